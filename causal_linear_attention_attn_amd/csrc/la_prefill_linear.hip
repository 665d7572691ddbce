// Chunked prefill for the LINEAR rule (elu+1 kernel, per-head decay, eps).
//
// Method ("What Is Linear Attention?" sections 2, 4, 5.1; "Efficient
// attention variants" sections 5, 7.1, 8; "Transformers Are RNNs"):
//     S_t = gamma S_{t-1} + phi(k_t) v_t^T,  z_t = gamma z_{t-1} + phi(k_t)
//     o_t = phi(q_t)^T S_t / (phi(q_t) . z_t + eps)
// evaluated chunk by chunk (the pages' chunkwise form: parallel inside a
// chunk, state passed between chunks).  For a chunk of C tokens starting
// from state (S-, z-), with Phi_q, Phi_k the chunk's features and chunk-local
// indices i, j:
//     A      = (Phi_q Phi_k^T) (.) D,  D_ij = gamma^(i-j) [j <= i]
//     num_i  = gamma^(i+1) phi(q_i)^T S-  +  (A V)_i
//     den_i  = gamma^(i+1) phi(q_i) . z-  +  (A 1)_i  +  eps
//     S+     = gamma^C S-  +  Phi_k^T diag(w) V,  w_j = gamma^(C-1-j)
//     z+     = gamma^C z-  +  Phi_k^T w
// which is the recurrence unrolled over the chunk.
//
// Long sequences are split into segments processed in parallel (a two-level
// scan, "Transformers Are RNNs": the recurrence is a prefix sum, so it can be
// scanned in parallel):
//   phase 1  summary_kernel  per (segment, head): the segment's own decayed
//            contribution (dS, dz) -- the chunk update from a zero state;
//   phase 2  scan_kernel     per head: prefix over segments,
//            P_{s+1} = gamma^L P_s + dS_s, P_0 = (S_in, z_in);
//   phase 3  chunk_kernel    per (segment, head): outputs from P_s, chunk by
//            chunk; the last segment writes (S_out, z_out).
// With one segment, phase 3 runs alone from (S_in, z_in).  The planner picks
// the segment count so that one launch fills every workgroup slot once.
//
// Data layout: q, k [BH, N, d], v, o [BH, N, dv] (row-major, dtype T);
// workspace slots [nseg][BH][d*dv + d] fp32 (state then normaliser).
//
// Per chunk, the kernel streams q, k, v once from HBM and writes o once.
// Global loads are issued one chunk ahead into registers (the next chunk's
// loads are in flight while the current chunk computes); each thread owns
// whole 16-byte column blocks of a few consecutive rows, so every wave reads
// contiguous row segments.  Tiles live in LDS: Phi_q and Phi_k row-major
// (token rows), Phi_k^T scaled by w and V^T (feature rows: the token
// contraction needs consecutive tokens per lane), a T-precision copy S^T of
// the fp32 state for the state read, and an output tile that turns the
// matrix-core output layout into 16-byte row stores.  The fp32 state itself
// lives in matrix-core accumulators and is never rounded.  All contractions
// run on the matrix cores (bf16 inputs: 16x16x32 bf16; fp32 inputs: 16x16x4
// fp32).  Powers of gamma come from a per-head table gamma^m, m = 0..C.
#include <atomic>

#include "la_common.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kLdsBytes = 160 * 1024;

template <typename T, int DK_, int DV_, int C_, int NW_>
struct Cfg {
  using type = T;
  using vec = typename Vec16<T>::type;
  static constexpr int DK = DK_, DV = DV_, C = C_, NW = NW_;
  static constexpr int NT = NW * kWave;
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte vector
  static constexpr int QLD = DK + VEC;  // row stride of Phi_q / Phi_k tiles
  static constexpr int TLD = C + VEC;   // row stride of Phi_k^T / V^T tiles
  static constexpr int SLD = DK + VEC;  // row stride of the S^T copy
  static constexpr int OLD = DV + VEC;  // row stride of the output tile
  static constexpr int NRB = C / 16;    // 16-row blocks of a chunk
  static constexpr int NG = NW / NRB;   // waves sharing one row block
  static constexpr int NPW = (DV / 16) / NG;  // output column tiles per wave
  static constexpr int NWN = NW / 4;    // state tiles: wave groups along dv
  static constexpr int TFW = (DK / 16) / 4;   // state row tiles per wave
  static constexpr int TNW = (DV / 16) / NWN; // state column tiles per wave
  static constexpr int KSD = DK / 32;   // k-steps over features
  static constexpr int KSC = C / 32;    // k-steps over tokens
  static constexpr int QCB = DK / VEC;  // 16-byte column blocks per q/k row
  static constexpr int VCB = DV / VEC;  // ... per v/o row
  static constexpr int RQ = C * DK / (VEC * NT);  // q/k rows per thread
  static constexpr int RV = C * DV / (VEC * NT);  // v/o rows per thread
  static_assert(NG >= 1 && NPW >= 1 && TFW >= 1 && TNW >= 1, "bad tiling");
  static_assert(NRB % 2 == 0, "chunk must hold an even number of row blocks");
  static_assert(RQ >= 1 && RQ * VEC * NT == C * DK, "q/k rows per thread");
  static_assert(RV >= 1 && RV * VEC * NT == C * DV, "v/o rows per thread");
};

template <class CF>
struct alignas(16) SmemChunk {
  using T = typename CF::type;
  T Qs[CF::C * CF::QLD];
  T Ks[CF::C * CF::QLD];
  T Kt[CF::DK * CF::TLD];
  T Vt[CF::DV * CF::TLD];
  T St[CF::DV * CF::SLD];
  T Os[CF::C * CF::OLD];
  float zs[CF::DK];
  float pw[CF::C + 4];  // gamma^m, m = 0..C
};

template <class CF>
struct alignas(16) SmemSummary {
  using T = typename CF::type;
  T Kt[CF::DK * CF::TLD];
  T Vt[CF::DV * CF::TLD];
  float pw[CF::C + 4];
};

// This thread's rows of one chunk, as loaded (raw 16-byte vectors).
template <class CF>
struct ChunkRegs {
  typename CF::vec q[CF::RQ], k[CF::RQ], v[CF::RV];
};

// Per-head buffer resources of q, k, v and o.  Every global access of the
// prefill goes through them, with out-of-range lanes given an offset past
// the resource (zero on load, dropped on store).
struct HeadBufs {
  __amdgpu_buffer_rsrc_t q, k, v, o;
};

template <typename T>
__device__ __forceinline__ HeadBufs head_bufs(const PrefillParams &p, int bh) {
  const size_t qk = (size_t)p.N * p.d, vo = (size_t)p.N * p.dv;
  HeadBufs hb;
  hb.q = buf_rsrc(reinterpret_cast<const T *>(p.q) + (size_t)bh * qk,
                  (uint32_t)(qk * sizeof(T)));
  hb.k = buf_rsrc(reinterpret_cast<const T *>(p.k) + (size_t)bh * qk,
                  (uint32_t)(qk * sizeof(T)));
  hb.v = buf_rsrc(reinterpret_cast<const T *>(p.v) + (size_t)bh * vo,
                  (uint32_t)(vo * sizeof(T)));
  hb.o = buf_rsrc(reinterpret_cast<const T *>(p.o) + (size_t)bh * vo,
                  (uint32_t)(vo * sizeof(T)));
  return hb;
}

// One 16-byte column block of row `tok` of a [N, ncols] tensor (zero where
// the row or a column is outside it).  VK: ncols is a multiple of the vector
// width, so a block is either wholly inside or wholly outside.
template <typename T, bool VK>
__device__ __forceinline__ typename Vec16<T>::type load_block(
    __amdgpu_buffer_rsrc_t r, int tok, int col0, int ncols, bool row_ok) {
  constexpr int VEC = 16 / (int)sizeof(T);
  if constexpr (VK) {
    const bool ok = row_ok && col0 < ncols;
    return buf_load16<T>(r, ok ? (uint32_t)(((size_t)tok * ncols + col0) * sizeof(T))
                               : kOOB);
  } else {
    typename Vec16<T>::type x;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const bool ok = row_ok && col0 + e < ncols;
      x[e] = buf_load1(r, ok ? (uint32_t)(((size_t)tok * ncols + col0 + e) * sizeof(T))
                             : kOOB, (T *)nullptr);
    }
    return x;
  }
}

template <class CF, bool WITH_Q, bool VK>
__device__ __forceinline__ void prefetch(ChunkRegs<CF> &R, const PrefillParams &p,
                                         const HeadBufs &hb, int c0, int Lc) {
  using T = typename CF::type;
  const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
#pragma unroll
  for (int r = 0; r < CF::RQ; ++r) {
    const int row = qrg * CF::RQ + r;
    if constexpr (WITH_Q)
      R.q[r] = load_block<T, VK>(hb.q, c0 + row, qcb * CF::VEC, p.d, row < Lc);
    R.k[r] = load_block<T, VK>(hb.k, c0 + row, qcb * CF::VEC, p.d, row < Lc);
  }
  const int vcb = threadIdx.x % CF::VCB, vrg = threadIdx.x / CF::VCB;
#pragma unroll
  for (int r = 0; r < CF::RV; ++r) {
    const int row = vrg * CF::RV + r;
    R.v[r] = load_block<T, VK>(hb.v, c0 + row, vcb * CF::VEC, p.dv, row < Lc);
  }
}

// Registers -> LDS tiles.  Feature-map padding rule: lanes outside the
// tensor (tokens past N, features past d) are zero AFTER phi (phi(0) = 1
// would be wrong).
template <class CF, bool WITH_Q>
__device__ __forceinline__ void commit(const ChunkRegs<CF> &R,
                                       typename CF::type *Qs,
                                       typename CF::type *Ks,
                                       typename CF::type *Kt,
                                       typename CF::type *Vt, const float *pw,
                                       const PrefillParams &p, int Lc) {
  using T = typename CF::type;
  constexpr int VEC = CF::VEC;
  const bool elu = p.fmap != 0;
  const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
  const int col0 = qcb * VEC;
  float kw[VEC][CF::RQ];
#pragma unroll
  for (int r = 0; r < CF::RQ; ++r) {
    const int row = qrg * CF::RQ + r;
    const bool ok = row < Lc;
    float x[VEC];
    if constexpr (WITH_Q) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float xq = to_f32(R.q[r][e]);
        x[e] = (ok && col0 + e < p.d) ? (elu ? phi_elu1(xq) : xq) : 0.f;
      }
      lds_store_n<T, VEC>(Qs + row * CF::QLD + col0, x);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float xk = to_f32(R.k[r][e]);
      x[e] = (ok && col0 + e < p.d) ? (elu ? phi_elu1(xk) : xk) : 0.f;
    }
    if constexpr (WITH_Q) lds_store_n<T, VEC>(Ks + row * CF::QLD + col0, x);
    const float w = ok ? pw[Lc - 1 - row] : 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) kw[e][r] = x[e] * w;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e)
    lds_store_n<T, CF::RQ>(Kt + (col0 + e) * CF::TLD + qrg * CF::RQ, kw[e]);

  const int vcb = threadIdx.x % CF::VCB, vrg = threadIdx.x / CF::VCB;
  float vt[VEC][CF::RV];
#pragma unroll
  for (int r = 0; r < CF::RV; ++r)
#pragma unroll
    for (int e = 0; e < VEC; ++e) vt[e][r] = to_f32(R.v[r][e]);
#pragma unroll
  for (int e = 0; e < VEC; ++e)
    lds_store_n<T, CF::RV>(Vt + (vcb * VEC + e) * CF::TLD + vrg * CF::RV, vt[e]);
}

// S <- gamma^Lc S + Phi_k^T diag(w) V and z <- gamma^Lc z + Phi_k^T w for the
// state tiles this wave owns (Kt already carries the weights w).
template <class CF>
__device__ __forceinline__ void state_update(
    f32x4 (&Sacc)[CF::TFW][CF::TNW], float (&zreg)[CF::TFW],
    const typename CF::type *Kt, const typename CF::type *Vt, float gC, int wf,
    int wn, int li, int lg) {
  using T = typename CF::type;
#pragma unroll
  for (int a = 0; a < CF::TFW; ++a) {
    const int tf = wf * CF::TFW + a;
#pragma unroll
    for (int b = 0; b < CF::TNW; ++b) Sacc[a][b] *= gC;
    float zsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < CF::KSC; ++ks) {
      Frag<T> kf;
      lds_frag(kf, Kt + (16 * tf + li) * CF::TLD + 32 * ks + 8 * lg);
      if (wn == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) zsum += frag_elem(kf, e);
      }
#pragma unroll
      for (int b = 0; b < CF::TNW; ++b) {
        const int tn = wn * CF::TNW + b;
        Frag<T> vf;
        lds_frag(vf, Vt + (16 * tn + li) * CF::TLD + 32 * ks + 8 * lg);
        mma(Sacc[a][b], kf, vf);
      }
    }
    if (wn == 0) zreg[a] = fmaf(gC, zreg[a], sum_groups(zsum));
  }
}

// T-precision copy of the state for the next chunk's read: St[n][f] = S[f][n].
template <class CF>
__device__ __forceinline__ void write_state_copy(
    typename CF::type *St, float *zs, const f32x4 (&Sacc)[CF::TFW][CF::TNW],
    const float (&zreg)[CF::TFW], int wf, int wn, int li, int lg) {
#pragma unroll
  for (int a = 0; a < CF::TFW; ++a) {
    const int tf = wf * CF::TFW + a;
#pragma unroll
    for (int b = 0; b < CF::TNW; ++b) {
      const int tn = wn * CF::TNW + b;
      lds_store4(St + (16 * tn + li) * CF::SLD + 16 * tf + 4 * lg, Sacc[a][b][0],
                 Sacc[a][b][1], Sacc[a][b][2], Sacc[a][b][3]);
    }
    if (wn == 0 && lg == 0) zs[16 * tf + li] = zreg[a];
  }
}

template <class CF>
__device__ __forceinline__ void fill_powers(float *pw, float log2g) {
  for (int m = threadIdx.x; m <= CF::C; m += CF::NT) pw[m] = exp2f((float)m * log2g);
}

template <class CF, bool VK>
__global__ void __launch_bounds__(CF::NT) chunk_kernel(PrefillParams p) {
  using T = typename CF::type;
  using V = typename CF::vec;
  __shared__ SmemChunk<CF> sm;

  const int seg = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const size_t rec = (size_t)d * dv + d;
  const HeadBufs hb = head_bufs<T>(p, bh);
  const int t_begin = seg * p.seg_len;
  const int t_end = min(N, t_begin + p.seg_len);

  const float *S0, *z0;
  if (p.nseg > 1) {
    S0 = p.ws + ((size_t)seg * p.BH + bh) * rec;
    z0 = S0 + (size_t)d * dv;
  } else {
    S0 = p.S_in ? p.S_in + (size_t)bh * d * dv : nullptr;
    z0 = p.z_in ? p.z_in + (size_t)bh * d : nullptr;
  }

  const int rb = wv % CF::NRB, ng = wv / CF::NRB;  // output role
  const int wf = wv % 4, wn = wv / 4;              // state-tile role
  const int irow = 16 * rb + li;  // chunk row this lane carries as an operand

  f32x4 Sacc[CF::TFW][CF::TNW];
  float zreg[CF::TFW];
#pragma unroll
  for (int a = 0; a < CF::TFW; ++a) {
    const int tf = wf * CF::TFW + a;
#pragma unroll
    for (int b = 0; b < CF::TNW; ++b) {
      const int n = 16 * (wn * CF::TNW + b) + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * tf + 4 * lg + r;
        Sacc[a][b][r] = (S0 && f < d && n < dv) ? S0[(size_t)f * dv + n] : 0.f;
      }
    }
    const int fz = 16 * tf + li;
    zreg[a] = (z0 && fz < d) ? z0[fz] : 0.f;
  }
  // the first chunk's loads go out after the state loads (loads complete in
  // issue order, so waiting for the state does not wait for the chunk)
  ChunkRegs<CF> R;
  prefetch<CF, true, VK>(R, p, hb, t_begin, min(CF::C, N - t_begin));
  fill_powers<CF>(sm.pw, p.gamma ? log2f(p.gamma[bh % p.H]) : 0.f);
  write_state_copy<CF>(sm.St, sm.zs, Sacc, zreg, wf, wn, li, lg);
  __syncthreads();

  for (int c0 = t_begin; c0 < t_end; c0 += CF::C) {
    const int Lc = min(CF::C, N - c0);
    commit<CF, true>(R, sm.Qs, sm.Ks, sm.Kt, sm.Vt, sm.pw, p, Lc);
    __syncthreads();
    if (c0 + CF::C < t_end)
      prefetch<CF, true, VK>(R, p, hb, c0 + CF::C, min(CF::C, N - c0 - CF::C));

    // ---- state read: gamma^(i+1) phi(q_i)^T S-, and phi(q_i) . z- ----
    Frag<T> qf[CF::KSD];
    float dz = 0.f;
#pragma unroll
    for (int ks = 0; ks < CF::KSD; ++ks) {
      lds_frag(qf[ks], sm.Qs + irow * CF::QLD + 32 * ks + 8 * lg);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dz = fmaf(frag_elem(qf[ks], e), sm.zs[32 * ks + 8 * lg + e], dz);
    }
    f32x4 acc[CF::NPW];
#pragma unroll
    for (int nt = 0; nt < CF::NPW; ++nt) {
      acc[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
      const int n = 16 * (ng * CF::NPW + nt) + li;
#pragma unroll
      for (int ks = 0; ks < CF::KSD; ++ks) {
        Frag<T> sf;
        lds_frag(sf, sm.St + n * CF::SLD + 32 * ks + 8 * lg);
        mma(acc[nt], qf[ks], sf);
      }
    }
    dz = sum_groups(dz) * sm.pw[irow + 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sc = sm.pw[16 * rb + 4 * lg + r + 1];
#pragma unroll
      for (int nt = 0; nt < CF::NPW; ++nt) acc[nt][r] *= sc;
    }

    // ---- intra-chunk: A = (Phi_q Phi_k^T) (.) D, computed as A^T tiles ----
    // at[tj][r] = A[i = 16 rb + li][j = 16 tj + 4 lg + r]
    f32x4 at[CF::NRB];
    float dintra = 0.f;
#pragma unroll
    for (int tj = 0; tj < CF::NRB; ++tj) {
      at[tj] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (tj <= rb) {
#pragma unroll
        for (int ks = 0; ks < CF::KSD; ++ks) {
          Frag<T> kf;
          lds_frag(kf, sm.Ks + (16 * tj + li) * CF::QLD + 32 * ks + 8 * lg);
          mma(at[tj], kf, qf[ks]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lag = irow - (16 * tj + 4 * lg + r);
          float x = lag >= 0 ? at[tj][r] * sm.pw[lag] : 0.f;
          x = to_f32(from_f32<T>(x));  // the weight the product below uses
          at[tj][r] = x;
          dintra += x;
        }
      }
    }
    dintra = sum_groups(dintra);
    // A V: two A^T tiles form one 32-token operand (slots e < 4 from tile
    // 2pp, e >= 4 from tile 2pp+1), matched by the same tokens of V^T.
#pragma unroll
    for (int pp = 0; pp < CF::NRB / 2; ++pp) {
      if (2 * pp <= rb) {
        Frag<T> af;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          frag_set(af, e, at[2 * pp][e]);
          frag_set(af, 4 + e, at[2 * pp + 1][e]);
        }
#pragma unroll
        for (int nt = 0; nt < CF::NPW; ++nt) {
          const int n = 16 * (ng * CF::NPW + nt) + li;
          Frag<T> vf;
          lds_half(vf, sm.Vt + n * CF::TLD + 32 * pp + 4 * lg, 0);
          lds_half(vf, sm.Vt + n * CF::TLD + 32 * pp + 16 + 4 * lg, 4);
          mma(acc[nt], af, vf);
        }
      }
    }

    // ---- normalise into the output tile ----
    const float den = dz + dintra + p.eps;  // for row irow
    float rden[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rden[r] = 1.f / __shfl(den, 4 * lg + r);
#pragma unroll
    for (int nt = 0; nt < CF::NPW; ++nt) {
      const int n = 16 * (ng * CF::NPW + nt) + li;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sm.Os[(16 * rb + 4 * lg + r) * CF::OLD + n] = from_f32<T>(acc[nt][r] * rden[r]);
    }

    // ---- carry the state across the chunk ----
    state_update<CF>(Sacc, zreg, sm.Kt, sm.Vt, sm.pw[Lc], wf, wn, li, lg);
    __syncthreads();
    write_state_copy<CF>(sm.St, sm.zs, Sacc, zreg, wf, wn, li, lg);
    // 16-byte row stores of the output tile
    {
      const int vcb = threadIdx.x % CF::VCB, vrg = threadIdx.x / CF::VCB;
      const int col0 = vcb * CF::VEC;
#pragma unroll
      for (int r = 0; r < CF::RV; ++r) {
        const int row = vrg * CF::RV + r;
        const V val = *reinterpret_cast<const V *>(sm.Os + row * CF::OLD + col0);
        const size_t el = (size_t)(c0 + row) * dv + col0;
        if constexpr (VK) {
          const bool ok = row < Lc && col0 < dv;
          buf_store16<T>(hb.o, ok ? (uint32_t)(el * sizeof(T)) : kOOB, val);
        } else {
#pragma unroll
          for (int e = 0; e < CF::VEC; ++e) {
            const bool ok = row < Lc && col0 + e < dv;
            buf_store1(hb.o, ok ? (uint32_t)((el + e) * sizeof(T)) : kOOB, val[e]);
          }
        }
      }
    }
  }

  if (seg == p.nseg - 1) {
    if (p.S_out) {
      float *So = p.S_out + (size_t)bh * d * dv;
#pragma unroll
      for (int a = 0; a < CF::TFW; ++a)
#pragma unroll
        for (int b = 0; b < CF::TNW; ++b) {
          const int n = 16 * (wn * CF::TNW + b) + li;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int f = 16 * (wf * CF::TFW + a) + 4 * lg + r;
            if (f < d && n < dv) So[(size_t)f * dv + n] = Sacc[a][b][r];
          }
        }
    }
    if (p.z_out && wn == 0 && lg == 0) {
#pragma unroll
      for (int a = 0; a < CF::TFW; ++a) {
        const int f = 16 * (wf * CF::TFW + a) + li;
        if (f < d) p.z_out[(size_t)bh * d + f] = zreg[a];
      }
    }
  }
}

// Phase 1: each segment's own contribution, from a zero state (all but the
// last segment; those are whole multiples of the chunk length).
template <class CF, bool VK>
__global__ void __launch_bounds__(CF::NT) summary_kernel(PrefillParams p) {
  using T = typename CF::type;
  __shared__ SmemSummary<CF> sm;
  const int seg = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const size_t rec = (size_t)d * dv + d;
  const HeadBufs hb = head_bufs<T>(p, bh);
  const int t_begin = seg * p.seg_len;
  const int t_end = t_begin + p.seg_len;
  const int wf = wv % 4, wn = wv / 4;

  ChunkRegs<CF> R;
  prefetch<CF, false, VK>(R, p, hb, t_begin, CF::C);
  fill_powers<CF>(sm.pw, p.gamma ? log2f(p.gamma[bh % p.H]) : 0.f);

  f32x4 Sacc[CF::TFW][CF::TNW];
  float zreg[CF::TFW];
#pragma unroll
  for (int a = 0; a < CF::TFW; ++a) {
    zreg[a] = 0.f;
#pragma unroll
    for (int b = 0; b < CF::TNW; ++b) Sacc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  const float gC = sm.pw[CF::C];
  for (int c0 = t_begin; c0 < t_end; c0 += CF::C) {
    commit<CF, false>(R, nullptr, nullptr, sm.Kt, sm.Vt, sm.pw, p, CF::C);
    __syncthreads();
    if (c0 + CF::C < t_end) prefetch<CF, false, VK>(R, p, hb, c0 + CF::C, CF::C);
    state_update<CF>(Sacc, zreg, sm.Kt, sm.Vt, gC, wf, wn, li, lg);
    __syncthreads();
  }
  float *dst = p.ws + ((size_t)(seg + 1) * p.BH + bh) * rec;
#pragma unroll
  for (int a = 0; a < CF::TFW; ++a) {
#pragma unroll
    for (int b = 0; b < CF::TNW; ++b) {
      const int n = 16 * (wn * CF::TNW + b) + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * (wf * CF::TFW + a) + 4 * lg + r;
        if (f < d && n < dv) dst[(size_t)f * dv + n] = Sacc[a][b][r];
      }
    }
    const int f = 16 * (wf * CF::TFW + a) + li;
    if (wn == 0 && lg == 0 && f < d) dst[(size_t)d * dv + f] = zreg[a];
  }
}

// Phase 2: prefix over segments, in place: slot 0 <- (S_in, z_in),
// slot s <- gamma^L slot (s-1) + dS_(s-1) for s >= 1.
__global__ void __launch_bounds__(256) scan_kernel(PrefillParams p) {
  const int bh = blockIdx.y;
  const size_t rec = (size_t)p.d * p.dv + p.d;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= rec) return;
  const float log2g = p.gamma ? log2f(p.gamma[bh % p.H]) : 0.f;
  const float gL = exp2f((float)p.seg_len * log2g);
  const size_t dd = (size_t)p.d * p.dv;
  float acc;
  if (e < dd)
    acc = p.S_in ? p.S_in[(size_t)bh * dd + e] : 0.f;
  else
    acc = p.z_in ? p.z_in[(size_t)bh * p.d + (e - dd)] : 0.f;
  float *base = p.ws + (size_t)bh * rec + e;
  const size_t stride = (size_t)p.BH * rec;
  base[0] = acc;
  for (int s = 1; s < p.nseg; ++s) {
    acc = fmaf(gL, acc, base[s * stride]);
    base[s * stride] = acc;
  }
}

template <class CF, bool VK>
hipError_t run_vk(const PrefillParams &p, hipStream_t s) {
  static_assert(sizeof(SmemChunk<CF>) <= kLdsBytes, "LDS budget");
  if (p.nseg > 1) {
    prof_begin(s);
    hipLaunchKernelGGL((summary_kernel<CF, VK>), dim3(p.nseg - 1, p.BH), dim3(CF::NT),
                       0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_end("linear_summary", s);
    const size_t rec = (size_t)p.d * p.dv + p.d;
    prof_begin(s);
    hipLaunchKernelGGL(scan_kernel, dim3((unsigned)((rec + 255) / 256), p.BH),
                       dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_end("linear_scan", s);
  }
  prof_begin(s);
  hipLaunchKernelGGL((chunk_kernel<CF, VK>), dim3(p.nseg, p.BH), dim3(CF::NT), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) prof_end("linear_chunk", s);
  return e;
}

template <class CF>
hipError_t run(const PrefillParams &p, hipStream_t s) {
  return p.vec_ok ? run_vk<CF, true>(p, s) : run_vk<CF, false>(p, s);
}

// Workgroups of chunk_kernel<CF> that fit on one CU (queried once).
template <class CF>
int resident_per_cu() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, chunk_kernel<CF, true>, CF::NT, 0) !=
          hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  cached.store(n, std::memory_order_relaxed);
  return n;
}

// Instantiations: bf16 uses 64-token chunks; fp32 uses 32-token chunks
// (64 at d = dv = 64) so that its fp32 tiles fit in LDS.
using B64x64 = Cfg<bf16, 64, 64, 64, 4>;
using B64x128 = Cfg<bf16, 64, 128, 64, 8>;
using B128x64 = Cfg<bf16, 128, 64, 64, 8>;
using B128x128 = Cfg<bf16, 128, 128, 64, 8>;
using F64x64 = Cfg<float, 64, 64, 64, 4>;
using F64x128 = Cfg<float, 64, 128, 32, 4>;
using F128x64 = Cfg<float, 128, 64, 32, 4>;
using F128x128 = Cfg<float, 128, 128, 32, 4>;

template <class CF>
void fill_plan(LinearPlan &pl) {
  pl.chunk = CF::C;
  pl.threads = CF::NT;
  pl.per_cu = resident_per_cu<CF>();
}

}  // namespace

LinearPlan plan_linear(int BH, int N, int d, int dv, bool bf16_io) {
  LinearPlan pl{};
  pl.dk = d <= 64 ? 64 : 128;
  pl.dv_pad = dv <= 64 ? 64 : 128;
  if (bf16_io) {
    if (pl.dk == 64) pl.dv_pad == 64 ? fill_plan<B64x64>(pl) : fill_plan<B64x128>(pl);
    else pl.dv_pad == 64 ? fill_plan<B128x64>(pl) : fill_plan<B128x128>(pl);
  } else {
    if (pl.dk == 64) pl.dv_pad == 64 ? fill_plan<F64x64>(pl) : fill_plan<F64x128>(pl);
    else pl.dv_pad == 64 ? fill_plan<F128x64>(pl) : fill_plan<F128x128>(pl);
  }
  const long chunks = N > 0 ? ((long)N + pl.chunk - 1) / pl.chunk : 0;
  long nseg = 1;
  if (chunks > 1 && BH > 0) {
    // one launch fills every resident workgroup slot once
    const long slots = (long)device_cu_count() * pl.per_cu;
    nseg = (slots + BH / 2) / BH;
    if (nseg > chunks) nseg = chunks;
    if (nseg < 1) nseg = 1;
  }
  const long cps = chunks > 0 ? (chunks + nseg - 1) / nseg : 1;
  nseg = chunks > 0 ? (chunks + cps - 1) / cps : 1;
  pl.nseg = (int)nseg;
  pl.seg_len = (int)(cps * pl.chunk);
  pl.ws_bytes = nseg > 1 ? (size_t)nseg * BH * ((size_t)d * dv + d) * sizeof(float)
                         : 0;
  return pl;
}

hipError_t launch_linear_prefill(const PrefillParams &p, const LinearPlan &pl,
                                 bool bf16_io, hipStream_t s) {
  if (bf16_io) {
    if (pl.dk == 64) return pl.dv_pad == 64 ? run<B64x64>(p, s) : run<B64x128>(p, s);
    return pl.dv_pad == 64 ? run<B128x64>(p, s) : run<B128x128>(p, s);
  }
  if (pl.dk == 64) return pl.dv_pad == 64 ? run<F64x64>(p, s) : run<F64x128>(p, s);
  return pl.dv_pad == 64 ? run<F128x64>(p, s) : run<F128x128>(p, s);
}

}  // namespace la
