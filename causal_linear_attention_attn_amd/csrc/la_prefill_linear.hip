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
// With one segment, phase 3 runs alone from (S_in, z_in).
//
// Data layout: q, k [BH, N, d], v, o [BH, N, dv] (row-major, dtype T);
// workspace slots [nseg][BH][d*dv + d] fp32 (state then normaliser).
//
// Tiles live in LDS: Phi_q and Phi_k row-major (token rows), Phi_k^T scaled
// by w and V^T (feature rows: the token contraction needs consecutive tokens
// per lane), and a T-precision copy S^T of the fp32 state for the state read.
// The fp32 state itself lives in matrix-core accumulators and is never
// rounded.  All contractions run on the matrix cores (bf16 inputs: 16x16x32
// bf16; fp32 inputs: 16x16x4 fp32).
#include "la_common.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

template <typename T, int DK_, int DV_, int C_, int NW_>
struct Cfg {
  using type = T;
  static constexpr int DK = DK_, DV = DV_, C = C_, NW = NW_;
  static constexpr int NT = NW * kWave;
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte vector
  static constexpr int QLD = DK + VEC;  // row stride of Phi_q / Phi_k tiles
  static constexpr int TLD = C + VEC;   // row stride of Phi_k^T / V^T tiles
  static constexpr int SLD = DK + VEC;  // row stride of the S^T copy
  static constexpr int NRB = C / 16;    // 16-row blocks of a chunk
  static constexpr int NG = NW / NRB;   // waves sharing one row block
  static constexpr int NPW = (DV / 16) / NG;  // output column tiles per wave
  static constexpr int NWN = NW / 4;    // state tiles: wave groups along dv
  static constexpr int TFW = (DK / 16) / 4;   // state row tiles per wave
  static constexpr int TNW = (DV / 16) / NWN; // state column tiles per wave
  static constexpr int KSD = DK / 32;   // k-steps over features
  static constexpr int KSC = C / 32;    // k-steps over tokens
  static_assert(NG >= 1 && NPW >= 1 && TFW >= 1 && TNW >= 1, "bad tiling");
  static_assert(NRB % 2 == 0, "chunk must hold an even number of row blocks");
};

template <class CF>
struct alignas(16) SmemChunk {
  using T = typename CF::type;
  T Qs[CF::C * CF::QLD];
  T Ks[CF::C * CF::QLD];
  T Kt[CF::DK * CF::TLD];
  T Vt[CF::DV * CF::TLD];
  T St[CF::DV * CF::SLD];
  float zs[CF::DK];
};

template <class CF>
struct alignas(16) SmemSummary {
  using T = typename CF::type;
  T Kt[CF::DK * CF::TLD];
  T Vt[CF::DV * CF::TLD];
};

// VEC consecutive elements of one row as fp32; zero outside the tensor.
template <typename T, int VEC>
__device__ __forceinline__ void load_vec(float (&x)[VEC], const T *row, int col0,
                                         int ncols, bool row_ok, bool vec_ok) {
  if (!row_ok) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) x[e] = 0.f;
    return;
  }
  if (vec_ok && col0 + VEC <= ncols) {
    if constexpr (sizeof(T) == 2) {
      const bf16x8 r = *reinterpret_cast<const bf16x8 *>(row + col0);
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = (float)r[e];
    } else {
      const f32x4 r = *reinterpret_cast<const f32x4 *>(row + col0);
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = r[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      x[e] = (col0 + e < ncols) ? to_f32(row[col0 + e]) : 0.f;
  }
}

template <typename T, int VEC>
__device__ __forceinline__ void store_row_vec(T *dst, const float (&x)[VEC]) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < VEC; ++e) r[e] = (bf16)x[e];
    *reinterpret_cast<bf16x8 *>(dst) = r;
  } else {
    *reinterpret_cast<f32x4 *>(dst) = (f32x4){x[0], x[1], x[2], x[3]};
  }
}

// Stage one chunk into LDS.  Work unit: 4 token rows x VEC columns.
// Feature-map padding rule: lanes outside the tensor (tokens past N, features
// past d) are zero AFTER phi (phi(0) = 1 would be wrong).
template <class CF, bool WITH_ROWS>
__device__ __forceinline__ void stage_chunk(
    typename CF::type *Qs, typename CF::type *Ks, typename CF::type *Kt,
    typename CF::type *Vt, const PrefillParams &p, const typename CF::type *qh,
    const typename CF::type *kh, const typename CF::type *vh, int c0, int Lc,
    float log2g) {
  using T = typename CF::type;
  constexpr int VEC = CF::VEC, C = CF::C;
  constexpr int UQ = (C / 4) * (CF::DK / VEC);
  constexpr int UV = (C / 4) * (CF::DV / VEC);
  const int d = p.d, dv = p.dv;
  const bool vec_ok = p.vec_ok != 0;
  const bool elu = p.fmap != 0;

  if constexpr (WITH_ROWS) {
    for (int u = threadIdx.x; u < UQ; u += CF::NT) {
      const int r0 = (u / (CF::DK / VEC)) * 4, col0 = (u % (CF::DK / VEC)) * VEC;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = r0 + rr;
        float x[VEC];
        load_vec<T, VEC>(x, qh + (size_t)(c0 + r) * d, col0, d, r < Lc, vec_ok);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          x[e] = (r < Lc && col0 + e < d) ? (elu ? phi_elu1(x[e]) : x[e]) : 0.f;
        store_row_vec<T, VEC>(Qs + r * CF::QLD + col0, x);
      }
    }
  }
  for (int u = threadIdx.x; u < UQ; u += CF::NT) {
    const int r0 = (u / (CF::DK / VEC)) * 4, col0 = (u % (CF::DK / VEC)) * VEC;
    float kt[4][VEC];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = r0 + rr;
      float x[VEC];
      load_vec<T, VEC>(x, kh + (size_t)(c0 + r) * d, col0, d, r < Lc, vec_ok);
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        x[e] = (r < Lc && col0 + e < d) ? (elu ? phi_elu1(x[e]) : x[e]) : 0.f;
      if constexpr (WITH_ROWS) store_row_vec<T, VEC>(Ks + r * CF::QLD + col0, x);
      const float w = r < Lc ? exp2f((float)(Lc - 1 - r) * log2g) : 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) kt[rr][e] = x[e] * w;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      lds_store4(Kt + (col0 + e) * CF::TLD + r0, kt[0][e], kt[1][e], kt[2][e],
                 kt[3][e]);
  }
  for (int u = threadIdx.x; u < UV; u += CF::NT) {
    const int r0 = (u / (CF::DV / VEC)) * 4, col0 = (u % (CF::DV / VEC)) * VEC;
    float vt[4][VEC];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      load_vec<T, VEC>(vt[rr], vh + (size_t)(c0 + r0 + rr) * dv, col0, dv,
                       r0 + rr < Lc, vec_ok);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      lds_store4(Vt + (col0 + e) * CF::TLD + r0, vt[0][e], vt[1][e], vt[2][e],
                 vt[3][e]);
  }
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
__global__ void __launch_bounds__(CF::NT) chunk_kernel(PrefillParams p) {
  using T = typename CF::type;
  __shared__ SmemChunk<CF> sm;

  const int seg = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const float log2g = p.gamma ? log2f(p.gamma[bh % p.H]) : 0.f;
  const size_t rec = (size_t)d * dv + d;
  const T *qh = reinterpret_cast<const T *>(p.q) + (size_t)bh * N * d;
  const T *kh = reinterpret_cast<const T *>(p.k) + (size_t)bh * N * d;
  const T *vh = reinterpret_cast<const T *>(p.v) + (size_t)bh * N * dv;
  T *oh = reinterpret_cast<T *>(p.o) + (size_t)bh * N * dv;
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
  write_state_copy<CF>(sm.St, sm.zs, Sacc, zreg, wf, wn, li, lg);

  for (int c0 = t_begin; c0 < t_end; c0 += CF::C) {
    const int Lc = min(CF::C, N - c0);
    stage_chunk<CF, true>(sm.Qs, sm.Ks, sm.Kt, sm.Vt, p, qh, kh, vh, c0, Lc,
                          log2g);
    __syncthreads();

    // ---- state read: gamma^(i+1) phi(q_i)^T S-, and phi(q_i) . z- ----
    const int irow = 16 * rb + li;  // row this lane carries as an operand
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
    dz = sum_groups(dz) * exp2f((float)(irow + 1) * log2g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sc = exp2f((float)(16 * rb + 4 * lg + r + 1) * log2g);
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
          float x = lag >= 0 ? at[tj][r] * exp2f((float)lag * log2g) : 0.f;
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

    // ---- normalise and store ----
    const float den = dz + dintra + p.eps;  // for row irow
    float dr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dr[r] = __shfl(den, 4 * lg + r);
#pragma unroll
    for (int nt = 0; nt < CF::NPW; ++nt) {
      const int n = 16 * (ng * CF::NPW + nt) + li;
      if (n < dv) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * rb + 4 * lg + r;
          if (i < Lc) oh[(size_t)(c0 + i) * dv + n] = from_f32<T>(acc[nt][r] / dr[r]);
        }
      }
    }

    // ---- carry the state across the chunk ----
    state_update<CF>(Sacc, zreg, sm.Kt, sm.Vt, exp2f((float)Lc * log2g), wf, wn,
                     li, lg);
    __syncthreads();
    write_state_copy<CF>(sm.St, sm.zs, Sacc, zreg, wf, wn, li, lg);
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
template <class CF>
__global__ void __launch_bounds__(CF::NT) summary_kernel(PrefillParams p) {
  using T = typename CF::type;
  __shared__ SmemSummary<CF> sm;
  const int seg = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const float log2g = p.gamma ? log2f(p.gamma[bh % p.H]) : 0.f;
  const size_t rec = (size_t)d * dv + d;
  const T *kh = reinterpret_cast<const T *>(p.k) + (size_t)bh * N * d;
  const T *vh = reinterpret_cast<const T *>(p.v) + (size_t)bh * N * dv;
  const int t_begin = seg * p.seg_len;
  const int t_end = t_begin + p.seg_len;
  const int wf = wv % 4, wn = wv / 4;

  f32x4 Sacc[CF::TFW][CF::TNW];
  float zreg[CF::TFW];
#pragma unroll
  for (int a = 0; a < CF::TFW; ++a) {
    zreg[a] = 0.f;
#pragma unroll
    for (int b = 0; b < CF::TNW; ++b) Sacc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  const float gC = exp2f((float)CF::C * log2g);
  for (int c0 = t_begin; c0 < t_end; c0 += CF::C) {
    stage_chunk<CF, false>(nullptr, nullptr, sm.Kt, sm.Vt, p, nullptr, kh, vh,
                           c0, CF::C, log2g);
    __syncthreads();
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

template <class CF>
hipError_t run(const PrefillParams &p, hipStream_t s) {
  if (p.nseg > 1) {
    prof_begin(s);
    hipLaunchKernelGGL(summary_kernel<CF>, dim3(p.nseg - 1, p.BH), dim3(CF::NT),
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
  hipLaunchKernelGGL(chunk_kernel<CF>, dim3(p.nseg, p.BH), dim3(CF::NT), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) prof_end("linear_chunk", s);
  return e;
}

// Instantiations: bf16 uses 64-token chunks; fp32 at 128 x 128 uses 32-token
// chunks so that its fp32 tiles fit in LDS.
using B64x64 = Cfg<bf16, 64, 64, 64, 4>;
using B64x128 = Cfg<bf16, 64, 128, 64, 8>;
using B128x64 = Cfg<bf16, 128, 64, 64, 8>;
using B128x128 = Cfg<bf16, 128, 128, 64, 8>;
using F64x64 = Cfg<float, 64, 64, 64, 4>;
using F64x128 = Cfg<float, 64, 128, 64, 4>;
using F128x64 = Cfg<float, 128, 64, 64, 4>;
using F128x128 = Cfg<float, 128, 128, 32, 4>;

}  // namespace

LinearPlan plan_linear(int BH, int N, int d, int dv, bool bf16_io) {
  LinearPlan pl{};
  pl.dk = d <= 64 ? 64 : 128;
  pl.dv_pad = dv <= 64 ? 64 : 128;
  const bool big = pl.dk == 128 && pl.dv_pad == 128;
  pl.chunk = (!bf16_io && big) ? 32 : 64;
  pl.threads = bf16_io ? ((pl.dk == 64 && pl.dv_pad == 64) ? 256 : 512) : 256;
  const long chunks = N > 0 ? ((long)N + pl.chunk - 1) / pl.chunk : 0;
  long nseg = 1;
  if (chunks > 1 && BH > 0) {
    const long target = 2L * device_cu_count();  // workgroups per launch
    nseg = (target + BH - 1) / BH;
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
