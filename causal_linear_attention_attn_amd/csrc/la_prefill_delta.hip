// Chunked prefill for the gated DELTA rule.
//
// Method ("What Is Linear Attention?" sections 5.2-5.3): per token,
//     S_t = S_{t-1} + g_t k_t (v_t - S_{t-1}^T k_t)^T,     o_t = S_t^T q_t
// with raw q and k, S stored [d, dv].  The pages give no chunked form; the
// one used here follows by substitution.  For a chunk of C tokens (rows of
// K, Q, V; gates g) entering with state S-, write u_j = g_j (v_j - S_{j-1}^T
// k_j) for the row that token j adds (S_j = S_{j-1} + k_j u_j^T).  Unrolling
// S_{j-1} = S- + sum_{i<j} k_i u_i^T gives the lower-triangular system
//     (I + diag(g) L) U = diag(g) (V - K S-),   L = strict_lower(K K^T)
// so with T = (I + diag(g) L)^(-1) diag(g) and Y = V - K S-:
//     U  = T Y
//     O  = Q S- + P U = Q S- + R Y,   P = lower_incl(Q K^T),  R = P T
//     S+ = S- + K^T U
// T and R depend only on the chunk's q, k and g, so they are computed for
// every chunk in parallel (prep_kernel); the state-dependent part is a
// sequential pass over chunks (seq_kernel).  The columns of S are
// independent, so the sequential pass is split along dv into slices of W
// columns, one workgroup per (head, slice).
//
// prep_kernel, one workgroup per (chunk, head):
//   K K^T and Q K^T on the matrix cores (lower tiles only); the unit lower
//   triangular inverse X = (I + diag(g) L)^(-1) in fp32, 16x16 diagonal
//   blocks by forward substitution, then the blocks below the diagonal
//   block row by block row, X_ij = -X_ii sum_{j<=m<i} N_im X_mj with
//   N = diag(g) L; T = X diag(g); R = P T on the fp32 matrix cores.
//   T and R are stored in the input precision, [BH][chunk][C][C].
// seq_kernel, one workgroup per (head, dv slice), chunk after chunk:
//   X = K S-, Z = Q S- (S- read from a T-precision copy of the fp32 state);
//   Y = V - X;  U = T Y;  O = Z + R Y;  S+ = S- + K^T U (fp32 accumulators,
//   never rounded).  Global loads run one chunk ahead in registers; K^T is
//   double-buffered so the next chunk's tiles are written while the state
//   update of the current one still reads the old K^T.
//
// Workgroups of one head's slices read the same q, k, T, R: the launch maps
// them onto one XCD (consecutive workgroup ids alternate XCDs) so those
// reads hit that XCD's L2.
#include <atomic>

#include "la_common.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kXcds = 8;

template <typename T, int DK_, int C_, int W_>
struct DCfg {
  using type = T;
  using vec = typename Vec16<T>::type;
  static constexpr int DK = DK_, C = C_, W = W_;
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int NRB = C / 16;    // 16-row blocks of a chunk
  static constexpr int NCT = W / 16;    // 16-column tiles of a value slice
  static constexpr int NW = NRB * NCT;  // waves of the sequential pass
  static constexpr int NT = NW * kWave;
  static constexpr int NFT = DK / 16;   // 16-row tiles of the state
  static constexpr int FPW = NFT / NRB; // state row tiles per wave
  static constexpr int KSD = DK / 32;   // k-steps over features
  static constexpr int QLD = DK + VEC;  // row stride: Qs, Ks, St
  static constexpr int CLD = C + VEC;   // row stride: Kt, Ts, Rs, Yt, Ut
  static constexpr int VLD = W + VEC;   // row stride: Vs, Os
  static constexpr int QCB = DK / VEC;  // 16-byte blocks per q/k row
  static constexpr int RQ = C * DK / (VEC * NT);  // q/k rows per thread
  static constexpr int TCB = C / VEC;   // 16-byte blocks per T/R row
  static constexpr int RT = C * C / (VEC * NT);   // T/R rows per thread
  static constexpr int WCB = W / VEC;   // 16-byte blocks per value-slice row
  static constexpr int NVB = C * WCB;   // 16-byte blocks of a value slice
  static_assert(NRB >= 1 && NCT >= 1 && FPW >= 1 && NFT % NRB == 0, "tiling");
  static_assert(RQ >= 1 && RQ * VEC * NT == C * DK, "q/k rows per thread");
  static_assert(RT >= 1 && RT * VEC * NT == C * C, "T/R rows per thread");
  static_assert(NVB <= NT, "one value block per thread at most");
};

// ---------------------------------------------------------------------------
// prep_kernel
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 256;

template <class CF>
struct alignas(16) SmemPrep {
  using T = typename CF::type;
  static constexpr int FLD = CF::C + 4;  // fp32 row stride (16-byte rows)
  T Ks[CF::C * CF::QLD];
  T Qs[CF::C * CF::QLD];
  float Nm[CF::C * FLD];  // diag(g) strict_lower(K K^T); later T^T
  float Pm[CF::C * FLD];  // lower_incl(Q K^T)
  float Xm[CF::C * FLD];  // (I + N)^(-1); later T
  float Ym[CF::C * 16];   // partial products of the block solve
  float gs[CF::C];
};

template <class CF, bool VK>
__global__ void __launch_bounds__(kPrepThreads) prep_kernel(PrefillParams p) {
  using T = typename CF::type;
  constexpr int C = CF::C, VEC = CF::VEC, FLD = SmemPrep<CF>::FLD;
  constexpr int NRB = CF::NRB;
  __shared__ SmemPrep<CF> sm;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int N = p.N, d = p.d;
  const int c0 = chunk * C;
  const int Lc = min(C, N - c0);

  // ---- q, k rows and gates into LDS (zero past the sequence) ----
  {
    const size_t qk = (size_t)N * d;
    const __amdgpu_buffer_rsrc_t rq =
        buf_rsrc(reinterpret_cast<const T *>(p.q) + (size_t)bh * qk, (uint32_t)(qk * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rk =
        buf_rsrc(reinterpret_cast<const T *>(p.k) + (size_t)bh * qk, (uint32_t)(qk * sizeof(T)));
    constexpr int NB = C * CF::QCB;  // 16-byte blocks per tile
    for (int b = tid; b < NB; b += kPrepThreads) {
      const int row = b / CF::QCB, col0 = (b % CF::QCB) * VEC;
      const bool ok = row < Lc;
      typename CF::vec xq, xk;
      if constexpr (VK) {
        const uint32_t off = (ok && col0 < d)
                                 ? (uint32_t)(((size_t)(c0 + row) * d + col0) * sizeof(T))
                                 : kOOB;
        xq = buf_load16<T>(rq, off);
        xk = buf_load16<T>(rk, off);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t off = (ok && col0 + e < d)
                                   ? (uint32_t)(((size_t)(c0 + row) * d + col0 + e) * sizeof(T))
                                   : kOOB;
          xq[e] = buf_load1(rq, off, (T *)nullptr);
          xk[e] = buf_load1(rk, off, (T *)nullptr);
        }
      }
      *reinterpret_cast<typename CF::vec *>(sm.Qs + row * CF::QLD + col0) = xq;
      *reinterpret_cast<typename CF::vec *>(sm.Ks + row * CF::QLD + col0) = xk;
    }
    if (tid < C) sm.gs[tid] = tid < Lc ? p.g[(size_t)bh * N + c0 + tid] : 0.f;
  }
  __syncthreads();

  // ---- K K^T and Q K^T, lower tiles, on the matrix cores ----
  // Wave w handles row block w (and w + 4 when the chunk has more blocks).
  for (int rb = wv; rb < NRB; rb += kPrepThreads / kWave) {
    Frag<T> kr[CF::KSD], qr[CF::KSD];
#pragma unroll
    for (int ks = 0; ks < CF::KSD; ++ks) {
      lds_frag(kr[ks], sm.Ks + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
      lds_frag(qr[ks], sm.Qs + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
    }
    for (int tj = 0; tj < NRB; ++tj) {
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
      if (tj <= rb) {
#pragma unroll
        for (int ks = 0; ks < CF::KSD; ++ks) {
          Frag<T> kc;
          lds_frag(kc, sm.Ks + (16 * tj + li) * CF::QLD + 32 * ks + 8 * lg);
          // output tile rows = keys j of block tj, column = row i of block rb
          mma(kk, kc, kr[ks]);
          mma(qk, kc, qr[ks]);
        }
      }
      // lane holds (i = 16 rb + li, j = 16 tj + 4 lg + r)
      const int i = 16 * rb + li;
      const float gi = sm.gs[i];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * tj + 4 * lg + r;
        sm.Nm[i * FLD + j] = j < i ? gi * kk[r] : 0.f;
        sm.Pm[i * FLD + j] = j <= i ? qk[r] : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- inverse of the unit lower triangular I + N ----
  // Diagonal 16x16 blocks: lane 16 b + c solves column c of block b by
  // forward substitution (x_c = 1; x_i = -sum_{m<i} N_im x_m for i > c).
  if (wv == 0 && lane < 16 * NRB) {
    const int b = lane >> 4, c = lane & 15;
    const float *Nb = sm.Nm + (16 * b) * FLD + 16 * b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s = fmaf(Nb[i * FLD + m], x[m], s);
      x[i] = i == c ? 1.f : (i < c ? 0.f : -s);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.Xm[(16 * b + i) * FLD + 16 * b + c] = x[i];
  }
  // zero the strictly upper blocks
  for (int e = tid; e < C * C; e += kPrepThreads) {
    const int i = e / C, j = e % C;
    if ((j >> 4) > (i >> 4)) sm.Xm[i * FLD + j] = 0.f;
  }
  __syncthreads();
  // Blocks below the diagonal, one block row at a time:
  //   Y_ij = sum_{j<=m<i} N_im X_mj,   X_ij = -X_ii Y_ij.
  {
    const int r = tid >> 4, c = tid & 15;  // one element of a 16x16 block
    for (int bi = 1; bi < NRB; ++bi) {
      for (int bj = 0; bj < bi; ++bj) {
        float s = 0.f;
        for (int bm = bj; bm < bi; ++bm) {
          const float *Nr = sm.Nm + (16 * bi + r) * FLD + 16 * bm;
          const float *Xc = sm.Xm + (16 * bm) * FLD + 16 * bj + c;
#pragma unroll
          for (int m = 0; m < 16; ++m) s = fmaf(Nr[m], Xc[m * FLD], s);
        }
        sm.Ym[(bj * 16 + r) * 16 + c] = s;
      }
      __syncthreads();
      for (int bj = 0; bj < bi; ++bj) {
        const float *Xr = sm.Xm + (16 * bi + r) * FLD + 16 * bi;
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) s = fmaf(Xr[m], sm.Ym[(bj * 16 + m) * 16 + c], s);
        sm.Xm[(16 * bi + r) * FLD + 16 * bj + c] = -s;
      }
      __syncthreads();
    }
  }

  // ---- T = X diag(g): kept row-major in Xm and transposed (fp32) in Nm ----
  for (int e = tid; e < C * C; e += kPrepThreads) {
    const int i = e / C, j = e % C;
    const float t = sm.Xm[i * FLD + j] * sm.gs[j];
    sm.Xm[i * FLD + j] = t;
    sm.Nm[j * FLD + i] = t;
  }
  __syncthreads();

  // ---- R = P T (lower tiles) on the fp32 matrix cores; stores ----
  const size_t slot = ((size_t)bh * gridDim.x + chunk) * C * C;
  T *Tw = reinterpret_cast<T *>(p.ws) + 2 * slot;
  T *Rw = Tw + (size_t)C * C;
  for (int t = wv; t < NRB * NRB; t += kPrepThreads / kWave) {
    const int ti = t / NRB, tj = t % NRB;  // output tile (rows ti, columns tj)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti) {
      // m runs over [16 tj, 16 ti + 16); P and T are zero outside their
      // triangles, so whole 32-wide steps covering that range are exact.
      for (int ks = (16 * tj) / 32; ks <= (16 * ti + 15) / 32; ++ks) {
        Frag<float> a, b;
        lds_frag(a, sm.Pm + (16 * ti + li) * FLD + 32 * ks + 8 * lg);
        lds_frag(b, sm.Nm + (16 * tj + li) * FLD + 32 * ks + 8 * lg);
        mma(acc, a, b);
      }
    }
    // lane holds R[16 ti + 4 lg + r][16 tj + li]
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Rw[(size_t)(16 * ti + 4 * lg + r) * C + 16 * tj + li] = from_f32<T>(acc[r]);
  }
  for (int e = tid; e < C * C; e += kPrepThreads)
    Tw[e] = from_f32<T>(sm.Xm[(e / C) * FLD + e % C]);
}

// ---------------------------------------------------------------------------
// seq_kernel
// ---------------------------------------------------------------------------
template <class CF>
struct alignas(16) SmemSeq {
  using T = typename CF::type;
  T Qs[CF::C * CF::QLD];
  T Ks[CF::C * CF::QLD];
  T Kt[2][CF::DK * CF::CLD];  // K^T, double-buffered
  T Ts[CF::C * CF::CLD];
  T Rs[CF::C * CF::CLD];
  T Vs[CF::C * CF::VLD];
  T Yt[CF::W * CF::CLD];      // (V - K S)^T
  T Ut[CF::W * CF::CLD];      // U^T
  T St[CF::W * CF::QLD];      // S^T, T-precision copy of the fp32 state
  T Os[CF::C * CF::VLD];
};

template <class CF>
struct SeqRegs {
  typename CF::vec q[CF::RQ], k[CF::RQ], t[CF::RT], r[CF::RT], v;
};

template <class CF, bool VK>
__device__ __forceinline__ void seq_prefetch(SeqRegs<CF> &R, const PrefillParams &p,
                                             const __amdgpu_buffer_rsrc_t (&rs)[5],
                                             int c0, int chunk, int n0) {
  using T = typename CF::type;
  constexpr int VEC = CF::VEC;
  const int tid = threadIdx.x;
  const int Lc = min(CF::C, p.N - c0);
  {
    const int cb = tid % CF::QCB, rg = tid / CF::QCB;
#pragma unroll
    for (int r = 0; r < CF::RQ; ++r) {
      const int row = rg * CF::RQ + r;
      R.q[r] = [&] {
        if constexpr (VK) {
          const bool ok = row < Lc && cb * VEC < p.d;
          return buf_load16<T>(rs[0], ok ? (uint32_t)(((size_t)(c0 + row) * p.d + cb * VEC) * sizeof(T)) : kOOB);
        } else {
          typename CF::vec x;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const bool ok = row < Lc && cb * VEC + e < p.d;
            x[e] = buf_load1(rs[0], ok ? (uint32_t)(((size_t)(c0 + row) * p.d + cb * VEC + e) * sizeof(T)) : kOOB, (T *)nullptr);
          }
          return x;
        }
      }();
      R.k[r] = [&] {
        if constexpr (VK) {
          const bool ok = row < Lc && cb * VEC < p.d;
          return buf_load16<T>(rs[1], ok ? (uint32_t)(((size_t)(c0 + row) * p.d + cb * VEC) * sizeof(T)) : kOOB);
        } else {
          typename CF::vec x;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const bool ok = row < Lc && cb * VEC + e < p.d;
            x[e] = buf_load1(rs[1], ok ? (uint32_t)(((size_t)(c0 + row) * p.d + cb * VEC + e) * sizeof(T)) : kOOB, (T *)nullptr);
          }
          return x;
        }
      }();
    }
  }
  {
    // T and R of this chunk: contiguous C x C tiles
    const uint32_t base = (uint32_t)chunk * (uint32_t)(2 * CF::C * CF::C) * sizeof(T);
#pragma unroll
    for (int r = 0; r < CF::RT; ++r) {
      const uint32_t e = (uint32_t)(tid + r * CF::NT) * VEC;  // element in the tile
      R.t[r] = buf_load16<T>(rs[2], base + e * sizeof(T));
      R.r[r] = buf_load16<T>(rs[2], base + (e + CF::C * CF::C) * sizeof(T));
    }
  }
  {
    const int row = tid / CF::WCB, cb = tid % CF::WCB;
    const int col0 = n0 + cb * VEC;
    const bool in = tid < CF::NVB && row < Lc;
    if constexpr (VK) {
      const bool ok = in && col0 < p.dv;
      R.v = buf_load16<T>(rs[3], ok ? (uint32_t)(((size_t)(c0 + row) * p.dv + col0) * sizeof(T)) : kOOB);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const bool ok = in && col0 + e < p.dv;
        R.v[e] = buf_load1(rs[3], ok ? (uint32_t)(((size_t)(c0 + row) * p.dv + col0 + e) * sizeof(T)) : kOOB, (T *)nullptr);
      }
    }
  }
}

// Registers -> LDS tiles for one chunk (K^T into buffer `kb`).
template <class CF>
__device__ __forceinline__ void seq_commit(const SeqRegs<CF> &R, SmemSeq<CF> &sm, int kb) {
  using T = typename CF::type;
  using V = typename CF::vec;
  constexpr int VEC = CF::VEC;
  const int tid = threadIdx.x;
  {
    const int cb = tid % CF::QCB, rg = tid / CF::QCB;
    const int col0 = cb * VEC;
#pragma unroll
    for (int r = 0; r < CF::RQ; ++r) {
      const int row = rg * CF::RQ + r;
      *reinterpret_cast<V *>(sm.Qs + row * CF::QLD + col0) = R.q[r];
      *reinterpret_cast<V *>(sm.Ks + row * CF::QLD + col0) = R.k[r];
    }
    // K^T: this thread's RQ consecutive rows, column by column
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float x[CF::RQ];
#pragma unroll
      for (int r = 0; r < CF::RQ; ++r) x[r] = to_f32(R.k[r][e]);
      lds_store_n<T, CF::RQ>(sm.Kt[kb] + (col0 + e) * CF::CLD + rg * CF::RQ, x);
    }
  }
#pragma unroll
  for (int r = 0; r < CF::RT; ++r) {
    const int e = (tid + r * CF::NT) * VEC;
    const int row = e / CF::C, col = e % CF::C;
    *reinterpret_cast<V *>(sm.Ts + row * CF::CLD + col) = R.t[r];
    *reinterpret_cast<V *>(sm.Rs + row * CF::CLD + col) = R.r[r];
  }
  if (tid < CF::NVB) {
    const int row = tid / CF::WCB, cb = tid % CF::WCB;
    *reinterpret_cast<V *>(sm.Vs + row * CF::VLD + cb * VEC) = R.v;
  }
}

template <class CF, bool VK>
__global__ void __launch_bounds__(CF::NT) seq_kernel(PrefillParams p, int nslices,
                                                     int xcd_map) {
  using T = typename CF::type;
  constexpr int C = CF::C, W = CF::W;
  __shared__ SmemSeq<CF> sm;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int rb = wv % CF::NRB, ct = wv / CF::NRB;

  // workgroup -> (head, slice); with xcd_map the slices of one head share
  // an XCD (workgroup b runs on XCD b % 8)
  const int b = blockIdx.x;
  int bh, slice;
  if (xcd_map) {
    const int j = b / kXcds;
    slice = j % nslices;
    bh = (j / nslices) * kXcds + b % kXcds;
  } else {
    bh = b / nslices;
    slice = b % nslices;
  }
  const int n0 = slice * W;
  const int N = p.N, d = p.d, dv = p.dv;
  const int nch = (N + C - 1) / C;

  __amdgpu_buffer_rsrc_t rs[5];
  {
    const size_t qk = (size_t)N * d, vo = (size_t)N * dv;
    rs[0] = buf_rsrc(reinterpret_cast<const T *>(p.q) + (size_t)bh * qk, (uint32_t)(qk * sizeof(T)));
    rs[1] = buf_rsrc(reinterpret_cast<const T *>(p.k) + (size_t)bh * qk, (uint32_t)(qk * sizeof(T)));
    const size_t tr = (size_t)nch * 2 * C * C;
    rs[2] = buf_rsrc(reinterpret_cast<const T *>(p.ws) + (size_t)bh * tr, (uint32_t)(tr * sizeof(T)));
    rs[3] = buf_rsrc(reinterpret_cast<const T *>(p.v) + (size_t)bh * vo, (uint32_t)(vo * sizeof(T)));
    rs[4] = buf_rsrc(reinterpret_cast<const T *>(p.o) + (size_t)bh * vo, (uint32_t)(vo * sizeof(T)));
  }

  // fp32 state slice: wave holds row tiles tf = rb * FPW + a, column tile ct
  f32x4 Sacc[CF::FPW];
  const float *S0 = p.S_in ? p.S_in + (size_t)bh * d * dv : nullptr;
  const int ncol = n0 + 16 * ct + li;
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a) {
    const int tf = rb * CF::FPW + a;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = 16 * tf + 4 * lg + r;
      Sacc[a][r] = (S0 && f < d && ncol < dv) ? S0[(size_t)f * dv + ncol] : 0.f;
    }
  }
  SeqRegs<CF> R;
  seq_prefetch<CF, VK>(R, p, rs, 0, 0, n0);
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a) {
    const int tf = rb * CF::FPW + a;
    lds_store4(sm.St + (16 * ct + li) * CF::QLD + 16 * tf + 4 * lg, Sacc[a][0], Sacc[a][1],
               Sacc[a][2], Sacc[a][3]);
  }
  seq_commit<CF>(R, sm, 0);
  if (nch > 1) seq_prefetch<CF, VK>(R, p, rs, C, 1, n0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int c0 = c * C;
    const int Lc = min(C, N - c0);
    const int kb = c & 1;
    // ---- X = K S-, Z = Q S- (tile rb, ct) ----
    f32x4 X = {0.f, 0.f, 0.f, 0.f}, Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < CF::KSD; ++ks) {
      Frag<T> kf, qf, sf;
      lds_frag(sf, sm.St + (16 * ct + li) * CF::QLD + 32 * ks + 8 * lg);
      lds_frag(kf, sm.Ks + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
      lds_frag(qf, sm.Qs + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
      mma(X, kf, sf);
      mma(Z, qf, sf);
    }
    // ---- Y = V - X, stored transposed (tokens contiguous) ----
    // lane holds rows 16 rb + 4 lg + r, column 16 ct + li
    {
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        y[r] = to_f32(sm.Vs[(16 * rb + 4 * lg + r) * CF::VLD + 16 * ct + li]) - X[r];
      lds_store4(sm.Yt + (16 * ct + li) * CF::CLD + 16 * rb + 4 * lg, y[0], y[1], y[2], y[3]);
    }
    __syncthreads();
    // ---- U = T Y, O = Z + R Y (T and R are lower triangular) ----
    {
      f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        if (32 * ks <= 16 * rb + 15) {
          Frag<T> tf, rf, yf;
          lds_frag(yf, sm.Yt + (16 * ct + li) * CF::CLD + 32 * ks + 8 * lg);
          lds_frag(tf, sm.Ts + (16 * rb + li) * CF::CLD + 32 * ks + 8 * lg);
          lds_frag(rf, sm.Rs + (16 * rb + li) * CF::CLD + 32 * ks + 8 * lg);
          mma(U, tf, yf);
          mma(Z, rf, yf);
        }
      }
      lds_store4(sm.Ut + (16 * ct + li) * CF::CLD + 16 * rb + 4 * lg, U[0], U[1], U[2], U[3]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sm.Os[(16 * rb + 4 * lg + r) * CF::VLD + 16 * ct + li] = from_f32<T>(Z[r]);
    }
    __syncthreads();
    // ---- next chunk's tiles (K^T into the other buffer), next loads ----
    if (c + 1 < nch) {
      seq_commit<CF>(R, sm, kb ^ 1);
      if (c + 2 < nch) seq_prefetch<CF, VK>(R, p, rs, c0 + 2 * C, c + 2, n0);
    }
    // ---- output rows of the slice ----
    if (tid < CF::NVB) {
      const int row = tid / CF::WCB, cb = tid % CF::WCB;
      const int col0 = n0 + cb * CF::VEC;
      const typename CF::vec val =
          *reinterpret_cast<const typename CF::vec *>(sm.Os + row * CF::VLD + cb * CF::VEC);
      const size_t el = (size_t)(c0 + row) * dv + col0;
      if constexpr (VK) {
        const bool ok = row < Lc && col0 < dv;
        buf_store16_nt<T>(rs[4], ok ? (uint32_t)(el * sizeof(T)) : kOOB, val);
      } else {
#pragma unroll
        for (int e = 0; e < CF::VEC; ++e) {
          const bool ok = row < Lc && col0 + e < dv;
          buf_store1(rs[4], ok ? (uint32_t)((el + e) * sizeof(T)) : kOOB, val[e]);
        }
      }
    }
    // ---- S+ = S- + K^T U, and its T-precision copy ----
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a) {
      const int tf = rb * CF::FPW + a;
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        Frag<T> kf, uf;
        lds_frag(kf, sm.Kt[kb] + (16 * tf + li) * CF::CLD + 32 * ks + 8 * lg);
        lds_frag(uf, sm.Ut + (16 * ct + li) * CF::CLD + 32 * ks + 8 * lg);
        mma(Sacc[a], kf, uf);
      }
      lds_store4(sm.St + (16 * ct + li) * CF::QLD + 16 * tf + 4 * lg, Sacc[a][0],
                 Sacc[a][1], Sacc[a][2], Sacc[a][3]);
    }
    __syncthreads();
  }

  if (p.S_out) {
    float *So = p.S_out + (size_t)bh * d * dv;
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a) {
      const int tf = rb * CF::FPW + a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * tf + 4 * lg + r;
        if (f < d && ncol < dv) So[(size_t)f * dv + ncol] = Sacc[a][r];
      }
    }
  }
}

template <class CF, bool VK>
hipError_t run_vk(const PrefillParams &p, hipStream_t s) {
  static_assert(sizeof(SmemPrep<CF>) <= 160 * 1024, "LDS budget (prep)");
  static_assert(sizeof(SmemSeq<CF>) <= 160 * 1024, "LDS budget (seq)");
  const int nch = (p.N + CF::C - 1) / CF::C;
  prof_begin(s);
  hipLaunchKernelGGL((prep_kernel<CF, VK>), dim3(nch, p.BH), dim3(kPrepThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_end("delta_prep", s);
  const int nsl = (p.dv + CF::W - 1) / CF::W;
  const int xcd_map = (p.BH % kXcds) == 0;
  prof_begin(s);
  hipLaunchKernelGGL((seq_kernel<CF, VK>), dim3(p.BH * nsl), dim3(CF::NT), 0, s, p, nsl,
                     xcd_map);
  e = hipGetLastError();
  if (e == hipSuccess) prof_end("delta_seq", s);
  return e;
}

template <class CF>
hipError_t run(const PrefillParams &p, hipStream_t s) {
  return p.vec_ok ? run_vk<CF, true>(p, s) : run_vk<CF, false>(p, s);
}

// bf16: 64-token chunks, 16-column slices (4 waves); fp32: 32-token chunks,
// 32-column slices (4 waves), so that the fp32 tiles fit in LDS.
using DB64 = DCfg<bf16, 64, 64, 16>;
using DB128 = DCfg<bf16, 128, 64, 16>;
using DF64 = DCfg<float, 64, 32, 32>;
using DF128 = DCfg<float, 128, 32, 32>;

}  // namespace

int delta_chunk_len(bool bf16_io) { return bf16_io ? DB64::C : DF64::C; }

size_t delta_workspace_bytes(int BH, int N, bool bf16_io) {
  const int C = delta_chunk_len(bf16_io);
  const size_t nch = ((size_t)N + C - 1) / C;
  return (size_t)BH * nch * 2 * C * C * (bf16_io ? 2 : 4);
}

hipError_t launch_delta_prefill(const PrefillParams &p, bool bf16_io, hipStream_t s) {
  if (bf16_io) return p.d <= 64 ? run<DB64>(p, s) : run<DB128>(p, s);
  return p.d <= 64 ? run<DF64>(p, s) : run<DF128>(p, s);
}

}  // namespace la
