// Backward of the LINEAR rule's chunked prefill (training): dq, dk, dv and
// the gradient of the initial state, from the forward's inputs, its output
// o, its per-token denominators and the gradient of the loss with respect
// to o (and, optionally, to the final state).
//
// The pages motivate parallel training ("What Is Linear Attention?" 8,
// "Efficient attention variants" 8 and 10) but give no gradient formulas;
// these are derived from the recurrence.  The normaliser rides along as an
// extra value column, as in the forward: with v'_t = [v_t | 1] and the
// state S'_t = [S_t | z_t],
//     num'_t = S'_t^T phi(q_t),  o_t = num_t / den_t,  den_t = phi(q_t).z_t + eps,
// so dL/dnum'_t = dn_t = [g_t / den_t | -(g_t . o_t) / den_t] (g_t = dL/do_t),
// and the rest is the gradient of unnormalised linear attention with values
// v' and output gradients dn.  For a chunk of L tokens (local indices
// t, j), entering state S'_in, decay D_tj = gamma^(t-j) for j <= t else 0,
// A = phi(Q) phi(K)^T . D and dA = (dN V'^T) . D:
//     dphi(q_t) = gamma^(t+1) S'_in dn_t + sum_j dA_tj phi(k_j)
//     dphi(k_j) = sum_t dA_tj phi(q_t) + gamma^(L-1-j) Sh v'_j
//     dv'_j     = sum_t A_tj dn_t      + gamma^(L-1-j) Sh^T phi(k_j)
// where Sh is the adjoint of the state after the chunk (gradient from all
// later tokens and the final-state gradient), carried backward as
//     Sh <- gamma^L Sh + sum_t gamma^(t+1) phi(q_t) dn_t^T,
// and the forward state is carried as in the forward pass.  Every decay
// factor is at most 1.  dq = dphi(q) phi'(q), dk = dphi(k) phi'(k), with
// phi'(x) = min(phi(x), 1) for elu+1.
//
// Kernels (per (segment, head); segments as in the forward):
//   the forward's summary and scan kernels   forward state entering each segment
//                                            (or the forward's own, left in its workspace)
//   bwd_dq_kernel                            dq, chunks left to right, forward state; also
//                                            each segment's own adjoint, from zero at its
//                                            end (the terms are summed in any order:
//                                            sum_t gamma^(t - t_begin + 1) phi(q_t) dn_t^T)
//   bwd_rscan_kernel                         adjoint entering each segment from the right
//   bwd_dkv_kernel                           dk, dv, chunks right to left, adjoint state;
//                                            segment 0 writes the initial-state gradient
// Every product runs on the matrix cores from LDS tiles (bf16 operands,
// fp32 accumulation; fp32 inputs use fp32 operands); the carried states
// stay in fp32 accumulators.
#include "la_common.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kMaxSegB = 32;  // the forward's most segments per sequence
// Gradient rows leave through an LDS staging tile as whole 16-byte row
// blocks (written out after the chunk's last barrier, so no barrier of their
// own), not as 2-byte stores straight from the accumulators.
constexpr bool kStageOut = true;

template <typename T, int DK_, int DV_, int C_, int NW_, int WPE_DQ_>
struct BCfg {
  using type = T;
  using vec = typename Vec16<T>::type;
  static constexpr int DK = DK_, DV = DV_, C = C_, NW = NW_;
  static constexpr int NT = NW * kWave;
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int PAD = sizeof(T) == 2 ? 16 : 4;
  static constexpr int DVK = DV + 32;    // value side as a contraction: values,
                                         // the normaliser column, zeros
  static constexpr int NVP = DV / 16 + 1;  // value-side tiles incl. the normaliser tile
  static constexpr int LDK = DK + PAD;     // row strides of the LDS tiles
  static constexpr int LDV = DVK + PAD;
  static constexpr int LDO = DV + PAD;
  // C x C tiles and the gradient staging tiles: rows of 80 or 144 bytes
  // (bf16), so the 16-byte fragment reads of 16 consecutive rows and the
  // staging writes of rows 4 apart fall in distinct banks
  static constexpr int PADS = sizeof(T) == 2 ? 8 : 4;
  static constexpr int LDC = C + PADS;
  static constexpr int LDKS = DK + PADS, LDOS = DV + PADS;
  static constexpr int NTB = C / 16;   // token blocks
  static constexpr int NFB = DK / 16;  // feature blocks
  static constexpr int NST = NFB * NVP;               // state tiles
  static constexpr int SPW = (NST + NW - 1) / NW;     // state tiles per wave
  static constexpr int QCB = DK / VEC, VCB = DV / VEC;  // 16-byte blocks per row
  static constexpr int XCB = 32 / VEC;                 // blocks of the extra columns
  // resident waves per SIMD the dq kernel's registers must allow (what its
  // LDS admits)
  static constexpr int WPE_DQ = WPE_DQ_;
  // ... and the dk/dv kernel's (four-wave bf16 workgroups: its LDS admits
  // three per CU)
  static constexpr int WPE_DKV = (NW == 4 && sizeof(T) == 2) ? 3 : 1;
  static_assert(C % 32 == 0 && DK % 32 == 0 && DV % 16 == 0, "tile sizes");
  // row loops run whole waves (the dn row reduction shuffles within a wave)
  static_assert((C * QCB) % kWave == 0 && (C * VCB) % kWave == 0, "whole-wave row loops");
  static_assert(VCB >= XCB && VCB <= kWave, "row groups within a wave");
};

template <class BC>
struct alignas(16) SmemDq {
  using T = typename BC::type;
  T Fq[BC::C * BC::LDK];  // phi(q)
  T Fk[BC::C * BC::LDK];  // phi(k)
  T KW[BC::C * BC::LDK];  // gamma^(L-1-j) phi(k_j)
  T Vp[BC::C * BC::LDV];  // [v | 1 | 0]
  T dN[BC::C * BC::LDV];  // [g / den | -(g.o) / den | 0]
  T dA[BC::C * BC::LDC];  // (dN V'^T) . D
  T St[BC::DK * BC::LDV]; // the forward state [S | z | 0], rows = features
  float pw[BC::C + 4];    // gamma^m
  float kw[BC::C];        // gamma^(L-1-j), 0 past the chunk
  T Os[kStageOut ? BC::C * BC::LDKS : 1];  // dq staging
};

// The weighted queries gamma^(t+1) phi(q_t) of the adjoint's update are
// formed from phi(q) in registers; without a decay (DEC false) there is no
// power table.
template <class BC, bool DEC>
struct alignas(16) SmemDkv {
  using T = typename BC::type;
  T Fq[BC::C * BC::LDK];
  T Fk[BC::C * BC::LDK];
  T Vp[BC::C * BC::LDV];
  T dN[BC::C * BC::LDV];
  T Ad[BC::C * BC::LDC];  // A . D
  T dA[BC::C * BC::LDC];  // dA . D
  T Sh[BC::DK * BC::LDV]; // the adjoint [Sh | zh | 0], rows = features
  float pw[DEC ? BC::C + 4 : 4];
  T Ok[kStageOut ? BC::C * BC::LDKS : 1];  // dk staging
  T Ov[kStageOut ? BC::C * BC::LDOS : 1];  // dv staging
};

// ---- operands -------------------------------------------------------------
// frag_rk: M[i][k] (k contiguous); frag_kr: M[k][i] (transposed read).  Lane
// (li, lg) gets index i0 + li and k slots k0 + 8 lg .. + 7 either way.
template <typename T>
__device__ __forceinline__ void frag_rk(Frag<T> &f, const T *M, int ld, int i0, int k0, int li,
                                        int lg) {
  lds_frag(f, M + (i0 + li) * ld + k0 + 8 * lg);
}
template <typename T>
__device__ __forceinline__ void frag_kr(Frag<T> &f, const T *M, int ld, int i0, int k0, int li,
                                        int lg) {
  lds_frag_tr(f, M, ld, k0 + 8 * lg, k0 + 8 * lg + 4, i0, li);
}

// One 16-byte block of row `tok` of a [N, ncols] tensor, zero outside.
template <typename T, bool VK>
__device__ __forceinline__ typename Vec16<T>::type load_vec(__amdgpu_buffer_rsrc_t r, int tok,
                                                            int col0, int ncols, bool row_ok) {
  constexpr int VEC = 16 / (int)sizeof(T);
  if constexpr (VK) {
    const bool ok = row_ok && col0 < ncols;
    return buf_load16<T>(r, ok ? (uint32_t)(((size_t)tok * ncols + col0) * sizeof(T)) : kOOB);
  } else {
    typename Vec16<T>::type x;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const bool ok = row_ok && col0 + e < ncols;
      x[e] = buf_load1(r, ok ? (uint32_t)(((size_t)tok * ncols + col0 + e) * sizeof(T)) : kOOB,
                       (T *)nullptr);
    }
    return x;
  }
}

template <typename T, bool VK>
__device__ __forceinline__ void store_vec(__amdgpu_buffer_rsrc_t r, int tok, int col0, int ncols,
                                          bool row_ok, typename Vec16<T>::type x) {
  constexpr int VEC = 16 / (int)sizeof(T);
  if constexpr (VK) {
    const bool ok = row_ok && col0 < ncols;
    buf_store16_nt<T>(r, ok ? (uint32_t)(((size_t)tok * ncols + col0) * sizeof(T)) : kOOB, x);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const bool ok = row_ok && col0 + e < ncols;
      buf_store1(r, ok ? (uint32_t)(((size_t)tok * ncols + col0 + e) * sizeof(T)) : kOOB, x[e]);
    }
  }
}

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void *base, int bh, int N,
                                                            int ncols) {
  const size_t n = (size_t)N * ncols;
  return buf_rsrc(reinterpret_cast<const T *>(base) + (size_t)bh * n, (uint32_t)(n * sizeof(T)));
}

__device__ __forceinline__ float feat(float x, int fmap) {
  return fmap ? phi_elu1(x) : x;
}

// ---- one chunk: loads into registers (issued a chunk ahead), then LDS -------
// Thread i handles blocks i, i + NT, ... of the chunk's rows (QCB or VCB
// 16-byte blocks per row); NQ / NV such blocks at most.
template <class BC>
struct BRegs {
  static constexpr int NQ = (BC::C * BC::QCB + BC::NT - 1) / BC::NT;
  static constexpr int NV = (BC::C * BC::VCB + BC::NT - 1) / BC::NT;
  typename BC::vec q[NQ], k[NQ], v[NV], o[NV], g[NV];
  float den[NV];
};

struct HeadRsrc {
  __amdgpu_buffer_rsrc_t q, k, v, o, g, den;
};

// LQ, LK, LV: load q, k, v; LOG: load o, dL/do and the denominators.
template <class BC, bool VK, bool LQ, bool LK, bool LV, bool LOG>
__device__ __forceinline__ void load_chunk(BRegs<BC> &R, const HeadRsrc &hr, int c0, int Lc,
                                           int d, int dv) {
  using T = typename BC::type;
#pragma unroll
  for (int n = 0; n < BRegs<BC>::NQ; ++n) {
    const int i = threadIdx.x + n * BC::NT;
    const int row = i / BC::QCB, col0 = (i % BC::QCB) * BC::VEC;
    const bool ok = i < BC::C * BC::QCB && row < Lc;
    if constexpr (LQ) R.q[n] = load_vec<T, VK>(hr.q, c0 + row, col0, d, ok);
    if constexpr (LK) R.k[n] = load_vec<T, VK>(hr.k, c0 + row, col0, d, ok);
  }
#pragma unroll
  for (int n = 0; n < BRegs<BC>::NV; ++n) {
    const int i = threadIdx.x + n * BC::NT;
    const int row = i / BC::VCB, col0 = (i % BC::VCB) * BC::VEC;
    const bool ok = i < BC::C * BC::VCB && row < Lc;
    if constexpr (LV) R.v[n] = load_vec<T, VK>(hr.v, c0 + row, col0, dv, ok);
    if constexpr (LOG) {
      R.o[n] = load_vec<T, VK>(hr.o, c0 + row, col0, dv, ok);
      R.g[n] = load_vec<T, VK>(hr.g, c0 + row, col0, dv, ok);
      R.den[n] = buf_load1(hr.den, ok ? (uint32_t)((c0 + row) * 4) : kOOB, (float *)nullptr);
    }
  }
}

// phi(q) or phi(k) rows into F (if set) and weighted rows wt[row] phi(.)
// into W (if set); rows past the chunk and feature columns past d are zero.
template <class BC>
__device__ __forceinline__ void commit_feat(typename BC::type *F, typename BC::type *W,
                                            const float *wt,
                                            const typename BC::vec (&X)[BRegs<BC>::NQ], int Lc,
                                            int d, int fmap) {
  using T = typename BC::type;
  using V = typename BC::vec;
#pragma unroll
  for (int n = 0; n < BRegs<BC>::NQ; ++n) {
    const int i = threadIdx.x + n * BC::NT;
    if (i >= BC::C * BC::QCB) break;
    const int row = i / BC::QCB, col0 = (i % BC::QCB) * BC::VEC;
    V f, w;
    const float s = W ? wt[row] : 0.f;
#pragma unroll
    for (int e = 0; e < BC::VEC; ++e) {
      const float y = (row < Lc && col0 + e < d) ? feat(to_f32(X[n][e]), fmap) : 0.f;
      f[e] = from_f32<T>(y);
      w[e] = from_f32<T>(y * s);
    }
    if (F) *reinterpret_cast<V *>(F + row * BC::LDK + col0) = f;
    if (W) *reinterpret_cast<V *>(W + row * BC::LDK + col0) = w;
  }
}

// [v | 1 | 0] rows (the ones column only for tokens of the chunk).
template <class BC>
__device__ __forceinline__ void commit_values(typename BC::type *Vp, const BRegs<BC> &R,
                                              int Lc) {
  using T = typename BC::type;
  using V = typename BC::vec;
#pragma unroll
  for (int n = 0; n < BRegs<BC>::NV; ++n) {
    const int i = threadIdx.x + n * BC::NT;
    if (i >= BC::C * BC::VCB) break;
    const int row = i / BC::VCB, cb = i % BC::VCB, col0 = cb * BC::VEC;
    *reinterpret_cast<V *>(Vp + row * BC::LDV + col0) = R.v[n];
    if (cb < BC::XCB) {
      V x;
#pragma unroll
      for (int e = 0; e < BC::VEC; ++e) x[e] = from_f32<T>(0.f);
      if (cb == 0 && row < Lc) x[0] = from_f32<T>(1.f);
      *reinterpret_cast<V *>(Vp + row * BC::LDV + BC::DV + col0) = x;
    }
  }
}

// [g / den | -(g . o) / den | 0] rows; zero past the chunk.  The threads of
// one row are VCB consecutive lanes and every iteration runs whole waves, so
// the row's dot product is a shuffle reduction.
template <class BC>
__device__ __forceinline__ void commit_dn(typename BC::type *dN, const BRegs<BC> &R, int Lc) {
  using T = typename BC::type;
  using V = typename BC::vec;
#pragma unroll
  for (int n = 0; n < BRegs<BC>::NV; ++n) {
    const int i = threadIdx.x + n * BC::NT;
    if (i >= BC::C * BC::VCB) break;
    const int row = i / BC::VCB, cb = i % BC::VCB, col0 = cb * BC::VEC;
    const float rd = row < Lc ? 1.f / R.den[n] : 0.f;
    float dot = 0.f;
    V x;
#pragma unroll
    for (int e = 0; e < BC::VEC; ++e) {
      const float ge = to_f32(R.g[n][e]);
      dot = fmaf(ge, to_f32(R.o[n][e]), dot);
      x[e] = from_f32<T>(ge * rd);
    }
    dot = lane_sum<BC::VCB>(dot);
    *reinterpret_cast<V *>(dN + row * BC::LDV + col0) = x;
    if (cb < BC::XCB) {
      V y;
#pragma unroll
      for (int e = 0; e < BC::VEC; ++e) y[e] = from_f32<T>(0.f);
      if (cb == 0) y[0] = from_f32<T>(-dot * rd);
      *reinterpret_cast<V *>(dN + row * BC::LDV + BC::DV + col0) = y;
    }
  }
}

// One accumulator tile (rows 16 t0 + 4 lg + r, column 16 c0 + li) straight
// to global memory: rows past the chunk and columns past ncols are dropped.
// The tile's 16 x 16 elements are written by one wave together, so its
// partial lines merge in the cache before they reach memory.
template <typename T>
__device__ __forceinline__ void store_tile(__amdgpu_buffer_rsrc_t r, const f32x4 &acc, int c0,
                                           int row0, int col, int Lc, int ncols, int lg) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = row0 + 4 * lg + rr;
    const bool ok = row < Lc && col < ncols;
    buf_store1(r, ok ? (uint32_t)(((size_t)(c0 + row) * ncols + col) * sizeof(T)) : kOOB,
               from_f32<T>(acc[rr]));
  }
}

// ---- carried state: fp32 accumulator tiles st = wv + NW i ---------------------
// tile st covers features 16 (st / NVP) .. and value columns 16 (st % NVP) ..;
// the last value tile is the normaliser's ([z | 0 ... 0]).
template <class BC>
__device__ __forceinline__ void state_load(f32x4 (&Sa)[BC::SPW], const float *S, const float *z,
                                           int d, int dv, int wv, int li, int lg) {
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) {
    const int st = wv + BC::NW * i;
    const int fb = st / BC::NVP, vb = st % BC::NVP;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = 16 * fb + 4 * lg + r;
      float x = 0.f;
      if (st < BC::NST && f < d) {
        if (vb < BC::NVP - 1) {
          const int c = 16 * vb + li;
          if (S && c < dv) x = S[(size_t)f * dv + c];
        } else if (li == 0 && z) {
          x = z[f];
        }
      }
      Sa[i][r] = x;
    }
  }
}

// The same tiles from a forward workspace slot, where S is stored
// transposed (element (f, n) at n d + f, then z at d dv + f): a lane's four
// rows of one column are 16 contiguous bytes (vec: d % 4 == 0 and the slot
// is 16-byte aligned; the four rows are then all inside or all past d).
template <class BC>
__device__ __forceinline__ void slot_load(f32x4 (&Sa)[BC::SPW], const float *slot, int d,
                                          int dv, bool vec, int wv, int li, int lg) {
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) {
    const int st = wv + BC::NW * i;
    const int fb = st / BC::NVP, vb = st % BC::NVP;
    const int f = 16 * fb + 4 * lg;
    const int c = 16 * vb + li;
    const bool val = vb < BC::NVP - 1;
    const bool ok = st < BC::NST && (val ? c < dv : li == 0);
    const float *src = slot + (val ? (size_t)c * d : (size_t)d * dv) + f;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (vec) {
      if (ok && f < d) x = *reinterpret_cast<const f32x4 *>(src);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = ok && f + r < d ? src[r] : 0.f;
    }
    Sa[i] = x;
  }
}

// ... and into a slot in that layout (the adjoint's reverse slots use it too).
template <class BC>
__device__ __forceinline__ void slot_store(const f32x4 (&Sa)[BC::SPW], float *slot, int d,
                                           int dv, bool vec, int wv, int li, int lg) {
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) {
    const int st = wv + BC::NW * i;
    const int fb = st / BC::NVP, vb = st % BC::NVP;
    const int f = 16 * fb + 4 * lg;
    const int c = 16 * vb + li;
    const bool val = vb < BC::NVP - 1;
    const bool ok = st < BC::NST && (val ? c < dv : li == 0);
    float *dst = slot + (val ? (size_t)c * d : (size_t)d * dv) + f;
    if (vec) {
      if (ok && f < d) *reinterpret_cast<f32x4 *>(dst) = Sa[i];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (ok && f + r < d) dst[r] = Sa[i][r];
    }
  }
}

template <class BC>
__device__ __forceinline__ void state_store(const f32x4 (&Sa)[BC::SPW], float *S, float *z, int d,
                                            int dv, int wv, int li, int lg) {
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) {
    const int st = wv + BC::NW * i;
    const int fb = st / BC::NVP, vb = st % BC::NVP;
    if (st >= BC::NST) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = 16 * fb + 4 * lg + r;
      if (f >= d) continue;
      if (vb < BC::NVP - 1) {
        const int c = 16 * vb + li;
        if (S && c < dv) S[(size_t)f * dv + c] = Sa[i][r];
      } else if (li == 0 && z) {
        z[f] = Sa[i][r];
      }
    }
  }
}

// bf16 (or fp32) copy of the state into an LDS tile [DK][LDV], columns
// 0 .. DV+15 (the zero columns past them are written once at the start).
template <class BC>
__device__ __forceinline__ void state_copy(typename BC::type *M, const f32x4 (&Sa)[BC::SPW],
                                           int wv, int li, int lg) {
  using T = typename BC::type;
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) {
    const int st = wv + BC::NW * i;
    if (st >= BC::NST) continue;
    const int fb = st / BC::NVP, vb = st % BC::NVP;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      M[(16 * fb + 4 * lg + r) * BC::LDV + 16 * vb + li] = from_f32<T>(Sa[i][r]);
  }
}

template <class BC>
__device__ __forceinline__ void zero_tail_columns(typename BC::type *M) {
  using T = typename BC::type;
  for (int i = threadIdx.x; i < BC::DK * 16; i += BC::NT)
    M[(i / 16) * BC::LDV + BC::DV + 16 + (i % 16)] = from_f32<T>(0.f);
}

// S += sum_t X[t][f] Y[t][c] over the chunk's tokens (both operands
// token-major), after S *= scale.
template <class BC>
__device__ __forceinline__ void state_update(f32x4 (&Sa)[BC::SPW], const typename BC::type *X,
                                             const typename BC::type *Y, float scale, int wv,
                                             int li, int lg, const float *wt = nullptr,
                                             float wsc = 1.f) {
  using T = typename BC::type;
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) {
    const int st = wv + BC::NW * i;
    if (st >= BC::NST) continue;
    const int fb = st / BC::NVP, vb = st % BC::NVP;
#pragma unroll
    for (int r = 0; r < 4; ++r) Sa[i][r] *= scale;
#pragma unroll
    for (int ks = 0; ks < BC::C / 32; ++ks) {
      Frag<T> a, b;
      frag_kr(a, X, BC::LDK, 16 * fb, 32 * ks, li, lg);
      if (wt) {  // per-token weights wsc * wt[t] on X's rows (this lane's k slots)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          a.v[e] = from_f32<T>(to_f32(a.v[e]) * (wt[32 * ks + 8 * lg + e] * wsc));
      }
      frag_kr(b, Y, BC::LDV, 16 * vb, 32 * ks, li, lg);
      mma(Sa[i], a, b);
    }
  }
}

// Masked, decayed C x C product tiles: M[t][j] = D_tj sum_k X[t][k] Y[j][k]
// (K = KS k-steps, both operands k-contiguous); tiles above the diagonal
// are written as zeros.
template <class BC, int KS, int LDX>
__device__ __forceinline__ void tri_tiles(typename BC::type *M, const typename BC::type *X,
                                          const typename BC::type *Y, const float *pw,
                                          bool decay, int wv, int li, int lg) {
  using T = typename BC::type;
  constexpr int NTI = BC::NTB * BC::NTB;
#pragma unroll
  for (int n = 0; n < (NTI + BC::NW - 1) / BC::NW; ++n) {
    const int ti = wv + BC::NW * n;
    if (ti >= NTI) break;
    const int tt = ti / BC::NTB, jt = ti % BC::NTB;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (jt <= tt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<T> a, b;
        frag_rk(a, X, LDX, 16 * tt, 32 * ks, li, lg);
        frag_rk(b, Y, LDX, 16 * jt, 32 * ks, li, lg);
        mma(acc, a, b);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tt + 4 * lg + r, j = 16 * jt + li;
      M[t * BC::LDC + j] = from_f32<T>(j <= t ? (decay ? acc[r] * pw[t - j] : acc[r]) : 0.f);
    }
  }
}

// A tile into an LDS staging tile (row stride ld), or straight to memory.
template <class BC>
__device__ __forceinline__ void out_tile(typename BC::type *M, int ld,
                                         __amdgpu_buffer_rsrc_t r, const f32x4 &acc, int c0,
                                         int row0, int col, int Lc, int ncols, int lg) {
  if constexpr (kStageOut) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      M[(row0 + 4 * lg + rr) * ld + col] = from_f32<typename BC::type>(acc[rr]);
  } else {
    store_tile<typename BC::type>(r, acc, c0, row0, col, Lc, ncols, lg);
  }
}

// Rows of a staging tile to memory (rows past the chunk, columns past ncols
// dropped).
template <class BC, bool VK>
__device__ __forceinline__ void store_rows(__amdgpu_buffer_rsrc_t r, const typename BC::type *M,
                                           int ld, int NCB, int c0, int Lc, int ncols) {
  using V = typename BC::vec;
  for (int i = threadIdx.x; i < BC::C * NCB; i += BC::NT) {
    const int row = i / NCB, col0 = (i % NCB) * BC::VEC;
    store_vec<typename BC::type, VK>(r, c0 + row, col0, ncols, row < Lc,
                                     *reinterpret_cast<const V *>(M + row * ld + col0));
  }
}

// ---- dq: chunks left to right, forward state --------------------------------
// DEC: per-head decay (p.gamma set); without it every decay factor is 1 and
// the weighted copies of phi(q), phi(k) are the unweighted ones
template <class BC, bool VK, bool DEC>
__global__ void __launch_bounds__(BC::NT, BC::WPE_DQ) bwd_dq_kernel(BwdParams p) {
  using T = typename BC::type;
  __shared__ SmemDq<BC> sm;
  const int seg = blockIdx.x, bh = grid_head();
  if (bh >= p.BH) return;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const int t_begin = seg * p.seg_len, t_end = min(N, t_begin + p.seg_len);
  HeadRsrc hr;
  hr.q = head_rsrc<T>(p.q, bh, N, d);
  hr.k = head_rsrc<T>(p.k, bh, N, d);
  hr.v = head_rsrc<T>(p.v, bh, N, dv);
  hr.o = head_rsrc<T>(p.o, bh, N, dv);
  hr.g = head_rsrc<T>(p.dout, bh, N, dv);
  hr.den = head_rsrc<float>(p.den, bh, N, 1);
  const __amdgpu_buffer_rsrc_t rdq = head_rsrc<T>(p.dq, bh, N, d);
  const float lg2 = DEC ? log2f(p.gamma[bh % p.H]) : 0.f;
  constexpr bool decay = DEC;
  for (int m = threadIdx.x; m <= BC::C; m += BC::NT) sm.pw[m] = exp2f((float)m * lg2);
  zero_tail_columns<BC>(sm.St);

  f32x4 Sa[BC::SPW];
  if (p.nseg > 1)
    slot_load<BC>(Sa, p.ws_f + ((size_t)seg * p.BH + bh) * p.wrec, d, dv, p.slot_vec, wv, li,
                  lg);
  else
    state_load<BC>(Sa, p.S_in ? p.S_in + (size_t)bh * d * dv : nullptr,
                   p.z_in ? p.z_in + (size_t)bh * d : nullptr, d, dv, wv, li, lg);
  // this segment's own adjoint (segments after the first), for the reverse scan
  f32x4 Ra[BC::SPW];
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) Ra[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  BRegs<BC> R;
  load_chunk<BC, VK, true, true, true, true>(R, hr, t_begin, min(BC::C, N - t_begin), d, dv);
  __syncthreads();

  for (int c0 = t_begin; c0 < t_end; c0 += BC::C) {
    const int Lc = min(BC::C, N - c0);
    if constexpr (decay) {
      for (int j = threadIdx.x; j < BC::C; j += BC::NT) sm.kw[j] = j < Lc ? sm.pw[Lc - 1 - j] : 0.f;
      __syncthreads();
    }
    commit_feat<BC>(sm.Fq, nullptr, nullptr, R.q, Lc, d, p.fmap);
    // without decay the weighted keys are phi(k) itself (zero past the chunk)
    commit_feat<BC>(sm.Fk, decay ? sm.KW : nullptr, sm.kw, R.k, Lc, d, p.fmap);
    commit_values<BC>(sm.Vp, R, Lc);
    commit_dn<BC>(sm.dN, R, Lc);
    state_copy<BC>(sm.St, Sa, wv, li, lg);
    if (c0 + BC::C < t_end)  // the next chunk's rows are in flight during this one
      load_chunk<BC, VK, true, true, true, true>(R, hr, c0 + BC::C, min(BC::C, N - c0 - BC::C),
                                                 d, dv);
    __syncthreads();

    tri_tiles<BC, BC::DVK / 32, BC::LDV>(sm.dA, sm.dN, sm.Vp, sm.pw, decay, wv, li, lg);
    __syncthreads();

    // dphi(q) = gamma^(t+1) dN S'_in^T + dA phi(K), then phi'(q)
    constexpr int NQT = BC::NTB * BC::NFB;
#pragma unroll
    for (int n = 0; n < (NQT + BC::NW - 1) / BC::NW; ++n) {
      const int ti = wv + BC::NW * n;
      if (ti >= NQT) break;
      const int tt = ti / BC::NFB, fb = ti % BC::NFB;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < BC::DVK / 32; ++ks) {
        Frag<T> a, b;
        frag_rk(a, sm.dN, BC::LDV, 16 * tt, 32 * ks, li, lg);
        frag_rk(b, sm.St, BC::LDV, 16 * fb, 32 * ks, li, lg);
        mma(acc, a, b);
      }
      if constexpr (decay) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= sm.pw[16 * tt + 4 * lg + r + 1];
      }
      const int kend = (16 * tt + 16 + 31) / 32;
#pragma unroll
      for (int ks = 0; ks < BC::C / 32; ++ks) {
        if (ks >= kend) break;
        Frag<T> a, b;
        frag_rk(a, sm.dA, BC::LDC, 16 * tt, 32 * ks, li, lg);
        frag_kr(b, sm.Fk, BC::LDK, 16 * fb, 32 * ks, li, lg);
        mma(acc, a, b);
      }
      if (p.fmap) {
        float fq[4];
        lds_col4(fq, sm.Fq, BC::LDK, 16 * tt + 4 * lg, 16 * fb, li);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= fminf(fq[r], 1.f);
      }
      out_tile<BC>(sm.Os, BC::LDKS, rdq, acc, c0, 16 * tt, 16 * fb + li, Lc, d, lg);
    }
    // forward state across the chunk
    state_update<BC>(Sa, decay ? sm.KW : sm.Fk, sm.Vp, decay ? sm.pw[Lc] : 1.f, wv, li, lg);
    // the segment's adjoint: += sum_t gamma^(c0 - t_begin + t + 1) phi(q_t) dn_t^T
    if (seg > 0)
      state_update<BC>(Ra, sm.Fq, sm.dN, 1.f, wv, li, lg, decay ? sm.pw + 1 : nullptr,
                       decay ? exp2f((float)(c0 - t_begin) * lg2) : 1.f);
    __syncthreads();
    if constexpr (kStageOut) store_rows<BC, VK>(rdq, sm.Os, BC::LDKS, BC::QCB, c0, Lc, d);
  }
  if (seg > 0)  // into reverse slot seg - 1
    slot_store<BC>(Ra, p.ws_r + ((size_t)(seg - 1) * p.BH + bh) * p.wrec, d, dv, p.slot_vec, wv,
                   li, lg);
}

// ---- dk, dv: chunks right to left, adjoint state ------------------------------
template <class BC, bool VK, bool DEC>
__global__ void __launch_bounds__(BC::NT, BC::WPE_DKV) bwd_dkv_kernel(BwdParams p) {
  using T = typename BC::type;
  __shared__ SmemDkv<BC, DEC> sm;
  const int seg = blockIdx.x, bh = grid_head();
  if (bh >= p.BH) return;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const int t_begin = seg * p.seg_len, t_end = min(N, t_begin + p.seg_len);
  HeadRsrc hr;
  hr.q = head_rsrc<T>(p.q, bh, N, d);
  hr.k = head_rsrc<T>(p.k, bh, N, d);
  hr.v = head_rsrc<T>(p.v, bh, N, dv);
  hr.o = head_rsrc<T>(p.o, bh, N, dv);
  hr.g = head_rsrc<T>(p.dout, bh, N, dv);
  hr.den = head_rsrc<float>(p.den, bh, N, 1);
  const __amdgpu_buffer_rsrc_t rdk = head_rsrc<T>(p.dk, bh, N, d),
                               rdv = head_rsrc<T>(p.dv_, bh, N, dv);
  const float lg2 = DEC ? log2f(p.gamma[bh % p.H]) : 0.f;
  constexpr bool decay = DEC;
  if constexpr (DEC)
    for (int m = threadIdx.x; m <= BC::C; m += BC::NT) sm.pw[m] = exp2f((float)m * lg2);
  zero_tail_columns<BC>(sm.Sh);

  f32x4 Sa[BC::SPW];
  if (p.nseg > 1)
    slot_load<BC>(Sa, p.ws_r + ((size_t)seg * p.BH + bh) * p.wrec, d, dv, p.slot_vec, wv, li,
                  lg);
  else
    state_load<BC>(Sa, p.dS_out ? p.dS_out + (size_t)bh * d * dv : nullptr,
                   p.dz_out ? p.dz_out + (size_t)bh * d : nullptr, d, dv, wv, li, lg);
  const int last = t_begin + ((t_end - t_begin - 1) / BC::C) * BC::C;
  BRegs<BC> R;
  load_chunk<BC, VK, true, true, true, true>(R, hr, last, min(BC::C, N - last), d, dv);
  __syncthreads();

  for (int c0 = last; c0 >= t_begin; c0 -= BC::C) {
    const int Lc = min(BC::C, N - c0);
    commit_feat<BC>(sm.Fq, nullptr, nullptr, R.q, Lc, d, p.fmap);
    commit_feat<BC>(sm.Fk, nullptr, nullptr, R.k, Lc, d, p.fmap);
    commit_values<BC>(sm.Vp, R, Lc);
    commit_dn<BC>(sm.dN, R, Lc);
    state_copy<BC>(sm.Sh, Sa, wv, li, lg);
    if (c0 > t_begin)  // the previous chunk's rows are in flight during this one
      load_chunk<BC, VK, true, true, true, true>(R, hr, c0 - BC::C, BC::C, d, dv);
    __syncthreads();

    tri_tiles<BC, BC::DK / 32, BC::LDK>(sm.Ad, sm.Fq, sm.Fk, sm.pw, decay, wv, li, lg);
    tri_tiles<BC, BC::DVK / 32, BC::LDV>(sm.dA, sm.dN, sm.Vp, sm.pw, decay, wv, li, lg);
    __syncthreads();
    // dphi(k) = gamma^(L-1-j) V' Sh^T + dA^T phi(Q), then phi'(k)
    constexpr int NKT = BC::NTB * BC::NFB;
#pragma unroll
    for (int n = 0; n < (NKT + BC::NW - 1) / BC::NW; ++n) {
      const int ti = wv + BC::NW * n;
      if (ti >= NKT) break;
      const int jt = ti / BC::NFB, fb = ti % BC::NFB;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < BC::DVK / 32; ++ks) {
        Frag<T> a, b;
        frag_rk(a, sm.Vp, BC::LDV, 16 * jt, 32 * ks, li, lg);
        frag_rk(b, sm.Sh, BC::LDV, 16 * fb, 32 * ks, li, lg);
        mma(acc, a, b);
      }
      if constexpr (decay) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= sm.pw[max(Lc - 1 - (16 * jt + 4 * lg + r), 0)];
      }
#pragma unroll
      for (int ks = 0; ks < BC::C / 32; ++ks) {
        if (ks < (16 * jt) / 32) continue;
        Frag<T> a, b;
        frag_kr(a, sm.dA, BC::LDC, 16 * jt, 32 * ks, li, lg);
        frag_kr(b, sm.Fq, BC::LDK, 16 * fb, 32 * ks, li, lg);
        mma(acc, a, b);
      }
      if (p.fmap) {
        float fk[4];
        lds_col4(fk, sm.Fk, BC::LDK, 16 * jt + 4 * lg, 16 * fb, li);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= fminf(fk[r], 1.f);
      }
      out_tile<BC>(sm.Ok, BC::LDKS, rdk, acc, c0, 16 * jt, 16 * fb + li, Lc, d, lg);
    }
    // dv' = gamma^(L-1-j) phi(K) Sh + (A . D)^T dN  (value columns only)
    constexpr int NVT = BC::NTB * (BC::NVP - 1);
#pragma unroll
    for (int n = 0; n < (NVT + BC::NW - 1) / BC::NW; ++n) {
      const int ti = wv + BC::NW * n;
      if (ti >= NVT) break;
      const int jt = ti / (BC::NVP - 1), vb = ti % (BC::NVP - 1);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < BC::DK / 32; ++ks) {
        Frag<T> a, b;
        frag_rk(a, sm.Fk, BC::LDK, 16 * jt, 32 * ks, li, lg);
        frag_kr(b, sm.Sh, BC::LDV, 16 * vb, 32 * ks, li, lg);
        mma(acc, a, b);
      }
      if constexpr (decay) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= sm.pw[max(Lc - 1 - (16 * jt + 4 * lg + r), 0)];
      }
#pragma unroll
      for (int ks = 0; ks < BC::C / 32; ++ks) {
        if (ks < (16 * jt) / 32) continue;
        Frag<T> a, b;
        frag_kr(a, sm.Ad, BC::LDC, 16 * jt, 32 * ks, li, lg);
        frag_kr(b, sm.dN, BC::LDV, 16 * vb, 32 * ks, li, lg);
        mma(acc, a, b);
      }
      out_tile<BC>(sm.Ov, BC::LDOS, rdv, acc, c0, 16 * jt, 16 * vb + li, Lc, dv, lg);
    }
    // adjoint across the chunk: Sh <- gamma^L Sh + (gamma^(t+1) phi(Q))^T dN
    state_update<BC>(Sa, sm.Fq, sm.dN, decay ? sm.pw[Lc] : 1.f, wv, li, lg,
                     decay ? sm.pw + 1 : nullptr);
    __syncthreads();
    if constexpr (kStageOut) {
      store_rows<BC, VK>(rdk, sm.Ok, BC::LDKS, BC::QCB, c0, Lc, d);
      store_rows<BC, VK>(rdv, sm.Ov, BC::LDOS, BC::VCB, c0, Lc, dv);
    }
  }

  if (seg == 0)
    state_store<BC>(Sa, p.dS_in ? p.dS_in + (size_t)bh * d * dv : nullptr,
                    p.dz_in ? p.dz_in + (size_t)bh * d : nullptr, d, dv, wv, li, lg);
}

// Adjoint entering each segment from the right, in place: slot nseg-1 <-
// (dS_out, dz_out); slot s <- gamma^len(s+1) slot (s+1) + dSh_(s+1) (which the
// reverse summary left in slot s).  One thread per record element; every
// record is loaded before the chain.
// CH: per-channel segment decays, from the third part of each reverse slot
// (dq of segment s + 1 left it in slot s).
template <bool CH>
__global__ void __launch_bounds__(256) bwd_rscan_kernel(BwdParams p) {
  const int bh = grid_head();
  if (bh >= p.BH) return;
  const size_t dd = (size_t)p.d * p.dv;
  const size_t rec = dd + p.d;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= rec) return;
  const int nseg = p.nseg;
  const float lg2 = p.gamma ? log2f(p.gamma[bh % p.H]) : 0.f;
  const float gfull = exp2f((float)p.seg_len * lg2);
  const float glast = exp2f((float)(p.N - (nseg - 1) * p.seg_len) * lg2);
  float *base = p.ws_r + (size_t)bh * p.wrec + e;
  const size_t stride = (size_t)p.BH * p.wrec;
  float dS[kMaxSegB];
#pragma unroll
  for (int s = 0; s < kMaxSegB - 1; ++s) dS[s] = s < nseg - 1 ? base[s * stride] : 0.f;
  [[maybe_unused]] float lgd[CH ? kMaxSegB : 1];
  if constexpr (CH) {
    const size_t f = e < dd ? e % p.d : e - dd;  // the element's state row
    const float *ld = p.ws_r + (size_t)bh * p.wrec + dd + p.d + f;
#pragma unroll
    for (int s = 0; s < kMaxSegB - 1; ++s) lgd[s] = s < nseg - 1 ? ld[s * stride] : 0.f;
  }
  float acc;
  if (e < dd)  // slot element e is S[f][n] with n = e / d, f = e % d
    acc = p.dS_out ? p.dS_out[(size_t)bh * dd + (e % p.d) * p.dv + e / p.d] : 0.f;
  else
    acc = p.dz_out ? p.dz_out[(size_t)bh * p.d + (e - dd)] : 0.f;
  base[(size_t)(nseg - 1) * stride] = acc;
#pragma unroll
  for (int s = kMaxSegB - 2; s >= 0; --s) {
    if (s < nseg - 1) {
      float g = s + 1 == nseg - 1 ? glast : gfull;
      if constexpr (CH) g = exp2f(lgd[s]);
      acc = fmaf(g, acc, dS[s]);
      base[s * stride] = acc;
    }
  }
}

// ---- per-key-channel decay (GLA; a separate instantiation) -----------------
// With S_t = diag(alpha_t) S_(t-1) + phi(k_t) v'_t^T, inside a chunk (local
// t, j; lb_t = sum_(s<=t) log2 alpha_s per channel, from the chunk start)
// every decayed product is a plain one of q~_t = phi(q_t) 2^lb_t and
// k~_j = phi(k_j) 2^-lb_j, so the gradients are those of the undecayed rule
// with those features and the mask in place of D:
//     dphi(q_t) = 2^lb_t (S'_in dn_t + sum_(j<=t) dA_tj k~_j)
//     dphi(k_j) = 2^-lb_j (sum_(t>=j) dA_tj q~_t + 2^lb_L Sh v'_j)
//     dv'_j     = sum_(t>=j) A_tj dn_t + Sh^T (phi(k_j) 2^(lb_L - lb_j))
//     Sh       <- 2^lb_L Sh + sum_t (phi(q_t) 2^lb_t) dn_t^T      (rows scaled per channel)
// (dA_tj = dn_t . v'_j, A the decayed scores).  The decay's own gradient,
// d log alpha_s = alpha_s sum_c Sh_s S_(s-1) (per channel; [S | z]), is,
// for s in a chunk entered with S- and left with the adjoint Sh+ of the
// later tokens, the sum of every product that spans token s:
//     2^lb_L <Sh+, S->                                  (the whole chunk)
//   + sum_(j<s)  phi(k_j) 2^(lb_L - lb_j) (Sh+ v'_j)    (keys before s, later tokens)
//   + sum_(t>=s) phi(q_t) 2^lb_t (S- dn_t)              (queries from s, earlier tokens)
//   + sum_(t>=s) sum_(j<s) phi(q_t) phi(k_j) 2^(lb_t - lb_j) dA_tj
// Every term carries alpha_s, so dalpha_s = that / alpha_s keeps its
// relative precision however small alpha_s is (a telescoped form, summing
// phi(q) dphi(q) - phi(k) dphi(k), cancels terms without alpha_s and would
// lose it).  The dq kernel leaves the third sum's terms per token and the
// state entering every chunk; the dk/dv kernel forms the rest.
// The factors are kept in range as in the forward: each 16-token block b
// has references R_b (lb before it), M_b (at its eighth token) and E_b (at
// its last); the tiles hold phi(q) 2^(lb_t - M_b) and phi(k) 2^(M_b - lb_t)
// (within alpha^-8 of phi, log2 alpha clamped at -15), and every other
// factor is a chain of terms that are each at most 1 (see each use).
constexpr float kLog2AlphaMinB = -15.f;

template <class BC>
struct alignas(16) ChanB {
  static constexpr int LDL = BC::DK + 4;
  float lbr[BC::C * LDL];      // lb_t - M_b(t) (rows past the chunk: lb stays)
  float mr[2][BC::DK];         // M_b - R_b (R_0 = 0, R_1 = E_0)
  float rf[2][BC::DK];         // 2^R_b
  float fm[2][BC::DK];         // 2^M_b
  float fl[2][BC::DK];         // 2^(lb_L - M_b)
  float em[2][BC::DK];         // E_b - M_b
  float le[2][BC::DK];         // 2^(lb_L - E_b)
  float qf[2][BC::DK];         // dq: 2^(R_b + log2 decay of the segment before the chunk)
  float mm[BC::DK];            // 2^(M_1 - M_0)
  float dl[BC::DK];            // 2^lb_L
  float anc[BC::DK];           // dk/dv: sum_c Sh+ S+ per channel
  double tot[BC::DK];          // dq: log2 decay of the segment up to the chunk
};

// The chunk's alpha rows, loaded a chunk ahead (element i of the C x DK
// block, row-major, i = thread + n NT), then staged in the exponent tile.
template <class BC>
struct ARegs {
  static_assert((BC::C * BC::DK) % BC::NT == 0, "whole steps");
  static constexpr int NA = BC::C * BC::DK / BC::NT;
  float a[NA];
};

template <class BC>
__device__ __forceinline__ void load_alpha(ARegs<BC> &A, __amdgpu_buffer_rsrc_t ra, int c0,
                                           int Lc, int d) {
#pragma unroll
  for (int n = 0; n < ARegs<BC>::NA; ++n) {
    const int i = threadIdx.x + n * BC::NT;
    const int row = i / BC::DK, col = i % BC::DK;
    const bool ok = row < Lc && col < d;
    A.a[n] = buf_load1(ra, ok ? (uint32_t)(((size_t)(c0 + row) * d + col) * 4) : kOOB,
                       (float *)nullptr);
  }
}

template <class BC>
__device__ __forceinline__ void stage_alpha(ChanB<BC> &cb, const ARegs<BC> &A) {
#pragma unroll
  for (int n = 0; n < ARegs<BC>::NA; ++n) {
    const int i = threadIdx.x + n * BC::NT;
    cb.lbr[(i / BC::DK) * ChanB<BC>::LDL + i % BC::DK] = A.a[n];
  }
}

// Threads per channel of the per-channel passes (lanes next to each other),
// each with JP consecutive tokens of the chunk.
template <class BC>
struct ChanSplit {
  static constexpr int P = BC::NT / BC::DK, JP = BC::C / P;
  static_assert(P * BC::DK == BC::NT && JP * P == BC::C && (P & (P - 1)) == 0 && P <= 16,
                "threads per channel");
};

// The value v of lane OWNER of this thread's group of P adjacent lanes
// (first lane base): for P = 4 a DPP quad broadcast of both halves, else a
// lane shuffle.
template <int P, int OWNER>
__device__ __forceinline__ double group_lane(double v, int base) {
  if constexpr (P == 4) {
    constexpr int ctrl = OWNER * 0x55;  // quad_perm [OWNER, OWNER, OWNER, OWNER]
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    i32x2 w = __builtin_bit_cast(i32x2, v);
    w.x = __builtin_amdgcn_update_dpp(0, w.x, ctrl, 0xF, 0xF, false);
    w.y = __builtin_amdgcn_update_dpp(0, w.y, ctrl, 0xF, 0xF, false);
    return __builtin_bit_cast(double, w);
  } else {
    return __shfl(v, base + OWNER);
  }
}

// before += the parts of the group's lanes M .. P - 2 that precede lane pp.
template <int P, int M>
__device__ __forceinline__ void add_earlier_parts(double &before, double part, int base, int pp) {
  if constexpr (M < P - 1) {
    const double x = group_lane<P, M>(part, base);
    if (M < pp) before += x;
    add_earlier_parts<P, M + 1>(before, part, base, pp);
  }
}

// The chunk's prefix sums (fp64; P threads per channel, each over its JP
// tokens of the staged alpha column, replaced in place by the exponents;
// channels past d and rows past the chunk take alpha = 1) and the tables
// above.  TOT: also the running segment decay.
template <class BC, bool TOT>
__device__ __forceinline__ void chan_tables(ChanB<BC> &cb, int Lc, int d) {
  static_assert(BC::C == 32, "two 16-token blocks per chunk");
  constexpr int LDL = ChanB<BC>::LDL, P = ChanSplit<BC>::P, JP = ChanSplit<BC>::JP;
  const int f = threadIdx.x / P, pp = threadIdx.x % P;
  const int base = (threadIdx.x & 63) - pp;
  double lb[JP];
  double part = 0.0;
#pragma unroll
  for (int jj = 0; jj < JP; ++jj) {
    const int t = pp * JP + jj;
    const float a = (t < Lc && f < d) ? cb.lbr[t * LDL + f] : 1.f;
    part += (double)fmaxf(log2f(a), kLog2AlphaMinB);
    lb[jj] = part;
  }
  double before = 0.0;  // the earlier threads' parts
  add_earlier_parts<P, 0>(before, part, base, pp);
#pragma unroll
  for (int jj = 0; jj < JP; ++jj) lb[jj] += before;
  // block references: M_b at token 16 b + 7, E_b at 16 b + 15 (E_1 = lb_L)
  const double M0 = group_lane<P, 7 / JP>(lb[7 % JP], base);
  const double E0 = group_lane<P, 15 / JP>(lb[15 % JP], base);
  const double M1 = group_lane<P, 23 / JP>(lb[23 % JP], base);
  const double L = group_lane<P, 31 / JP>(lb[31 % JP], base);
#pragma unroll
  for (int jj = 0; jj < JP; ++jj) {
    const int t = pp * JP + jj;
    cb.lbr[t * LDL + f] = (float)(lb[jj] - (t < 16 ? M0 : M1));
  }
  if (pp == 0) {
    const double M[2] = {M0, M1}, E[2] = {E0, L}, R[2] = {0.0, E0};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      cb.mr[b][f] = (float)(M[b] - R[b]);
      cb.rf[b][f] = exp2f((float)R[b]);
      cb.fm[b][f] = exp2f((float)M[b]);
      cb.em[b][f] = (float)(E[b] - M[b]);
      cb.fl[b][f] = exp2f((float)(L - M[b]));
      cb.le[b][f] = exp2f((float)(L - E[b]));
    }
    cb.mm[f] = exp2f((float)(M1 - M0));
    cb.dl[f] = exp2f((float)L);
    if constexpr (TOT) {
      const double seg = cb.tot[f];
#pragma unroll
      for (int b = 0; b < 2; ++b) cb.qf[b][f] = exp2f((float)(seg + R[b]));
      cb.tot[f] = seg + L;
    }
  }
}

// phi rows times 2^(sgn lbr) into F (zero past the chunk and past d); RB:
// times 2^(lbr + M_b - R_b) = 2^(lb_t - R_b) instead (at most 1).
template <class BC, bool RB = false>
__device__ __forceinline__ void commit_feat_ch(typename BC::type *F, const ChanB<BC> &cb,
                                               float sgn,
                                               const typename BC::vec (&X)[BRegs<BC>::NQ],
                                               int Lc, int d, int fmap) {
  using T = typename BC::type;
  using V = typename BC::vec;
#pragma unroll
  for (int n = 0; n < BRegs<BC>::NQ; ++n) {
    const int i = threadIdx.x + n * BC::NT;
    if (i >= BC::C * BC::QCB) break;
    const int row = i / BC::QCB, col0 = (i % BC::QCB) * BC::VEC;
    V f;
#pragma unroll
    for (int e = 0; e < BC::VEC; ++e) {
      const float y = (row < Lc && col0 + e < d) ? feat(to_f32(X[n][e]), fmap) : 0.f;
      const float x = cb.lbr[row * ChanB<BC>::LDL + col0 + e];
      f[e] = from_f32<T>(y * exp2f(RB ? x + cb.mr[row >> 4][col0 + e] : sgn * x));
    }
    *reinterpret_cast<V *>(F + row * BC::LDK + col0) = f;
  }
}

// S <- diag(rs) S + sum_t (X[t][f] op[b(t)][f]) Y[t][c]: X token-major with
// channels as rows of S, op one factor per 16-token block and channel (a
// lane's eight k slots are tokens 8 lg .. 8 lg + 7, all in block lg / 2).
template <class BC>
__device__ __forceinline__ void state_update_ch(f32x4 (&Sa)[BC::SPW],
                                                const typename BC::type *X,
                                                const typename BC::type *Y, const float *rs,
                                                const float (*op)[BC::DK], int wv, int li,
                                                int lg) {
  using T = typename BC::type;
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) {
    const int st = wv + BC::NW * i;
    if (st >= BC::NST) continue;
    const int fb = st / BC::NVP, vb = st % BC::NVP;
#pragma unroll
    for (int r = 0; r < 4; ++r) Sa[i][r] *= rs[16 * fb + 4 * lg + r];
    Frag<T> a, b;
    frag_kr(a, X, BC::LDK, 16 * fb, 0, li, lg);
    const float w = op[lg >> 1][16 * fb + li];
#pragma unroll
    for (int e = 0; e < 8; ++e) a.v[e] = from_f32<T>(to_f32(a.v[e]) * w);
    frag_kr(b, Y, BC::LDV, 16 * vb, 0, li, lg);
    mma(Sa[i], a, b);
  }
}

// Decayed scores A[t][j] = sum_f Qh[t][f] Kh[j][f] (2^(M_1 - M_0))_f for the
// key block before the query block (the tiles are block-relative), zero
// above the diagonal.
template <class BC>
__device__ __forceinline__ void tri_tiles_ch(typename BC::type *M, const typename BC::type *X,
                                             const typename BC::type *Y, const float *mm,
                                             int wv, int li, int lg) {
  using T = typename BC::type;
  constexpr int NTI = BC::NTB * BC::NTB;
#pragma unroll
  for (int n = 0; n < (NTI + BC::NW - 1) / BC::NW; ++n) {
    const int ti = wv + BC::NW * n;
    if (ti >= NTI) break;
    const int tt = ti / BC::NTB, jt = ti % BC::NTB;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (jt <= tt) {
#pragma unroll
      for (int ks = 0; ks < BC::DK / 32; ++ks) {
        Frag<T> a, b;
        frag_rk(a, X, BC::LDK, 16 * tt, 32 * ks, li, lg);
        frag_rk(b, Y, BC::LDK, 16 * jt, 32 * ks, li, lg);
        if (jt < tt) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            b.v[e] = from_f32<T>(to_f32(b.v[e]) * mm[32 * ks + 8 * lg + e]);
        }
        mma(acc, a, b);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tt + 4 * lg + r, j = 16 * jt + li;
      M[t * BC::LDC + j] = from_f32<T>(j <= t ? acc[r] : 0.f);
    }
  }
}

template <class BC>
constexpr int ch_waves_per_simd(size_t lds) {
  const int wg = (int)((160 * 1024) / lds);
  const int w = wg * BC::NW / 4;
  return w < 1 ? 1 : (w > 2 ? 2 : w);
}

// ---- dq with a per-channel decay: chunks left to right, forward state ------
template <class BC>
struct alignas(16) SmemDqCh {
  SmemDq<BC> m;  // Fk holds phi(k) 2^(M_b - lb_j); KW, pw, kw unused
  ChanB<BC> c;
};

template <class BC, bool VK>
__global__ void __launch_bounds__(BC::NT, ch_waves_per_simd<BC>(sizeof(SmemDqCh<BC>)))
    bwd_dq_ch_kernel(BwdParams p) {
  using T = typename BC::type;
  __shared__ SmemDqCh<BC> smc;
  SmemDq<BC> &sm = smc.m;
  ChanB<BC> &cb = smc.c;
  const int seg = blockIdx.x, bh = grid_head();
  if (bh >= p.BH) return;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const int t_begin = seg * p.seg_len, t_end = min(N, t_begin + p.seg_len);
  constexpr int LDL = ChanB<BC>::LDL;
  HeadRsrc hr;
  hr.q = head_rsrc<T>(p.q, bh, N, d);
  hr.k = head_rsrc<T>(p.k, bh, N, d);
  hr.v = head_rsrc<T>(p.v, bh, N, dv);
  hr.o = head_rsrc<T>(p.o, bh, N, dv);
  hr.g = head_rsrc<T>(p.dout, bh, N, dv);
  hr.den = head_rsrc<float>(p.den, bh, N, 1);
  const __amdgpu_buffer_rsrc_t rdq = head_rsrc<T>(p.dq, bh, N, d);
  const __amdgpu_buffer_rsrc_t ra = head_rsrc<float>(p.alpha, bh, N, d);
  float *ux = p.ux + (size_t)bh * N * d;
  const int nch = (N + BC::C - 1) / BC::C;
  zero_tail_columns<BC>(sm.St);
  for (int f = threadIdx.x; f < BC::DK; f += BC::NT) cb.tot[f] = 0.0;

  f32x4 Sa[BC::SPW];
  if (p.nseg > 1)
    slot_load<BC>(Sa, p.ws_f + ((size_t)seg * p.BH + bh) * p.wrec, d, dv, p.slot_vec, wv, li,
                  lg);
  else
    state_load<BC>(Sa, p.S_in ? p.S_in + (size_t)bh * d * dv : nullptr,
                   p.z_in ? p.z_in + (size_t)bh * d : nullptr, d, dv, wv, li, lg);
  f32x4 Ra[BC::SPW];  // this segment's own adjoint (segments after the first)
#pragma unroll
  for (int i = 0; i < BC::SPW; ++i) Ra[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  BRegs<BC> R;
  load_chunk<BC, VK, true, true, true, true>(R, hr, t_begin, min(BC::C, N - t_begin), d, dv);
  ARegs<BC> A;
  load_alpha<BC>(A, ra, t_begin, min(BC::C, N - t_begin), d);
  __syncthreads();

  for (int c0 = t_begin; c0 < t_end; c0 += BC::C) {
    const int Lc = min(BC::C, N - c0);
    stage_alpha<BC>(cb, A);
    __syncthreads();
    chan_tables<BC, true>(cb, Lc, d);
    if (c0 + BC::C < t_end) load_alpha<BC>(A, ra, c0 + BC::C, min(BC::C, N - c0 - BC::C), d);
    __syncthreads();
    commit_feat<BC>(sm.Fq, nullptr, nullptr, R.q, Lc, d, p.fmap);
    commit_feat_ch<BC>(sm.Fk, cb, -1.f, R.k, Lc, d, p.fmap);
    if (seg > 0) commit_feat_ch<BC, true>(sm.KW, cb, 1.f, R.q, Lc, d, p.fmap);
    commit_values<BC>(sm.Vp, R, Lc);
    commit_dn<BC>(sm.dN, R, Lc);
    state_copy<BC>(sm.St, Sa, wv, li, lg);
    // the state entering the chunk, for the dk/dv kernel's dalpha
    slot_store<BC>(Sa, p.chs + ((size_t)bh * nch + c0 / BC::C) * p.wrec, d, dv, p.slot_vec, wv,
                   li, lg);
    if (c0 + BC::C < t_end)
      load_chunk<BC, VK, true, true, true, true>(R, hr, c0 + BC::C, min(BC::C, N - c0 - BC::C),
                                                 d, dv);
    __syncthreads();

    tri_tiles<BC, BC::DVK / 32, BC::LDV>(sm.dA, sm.dN, sm.Vp, sm.pw, false, wv, li, lg);
    __syncthreads();

    // dphi(q_t) = 2^lb_t S'_in dn_t (as 2^(lb_t - R_b) 2^R_b, both <= 1)
    //           + 2^(lb_t - M_b) sum_j dA_tj phi(k_j) 2^(M_b - lb_j)
    // (keys of the block before: 2^(M_1 - M_0) <= 1 on their tile entries)
    constexpr int NQT = BC::NTB * BC::NFB;
#pragma unroll
    for (int n = 0; n < (NQT + BC::NW - 1) / BC::NW; ++n) {
      const int ti = wv + BC::NW * n;
      if (ti >= NQT) break;
      const int tt = ti / BC::NFB, fb = ti % BC::NFB;
      f32x4 acs = {0.f, 0.f, 0.f, 0.f}, acd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < BC::DVK / 32; ++ks) {
        Frag<T> a, b;
        frag_rk(a, sm.dN, BC::LDV, 16 * tt, 32 * ks, li, lg);
        frag_rk(b, sm.St, BC::LDV, 16 * fb, 32 * ks, li, lg);
        mma(acs, a, b);
      }
      {
        Frag<T> a, b;
        frag_rk(a, sm.dA, BC::LDC, 16 * tt, 0, li, lg);
        frag_kr(b, sm.Fk, BC::LDK, 16 * fb, 0, li, lg);
        if (tt == 1 && (lg >> 1) == 0) {
          const float w = cb.mm[16 * fb + li];
#pragma unroll
          for (int e = 0; e < 8; ++e) b.v[e] = from_f32<T>(to_f32(b.v[e]) * w);
        }
        mma(acd, a, b);
      }
      f32x4 acc;
      const int f = 16 * fb + li;
      float fq4[4];
      lds_col4(fq4, sm.Fq, BC::LDK, 16 * tt + 4 * lg, 16 * fb, li);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * lg + r;
        const float lr = cb.lbr[t * LDL + f];
        const float sp = acs[r] * (exp2f(lr + cb.mr[tt][f]) * cb.rf[tt][f]);
        const float dphi = sp + acd[r] * exp2f(lr);
        const float fq = fq4[r];
        if (t < Lc && f < d) ux[(size_t)(c0 + t) * d + f] = fq * sp;  // dalpha's third sum
        acc[r] = dphi * (p.fmap ? fminf(fq, 1.f) : 1.f);
      }
      out_tile<BC>(sm.Os, BC::LDKS, rdq, acc, c0, 16 * tt, f, Lc, d, lg);
    }
    // forward state across the chunk: S <- 2^lb_L S + sum_j (phi(k_j) 2^(lb_L - lb_j)) v'_j^T
    state_update_ch<BC>(Sa, sm.Fk, sm.Vp, cb.dl, cb.fl, wv, li, lg);
    // the segment's adjoint: += sum_t (phi(q_t) 2^(seg decay before t, incl. t)) dn_t^T
    if (seg > 0) {
#pragma unroll
      for (int i = 0; i < BC::SPW; ++i) {
        const int st = wv + BC::NW * i;
        if (st >= BC::NST) continue;
        const int fb = st / BC::NVP, vb = st % BC::NVP;
        const int f = 16 * fb + li;
        Frag<T> a, bb;
        frag_kr(a, sm.KW, BC::LDK, 16 * fb, 0, li, lg);  // phi(q) 2^(lb_t - R_b)
        const float w0 = cb.qf[lg >> 1][f];
#pragma unroll
        for (int e = 0; e < 8; ++e) a.v[e] = from_f32<T>(to_f32(a.v[e]) * w0);
        frag_kr(bb, sm.dN, BC::LDV, 16 * vb, 0, li, lg);
        mma(Ra[i], a, bb);
      }
    }
    __syncthreads();
    store_rows<BC, VK>(rdq, sm.Os, BC::LDKS, BC::QCB, c0, Lc, d);
  }
  if (seg > 0) {  // into reverse slot seg - 1, with the segment's log2 decay per channel
    float *slot = p.ws_r + ((size_t)(seg - 1) * p.BH + bh) * p.wrec;
    slot_store<BC>(Ra, slot, d, dv, p.slot_vec, wv, li, lg);
    for (int f = threadIdx.x; f < d; f += BC::NT)
      slot[(size_t)d * dv + d + f] = (float)cb.tot[f];
  }
}

// ---- dk, dv with a per-channel decay: chunks right to left, adjoint state ---
// The cross-block sums of dalpha's fourth sum, per token and channel (fp32,
// row stride LDX), then the token ranges' totals of its terms ([NW][DK]),
// in the adjoint copy's tile.
template <class BC>
struct CrossB {
  static constexpr int LDX = BC::DK + 4;
  static constexpr size_t bytes = ((size_t)BC::C * LDX + (size_t)BC::NW * BC::DK) * sizeof(float);
  static_assert(BC::C == 32 && BC::NTB == 2, "two 16-token blocks per chunk");
};

// xc[j][f] = Y_j (j in block 0) and xc[t][f] = Z_t (t in block 1), with
// Y_j = mm sum_(t in block 1) q^_t dA_tj and Z_t = mm sum_(j in block 0)
// dA_tj k^_j (q^ = Fq, k^ = Kh, mm = 2^(M_1 - M_0) per channel); the final
// phase multiplies by k^_j or q^_t.  Wave w takes the feature tiles w,
// w + NW, ... of both.
template <class BC>
__device__ __forceinline__ void cross_block_terms(float *xc, const typename BC::type *dA,
                                                  const typename BC::type *Fq,
                                                  const typename BC::type *Kh, const float *mm,
                                                  int wv, int li, int lg) {
  using T = typename BC::type;
  constexpr int LDX = CrossB<BC>::LDX;
  const T zero = from_f32<T>(0.f);
  for (int fb = wv; fb < BC::NFB; fb += BC::NW) {
    const int f = 16 * fb + li;
    const float m = mm[f];
    {  // Y: keys of block 0 (rows 4 lg + r), queries of block 1 only
      Frag<T> a, b;
      frag_kr(a, dA, BC::LDC, 0, 0, li, lg);
      frag_kr(b, Fq, BC::LDK, 16 * fb, 0, li, lg);
      if (lg < 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) b.v[e] = zero;
      }
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      mma(y, a, b);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * lg + r;
        xc[j * LDX + f] = y[r] * m;
      }
    }
    {  // Z: queries of block 1 (rows 16 + 4 lg + r), keys of block 0 only
      Frag<T> a, b;
      frag_rk(a, dA, BC::LDC, 16, 0, li, lg);
      if (lg >= 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a.v[e] = zero;
      }
      frag_kr(b, Kh, BC::LDK, 16 * fb, 0, li, lg);
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      mma(z, a, b);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 + 4 * lg + r;
        xc[t * LDX + f] = z[r] * m;
      }
    }
  }
}

template <class BC>
struct alignas(16) SmemDkvCh {
  static_assert(sizeof(SmemDkv<BC, false>::Sh) >= CrossB<BC>::bytes,
                "the cross-block terms and their range totals fit the adjoint copy's tile");
  static_assert(sizeof(SmemDkv<BC, false>::Ok) >= BC::NVP * BC::DK * sizeof(float) &&
                    sizeof(SmemDkv<BC, false>::Ok) >= 2 * BC::NW * 64 * sizeof(float),
                "the anchor partials and the dalpha range totals fit the dk staging tile");
  SmemDkv<BC, false> m;  // Fq holds phi(q) 2^(lb_t - M_b), Fk phi(k)
  typename BC::type Kh[BC::C * BC::LDK];  // phi(k) 2^(M_b - lb_j)
  ChanB<BC> c;
};

template <class BC, bool VK>
__global__ void __launch_bounds__(BC::NT, ch_waves_per_simd<BC>(sizeof(SmemDkvCh<BC>)))
    bwd_dkv_ch_kernel(BwdParams p) {
  using T = typename BC::type;
  __shared__ SmemDkvCh<BC> smc;
  SmemDkv<BC, false> &sm = smc.m;
  ChanB<BC> &cb = smc.c;
  T *Kh = smc.Kh;
  const int seg = blockIdx.x, bh = grid_head();
  if (bh >= p.BH) return;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const int t_begin = seg * p.seg_len, t_end = min(N, t_begin + p.seg_len);
  constexpr int LDL = ChanB<BC>::LDL;
  HeadRsrc hr;
  hr.q = head_rsrc<T>(p.q, bh, N, d);
  hr.k = head_rsrc<T>(p.k, bh, N, d);
  hr.v = head_rsrc<T>(p.v, bh, N, dv);
  hr.o = head_rsrc<T>(p.o, bh, N, dv);
  hr.g = head_rsrc<T>(p.dout, bh, N, dv);
  hr.den = head_rsrc<float>(p.den, bh, N, 1);
  const __amdgpu_buffer_rsrc_t rdk = head_rsrc<T>(p.dk, bh, N, d),
                               rdv = head_rsrc<T>(p.dv_, bh, N, dv);
  const __amdgpu_buffer_rsrc_t ra = head_rsrc<float>(p.alpha, bh, N, d);
  const float *al = p.alpha + (size_t)bh * N * d;
  const float *ux = p.ux + (size_t)bh * N * d;
  float *dal = p.dalpha + (size_t)bh * N * d;
  const int nch = (N + BC::C - 1) / BC::C;
  zero_tail_columns<BC>(sm.Sh);

  f32x4 Sa[BC::SPW];
  if (p.nseg > 1)
    slot_load<BC>(Sa, p.ws_r + ((size_t)seg * p.BH + bh) * p.wrec, d, dv, p.slot_vec, wv, li,
                  lg);
  else
    state_load<BC>(Sa, p.dS_out ? p.dS_out + (size_t)bh * d * dv : nullptr,
                   p.dz_out ? p.dz_out + (size_t)bh * d : nullptr, d, dv, wv, li, lg);
  const int last = t_begin + ((t_end - t_begin - 1) / BC::C) * BC::C;
  BRegs<BC> R;
  load_chunk<BC, VK, true, true, true, true>(R, hr, last, min(BC::C, N - last), d, dv);
  ARegs<BC> A;
  load_alpha<BC>(A, ra, last, min(BC::C, N - last), d);
  __syncthreads();

  constexpr int NKT = BC::NTB * BC::NFB;
  constexpr int KPW = (NKT + BC::NW - 1) / BC::NW;  // dk tiles per wave
  constexpr int LDX = CrossB<BC>::LDX;
  const float amin = exp2f(kLog2AlphaMinB);
  for (int c0 = last; c0 >= t_begin; c0 -= BC::C) {
    const int Lc = min(BC::C, N - c0);
    // (the previous chunk's cross-block terms overwrote the adjoint copy's
    // zero columns)
    if (c0 != last) zero_tail_columns<BC>(sm.Sh);
    stage_alpha<BC>(cb, A);
    __syncthreads();
    chan_tables<BC, false>(cb, Lc, d);
    __syncthreads();
    // <Sh+, S-> per channel (Sh+: this wave's adjoint tiles as they enter
    // the chunk; S-: the forward state entering it, left by dq): one partial
    // per channel and value tile, in the dk staging tile (free until the dk
    // tiles), summed in a fixed order below
    float *partv = reinterpret_cast<float *>(sm.Ok);
    {
      f32x4 Sm[BC::SPW];  // loaded together, in the adjoint tiles' layout
      slot_load<BC>(Sm, p.chs + ((size_t)bh * nch + c0 / BC::C) * p.wrec, d, dv, p.slot_vec, wv,
                    li, lg);
#pragma unroll
      for (int i = 0; i < BC::SPW; ++i) {
        const int st = wv + BC::NW * i;
        const int fb = st / BC::NVP, vb = st % BC::NVP;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * fb + 4 * lg + r;
          float part = Sa[i][r] * Sm[i][r];
          part = lane_sum<16>(part);
          if (li == 0 && st < BC::NST) partv[vb * BC::DK + f] = part;
        }
      }
    }
    commit_feat_ch<BC>(sm.Fq, cb, 1.f, R.q, Lc, d, p.fmap);
    commit_feat<BC>(sm.Fk, nullptr, nullptr, R.k, Lc, d, p.fmap);
    commit_feat_ch<BC>(Kh, cb, -1.f, R.k, Lc, d, p.fmap);
    commit_values<BC>(sm.Vp, R, Lc);
    commit_dn<BC>(sm.dN, R, Lc);
    state_copy<BC>(sm.Sh, Sa, wv, li, lg);
    __syncthreads();

    tri_tiles_ch<BC>(sm.Ad, sm.Fq, Kh, cb.mm, wv, li, lg);
    tri_tiles<BC, BC::DVK / 32, BC::LDV>(sm.dA, sm.dN, sm.Vp, sm.pw, false, wv, li, lg);
    for (int f = threadIdx.x; f < d; f += BC::NT) {
      float a = 0.f;
      for (int vb = 0; vb < BC::NVP; ++vb) a += partv[vb * BC::DK + f];
      cb.anc[f] = a;
    }
    __syncthreads();
    // dphi(k_j) = 2^(lb_L - lb_j) V' Sh^T (as 2^(E_b - lb_j) 2^(lb_L - E_b))
    //           + 2^(M_b - lb_j) sum_t dA_tj phi(q_t) 2^(lb_t - M_b)
    // (queries of the block after: 2^(M_1 - M_0) <= 1 on their tile entries);
    // dalpha's second sum's terms phi(k_j) (state part) kept in registers
    float xr[KPW][4];
#pragma unroll
    for (int n = 0; n < KPW; ++n) {
      const int ti = wv + BC::NW * n;
      if (ti >= NKT) break;
      const int jt = ti / BC::NFB, fb = ti % BC::NFB;
      f32x4 acs = {0.f, 0.f, 0.f, 0.f}, aci = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < BC::DVK / 32; ++ks) {
        Frag<T> a, b;
        frag_rk(a, sm.Vp, BC::LDV, 16 * jt, 32 * ks, li, lg);
        frag_rk(b, sm.Sh, BC::LDV, 16 * fb, 32 * ks, li, lg);
        mma(acs, a, b);
      }
      {
        Frag<T> a, b;
        frag_kr(a, sm.dA, BC::LDC, 16 * jt, 0, li, lg);
        frag_kr(b, sm.Fq, BC::LDK, 16 * fb, 0, li, lg);
        if (jt == 0 && (lg >> 1) == 1) {
          const float w = cb.mm[16 * fb + li];
#pragma unroll
          for (int e = 0; e < 8; ++e) b.v[e] = from_f32<T>(to_f32(b.v[e]) * w);
        }
        mma(aci, a, b);
      }
      f32x4 acc;
      const int f = 16 * fb + li;
      float fk4[4];
      lds_col4(fk4, sm.Fk, BC::LDK, 16 * jt + 4 * lg, 16 * fb, li);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jt + 4 * lg + r;
        const float lr = cb.lbr[j * LDL + f];
        const float sp = acs[r] * (exp2f(cb.em[jt][f] - lr) * cb.le[jt][f]);
        const float dphi = sp + aci[r] * exp2f(-lr);
        const float fk = fk4[r];
        xr[n][r] = fk * sp;
        acc[r] = dphi * (p.fmap ? fminf(fk, 1.f) : 1.f);
      }
      out_tile<BC>(sm.Ok, BC::LDKS, rdk, acc, c0, 16 * jt, f, Lc, d, lg);
    }
    // dv' = (phi(k_j) 2^(lb_L - lb_j)) Sh + A^T dN  (value columns only)
    constexpr int NVT = BC::NTB * (BC::NVP - 1);
#pragma unroll
    for (int n = 0; n < (NVT + BC::NW - 1) / BC::NW; ++n) {
      const int ti = wv + BC::NW * n;
      if (ti >= NVT) break;
      const int jt = ti / (BC::NVP - 1), vb = ti % (BC::NVP - 1);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < BC::DK / 32; ++ks) {
        Frag<T> a, b;
        frag_rk(a, Kh, BC::LDK, 16 * jt, 32 * ks, li, lg);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          a.v[e] = from_f32<T>(to_f32(a.v[e]) * cb.fl[jt][32 * ks + 8 * lg + e]);
        frag_kr(b, sm.Sh, BC::LDV, 16 * vb, 32 * ks, li, lg);
        mma(acc, a, b);
      }
      {
        Frag<T> a, b;
        frag_kr(a, sm.Ad, BC::LDC, 16 * jt, 0, li, lg);
        frag_kr(b, sm.dN, BC::LDV, 16 * vb, 0, li, lg);
        mma(acc, a, b);
      }
      out_tile<BC>(sm.Ov, BC::LDOS, rdv, acc, c0, 16 * jt, 16 * vb + li, Lc, dv, lg);
    }
    // adjoint across the chunk: Sh <- 2^lb_L Sh + sum_t (phi(q_t) 2^lb_t) dn_t^T
    state_update_ch<BC>(Sa, sm.Fq, sm.dN, cb.dl, cb.fm, wv, li, lg);
    __syncthreads();
    store_rows<BC, VK>(rdk, sm.Ok, BC::LDKS, BC::QCB, c0, Lc, d);
    store_rows<BC, VK>(rdv, sm.Ov, BC::LDOS, BC::VCB, c0, Lc, dv);
    // dalpha: the second sum's terms into the (now unused) exponent tile, then
    // per channel their prefix over the keys before s, the third sum's suffix
    // from dq's terms, and the fourth split by the chunk's two 16-token
    // blocks: its pairs across the blocks from two matrix products, its pairs
    // inside s's block as a running G_j = sum_(t>=s) phi(q_t) 2^(lb_t - M)
    // dA_tj over the block's keys j < s
#pragma unroll
    for (int n = 0; n < KPW; ++n) {
      const int ti = wv + BC::NW * n;
      if (ti >= NKT) break;
      const int jt = ti / BC::NFB, fb = ti % BC::NFB;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        cb.lbr[(16 * jt + 4 * lg + r) * LDL + 16 * fb + li] = xr[n][r];
    }
    // the fourth sum's pairs across the chunk's two token blocks (query t in
    // block 1, key j in block 0), per channel, into the adjoint copy's tile
    // (free now): for a key j, phi(k_j)-side times Y_j = sum_(t in block 1)
    // phi(q_t)-side dA_tj (it enters every s of block 0 after j); for a query
    // t, phi(q_t)-side times Z_t = sum_(j in block 0) dA_tj phi(k_j)-side (it
    // enters every s of block 1 up to t).  Both products are taken on the
    // matrix cores with the other block's k slots zeroed (lanes lg < 2 hold
    // the tokens of block 0); the factor 2^(M_1 - M_0) of the pairs is per
    // channel and goes on after the product.
    float *xc = reinterpret_cast<float *>(sm.Sh);
    cross_block_terms<BC>(xc, sm.dA, sm.Fq, Kh, cb.mm, wv, li, lg);
    __syncthreads();
    {
      // wave wv takes the JP tokens pp JP .. of channels 64 fg + lane
      // (pp = wv % P, fg = wv / P): every lane sums its own channel, no
      // exchange inside the walk
      constexpr int FG = BC::DK / 64, P = BC::NW / FG, JP = BC::C / P;
      static_assert(FG * 64 == BC::DK && P * FG == BC::NW && JP * P == BC::C, "token ranges");
      static_assert(16 % JP == 0, "a token range lies in one 16-token block");
      const int pp = wv % P, f = 64 * (wv / P) + lane;
      const int s0 = pp * JP, blk = s0 / 16;
      const bool fok = f < d;
      float* ytot = partv;                // [P][DK] the ranges' totals (staging tile,
      float* utot = partv + P * BC::DK;   // free again after the dk/dv rows went out)
      float* ctot = xc + BC::C * LDX;     // (after the cross terms)
      float base[JP], alr[JP], cx[JP];
      float yt = 0.f, ut = 0.f, ct = 0.f;
#pragma unroll
      for (int jj = 0; jj < JP; ++jj) {
        const int t = s0 + jj;
        const bool ok = fok && t < Lc;
        const size_t at = (size_t)(c0 + t) * d + f;
        base[jj] = ok ? cb.lbr[t * LDL + f] : 0.f;  // the second sum's term of key t
        // the cross-block term of token t: k^_t Y_t (block 0), q^_t Z_t (block 1)
        cx[jj] = ok ? xc[t * LDX + f] * to_f32((blk == 0 ? Kh : sm.Fq)[t * BC::LDK + f]) : 0.f;
        alr[jj] = ok ? al[at] : 1.f;
        yt += base[jj];
        ct += cx[jj];
        ut += ok ? ux[at] : 0.f;
      }
      ytot[pp * BC::DK + f] = yt;
      utot[pp * BC::DK + f] = ut;
      ctot[pp * BC::DK + f] = ct;
      __syncthreads();
      // the first sum, then the other ranges' parts: the second sum's over the
      // ranges before, the third's over those after; the cross-block terms
      // over the ranges of the same block before (block 0: keys) or after
      // (block 1: queries)
      float run = cb.anc[f] * cb.dl[f], suf = 0.f, cc = 0.f;
      for (int m = 0; m < P; ++m) {
        if (m < pp) run += ytot[m * BC::DK + f];
        if (m > pp) suf += utot[m * BC::DK + f];
        if (blk == 0 ? m < pp : m > pp) cc += ctot[m * BC::DK + f];
      }
      // prefix of the second sum over the keys before s (exclusive), suffix of
      // the third from s (inclusive); the cross-block terms likewise by block;
      // sums only, every term kept carries alpha_s
      float pre[JP];
      if (blk == 0) {  // (uniform)
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) {
          pre[jj] = run + cc;
          run += base[jj];
          cc += cx[jj];
        }
#pragma unroll
        for (int jj = JP - 1; jj >= 0; --jj) {
          const int t = s0 + jj;
          suf += (fok && t < Lc) ? ux[(size_t)(c0 + t) * d + f] : 0.f;
          base[jj] = pre[jj] + suf;
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) {
          pre[jj] = run;
          run += base[jj];
        }
#pragma unroll
        for (int jj = JP - 1; jj >= 0; --jj) {
          const int t = s0 + jj;
          suf += (fok && t < Lc) ? ux[(size_t)(c0 + t) * d + f] : 0.f;
          cc += cx[jj];
          base[jj] = pre[jj] + suf + cc;
        }
      }
      // the fourth sum's pairs inside the range's block: G_j = sum_(t>=s)
      // phi(q_t) 2^(lb_t - M) dA_tj for the block's keys j < s, walking t down
      // from the block's end to this range's first token, eight keys at a
      // time (only the groups below the range's last token).  Branch-free: the
      // row's entries past the diagonal are zero, and a key j >= t enters G_j
      // only with terms of queries at or after j, which an output s <= j never
      // reads; the output masks its keys.  (Query and key share the block's
      // reference M, so no factor enters.)
      using T = typename BC::type;
      const int tl = min(Lc, 16 * blk + 16) - 1;
      for (int j0 = 16 * blk; j0 < s0 + JP - 1; j0 += 8) {  // (uniform)
        float G[8], kq[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          G[jj] = 0.f;
          kq[jj] = to_f32(Kh[(j0 + jj) * BC::LDK + f]);
        }
        for (int t = tl; t >= s0; --t) {  // (uniform)
          const float qk = to_f32(sm.Fq[t * BC::LDK + f]);
          T arow[8];  // row t of dA at these keys (the same for every lane)
          __builtin_memcpy(arow, sm.dA + t * BC::LDC + j0, sizeof(arow));
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) G[jj] = fmaf(qk, to_f32(arow[jj]), G[jj]);
          if (t < s0 + JP) {  // an output of this range: add sum_(j<t) k^_j G_j
            float a4 = 0.f;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) a4 = fmaf(j0 + jj < t ? kq[jj] : 0.f, G[jj], a4);
#pragma unroll
            for (int jj = 0; jj < JP; ++jj) base[jj] += s0 + jj == t ? a4 : 0.f;
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < JP; ++jj) {
        const int t = s0 + jj;
        if (fok && t < Lc)
          dal[(size_t)(c0 + t) * d + f] = alr[jj] >= amin ? base[jj] / alr[jj] : 0.f;
      }
    }
    // the previous chunk's rows go out only now (registers the walk needed)
    if (c0 > t_begin) {
      load_chunk<BC, VK, true, true, true, true>(R, hr, c0 - BC::C, BC::C, d, dv);
      load_alpha<BC>(A, ra, c0 - BC::C, BC::C, d);
    }
    __syncthreads();
  }

  if (seg == 0)
    state_store<BC>(Sa, p.dS_in ? p.dS_in + (size_t)bh * d * dv : nullptr,
                    p.dz_in ? p.dz_in + (size_t)bh * d : nullptr, d, dv, wv, li, lg);
}

template <class BC, bool VK>
hipError_t run_bwd(const BwdParams &p, hipStream_t s) {
  static_assert(sizeof(SmemDq<BC>) <= 160 * 1024 && sizeof(SmemDkv<BC, true>) <= 160 * 1024,
                "LDS budget");
  // dq also leaves each segment's own adjoint in the reverse slots; the
  // reverse scan then turns them into the adjoint entering each segment
  const dim3 grid = head_grid(p.nseg, p.BH);
  hipError_t e = p.gamma ? launch_kernel("linear_bwd_dq", bwd_dq_kernel<BC, VK, true>, grid,
                                         dim3(BC::NT), s, p)
                         : launch_kernel("linear_bwd_dq", bwd_dq_kernel<BC, VK, false>, grid,
                                         dim3(BC::NT), s, p);
  if (e != hipSuccess) return e;
  if (p.nseg > 1) {
    const size_t rec = (size_t)p.d * p.dv + p.d;
    e = launch_kernel("linear_bwd_rscan", bwd_rscan_kernel<false>,
                      head_grid((unsigned)((rec + 255) / 256), p.BH), dim3(256), s, p);
    if (e != hipSuccess) return e;
  }
  return p.gamma ? launch_kernel("linear_bwd_dkv", bwd_dkv_kernel<BC, VK, true>, grid,
                                 dim3(BC::NT), s, p)
                 : launch_kernel("linear_bwd_dkv", bwd_dkv_kernel<BC, VK, false>, grid,
                                 dim3(BC::NT), s, p);
}

// The dk/dv kernel with a per-channel decay takes its operand tiles' rows
// 8 elements past the tile widths (bf16) instead of 16: measured faster
// there (the GLA training step's dk/dv 340 -> 316 us), while the plain
// kernels and dq measured slower with it.
template <class BC>
struct NarrowRows : BC {
  static constexpr int PAD = sizeof(typename BC::type) == 2 ? 8 : BC::PAD;
  static constexpr int LDK = BC::DK + PAD, LDV = BC::DVK + PAD, LDO = BC::DV + PAD;
};

template <class BC, bool VK>
hipError_t run_bwd_ch(const BwdParams &p, hipStream_t s) {
  static_assert(sizeof(SmemDqCh<BC>) <= 160 * 1024 &&
                    sizeof(SmemDkvCh<NarrowRows<BC>>) <= 160 * 1024,
                "LDS budget");
  static_assert(BC::C == kChanBwdChunk, "chunk of the per-channel kernels");
  const dim3 grid = head_grid(p.nseg, p.BH);
  hipError_t e = launch_kernel("linear_bwd_dq", bwd_dq_ch_kernel<BC, VK>, grid, dim3(BC::NT), s, p);
  if (e != hipSuccess) return e;
  if (p.nseg > 1) {
    const size_t rec = (size_t)p.d * p.dv + p.d;
    e = launch_kernel("linear_bwd_rscan", bwd_rscan_kernel<true>,
                      head_grid((unsigned)((rec + 255) / 256), p.BH), dim3(256), s, p);
    if (e != hipSuccess) return e;
  }
  return launch_kernel("linear_bwd_dkv", bwd_dkv_ch_kernel<NarrowRows<BC>, VK>, grid,
                       dim3(BC::NT), s, p);
}

template <class BC>
hipError_t run_bwd_vk(const BwdParams &p, hipStream_t s) {
  if (p.alpha) {
    if constexpr (sizeof(SmemDqCh<BC>) <= 160 * 1024 &&
                  sizeof(SmemDkvCh<NarrowRows<BC>>) <= 160 * 1024)
      return p.vec_ok ? run_bwd_ch<BC, true>(p, s) : run_bwd_ch<BC, false>(p, s);
    else
      return hipErrorInvalidValue;
  }
  return p.vec_ok ? run_bwd<BC, true>(p, s) : run_bwd<BC, false>(p, s);
}

// bf16: 64-token chunks at d = dv = 64, 32-token chunks (and eight waves)
// with 128-wide tiles; fp32: 32-token chunks, feature and value tiles of
// 64 and 64, 64 and 128, or 128 and 64 (128 and 128 exceed the LDS: the
// fp32 state tile alone takes 84 KB).
using BB64x64 = BCfg<bf16, 64, 64, 32, 4, 3>;
using BB64x128 = BCfg<bf16, 64, 128, 32, 8, 2>;
using BB128x64 = BCfg<bf16, 128, 64, 32, 8, 2>;
using BB128x128 = BCfg<bf16, 128, 128, 32, 8, 2>;
using BF64x64 = BCfg<float, 64, 64, 32, 4, 1>;
using BF64x128 = BCfg<float, 64, 128, 32, 4, 1>;
using BF128x64 = BCfg<float, 128, 64, 32, 4, 1>;

// ---- fp32 with d and dv both above 64: value-column halves ------------------
// Every gradient is linear in the value columns: splitting them into two
// halves (each with its own normaliser column carrying that half's share of
// g.o, which add up to the whole), dq and dk (and dL/dz_in) are the sums of
// the halves' results, dv and dL/dS_in their column blocks.  These kernels
// move fp32 rows between the whole width n and the halves [0, na), [na, n).
__global__ void __launch_bounds__(256) split_cols_kernel(const float *src, float *a, float *b,
                                                         size_t rows, int n, int na) {
  const size_t total = rows * (size_t)n;
  const int nb = n - na;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / (size_t)n;
    const int c = (int)(i - r * (size_t)n);
    const float x = src[i];
    if (c < na)
      a[r * na + c] = x;
    else
      b[r * nb + (c - na)] = x;
  }
}

__global__ void __launch_bounds__(256) join_cols_kernel(float *dst, const float *a,
                                                        const float *b, size_t rows, int n,
                                                        int na) {
  const size_t total = rows * (size_t)n;
  const int nb = n - na;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / (size_t)n;
    const int c = (int)(i - r * (size_t)n);
    dst[i] = c < na ? a[r * na + c] : b[r * nb + (c - na)];
  }
}

__global__ void __launch_bounds__(256) add_into_kernel(float *dst, const float *src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] += src[i];
}

unsigned glue_blocks(size_t n) {
  const size_t b = (n + 255) / 256;
  return (unsigned)(b < 4096 ? (b ? b : 1) : 4096);
}

}  // namespace

hipError_t launch_split_cols(const float *src, float *a, float *b, size_t rows, int n, int na,
                             hipStream_t s) {
  if (rows == 0 || n <= na || na <= 0) return hipErrorInvalidValue;
  return launch_kernel("linear_bwd_split", split_cols_kernel,
                       dim3(glue_blocks(rows * (size_t)n)), dim3(256), s, src, a, b, rows, n,
                       na);
}

hipError_t launch_join_cols(float *dst, const float *a, const float *b, size_t rows, int n,
                            int na, hipStream_t s) {
  if (rows == 0 || n <= na || na <= 0) return hipErrorInvalidValue;
  return launch_kernel("linear_bwd_join", join_cols_kernel,
                       dim3(glue_blocks(rows * (size_t)n)), dim3(256), s, dst, a, b, rows, n,
                       na);
}

hipError_t launch_add_into(float *dst, const float *src, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return launch_kernel("linear_bwd_add", add_into_kernel, dim3(glue_blocks(n)), dim3(256), s,
                       dst, src, n);
}

bool linear_backward_supported(int d, int dv, bool bf16_io) {
  return bf16_io || d <= 64 || dv <= 64;
}

bool linear_backward_channel_supported(int d, int dv, bool bf16_io) {
  // the fp32 128-feature tiles of the per-channel kernels exceed the LDS
  return linear_backward_supported(d, dv, bf16_io) && (bf16_io || d <= 64);
}

hipError_t launch_linear_backward(const BwdParams &p, bool bf16_io, hipStream_t s) {
  if (!linear_backward_supported(p.d, p.dv, bf16_io)) return hipErrorInvalidValue;
  if (p.alpha && (p.gamma || !linear_backward_channel_supported(p.d, p.dv, bf16_io)))
    return hipErrorInvalidValue;
  if (!bf16_io) {
    if (p.d <= 64) return p.dv <= 64 ? run_bwd_vk<BF64x64>(p, s) : run_bwd_vk<BF64x128>(p, s);
    return run_bwd_vk<BF128x64>(p, s);
  }
  if (p.d <= 64) return p.dv <= 64 ? run_bwd_vk<BB64x64>(p, s) : run_bwd_vk<BB64x128>(p, s);
  return p.dv <= 64 ? run_bwd_vk<BB128x64>(p, s) : run_bwd_vk<BB128x128>(p, s);
}

}  // namespace la
