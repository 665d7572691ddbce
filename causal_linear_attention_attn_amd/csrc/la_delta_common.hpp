// Definitions shared by the gated-delta-rule prefill (la_prefill_delta.hip)
// and its backward (la_backward_delta.hip): the chunk configuration, the
// per-chunk record layout, the operand loads, and the per-chunk preparation
// kernel (the chunk's triangular solve and the products that depend only on
// its q, k, g and alpha).  The chunked form is derived in
// la_prefill_delta.hip.
#pragma once

#include "la_common.hpp"
#include "la_internal.hpp"

namespace la {
namespace {


constexpr int kXcds = 8;
constexpr int kThreads = 256;  // both kernels: 4 waves
constexpr int kWaves = kThreads / kWave;

template <typename T, int DK_, int C_, int W_>
struct DCfg {
  using type = T;
  using vec = typename Vec16<T>::type;
  static constexpr bool SPLIT = sizeof(T) == 2;  // bf16: hi/lo parts in prep
  static constexpr int DK = DK_, C = C_, W = W_;
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int NRB = C / 16;    // 16-token row blocks of a chunk
  static constexpr int NCT = W / 16;    // 16-column tiles of a value slice
  static constexpr int NGRP = kWaves / NRB;  // column groups of waves
  static constexpr int TW = NCT / NGRP;      // column tiles per wave
  static constexpr int NFT = DK / 16;   // 16-row tiles of the state
  static constexpr int FPW = NFT / kWaves;   // state row tiles per wave
  static constexpr int KSD = DK / 32;   // k-steps over features
  static constexpr int KSC = C / 32;    // k-steps over tokens
  static constexpr int QLD = DK + 2 * VEC;  // row stride: Ks (prep), St (seq); 16 past DK
                                            // (measured 1.5 % faster than 8 in the pass)
  static constexpr int YLD = W + 16;    // row stride: Ys (transpose reads)
  static constexpr int FLD = C + 4;     // fp32 row stride: Nm (prep; + 4 measured faster than + 8)
  static constexpr int TLD = C + VEC;   // row stride: T^T parts (prep)
  static constexpr int QCB = DK / VEC;  // 16-byte blocks per q/k row
  static constexpr size_t WT = (size_t)DK * C;     // Wt elements per chunk
  static constexpr size_t REC = WT + (size_t)C * C;  // workspace elements per chunk
  // the backward's records: Wt, then Wt^T and R^T in the transposed
  // fragment order (rows = tokens) its reverse pass reads
  static constexpr size_t RECB = 2 * WT + (size_t)C * C;
  // register sets of seq_kernel operands (chunks in flight + 1)
  static constexpr int NSET = sizeof(T) == 2 ? 3 : 2;
  static_assert(NRB >= 1 && NGRP >= 1 && NGRP * NRB == kWaves, "row blocks");
  static_assert(TW >= 1 && TW * NGRP == NCT, "column tiles");
  static_assert(FPW >= 1 && FPW * kWaves == NFT, "state tiles");
  static_assert(KSC >= 1, "chunk of at least 32 tokens");
};

// 8 consecutive elements of row `row` (columns col0..col0+7) of a row-major
// [rows, ncols] tensor as an operand fragment; zero outside it.
template <typename T, bool VK>
__device__ __forceinline__ void load_frag8(Frag<T> &f, __amdgpu_buffer_rsrc_t r, int row,
                                           int col0, int ncols, bool row_ok) {
  constexpr int VEC = 16 / (int)sizeof(T);
#pragma unroll
  for (int h = 0; h < 8 / VEC; ++h) {
    const int c = col0 + h * VEC;
    typename Vec16<T>::type x;
    if constexpr (VK) {
      const bool ok = row_ok && c < ncols;
      x = buf_load16<T>(r, ok ? (uint32_t)(((size_t)row * ncols + c) * sizeof(T)) : kOOB);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const bool ok = row_ok && c + e < ncols;
        x[e] = buf_load1(r, ok ? (uint32_t)(((size_t)row * ncols + c + e) * sizeof(T)) : kOOB,
                         (T *)nullptr);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) f.v[h * VEC + e] = x[e];
  }
}

// Four fp32 values to four consecutive T in global memory (8 or 16 bytes).
__device__ __forceinline__ void store4_t(bf16 *dst, f32x4 a) {
  *reinterpret_cast<bf16x4 *>(dst) = (bf16x4){(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
}
__device__ __forceinline__ void store4_t(float *dst, f32x4 a) {
  *reinterpret_cast<f32x4 *>(dst) = a;
}

// High and low parts of an fp32 value in T (exact split for bf16; fp32
// keeps the whole value in the high part).
template <typename T>
__device__ __forceinline__ void split2(float x, T &hi, T &lo) {
  hi = from_f32<T>(x);
  lo = from_f32<T>(x - to_f32(hi));
}

// Element offset of entry (row, col) of a chunk's Wt [DK x C] or R [C x C]
// within its part of the record, in operand-fragment order: 16-row tile,
// then 32-column k-step, then lane (lg * 16 + li holds row 16 tile + li,
// columns 32 ks + 8 lg .. +7), then those 8 elements.  A wave's fragment of
// one (tile, k-step) is then 64 lanes x 8 contiguous elements, which
// seq_kernel loads straight into registers with whole-line loads.
template <int KS>
__device__ __forceinline__ size_t frag_off_k(int row, int col) {
  const int w = col & 31;
  return ((((size_t)(row >> 4) * KS + (col >> 5)) * 64 + (w >> 3) * 16 + (row & 15))
          << 3) + (w & 7);
}
// ... of a matrix whose columns are the chunk's tokens (KSC k-steps)
template <class CF>
__device__ __forceinline__ size_t frag_off(int row, int col) {
  return frag_off_k<CF::KSC>(row, col);
}

// ---------------------------------------------------------------------------
// prep_kernel
// ---------------------------------------------------------------------------
template <class CF>
struct alignas(16) SmemPrep {
  using T = typename CF::type;
  T Ks[CF::C * CF::QLD];     // k rows
  union {
    float Nm[CF::C * CF::FLD];  // N = diag(g) strict_lower(K K^T), then in
                                // place X = (I + N)^(-1)
    T Tt[2][CF::C * CF::TLD];   // T^T high / low parts (after the solve)
  };
  float gs[CF::C];
  float lb[CF::C];            // log b_j: prefix sums of log alpha
  float wl[CF::C];            // b_L / b_j (Wt's token weights)
};

// BWD: the backward's records (Wt, then Wt^T and R^T with the tokens as
// fragment rows: CF::RECB elements per chunk) instead of the prefill's
// (Wt, R: CF::REC).
template <class CF, bool VK, bool DECAY, bool BWD = false>
__global__ void __launch_bounds__(kThreads) prep_kernel(PrefillParams p) {
  using T = typename CF::type;
  constexpr int C = CF::C, FLD = CF::FLD, TLD = CF::TLD, NRB = CF::NRB;
  __shared__ SmemPrep<CF> sm;
  const int chunk = blockIdx.x, bh = grid_head();
  if (bh >= p.BH) return;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int N = p.N, d = p.d;
  const int c0 = chunk * C;
  const int Lc = min(C, N - c0);
  const size_t qk = (size_t)N * d;
  const __amdgpu_buffer_rsrc_t rq =
      buf_rsrc(reinterpret_cast<const T *>(p.q) + (size_t)bh * qk, (uint32_t)(qk * sizeof(T)));
  const __amdgpu_buffer_rsrc_t rk =
      buf_rsrc(reinterpret_cast<const T *>(p.k) + (size_t)bh * qk, (uint32_t)(qk * sizeof(T)));

  // ---- k rows and gates into LDS; this wave's q rows into registers ----
  for (int b = tid; b < C * CF::QCB; b += kThreads) {
    const int row = b / CF::QCB, col0 = (b % CF::QCB) * CF::VEC;
    typename CF::vec x;
    if constexpr (VK) {
      const bool ok = row < Lc && col0 < d;
      x = buf_load16<T>(rk, ok ? (uint32_t)(((size_t)(c0 + row) * d + col0) * sizeof(T)) : kOOB);
    } else {
#pragma unroll
      for (int e = 0; e < CF::VEC; ++e) {
        const bool ok = row < Lc && col0 + e < d;
        x[e] = buf_load1(rk, ok ? (uint32_t)(((size_t)(c0 + row) * d + col0 + e) * sizeof(T))
                                : kOOB, (T *)nullptr);
      }
    }
    *reinterpret_cast<typename CF::vec *>(sm.Ks + row * CF::QLD + col0) = x;
  }
  if (tid < C) sm.gs[tid] = tid < Lc ? p.g[(size_t)bh * N + c0 + tid] : 0.f;
  // log-cumulative decay over the chunk (alpha = 1 past the end): an
  // inclusive prefix sum across the lanes of wave 0
  constexpr bool decay = DECAY;  // a decay alpha was given
  if (decay && wv == 0) {
    float x = lane < Lc ? logf(p.alpha[(size_t)bh * N + c0 + lane]) : 0.f;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const float y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane < C) sm.lb[lane] = x;
  }
  const int rb = wv;  // row block of this wave (waves >= NRB idle in row-block work)
  Frag<T> qf[CF::KSD];
  if (rb < NRB) {
#pragma unroll
    for (int ks = 0; ks < CF::KSD; ++ks)
      load_frag8<T, VK>(qf[ks], rq, c0 + 16 * rb + li, 32 * ks + 8 * lg, d,
                        16 * rb + li < Lc);
  }
  __syncthreads();

  // ---- K K^T (-> N in LDS) and Q K^T (-> registers), lower tiles ----
  // Tiles are computed transposed: pq[tj][r] = q_i . k_j with i = 16 rb + li,
  // j = 16 tj + 4 lg + r (lane keeps one query row, four keys).
  f32x4 pq[NRB];
#pragma unroll
  for (int tj = 0; tj < NRB; ++tj) pq[tj] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (rb < NRB) {
    Frag<T> kr[CF::KSD];
#pragma unroll
    for (int ks = 0; ks < CF::KSD; ++ks)
      lds_frag(kr[ks], sm.Ks + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
    const int i = 16 * rb + li;
    const float gi = sm.gs[i];
    const float lbi = decay ? sm.lb[i] : 0.f;
#pragma unroll
    for (int tj = 0; tj < NRB; ++tj) {
      if (tj <= rb) {
        f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < CF::KSD; ++ks) {
          Frag<T> kc;
          lds_frag(kc, sm.Ks + (16 * tj + li) * CF::QLD + 32 * ks + 8 * lg);
          mma(kk, kc, kr[ks]);
          mma(pq[tj], kc, qf[ks]);
        }
        float n4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * tj + 4 * lg + r;
          const float dec = decay ? expf(lbi - sm.lb[min(j, i)]) : 1.f;  // b_i / b_j
          n4[r] = j < i ? gi * kk[r] * dec : 0.f;
          pq[tj][r] = j <= i ? pq[tj][r] * dec : 0.f;
        }
        lds_store4(sm.Nm + i * FLD + 16 * tj + 4 * lg, n4[0], n4[1], n4[2], n4[3]);
      }
    }
  }
  __syncthreads();
  if (decay && tid < C) {  // b_j for the sequential pass, b_L / b_j for Wt
    float *bdst = reinterpret_cast<float *>(reinterpret_cast<T *>(p.ws) +
                                            (size_t)p.BH * gridDim.x *
                                                (BWD ? CF::RECB : CF::REC)) +
                  ((size_t)bh * gridDim.x + chunk) * C;
    bdst[tid] = BWD ? sm.lb[tid] : expf(sm.lb[tid]);  // the backward takes log b
    sm.wl[tid] = expf(sm.lb[C - 1] - sm.lb[tid]);
  }

  // ---- X = (I + N)^(-1), unit lower triangular, in place over N ----
  // Diagonal 16x16 blocks: lane 16 b + c solves column c of block b by
  // forward substitution (x_c = 1; x_i = -sum_{m<i} N_im x_m for i > c);
  // a block's N is read in full before its X is written (one wave, in
  // order), and nothing else needs it.  Blocks above the diagonal are
  // zeroed meanwhile (N never wrote them).
  if (wv == 0 && lane < 16 * NRB) {
    const int b = lane >> 4, c = lane & 15;
    float *Nb = sm.Nm + (16 * b) * FLD + 16 * b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s = fmaf(Nb[i * FLD + m], x[m], s);
      x[i] = i == c ? 1.f : (i < c ? 0.f : -s);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Nb[i * FLD + c] = x[i];
  }
  for (int e = tid; e < C * C; e += kThreads) {  // strictly upper blocks
    const int i = e / C, j = e % C;
    if ((j >> 4) > (i >> 4)) sm.Nm[i * FLD + j] = 0.f;
  }
  __syncthreads();
  // Blocks below, block row by block row, on the matrix cores in fp32
  // (16x16x4 products, so X keeps full fp32 accuracy): wave w takes column
  // block j = w < i; Y_j = sum_{m=j}^{i-1} N_im X_mj stays in its registers
  // (the accumulator layout, lane (li, lg) holding rows 4 lg + r of column
  // li, is the B operand layout of the second product); after a barrier
  // (every read of block row i of N is done), X_ij = -X_ii Y_j replaces N_ij.
  // A operands take the lane's four consecutive columns 4 lg .. 4 lg + 3 of
  // row li as its k slots (one 16-byte LDS read); B operands the same k rows.
  for (int bi = 1; bi < NRB; ++bi) {
    const int bj = wv;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (bj < bi) {
      for (int bm = bj; bm < bi; ++bm) {
        const f32x4 a =
            *reinterpret_cast<const f32x4 *>(sm.Nm + (16 * bi + li) * FLD + 16 * bm + 4 * lg);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float bk = sm.Nm[(16 * bm + 4 * lg + kk) * FLD + 16 * bj + li];
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], bk, y, 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (bj < bi) {
      const f32x4 a =
          *reinterpret_cast<const f32x4 *>(sm.Nm + (16 * bi + li) * FLD + 16 * bi + 4 * lg);
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) x = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], y[kk], x, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.Nm[(16 * bi + 4 * lg + r) * FLD + 16 * bj + li] = -x[r];
    }
    __syncthreads();
  }

  // ---- T^T (T = X diag(g)) as high and low parts, over X's storage (so X
  //      is first taken into registers); for Wt with decay, column j
  //      carries w_j = b_L / b_j ----
  constexpr int NE = C * C / kThreads;
  static_assert(NE * kThreads == C * C, "T elements per thread");
  float xt[NE];  // T^T[i][j] = T[j][i] = X[j][i] g_i, element e = tid + m * kThreads
#pragma unroll
  for (int m = 0; m < NE; ++m) {
    const int e = tid + m * kThreads, i = e / C, j = e % C;
    xt[m] = sm.Nm[j * FLD + i] * sm.gs[i];
  }
  __syncthreads();
  auto split_t = [&](bool weighted) {
#pragma unroll
    for (int m = 0; m < NE; ++m) {
      const int e = tid + m * kThreads, i = e / C, j = e % C;
      float x = xt[m];
      if (weighted) x *= sm.wl[j];
      T hi, lo;
      split2<T>(x, hi, lo);
      sm.Tt[0][i * TLD + j] = hi;
      sm.Tt[1][i * TLD + j] = lo;
    }
  };
  split_t(decay);
  __syncthreads();

  T *out = reinterpret_cast<T *>(p.ws) +
           ((size_t)bh * gridDim.x + chunk) * (BWD ? CF::RECB : CF::REC);
  // ---- Wt = K^T T, computed as W = T^T K (rows i, columns f) ----
  // stored transposed, Wt[f][i]: the lane's four rows i are contiguous.
  for (int t = wv; t < NRB * CF::NFT; t += kWaves) {
    const int ti = t / CF::NFT, tf = t % CF::NFT;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < CF::KSC; ++ks) {
      if (32 * ks + 31 < 16 * ti) continue;  // T^T[i][j] = 0 for j < i
      Frag<T> kf;
      lds_frag_tr(kf, sm.Ks, CF::QLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * tf, li);
#pragma unroll
      for (int h = 0; h < (CF::SPLIT ? 2 : 1); ++h) {
        Frag<T> a;
        lds_frag(a, sm.Tt[h] + (16 * ti + li) * TLD + 32 * ks + 8 * lg);
        mma(acc, a, kf);
      }
    }
    // lane holds W[i = 16 ti + 4 lg + r][f = 16 tf + li], i.e. Wt[f][i..i+3]
    store4_t(out + frag_off<CF>(16 * tf + li, 16 * ti + 4 * lg), acc);
  }
  if constexpr (BWD) {
    // ---- Wt^T rows for the backward: the same product as Wt = K^T T with
    //      the operands' roles swapped, so the lane holds Wt[f..f+3][i]: row i
    //      of Wt^T, four consecutive features ----
    T *Wtt = out + CF::WT;
    for (int t = wv; t < NRB * CF::NFT; t += kWaves) {
      const int ti = t / CF::NFT, tf = t % CF::NFT;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < CF::KSC; ++ks) {
        if (32 * ks + 31 < 16 * ti) continue;
        Frag<T> kf;
        lds_frag_tr(kf, sm.Ks, CF::QLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * tf, li);
#pragma unroll
        for (int h = 0; h < (CF::SPLIT ? 2 : 1); ++h) {
          Frag<T> a;
          lds_frag(a, sm.Tt[h] + (16 * ti + li) * TLD + 32 * ks + 8 * lg);
          mma(acc, kf, a);
        }
      }
      store4_t(Wtt + frag_off_k<CF::KSD>(16 * ti + li, 16 * tf + 4 * lg), acc);
    }
  }
  if (decay) {  // R takes T itself
    __syncthreads();
    split_t(false);
    __syncthreads();
  }
  // ---- R^T = T^T P^T (rows m, columns i = this wave's row block) ----
  // stored as R[i][m]: the lane's four rows m are contiguous.
  if (rb < NRB) {
    T *Rw = out + (BWD ? 2 * CF::WT : CF::WT);
    const int i = 16 * rb + li;
    for (int tm = 0; tm <= rb; ++tm) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < NRB / 2; ++pp) {
        if (2 * pp > rb || 32 * pp + 31 < 16 * tm) continue;
        // k slots: 0..3 -> keys 32 pp + 4 lg + e, 4..7 -> 32 pp + 16 + 4 lg + e
        Frag<T> bh_, bl_;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          T h0, l0, h1, l1;
          split2<T>(pq[2 * pp][e], h0, l0);
          split2<T>(2 * pp + 1 < NRB ? pq[2 * pp + 1][e] : 0.f, h1, l1);
          bh_.v[e] = h0; bh_.v[4 + e] = h1;
          bl_.v[e] = l0; bl_.v[4 + e] = l1;
        }
        Frag<T> ah, al;
        lds_half(ah, sm.Tt[0] + (16 * tm + li) * TLD + 32 * pp + 4 * lg, 0);
        lds_half(ah, sm.Tt[0] + (16 * tm + li) * TLD + 32 * pp + 16 + 4 * lg, 4);
        // (BWD: operands swapped, acc = R[i..i+3][m], the lane's part of
        // row m of R^T)
        if constexpr (BWD) mma(acc, bh_, ah);
        else mma(acc, ah, bh_);
        if constexpr (CF::SPLIT) {
          lds_half(al, sm.Tt[1] + (16 * tm + li) * TLD + 32 * pp + 4 * lg, 0);
          lds_half(al, sm.Tt[1] + (16 * tm + li) * TLD + 32 * pp + 16 + 4 * lg, 4);
          if constexpr (BWD) {
            mma(acc, bl_, ah);
            mma(acc, bh_, al);
          } else {
            mma(acc, ah, bl_);
            mma(acc, al, bh_);
          }
        }
      }
      // lane holds R^T[m = 16 tm + 4 lg + r][i], i.e. R[i][m..m+3]
      if constexpr (BWD)
        store4_t(Rw + frag_off<CF>(16 * tm + li, 16 * rb + 4 * lg), acc);
      else
        store4_t(Rw + frag_off<CF>(i, 16 * tm + 4 * lg), acc);
    }
    // tiles of R above the diagonal are zero
    for (int tm = rb + 1; tm < NRB; ++tm)
      store4_t(Rw + (BWD ? frag_off<CF>(16 * tm + li, 16 * rb + 4 * lg)
                         : frag_off<CF>(i, 16 * tm + 4 * lg)),
               (f32x4){0.f, 0.f, 0.f, 0.f});
  }
}

template <typename T> struct Vec4;
template <> struct Vec4<bf16> { using type = bf16x4; };
template <> struct Vec4<float> { using type = f32x4; };

// Four consecutive T (8 bytes bf16, 16 bytes fp32) as loaded.
__device__ __forceinline__ bf16x4 buf_load4_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16 *) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ f32x4 buf_load4_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, float *) {
  return buf_load16<float>(r, off);
}

// 8 contiguous record elements at byte offset `off` as a fragment (zero
// past the resource).
__device__ __forceinline__ void load_rec_frag(Frag<bf16> &f, __amdgpu_buffer_rsrc_t r,
                                              uint32_t off) {
  f.v = buf_load16<bf16>(r, off);
}
__device__ __forceinline__ void load_rec_frag(Frag<float> &f, __amdgpu_buffer_rsrc_t r,
                                              uint32_t off) {
  const f32x4 a = buf_load16<float>(r, off), b = buf_load16<float>(r, off + 16u);
  f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace
}  // namespace la
