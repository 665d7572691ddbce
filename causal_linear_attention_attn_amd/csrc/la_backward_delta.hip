// Backward of the gated DELTA rule's chunked prefill (training).
//
// The pages motivate parallel training ("What Is Linear Attention?" section
// 8; "Efficient attention variants" sections 8 and 10) but give no gradient
// formulas.  These are the reverse-mode derivatives of the chunk form of
// la_prefill_delta.hip.  For a chunk of C tokens (L of them valid) entering
// with state S- (b_j = alpha_0 ... alpha_j within the chunk, beta = b_(L-1),
// Db_ji = b_j / b_i; all b = 1 without a decay):
//     L  = strict_lower(K K^T) (.) Db,   P = lower_incl(Q K^T) (.) Db
//     X  = I + diag(g) L,   T = X^(-1) diag(g)
//     Y  = V - diag(b) K S-,   U = T Y        (row j of U: token j's write)
//     O  = diag(b) Q S- + P U,   S+ = beta S- + K^T diag(beta / b) U
// Given dO and Sh+ = dL/dS+ (later chunks and the final-state gradient):
//     dU = P^T dO + D,   D = diag(beta / b) K Sh+
//     lam = X^(-T) dU,   dY = diag(g) lam = Wt^T Sh+ + R^T dO      (= dV)
//     dS- = beta Sh+ + Q^T diag(b) dO - K^T diag(b) dY             (chain)
//     dQ = diag(b) dO S-^T + (dP (.) Mb) K,         dP = dO U^T, Mb = mask (.) Db
//     dK = (dP (.) Mb)^T Q - diag(b) dY S-^T + diag(beta / b) U Sh+^T + (G + G^T) K,
//          G = strict_lower(-dY U^T) (.) Db
//     dg_j = lam_j . r_j,   r = Y - L U   (so that u_j = g_j r_j)
// and with a decay, d log b_j collects b_j q_j . (dO S-^T)_j,
// -b_j k_j . (dY S-^T)_j, the row-minus-column sums of dP (.) P and of
// (-dY U^T) (.) L, minus u_j . D_j; d log beta = beta <Sh+, S-> + sum_j u_j . D_j
// joins b_(L-1); d log alpha_t = sum_(j >= t) d log b_j, dalpha = that / alpha.
//
// Kernels (bf16; the prefill's per-chunk preparation runs first, writing
// Wt and, for the reverse pass, Wt^T and R^T with the tokens as fragment
// rows):
//   bstate_kernel  per (head, 16 value columns), chunks in order: the
//                  prefill's chain (X = K S-, Y = V - diag(b) X,
//                  S+ = beta S- + Wt Y); stores each chunk's S- and Y;
//   brev_kernel    per (head, 16 value columns), chunks in reverse: dY from
//                  Sh+ and dO (written as dV), D, the adjoint chain above;
//                  stores each chunk's Sh+ and D; the last step gives dS_in;
//   bgrad_kernel   per (chunk, head), all in parallel: recomputes L, P, X^(-1),
//                  U, dU, lam from the stored Y, D and the inputs, then dQ,
//                  dK, dg and dalpha.
// Workspace: the preparation records, then the states S- and adjoints Sh+
// of every chunk (transposed, [DV][DK] bf16: a slice workgroup's 16 columns
// are 16 whole rows), then Y and D ([C][DV] bf16).
#include "la_delta_common.hpp"

namespace la {
namespace {

using DB64 = DCfg<bf16, 64, 64, 16>;
using DB128 = DCfg<bf16, 128, 64, 16>;

// Offsets (in elements of bf16, or floats for the decay products) of the
// workspace sections of one backward call.
struct BwdDeltaLayout {
  size_t rec;      // preparation records (bf16), start 0
  size_t dec;      // decay products b_j (fp32 index, after the records)
  size_t states;   // S- per chunk, [DK][DV]
  size_t adj;      // Sh+ per chunk, [DK][DV]
  size_t y;        // Y per chunk, [C][DV]
  size_t dd;       // D per chunk, [C][DV]
  size_t bytes;
};

constexpr size_t align_el(size_t n) { return (n + 127) & ~(size_t)127; }  // 256 bytes

template <class CF>
BwdDeltaLayout bwd_delta_layout(int BH, int N, int dvp) {
  BwdDeltaLayout L{};
  const size_t nch = ((size_t)N + CF::C - 1) / CF::C;
  const size_t heads = (size_t)BH * nch;
  L.rec = 0;
  const size_t rec_bytes = heads * CF::RECB * 2 + heads * CF::C * 4;  // + decay products
  size_t off = align_el((rec_bytes + 1) / 2);
  L.dec = heads * CF::RECB / 2;  // float index of the products (prep's placement)
  L.states = off;
  off = align_el(off + heads * CF::DK * dvp);
  L.adj = off;
  off = align_el(off + heads * CF::DK * dvp);
  L.y = off;
  off = align_el(off + heads * CF::C * dvp);
  L.dd = off;
  off = align_el(off + heads * CF::C * dvp);
  L.bytes = off * 2;
  return L;
}

// Slices of one head share an XCD (workgroup b runs on XCD b % 8).
__device__ __forceinline__ void head_slice(int b, int nslices, int xcd_map, int &bh, int &slice) {
  if (xcd_map) {
    const int j = b / kXcds;
    slice = j % nslices;
    bh = (j / nslices) * kXcds + b % kXcds;
  } else {
    bh = b / nslices;
    slice = b % nslices;
  }
}

// Four consecutive values (8 bytes bf16) of row `row` of a [rows, ncols]
// tensor at column col, zero outside.
template <bool VK>
__device__ __forceinline__ bf16x4 load4(__amdgpu_buffer_rsrc_t r, int row, int col, int ncols,
                                        bool row_ok) {
  if constexpr (VK) {
    return buf_load4_raw(r, row_ok && col < ncols
                                ? (uint32_t)(((size_t)row * ncols + col) * 2) : kOOB,
                         (bf16 *)nullptr);
  } else {
    bf16x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = buf_load1(r, row_ok && col + e < ncols
                              ? (uint32_t)(((size_t)row * ncols + col + e) * 2) : kOOB,
                       (bf16 *)nullptr);
    return x;
  }
}

template <bool VK>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, int row, int col, int ncols,
                                       bool row_ok, f32x4 a) {
  if constexpr (VK) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const bf16x4 h = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r,
                                          row_ok && col < ncols
                                              ? (int)(((size_t)row * ncols + col) * 2)
                                              : (int)kOOB,
                                          0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      buf_store1(r, row_ok && col + e < ncols ? (uint32_t)(((size_t)row * ncols + col + e) * 2)
                                              : kOOB,
                 (bf16)a[e]);
  }
}

// Whole-line blocks of q or k rows of one chunk (this thread's share of the
// workgroup's NT) and their staging into an LDS tile.
template <class CF, bool VK, int NT = kThreads>
struct RowBlocks {
  static constexpr int NB = CF::C * CF::QCB / NT;
  static_assert(NB * NT == CF::C * CF::QCB, "row blocks per thread");
  typename CF::vec x[NB];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int N, int d, int chunk) {
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int b = threadIdx.x + m * NT;
      const int row = chunk * CF::C + b / CF::QCB, col0 = (b % CF::QCB) * CF::VEC;
      if constexpr (VK) {
        x[m] = buf_load16<bf16>(r, (chunk >= 0 && row < N && col0 < d)
                                       ? (uint32_t)(((size_t)row * d + col0) * 2) : kOOB);
      } else {
#pragma unroll
        for (int e = 0; e < CF::VEC; ++e)
          x[m][e] = buf_load1(r, (chunk >= 0 && row < N && col0 + e < d)
                                     ? (uint32_t)(((size_t)row * d + col0 + e) * 2) : kOOB,
                              (bf16 *)nullptr);
      }
    }
  }
  __device__ __forceinline__ void stage(bf16 *tile) const {
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int b = threadIdx.x + m * NT;
      *reinterpret_cast<typename CF::vec *>(tile + (b / CF::QCB) * CF::QLD +
                                            (b % CF::QCB) * CF::VEC) = x[m];
    }
  }
};

// The state slice of the workgroup as its bf16 LDS copy holds it
// (Sl[n * QLD + f] = S[f][n0 + n]) to the chunk's transposed record
// [dvp][DK] (row n: column n of the state over the features), one 16-byte
// store per thread; feature rows past the head's d are zero in the state.
template <class CF>
__device__ __forceinline__ void store_state_rec(bf16 *rec, const bf16 *Sl, int n0) {
  constexpr int FB = CF::DK / 8;  // 16-byte blocks of a record row
  static_assert(CF::W * FB <= kThreads, "one block per thread");
  const int t = threadIdx.x;
  if (t < CF::W * FB) {
    const int n = t / FB, f0 = (t % FB) * 8;
    *reinterpret_cast<bf16x8 *>(rec + (size_t)(n0 + n) * CF::DK + f0) =
        *reinterpret_cast<const bf16x8 *>(Sl + n * CF::QLD + f0);
  }
}

// ---------------------------------------------------------------------------
// bstate_kernel: the prefill's chain, storing S- and Y of every chunk.
// ---------------------------------------------------------------------------
template <class CF>
struct alignas(16) SmemBState {
  bf16 K[2][CF::C * CF::QLD];
  bf16 Ys[CF::C * CF::YLD];
  bf16 St[CF::W * CF::QLD];
};

template <class CF, bool VK, bool DECAY>
__global__ void __launch_bounds__(kThreads) bstate_kernel(BwdDeltaParams p, int nslices,
                                                          int xcd_map) {
  static_assert(CF::W == 16 && CF::NRB == 4 && CF::NCT == 1, "16-column slices, 4 row blocks");
  constexpr int C = CF::C, FPW = CF::FPW, KSC = CF::KSC;
  __shared__ SmemBState<CF> sm;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int rb = wv;
  int bh, slice;
  head_slice(blockIdx.x, nslices, xcd_map, bh, slice);
  const int n0 = slice * 16;
  const int N = p.N, d = p.d, dv = p.dv, nch = p.nch, dvp = p.dvp;
  const size_t qk = (size_t)N * d, vo = (size_t)N * dv;
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc(reinterpret_cast<const bf16 *>(p.k) + bh * qk,
                                             (uint32_t)(qk * 2));
  const __amdgpu_buffer_rsrc_t rv = buf_rsrc(reinterpret_cast<const bf16 *>(p.v) + bh * vo,
                                             (uint32_t)(vo * 2));
  const bf16 *ws = reinterpret_cast<const bf16 *>(p.ws);
  const size_t trec = (size_t)nch * CF::RECB;
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(ws + bh * trec, (uint32_t)(trec * 2));
  // log b_j of every chunk (the preparation kernel's prefix sums of log alpha)
  const float *ldec = reinterpret_cast<const float *>(p.ws) + p.lay_dec + (size_t)bh * nch * C;
  bf16 *states = reinterpret_cast<bf16 *>(p.ws) + p.lay_states + (size_t)bh * nch * CF::DK * dvp;
  bf16 *ybase = reinterpret_cast<bf16 *>(p.ws) + p.lay_y + (size_t)bh * nch * C * dvp;
  const int col = n0 + 4 * lg;  // this lane's four value columns (X, Y)

  struct Ops {
    RowBlocks<CF, VK> k;
    Frag<bf16> w[FPW][KSC];
    bf16x4 v;
  };
  auto fetch = [&](Ops &o, int c) {
    o.k.load(rk, N, d, c < nch ? c : -1);
    const uint32_t base = (uint32_t)((size_t)c * CF::RECB * 2);
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
      for (int a = 0; a < FPW; ++a)
        load_rec_frag(o.w[a][ks], rw,
                      c < nch ? base + (uint32_t)((((size_t)((wv * FPW + a) * KSC + ks) * 64 +
                                                    lane) * 8) * 2)
                              : kOOB);
    const int t = c * C + 16 * rb + li;
    o.v = load4<VK>(rv, t, col, dv, c < nch && t < N);
  };

  f32x4 Sacc[FPW];
  const float *S0 = p.S_in ? p.S_in + (size_t)bh * d * dv : nullptr;
#pragma unroll
  for (int a = 0; a < FPW; ++a) {
    const int n = n0 + li;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = 16 * (wv * FPW + a) + 4 * lg + r;
      Sacc[a][r] = (S0 && f < d && n < dv) ? S0[(size_t)f * dv + n] : 0.f;
    }
    lds_store4(sm.St + li * CF::QLD + 16 * (wv * FPW + a) + 4 * lg, Sacc[a][0], Sacc[a][1],
               Sacc[a][2], Sacc[a][3]);
  }
  Ops cur, nxt;
  fetch(cur, 0);
  fetch(nxt, 1);
  cur.k.stage(sm.K[0]);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int u = c & 1;
    // the state entering the chunk
    store_state_rec<CF>(states + (size_t)c * CF::DK * dvp, sm.St, n0);
    // X^T = S'^T K^T for this wave's 16 tokens; Y = V - b X
    f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < CF::KSD; ++ks) {
      Frag<bf16> sf, kf;
      lds_frag(kf, sm.K[u] + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
      lds_frag(sf, sm.St + li * CF::QLD + 32 * ks + 8 * lg);
      mma(X, sf, kf);
    }
    float b_tok = 1.f, b_last = 1.f;
    if constexpr (DECAY) {
      b_tok = __expf(ldec[(size_t)c * C + 16 * rb + li]);
      b_last = __expf(ldec[(size_t)c * C + C - 1]);
    }
    f32x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = (float)cur.v[r] - b_tok * X[r];
    lds_store4(sm.Ys + (16 * rb + li) * CF::YLD + 4 * lg, y[0], y[1], y[2], y[3]);
    {  // Y record: every row of the chunk (zero past the sequence)
      bf16 *yr = ybase + ((size_t)c * C + 16 * rb + li) * dvp + col;
      if (col < dvp)
        *reinterpret_cast<bf16x4 *>(yr) = (bf16x4){(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
    }
    __syncthreads();
    // S+ = beta S- + Wt Y
#pragma unroll
    for (int a = 0; a < FPW; ++a) Sacc[a] *= b_last;
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      Frag<bf16> yf;
      lds_frag_tr(yf, sm.Ys, CF::YLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 0, li);
#pragma unroll
      for (int a = 0; a < FPW; ++a) mma(Sacc[a], cur.w[a][ks], yf);
    }
#pragma unroll
    for (int a = 0; a < FPW; ++a)
      lds_store4(sm.St + li * CF::QLD + 16 * (wv * FPW + a) + 4 * lg, Sacc[a][0], Sacc[a][1],
                 Sacc[a][2], Sacc[a][3]);
    nxt.k.stage(sm.K[u ^ 1]);
    cur = nxt;
    fetch(nxt, c + 2);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// brev_kernel: the adjoint chain over chunks in reverse.  NWR waves: with
// four, each takes one 16-token row block (dY and D) and a quarter of the
// state tiles; with eight (d = 128), the two waves of a row block take its
// dY and its D, and each wave an eighth of the state tiles, so that every
// SIMD holds two waves of the chain.
// ---------------------------------------------------------------------------
template <class CF>
struct alignas(16) SmemBRev {
  bf16 Q[2][CF::C * CF::QLD];
  bf16 K[2][CF::C * CF::QLD];
  bf16 dO[2][CF::C * CF::YLD];   // dO rows (this slice's columns)
  bf16 dOb[2][CF::C * CF::YLD];  // b dO
  bf16 dYb[CF::C * CF::YLD];     // -b dY
  bf16 Sh[CF::W * CF::QLD];      // Sh'^T: bf16 copy of the adjoint slice
};

template <class CF, bool VK, bool DECAY, int NWR>
__global__ void __launch_bounds__(NWR *kWave) brev_kernel(BwdDeltaParams p, int nslices,
                                                          int xcd_map) {
  static_assert(CF::W == 16 && CF::NRB == 4 && CF::NCT == 1, "16-column slices, 4 row blocks");
  constexpr int C = CF::C, KSC = CF::KSC, KSD = CF::KSD;
  constexpr int FPW = CF::NFT / NWR;  // state row tiles per wave
  constexpr bool SPLIT = NWR == 2 * CF::NRB;
  static_assert(FPW >= 1 && FPW * NWR == CF::NFT && (NWR == CF::NRB || SPLIT), "wave split");
  __shared__ SmemBRev<CF> sm;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int rb = wv % CF::NRB;
  // (wave-uniform) this wave computes its row block's dY, its D, or both
  const bool do_dy = !SPLIT || wv < CF::NRB, do_dd = !SPLIT || wv >= CF::NRB;
  int bh, slice;
  head_slice(blockIdx.x, nslices, xcd_map, bh, slice);
  const int n0 = slice * 16;
  const int N = p.N, d = p.d, dv = p.dv, nch = p.nch, dvp = p.dvp;
  const size_t qk = (size_t)N * d, vo = (size_t)N * dv;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(reinterpret_cast<const bf16 *>(p.q) + bh * qk,
                                             (uint32_t)(qk * 2));
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc(reinterpret_cast<const bf16 *>(p.k) + bh * qk,
                                             (uint32_t)(qk * 2));
  const __amdgpu_buffer_rsrc_t rdo = buf_rsrc(reinterpret_cast<const bf16 *>(p.dout) + bh * vo,
                                              (uint32_t)(vo * 2));
  const __amdgpu_buffer_rsrc_t rdv = buf_rsrc(reinterpret_cast<bf16 *>(p.dv_) + bh * vo,
                                              (uint32_t)(vo * 2));
  const bf16 *ws = reinterpret_cast<const bf16 *>(p.ws);
  const size_t trec = (size_t)nch * CF::RECB;
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(ws + bh * trec, (uint32_t)(trec * 2));
  const float *ldec = reinterpret_cast<const float *>(p.ws) + p.lay_dec + (size_t)bh * nch * C;
  bf16 *adj = reinterpret_cast<bf16 *>(p.ws) + p.lay_adj + (size_t)bh * nch * CF::DK * dvp;
  bf16 *dbase = reinterpret_cast<bf16 *>(p.ws) + p.lay_dd + (size_t)bh * nch * C * dvp;
  const int col = n0 + 4 * lg;

  struct Ops {
    RowBlocks<CF, VK, NWR * kWave> q, k;
    Frag<bf16> wt[KSD], rt[KSC];  // Wt^T and R^T rows of this wave's 16 tokens (dY)
    bf16x4 dout;
    float lb;  // log b of this lane's token
  };
  auto fetch = [&](Ops &o, int c) {
    const bool ok = c >= 0;
    o.q.load(rq, N, d, ok ? c : -1);
    o.k.load(rk, N, d, ok ? c : -1);
    const uint32_t base = ok ? (uint32_t)((size_t)c * CF::RECB * 2) : 0u;
    if (do_dy) {
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
        load_rec_frag(o.wt[ks], rw,
                      ok ? base + (uint32_t)((CF::WT + ((size_t)(rb * KSD + ks) * 64 + lane) * 8) *
                                             2)
                         : kOOB);
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks)
        load_rec_frag(o.rt[ks], rw,
                      ok ? base + (uint32_t)((2 * CF::WT +
                                              ((size_t)(rb * KSC + ks) * 64 + lane) * 8) * 2)
                         : kOOB);
    }
    const int t = c * C + 16 * rb + li;
    o.dout = load4<VK>(rdo, t, col, dv, ok && t < N);
    o.lb = (DECAY && ok) ? ldec[(size_t)c * C + 16 * rb + li] : 0.f;
  };
  auto stage = [&](const Ops &o, int u) {
    o.q.stage(sm.Q[u]);
    o.k.stage(sm.K[u]);
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (float)o.dout[e];
    const float b = DECAY ? __expf(o.lb) : 1.f;
    if (do_dy) lds_store4(sm.dO[u] + (16 * rb + li) * CF::YLD + 4 * lg, x[0], x[1], x[2], x[3]);
    if (do_dd)
      lds_store4(sm.dOb[u] + (16 * rb + li) * CF::YLD + 4 * lg, b * x[0], b * x[1], b * x[2],
                 b * x[3]);
  };

  f32x4 Sacc[FPW];
  const float *Sh0 = p.dS_out ? p.dS_out + (size_t)bh * d * dv : nullptr;
#pragma unroll
  for (int a = 0; a < FPW; ++a) {
    const int n = n0 + li;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = 16 * (wv * FPW + a) + 4 * lg + r;
      Sacc[a][r] = (Sh0 && f < d && n < dv) ? Sh0[(size_t)f * dv + n] : 0.f;
    }
    lds_store4(sm.Sh + li * CF::QLD + 16 * (wv * FPW + a) + 4 * lg, Sacc[a][0], Sacc[a][1],
               Sacc[a][2], Sacc[a][3]);
  }
  Ops cur, nxt;
  fetch(cur, nch - 1);
  fetch(nxt, nch - 2);
  stage(cur, (nch - 1) & 1);
  __syncthreads();
  for (int c = nch - 1; c >= 0; --c) {
    const int u = c & 1;
    const float lbeta = DECAY ? ldec[(size_t)c * C + C - 1] : 0.f;
    const float beta = DECAY ? __expf(lbeta) : 1.f;
    store_state_rec<CF>(adj + (size_t)c * CF::DK * dvp, sm.Sh, n0);
    // dY^T = Sh'^T Wt + dO^T R and D^T = Sh'^T K^T for this wave's 16 tokens
    f32x4 dy = {0.f, 0.f, 0.f, 0.f}, dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      Frag<bf16> sf, kf;
      lds_frag(sf, sm.Sh + li * CF::QLD + 32 * ks + 8 * lg);
      if (do_dy) mma(dy, sf, cur.wt[ks]);
      if (do_dd) {
        lds_frag(kf, sm.K[u] + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
        mma(dd, sf, kf);
      }
    }
    const int t = c * C + 16 * rb + li;  // this lane's token; dY[t][col .. col + 3]
    if (do_dy) {
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        if (32 * ks + 31 < 16 * rb) continue;  // R[j][t] = 0 for j < t
        Frag<bf16> of;
        lds_frag_tr(of, sm.dO[u], CF::YLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 0, li);
        mma(dy, of, cur.rt[ks]);
      }
      store4<VK>(rdv, t, col, dv, t < N, dy);
      const float nb = DECAY ? -__expf(cur.lb) : -1.f;
      lds_store4(sm.dYb + (16 * rb + li) * CF::YLD + 4 * lg, nb * dy[0], nb * dy[1], nb * dy[2],
                 nb * dy[3]);
    }
    if (do_dd) {
      const float wl = DECAY ? __expf(lbeta - cur.lb) : 1.f;  // beta / b_t
      bf16 *dr = dbase + ((size_t)c * C + 16 * rb + li) * dvp + col;
      if (col < dvp)
        *reinterpret_cast<bf16x4 *>(dr) = (bf16x4){(bf16)(wl * dd[0]), (bf16)(wl * dd[1]),
                                                   (bf16)(wl * dd[2]), (bf16)(wl * dd[3])};
    }
    __syncthreads();
    // Sh- = beta Sh+ + Q^T (b dO) + K^T (-b dY)
#pragma unroll
    for (int a = 0; a < FPW; ++a) Sacc[a] *= beta;
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      Frag<bf16> ob, yb;
      lds_frag_tr(ob, sm.dOb[u], CF::YLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 0, li);
      lds_frag_tr(yb, sm.dYb, CF::YLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 0, li);
#pragma unroll
      for (int a = 0; a < FPW; ++a) {
        Frag<bf16> qf, kf;
        const int f0 = 16 * (wv * FPW + a);
        lds_frag_tr(qf, sm.Q[u], CF::QLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, f0, li);
        lds_frag_tr(kf, sm.K[u], CF::QLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, f0, li);
        mma(Sacc[a], qf, ob);
        mma(Sacc[a], kf, yb);
      }
    }
#pragma unroll
    for (int a = 0; a < FPW; ++a)
      lds_store4(sm.Sh + li * CF::QLD + 16 * (wv * FPW + a) + 4 * lg, Sacc[a][0], Sacc[a][1],
                 Sacc[a][2], Sacc[a][3]);
    if (c > 0) stage(nxt, u ^ 1);
    cur = nxt;
    fetch(nxt, c - 2);
    __syncthreads();
  }
  if (p.dS_in) {
    float *Si = p.dS_in + (size_t)bh * d * dv;
#pragma unroll
    for (int a = 0; a < FPW; ++a) {
      const int n = n0 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * (wv * FPW + a) + 4 * lg + r;
        if (f < d && n < dv) Si[(size_t)f * dv + n] = Sacc[a][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bgrad_kernel: the per-chunk gradients, every chunk in parallel.  Its tiles
// fill the LDS, so one workgroup runs per CU; it has sixteen waves, four per
// 16-row block of the chunk, each taking a quarter of the block's output
// tiles (value column tiles of U, dU and lambda; feature tiles of dQ and dK;
// every fourth column block of L, P and dP), so that every SIMD holds four
// waves to cover each other's LDS and matrix-core latency.
constexpr int kGSplit = 4, kGWaves = 4 * kGSplit, kGThreads = kGWaves * kWave;
// ---------------------------------------------------------------------------
template <int DK_, int DV_>
struct GCfg {
  static constexpr int C = 64, DK = DK_, DV = DV_;
  static constexpr int NRB = C / 16, NFT = DK / 16, NVT = DV / 16;
  static constexpr int LDK = DK + 8, LDV = DV + 8, LDC = C + 8, LDX = C + 4;
};

template <class G>
struct alignas(16) SmemGrad {
  bf16 Qs[G::C * G::LDK], Ks[G::C * G::LDK];
  bf16 dOs[G::C * G::LDV], dYs[G::C * G::LDV], Ys[G::C * G::LDV], Ds[G::C * G::LDV],
      Us[G::C * G::LDV];
  bf16 Lb[G::C * G::LDC], Pb[G::C * G::LDC];  // L then G + G^T; P then dP (.) Mb
  float Xi[G::C * G::LDX];                    // X, then X^(-1)
  float gs[G::C], lb[G::C], al[G::C], Gi[G::C];
  float dlb[kGWaves][G::C];  // per-wave parts of d log b
  float dgp[kGSplit][G::C];  // the parts of dg; later the waves' parts of <Sh+, S->
};

// Rows of a [tokens, ncols] bf16 tensor (or a chunk record) into an LDS tile
// of `cols` columns (zero outside rows < nrows, columns < ncols).
template <bool VK>
__device__ __forceinline__ void tile_load(bf16 *tile, int ld, int cols, __amdgpu_buffer_rsrc_t r,
                                          int row0, int nrows, int ncols, int rstride) {
  const int cb = cols / 8;
  for (int b = threadIdx.x; b < 64 * cb; b += kGThreads) {
    const int row = b / cb, c0 = (b % cb) * 8;
    bf16x8 x;
    const bool ok = row < nrows;
    if constexpr (VK) {
      x = buf_load16<bf16>(r, ok && c0 < ncols
                                  ? (uint32_t)(((size_t)(row0 + row) * rstride + c0) * 2) : kOOB);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = buf_load1(r, ok && c0 + e < ncols
                                ? (uint32_t)(((size_t)(row0 + row) * rstride + c0 + e) * 2)
                                : kOOB,
                         (bf16 *)nullptr);
    }
    *reinterpret_cast<bf16x8 *>(tile + row * ld + c0) = x;
  }
}

// The first nrows rows of an LDS tile (cols columns, stride ld) to rows
// row0 .. of a [N, ncols] bf16 tensor (columns past ncols not written),
// every thread 16-byte blocks (VK: ncols % 8 == 0 and 16-byte aligned rows).
template <bool VK>
__device__ __forceinline__ void tile_store(const bf16 *tile, int ld, int cols, bf16 *out,
                                           int row0, int nrows, int ncols) {
  const int cb = cols / 8;
  for (int b = threadIdx.x; b < 64 * cb; b += kGThreads) {
    const int row = b / cb, c0 = (b % cb) * 8;
    if (row >= nrows) continue;
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(tile + row * ld + c0);
    bf16 *dst = out + (size_t)(row0 + row) * ncols + c0;
    if constexpr (VK) {
      if (c0 < ncols) *reinterpret_cast<bf16x8 *>(dst) = x;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < ncols) dst[e] = x[e];
    }
  }
}

// A transposed state record [dvp][DK] (row n: the state's column n), DV
// rows of it, in registers: loaded ahead of the phase that stages it into an
// LDS tile (stride ld), so that its latency overlaps the phases before;
// rows past dv are zero.  Every thread takes 16-byte blocks.
template <int DK, int DV>
struct RecRegs {
  static constexpr int CB = DK / 8, NB = (DV * CB + kGThreads - 1) / kGThreads;
  bf16x8 x[NB];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int dv) {
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int b = threadIdx.x + m * kGThreads, n = b / CB, f0 = (b % CB) * 8;
      x[m] = buf_load16<bf16>(r, b < DV * CB && n < dv ? (uint32_t)(((size_t)n * DK + f0) * 2)
                                                        : kOOB);
    }
  }
  __device__ __forceinline__ void stage(bf16 *tile, int ld) const {
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int b = threadIdx.x + m * kGThreads;
      if (b < DV * CB) *reinterpret_cast<bf16x8 *>(tile + (b / CB) * ld + (b % CB) * 8) = x[m];
    }
  }
};

__device__ __forceinline__ float sum16(float x) {  // over the 16 lanes li of a slot group
  return lane_sum<16>(x);
}

template <class G, bool VK, bool DECAY>
__global__ void __launch_bounds__(kGThreads) bgrad_kernel(BwdDeltaParams p) {
  constexpr int C = G::C, DK = G::DK, DV = G::DV, NRB = G::NRB;
  constexpr int NVH = G::NVT / kGSplit, NFH = G::NFT / kGSplit;  // a wave's value / feature tiles
  static_assert(kGSplit * NRB == kGWaves && kGSplit * NVH == G::NVT && kGSplit * NFH == G::NFT,
                "wave split");
  constexpr int LDK = G::LDK, LDV = G::LDV, LDC = G::LDC, LDX = G::LDX;
  __shared__ SmemGrad<G> sm;
  const int chunk = blockIdx.x, bh = grid_head();
  if (bh >= p.BH) return;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
  // part h of row block rb; the waves w, w + 4, ... of one SIMD alternate
  // between an early and a late row block, whose triangular parts differ
  // in length
  const int h = wv >> 2, rb = (h & 1) ? NRB - 1 - (wv & 3) : (wv & 3);
  const int N = p.N, d = p.d, dv = p.dv, nch = p.nch, dvp = p.dvp;
  const int c0 = chunk * C, Lc = min(C, N - c0);
  const size_t qk = (size_t)N * d, vo = (size_t)N * dv;
  const bf16 *wsb = reinterpret_cast<const bf16 *>(p.ws);
  const size_t rec_s = (size_t)DK * dvp, rec_y = (size_t)C * dvp;
  const size_t ci = (size_t)bh * nch + chunk;
  const __amdgpu_buffer_rsrc_t rS = buf_rsrc(wsb + p.lay_states + ci * rec_s,
                                             (uint32_t)(rec_s * 2));
  const __amdgpu_buffer_rsrc_t rA = buf_rsrc(wsb + p.lay_adj + ci * rec_s, (uint32_t)(rec_s * 2));
  const float *ldec = reinterpret_cast<const float *>(p.ws) + p.lay_dec + ci * C;

  // ---- load the chunk's tiles ----
  {
    const bf16 *q = reinterpret_cast<const bf16 *>(p.q) + bh * qk;
    const bf16 *k = reinterpret_cast<const bf16 *>(p.k) + bh * qk;
    const bf16 *dout = reinterpret_cast<const bf16 *>(p.dout) + bh * vo;
    const bf16 *dy = reinterpret_cast<const bf16 *>(p.dv_) + bh * vo;
    tile_load<VK>(sm.Qs, LDK, DK, buf_rsrc(q, (uint32_t)(qk * 2)), c0, Lc, d, d);
    tile_load<VK>(sm.Ks, LDK, DK, buf_rsrc(k, (uint32_t)(qk * 2)), c0, Lc, d, d);
    tile_load<VK>(sm.dOs, LDV, DV, buf_rsrc(dout, (uint32_t)(vo * 2)), c0, Lc, dv, dv);
    tile_load<VK>(sm.dYs, LDV, DV, buf_rsrc(dy, (uint32_t)(vo * 2)), c0, Lc, dv, dv);
    tile_load<true>(sm.Ys, LDV, DV, buf_rsrc(wsb + p.lay_y + ci * rec_y, (uint32_t)(rec_y * 2)),
                    0, C, dv, dvp);
    tile_load<true>(sm.Ds, LDV, DV, buf_rsrc(wsb + p.lay_dd + ci * rec_y, (uint32_t)(rec_y * 2)),
                    0, C, dv, dvp);
  }
  if (tid < C) {
    sm.gs[tid] = tid < Lc ? p.g[(size_t)bh * N + c0 + tid] : 0.f;
    sm.lb[tid] = DECAY ? ldec[tid] : 0.f;  // log b_j (constant past the chunk)
    sm.al[tid] = (DECAY && tid < Lc) ? p.alpha[(size_t)bh * N + c0 + tid] : 1.f;
  }
  for (int e = tid; e < kGWaves * C; e += kGThreads) (&sm.dlb[0][0])[e] = 0.f;
  for (int e = tid; e < C * LDC; e += kGThreads) {
    sm.Lb[e] = (bf16)0.f;
    sm.Pb[e] = (bf16)0.f;
  }
  for (int e = tid; e < C * C; e += kGThreads) sm.Xi[(e / C) * LDX + e % C] = 0.f;
  __syncthreads();
  const float lbeta = DECAY ? sm.lb[C - 1] : 0.f;

  // ---- L, P (bf16) and N = diag(g) L (fp32), lower tiles; lane: row
  //      i = 16 rb + li, columns j = 16 tj + 4 lg + r ----
  {
    const int i = 16 * rb + li;
    Frag<bf16> kr[DK / 32], qr[DK / 32];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      lds_frag(kr[ks], sm.Ks + i * LDK + 32 * ks + 8 * lg);
      lds_frag(qr[ks], sm.Qs + i * LDK + 32 * ks + 8 * lg);
    }
    const float gi = sm.gs[i], lbi = sm.lb[i];
#pragma unroll
    for (int tj = 0; tj < NRB; ++tj) {
      if (tj > rb || tj % kGSplit != h) continue;
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        Frag<bf16> kc;
        lds_frag(kc, sm.Ks + (16 * tj + li) * LDK + 32 * ks + 8 * lg);
        mma(kk, kc, kr[ks]);
        mma(pq, kc, qr[ks]);
      }
      float l4[4], p4[4], n4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * tj + 4 * lg + r;
        const float db = DECAY ? __expf(lbi - sm.lb[min(j, i)]) : 1.f;
        l4[r] = j < i ? kk[r] * db : 0.f;
        p4[r] = j <= i ? pq[r] * db : 0.f;
        n4[r] = gi * l4[r];
      }
      lds_store4(sm.Lb + i * LDC + 16 * tj + 4 * lg, l4[0], l4[1], l4[2], l4[3]);
      lds_store4(sm.Pb + i * LDC + 16 * tj + 4 * lg, p4[0], p4[1], p4[2], p4[3]);
      *reinterpret_cast<f32x4 *>(sm.Xi + i * LDX + 16 * tj + 4 * lg) =
          (f32x4){n4[0], n4[1], n4[2], n4[3]};
    }
  }
  __syncthreads();

  // ---- X^(-1), X = I + N unit lower triangular, in place (as the
  //      preparation kernel: diagonal blocks by forward substitution, then
  //      block rows on the fp32 matrix cores) ----
  if (wv == 0 && lane < 16 * NRB) {
    const int b = lane >> 4, c = lane & 15;
    float *Nb = sm.Xi + (16 * b) * LDX + 16 * b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s = fmaf(Nb[i * LDX + m], x[m], s);
      x[i] = i == c ? 1.f : (i < c ? 0.f : -s);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Nb[i * LDX + c] = x[i];
  }
  __syncthreads();
  for (int bi = 1; bi < NRB; ++bi) {
    const int bj = wv;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (bj < bi) {
      for (int bm = bj; bm < bi; ++bm) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(sm.Xi + (16 * bi + li) * LDX + 16 * bm +
                                                         4 * lg);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float bk = sm.Xi[(16 * bm + 4 * lg + kk) * LDX + 16 * bj + li];
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], bk, y, 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (bj < bi) {
      const f32x4 a =
          *reinterpret_cast<const f32x4 *>(sm.Xi + (16 * bi + li) * LDX + 16 * bi + 4 * lg);
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], y[kk], x, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.Xi[(16 * bi + 4 * lg + r) * LDX + 16 * bj + li] = -x[r];
    }
    __syncthreads();
  }

  // ---- U = X^(-1) diag(g) Y (fp32 matrix cores): rows of this wave's block,
  //      its part of the value tiles (ct = NVH h + c) ----
  // (per 16-wide k block: the lane's four consecutive k of its row of X^(-1)
  // in one 16-byte read, k = 16 bm + 4 lg + kk in product kk)
  // (every value-column tile advances together: independent accumulators)
  {
    f32x4 acc[NVH];
#pragma unroll
    for (int c = 0; c < NVH; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int bm = 0; bm <= rb; ++bm) {
      const f32x4 a =
          *reinterpret_cast<const f32x4 *>(sm.Xi + (16 * rb + li) * LDX + 16 * bm + 4 * lg);
      float yk[NVH][4];  // Y rows 16 bm + 4 lg .. + 3 of column 16 ct + li
#pragma unroll
      for (int c = 0; c < NVH; ++c)
        lds_col4(yk[c], sm.Ys, LDV, 16 * bm + 4 * lg, 16 * (NVH * h + c), li);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k = 16 * bm + 4 * lg + kk;
        const float gk = sm.gs[k];
#pragma unroll
        for (int c = 0; c < NVH; ++c) {
          const float b = gk * yk[c][kk];
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk], b, acc[c], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NVH; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sm.Us[(16 * rb + 4 * lg + r) * LDV + 16 * (NVH * h + c) + li] = (bf16)acc[c][r];
  }
  __syncthreads();

  // ---- G_i = u_i . D_i (decay; the first part), then dU = P^T dO + D into Ds ----
  if (DECAY && h == 0) {
    const int i = 16 * rb + li;
    float s = 0.f;
    for (int n = lg * (DV / 4); n < (lg + 1) * (DV / 4); ++n)
      s = fmaf((float)sm.Us[i * LDV + n], (float)sm.Ds[i * LDV + n], s);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (lg == 0) sm.Gi[i] = s;
  }
  f32x4 du[NVH];
#pragma unroll
  for (int c = 0; c < NVH; ++c) {
    float x[4];
    lds_col4(x, sm.Ds, LDV, 16 * rb + 4 * lg, 16 * (NVH * h + c), li);
#pragma unroll
    for (int r = 0; r < 4; ++r) du[c][r] = x[r];
  }
#pragma unroll
  for (int ks = 0; ks < C / 32; ++ks) {
    if (32 * ks + 31 < 16 * rb) continue;  // P[j][i] = 0 for j < i
    Frag<bf16> pf;
    lds_frag_tr(pf, sm.Pb, LDC, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * rb, li);
#pragma unroll
    for (int c = 0; c < NVH; ++c) {
      Frag<bf16> of;
      lds_frag_tr(of, sm.dOs, LDV, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * (NVH * h + c),
                  li);
      mma(du[c], pf, of);
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NVH; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sm.Ds[(16 * rb + 4 * lg + r) * LDV + 16 * (NVH * h + c) + li] = (bf16)du[c][r];
  __syncthreads();

  RecRegs<DK, DV> srec;  // S- of the chunk, staged after this phase
  srec.load(rS, dv);
  // ---- lam = X^(-T) dU and r = Y - L U (same tiles); dg_j = lam_j . r_j ----
  {
    f32x4 lam[NVH];
#pragma unroll
    for (int c = 0; c < NVH; ++c) lam[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int k0 = 16 * rb; k0 < C; k0 += 4) {
      const float a = sm.Xi[(k0 + lg) * LDX + 16 * rb + li];
#pragma unroll
      for (int c = 0; c < NVH; ++c) {
        const float b = (float)sm.Ds[(k0 + lg) * LDV + 16 * (NVH * h + c) + li];
        lam[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, lam[c], 0, 0, 0);
      }
    }
    float dgp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks) {
      if (32 * ks > 16 * rb + 15) continue;  // L[i][j] = 0 for j >= i
      Frag<bf16> lf;
      lds_frag(lf, sm.Lb + (16 * rb + li) * LDC + 32 * ks + 8 * lg);
#pragma unroll
      for (int c = 0; c < NVH; ++c) {
        Frag<bf16> uf;
        lds_frag_tr(uf, sm.Us, LDV, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * (NVH * h + c),
                    li);
        f32x4 lu = {0.f, 0.f, 0.f, 0.f};
        mma(lu, lf, uf);
#pragma unroll
        for (int r = 0; r < 4; ++r) dgp[r] = fmaf(-lam[c][r], lu[r], dgp[r]);
      }
    }
#pragma unroll
    for (int c = 0; c < NVH; ++c) {
      float y[4];
      lds_col4(y, sm.Ys, LDV, 16 * rb + 4 * lg, 16 * (NVH * h + c), li);
#pragma unroll
      for (int r = 0; r < 4; ++r) dgp[r] = fmaf(lam[c][r], y[r], dgp[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = sum16(dgp[r]);
      if (li == 0) sm.dgp[h][16 * rb + 4 * lg + r] = s;
    }
  }
  __syncthreads();
  if (tid < Lc) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kGSplit; ++w) s += sm.dgp[w][tid];
    p.dg[(size_t)bh * N + c0 + tid] = s;
  }

  // ---- dP = dO U^T, -dY U^T (lower tiles): P's and L's gradients, the
  //      decay's row/column sums; Pb <- dP (.) Mb, Lb <- G + G^T.  The
  //      chunk's S- goes to the Ys / Ds tiles meanwhile (no longer read) ----
  bf16 *const Sm = sm.Ys;  // S-^T [DV][DK], stride LDK, over Ys and then Ds
  static_assert(DV * LDK <= 2 * C * LDV, "S- fits the Y and D tiles");
  srec.stage(Sm, LDK);
  RecRegs<DK, DV> arec;  // Sh+ of the chunk, staged for the dK phase
  arec.load(rA, dv);
  {
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    for (int tj = h; tj <= rb; tj += kGSplit) {
      f32x4 dp = {0.f, 0.f, 0.f, 0.f}, dl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DV / 32; ++ks) {
        Frag<bf16> of, yf, uf;
        lds_frag(of, sm.dOs + (16 * rb + li) * LDV + 32 * ks + 8 * lg);
        lds_frag(yf, sm.dYs + (16 * rb + li) * LDV + 32 * ks + 8 * lg);
        lds_frag(uf, sm.Us + (16 * tj + li) * LDV + 32 * ks + 8 * lg);
        mma(dp, of, uf);
        mma(dl, yf, uf);
      }
      // lane: rows i = 16 rb + 4 lg + r, column j = 16 tj + li
      const int j = 16 * tj + li;
      float cs = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * rb + 4 * lg + r;
        const float db = DECAY ? __expf(sm.lb[i] - sm.lb[min(j, i)]) : 1.f;
        const float pv = j <= i ? (float)sm.Pb[i * LDC + j] : 0.f;
        const float lv = j < i ? (float)sm.Lb[i * LDC + j] : 0.f;
        const float pg = j <= i ? dp[r] * db : 0.f;
        const float gv = j < i ? -dl[r] * db : 0.f;
        if constexpr (DECAY) {
          const float e = (j <= i ? dp[r] * pv : 0.f) + (j < i ? -dl[r] * lv : 0.f);
          rs[r] += e;
          cs += e;
        }
        // own lower-triangle element (read above), and G's mirror above the
        // diagonal (no lane reads or writes it otherwise)
        if (j <= i) {
          sm.Pb[i * LDC + j] = (bf16)pg;
          sm.Lb[i * LDC + j] = (bf16)gv;
        }
        if (j < i) sm.Lb[j * LDC + i] = (bf16)gv;
      }
      if constexpr (DECAY) {
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
        if (lg == 0) sm.dlb[wv][j] -= cs;
      }
    }
    if constexpr (DECAY) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = sum16(rs[r]);
        if (li == 0) sm.dlb[wv][16 * rb + 4 * lg + r] += s;
      }
    }
  }
  __syncthreads();

  bf16 *dqo = reinterpret_cast<bf16 *>(p.dq) + bh * qk;
  bf16 *dko = reinterpret_cast<bf16 *>(p.dk) + bh * qk;
  // dQ, then dK rows staged in the X^(-1) tile (no longer read), then
  // stored as whole rows
  bf16 *const Gst = reinterpret_cast<bf16 *>(sm.Xi);
  static_assert(sizeof(sm.Xi) >= sizeof(bf16) * C * LDK, "gradient rows fit the X tile");
  // ---- dQ = diag(b) dO S-^T + (dP (.) Mb) K; d log b_i += b_i q_i . (dO S-^T)_i ----
  {
    float da[4] = {0.f, 0.f, 0.f, 0.f};
    Frag<bf16> ofr[DV / 32], pfr[C / 32];  // this wave's rows of dO and of dP (.) Mb
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks)
      lds_frag(ofr[ks], sm.dOs + (16 * rb + li) * LDV + 32 * ks + 8 * lg);
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks)
      lds_frag(pfr[ks], sm.Pb + (16 * rb + li) * LDC + 32 * ks + 8 * lg);
#pragma unroll 2
    for (int tf = NFH * h; tf < NFH * (h + 1); ++tf) {
      f32x4 t1 = {0.f, 0.f, 0.f, 0.f}, t2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DV / 32; ++ks) {
        Frag<bf16> sf;
        lds_frag_tr(sf, Sm, LDK, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * tf, li);
        mma(t1, ofr[ks], sf);
      }
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        if (32 * ks > 16 * rb + 15) continue;
        Frag<bf16> kf;
        lds_frag_tr(kf, sm.Ks, LDK, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * tf, li);
        mma(t2, pfr[ks], kf);
      }
      const int f = 16 * tf + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * rb + 4 * lg + r;
        const float b = DECAY ? __expf(sm.lb[i]) : 1.f;
        if (DECAY) da[r] = fmaf(b * t1[r], (float)sm.Qs[i * LDK + f], da[r]);
        Gst[i * LDK + f] = (bf16)fmaf(b, t1[r], t2[r]);
      }
    }
    if constexpr (DECAY) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = sum16(da[r]);
        if (li == 0) sm.dlb[wv][16 * rb + 4 * lg + r] += s;
      }
    }
    __syncthreads();
    tile_store<VK>(Gst, LDK, DK, dqo, c0, Lc, d);
  }
  // ---- dK = (dP (.) Mb)^T Q - diag(b) dY S-^T + diag(beta / b) U Sh+^T + (G + G^T) K;
  //      d log b_j -= b_j k_j . (dY S-^T)_j.  Sh+ goes to the dO and dY
  //      tiles (no longer read once the dY rows are in registers); beta
  //      <Sh+, S-> alongside ----
  bf16 *const Shs = sm.dOs;  // Sh+^T [DV][DK], stride LDK, over dOs and then dYs
  static_assert(offsetof(SmemGrad<G>, dYs) == offsetof(SmemGrad<G>, dOs) + sizeof(sm.dOs),
                "the dO and dY tiles are adjacent");
  float shs = 0.f;  // this thread's part of <Sh+, S->
  {
    float da[4] = {0.f, 0.f, 0.f, 0.f};
    // this wave's rows j of (G + G^T), of (dP (.) Mb)^T, of dY and of U
    Frag<bf16> gfr[C / 32], ptr_[C / 32], yfr[DV / 32], ufr[DV / 32];
#pragma unroll
    for (int ks = 0; ks < C / 32; ++ks) {
      lds_frag(gfr[ks], sm.Lb + (16 * rb + li) * LDC + 32 * ks + 8 * lg);
      lds_frag_tr(ptr_[ks], sm.Pb, LDC, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * rb, li);
    }
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks) {
      lds_frag(yfr[ks], sm.dYs + (16 * rb + li) * LDV + 32 * ks + 8 * lg);
      lds_frag(ufr[ks], sm.Us + (16 * rb + li) * LDV + 32 * ks + 8 * lg);
    }
    __syncthreads();  // dQ's rows are out of the X tile, every wave has its dY rows
    arec.stage(Shs, LDK);
    __syncthreads();
    if constexpr (DECAY) {
      for (int e = tid; e < DV * (DK / 8); e += kGThreads) {
        const int row = e / (DK / 8), f0 = (e % (DK / 8)) * 8;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Shs + row * LDK + f0);
        const bf16x8 b = *reinterpret_cast<const bf16x8 *>(Sm + row * LDK + f0);
#pragma unroll
        for (int m = 0; m < 8; ++m) shs = fmaf((float)a[m], (float)b[m], shs);
      }
    }
    for (int tf = NFH * h; tf < NFH * (h + 1); ++tf) {
      f32x4 t1 = {0.f, 0.f, 0.f, 0.f}, t2 = {0.f, 0.f, 0.f, 0.f}, t3 = {0.f, 0.f, 0.f, 0.f},
            t4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        Frag<bf16> kf;
        lds_frag_tr(kf, sm.Ks, LDK, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * tf, li);
        mma(t4, gfr[ks], kf);
        if (32 * ks + 31 < 16 * rb) continue;  // dP (.) Mb [i][j] = 0 for i < j
        Frag<bf16> qf;
        lds_frag_tr(qf, sm.Qs, LDK, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * tf, li);
        mma(t1, ptr_[ks], qf);
      }
#pragma unroll
      for (int ks = 0; ks < DV / 32; ++ks) {
        Frag<bf16> sf, hf;
        lds_frag_tr(sf, Sm, LDK, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * tf, li);
        lds_frag_tr(hf, Shs, LDK, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * tf, li);
        mma(t2, yfr[ks], sf);
        mma(t3, ufr[ks], hf);
      }
      const int f = 16 * tf + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * rb + 4 * lg + r;
        const float b = DECAY ? __expf(sm.lb[j]) : 1.f;
        const float wl = DECAY ? __expf(lbeta - sm.lb[j]) : 1.f;
        if (DECAY) da[r] = fmaf(-b * t2[r], (float)sm.Ks[j * LDK + f], da[r]);
        const float g = t1[r] - b * t2[r] + wl * t3[r] + t4[r];
        Gst[j * LDK + f] = (bf16)g;
      }
    }
    if constexpr (DECAY) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = sum16(da[r]);
        if (li == 0) sm.dlb[wv][16 * rb + 4 * lg + r] += s;
      }
    }
    __syncthreads();
    tile_store<VK>(Gst, LDK, DK, dko, c0, Lc, d);
  }
  if constexpr (DECAY) {
    float s = shs;  // beta <Sh+, S-> over the chunk's records
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) s += __shfl_xor(s, o);
    float *const red = &sm.dgp[0][0];
    static_assert(sizeof(sm.dgp) >= kGWaves * sizeof(float), "one slot per wave");
    if (lane == 0) red[wv] = s;
    __syncthreads();
    if (wv == 0) {
      // d log b_j for the chunk's tokens (lane j), then d log alpha_t as the
      // suffix sums, dalpha = d log alpha / alpha
      const int j = lane;
      float x = -sm.Gi[j], shsum = 0.f;
#pragma unroll
      for (int w = 0; w < kGWaves; ++w) {
        x += sm.dlb[w][j];
        shsum += red[w];
      }
      float gsum = sm.Gi[j];
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) gsum += __shfl_xor(gsum, o);
      const float dlbeta = __expf(lbeta) * shsum + gsum;
      if (j == Lc - 1) x += dlbeta;
      if (j >= Lc) x = 0.f;
      // suffix sum: sum over j' >= j
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const float y = __shfl_down(x, o);
        if (j + o < kWave) x += y;
      }
      if (j < Lc) p.dalpha[(size_t)bh * N + c0 + j] = x / sm.al[j];
    }
  }
}

template <class CF, class G, bool VK, bool DECAY>
hipError_t run_bwd(const BwdDeltaParams &bp, const PrefillParams &pp, hipStream_t s) {
  static_assert(sizeof(SmemGrad<G>) <= 160 * 1024, "LDS budget (gradient kernel)");
  static_assert(sizeof(SmemBRev<CF>) <= 160 * 1024, "LDS budget (reverse pass)");
  const int nch = bp.nch;
  hipError_t e = launch_kernel("delta_bwd_prep", prep_kernel<CF, VK, DECAY, true>,
                               head_grid(nch, bp.BH), dim3(kThreads), s, pp);
  if (e != hipSuccess) return e;
  const int nsl = (bp.dv + 15) / 16;
  const int xcd_map = (bp.BH % kXcds) == 0;
  e = launch_kernel("delta_bwd_state", bstate_kernel<CF, VK, DECAY>, dim3(bp.BH * nsl),
                    dim3(kThreads), s, bp, nsl, xcd_map);
  if (e != hipSuccess) return e;
  constexpr int NWR = CF::NFT >= 8 ? 8 : 4;  // the reverse pass's waves
  e = launch_kernel("delta_bwd_rev", brev_kernel<CF, VK, DECAY, NWR>, dim3(bp.BH * nsl),
                    dim3(NWR * kWave), s, bp, nsl, xcd_map);
  if (e != hipSuccess) return e;
  return launch_kernel("delta_bwd_grad", bgrad_kernel<G, VK, DECAY>, head_grid(nch, bp.BH),
                       dim3(kGThreads), s, bp);
}

template <class CF, int DV>
hipError_t run_bwd_dv(const BwdDeltaParams &bp, const PrefillParams &pp, hipStream_t s) {
  using G = GCfg<CF::DK, DV>;
  if (bp.vec_ok)
    return bp.alpha ? run_bwd<CF, G, true, true>(bp, pp, s) : run_bwd<CF, G, true, false>(bp, pp, s);
  return bp.alpha ? run_bwd<CF, G, false, true>(bp, pp, s) : run_bwd<CF, G, false, false>(bp, pp, s);
}

}  // namespace

BwdDeltaSizes delta_backward_sizes(int BH, int N, int d, int dv) {
  BwdDeltaSizes z{};
  const int dvp = dv <= 64 ? 64 : 128;
  const BwdDeltaLayout L = d <= 64 ? bwd_delta_layout<DB64>(BH, N, dvp)
                                   : bwd_delta_layout<DB128>(BH, N, dvp);
  z.bytes = L.bytes;
  z.dvp = dvp;
  z.nch = (N + 63) / 64;
  z.dec = L.dec;
  z.states = L.states;
  z.adj = L.adj;
  z.y = L.y;
  z.dd = L.dd;
  return z;
}

hipError_t launch_delta_backward(const BwdDeltaParams &bp, hipStream_t s) {
  PrefillParams pp{};  // the preparation kernel's view of the inputs
  pp.BH = bp.BH;
  pp.H = bp.H;
  pp.N = bp.N;
  pp.d = bp.d;
  pp.dv = bp.dv;
  pp.q = bp.q;
  pp.k = bp.k;
  pp.v = bp.v;
  pp.g = bp.g;
  pp.alpha = bp.alpha;
  pp.ws = reinterpret_cast<float *>(bp.ws);
  if (bp.d <= 64)
    return bp.dvp == 64 ? run_bwd_dv<DB64, 64>(bp, pp, s) : run_bwd_dv<DB64, 128>(bp, pp, s);
  return bp.dvp == 64 ? run_bwd_dv<DB128, 64>(bp, pp, s) : run_bwd_dv<DB128, 128>(bp, pp, s);
}

}  // namespace la
