// Chunked prefill for the LINEAR rule (elu+1 kernel, per-head decay, eps).
//
// Method ("What Is Linear Attention?" sections 2, 4, 5.1; "Efficient
// attention variants" sections 5, 7.1, 8; "Transformers Are RNNs"):
//     S_t = gamma S_{t-1} + phi(k_t) v_t^T,  z_t = gamma z_{t-1} + phi(k_t)
//     o_t = phi(q_t)^T S_t / (phi(q_t) . z_t + eps)
// evaluated chunk by chunk (the pages' chunkwise form: parallel inside a
// chunk, state passed between chunks).  For a chunk of L tokens entering with
// state (S-, z-), chunk-local indices i, j, unrolling the recurrence gives
//     num_i = gamma^(i+1) phi(q_i) S-  +  sum_{j<=i} gamma^(i-j) (phi(q_i).phi(k_j)) v_j
//     den_i = gamma^(i+1) phi(q_i).z- +  sum_{j<=i} gamma^(i-j) (phi(q_i).phi(k_j))  + eps
//     S+    = gamma^L S- + sum_j gamma^(L-1-j) phi(k_j) v_j^T   (z+ likewise)
// and o_i = num_i / den_i.  Every decay factor there is a power gamma^m with
// m >= 0, and each is applied where it occurs: the scores take gamma^(i-j)
// after their product (one exponential per four scores of a lane, gamma^e
// times the constants gamma^-r, r < 4), the state read gamma^(i+1) per query
// row (one value per lane: each lane holds one token), and the key fragments
// of the state update gamma^(L-1-j) per token.  No factor exceeds 1, so
// nothing overflows for any gamma in (0, 1]; a factor that underflows stands
// for a contribution far below fp32 resolution next to the token's own.
// log2 gamma is clamped at -40, which keeps gamma^-3 finite (below
// gamma = 2^-40 every earlier token then weighs under 2^-40 of its own).
// The segment summaries only accumulate the state, with weighted keys
// kw_j = gamma^(L-1-j) phi(k_j): S+ = gamma^L S- + KW^T V.
//
// The normaliser rides along as one more 16-column tile of the value side:
// the state is kept as [S | z z ... z] (z replicated over 16 columns) and V
// is extended by a tile of ones, so one matrix product gives numerator and
// denominator together.  Outputs are computed transposed (O^T = S'^T Phi_q^T
// + V'^T A^T), which gives each lane four consecutive output columns of one
// token and the denominator of that same token.
//
// LDS tiles are all row-major: Phi_q, Phi_k and V rows as loaded (16-byte
// stores), the state copy S'^T (value columns + normaliser rows by
// features), and an output staging tile.  Token contractions (A V and
// Phi_k^T V) read transposed fragments with the gfx950 LDS transpose load, so
// no tile is ever written transposed.  Scores are computed transposed (Phi_k
// as the A operand, Phi_q as B), which leaves in each lane one query row and
// four consecutive keys: two such tiles form the A^T operand of the next
// product straight from registers.  The fp32 state lives in matrix-core
// accumulators and is never rounded; its bf16 copy feeds the next chunk's
// read.
//
// Long sequences are split into segments processed in parallel (a two-level
// scan, "Transformers Are RNNs": the recurrence is a prefix sum):
//   summary_kernel  per (segment, head), all but the last segment: the
//                   segment's own contribution (dS, dz), i.e. the state
//                   update from a zero state;
//   scan_kernel     per head: P_0 = (S_in, z_in), P_s = gamma^Lseg P_(s-1)
//                   + dS_(s-1), every record loaded before the chain;
//   chunk_kernel    per (segment, head): outputs from P_s, chunk by chunk;
//                   the last segment writes (S_out, z_out).
// With one segment only chunk_kernel runs, from (S_in, z_in).
//
// Per-key-channel decay (GLA, "Efficient attention variants" 7.2; the CH
// instantiations): S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T, z alike.
// With lb_j = sum_{t<=j} log2 alpha_t (chunk-local, per channel), the score
// of query j and key i <= j is sum_f phi(q_j)_f phi(k_i)_f 2^(lb_j - lb_i)_f.
// Each 16-token block b of the chunk has references R_b = lb before it (0
// for the first), M_b = lb at its eighth token and E_b = lb at its last, and
// the tiles hold
//     q^_j = phi(q_j) (.) 2^(lb_j - M_b(j)),   k^_i = phi(k_i) (.) 2^(M_b(i) - lb_i),
// every factor within alpha^(-8).  A diagonal score tile is q^ . k^ as it
// stands.  Elsewhere every product is taken as a chain of factors that each
// stay in range, so that a factor can underflow only where the weight it
// belongs to is negligible: the query side of a tile of query block r
// against key block b < r is (q^ (.) 2^(M_r - R_r)) (.) 2^(R_r - E_b) (the
// second factor only for b < r-1: R_r = E_(r-1)), the key side k^ (.)
// 2^(E_b - M_b); the state read takes (q^ (.) 2^(M_r - R_r)) (.) 2^R_r against
// the plain state copy; and the state update is S+ = diag(2^lb_L) S- +
// sum_i ((k^_i (.) 2^(E_b - M_b)) (.) 2^(lb_L - E_b)) v_i^T (z alike).  The
// range argument needs alpha^(-8) finite: log2 alpha is clamped at -15
// (alpha at least 2^-15; below it an earlier token already weighs under
// 2^-15 of the current one).  The prefix sums are taken per chunk in fp64
// (one thread per channel) and stored relative to each row's reference, so
// the exponents keep fp32 accuracy however long the decay has run; a
// segment summary weights its keys by 2^(lb_L - lb_i) (reference L for every
// row) and also carries the segment's total log2 decay per channel, which
// the scan applies row by row.
//
// Data layout: q, k [BH, N, d], v, o [BH, N, dv] (row-major, dtype T);
// alpha [BH, N, d] fp32 (CH); workspace slots [nseg][BH][d*dv + 2d] fp32
// (state transposed, element (f, n) at n d + f; normaliser; then the
// segment's log2 decay per channel for CH).
// Global traffic goes through buffer resources (bounds by offset, no
// branches between a load and its use), issued one chunk ahead.
#include <atomic>
#include <type_traits>

#include "la_common.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kLdsBytes = 160 * 1024;
constexpr size_t kStreamBytes = (size_t)256 << 20;  // last-level (MALL) cache size
constexpr int kMaxSeg = 32;  // most segments per sequence

// fp32 elements of one workspace slot record: S (d x dv), z (d), and the
// segment's log2 decay per channel (d; used with a per-channel decay).
__host__ __device__ inline size_t ws_rec(int d, int dv) {
  return (size_t)d * dv + 2 * (size_t)d;
}

template <typename T, int DK_, int DV_, int C_, int NW_>
struct Cfg {
  using type = T;
  using vec = typename Vec16<T>::type;
  static constexpr int DK = DK_, DV = DV_, C = C_, NW = NW_;
  static constexpr int NT = NW * kWave;
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte vector
  static constexpr int QLD = DK + VEC;  // row strides: Qs, Ks, St
  static constexpr int KLD = DK + VEC;
  static constexpr int SLD = DK + VEC;
  static constexpr int VLD = DV + VEC;  // row stride: Os
  // row stride of Vs, read only through transpose loads: 8 consecutive rows
  // of 32 bytes then fall in distinct LDS banks
  static constexpr int VTLD = sizeof(T) == 2 ? DV + 16 : DV + 4;
  static constexpr int NRB = C / 16;    // 16-token row blocks of a chunk
  static constexpr int NG = NW / NRB;   // waves per row block (output role)
  static constexpr int NVT = DV / 16;   // value column tiles
  static constexpr int NPW = NVT / NG;  // value tiles per wave (output role)
  static constexpr int NCT = NVT + 1;   // state column tiles incl. the normaliser
  static constexpr int NFT = DK / 16;   // state row tiles
  static constexpr int FPW = NFT >= NW ? NFT / NW : 1;  // state row tiles per wave
  static constexpr int NWC = NFT >= NW ? 1 : NW / NFT;  // state column groups
  static constexpr int TPW = (NCT + NWC - 1) / NWC;     // state column tiles per wave
  static constexpr int KSD = DK / 32;   // k-steps over features
  static constexpr int KSC = C / 32;    // k-steps over tokens
  static constexpr int QCB = DK / VEC;  // 16-byte blocks per q/k row
  static constexpr int VCB = DV / VEC;  // ... per v/o row
  static constexpr int RQ = C * DK / (VEC * NT);  // q/k rows per thread
  static constexpr int RV = C * DV / (VEC * NT);  // v/o rows per thread
  static constexpr int SROWS = DV + 1;  // rows of the S'^T copy (z once: row DV)
  // resident waves per SIMD the register allocation must allow
  static constexpr int WPE = sizeof(T) == 4 ? 1 : (NW <= 4 ? 3 : 2);
  // chunks whose k, v rows summary_kernel keeps in flight: eight-wave bf16
  // workgroups (d or dv of 128) run at most one per CU on long sequences,
  // where a second chunk in flight measured 6% faster; four-wave ones keep
  // one (a deeper prefetch measured slower there).
  static constexpr int PD = (sizeof(T) == 2 && NW == 8) ? 2 : 1;
  static_assert(NG >= 1 && NPW >= 1 && NPW * NG == NVT, "output tiling");
  static_assert(FPW * NW == NFT || NWC * NFT == NW, "state tiling");
  static_assert(NRB % 2 == 0, "chunk must hold an even number of row blocks");
  static_assert(RQ >= 1 && RQ * VEC * NT == C * DK, "q/k rows per thread");
  static_assert(RV >= 1 && RV * VEC * NT == C * DV, "v/o rows per thread");
};

template <class CF>
struct alignas(16) SmemChunk {
  using T = typename CF::type;
  T Qs[CF::C * CF::QLD];      // phi(q) rows
  T Ks[CF::C * CF::KLD];      // weighted phi(k) rows
  T Vs[CF::C * CF::VTLD];     // v rows
  T St[CF::SROWS * CF::SLD];  // gamma^L [S | z]^T for the next state read
  T Os[CF::C * CF::VLD];      // output staging
  float pw[CF::C + 4];        // gamma^m, m = 0..C (decay folded into key weights)
};

template <class CF>
struct alignas(16) SmemSummary {
  using T = typename CF::type;
  T Ks[CF::C * CF::KLD];
  T Vs[CF::C * CF::VTLD];
  float pw[CF::C + 4];
};

// This thread's rows of one chunk, as loaded (raw 16-byte vectors).
template <class CF>
struct ChunkRegs {
  typename CF::vec q[CF::RQ], k[CF::RQ], v[CF::RV];
};

// Per-key-channel decay (CH): this thread's alpha values for its q/k rows
// (VEC channels per row), and the LDS of one chunk's prefix sums.
template <class CF>
struct ChanRegs {
  f32x4 a[CF::RQ][CF::VEC / 4];
};

template <class CF>
struct alignas(16) SmemChan {
  static constexpr int LDL = CF::DK + 4;  // row stride of lb
  static constexpr int NRB = CF::NRB;
  static constexpr int NP = (NRB - 1) * (NRB - 2) / 2;  // block pairs b <= r - 2
  // log2 alpha as loaded, then each row's exponent lb_j - ref_j (ref_j =
  // M_b(j) in the chunk kernel, lb_L in the segment summaries)
  float lb[CF::C * LDL];
  float th[NRB][CF::DK], tl[NRB][CF::DK];  // block sums of log2 alpha (fp64 as hi + lo)
  float el[CF::DK];  // 2^lb_L: the chunk's decay of the state
  union {
    struct {  // chunk kernel (the factors of 1 are not stored)
      float qa[NRB][CF::DK];               // 2^(M_r - R_r)
      float cp[NP > 0 ? NP : 1][CF::DK];   // 2^(R_r - E_b), b <= r-2: (r-2)(r-1)/2 + b
      float kb[NRB][CF::DK];               // 2^(E_b - M_b)
      float kf[NRB > 1 ? NRB - 1 : 1][CF::DK];  // 2^(lb_L - E_b), b < NRB-1
      float sf[NRB > 1 ? NRB - 1 : 1][CF::DK];  // 2^R_r, r >= 1: row r - 1
    };
    float tot[CF::DK];  // segment summaries: log2 decay of the segment so far
  };
};
// log2 alpha below this is clamped (alpha >= 2^-15; see the file header)
constexpr float kLog2AlphaMin = -15.f;
struct NoChan {};
template <class CF>
__device__ __forceinline__ const SmemChan<CF> *chan_ptr(const SmemChan<CF> &s) {
  return &s;
}
template <class CF>
__device__ __forceinline__ const SmemChan<CF> *chan_ptr(const NoChan &) {
  return nullptr;
}
template <class CF, bool CH>
using ChanSmem = typename std::conditional<CH, SmemChan<CF>, NoChan>::type;

// Per-head buffer resources of q, k, v and o.
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
// width, so a block is either wholly inside or wholly outside.  NT: a
// non-temporal (streaming) load, for data no later kernel can find in cache.
template <typename T, bool VK, bool NT = false>
__device__ __forceinline__ typename Vec16<T>::type load_block(
    __amdgpu_buffer_rsrc_t r, int tok, int col0, int ncols, bool row_ok) {
  constexpr int VEC = 16 / (int)sizeof(T);
  if constexpr (VK) {
    const bool ok = row_ok && col0 < ncols;
    const uint32_t off = ok ? (uint32_t)(((size_t)tok * ncols + col0) * sizeof(T)) : kOOB;
    if constexpr (NT) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      return __builtin_bit_cast(typename Vec16<T>::type,
                                __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
    }
    return buf_load16<T>(r, off);
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

// alpha rows of a chunk for this thread's q/k rows (zeros outside; they
// become factors of 1 in chan_logs).
template <class CF, bool VK>
__device__ __forceinline__ void chan_prefetch(ChanRegs<CF> &A, __amdgpu_buffer_rsrc_t ra,
                                              const PrefillParams &p, int c0, int Lc) {
  const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
#pragma unroll
  for (int r = 0; r < CF::RQ; ++r) {
    const int row = qrg * CF::RQ + r;
    const size_t t = (size_t)(c0 + row);
#pragma unroll
    for (int h = 0; h < CF::VEC / 4; ++h) {
      const int col = qcb * CF::VEC + 4 * h;
      if constexpr (VK) {
        A.a[r][h] = buf_load16<float>(
            ra, row < Lc && col < p.d ? (uint32_t)((t * p.d + col) * 4) : kOOB);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          A.a[r][h][e] = buf_load1(
              ra, row < Lc && col + e < p.d ? (uint32_t)((t * p.d + col + e) * 4) : kOOB,
              (float *)nullptr);
      }
    }
  }
}

// log2 alpha of this thread's elements into lb (0 for rows past the chunk
// and columns past d, i.e. a factor of 1).
template <class CF>
__device__ __forceinline__ void chan_logs(const ChanRegs<CF> &A, SmemChan<CF> &sc, int d,
                                          int Lc) {
  const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
#pragma unroll
  for (int r = 0; r < CF::RQ; ++r) {
    const int row = qrg * CF::RQ + r;
#pragma unroll
    for (int h = 0; h < CF::VEC / 4; ++h) {
      const int col = qcb * CF::VEC + 4 * h;
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = row < Lc && col + e < d ? fmaxf(__log2f(A.a[r][h][e]), kLog2AlphaMin) : 0.f;
      *reinterpret_cast<f32x4 *>(sc.lb + row * SmemChan<CF>::LDL + col) = x;
    }
  }
}

// Prefix sums of log2 alpha down each column in fp64, one thread per
// (channel, 16-row block): the block's own sums first, then, with every
// block's total at hand, each row's exponent relative to its reference
// written back in place, the state decay el and the factor tables of the
// chunk kernel, or (segment summaries, total) the running log2 decay of the
// segment.  Rows past Lc add factors of 1.  Two barriers: one inside, one
// for the caller after it.
template <class CF>
__device__ __forceinline__ void chan_prefix(SmemChan<CF> &sc, bool total) {
  constexpr int LDL = SmemChan<CF>::LDL, NRB = CF::NRB;
  static_assert(NRB * CF::DK <= CF::NT, "one thread per channel and block");
  const int t = threadIdx.x, f = t % CF::DK, b = t / CF::DK;
  const bool act = b < NRB;
  double loc7 = 0.0;
  if (act) {
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      acc += (double)sc.lb[(16 * b + j) * LDL + f];
      if (j == 7) loc7 = acc;
    }
    const float hi = (float)acc;
    sc.th[b][f] = hi;
    sc.tl[b][f] = (float)(acc - (double)hi);
  }
  __syncthreads();
  if (act) {
    double off = 0.0, x = 0.0, offs[NRB];
#pragma unroll
    for (int c = 0; c < NRB; ++c) {
      const double T = (double)sc.th[c][f] + (double)sc.tl[c][f];
      offs[c] = x;  // R_c: the sum of the blocks before c
      x += T;
      if (c < b) off += T;
    }
    // exponent of row j: lb_j - M_b = (own sums to j) - loc7 in the chunk
    // kernel; lb_j - lb_L = off + (own sums to j) - x in the summaries
    const double ref = total ? x - off : loc7;
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float *cell = sc.lb + (16 * b + j) * LDL + f;
      acc += (double)*cell;
      *cell = (float)(acc - ref);
    }
    if (b == 0) {
      sc.el[f] = exp2f((float)x);  // x = lb[C-1] = lb[Lc-1]
      if (total) sc.tot[f] += (float)x;
    }
    if (!total) {
      const double E = off + (double)sc.th[b][f] + (double)sc.tl[b][f];
      sc.qa[b][f] = exp2f((float)loc7);              // M_b - R_b
      sc.kb[b][f] = exp2f((float)(E - off - loc7));  // E_b - M_b
      if (b + 1 < NRB) sc.kf[b][f] = exp2f((float)(x - E));
      if (b >= 1) sc.sf[b - 1][f] = exp2f((float)off);
#pragma unroll
      for (int c = 0; c + 2 <= NRB - 1; ++c) {  // pairs (b, c), c <= b - 2: R_b - E_c
        if (c + 2 <= b) {
          const double Ec = offs[c] + (double)sc.th[c][f] + (double)sc.tl[c][f];
          sc.cp[(b - 2) * (b - 1) / 2 + c][f] = exp2f((float)(off - Ec));
        }
      }
    }
  }
}

// A fragment's eight values times eight per-channel factors (fp32 product,
// rounded back to the fragment's type).
template <typename T>
__device__ __forceinline__ Frag<T> frag_scaled(const Frag<T> &f, const float *fac) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(fac);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(fac + 4);
  Frag<T> o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o.v[e] = from_f32<T>(to_f32(f.v[e]) * a[e]);
    o.v[4 + e] = from_f32<T>(to_f32(f.v[4 + e]) * b[e]);
  }
  return o;
}

// ---- short causal convolution of q, k, v (the CV instantiations) ----------
// y_t = sum_j w_j x_(t-j') over the last w tokens, per head and channel
// ("What Is Linear Attention?" 5.4).  Fused into the row commit: a chunk's
// raw rows go to LDS, each thread reads the kConvHalo rows before its own
// (the first rows of a chunk find them in a small halo buffer that holds the
// previous chunk's last raw rows), convolves in fp32 and continues with the
// feature map as before.  Filters sit in LDS as a table of kConvTaps rows,
// aligned so that the last row multiplies the current token; rows for taps
// past the filter width and columns past d / dv are zero.
constexpr int kConvTaps = 4;              // widest filter
constexpr int kConvHalo = kConvTaps - 1;  // raw rows a chunk needs from before it

template <class CF>
struct alignas(16) SmemConv {
  using T = typename CF::type;
  static constexpr int WLD = 2 * CF::DK + CF::DV;  // table row: [q | k | v] columns
  float w[kConvTaps * WLD];
  T hq[kConvHalo * CF::QLD];  // the raw rows before the chunk, oldest first
  T hk[kConvHalo * CF::QLD];
  T hv[kConvHalo * CF::VLD];
};
struct NoConv {};
template <class CF, bool CV>
using ConvSmem = typename std::conditional<CV, SmemConv<CF>, NoConv>::type;
template <class CF>
__device__ __forceinline__ SmemConv<CF> *conv_ptr(SmemConv<CF> &s) {
  return &s;
}
template <class CF>
__device__ __forceinline__ SmemConv<CF> *conv_ptr(NoConv &) {
  return nullptr;
}

// Filter table, and the kConvHalo raw rows before token t0: from q, k, v,
// or, before the sequence, from the cache `src` (this head's w-1 rows of
// [q | k | v], oldest first; zeros if null).  `copy`, if set, receives the
// cache rows read (so that a later kernel may read them while the cache
// itself is overwritten).
template <class CF>
__device__ void conv_init(SmemConv<CF> &cs, const PrefillParams &p, int bh, int t0,
                          const typename CF::type *src, typename CF::type *copy) {
  using T = typename CF::type;
  constexpr int WLD = SmemConv<CF>::WLD;
  const int d = p.d, dv = p.dv, w = p.conv_width, wc = 2 * d + dv;
  const float *W = p.conv_w + (size_t)(bh % p.H) * w * wc;
  const T *x[3] = {reinterpret_cast<const T *>(p.q) + (size_t)bh * p.N * d,
                   reinterpret_cast<const T *>(p.k) + (size_t)bh * p.N * d,
                   reinterpret_cast<const T *>(p.v) + (size_t)bh * p.N * dv};
  for (int i = threadIdx.x; i < kConvHalo * WLD + kConvTaps * WLD; i += CF::NT) {
    const bool is_w = i >= kConvHalo * WLD;
    const int i2 = is_w ? i - kConvHalo * WLD : i;
    const int row = i2 / WLD, c = i2 % WLD;
    // tensor (0 q, 1 k, 2 v), its column and width, and the channel in [q | k | v]
    const int tsr = c < CF::DK ? 0 : c < 2 * CF::DK ? 1 : 2;
    const int col = c - tsr * CF::DK;
    const int width = tsr == 2 ? dv : d;
    const int ch = tsr * d + col;
    if (is_w) {
      const int tap = row - (kConvTaps - w);
      cs.w[i2] = (col < width && tap >= 0) ? W[(size_t)tap * wc + ch] : 0.f;
      continue;
    }
    const int tok = t0 - kConvHalo + row;
    T val = from_f32<T>(0.f);
    if (col < width) {
      if (tok >= 0) {
        val = x[tsr][(size_t)tok * width + col];
      } else if (src && tok >= 1 - w) {
        val = src[(size_t)(tok + w - 1) * wc + ch];
        if (copy) copy[(size_t)(tok + w - 1) * wc + ch] = val;
      }
    }
    T *h = tsr == 0 ? cs.hq : tsr == 1 ? cs.hk : cs.hv;
    h[row * (tsr == 2 ? CF::VLD : CF::QLD) + col] = val;
  }
}

// Convolved rows row0 .. row0+NR-1 at columns col0 .. col0+VEC-1 of one
// tensor: the NR rows this thread loaded (`own`) and the kConvHalo rows
// before them, read from the raw rows in LDS (`raw`, stride ld) or, before
// the chunk, from the halo buffer (stride hld).
template <class CF, int NR>
__device__ __forceinline__ void conv_rows(float (&y)[NR][CF::VEC],
                                          const typename CF::vec (&own)[NR],
                                          const typename CF::type *raw, int ld,
                                          const typename CF::type *halo, int hld, int row0,
                                          int col0, const float *wt) {
  using T = typename CF::type;
  using V = typename CF::vec;
  constexpr int VEC = CF::VEC;
  float win[NR + kConvHalo][VEC];
#pragma unroll
  for (int h = 0; h < kConvHalo; ++h) {
    const int r = row0 - kConvHalo + h;
    const T *src = r >= 0 ? raw + r * ld + col0 : halo + (r + kConvHalo) * hld + col0;
    const V x = *reinterpret_cast<const V *>(src);
#pragma unroll
    for (int e = 0; e < VEC; ++e) win[h][e] = to_f32(x[e]);
  }
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) win[kConvHalo + i][e] = to_f32(own[i][e]);
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[i][e] = 0.f;
#pragma unroll
  for (int j = 0; j < kConvTaps; ++j) {
    float wj[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) wj[e] = wt[j * SmemConv<CF>::WLD + col0 + e];
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[i][e] = fmaf(wj[e], win[i + j][e], y[i][e]);
  }
}

// This thread's convolved rows (fp32), and its final rows as they go to LDS
// once every thread has read its window.
template <class CF, bool WITH_Q>
struct ConvOut {
  float q[WITH_Q ? CF::RQ : 1][CF::VEC];
  float k[CF::RQ][CF::VEC];
  float v[CF::RV][CF::VEC];
};
template <class CF, bool WITH_Q>
struct ConvRows {
  typename CF::vec q[WITH_Q ? CF::RQ : 1], k[CF::RQ], v[CF::RV];
};
template <class CF>
__device__ __forceinline__ typename CF::vec pack_vec(const float (&x)[CF::VEC]) {
  typename CF::vec v;
#pragma unroll
  for (int e = 0; e < CF::VEC; ++e) v[e] = from_f32<typename CF::type>(x[e]);
  return v;
}

// Convolve this thread's rows of the chunk.  The raw rows are staged in
// Qs / Ks / Vs (a barrier, then each thread reads its window); the caller
// overwrites them with the final rows after a second barrier.
template <class CF, bool WITH_Q>
__device__ __forceinline__ void conv_gather(ConvOut<CF, WITH_Q> &Y, const ChunkRegs<CF> &R,
                                            typename CF::type *Qs, typename CF::type *Ks,
                                            typename CF::type *Vs, const SmemConv<CF> &cs) {
  using V = typename CF::vec;
  const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
  const int vcb = threadIdx.x % CF::VCB, vrg = threadIdx.x / CF::VCB;
  const int qc0 = qcb * CF::VEC, vc0 = vcb * CF::VEC;
#pragma unroll
  for (int r = 0; r < CF::RQ; ++r) {
    const int row = qrg * CF::RQ + r;
    if constexpr (WITH_Q) *reinterpret_cast<V *>(Qs + row * CF::QLD + qc0) = R.q[r];
    *reinterpret_cast<V *>(Ks + row * CF::KLD + qc0) = R.k[r];
  }
#pragma unroll
  for (int r = 0; r < CF::RV; ++r)
    *reinterpret_cast<V *>(Vs + (vrg * CF::RV + r) * CF::VTLD + vc0) = R.v[r];
  __syncthreads();
  if constexpr (WITH_Q)
    conv_rows<CF, CF::RQ>(Y.q, R.q, Qs, CF::QLD, cs.hq, CF::QLD, qrg * CF::RQ, qc0, cs.w);
  conv_rows<CF, CF::RQ>(Y.k, R.k, Ks, CF::KLD, cs.hk, CF::QLD, qrg * CF::RQ, qc0,
                        cs.w + CF::DK);
  conv_rows<CF, CF::RV>(Y.v, R.v, Vs, CF::VTLD, cs.hv, CF::VLD, vrg * CF::RV, vc0,
                        cs.w + 2 * CF::DK);
}

// After the second barrier: the chunk's last kConvHalo raw rows become the
// next chunk's halo.
template <class CF>
__device__ __forceinline__ void conv_halo(const ChunkRegs<CF> &R, SmemConv<CF> &cs,
                                          bool with_q) {
  using V = typename CF::vec;
  const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
  const int vcb = threadIdx.x % CF::VCB, vrg = threadIdx.x / CF::VCB;
  const int qc0 = qcb * CF::VEC, vc0 = vcb * CF::VEC;
#pragma unroll
  for (int r = 0; r < CF::RQ; ++r) {
    const int h = qrg * CF::RQ + r - (CF::C - kConvHalo);
    if (h >= 0) {
      if (with_q) *reinterpret_cast<V *>(cs.hq + h * CF::QLD + qc0) = R.q[r];
      *reinterpret_cast<V *>(cs.hk + h * CF::QLD + qc0) = R.k[r];
    }
  }
#pragma unroll
  for (int r = 0; r < CF::RV; ++r) {
    const int h = vrg * CF::RV + r - (CF::C - kConvHalo);
    if (h >= 0) *reinterpret_cast<V *>(cs.hv + h * CF::VLD + vc0) = R.v[r];
  }
}

// The cache after the sequence: its last w-1 raw tokens (from the cache
// before it when the sequence is shorter).  Every value is loaded before
// the barrier and stored after it, so conv_out may alias conv_in.
template <class CF>
__device__ void conv_final(const PrefillParams &p, int bh) {
  using T = typename CF::type;
  const int d = p.d, dv = p.dv, N = p.N, w = p.conv_width, wc = 2 * d + dv;
  const int n = (w - 1) * wc;
  constexpr int MAXE = (kConvHalo * 3 * LA_MAXD + CF::NT - 1) / CF::NT;
  const T *in = p.conv_in ? reinterpret_cast<const T *>(p.conv_in) + (size_t)bh * n : nullptr;
  const T *x[3] = {reinterpret_cast<const T *>(p.q) + (size_t)bh * N * d,
                   reinterpret_cast<const T *>(p.k) + (size_t)bh * N * d,
                   reinterpret_cast<const T *>(p.v) + (size_t)bh * N * dv};
  T val[MAXE];
#pragma unroll
  for (int m = 0; m < MAXE; ++m) {
    const int i = threadIdx.x + m * CF::NT;
    val[m] = from_f32<T>(0.f);
    if (i < n) {
      const int row = i / wc, ch = i % wc;
      const int tok = N - (w - 1) + row;
      const int tsr = ch < d ? 0 : ch < 2 * d ? 1 : 2;
      const int col = ch - tsr * d, width = tsr == 2 ? dv : d;
      if (tok >= 0) val[m] = x[tsr][(size_t)tok * width + col];
      else if (in) val[m] = in[(size_t)(tok + w - 1) * wc + ch];
    }
  }
  __syncthreads();
  T *out = reinterpret_cast<T *>(p.conv_out) + (size_t)bh * n;
#pragma unroll
  for (int m = 0; m < MAXE; ++m) {
    const int i = threadIdx.x + m * CF::NT;
    if (i < n) out[i] = val[m];
  }
}

template <class CF, bool WITH_Q, bool VK, bool NT = false>
__device__ __forceinline__ void prefetch(ChunkRegs<CF> &R, const PrefillParams &p,
                                         const HeadBufs &hb, int c0, int Lc) {
  using T = typename CF::type;
  const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
#pragma unroll
  for (int r = 0; r < CF::RQ; ++r) {
    const int row = qrg * CF::RQ + r;
    if constexpr (WITH_Q)
      R.q[r] = load_block<T, VK, NT>(hb.q, c0 + row, qcb * CF::VEC, p.d, row < Lc);
    R.k[r] = load_block<T, VK, NT>(hb.k, c0 + row, qcb * CF::VEC, p.d, row < Lc);
  }
  const int vcb = threadIdx.x % CF::VCB, vrg = threadIdx.x / CF::VCB;
#pragma unroll
  for (int r = 0; r < CF::RV; ++r) {
    const int row = vrg * CF::RV + r;
    R.v[r] = load_block<T, VK, NT>(hb.v, c0 + row, vcb * CF::VEC, p.dv, row < Lc);
  }
}

// Registers -> LDS: phi(q) rows, phi(k) rows, v rows.  Keys past the chunk
// get weight 0 and feature columns past d are zeroed (phi(0) = 1 would
// otherwise count them); queries need no mask (their padded features meet
// zero keys and zero state rows).  The feature map and the column mask are
// uniform per launch and taken as branches, so the common case carries no
// per-element selects.  The segment summary (no queries) weights its keys by
// gamma^(Lc-1-j); the chunk kernel's keys stay unweighted (it applies the
// decay to its scores and key fragments).
template <class CF, bool WITH_Q, bool ELU, bool CH, bool CV, bool KW>
__device__ __forceinline__ void commit_rows(const ChunkRegs<CF> &R,
                                            const ConvOut<CF, WITH_Q> *Y,
                                            ConvRows<CF, WITH_Q> *P,
                                            typename CF::type *Qs,
                                            typename CF::type *Ks, const float *pw,
                                            const PrefillParams &p, int Lc,
                                            const SmemChan<CF> *sc) {
  using T = typename CF::type;
  constexpr int VEC = CF::VEC;
  const bool weighted = (KW && p.gamma != nullptr) || Lc < CF::C;
  const bool colmask = p.d < CF::DK;  // feature columns past d
  const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
  const int col0 = qcb * VEC;
  // per-channel decay: q^ = phi(q) 2^D, k^ = phi(k) 2^-D with D = lb_row -
  // ref_row as chan_prefix leaves it (ref: the row's block reference in the
  // chunk kernel, lb_L in the segment summaries)
  constexpr int LDL = SmemChan<CF>::LDL;
#pragma unroll
  for (int r = 0; r < CF::RQ; ++r) {
    const int row = qrg * CF::RQ + r;
    const float *lbr = CH ? sc->lb + row * LDL + col0 : nullptr;
    float x[VEC];
    if constexpr (WITH_Q) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float xq;
        if constexpr (CV) xq = Y->q[r][e];
        else xq = to_f32(R.q[r][e]);
        x[e] = ELU ? phi_elu1(xq) : xq;
        if constexpr (CH) x[e] *= exp2f(lbr[e]);
      }
      if constexpr (CV) P->q[r] = pack_vec<CF>(x);
      else lds_store_n<T, VEC>(Qs + row * CF::QLD + col0, x);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float xk;
      if constexpr (CV) xk = Y->k[r][e];
      else xk = to_f32(R.k[r][e]);
      x[e] = ELU ? phi_elu1(xk) : xk;
      if constexpr (CH) x[e] *= exp2f(-lbr[e]);
    }
    // key weights: 0 past the chunk; gamma^(Lc-1-j) where the decay is
    // folded into the keys (KW)
    const float w = !weighted ? 1.f : row >= Lc ? 0.f : KW ? pw[Lc - 1 - row] : 1.f;
    if (__builtin_expect(colmask, 0)) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = col0 + e < p.d ? x[e] * w : 0.f;
      if constexpr (CV) P->k[r] = pack_vec<CF>(x);
      else lds_store_n<T, VEC>(Ks + row * CF::KLD + col0, x);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] *= w;
      if constexpr (CV) P->k[r] = pack_vec<CF>(x);
      else lds_store_n<T, VEC>(Ks + row * CF::KLD + col0, x);
    }
  }
}

template <class CF, bool WITH_Q, bool CH, bool CV, bool KW>
__device__ __forceinline__ void commit(const ChunkRegs<CF> &R, typename CF::type *Qs,
                                       typename CF::type *Ks, typename CF::type *Vs,
                                       const float *pw, const PrefillParams &p, int Lc,
                                       const SmemChan<CF> *sc = nullptr,
                                       SmemConv<CF> *cs = nullptr) {
  using T = typename CF::type;
  using V = typename CF::vec;
  const int vcb = threadIdx.x % CF::VCB, vrg = threadIdx.x / CF::VCB;
  if constexpr (CV) {
    // final rows computed in registers while the raw rows are still staged
    ConvRows<CF, WITH_Q> P;
    {
      ConvOut<CF, WITH_Q> Y;
      conv_gather<CF, WITH_Q>(Y, R, Qs, Ks, Vs, *cs);
      if (p.fmap != 0)
        commit_rows<CF, WITH_Q, true, CH, true, KW>(R, &Y, &P, Qs, Ks, pw, p, Lc, sc);
      else
        commit_rows<CF, WITH_Q, false, CH, true, KW>(R, &Y, &P, Qs, Ks, pw, p, Lc, sc);
#pragma unroll
      for (int r = 0; r < CF::RV; ++r) P.v[r] = pack_vec<CF>(Y.v[r]);
    }
    __syncthreads();
    conv_halo<CF>(R, *cs, WITH_Q);
    const int qcb = threadIdx.x % CF::QCB, qrg = threadIdx.x / CF::QCB;
#pragma unroll
    for (int r = 0; r < CF::RQ; ++r) {
      const int row = qrg * CF::RQ + r;
      if constexpr (WITH_Q) *reinterpret_cast<V *>(Qs + row * CF::QLD + qcb * CF::VEC) = P.q[r];
      *reinterpret_cast<V *>(Ks + row * CF::KLD + qcb * CF::VEC) = P.k[r];
    }
#pragma unroll
    for (int r = 0; r < CF::RV; ++r) {
      const int row = vrg * CF::RV + r;
      *reinterpret_cast<V *>(Vs + row * CF::VTLD + vcb * CF::VEC) = P.v[r];
    }
  } else {
    if (p.fmap != 0)
      commit_rows<CF, WITH_Q, true, CH, false, KW>(R, nullptr, nullptr, Qs, Ks, pw, p, Lc, sc);
    else
      commit_rows<CF, WITH_Q, false, CH, false, KW>(R, nullptr, nullptr, Qs, Ks, pw, p, Lc, sc);
#pragma unroll
    for (int r = 0; r < CF::RV; ++r) {
      const int row = vrg * CF::RV + r;
      *reinterpret_cast<V *>(Vs + row * CF::VTLD + vcb * CF::VEC) = R.v[r];
    }
  }
}

// State-tile ownership: row tiles tf = srow(w, a), column tiles tn = scol(w, b).
template <class CF>
__device__ __forceinline__ int srow(int wv, int a) {
  return CF::NFT >= CF::NW ? wv * CF::FPW + a : wv % CF::NFT;
}
template <class CF>
__device__ __forceinline__ int scol(int wv, int b) {
  return CF::NFT >= CF::NW ? b : wv / CF::NFT + CF::NWC * b;
}

// [S | z] <- gamma^L [S | z] + KW^T [V | 1] for this wave's tiles.
template <class CF>
__device__ __forceinline__ void state_update(f32x4 (&Sacc)[CF::FPW][CF::TPW],
                                             const typename CF::type *Ks,
                                             const typename CF::type *Vs, float gL,
                                             bool decay, int wv, int li, int lg) {
  using T = typename CF::type;
  if (decay) {
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
      for (int b = 0; b < CF::TPW; ++b) Sacc[a][b] *= gL;
  }
  Frag<T> ones;
  frag_fill(ones, 1.f);
#pragma unroll
  for (int ks = 0; ks < CF::KSC; ++ks) {
    // slots 0..3: tokens 32 ks + 4 lg + e, slots 4..7: 32 ks + 16 + 4 lg + e
    // (one transpose read then covers 8 consecutive rows per 32 lanes)
    const int t0 = 32 * ks + 4 * lg;
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a) {
      Frag<T> kf;
      lds_frag_tr(kf, Ks, CF::KLD, t0, t0 + 16, 16 * srow<CF>(wv, a), li);
#pragma unroll
      for (int b = 0; b < CF::TPW; ++b) {
        const int tn = scol<CF>(wv, b);
        if (tn < CF::NVT) {
          Frag<T> vf;
          lds_frag_tr(vf, Vs, CF::VTLD, t0, t0 + 16, 16 * tn, li);
          mma(Sacc[a][b], kf, vf);
        } else if (tn == CF::NVT) {
          mma(Sacc[a][b], kf, ones);
        }
      }
    }
  }
}

// The state update with a per-channel decay (chunk kernel): each key
// fragment row (channel f) takes 2^(E_b - M_b), then 2^(lb_L - E_b), of its
// token block b; a fragment's slots 0..3 hold tokens of block 2 ks, slots
// 4..7 of 2 ks + 1.
template <class CF>
__device__ __forceinline__ void state_update_chan(f32x4 (&Sacc)[CF::FPW][CF::TPW],
                                                  const typename CF::type *Ks,
                                                  const typename CF::type *Vs,
                                                  const SmemChan<CF> &sc, int wv, int li,
                                                  int lg) {
  using T = typename CF::type;
  Frag<T> ones;
  frag_fill(ones, 1.f);
#pragma unroll
  for (int ks = 0; ks < CF::KSC; ++ks) {
    const int t0 = 32 * ks + 4 * lg;
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a) {
      const int f = 16 * srow<CF>(wv, a) + li;
      Frag<T> kf;
      lds_frag_tr(kf, Ks, CF::KLD, t0, t0 + 16, 16 * srow<CF>(wv, a), li);
      const int b0 = 2 * ks, b1 = 2 * ks + 1;
      const float a0 = sc.kb[b0][f], a1 = sc.kb[b1][f];
      const float c0 = b0 + 1 < CF::NRB ? sc.kf[b0][f] : 1.f;
      const float c1 = b1 + 1 < CF::NRB ? sc.kf[b1 < CF::NRB - 1 ? b1 : 0][f] : 1.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf.v[e] = from_f32<T>((to_f32(kf.v[e]) * a0) * c0);
        kf.v[4 + e] = from_f32<T>((to_f32(kf.v[4 + e]) * a1) * c1);
      }
#pragma unroll
      for (int b = 0; b < CF::TPW; ++b) {
        const int tn = scol<CF>(wv, b);
        if (tn < CF::NVT) {
          Frag<T> vf;
          lds_frag_tr(vf, Vs, CF::VTLD, t0, t0 + 16, 16 * tn, li);
          mma(Sacc[a][b], kf, vf);
        } else if (tn == CF::NVT) {
          mma(Sacc[a][b], kf, ones);
        }
      }
    }
  }
}

// gamma^-1, gamma^-2, gamma^-3 from the clamped log2 gamma (finite).
struct InvPow {
  float c1, c2, c3;
};
__device__ __forceinline__ InvPow inv_pows(float lg2) {
  InvPow c;
  c.c1 = exp2f(-lg2);
  c.c2 = exp2f(-2.f * lg2);
  c.c3 = exp2f(-3.f * lg2);
  return c;
}

// log2 of a per-head decay, clamped at -40 (see the file header).
__device__ __forceinline__ float decay_log2(const float *gamma, int h) {
  return gamma ? fmaxf(log2f(gamma[h]), -40.f) : 0.f;
}

// [S | z] <- gamma^Lc [S | z] + Phi_k^T diag(w) [V | 1] for this wave's
// tiles, w_j = gamma^(Lc-1-j): the chunk kernel's keys are unweighted in LDS,
// so the weights go onto the key fragments in registers (a lane's eight
// slots are tokens t0..t0+3 and t0+16..t0+19).  Rows past the chunk are
// zero in LDS, so their (finite) weights do not matter.
template <class CF>
__device__ __forceinline__ void state_update_decay(f32x4 (&Sacc)[CF::FPW][CF::TPW],
                                                   const typename CF::type *Ks,
                                                   const typename CF::type *Vs, int Lc,
                                                   float lg2, int wv, int li, int lg) {
  using T = typename CF::type;
  const float gL = exp2f((float)Lc * lg2);
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
    for (int b = 0; b < CF::TPW; ++b) Sacc[a][b] *= gL;
  const InvPow c = inv_pows(lg2);
  Frag<T> ones;
  frag_fill(ones, 1.f);
#pragma unroll
  for (int ks = 0; ks < CF::KSC; ++ks) {
    const int t0 = 32 * ks + 4 * lg;
    float w[8];
    {
      const float blo = exp2f((float)max(Lc - 1 - t0, 0) * lg2);
      const float bhi = exp2f((float)max(Lc - 1 - (t0 + 16), 0) * lg2);
      w[0] = blo; w[1] = blo * c.c1; w[2] = blo * c.c2; w[3] = blo * c.c3;
      w[4] = bhi; w[5] = bhi * c.c1; w[6] = bhi * c.c2; w[7] = bhi * c.c3;
    }
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a) {
      Frag<T> kf;
      lds_frag_tr(kf, Ks, CF::KLD, t0, t0 + 16, 16 * srow<CF>(wv, a), li);
#pragma unroll
      for (int e = 0; e < 8; ++e) frag_set(kf, e, frag_elem(kf, e) * w[e]);
#pragma unroll
      for (int b = 0; b < CF::TPW; ++b) {
        const int tn = scol<CF>(wv, b);
        if (tn < CF::NVT) {
          Frag<T> vf;
          lds_frag_tr(vf, Vs, CF::VTLD, t0, t0 + 16, 16 * tn, li);
          mma(Sacc[a][b], kf, vf);
        } else if (tn == CF::NVT) {
          mma(Sacc[a][b], kf, ones);
        }
      }
    }
  }
}

// Scale the state (decay only) and write its T-precision copy, transposed:
// St[n][f] = S[f][n].
template <class CF>
__device__ __forceinline__ void rescale_and_copy_state(typename CF::type *St,
                                                       f32x4 (&Sacc)[CF::FPW][CF::TPW],
                                                       float scale, bool decay, int wv,
                                                       int li, int lg) {
  if (decay) {
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
      for (int b = 0; b < CF::TPW; ++b) Sacc[a][b] *= scale;
  }
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a) {
    const int tf = srow<CF>(wv, a);
#pragma unroll
    for (int b = 0; b < CF::TPW; ++b) {
      const int tn = scol<CF>(wv, b);
      // (the normaliser tile holds z in all 16 columns: one row of it)
      if (tn < CF::NVT || (tn == CF::NVT && li == 0))
        lds_store4(St + (tn < CF::NVT ? 16 * tn + li : CF::DV) * CF::SLD + 16 * tf + 4 * lg,
                   Sacc[a][b][0], Sacc[a][b][1], Sacc[a][b][2], Sacc[a][b][3]);
    }
  }
}

// Per-row factors on this wave's [S | z] tiles (per-channel decay).
template <class CF>
__device__ __forceinline__ void chan_scale(f32x4 (&Sacc)[CF::FPW][CF::TPW], const float *fac,
                                           int wv, int lg) {
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a) {
    const int tf = srow<CF>(wv, a);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float f = fac[16 * tf + 4 * lg + r];
#pragma unroll
      for (int b = 0; b < CF::TPW; ++b) Sacc[a][b][r] *= f;
    }
  }
}

// Load this wave's [S | z] tiles from an fp32 state (rows f < d, columns
// n < dv; the normaliser tile repeats z in every column).
template <class CF>
__device__ __forceinline__ void load_state(f32x4 (&Sacc)[CF::FPW][CF::TPW], const float *S0,
                                           const float *z0, int d, int dv, int wv, int li,
                                           int lg) {
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a) {
    const int tf = srow<CF>(wv, a);
#pragma unroll
    for (int b = 0; b < CF::TPW; ++b) {
      const int tn = scol<CF>(wv, b);
      const int n = 16 * tn + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * tf + 4 * lg + r;
        float x = 0.f;
        if (tn < CF::NVT) {
          if (S0 && f < d && n < dv) x = S0[(size_t)f * dv + n];
        } else if (tn == CF::NVT) {
          if (z0 && f < d) x = z0[f];
        }
        Sacc[a][b][r] = x;
      }
    }
  }
}

// Workspace slots hold S transposed, element (f, n) at n d + f, then z at
// d dv + f: a lane's four rows f..f+3 of one column are then 16 contiguous
// bytes, one vector access (vec: d % 4 == 0 and the workspace is 16-byte
// aligned; f is a multiple of 4, so the four rows are all inside or all
// past d).  Load this wave's [S | z] tiles from a slot.
template <class CF>
__device__ __forceinline__ void load_slot(f32x4 (&Sacc)[CF::FPW][CF::TPW], const float *slot,
                                          int d, int dv, bool vec, int wv, int li, int lg) {
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a) {
    const int f = 16 * srow<CF>(wv, a) + 4 * lg;
#pragma unroll
    for (int b = 0; b < CF::TPW; ++b) {
      const int tn = scol<CF>(wv, b);
      const int n = 16 * tn + li;
      // source of the lane's four values (the normaliser tile repeats z)
      const bool ok = tn < CF::NVT ? n < dv : tn == CF::NVT;
      const float *src = slot + (tn < CF::NVT ? (size_t)n * d : (size_t)d * dv) + f;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (vec) {
        if (ok && f < d) x = *reinterpret_cast<const f32x4 *>(src);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = ok && f + r < d ? src[r] : 0.f;
      }
      Sacc[a][b] = x;
    }
  }
}

// Store this wave's [S | z] tiles to a slot (layout above).
template <class CF>
__device__ __forceinline__ void store_slot(const f32x4 (&Sacc)[CF::FPW][CF::TPW], float *slot,
                                           int d, int dv, bool vec, int wv, int li, int lg) {
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a) {
    const int f = 16 * srow<CF>(wv, a) + 4 * lg;
#pragma unroll
    for (int b = 0; b < CF::TPW; ++b) {
      const int tn = scol<CF>(wv, b);
      const int n = 16 * tn + li;
      const bool ok = tn < CF::NVT ? n < dv : (tn == CF::NVT && li == 0);
      float *dst = slot + (tn < CF::NVT ? (size_t)n * d : (size_t)d * dv) + f;
      if (vec) {
        if (ok && f < d) *reinterpret_cast<f32x4 *>(dst) = Sacc[a][b];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (ok && f + r < d) dst[r] = Sacc[a][b][r];
      }
    }
  }
}

// Store this wave's [S | z] tiles to an fp32 state.
template <class CF>
__device__ __forceinline__ void store_state(const f32x4 (&Sacc)[CF::FPW][CF::TPW], float *S1,
                                            float *z1, int d, int dv, int wv, int li, int lg) {
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a) {
    const int tf = srow<CF>(wv, a);
#pragma unroll
    for (int b = 0; b < CF::TPW; ++b) {
      const int tn = scol<CF>(wv, b);
      const int n = 16 * tn + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * tf + 4 * lg + r;
        if (tn < CF::NVT) {
          if (S1 && f < d && n < dv) S1[(size_t)f * dv + n] = Sacc[a][b][r];
        } else if (tn == CF::NVT) {
          if (z1 && li == 0 && f < d) z1[f] = Sacc[a][b][r];
        }
      }
    }
  }
}

template <class CF>
__device__ __forceinline__ void fill_powers(float *pw, float log2g) {
  for (int m = threadIdx.x; m <= CF::C; m += CF::NT) pw[m] = exp2f((float)m * log2g);
}

// How a per-head decay enters the chunk kernel (see the file header):
// none; folded into the key weights and the state copy (gamma >= 1/2); or
// each factor applied where it occurs (faster decays).
enum DecayMode : int { kDecNone = 0, kDecKeys = 1, kDecElem = 2 };

// Outputs of one chunk for one output role: query row block RB (compile-time,
// so the causal structure of the score tiles costs no branches or selects)
// and column group cg of the value tiles; normalised rows go to the staging
// tile Os.  MODE kDecElem: the scores take gamma^(i-j) and the state read
// gamma^(i+1) (lg2 = log2 gamma); kDecKeys: numerator and denominator carry
// gamma^(L-1-i), so eps does too.
// CH: per-channel decay, factors from the tables of sc (see the file header).
template <class CF, int RB, bool DN, int MODE, bool CH>
__device__ __forceinline__ void chunk_outputs(SmemChunk<CF> &sm, const SmemChan<CF> *sc,
                                              const PrefillParams &p, int Lc, int cg, int li,
                                              int lg, float *den_row, float lg2) {
  using T = typename CF::type;
  const int irow = 16 * RB + li;  // this lane's query row
  // ---- scores, transposed: at[tj][r] = phi(q_i) . phi(k_j), i = irow,
  //      j = 16 tj + 4 lg + r (lower triangle only) ----
  Frag<T> qf[CF::KSD];
#pragma unroll
  for (int ks = 0; ks < CF::KSD; ++ks)
    lds_frag(qf[ks], sm.Qs + irow * CF::QLD + 32 * ks + 8 * lg);
  // per-channel decay: the queries against the block boundary, q^ 2^(M_RB - R_RB)
  [[maybe_unused]] Frag<T> qt[CH ? CF::KSD : 1];
  if constexpr (CH) {
#pragma unroll
    for (int ks = 0; ks < CF::KSD; ++ks)
      qt[ks] = frag_scaled(qf[ks], sc->qa[RB] + 32 * ks + 8 * lg);
  }
  f32x4 at[CF::NRB];
#pragma unroll
  for (int tj = 0; tj < CF::NRB; ++tj) {
    at[tj] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (tj <= RB) {
#pragma unroll
      for (int ks = 0; ks < CF::KSD; ++ks) {
        Frag<T> kf;
        lds_frag(kf, sm.Ks + (16 * tj + li) * CF::KLD + 32 * ks + 8 * lg);
        if (CH && tj < RB) {  // key block tj before the query block (see the header)
          const int c0 = 32 * ks + 8 * lg;
          kf = frag_scaled(kf, sc->kb[tj] + c0);
          if (tj + 1 < RB)
            mma(at[tj], kf, frag_scaled(qt[ks], sc->cp[(RB - 2) * (RB - 1) / 2 + tj] + c0));
          else
            mma(at[tj], kf, qt[ks]);
        } else {
          mma(at[tj], kf, qf[ks]);
        }
      }
    }
  }
  if constexpr (MODE == kDecElem) {  // gamma^(i-j) = gamma^e gamma^-r, e = i - 16 tj - 4 lg
    const InvPow c = inv_pows(lg2);
#pragma unroll
    for (int tj = 0; tj <= RB; ++tj) {
      // e < 0 only where all four keys are masked below (then any finite factor)
      const float f = exp2f((float)max(irow - 16 * tj - 4 * lg, 0) * lg2);
      at[tj][0] *= f;
      at[tj][1] *= f * c.c1;
      at[tj][2] *= f * c.c2;
      at[tj][3] *= f * c.c3;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) at[RB][r] = 4 * lg + r <= li ? at[RB][r] : 0.f;

  // ---- O^T = [S' | z']^T Phi_q^T + [V | 1]^T A^T, with the state copy
  //      S' = S- (row factor gamma^(i+1) applied after the product, kDecElem)
  //      or S' = gamma^L S- (kDecKeys) ----
  f32x4 acc[CF::NPW], accd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int a = 0; a < CF::NPW; ++a) acc[a] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < CF::KSD; ++ks) {
    // (per-channel decay: the state read takes (q^ 2^(M_RB - R_RB)) 2^R_RB)
    Frag<T> qs = qf[ks];
    if constexpr (CH) qs = RB ? frag_scaled(qt[ks], sc->sf[RB ? RB - 1 : 0] + 32 * ks + 8 * lg)
                              : qt[ks];
#pragma unroll
    for (int a = 0; a < CF::NPW; ++a) {
      Frag<T> sf;
      lds_frag(sf, sm.St + (16 * (cg * CF::NPW + a) + li) * CF::SLD + 32 * ks + 8 * lg);
      mma(acc[a], sf, qs);
    }
    Frag<T> zf;
    lds_frag(zf, sm.St + CF::DV * CF::SLD + 32 * ks + 8 * lg);  // z, every lane
    mma(accd, zf, qs);
  }
  if constexpr (MODE == kDecElem) {
    const float gq = exp2f((float)(irow + 1) * lg2);
#pragma unroll
    for (int a = 0; a < CF::NPW; ++a) acc[a] *= gq;
    accd *= gq;
  }
  Frag<T> ones;
  frag_fill(ones, 1.f);
#pragma unroll
  for (int pp = 0; pp < CF::NRB / 2; ++pp) {
    if (2 * pp <= RB) {
      // slots 0..3: keys 32 pp + 4 lg + e; slots 4..7: 32 pp + 16 + 4 lg + e
      Frag<T> af;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        frag_set(af, e, at[2 * pp][e]);
        frag_set(af, 4 + e, at[2 * pp + 1][e]);
      }
      const int tlo = 32 * pp + 4 * lg, thi = tlo + 16;
#pragma unroll
      for (int a = 0; a < CF::NPW; ++a) {
        Frag<T> vf;
        lds_frag_tr(vf, sm.Vs, CF::VTLD, tlo, thi, 16 * (cg * CF::NPW + a), li);
        mma(acc[a], vf, af);
      }
      mma(accd, ones, af);
    }
  }

  // ---- normalise: lane holds columns 16 tn + 4 lg + r of token irow ----
  {
    const float den =
        accd[0] + (MODE == kDecKeys ? p.eps * sm.pw[max(Lc - 1 - irow, 0)] : p.eps);
    const float rd = __builtin_amdgcn_rcpf(den);
    // the token's own denominator phi(q).z + eps (kDecKeys: den carries
    // gamma^(L-1-i))
    if constexpr (DN) {
      if (cg == 0 && lg == 0 && irow < Lc)
        den_row[irow] = MODE == kDecKeys ? accd[0] / sm.pw[Lc - 1 - irow] + p.eps : den;
    }
#pragma unroll
    for (int a = 0; a < CF::NPW; ++a)
      lds_store4(sm.Os + irow * CF::VLD + 16 * (cg * CF::NPW + a) + 4 * lg,
                 acc[a][0] * rd, acc[a][1] * rd, acc[a][2] * rd, acc[a][3] * rd);
  }

}

// The chunk loop of one segment (chunk_kernel), for one way of applying a
// per-head decay (MODE).
template <class CF, bool VK, bool CH, bool CV, bool DN, int MODE>
__device__ __forceinline__ void chunk_loop(SmemChunk<CF> &sm, ChanSmem<CF, CH> &sc,
                                           ConvSmem<CF, CV> &cs, const PrefillParams &p,
                                           const HeadBufs &hb,
                                           f32x4 (&Sacc)[CF::FPW][CF::TPW], ChunkRegs<CF> &R,
                                           ChanRegs<CF> &A, __amdgpu_buffer_rsrc_t ra, int bh,
                                           int t_begin, int t_end, float lg2, int wv, int li,
                                           int lg) {
  using T = typename CF::type;
  using V = typename CF::vec;
  const int d = p.d, dv = p.dv, N = p.N;
  constexpr bool KEYS = MODE == kDecKeys;
  if constexpr (!CH)
    rescale_and_copy_state<CF>(sm.St, Sacc, KEYS ? sm.pw[min(CF::C, N - t_begin)] : 1.f, KEYS,
                               wv, li, lg);

  const int rb = wv % CF::NRB, cg = wv / CF::NRB;  // output role
  for (int c0 = t_begin; c0 < t_end; c0 += CF::C) {
    const int Lc = min(CF::C, N - c0);
    if constexpr (CH) {  // the chunk's per-channel decay prefix sums
      chan_logs<CF>(A, sc, d, Lc);
      __syncthreads();
      chan_prefix<CF>(sc, false);
      __syncthreads();
    }
    commit<CF, true, CH, CV, KEYS>(R, sm.Qs, sm.Ks, sm.Vs, sm.pw, p, Lc, chan_ptr<CF>(sc),
                                   conv_ptr<CF>(cs));
    if constexpr (CH) {  // the state copy as it stands (factors on the queries)
      rescale_and_copy_state<CF>(sm.St, Sacc, 1.f, false, wv, li, lg);
      if (c0 + CF::C < t_end)
        chan_prefetch<CF, VK>(A, ra, p, c0 + CF::C, min(CF::C, N - c0 - CF::C));
    }
    if (c0 + CF::C < t_end)
      prefetch<CF, true, VK>(R, p, hb, c0 + CF::C, min(CF::C, N - c0 - CF::C));
    __syncthreads();

    float *dno = DN ? p.den_out + (size_t)bh * N + c0 : nullptr;
    if constexpr (CF::NRB == 2) {
      if (rb == 0) chunk_outputs<CF, 0, DN, MODE, CH>(sm, chan_ptr<CF>(sc), p, Lc, cg, li, lg, dno, lg2);
      else chunk_outputs<CF, 1, DN, MODE, CH>(sm, chan_ptr<CF>(sc), p, Lc, cg, li, lg, dno, lg2);
    } else {
      static_assert(CF::NRB == 4, "row blocks per chunk");
      switch (rb) {
        case 0: chunk_outputs<CF, 0, DN, MODE, CH>(sm, chan_ptr<CF>(sc), p, Lc, cg, li, lg, dno, lg2); break;
        case 1: chunk_outputs<CF, 1, DN, MODE, CH>(sm, chan_ptr<CF>(sc), p, Lc, cg, li, lg, dno, lg2); break;
        case 2: chunk_outputs<CF, 2, DN, MODE, CH>(sm, chan_ptr<CF>(sc), p, Lc, cg, li, lg, dno, lg2); break;
        default: chunk_outputs<CF, 3, DN, MODE, CH>(sm, chan_ptr<CF>(sc), p, Lc, cg, li, lg, dno, lg2); break;
      }
    }

    // ---- carry the state across the chunk ----
    // (the accumulator already carries gamma^Lc with the decay folded into
    // the keys, or diag(exp(lb_m)) with a per-channel decay: scaled before
    // the copy)
    if constexpr (CH) {  // S+ = diag(2^lb_L) S- + sum_i (keys to the chunk end) v_i^T
      chan_scale<CF>(Sacc, sc.el, wv, lg);
      state_update_chan<CF>(Sacc, sm.Ks, sm.Vs, sc, wv, li, lg);
    } else if constexpr (MODE == kDecElem) {
      state_update_decay<CF>(Sacc, sm.Ks, sm.Vs, Lc, lg2, wv, li, lg);
    } else {
      state_update<CF>(Sacc, sm.Ks, sm.Vs, 1.f, false, wv, li, lg);
    }
    __syncthreads();
    if constexpr (!CH) {
      if (c0 + CF::C < t_end)
        rescale_and_copy_state<CF>(sm.St, Sacc,
                                   KEYS ? sm.pw[min(CF::C, N - c0 - CF::C)] : 1.f, KEYS, wv,
                                   li, lg);
    }
    // 16-byte row stores of the output tile
    {
      const int vcb = threadIdx.x % CF::VCB, vrg = threadIdx.x / CF::VCB;
      const int col0 = vcb * CF::VEC;
#pragma unroll
      for (int r = 0; r < CF::RV; ++r) {
        const int row = vrg * CF::RV + r;
        const V val = *reinterpret_cast<const V *>(sm.Os + row * CF::VLD + col0);
        const size_t el = (size_t)(c0 + row) * dv + col0;
        if constexpr (VK) {
          const bool ok = row < Lc && col0 < dv;
          buf_store16_nt<T>(hb.o, ok ? (uint32_t)(el * sizeof(T)) : kOOB, val);
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
}

// Resident waves per SIMD the register allocation must allow: the
// per-channel decay and the convolution need more registers than three
// waves leave.
template <class CF>
constexpr int wpe_at_most_2() {
  return CF::WPE < 2 ? CF::WPE : 2;
}

// DN: also write each token's denominator (den_out; not with the fused
// convolution); DEC: per-head decay gamma (compiled in only where given)
template <class CF, bool VK, bool CH, bool CV, bool DN, bool DEC>
__global__ void __launch_bounds__(CF::NT, (CH || CV) ? wpe_at_most_2<CF>() : CF::WPE)
    chunk_kernel(PrefillParams p) {
  using T = typename CF::type;
  using V = typename CF::vec;
  __shared__ SmemChunk<CF> sm;
  __shared__ ChanSmem<CF, CH> sc;  // per-channel decay (CH) only
  __shared__ ConvSmem<CF, CV> cs;  // short convolution (CV) only

  const int seg = blockIdx.x, bh = grid_head();
  if (bh >= p.BH) return;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv, N = p.N;
  const HeadBufs hb = head_bufs<T>(p, bh);
  const int t_begin = seg * p.seg_len;
  const int t_end = min(N, t_begin + p.seg_len);

  // state entering this segment: slot seg of the scanned workspace, or
  // (S_in, z_in) with a single segment
  f32x4 Sacc[CF::FPW][CF::TPW];
  if (p.nseg > 1)
    load_slot<CF>(Sacc, p.ws + ((size_t)seg * p.BH + bh) * ws_rec(d, dv), d, dv, p.slot_vec,
                  wv, li, lg);
  else
    load_state<CF>(Sacc, p.S_in ? p.S_in + (size_t)bh * d * dv : nullptr,
                   p.z_in ? p.z_in + (size_t)bh * d : nullptr, d, dv, wv, li, lg);
  // the first chunk's loads go out after the state loads (loads complete in
  // issue order, so waiting for the state does not wait for the chunk)
  ChunkRegs<CF> R;
  prefetch<CF, true, VK>(R, p, hb, t_begin, min(CF::C, N - t_begin));
  [[maybe_unused]] ChanRegs<CF> A;
  [[maybe_unused]] const __amdgpu_buffer_rsrc_t ra =
      CH ? buf_rsrc(p.alpha + (size_t)bh * N * d, (uint32_t)((size_t)N * d * 4)) : hb.q;
  if constexpr (CH) chan_prefetch<CF, VK>(A, ra, p, t_begin, min(CF::C, N - t_begin));
  if constexpr (CV)  // the tokens before segment 0 come from the cache (or its copy)
    conv_init<CF>(cs, p, bh, t_begin,
                  p.conv_src ? reinterpret_cast<const T *>(p.conv_src) +
                                   (size_t)bh * (p.conv_width - 1) * (2 * d + dv)
                             : nullptr,
                  nullptr);
  const float lg2 = DEC ? decay_log2(p.gamma, bh % p.H) : 0.f;
  if constexpr (DEC) fill_powers<CF>(sm.pw, lg2);
  __syncthreads();
  if constexpr (DEC) {
    // gamma >= 1/2: decay folded into the key weights and the state copy
    // (factors within gamma^C of 1); faster decays: every factor where it
    // occurs (uniform per workgroup)
    if (lg2 >= -1.f)
      chunk_loop<CF, VK, CH, CV, DN, kDecKeys>(sm, sc, cs, p, hb, Sacc, R, A, ra, bh,
                                               t_begin, t_end, lg2, wv, li, lg);
    else
      chunk_loop<CF, VK, CH, CV, DN, kDecElem>(sm, sc, cs, p, hb, Sacc, R, A, ra, bh,
                                               t_begin, t_end, lg2, wv, li, lg);
  } else {
    chunk_loop<CF, VK, CH, CV, DN, kDecNone>(sm, sc, cs, p, hb, Sacc, R, A, ra, bh, t_begin,
                                             t_end, lg2, wv, li, lg);
  }

  if (seg == p.nseg - 1) {
    store_state<CF>(Sacc, p.S_out ? p.S_out + (size_t)bh * d * dv : nullptr,
                    p.z_out ? p.z_out + (size_t)bh * d : nullptr, d, dv, wv, li, lg);
    if constexpr (CV) {
      if (p.conv_out) conv_final<CF>(p, bh);
    }
  }
}

// Phase 1: each segment's own contribution, from a zero state (all but the
// last segment; those are whole multiples of the chunk length).
// NT: streaming loads of k and v (the launch's k and v exceed the last-level
// cache, so the chunk kernel will not find them there).
template <class CF, bool VK, bool CH, bool CV, bool NT = false>
__global__ void __launch_bounds__(CF::NT, (CH && CV) ? wpe_at_most_2<CF>() : CF::WPE)
    summary_kernel(PrefillParams p) {
  using T = typename CF::type;
  __shared__ SmemSummary<CF> sm;
  __shared__ ChanSmem<CF, CH> sc;  // per-channel decay (CH) only
  __shared__ ConvSmem<CF, CV> cs;  // short convolution (CV) only
  // part `part` of segment `seg`: with two parts per segment the first
  // covers split_len tokens, the second the rest (whole chunks both)
  const int seg = blockIdx.x / p.nsplit, part = blockIdx.x % p.nsplit, bh = grid_head();
  if (bh >= p.BH) return;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int d = p.d, dv = p.dv;
  const HeadBufs hb = head_bufs<T>(p, bh);
  const int t_begin = seg * p.seg_len + part * p.split_len;
  const int t_end = part + 1 == p.nsplit ? (seg + 1) * p.seg_len : t_begin + p.split_len;
  const bool decay = p.gamma != nullptr;

  // k and v rows of the next PD chunks are in flight while one is reduced
  // (CF::PD; the per-channel decay and the convolution keep one chunk).
  constexpr int PD = (CH || CV) ? 1 : CF::PD;
  ChunkRegs<CF> R[PD];
#pragma unroll
  for (int u = 0; u < PD; ++u)
    if (t_begin + u * CF::C < t_end)
      prefetch<CF, false, VK, NT>(R[u], p, hb, t_begin + u * CF::C, CF::C);
  [[maybe_unused]] ChanRegs<CF> A;
  [[maybe_unused]] const __amdgpu_buffer_rsrc_t ra =
      CH ? buf_rsrc(p.alpha + (size_t)bh * p.N * d, (uint32_t)((size_t)p.N * d * 4)) : hb.q;
  if constexpr (CH) {
    chan_prefetch<CF, VK>(A, ra, p, t_begin, CF::C);
    if (threadIdx.x < CF::DK) sc.tot[threadIdx.x] = 0.f;
  }
  if constexpr (CV) {  // segment 0 reads the cache and leaves a copy for chunk_kernel
    const size_t crow = (size_t)bh * (p.conv_width - 1) * (2 * d + dv);
    conv_init<CF>(cs, p, bh, t_begin,
                  p.conv_in ? reinterpret_cast<const T *>(p.conv_in) + crow : nullptr,
                  p.conv_copy ? reinterpret_cast<T *>(p.conv_copy) + crow : nullptr);
  }
  fill_powers<CF>(sm.pw, decay_log2(p.gamma, bh % p.H));

  f32x4 Sacc[CF::FPW][CF::TPW];
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
    for (int b = 0; b < CF::TPW; ++b) Sacc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const float gC = sm.pw[CF::C];
  for (int c0 = t_begin; c0 < t_end; c0 += PD * CF::C) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {  // register set u holds chunk c0 + u C
      const int cc = c0 + u * CF::C;
      if (cc >= t_end) break;
      if constexpr (CH) {
        chan_logs<CF>(A, sc, d, CF::C);
        __syncthreads();
        chan_prefix<CF>(sc, true);
        __syncthreads();
      }
      commit<CF, false, CH, CV, true>(R[u], nullptr, sm.Ks, sm.Vs, sm.pw, p, CF::C,
                                chan_ptr<CF>(sc), conv_ptr<CF>(cs));
      if constexpr (CH) {  // S+ = diag(2^lb_L) S- + K^^T V, keys weighted 2^(lb_L - lb_i)
        chan_scale<CF>(Sacc, sc.el, wv, lg);
        if (cc + CF::C < t_end) chan_prefetch<CF, VK>(A, ra, p, cc + CF::C, CF::C);
      }
      if (cc + PD * CF::C < t_end)
        prefetch<CF, false, VK, NT>(R[u], p, hb, cc + PD * CF::C, CF::C);
      __syncthreads();
      state_update<CF>(Sacc, sm.Ks, sm.Vs, gC, decay, wv, li, lg);
      __syncthreads();
    }
  }
  // the first part's record in slot seg + 1, the second's in slot nseg + seg
  const int slot = part == 0 ? seg + 1 : p.nseg + seg;
  float *dst = p.ws + ((size_t)slot * p.BH + bh) * ws_rec(d, dv);
  store_slot<CF>(Sacc, dst, d, dv, p.slot_vec, wv, li, lg);
  if constexpr (CH) {  // the segment's log2 decay per channel (own thread's sum)
    if (threadIdx.x < d) dst[(size_t)d * dv + d + threadIdx.x] = sc.tot[threadIdx.x];
  }
}

// Phase 2: prefix over segments, in place: slot 0 <- (S_in, z_in),
// slot s <- gamma^Lseg slot (s-1) + dS_(s-1) for s >= 1, where dS_(s-1) is
// the contribution of segment s-1: its summary record (slot s), or with two
// summary parts gamma^Lb A + B (A in slot s, B, the last Lb tokens, in slot
// nseg + s - 1).  With a per-channel decay the factors of row f are 2 to
// the parts' log2 decays of channel f, stored with the records.  One thread
// per record element; every record is loaded before the dependent chain.
template <bool CH, bool TWO>
__global__ void __launch_bounds__(256) scan_kernel(PrefillParams p) {
  const int bh = grid_head();
  if (bh >= p.BH) return;
  const size_t dd = (size_t)p.d * p.dv;
  const size_t rec = dd + p.d;               // scanned elements: S then z
  const size_t wr = ws_rec(p.d, p.dv);       // slot record stride
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= rec) return;
  constexpr bool two = TWO;  // two summary parts per segment (nsplit 2)
  const float lgam = decay_log2(p.gamma, bh % p.H);
  const float gL = exp2f((float)p.seg_len * lgam);
  const float gB = exp2f((float)(p.seg_len - p.split_len) * lgam);
  float *base = p.ws + (size_t)bh * wr + e;
  const float *bsec = p.ws + ((size_t)p.nseg * p.BH + bh) * wr + e;  // second parts
  const size_t stride = (size_t)p.BH * wr;
  float dS[kMaxSeg];
  [[maybe_unused]] float dB[TWO ? kMaxSeg : 1];
#pragma unroll
  for (int s = 1; s < kMaxSeg; ++s) {
    dS[s] = s < p.nseg ? base[s * stride] : 0.f;
    if constexpr (TWO) dB[s] = s < p.nseg ? bsec[(s - 1) * stride] : 0.f;
  }
  [[maybe_unused]] float lgd[kMaxSeg];
  [[maybe_unused]] float lgb[TWO ? kMaxSeg : 1];
  if constexpr (CH) {
    const size_t f = e < dd ? e % p.d : e - dd;  // the element's state row
    const float *ld = p.ws + (size_t)bh * wr + dd + p.d + f;
    const float *lb = p.ws + ((size_t)p.nseg * p.BH + bh) * wr + dd + p.d + f;
#pragma unroll
    for (int s = 1; s < kMaxSeg; ++s) {
      lgd[s] = s < p.nseg ? ld[s * stride] : 0.f;
      if constexpr (TWO) lgb[s] = s < p.nseg ? lb[(s - 1) * stride] : 0.f;
    }
  }
  float acc;
  if (e < dd)  // slot element e is S[f][n] with n = e / d, f = e % d
    acc = p.S_in ? p.S_in[(size_t)bh * dd + (e % p.d) * p.dv + e / p.d] : 0.f;
  else
    acc = p.z_in ? p.z_in[(size_t)bh * p.d + (e - dd)] : 0.f;
  base[0] = acc;
#pragma unroll
  for (int s = 1; s < kMaxSeg; ++s) {
    if (s < p.nseg) {
      float g = gL, seg_part = dS[s];
      if constexpr (TWO) {
        float gb = gB;
        if constexpr (CH) {
          g = exp2f(lgd[s] + lgb[s]);
          gb = exp2f(lgb[s]);
        }
        seg_part = fmaf(gb, seg_part, dB[s]);
      } else if constexpr (CH) {
        g = exp2f(lgd[s]);
      }
      acc = fmaf(g, acc, seg_part);
      base[s * stride] = acc;
    }
  }
}

template <bool CH>
hipError_t launch_scan(const PrefillParams &p, hipStream_t s) {
  const size_t rec = (size_t)p.d * p.dv + p.d;
  const dim3 grid = head_grid((unsigned)((rec + 255) / 256), p.BH);
  return p.nsplit == 2 ? launch_kernel("linear_scan", scan_kernel<CH, true>, grid, dim3(256), s, p)
                       : launch_kernel("linear_scan", scan_kernel<CH, false>, grid, dim3(256), s, p);
}

// LDS of one chunk_kernel workgroup
template <class CF, bool CH, bool CV>
constexpr size_t chunk_lds() {
  return sizeof(SmemChunk<CF>) + (CH ? sizeof(SmemChan<CF>) : 0) +
         (CV ? sizeof(SmemConv<CF>) : 0);
}

// The chunk kernel's tile strides: at d = 128 (bf16) the plain kernel's
// Qs, Ks and state-copy rows take 16 more elements, which spreads its
// output phase's LDS reads over more banks (measured faster at B1 H32
// N131072); the per-channel-decay and convolution variants keep the
// tighter rows (with both, that tile size would not fit in the LDS).
template <class CF>
struct WideRows : CF {
  static constexpr int QLD = CF::DK + 2 * CF::VEC;
  static constexpr int KLD = QLD, SLD = QLD;
};
template <class CF, bool CH, bool CV>
using ChunkCfg =
    typename std::conditional<!CH && !CV && CF::DK == 128 && sizeof(typename CF::type) == 2,
                              WideRows<CF>, CF>::type;

template <class CF0, bool VK, bool CH, bool CV>
hipError_t run_vkcc(const PrefillParams &p, hipStream_t s) {
  using CF = ChunkCfg<CF0, CH, CV>;  // (the summary keeps CF0)
  if constexpr (chunk_lds<CF, CH, CV>() > kLdsBytes) {
    return hipErrorNotSupported;  // refused on the host before any launch
  } else {
  if (p.nseg > 1) {
    const dim3 grid = head_grid((p.nseg - 1) * p.nsplit, p.BH);
    // k and v beyond the last-level cache (256 MB): streaming loads
    const bool stream = (size_t)p.BH * p.N * (p.d + p.dv) * sizeof(typename CF::type) >
                        kStreamBytes;
    hipError_t e;
    if constexpr (!CH && !CV && VK)
      e = stream ? launch_kernel("linear_summary", summary_kernel<CF0, VK, false, false, true>,
                                 grid, dim3(CF::NT), s, p)
                 : launch_kernel("linear_summary", summary_kernel<CF0, VK, CH, CV>, grid,
                                 dim3(CF::NT), s, p);
    else
      e = launch_kernel("linear_summary", summary_kernel<CF0, VK, CH, CV>, grid, dim3(CF::NT), s,
                        p);
    if (e != hipSuccess) return e;
    e = launch_scan<CH>(p, s);
    if (e != hipSuccess) return e;
  }
  const dim3 grid = head_grid(p.nseg, p.BH);
  if constexpr (CH) {  // (a per-channel decay excludes gamma)
    if constexpr (!CV) {  // (with den_out a convolution runs as a pass of its own)
      if (p.den_out)
        return launch_kernel("linear_chunk", chunk_kernel<CF, VK, true, false, true, false>,
                             grid, dim3(CF::NT), s, p);
    }
    return launch_kernel("linear_chunk", chunk_kernel<CF, VK, CH, CV, false, false>, grid,
                         dim3(CF::NT), s, p);
  } else {
    const bool dec = p.gamma != nullptr;
    if constexpr (!CV) {
      if (p.den_out)
        return dec ? launch_kernel("linear_chunk", chunk_kernel<CF, VK, false, false, true, true>,
                                   grid, dim3(CF::NT), s, p)
                   : launch_kernel("linear_chunk", chunk_kernel<CF, VK, false, false, true, false>,
                                   grid, dim3(CF::NT), s, p);
    }
    return dec ? launch_kernel("linear_chunk", chunk_kernel<CF, VK, CH, CV, false, true>, grid,
                               dim3(CF::NT), s, p)
               : launch_kernel("linear_chunk", chunk_kernel<CF, VK, CH, CV, false, false>, grid,
                               dim3(CF::NT), s, p);
  }
  }
}

// a per-key-channel decay and a short convolution get their own
// instantiations (none of their work is compiled into the others)
template <class CF, bool VK, bool CH>
hipError_t run_vkc(const PrefillParams &p, hipStream_t s) {
  return p.conv_w ? run_vkcc<CF, VK, CH, true>(p, s) : run_vkcc<CF, VK, CH, false>(p, s);
}

template <class CF, bool VK>
hipError_t run_vk(const PrefillParams &p, hipStream_t s) {
  return p.alpha ? run_vkc<CF, VK, true>(p, s) : run_vkc<CF, VK, false>(p, s);
}

template <class CF>
hipError_t run(const PrefillParams &p, hipStream_t s) {
  return p.vec_ok ? run_vk<CF, true>(p, s) : run_vk<CF, false>(p, s);
}

// summary + scan only (the segment-entering states); the per-head decay
// is read by the plain instantiation, a per-channel decay has its own
template <class CF>
hipError_t run_prefix(const PrefillParams &p, hipStream_t s) {
  if (p.nseg <= 1) return hipSuccess;
  const dim3 grid = head_grid((p.nseg - 1) * p.nsplit, p.BH);
  hipError_t e;
  if (p.alpha)
    e = p.vec_ok ? launch_kernel("linear_summary", summary_kernel<CF, true, true, false>, grid,
                                 dim3(CF::NT), s, p)
                 : launch_kernel("linear_summary", summary_kernel<CF, false, true, false>, grid,
                                 dim3(CF::NT), s, p);
  else
    e = p.vec_ok ? launch_kernel("linear_summary", summary_kernel<CF, true, false, false>, grid,
                                 dim3(CF::NT), s, p)
                 : launch_kernel("linear_summary", summary_kernel<CF, false, false, false>, grid,
                                 dim3(CF::NT), s, p);
  if (e != hipSuccess) return e;
  return p.alpha ? launch_scan<true>(p, s) : launch_scan<false>(p, s);
}

// Workgroups of chunk_kernel<CF> that fit on one CU (queried once per
// instantiation).
template <class CF, bool CH, bool CV>
int resident_per_cu() {
  if constexpr (chunk_lds<ChunkCfg<CF, CH, CV>, CH, CV>() > kLdsBytes) {
    return 1;  // refused at launch anyway
  } else {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, chunk_kernel<ChunkCfg<CF, CH, CV>, true, CH, CV, false, false>, CF::NT, 0) !=
            hipSuccess ||
        n < 1) {
      (void)hipGetLastError();
      n = 1;
    }
    cached.store(n, std::memory_order_relaxed);
    return n;
  }
}

// Instantiations: bf16 uses 64-token chunks; fp32 uses 32-token chunks
// beyond d = dv = 64 so that its fp32 tiles fit in LDS.
using B64x64 = Cfg<bf16, 64, 64, 64, 4>;
using B64x128 = Cfg<bf16, 64, 128, 64, 8>;
using B128x64 = Cfg<bf16, 128, 64, 64, 8>;
using B128x128 = Cfg<bf16, 128, 128, 64, 8>;
using F64x64 = Cfg<float, 64, 64, 64, 4>;
using F64x128 = Cfg<float, 64, 128, 32, 8>;
using F128x64 = Cfg<float, 128, 64, 32, 8>;
using F128x128 = Cfg<float, 128, 128, 32, 8>;

template <class CF>
void fill_plan(LinearPlan &pl, bool conv, bool chan) {
  pl.chunk = CF::C;
  pl.threads = CF::NT;
  if (chan)
    pl.per_cu = conv ? resident_per_cu<CF, true, true>() : resident_per_cu<CF, true, false>();
  else
    pl.per_cu = conv ? resident_per_cu<CF, false, true>() : resident_per_cu<CF, false, false>();
}

}  // namespace

LinearPlan plan_linear(int BH, int N, int d, int dv, bool bf16_io, int conv_width, bool chan) {
  LinearPlan pl{};
  pl.dk = d <= 64 ? 64 : 128;
  pl.dv_pad = dv <= 64 ? 64 : 128;
  const bool cv = conv_width > 0;
  if (bf16_io) {
    if (pl.dk == 64) pl.dv_pad == 64 ? fill_plan<B64x64>(pl, cv, chan) : fill_plan<B64x128>(pl, cv, chan);
    else pl.dv_pad == 64 ? fill_plan<B128x64>(pl, cv, chan) : fill_plan<B128x128>(pl, cv, chan);
  } else {
    if (pl.dk == 64) pl.dv_pad == 64 ? fill_plan<F64x64>(pl, cv, chan) : fill_plan<F64x128>(pl, cv, chan);
    else pl.dv_pad == 64 ? fill_plan<F128x64>(pl, cv, chan) : fill_plan<F128x128>(pl, cv, chan);
  }
  const long chunks = N > 0 ? ((long)N + pl.chunk - 1) / pl.chunk : 0;
  long nseg = 1;
  if (chunks > 1 && BH > 0) {
    // one launch fills every resident workgroup slot once
    const long slots = (long)device_cu_count() * pl.per_cu;
    nseg = (slots + BH / 2) / BH;
    if (nseg > chunks) nseg = chunks;
    if (nseg > kMaxSeg) nseg = kMaxSeg;
    if (nseg < 1) nseg = 1;
  }
  const long cps = chunks > 0 ? (chunks + nseg - 1) / nseg : 1;
  nseg = chunks > 0 ? (chunks + cps - 1) / cps : 1;
  pl.nseg = (int)nseg;
  pl.seg_len = (int)(cps * pl.chunk);
  // When its workgroups would not cover the CUs (few heads, long segments),
  // the summary kernel splits each segment in two parts of whole chunks (its
  // workgroups then walk half as many chunks each, and twice as many run);
  // the scan combines the parts.  Records: nseg slots, then one more per
  // summarised segment for the second parts.  With enough workgroups the
  // split measured slower (more records to write and scan).
  pl.nsplit = nseg > 1 && cps >= 2 && (nseg - 1) * (long)BH < device_cu_count() ? 2 : 1;
  pl.split_len = (int)(((cps + 1) / 2) * pl.chunk);
  pl.wrec = ws_rec(d, dv);
  const size_t nrec = nseg > 1 ? (size_t)nseg + (size_t)(pl.nsplit - 1) * (nseg - 1) : 0;
  pl.ws_bytes = nrec * BH * pl.wrec * sizeof(float);
  pl.conv_off = pl.ws_bytes;
  if (nseg > 1 && conv_width > 1)  // room for the summary kernel's copy of the cache
    pl.ws_bytes += (size_t)BH * (conv_width - 1) * (2 * d + dv) * (bf16_io ? 2 : 4);
  return pl;
}

// A short convolution together with a per-key-channel decay does not fit
// the LDS of the fp32 instantiation with d and dv above 64.
bool linear_combo_supported(int d, int dv, bool bf16_io, bool chan, bool conv) {
  if (bf16_io || !chan || !conv || d <= 64 || dv <= 64) return true;
  return chunk_lds<F128x128, true, true>() <= kLdsBytes;
}

hipError_t launch_linear_state_prefix(const PrefillParams &p, const LinearPlan &pl,
                                      bool bf16_io, hipStream_t s) {
  if (bf16_io) {
    if (pl.dk == 64) return pl.dv_pad == 64 ? run_prefix<B64x64>(p, s) : run_prefix<B64x128>(p, s);
    return pl.dv_pad == 64 ? run_prefix<B128x64>(p, s) : run_prefix<B128x128>(p, s);
  }
  if (pl.dk == 64) return pl.dv_pad == 64 ? run_prefix<F64x64>(p, s) : run_prefix<F64x128>(p, s);
  return pl.dv_pad == 64 ? run_prefix<F128x64>(p, s) : run_prefix<F128x128>(p, s);
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
