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
//     U  = T Y,   O = Q S- + P U = Q S- + R Y,   P = lower_incl(Q K^T),  R = P T
//     S+ = S- + K^T U = S- + Wt Y,               Wt = K^T T   (d x C)
// With the scalar decay alpha of Gated DeltaNet ("Efficient attention
// variants" 7.4: S_t = alpha_t S_{t-1} + g_t k_t (v_t - alpha_t S_{t-1}^T
// k_t)^T), let b_j = alpha_0 ... alpha_j within the chunk.  Unrolling the
// same way puts b_j / b_i on every pair j > i:
//     L = strict_lower(K K^T) (.) [b_j / b_i],  P = lower_incl(Q K^T) (.) [b_j / b_i]
//     Y = V - diag(b) K S-,  O = diag(b) Q S- + R Y,  R = P T,
//     S+ = b_L S- + Wt Y,    Wt = K^T diag(b_L / b) T   (b_L = b of the last token)
// prep forms the ratios from log-cumulative decays (a prefix sum of log
// alpha over the chunk), so every factor is exp of a non-positive number.
// Wt and R depend only on the chunk's q, k and g, so they are computed for
// every chunk in parallel (prep_kernel); the state-dependent part is a
// sequential pass over chunks (seq_kernel) with one matrix product on the
// chain per step: X = K S-, then S+ = S- + Wt (V - X).  The columns of S are
// independent, so the sequential pass is split along dv into slices.
//
// prep_kernel, one workgroup per (chunk, head):
//   K K^T and Q K^T on the matrix cores (lower tiles; the Q K^T tiles stay
//   in registers); X = (I + N)^(-1), N = diag(g) strict_lower(K K^T), in
//   fp32: 16x16 diagonal blocks by forward substitution, then the blocks
//   below, block row by block row, X_ij = -X_ii sum_{j<=m<i} N_im X_mj
//   (fp32 matrix-core products);
//   T = X diag(g).  Wt = K^T T and R^T = T^T P^T on the matrix cores with T
//   (and P) split into bf16 high and low parts, so both keep fp32-level
//   accuracy before the final rounding.  Stored in the input precision:
//   per chunk [Wt: DK x C][R: C x C], each in operand-fragment order
//   (frag_off), so a wave's fragment is one contiguous 1 KiB block.
// seq_kernel, one workgroup (4 waves) per (head, slice of W value columns;
// bf16 runs seq2_kernel below, the same pass with eight waves split by role):
//   per chunk, wave (row block rb, column group): X^T = S'^T K^T and
//   Z^T = S'^T Q^T from a T-precision copy S' of the fp32 state; Y = V - X
//   into LDS; O^T = Z^T + Y^T R^T, stored straight from registers; the
//   state rows the wave owns: S += Wt Y (fp32 accumulators, never rounded).
//   No wave reads another's R or Wt rows, so these go from memory straight
//   into operand registers, two chunks ahead (three register sets); k and
//   q are loaded as whole-line blocks with them and staged through LDS (a
//   k/q fragment would span 16 rows per load).  A chunk costs two barriers.
//
// Workgroups of one head's slices read the same q, k, R, Wt: the launch maps
// them onto one XCD (consecutive workgroup ids alternate XCDs) so those
// reads hit that XCD's L2.
#include <atomic>

#include "la_delta_common.hpp"

namespace la {
namespace {

// ---------------------------------------------------------------------------
// seq_kernel
// ---------------------------------------------------------------------------
// LDS of seq_kernel: only what the waves exchange each chunk (row strides
// padded so that 16-lane fragment reads of 16 rows hit distinct banks).
template <class CF>
struct alignas(16) SmemSeq {
  using T = typename CF::type;
  T K[CF::NSET][CF::C * CF::QLD];  // k rows of the chunk of register set u
  T Q[CF::NSET][CF::C * CF::QLD];  // q rows
  T Ys[CF::C * CF::YLD];   // Y = V - K S- rows (this slice's columns)
  T St[CF::W * CF::QLD];   // S'^T: T-precision copy of the fp32 state slice
};

// One chunk's operands, in registers.  No wave reads another's R or Wt
// rows, so those go from memory straight into operand fragments: the R rows
// of the wave's 16 tokens (record blocks (rb, ks)) and the Wt rows of its
// state row tiles (blocks (tf, ks)); likewise the four v values of the
// lane's token and the decay products b of that token and of the chunk's
// last token.  k and q are loaded as whole-line 16-byte blocks (this
// thread's share of the workgroup's) and staged through LDS: an operand
// fragment of them would span 16 rows per load.
template <class CF>
struct SeqOps {
  using T = typename CF::type;
  static constexpr int NQ = CF::C * CF::QCB / kThreads;  // k (and q) blocks per thread
  static_assert(NQ * kThreads == CF::C * CF::QCB, "k/q blocks per thread");
  typename CF::vec kb[NQ], qb[NQ];  // whole-line blocks, staged to LDS
  Frag<T> r[CF::KSC], w[CF::FPW][CF::KSC];
  typename Vec4<T>::type v[CF::TW];  // as loaded: converted where used, so
                                     // no instruction touches it in flight
  float b_tok, b_last;
};

// Issue the loads of chunk `chunk`'s operands for this wave (nothing waits
// here).  Chunks past the end read as zeros: tokens past N fail the bounds,
// records past the last chunk lie past the workspace resource.
template <class CF, bool VK, bool DECAY>
__device__ __forceinline__ void seq_fetch(SeqOps<CF> &o, const PrefillParams &p,
                                          const __amdgpu_buffer_rsrc_t (&rs)[5],
                                          __amdgpu_buffer_rsrc_t rdec, int chunk, int n0,
                                          int wv, int rb, int ct0, int lane) {
  using T = typename CF::type;
  constexpr int C = CF::C;
  const int li = lane & 15, lg = lane >> 4;
  const int t = chunk * C + 16 * rb + li;
  const bool tok_ok = t < p.N;
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < SeqOps<CF>::NQ; ++m) {
    const int b = tid + m * kThreads;
    const int row = chunk * C + b / CF::QCB, col0 = (b % CF::QCB) * CF::VEC;
    if constexpr (VK) {
      const uint32_t off = (row < p.N && col0 < p.d)
                               ? (uint32_t)(((size_t)row * p.d + col0) * sizeof(T)) : kOOB;
      o.kb[m] = buf_load16<T>(rs[1], off);
      o.qb[m] = buf_load16<T>(rs[0], off);
    } else {
#pragma unroll
      for (int e = 0; e < CF::VEC; ++e) {
        const uint32_t off = (row < p.N && col0 + e < p.d)
                                 ? (uint32_t)(((size_t)row * p.d + col0 + e) * sizeof(T)) : kOOB;
        o.kb[m][e] = buf_load1(rs[1], off, (T *)nullptr);
        o.qb[m][e] = buf_load1(rs[0], off, (T *)nullptr);
      }
    }
  }
  const uint32_t base = (uint32_t)((size_t)chunk * CF::REC * sizeof(T));
#pragma unroll
  for (int ks = 0; ks < CF::KSC; ++ks) {
    // (blocks of keys past the row block are zero; loaded anyway, so the
    // number of loads in flight does not depend on the wave)
    load_rec_frag(o.r[ks], rs[2],
                    base + (uint32_t)((CF::WT + ((size_t)(rb * CF::KSC + ks) * 64 + lane) * 8) *
                                      sizeof(T)));
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a)
      load_rec_frag(o.w[a][ks], rs[2],
                    base + (uint32_t)((((size_t)((wv * CF::FPW + a) * CF::KSC + ks) * 64 + lane) *
                                       8) * sizeof(T)));
  }
#pragma unroll
  for (int b2 = 0; b2 < CF::TW; ++b2) {
    const int col = n0 + 16 * (ct0 + b2) + 4 * lg;
    if constexpr (VK) {
      o.v[b2] = buf_load4_raw(rs[3], tok_ok && col < p.dv
                                         ? (uint32_t)(((size_t)t * p.dv + col) * sizeof(T))
                                         : kOOB,
                              (T *)nullptr);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = tok_ok && col + e < p.dv;
        o.v[b2][e] = buf_load1(
            rs[3], ok ? (uint32_t)(((size_t)t * p.dv + col + e) * sizeof(T)) : kOOB, (T *)nullptr);
      }
    }
  }
  if constexpr (DECAY) {
    o.b_tok = buf_load1(rdec, (uint32_t)((chunk * C + 16 * rb + li) * 4), (float *)nullptr);
    o.b_last = buf_load1(rdec, (uint32_t)((chunk * C + C - 1) * 4), (float *)nullptr);
  } else {
    o.b_tok = o.b_last = 1.f;
  }
}

// This thread's k and q blocks of a register set into LDS tiles.
template <class CF>
__device__ __forceinline__ void seq_stage(const SeqOps<CF> &o, typename CF::type *K,
                                          typename CF::type *Q) {
  using V = typename CF::vec;
#pragma unroll
  for (int m = 0; m < SeqOps<CF>::NQ; ++m) {
    const int b = threadIdx.x + m * kThreads;
    const int row = b / CF::QCB, col0 = (b % CF::QCB) * CF::VEC;
    *reinterpret_cast<V *>(K + row * CF::QLD + col0) = o.kb[m];
    *reinterpret_cast<V *>(Q + row * CF::QLD + col0) = o.qb[m];
  }
}

template <class CF, bool VK, bool DECAY>
__global__ void __launch_bounds__(kThreads) seq_kernel(PrefillParams p, int nslices,
                                                       int xcd_map) {
  using T = typename CF::type;
  constexpr int C = CF::C, W = CF::W, NS = CF::NSET;
  __shared__ SmemSeq<CF> sm;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int rb = wv % CF::NRB, ct0 = (wv / CF::NRB) * CF::TW;

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
    const size_t tr = (size_t)nch * CF::REC;
    rs[2] = buf_rsrc(reinterpret_cast<const T *>(p.ws) + (size_t)bh * tr, (uint32_t)(tr * sizeof(T)));
    rs[3] = buf_rsrc(reinterpret_cast<const T *>(p.v) + (size_t)bh * vo, (uint32_t)(vo * sizeof(T)));
    rs[4] = buf_rsrc(reinterpret_cast<const T *>(p.o) + (size_t)bh * vo, (uint32_t)(vo * sizeof(T)));
  }
  // decay products b_j of every chunk of this head (written by prep)
  const __amdgpu_buffer_rsrc_t rdec = buf_rsrc(
      reinterpret_cast<const float *>(reinterpret_cast<const T *>(p.ws) +
                                      (size_t)p.BH * nch * CF::REC) + (size_t)bh * nch * C,
      (uint32_t)((size_t)nch * C * sizeof(float)));

  // Operands run NS - 1 chunks ahead: register set u serves chunks
  // u, u + NS, u + 2 NS, ... (the loop is unrolled by NS so every set index
  // is static) and is refilled with chunk c + NS as soon as chunk c is done.
  SeqOps<CF> set[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u)
    seq_fetch<CF, VK, DECAY>(set[u], p, rs, rdec, u, n0, wv, rb, ct0, lane);

  // fp32 state slice: wave holds row tiles tf = wv * FPW + a, every column tile
  f32x4 Sacc[CF::FPW][CF::NCT];
  const float *S0 = p.S_in ? p.S_in + (size_t)bh * d * dv : nullptr;
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
    for (int c = 0; c < CF::NCT; ++c) {
      const int n = n0 + 16 * c + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * (wv * CF::FPW + a) + 4 * lg + r;
        Sacc[a][c][r] = (S0 && f < d && n < dv) ? S0[(size_t)f * dv + n] : 0.f;
      }
    }
#pragma unroll
  for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
    for (int c = 0; c < CF::NCT; ++c)
      lds_store4(sm.St + (16 * c + li) * CF::QLD + 16 * (wv * CF::FPW + a) + 4 * lg,
                 Sacc[a][c][0], Sacc[a][c][1], Sacc[a][c][2], Sacc[a][c][3]);
  seq_stage<CF>(set[0], sm.K[0], sm.Q[0]);
  __syncthreads();

  // chunk c = (group) + u: k, q in LDS tile u; its other operands in set u.
  // At the end of the chunk the next chunk's k, q (set u1) go to tile u1,
  // last read two chunks earlier, and set u is refilled with chunk c + NS.
  auto step = [&](SeqOps<CF> &op, const SeqOps<CF> &opn, const T *Kt, const T *Qt, T *Kn,
                  T *Qn, const int c) {
    const int t = c * C + 16 * rb + li;  // this lane's token
    const bool tok_ok = t < N;

    // ---- X^T = S'^T K^T, Z^T = S'^T Q^T (rows n, columns: this row block) ----
    f32x4 X[CF::TW], Z[CF::TW];
#pragma unroll
    for (int b2 = 0; b2 < CF::TW; ++b2) {
      X[b2] = (f32x4){0.f, 0.f, 0.f, 0.f};
      Z[b2] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < CF::KSD; ++ks) {
#pragma unroll
      for (int b2 = 0; b2 < CF::TW; ++b2) {
        Frag<T> sf, kf, qf;
        lds_frag(kf, Kt + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
        lds_frag(qf, Qt + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
        lds_frag(sf, sm.St + (16 * (ct0 + b2) + li) * CF::QLD + 32 * ks + 8 * lg);
        mma(X[b2], sf, kf);
        mma(Z[b2], sf, qf);
      }
    }
    if (DECAY) {  // X and Q S- rows carry b of their token
#pragma unroll
      for (int b2 = 0; b2 < CF::TW; ++b2) {
        X[b2] *= op.b_tok;
        Z[b2] *= op.b_tok;
      }
    }
    // ---- Y = V - X: lane holds columns 16 ct + 4 lg + r of token t ----
#pragma unroll
    for (int b2 = 0; b2 < CF::TW; ++b2)
      lds_store4(sm.Ys + (16 * rb + li) * CF::YLD + 16 * (ct0 + b2) + 4 * lg,
                 to_f32(op.v[b2][0]) - X[b2][0], to_f32(op.v[b2][1]) - X[b2][1],
                 to_f32(op.v[b2][2]) - X[b2][2], to_f32(op.v[b2][3]) - X[b2][3]);
    __syncthreads();

    // ---- O^T = Z^T + Y^T R^T (keys j <= this row block) ----
#pragma unroll
    for (int ks = 0; ks < CF::KSC; ++ks) {
      if (32 * ks > 16 * rb + 15) continue;
#pragma unroll
      for (int b2 = 0; b2 < CF::TW; ++b2) {
        Frag<T> yf;
        lds_frag_tr(yf, sm.Ys, CF::YLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4,
                    16 * (ct0 + b2), li);
        mma(Z[b2], yf, op.r[ks]);
      }
    }
#pragma unroll
    for (int b2 = 0; b2 < CF::TW; ++b2) {
      const int col = n0 + 16 * (ct0 + b2) + 4 * lg;
      if constexpr (VK) {
        buf_store4_nt(rs[4],
                      tok_ok && col < dv ? (uint32_t)(((size_t)t * dv + col) * sizeof(T)) : kOOB,
                      Z[b2], (T *)nullptr);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool oke = tok_ok && col + e < dv;
          buf_store1(rs[4], oke ? (uint32_t)(((size_t)t * dv + col + e) * sizeof(T)) : kOOB,
                     from_f32<T>(Z[b2][e]));
        }
      }
    }
    // ---- S+ = b_L S- + Wt Y for this wave's state rows; T-precision copy ----
    if (DECAY) {
#pragma unroll
      for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
        for (int c2 = 0; c2 < CF::NCT; ++c2) Sacc[a][c2] *= op.b_last;
    }
#pragma unroll
    for (int ks = 0; ks < CF::KSC; ++ks) {
#pragma unroll
      for (int c2 = 0; c2 < CF::NCT; ++c2) {
        Frag<T> yf;
        lds_frag_tr(yf, sm.Ys, CF::YLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 16 * c2, li);
#pragma unroll
        for (int a = 0; a < CF::FPW; ++a) mma(Sacc[a][c2], op.w[a][ks], yf);
      }
    }
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
      for (int c2 = 0; c2 < CF::NCT; ++c2)
        lds_store4(sm.St + (16 * c2 + li) * CF::QLD + 16 * (wv * CF::FPW + a) + 4 * lg,
                   Sacc[a][c2][0], Sacc[a][c2][1], Sacc[a][c2][2], Sacc[a][c2][3]);
    seq_stage<CF>(opn, Kn, Qn);
    seq_fetch<CF, VK, DECAY>(op, p, rs, rdec, c + NS, n0, wv, rb, ct0, lane);
    __syncthreads();
  };
  // Whole groups of NS chunks without a branch between them: every load of
  // a register set is then followed by the loads of the other NS - 1 sets
  // before its use, and the compiler's wait counts let those stay in flight.
  int cb = 0;
  for (; cb + NS <= nch; cb += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int u1 = (u + 1) % NS;
      step(set[u], set[u1], sm.K[u], sm.Q[u], sm.K[u1], sm.Q[u1], cb + u);
    }
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) {
    const int u1 = (u + 1) % NS;
    if (cb + u < nch) step(set[u], set[u1], sm.K[u], sm.Q[u], sm.K[u1], sm.Q[u1], cb + u);
  }

  if (p.S_out) {
    float *So = p.S_out + (size_t)bh * d * dv;
#pragma unroll
    for (int a = 0; a < CF::FPW; ++a)
#pragma unroll
      for (int c = 0; c < CF::NCT; ++c) {
        const int n = n0 + 16 * c + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * (wv * CF::FPW + a) + 4 * lg + r;
          if (f < d && n < dv) So[(size_t)f * dv + n] = Sacc[a][c][r];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// seq2_kernel (bf16): the sequential pass with the work split by role.
// Eight waves: four chain waves (row block rb = wave) compute X = K S-,
// Y = V - X and the state update of their state rows, loading only k, Wt
// and v; four output waves (row block rb = wave - 4) compute Q S- and
// O = Q S- + R Y, loading only q and R.  Both read S' before the first
// barrier and Y after it; the chain waves write S' and the next chunk's k
// tile, the output waves its q tile, before the second.  The loads per
// chunk are those of seq_kernel; the chain waves issue less than half of
// them, and two waves share each SIMD.
// ---------------------------------------------------------------------------
constexpr int kThreads2 = 512;

template <class CF>
struct alignas(16) SmemSeq2 {
  using T = typename CF::type;
  T K[CF::NSET][CF::C * CF::QLD];  // k rows of the chunk of register set u
  T Q[CF::NSET][CF::C * CF::QLD];  // q rows
  T Ys[CF::C * CF::YLD];
  T St[CF::W * CF::QLD];
  float bs[CF::NSET][CF::C];       // decay products b_j of the chunk (with a decay)
};

// A role's share of one chunk's operands (256 threads stage its k or q).
template <class CF>
struct ChainOps {
  static constexpr int NB = CF::C * CF::QCB / kThreads;
  static_assert(NB * kThreads == CF::C * CF::QCB, "k blocks per thread");
  typename CF::vec kb[NB];
  Frag<typename CF::type> w[CF::FPW][CF::KSC];
  typename Vec4<typename CF::type>::type v;
};
// (with a decay, output wave 0 also loads the chunk's C decay products, one
// per lane, and stages them into LDS with the q tile: one load per chunk
// instead of one per wave and product)
template <class CF>
struct OutOps {
  static constexpr int NB = CF::C * CF::QCB / kThreads;
  typename CF::vec qb[NB];
  Frag<typename CF::type> r[CF::KSC];
  float bv;
};

// Whole-line 16-byte blocks of rows of q or k (thread rt of the role's 256).
template <class CF, bool VK, int NB>
__device__ __forceinline__ void load_rows(typename CF::vec (&x)[NB], __amdgpu_buffer_rsrc_t r,
                                          const PrefillParams &p, int chunk, int rt) {
  using T = typename CF::type;
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int b = rt + m * kThreads;
    const int row = chunk * CF::C + b / CF::QCB, col0 = (b % CF::QCB) * CF::VEC;
    if constexpr (VK) {
      x[m] = buf_load16<T>(r, (row < p.N && col0 < p.d)
                                  ? (uint32_t)(((size_t)row * p.d + col0) * sizeof(T)) : kOOB);
    } else {
#pragma unroll
      for (int e = 0; e < CF::VEC; ++e)
        x[m][e] = buf_load1(r, (row < p.N && col0 + e < p.d)
                                   ? (uint32_t)(((size_t)row * p.d + col0 + e) * sizeof(T))
                                   : kOOB, (T *)nullptr);
    }
  }
}
template <class CF, int NB>
__device__ __forceinline__ void stage_rows(const typename CF::vec (&x)[NB],
                                           typename CF::type *tile, int rt) {
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int b = rt + m * kThreads;
    *reinterpret_cast<typename CF::vec *>(tile + (b / CF::QCB) * CF::QLD +
                                          (b % CF::QCB) * CF::VEC) = x[m];
  }
}

template <class CF, bool VK, bool DECAY>
__global__ void __launch_bounds__(kThreads2) seq2_kernel(PrefillParams p, int nslices,
                                                         int xcd_map) {
  using T = typename CF::type;
  constexpr int C = CF::C, W = CF::W, NS = CF::NSET, FPW = CF::FPW, KSC = CF::KSC;
  static_assert(CF::NRB == 4 && CF::NCT == 1 && FPW * 4 == CF::NFT, "role split tiling");
  static_assert(C == kWave, "one decay product per lane of a wave");
  __shared__ SmemSeq2<CF> sm;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = wv < 4;
  const int rb = chain ? wv : wv - 4;  // row block; chain waves also own state rows
  const int rt = chain ? tid : tid - kThreads;  // thread index within the role
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;

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
    const size_t tr = (size_t)nch * CF::REC;
    rs[2] = buf_rsrc(reinterpret_cast<const T *>(p.ws) + (size_t)bh * tr, (uint32_t)(tr * sizeof(T)));
    rs[3] = buf_rsrc(reinterpret_cast<const T *>(p.v) + (size_t)bh * vo, (uint32_t)(vo * sizeof(T)));
    rs[4] = buf_rsrc(reinterpret_cast<const T *>(p.o) + (size_t)bh * vo, (uint32_t)(vo * sizeof(T)));
  }
  const __amdgpu_buffer_rsrc_t rdec = buf_rsrc(
      reinterpret_cast<const float *>(reinterpret_cast<const T *>(p.ws) +
                                      (size_t)p.BH * nch * CF::REC) + (size_t)bh * nch * C,
      (uint32_t)((size_t)nch * C * sizeof(float)));
  const int col = n0 + 4 * lg;  // this lane's four value columns

  if (chain) {
    auto fetch = [&](ChainOps<CF> &o, int chunk) {
      load_rows<CF, VK>(o.kb, rs[1], p, chunk, rt);
      const uint32_t base = (uint32_t)((size_t)chunk * CF::REC * sizeof(T));
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
        for (int a = 0; a < FPW; ++a)
          load_rec_frag(o.w[a][ks], rs[2],
                        base + (uint32_t)((((size_t)((rb * FPW + a) * KSC + ks) * 64 + lane) * 8) *
                                          sizeof(T)));
      const int t = chunk * C + 16 * rb + li;
      const bool ok = t < N;
      if constexpr (VK) {
        o.v = buf_load4_raw(rs[3], ok && col < dv ? (uint32_t)(((size_t)t * dv + col) * sizeof(T))
                                                  : kOOB, (T *)nullptr);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o.v[e] = buf_load1(rs[3], ok && col + e < dv
                                        ? (uint32_t)(((size_t)t * dv + col + e) * sizeof(T))
                                        : kOOB, (T *)nullptr);
      }
    };
    ChainOps<CF> set[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) fetch(set[u], u);
    f32x4 Sacc[FPW];
    const float *S0 = p.S_in ? p.S_in + (size_t)bh * d * dv : nullptr;
#pragma unroll
    for (int a = 0; a < FPW; ++a) {
      const int n = n0 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 16 * (rb * FPW + a) + 4 * lg + r;
        Sacc[a][r] = (S0 && f < d && n < dv) ? S0[(size_t)f * dv + n] : 0.f;
      }
      lds_store4(sm.St + li * CF::QLD + 16 * (rb * FPW + a) + 4 * lg, Sacc[a][0], Sacc[a][1],
                 Sacc[a][2], Sacc[a][3]);
    }
    stage_rows<CF>(set[0].kb, sm.K[0], rt);
    __syncthreads();

    auto step = [&](ChainOps<CF> &op, const ChainOps<CF> &opn, const T *Kt, T *Kn,
                    const float *bt, int c) {
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < CF::KSD; ++ks) {
        Frag<T> sf, kf;
        lds_frag(kf, Kt + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
        lds_frag(sf, sm.St + li * CF::QLD + 32 * ks + 8 * lg);
        mma(X, sf, kf);
      }
      float b_last = 1.f;
      if (DECAY) {
        X *= bt[16 * rb + li];
        b_last = bt[C - 1];
      }
      lds_store4(sm.Ys + (16 * rb + li) * CF::YLD + 4 * lg, to_f32(op.v[0]) - X[0],
                 to_f32(op.v[1]) - X[1], to_f32(op.v[2]) - X[2], to_f32(op.v[3]) - X[3]);
      __syncthreads();
      if (DECAY) {
#pragma unroll
        for (int a = 0; a < FPW; ++a) Sacc[a] *= b_last;
      }
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        Frag<T> yf;
        lds_frag_tr(yf, sm.Ys, CF::YLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 0, li);
#pragma unroll
        for (int a = 0; a < FPW; ++a) mma(Sacc[a], op.w[a][ks], yf);
      }
#pragma unroll
      for (int a = 0; a < FPW; ++a)
        lds_store4(sm.St + li * CF::QLD + 16 * (rb * FPW + a) + 4 * lg, Sacc[a][0], Sacc[a][1],
                   Sacc[a][2], Sacc[a][3]);
      stage_rows<CF>(opn.kb, Kn, rt);
      fetch(op, c + NS);
      __syncthreads();
    };
    int cb = 0;
    for (; cb + NS <= nch; cb += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int u1 = (u + 1) % NS;
        step(set[u], set[u1], sm.K[u], sm.K[u1], sm.bs[u], cb + u);
      }
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      const int u1 = (u + 1) % NS;
      if (cb + u < nch) step(set[u], set[u1], sm.K[u], sm.K[u1], sm.bs[u], cb + u);
    }
    if (p.S_out) {
      float *So = p.S_out + (size_t)bh * d * dv;
#pragma unroll
      for (int a = 0; a < FPW; ++a) {
        const int n = n0 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * (rb * FPW + a) + 4 * lg + r;
          if (f < d && n < dv) So[(size_t)f * dv + n] = Sacc[a][r];
        }
      }
    }
  } else {
    auto fetch = [&](OutOps<CF> &o, int chunk) {
      load_rows<CF, VK>(o.qb, rs[0], p, chunk, rt);
      const uint32_t base = (uint32_t)((size_t)chunk * CF::REC * sizeof(T));
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks)  // (blocks past the row block are zero)
        load_rec_frag(o.r[ks], rs[2],
                      base + (uint32_t)((CF::WT + ((size_t)(rb * KSC + ks) * 64 + lane) * 8) *
                                        sizeof(T)));
      if (DECAY && rb == 0)  // past the last chunk: zeros (never used)
        o.bv = buf_load1(rdec, (uint32_t)((chunk * C + lane) * 4), (float *)nullptr);
    };
    auto stage_b = [&](const OutOps<CF> &o, float *dst) {
      if (DECAY && rb == 0) dst[lane] = o.bv;
    };
    OutOps<CF> set[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) fetch(set[u], u);
    stage_rows<CF>(set[0].qb, sm.Q[0], rt);
    stage_b(set[0], sm.bs[0]);
    __syncthreads();

    auto step = [&](OutOps<CF> &op, const OutOps<CF> &opn, const T *Qt, T *Qn, const float *bt,
                    float *bn, int c) {
      const int t = c * C + 16 * rb + li;
      f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < CF::KSD; ++ks) {
        Frag<T> sf, qf;
        lds_frag(qf, Qt + (16 * rb + li) * CF::QLD + 32 * ks + 8 * lg);
        lds_frag(sf, sm.St + li * CF::QLD + 32 * ks + 8 * lg);
        mma(Z, sf, qf);
      }
      if (DECAY) Z *= bt[16 * rb + li];
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        if (32 * ks > 16 * rb + 15) continue;
        Frag<T> yf;
        lds_frag_tr(yf, sm.Ys, CF::YLD, 32 * ks + 8 * lg, 32 * ks + 8 * lg + 4, 0, li);
        mma(Z, yf, op.r[ks]);
      }
      if constexpr (VK) {
        buf_store4_nt(rs[4], t < N && col < dv ? (uint32_t)(((size_t)t * dv + col) * sizeof(T))
                                               : kOOB, Z, (T *)nullptr);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_store1(rs[4], t < N && col + e < dv
                                ? (uint32_t)(((size_t)t * dv + col + e) * sizeof(T)) : kOOB,
                     from_f32<T>(Z[e]));
      }
      stage_rows<CF>(opn.qb, Qn, rt);
      stage_b(opn, bn);
      fetch(op, c + NS);
      __syncthreads();
    };
    int cb = 0;
    for (; cb + NS <= nch; cb += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int u1 = (u + 1) % NS;
        step(set[u], set[u1], sm.Q[u], sm.Q[u1], sm.bs[u], sm.bs[u1], cb + u);
      }
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      const int u1 = (u + 1) % NS;
      if (cb + u < nch) step(set[u], set[u1], sm.Q[u], sm.Q[u1], sm.bs[u], sm.bs[u1], cb + u);
    }
  }
}

template <class CF, bool VK, bool DECAY>
hipError_t run_vkd(const PrefillParams &p, hipStream_t s) {
  static_assert(sizeof(SmemPrep<CF>) <= 64 * 1024, "LDS budget (prep)");
  static_assert(sizeof(SmemSeq<CF>) <= 160 * 1024, "LDS budget (seq)");
  const int nch = (p.N + CF::C - 1) / CF::C;
  hipError_t e = launch_kernel("delta_prep", prep_kernel<CF, VK, DECAY>, head_grid(nch, p.BH),
                               dim3(kThreads), s, p);
  if (e != hipSuccess) return e;
  const int nsl = (p.dv + CF::W - 1) / CF::W;
  const int xcd_map = (p.BH % kXcds) == 0;
  if constexpr (CF::NRB == 4 && CF::NCT == 1) {  // bf16: waves split by role
    static_assert(sizeof(SmemSeq2<CF>) <= 160 * 1024, "LDS budget (seq2)");
    return launch_kernel("delta_seq", seq2_kernel<CF, VK, DECAY>, dim3(p.BH * nsl),
                         dim3(kThreads2), s, p, nsl, xcd_map);
  } else {
    return launch_kernel("delta_seq", seq_kernel<CF, VK, DECAY>, dim3(p.BH * nsl),
                         dim3(kThreads), s, p, nsl, xcd_map);
  }
}

// the decay-free rule gets its own instantiation (no decay work compiled in)
template <class CF, bool VK>
hipError_t run_vk(const PrefillParams &p, hipStream_t s) {
  return p.alpha ? run_vkd<CF, VK, true>(p, s) : run_vkd<CF, VK, false>(p, s);
}

template <class CF>
hipError_t run(const PrefillParams &p, hipStream_t s) {
  return p.vec_ok ? run_vk<CF, true>(p, s) : run_vk<CF, false>(p, s);
}

// bf16: 64-token chunks, 16-column slices; fp32: 32-token chunks,
// 32-column slices.
using DB64 = DCfg<bf16, 64, 64, 16>;
using DB128 = DCfg<bf16, 128, 64, 16>;
using DF64 = DCfg<float, 64, 32, 32>;
using DF128 = DCfg<float, 128, 32, 32>;

}  // namespace

size_t delta_workspace_bytes(int BH, int N, int d, bool bf16_io) {
  const int C = bf16_io ? DB64::C : DF64::C;
  const size_t DK = d <= 64 ? 64 : 128;
  const size_t nch = ((size_t)N + C - 1) / C;
  // per chunk: the [Wt | R] record in the input precision, then (after all
  // records) C fp32 decay products b_j, used when a decay is given
  return (size_t)BH * nch * ((DK * C + (size_t)C * C) * (bf16_io ? 2 : 4) + (size_t)C * 4);
}

hipError_t launch_delta_prefill(const PrefillParams &p, bool bf16_io, hipStream_t s) {
  if (bf16_io) return p.d <= 64 ? run<DB64>(p, s) : run<DB128>(p, s);
  return p.d <= 64 ? run<DF64>(p, s) : run<DF128>(p, s);
}

}  // namespace la
