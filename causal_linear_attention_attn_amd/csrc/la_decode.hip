// Single-token decode step against a persistent fp32 state, updated in place.
//
// LINEAR ("What Is Linear Attention?" section 4 with the decay of 5.1;
// "LLM inference optimisation (3)", recurrent form: read once, add once):
//     S <- gamma S + phi(k) v^T,  z <- gamma z + phi(k)
//     o  = S^T phi(q) / (phi(q) . z + eps)
//   or, with a per-key-channel decay ("Efficient attention variants" 7.2,
//   GLA), gamma replaced by alpha_r on row r of S and entry r of z.
// DELTA ("What Is Linear Attention?" 5.2-5.3), with the optional scalar
// decay alpha of Gated DeltaNet ("Efficient attention variants" 7.4: decay
// first, the error is taken on the decayed state):
//     b = S^T k,  u = v - alpha b,  S <- alpha S + g k u^T,
//     o = S_new^T q = alpha S_old^T q + g (k . q) u
//
// With a short causal convolution ("What Is Linear Attention?" 5.4; either
// rule, the CV instantiations) q, k and v are first convolved with the w-1
// raw tokens of the conv cache, which then shifts by one token: thread t
// owns channel t of q, k and v in every cache row, so the in-place update
// needs no synchronisation.
//
// The step is bound by HBM: each (b,h) state block (d x dv fp32, 64 KiB at
// d = dv = 128) is read once and written once.  One workgroup of 256 threads
// owns one block; consecutive threads own consecutive VEC-wide column groups
// of a row, so each wave moves whole rows (coalesced dwordx4 traffic), and
// each thread walks rows rg, rg + RG, ... .  All of a thread's rows are
// loaded before any is used so that every load is in flight at once, and the
// block's loads are issued before the token's q, k, v are read.  Column
// sums (the reads S^T phi(q), S^T k, S^T q) are reduced across the RG row
// groups through LDS in a fixed order: no atomics, deterministic.
#include "la_common.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kDecThreads = 256;

__device__ __forceinline__ float block_sum(float x, float *red) {
  // all threads of a 256-thread block call this; returns the sum everywhere
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Channel c of one token through the short convolution: the filter's taps
// run over the cache rows (oldest first) and then x; the cache moves up one
// row and x becomes its last row.  Same fp32 chain as the prefill.
template <typename T>
__device__ __forceinline__ float conv_channel(T *cache, const float *W, int w, int wc,
                                              int c, T x) {
  constexpr int kHalo = 3;  // widest filter minus one
  T old[kHalo];
#pragma unroll
  for (int j = 0; j < kHalo; ++j) old[j] = j < w - 1 ? cache[(size_t)j * wc + c] : T{};
  float y = 0.f;
#pragma unroll
  for (int j = 0; j < kHalo; ++j)
    if (j < w - 1) y = fmaf(W[(size_t)j * wc + c], to_f32(old[j]), y);
  y = fmaf(W[(size_t)(w - 1) * wc + c], to_f32(x), y);
#pragma unroll
  for (int j = 0; j + 1 < kHalo; ++j)
    if (j + 1 < w - 1) cache[(size_t)j * wc + c] = old[j + 1];
  if (w > 1) cache[(size_t)(w - 2) * wc + c] = x;
  return y;
}

template <typename T, int VEC, bool DELTA, bool CV>
__global__ void __launch_bounds__(kDecThreads)
decode_kernel(DecodeParams p) {
  constexpr int ROWS = 64 / VEC;  // rows per thread at most (d <= 128)
  __shared__ float s_q[LA_MAXD], s_k[LA_MAXD], s_v[LA_MAXD], s_al[LA_MAXD];
  __shared__ float s_part[2][kDecThreads * VEC];
  __shared__ float s_a[LA_MAXD], s_b[LA_MAXD];
  __shared__ float s_red[4];

  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const int d = p.d, dv = p.dv;
  const int colsv = dv / VEC;          // column groups per row
  const int RG = kDecThreads / colsv;  // row groups
  const int cv = t % colsv, rg = t / colsv;
  const bool active = rg < RG;
  const int c0 = cv * VEC;

  // The state block goes out first: its loads are in flight while the
  // token's q, k, v arrive (those are tiny, but a full memory latency).
  const size_t blk = (size_t)d * dv;
  const __amdgpu_buffer_rsrc_t rS = buf_rsrc(p.S + (size_t)bh * blk, (uint32_t)(blk * 4));
  float sr[ROWS][VEC];
#pragma unroll
  for (int m = 0; m < ROWS; ++m) {
    const int r = rg + RG * m;
    const bool ok = active && r < d;
    const uint32_t off = ok ? (uint32_t)(((size_t)r * dv + c0) * 4) : kOOB;
    if constexpr (VEC == 4) {
      const f32x4 x = buf_load16<float>(rS, off);
#pragma unroll
      for (int e = 0; e < 4; ++e) sr[m][e] = x[e];
    } else {
      sr[m][0] = buf_load1(rS, off, (float *)nullptr);
    }
  }

  const T *q = reinterpret_cast<const T *>(p.q) + (size_t)bh * d;
  const T *k = reinterpret_cast<const T *>(p.k) + (size_t)bh * d;
  const T *v = reinterpret_cast<const T *>(p.v) + (size_t)bh * dv;
  [[maybe_unused]] const int wc = 2 * d + dv;
  [[maybe_unused]] T *ccache = nullptr;
  [[maybe_unused]] const float *cw = nullptr;
  if constexpr (CV) {
    ccache = reinterpret_cast<T *>(p.conv_cache) + (size_t)bh * (p.conv_width - 1) * wc;
    cw = p.conv_w + (size_t)(bh % p.H) * p.conv_width * wc;
  }
  float zold = 0.f;
  if (t < d) {
    float xq, xk;
    if constexpr (CV) {
      xq = conv_channel<T>(ccache, cw, p.conv_width, wc, t, q[t]);
      xk = conv_channel<T>(ccache, cw, p.conv_width, wc, d + t, k[t]);
    } else {
      xq = to_f32(q[t]);
      xk = to_f32(k[t]);
    }
    if (!DELTA && p.fmap) { xq = phi_elu1(xq); xk = phi_elu1(xk); }
    s_q[t] = xq;
    s_k[t] = xk;
    if (!DELTA) zold = p.z[(size_t)bh * d + t];
    if (!DELTA) s_al[t] = p.alpha ? p.alpha[(size_t)bh * d + t] : 1.f;
  }
  if (t < dv) {
    if constexpr (CV) s_v[t] = conv_channel<T>(ccache, cw, p.conv_width, wc, 2 * d + t, v[t]);
    else s_v[t] = to_f32(v[t]);
  }
  const float gam = (!DELTA && p.gamma) ? p.gamma[bh % p.H] : 1.f;
  const bool chan = !DELTA && p.alpha != nullptr;  // per-channel decay
  const float gate = DELTA ? p.g[bh] : 0.f;
  const float al = (DELTA && p.alpha) ? p.alpha[bh] : 1.f;
  __syncthreads();

  float acc[VEC], acc2[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) { acc[e] = 0.f; acc2[e] = 0.f; }

  if constexpr (!DELTA) {
    // update in place (each row stored as soon as it is done) and
    // accumulate phi(q)^T S_new for this thread's columns
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
      const int r = rg + RG * m;
      const bool ok = active && r < d;
      const float fk = ok ? s_k[r] : 0.f, fq = ok ? s_q[r] : 0.f;
      const float gr = chan ? (ok ? s_al[r] : 1.f) : gam;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float sn = fmaf(gr, sr[m][e], fk * s_v[c0 + e]);
        sr[m][e] = sn;
        acc[e] = fmaf(fq, sn, acc[e]);
      }
      const uint32_t off = ok ? (uint32_t)(((size_t)r * dv + c0) * 4) : kOOB;
      if constexpr (VEC == 4)
        buf_store16_nt<float>(rS, off, (f32x4){sr[m][0], sr[m][1], sr[m][2], sr[m][3]});
      else
        buf_store1(rS, off, sr[m][0]);
    }
    // normaliser: z <- gamma z + phi(k); den = phi(q) . z_new
    float dz = 0.f;
    if (t < d) {
      const float zn = fmaf(chan ? s_al[t] : gam, zold, s_k[t]);
      p.z[(size_t)bh * d + t] = zn;
      dz = s_q[t] * zn;
    }
    const float den = block_sum(dz, s_red) + p.eps;
    if (active) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_part[0][rg * dv + c0 + e] = acc[e];
    }
    __syncthreads();
    if (t < dv) {
      float num = 0.f;
      for (int r2 = 0; r2 < RG; ++r2) num += s_part[0][r2 * dv + t];
      reinterpret_cast<T *>(p.o)[(size_t)bh * dv + t] = from_f32<T>(num / den);
    }
  } else {
    // column dots of the OLD state with k and q, from the same read
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
      const int r = rg + RG * m;
      const bool ok = active && r < d;
      const float kr = ok ? s_k[r] : 0.f, qr = ok ? s_q[r] : 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        acc[e] = fmaf(kr, sr[m][e], acc[e]);
        acc2[e] = fmaf(qr, sr[m][e], acc2[e]);
      }
    }
    const float qk = block_sum(t < d ? s_q[t] * s_k[t] : 0.f, s_red);
    if (active) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        s_part[0][rg * dv + c0 + e] = acc[e];
        s_part[1][rg * dv + c0 + e] = acc2[e];
      }
    }
    __syncthreads();
    if (t < dv) {
      float b = 0.f, a = 0.f;
      for (int r2 = 0; r2 < RG; ++r2) {
        b += s_part[0][r2 * dv + t];
        a += s_part[1][r2 * dv + t];
      }
      const float u = fmaf(-al, b, s_v[t]);  // residual v - alpha S_old^T k
      s_b[t] = u;
      s_a[t] = a;
      reinterpret_cast<T *>(p.o)[(size_t)bh * dv + t] =
          from_f32<T>(fmaf(gate * qk, u, al * a));
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
      const int r = rg + RG * m;
      const bool ok = active && r < d;
      const float gk = ok ? gate * s_k[r] : 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) sr[m][e] = fmaf(gk, s_b[c0 + e], al * sr[m][e]);
      const uint32_t off = ok ? (uint32_t)(((size_t)r * dv + c0) * 4) : kOOB;
      if constexpr (VEC == 4)
        buf_store16_nt<float>(rS, off, (f32x4){sr[m][0], sr[m][1], sr[m][2], sr[m][3]});
      else
        buf_store1(rS, off, sr[m][0]);
    }
  }
}

__global__ void fill_kernel(float *dst, size_t n, float value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = value;
}

__global__ void zero_bytes_kernel(unsigned char *dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = 0;
}

__global__ void copy_bytes_kernel(unsigned char *dst, const unsigned char *src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void copy_kernel(float *dst, const float *src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

template <typename T, int VEC, bool DELTA>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t s) {
  if (p.conv_w)
    return launch_kernel(DELTA ? "delta_decode" : "linear_decode",
                         decode_kernel<T, VEC, DELTA, true>, dim3(p.BH), dim3(kDecThreads), s, p);
  return launch_kernel(DELTA ? "delta_decode" : "linear_decode",
                       decode_kernel<T, VEC, DELTA, false>, dim3(p.BH), dim3(kDecThreads), s, p);
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, bool bf16_io, bool delta,
                         int vec, hipStream_t s) {
  if (bf16_io) {
    if (delta) return vec == 4 ? launch_decode_t<bf16, 4, true>(p, s)
                               : launch_decode_t<bf16, 1, true>(p, s);
    return vec == 4 ? launch_decode_t<bf16, 4, false>(p, s)
                    : launch_decode_t<bf16, 1, false>(p, s);
  }
  if (delta) return vec == 4 ? launch_decode_t<float, 4, true>(p, s)
                             : launch_decode_t<float, 1, true>(p, s);
  return vec == 4 ? launch_decode_t<float, 4, false>(p, s)
                  : launch_decode_t<float, 1, false>(p, s);
}

hipError_t launch_fill(float *dst, size_t n, float value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst,
                     n, value);
  return hipGetLastError();
}

hipError_t launch_zero_bytes(void *dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_bytes_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<unsigned char *>(dst), n);
  return hipGetLastError();
}

hipError_t launch_copy_bytes(void *dst, const void *src, size_t n, hipStream_t s) {
  if (n == 0 || dst == src) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_bytes_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<unsigned char *>(dst), static_cast<const unsigned char *>(src),
                     n);
  return hipGetLastError();
}

hipError_t launch_copy(float *dst, const float *src, size_t n, hipStream_t s) {
  if (n == 0 || dst == src) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst,
                     src, n);
  return hipGetLastError();
}

}  // namespace la
