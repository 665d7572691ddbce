// Short causal convolution of q, k and v as a pass of its own (ahead of the
// gated DELTA rule, and of the LINEAR rule's training forward), and its
// backward.
//
// "What Is Linear Attention?" section 5.4 puts a short convolution over the
// most recent tokens in front of the linear layer (beside the decay, the
// delta update and the gate) and keeps those tokens as a conv cache next to
// the state.  Per head h and channel c of [q | k | v] (2d + dv channels),
// with filter taps W[h][j][c], tap w-1 on the current token:
//     y_t[c] = sum_{j=0..w-1} W[h][j][c] x_(t-(w-1)+j)[c]
// where tokens before the sequence come from the conv cache (rows oldest
// first) or are zero without one.  The LINEAR prefill fuses this into its
// chunk loads; the delta rule reads q, k and v in two kernels (the
// preparation pass and the sequential pass, which stages them differently),
// and the LINEAR training forward hands the convolved inputs on to its
// backward, so for those the convolved q, k, v are written once, in the
// input precision, to the workspace, and the rule runs on those copies.  The sums are taken
// in fp32 in tap order and rounded once, as the matrix cores would take
// them.
//
// conv_qkv_kernel: one thread per (token, E consecutive channels) of one of
// q, k, v (E = 16 bytes of channels where every row allows it, else 1);
// heads along grid y/z.  conv_cache_kernel, launched after it (so the cache
// may be updated in place): one thread per (head, channel) walks the w-1
// cache rows oldest first, so a row is read before it is overwritten.
#include "la_common.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kConvThreads = 256;
constexpr int kMaxConvW = 4;  // widest filter

template <typename T, int E>
__device__ __forceinline__ void load_e(const T *src, float (&x)[E]) {
  if constexpr (E * sizeof(T) == 16) {
    const typename Vec16<T>::type v = *reinterpret_cast<const typename Vec16<T>::type *>(src);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = to_f32(v[e]);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = to_f32(src[e]);
  }
}

template <typename T, int E>
__global__ void __launch_bounds__(kConvThreads) conv_qkv_kernel(ConvParams p) {
  const int bh = grid_head();
  if (bh >= p.BH) return;
  const int d = p.d, dv = p.dv, w = p.width, N = p.N;
  const int wc = 2 * d + dv;
  const int nb = wc / E;  // E divides d and dv
  const size_t idx = (size_t)blockIdx.x * kConvThreads + threadIdx.x;
  if (idx >= (size_t)N * nb) return;
  const int t = (int)(idx / nb), c0 = (int)(idx % nb) * E;
  const T *x;
  T *y;
  int c, ld;
  if (c0 < d) {
    x = reinterpret_cast<const T *>(p.q); y = reinterpret_cast<T *>(p.yq); c = c0; ld = d;
  } else if (c0 < 2 * d) {
    x = reinterpret_cast<const T *>(p.k); y = reinterpret_cast<T *>(p.yk); c = c0 - d; ld = d;
  } else {
    x = reinterpret_cast<const T *>(p.v); y = reinterpret_cast<T *>(p.yv); c = c0 - 2 * d;
    ld = dv;
  }
  x += (size_t)bh * N * ld + c;
  y += (size_t)bh * N * ld + (size_t)t * ld + c;
  const float *W = p.w + (size_t)(bh % p.H) * w * wc + c0;
  const T *cache =
      p.cache_in ? reinterpret_cast<const T *>(p.cache_in) + (size_t)bh * (w - 1) * wc + c0
                 : nullptr;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int j = 0; j < w; ++j) {
    const int src = t - (w - 1) + j;  // token index; below 0: cache row w-1+src
    float xv[E];
    if (src >= 0) {
      load_e<T, E>(x + (size_t)src * ld, xv);
    } else if (cache) {
      load_e<T, E>(cache + (size_t)(w - 1 + src) * wc, xv);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) xv[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(W[(size_t)j * wc + e], xv[e], acc[e]);
  }
  if constexpr (E * sizeof(T) == 16) {
    typename Vec16<T>::type out;
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = from_f32<T>(acc[e]);
    *reinterpret_cast<typename Vec16<T>::type *>(y) = out;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = from_f32<T>(acc[e]);
  }
}

// The conv cache after the sequence: the last w-1 raw tokens of the cache
// before it followed by the sequence.
template <typename T>
__global__ void __launch_bounds__(kConvThreads) conv_cache_kernel(ConvParams p) {
  const int d = p.d, dv = p.dv, w = p.width, N = p.N;
  const int wc = 2 * d + dv;
  const size_t idx = (size_t)blockIdx.x * kConvThreads + threadIdx.x;
  if (idx >= (size_t)p.BH * wc) return;
  const int bh = (int)(idx / wc), ch = (int)(idx % wc);
  const T *x;
  int c, ld;
  if (ch < d) {
    x = reinterpret_cast<const T *>(p.q); c = ch; ld = d;
  } else if (ch < 2 * d) {
    x = reinterpret_cast<const T *>(p.k); c = ch - d; ld = d;
  } else {
    x = reinterpret_cast<const T *>(p.v); c = ch - 2 * d; ld = dv;
  }
  x += (size_t)bh * N * ld + c;
  const T *cin =
      p.cache_in ? reinterpret_cast<const T *>(p.cache_in) + (size_t)bh * (w - 1) * wc + ch
                 : nullptr;
  T *cout = reinterpret_cast<T *>(p.cache_out) + (size_t)bh * (w - 1) * wc + ch;
  for (int r = 0; r < w - 1; ++r) {  // new row r is token N-(w-1)+r
    const int src = N - (w - 1) + r;
    T val;
    if (src >= 0) val = x[(size_t)src * ld];
    else val = cin ? cin[(size_t)(w - 1 + src) * wc] : T{};  // old row N + r > r
    cout[(size_t)r * wc] = val;
  }
}

// ---- backward ---------------------------------------------------------------
// With x~ = [cache | x] (row r is token r - (w-1)) and y_s = sum_j W_j x~_(s+j):
//   dx~_r = sum_j W_j dy_(r-j)   (0 <= r - j < N), plus dL/d(returned cache)
//           on the last w-1 rows of x~;
//   dW_j  = sum over sequences and s of dy_s x~_(s+j)   (per head, channel).
// conv_dx_kernel: one thread per (row r of x~, channel) of one of q, k, v
// (rows before the sequence give the cache gradient, when asked for).
// conv_dw_partial_kernel: one thread per (sequence, token block, channel),
// the block's sums for every tap; conv_dw_reduce_kernel adds the blocks of a
// head in a fixed order.
template <typename T>
__device__ __forceinline__ void conv_channel_ptrs(const ConvBwdParams &p, int bh, int ch,
                                                  const T *&x, const T *&dy, T *&dx, int &c,
                                                  int &ld) {
  const int d = p.d, dv = p.dv;
  int which;
  if (ch < d) { which = 0; c = ch; ld = d; }
  else if (ch < 2 * d) { which = 1; c = ch - d; ld = d; }
  else { which = 2; c = ch - 2 * d; ld = dv; }
  const size_t base = (size_t)bh * p.N * ld + c;
  x = reinterpret_cast<const T *>(which == 0 ? p.q : which == 1 ? p.k : p.v) + base;
  dy = reinterpret_cast<const T *>(which == 0 ? p.dyq : which == 1 ? p.dyk : p.dyv) + base;
  dx = reinterpret_cast<T *>(which == 0 ? p.dq : which == 1 ? p.dk : p.dv_) + base;
}

template <typename T>
__global__ void __launch_bounds__(kConvThreads) conv_dx_kernel(ConvBwdParams p) {
  const int bh = grid_head();
  if (bh >= p.BH) return;
  const int w = p.width, N = p.N, wc = 2 * p.d + p.dv;
  const size_t idx = (size_t)blockIdx.x * kConvThreads + threadIdx.x;
  const size_t rows = (size_t)N + w - 1;  // rows of x~
  if (idx >= rows * wc) return;
  const int r = (int)(idx / wc), ch = (int)(idx % wc);
  if (r < w - 1 && !p.dcache_in) return;  // no cache gradient asked for
  const T *x, *dy;
  T *dx;
  int c, ld;
  conv_channel_ptrs<T>(p, bh, ch, x, dy, dx, c, ld);
  (void)x;
  const float *W = p.w + (size_t)(bh % p.H) * w * wc + ch;
  float acc = 0.f;
  for (int j = 0; j < w; ++j) {
    const int s = r - j;
    if (s >= 0 && s < N) acc = fmaf(W[(size_t)j * wc], to_f32(dy[(size_t)s * ld]), acc);
  }
  const size_t crow = (size_t)bh * (w - 1) * wc + ch;
  const int r_out = r - (N + w - 1 - (w - 1));  // row of the returned cache (last w-1 of x~)
  if (p.dcache_out && r_out >= 0)
    acc += to_f32(reinterpret_cast<const T *>(p.dcache_out)[crow + (size_t)r_out * wc]);
  if (r >= w - 1)
    dx[(size_t)(r - (w - 1)) * ld] = from_f32<T>(acc);
  else
    reinterpret_cast<T *>(p.dcache_in)[crow + (size_t)r * wc] = from_f32<T>(acc);
}

constexpr int kDwTokens = 256;  // tokens per partial sum of the filter gradient

template <typename T>
__global__ void __launch_bounds__(kConvThreads) conv_dw_partial_kernel(ConvBwdParams p) {
  const int w = p.width, N = p.N, wc = 2 * p.d + p.dv;
  const int nblk = (N + kDwTokens - 1) / kDwTokens;
  const int bh = grid_head();
  if (bh >= p.BH) return;
  const int blk = blockIdx.x % nblk;
  const int ch = (blockIdx.x / nblk) * kConvThreads + threadIdx.x;
  if (ch >= wc) return;
  const T *x, *dy;
  T *dx;
  int c, ld;
  conv_channel_ptrs<T>(p, bh, ch, x, dy, dx, c, ld);
  (void)dx;
  const T *cache = p.cache_in ? reinterpret_cast<const T *>(p.cache_in) +
                                    (size_t)bh * (w - 1) * wc + ch
                              : nullptr;
  float acc[kMaxConvW];
#pragma unroll
  for (int j = 0; j < kMaxConvW; ++j) acc[j] = 0.f;
  const int s0 = blk * kDwTokens, s1 = min(N, s0 + kDwTokens);
  for (int s = s0; s < s1; ++s) {
    const float g = to_f32(dy[(size_t)s * ld]);
#pragma unroll
    for (int j = 0; j < kMaxConvW; ++j) {
      if (j < w) {
        const int t = s + j - (w - 1);  // token of x~ row s + j
        const float xv = t >= 0 ? to_f32(x[(size_t)t * ld])
                         : cache ? to_f32(cache[(size_t)(w - 1 + t) * wc]) : 0.f;
        acc[j] = fmaf(g, xv, acc[j]);
      }
    }
  }
  float *out = p.dw_part + ((size_t)bh * nblk + blk) * w * wc + ch;
  for (int j = 0; j < w; ++j) out[(size_t)j * wc] = acc[j];
}

__global__ void __launch_bounds__(kConvThreads) conv_dw_reduce_kernel(ConvBwdParams p) {
  const int w = p.width, wc = 2 * p.d + p.dv;
  const int nblk = (p.N + kDwTokens - 1) / kDwTokens;
  const size_t idx = (size_t)blockIdx.x * kConvThreads + threadIdx.x;
  if (idx >= (size_t)p.H * w * wc) return;
  const int h = (int)(idx / ((size_t)w * wc));
  const size_t jc = idx % ((size_t)w * wc);
  const int B = p.BH / p.H;
  float acc = 0.f;
  for (int b = 0; b < B; ++b)
    for (int k = 0; k < nblk; ++k)
      acc += p.dw_part[(((size_t)b * p.H + h) * nblk + k) * w * wc + jc];
  p.dw[idx] = acc;
}

template <typename T>
hipError_t run_bwd(const ConvBwdParams &p, hipStream_t s) {
  const int wc = 2 * p.d + p.dv;
  const size_t rows = (size_t)p.N + p.width - 1;
  hipError_t e = launch_kernel(
      "conv_dx", conv_dx_kernel<T>,
      head_grid((unsigned)((rows * wc + kConvThreads - 1) / kConvThreads), p.BH),
      dim3(kConvThreads), s, p);
  if (e != hipSuccess || p.N == 0) return e;
  const int nblk = (p.N + kDwTokens - 1) / kDwTokens;
  const unsigned ncb = (unsigned)((wc + kConvThreads - 1) / kConvThreads);
  e = launch_kernel("conv_dw", conv_dw_partial_kernel<T>, head_grid(ncb * nblk, p.BH),
                    dim3(kConvThreads), s, p);
  if (e != hipSuccess) return e;
  const size_t nw = (size_t)p.H * p.width * wc;
  return launch_kernel("conv_dw_reduce", conv_dw_reduce_kernel,
                       dim3((unsigned)((nw + kConvThreads - 1) / kConvThreads)),
                       dim3(kConvThreads), s, p);
}

template <typename T>
hipError_t run(const ConvParams &p, bool vec, hipStream_t s) {
  constexpr int EV = 16 / (int)sizeof(T);
  const int wc = 2 * p.d + p.dv;
  hipError_t e;
  if (vec) {
    const unsigned nx = (unsigned)(((size_t)p.N * (wc / EV) + kConvThreads - 1) / kConvThreads);
    e = launch_kernel("conv_qkv", conv_qkv_kernel<T, EV>, head_grid(nx, p.BH),
                      dim3(kConvThreads), s, p);
  } else {
    const unsigned nx = (unsigned)(((size_t)p.N * wc + kConvThreads - 1) / kConvThreads);
    e = launch_kernel("conv_qkv", conv_qkv_kernel<T, 1>, head_grid(nx, p.BH),
                      dim3(kConvThreads), s, p);
  }
  if (e != hipSuccess || !p.cache_out || p.width < 2) return e;
  const unsigned nc = (unsigned)(((size_t)p.BH * wc + kConvThreads - 1) / kConvThreads);
  return launch_kernel("conv_cache", conv_cache_kernel<T>, dim3(nc), dim3(kConvThreads), s, p);
}

}  // namespace

hipError_t launch_conv_qkv(const ConvParams &p, bool bf16_io, bool vec, hipStream_t s) {
  return bf16_io ? run<bf16>(p, vec, s) : run<float>(p, vec, s);
}

size_t conv_dw_partial_floats(int BH, int N, int d, int dv, int width) {
  const size_t nblk = ((size_t)N + kDwTokens - 1) / kDwTokens;
  return (size_t)BH * nblk * width * (2 * (size_t)d + dv);
}

hipError_t launch_conv_backward(const ConvBwdParams &p, bool bf16_io, hipStream_t s) {
  return bf16_io ? run_bwd<bf16>(p, s) : run_bwd<float>(p, s);
}

}  // namespace la
