// Device helpers shared by the linattn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Head of a workgroup in a grid built by head_grid (la_internal.hpp).
__device__ __forceinline__ int grid_head() {
  return (int)(blockIdx.y + 65535u * blockIdx.z);
}
constexpr int LA_MAXD = 128;  // largest d and dv

// ---------------------------------------------------------------------------
// Element conversion.  bf16 -> f32 is exact; f32 -> bf16 rounds to nearest
// even (v_cvt_pk_bf16_f32 on gfx950).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// elu(x)+1 with alpha 1: x+1 above zero, e^x at or below, written as
// max(x + 1, e^-|x|).  The two agree exactly in real arithmetic: for x <= 0,
// e^x >= 1 + x; for x > 0, e^-x < 1 < 1 + x.  No positive exponent is
// formed, and the form needs no compare-and-select (the sign and absolute
// value fold into the multiply ahead of the exponential).
__device__ __forceinline__ float phi_elu1(float x) {
  return fmaxf(x + 1.f, __expf(-fabsf(x)));
}

// ---------------------------------------------------------------------------
// Matrix-core fragments.  One "k-step" contracts 32 values of k.  Lane l of a
// wave holds row (A) / column (B) l%16 and the eight k values of slot group
// l/16.  The A and B operand slots are laid out identically, so any
// consistent assignment of logical k to the (group, element) slots gives the
// same sum; the kernels rely on that to feed accumulator tiles back in as
// operands without a layout change.
// Accumulator layout (16x16 fp32): lane l holds rows 4*(l/16)+r, r=0..3, of
// column l%16.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<bf16> &a,
                                    const Frag<bf16> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
// fp32 inputs: eight 16x16x4 products, element e of every slot group at a time.
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &a,
                                    const Frag<float> &b) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// 8 consecutive elements from LDS (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ void lds_frag(Frag<bf16> &f, const bf16 *p) {
  f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void lds_frag(Frag<float> &f, const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// 4 consecutive elements into slots [off, off+4) of a fragment.
__device__ __forceinline__ void lds_half(Frag<bf16> &f, const bf16 *p, int off) {
  const bf16x4 h = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) f.v[off + e] = h[e];
}
__device__ __forceinline__ void lds_half(Frag<float> &f, const float *p, int off) {
  const f32x4 h = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) f.v[off + e] = h[e];
}
template <typename T>
__device__ __forceinline__ float frag_elem(const Frag<T> &f, int e) {
  return to_f32(f.v[e]);
}
template <typename T>
__device__ __forceinline__ void frag_set(Frag<T> &f, int e, float x) {
  f.v[e] = from_f32<T>(x);
}

// Transposed fragment from a row-major LDS tile M (rows = the contraction
// index, e.g. tokens; columns = the operand's row/column index).  Lane
// (li, lg) receives column c0 + li; its slots 0..3 hold rows t_lo..t_lo+3 and
// slots 4..7 rows t_hi..t_hi+3 (t_lo, t_hi may differ between slot groups).
// bf16: two gfx950 LDS transpose reads (ds_read_b64_tr_b16): in each group
// of 16 lanes, lane li names row t + li/4, columns c0 + 4 (li%4) .. +3, and
// receives column c0 + li of the four rows.  fp32: eight strided reads.
__device__ __forceinline__ void lds_frag_tr(Frag<bf16> &f, const bf16 *M, int ld,
                                            int t_lo, int t_hi, int c0, int li) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lbf16x4;
  typedef __attribute__((address_space(3))) lbf16x4 lds_bf16x4;
  const int off = (li >> 2) * ld + c0 + 4 * (li & 3);
  const lbf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4 *)(M + t_lo * ld + off));
  const lbf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4 *)(M + t_hi * ld + off));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = a[e];
    f.v[4 + e] = b[e];
  }
}
__device__ __forceinline__ void lds_frag_tr(Frag<float> &f, const float *M, int ld,
                                            int t_lo, int t_hi, int c0, int li) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = M[(t_lo + e) * ld + c0 + li];
    f.v[4 + e] = M[(t_hi + e) * ld + c0 + li];
  }
}

// Rows t..t+3 of column c0 + li of a row-major LDS tile, as fp32: the
// accumulator layout of a 16 x 16 product (lane (li, lg) holds rows 4 lg + r
// of column li), with t the same for the 16 lanes of a slot group.  bf16:
// one transpose read (as in lds_frag_tr) instead of four 2-byte reads;
// fp32: four strided reads.
__device__ __forceinline__ void lds_col4(float (&x)[4], const bf16 *M, int ld, int t, int c0,
                                         int li) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lbf16x4;
  typedef __attribute__((address_space(3))) lbf16x4 lds_bf16x4;
  const lbf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4 *)(M + t * ld + (li >> 2) * ld + c0 + 4 * (li & 3)));
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = (float)a[e];
}
__device__ __forceinline__ void lds_col4(float (&x)[4], const float *M, int ld, int t, int c0,
                                         int li) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = M[(t + e) * ld + c0 + li];
}
template <typename T>
__device__ __forceinline__ void frag_fill(Frag<T> &f, float x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = from_f32<T>(x);
}

// Four consecutive T to LDS.
__device__ __forceinline__ void lds_store4(bf16 *p, float a, float b, float c,
                                           float d) {
  *reinterpret_cast<bf16x4 *>(p) = (bf16x4){(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
__device__ __forceinline__ void lds_store4(float *p, float a, float b, float c,
                                           float d) {
  *reinterpret_cast<f32x4 *>(p) = (f32x4){a, b, c, d};
}

// 16-byte vector of T (8 bf16 or 4 fp32).
template <typename T> struct Vec16;
template <> struct Vec16<bf16> { using type = bf16x8; };
template <> struct Vec16<float> { using type = f32x4; };

// R consecutive T to LDS from fp32 values (R * sizeof(T) = 2..32 bytes).
template <typename T, int R>
__device__ __forceinline__ void lds_store_n(T *p, const float (&x)[R]) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (R == 1) {
      p[0] = (bf16)x[0];
    } else if constexpr (R == 2) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<bf16x2 *>(p) = (bf16x2){(bf16)x[0], (bf16)x[1]};
    } else if constexpr (R == 4) {
      lds_store4(p, x[0], x[1], x[2], x[3]);
    } else {
      static_assert(R == 8, "unsupported width");
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
      *reinterpret_cast<bf16x8 *>(p) = v;
    }
  } else if constexpr (R == 1) {
    p[0] = x[0];
  } else if constexpr (R == 2) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<f32x2 *>(p) = (f32x2){x[0], x[1]};
  } else {
    static_assert(R % 4 == 0, "unsupported width");
#pragma unroll
    for (int e = 0; e < R; e += 4)
      *reinterpret_cast<f32x4 *>(p + e) = (f32x4){x[e], x[e + 1], x[e + 2], x[e + 3]};
  }
}

// ---------------------------------------------------------------------------
// Buffer-resource loads and stores.  A raw buffer access whose byte offset
// lies at or past the resource's size returns zeros (loads) or is dropped
// (stores) in hardware, so bounds checks become offset selects instead of
// branches: no divergent control flow sits between a load and its use, and
// the compiler can keep every prefetched load in flight across the compute.
// ---------------------------------------------------------------------------
constexpr uint32_t kOOB = 0x7ffffff0u;  // an offset past any resource used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base,
                                                           uint32_t bytes) {
  // dword 3 = 0x00020000: 32-bit data format, the gfx9-family raw-buffer setting
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)bytes, 0x00020000);
}

template <typename T>
__device__ __forceinline__ typename Vec16<T>::type buf_load16(
    __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return __builtin_bit_cast(typename Vec16<T>::type, x);
}

__device__ __forceinline__ float buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                           float *) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ bf16 buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                          bf16 *) {
  return __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}

// Four consecutive T (8 bytes bf16, 16 bytes fp32), as fp32.
__device__ __forceinline__ f32x4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16 *) {
  const bf16x4 h = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
  return (f32x4){(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
__device__ __forceinline__ f32x4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off, float *) {
  return buf_load16<float>(r, off);
}

template <typename T>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                            typename Vec16<T>::type v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
}
// Streaming store: the cache-policy operand's non-temporal bit (bit 1 in
// the gfx94x/gfx950 encoding: bit 0 sc0, bit 1 nt, bit 4 sc1).  Used for
// data written once and not read back by the same kernel (outputs, the
// decode state write-back, which is larger than the last-level cache).
template <typename T>
__device__ __forceinline__ void buf_store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                               typename Vec16<T>::type v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 2);
}
// Four fp32 values as four consecutive T (8 bytes bf16, 16 bytes fp32),
// streaming (non-temporal) store.
__device__ __forceinline__ void buf_store4_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 a,
                                              bf16 *) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const bf16x4 h = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, (int)off, 0, 2);
}
__device__ __forceinline__ void buf_store4_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 a,
                                              float *) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), r, (int)off, 0, 2);
}
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                           float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store1(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                           bf16 x) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, x), r, (int)off, 0, 0);
}

// One DPP lane move inside 16-lane rows (CTRL: a quad permutation, or the
// half-row / row mirror), a VALU operand modifier with no trip through the
// LDS unit.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W consecutive lanes (a power of two up to 64),
// the same value in every lane of a group: lanes l ^ 1 and l ^ 2 by quad
// permutations, then the other quad of the half-row and the other half of
// the row by the mirrors (each step adds a group to its mirror image, so
// every lane ends with the whole sum), then across rows by lane shuffles.
template <int W>
__device__ __forceinline__ float lane_sum(float x) {
  static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "group width");
  x += dpp_move<0xB1>(x);                         // quad_perm [1, 0, 3, 2]
  if constexpr (W >= 4) x += dpp_move<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if constexpr (W >= 8) x += dpp_move<0x141>(x);  // row_half_mirror
  if constexpr (W >= 16) x += dpp_move<0x140>(x); // row_mirror
  if constexpr (W >= 32) x += __shfl_xor(x, 16);
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Sum over the four slot groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace la
