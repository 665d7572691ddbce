// Host-side interface between the C ABI (la_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

// Chunk length and tile sizes a linear prefill instantiation uses.
struct LinearPlan {
  int dk, dv_pad;   // padded feature / value dims (64 or 128)
  int chunk;        // tokens per chunk
  int threads;      // workgroup size
  int per_cu;       // resident workgroups per CU
  int nseg;         // segments per sequence (>= 1)
  int seg_len;      // tokens per segment (multiple of chunk)
  size_t ws_bytes;  // workspace bytes
};

struct PrefillParams {
  int BH, H, N, d, dv;
  int fmap;      // 1 = elu+1
  int vec_ok;    // 16-byte vector loads of q, k, v rows are legal
  const void *q, *k, *v;
  const float *gamma;  // [H] or nullptr
  const float *g;      // delta gate [BH, N]
  float eps;
  const float *S_in, *z_in;
  float *S_out, *z_out;
  void *o;
  float *ws;
  int nseg, seg_len;
};

struct DecodeParams {
  int BH, H, d, dv;
  int fmap;
  const void *q, *k, *v;
  const float *gamma, *g;
  float eps;
  float *S, *z;
  void *o;
};

int device_cu_count();  // cached per device

// Kernel timing hooks (no-ops unless profiling is enabled): call prof_begin
// before and prof_end after each kernel launch.
void prof_begin(hipStream_t s);
void prof_end(const char *name, hipStream_t s);

LinearPlan plan_linear(int BH, int N, int d, int dv, bool bf16);
hipError_t launch_linear_prefill(const PrefillParams &p, const LinearPlan &plan,
                                 bool bf16, hipStream_t s);
// Gated delta rule: workspace (per-chunk Wt and R tiles) and the two-kernel
// launch (per-chunk prep, then the sequential pass).
size_t delta_workspace_bytes(int BH, int N, int d, bool bf16);
hipError_t launch_delta_prefill(const PrefillParams &p, bool bf16, hipStream_t s);
hipError_t launch_decode(const DecodeParams &p, bool bf16, bool delta, int vec,
                         hipStream_t s);
hipError_t launch_fill(float *dst, size_t n, float value, hipStream_t s);
hipError_t launch_copy(float *dst, const float *src, size_t n, hipStream_t s);

}  // namespace la
