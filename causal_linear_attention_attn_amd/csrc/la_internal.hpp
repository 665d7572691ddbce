// Host-side interface between the C ABI (la_api.hip) and the kernel files.
#pragma once

#include <hip/hip_ext.h>
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
  int nsplit;       // summary workgroups per segment (1 or 2)
  int split_len;    // tokens in a segment's first summary part (nsplit 2)
  size_t wrec;      // floats per workspace slot record
  size_t ws_bytes;  // workspace bytes
  size_t conv_off;  // byte offset of the conv cache copy (with a convolution
                    // over several segments; it ends the workspace)
};

struct PrefillParams {
  int BH, H, N, d, dv;
  int fmap;      // 1 = elu+1
  int vec_ok;    // 16-byte vector loads of q, k, v rows are legal
  const void *q, *k, *v;
  const float *gamma;  // [H] or nullptr
  const float *g;      // delta gate [BH, N]
  const float *alpha;  // delta decay [BH, N] or nullptr
  float eps;
  const float *S_in, *z_in;
  float *S_out, *z_out;
  void *o;
  float *ws;
  int nseg, seg_len;
  int nsplit, split_len;  // summary parts per segment, tokens in the first
  int slot_vec;  // workspace slots take 16-byte accesses (d % 4 == 0, ws aligned)
  // short causal convolution of q, k, v (LINEAR rule): filters [H, w, 2d+dv]
  // fp32, or nullptr; cache rows [BH, w-1, 2d+dv] of dtype T
  const float *conv_w;
  int conv_width;
  const void *conv_in;   // tokens before the sequence (nullptr = zeros)
  void *conv_out;        // last w-1 raw tokens after it (nullptr = not written)
  const void *conv_src;  // where the chunk kernel reads the tokens before
                         // segment 0: conv_in, or the summary kernel's copy
  void *conv_copy;       // summary kernel: copy conv_in here (nullptr = no)
  float *den_out;        // [BH, N] per-token denominators, or nullptr
};

// Short causal convolution of q, k, v into workspace copies (ahead of the
// delta rule's prefill), and the conv cache after the sequence.
struct ConvParams {
  int BH, H, N, d, dv, width;
  const float *w;         // [H, width, 2d+dv] filters
  const void *q, *k, *v;  // [BH, N, d], [BH, N, d], [BH, N, dv]
  const void *cache_in;   // [BH, width-1, 2d+dv] or nullptr (zeros)
  void *yq, *yk, *yv;     // convolved copies, layouts as q, k, v
  void *cache_out;        // [BH, width-1, 2d+dv] or nullptr (not written)
};
// vec: d and dv multiples of 16 bytes of elements and every buffer 16-byte
// aligned
hipError_t launch_conv_qkv(const ConvParams &p, bool bf16_io, bool vec, hipStream_t s);
// Backward of the convolution: from dL/dy (the convolved q, k, v), dL/dx,
// dL/d(filters) and dL/d(cache before the sequence).
struct ConvBwdParams {
  int BH, H, N, d, dv, width;
  const float *w;            // [H, width, 2d+dv]
  const void *q, *k, *v;     // raw inputs
  const void *cache_in;      // or nullptr (zeros)
  const void *dyq, *dyk, *dyv;  // dL/d(convolved q, k, v)
  const void *dcache_out;    // dL/d(returned cache) or nullptr (zero)
  void *dq, *dk, *dv_;       // dL/d(raw q, k, v)
  void *dcache_in;           // or nullptr (not written)
  float *dw;                 // [H, width, 2d+dv]
  float *dw_part;            // workspace: conv_dw_partial_floats floats
};
size_t conv_dw_partial_floats(int BH, int N, int d, int dv, int width);
hipError_t launch_conv_backward(const ConvBwdParams &p, bool bf16_io, hipStream_t s);

// Backward of the LINEAR rule's prefill.
struct BwdParams {
  int BH, H, N, d, dv;
  int fmap;
  int vec_ok;
  const void *q, *k, *v, *o, *dout;  // forward inputs and output, dL/do
  const float *den;                  // [BH, N] forward denominators
  const float *gamma;                // [H] or nullptr
  const float *S_in, *z_in;          // forward initial state or nullptr
  const float *dS_out, *dz_out;      // dL/d(final state) or nullptr
  void *dq, *dk, *dv_;
  float *dS_in, *dz_in;              // dL/d(initial state) or nullptr
  float *ws_f, *ws_r;                // forward-state and adjoint slots
  size_t wrec;                       // floats per slot record
  int nseg, seg_len;
  int slot_vec;                      // forward slots take 16-byte accesses
  // per-key-channel decay (GLA): alpha [BH, N, d] fp32 or nullptr; then
  // ux [BH, N, d] fp32 (phi(q) . dphi(q) per token and channel), chs
  // [BH, nchunks] slot records of wrec floats (the forward state after each
  // chunk) and the output dalpha [BH, N, d]
  const float *alpha;
  float *ux, *chs, *dalpha;
};

struct DecodeParams {
  int BH, H, d, dv;
  int fmap;
  const void *q, *k, *v;
  const float *gamma, *g;
  const float *alpha;  // delta decay [BH] or nullptr
  float eps;
  float *S, *z;
  void *o;
  const float *conv_w;  // [H, w, 2d+dv] or nullptr
  int conv_width;
  void *conv_cache;     // [BH, w-1, 2d+dv], dtype T, updated in place
};

// Backward of the gated delta rule (bf16).
struct BwdDeltaParams {
  int BH, H, N, d, dv;
  int dvp;       // value width of the state records (64 or 128)
  int nch;       // chunks per sequence
  int vec_ok;    // 16-byte loads of q, k rows and 8-byte ones of v, dL/do rows
  const void *q, *k, *v, *dout;      // forward inputs, dL/do
  const float *g, *alpha;            // [BH, N]; alpha nullptr = no decay
  const float *S_in, *dS_out;        // forward initial state, dL/d(final state)
  void *dq, *dk, *dv_;               // outputs (dtype of q)
  float *dg, *dalpha, *dS_in;        // [BH, N], [BH, N] (with a decay), [BH, d, dv]
  void *ws;                          // workspace, sections below
  size_t lay_dec, lay_states, lay_adj, lay_y, lay_dd;  // element offsets
};
struct BwdDeltaSizes {
  size_t bytes;
  int dvp, nch;
  size_t dec, states, adj, y, dd;
};
BwdDeltaSizes delta_backward_sizes(int BH, int N, int d, int dv);
hipError_t launch_delta_backward(const BwdDeltaParams &p, hipStream_t s);

int device_cu_count();  // cached per device

// Grids with one row of workgroups per head put the head on y and, past the
// y limit, on z: head = blockIdx.y + kGridY * blockIdx.z (workgroups with a
// head index past B*H return at once).
constexpr int kGridY = 65535;
inline dim3 head_grid(unsigned nx, int BH) {
  const unsigned y = BH < kGridY ? (unsigned)BH : (unsigned)kGridY;
  return dim3(nx, y, (unsigned)((BH + kGridY - 1) / kGridY));
}

// Kernel timing (off unless la_profile_enable turned it on).  A launch
// through launch_kernel takes a pair of events from prof_slot and hands them
// to the dispatch itself (hipExtLaunchKernel stamps them when the kernel
// starts and ends, so launch latency is not counted); prof_commit files the
// record under `name` if the launch succeeded.  Off, the slot is empty and
// the launch is a plain hipLaunchKernelGGL.
struct ProfSlot {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfSlot prof_slot();
void prof_commit(const char *name, ProfSlot slot, hipError_t launch_status);

template <typename... Args, typename F = void (*)(Args...)>
hipError_t launch_kernel(const char *name, F kernel, dim3 grid, dim3 block, hipStream_t s,
                         Args... args) {
  const ProfSlot ps = prof_slot();
  if (ps.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ps.start, ps.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  const hipError_t e = hipGetLastError();
  prof_commit(name, ps, e);
  return e;
}

// conv_width > 0: a short convolution runs in front of q, k, v; chan: a
// per-key-channel decay (its kernels' occupancy sets the segment count)
LinearPlan plan_linear(int BH, int N, int d, int dv, bool bf16, int conv_width,
                       bool chan = false);
bool linear_combo_supported(int d, int dv, bool bf16, bool chan_decay, bool conv);
// The forward's summary and scan kernels only: the state entering each
// segment, in the workspace slots (nothing to do with one segment).
hipError_t launch_linear_state_prefix(const PrefillParams &p, const LinearPlan &plan,
                                      bool bf16, hipStream_t s);
// Tile configurations the backward kernels have for these widths (fp32 with
// d and dv both above 64 has none: the API runs it over value halves).
bool linear_backward_supported(int d, int dv, bool bf16);
bool linear_backward_channel_supported(int d, int dv, bool bf16);  // with alpha
hipError_t launch_linear_backward(const BwdParams &p, bool bf16, hipStream_t s);
// fp32 rows [rows, n] <-> column blocks [rows, na] and [rows, n - na]; dst += src.
hipError_t launch_split_cols(const float *src, float *a, float *b, size_t rows, int n, int na,
                             hipStream_t s);
hipError_t launch_join_cols(float *dst, const float *a, const float *b, size_t rows, int n,
                            int na, hipStream_t s);
hipError_t launch_add_into(float *dst, const float *src, size_t n, hipStream_t s);
// tokens per chunk of the backward kernels with a per-channel decay
constexpr int kChanBwdChunk = 32;
hipError_t launch_linear_prefill(const PrefillParams &p, const LinearPlan &plan,
                                 bool bf16, hipStream_t s);
// Gated delta rule: workspace (per-chunk Wt and R tiles) and the two-kernel
// launch (per-chunk prep, then the sequential pass).
size_t delta_workspace_bytes(int BH, int N, int d, bool bf16);
hipError_t launch_delta_prefill(const PrefillParams &p, bool bf16, hipStream_t s);
hipError_t launch_decode(const DecodeParams &p, bool bf16, bool delta, int vec,
                         hipStream_t s);
hipError_t launch_zero_bytes(void *dst, size_t bytes, hipStream_t s);
hipError_t launch_copy_bytes(void *dst, const void *src, size_t bytes, hipStream_t s);
hipError_t launch_fill(float *dst, size_t n, float value, hipStream_t s);
hipError_t launch_copy(float *dst, const float *src, size_t n, hipStream_t s);

}  // namespace la
