// C ABI of liblinattn.so: argument validation, planning and kernel dispatch.
// Every check runs before anything is enqueued (see include/linattn.h).
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/linattn.h"
#include "la_internal.hpp"

namespace la {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 256;  // no device visible (e.g. a workspace query on a build host)
  }
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || v <= 0) {
    (void)hipGetLastError();
    v = 256;
  }
  if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// ---- kernel timing log -----------------------------------------------------
namespace {
struct ProfRec {
  const char *name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;
constexpr size_t kMaxRecs = 65536;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}

void clear_log_locked() {
  for (auto &r : g_recs) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
}
}  // namespace

ProfSlot prof_slot() {
  ProfSlot ps;
  if (!g_prof_on.load(std::memory_order_relaxed)) return ps;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_recs.size() >= kMaxRecs) return ps;
  ps.start = take_event();
  ps.stop = ps.start ? take_event() : nullptr;
  if (!ps.stop) {
    if (ps.start) g_pool.push_back(ps.start);
    ps.start = nullptr;
  }
  return ps;
}

void prof_commit(const char *name, ProfSlot ps, hipError_t launch_status) {
  if (!ps.start) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (launch_status == hipSuccess && g_prof_on.load(std::memory_order_relaxed)) {
    g_recs.push_back({name, ps.start, ps.stop});
  } else {
    g_pool.push_back(ps.start);
    g_pool.push_back(ps.stop);
  }
}

}  // namespace la

namespace {

// A dispatch's grid is at most 2^32 - 1 work-items along each axis.
constexpr unsigned long long kMaxGridItems = 0xffffffffull;
constexpr size_t kMaxHeadBytes = 0x7fff0000u;
constexpr int kMaxConvWidth = 4;

bool dims_ok(int d, int dv) {
  return d >= 1 && d <= LA_MAX_DIM && dv >= 1 && dv <= LA_MAX_DIM;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int to_status(hipError_t e) { return e == hipSuccess ? LA_OK : LA_EHIP; }

// Shape / mode checks shared by the workspace query and the prefill itself.
int check_prefill_shape(const la_prefill_args *a) {
  if (!a) return LA_EINVAL;
  if (a->B < 0 || a->H < 0 || a->N < 0 || !dims_ok(a->d, a->dv)) return LA_EINVAL;
  if ((long long)a->B * a->H > 0x7fffffffLL) return LA_EUNSUPPORTED;
  if (a->dtype != LA_F32 && a->dtype != LA_BF16) return LA_EINVAL;
  if (a->rule != LA_RULE_LINEAR && a->rule != LA_RULE_DELTA) return LA_EINVAL;
  if (a->fmap != LA_FMAP_IDENTITY && a->fmap != LA_FMAP_ELU1) return LA_EINVAL;
  if (a->rule == LA_RULE_DELTA && a->fmap != LA_FMAP_IDENTITY) return LA_EINVAL;
  // the delta rule's sequential pass runs 512 threads per (head, 16 value
  // columns) along one grid axis; every other grid puts heads on y and z
  if (a->rule == LA_RULE_DELTA &&
      (unsigned long long)a->B * a->H * ((a->dv + 15) / 16) * 512 > kMaxGridItems)
    return LA_EUNSUPPORTED;
  // one head's q/k/v/o must be addressable with 32-bit byte offsets
  const size_t esz = a->dtype == LA_BF16 ? 2 : 4;
  const size_t dmax = a->d > a->dv ? a->d : a->dv;
  if ((size_t)a->N * dmax * esz > kMaxHeadBytes) return LA_EUNSUPPORTED;
  if (a->conv_weight) {
    if (a->conv_width < 1 || a->conv_width > kMaxConvWidth) return LA_EINVAL;
    if (a->rule == LA_RULE_LINEAR &&
        !la::linear_combo_supported(a->d, a->dv, a->dtype == LA_BF16, a->alpha != nullptr,
                                    true))
      return LA_EUNSUPPORTED;
  } else if (a->conv_width != 0 || a->conv_in || a->conv_out) {
    return LA_EINVAL;
  }
  return LA_OK;
}

// Bytes of one conv cache [B,H,w-1,2d+dv] (0 without a convolution).
size_t conv_cache_bytes(size_t BH, int d, int dv, int width, bool bf16_io) {
  return width > 1 ? BH * (size_t)(width - 1) * (2 * (size_t)d + dv) * (bf16_io ? 2 : 4) : 0;
}

// The delta rule behind a convolution runs on convolved copies of q, k, v
// at the start of the workspace (each region 256-byte aligned); the rule's
// own workspace follows.
size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
// Bytes of three [B,H,N,*] copies of q, k, v (or of their gradients), each
// region 256-byte aligned.
size_t qkv_copy_bytes(size_t rows, int d, int dv, size_t esz) {
  return 2 * round256(rows * d * esz) + round256(rows * dv * esz);
}
// The prefills that run the convolution as a pass of its own: the delta
// rule, and the LINEAR rule with denominators (a training forward).
bool conv_pass(const la_prefill_args *a) {
  return a->conv_weight && (a->rule == LA_RULE_DELTA || a->den_out);
}
size_t conv_copy_bytes(const la_prefill_args *a) {
  if (!conv_pass(a)) return 0;
  return qkv_copy_bytes((size_t)a->B * a->H * a->N, a->d, a->dv, a->dtype == LA_BF16 ? 2 : 4);
}

// Convolution pass into the three copies at `base` (the conv cache after
// the sequence to cache_out, when given).
hipError_t run_conv_pass(int BH, int H, int N, int d, int dv, bool bf16_io, const float *w,
                         int width, const void *q, const void *k, const void *v,
                         const void *cache_in, void *cache_out, char *base, hipStream_t s,
                         const void **yq, const void **yk, const void **yv) {
  const size_t esz = bf16_io ? 2 : 4, rows = (size_t)BH * N;
  la::ConvParams c{};
  c.BH = BH;
  c.H = H;
  c.N = N;
  c.d = d;
  c.dv = dv;
  c.width = width;
  c.w = w;
  c.q = q;
  c.k = k;
  c.v = v;
  c.cache_in = cache_in;
  c.cache_out = cache_out;
  c.yq = base;
  c.yk = base + round256(rows * d * esz);
  c.yv = base + 2 * round256(rows * d * esz);
  *yq = c.yq;
  *yk = c.yk;
  *yv = c.yv;
  const bool vec16 = ((size_t)d * esz) % 16 == 0 && ((size_t)dv * esz) % 16 == 0 &&
                     aligned16(q) && aligned16(k) && aligned16(v) && aligned16(base) &&
                     (!cache_in || aligned16(cache_in));
  return la::launch_conv_qkv(c, bf16_io, vec16, s);
}

bool overlap(const void *a, const void *b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return n > 0 && x < y + n && y < x + n;
}

}  // namespace

extern "C" {

int32_t la_abi_version(void) { return 7; }

const char *la_status_str(int s) {
  switch (s) {
    case LA_OK: return "ok";
    case LA_EINVAL: return "invalid argument";
    case LA_EUNSUPPORTED: return "unsupported configuration";
    case LA_EHIP: return "HIP launch or runtime error";
    case LA_EWORKSPACE: return "workspace missing or too small";
    case LA_ESCRATCH: return "request needs more than the static scratch of la_prefill_noalloc";
    default: return "unknown status";
  }
}

size_t la_prefill_workspace_size(const la_prefill_args *a) {
  if (check_prefill_shape(a) != LA_OK) return (size_t)-1;
  const int BH = a->B * a->H;
  if (BH == 0 || a->N == 0) return 0;
  if (a->rule == LA_RULE_LINEAR)
    return conv_copy_bytes(a) +
           la::plan_linear(BH, a->N, a->d, a->dv, a->dtype == LA_BF16,
                           a->conv_weight && !conv_pass(a) ? a->conv_width : 0,
                           a->alpha != nullptr)
               .ws_bytes;
  return conv_copy_bytes(a) + la::delta_workspace_bytes(BH, a->N, a->d, a->dtype == LA_BF16);
}

int la_prefill(const la_prefill_args *a, void *stream) {
  int st = check_prefill_shape(a);
  if (st != LA_OK) return st;
  const int BH = a->B * a->H;
  const bool linear = a->rule == LA_RULE_LINEAR;
  if (linear) {
    if (a->g || (a->alpha && a->gamma) || !(a->eps >= 0.f) || !std::isfinite(a->eps))
      return LA_EINVAL;
    // one head's per-channel decay (fp32) must be addressable with 32-bit offsets
    if (a->alpha && (size_t)a->N * a->d * 4 > kMaxHeadBytes) return LA_EUNSUPPORTED;
  } else {
    if (!a->g && BH > 0 && a->N > 0) return LA_EINVAL;
    if (a->gamma || a->z_in || a->z_out || a->den_out) return LA_EINVAL;
  }
  if (BH > 0 && a->N > 0 && (!a->q || !a->k || !a->v || !a->o)) return LA_EINVAL;
  const bool bf16_io = a->dtype == LA_BF16;
  const int cw = a->conv_weight ? a->conv_width : 0;
  const size_t ncache = conv_cache_bytes((size_t)BH, a->d, a->dv, cw, bf16_io);
  if (a->conv_in && a->conv_out && a->conv_in != a->conv_out &&
      overlap(a->conv_in, a->conv_out, ncache))
    return LA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (BH == 0) return LA_OK;

  const size_t nS = (size_t)BH * a->d * a->dv, nz = (size_t)BH * a->d;
  if (a->N == 0) {  // no tokens: the state passes through unchanged
    hipError_t e = hipSuccess;
    if (a->S_out)
      e = a->S_in ? la::launch_copy(a->S_out, a->S_in, nS, s)
                  : la::launch_fill(a->S_out, nS, 0.f, s);
    if (e == hipSuccess && a->z_out)
      e = a->z_in ? la::launch_copy(a->z_out, a->z_in, nz, s)
                  : la::launch_fill(a->z_out, nz, 0.f, s);
    if (e == hipSuccess && a->conv_out)  // and so does the conv cache
      e = a->conv_in ? la::launch_copy_bytes(a->conv_out, a->conv_in, ncache, s)
                     : la::launch_zero_bytes(a->conv_out, ncache, s);
    return to_status(e);
  }
  la::LinearPlan plan{};
  size_t ws_need;
  if (linear) {
    plan = la::plan_linear(BH, a->N, a->d, a->dv, bf16_io, conv_pass(a) ? 0 : cw,
                           a->alpha != nullptr);
    ws_need = conv_copy_bytes(a) + plan.ws_bytes;
    if (conv_pass(a) && !aligned16(a->workspace)) return LA_EINVAL;
  } else {
    ws_need = la::delta_workspace_bytes(BH, a->N, a->d, bf16_io);
    // one head's T and R tiles must be addressable with 32-bit byte offsets
    if (ws_need / (size_t)BH > kMaxHeadBytes) return LA_EUNSUPPORTED;
    ws_need += conv_copy_bytes(a);
  }
  if (ws_need > 0 && (!a->workspace || a->workspace_bytes < ws_need))
    return LA_EWORKSPACE;
  // the delta rule moves its per-chunk records with 16-byte accesses
  if (!linear && ws_need > 0 && !aligned16(a->workspace)) return LA_EINVAL;

  la::PrefillParams p{};
  p.BH = BH;
  p.H = a->H;
  p.N = a->N;
  p.d = a->d;
  p.dv = a->dv;
  p.fmap = a->fmap == LA_FMAP_ELU1;
  const int vec = bf16_io ? 8 : 4;
  p.vec_ok = (a->d % vec == 0) && (a->dv % vec == 0) && aligned16(a->q) &&
             aligned16(a->k) && aligned16(a->v) && aligned16(a->o);
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.gamma = a->gamma;
  p.g = a->g;
  p.alpha = a->alpha;
  p.eps = a->eps;
  p.S_in = a->S_in;
  p.z_in = a->z_in;
  p.S_out = a->S_out;
  p.z_out = a->z_out;
  p.o = a->o;
  p.den_out = a->den_out;
  p.ws = reinterpret_cast<float *>(a->workspace);
  if (conv_pass(a)) {  // the rule runs on convolved copies of q, k, v
    char *base = static_cast<char *>(a->workspace);
    const hipError_t e =
        run_conv_pass(BH, a->H, a->N, a->d, a->dv, bf16_io, a->conv_weight, cw, a->q, a->k,
                      a->v, a->conv_in, a->conv_out, base, s, &p.q, &p.k, &p.v);
    if (e != hipSuccess) return LA_EHIP;
    p.vec_ok = (a->d % vec == 0) && (a->dv % vec == 0) && aligned16(a->o);
    p.ws = reinterpret_cast<float *>(base + conv_copy_bytes(a));
  }
  if (!linear) return to_status(la::launch_delta_prefill(p, bf16_io, s));
  p.nseg = plan.nseg;
  p.seg_len = plan.seg_len;
  p.nsplit = plan.nsplit;
  p.split_len = plan.split_len;
  p.slot_vec = (a->d % 4 == 0) && aligned16(p.ws);
  if (conv_pass(a)) return to_status(la::launch_linear_prefill(p, plan, bf16_io, s));
  p.conv_w = a->conv_weight;
  p.conv_width = cw;
  if (cw > 1) {
    p.conv_in = a->conv_in;
    p.conv_out = a->conv_out;
    // over several segments chunk_kernel reads the summary kernel's copy of
    // the cache, so that conv_out may alias conv_in
    const bool copy = plan.nseg > 1 && a->conv_in;
    void *cp = copy ? static_cast<char *>(a->workspace) + plan.conv_off : nullptr;
    p.conv_copy = cp;
    p.conv_src = copy ? cp : a->conv_in;
  }
  return to_status(la::launch_linear_prefill(p, plan, bf16_io, s));
}

namespace {

// The convolution fields of the backward arguments.
int check_conv_grads(const float *w, int width, const void *cin, const void *gout,
                     const float *gw, const void *gin) {
  if (w) {
    if (width < 1 || width > kMaxConvWidth || !gw) return LA_EINVAL;
  } else if (width != 0 || cin || gout || gw || gin) {
    return LA_EINVAL;
  }
  return LA_OK;
}

// Backward gradients with no tokens for the convolution's parameters: the
// filters get none, the cache before the sequence passes straight through
// to the cache after it.
hipError_t conv_grads_no_tokens(int BH, int H, int d, int dv, int width, bool bf16_io,
                                const void *gout, float *gw, void *gin, hipStream_t s) {
  hipError_t e = la::launch_fill(gw, (size_t)H * width * (2 * (size_t)d + dv), 0.f, s);
  const size_t n = conv_cache_bytes((size_t)BH, d, dv, width, bf16_io);
  if (e == hipSuccess && gin && n)
    e = gout ? la::launch_copy_bytes(gin, gout, n, s) : la::launch_zero_bytes(gin, n, s);
  return e;
}

// Workspace of a backward call with the forward's short convolution:
// dL/d(convolved q, k, v), the filter gradient's partial sums, and (unless
// the forward's workspace is given) the convolved q, k, v themselves; then
// the rule's own state slots.
struct BwdLayout {
  size_t grads, part, copies, slots, total;
};
BwdLayout conv_bwd_layout(int BH, int N, int d, int dv, size_t esz, int width, bool conv,
                          bool fwd, size_t slot_bytes) {
  BwdLayout L{};
  const size_t rows = (size_t)BH * N;
  size_t off = 0;
  if (conv) {
    L.grads = off;
    off += qkv_copy_bytes(rows, d, dv, esz);
    L.part = off;
    off += round256(la::conv_dw_partial_floats(BH, N, d, dv, width) * sizeof(float));
    if (!fwd) {
      L.copies = off;
      off += qkv_copy_bytes(rows, d, dv, esz);
    }
  }
  L.slots = off;
  L.total = off + slot_bytes;
  return L;
}

// The convolution's chain rule after a rule's backward (dy: dL/d(convolved
// q, k, v)).
hipError_t conv_backward(int BH, int H, int N, int d, int dv, bool bf16_io, const float *w,
                         int width, const void *q, const void *k, const void *v,
                         const void *cin, const void *dyq, const void *dyk, const void *dyv,
                         const void *gout, void *dq, void *dk, void *dv_, void *gin, float *gw,
                         char *part, hipStream_t s) {
  la::ConvBwdParams c{};
  c.BH = BH;
  c.H = H;
  c.N = N;
  c.d = d;
  c.dv = dv;
  c.width = width;
  c.w = w;
  c.q = q;
  c.k = k;
  c.v = v;
  c.cache_in = cin;
  c.dyq = dyq;
  c.dyk = dyk;
  c.dyv = dyv;
  c.dcache_out = width > 1 ? gout : nullptr;
  c.dq = dq;
  c.dk = dk;
  c.dv_ = dv_;
  c.dcache_in = width > 1 ? gin : nullptr;
  c.dw = gw;
  c.dw_part = reinterpret_cast<float *>(part);
  return la::launch_conv_backward(c, bf16_io, s);
}

// The three regions of a q, k, v copy starting at base.
void qkv_regions(char *base, size_t rows, int d, size_t esz, void **q, void **k, void **v) {
  *q = base;
  *k = base + round256(rows * d * esz);
  *v = base + 2 * round256(rows * d * esz);
}

int check_backward_shape(const la_backward_args *a) {
  if (!a) return LA_EINVAL;
  if (a->B < 0 || a->H < 0 || a->N < 0 || !dims_ok(a->d, a->dv)) return LA_EINVAL;
  if ((long long)a->B * a->H > 0x7fffffffLL) return LA_EUNSUPPORTED;
  if (a->dtype != LA_F32 && a->dtype != LA_BF16) return LA_EINVAL;
  if (a->fmap != LA_FMAP_IDENTITY && a->fmap != LA_FMAP_ELU1) return LA_EINVAL;
  const size_t esz = a->dtype == LA_BF16 ? 2 : 4;
  const size_t dmax = a->d > a->dv ? a->d : a->dv;
  if ((size_t)a->N * dmax * esz > kMaxHeadBytes) return LA_EUNSUPPORTED;
  if (a->alpha) {  // per-key-channel decay (GLA)
    if (a->gamma) return LA_EINVAL;
    if (!la::linear_backward_channel_supported(a->d, a->dv, a->dtype == LA_BF16))
      return LA_EUNSUPPORTED;
    if ((size_t)a->N * a->d * 4 > kMaxHeadBytes) return LA_EUNSUPPORTED;
  } else if (a->grad_alpha) {
    return LA_EINVAL;
  }
  return check_conv_grads(a->conv_weight, a->conv_width, a->conv_in, a->grad_conv_out,
                          a->grad_conv_weight, a->grad_conv_in);
}

// Adjoint slots (one copy of the forward's segment slots), and in front of
// them the forward-state slots unless the forward's workspace is reused.
size_t backward_ws_bytes(const la::LinearPlan &pl, bool reuse) {
  return (reuse ? 1 : 2) * pl.ws_bytes;
}

// fp32 with d and dv both above 64 has no tile configuration for the whole
// value width (the fp32 state tile would not fit the LDS beside the operand
// tiles), so the rule's backward runs over the value columns [0, 64) and
// [64, dv) in turn: each half's normaliser column carries that half's share
// of g.o (the shares add up to the whole), so dq, dk and dL/dz_in are the
// sums of the halves' results and dv, dL/dS_in their column blocks; the
// final-normaliser gradient enters the first half only.
constexpr int kSplitCols = 64;
bool split_values(int d, int dv, bool bf16) { return !la::linear_backward_supported(d, dv, bf16); }

// Regions (bytes from the start of the rule's part of the workspace) of a
// split backward: the halves' v, o, dL/do, dv, the second half's dq and dk,
// S_in, dL/dS_out, dL/dS_in by halves, the second half's dL/dz_in, then
// state slots for one half at a time.
struct SplitLayout {
  size_t v[2], o[2], go[2], gv[2], gq, gk, sin[2], gso[2], gsi[2], gz, slots, total;
};
SplitLayout split_layout(int BH, int N, int d, int dv) {
  SplitLayout L{};
  const size_t rows = (size_t)BH * N, srows = (size_t)BH * d;
  const int n[2] = {kSplitCols, dv - kSplitCols};
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t at = off;
    off += round256(floats * sizeof(float));
    return at;
  };
  for (int h = 0; h < 2; ++h) {
    L.v[h] = take(rows * n[h]);
    L.o[h] = take(rows * n[h]);
    L.go[h] = take(rows * n[h]);
    L.gv[h] = take(rows * n[h]);
    L.sin[h] = take(srows * n[h]);
    L.gso[h] = take(srows * n[h]);
    L.gsi[h] = take(srows * n[h]);
  }
  L.gq = take(rows * d);
  L.gk = take(rows * d);
  L.gz = take(srows);
  L.slots = off;
  size_t slot_bytes = 0;
  for (int h = 0; h < 2; ++h) {
    const la::LinearPlan pl = la::plan_linear(BH, N, d, n[h], false, 0);  // (no decay: fp32)
    if (pl.nseg > 1 && backward_ws_bytes(pl, false) > slot_bytes)
      slot_bytes = backward_ws_bytes(pl, false);
  }
  L.total = off + slot_bytes;
  return L;
}

// With a per-channel decay, after the state slots: phi(q) . dphi(q) per
// token and channel (fp32 [BH, N, d]) and the forward state after every
// chunk (slot records, [BH, nchunks]).
struct ChanBwdLayout {
  size_t ux, chs, total;
};
ChanBwdLayout chan_bwd_layout(int BH, int N, int d, int dv) {
  ChanBwdLayout L{};
  const size_t nch = ((size_t)N + la::kChanBwdChunk - 1) / la::kChanBwdChunk;
  const size_t wrec = (size_t)d * dv + 2 * (size_t)d;
  L.ux = 0;
  L.chs = round256((size_t)BH * N * d * sizeof(float));
  L.total = L.chs + round256((size_t)BH * nch * wrec * sizeof(float));
  return L;
}

// Bytes of the rule's part of a backward workspace (state slots, the
// per-channel decay's buffers, and the halves' buffers when the value
// columns are split).
size_t rule_ws_bytes(int BH, int N, int d, int dv, bool bf16, bool fwd, bool chan) {
  if (split_values(d, dv, bf16)) return split_layout(BH, N, d, dv).total;
  const la::LinearPlan plan = la::plan_linear(BH, N, d, dv, bf16, 0, chan);
  const size_t slots = plan.nseg > 1 ? backward_ws_bytes(plan, fwd) : 0;
  return chan ? round256(slots) + chan_bwd_layout(BH, N, d, dv).total : slots;
}

// One LINEAR-rule backward (no convolution) over tensors of width dv.
struct RuleBwd {
  int BH, H, N, d, dv, fmap;
  bool bf16;
  const void *q, *k, *v, *o, *dout;
  const float *den, *gamma, *S_in, *z_in, *dS_out, *dz_out, *alpha;
  void *dq, *dk, *dv_;
  float *dS_in, *dz_in, *dalpha;
};

// wsb: the rule's part of the workspace (rule_ws_bytes: state slots of
// backward_ws_bytes(plan, fwd_slots given), then the per-channel decay's
// buffers); fwd_slots: the forward's own segment states (same plan), or
// nullptr to recompute.
hipError_t rule_backward(const RuleBwd &r, char *wsb, const float *fwd_slots, hipStream_t s) {
  const bool chan = r.alpha != nullptr;
  const la::LinearPlan plan = la::plan_linear(r.BH, r.N, r.d, r.dv, r.bf16, 0, chan);
  const bool reuse = plan.nseg > 1 && fwd_slots != nullptr;
  float *ws = plan.nseg > 1 ? reinterpret_cast<float *>(wsb) : nullptr;
  const int vec = r.bf16 ? 8 : 4;
  const bool vec_ok = (r.d % vec == 0) && (r.dv % vec == 0) && aligned16(r.q) &&
                      aligned16(r.k) && aligned16(r.v) && aligned16(r.o) &&
                      aligned16(r.dout) && aligned16(r.dq) && aligned16(r.dk) &&
                      aligned16(r.dv_);
  float *ws_r = ws ? ws + (reuse ? 0 : plan.ws_bytes / sizeof(float)) : nullptr;
  const float *ws_f = reuse ? fwd_slots : ws;
  if (plan.nseg > 1 && !reuse) {  // the forward state entering each segment
    la::PrefillParams fp{};
    fp.BH = r.BH;
    fp.H = r.H;
    fp.N = r.N;
    fp.d = r.d;
    fp.dv = r.dv;
    fp.fmap = r.fmap;
    fp.vec_ok = vec_ok;
    fp.q = r.q;
    fp.k = r.k;
    fp.v = r.v;
    fp.gamma = r.gamma;
    fp.alpha = r.alpha;
    fp.S_in = r.S_in;
    fp.z_in = r.z_in;
    fp.ws = ws;
    fp.nseg = plan.nseg;
    fp.nsplit = plan.nsplit;
    fp.split_len = plan.split_len;
    fp.slot_vec = (r.d % 4 == 0) && aligned16(ws);
    fp.seg_len = plan.seg_len;
    const hipError_t e = la::launch_linear_state_prefix(fp, plan, r.bf16, s);
    if (e != hipSuccess) return e;
  }
  la::BwdParams p{};
  p.BH = r.BH;
  p.H = r.H;
  p.N = r.N;
  p.d = r.d;
  p.dv = r.dv;
  p.fmap = r.fmap;
  p.vec_ok = vec_ok;
  p.q = r.q;
  p.k = r.k;
  p.v = r.v;
  p.o = r.o;
  p.dout = r.dout;
  p.den = r.den;
  p.gamma = r.gamma;
  p.S_in = r.S_in;
  p.z_in = r.z_in;
  p.dS_out = r.dS_out;
  p.dz_out = r.dz_out;
  p.dq = r.dq;
  p.dk = r.dk;
  p.dv_ = r.dv_;
  p.dS_in = r.dS_in;
  p.dz_in = r.dz_in;
  p.ws_f = const_cast<float *>(ws_f);  // read only by the backward kernels
  p.ws_r = ws_r;
  p.wrec = plan.wrec;  // (slot records; also the per-chunk states with alpha)
  p.nseg = plan.nseg;
  p.seg_len = plan.seg_len;
  p.slot_vec = (r.d % 4 == 0) && aligned16(ws_f) && aligned16(ws_r);
  if (chan) {
    const size_t slots = plan.nseg > 1 ? backward_ws_bytes(plan, reuse) : 0;
    char *cw = wsb + round256(slots);
    const ChanBwdLayout C = chan_bwd_layout(r.BH, r.N, r.d, r.dv);
    p.alpha = r.alpha;
    p.dalpha = r.dalpha;
    p.ux = reinterpret_cast<float *>(cw + C.ux);
    p.chs = reinterpret_cast<float *>(cw + C.chs);
  }
  return la::launch_linear_backward(p, r.bf16, s);
}

// The fp32 backward over two value halves (see split_values), in the
// rule's part of the workspace (split_layout).
hipError_t rule_backward_split(const RuleBwd &r, char *ws, hipStream_t s) {
  const SplitLayout L = split_layout(r.BH, r.N, r.d, r.dv);
  const size_t rows = (size_t)r.BH * r.N, srows = (size_t)r.BH * r.d;
  const int na = kSplitCols;
  auto at = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
  hipError_t e = hipSuccess;
  auto split = [&](const void *src, size_t nrows, const size_t (&dst)[2]) {
    if (e == hipSuccess)
      e = la::launch_split_cols(static_cast<const float *>(src), at(dst[0]), at(dst[1]), nrows,
                                r.dv, na, s);
  };
  split(r.v, rows, L.v);
  split(r.o, rows, L.o);
  split(r.dout, rows, L.go);
  if (r.S_in) split(r.S_in, srows, L.sin);
  if (r.dS_out) split(r.dS_out, srows, L.gso);
  for (int h = 0; h < 2 && e == hipSuccess; ++h) {
    RuleBwd x = r;
    x.dv = h ? r.dv - na : na;
    x.v = at(L.v[h]);
    x.o = at(L.o[h]);
    x.dout = at(L.go[h]);
    x.S_in = r.S_in ? at(L.sin[h]) : nullptr;
    x.dS_out = r.dS_out ? at(L.gso[h]) : nullptr;
    x.dz_out = h ? nullptr : r.dz_out;
    x.dq = h ? at(L.gq) : r.dq;
    x.dk = h ? at(L.gk) : r.dk;
    x.dv_ = at(L.gv[h]);
    x.dS_in = r.dS_in ? at(L.gsi[h]) : nullptr;
    x.dz_in = r.dz_in ? (h ? at(L.gz) : r.dz_in) : nullptr;
    e = rule_backward(x, ws + L.slots, nullptr, s);
  }
  if (e == hipSuccess) e = la::launch_add_into(static_cast<float *>(r.dq), at(L.gq), rows * r.d, s);
  if (e == hipSuccess) e = la::launch_add_into(static_cast<float *>(r.dk), at(L.gk), rows * r.d, s);
  if (e == hipSuccess)
    e = la::launch_join_cols(static_cast<float *>(r.dv_), at(L.gv[0]), at(L.gv[1]), rows, r.dv,
                             na, s);
  if (e == hipSuccess && r.dS_in)
    e = la::launch_join_cols(r.dS_in, at(L.gsi[0]), at(L.gsi[1]), srows, r.dv, na, s);
  if (e == hipSuccess && r.dz_in) e = la::launch_add_into(r.dz_in, at(L.gz), srows, s);
  return e;
}

}  // namespace

size_t la_backward_workspace_size(const la_backward_args *a) {
  if (check_backward_shape(a) != LA_OK) return (size_t)-1;
  const int BH = a->B * a->H;
  if (BH == 0 || a->N == 0) return 0;
  const bool bf16 = a->dtype == LA_BF16, fwd = a->fwd_workspace != nullptr;
  return conv_bwd_layout(BH, a->N, a->d, a->dv, bf16 ? 2 : 4, a->conv_width,
                         a->conv_weight != nullptr, fwd,
                         rule_ws_bytes(BH, a->N, a->d, a->dv, bf16, fwd, a->alpha != nullptr))
      .total;
}

int la_backward(const la_backward_args *a, void *stream) {
  int st = check_backward_shape(a);
  if (st != LA_OK) return st;
  const int BH = a->B * a->H;
  if (BH > 0 && a->N > 0 &&
      (!a->q || !a->k || !a->v || !a->o || !a->den || !a->grad_o || !a->grad_q ||
       !a->grad_k || !a->grad_v || (a->alpha && !a->grad_alpha)))
    return LA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (BH == 0) return LA_OK;
  const size_t nS = (size_t)BH * a->d * a->dv, nz = (size_t)BH * a->d;
  if (a->N == 0) {  // no tokens: the final state is the initial state
    hipError_t e = hipSuccess;
    if (a->grad_S_in)
      e = a->grad_S_out ? la::launch_copy(a->grad_S_in, a->grad_S_out, nS, s)
                        : la::launch_fill(a->grad_S_in, nS, 0.f, s);
    if (e == hipSuccess && a->grad_z_in)
      e = a->grad_z_out ? la::launch_copy(a->grad_z_in, a->grad_z_out, nz, s)
                        : la::launch_fill(a->grad_z_in, nz, 0.f, s);
    if (e == hipSuccess && a->conv_weight)
      e = conv_grads_no_tokens(BH, a->H, a->d, a->dv, a->conv_width, a->dtype == LA_BF16,
                               a->grad_conv_out, a->grad_conv_weight, a->grad_conv_in, s);
    return to_status(e);
  }
  const bool bf16_io = a->dtype == LA_BF16;
  const size_t esz = bf16_io ? 2 : 4, rows = (size_t)BH * a->N;
  const bool conv = a->conv_weight != nullptr;
  const bool chan = a->alpha != nullptr;
  const la::LinearPlan plan = la::plan_linear(BH, a->N, a->d, a->dv, bf16_io, 0, chan);
  const bool split = split_values(a->d, a->dv, bf16_io);
  // the forward's own records, when given (same plan, same slots); else
  // this call's workspace, filled below
  const bool reuse = !split && plan.nseg > 1 && a->fwd_workspace != nullptr;
  const BwdLayout L =
      conv_bwd_layout(BH, a->N, a->d, a->dv, esz, a->conv_width, conv, a->fwd_workspace != nullptr,
                      rule_ws_bytes(BH, a->N, a->d, a->dv, bf16_io, a->fwd_workspace != nullptr,
                                    chan));
  if (L.total > 0 && (!a->workspace || a->workspace_bytes < L.total)) return LA_EWORKSPACE;
  if (L.total > 0 && ((conv || chan) ? !aligned16(a->workspace)
                                    : (reinterpret_cast<uintptr_t>(a->workspace) & 3u) != 0))
    return LA_EINVAL;
  // the forward's workspace: [convolved q, k, v (with a convolution) | state slots]
  const size_t fwd_copies = conv ? qkv_copy_bytes(rows, a->d, a->dv, esz) : 0;
  if (a->fwd_workspace && (conv || plan.nseg > 1)) {
    if (a->fwd_workspace_bytes < fwd_copies + (plan.nseg > 1 ? plan.ws_bytes : 0))
      return LA_EWORKSPACE;
    if (conv ? !aligned16(a->fwd_workspace)
             : (reinterpret_cast<uintptr_t>(a->fwd_workspace) & 3u) != 0)
      return LA_EINVAL;
  }
  char *base = static_cast<char *>(a->workspace);
  // the rule's inputs and gradients: q, k, v themselves, or with a
  // convolution the convolved copies and dL/d(those copies)
  const void *q = a->q, *k = a->k, *v = a->v;
  void *gq = a->grad_q, *gk = a->grad_k, *gv = a->grad_v;
  if (conv) {
    if (a->fwd_workspace) {
      void *fq, *fk, *fv;
      qkv_regions(const_cast<char *>(static_cast<const char *>(a->fwd_workspace)), rows, a->d,
                  esz, &fq, &fk, &fv);
      q = fq;
      k = fk;
      v = fv;
    } else {
      const hipError_t e =
          run_conv_pass(BH, a->H, a->N, a->d, a->dv, bf16_io, a->conv_weight, a->conv_width,
                        a->q, a->k, a->v, a->conv_in, nullptr, base + L.copies, s, &q, &k, &v);
      if (e != hipSuccess) return LA_EHIP;
    }
    qkv_regions(base + L.grads, rows, a->d, esz, &gq, &gk, &gv);
  }
  RuleBwd r{};
  r.BH = BH;
  r.H = a->H;
  r.N = a->N;
  r.d = a->d;
  r.dv = a->dv;
  r.fmap = a->fmap == LA_FMAP_ELU1;
  r.bf16 = bf16_io;
  r.q = q;
  r.k = k;
  r.v = v;
  r.o = a->o;
  r.dout = a->grad_o;
  r.den = a->den;
  r.gamma = a->gamma;
  r.S_in = a->S_in;
  r.z_in = a->z_in;
  r.dS_out = a->grad_S_out;
  r.dz_out = a->grad_z_out;
  r.dq = gq;
  r.dk = gk;
  r.dv_ = gv;
  r.dS_in = a->grad_S_in;
  r.dz_in = a->grad_z_in;
  r.alpha = a->alpha;
  r.dalpha = a->grad_alpha;
  hipError_t e;
  if (split) {
    e = rule_backward_split(r, base + L.slots, s);
  } else {
    const float *fwd_slots =
        reuse ? reinterpret_cast<const float *>(static_cast<const char *>(a->fwd_workspace) +
                                                fwd_copies)
              : nullptr;
    e = rule_backward(r, base ? base + L.slots : nullptr, fwd_slots, s);
  }
  if (e != hipSuccess || !conv) return to_status(e);
  return to_status(conv_backward(BH, a->H, a->N, a->d, a->dv, bf16_io, a->conv_weight,
                                 a->conv_width, a->q, a->k, a->v, a->conv_in, gq, gk, gv,
                                 a->grad_conv_out, a->grad_q, a->grad_k, a->grad_v,
                                 a->grad_conv_in, a->grad_conv_weight, base + L.part, s));
}

namespace {

int check_delta_backward_shape(const la_delta_backward_args *a) {
  if (!a) return LA_EINVAL;
  if (a->B < 0 || a->H < 0 || a->N < 0 || !dims_ok(a->d, a->dv)) return LA_EINVAL;
  if ((long long)a->B * a->H > 0x7fffffffLL) return LA_EUNSUPPORTED;
  if (a->dtype != LA_F32 && a->dtype != LA_BF16) return LA_EINVAL;
  if (a->dtype != LA_BF16) return LA_EUNSUPPORTED;
  // the state and reverse passes run 256 threads per (head, 16 value
  // columns) along one grid axis
  if ((unsigned long long)a->B * a->H * ((a->dv + 15) / 16) * 256 > kMaxGridItems)
    return LA_EUNSUPPORTED;
  const size_t dmax = a->d > a->dv ? a->d : a->dv;
  if ((size_t)a->N * dmax * 2 > kMaxHeadBytes) return LA_EUNSUPPORTED;
  // one head's preparation records must be addressable with 32-bit offsets
  const size_t nch = ((size_t)a->N + 63) / 64, dk = a->d <= 64 ? 64 : 128;
  if (nch * (2 * dk * 64 + 64 * 64) * 2 > kMaxHeadBytes) return LA_EUNSUPPORTED;
  return check_conv_grads(a->conv_weight, a->conv_width, a->conv_in, a->grad_conv_out,
                          a->grad_conv_weight, a->grad_conv_in);
}

}  // namespace

size_t la_delta_backward_workspace_size(const la_delta_backward_args *a) {
  if (check_delta_backward_shape(a) != LA_OK) return (size_t)-1;
  const int BH = a->B * a->H;
  if (BH == 0 || a->N == 0) return 0;
  return conv_bwd_layout(BH, a->N, a->d, a->dv, 2, a->conv_width, a->conv_weight != nullptr,
                         false, la::delta_backward_sizes(BH, a->N, a->d, a->dv).bytes)
      .total;
}

int la_delta_backward(const la_delta_backward_args *a, void *stream) {
  int st = check_delta_backward_shape(a);
  if (st != LA_OK) return st;
  const int BH = a->B * a->H;
  if ((a->alpha != nullptr) != (a->grad_alpha != nullptr) && BH > 0 && a->N > 0)
    return LA_EINVAL;
  if (BH > 0 && a->N > 0 &&
      (!a->q || !a->k || !a->v || !a->g || !a->grad_o || !a->grad_q || !a->grad_k ||
       !a->grad_v || !a->grad_g))
    return LA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (BH == 0) return LA_OK;
  const size_t nS = (size_t)BH * a->d * a->dv;
  if (a->N == 0) {  // no tokens: the final state is the initial state
    hipError_t e = hipSuccess;
    if (a->grad_S_in)
      e = a->grad_S_out ? la::launch_copy(a->grad_S_in, a->grad_S_out, nS, s)
                        : la::launch_fill(a->grad_S_in, nS, 0.f, s);
    if (e == hipSuccess && a->conv_weight)
      e = conv_grads_no_tokens(BH, a->H, a->d, a->dv, a->conv_width, true, a->grad_conv_out,
                               a->grad_conv_weight, a->grad_conv_in, s);
    return to_status(e);
  }
  const la::BwdDeltaSizes z = la::delta_backward_sizes(BH, a->N, a->d, a->dv);
  const bool conv = a->conv_weight != nullptr;
  const size_t rows = (size_t)BH * a->N;
  const BwdLayout L = conv_bwd_layout(BH, a->N, a->d, a->dv, 2, a->conv_width, conv, false, z.bytes);
  if (!a->workspace || a->workspace_bytes < L.total) return LA_EWORKSPACE;
  if (!aligned16(a->workspace)) return LA_EINVAL;
  char *base = static_cast<char *>(a->workspace);
  // the rule's inputs and gradients: q, k, v themselves, or with a
  // convolution the convolved copies and dL/d(those copies)
  const void *q = a->q, *k = a->k, *v = a->v;
  void *gq = a->grad_q, *gk = a->grad_k, *gv = a->grad_v;
  if (conv) {
    const hipError_t e =
        run_conv_pass(BH, a->H, a->N, a->d, a->dv, true, a->conv_weight, a->conv_width, a->q,
                      a->k, a->v, a->conv_in, nullptr, base + L.copies, s, &q, &k, &v);
    if (e != hipSuccess) return LA_EHIP;
    qkv_regions(base + L.grads, rows, a->d, 2, &gq, &gk, &gv);
  }
  la::BwdDeltaParams p{};
  p.BH = BH;
  p.H = a->H;
  p.N = a->N;
  p.d = a->d;
  p.dv = a->dv;
  p.dvp = z.dvp;
  p.nch = z.nch;
  p.vec_ok = (a->d % 8 == 0) && (a->dv % 8 == 0) && aligned16(q) && aligned16(k) &&
             aligned16(v) && aligned16(a->grad_o) && aligned16(gq) && aligned16(gk) &&
             aligned16(gv);
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = a->grad_o;
  p.g = a->g;
  p.alpha = a->alpha;
  p.S_in = a->S_in;
  p.dS_out = a->grad_S_out;
  p.dq = gq;
  p.dk = gk;
  p.dv_ = gv;
  p.dg = a->grad_g;
  p.dalpha = a->grad_alpha;
  p.dS_in = a->grad_S_in;
  p.ws = base + L.slots;
  p.lay_dec = z.dec;
  p.lay_states = z.states;
  p.lay_adj = z.adj;
  p.lay_y = z.y;
  p.lay_dd = z.dd;
  hipError_t e = la::launch_delta_backward(p, s);
  if (e != hipSuccess || !conv) return to_status(e);
  return to_status(conv_backward(BH, a->H, a->N, a->d, a->dv, true, a->conv_weight,
                                 a->conv_width, a->q, a->k, a->v, a->conv_in, gq, gk, gv,
                                 a->grad_conv_out, a->grad_q, a->grad_k, a->grad_v,
                                 a->grad_conv_in, a->grad_conv_weight, base + L.part, s));
}

int la_decode_step(const la_decode_args *a, void *stream) {
  if (!a) return LA_EINVAL;
  if (a->B < 0 || a->H < 0 || !dims_ok(a->d, a->dv)) return LA_EINVAL;
  if (a->dtype != LA_F32 && a->dtype != LA_BF16) return LA_EINVAL;
  if (a->rule != LA_RULE_LINEAR && a->rule != LA_RULE_DELTA) return LA_EINVAL;
  if (a->fmap != LA_FMAP_IDENTITY && a->fmap != LA_FMAP_ELU1) return LA_EINVAL;
  const bool delta = a->rule == LA_RULE_DELTA;
  const long long BH = (long long)a->B * a->H;
  // one 256-thread workgroup per (b, h) along one grid axis
  if ((unsigned long long)BH * 256 > kMaxGridItems) return LA_EUNSUPPORTED;
  if (delta) {
    if (a->fmap != LA_FMAP_IDENTITY || a->gamma || a->z) return LA_EINVAL;
    if (BH > 0 && !a->g) return LA_EINVAL;
  } else {
    if (a->g || (a->alpha && a->gamma) || !(a->eps >= 0.f) || !std::isfinite(a->eps))
      return LA_EINVAL;
    if (BH > 0 && !a->z) return LA_EINVAL;
  }
  if (a->conv_weight) {
    if (a->conv_width < 1 || a->conv_width > kMaxConvWidth) return LA_EINVAL;
    if (BH > 0 && a->conv_width > 1 && !a->conv_cache) return LA_EINVAL;
  } else if (a->conv_width != 0 || a->conv_cache) {
    return LA_EINVAL;
  }
  if (BH == 0) return LA_OK;
  if (!a->q || !a->k || !a->v || !a->o || !a->S) return LA_EINVAL;

  la::DecodeParams p{};
  p.BH = (int)BH;
  p.H = a->H;
  p.d = a->d;
  p.dv = a->dv;
  p.fmap = a->fmap == LA_FMAP_ELU1;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.gamma = a->gamma;
  p.g = a->g;
  p.alpha = a->alpha;
  p.eps = a->eps;
  p.S = a->S;
  p.z = a->z;
  p.o = a->o;
  p.conv_w = a->conv_weight;
  p.conv_width = a->conv_weight ? a->conv_width : 0;
  p.conv_cache = a->conv_cache;
  const int vec = (a->dv % 4 == 0 && aligned16(a->S)) ? 4 : 1;
  return to_status(la::launch_decode(p, a->dtype == LA_BF16, delta, vec,
                                     reinterpret_cast<hipStream_t>(stream)));
}

int la_state_init(float *S, float *z, int32_t B, int32_t H, int32_t d,
                  int32_t dv, void *stream) {
  if (B < 0 || H < 0 || !dims_ok(d, dv)) return LA_EINVAL;
  const size_t BH = (size_t)B * H;
  if (BH == 0) return LA_OK;
  if (!S) return LA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = la::launch_fill(S, BH * d * dv, 0.f, s);
  if (e == hipSuccess && z) e = la::launch_fill(z, BH * d, 0.f, s);
  return to_status(e);
}

int la_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(la::g_prof_mu);
  la::clear_log_locked();
  la::g_prof_on.store(on != 0, std::memory_order_relaxed);
  return LA_OK;
}

int la_profile_collect(la_kernel_time *out, int max) {
  std::lock_guard<std::mutex> lk(la::g_prof_mu);
  int n = 0;
  bool err = false;
  for (const auto &r : la::g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess ||
        hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      (void)hipGetLastError();
      err = true;
      break;
    }
    if (out && n < max) out[n] = la_kernel_time{r.name, ms};
    ++n;
  }
  la::clear_log_locked();
  if (err) return -1;
  return n < max ? n : max;
}

}  // extern "C"
