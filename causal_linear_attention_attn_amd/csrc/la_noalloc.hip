// la_prefill_noalloc: la_prefill with its workspace in a static device
// array, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ object of LA_NOALLOC_SCRATCH_BYTES;
// every GPU the library runs on holds its own copy until the process ends.
// In host code its name is only a host-side stand-in, never a device
// address: on the first call on a device (with that device current) the
// device address is taken with hipGetSymbolAddress and kept per device, and
// only that address is handed to the kernels.  Nothing here allocates: the
// call validates, looks up the kept address and runs la_prefill on it.
// The prefill kernels write every workspace element they read before
// reading it (segment records, scan slots, the conv-cache copy, the delta
// rule's per-chunk records), so nothing is cleared between calls.  Calls
// that overlap on one GPU (two streams, two threads) share the array and
// race; the caller serialises them.
#include <mutex>

#include "../../include/linattn.h"
#include "la_internal.hpp"

namespace {

constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_addr[kMaxDevices];  // device address of `scratch`, per device

// Device address of this device's scratch array (nullptr on failure).
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_addr[dev] = p;
  }
  return g_addr[dev];
}

}  // namespace

extern "C" int la_prefill_noalloc(const la_prefill_args *a, void *stream) {
  if (!a) return LA_EINVAL;
  if (a->workspace || a->workspace_bytes) return LA_EINVAL;
  const size_t need = la_prefill_workspace_size(a);
  if (need == (size_t)-1 || need == 0) return la_prefill(a, stream);  // its own checks
  if (need > kScratchBytes) return LA_ESCRATCH;
  void *ws = scratch_address();
  if (!ws) return LA_EHIP;
  la_prefill_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = kScratchBytes;
  return la_prefill(&b, stream);
}
