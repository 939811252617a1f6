// noalloc.hip -- selective_scan_fwd_noalloc: the forward call with its scratch memory in a
// file-scope device array instead of a caller workspace, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in every GPU's copy of the code object for the life of the process.  Its
// device address is taken once per device, with that device current, by hipGetSymbolAddress;
// host code uses only that address, never the symbol (on the host the symbol is a stand-in,
// not device memory).  Every call on one GPU shares that GPU's array: calls that may overlap
// on one GPU (several streams, several host threads) race.  The array's contents need no
// clearing between calls: the segment pass writes every slot the carry and the output pass
// then read.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"
#include "sss.h"

namespace sss {
namespace {

constexpr size_t kScratchBytes = (size_t)96 << 20;  // SSS_NOALLOC_SCRATCH_BYTES in sss.h
static_assert(kScratchBytes == SSS_NOALLOC_SCRATCH_BYTES, "scratch size and its public value");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDev = 64;
std::atomic<void*> g_scratch[kMaxDev];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (nullptr on failure).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace
}  // namespace sss

extern "C" int selective_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const float* B,
                                          const float* C, const float* D_skip, const void* z, const float* h0,
                                          float* y, float* h_last, int64_t batch, int64_t seqlen, int64_t dim,
                                          int64_t dstate, int io_dtype, sss_stream_t stream) {
  // argument errors first (the same checks and codes as selective_scan_fwd), before the
  // scratch address is looked up
  if (!x || !delta || !A || !B || !C || !y) return SSS_ERR_NULL_ARG;
  void* ws = sss::device_scratch();
  if (ws == nullptr) return SSS_ERR_HIP;
  // the plan is sized to the array: fewer time segments when the usual plan needs more
  // scratch than it holds (a single segment needs none, so no valid shape is refused for its
  // size; sel_fwd_impl still checks the plan against the array and returns SSS_ERR_WORKSPACE
  // if it ever exceeded it)
  return sss::sel_fwd_impl(x, delta, A, B, C, D_skip, z, h0, y, h_last, nullptr, 0u, batch, seqlen, dim, dstate,
                           io_dtype, ws, sss::kScratchBytes, sss::kScratchBytes, stream);
}
