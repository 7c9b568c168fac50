// fsa_backward_noalloc: the backward pass with its scratch (per-row softmax
// terms and per-tile dalpha partials) in a fixed device array instead of a
// caller workspace, for callers that cannot allocate device memory.
//
// The array lives in this file. Host code never passes its name to a kernel:
// in host code the name is a host-side stand-in, not a device address. The
// device address is looked up once per device with hipGetSymbolAddress (that
// device current) and kept; every use goes through the kept address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fsa.h"
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr size_t kScratchBytes = FSA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device

// Device address of the scratch array on the stream's device: looked up on
// the first call for that device, with that device made current for the
// lookup and the caller's current device restored after it.
int scratch_on(hipStream_t s, void** out) {
  int dev = 0;
  // the null stream runs on the current device
  hipError_t e = s == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return status_of(e);
  if (dev < 0 || dev >= kMaxDevices) return FSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return status_of(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return status_of(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return status_of(e);
    if (r != hipSuccess) return status_of(r);
    if (p == nullptr) return FSA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FSA_OK;
}

}  // namespace
}  // namespace fsa

extern "C" int fsa_backward_noalloc(const void* q, const void* k, const void* v,
                                    const void* dout, const float* lse, int dtype,
                                    int B, int H, int T, int D, float alpha,
                                    int window, int pattern, float* dq, float* dk,
                                    float* dv, float* dalpha, void* stream) {
  bool empty = false;
  int st = fsa::check_backward_call(q, k, v, dout, lse, dtype, B, H, T, D, alpha,
                                    window, pattern, dq, dk, dv, dalpha, &empty);
  if (st != FSA_OK) return st;
  if (empty)                                          // writes dalpha only
    return fsa_backward_ex(q, k, v, dout, lse, dtype, B, H, T, D, alpha, window,
                           pattern, dq, dk, dv, dalpha, nullptr, 0, stream);
  if (fsa_backward_workspace_size(B, H, T, D, dtype) > fsa::kScratchBytes)
    return FSA_ERR_SCRATCH;
  void* ws = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = fsa::scratch_on(s, &ws);
  if (st != FSA_OK) return st;
  return fsa_backward_ex(q, k, v, dout, lse, dtype, B, H, T, D, alpha, window,
                         pattern, dq, dk, dv, dalpha, ws, fsa::kScratchBytes, stream);
}
