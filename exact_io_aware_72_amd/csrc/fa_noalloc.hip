// fa_backward_noalloc: the backward pass with its D workspace in a
// file-scope device array instead of caller-supplied memory, for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array is the `scratch` below, FA_NOALLOC_MAX_ROWS floats (16 MiB) per
// GPU the library runs on, held until the process ends. Host code never
// passes its name to a kernel: on first use on a device, with that device
// current, hipGetSymbolAddress gives that device's copy's address, which is
// kept per device and passed to the kernels like the workspace argument of
// fa_backward. Every call on one GPU shares that GPU's array; the
// preprocess kernel rewrites every entry the later kernels read (B*H*N of
// them), so nothing needs clearing, but calls that overlap on one GPU (on
// different streams, or from several threads without ordering) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_kernels.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_ptr[kMaxDevices] = {};

// This device's copy of `scratch`, resolved once per device.
hipError_t scratch_ptr(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

FA_EXPORT int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                                  const void* dout, const float* lse, void* dq, void* dk,
                                  void* dv, int B, int H, int N, int d, float scale, int causal,
                                  float dropout_p, uint64_t seed, void* stream, int dtype) {
  const int st = fa::check_backward_args(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale,
                                         causal, dropout_p, seed, dtype);
  if (st != FA_OK) return st;
  // check_backward_args bounds B * N * H by 2^36, so the product is exact.
  if ((int64_t)B * H * N > (int64_t)FA_NOALLOC_MAX_ROWS) return FA_ERR_SHAPE;
  float* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return fa::record_hip_error(e);  // nothing launched
  return fa_backward(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, d, scale, causal, dropout_p,
                     seed, stream, dtype);
}
