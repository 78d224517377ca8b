// Measurement aid: the sustained rate of the bf16 matrix cores on given
// operand data, with no memory traffic, LDS or vector work around them.
//
// The attention kernels' roofline is the published dense bf16 matrix-core
// peak, but what the chip sustains also depends on the operand bits: the
// same instruction stream runs at a lower rate on random data than on
// constant data (the chip holds its power budget by lowering the clock and
// the issue rate). Timing this kernel on the workload's own value
// distribution gives the ceiling the attention kernels can reach on that
// data.
//
// Each wave loads sixteen 32x32x16 operand fragments (lane L reads 16-byte
// entry f * 64 + L of the operand buffer for fragment f) and then issues
// `iters` x 16 products into four independent accumulators: A_i B_i for
// i = 0..7 and B_i A_{(i+1) mod 8} for i = 0..7, accumulator i mod 4. Each
// lane writes the sum of its 64 accumulator registers, so the sum over a
// wave's lanes is iters times the sum of all elements of those 16 products.
#include "../../include/fa.h"
#include "fa_device.h"

namespace fa {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(const u32x4* __restrict__ frag,
                                                                   float* __restrict__ out,
                                                                   int iters) {
  const int lane = threadIdx.x & 63;
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = frag[i * 64 + lane];
    b[i] = frag[(8 + i) * 64 + lane];
  }
  f32x16 c[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i & 3] = mfma32x32x16(a[i], b[i], c[i & 3]);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i & 3] = mfma32x32x16(b[i], a[(i + 1) & 7], c[i & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace fa

// C entry point (declared in fa.h): arguments are checked before any HIP
// call; FA_ERR_HIP carries no detail string here (fa_status_string reports
// the last error of the attention entry points only).
extern "C" __attribute__((visibility("default"))) int fa_probe_mfma_rate(const void* operands,
                                                                        float* out, int blocks,
                                                                        int iters, void* stream) {
  if (operands == nullptr || out == nullptr) return FA_ERR_NULL;
  if (((reinterpret_cast<uintptr_t>(operands) | reinterpret_cast<uintptr_t>(out)) & 15u) != 0)
    return FA_ERR_ALIGN;
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 24)) return FA_ERR_ARG;
  hipLaunchKernelGGL(fa::probe_mfma_kernel, dim3(blocks), dim3(fa::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const fa::u32x4*>(operands), out, iters);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
