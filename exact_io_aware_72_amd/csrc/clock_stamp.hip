// Clock stamps for the benchmark: the shader-cycle counter (s_memtime) and
// the fixed 100 MHz real-time counter (s_memrealtime), read by one wave per
// work-group, with the XCD and the CU (shader engine, array and CU fields of
// HW_ID) that the wave ran on. Two stamps on a stream, before and after a
// timed region, give each XCD's mean shader clock over that region as
// 100 MHz * (cycles elapsed) / (real-time ticks elapsed), from stamps taken
// on the same CU. Not part of the attention library: built as its own
// shared object for measurement.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_clock.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

__global__ __launch_bounds__(64) void clock_stamp_kernel(uint64_t* out) {
  if (threadIdx.x != 0) return;
  uint32_t xcc, hwid;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID, 8, 8)" : "=s"(hwid));  // CU, SH, SE
  const uint64_t cyc = __builtin_amdgcn_s_memtime();
  const uint64_t rt = __builtin_amdgcn_s_memrealtime();
  uint64_t* o = out + 4 * blockIdx.x;
  o[0] = xcc;
  o[1] = cyc;
  o[2] = rt;
  o[3] = hwid;
}

}  // namespace

FA_EXPORT int fa_clock_stamp(uint64_t* out, int blocks, void* stream) {
  if (out == nullptr || (reinterpret_cast<uintptr_t>(out) & 7u) != 0) return -1;
  if (blocks < 1 || blocks > 1024) return -1;
  hipLaunchKernelGGL(clock_stamp_kernel, dim3(blocks), dim3(64), 0,
                     static_cast<hipStream_t>(stream), out);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}
