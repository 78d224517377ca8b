/*
 * Clock stamps for benchmarking (libfa_clock.so, separate from the attention
 * library libfa.so): the mean shader clock of each XCD over a timed region.
 *
 * fa_clock_stamp enqueues, on `stream`, a kernel of `blocks` work-groups of
 * one wave; work-group i writes four uint64 values to out[4i .. 4i+3]: the
 * XCD it ran on (the XCC_ID hardware register, 0..7), the shader-cycle
 * counter (s_memtime), the real-time counter (s_memrealtime, 100 MHz), and
 * bits 8..15 of the HW_ID register (CU, shader array and shader engine of
 * the wave). Work-groups are dispatched round-robin over the XCDs, so 8
 * work-groups cover all of them. Two stamps around a region give each
 * XCD's mean clock as 100 MHz * delta(cycles) / delta(real time), from
 * stamps matched by XCD and CU.
 *   out     device, 8-byte aligned, 4 * blocks uint64 values, written
 *   blocks  1 .. 1024
 * Returns 0 when enqueued, -1 for a NULL or misaligned `out` or a block
 * count out of range (nothing launched), -8 if the launch failed.
 */
#ifndef FA_CLOCK_H_
#define FA_CLOCK_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int fa_clock_stamp(uint64_t* out, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_CLOCK_H_ */
