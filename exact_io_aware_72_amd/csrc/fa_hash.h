// Dropout keep-mask counter hash, regenerated identically by the forward
// and both backward kernels so the N x N mask is never stored.
//
// The pages fuse dropout into the attention kernel without naming a
// generator. This library's generator keys one 64-bit value per head, one
// 32-bit value per query row and one per pair of key columns, and mixes them
// per (row, pair):
//   G    = 0x9E3779B97F4A7C15
//   mix64: SplitMix64 output function (Steele, Lea and Flood, OOPSLA 2014)
//   fmix32: MurmurHash3 32-bit finalizer (Appleby, public domain)
//   K_bh = mix64(seed + G*(1 + b*H + h))
//   A_i  = lo32(mix64(K_bh + G*(2i+1))),  B_c = lo32(mix64(K_bh + G*(2c+2)))
//   w    = fmix32(A_i ^ B_c): key j = 2c draws its low 16 bits, j = 2c+1 its high 16
//   keep(i, j) = u_ij >= T,  T = floor(p * 2^16)
// One hash gives two 16-bit draws, so a row's two neighbouring keys share one
// finalizer (two 32-bit multiplies, quarter-rate on the vector ALUs).
//
// The first step of fmix32, x ^= x >> 16, is linear over XOR, so row and pair
// keys are kept with it applied (premix) and the per-pair work starts at the
// first multiply. Of the last step, y ^= y >> 16, the high half of the result
// is the high half of y, so odd keys compare y itself against T << 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint64_t splitmix64_out(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ __forceinline__ uint64_t head_key(uint64_t seed, int b, int h, int H) {
  return splitmix64_out(seed + kGolden * (uint64_t)(1 + (int64_t)b * H + h));
}

__host__ __device__ __forceinline__ uint32_t premix(uint32_t x) { return x ^ (x >> 16); }

// premix(A_i)
__host__ __device__ __forceinline__ uint32_t row_key(uint64_t kbh, int i) {
  return premix((uint32_t)splitmix64_out(kbh + kGolden * (2ull * (uint64_t)i + 1ull)));
}

// premix(B_c) for the key pair c = j >> 1
__host__ __device__ __forceinline__ uint32_t pair_key(uint64_t kbh, int c) {
  return premix((uint32_t)splitmix64_out(kbh + kGolden * (2ull * (uint64_t)c + 2ull)));
}

// fmix32 without its first and last steps: the y with fmix32(A ^ B) =
// y ^ (y >> 16), from the premixed row and pair keys.
__host__ __device__ __forceinline__ uint32_t pair_mix(uint32_t arow, uint32_t bpair) {
  uint32_t x = arow ^ bpair;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  return x;
}

// Even key 2c: low 16 bits of fmix32, lo16(y) ^ hi16(y).
__host__ __device__ __forceinline__ bool keep_even(uint32_t y, uint32_t t16) {
  return (uint32_t)(uint16_t)(y ^ (y >> 16)) >= t16;
}

// Odd key 2c + 1: high 16 bits of fmix32, hi16(y).
__host__ __device__ __forceinline__ bool keep_odd(uint32_t y, uint32_t t16) { return y >= (t16 << 16); }

__host__ __device__ __forceinline__ bool keep_key(uint32_t y, int j, uint32_t t16) {
  return (j & 1) ? keep_odd(y, t16) : keep_even(y, t16);
}

}  // namespace fa
