// Dropout keep-mask counter hash, regenerated identically by the forward
// and both backward kernels so the N x N mask is never stored.
//
// The pages fuse dropout into the attention kernel without naming a
// generator. This library's generator keys one 64-bit value per head, one
// 32-bit value per query row and per key column, and mixes them per element:
//   G    = 0x9E3779B97F4A7C15
//   mix64: SplitMix64 output function (Steele, Lea and Flood, OOPSLA 2014)
//   fmix32: MurmurHash3 32-bit finalizer (Appleby, public domain)
//   K_bh = mix64(seed + G*(1 + b*H + h))
//   A_i  = lo32(mix64(K_bh + G*(2i+1))),  B_j = lo32(mix64(K_bh + G*(2j+2)))
//   keep(i, j) = fmix32(A_i ^ B_j) >= T,  T = floor(p * 2^32)
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

__host__ __device__ __forceinline__ uint32_t murmur3_fmix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return x;
}

__host__ __device__ __forceinline__ uint64_t head_key(uint64_t seed, int b, int h, int H) {
  return splitmix64_out(seed + kGolden * (uint64_t)(1 + (int64_t)b * H + h));
}

__host__ __device__ __forceinline__ uint32_t row_key(uint64_t kbh, int i) {
  return (uint32_t)splitmix64_out(kbh + kGolden * (2ull * (uint64_t)i + 1ull));
}

__host__ __device__ __forceinline__ uint32_t col_key(uint64_t kbh, int j) {
  return (uint32_t)splitmix64_out(kbh + kGolden * (2ull * (uint64_t)j + 2ull));
}

__host__ __device__ __forceinline__ bool keep(uint32_t a, uint32_t b, uint32_t threshold) {
  return murmur3_fmix32(a ^ b) >= threshold;
}

}  // namespace fa
