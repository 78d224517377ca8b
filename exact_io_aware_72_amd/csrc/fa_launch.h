// Host-side launch helpers of the forward launchers: device and occupancy
// queries, and the choice of causal block pairing (map_block_pairs /
// map_block_pair in fa_device.h).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace fa {

// CUs of the current device (cached per device; 0 if the query fails).
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Work-groups of `Kernel` that one CU holds at once (cached per instance;
// the kernels' resources do not depend on the device among gfx950 parts).
template <auto Kernel>
int resident_per_cu(int threads) {
  static std::atomic<int> cache{-1};
  int n = cache.load(std::memory_order_relaxed);
  if (n < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(Kernel), threads, 0) !=
        hipSuccess)
      n = 0;
    cache.store(n, std::memory_order_relaxed);
  }
  return n;
}

// Causal masks give the blocks of a head linearly growing (or shrinking)
// work, so blocks are paired:
// - a grid that the device holds at once, as an even number of work-groups
//   per CU: the work-groups of each CU take complementary blocks
//   (pair_slots, map_block_pairs), so every CU gets equal work;
// - with group_mode, a larger grid, when the paired grid still fills the
//   device: each work-group takes a complementary pair (pair_blocks,
//   map_block_pair),
//   one block over ascending tiles and the other over descending ones.
//   Every work-group then does the same work, and at any moment the
//   work-groups of one head read only two tiles of the streamed operands
//   (position t of one sweep and position const - t of the other), which
//   the XCD's L2 holds.
struct BlockPairing {
  int grid;          // work-groups to launch
  int pair_slots;    // > 0: resident pairing across the work-groups of a CU
  int cus_per_xcd;
  int pair_blocks;   // 1: one pair of blocks per work-group
};

template <auto Kernel>
BlockPairing plan_block_pairs(int nblk, int BH, int threads, bool eligible, bool resident_mode,
                              bool group_mode) {
  BlockPairing r{nblk * BH, 0, 0, 0};
  if (!eligible) return r;
  const int ncu = device_cus();
  const int cap = ncu * resident_per_cu<Kernel>(threads);
  const int n = nblk * BH;
  if (n <= cap) {
    if (resident_mode && (BH & 7) == 0 && (nblk & 1) == 0 && ncu > 0 && (ncu & 7) == 0 && n % ncu == 0 &&
        ((n / ncu) & 1) == 0) {
      r.pair_slots = n / ncu;
      r.cus_per_xcd = ncu / 8;
    }
  } else if (group_mode && (nblk + 1) / 2 * BH >= cap) {
    r.pair_blocks = 1;
    r.grid = (nblk + 1) / 2 * BH;
  }
  return r;
}

}  // namespace fa
