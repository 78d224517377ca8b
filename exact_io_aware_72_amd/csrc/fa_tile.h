// LDS tile layout for the gfx950 kernels, filled by direct global->LDS loads.
//
// A tile holds R rows of D bf16 values (one row per key or query), row-major,
// cut into groups of eight 16-byte chunks (128 bytes of a row per group) plus,
// for D = 80, a tail group of two chunks (32 bytes of a row). Within a group
// the chunk position is XOR-swizzled by the row so that the matrix-core
// operand reads of one LDS pass land in distinct banks:
//   kRow: 16-byte reads, lane = row, one chunk column (operands along D);
//   kTr:  8-byte transposing reads (ds_read_b64_tr_b16), four rows and two
//         chunks per 16 lanes (operands along the rows);
//   kBoth: both of the above from one copy of the tile.
// A direct-to-LDS buffer load writes 64 consecutive 16-byte slots (one per
// lane, in lane order), so each load instruction fills 8 rows of one group
// (or 32 rows of the tail) and the swizzle is applied by choosing which chunk
// each lane fetches. Rows at or past the end of the sequence are fetched
// through the buffer's range check and arrive as zeros.
#pragma once

#include "fa_device.h"

namespace fa {

enum class Swz { kRow, kTr, kBoth };

template <int R, int D, Swz S>
struct Tile {
  static constexpr int NG = D / 64;          // full 8-chunk groups
  static constexpr int TC = (D % 64) / 8;    // chunks in the tail group
  static_assert((TC == 0 || TC == 2) && D % 16 == 0, "head dim must be 64, 80 or 128");
  static_assert(R % 32 == 0, "tile rows must be a multiple of 32");
  static constexpr int GBYTES = R * 128;     // bytes of one full group
  static constexpr int TAIL = NG * GBYTES;   // offset of the tail group
  static constexpr int BYTES = R * D * 2;
  static constexpr int NFULL = NG * (R / 8);  // load instructions for the full groups
  static constexpr int NTAIL = TC ? R / 32 : 0;
  static constexpr int NLOAD = NFULL + NTAIL;

  // Chunk swizzle of row r. kRow: distinct over any 8 (and, by row parity,
  // 16) consecutive rows. kTr: rows 4k..4k+3 get values differing in bits 1-2,
  // so two adjacent chunks of four rows land in 8 distinct positions. kBoth
  // satisfies both conditions.
  __device__ __forceinline__ static int sw(int r) {
    if constexpr (S == Swz::kRow) return (r ^ (r >> 3)) & 7;
    if constexpr (S == Swz::kTr) return (((r & 3) << 1) ^ (r >> 2)) & 7;
    return ((((r & 3) << 1) | ((r >> 2) & 1)) ^ (((r >> 3) & 1) << 1)) & 7;
  }
  __device__ __forceinline__ static int swt(int r) {
    return S == Swz::kTr ? 0 : (((r >> 2) ^ (r >> 3)) & 1);
  }
  // Load instruction i (0 <= i < NLOAD): the LDS byte offset it writes
  // (uniform over the wave) and the row and 16-byte chunk this lane fetches.
  __device__ __forceinline__ static void load_slot(int i, int lane, int& lds_off, int& row,
                                                   int& chunk) {
    if (i < NFULL) {
      const int gi = i / (R / 8), rb = (i % (R / 8)) * 8;
      row = rb + (lane >> 3);
      chunk = 8 * gi + ((lane & 7) ^ sw(row));
      lds_off = gi * GBYTES + rb * 128;
    } else {
      const int rb = (i - NFULL) * 32;
      row = rb + (lane >> 1);
      chunk = 8 * NG + ((lane & 1) ^ swt(row));
      lds_off = TAIL + rb * 32;
    }
  }

  // kRow read of the 16-byte chunk `chunk` of row r (byte offset in the tile).
  __device__ __forceinline__ static int row_chunk_off(int r, int chunk) {
    if (chunk < 8 * NG) return (chunk >> 3) * GBYTES + r * 128 + (((chunk & 7) ^ sw(r)) << 4);
    return TAIL + r * 32 + (((chunk - 8 * NG) ^ swt(r)) << 4);
  }
};

// LDS tile of R rows of D FP8 bytes (one byte per element), for 16-byte row
// reads (matrix-core operands along D). Rows are 64 bytes (D = 64) or 128
// bytes (D = 80 or 128; the chunks past D are filled with zeros); the chunk
// position is XOR-swizzled by the row so that the 16 lanes of one LDS pass
// (16 consecutive rows, one chunk column) hit 16 distinct 16-byte bank
// groups: (r ^ r >> 3) & 7 for 8-chunk rows as in Tile<.., kRow>, (r >> 2) & 3
// for 4-chunk rows (rows r, r + 4, r + 8, r + 12 share a bank group base).
template <int R, int D>
struct Fp8Tile {
  static_assert(D == 64 || D == 80 || D == 128, "head dim must be 64, 80 or 128");
  static constexpr int RB = D == 64 ? 64 : 128;  // LDS bytes per row
  static constexpr int CPR = RB / 16;             // chunks per row
  static constexpr int VALID = (D + 15) / 16;     // chunks holding data
  static constexpr int BYTES = R * RB;
  static constexpr int RPL = 64 / CPR;            // rows per load instruction
  static_assert(R % RPL == 0, "whole load instructions");
  static constexpr int NLOAD = R / RPL;

  __device__ __forceinline__ static int sw(int r) {
    return CPR == 8 ? ((r ^ (r >> 3)) & 7) : ((r >> 2) & 3);
  }
  // Load instruction i: LDS byte offset (uniform), and the row and chunk
  // this lane fetches; chunk >= VALID must be fetched as zeros.
  __device__ __forceinline__ static void load_slot(int i, int lane, int& lds_off, int& row,
                                                   int& chunk) {
    row = i * RPL + lane / CPR;
    chunk = (lane % CPR) ^ sw(row);
    lds_off = i * 1024;
  }
  // Byte offset of chunk c of row r.
  __device__ __forceinline__ static int off(int r, int c) { return r * RB + ((c ^ sw(r)) << 4); }
};

// Direct global->LDS load of 16 bytes per lane: lane L's data lands at
// lds + 16 * L. `lds` must be the same for the whole wave.
__device__ __forceinline__ void lds_dma_16(BufRes r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte values read by lanes i / 4 + 4 j (j = 0..3), i.e. four
// rows of one column when lanes 4j + a address row j, columns 4a..4a+3.
__device__ __forceinline__ u32x2 ld_lds_tr16(const char* base, int off) {
  const auto v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(const_cast<char*>(base) + off));
  return __builtin_bit_cast(u32x2, v);
}

// Race-detection builds (-DFA_LDS_POISON): once every wave is past the
// barrier after its last read of an LDS stage, and before the next tile's
// loads into that stage are issued, the stage is filled with all-ones bytes
// (NaN as bf16 and as fp32). A read that runs ahead of those loads, or a
// stage reused too early, then shows up as NaN outputs instead of stale but
// plausible values. Regular builds compile this to nothing.
#ifdef FA_LDS_POISON
constexpr bool kLdsPoison = true;
#else
constexpr bool kLdsPoison = false;
#endif
// Every thread of the work-group must call this (it ends with a barrier);
// threads tid = 0 .. nt-1 fill `bytes` bytes (a multiple of 16) at `stage`.
__device__ __forceinline__ void poison_stage(char* stage, int bytes, int tid, int nt) {
  if constexpr (kLdsPoison) {
    for (int i = tid; i < bytes / 16; i += nt)
      reinterpret_cast<u32x4*>(stage)[i] = u32x4{~0u, ~0u, ~0u, ~0u};
    __syncthreads();  // stored before any wave issues its loads into the stage
  }
}

// Waits for this wave's outstanding global loads (direct-to-LDS included)
// and nothing else: s_waitcnt vmcnt(0) with expcnt and lgkmcnt at maximum.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace fa
