// Device helpers for the gfx950 attention kernels: vector types, the bf16 and
// FP8 matrix-core instructions, LDS/global accesses, bf16 packing, lane
// exchanges, scheduling hints, sequence/block bookkeeping, and the
// contraction-index relabelling that lets a score tile held in accumulator
// registers feed the next matrix product without going through LDS.
//
// Matrix-core layout used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16, row m, column k):  lane L holds A[L % 32][8*(L/32) + j], j = 0..7
//   B (16 x 32, row k, column n):  lane L holds B[8*(L/32) + j][L % 32], j = 0..7
//   C (32 x 32):                   lane L, register r holds
//                                  C[8*(r/4) + 4*(L/32) + (r%4)][L % 32], r = 0..15
// The pairing of A and B elements along k is by (L/32, j) for both operands,
// so any relabelling of k applied to both operands leaves the product
// unchanged. A C tile therefore serves directly as the B operand of a product
// that contracts over its row index, provided the A operand is read with the
// same relabelling: for the 16 rows 16t..16t+15 of a C tile, lane half s
// supplies rows {16t + 4s + 0..3, 16t + 8 + 4s + 0..3} (c_row below), and the
// transposing LDS reads that build the matching A operand fetch those rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWave = 64;

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x64_f8f6f4 with both operands OCP FP8 E4M3 (format code
// 0): A is 32 x 64, B is 64 x 32, 32 bytes per lane each (a0 then a1). Lane
// L supplies row (A) or column (B) L % 32; the 32 bytes of lane half L / 32
// cover 32 consecutive contraction indices, and A and B pair the same
// indices, so both operands are loaded with one lane -> chunk map. Zero
// scale operands select the unscaled instruction.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1,
                                                   f32x16 c) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                   (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two floats -> two bf16 (round to nearest even) in one 32-bit word, lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// acc + lo + hi of the two bf16 halves of w, in one v_dot2 with ones. The
// word is taken by value: clang's __builtin_bit_cast applied directly to an
// ext-vector element reads the wrong element.
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Buffer resource over one (batch, head) slice: offsets are bytes from the
// slice start, and any 16-byte read at or past `bytes` returns zeros (the
// hardware range check), which is how rows past N are padded.
typedef __amdgpu_buffer_rsrc_t BufRes;
__device__ __forceinline__ BufRes make_bufres(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// Buffer resource over rows [row0, row0 + cap) of a (batch, head) slice
// whose rows lie `stride` bytes apart, cut at row n: reads of rows at or past
// n return zeros. Offsets are bytes from row row0, and the range is at most
// cap * stride bytes, so offsets stay 32-bit for slices of any size.
__device__ __forceinline__ BufRes rows_bufres(const void* slice, int row0, int n, int cap,
                                              uint32_t stride) {
  // readfirstlane: the clamp may be selected as a vector instruction, and a
  // resource held in vector registers would need a waterfall loop per load.
  const int rows = __builtin_amdgcn_readfirstlane(min(max(n - row0, 0), cap));
  return make_bufres(static_cast<const char*>(slice) + (int64_t)row0 * stride,
                     (uint32_t)rows * stride);
}
__device__ __forceinline__ u32x4 buf_load_128(BufRes r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(BufRes r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

__device__ __forceinline__ u32x4 ld_global_128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_global_64(void* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}
__device__ __forceinline__ u32x4 ld_lds_128(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// Exchange between lane L and lane L ^ 32 without LDS (v_permlane32_swap):
// swapping x with itself leaves {x_L, x_(L^32)} in the two results, in the
// same order on both lane halves, so the combined value is bitwise identical
// on lanes L and L ^ 32.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scheduling hint for a fully unrolled loop of `steps` steps, each issuing
// `reads` LDS reads and `mfmas` matrix products that consume them: the reads
// of the first `ahead` steps go first, then every step's products are
// followed by the reads of the step `ahead` steps later. Placed after the loop, in the same
// basic block; it only constrains instruction order.
// `first` extra reads (operands of other work in the block) join the first
// group; `ahead` is the lookahead in steps. `ds_mask` selects the LDS
// instruction class (0x100: reads; 0x080: any LDS access, which also covers
// the transposing reads).
template <int steps, int reads, int mfmas, int first = 0, int ahead = 2, int ds_mask = 0x100>
__device__ __forceinline__ void sched_lds_ahead() {
  constexpr int kMfma = 0x008, kDsRead = ds_mask;
  __builtin_amdgcn_sched_group_barrier(kDsRead, first + ahead * reads, 0);
#pragma unroll
  for (int c = 0; c < steps; ++c) {
    __builtin_amdgcn_sched_group_barrier(kMfma, mfmas, 0);
    if (c + ahead < steps) __builtin_amdgcn_sched_group_barrier(kDsRead, reads, 0);
  }
}

// Row index within a 32-row C tile held by accumulator register r of lane half s.
__device__ __forceinline__ constexpr int c_row(int r, int s) { return 8 * (r >> 2) + 4 * s + (r & 3); }

// Rows of one (sequence, head) pair: the sequence length, the element offset
// of its first row in the [.., H, d] tensors, and the offset of its first
// entry in the per-row statistics (lse, D). Fixed-length batches (cu ==
// nullptr): sequence s is batch item s of N rows, statistics [B][H][N].
// Packed variable-length batches: sequence s holds rows cu[s]..cu[s+1]-1 of
// [total, H, d] tensors, statistics [H][total]; offsets are clamped to
// [0, total] and lengths to max_n so that malformed offsets cannot address
// memory outside the tensors.
struct SeqRows {
  int n;
  int64_t base;
  int64_t stat;
};
__device__ __forceinline__ SeqRows seq_rows(const int* cu, int total, int s, int h, int H, int D,
                                            int max_n) {
  SeqRows r;
  if (cu == nullptr) {
    r.n = max_n;
    r.base = ((int64_t)s * max_n * H + h) * D;
    r.stat = ((int64_t)s * H + h) * max_n;
  } else {
    const int a = min(max(cu[s], 0), total);
    const int e = min(max(cu[s + 1], a), total);
    r.n = min(e - a, max_n);
    r.base = ((int64_t)a * H + h) * D;
    r.stat = (int64_t)h * total + a;
  }
  return r;
}

// Block-sparse masks (layout in fa_kernels.h): the kernels visit only kept
// blocks, so their tiles (64 or 32 rows) never straddle a block edge. One
// wave collects a work-group's kept blocks into an LDS list.
struct KeptBlocks {
  int count;  // kept blocks
  int last;   // index of the last kept block, -1 if none
};
// Scans m[j * stride] for j in [first, n) with one wave and returns the kept
// count and last index (uniform over the wave). With `write`, also stores the
// kept indices in ascending order to list[0 .. count-1] (LDS).
__device__ __forceinline__ KeptBlocks collect_blocks(const uint8_t* m, int64_t stride, int first,
                                                     int n, uint16_t* list, int lane, bool write) {
  KeptBlocks r{0, -1};
  for (int j0 = first; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    const bool kept = j < n && m[(int64_t)j * stride] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(kept);
    if (write && kept) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      list[r.count + below] = (uint16_t)j;
    }
    if (bal != 0) r.last = j0 + 63 - __builtin_clzll(bal);
    r.count += __builtin_popcountll(bal);
  }
  return r;
}
// Tiles of TILE rows over the kept blocks: T = 128 / TILE per block, except
// that tiles of the last kept block starting at or past `limit` are dropped.
template <int TILE>
__device__ __forceinline__ int kept_tiles(KeptBlocks kb, int limit) {
  constexpr int T = kSparseBlock / TILE;
  if (kb.count == 0) return 0;
  const int in_last = min(T, (limit - kb.last * kSparseBlock + TILE - 1) / TILE);
  return (kb.count - 1) * T + in_last;
}
// First row of tile t of the kept-block list (uniform).
template <int TILE>
__device__ __forceinline__ int kept_tile_start(const uint16_t* list, int t) {
  constexpr int T = kSparseBlock / TILE;
  const int blk = __builtin_amdgcn_readfirstlane((int)list[t / T]);
  return blk * kSparseBlock + (t % T) * TILE;
}

// Maps a linear work-group id to (block, batch*heads index). All blocks of a
// (b, h) pair land on the same XCD (work-groups are dispatched round-robin
// over the 8 XCDs), so K/V tiles re-read by neighbouring blocks stay in that
// XCD's L2. Pairs are dealt to XCDs by index modulo 8, which spreads the
// heads of each sequence over the XCDs: sequences of different lengths then
// load the XCDs evenly (when the head count is a multiple of 8). Consecutive ids sweep all pairs of one XCD before the next
// block rank, so the rank order (heaviest first for causal masks) holds on
// every XCD.
struct BlockMap {
  int rank;
  int bh;
};
__device__ __forceinline__ BlockMap map_block(int id, int nblk, int BH) {
  BlockMap m;
  if ((BH & 7) == 0) {
    const int xcd = id & 7;
    const int local = id >> 3;
    const int hpx = BH >> 3;
    m.rank = local / hpx;
    m.bh = (local - m.rank * hpx) * 8 + xcd;
  } else {
    m.rank = id / BH;
    m.bh = id - m.rank * BH;
  }
  (void)nblk;
  return m;
}

// Complementary causal block pairs, one pair per work-group: a linear id
// maps to (pair index, batch*heads index). Heads are dealt to XCDs as in
// map_block; within an XCD consecutive ids take consecutive pairs of one
// head, so the work-groups resident at once share that head's K/V.
__device__ __forceinline__ BlockMap map_block_pair(int id, int npairs, int BH) {
  BlockMap m;
  if ((BH & 7) == 0) {
    const int xcd = id & 7;
    const int local = id >> 3;
    const int hl = local / npairs;
    m.rank = local - hl * npairs;
    m.bh = hl * 8 + xcd;
  } else {
    m.rank = id / BH;
    m.bh = id - m.rank * BH;
  }
  return m;
}

// Causal blocks when the whole grid is resident at once: the grid is
// 8 XCDs x `cpx` CUs x `slots` work-groups, `slots` even and within the
// kernel's occupancy. Work-groups are dispatched round-robin over the XCDs
// and, within an XCD, breadth-first over its CUs, so the `slots` work-groups
// of one CU are the ids of one XCD whose local index is equal mod `cpx`.
// Those take slots / 2 complementary rank pairs (r, nblk - 1 - r) of one
// head each, whose causal work sums to nblk + 1 blocks: every CU gets the
// same work, where rank-major order leaves up to 1.4x between CUs. Heads are
// dealt to XCDs as in map_block.
__device__ __forceinline__ BlockMap map_block_pairs(int id, int nblk, int BH, int slots, int cpx) {
  BlockMap m;
  const int xcd = id & 7;
  const int local = id >> 3;
  const int hpx = BH >> 3;
  const int c = local % cpx, j = local / cpx;
  const int half = slots >> 1;
  const int pair = (j % half) * cpx + c;  // < half * cpx = hpx * nblk / 2
  const int r = pair / hpx;
  m.bh = (pair - r * hpx) * 8 + xcd;
  m.rank = j < half ? r : nblk - 1 - r;
  return m;
}

}  // namespace fa
