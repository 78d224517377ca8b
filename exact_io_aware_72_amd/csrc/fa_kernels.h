// Internal launch interface between the C ABI (fa_api.cpp) and the kernels.
// Arguments are validated by the caller before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Block-sparse masks: one byte per (128-query block, 128-key block) of a
// (b, h) pair, row-major over an nb x nb grid (nb = ceil(N / 128)); nonzero
// means the block is computed, zero that its scores are -inf.
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxBlocks = 1024;  // so N <= 131072 with a block mask

struct AttnArgs {
  // inputs
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const void* o = nullptr;     // forward output, read by the backward
  const void* dout = nullptr;  // upstream gradient dO
  const float* lse = nullptr;  // [B][H][N] natural-log logsumexp
  const float* dsum = nullptr; // [B][H][N] D = rowsum(dO * O)
  // outputs
  void* o_out = nullptr;
  float* lse_out = nullptr;
  float* dsum_out = nullptr;
  void* dq = nullptr;
  void* dk = nullptr;
  void* dv = nullptr;
  // problem. Fixed-length batches: B items of N rows each, statistics
  // [B][H][N]. Packed variable-length batches (cu_seqlens != nullptr): B
  // sequences, sequence s holding rows cu_seqlens[s]..cu_seqlens[s+1]-1 of
  // [total][H][d] tensors, N = the longest sequence, statistics [H][total].
  int B = 0, H = 0, N = 0, d = 0;
  const int* cu_seqlens = nullptr;
  int total = 0;
  // Block-sparse mask (fixed-length batches only): for (b, h), the nb x nb
  // bytes at block_mask + b * mask_stride_b + h * mask_stride_h, nb =
  // ceil(N / 128); nonzero = the 128 x 128 block is computed. nullptr: dense.
  const uint8_t* block_mask = nullptr;
  int64_t mask_stride_b = 0, mask_stride_h = 0;
  // Split-KV forward: N query rows against Nk key rows per batch item, the
  // key range cut into num_splits parts whose partial results (O_s fp32
  // [num_splits][B][H][N][d], LSE_s [num_splits][B][H][N]) are combined.
  int Nk = 0, num_splits = 1;
  float* split_o = nullptr;
  float* split_lse = nullptr;
  // FP8 scores: q and k hold OCP E4M3 bytes; scales per 128 query rows and
  // per 64 key rows ([B][H][blocks]).
  const float* q_scale = nullptr;
  const float* k_scale = nullptr;
  float scale = 0.f;
  bool causal = false;
  bool dropout = false;
  uint32_t drop_threshold = 0;  // keep iff the 16-bit draw >= threshold
  float drop_rescale = 1.f;     // 1 / (1 - p) in fp32
  uint64_t seed = 0;
};

hipError_t launch_forward_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_forward_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_forward_splitkv_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_forward_fp8(const AttnArgs& a, hipStream_t s);
hipError_t launch_quantize_fp8(const void* x, uint8_t* xq, float* scales, int B, int N, int H,
                               int d, int block_rows, hipStream_t s);
hipError_t launch_bwd_preprocess(const AttnArgs& a, hipStream_t s, bool bf16);
hipError_t launch_bwd_dkdv_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_f32(const AttnArgs& a, hipStream_t s);
// Status code for a failed HIP call, recording its text for fa_status_string
// (fa_api.cpp).
int record_hip_error(hipError_t e);

// Argument checks of fa_backward without the workspace (fa_api.cpp).
int check_backward_args(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int H, int N, int d, float scale, int causal, float dropout_p,
                        uint64_t seed, int dtype);

hipError_t launch_dropout_mask(uint64_t seed, int b, int h, int H, uint32_t threshold, int row0,
                               int col0, int rows, int cols, uint8_t* out, hipStream_t s);

}  // namespace fa
