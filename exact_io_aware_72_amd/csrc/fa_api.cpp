// C ABI of the attention library: argument validation, status codes and
// dispatch to the gfx950 kernels. Every check runs before any HIP call, so a
// rejected call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "../../include/fa.h"
#include "fa_kernels.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_hip_error = "no HIP error recorded";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_hip_error = std::string("HIP error ") + std::to_string((int)e) + ": " + hipGetErrorString(e);
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape, head-dim and dtype rules shared by every tensor entry point.
int check_problem(int B, int H, int N, int d, int dtype) {
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 80 && d != 128) return FA_ERR_HEADDIM;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  // Element count must fit comfortably in 64-bit byte offsets, and grids
  // (at most one work-group per 16 rows, or per 32-row block per head) in
  // 32 bits.
  // B * N fits in 64 bits; comparing it with 2^36 / H decides
  // B * N * H > 2^36 without forming a product that could overflow. Every
  // product below is then bounded by the row count.
  const int64_t bn = (int64_t)B * N;
  if (bn > ((int64_t)1 << 36) / H) return FA_ERR_SHAPE;
  const int64_t rows = bn * H;
  if ((rows + 15) / 16 > (int64_t)INT32_MAX) return FA_ERR_SHAPE;
  if ((int64_t)((N + 31) / 32) * B * H > (int64_t)INT32_MAX) return FA_ERR_SHAPE;
  // The kernels read rows through buffer resources based at each block,
  // tile or window start, with 32-bit offsets from there (a row is at most
  // H * d * 4 <= 2^22 bytes), and per-row statistics with 32-bit offsets
  // (N * 4 < 2^32). A batch item itself may exceed 4 GiB.
  if (N >= (1 << 30)) return FA_ERR_SHAPE;
  if ((int64_t)H * d > (1 << 20)) return FA_ERR_SHAPE;
  return FA_OK;
}

// The keep decision compares 16-bit draws with floor(p * 2^16): a p in
// (0, 2^-16) would drop nothing yet still rescale, so it is rejected.
int check_dropout(float p) {
  if (!(p >= 0.0f && p < 1.0f)) return FA_ERR_DROPOUT;  // also rejects NaN
  if (p > 0.0f && p < 1.0f / 65536.0f) return FA_ERR_DROPOUT;
  return FA_OK;
}

// The kernels take the row max of raw scores and scale it afterwards, which
// needs scale > 0 (the pages' scale is 1/sqrt(d)).
int check_scale(float scale) { return (std::isfinite(scale) && scale > 0.0f) ? FA_OK : FA_ERR_ARG; }

// Keep threshold T = floor(p * 2^16) on the 16-bit draws; p < 1 keeps T <= 65535.
uint32_t drop_threshold16(float p) { return (uint32_t)std::floor((double)p * 65536.0); }

void set_dropout(fa::AttnArgs& a, float p, uint64_t seed) {
  a.dropout = p > 0.0f;
  a.seed = seed;
  a.drop_threshold = drop_threshold16(p);
  a.drop_rescale = (float)(1.0 / (1.0 - (double)p));
}

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr) return FA_ERR_NULL;
  for (const void* p : ps)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  return FA_OK;
}

#define FA_TRY(x)             \
  do {                        \
    const int st_ = (x);      \
    if (st_ != FA_OK) return st_; \
  } while (0)

}  // namespace

FA_EXPORT int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int N, int d, float scale, int causal, float dropout_p,
                         uint64_t seed, void* stream, int dtype) {
  FA_TRY(check_problem(B, H, N, d, dtype));
  FA_TRY(check_dropout(dropout_p));
  FA_TRY(check_scale(scale));
  FA_TRY(check_ptrs({q, k, v, o, lse}));
  fa::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o_out = o;
  a.lse_out = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  set_dropout(a, dropout_p, seed);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(dtype == FA_BF16 ? fa::launch_forward_bf16(a, s)
                                     : fa::launch_forward_f32(a, s));
}

FA_EXPORT size_t fa_backward_workspace_bytes(int B, int H, int N, int d) {
  if (check_problem(B, H, N, d, FA_BF16) != FA_OK) return 0;
  return (size_t)4 * (size_t)B * (size_t)H * (size_t)N;
}

FA_EXPORT int fa_backward_preprocess(const void* o, const void* dout, float* workspace, int B,
                                     int H, int N, int d, void* stream, int dtype) {
  FA_TRY(check_problem(B, H, N, d, dtype));
  FA_TRY(check_ptrs({o, dout, workspace}));
  fa::AttnArgs a;
  a.o = o;
  a.dout = dout;
  a.dsum_out = workspace;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  return hip_status(fa::launch_bwd_preprocess(a, static_cast<hipStream_t>(stream),
                                              dtype == FA_BF16));
}

namespace {
int fill_bwd(fa::AttnArgs& a, const void* q, const void* k, const void* v, const void* dout,
             const float* lse, const float* ws, int B, int H, int N, int d, float scale,
             int causal, float dropout_p, uint64_t seed, int dtype) {
  FA_TRY(check_problem(B, H, N, d, dtype));
  FA_TRY(check_dropout(dropout_p));
  FA_TRY(check_scale(scale));
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dsum = ws;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  set_dropout(a, dropout_p, seed);
  return FA_OK;
}
}  // namespace

FA_EXPORT int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dout,
                               const float* lse, const float* workspace, void* dk, void* dv, int B,
                               int H, int N, int d, float scale, int causal, float dropout_p,
                               uint64_t seed, void* stream, int dtype) {
  fa::AttnArgs a;
  FA_TRY(fill_bwd(a, q, k, v, dout, lse, workspace, B, H, N, d, scale, causal, dropout_p, seed,
                  dtype));
  FA_TRY(check_ptrs({q, k, v, dout, lse, workspace, dk, dv}));
  a.dk = dk;
  a.dv = dv;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(dtype == FA_BF16 ? fa::launch_bwd_dkdv_bf16(a, s)
                                     : fa::launch_bwd_dkdv_f32(a, s));
}

FA_EXPORT int fa_backward_dq(const void* q, const void* k, const void* v, const void* dout,
                             const float* lse, const float* workspace, void* dq, int B, int H,
                             int N, int d, float scale, int causal, float dropout_p, uint64_t seed,
                             void* stream, int dtype) {
  fa::AttnArgs a;
  FA_TRY(fill_bwd(a, q, k, v, dout, lse, workspace, B, H, N, d, scale, causal, dropout_p, seed,
                  dtype));
  FA_TRY(check_ptrs({q, k, v, dout, lse, workspace, dq}));
  a.dq = dq;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(dtype == FA_BF16 ? fa::launch_bwd_dq_bf16(a, s)
                                     : fa::launch_bwd_dq_f32(a, s));
}

FA_EXPORT int fa_backward(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          float* workspace, int B, int H, int N, int d, float scale, int causal,
                          float dropout_p, uint64_t seed, void* stream, int dtype) {
  fa::AttnArgs a;
  FA_TRY(fill_bwd(a, q, k, v, dout, lse, workspace, B, H, N, d, scale, causal, dropout_p, seed,
                  dtype));
  FA_TRY(check_ptrs({q, k, v, o, dout, lse, dq, dk, dv, workspace}));
  a.o = o;
  a.dsum_out = workspace;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == FA_BF16;
  FA_TRY(hip_status(fa::launch_bwd_preprocess(a, s, bf16)));
  FA_TRY(hip_status(bf16 ? fa::launch_bwd_dkdv_bf16(a, s) : fa::launch_bwd_dkdv_f32(a, s)));
  return hip_status(bf16 ? fa::launch_bwd_dq_bf16(a, s) : fa::launch_bwd_dq_f32(a, s));
}

namespace fa {
int record_hip_error(hipError_t e) { return hip_status(e); }

// Every check fa_backward makes except the workspace pointer's, for entry
// points that supply the workspace themselves; no HIP call.
int check_backward_args(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int H, int N, int d, float scale, int causal, float dropout_p,
                        uint64_t seed, int dtype) {
  fa::AttnArgs a;
  FA_TRY(fill_bwd(a, q, k, v, dout, lse, nullptr, B, H, N, d, scale, causal, dropout_p, seed,
                  dtype));
  return check_ptrs({q, k, v, o, dout, lse, dq, dk, dv});
}
}  // namespace fa

// ---------------------------------------------------------------------------
// Packed variable-length batches.
namespace {
int check_varlen(const int* cu, int num_seqs, int total, int max_seqlen, int H, int d,
                 int dtype) {
  // Per-sequence rules are those of a fixed-length batch of num_seqs items of
  // max_seqlen rows (grid sizes, 32-bit offsets within one sequence).
  FA_TRY(check_problem(num_seqs, H, max_seqlen, d, dtype));
  if (cu == nullptr) return FA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(cu) & 3u) != 0) return FA_ERR_ALIGN;
  if (total < 0) return FA_ERR_SHAPE;
  if ((int64_t)total * H > (int64_t)1 << 36) return FA_ERR_SHAPE;
  if (((int64_t)total * H + 15) / 16 > (int64_t)INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}
void set_varlen(fa::AttnArgs& a, const int* cu, int num_seqs, int total, int max_seqlen, int H,
                int d) {
  a.cu_seqlens = cu;
  a.total = total;
  a.B = num_seqs;
  a.N = max_seqlen;
  a.H = H;
  a.d = d;
}
}  // namespace

FA_EXPORT int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* cu_seqlens, int num_seqs, int total, int max_seqlen,
                                int H, int d, float scale, int causal, float dropout_p,
                                uint64_t seed, void* stream, int dtype) {
  FA_TRY(check_varlen(cu_seqlens, num_seqs, total, max_seqlen, H, d, dtype));
  FA_TRY(check_dropout(dropout_p));
  FA_TRY(check_scale(scale));
  if (total == 0) return FA_OK;  // nothing to compute
  FA_TRY(check_ptrs({q, k, v, o, lse}));
  fa::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o_out = o;
  a.lse_out = lse;
  set_varlen(a, cu_seqlens, num_seqs, total, max_seqlen, H, d);
  a.scale = scale;
  a.causal = causal != 0;
  set_dropout(a, dropout_p, seed);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(dtype == FA_BF16 ? fa::launch_forward_bf16(a, s)
                                     : fa::launch_forward_f32(a, s));
}

FA_EXPORT size_t fa_backward_varlen_workspace_bytes(int total, int H, int d) {
  if (total < 0 || H < 1 || (d != 64 && d != 80 && d != 128)) return 0;
  if ((int64_t)total * H > (int64_t)1 << 36) return 0;
  return (size_t)4 * (size_t)H * (size_t)total;
}

FA_EXPORT int fa_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                 float* workspace, const int* cu_seqlens, int num_seqs, int total,
                                 int max_seqlen, int H, int d, float scale, int causal,
                                 float dropout_p, uint64_t seed, void* stream, int dtype) {
  FA_TRY(check_varlen(cu_seqlens, num_seqs, total, max_seqlen, H, d, dtype));
  FA_TRY(check_dropout(dropout_p));
  FA_TRY(check_scale(scale));
  if (total == 0) return FA_OK;  // nothing to compute
  FA_TRY(check_ptrs({q, k, v, o, dout, lse, dq, dk, dv, workspace}));
  fa::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dsum = workspace;
  a.dsum_out = workspace;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  set_varlen(a, cu_seqlens, num_seqs, total, max_seqlen, H, d);
  a.scale = scale;
  a.causal = causal != 0;
  set_dropout(a, dropout_p, seed);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == FA_BF16;
  FA_TRY(hip_status(fa::launch_bwd_preprocess(a, s, bf16)));
  FA_TRY(hip_status(bf16 ? fa::launch_bwd_dkdv_bf16(a, s) : fa::launch_bwd_dkdv_f32(a, s)));
  return hip_status(bf16 ? fa::launch_bwd_dq_bf16(a, s) : fa::launch_bwd_dq_f32(a, s));
}

// ---------------------------------------------------------------------------
// Block-sparse masks.
namespace {
int check_block_mask(const uint8_t* m, int64_t sb, int64_t sh, int N) {
  if (m == nullptr) return FA_ERR_NULL;
  if (sb < 0 || sh < 0) return FA_ERR_ARG;
  if (N > fa::kSparseBlock * fa::kSparseMaxBlocks) return FA_ERR_SHAPE;
  return FA_OK;
}
}  // namespace

FA_EXPORT int fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o,
                                     float* lse, const uint8_t* block_mask, int64_t mask_stride_b,
                                     int64_t mask_stride_h, int B, int H, int N, int d,
                                     float scale, int causal, float dropout_p, uint64_t seed,
                                     void* stream, int dtype) {
  FA_TRY(check_problem(B, H, N, d, dtype));
  FA_TRY(check_dropout(dropout_p));
  FA_TRY(check_scale(scale));
  FA_TRY(check_block_mask(block_mask, mask_stride_b, mask_stride_h, N));
  FA_TRY(check_ptrs({q, k, v, o, lse}));
  fa::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o_out = o;
  a.lse_out = lse;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.block_mask = block_mask;
  a.mask_stride_b = mask_stride_b;
  a.mask_stride_h = mask_stride_h;
  a.scale = scale;
  a.causal = causal != 0;
  set_dropout(a, dropout_p, seed);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(dtype == FA_BF16 ? fa::launch_forward_bf16(a, s)
                                     : fa::launch_forward_f32(a, s));
}

FA_EXPORT int fa_backward_blocksparse(const void* q, const void* k, const void* v, const void* o,
                                      const void* dout, const float* lse, void* dq, void* dk,
                                      void* dv, float* workspace, const uint8_t* block_mask,
                                      int64_t mask_stride_b, int64_t mask_stride_h, int B, int H,
                                      int N, int d, float scale, int causal, float dropout_p,
                                      uint64_t seed, void* stream, int dtype) {
  fa::AttnArgs a;
  FA_TRY(fill_bwd(a, q, k, v, dout, lse, workspace, B, H, N, d, scale, causal, dropout_p, seed,
                  dtype));
  FA_TRY(check_block_mask(block_mask, mask_stride_b, mask_stride_h, N));
  FA_TRY(check_ptrs({q, k, v, o, dout, lse, dq, dk, dv, workspace}));
  a.o = o;
  a.dsum_out = workspace;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.block_mask = block_mask;
  a.mask_stride_b = mask_stride_b;
  a.mask_stride_h = mask_stride_h;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == FA_BF16;
  FA_TRY(hip_status(fa::launch_bwd_preprocess(a, s, bf16)));
  FA_TRY(hip_status(bf16 ? fa::launch_bwd_dkdv_bf16(a, s) : fa::launch_bwd_dkdv_f32(a, s)));
  return hip_status(bf16 ? fa::launch_bwd_dq_bf16(a, s) : fa::launch_bwd_dq_f32(a, s));
}

// ---------------------------------------------------------------------------
// Split-KV forward.
namespace {
constexpr int kMaxSplits = 128;

int check_splitkv(int B, int H, int Nq, int Nk, int d, int causal, int num_splits, int dtype) {
  FA_TRY(check_problem(B, H, Nq, d, dtype));
  FA_TRY(check_problem(B, H, Nk, d, dtype));
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (causal && Nk < Nq) return FA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_ARG;
  const int64_t wgs = (int64_t)((Nq + 127) / 128) * B * H * (num_splits ? num_splits : kMaxSplits);
  if (wgs > (int64_t)INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

int pick_splits(int B, int H, int Nq, int Nk) {
  // Enough work-groups for two per compute unit (256 CUs), and at least four
  // 64-key tiles per part.
  const int64_t wgs = (int64_t)((Nq + 127) / 128) * B * H;
  if (wgs >= 512) return 1;
  const int tiles = (Nk + 63) / 64;
  int s = (int)((512 + wgs - 1) / wgs);
  s = std::min(s, std::max(1, tiles / 4));
  return std::max(1, std::min(s, kMaxSplits));
}
}  // namespace

FA_EXPORT int fa_splitkv_num_splits(int B, int H, int Nq, int Nk, int d) {
  if (check_splitkv(B, H, Nq, Nk, d, 0, 0, FA_BF16) != FA_OK) return 0;
  return pick_splits(B, H, Nq, Nk);
}

FA_EXPORT size_t fa_forward_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits) {
  if (num_splits < 1 || num_splits > kMaxSplits) return 0;
  if (check_problem(B, H, Nq, d, FA_BF16) != FA_OK) return 0;
  return (size_t)4 * (size_t)num_splits * (size_t)B * (size_t)H * (size_t)Nq * (size_t)(d + 1);
}

FA_EXPORT int fa_forward_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                                 float* workspace, int B, int H, int Nq, int Nk, int d,
                                 float scale, int causal, int num_splits, void* stream,
                                 int dtype) {
  FA_TRY(check_splitkv(B, H, Nq, Nk, d, causal, num_splits, dtype));
  FA_TRY(check_scale(scale));
  FA_TRY(check_ptrs({q, k, v, o, lse, workspace}));
  fa::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o_out = o;
  a.lse_out = lse;
  a.B = B;
  a.H = H;
  a.N = Nq;
  a.Nk = Nk;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.num_splits = num_splits ? num_splits : pick_splits(B, H, Nq, Nk);
  a.split_o = workspace;
  a.split_lse = workspace + (size_t)a.num_splits * B * H * Nq * d;
  return hip_status(fa::launch_forward_splitkv_bf16(a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// FP8 scores.
FA_EXPORT int fa_quantize_fp8(const void* x, uint8_t* xq, float* scales, int B, int N, int H,
                              int d, int block_rows, void* stream) {
  FA_TRY(check_problem(B, H, N, d, FA_BF16));
  if (block_rows != 64 && block_rows != 128) return FA_ERR_ARG;
  FA_TRY(check_ptrs({x, xq, scales}));
  return hip_status(fa::launch_quantize_fp8(x, xq, scales, B, N, H, d, block_rows,
                                            static_cast<hipStream_t>(stream)));
}

FA_EXPORT int fa_forward_fp8(const uint8_t* q8, const uint8_t* k8, const void* v, void* o,
                             float* lse, const float* q_scale, const float* k_scale, int B, int H,
                             int N, int d, float scale, int causal, void* stream) {
  FA_TRY(check_problem(B, H, N, d, FA_BF16));
  FA_TRY(check_scale(scale));
  FA_TRY(check_ptrs({q8, k8, v, o, lse}));
  if (q_scale == nullptr || k_scale == nullptr) return FA_ERR_NULL;
  if (((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale)) & 3u) != 0)
    return FA_ERR_ALIGN;
  fa::AttnArgs a;
  a.q = q8;
  a.k = k8;
  a.v = v;
  a.o_out = o;
  a.lse_out = lse;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  return hip_status(fa::launch_forward_fp8(a, static_cast<hipStream_t>(stream)));
}

FA_EXPORT int fa_dropout_mask(uint64_t seed, int b, int h, int H, float dropout_p, int row0,
                              int col0, int rows, int cols, uint8_t* out, void* stream) {
  FA_TRY(check_dropout(dropout_p));
  if (out == nullptr) return FA_ERR_NULL;
  if (H < 1 || b < 0 || h < 0 || h >= H || row0 < 0 || col0 < 0 || rows < 1 || cols < 1)
    return FA_ERR_ARG;
  if ((int64_t)rows * cols >= ((int64_t)1 << 31)) return FA_ERR_ARG;
  if ((int64_t)row0 + rows > INT32_MAX || (int64_t)col0 + cols > INT32_MAX) return FA_ERR_ARG;
  const uint32_t thr = drop_threshold16(dropout_p);
  return hip_status(fa::launch_dropout_mask(seed, b, h, H, thr, row0, col0, rows, cols, out,
                                            static_cast<hipStream_t>(stream)));
}

FA_EXPORT const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: B, H, N must be >= 1 and sizes must fit";
    case FA_ERR_HEADDIM: return "unsupported head dimension (supported: 64, 80, 128)";
    case FA_ERR_DTYPE: return "unsupported dtype (FA_F32 or FA_BF16)";
    case FA_ERR_DROPOUT: return "dropout_p must lie in [0, 1)";
    case FA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FA_ERR_UNSUPPORTED: return "request not supported by this build";
    case FA_ERR_HIP: return g_hip_error.c_str();
    case FA_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

FA_EXPORT const char* fa_version(void) { return "fa-mi355x 0.1.0 gfx950"; }
