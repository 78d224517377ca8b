/*
 * fa.h — C ABI of the exact IO-aware attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(Q K^T * scale) V,     scale = 1/sqrt(d) normally,
 * tile by tile, with an online softmax, never writing the N x N score or
 * probability matrices to device memory, and saving the per-row logsumexp so
 * that the backward pass recomputes the probabilities instead of storing them.
 * ("FlashAttention for Efficient Training", sections 2.1 "Forward Pass with
 * Recomputation", 3.1 "Workflow Breakdown" and 3.2 "Precision Handling and
 * Numerical Stability"; "How FlashAttention Optimizes GPU Memory for Fast AI
 * Training", sections "1. Tiling", "2. Online Softmax", "3. Kernel Fusion" and
 * "4. Recomputation in the Backward Pass".)
 *
 * Conventions shared by every entry point:
 *   - Tensors q, k, v, o, dout, dq, dk, dv are contiguous [B][N][H][d] arrays
 *     (the (batch, seq_len, num_heads, head_dim) layout of the PyTorch usage
 *     example, section 4.2 of the first page) of the element type `dtype`.
 *     lse and the backward workspace are contiguous [B][H][N] float arrays.
 *   - Every pointer is a DEVICE pointer owned by the caller, aligned to 16
 *     bytes. The library never allocates, frees, or synchronises, and keeps no
 *     mutable global state: all calls are safe from several host threads.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *     is enqueued on it and the call returns without waiting; FA_OK means
 *     "enqueued". Device faults surface at the caller's next synchronisation.
 *   - Arguments are validated before any HIP call; on any error nothing is
 *     launched and nothing is written. No C++ exception crosses this ABI.
 *   - Supported: d in {64, 80, 128}; 1 <= N < 2^30 (tails handled by
 *     masks), H*d <= 2^20, B*N*H <= 2^36; a batch item may exceed 4 GiB;
 *     dtype FA_BF16 (bf16 storage, fp32 accumulation, bf16 matrix cores) or
 *     FA_F32 (fp32 throughout). Causal masking keeps key j for query i iff
 *     j <= i (queries and keys share positions 0..N-1).
 *   - Dropout: dropout_p = 0 or 2^-16 <= dropout_p < 1 (the draws have 16
 *     bits, so a smaller nonzero p could drop nothing; it is rejected with
 *     FA_ERR_DROPOUT). Probabilities are dropped after the
 *     softmax normalisation with the keep mask of a counter hash of
 *     (seed, b, h, row, col) and kept ones are scaled by 1/(1 - dropout_p);
 *     the logsumexp is that of the undropped probabilities. `seed` is used
 *     only when dropout_p > 0. The backward pass must receive the same
 *     (dropout_p, seed) as the forward pass. The hash is specified in the
 *     comment of fa_dropout_mask below.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  FA_ERR_SHAPE = -2,       /* B, H or N < 1, N >= 2^30, H*d > 2^20, or a size
                              that overflows                                    */
  FA_ERR_HEADDIM = -3,     /* d not in {64, 80, 128}                             */
  FA_ERR_DTYPE = -4,       /* dtype not FA_F32 / FA_BF16                         */
  FA_ERR_DROPOUT = -5,     /* dropout_p NaN, outside [0, 1) or in (0, 2^-16)     */
  FA_ERR_ALIGN = -6,       /* a pointer is not 16-byte aligned                   */
  FA_ERR_UNSUPPORTED = -7, /* valid request this build does not implement       */
  FA_ERR_HIP = -8,         /* a HIP runtime call failed; see fa_status_string    */
  FA_ERR_ARG = -9          /* other invalid argument (scale not finite and > 0,
                              bad mask window)                                  */
} fa_status;

/*
 * Forward pass (steps: stage Q tile, stream K/V tiles, S = scale*Q K^T,
 * causal tile skip and mask, online softmax, dropout, O += P V, epilogue).
 *   q, k, v  [B][N][H][d] inputs (dtype)
 *   o        [B][N][H][d] output (dtype): O = (P o Z / (1-p)) V
 *   lse      [B][H][N] float output: natural-log logsumexp of the scaled,
 *            masked scores of each query row (undropped)
 *   scale    multiplier of Q K^T, finite and > 0; normally 1/sqrt(d)
 *   causal   0 = full attention, nonzero = causal mask
 * Definition: "FlashAttention for Efficient Training", section 1.1
 * (Attention(Q,K,V)), section 3.1 (S_ij = Q_i K_j^T / sqrt(d_k), online
 * softmax) and section 3.2 (log_softmax = x - logsumexp(x)).
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               float dropout_p, uint64_t seed, void* stream, int dtype);

/* Bytes of the float workspace fa_backward needs: 4*B*H*N (the row terms
 * D_i = sum_c dO_ic O_ic). Returns 0 if the sizes are invalid. */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass. Runs fa_backward_preprocess, fa_backward_dkdv and
 * fa_backward_dq on `stream`, in that order.
 *   q, k, v, o, dout  [B][N][H][d] (dtype); o and lse from fa_forward with
 *                     the same arguments
 *   lse               [B][H][N] float from fa_forward
 *   dq, dk, dv        [B][N][H][d] outputs (dtype), fully overwritten
 *   workspace         float array of fa_backward_workspace_bytes(...) bytes;
 *                     receives D = rowsum(dout o o) as [B][H][N]
 * Gradients of L = sum(dout o O): dV = P~^T dO ("FlashAttention for Efficient
 * Training", section 3.2 "Integration with Autograd Engines"), dQ and dK by
 * the chain rule of the same section: dP = (dO V^T) o Z/(1-p),
 * dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q. No atomics: results
 * are bitwise reproducible run to run.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                float* workspace, int B, int H, int N, int d, float scale,
                int causal, float dropout_p, uint64_t seed, void* stream, int dtype);

/*
 * Backward pass without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, results and error codes
 * as fa_backward, minus `workspace`: D goes to a fixed device array inside
 * the library, FA_NOALLOC_MAX_ROWS floats (16 MiB) per GPU, held until the
 * process ends. Requires B*H*N <= FA_NOALLOC_MAX_ROWS (else FA_ERR_SHAPE,
 * nothing launched). The library allocates nothing. All calls on one GPU
 * share that GPU's array, which keeps the last call's contents: calls that
 * overlap on one GPU (different streams, or threads without ordering) race
 * and must be serialised by the caller. The first call on a device looks up
 * the array's device address (hipGetSymbolAddress); a failure there returns
 * FA_ERR_HIP with nothing launched.
 */
#define FA_NOALLOC_MAX_ROWS (1 << 22)
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, float scale, int causal,
                        float dropout_p, uint64_t seed, void* stream, int dtype);

/* Step B1 alone: workspace[b][h][i] = sum_c dout[b][i][h][c] * o[b][i][h][c]
 * in fp32. Same argument rules as fa_backward. */
int fa_backward_preprocess(const void* o, const void* dout, float* workspace,
                           int B, int H, int N, int d, void* stream, int dtype);

/* Step B2 alone: dk and dv, one work-group per key block, looping over the
 * query blocks that see it. Needs the workspace written by step B1. */
int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dout,
                     const float* lse, const float* workspace, void* dk, void* dv,
                     int B, int H, int N, int d, float scale, int causal,
                     float dropout_p, uint64_t seed, void* stream, int dtype);

/* Step B3 alone: dq, one work-group per query block, looping over the key
 * blocks it sees. Needs the workspace written by step B1. */
int fa_backward_dq(const void* q, const void* k, const void* v, const void* dout,
                   const float* lse, const float* workspace, void* dq,
                   int B, int H, int N, int d, float scale, int causal,
                   float dropout_p, uint64_t seed, void* stream, int dtype);

/*
 * Packed variable-length batches ("FlashAttention for Efficient Training",
 * section 5.2 "Handling Variable Sequence Lengths": a query attends only to
 * the keys of its own sequence, scores of other positions being -inf, and
 * no work is spent on padding). Sequence s holds rows
 * cu_seqlens[s] .. cu_seqlens[s+1]-1 of the packed tensors; positions,
 * causal masking and the dropout hash (with b = s) count from the sequence
 * start.
 *   q, k, v, o, dout, dq, dk, dv  [total][H][d] (dtype)
 *   lse, workspace                [H][total] float
 *   cu_seqlens  DEVICE int32 array of num_seqs + 1 non-decreasing offsets
 *               in [0, total] (normally cu_seqlens[0] = 0); every sequence
 *               at most max_seqlen rows. Offsets are clamped to
 *               [0, total] and lengths to max_seqlen on the device, so a
 *               malformed array cannot address memory outside the tensors
 *               (the results are then unspecified); rows outside every
 *               sequence are not written.
 *   num_seqs >= 1, max_seqlen >= 1, total >= 0 (total == 0: returns FA_OK
 *   after the argument checks above, touching nothing); other arguments and errors
 *   as for fa_forward / fa_backward (the shape rules apply to a batch of
 *   num_seqs items of max_seqlen rows). cu_seqlens needs 4-byte alignment.
 */
int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int* cu_seqlens, int num_seqs, int total, int max_seqlen,
                      int H, int d, float scale, int causal, float dropout_p, uint64_t seed,
                      void* stream, int dtype);

/* Bytes of the workspace fa_backward_varlen needs: 4*H*total (D as [H][total]).
 * Returns 0 if the sizes are invalid. */
size_t fa_backward_varlen_workspace_bytes(int total, int H, int d);

int fa_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       float* workspace, const int* cu_seqlens, int num_seqs, int total,
                       int max_seqlen, int H, int d, float scale, int causal, float dropout_p,
                       uint64_t seed, void* stream, int dtype);

/*
 * Block-sparse attention ("FlashAttention for Efficient Training", section 3.2,
 * "Block-Sparse Attention Support": only the nonzero blocks of the attention
 * matrix are computed). Fixed-length [B][N][H][d] tensors as for fa_forward /
 * fa_backward, plus a mask over 128 x 128 blocks of the score matrix:
 *   block_mask  DEVICE bytes; for head (b, h) the nb x nb row-major grid at
 *               block_mask + b * mask_stride_b + h * mask_stride_h, with
 *               nb = ceil(N / 128); entry [i][j] nonzero: the scores of query
 *               block i against key block j are computed; zero: they are -inf
 *               (no work is done for them). Strides are in bytes, >= 0 (0
 *               shares one grid across batch items or heads); no alignment.
 *   N <= 131072.
 * With causal != 0 the causal mask applies as well. A query row whose
 * visible keys are all masked gets O = 0 and LSE = -inf, and zero gradients.
 * The backward takes the same mask as the forward that produced o and lse;
 * its workspace is fa_backward_workspace_bytes(B, H, N, d). Other arguments
 * and errors as for fa_forward / fa_backward; additionally FA_ERR_NULL for a
 * null mask, FA_ERR_ARG for a negative stride, FA_ERR_SHAPE for N > 131072.
 */
int fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                           const uint8_t* block_mask, int64_t mask_stride_b,
                           int64_t mask_stride_h, int B, int H, int N, int d, float scale,
                           int causal, float dropout_p, uint64_t seed, void* stream, int dtype);

int fa_backward_blocksparse(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            float* workspace, const uint8_t* block_mask, int64_t mask_stride_b,
                            int64_t mask_stride_h, int B, int H, int N, int d, float scale,
                            int causal, float dropout_p, uint64_t seed, void* stream, int dtype);

/*
 * Split-KV forward for shapes with little parallelism (few batch items and
 * heads, short query blocks against long key sequences, e.g. decoding):
 * per-tile softmax results are merged by a reduction ("FlashAttention for
 * Efficient Training", section 2.3, "Practical Implementation"; its section
 * 6.1, "Limited Parallelism for Small Batch Sizes", names small batches and
 * few heads as the case of idle compute units). The key range is cut into
 * num_splits parts computed by separate work-groups; each part's normalised
 * output O_s and logsumexp LSE_s are merged exactly:
 * LSE = ln sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s.
 *   q, o      [B][Nq][H][d] bf16;  k, v  [B][Nk][H][d] bf16;  lse [B][H][Nq] fp32
 *   causal    key j is visible to query i iff j <= i + (Nk - Nq): the queries
 *             are the last Nq positions of the key sequence (needs Nk >= Nq)
 *   num_splits  1..128, or 0 to let fa_splitkv_num_splits choose
 *   workspace fa_forward_splitkv_workspace_bytes(B, H, Nq, d, num_splits)
 *             bytes of device memory (fp32 partial results), 16-byte aligned;
 *             with num_splits = 0 size it for 128 parts or for the number
 *             fa_splitkv_num_splits returns
 * No dropout (an inference path). dtype must be FA_BF16 (FA_ERR_UNSUPPORTED
 * otherwise). Other arguments and errors as for fa_forward; FA_ERR_ARG for
 * num_splits outside 0..128, FA_ERR_SHAPE for causal with Nk < Nq.
 */
int fa_splitkv_num_splits(int B, int H, int Nq, int Nk, int d);
size_t fa_forward_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits);
int fa_forward_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                       float* workspace, int B, int H, int Nq, int Nk, int d, float scale,
                       int causal, int num_splits, void* stream, int dtype);

/*
 * FP8 scores ("FlashAttention for Efficient Training", section 6.2,
 * "Quantization and Mixed-Precision Approaches": Q K^T ~ S_Q * Q8 * K8^T * S_K
 * with quantised queries and keys and their scaling factors). Q K^T runs on
 * the FP8 matrix cores; the softmax, P V (bf16) and outputs are as in
 * fa_forward. An inference path: forward only, no dropout; d = 64, 80, 128.
 *
 * fa_quantize_fp8: x bf16 [B][N][H][d] -> xq OCP FP8 E4M3 bytes [B][N][H][d]
 *   and scales fp32 [B][H][ceil(N / block_rows)], block_rows 128 (queries) or
 *   64 (keys). Per (b, h, block): amax = max |x|, scale = amax / 448 (1 for
 *   an all-zero block), xq = E4M3(x * (448 / amax)) rounded to nearest even,
 *   all in fp32.
 * fa_forward_fp8: q8, k8 from fa_quantize_fp8 (block_rows 128 and 64), v bf16
 *   [B][N][H][d]; o bf16 and lse fp32 as fa_forward. Scores are
 *   scale * q_scale[b][h][i / 128] * k_scale[b][h][j / 64] * (q8_i . k8_j).
 * Errors as for fa_forward; FA_ERR_ARG for another block_rows. Scale arrays
 * need 4-byte alignment. xq rows of d bytes must be 16-byte aligned like the
 * other tensors (d is a multiple of 16).
 */
int fa_quantize_fp8(const void* x, uint8_t* xq, float* scales, int B, int N, int H, int d,
                    int block_rows, void* stream);
int fa_forward_fp8(const uint8_t* q8, const uint8_t* k8, const void* v, void* o, float* lse,
                   const float* q_scale, const float* k_scale, int B, int H, int N, int d,
                   float scale, int causal, void* stream);

/*
 * Writes the dropout keep mask of head (b, h) for rows row0..row0+rows-1 and
 * columns col0..col0+cols-1 to out[rows][cols] (device, 1 = keep), with the
 * same device function the kernels use. The pages fuse dropout into the
 * kernel without naming a generator; this library's generator is:
 *   G = 0x9E3779B97F4A7C15;  mix64 = SplitMix64 output function;
 *   fmix32 = MurmurHash3 32-bit finalizer;
 *   K_bh = mix64(seed + G*(1 + b*H + h));
 *   A_i = lo32(mix64(K_bh + G*(2i+1)));  B_c = lo32(mix64(K_bh + G*(2c+2)));
 *   w = fmix32(A_i ^ B_c), whose low 16 bits are the draw u_ij of column j = 2c
 *   and whose high 16 bits that of j = 2c + 1   (all mod 2^64 / 2^32);
 *   keep(i, j) = u_ij >= floor(dropout_p * 2^16), a keep probability within
 *   2^-16 of 1 - dropout_p.
 * Requires 0 <= b, 0 <= h < H, row0, col0 >= 0, rows, cols >= 1,
 * rows * cols < 2^31, out non-NULL (any alignment).
 */
int fa_dropout_mask(uint64_t seed, int b, int h, int H, float dropout_p,
                    int row0, int col0, int rows, int cols, uint8_t* out,
                    void* stream);

/* Human-readable text for a status code. For FA_ERR_HIP it carries the HIP
 * error of the last failing call on this host thread. Never NULL. */
const char* fa_status_string(int status);

/* Library version string, e.g. "fa-mi355x 0.1.0 gfx950". */
const char* fa_version(void);


#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
