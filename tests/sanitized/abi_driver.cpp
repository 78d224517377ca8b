// Drives every attention entry point of fa.h through fa_api.cpp with the
// launchers stubbed out: valid arguments must return FA_OK and launch,
// invalid ones their documented status and launch nothing. Built with
// -fsanitize=address,undefined on the host, so any out-of-bounds access,
// overflow or undefined behaviour in the validation code aborts the run.
// Pointers are aligned stand-in addresses that nothing dereferences.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "fa.h"

namespace fa {
extern int g_launches;
}

static int failures = 0;

#define EXPECT(call, want, launches)                                                        \
  do {                                                                                      \
    const int before_ = fa::g_launches;                                                     \
    const int got_ = (call);                                                                \
    const int launched_ = fa::g_launches - before_;                                         \
    if (got_ != (want) || (launches >= 0 && launched_ != launches)) {                       \
      std::printf("FAIL line %d: %s -> %d (want %d), %d launches\n", __LINE__, #call, got_, \
                  (int)(want), launched_);                                                  \
      ++failures;                                                                           \
    }                                                                                       \
  } while (0)

int main() {
  void* P = reinterpret_cast<void*>(0x10000);   // 16-byte aligned stand-in
  void* M = reinterpret_cast<void*>(0x10004);   // misaligned
  float* F = static_cast<float*>(P);
  const int* CU = static_cast<const int*>(P);
  const uint8_t* U8 = static_cast<const uint8_t*>(P);
  uint8_t* W8 = static_cast<uint8_t*>(P);
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();

  // forward
  EXPECT(fa_forward(P, P, P, P, F, 2, 4, 300, 128, 0.088f, 1, 0.1f, 7, nullptr, FA_BF16), FA_OK, 1);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 256, 64, 0.125f, 0, 0.f, 0, nullptr, FA_F32), FA_OK, 1);
  EXPECT(fa_forward(nullptr, P, P, P, F, 1, 1, 16, 64, 0.125f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_NULL, 0);
  EXPECT(fa_forward(P, P, P, P, nullptr, 1, 1, 16, 64, 0.125f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_NULL, 0);
  EXPECT(fa_forward(P, M, P, P, F, 1, 1, 16, 64, 0.125f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_ALIGN, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 16, 96, 0.125f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_HEADDIM, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 16, 64, 0.125f, 0, 0.f, 0, nullptr, 7), FA_ERR_DTYPE, 0);
  EXPECT(fa_forward(P, P, P, P, F, 0, 1, 16, 64, 0.125f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_SHAPE, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, -5, 64, 0.125f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_SHAPE, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 64, 2000000000, 128, 0.1f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_SHAPE, 0);
  EXPECT(fa_forward(P, P, P, P, F, 2147483647, 2147483647, 2147483647, 128, 0.1f, 0, 0.f, 0, nullptr, FA_BF16),
         FA_ERR_SHAPE, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 16, 64, 0.125f, 0, 1.f, 0, nullptr, FA_BF16), FA_ERR_DROPOUT, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 16, 64, 0.125f, 0, nan, 0, nullptr, FA_BF16), FA_ERR_DROPOUT, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 16, 64, 0.125f, 0, -0.5f, 0, nullptr, FA_BF16), FA_ERR_DROPOUT, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 16, 64, 0.f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_ARG, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 16, 64, inf, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_ARG, 0);
  EXPECT(fa_forward(P, P, P, P, F, 1, 1, 16, 64, nan, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_ARG, 0);

  // backward: fused call (three launches) and its steps
  EXPECT(fa_backward(P, P, P, P, P, F, P, P, P, F, 2, 4, 300, 80, 0.11f, 1, 0.1f, 3, nullptr, FA_BF16), FA_OK, 3);
  EXPECT(fa_backward(P, P, P, P, P, F, P, P, P, F, 1, 2, 100, 64, 0.125f, 0, 0.f, 0, nullptr, FA_F32), FA_OK, 3);
  EXPECT(fa_backward(P, P, P, P, P, F, P, P, P, nullptr, 1, 1, 16, 64, 0.125f, 0, 0.f, 0, nullptr, FA_BF16),
         FA_ERR_NULL, 0);
  EXPECT(fa_backward(P, P, P, P, M, F, P, P, P, F, 1, 1, 16, 64, 0.125f, 0, 0.f, 0, nullptr, FA_BF16), FA_ERR_ALIGN, 0);
  EXPECT(fa_backward(P, P, P, P, P, F, P, P, P, F, 1, 1, 16, 64, 0.125f, 0, 2.f, 0, nullptr, FA_BF16), FA_ERR_DROPOUT, 0);
  EXPECT(fa_backward_preprocess(P, P, F, 1, 2, 100, 128, nullptr, FA_BF16), FA_OK, 1);
  EXPECT(fa_backward_preprocess(P, nullptr, F, 1, 2, 100, 128, nullptr, FA_BF16), FA_ERR_NULL, 0);
  EXPECT(fa_backward_dkdv(P, P, P, P, F, F, P, P, 1, 2, 100, 128, 0.1f, 1, 0.f, 0, nullptr, FA_BF16), FA_OK, 1);
  EXPECT(fa_backward_dkdv(P, P, P, P, F, F, P, P, 1, 2, 100, 72, 0.1f, 1, 0.f, 0, nullptr, FA_BF16), FA_ERR_HEADDIM, 0);
  EXPECT(fa_backward_dq(P, P, P, P, F, F, P, 1, 2, 100, 128, 0.1f, 1, 0.f, 0, nullptr, FA_BF16), FA_OK, 1);
  EXPECT(fa_backward_dq(P, P, P, P, F, F, P, 1, 2, 100, 128, -1.f, 1, 0.f, 0, nullptr, FA_BF16), FA_ERR_ARG, 0);
  if (fa_backward_workspace_bytes(2, 16, 8192, 128) != (size_t)4 * 2 * 16 * 8192) {
    std::printf("FAIL workspace bytes\n");
    ++failures;
  }
  (void)fa_backward_workspace_bytes(2147483647, 2147483647, 2147483647, 128);  // no UB
  (void)fa_backward_workspace_bytes(-1, 1, 1, 64);

  // packed variable-length batches
  EXPECT(fa_forward_varlen(P, P, P, P, F, CU, 3, 900, 512, 4, 128, 0.1f, 1, 0.f, 0, nullptr, FA_BF16), FA_OK, 1);
  EXPECT(fa_forward_varlen(P, P, P, P, F, nullptr, 3, 900, 512, 4, 128, 0.1f, 1, 0.f, 0, nullptr, FA_BF16),
         FA_ERR_NULL, 0);
  EXPECT(fa_forward_varlen(P, P, P, P, F, reinterpret_cast<const int*>(0x10002), 3, 900, 512, 4, 128, 0.1f, 1,
                           0.f, 0, nullptr, FA_BF16), FA_ERR_ALIGN, 0);
  EXPECT(fa_forward_varlen(P, P, P, P, F, CU, -1, 900, 512, 4, 128, 0.1f, 1, 0.f, 0, nullptr, FA_BF16), FA_ERR_SHAPE, 0);
  EXPECT(fa_forward_varlen(P, P, P, P, F, CU, 3, -1, 512, 4, 128, 0.1f, 1, 0.f, 0, nullptr, FA_BF16), FA_ERR_SHAPE, 0);
  EXPECT(fa_backward_varlen(P, P, P, P, P, F, P, P, P, F, CU, 3, 900, 512, 4, 80, 0.1f, 1, 0.1f, 1, nullptr,
                            FA_BF16), FA_OK, 3);
  (void)fa_backward_varlen_workspace_bytes(2147483647, 2147483647, 128);

  // block-sparse
  EXPECT(fa_forward_blocksparse(P, P, P, P, F, U8, 0, 0, 1, 2, 1000, 128, 0.1f, 0, 0.f, 0, nullptr, FA_BF16),
         FA_OK, 1);
  EXPECT(fa_forward_blocksparse(P, P, P, P, F, nullptr, 0, 0, 1, 2, 1000, 128, 0.1f, 0, 0.f, 0, nullptr,
                                FA_BF16), FA_ERR_NULL, 0);
  EXPECT(fa_forward_blocksparse(P, P, P, P, F, U8, -64, 0, 1, 2, 1000, 128, 0.1f, 0, 0.f, 0, nullptr, FA_BF16),
         FA_ERR_ARG, 0);
  EXPECT(fa_backward_blocksparse(P, P, P, P, P, F, P, P, P, F, U8, 64, 64, 1, 2, 1000, 128, 0.1f, 1, 0.1f, 5,
                                 nullptr, FA_BF16), FA_OK, 3);

  // split-KV
  const int ns = fa_splitkv_num_splits(4, 16, 1, 65536, 128);
  if (ns < 1) {
    std::printf("FAIL num_splits %d\n", ns);
    ++failures;
  }
  (void)fa_forward_splitkv_workspace_bytes(2147483647, 2147483647, 2147483647, 128, 8);
  EXPECT(fa_forward_splitkv(P, P, P, P, F, F, 4, 16, 1, 65536, 128, 0.1f, 1, 0, nullptr, FA_BF16), FA_OK, 1);
  EXPECT(fa_forward_splitkv(P, P, P, P, F, F, 4, 16, 1, 65536, 128, 0.1f, 1, 100000, nullptr, FA_BF16),
         FA_ERR_ARG, 0);

  // FP8 scores
  EXPECT(fa_quantize_fp8(P, W8, F, 2, 8192, 16, 128, 128, nullptr), FA_OK, 1);
  EXPECT(fa_quantize_fp8(P, W8, F, 2, 8192, 16, 128, 48, nullptr), FA_ERR_ARG, 0);
  EXPECT(fa_forward_fp8(U8, U8, P, P, F, F, F, 2, 16, 8192, 128, 0.088f, 1, nullptr), FA_OK, 1);
  EXPECT(fa_forward_fp8(U8, U8, P, P, F, nullptr, F, 2, 16, 8192, 128, 0.088f, 1, nullptr), FA_ERR_NULL, 0);

  // dropout mask hook
  EXPECT(fa_dropout_mask(2026, 0, 3, 8, 0.1f, 0, 0, 64, 64, W8, nullptr), FA_OK, 1);
  EXPECT(fa_dropout_mask(2026, 0, 8, 8, 0.1f, 0, 0, 64, 64, W8, nullptr), FA_ERR_ARG, 0);
  EXPECT(fa_dropout_mask(2026, 0, 0, 8, 0.1f, 0, 0, 65536, 65536, W8, nullptr), FA_ERR_ARG, 0);
  EXPECT(fa_dropout_mask(2026, 0, 0, 8, 0.1f, 2147483647, 0, 2, 2, W8, nullptr), FA_ERR_ARG, 0);

  // status strings for every code, and an unknown one
  for (int s = -12; s <= 1; ++s) {
    const char* t = fa_status_string(s);
    if (t == nullptr || std::strlen(t) == 0) {
      std::printf("FAIL status string %d\n", s);
      ++failures;
    }
  }
  if (std::strlen(fa_version()) == 0) ++failures;

  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
