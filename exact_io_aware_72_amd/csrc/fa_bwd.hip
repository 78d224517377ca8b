// Backward pass of exact attention on gfx950, by recomputation.
//
// The forward pass saved only O and the row logsumexp; the backward pass
// rebuilds each probability tile from Q, K and that logsumexp instead of
// reading a stored N x N matrix ("FlashAttention for Efficient Training",
// sections 2.1 "Forward Pass with Recomputation" and 3.2 "Integration with
// Autograd Engines"; "How FlashAttention Optimizes GPU Memory for Fast AI
// Training", section "4. Recomputation in the Backward Pass").
//
// Gradients of L = sum(dO * O) (chain rule of section 3.2 of the first page):
//   P   = exp(scale*Q K^T - LSE)          (recomputed, causal-masked)
//   P~  = P * Z / (1 - p)                 (Z: dropout keep mask)
//   dV  = P~^T dO                         (the page's dV formula)
//   dP  = (dO V^T) * Z / (1 - p)
//   D_i = sum_c dO_ic O_ic                (= sum_j P_ij dP_ij)
//   dS  = P * (dP - D)
//   dQ  = scale * dS K,    dK = scale * dS^T Q
// Three kernels: B1 computes D; B2 owns a block of keys and accumulates dK
// and dV over the query tiles that see it; B3 owns a block of queries and
// accumulates dQ over its key tiles. B2 and B3 only read what B1 and the
// forward pass wrote, so no atomics are needed and results are reproducible.
#include "fa_device.h"
#include "fa_hash.h"
#include "fa_kernels.h"

namespace fa {
namespace {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* dsum;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N;
  float scale;
  float c2;  // scale * log2(e)
  uint32_t drop_t;
  float drop_r;
  uint64_t seed;
};

BwdParams make_params(const AttnArgs& a) {
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.dout = a.dout;
  p.lse = a.lse;
  p.dsum = a.dsum;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.B = a.B;
  p.H = a.H;
  p.N = a.N;
  p.scale = a.scale;
  p.c2 = a.scale * kLog2e;
  p.drop_t = a.drop_threshold;
  p.drop_r = a.drop_rescale;
  p.seed = a.seed;
  return p;
}

// ---------------------------------------------------------------------------
// B1: D[b][h][i] = sum_c dO[b][i][h][c] * O[b][i][h][c], fp32. Sixteen lanes
// per row, 16-byte loads; bound by HBM bandwidth.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const void* __restrict__ o,
                                                      const void* __restrict__ dout,
                                                      float* __restrict__ dsum, int B, int H,
                                                      int N) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NCH = D * ESZ / 16;
  const int64_t rows = (int64_t)B * N * H;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const char* orow = static_cast<const char*>(o) + row * D * ESZ;
    const char* drow = static_cast<const char*>(dout) + row * D * ESZ;
    for (int c = sub; c < NCH; c += 16) {
      const u32x4 a = ld_global_128(orow + c * 16);
      const u32x4 g = ld_global_128(drow + c * 16);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (BF16) {
          acc = fmaf(bf16_lo(a[w]), bf16_lo(g[w]), acc);
          acc = fmaf(bf16_hi(a[w]), bf16_hi(g[w]), acc);
        } else {
          acc = fmaf(__uint_as_float(a[w]), __uint_as_float(g[w]), acc);
        }
      }
    }
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (row < rows && sub == 0) {
    const int h = (int)(row % H);
    const int64_t bn = row / H;
    const int n = (int)(bn % N);
    const int b = (int)(bn / N);
    dsum[((int64_t)b * H + h) * N + n] = acc;
  }
}

// ---------------------------------------------------------------------------
// B2 (bf16): one work-group of 8 waves per (block of 256 keys, b, h); each
// wave owns 32 keys, with their K rows in registers, their V rows in LDS
// (read once per query tile) and dK^T, dV^T accumulators (lane = key).
// Query tiles of 32 rows stream through LDS, staged once for all 8 waves and
// stored twice: row-major (A operand of S = Q K^T and dP = dO V^T) and
// transposed with the contraction relabelling (A operand of dK^T += Q^T dS
// and dV^T += dO^T P~).
template <int D, bool DROP>
struct DkdvCfg {
  static constexpr int NT = 512;   // 8 waves
  static constexpr int BK = 256;   // keys per work-group
  static constexpr int BQ = 32;    // queries per tile
  static constexpr int NKC = D / 16;
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int NDB = DP / 32;
  static constexpr int KCH = D / 8;
  static constexpr int RS = (D + 8) * 2;   // bytes per row-major row
  static constexpr int TS = (BQ + 8) * 2;  // bytes per transposed row
  static constexpr int NAT = BQ * RS;
  static constexpr int TRN = DP * TS;
  static constexpr int VBLK = BK * RS;     // this block's V rows
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_QT = NAT;
  static constexpr int OFF_DO = NAT + TRN;
  static constexpr int OFF_DOT = 2 * NAT + TRN;
  static constexpr int OFF_LSE = 2 * (NAT + TRN);
  static constexpr int OFF_DS = OFF_LSE + BQ * 4;
  static constexpr int OFF_AR = OFF_DS + BQ * 4;
  static constexpr int BUF = OFF_AR + (DROP ? BQ * 4 : 0);
  static constexpr int ITEMS1 = (BQ / 4) * KCH;  // 4-row x 16-byte items per tensor
  static constexpr int STAT0 = 256;              // first thread loading row statistics
  static_assert(2 * ITEMS1 <= STAT0, "staging items fit below the statistics threads");
  static constexpr int V_ITEMS = BK * KCH;
  static constexpr int V_PER_T = (V_ITEMS + NT - 1) / NT;
};

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(512) void bwd_dkdv_bf16_kernel(BwdParams p) {
  using C = DkdvCfg<D, DROP>;
  __shared__ __align__(16) char smem[C::VBLK + 2 * C::BUF];
  char* const vblk = smem;
  char* const bufs = smem + C::VBLK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int N = p.N, H = p.H;
  const int nkb = (N + C::BK - 1) / C::BK;
  const BlockMap bm = map_block(blockIdx.x, nkb, p.B * H);
  const int kblk = bm.rank;  // causal: key block 0 sees the most queries
  const int b = bm.bh / H, h = bm.bh - b * H;
  const int k0 = kblk * C::BK;
  const int kw0 = k0 + wave * 32;
  const int mykey = kw0 + l32;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * N * H + h) * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + base;
  const uint16_t* dOg = static_cast<const uint16_t*>(p.dout) + base;
  // Buffer resources over this head: reads of rows >= N return zeros. Zero Q
  // and dO rows (with zero LSE and D) contribute exactly nothing to dK, dV.
  const uint32_t rs2 = (uint32_t)(H * D * 2);
  const uint32_t nbytes = (uint32_t)N * rs2;
  const BufRes rq = make_bufres(Qg, nbytes), rk = make_bufres(Kg, nbytes);
  const BufRes rv = make_bufres(Vg, nbytes), rdo = make_bufres(dOg, nbytes);
  const BufRes rl = make_bufres(p.lse + ((int64_t)b * H + h) * N, (uint32_t)N * 4);
  const BufRes rd = make_bufres(p.dsum + ((int64_t)b * H + h) * N, (uint32_t)N * 4);

  if constexpr (C::DP > D) {
    // transposed rows d >= D feed only discarded accumulator rows
    constexpr int PAD16 = (C::DP - D) * C::TS / 16;
    for (int i = tid; i < 2 * 2 * PAD16; i += C::NT) {
      const int which = i / PAD16, j = i - which * PAD16;
      const int bsel = which >> 1;
      const int off = (which & 1) ? C::OFF_DOT : C::OFF_QT;
      st_lds_128(bufs + bsel * C::BUF + off + D * C::TS, j * 16, u32x4{0, 0, 0, 0});
    }
  }

  // This block's V rows, row-major in LDS (B operand of dP = dO V^T).
#pragma unroll
  for (int i = 0; i < C::V_PER_T; ++i) {
    const int item = tid + i * C::NT;
    if (C::V_ITEMS % C::NT == 0 || item < C::V_ITEMS) {
      const int r = item / C::KCH, c = item - r * C::KCH;
      st_lds_128(vblk, r * C::RS + c * 16, buf_load_128(rv, (uint32_t)(k0 + r) * rs2 + 16 * c));
    }
  }
  u32x4 kreg[C::NKC];
#pragma unroll
  for (int c = 0; c < C::NKC; ++c)
    kreg[c] = buf_load_128(rk, (uint32_t)mykey * rs2 + (16 * c + 8 * hf) * 2);
  const int vrow = (wave * 32 + l32) * C::RS + 16 * hf;  // this lane's V row in LDS

  uint64_t kbh = 0;
  uint32_t bcol = 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    bcol = col_key(kbh, mykey);
  }

  const int qstart = CAUSAL ? k0 : 0;
  const int ntiles = (N - qstart + C::BQ - 1) / C::BQ;

  u32x4 st[4];
  float sx = 0.f;
  auto load_tile = [&](int qt0) {
    if (tid < 2 * C::ITEMS1) {
      const int which = tid / C::ITEMS1, it = tid - which * C::ITEMS1;
      const StageItem si = stage_item(it, C::BQ / 4, C::KCH);
      const BufRes src = which ? rdo : rq;
      const uint32_t off = (uint32_t)(qt0 + 4 * si.g) * rs2 + 16 * si.c;
#pragma unroll
      for (int j = 0; j < 4; ++j) st[j] = buf_load_128(src, off + j * rs2);
    } else if (tid >= C::STAT0) {
      const int which = (tid - C::STAT0) >> 5;
      const int q = qt0 + (tid & 31);
      if (which == 0) {
        sx = buf_load_f32(rl, (uint32_t)q * 4) * kLog2e;
      } else if (which == 1) {
        sx = buf_load_f32(rd, (uint32_t)q * 4);
      } else if (DROP && which == 2) {
        sx = __uint_as_float(row_key(kbh, q));
      }
    }
  };
  auto store_tile = [&](char* buf) {
    if (tid < 2 * C::ITEMS1) {
      const int which = tid / C::ITEMS1, it = tid - which * C::ITEMS1;
      const StageItem si = stage_item(it, C::BQ / 4, C::KCH);
      char* nat = buf + (which ? C::OFF_DO : C::OFF_Q);
      char* trn = buf + (which ? C::OFF_DOT : C::OFF_QT);
#pragma unroll
      for (int j = 0; j < 4; ++j) st_lds_128(nat, (4 * si.g + j) * C::RS + si.c * 16, st[j]);
      st_lds_transpose4x8(trn, C::TS, 8 * si.c, perm_pos4(si.g), st[0], st[1], st[2], st[3]);
    } else if (tid >= C::STAT0 && tid < C::STAT0 + (DROP ? 96 : 64)) {
      const int which = (tid - C::STAT0) >> 5;
      const int off = which == 0 ? C::OFF_LSE : (which == 1 ? C::OFF_DS : C::OFF_AR);
      *reinterpret_cast<float*>(buf + off + (tid & 31) * 4) = sx;
    }
  };

  f32x16 dkacc[C::NDB], dvacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  load_tile(qstart);
  store_tile(bufs);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const char* buf = bufs + (t & 1) * C::BUF;
    const int qt0 = qstart + t * C::BQ;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(qt0 + C::BQ);
    if (!CAUSAL || qt0 + C::BQ - 1 >= kw0) {
      // S = Q K^T and dP = dO V^T : lane = key, register r -> query qt0 + c_row(r, hf)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NKC; ++c) {
        const int col = (16 * c + 8 * hf) * 2;
        s = mfma32x32x16(ld_lds_128(buf + C::OFF_Q, l32 * C::RS + col), kreg[c], s);
        dp = mfma32x32x16(ld_lds_128(buf + C::OFF_DO, l32 * C::RS + col),
                          ld_lds_128(vblk, vrow + 32 * c), dp);
      }
      const bool need_mask = CAUSAL && (qt0 < kw0 + 31);
      float pt[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l2 = ld_lds_f32x4(buf + C::OFF_LSE, (8 * g + 4 * hf) * 4);
        const f32x4 dd = ld_lds_f32x4(buf + C::OFF_DS, (8 * g + 4 * hf) * 4);
        u32x4 ar = {0, 0, 0, 0};
        if constexpr (DROP) ar = ld_lds_u32x4(buf + C::OFF_AR, (8 * g + 4 * hf) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = exp2_hw(fmaf(s[r], p.c2, -l2[e]));
          if (need_mask) pv = mykey > qt0 + c_row(r, hf) ? 0.f : pv;
          float dpv = dp[r];
          if constexpr (DROP) {
            const bool kp = keep(ar[e], bcol, p.drop_t);
            pt[r] = kp ? pv * p.drop_r : 0.f;
            dpv = kp ? dpv * p.drop_r : 0.f;
          } else {
            pt[r] = pv;
          }
          s[r] = pv * (dpv - dd[e]);  // dS
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int rb = kt * 8;
        const u32x4 pop = {pack_bf16x2(pt[rb + 0], pt[rb + 1]), pack_bf16x2(pt[rb + 2], pt[rb + 3]),
                           pack_bf16x2(pt[rb + 4], pt[rb + 5]), pack_bf16x2(pt[rb + 6], pt[rb + 7])};
        const u32x4 sop = {pack_bf16x2(s[rb + 0], s[rb + 1]), pack_bf16x2(s[rb + 2], s[rb + 3]),
                           pack_bf16x2(s[rb + 4], s[rb + 5]), pack_bf16x2(s[rb + 6], s[rb + 7])};
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const int off = (db * 32 + l32) * C::TS + (16 * kt + 8 * hf) * 2;
          dvacc[db] = mfma32x32x16(ld_lds_128(buf + C::OFF_DOT, off), pop, dvacc[db]);
          dkacc[db] = mfma32x32x16(ld_lds_128(buf + C::OFF_QT, off), sop, dkacc[db]);
        }
      }
    }
    if (more) store_tile(bufs + ((t + 1) & 1) * C::BUF);
    __syncthreads();
  }

  if (mykey < N) {
    uint16_t* dkrow = static_cast<uint16_t*>(p.dk) + base + (int64_t)mykey * rs;
    uint16_t* dvrow = static_cast<uint16_t*>(p.dv) + base + (int64_t)mykey * rs;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hf;
        if (d0 < D) {
          const u32x2 wk = {pack_bf16x2(dkacc[db][4 * g] * sc, dkacc[db][4 * g + 1] * sc),
                            pack_bf16x2(dkacc[db][4 * g + 2] * sc, dkacc[db][4 * g + 3] * sc)};
          const u32x2 wv = {pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]),
                            pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3])};
          st_global_64(dkrow + d0, wk);
          st_global_64(dvrow + d0, wv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// B3 (bf16): one work-group per (block of 128 queries, b, h); each wave owns
// 32 queries with Q and dO rows in registers and a dQ^T accumulator
// (lane = query). Key tiles of 32 rows stream through LDS: K row-major
// (A operand of S^T = K Q^T), K transposed with the contraction relabelling
// (A operand of dQ^T += K^T dS^T) and V row-major (A operand of
// dP^T = V dO^T).
template <int D, bool DROP>
struct DqCfg {
  static constexpr int NT = 256;
  static constexpr int BQ = 128;
  static constexpr int BK = 32;
  static constexpr int NKC = D / 16;
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int NDB = DP / 32;
  static constexpr int KCH = D / 8;
  static constexpr int RS = (D + 8) * 2;
  static constexpr int TS = (BK + 8) * 2;
  static constexpr int NAT = BK * RS;
  static constexpr int TRN = DP * TS;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_KT = NAT;
  static constexpr int OFF_V = NAT + TRN;
  static constexpr int OFF_BC = 2 * NAT + TRN;
  static constexpr int BUF = OFF_BC + (DROP ? BK * 4 : 0);
  static constexpr int ITEMS1 = (BK / 4) * KCH;
  static_assert(2 * ITEMS1 <= NT, "one staging item per thread");
};

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256) void bwd_dq_bf16_kernel(BwdParams p) {
  using C = DqCfg<D, DROP>;
  __shared__ __align__(16) char smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int N = p.N, H = p.H;
  const int nqb = (N + C::BQ - 1) / C::BQ;
  const BlockMap bm = map_block(blockIdx.x, nqb, p.B * H);
  const int qb = CAUSAL ? (nqb - 1 - bm.rank) : bm.rank;
  const int b = bm.bh / H, h = bm.bh - b * H;
  const int q0 = qb * C::BQ;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + l32;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * N * H + h) * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + base;
  const uint16_t* dOg = static_cast<const uint16_t*>(p.dout) + base;

  if constexpr (C::DP > D) {
    constexpr int PAD16 = (C::DP - D) * C::TS / 16;
    for (int i = tid; i < 2 * PAD16; i += C::NT) {
      const int bsel = i / PAD16, j = i - bsel * PAD16;
      st_lds_128(smem + bsel * C::BUF + C::OFF_KT + D * C::TS, j * 16, u32x4{0, 0, 0, 0});
    }
  }

  // Buffer resources over this head: reads of rows >= N return zeros.
  const uint32_t rs2 = (uint32_t)(H * D * 2);
  const uint32_t nbytes = (uint32_t)N * rs2;
  const BufRes rq = make_bufres(Qg, nbytes), rk = make_bufres(Kg, nbytes);
  const BufRes rv = make_bufres(Vg, nbytes), rdo = make_bufres(dOg, nbytes);
  const int64_t statoff = ((int64_t)b * H + h) * N;
  const BufRes rl = make_bufres(p.lse + statoff, (uint32_t)N * 4);
  const BufRes rd = make_bufres(p.dsum + statoff, (uint32_t)N * 4);

  u32x4 qreg[C::NKC], doreg[C::NKC];
  const bool qok = myq < N;
#pragma unroll
  for (int c = 0; c < C::NKC; ++c) {
    const uint32_t off = (uint32_t)myq * rs2 + (16 * c + 8 * hf) * 2;
    qreg[c] = buf_load_128(rq, off);
    doreg[c] = buf_load_128(rdo, off);
  }
  // Rows past N: zero Q, dO, LSE and D give dS = 0 (never stored anyway).
  const float lse2 = buf_load_f32(rl, (uint32_t)myq * 4) * kLog2e;
  const float dq_d = buf_load_f32(rd, (uint32_t)myq * 4);
  uint64_t kbh = 0;
  uint32_t arow = 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    arow = row_key(kbh, myq);
  }

  const int kend = CAUSAL ? min(N, q0 + C::BQ) : N;
  const int ntiles = (kend + C::BK - 1) / C::BK;

  u32x4 st[4];
  uint32_t bst = 0;
  auto load_tile = [&](int k0) {
    if (tid < 2 * C::ITEMS1) {
      const int which = tid / C::ITEMS1, it = tid - which * C::ITEMS1;
      const StageItem si = stage_item(it, C::BK / 4, C::KCH);
      const BufRes src = which ? rv : rk;
      const uint32_t off = (uint32_t)(k0 + 4 * si.g) * rs2 + 16 * si.c;
#pragma unroll
      for (int j = 0; j < 4; ++j) st[j] = buf_load_128(src, off + j * rs2);
    }
    if constexpr (DROP) {
      if (tid >= 224) bst = col_key(kbh, k0 + (tid - 224));
    }
  };
  auto store_tile = [&](char* buf) {
    if (tid < 2 * C::ITEMS1) {
      const int which = tid / C::ITEMS1, it = tid - which * C::ITEMS1;
      const StageItem si = stage_item(it, C::BK / 4, C::KCH);
      char* nat = buf + (which ? C::OFF_V : C::OFF_K);
#pragma unroll
      for (int j = 0; j < 4; ++j) st_lds_128(nat, (4 * si.g + j) * C::RS + si.c * 16, st[j]);
      if (which == 0)
        st_lds_transpose4x8(buf + C::OFF_KT, C::TS, 8 * si.c, perm_pos4(si.g), st[0], st[1], st[2],
                            st[3]);
    }
    if constexpr (DROP) {
      if (tid >= 224) *reinterpret_cast<uint32_t*>(buf + C::OFF_BC + (tid - 224) * 4) = bst;
    }
  };

  f32x16 dqacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) dqacc[db] = f32x16{};

  load_tile(0);
  store_tile(smem);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const char* buf = smem + (t & 1) * C::BUF;
    const int k0 = t * C::BK;
    if (t + 1 < ntiles) load_tile(k0 + C::BK);
    const bool active = !CAUSAL || (k0 <= qw0 + 31);
    if (active) {
      // S^T = K Q^T : lane = query, register r -> key k0 + c_row(r, hf)
      f32x16 s = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NKC; ++c)
        s = mfma32x32x16(ld_lds_128(buf + C::OFF_K, l32 * C::RS + (16 * c + 8 * hf) * 2), qreg[c],
                         s);
      f32x16 dp = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NKC; ++c)
        dp = mfma32x32x16(ld_lds_128(buf + C::OFF_V, l32 * C::RS + (16 * c + 8 * hf) * 2),
                          doreg[c], dp);
      const bool need_mask = (k0 + C::BK > N) || (CAUSAL && k0 + C::BK - 1 > qw0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 bc = {0, 0, 0, 0};
        if constexpr (DROP) bc = ld_lds_u32x4(buf + C::OFF_BC, (8 * g + 4 * hf) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = exp2_hw(s[r] * p.c2 - lse2);
          if (need_mask) {
            const int key = k0 + c_row(r, hf);
            if (key >= N || (CAUSAL && key > myq)) pv = 0.f;
          }
          float dpv = dp[r];
          if constexpr (DROP) dpv = keep(arow, bc[e], p.drop_t) ? dpv * p.drop_r : 0.f;
          s[r] = pv * (dpv - dq_d);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int rb = kt * 8;
        const u32x4 sop = {pack_bf16x2(s[rb + 0], s[rb + 1]), pack_bf16x2(s[rb + 2], s[rb + 3]),
                           pack_bf16x2(s[rb + 4], s[rb + 5]), pack_bf16x2(s[rb + 6], s[rb + 7])};
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          dqacc[db] = mfma32x32x16(
              ld_lds_128(buf + C::OFF_KT, (db * 32 + l32) * C::TS + (16 * kt + 8 * hf) * 2), sop,
              dqacc[db]);
      }
    }
    if (t + 1 < ntiles) store_tile(smem + ((t + 1) & 1) * C::BUF);
    __syncthreads();
  }

  if (qok) {
    uint16_t* dqrow = static_cast<uint16_t*>(p.dq) + base + (int64_t)myq * rs;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hf;
        if (d0 < D) {
          const u32x2 w = {pack_bf16x2(dqacc[db][4 * g] * sc, dqacc[db][4 * g + 1] * sc),
                           pack_bf16x2(dqacc[db][4 * g + 2] * sc, dqacc[db][4 * g + 3] * sc)};
          st_global_64(dqrow + d0, w);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 backward on the vector ALUs: four threads per row, each owning a
// quarter of the head dimension; tiles of 16 rows in LDS.
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(128) void bwd_dkdv_f32_kernel(BwdParams p) {
  constexpr int BKW = 32, BQ = 16, DQ = D / 4;
  __shared__ __align__(16) float qs[BQ][D];
  __shared__ __align__(16) float gs[BQ][D];
  __shared__ float l2s[BQ], dss[BQ];
  __shared__ uint32_t ars[BQ];

  const int tid = threadIdx.x;
  const int ki = tid >> 2, part = tid & 3;
  const int N = p.N, H = p.H;
  const int nkb = (N + BKW - 1) / BKW;
  const BlockMap bm = map_block(blockIdx.x, nkb, p.B * H);
  const int b = bm.bh / H, h = bm.bh - b * H;
  const int k0 = bm.rank * BKW;
  const int mykey = k0 + ki;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * N * H + h) * D;
  const float* Qg = static_cast<const float*>(p.q) + base;
  const float* Kg = static_cast<const float*>(p.k) + base;
  const float* Vg = static_cast<const float*>(p.v) + base;
  const float* dOg = static_cast<const float*>(p.dout) + base;
  const int64_t statoff = ((int64_t)b * H + h) * N;

  float kv[DQ], vv[DQ], dk[DQ], dv[DQ];
  const bool kok = mykey < N;
#pragma unroll
  for (int c = 0; c < DQ; ++c) {
    kv[c] = kok ? Kg[(int64_t)mykey * rs + part * DQ + c] : 0.f;
    vv[c] = kok ? Vg[(int64_t)mykey * rs + part * DQ + c] : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  uint64_t kbh = 0;
  uint32_t bcol = 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    bcol = col_key(kbh, mykey);
  }
  const int qstart = CAUSAL ? k0 : 0;
  for (int qt0 = qstart; qt0 < N; qt0 += BQ) {
    __syncthreads();
    for (int i = tid; i < BQ * D / 4; i += 128) {
      const int r = i / (D / 4), c = (i - r * (D / 4)) * 4;
      const int q = qt0 + r;
      f32x4 qx = {0.f, 0.f, 0.f, 0.f}, gx = {0.f, 0.f, 0.f, 0.f};
      if (q < N) {
        qx = *reinterpret_cast<const f32x4*>(Qg + (int64_t)q * rs + c);
        gx = *reinterpret_cast<const f32x4*>(dOg + (int64_t)q * rs + c);
      }
      *reinterpret_cast<f32x4*>(&qs[r][c]) = qx;
      *reinterpret_cast<f32x4*>(&gs[r][c]) = gx;
    }
    if (tid < BQ) {
      const int q = qt0 + tid;
      l2s[tid] = q < N ? p.lse[statoff + q] * kLog2e : INFINITY;
      dss[tid] = q < N ? p.dsum[statoff + q] : 0.f;
      if constexpr (DROP) ars[tid] = row_key(kbh, q);
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < BQ; ++i) {
      float sv = 0.f, dpv = 0.f;
#pragma unroll
      for (int c = 0; c < DQ; ++c) {
        sv = fmaf(kv[c], qs[i][part * DQ + c], sv);
        dpv = fmaf(vv[c], gs[i][part * DQ + c], dpv);
      }
      sv += __shfl_xor(sv, 1);
      sv += __shfl_xor(sv, 2);
      dpv += __shfl_xor(dpv, 1);
      dpv += __shfl_xor(dpv, 2);
      const int q = qt0 + i;
      float pv = exp2_hw(sv * p.c2 - l2s[i]);
      if (CAUSAL && mykey > q) pv = 0.f;
      float ptv = pv;
      if constexpr (DROP) {
        const bool kp = keep(ars[i], bcol, p.drop_t);
        ptv = kp ? pv * p.drop_r : 0.f;
        dpv = kp ? dpv * p.drop_r : 0.f;
      }
      const float dsv = pv * (dpv - dss[i]);
#pragma unroll
      for (int c = 0; c < DQ; ++c) {
        dv[c] = fmaf(ptv, gs[i][part * DQ + c], dv[c]);
        dk[c] = fmaf(dsv, qs[i][part * DQ + c], dk[c]);
      }
    }
  }
  if (kok) {
    float* dkrow = static_cast<float*>(p.dk) + base + (int64_t)mykey * rs + part * DQ;
    float* dvrow = static_cast<float*>(p.dv) + base + (int64_t)mykey * rs + part * DQ;
#pragma unroll
    for (int c = 0; c < DQ; ++c) {
      dkrow[c] = dk[c] * p.scale;
      dvrow[c] = dv[c];
    }
  }
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(128) void bwd_dq_f32_kernel(BwdParams p) {
  constexpr int BQW = 32, BK = 16, DQ = D / 4;
  __shared__ __align__(16) float ks[BK][D];
  __shared__ __align__(16) float vs[BK][D];
  __shared__ uint32_t bcs[BK];

  const int tid = threadIdx.x;
  const int qi = tid >> 2, part = tid & 3;
  const int N = p.N, H = p.H;
  const int nqb = (N + BQW - 1) / BQW;
  const BlockMap bm = map_block(blockIdx.x, nqb, p.B * H);
  const int qb = CAUSAL ? (nqb - 1 - bm.rank) : bm.rank;
  const int b = bm.bh / H, h = bm.bh - b * H;
  const int q0 = qb * BQW;
  const int myq = q0 + qi;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * N * H + h) * D;
  const float* Qg = static_cast<const float*>(p.q) + base;
  const float* Kg = static_cast<const float*>(p.k) + base;
  const float* Vg = static_cast<const float*>(p.v) + base;
  const float* dOg = static_cast<const float*>(p.dout) + base;
  const int64_t statoff = ((int64_t)b * H + h) * N;

  const bool qok = myq < N;
  float qv[DQ], gv[DQ], dq[DQ];
#pragma unroll
  for (int c = 0; c < DQ; ++c) {
    qv[c] = qok ? Qg[(int64_t)myq * rs + part * DQ + c] : 0.f;
    gv[c] = qok ? dOg[(int64_t)myq * rs + part * DQ + c] : 0.f;
    dq[c] = 0.f;
  }
  const float lse2 = qok ? p.lse[statoff + myq] * kLog2e : INFINITY;
  const float dd = qok ? p.dsum[statoff + myq] : 0.f;
  uint64_t kbh = 0;
  uint32_t arow = 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    arow = row_key(kbh, myq);
  }
  const int kend = CAUSAL ? min(N, q0 + BQW) : N;
  for (int k0 = 0; k0 < kend; k0 += BK) {
    __syncthreads();
    for (int i = tid; i < BK * D / 4; i += 128) {
      const int r = i / (D / 4), c = (i - r * (D / 4)) * 4;
      const int key = k0 + r;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < N) {
        kx = *reinterpret_cast<const f32x4*>(Kg + (int64_t)key * rs + c);
        vx = *reinterpret_cast<const f32x4*>(Vg + (int64_t)key * rs + c);
      }
      *reinterpret_cast<f32x4*>(&ks[r][c]) = kx;
      *reinterpret_cast<f32x4*>(&vs[r][c]) = vx;
    }
    if constexpr (DROP) {
      if (tid < BK) bcs[tid] = col_key(kbh, k0 + tid);
    }
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < BK; ++j) {
      float sv = 0.f, dpv = 0.f;
#pragma unroll
      for (int c = 0; c < DQ; ++c) {
        sv = fmaf(qv[c], ks[j][part * DQ + c], sv);
        dpv = fmaf(gv[c], vs[j][part * DQ + c], dpv);
      }
      sv += __shfl_xor(sv, 1);
      sv += __shfl_xor(sv, 2);
      dpv += __shfl_xor(dpv, 1);
      dpv += __shfl_xor(dpv, 2);
      const int key = k0 + j;
      float pv = exp2_hw(sv * p.c2 - lse2);
      if (key >= N || (CAUSAL && key > myq)) pv = 0.f;
      if constexpr (DROP) dpv = keep(arow, bcs[j], p.drop_t) ? dpv * p.drop_r : 0.f;
      const float dsv = pv * (dpv - dd);
#pragma unroll
      for (int c = 0; c < DQ; ++c) dq[c] = fmaf(dsv, ks[j][part * DQ + c], dq[c]);
    }
  }
  if (qok) {
    float* dqrow = static_cast<float*>(p.dq) + base + (int64_t)myq * rs + part * DQ;
#pragma unroll
    for (int c = 0; c < DQ; ++c) dqrow[c] = dq[c] * p.scale;
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dropout_mask_kernel(uint64_t seed, int b, int h, int H,
                                                           uint32_t thr, int row0, int col0,
                                                           int rows, int cols, uint8_t* out) {
  const uint64_t kbh = head_key(seed, b, h, H);
  const int64_t total = (int64_t)rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / cols), c = (int)(i - (int64_t)r * cols);
    out[i] = keep(row_key(kbh, row0 + r), col_key(kbh, col0 + c), thr) ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
#define FA_DISPATCH_CD(KERNEL, D, causal, drop, grid, block, s, prm)                         \
  do {                                                                                       \
    if (causal) {                                                                            \
      if (drop)                                                                              \
        hipLaunchKernelGGL((KERNEL<D, true, true>), grid, block, 0, s, prm);                 \
      else                                                                                   \
        hipLaunchKernelGGL((KERNEL<D, true, false>), grid, block, 0, s, prm);                \
    } else {                                                                                 \
      if (drop)                                                                              \
        hipLaunchKernelGGL((KERNEL<D, false, true>), grid, block, 0, s, prm);                \
      else                                                                                   \
        hipLaunchKernelGGL((KERNEL<D, false, false>), grid, block, 0, s, prm);               \
    }                                                                                        \
  } while (0)

#define FA_DISPATCH(KERNEL, d, causal, drop, grid, block, s, prm)                  \
  do {                                                                             \
    switch (d) {                                                                   \
      case 64: FA_DISPATCH_CD(KERNEL, 64, causal, drop, grid, block, s, prm); break;   \
      case 80: FA_DISPATCH_CD(KERNEL, 80, causal, drop, grid, block, s, prm); break;   \
      case 128: FA_DISPATCH_CD(KERNEL, 128, causal, drop, grid, block, s, prm); break; \
      default: return hipErrorInvalidValue;                                        \
    }                                                                              \
  } while (0)

}  // namespace

hipError_t launch_bwd_preprocess(const AttnArgs& a, hipStream_t s, bool bf16) {
  const int64_t rows = (int64_t)a.B * a.N * a.H;
  const dim3 grid((unsigned)((rows + 15) / 16)), block(256);
#define FA_PRE(D)                                                                             \
  case D:                                                                                     \
    if (bf16)                                                                                 \
      hipLaunchKernelGGL((bwd_pre_kernel<D, true>), grid, block, 0, s, a.o, a.dout, a.dsum_out, \
                         a.B, a.H, a.N);                                                      \
    else                                                                                      \
      hipLaunchKernelGGL((bwd_pre_kernel<D, false>), grid, block, 0, s, a.o, a.dout,          \
                         a.dsum_out, a.B, a.H, a.N);                                          \
    break;
  switch (a.d) {
    FA_PRE(64)
    FA_PRE(80)
    FA_PRE(128)
    default: return hipErrorInvalidValue;
  }
#undef FA_PRE
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const AttnArgs& a, hipStream_t s) {
  const BwdParams prm = make_params(a);
  const dim3 grid((unsigned)(((a.N + 255) / 256) * a.B * a.H)), block(512);
  FA_DISPATCH(bwd_dkdv_bf16_kernel, a.d, a.causal, a.dropout, grid, block, s, prm);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const AttnArgs& a, hipStream_t s) {
  const BwdParams prm = make_params(a);
  const dim3 grid((unsigned)(((a.N + 127) / 128) * a.B * a.H)), block(256);
  FA_DISPATCH(bwd_dq_bf16_kernel, a.d, a.causal, a.dropout, grid, block, s, prm);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const AttnArgs& a, hipStream_t s) {
  const BwdParams prm = make_params(a);
  const dim3 grid((unsigned)(((a.N + 31) / 32) * a.B * a.H)), block(128);
  FA_DISPATCH(bwd_dkdv_f32_kernel, a.d, a.causal, a.dropout, grid, block, s, prm);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const AttnArgs& a, hipStream_t s) {
  const BwdParams prm = make_params(a);
  const dim3 grid((unsigned)(((a.N + 31) / 32) * a.B * a.H)), block(128);
  FA_DISPATCH(bwd_dq_f32_kernel, a.d, a.causal, a.dropout, grid, block, s, prm);
  return hipGetLastError();
}

hipError_t launch_dropout_mask(uint64_t seed, int b, int h, int H, uint32_t threshold, int row0,
                               int col0, int rows, int cols, uint8_t* out, hipStream_t s) {
  const int64_t total = (int64_t)rows * cols;
  const int64_t want = (total + 255) / 256;
  const unsigned nblk = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(dropout_mask_kernel, dim3(nblk), dim3(256), 0, s, seed, b, h, H, threshold,
                     row0, col0, rows, cols, out);
  return hipGetLastError();
}

}  // namespace fa
