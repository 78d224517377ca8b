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
#include "fa_tile.h"

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
  int B, H, N;  // N: rows per sequence (the longest one for packed batches)
  const int* cu;  // packed variable-length batch offsets, or nullptr
  int total;
  const uint8_t* bmask;  // block-sparse mask, or nullptr
  int64_t msb, msh;
  float scale;
  float c2;  // scale * log2(e)
  uint32_t drop_t;
  float drop_r;
  uint64_t seed;
  int pair_blocks;  // dQ, causal: complementary query block pairs per work-group
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
  p.cu = a.cu_seqlens;
  p.total = a.total;
  p.bmask = a.block_mask;
  p.msb = a.mask_stride_b;
  p.msh = a.mask_stride_h;
  p.scale = a.scale;
  p.c2 = a.scale * kLog2e;
  p.drop_t = a.drop_threshold;
  p.drop_r = a.drop_rescale;
  p.seed = a.seed;
  p.pair_blocks = 0;  // set by the dQ launcher
  return p;
}

// ---------------------------------------------------------------------------
// B1: D[b][h][i] = sum_c dO[b][i][h][c] * O[b][i][h][c], fp32. Sixteen lanes
// per row, 16-byte loads; bound by HBM bandwidth.
// Rows are (token, head) pairs in storage order; the statistics index is
// [b][h][n] for fixed-length batches (total == 0) and [h][token] for packed
// variable-length batches of `total` tokens.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const void* __restrict__ o,
                                                      const void* __restrict__ dout,
                                                      float* __restrict__ dsum, int B, int H,
                                                      int N, int total) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NCH = D * ESZ / 16;
  const int64_t rows = total ? (int64_t)total * H : (int64_t)B * N * H;
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
    if (total) {
      dsum[(int64_t)h * total + bn] = acc;
    } else {
      const int n = (int)(bn % N);
      const int b = (int)(bn / N);
      dsum[((int64_t)b * H + h) * N + n] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Offsets shared by the two bf16 backward kernels, for a 32-row tile in the
// kBoth layout (rows = queries or keys, columns = d).
//   Row reads (16 bytes, lane = row l32, chunk 2c + hf): four per-lane
//   offsets, one per value of c & 3; the group of chunk 2c adds a constant.
//   Transposing reads for the A operand of a product contracting over the
//   rows: 16-lane group g covers rows 4(g/2) + j (+ 8h + 16kt) and columns
//   16(g%2) + 4a (+ 32db) for lane 4j + a; the uniform part of the swizzle,
//   (db & 1, h), selects one of four per-lane offsets.
template <int D>
struct Both32 {
  using T = Tile<32, D, Swz::kBoth>;
  int row[4];     // row reads, full groups
  int row_tail;   // row reads, tail group (D = 80)
  int tr[4];      // transposing reads, full groups
  int tr_tail[2]; // transposing reads, tail group, by h
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hf = lane >> 5;
    const int x = hf ^ T::sw(l32);
#pragma unroll
    for (int u = 0; u < 4; ++u) row[u] = l32 * 128 + (((2 * u) ^ x) << 4);
    row_tail = T::TAIL + l32 * 32 + ((hf ^ T::swt(l32)) << 4);
    const int g = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
    const int s = g >> 1, gh = g & 1;
    const int lp = (2 * gh) ^ (a >> 1) ^ (2 * j) ^ s;
#pragma unroll
    for (int u = 0; u < 4; ++u) tr[u] = (4 * s + j) * 128 + ((lp ^ (2 * u)) << 4) + 8 * (a & 1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      tr_tail[hh] = T::TAIL + (4 * s + j) * 32 + (((a >> 1) ^ s ^ hh) << 4) + 8 * (a & 1);
  }
  // Row read of k-step c (d = 16c .. 16c + 15).
  __device__ __forceinline__ int row_off(int c) const {
    return (2 * c < 8 * T::NG) ? (c >> 2) * T::GBYTES + row[c & 3] : row_tail;
  }
  // The two transposing reads (h = 0, 1) of d-block db and row step kt.
  __device__ __forceinline__ u32x4 tr_frag(const char* tile, int db, int kt) const {
    u32x2 v0, v1;
    if (4 * db < 8 * T::NG) {
      const int gb = (db >> 1) * T::GBYTES + 2048 * kt;
      const int u = 2 * (db & 1);
      v0 = ld_lds_tr16(tile, gb + tr[u]);
      v1 = ld_lds_tr16(tile, gb + 1024 + tr[u + 1]);
    } else {
      v0 = ld_lds_tr16(tile, tr_tail[0] + 512 * kt);
      v1 = ld_lds_tr16(tile, tr_tail[1] + 512 * kt + 256);
    }
    return u32x4{v0[0], v0[1], v1[0], v1[1]};
  }
};

// Instruction order of the dQ step after the score products: the NKC dP^T
// products, each followed by V2 vector instructions (exponentials, dropout
// hashes) and one V-row LDS read two steps ahead; the dS work of the first
// 16-key step (V3a instructions); then the NDB dQ products of that step,
// each followed by V3b vector instructions of the second step's dS and two
// transposing reads; then the second step's NDB products.
template <int NKC, int NDB, int PRE, int V2, int V3a, int V3b>
__device__ __forceinline__ void sched_dq_order() {
  constexpr int kValu = 0x002, kMfma = 0x008, kDs = 0x080;
  __builtin_amdgcn_sched_group_barrier(kDs, PRE + 2, 0);
#pragma unroll
  for (int i = 0; i < NKC; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kValu, V2, 0);
    if (i + 2 < NKC)
      __builtin_amdgcn_sched_group_barrier(kDs, 1, 0);
    else
      __builtin_amdgcn_sched_group_barrier(kDs, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kValu, V3a, 0);
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kValu, V3b, 0);
    __builtin_amdgcn_sched_group_barrier(kDs, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    if (i + 1 < NDB) __builtin_amdgcn_sched_group_barrier(kDs, 2, 0);
  }
}
// Vector work per dQ step: 16 FMAs and 16 exponentials (with dropout also
// 8 hashes, about 40 instructions), then per 16-key step 8 multiplies and
// 4 packs (with dropout 8 keep tests and selects more).
template <int NKC, int NDB, bool DROP>
__device__ __forceinline__ void sched_dq_phases() {
  if constexpr (DROP)
    sched_dq_order<NKC, NDB, 4, (72 + NKC - 1) / NKC, 36, (36 + NDB - 1) / NDB>();
  else
    sched_dq_order<NKC, NDB, 0, (32 + NKC - 1) / NKC, 12, (12 + NDB - 1) / NDB>();
}

// ---------------------------------------------------------------------------
// B2 (bf16): one work-group of NW waves per (block of 32 NW keys, b, h); each
// wave owns 32 keys (lane = key) with their K rows in registers, the block's
// V rows in LDS, and dK^T, dV^T accumulators. Query tiles of 32 rows of Q and
// dO stream through two LDS stages by direct-to-LDS loads; one copy of each
// serves the row reads (A operand of S = Q K^T and dP = dO V^T) and the
// transposing reads (A operand of dK^T += Q^T dS and dV^T += dO^T P~).
template <int D>
struct DkdvCfg {
  static constexpr int NW = 4;     // waves per work-group (32 keys each)
  static constexpr int NT = 64 * NW;
  static constexpr int BK = 32 * NW;  // keys per work-group
  static constexpr int BQ = 32;    // queries per tile
  static constexpr int NKC = D / 16;
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int NDB = DP / 32;
  using QT = Tile<BQ, D, Swz::kBoth>;  // Q and dO tiles
  using VB = Tile<BK, D, Swz::kRow>;   // the block's V rows
  static constexpr int STAGE = 2 * QT::BYTES;
  static constexpr int NLOAD = 2 * QT::NLOAD;
  static constexpr int LPW = (NLOAD + NW - 1) / NW;
  static constexpr int VLPW = (VB::NLOAD + NW - 1) / NW;
};

// QG query groups: with QG = 2 the work-group has two groups of NW waves
// over the same keys; group g takes query tiles g, g + 2, ... with its own LDS
// stages, and the groups' dK/dV partial sums are added in LDS in a fixed
// order at the end. Block-sparse runs use it: a key block whose mask column
// keeps many query blocks (a global key block) otherwise sets the critical
// path of the whole launch.
template <int D, bool CAUSAL, bool DROP, bool SPARSE, int QG = 1>
__global__ __launch_bounds__(DkdvCfg<D>::NT * QG) void bwd_dkdv_bf16_kernel(BwdParams p) {
  using C = DkdvCfg<D>;
  using QT = typename C::QT;
  using VB = typename C::VB;
  __shared__ __align__(16) char vblk[VB::BYTES];
  __shared__ __align__(16) char st0[QG][C::STAGE];
  __shared__ __align__(16) char st1[QG][C::STAGE];
  // Per-stage statistics of the tile's queries: lse * log2(e), D, row keys.
  __shared__ __align__(16) float ls0[QG][C::BQ];
  __shared__ __align__(16) float ls1[QG][C::BQ];
  __shared__ __align__(16) float dd0[QG][C::BQ];
  __shared__ __align__(16) float dd1[QG][C::BQ];
  __shared__ __align__(16) uint32_t ar0[QG][DROP ? C::BQ : 1];
  __shared__ __align__(16) uint32_t ar1[QG][DROP ? C::BQ : 1];
  __shared__ uint16_t kept[SPARSE ? kSparseMaxBlocks : 1];  // kept query blocks
  static_assert(!SPARSE || C::BK == kSparseBlock, "a work-group covers one mask column");
  static_assert(QG == 1 || QG == 2, "one or two query groups");
  // The group-sum buffer (one accumulator block of every wave) fits in st0.
  static_assert(QG == 1 || C::NW * 16 * 64 * 4 <= QG * C::STAGE, "reduction buffer");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = QG == 1 ? 0 : wave / C::NW;       // query group
  const int wv = wave % C::NW;                      // wave within the group: keys kw0 .. kw0 + 31
  const int gt = QG == 1 ? tid : tid - qg * C::NT;  // thread within the group
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H;
  const int nkb = (p.N + C::BK - 1) / C::BK;
  const BlockMap bm = map_block(blockIdx.x, nkb, p.B * H);
  const int kblk = bm.rank;  // causal: key block 0 sees the most queries
  const int b = bm.bh / H, h = bm.bh - b * H;
  const SeqRows sr = seq_rows(p.cu, p.total, b, h, H, D, p.N);
  const int N = sr.n;
  const int k0 = kblk * C::BK;
  if (k0 >= N) return;  // block past the end of a shorter sequence
  const int kw0 = k0 + wv * 32;
  const int mykey = kw0 + l32;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = sr.base;
  const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + base;
  const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + base;
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + base;
  const uint16_t* dOg = static_cast<const uint16_t*>(p.dout) + base;
  const uint32_t rs2 = (uint32_t)(H * D * 2);
  const int64_t statoff = sr.stat;
  const BufRes rl = make_bufres(p.lse + statoff, (uint32_t)N * 4);
  const BufRes rd = make_bufres(p.dsum + statoff, (uint32_t)N * 4);

  // The block's V rows into LDS (rows >= N arrive as zeros).
  {
    const BufRes rvb = rows_bufres(Vg, k0, N, C::BK, rs2);
#pragma unroll
    for (int m = 0; m < C::VLPW; ++m) {
      const int i = wv + C::NW * m;
      if ((QG == 1 || qg == 0) && i < VB::NLOAD) {
        int off, row, ch;
        VB::load_slot(i, lane, off, row, ch);
        lds_dma_16(rvb, vblk + off, (uint32_t)row * rs2 + 16 * ch);
      }
    }
  }
  // This lane's K row (B operand of S = Q K^T); zeros past N.
  const BufRes rk = rows_bufres(Kg, k0, N, C::BK, rs2);
  u32x4 kreg[C::NKC];
#pragma unroll
  for (int c = 0; c < C::NKC; ++c)
    kreg[c] = buf_load_128(rk, (uint32_t)(mykey - k0) * rs2 + (16 * c + 8 * hf) * 2);
  // This lane's V row in LDS (B operand of dP = dO V^T).
  const int vr = wv * 32 + l32;
  const int vx = hf ^ VB::sw(vr);
  int vrow[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) vrow[u] = vr * 128 + (((2 * u) ^ vx) << 4);
  const int vrow_tail = VB::TAIL + vr * 32 + ((hf ^ VB::swt(vr)) << 4);

  // Dropout: lanes 2c and 2c + 1 hold the two keys of one pair (mykey is
  // kw0 + l32 with kw0 even) over the same query rows, so one hash serves
  // both. Each lane of the two hashes two of every four rows (even lane rows
  // 0, 1, odd lane rows 2, 3) and passes the 16-bit draws of its partner's
  // key across; byte selectors pick the halves: own = this key's draws of the
  // two rows, send = the partner key's.
  uint64_t kbh = 0;
  uint32_t bpair = 0, sel_own = 0, sel_send = 0;
  const bool odd = (lane & 1) != 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    bpair = pair_key(kbh, mykey >> 1);
    sel_own = odd ? 0x07060302u : 0x05040100u;  // high (odd key) or low (even key) halves
    sel_send = odd ? 0x05040100u : 0x07060302u;
  }

  const int qstart = CAUSAL ? k0 : 0;
  int ntiles;
  if constexpr (SPARSE) {
    // Kept query blocks of this key block (a mask column), ascending; under
    // the causal mask only blocks from the diagonal on.
    const int nb = (N + kSparseBlock - 1) / kSparseBlock;
    const uint8_t* mcol = p.bmask + b * p.msb + h * p.msh + kblk;
    const KeptBlocks kb = collect_blocks(mcol, nb, CAUSAL ? kblk : 0, nb, kept, lane, wave == 0);
    ntiles = kept_tiles<C::BQ>(kb, N);
    __syncthreads();
  } else {
    ntiles = (N - qstart + C::BQ - 1) / C::BQ;
  }
  auto tile_start = [&](int t) {
    return SPARSE ? kept_tile_start<C::BQ>(kept, t) : qstart + t * C::BQ;
  };

  // This wave's share of the tile loads: Q instructions, then dO.
  uint32_t dsrc[C::LPW];
  int dlds[C::LPW];
#pragma unroll
  for (int m = 0; m < C::LPW; ++m) {
    const int i = wv + C::NW * m;
    int off = 0, row = 0, ch = 0;
    if (i < QT::NLOAD) {
      QT::load_slot(i, lane, off, row, ch);
    } else if (i < C::NLOAD) {
      QT::load_slot(i - QT::NLOAD, lane, off, row, ch);
      off += QT::BYTES;
    }
    dsrc[m] = (uint32_t)row * rs2 + 16 * ch;
    dlds[m] = off;
  }
  // Statistics of a query tile: threads 0-31 of the group load lse, 32-63
  // load D, 64-95 hash the row keys; stored after the tile's compute. Rows
  // past N read zeros (their Q and dO rows are zero too, so they add nothing).
  float sx = 0.f;
  auto stat_load = [&](int qt0) {
    if (gt < 32) {
      sx = buf_load_f32(rl, (uint32_t)(qt0 + gt) * 4);
    } else if (gt < 64) {
      sx = buf_load_f32(rd, (uint32_t)(qt0 + gt - 32) * 4);
    } else if (DROP && gt < 96) {
      sx = __uint_as_float(row_key(kbh, qt0 + gt - 64));
    }
  };
  auto stat_store = [&](float* ls, float* dd, uint32_t* ar) {
    if (gt < 32) {
      ls[gt] = DROP ? sx * kLog2e : -sx / p.scale;  // without dropout: start of the S accumulator
    } else if (gt < 64) {
      dd[gt - 32] = DROP ? sx : -sx;  // without dropout the dP accumulator starts at -D
    } else if (DROP && gt < 96) {
      ar[gt - 64] = __float_as_uint(sx);
    }
  };
  auto issue = [&](char* stage, int qt0) {
    const BufRes rq = rows_bufres(Qg, qt0, N, C::BQ, rs2);
    const BufRes ro = rows_bufres(dOg, qt0, N, C::BQ, rs2);
#pragma unroll
    for (int m = 0; m < C::LPW; ++m) {
      const int i = wv + C::NW * m;
      if (i < C::NLOAD) lds_dma_16(i < QT::NLOAD ? rq : ro, stage + dlds[m], dsrc[m]);
    }
  };

  Both32<D> ofs;
  ofs.init(lane);

  f32x16 dkacc[C::NDB], dvacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  // One query tile without dropout, in issue order: each group of
  // instructions below is kept in place by a scheduling barrier, so the
  // matrix products and the vector work of the same tile alternate within
  // the wave. The S accumulator starts at -lse/scale and the dP accumulator
  // at -D (both from the per-stage arrays), so P = exp2(S * scale log2 e)
  // and dS = P * dP need one multiply each per element.
  auto dkdv_tile_nodrop = [&](const char* cur, const float* lsc, const float* ddc, int qt0) {
    constexpr int NKC = C::NKC, NT = 2 * C::NDB;
    // Phase 1: S = Q K^T (K in registers, Q rows from LDS).
    f32x16 s;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(lsc + 8 * g + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * g + e] = x[e];
    }
#pragma unroll
    for (int c = 0; c < NKC; ++c) s = mfma32x32x16(ld_lds_128(cur, ofs.row_off(c)), kreg[c], s);
    sched_lds_ahead<NKC, 1, 1, 4>();
    __builtin_amdgcn_sched_barrier(0);
    if (CAUSAL && qt0 < kw0 + 31) {
      // diagonal tile: keys after the query get probability exp2(-inf) = 0
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = mykey > qt0 + c_row(r, hf) ? -INFINITY : s[r];
    }
    __builtin_amdgcn_sched_barrier(0);
    // dP = dO V^T (dO rows and the block's V rows from LDS), starting at -D.
    f32x16 dp;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(ddc + 8 * g + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * g + e] = x[e];
    }
    // Phases 2-4 as one sequence of NKC + 4 NDB products (dP, then dV,
    // then dK), each followed by the LDS reads of the product two places
    // later and by a share of the vector work: probability e (multiply +
    // exp2) after product (e (NKC + NDB)) / 16, dS value e after product
    // NKC + (3 NDB e) / 16, and each pack right after its last input. The
    // shares are spread so that no product carries more than about one and
    // a half exponentials, and every operand is ready before the product
    // that takes it (P^T of step kt before the dV products of step kt, dS
    // of step kt before the dK products of step kt).
    constexpr int NP = NKC + 4 * C::NDB;   // products after the S phase
    constexpr int SP = NKC + C::NDB;       // slots that carry probabilities
    constexpr int SS = 3 * C::NDB;         // slots that carry dS values
    u32x4 xa[NKC], xb[NKC];
    u32x4 ta[NT], tb[NT];  // transposing-read operands of the dV and dK products
    auto ops = [&](int j) {
      if (j < NKC) {
        const int o = ofs.row_off(j);
        const int vo = (2 * j < 8 * VB::NG) ? (j >> 2) * VB::GBYTES + vrow[j & 3] : vrow_tail;
        xa[j] = ld_lds_128(cur, QT::BYTES + o);
        xb[j] = ld_lds_128(vblk, vo);
      } else if (j < NKC + NT) {
        const int t = j - NKC;
        ta[t] = ofs.tr_frag(cur + QT::BYTES, t % C::NDB, t / C::NDB);
      } else if (j < NP) {
        const int t = j - NKC - NT;
        tb[t] = ofs.tr_frag(cur, t % C::NDB, t / C::NDB);
      }
    };
    ops(0);
    ops(1);
    float pv[16], dsv[16];
    u32x4 pop[2], sop[2];
    auto pack8 = [&](const float* x) {
      return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j < NKC) {
        dp = mfma32x32x16(xa[j], xb[j], dp);
      } else if (j < NKC + NT) {
        const int t = j - NKC;
        dvacc[t % C::NDB] = mfma32x32x16(ta[t], pop[t / C::NDB], dvacc[t % C::NDB]);
      } else {
        const int t = j - NKC - NT;
        dkacc[t % C::NDB] = mfma32x32x16(tb[t], sop[t / C::NDB], dkacc[t % C::NDB]);
      }
      ops(j + 2);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((e * SP) / 16 == j) pv[e] = exp2_hw(s[e] * p.c2);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        if (((8 * kt + 7) * SP) / 16 == j) pop[kt] = pack8(pv + 8 * kt);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (NKC + (e * SS) / 16 == j) dsv[e] = pv[e] * dp[e];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        if (NKC + ((8 * kt + 7) * SS) / 16 == j) sop[kt] = pack8(dsv + 8 * kt);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step of this group over kept query tile t (t >= ntiles: the group has
  // no tile in this step and only takes part in the barrier).
  auto step = [&](const char* cur, const float* lsc, const float* ddc, const uint32_t* arc,
                  char* nxt, float* lsn, float* ddn, uint32_t* arn, int t) {
    wait_vmem();
    __syncthreads();
    if constexpr (kLdsPoison) poison_stage(nxt, C::STAGE, gt, C::NT);
    const bool valid = QG == 1 || t < ntiles;  // one group: every step has a tile
    const int qt0 = valid ? tile_start(t) : 0;
    const bool more = t + QG < ntiles;
    if (more) {
      const int qn = tile_start(t + QG);
      stat_load(qn);
      issue(nxt, qn);
    }
    if (valid && (!CAUSAL || qt0 + C::BQ - 1 >= kw0)) {
      if constexpr (!DROP) {
        dkdv_tile_nodrop(cur, lsc, ddc, qt0);
      } else {
      // S = Q K^T and dP = dO V^T : lane = key, register r -> query qt0 + c_row(r, hf)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NKC; ++c) {
        const int o = ofs.row_off(c);
        const int vo = (2 * c < 8 * VB::NG) ? (c >> 2) * VB::GBYTES + vrow[c & 3] : vrow_tail;
        s = mfma32x32x16(ld_lds_128(cur, o), kreg[c], s);
        dp = mfma32x32x16(ld_lds_128(cur, QT::BYTES + o), ld_lds_128(vblk, vo), dp);
      }
      // Issue order: the three LDS reads of step c + 2 go out before the two
      // products of step c, so read latency overlaps the matrix cores.
      sched_lds_ahead<C::NKC, 3, 2>();
      if (CAUSAL && qt0 < kw0 + 31) {
        // diagonal tile: keys after the query get probability exp2(-inf) = 0
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = mykey > qt0 + c_row(r, hf) ? -INFINITY : s[r];
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float pt[8], dsv[8];
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int g = 2 * kt + gg;
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(lsc + 8 * g + 4 * hf);
          const f32x4 dd = *reinterpret_cast<const f32x4*>(ddc + 8 * g + 4 * hf);
          // Dropout draws of rows 8g + 4hf + e: e = 0, 1 in dr01, e = 2, 3 in
          // dr23 (low half, high half).
          uint32_t dr01 = 0, dr23 = 0;
          if constexpr (DROP) {
            const u32x2 ar = *reinterpret_cast<const u32x2*>(arc + 8 * g + 4 * hf + (odd ? 2 : 0));
            uint32_t fa = pair_mix(ar[0], bpair), fb = pair_mix(ar[1], bpair);
            fa ^= fa >> 16;  // fmix32: low half the even key's draw, high half the odd key's
            fb ^= fb >> 16;
            const uint32_t own = __builtin_amdgcn_perm(fb, fa, sel_own);
            const uint32_t send = __builtin_amdgcn_perm(fb, fa, sel_send);
            const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
            dr01 = odd ? recv : own;
            dr23 = odd ? own : recv;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const float pv = exp2_hw(fmaf(s[r], p.c2, -l2[e]));
            float dpv = dp[r];
            float ptv = pv;
            if constexpr (DROP) {
              const uint32_t dw = e < 2 ? dr01 : dr23;
              const bool kp = (e & 1) ? dw >= (p.drop_t << 16) : (dw & 0xFFFFu) >= p.drop_t;
              const float mr = kp ? p.drop_r : 0.f;
              ptv = pv * mr;
              dpv *= mr;
            }
            pt[4 * gg + e] = ptv;
            dsv[4 * gg + e] = pv * (dpv - dd[e]);
          }
        }
        const u32x4 pop = {pack_bf16x2(pt[0], pt[1]), pack_bf16x2(pt[2], pt[3]),
                           pack_bf16x2(pt[4], pt[5]), pack_bf16x2(pt[6], pt[7])};
        const u32x4 sop = {pack_bf16x2(dsv[0], dsv[1]), pack_bf16x2(dsv[2], dsv[3]),
                           pack_bf16x2(dsv[4], dsv[5]), pack_bf16x2(dsv[6], dsv[7])};
        // dV^T += dO^T P~ and dK^T += Q^T dS over the 16 queries of step kt.
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          dvacc[db] = mfma32x32x16(ofs.tr_frag(cur + QT::BYTES, db, kt), pop, dvacc[db]);
          dkacc[db] = mfma32x32x16(ofs.tr_frag(cur, db, kt), sop, dkacc[db]);
        }
      }
      // Statistics reads first, then the four transposing reads of step i + 1
      // ahead of the two products of step i.
      sched_lds_ahead<2 * C::NDB, 4, 2, DROP ? 12 : 8, 1>();
      }
    }
    if (more) stat_store(lsn, ddn, arn);
  };

  const int nsteps = (ntiles + QG - 1) / QG;  // the same count for every group
  if constexpr (kLdsPoison) poison_stage(st0[qg], C::STAGE, gt, C::NT);
  if (qg < ntiles) {
    stat_load(tile_start(qg));
    issue(st0[qg], tile_start(qg));
    stat_store(ls0[qg], dd0[qg], ar0[qg]);
  }
  for (int s = 0; s < nsteps; s += 2) {
    step(st0[qg], ls0[qg], dd0[qg], ar0[qg], st1[qg], ls1[qg], dd1[qg], ar1[qg], qg + QG * s);
    if (s + 1 < nsteps)
      step(st1[qg], ls1[qg], dd1[qg], ar1[qg], st0[qg], ls0[qg], dd0[qg], ar0[qg], qg + QG * (s + 1));
  }

  if constexpr (QG == 2) {
    // Group 1's sums into group 0's, one accumulator block at a time through
    // st0 (free once every wave has passed the barrier): slot (wave, r, lane).
    float* red = reinterpret_cast<float*>(&st0[0][0]);
#pragma unroll
    for (int tsel = 0; tsel < 2; ++tsel) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        f32x16& acc = tsel ? dvacc[db] : dkacc[db];
        __syncthreads();
        if (qg == 1) {
#pragma unroll
          for (int r = 0; r < 16; ++r) red[(wv * 16 + r) * 64 + lane] = acc[r];
        }
        __syncthreads();
        if (qg == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] += red[(wv * 16 + r) * 64 + lane];
        }
      }
    }
  }

  if ((QG == 1 || qg == 0) && mykey < N) {
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
// (lane = query). Key tiles of 32 rows of K and V stream through two LDS
// stages by direct-to-LDS loads: K row reads (A operand of S^T = K Q^T) and
// K transposing reads (A operand of dQ^T += K^T dS^T) from one copy, V row
// reads (A operand of dP^T = V dO^T).
template <int D, int NW = 4>
struct DqCfg {
  static constexpr int NT = 64 * NW;  // NW waves of 32 queries
  static constexpr int BQ = 32 * NW;
  static constexpr int BK = 32;
  static constexpr int NKC = D / 16;
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int NDB = DP / 32;
  using KT = Tile<BK, D, Swz::kBoth>;
  using VT = Tile<BK, D, Swz::kRow>;
  static constexpr int STAGE = KT::BYTES + VT::BYTES;
  static constexpr int NLOAD = KT::NLOAD + VT::NLOAD;
  static constexpr int LPW = (NLOAD + NW - 1) / NW;
};

// NW = 8 (256 queries per work-group) at long sequences: each K/V tile then
// serves twice the queries, which halves the K/V bytes streamed from L2 and
// beyond per query (the key-range prefixes of co-resident work-groups do not
// share L2 lines at 32K+ keys).
template <int D, bool CAUSAL, bool DROP, bool SPARSE, int NW = 4>
__global__ __launch_bounds__(64 * NW) void bwd_dq_bf16_kernel(BwdParams p) {
  using C = DqCfg<D, NW>;
  using KT = typename C::KT;
  using VT = typename C::VT;
  __shared__ __align__(16) char st0[C::STAGE];
  __shared__ __align__(16) char st1[C::STAGE];
  __shared__ __align__(16) uint32_t bc0[DROP ? C::BK / 2 : 1];  // dropout keys of the tile's key pairs
  __shared__ __align__(16) uint32_t bc1[DROP ? C::BK / 2 : 1];
  __shared__ uint16_t kept[SPARSE ? kSparseMaxBlocks : 1];  // kept key blocks
  static_assert(!SPARSE || C::BQ == kSparseBlock, "a work-group covers one mask row");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H;
  const int nqb = (p.N + C::BQ - 1) / C::BQ;
  // Causal, eight-wave groups without dropout (long sequences), with
  // p.pair_blocks: the pair of query blocks (nqb - 1 - j, j) per
  // work-group, the second over descending key tiles, so that the
  // work-groups of a head sweep the same K/V tiles together. Other
  // instances take one block per work-group (heaviest first) and compile
  // to a single pass.
  constexpr int kPasses = (NW == 8 && CAUSAL && !DROP && !SPARSE) ? 2 : 1;
  const bool paired = kPasses == 2 && p.pair_blocks;
  const BlockMap bm = paired ? map_block_pair(blockIdx.x, (nqb + 1) / 2, p.B * H)
                             : map_block(blockIdx.x, nqb, p.B * H);
  const int b = bm.bh / H, h = bm.bh - b * H;
  const SeqRows sr = seq_rows(p.cu, p.total, b, h, H, D, p.N);
  const int N = sr.n;
  int qb_first, qb_second = -1;
  if (paired) {
    const int nb = (N + C::BQ - 1) / C::BQ;
    if (bm.rank >= (nb + 1) / 2) return;
    qb_first = nb - 1 - bm.rank;
    if (bm.rank < qb_first) qb_second = bm.rank;
  } else {
    qb_first = CAUSAL ? (nqb - 1 - bm.rank) : bm.rank;
  }
#pragma unroll 1
  for (int pass = 0; pass < kPasses; ++pass) {
    const int qb = pass == 0 ? qb_first : qb_second;
    if (qb < 0) break;
    const bool rev = pass > 0;  // the key tiles in descending order
    // The previous block's last tile may still be read from a stage.
    if (pass > 0) __syncthreads();
    const int q0 = qb * C::BQ;
    if (q0 >= N) break;  // block past the end of a shorter sequence
    const int qw0 = q0 + wave * 32;
    const int myq = qw0 + l32;
    const int64_t rs = (int64_t)H * D;
    const int64_t base = sr.base;
    const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + base;
    const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + base;
    const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + base;
    const uint16_t* dOg = static_cast<const uint16_t*>(p.dout) + base;
    const uint32_t rs2 = (uint32_t)(H * D * 2);
    const BufRes rq = rows_bufres(Qg, q0, N, C::BQ, rs2), rdo = rows_bufres(dOg, q0, N, C::BQ, rs2);
    const int64_t statoff = sr.stat;
    const BufRes rl = make_bufres(p.lse + statoff, (uint32_t)N * 4);
    const BufRes rd = make_bufres(p.dsum + statoff, (uint32_t)N * 4);

    // Rows past N: zero Q, dO, LSE and D give dS = 0 (never stored anyway).
    u32x4 qreg[C::NKC], doreg[C::NKC];
  #pragma unroll
    for (int c = 0; c < C::NKC; ++c) {
      const uint32_t off = (uint32_t)(myq - q0) * rs2 + (16 * c + 8 * hf) * 2;
      qreg[c] = buf_load_128(rq, off);
      doreg[c] = buf_load_128(rdo, off);
    }
    const float lse2 = buf_load_f32(rl, (uint32_t)myq * 4) * kLog2e;
    const float dq_d = buf_load_f32(rd, (uint32_t)myq * 4);
    uint64_t kbh = 0;
    uint32_t arow = 0;
    if constexpr (DROP) {
      kbh = head_key(p.seed, b, h, H);
      arow = row_key(kbh, myq);
    }

    const int kend = CAUSAL ? min(N, q0 + C::BQ) : N;
    int ntiles;
    if constexpr (SPARSE) {
      const int nb = (N + kSparseBlock - 1) / kSparseBlock;
      const uint8_t* mrow = p.bmask + b * p.msb + h * p.msh + (int64_t)qb * nb;
      const KeptBlocks kb =
          collect_blocks(mrow, 1, 0, (kend + kSparseBlock - 1) / kSparseBlock, kept, lane, wave == 0);
      ntiles = kept_tiles<C::BK>(kb, kend);
      __syncthreads();
    } else {
      ntiles = (kend + C::BK - 1) / C::BK;
    }
    auto tile_start = [&](int t) {
      if (rev) t = ntiles - 1 - t;
      return SPARSE ? kept_tile_start<C::BK>(kept, t) : t * C::BK;
    };

    // This wave's share of the tile loads: K instructions, then V.
    uint32_t dsrc[C::LPW];
    int dlds[C::LPW];
  #pragma unroll
    for (int m = 0; m < C::LPW; ++m) {
      const int i = wave + NW * m;
      int off = 0, row = 0, ch = 0;
      if (i < KT::NLOAD) {
        KT::load_slot(i, lane, off, row, ch);
      } else if (i < C::NLOAD) {
        VT::load_slot(i - KT::NLOAD, lane, off, row, ch);
        off += KT::BYTES;
      }
      dsrc[m] = (uint32_t)row * rs2 + 16 * ch;
      dlds[m] = off;
    }
    auto issue = [&](char* stage, uint32_t* bc, int k0) {
      const BufRes rk = rows_bufres(Kg, k0, N, C::BK, rs2);
      const BufRes rv = rows_bufres(Vg, k0, N, C::BK, rs2);
  #pragma unroll
      for (int m = 0; m < C::LPW; ++m) {
        const int i = wave + NW * m;
        if (i < C::NLOAD) lds_dma_16(i < KT::NLOAD ? rk : rv, stage + dlds[m], dsrc[m]);
      }
      if constexpr (DROP) {
        if (tid < C::BK / 2) bc[tid] = pair_key(kbh, (k0 >> 1) + tid);
      }
    };

    Both32<D> ofs;
    ofs.init(lane);
    const int vx = hf ^ VT::sw(l32);
    int vrow[4];
  #pragma unroll
    for (int u = 0; u < 4; ++u) vrow[u] = KT::BYTES + l32 * 128 + (((2 * u) ^ vx) << 4);
    const int vrow_tail = KT::BYTES + VT::TAIL + l32 * 32 + ((hf ^ VT::swt(l32)) << 4);

    f32x16 dqacc[C::NDB];
  #pragma unroll
    for (int db = 0; db < C::NDB; ++db) dqacc[db] = f32x16{};
    f32x16 negd;  // -D of this lane's query: start of the dP^T accumulator (no dropout)
  #pragma unroll
    for (int r = 0; r < 16; ++r) negd[r] = -dq_d;

    auto step = [&](const char* cur, const uint32_t* bcc, char* nxt, uint32_t* bcn, int t) {
      wait_vmem();
      __syncthreads();
      if constexpr (kLdsPoison) poison_stage(nxt, C::STAGE, tid, C::NT);
      const int k0 = tile_start(t);
      if (t + 1 < ntiles) issue(nxt, bcn, tile_start(t + 1));
      if (CAUSAL && k0 > qw0 + 31) return;
      // Phase 1. S^T = K Q^T : lane = query, register r -> key k0 + c_row(r, hf).
      f32x16 s = f32x16{};
  #pragma unroll
      for (int c = 0; c < C::NKC; ++c) s = mfma32x32x16(ld_lds_128(cur, ofs.row_off(c)), qreg[c], s);
      sched_lds_ahead<C::NKC, 1, 1>();
      __builtin_amdgcn_sched_barrier(0);  // the later phases are ordered on their own
      if ((k0 + C::BK > N) || (CAUSAL && k0 + C::BK - 1 > qw0)) {
        // tail or diagonal tile: keys past N or after the query get exp2(-inf) = 0
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + c_row(r, hf);
          s[r] = (key >= N || (CAUSAL && key > myq)) ? -INFINITY : s[r];
        }
      }
      // Phase 2. dP^T = V dO^T on the matrix cores while the vector ALUs form
      // P^T; without dropout the accumulator starts at -D of this lane's query.
      f32x16 dp = DROP ? f32x16{} : negd;
  #pragma unroll
      for (int c = 0; c < C::NKC; ++c) {
        const int vo = (2 * c < 8 * VT::NG) ? (c >> 2) * VT::GBYTES + vrow[c & 3] : vrow_tail;
        dp = mfma32x32x16(ld_lds_128(cur, vo), doreg[c], dp);
      }
      float pv[16];
      // Registers 4g + e hold keys 8g + 4hf + e; keys (e, e + 1), e = 0, 2, are
      // a pair and share one dropout hash.
      uint32_t yd[DROP ? 4 : 1][2];
  #pragma unroll
      for (int g = 0; g < 4; ++g) {
        if constexpr (DROP) {
          const u32x2 bc = *reinterpret_cast<const u32x2*>(bcc + 4 * g + 2 * hf);
          yd[g][0] = pair_mix(arow, bc[0]);
          yd[g][1] = pair_mix(arow, bc[1]);
        }
  #pragma unroll
        for (int e = 0; e < 4; ++e) pv[4 * g + e] = exp2_hw(fmaf(s[4 * g + e], p.c2, -lse2));
      }
      // Phase 3. dS^T = P^T (dP^T - D) per 16-key step, and dQ^T += K^T dS^T.
  #pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float dsv[8];
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * kt + i, g = r >> 2, e = r & 3;
          if constexpr (DROP) {
            const uint32_t y = yd[DROP ? g : 0][e >> 1];
            const bool kp = (e & 1) ? keep_odd(y, p.drop_t) : keep_even(y, p.drop_t);
            dsv[i] = pv[r] * ((kp ? dp[r] * p.drop_r : 0.f) - dq_d);
          } else {
            dsv[i] = pv[r] * dp[r];
          }
        }
        const u32x4 sop = {pack_bf16x2(dsv[0], dsv[1]), pack_bf16x2(dsv[2], dsv[3]),
                           pack_bf16x2(dsv[4], dsv[5]), pack_bf16x2(dsv[6], dsv[7])};
  #pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          dqacc[db] = mfma32x32x16(ofs.tr_frag(cur, db, kt), sop, dqacc[db]);
      }
      sched_dq_phases<C::NKC, C::NDB, DROP>();
    };

    if constexpr (kLdsPoison) poison_stage(st0, C::STAGE, tid, C::NT);
    if (ntiles > 0) issue(st0, bc0, tile_start(0));
    for (int t = 0; t < ntiles; t += 2) {
      step(st0, bc0, st1, bc1, t);
      if (t + 1 < ntiles) step(st1, bc1, st0, bc0, t + 1);
    }

    if (myq < N) {
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
  const int H = p.H;
  const int nkb = (p.N + BKW - 1) / BKW;
  const BlockMap bm = map_block(blockIdx.x, nkb, p.B * H);
  const int b = bm.bh / H, h = bm.bh - b * H;
  const SeqRows sr = seq_rows(p.cu, p.total, b, h, H, D, p.N);
  const int N = sr.n;
  const int k0 = bm.rank * BKW;
  if (k0 >= N) return;  // block past the end of a shorter sequence
  const int mykey = k0 + ki;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = sr.base;
  const float* Qg = static_cast<const float*>(p.q) + base;
  const float* Kg = static_cast<const float*>(p.k) + base;
  const float* Vg = static_cast<const float*>(p.v) + base;
  const float* dOg = static_cast<const float*>(p.dout) + base;
  const int64_t statoff = sr.stat;

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
  uint32_t bpair = 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    bpair = pair_key(kbh, mykey >> 1);
  }
  const int qstart = CAUSAL ? k0 : 0;
  const int nb = (N + kSparseBlock - 1) / kSparseBlock;
  const uint8_t* mcol =  // this key block's column of the block mask
      p.bmask ? p.bmask + b * p.msb + h * p.msh + k0 / kSparseBlock : nullptr;
  for (int qt0 = qstart; qt0 < N; qt0 += BQ) {
    if (mcol != nullptr && mcol[(int64_t)(qt0 / kSparseBlock) * nb] == 0) continue;  // uniform
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
        const bool kp = keep_key(pair_mix(ars[i], bpair), mykey, p.drop_t);
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
  __shared__ uint32_t bcs[BK / 2];  // dropout keys of the tile's key pairs

  const int tid = threadIdx.x;
  const int qi = tid >> 2, part = tid & 3;
  const int H = p.H;
  const int nqb = (p.N + BQW - 1) / BQW;
  const BlockMap bm = map_block(blockIdx.x, nqb, p.B * H);
  const int qb = CAUSAL ? (nqb - 1 - bm.rank) : bm.rank;
  const int b = bm.bh / H, h = bm.bh - b * H;
  const SeqRows sr = seq_rows(p.cu, p.total, b, h, H, D, p.N);
  const int N = sr.n;
  const int q0 = qb * BQW;
  if (q0 >= N) return;  // block past the end of a shorter sequence
  const int myq = q0 + qi;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = sr.base;
  const float* Qg = static_cast<const float*>(p.q) + base;
  const float* Kg = static_cast<const float*>(p.k) + base;
  const float* Vg = static_cast<const float*>(p.v) + base;
  const float* dOg = static_cast<const float*>(p.dout) + base;
  const int64_t statoff = sr.stat;

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
  const uint8_t* mrow =  // this query block's row of the block mask
      p.bmask ? p.bmask + b * p.msb + h * p.msh +
                    (int64_t)(q0 / kSparseBlock) * ((N + kSparseBlock - 1) / kSparseBlock)
              : nullptr;
  for (int k0 = 0; k0 < kend; k0 += BK) {
    if (mrow != nullptr && mrow[k0 / kSparseBlock] == 0) continue;  // uniform over the block
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
      if (tid < BK / 2) bcs[tid] = pair_key(kbh, (k0 >> 1) + tid);
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
      if constexpr (DROP) dpv = keep_key(pair_mix(arow, bcs[j >> 1]), j, p.drop_t) ? dpv * p.drop_r : 0.f;
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
    const int j = col0 + c;
    out[i] = keep_key(pair_mix(row_key(kbh, row0 + r), pair_key(kbh, j >> 1)), j, thr) ? 1 : 0;
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

// bf16 matrix-core kernels: (d, causal, dropout, block-sparse) instances.
template <int D, bool SPARSE>
hipError_t launch_dkdv_ds(const BwdParams& prm, bool causal, bool drop, dim3 grid, dim3 block,
                          hipStream_t s) {
  // Block-sparse: two query groups per work-group (see the kernel).
  constexpr int QG = SPARSE ? 2 : 1;
  block.x *= QG;
  if (causal) {
    if (drop)
      hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, true, true, SPARSE, QG>), grid, block, 0, s, prm);
    else
      hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, true, false, SPARSE, QG>), grid, block, 0, s, prm);
  } else {
    if (drop)
      hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, false, true, SPARSE, QG>), grid, block, 0, s, prm);
    else
      hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, false, false, SPARSE, QG>), grid, block, 0, s, prm);
  }
  return hipGetLastError();
}

template <int D, bool SPARSE>
hipError_t launch_dq_ds(const BwdParams& prm, bool causal, bool drop, dim3 grid, dim3 block,
                        hipStream_t s) {
  // A block-mask row covers 128 queries: block-sparse runs keep four waves.
  if constexpr (!SPARSE) {
    if (prm.N >= 32768) {
      const int nq8 = (prm.N + 255) / 256;
      const dim3 grid8((unsigned)(nq8 * prm.B * prm.H)), block8(512);
      if (causal) {
        if (drop) {
          hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, true, true, false, 8>), grid8, block8, 0, s, prm);
        } else {
          // Query block pairs per work-group (see the kernel). Measured at
          // N = 32768, d = 80: 2.50 -> 0.93 GB fetched from beyond L2 per
          // launch at the same time (3.700 / 3.704 ms); four-wave dQ at
          // N = 8192 and the dropout kernels were slower paired.
          BwdParams pp = prm;
          pp.pair_blocks = prm.cu == nullptr;
          const dim3 gridp((unsigned)((pp.pair_blocks ? (nq8 + 1) / 2 : nq8) * prm.B * prm.H));
          hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, true, false, false, 8>), gridp, block8, 0, s, pp);
        }
      } else {
        if (drop)
          hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, false, true, false, 8>), grid8, block8, 0, s, prm);
        else
          hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, false, false, false, 8>), grid8, block8, 0, s, prm);
      }
      return hipGetLastError();
    }
  }
  if (causal) {
    if (drop)
      hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, true, true, SPARSE>), grid, block, 0, s, prm);
    else
      hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, true, false, SPARSE>), grid, block, 0, s, prm);
  } else {
    if (drop)
      hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, false, true, SPARSE>), grid, block, 0, s, prm);
    else
      hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, false, false, SPARSE>), grid, block, 0, s, prm);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_d(const BwdParams& prm, bool causal, bool drop, dim3 grid, dim3 block,
                         hipStream_t s) {
  return prm.bmask ? launch_dkdv_ds<D, true>(prm, causal, drop, grid, block, s)
                   : launch_dkdv_ds<D, false>(prm, causal, drop, grid, block, s);
}

template <int D>
hipError_t launch_dq_d(const BwdParams& prm, bool causal, bool drop, dim3 grid, dim3 block,
                       hipStream_t s) {
  return prm.bmask ? launch_dq_ds<D, true>(prm, causal, drop, grid, block, s)
                   : launch_dq_ds<D, false>(prm, causal, drop, grid, block, s);
}

}  // namespace

hipError_t launch_bwd_preprocess(const AttnArgs& a, hipStream_t s, bool bf16) {
  const int64_t rows = a.cu_seqlens ? (int64_t)a.total * a.H : (int64_t)a.B * a.N * a.H;
  const int total = a.cu_seqlens ? a.total : 0;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 15) / 16)), block(256);
#define FA_PRE(D)                                                                             \
  case D:                                                                                     \
    if (bf16)                                                                                 \
      hipLaunchKernelGGL((bwd_pre_kernel<D, true>), grid, block, 0, s, a.o, a.dout, a.dsum_out, \
                         a.B, a.H, a.N, total);                                               \
    else                                                                                      \
      hipLaunchKernelGGL((bwd_pre_kernel<D, false>), grid, block, 0, s, a.o, a.dout,          \
                         a.dsum_out, a.B, a.H, a.N, total);                                   \
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
  constexpr int BK = DkdvCfg<64>::BK, NT = DkdvCfg<64>::NT;
  const dim3 grid((unsigned)(((a.N + BK - 1) / BK) * a.B * a.H)), block(NT);
  switch (a.d) {
    case 64: return launch_dkdv_d<64>(prm, a.causal, a.dropout, grid, block, s);
    case 80: return launch_dkdv_d<80>(prm, a.causal, a.dropout, grid, block, s);
    case 128: return launch_dkdv_d<128>(prm, a.causal, a.dropout, grid, block, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq_bf16(const AttnArgs& a, hipStream_t s) {
  const BwdParams prm = make_params(a);
  const dim3 grid((unsigned)(((a.N + 127) / 128) * a.B * a.H)), block(256);
  switch (a.d) {
    case 64: return launch_dq_d<64>(prm, a.causal, a.dropout, grid, block, s);
    case 80: return launch_dq_d<80>(prm, a.causal, a.dropout, grid, block, s);
    case 128: return launch_dq_d<128>(prm, a.causal, a.dropout, grid, block, s);
    default: return hipErrorInvalidValue;
  }
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
