// Forward pass of exact attention on gfx950.
//
// One work-group owns BM query rows of one (batch, head) and streams the key
// and value tiles of that head through LDS ("FlashAttention for Efficient
// Training", section 3.1 "Workflow Breakdown": load blocks into fast memory,
// compute the local scores and partial softmax, update the output block).
// The score tile S, its probabilities P and the output accumulator stay in
// registers; only O and the row logsumexp are written
// ("How FlashAttention Optimizes GPU Memory for Fast AI Training", sections
// "1. Tiling", "2. Online Softmax", "3. Kernel Fusion").
//
// bf16 path, per wave (32 query rows, one per lane pair L and L+32):
//   S^T = K_j Q^T on the matrix cores, so each lane holds scores of ONE query;
//   the row max needs one exchange between the two lane halves and the row
//   sum none until the end; the output rescale is one multiply per register.
//   O^T += V_j^T P^T with P^T taken straight from the score registers; V_j is
//   staged in LDS transposed (and with the contraction relabelling of
//   fa_device.h) for that operand.
//   Online softmax in base 2 with scale*log2(e) folded into one multiply:
//   m' = max(m, max_j x_j), alpha = 2^(m - m'), p = 2^(x - m'),
//   l = alpha*l + sum p, O = alpha*O + P V (section 3.2 "Precision Handling and
//   Numerical Stability": running max and sum, rescaled partial outputs).
//   LSE = ln2 * (m + log2 l).
// Causal: key tiles wholly after the block's last query are never loaded;
// a wave skips tiles wholly after its own last query; diagonal tiles are
// masked per element.
#include "fa_device.h"
#include <type_traits>

#include "fa_hash.h"
#include "fa_kernels.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

#define FA_HIP_RETURN_IF(x)            \
  do {                                 \
    const hipError_t e_ = (x);         \
    if (e_ != hipSuccess) return e_;   \
  } while (0)

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, H, N;  // N: rows per sequence (the longest one for packed batches)
  const int* cu;  // packed variable-length batch offsets, or nullptr
  int total;
  const uint8_t* bmask;  // block-sparse mask, or nullptr
  int64_t msb, msh;
  // Causal, whole grid resident: work-groups per CU and CUs per XCD for
  // map_block_pairs; pair_slots = 0 keeps the rank-major map_block.
  int pair_slots, cus_per_xcd;
  int pair_blocks;  // causal: complementary block pairs per work-group
  // Split-KV: Nk key rows per batch item (N query rows), the key range cut
  // into nsplit parts; part s writes O_s (fp32, normalised) and LSE_s.
  int Nk, nsplit;
  float* ws_o;    // [nsplit][B][H][N][D]
  float* ws_lse;  // [nsplit][B][H][N]
  // FP8 scores: Q and K as OCP E4M3 bytes [B][N][H][D] with one scale per
  // 128 query rows ([B][H][ceil(N/128)]) and per 64 key rows
  // ([B][H][ceil(N/64)]); scores are scale_q * scale_k * (Q8 . K8).
  const uint8_t* q8;
  const uint8_t* k8;
  const float* q_scale;
  const float* k_scale;
  float c2;  // scale * log2(e)
  uint32_t drop_t;
  float drop_r;
  uint64_t seed;
};

template <int D, bool FP8 = false, int NW_ = 4>
struct FwdCfg {
  static constexpr int NW = NW_;                 // waves, 32 query rows each
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;             // query rows per work-group
  static constexpr int BN = 64;                  // keys per tile
  static constexpr int NKC = D / 16;             // k-steps of S^T = K Q^T
  static constexpr int DP = (D + 31) / 32 * 32;  // rows of O^T computed (d padded to 32)
  static constexpr int NDB = DP / 32;
  // K tile: 16-byte row reads (bf16, or FP8 bytes).
  using KT = typename std::conditional<FP8, Fp8Tile<BN, D>, Tile<BN, D, Swz::kRow>>::type;
  using VT = Tile<BN, D, Swz::kTr>;              // V tile: transposing reads
  static constexpr int STAGE = KT::BYTES + VT::BYTES;
  static constexpr int NLOAD = KT::NLOAD + VT::NLOAD;  // load instructions per tile
  static constexpr int LPW = (NLOAD + NW - 1) / NW;    // per wave
};

// At most two waves per SIMD: with the smaller FP8 tiles three work-groups
// would fit a CU, and the register budget of three waves keeps the compiler
// from issuing the V reads ahead of the P V products. The bf16 d = 64 kernels
// fit in 128 registers and may run four waves per SIMD (four work-groups per
// CU), which hides more latency on short sequences: 5% faster at N = 2048 and
// 8% at N = 1024, unchanged from N = 8192.
template <int D, bool CAUSAL, bool DROP, bool SPARSE, bool SPLIT, bool FP8, int NW = 4>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(1, ((D == 64 && !FP8) || NW == 16) ? 4 : 2))) void fwd_bf16_kernel(
    FwdParams p) {
  using C = FwdCfg<D, FP8, NW>;
  using KT = typename C::KT;
  using VT = typename C::VT;
  // Two stages of K and V tiles; separate arrays so that reads of one stage
  // only wait for the loads into that stage.
  __shared__ __align__(16) char st0[C::STAGE];
  __shared__ __align__(16) char st1[C::STAGE];
  __shared__ __align__(16) uint32_t ck0[DROP ? C::BN / 2 : 1];  // dropout keys of the tile's key pairs
  __shared__ __align__(16) uint32_t ck1[DROP ? C::BN / 2 : 1];
  __shared__ uint16_t kept[SPARSE ? kSparseMaxBlocks : 1];  // kept key blocks
  static_assert(!SPARSE || C::BM == kSparseBlock, "a work-group covers one mask row");
  static_assert(!(SPLIT && (SPARSE || DROP)), "split-KV runs without dropout or block masks");
  static_assert(!FP8 || (!SPLIT && !SPARSE && !DROP),
                "FP8 scores run without dropout, block masks or split-KV");
  constexpr int NK8 = (D + 63) / 64;  // FP8: 64-wide contraction steps of S^T = K Q^T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile decisions are scalar
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H;
  const int nqb = (p.N + C::BM - 1) / C::BM;
  int wgid = blockIdx.x, split = 0;
  if constexpr (SPLIT) {
    split = wgid % p.nsplit;
    wgid /= p.nsplit;
  }
  // Causal blocks: one per work-group (rank-major, or paired across the
  // work-groups of a CU), or with p.pair_blocks a complementary pair
  // (nqb - 1 - j, then j) per work-group, so that every work-group has the
  // same work and co-resident groups sweep the same K/V tiles in step.
  const bool paired = CAUSAL && !SPLIT && !SPARSE && p.pair_blocks;
  BlockMap bm;
  int qb_first = 0, qb_second = -1;
  if (paired) {
    bm = map_block_pair(wgid, (nqb + 1) / 2, p.B * H);
  } else {
    bm = (CAUSAL && !SPLIT && !SPARSE && p.pair_slots > 0)
             ? map_block_pairs(wgid, nqb, p.B * H, p.pair_slots, p.cus_per_xcd)
             : map_block(wgid, nqb, p.B * H);
    qb_first = CAUSAL ? (nqb - 1 - bm.rank) : bm.rank;
  }
  const int b = bm.bh / H, h = bm.bh - b * H;
  const SeqRows sr = seq_rows(p.cu, p.total, b, h, H, D, p.N);
  const int N = sr.n;             // query rows
  if (paired) {
    // Pairs of this sequence's own blocks (a packed batch's sequences have
    // their own block counts); pair indices past them have nothing to do.
    const int nb = (N + C::BM - 1) / C::BM;
    if (bm.rank >= (nb + 1) / 2) return;
    qb_first = nb - 1 - bm.rank;
    if (bm.rank < qb_first) qb_second = bm.rank;
  }
  const int Nk = SPLIT ? p.Nk : N;  // key rows
  // Causal: key j is visible to query i iff j <= i + coff; with Nk > N the
  // queries are the last N positions of the key sequence.
  const int coff = Nk - N;
  // rev: the key tiles in descending order (the second block of a pair).
  auto run_block = [&](const int qb, const bool rev) {
    const int q0 = qb * C::BM;
    if (q0 >= N) return;  // block past the end of a shorter sequence
    const int qw0 = q0 + wave * 32;
    const int myq = qw0 + l32;
    const int64_t rs = (int64_t)H * D;
    const int64_t base = sr.base;
    const int64_t kbase = SPLIT ? ((int64_t)b * Nk * H + h) * D : base;
    const uint16_t* Qg = p.q + base;
    const uint16_t* Vg = p.v + kbase;
    const uint32_t rs2 = (uint32_t)(H * D * 2);  // bytes between consecutive rows
    // K rows: bf16, or FP8 bytes (one byte per element).
    const char* Kb = FP8 ? reinterpret_cast<const char*>(p.k8 + kbase)
                         : reinterpret_cast<const char*>(p.k + kbase);
    const uint32_t rsk = FP8 ? (uint32_t)(H * D) : rs2;

    // Q operand (B of S^T = K Q^T): 8 d-values per lane per 16-wide chunk
    // (bf16), or 32 bytes per lane per 64-wide chunk (FP8, in qreg[2c],
    // qreg[2c+1]); rows >= N read as zeros through the buffer range check.
    u32x4 qreg[C::NKC];
    float qsc = 1.f;  // FP8: this query block's scale
    if constexpr (FP8) {
      const BufRes rq = rows_bufres(p.q8 + base, q0, N, C::BM, rsk);
  #pragma unroll
      for (int c = 0; c < NK8; ++c)
  #pragma unroll
        for (int u = 0; u < 2; ++u) {
          // chunks past D (D = 80) read as zeros through an out-of-range offset
          const int ch = 4 * c + 2 * hf + u;
          qreg[2 * c + u] = buf_load_128(rq, ch < KT::VALID ? (uint32_t)(myq - q0) * rsk + 16 * ch : 0x80000000u);
        }
      qsc = p.q_scale[((int64_t)b * H + h) * nqb + qb];
    } else {
      const BufRes rq = rows_bufres(Qg, q0, N, C::BM, rs2);
  #pragma unroll
      for (int c = 0; c < C::NKC; ++c)
        qreg[c] = buf_load_128(rq, (uint32_t)(myq - q0) * rs2 + (16 * c + 8 * hf) * 2);
    }
    // FP8: the key tiles' scales, one per 64 keys; the next tile's is loaded
    // with its tile (and so has arrived when that tile's loads have).
    const BufRes rks = make_bufres(FP8 ? p.k_scale + ((int64_t)b * H + h) * ((Nk + 63) / 64) : nullptr,
                                   FP8 ? (uint32_t)((Nk + 63) / 64) * 4 : 0u);
    float ksn = 1.f;

    uint64_t kbh = 0;
    uint32_t arow = 0;
    if constexpr (DROP) {
      kbh = head_key(p.seed, b, h, H);
      arow = row_key(kbh, myq);
    }

    const int kend = CAUSAL ? min(Nk, q0 + C::BM + coff) : Nk;
    int ntiles, tfirst = 0;
    if constexpr (SPLIT) {
      // This part's share of the key tiles: parts of equal tile counts.
      const int all = (kend + C::BN - 1) / C::BN;
      const int per = (all + p.nsplit - 1) / p.nsplit;
      tfirst = min(all, split * per);
      ntiles = min(all, tfirst + per) - tfirst;
    } else if constexpr (SPARSE) {
      // Kept key blocks of this query block, in ascending order.
      const int nb = (N + kSparseBlock - 1) / kSparseBlock;
      const uint8_t* mrow = p.bmask + b * p.msb + h * p.msh + (int64_t)qb * nb;
      const KeptBlocks kb =
          collect_blocks(mrow, 1, 0, (kend + kSparseBlock - 1) / kSparseBlock, kept, lane, wave == 0);
      ntiles = kept_tiles<C::BN>(kb, kend);
      __syncthreads();
    } else {
      ntiles = (kend + C::BN - 1) / C::BN;
    }
    auto tile_start = [&](int t) {
      if (rev) t = ntiles - 1 - t;
      return SPARSE ? kept_tile_start<C::BN>(kept, t) : (tfirst + t) * C::BN;
    };

    // This wave's share of the tile loads: K instructions first, then V.
    uint32_t dsrc[C::LPW];
    int dlds[C::LPW];
  #pragma unroll
    for (int m = 0; m < C::LPW; ++m) {
      const int i = (wave % C::NW) + C::NW * m;
      int off = 0, row = 0, ch = 0;
      if (i < KT::NLOAD) {
        KT::load_slot(i, lane, off, row, ch);
      } else if (i < C::NLOAD) {
        VT::load_slot(i - KT::NLOAD, lane, off, row, ch);
        off += KT::BYTES;
      }
      dsrc[m] = (uint32_t)row * (i < KT::NLOAD ? rsk : rs2) + 16 * ch;
      if constexpr (FP8) {
        // Chunks past D in a padded FP8 row: an offset beyond every buffer
        // range makes the load return zeros.
        if (i < KT::NLOAD && ch >= KT::VALID) dsrc[m] = 0x80000000u;
      }
      dlds[m] = off;
    }
    auto issue = [&](char* stage, uint32_t* ck, int k0) {
      // Resources start at row k0 and end at row N: rows past N arrive as zeros.
      const BufRes rk = rows_bufres(Kb, k0, Nk, C::BN, rsk);
      const BufRes rv = rows_bufres(Vg, k0, Nk, C::BN, rs2);
      if constexpr (FP8) ksn = buf_load_f32(rks, (uint32_t)(k0 >> 6) * 4);
  #pragma unroll
      for (int m = 0; m < C::LPW; ++m) {
        const int i = (wave % C::NW) + C::NW * m;
        if (i < C::NLOAD) lds_dma_16(i < KT::NLOAD ? rk : rv, stage + dlds[m], dsrc[m]);
      }
      if constexpr (DROP) {
        if (tid < C::BN / 2) ck[tid] = pair_key(kbh, (k0 >> 1) + tid);
      }
    };

    // Per-lane LDS offsets of the matrix-core operands (loop invariant).
    // K rows l32 (scores s0) and l32 + 32 (s1), chunk 2c + hf: the swizzle of
    // row l32 + 32 is that of row l32 with bit 2 flipped.
    const int xk = hf ^ KT::sw(l32);
    int ka[4] = {0, 0, 0, 0};
    int ktl = 0;
    if constexpr (!FP8) {
  #pragma unroll
      for (int u = 0; u < 4; ++u) ka[u] = l32 * 128 + (((2 * u) ^ xk) << 4);
      ktl = KT::TAIL + l32 * 32 + ((hf ^ KT::swt(l32)) << 4);
    }
    // FP8: 64-wide k-step c reads chunks 4c + 2hf + u (u = 0, 1) of rows l32
    // (fo) and l32 + 32 (fo2).
    int fo[NK8][2], fo2[NK8][2];
    if constexpr (FP8) {
  #pragma unroll
      for (int c = 0; c < NK8; ++c)
  #pragma unroll
        for (int u = 0; u < 2; ++u) {
          fo[c][u] = KT::off(l32, 4 * c + 2 * hf + u);
          fo2[c][u] = KT::off(l32 + 32, 4 * c + 2 * hf + u);
        }
    }
    // V: 16-lane group g reads rows 4(g/2) + j (+ 8h + 16kt), columns
    // 16(g%2) + 4a (+ 32db) for lane 4j + a of the group; the uniform part of
    // the swizzle selects one of four precomputed offsets.
    const int vg = lane >> 4, vj = (lane >> 2) & 3, va = lane & 3;
    const int vs = vg >> 1, vgh = vg & 1;
    const int vlp = (2 * vgh) ^ (va >> 1) ^ (2 * vj) ^ vs;
    int vaoff[4];
  #pragma unroll
    for (int u = 0; u < 4; ++u)
      vaoff[u] = KT::BYTES + (4 * vs + vj) * 128 + ((vlp ^ (2 * u)) << 4) + 8 * (va & 1);
    const int vtl = KT::BYTES + VT::TAIL + (4 * vs + vj) * 32 + 8 * va;

    // Running statistics in base-2 units of the scaled scores. The reference
    // max m only moves when a tile's max exceeds it by more than kLazy (then
    // O and l are rescaled); otherwise probabilities up to 2^kLazy are summed
    // against the old reference. O and l always share one reference, so the
    // final O / l and LSE are exact.
    constexpr float kLazy = 8.0f;
    const float c2 = p.c2;
    float m = -INFINITY, l = 0.f;
    f32x16 oacc[C::NDB];
  #pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16{};

    auto step = [&](const char* cur, const uint32_t* ckc, char* nxt, uint32_t* ckn, int t) {
      // Tile t has landed in `cur` once every wave's loads are done; after the
      // barrier nobody reads `nxt` any more, so the next tile can go there.
      wait_vmem();
      __syncthreads();
      if constexpr (kLdsPoison) poison_stage(nxt, C::STAGE, tid, C::NT);
      const int k0 = tile_start(t);
      // Exponent coefficient of this tile (FP8: times the two block scales).
      const float c2t = FP8 ? c2 * qsc * ksn : c2;
      if (t + 1 < ntiles) issue(nxt, ckn, tile_start(t + 1));
      if (CAUSAL && k0 > qw0 + 31 + coff) return;  // every key is after this wave's queries
      if (SPLIT && qw0 >= N) return;                // no query rows in this wave

      // S^T = K Q^T: lane = query, registers = keys (c_row layout).
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      if constexpr (FP8) {
  #pragma unroll
        for (int c = 0; c < NK8; ++c) {
          const u32x4 x0 = ld_lds_128(cur, fo[c][0]), x1 = ld_lds_128(cur, fo[c][1]);
          const u32x4 y0 = ld_lds_128(cur, fo2[c][0]), y1 = ld_lds_128(cur, fo2[c][1]);
          s0 = mfma32x32x64_fp8(x0, x1, qreg[2 * c], qreg[2 * c + 1], s0);
          s1 = mfma32x32x64_fp8(y0, y1, qreg[2 * c], qreg[2 * c + 1], s1);
        }
        sched_lds_ahead<NK8, 4, 2, 0, 1>();
      } else {
  #pragma unroll
      for (int c = 0; c < C::NKC; ++c) {
        int o0, o1;
        if (2 * c < 8 * KT::NG) {
          o0 = (c >> 2) * KT::GBYTES + ka[c & 3];
          o1 = (c >> 2) * KT::GBYTES + 4096 + ka[(c & 3) ^ 2];
        } else {
          o0 = ktl;
          o1 = ktl + 1024;
        }
        s0 = mfma32x32x16(ld_lds_128(cur, o0), qreg[c], s0);
        s1 = mfma32x32x16(ld_lds_128(cur, o1), qreg[c], s1);
      }
      sched_lds_ahead<C::NKC, 2, 2>();
      }
      if ((k0 + C::BN > Nk) || (CAUSAL && k0 + C::BN - 1 > qw0 + coff)) {
        const int lim = CAUSAL ? min(myq + coff, Nk - 1) : Nk - 1;  // last visible key
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + c_row(r, hf);
          s0[r] = key > lim ? -INFINITY : s0[r];
          s1[r] = key + 32 > lim ? -INFINITY : s1[r];
        }
      }
      float ma = fmaxf(s0[0], s0[1]), mb = fmaxf(s1[0], s1[1]);
  #pragma unroll
      for (int r = 2; r < 16; r += 2) {
        ma = fmaxf(fmaxf(ma, s0[r]), s0[r + 1]);
        mb = fmaxf(fmaxf(mb, s1[r]), s1[r + 1]);
      }
      const float mx = xor32_max(fmaxf(ma, mb)) * c2t;
      if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {
        const float mnew = fmaxf(m, mx);
        // Rows without a visible key so far (only in a split key range) have
        // l = 0 and O = 0: scale 0 instead of exp2(-inf - -inf).
        const float alpha = (SPLIT && m == -INFINITY) ? 0.f : exp2_hw(m - mnew);
        m = mnew;
        l *= alpha;
  #pragma unroll
        for (int db = 0; db < C::NDB; ++db) oacc[db] *= alpha;
      }
      // A part of a split key range can start with a tile in which some rows
      // see no key yet (m = -inf); they take reference 0 so that exp2 gives 0.
      const float nm = (SPLIT && m == -INFINITY) ? 0.f : -m;
  #pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = exp2_hw(fmaf(s0[r], c2t, nm));
        s1[r] = exp2_hw(fmaf(s1[r], c2t, nm));
      }
      if constexpr (DROP) {
        // l sums the probabilities before dropout.
        float ps0 = 0.f, ps1 = 0.f;
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          ps0 += s0[r];
          ps1 += s1[r];
        }
        l += ps0 + ps1;
        // Register 4g + e holds key 8g + 4hf + e: keys (e, e + 1) for e = 0, 2
        // are a pair and share one hash.
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 c0 = *reinterpret_cast<const u32x2*>(ckc + 4 * g + 2 * hf);
          const u32x2 c1 = *reinterpret_cast<const u32x2*>(ckc + 16 + 4 * g + 2 * hf);
  #pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const uint32_t y0 = pair_mix(arow, c0[e >> 1]);
            const uint32_t y1 = pair_mix(arow, c1[e >> 1]);
            s0[4 * g + e] = keep_even(y0, p.drop_t) ? s0[4 * g + e] : 0.f;
            s0[4 * g + e + 1] = keep_odd(y0, p.drop_t) ? s0[4 * g + e + 1] : 0.f;
            s1[4 * g + e] = keep_even(y1, p.drop_t) ? s1[4 * g + e] : 0.f;
            s1[4 * g + e + 1] = keep_odd(y1, p.drop_t) ? s1[4 * g + e + 1] : 0.f;
          }
        }
      }
      // P^T as the B operand, bf16, in 16-key steps; without dropout the row
      // sum is taken on these rounded values (v_dot2 with ones).
      u32x4 pop[4];
      float la = 0.f, lb = 0.f;
  #pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16& sv = (kt < 2) ? s0 : s1;
        const int rb = (kt & 1) * 8;
        pop[kt] = u32x4{pack_bf16x2(sv[rb + 0], sv[rb + 1]), pack_bf16x2(sv[rb + 2], sv[rb + 3]),
                        pack_bf16x2(sv[rb + 4], sv[rb + 5]), pack_bf16x2(sv[rb + 6], sv[rb + 7])};
        if constexpr (!DROP) {
  #pragma unroll
          for (int w = 0; w < 4; ++w) {
            float& acc = (w & 1) ? lb : la;
            acc = add_bf16_pair(pop[kt][w], acc);
          }
        }
      }
      if constexpr (!DROP) l += la + lb;
      // O^T += V^T P^T: V fragments by transposing reads (two per operand).
  #pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
  #pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          u32x2 v0, v1;
          if (4 * db < 8 * VT::NG) {
            const int gb = (db >> 1) * VT::GBYTES + 2048 * kt;
            const int u = 2 * ((db ^ kt) & 1);
            v0 = ld_lds_tr16(cur, gb + vaoff[u]);
            v1 = ld_lds_tr16(cur, gb + 1024 + vaoff[u + 1]);
          } else {
            v0 = ld_lds_tr16(cur, vtl + 512 * kt);
            v1 = ld_lds_tr16(cur, vtl + 512 * kt + 256);
          }
          const u32x4 aop = {v0[0], v0[1], v1[0], v1[1]};
          oacc[db] = mfma32x32x16(aop, pop[kt], oacc[db]);
        }
      }
    };

    if constexpr (kLdsPoison) poison_stage(st0, C::STAGE, tid, C::NT);
    if (ntiles > 0) issue(st0, ck0, tile_start(0));
    for (int t = 0; t < ntiles; t += 2) {
      step(st0, ck0, st1, ck1, t);
      if (t + 1 < ntiles) step(st1, ck1, st0, ck0, t + 1);
    }

    const float ltot = xor32_sum(l);
    if constexpr (SPLIT) {
      // Partial result of this key range, normalised by its own sum; a range
      // with no visible key gives O_s = 0 and LSE_s = -inf.
      if (myq < N) {
        const int64_t row = (((int64_t)split * p.B + b) * H + h) * N + myq;
        const float inv = ltot == 0.f ? 0.f : 1.f / ltot;
        float* orow = p.ws_o + row * D;
  #pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
  #pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = db * 32 + 8 * g + 4 * hf;
            if (d0 < D) {
              const f32x4 w = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                               oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
              *reinterpret_cast<f32x4*>(orow + d0) = w;
            }
          }
        }
        if (hf == 0) p.ws_lse[row] = ltot == 0.f ? -INFINITY : (m + log2_hw(ltot)) * kLn2;
      }
      return;
    }
    if (myq < N) {
      // A row whose blocks are all masked has no keys: O = 0, LSE = -inf.
      const float inv = (SPARSE && ltot == 0.f) ? 0.f : (DROP ? p.drop_r : 1.f) / ltot;
      uint16_t* orow = p.o + base + (int64_t)myq * rs;
  #pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * hf;
          if (d0 < D) {
            const u32x2 w = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                             pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
            st_global_64(orow + d0, w);
          }
        }
      }
      if (hf == 0) p.lse[sr.stat + myq] = (m + log2_hw(ltot)) * kLn2;
    }
  };
  run_block(qb_first, false);
  if (qb_second >= 0) {
    // The first block's last tile may still be read from a stage.
    __syncthreads();
    run_block(qb_second, true);
  }
}

// ---------------------------------------------------------------------------
// fp32 path on the fp32 matrix cores (v_mfma_f32_32x32x2_f32). A work-group
// of eight waves owns 32 query rows of one (batch, head); wave w takes the
// 32-key tiles w, w + 8, w + 16, ... of the key range, so that even a short
// sequence spreads over eight waves. Each wave keeps its own running max,
// sum and output (the online softmax of the bf16 path, rescaled on every
// tile) and reads its K and V rows from global memory straight into
// registers. At the end the eight partial results are merged through LDS in
// a fixed order: M = max_w m_w, O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w.
// Lanes as in the bf16 kernel: S^T = K Q^T with lane = query (both lane
// halves) and register r -> key c_row(r, half). Step c of the contraction
// takes dimension half * D/2 + c (relabelling the contraction index on both
// operands leaves the product unchanged), so a lane reads D/2 consecutive
// floats of its Q and K rows. P^T feeds O^T += V^T P^T directly: step c
// takes key c_row(c, half), whose probability is the lane's own register c.
struct FwdParamsF {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, H, N;
  const int* cu;
  int total;
  const uint8_t* bmask;
  int64_t msb, msh;
  float c2;
  uint32_t drop_t;
  float drop_r;
  uint64_t seed;
};

constexpr int kF32Waves = 8;  // waves per work-group (key tiles dealt round-robin)
constexpr int kF32Bm = 32;    // query rows per work-group

__device__ __forceinline__ f32x16 mfma32x32x2_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(64 * kF32Waves) void fwd_f32_kernel(FwdParamsF p) {
  constexpr int NW = kF32Waves, BM = kF32Bm, BN = 32, DH = D / 2;
  constexpr int NDB = (D + 31) / 32;
  __shared__ float red_m[NW][BM];
  __shared__ float red_l[NW][BM];
  __shared__ __align__(16) float red_o[NW][16][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H;
  const int nqb = (p.N + BM - 1) / BM;
  const BlockMap bm = map_block(blockIdx.x, nqb, p.B * H);
  const int qb = CAUSAL ? (nqb - 1 - bm.rank) : bm.rank;
  const int b = bm.bh / H, h = bm.bh - b * H;
  const SeqRows sr = seq_rows(p.cu, p.total, b, h, H, D, p.N);
  const int N = sr.n;
  const int q0 = qb * BM;
  if (q0 >= N) return;  // block past the end of a shorter sequence (whole work-group)
  const int myq = q0 + l32;
  const int64_t rs = (int64_t)H * D;
  const float* Qg = p.q + sr.base;
  const float* Kg = p.k + sr.base;
  const float* Vg = p.v + sr.base;

  // Buffer resources over this block's rows and each tile's rows: reads of
  // rows at or past N return zeros (hardware range check), so no load needs a
  // branch.
  const uint32_t rs4 = (uint32_t)rs * 4u;
  const BufRes rq = rows_bufres(Qg, q0, N, BM, rs4);
  // Rows per K/V resource window: the largest power of two with
  // win * rs4 <= 2^30 (rs4 <= 2^22 at the boundary, so win >= 128).
  const int win = 1 << (30 - (32 - __builtin_clz(rs4)));
  // This lane's query row, dimensions hf * DH .. hf * DH + DH - 1.
  float qf[DH];
#pragma unroll
  for (int c = 0; c < DH; c += 4) {
    const u32x4 x = buf_load_128(rq, (uint32_t)l32 * rs4 + (uint32_t)(hf * DH + c) * 4u);
    qf[c] = __uint_as_float(x[0]), qf[c + 1] = __uint_as_float(x[1]);
    qf[c + 2] = __uint_as_float(x[2]), qf[c + 3] = __uint_as_float(x[3]);
  }
  uint64_t kbh = 0;
  uint32_t arow = 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    arow = row_key(kbh, myq);
  }
  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  const uint8_t* mrow = nullptr;  // this query block's row of the block mask
  if (p.bmask != nullptr)
    mrow = p.bmask + b * p.msb + h * p.msh +
           (int64_t)(q0 / kSparseBlock) * ((N + kSparseBlock - 1) / kSparseBlock);

  float m = -INFINITY, l = 0.f;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  for (int t = wave; t < ntiles; t += NW) {
    const int k0 = t * BN;
    if (mrow != nullptr && mrow[k0 / kSparseBlock] == 0) continue;  // uniform over the wave
    // All of this tile's K and V loads are issued before its products, so
    // their latency is paid once. K: this lane's key row k0 + l32, the same
    // dimensions as its query row. V: step c of O^T += V^T P^T takes key
    // k0 + c_row(c, hf), column 32 db + l32 (columns past D, only for
    // D = 80, read zeros through an offset beyond the range).
    // K and V resources start at row kb, the start of the window of `win`
    // rows holding k0: offsets from there stay below 2^30 + 2^28 for slices
    // of any size, and in the usual case (the whole slice in one window,
    // kb = 0) they are the slice's own offsets, which depend on the tile and
    // are computed per tile rather than held across the loop.
    const int kb = k0 & -win, kr = k0 - kb;
    const BufRes rk = rows_bufres(Kg, kb, N, win + BN, rs4);
    const BufRes rv = rows_bufres(Vg, kb, N, win + BN, rs4);
    float kf[DH];
#pragma unroll
    for (int c = 0; c < DH; c += 4) {
      const u32x4 x = buf_load_128(rk, (uint32_t)(kr + l32) * rs4 + (uint32_t)(hf * DH + c) * 4u);
      kf[c] = __uint_as_float(x[0]), kf[c + 1] = __uint_as_float(x[1]);
      kf[c + 2] = __uint_as_float(x[2]), kf[c + 3] = __uint_as_float(x[3]);
    }
    float va[NDB][16];
    auto load_v = [&](int db) {
      const int col = 32 * db + l32;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint32_t off = (uint32_t)(kr + c_row(c, hf)) * rs4 + (uint32_t)col * 4u;
        va[db][c] = buf_load_f32(rv, col < D ? off : 0x80000000u);
      }
    };
    // At D = 128 the V loads are requested after the score products (the
    // K row's registers are free by then), still ahead of the softmax.
    constexpr int NEARLY = D == 128 ? 0 : NDB;
#pragma unroll
    for (int db = 0; db < NEARLY; ++db) load_v(db);
    __builtin_amdgcn_sched_barrier(0);  // the loads above stay ahead of the products
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < DH; ++c) s = mfma32x32x2_f32(kf[c], qf[c], s);
#pragma unroll
    for (int db = NEARLY; db < NDB; ++db) load_v(db);
    __builtin_amdgcn_sched_barrier(0);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + c_row(r, hf);
      float x = s[r] * p.c2;
      if (key >= N || (CAUSAL && key > myq)) x = -INFINITY;
      s[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = xor32_max(mx);
    const float mnew = fmaxf(m, mx);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = exp2_hw(m - mref);
    m = mnew;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = exp2_hw(s[r] - mref);
      ps += pv;
      s[r] = pv;
    }
    l = l * alpha + ps;  // this lane half's keys; the halves are added at the end
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    if constexpr (DROP) {
      // Lane j (j < 16) hashes the tile's key pair j; register r reads the
      // pair of its key (c_row(r, hf) >> 1) from that lane.
      const uint32_t pk = pair_key(kbh, (k0 >> 1) + (lane & 15));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ko = c_row(r, hf);
        const uint32_t y = pair_mix(arow, (uint32_t)__shfl((int)pk, ko >> 1));
        if (!keep_key(y, ko, p.drop_t)) s[r] = 0.f;
      }
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int c = 0; c < 16; ++c) o[db] = mfma32x32x2_f32(va[db][c], s[c], o[db]);
  }

  // Merge the eight waves' partial results in wave order.
  const float lw = xor32_sum(l);
  if (hf == 0) {
    red_m[wave][l32] = m;
    red_l[wave][l32] = lw;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][l32]);
  const float mref = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += red_l[w][l32] * exp2_hw(red_m[w][l32] - mref);
  const float sc = exp2_hw(m - mref);
  // A row whose blocks are all masked has no keys: O = 0, LSE = -inf.
  const float inv = L == 0.f ? 0.f : (DROP ? p.drop_r : 1.f) / L;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    if (db > 0) __syncthreads();  // the previous block's sums are read
#pragma unroll
    for (int r = 0; r < 16; ++r) red_o[wave][r][lane] = o[db][r] * sc;
    __syncthreads();
    if (wave < 4) {
      // wave g sums registers 4g .. 4g + 3: dimensions 32 db + 8g + 4hf + 0..3
      const int g = wave, d0 = 32 * db + 8 * g + 4 * hf;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += red_o[w][4 * g + e][lane];
      if (myq < N && d0 < D)
        *reinterpret_cast<f32x4*>(p.o + sr.base + (int64_t)myq * rs + d0) = acc * inv;
    }
  }
  if (wave == 0 && hf == 0 && myq < N) p.lse[sr.stat + myq] = (M + log2_hw(L)) * kLn2;
}

// Eight waves (256 query rows) per work-group share each K/V tile, which
// halves the tile loads and L2 reads per query row but leaves the waves of a
// group less balanced under the causal mask. Measured on MI355X, eight waves
// pay for head dims up to 80 from N = 8192 (d = 64: 16% faster at N = 8192;
// d = 80: 5% at N = 8192, 11% at N = 32768) and for the vector-ALU-bound
// dropout kernels at N >= 32768 (d = 128: 6% at N = 65536), and cost the
// d = 128 kernels without dropout 6-10% (N = 8192..32768; 6-8% at N = 8192
// in runs interleaved with the four-wave kernel).
template <int D, bool DROP>
bool fwd_eight_waves(int N) {
  return (D <= 80 && N >= 8192) || (DROP && N >= 32768);
}

// Sixteen waves (512 query rows, four waves per SIMD) from N = 32768 for
// head dims up to 80 without dropout, whose kernels fit in 128 registers:
// each K/V tile then serves twice the queries of the eight-wave group, which
// halves the K/V bytes fetched from beyond L2 (N = 32768 d = 80: 4.2 to
// 2.2 GB per launch, 2-2.5% faster). The d = 128 and dropout kernels need
// more than 128 registers and keep eight waves.
template <int D, bool DROP>
bool fwd_sixteen_waves(int N) {
  return D <= 80 && !DROP && N >= 32768;
}

// Launches a forward instance with the causal block pairing of
// plan_block_pairs (fa_launch.h): the descending sweep changes only the order
// of the online softmax's updates (results equal up to fp32 rounding order),
// and which work-group computes which block changes no result. Measured: the
// N = 32768 d = 80 forward fetches 0.52 GB per launch from beyond L2
// instead of 2.19 GB (the N = 8192 d = 128 one 0.25 GB instead of 0.82,
// but slower there, see below).
// A packed batch pairs each sequence's own blocks (the resident pairing
// across work-groups needs equal block counts and is not used there): the
// 16-sequence batch of 512..8192 tokens runs 12% faster.
template <auto Kernel>
hipError_t launch_fwd_grid(int nblocks, int threads, bool causal, const FwdParams& prm, hipStream_t s) {
  const int BH = prm.B * prm.H;
  // Pairs per work-group for packed batches and from N = 32768: measured
  // inside the benchmark's full training step (forward after the previous
  // step's backward), they made the N = 8192 d = 128 forward 3% slower
  // (0.514 against 0.497 ms), the N = 32768 d = 80 one 2% faster, the
  // N = 65536 dropout one no different, and the packed 16-sequence batch 6%
  // faster.
  const BlockPairing bp = plan_block_pairs<Kernel>(nblocks / BH, BH, threads, causal, prm.cu == nullptr,
                                                   prm.cu != nullptr || prm.N >= 32768);
  FwdParams p = prm;
  p.pair_slots = bp.pair_slots;
  p.cus_per_xcd = bp.cus_per_xcd;
  p.pair_blocks = bp.pair_blocks;
  hipLaunchKernelGGL(Kernel, dim3(bp.grid), dim3(threads), 0, s, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool DROP, bool SPARSE>
hipError_t launch_fwd_bf16_t(const FwdParams& prm, hipStream_t s) {
  // A block mask row covers 128 queries: block-sparse runs keep four waves.
  if constexpr (!SPARSE) {
    if constexpr (D <= 80 && !DROP) {  // the only instances built with sixteen waves
      if (fwd_sixteen_waves<D, DROP>(prm.N))
        return launch_fwd_grid<fwd_bf16_kernel<D, CAUSAL, DROP, SPARSE, false, false, 16>>(
            (prm.N + 511) / 512 * prm.B * prm.H, 1024, CAUSAL, prm, s);
    }
    if (fwd_eight_waves<D, DROP>(prm.N))
      return launch_fwd_grid<fwd_bf16_kernel<D, CAUSAL, DROP, SPARSE, false, false, 8>>(
          (prm.N + 255) / 256 * prm.B * prm.H, 512, CAUSAL, prm, s);
  }
  return launch_fwd_grid<fwd_bf16_kernel<D, CAUSAL, DROP, SPARSE, false, false, 4>>(
      (prm.N + 127) / 128 * prm.B * prm.H, 256, CAUSAL && !SPARSE, prm, s);
}

// Split-KV combine: for each query row, LSE = ln sum_s e^{LSE_s} and
// O = sum_s e^{LSE_s - LSE} O_s (the rescale of the online softmax applied
// across the parts). Sixteen lanes per row; bound by HBM bandwidth.
template <int D>
__global__ __launch_bounds__(256) void splitkv_combine_kernel(const float* __restrict__ ws_o,
                                                              const float* __restrict__ ws_lse,
                                                              uint16_t* __restrict__ o,
                                                              float* __restrict__ lse, int B,
                                                              int H, int N, int nsplit) {
  const int64_t rows = (int64_t)B * H * N;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // [b][h][q]
  const int sub = threadIdx.x & 15;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, ws_lse[sp * rows + row]);
  constexpr int PER = (D + 15) / 16;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float sum = 0.f;
  if (mx != -INFINITY) {
    for (int sp = 0; sp < nsplit; ++sp) {
      const float w = exp2_hw((ws_lse[sp * rows + row] - mx) * kLog2e);
      sum += w;
      const float* orow = ws_o + (sp * rows + row) * D;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (sub + 16 * j < D) acc[j] = fmaf(w, orow[sub + 16 * j], acc[j]);
    }
  }
  const int q = (int)(row % N);
  const int64_t bh = row / N;
  const int h = (int)(bh % H), b = (int)(bh / H);
  uint16_t* orow = o + (((int64_t)b * N + q) * H + h) * D;
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (sub + 16 * j < D) {
      const uint32_t w = pack_bf16x2(acc[j] * inv, 0.f);
      orow[sub + 16 * j] = (uint16_t)(w & 0xffffu);
    }
  }
  if (sub == 0) lse[row] = sum > 0.f ? mx + log2_hw(sum) * kLn2 : -INFINITY;
}

template <int D, bool SPARSE>
hipError_t launch_fwd_bf16_ds(const FwdParams& prm, bool causal, bool drop,
                              hipStream_t s) {
  if (causal)
    return drop ? launch_fwd_bf16_t<D, true, true, SPARSE>(prm, s)
                : launch_fwd_bf16_t<D, true, false, SPARSE>(prm, s);
  return drop ? launch_fwd_bf16_t<D, false, true, SPARSE>(prm, s)
              : launch_fwd_bf16_t<D, false, false, SPARSE>(prm, s);
}

template <int D>
hipError_t launch_fwd_bf16_d(const FwdParams& prm, bool causal, bool drop,
                             hipStream_t s) {
  return prm.bmask ? launch_fwd_bf16_ds<D, true>(prm, causal, drop, s)
                   : launch_fwd_bf16_ds<D, false>(prm, causal, drop, s);
}

template <int D, bool CAUSAL, bool DROP>
hipError_t launch_fwd_f32_t(const FwdParamsF& prm, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, DROP>), dim3(nblocks), dim3(64 * kF32Waves), 0, s,
                     prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_f32_d(const FwdParamsF& prm, bool causal, bool drop, int nblocks,
                            hipStream_t s) {
  if (causal)
    return drop ? launch_fwd_f32_t<D, true, true>(prm, nblocks, s)
                : launch_fwd_f32_t<D, true, false>(prm, nblocks, s);
  return drop ? launch_fwd_f32_t<D, false, true>(prm, nblocks, s)
              : launch_fwd_f32_t<D, false, false>(prm, nblocks, s);
}

}  // namespace

hipError_t launch_forward_bf16(const AttnArgs& a, hipStream_t s) {
  FwdParams prm{};
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.k = static_cast<const uint16_t*>(a.k);
  prm.v = static_cast<const uint16_t*>(a.v);
  prm.o = static_cast<uint16_t*>(a.o_out);
  prm.lse = a.lse_out;
  prm.B = a.B;
  prm.H = a.H;
  prm.N = a.N;
  prm.cu = a.cu_seqlens;
  prm.total = a.total;
  prm.bmask = a.block_mask;
  prm.msb = a.mask_stride_b;
  prm.msh = a.mask_stride_h;
  prm.Nk = a.N;
  prm.nsplit = 1;
  prm.ws_o = nullptr;
  prm.ws_lse = nullptr;
  prm.c2 = a.scale * kLog2e;
  prm.drop_t = a.drop_threshold;
  prm.drop_r = a.drop_rescale;
  prm.seed = a.seed;
  switch (a.d) {
    case 64: return launch_fwd_bf16_d<64>(prm, a.causal, a.dropout, s);
    case 80: return launch_fwd_bf16_d<80>(prm, a.causal, a.dropout, s);
    case 128: return launch_fwd_bf16_d<128>(prm, a.causal, a.dropout, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward_splitkv_bf16(const AttnArgs& a, hipStream_t s) {
  FwdParams prm{};
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.k = static_cast<const uint16_t*>(a.k);
  prm.v = static_cast<const uint16_t*>(a.v);
  prm.o = nullptr;
  prm.lse = nullptr;
  prm.B = a.B;
  prm.H = a.H;
  prm.N = a.N;
  prm.cu = nullptr;
  prm.total = 0;
  prm.bmask = nullptr;
  prm.Nk = a.Nk;
  prm.nsplit = a.num_splits;
  prm.ws_o = a.split_o;
  prm.ws_lse = a.split_lse;
  prm.c2 = a.scale * kLog2e;
  const int nqb = (a.N + 127) / 128;
  const dim3 grid((unsigned)(nqb * a.B * a.H * a.num_splits)), block(256);
#define FA_SPLIT(D)                                                                          \
  case D:                                                                                    \
    if (a.causal)                                                                            \
      hipLaunchKernelGGL((fwd_bf16_kernel<D, true, false, false, true, false>), grid, block, 0, s,  \
                         prm);                                                               \
    else                                                                                     \
      hipLaunchKernelGGL((fwd_bf16_kernel<D, false, false, false, true, false>), grid, block, 0, s, \
                         prm);                                                               \
    break;
  switch (a.d) {
    FA_SPLIT(64)
    FA_SPLIT(80)
    FA_SPLIT(128)
    default: return hipErrorInvalidValue;
  }
#undef FA_SPLIT
  FA_HIP_RETURN_IF(hipGetLastError());
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const dim3 cgrid((unsigned)((rows + 15) / 16));
  uint16_t* o = static_cast<uint16_t*>(a.o_out);
  switch (a.d) {
    case 64:
      hipLaunchKernelGGL((splitkv_combine_kernel<64>), cgrid, block, 0, s, a.split_o, a.split_lse,
                         o, a.lse_out, a.B, a.H, a.N, a.num_splits);
      break;
    case 80:
      hipLaunchKernelGGL((splitkv_combine_kernel<80>), cgrid, block, 0, s, a.split_o, a.split_lse,
                         o, a.lse_out, a.B, a.H, a.N, a.num_splits);
      break;
    default:
      hipLaunchKernelGGL((splitkv_combine_kernel<128>), cgrid, block, 0, s, a.split_o,
                         a.split_lse, o, a.lse_out, a.B, a.H, a.N, a.num_splits);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-block FP8 quantisation ("FlashAttention for Efficient Training", section
// 6.2 "Quantization and Mixed-Precision Approaches": scores from quantised
// queries and keys with scaling factors). One work-group per (b, h, block of
// R rows): amax = max |x| over the block, codes = E4M3(x * (448 / amax)) with
// round-to-nearest-even (v_cvt_pk_fp8_f32), scale = amax / 448 (1 for an
// all-zero block), so that x ~ scale * code.
template <int D, int R>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ x,
                                                           uint8_t* __restrict__ xq,
                                                           float* __restrict__ scales, int N,
                                                           int H) {
  // Work in 16-element chunks (32 bytes in, 16 bytes out): chunk c of the
  // block is row c / CPR, columns 16 (c % CPR) ..; thread t takes chunks
  // t, t + 256, ...
  constexpr int CPR = D / 16;
  constexpr int NCH = R * CPR;
  constexpr int PER = (NCH + 255) / 256;
  __shared__ float wmax[4];
  const int nblk = (N + R - 1) / R;
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int b = bh / H, h = bh - b * H;
  u32x4 v[PER][2];
  int64_t off[PER];
  bool ok[PER];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    const int row = blk * R + c / CPR;
    ok[i] = c < NCH && row < N;
    off[i] = (((int64_t)b * N + row) * H + h) * D + 16 * (c % CPR);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v[i][j] = ok[i] ? ld_global_128(x + off[i] + 8 * j) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i][j][e])), fabsf(bf16_hi(v[i][j][e]))));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = amax > 0.f ? 448.f / amax : 1.f;
  if (threadIdx.x == 0) scales[(int64_t)bh * nblk + blk] = amax > 0.f ? amax / 448.f : 1.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (!ok[i]) continue;
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // output word q: elements 4q .. 4q + 3
      const uint32_t e0 = v[i][q / 2][2 * (q & 1)], e1 = v[i][q / 2][2 * (q & 1) + 1];
      int t = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(e0) * inv, bf16_hi(e0) * inv, 0, false);
      t = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(e1) * inv, bf16_hi(e1) * inv, t, true);
      w[q] = (uint32_t)t;
    }
    *reinterpret_cast<u32x4*>(xq + off[i]) = w;
  }
}

template <int D>
void launch_quantize_fp8_d(const uint16_t* xs, uint8_t* xq, float* scales, int N, int H,
                           int block_rows, dim3 grid, hipStream_t s) {
  if (block_rows == 128)
    hipLaunchKernelGGL((quantize_fp8_kernel<D, 128>), grid, dim3(256), 0, s, xs, xq, scales, N, H);
  else
    hipLaunchKernelGGL((quantize_fp8_kernel<D, 64>), grid, dim3(256), 0, s, xs, xq, scales, N, H);
}

hipError_t launch_quantize_fp8(const void* x, uint8_t* xq, float* scales, int B, int N, int H,
                               int d, int block_rows, hipStream_t s) {
  if (block_rows != 128 && block_rows != 64) return hipErrorInvalidValue;
  const int nblk = (N + block_rows - 1) / block_rows;
  const dim3 grid((unsigned)(nblk * B * H));
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  switch (d) {
    case 64: launch_quantize_fp8_d<64>(xs, xq, scales, N, H, block_rows, grid, s); break;
    case 80: launch_quantize_fp8_d<80>(xs, xq, scales, N, H, block_rows, grid, s); break;
    case 128: launch_quantize_fp8_d<128>(xs, xq, scales, N, H, block_rows, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_forward_fp8(const AttnArgs& a, hipStream_t s) {
  FwdParams prm{};
  prm.q = nullptr;
  prm.k = nullptr;
  prm.v = static_cast<const uint16_t*>(a.v);
  prm.o = static_cast<uint16_t*>(a.o_out);
  prm.lse = a.lse_out;
  prm.B = a.B;
  prm.H = a.H;
  prm.N = a.N;
  prm.cu = nullptr;
  prm.total = 0;
  prm.bmask = nullptr;
  prm.Nk = a.N;
  prm.nsplit = 1;
  prm.q8 = static_cast<const uint8_t*>(a.q);
  prm.k8 = static_cast<const uint8_t*>(a.k);
  prm.q_scale = a.q_scale;
  prm.k_scale = a.k_scale;
  prm.c2 = a.scale * kLog2e;
  const dim3 grid((unsigned)(((a.N + 127) / 128) * a.B * a.H)), block(256);
#define FA_FP8(D)                                                                            \
  case D:                                                                                    \
    if (a.causal)                                                                            \
      hipLaunchKernelGGL((fwd_bf16_kernel<D, true, false, false, false, true>), grid, block, 0, \
                         s, prm);                                                            \
    else                                                                                     \
      hipLaunchKernelGGL((fwd_bf16_kernel<D, false, false, false, false, true>), grid, block, \
                         0, s, prm);                                                         \
    break;
  switch (a.d) {
    FA_FP8(64)
    FA_FP8(80)
    FA_FP8(128)
    default: return hipErrorInvalidValue;
  }
#undef FA_FP8
  return hipGetLastError();
}

hipError_t launch_forward_f32(const AttnArgs& a, hipStream_t s) {
  FwdParamsF prm;
  prm.q = static_cast<const float*>(a.q);
  prm.k = static_cast<const float*>(a.k);
  prm.v = static_cast<const float*>(a.v);
  prm.o = static_cast<float*>(a.o_out);
  prm.lse = a.lse_out;
  prm.B = a.B;
  prm.H = a.H;
  prm.N = a.N;
  prm.cu = a.cu_seqlens;
  prm.total = a.total;
  prm.bmask = a.block_mask;
  prm.msb = a.mask_stride_b;
  prm.msh = a.mask_stride_h;
  prm.c2 = a.scale * kLog2e;
  prm.drop_t = a.drop_threshold;
  prm.drop_r = a.drop_rescale;
  prm.seed = a.seed;
  const int nqb = (a.N + kF32Bm - 1) / kF32Bm;
  const int nblocks = nqb * a.B * a.H;
  switch (a.d) {
    case 64: return launch_fwd_f32_d<64>(prm, a.causal, a.dropout, nblocks, s);
    case 80: return launch_fwd_f32_d<80>(prm, a.causal, a.dropout, nblocks, s);
    case 128: return launch_fwd_f32_d<128>(prm, a.causal, a.dropout, nblocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
