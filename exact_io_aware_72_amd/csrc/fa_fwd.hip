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
#include "fa_hash.h"
#include "fa_kernels.h"

namespace fa {
namespace {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, H, N;
  float c2;  // scale * log2(e)
  uint32_t drop_t;
  float drop_r;
  uint64_t seed;
};

template <int D, bool DROP>
struct FwdCfg {
  static constexpr int NT = 256;                 // 4 waves
  static constexpr int BM = 128;                 // query rows per work-group
  static constexpr int BN = 64;                  // keys per tile
  static constexpr int NKC = D / 16;             // k-steps of S^T = K Q^T
  static constexpr int DP = (D + 31) / 32 * 32;  // rows of O^T computed (d padded to 32)
  static constexpr int NDB = DP / 32;
  static constexpr int KCH = D / 8;              // 16-byte chunks per row
  static constexpr int KS = (D + 8) * 2;         // LDS bytes per K row (padded)
  static constexpr int VS = (BN + 8) * 2;        // LDS bytes per V^T row (padded)
  static constexpr int KBYTES = BN * KS;
  static constexpr int VBYTES = DP * VS;
  static constexpr int BUF = KBYTES + VBYTES + (DROP ? BN * 4 : 0);
  static constexpr int K_ITEMS = BN * KCH;
  static constexpr int K_PER_T = (K_ITEMS + NT - 1) / NT;
  static constexpr int V_ITEMS = (BN / 4) * KCH;
  static constexpr int V_PER_T = (V_ITEMS + NT - 1) / NT;
};

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(FwdParams p) {
  using C = FwdCfg<D, DROP>;
  __shared__ __align__(16) char smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile decisions are scalar
  const int l32 = lane & 31, hf = lane >> 5;
  const int N = p.N, H = p.H;
  const int nqb = (N + C::BM - 1) / C::BM;
  const BlockMap bm = map_block(blockIdx.x, nqb, p.B * H);
  const int qb = CAUSAL ? (nqb - 1 - bm.rank) : bm.rank;
  const int b = bm.bh / H, h = bm.bh - b * H;
  const int q0 = qb * C::BM;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + l32;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * N * H + h) * D;
  const uint16_t* Qg = p.q + base;
  const uint16_t* Kg = p.k + base;
  const uint16_t* Vg = p.v + base;

  // Rows d >= D of the transposed V tiles only feed discarded output rows;
  // clear them once so they hold finite values.
  if constexpr (C::DP > D) {
    constexpr int PAD16 = (C::DP - D) * C::VS / 16;
    for (int i = tid; i < 2 * PAD16; i += C::NT) {
      const int bsel = i / PAD16, j = i - bsel * PAD16;
      st_lds_128(smem + bsel * C::BUF + C::KBYTES + D * C::VS, j * 16, u32x4{0, 0, 0, 0});
    }
  }

  // Buffer resources over this head's rows: reads of rows >= N return zeros.
  const uint32_t rs2 = (uint32_t)(H * D * 2);  // bytes between consecutive rows
  const BufRes rq = make_bufres(Qg, (uint32_t)N * rs2);
  const BufRes rk = make_bufres(Kg, (uint32_t)N * rs2);
  const BufRes rv = make_bufres(Vg, (uint32_t)N * rs2);

  // Q operand (B of S^T = K Q^T): 8 d-values per lane per 16-wide chunk.
  u32x4 qreg[C::NKC];
#pragma unroll
  for (int c = 0; c < C::NKC; ++c) qreg[c] = buf_load_128(rq, (uint32_t)myq * rs2 + (16 * c + 8 * hf) * 2);

  uint64_t kbh = 0;
  uint32_t arow = 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    arow = row_key(kbh, myq);
  }

  const int kend = CAUSAL ? min(N, q0 + C::BM) : N;
  const int ntiles = (kend + C::BN - 1) / C::BN;

  // Staging registers. Key rows past N read as zeros: their scores are
  // masked to -inf and their V rows meet zero probabilities.
  u32x4 kst[C::K_PER_T];
  u32x4 vst[C::V_PER_T][4];
  uint32_t bst = 0;

  auto load_tile = [&](int k0) {
    const uint32_t koff = (uint32_t)k0 * rs2;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int item = tid + i * C::NT;
      if (C::K_ITEMS % C::NT == 0 || item < C::K_ITEMS) {
        const int r = item / C::KCH, c = item - r * C::KCH;
        kst[i] = buf_load_128(rk, koff + (uint32_t)r * rs2 + 16 * c);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int item = tid + i * C::NT;
      if (C::V_ITEMS % C::NT == 0 || item < C::V_ITEMS) {
        const StageItem si = stage_item(item, C::BN / 4, C::KCH);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vst[i][j] = buf_load_128(rv, koff + (uint32_t)(4 * si.g + j) * rs2 + 16 * si.c);
      }
    }
    if constexpr (DROP) {
      if (tid < C::BN) bst = col_key(kbh, k0 + tid);
    }
  };
  auto store_tile = [&](char* buf) {
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int item = tid + i * C::NT;
      if (C::K_ITEMS % C::NT == 0 || item < C::K_ITEMS) {
        const int r = item / C::KCH, c = item - r * C::KCH;
        st_lds_128(buf, r * C::KS + c * 16, kst[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int item = tid + i * C::NT;
      if (C::V_ITEMS % C::NT == 0 || item < C::V_ITEMS) {
        const StageItem si = stage_item(item, C::BN / 4, C::KCH);
        st_lds_transpose4x8(buf + C::KBYTES, C::VS, 8 * si.c, perm_pos4(si.g), vst[i][0], vst[i][1],
                            vst[i][2], vst[i][3]);
      }
    }
    if constexpr (DROP) {
      if (tid < C::BN) *reinterpret_cast<uint32_t*>(buf + C::KBYTES + C::VBYTES + tid * 4) = bst;
    }
  };

  load_tile(0);
  store_tile(smem);
  __syncthreads();

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

  for (int t = 0; t < ntiles; ++t) {
    const char* buf = smem + (t & 1) * C::BUF;
    const int k0 = t * C::BN;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(k0 + C::BN);
    if (!CAUSAL || k0 <= qw0 + 31) {
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int c = 0; c < C::NKC; ++c) {
        const int col = (16 * c + 8 * hf) * 2;
        s0 = mfma32x32x16(ld_lds_128(buf, l32 * C::KS + col), qreg[c], s0);
        s1 = mfma32x32x16(ld_lds_128(buf, (32 + l32) * C::KS + col), qreg[c], s1);
      }
      if ((k0 + C::BN > N) || (CAUSAL && k0 + C::BN - 1 > qw0)) {
        const int lim = CAUSAL ? min(myq, N - 1) : N - 1;  // last visible key
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + c_row(r, hf);
          s0[r] = key > lim ? -INFINITY : s0[r];
          s1[r] = key + 32 > lim ? -INFINITY : s1[r];
        }
      }
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = xor32_max(mx) * c2;
      if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {
        const float mnew = fmaxf(m, mx);
        const float alpha = exp2_hw(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) oacc[db] *= alpha;
      }
      const float nm = -m;
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = exp2_hw(fmaf(s0[r], c2, nm));
        s1[r] = exp2_hw(fmaf(s1[r], c2, nm));
        ps0 += s0[r];
        ps1 += s1[r];
      }
      l += ps0 + ps1;
      if constexpr (DROP) {
        const char* bk = buf + C::KBYTES + C::VBYTES;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 c0 = ld_lds_u32x4(bk, (8 * g + 4 * hf) * 4);
          const u32x4 c1 = ld_lds_u32x4(bk, (32 + 8 * g + 4 * hf) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s0[4 * g + e] = keep(arow, c0[e], p.drop_t) ? s0[4 * g + e] : 0.f;
            s1[4 * g + e] = keep(arow, c1[e], p.drop_t) ? s1[4 * g + e] : 0.f;
          }
        }
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16& sv = (kt < 2) ? s0 : s1;
        const int rb = (kt & 1) * 8;
        const u32x4 bop = {pack_bf16x2(sv[rb + 0], sv[rb + 1]), pack_bf16x2(sv[rb + 2], sv[rb + 3]),
                           pack_bf16x2(sv[rb + 4], sv[rb + 5]), pack_bf16x2(sv[rb + 6], sv[rb + 7])};
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
          oacc[db] = mfma32x32x16(
              ld_lds_128(buf, C::KBYTES + (db * 32 + l32) * C::VS + (16 * kt + 8 * hf) * 2), bop,
              oacc[db]);
      }
    }
    if (more) store_tile(smem + ((t + 1) & 1) * C::BUF);
    __syncthreads();
  }

  const float ltot = xor32_sum(l);
  if (myq < N) {
    const float inv = (DROP ? p.drop_r : 1.f) / ltot;
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
    if (hf == 0) p.lse[((int64_t)b * H + h) * N + myq] = (m + log2_hw(ltot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: the same tiled online softmax on the vector ALUs, two threads
// per query row (each owns half of the head dimension). Used for fp32 inputs,
// where the bf16 matrix cores do not apply.
struct FwdParamsF {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, H, N;
  float c2;
  uint32_t drop_t;
  float drop_r;
  uint64_t seed;
};

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(128) void fwd_f32_kernel(FwdParamsF p) {
  constexpr int BM = 64, BN = 16, DH = D / 2;
  __shared__ __align__(16) float ks[BN][D];
  __shared__ __align__(16) float vs[BN][D];
  __shared__ uint32_t bk[BN];

  const int tid = threadIdx.x;
  const int qi = tid >> 1, part = tid & 1;
  const int N = p.N, H = p.H;
  const int nqb = (N + BM - 1) / BM;
  const BlockMap bm = map_block(blockIdx.x, nqb, p.B * H);
  const int qb = CAUSAL ? (nqb - 1 - bm.rank) : bm.rank;
  const int b = bm.bh / H, h = bm.bh - b * H;
  const int q0 = qb * BM;
  const int myq = q0 + qi;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)b * N * H + h) * D;

  float qv[DH], ov[DH];
  {
    const bool ok = myq < N;
    const float* qrow = p.q + base + (int64_t)(ok ? myq : 0) * rs + part * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      qv[c] = ok ? qrow[c] : 0.f;
      ov[c] = 0.f;
    }
  }
  uint64_t kbh = 0;
  uint32_t arow = 0;
  if constexpr (DROP) {
    kbh = head_key(p.seed, b, h, H);
    arow = row_key(kbh, myq);
  }
  const int kend = CAUSAL ? min(N, q0 + BM) : N;
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int i = tid; i < BN * D / 4; i += 128) {
      const int r = i / (D / 4), c = (i - r * (D / 4)) * 4;
      const int key = k0 + r;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < N) {
        kx = *reinterpret_cast<const f32x4*>(p.k + base + (int64_t)key * rs + c);
        vx = *reinterpret_cast<const f32x4*>(p.v + base + (int64_t)key * rs + c);
      }
      *reinterpret_cast<f32x4*>(&ks[r][c]) = kx;
      *reinterpret_cast<f32x4*>(&vs[r][c]) = vx;
    }
    if constexpr (DROP) {
      if (tid < BN) bk[tid] = col_key(kbh, k0 + tid);
    }
    __syncthreads();
    float s[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) acc = fmaf(qv[c], ks[j][part * DH + c], acc);
      acc += __shfl_xor(acc, 1);
      float x = acc * p.c2;
      const int key = k0 + j;
      if (key >= N || (CAUSAL && key > myq)) x = -INFINITY;
      s[j] = x;
      mx = fmaxf(mx, x);
    }
    const float mnew = fmaxf(m, mx);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = exp2_hw(m - mref);
    m = mnew;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float pv = exp2_hw(s[j] - mref);
      psum += pv;
      s[j] = pv;
      if constexpr (DROP) {
        if (!keep(arow, bk[j], p.drop_t)) s[j] = 0.f;
      }
    }
    l = l * alpha + psum;
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      float acc = ov[c] * alpha;
#pragma unroll
      for (int j = 0; j < BN; ++j) acc = fmaf(s[j], vs[j][part * DH + c], acc);
      ov[c] = acc;
    }
  }
  if (myq < N) {
    const float inv = (DROP ? p.drop_r : 1.f) / l;
    float* orow = p.o + base + (int64_t)myq * rs + part * DH;
#pragma unroll
    for (int c = 0; c < DH; ++c) orow[c] = ov[c] * inv;
    if (part == 0) p.lse[((int64_t)b * H + h) * N + myq] = (m + log2_hw(l)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool DROP>
hipError_t launch_fwd_bf16_t(const FwdParams& prm, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, DROP>), dim3(nblocks), dim3(256), 0, s, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_bf16_d(const FwdParams& prm, bool causal, bool drop, int nblocks,
                             hipStream_t s) {
  if (causal)
    return drop ? launch_fwd_bf16_t<D, true, true>(prm, nblocks, s)
                : launch_fwd_bf16_t<D, true, false>(prm, nblocks, s);
  return drop ? launch_fwd_bf16_t<D, false, true>(prm, nblocks, s)
              : launch_fwd_bf16_t<D, false, false>(prm, nblocks, s);
}

template <int D, bool CAUSAL, bool DROP>
hipError_t launch_fwd_f32_t(const FwdParamsF& prm, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, DROP>), dim3(nblocks), dim3(128), 0, s, prm);
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
  FwdParams prm;
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.k = static_cast<const uint16_t*>(a.k);
  prm.v = static_cast<const uint16_t*>(a.v);
  prm.o = static_cast<uint16_t*>(a.o_out);
  prm.lse = a.lse_out;
  prm.B = a.B;
  prm.H = a.H;
  prm.N = a.N;
  prm.c2 = a.scale * kLog2e;
  prm.drop_t = a.drop_threshold;
  prm.drop_r = a.drop_rescale;
  prm.seed = a.seed;
  const int nqb = (a.N + 127) / 128;
  const int nblocks = nqb * a.B * a.H;
  switch (a.d) {
    case 64: return launch_fwd_bf16_d<64>(prm, a.causal, a.dropout, nblocks, s);
    case 80: return launch_fwd_bf16_d<80>(prm, a.causal, a.dropout, nblocks, s);
    case 128: return launch_fwd_bf16_d<128>(prm, a.causal, a.dropout, nblocks, s);
    default: return hipErrorInvalidValue;
  }
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
  prm.c2 = a.scale * kLog2e;
  prm.drop_t = a.drop_threshold;
  prm.drop_r = a.drop_rescale;
  prm.seed = a.seed;
  const int nqb = (a.N + 63) / 64;
  const int nblocks = nqb * a.B * a.H;
  switch (a.d) {
    case 64: return launch_fwd_f32_d<64>(prm, a.causal, a.dropout, nblocks, s);
    case 80: return launch_fwd_f32_d<80>(prm, a.causal, a.dropout, nblocks, s);
    case 128: return launch_fwd_f32_d<128>(prm, a.causal, a.dropout, nblocks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
