// Kept-row projection, rotary embedding at original positions and KV emission.
//
// Above the gate only the kept tokens are processed and pruned tokens create no KV
// entries (aiproducthub.cn "斯坦福伯克利TokenGate 预填充提速11.3倍", section 事件详情;
// aisight.pl "TokenGate: Stanford i Berkeley ...", section "Jak to dziala";
// news.chathome.org TokenGate article, section "TokenGate の学習可能なトークンプルーニングの
// 仕組み").  This is the step right after the gather:
//     C = X_kept W_qkv^T (+ b)          W_qkv rows: Hq query heads, Hkv key heads, Hkv value heads
//     q, k rotated by pos_j (rotate-half: feature i pairs with i + d/2, angle pos theta^(-2i/d))
//     q -> q_out[j];  k, v, pos -> caches at slot0 + j (the cache holds the kept tokens only)
//
// Two kernels:
//  * rope_table: cos / sin of pos_j theta^(-2i/d) for every kept row and frequency.  The
//    angle reaches 1.3e5 rad at 128k positions, far beyond what a float32 product keeps
//    (its rounding alone would be 0.008 rad), so the angle is formed and reduced modulo
//    2 pi in float64 and only the reduced angle goes through a float32 sincos.  The same
//    launch writes the positions into the position cache;
//  * qkv_rope: a bf16 GEMM on v_mfma_f32_32x32x16_bf16 computed transposed, C^T[feature,
//    token] = W . X^T, so each lane of a 32x32 accumulator holds one token and 16 features.
//    A workgroup (8 waves) owns 256 features x BT tokens; each wave owns 128 features
//    (one head of 128 or two of 64) x 32 BTW tokens, so a feature i and its rotation
//    partner i + d/2 sit in the same lane and register of two accumulator tiles and the
//    rotation is element-wise in registers.  Both operands stream through an NS-stage
//    LDS ring by DMA (64-wide k-chunks, 128-byte rows XOR-swizzled by (row >> 1) & 7 so
//    the operand reads are conflict-free); the epilogue adds the bias, rotates q and k
//    with the table and writes bf16 rows through LDS, so each row leaves as whole lines.  The
//    tile grid is dealt to the XCDs in blocks that minimise the operand tiles each XCD's L2
//    must fetch.
#include <atomic>
#include <type_traits>

#include "tg_common.h"

namespace tg {

constexpr int kQkvWaves = 8;
constexpr int kQkvKC = 64;                  // k elements per stage
constexpr int kQkvRow = kQkvKC * 2;         // bytes per row per stage
constexpr int kQkvFeat = 256;               // features per workgroup
constexpr double kTwoPiHi = 6.283185307179586;          // 2 pi rounded to double
constexpr double kTwoPiLo = 2.4492935982947064e-16;     // 2 pi - kTwoPiHi

__device__ __forceinline__ int qkv_swz(int row) { return (row >> 1) & 7; }

// ---------------------------------------------------------------------------------
// rotation table: tab[j * (D/2) + i] = (cos, sin)(pos_j theta^(-2i/D))
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void rope_table_kernel(int m, const int32_t* __restrict__ pos, double log2_theta,
                                                         float2* __restrict__ tab, int32_t* __restrict__ pos_cache,
                                                         int64_t slot0) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)m * (D / 2)) return;
  const int tok = (int)(idx / (D / 2)), i = (int)(idx % (D / 2));
  const int32_t p = pos[tok];
  const double inv = exp2(-(2.0 * i / D) * log2_theta);
  const double ang = (double)p * inv;
  const double k = rint(ang * (1.0 / kTwoPiHi));
  double r = fma(-k, kTwoPiHi, ang);        // exact up to one rounding of a value below ~pi
  r = fma(-k, kTwoPiLo, r);
  float sr, cr;
  sincosf((float)r, &sr, &cr);
  tab[idx] = make_float2(cr, sr);
  if (i == 0 && pos_cache) pos_cache[slot0 + tok] = p;
}

template <int BTW, int NS>
struct QkvTile {
  static constexpr int F = kQkvFeat, AT = 4, WH = 2, WT = kQkvWaves / WH, BT = 32 * BTW * WT;
  static constexpr int WB = F * kQkvRow, XB = BT * kQkvRow, STAGE = WB + XB;
  static constexpr int WI = WB / 1024 / kQkvWaves, XI = XB / 1024 / kQkvWaves;   // DMAs per wave per stage
  static_assert(WI >= 1 && XI >= 1, "stage split over the waves");
  static_assert(NS * STAGE <= 160 * 1024, "LDS");
};

// 4 bf16 of one row: C values (lo) and their partners d/2 further (hi), rotated or not
__device__ __forceinline__ void store4(uint16_t* row, int i0, int half_d, const float* lo, const float* hi) {
  const u32x2 a = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
  const u32x2 b = {pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
  *reinterpret_cast<u32x2*>(row + i0) = a;
  *reinterpret_cast<u32x2*>(row + half_d + i0) = b;
}

template <int D, int BTW, int NS>
__global__ __launch_bounds__(kQkvWaves * 64, 1) void qkv_rope_kernel(
    int m, int d_model, const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, int n_feat, int hq, int hkv, const float2* __restrict__ tab,
    uint16_t* __restrict__ q_out, uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, int64_t slot0,
    int n_ft, int n_tt, int fb) {
  using T = QkvTile<BTW, NS>;
  constexpr int BT = T::BT, AT = T::AT, WT = T::WT;
  constexpr int HT = D / 64;                 // 32-wide accumulator tiles per half head
  constexpr int HPW = 128 / D;               // heads per wave
  // the ring, reused after the main loop as each wave's output staging area
  constexpr int SROWS = 32 * BTW, SPITCH = 128 * 2 + 16;   // 16 bytes of padding per row
  constexpr int RING = NS * T::STAGE, STAGING = kQkvWaves * SROWS * SPITCH;
  __shared__ __attribute__((aligned(16))) char ring[RING > STAGING ? RING : STAGING];
  const uint32_t lds0 = lds_addr(ring);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  // wave -> (feature half, token slice): the waves of one token slice sit on different
  // SIMDs, so a ragged last token tile (only its first slices hold tokens) costs less
  const int wh = wave % T::WH, wt = wave / T::WH;

  // workgroup -> (feature tile, token tile).  The dispatcher sends consecutive workgroups to
  // the 8 XCDs in turn, and an XCD runs about 32 of them at once (one per CU), which share
  // its L2.  With fb > 0 the tile grid is cut into blocks of fb feature tiles x 32 / fb
  // token tiles and each block goes whole to one XCD: its 32 workgroups fetch fb + 32 / fb
  // operand tiles (12 for fb = 4) instead of the 18 of 2 feature tiles x 16 token tiles.
  // Otherwise (grids too small to give every XCD two blocks), with n_ft a multiple of 8,
  // each XCD only ever sees n_ft / 8 feature tiles while the token tiles stream past.
  int ft, tt;
  if (fb > 0) {
    const int tb = 32 / fb, n_fb = n_ft / fb;
    const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const int blk = (j / 32) * 8 + xcd, loc = j % 32;
    ft = (blk % n_fb) * fb + loc % fb;
    tt = (blk / n_fb) * tb + loc / fb;
    if (blk >= n_fb * ((n_tt + tb - 1) / tb) || tt >= n_tt) return;   // padding of the last blocks
  } else if (n_ft % 8 == 0) {
    const int per = n_ft / 8, xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    ft = xcd * per + j % per;
    tt = j / per;
  } else {
    ft = blockIdx.x % n_ft;
    tt = blockIdx.x / n_ft;
  }
  const int f0 = ft * kQkvFeat, tok0 = tt * BT;
  // waves whose tokens or features all lie past the end skip the products (they still
  // share the loads and barriers)
  const bool busy = tok0 + 32 * BTW * wt < m && f0 + 128 * wh < n_feat;

  // DMA j of this wave fills rows 8 (I wave + j) + lane/8 of the W (or X) stage; the lane
  // writes physical chunk lane%8 of its row, which holds logical chunk (lane%8) ^ swz(row).
  // Rows past the end re-read the last row (their results are never stored).
  uint32_t wo[T::WI], wm[T::WI], xo[T::XI], xm[T::XI];
#pragma unroll
  for (int j = 0; j < T::WI; ++j) {
    const int r = 8 * (T::WI * wave + j) + lane / 8;
    const int rf = min(f0 + r, n_feat - 1) - f0;
    wo[j] = (uint32_t)(((int64_t)rf * d_model + 8 * ((lane % 8) ^ qkv_swz(r))) * 2);
    wm[j] = (uint32_t)((T::WI * wave + j) * 1024);
  }
#pragma unroll
  for (int j = 0; j < T::XI; ++j) {
    const int r = 8 * (T::XI * wave + j) + lane / 8;
    const int64_t rt = min(tok0 + r, m - 1) - tok0;
    xo[j] = (uint32_t)((rt * ldx + 8 * ((lane % 8) ^ qkv_swz(r))) * 2);
    xm[j] = (uint32_t)(T::WB + (T::XI * wave + j) * 1024);
  }
  const char* wg = reinterpret_cast<const char*>(w) + (int64_t)f0 * d_model * 2;
  const char* xg = reinterpret_cast<const char*>(x) + (int64_t)tok0 * ldx * 2;
  auto issue = [&](int c, int slot) {
#pragma unroll
    for (int j = 0; j < T::WI; ++j) dma_lds16(wo[j], wg + c * kQkvRow, lds0 + slot * T::STAGE + wm[j]);
#pragma unroll
    for (int j = 0; j < T::XI; ++j) dma_lds16(xo[j], xg + c * kQkvRow, lds0 + slot * T::STAGE + xm[j]);
  };

  uint32_t oa[kQkvKC / 16];
#pragma unroll
  for (int ks = 0; ks < kQkvKC / 16; ++ks) oa[ks] = (uint32_t)(l32 * kQkvRow + 16 * ((2 * ks + half) ^ qkv_swz(l32)));

  f32x16 acc[AT][BTW];
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BTW; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int nch = d_model / kQkvKC;
#pragma unroll
  for (int c = 0; c < NS - 1; ++c)
    if (c < nch) issue(c, c);

  auto step = [&](int c, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
    constexpr int per_chunk = T::WI + T::XI;
    // chunk c has landed once at most min(NS - 2, nch - 1 - c) later chunks are outstanding
    const int later = min(NS - 2, nch - 1 - c);
    if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NS > 3 ? 2 * per_chunk : 0) : "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NS > 2 ? per_chunk : 0) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // chunk c visible to all waves; chunk c - 1's slot free for reuse
    if (c + NS - 1 < nch) issue(c + NS - 1, (slot + NS - 1) % NS);
    if (!busy) return;
    const char* st = ring + slot * T::STAGE;
    // operands of k-step ks + 1 are read before the products of k-step ks (two register sets),
    // scheduling fences keeping them there
    constexpr int NKS = kQkvKC / 16;
    bf16x8 af[2][AT], bfr[2][BTW];
    auto load = [&](int ks, int buf) {
#pragma unroll
      for (int a = 0; a < AT; ++a)
        af[buf][a] = *reinterpret_cast<const bf16x8*>(st + oa[ks] + 32 * kQkvRow * (wh * AT + a));
#pragma unroll
      for (int b = 0; b < BTW; ++b)
        bfr[buf][b] = *reinterpret_cast<const bf16x8*>(st + T::WB + oa[ks] + 32 * kQkvRow * (wt * BTW + b));
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 1 < NKS) load(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BTW; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][a], bfr[ks & 1][b], acc[a][b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int c = 0; c < nch; c += NS) {   // unrolled by NS so the stage slot is a constant
    step(c, std::integral_constant<int, 0>{});
    if (NS > 1 && c + 1 < nch) step(c + 1, std::integral_constant<int, 1 % NS>{});
    if (NS > 2 && c + 2 < nch) step(c + 2, std::integral_constant<int, 2 % NS>{});
    if (NS > 3 && c + 3 < nch) step(c + 3, std::integral_constant<int, 3 % NS>{});
  }

  // epilogue: tile (a, b) holds token tok0 + 32 (wt BTW + b) + l32 and features
  // fw + 32 a + 8 g + 4 half + r (register 4 g + r), fw = the wave's first feature.
  // Results go through LDS so that each output row leaves as whole 16-byte-per-lane
  // lines (8-byte scattered stores left partly written lines for L2 to evict).
  const int fw = f0 + 128 * wh;
  __syncthreads();   // every wave is done with the ring
  if (fw >= n_feat) return;
  char* stage = ring + wave * SROWS * SPITCH;
  uint16_t* dst[HPW];
  int64_t stride[HPW];                                // elements between consecutive tokens
#pragma unroll
  for (int hp = 0; hp < HPW; ++hp) {
    const int hg = (fw + hp * D) / D;                 // head over the q | k | v concatenation
    const bool rotate = hg < hq + hkv;
    if (hg < hq) {
      dst[hp] = q_out + (int64_t)hg * D;
      stride[hp] = (int64_t)hq * D;
    } else if (hg < hq + hkv) {
      dst[hp] = k_cache + (slot0 * hkv + (hg - hq)) * D;
      stride[hp] = (int64_t)hkv * D;
    } else {
      dst[hp] = v_cache + (slot0 * hkv + (hg - hq - hkv)) * D;
      stride[hp] = (int64_t)hkv * D;
    }
    const float* hb = bias ? bias + (int64_t)hg * D : nullptr;
#pragma unroll
    for (int b = 0; b < BTW; ++b) {
      const int tok = tok0 + 32 * (wt * BTW + b) + l32;
      const int tc = min(tok, m - 1);
      const float2* trow = tab + (int64_t)tc * (D / 2);
      char* srow = stage + (32 * b + l32) * SPITCH + hp * D * 2;
#pragma unroll
      for (int at = 0; at < HT; ++at) {
        const int alo = hp * 2 * HT + at, ahi = alo + HT;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int i0 = 32 * at + 8 * g + 4 * half;   // feature in the first half of the head
          float lo[4], hi[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            lo[r] = acc[alo][b][4 * g + r];
            hi[r] = acc[ahi][b][4 * g + r];
          }
          if (hb) {
            const f32x4 bl = *reinterpret_cast<const f32x4*>(hb + i0);
            const f32x4 bh = *reinterpret_cast<const f32x4*>(hb + D / 2 + i0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              lo[r] += bl[r];
              hi[r] += bh[r];
            }
          }
          if (rotate) {
            const f32x4 cs01 = *reinterpret_cast<const f32x4*>(trow + i0);
            const f32x4 cs23 = *reinterpret_cast<const f32x4*>(trow + i0 + 2);
            const float c[4] = {cs01[0], cs01[2], cs23[0], cs23[2]};
            const float sn[4] = {cs01[1], cs01[3], cs23[1], cs23[3]};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float a = lo[r], e = hi[r];
              lo[r] = fmaf(a, c[r], -e * sn[r]);
              hi[r] = fmaf(e, c[r], a * sn[r]);
            }
          }
          store4(reinterpret_cast<uint16_t*>(srow), i0, D / 2, lo, hi);
        }
      }
    }
  }
  // copy-out: 16 lanes per token row of the wave's 128 features, 4 rows per instruction
  const int c16 = lane & 15, f = 8 * c16, hp = f / D, fi = f % D;
  uint16_t* drow = dst[0];
  int64_t dstride = stride[0];
#pragma unroll
  for (int h = 1; h < HPW; ++h)
    if (hp == h) { drow = dst[h]; dstride = stride[h]; }
#pragma unroll
  for (int j = 0; j < SROWS / 4; ++j) {
    const int r = 4 * j + (lane >> 4);
    const int tok = tok0 + 32 * wt * BTW + r;
    const u32x4 val = *reinterpret_cast<const u32x4*>(stage + r * SPITCH + 16 * c16);
    if (tok < m) *reinterpret_cast<u32x4*>(drow + (int64_t)tok * dstride + fi) = val;
  }
}

template <int D, int BTW, int NS>
static tg_status launch_qkv(int m, int d_model, const void* x, int64_t ldx, const void* w, const float* bias,
                            int hq, int hkv, const float2* tab, void* q_out, void* k_cache, void* v_cache,
                            int64_t slot0, hipStream_t st) {
  constexpr int BT = QkvTile<BTW, NS>::BT;
  const int n_feat = (hq + 2 * hkv) * D;
  const int n_ft = (n_feat + kQkvFeat - 1) / kQkvFeat;
  const int n_tt = (m + BT - 1) / BT;
  // XCD blocks (see the kernel) when every XCD gets at least two of them
  const int fb = n_ft % 4 == 0 ? 4 : (n_ft % 2 == 0 ? 2 : 1);
  const int64_t n_blocks = (int64_t)(n_ft / fb) * ((n_tt + 32 / fb - 1) / (32 / fb));
  const bool blocked = n_blocks >= 16;
  const int64_t grid = blocked ? 8 * 32 * ((n_blocks + 7) / 8) : (int64_t)n_ft * n_tt;
  if (grid > INT32_MAX) return TG_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((qkv_rope_kernel<D, BTW, NS>), dim3((unsigned)grid), dim3(kQkvWaves * 64), 0, st, m, d_model,
                     static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(w), bias, n_feat, hq, hkv,
                     tab, static_cast<uint16_t*>(q_out), static_cast<uint16_t*>(k_cache),
                     static_cast<uint16_t*>(v_cache), slot0, n_ft, n_tt, blocked ? fb : 0);
  TG_CHECK_LAUNCH();
  return TG_OK;
}

// Workgroups of the 256-token projection kernel that the current device runs at once
// (cached per device; 0 if unknown).
template <int D>
static int qkv_slots() {
  static std::atomic<int> cache[64];
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= 64) return 0;
  int v = cache[device].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(qkv_rope_kernel<D, 2, 2>),
                                                   kQkvWaves * 64, 0) != hipSuccess)
    return 0;
  v = cus * per_cu;
  cache[device].store(v, std::memory_order_relaxed);
  return v;
}

template <int D>
static tg_status qkv_rope(int m, int d_model, const void* x, int64_t ldx, const void* w, const float* bias, int hq,
                          int hkv, const int32_t* pos, float theta, void* q_out, void* k_cache, void* v_cache,
                          int32_t* pos_cache, int64_t slot0, float2* tab, hipStream_t st) {
  const int64_t n_tab = (int64_t)m * (D / 2);
  hipLaunchKernelGGL((rope_table_kernel<D>), dim3((unsigned)((n_tab + 255) / 256)), dim3(256), 0, st, m, pos,
                     std::log2((double)theta), tab, pos_cache, slot0);
  TG_CHECK_LAUNCH();
  // A ragged last token tile of r rows keeps only ceil(r / 64) of its four token slices busy
  // and costs about half a full tile.  When it would run in a round of its own (the full
  // tiles fill whole rounds of the chip, or leave too little room beside them), its rows go
  // to a second launch of 128-token tiles, whose waves hold 32 tokens each: twice the busy
  // waves at half the work each.
  constexpr int BT = QkvTile<2, 2>::BT;
  const int r = m % BT, full = m / BT;
  bool split = false;
  if (full > 0 && r > 0 && r <= BT / 2) {
    const int64_t n_ft = ((int64_t)(hq + 2 * hkv) * D + kQkvFeat - 1) / kQkvFeat;
    const int64_t f = n_ft * full, slots = qkv_slots<D>();
    if (slots > 0 && f >= slots) split = f % slots == 0 || f % slots + n_ft > slots;
  }
  if (!split) return launch_qkv<D, 2, 2>(m, d_model, x, ldx, w, bias, hq, hkv, tab, q_out, k_cache, v_cache, slot0, st);
  const int m0 = m - r;
  const tg_status s0 =
      launch_qkv<D, 2, 2>(m0, d_model, x, ldx, w, bias, hq, hkv, tab, q_out, k_cache, v_cache, slot0, st);
  if (s0 != TG_OK) return s0;
  return launch_qkv<D, 1, 3>(r, d_model, static_cast<const uint16_t*>(x) + (int64_t)m0 * ldx, ldx, w, bias, hq, hkv,
                             tab + (int64_t)m0 * (D / 2), static_cast<uint16_t*>(q_out) + (int64_t)m0 * hq * D,
                             k_cache, v_cache, slot0 + m0, st);
}

static size_t rope_table_bytes(int64_t m, int64_t head_dim) {
  return ((size_t)m * (size_t)(head_dim / 2) * sizeof(float2) + 255) & ~size_t(255);
}

}  // namespace tg

extern "C" size_t tg_qkv_rope_workspace_bytes(int64_t m, int32_t head_dim) {
  if (m < 0 || m > INT32_MAX || head_dim <= 0) return 0;
  return tg::rope_table_bytes(m, head_dim);
}

extern "C" tg_status tg_qkv_rope(int32_t dtype, int64_t m, int32_t d_model, const void* x_kept, int64_t ldx,
                                 const void* w_qkv, const float* b_qkv, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, const int32_t* pos, float rope_theta, void* q_out, void* k_cache,
                                 void* v_cache, int32_t* pos_cache, int64_t cache_slot0, int64_t cache_capacity,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  using namespace tg;
  if (dtype != TG_F32 && dtype != TG_BF16) return TG_ERR_INVALID_ARG;
  if (m < 0 || m > INT32_MAX || d_model <= 0 || ldx < d_model || n_q_heads <= 0 || n_kv_heads <= 0 ||
      head_dim <= 0)
    return TG_ERR_INVALID_ARG;
  if (!std::isfinite(rope_theta) || !(rope_theta > 1.0f)) return TG_ERR_INVALID_ARG;
  if (cache_slot0 < 0 || cache_capacity < 0 || cache_slot0 > cache_capacity - m) return TG_ERR_INVALID_ARG;
  if (dtype != TG_BF16 || (head_dim != 64 && head_dim != 128)) return TG_ERR_UNSUPPORTED;
  const int64_t n_feat = (int64_t)(n_q_heads + 2 * (int64_t)n_kv_heads) * head_dim;
  if (n_feat % 128 != 0 || n_feat > INT32_MAX) return TG_ERR_UNSUPPORTED;
  if (d_model % kQkvKC != 0 || ldx % 8 != 0) return TG_ERR_UNSUPPORTED;
  // 32-bit DMA offsets within one tile: 256 weight rows and 256 token rows
  if ((int64_t)kQkvFeat * d_model * 2 > INT32_MAX || (int64_t)kQkvFeat * ldx * 2 > INT32_MAX) return TG_ERR_UNSUPPORTED;
  if (m == 0) return TG_OK;
  if (!x_kept || !w_qkv || !pos || !q_out || !k_cache || !v_cache || !workspace) return TG_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return TG_ERR_INVALID_ARG;
  if (workspace_bytes < rope_table_bytes(m, head_dim)) return TG_ERR_WORKSPACE;
  const uintptr_t align = reinterpret_cast<uintptr_t>(x_kept) | reinterpret_cast<uintptr_t>(w_qkv) |
                          reinterpret_cast<uintptr_t>(q_out) | reinterpret_cast<uintptr_t>(k_cache) |
                          reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(b_qkv);
  if (align & 15u) return TG_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float2* tab = static_cast<float2*>(workspace);
  const int mm = static_cast<int>(m);
  return head_dim == 128
             ? qkv_rope<128>(mm, d_model, x_kept, ldx, w_qkv, b_qkv, n_q_heads, n_kv_heads, pos, rope_theta, q_out,
                             k_cache, v_cache, pos_cache, cache_slot0, tab, st)
             : qkv_rope<64>(mm, d_model, x_kept, ldx, w_qkv, b_qkv, n_q_heads, n_kv_heads, pos, rope_theta, q_out,
                            k_cache, v_cache, pos_cache, cache_slot0, tab, st);
}
