// Gate scorer: s[i] = b2 + sum_j w2[j] * GELU(b1[j] + x[i,:] . w1[j,:]).
//
// The MLP gate of TokenGate (aiproducthub.cn "斯坦福伯克利TokenGate 预填充提速11.3倍",
// section 事件详情; aisight.pl "TokenGate: Stanford i Berkeley ...", section
// "Jak to dziala") scores each token's post-attention residual with a small MLP.
//
// bf16 path: one workgroup of 8 waves owns BT tokens and ALL d_hidden units, so
// the GELU and the 1-wide w2 dot finish inside the workgroup (no partial hidden
// activations ever reach memory).  The product is computed transposed,
// C^T[hidden, token] = W1 . X^T, on v_mfma_f32_32x32x16_bf16: each lane of a
// 32x32 accumulator then holds one token and 16 hidden units, so the epilogue
// reduction over hidden units is mostly in-register.  Both operands are staged
// through LDS in k-chunks of 64 (double-buffered); X streams from HBM once and
// W1 (<= 1 MiB) is re-read from L2 by every workgroup.
#include <type_traits>

#include "tg_common.h"

namespace tg {

// GELU(h) = h * Phi(h), Phi the standard normal CDF.  Phi comes from the rational
// approximation of erfc in Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (|error| <= 1.5e-7 on erfc): for a = |h|/sqrt(2) >= 0,
//   erfc(a) ~= (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-a^2),  t = 1/(1 + p a),
// and Phi(h) = 1 - erfc(a)/2 for h >= 0, erfc(a)/2 for h < 0.  In float32 the GELU
// error stays below 4e-7 absolute.  This costs ~12 VALU ops and two transcendentals
// (rcp, exp2) per value and keeps few registers live.
__device__ __forceinline__ float gelu_exact(float h) {
  constexpr float p_over_sqrt2 = 0.3275911f * 0.70710678118654752f;
  constexpr float a1 = 0.5f * 0.254829592f, a2 = 0.5f * -0.284496736f, a3 = 0.5f * 1.421413741f,
                  a4 = 0.5f * -1.453152027f, a5 = 0.5f * 1.061405429f;   // halved: q = erfc/2
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(h), p_over_sqrt2, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float q = poly * __builtin_amdgcn_exp2f(h * h * (-0.5f * kLog2e));   // = erfc(|h|/sqrt2)/2
  const float hq = h * q;
  return h >= 0.0f ? h - hq : hq;
}

// ---------------------------------------------------------------------------------
// float32 path (small shapes): thread j of the block owns hidden unit j.
// ---------------------------------------------------------------------------------
constexpr int kF32Toks = 8;
constexpr int kF32KC = 256;

__global__ __launch_bounds__(256) void score_f32_kernel(int n, int d_model, int d_hidden,
                                                        const float* __restrict__ x, int64_t ldx,
                                                        const float* __restrict__ w1,
                                                        const float* __restrict__ b1,
                                                        const float* __restrict__ w2, float b2,
                                                        float* __restrict__ scores) {
  __shared__ float xs[kF32Toks][kF32KC];
  __shared__ float red[kF32Toks][4];
  const int t0 = blockIdx.x * kF32Toks;
  const int j = threadIdx.x;
  float acc[kF32Toks];
#pragma unroll
  for (int r = 0; r < kF32Toks; ++r) acc[r] = 0.f;

  for (int k0 = 0; k0 < d_model; k0 += kF32KC) {
    const int kc = min(kF32KC, d_model - k0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < kF32Toks * kF32KC; idx += 256) {
      const int r = idx / kF32KC, c = idx % kF32KC;
      xs[r][c] = (t0 + r < n && c < kc) ? x[(int64_t)(t0 + r) * ldx + k0 + c] : 0.f;
    }
    __syncthreads();
    if (j < d_hidden) {
      const float* wr = w1 + (int64_t)j * d_model + k0;
      for (int c = 0; c < kc; ++c) {
        const float w = wr[c];
#pragma unroll
        for (int r = 0; r < kF32Toks; ++r) acc[r] = fmaf(xs[r][c], w, acc[r]);
      }
    }
  }
  const float bb = (j < d_hidden && b1) ? b1[j] : 0.f;
  const float ww = (j < d_hidden) ? w2[j] : 0.f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < kF32Toks; ++r) {
    float v = (j < d_hidden) ? ww * gelu_exact(acc[r] + bb) : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[r][wave] = v;
  }
  __syncthreads();
  if (threadIdx.x < kF32Toks && t0 + threadIdx.x < n) {
    const int r = threadIdx.x;
    scores[t0 + r] = b2 + ((red[r][0] + red[r][1]) + (red[r][2] + red[r][3]));
  }
}

// ---------------------------------------------------------------------------------
// bf16 path
// ---------------------------------------------------------------------------------
constexpr int kScoreWaves = 8;
constexpr int kScoreKC = 64;              // k-chunk staged per step
constexpr int kScorePitch = kScoreKC + 8; // LDS row pitch in bf16 (144 B: conflict-free b128 reads)

template <int H, int BTW>
struct ScoreTile {
  static constexpr int HT = H / 32;               // 32-row hidden tiles in total
  // hidden tiles per wave: 4 where they divide evenly (128, 256), 3 for 192, else all
  static constexpr int AT = HT % 4 == 0 ? 4 : (HT % 3 == 0 ? 3 : HT);
  static constexpr int WH = HT / AT;              // waves along hidden
  static constexpr int WT = kScoreWaves / WH;     // waves along tokens
  static constexpr int BT = 32 * BTW * WT;        // tokens per workgroup
  static constexpr int W_PIECES = H * (kScoreKC / 8);   // 16-byte pieces of a W1 chunk
  static constexpr int X_PIECES = BT * (kScoreKC / 8);
  static constexpr int W_PER_T = W_PIECES / (kScoreWaves * 64);
  static constexpr int X_PER_T = X_PIECES / (kScoreWaves * 64);
  static_assert(HT % AT == 0 && kScoreWaves % WH == 0, "tile shape");
  static_assert(W_PIECES % (kScoreWaves * 64) == 0 && X_PIECES % (kScoreWaves * 64) == 0, "pieces");
};

template <int H, int BTW>
__global__ __launch_bounds__(kScoreWaves * 64) void score_bf16_kernel(
    int n, int d_model, const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ w1,
    const float* __restrict__ b1, const uint16_t* __restrict__ w2, float b2, float* __restrict__ scores) {
  using T = ScoreTile<H, BTW>;
  constexpr int BT = T::BT, AT = T::AT, WT = T::WT;
  __shared__ __attribute__((aligned(16))) uint16_t lw[2][H][kScorePitch];
  __shared__ __attribute__((aligned(16))) uint16_t lx[2][BT][kScorePitch];
  __shared__ __attribute__((aligned(16))) float w2f[H];
  __shared__ __attribute__((aligned(16))) float b1f[H];
  __shared__ float red[T::WH][BT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wh = wave / WT, wt = wave % WT;
  const int tok0 = blockIdx.x * BT;

  for (int i = tid; i < H; i += kScoreWaves * 64) {
    w2f[i] = bf16_to_f32(w2[i]);
    b1f[i] = b1 ? b1[i] : 0.f;
  }

  // global -> register staging of one k-chunk
  u32x4 wreg[T::W_PER_T], xreg[T::X_PER_T];
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::W_PER_T; ++i) {
      const int p = tid + i * kScoreWaves * 64;
      const int row = p / (kScoreKC / 8), c = p % (kScoreKC / 8);
      wreg[i] = *reinterpret_cast<const u32x4*>(w1 + (int64_t)row * d_model + k0 + c * 8);
    }
#pragma unroll
    for (int i = 0; i < T::X_PER_T; ++i) {
      const int p = tid + i * kScoreWaves * 64;
      const int row = p / (kScoreKC / 8), c = p % (kScoreKC / 8);
      const int tok = tok0 + row;
      xreg[i] = (tok < n) ? *reinterpret_cast<const u32x4*>(x + (int64_t)tok * ldx + k0 + c * 8)
                          : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < T::W_PER_T; ++i) {
      const int p = tid + i * kScoreWaves * 64;
      const int row = p / (kScoreKC / 8), c = p % (kScoreKC / 8);
      *reinterpret_cast<u32x4*>(&lw[buf][row][c * 8]) = wreg[i];
    }
#pragma unroll
    for (int i = 0; i < T::X_PER_T; ++i) {
      const int p = tid + i * kScoreWaves * 64;
      const int row = p / (kScoreKC / 8), c = p % (kScoreKC / 8);
      *reinterpret_cast<u32x4*>(&lx[buf][row][c * 8]) = xreg[i];
    }
  };

  f32x16 acc[AT][BTW];
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BTW; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int nchunks = d_model / kScoreKC;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nchunks) load_chunk((ch + 1) * kScoreKC);
#pragma unroll
    for (int ks = 0; ks < kScoreKC / 16; ++ks) {
      bf16x8 af[AT], bfr[BTW];
#pragma unroll
      for (int a = 0; a < AT; ++a)
        af[a] = *reinterpret_cast<const bf16x8*>(&lw[buf][32 * (wh * AT + a) + l32][16 * ks + 8 * half]);
#pragma unroll
      for (int b = 0; b < BTW; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8*>(&lx[buf][32 * (wt * BTW + b) + l32][16 * ks + 8 * half]);
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BTW; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
    if (ch + 1 < nchunks) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds token (32*(wt*BTW+b) + l32) and hidden units
  // 32*(wh*AT+a) + 8*g + 4*half + r  (g = 0..3, r = 0..3) of tile (a, b)
  float part[BTW];
#pragma unroll
  for (int b = 0; b < BTW; ++b) part[b] = 0.f;
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int hid = 32 * (wh * AT + a) + 8 * g + 4 * half;
      const f32x4 ww = *reinterpret_cast<const f32x4*>(&w2f[hid]);
      const f32x4 bb = *reinterpret_cast<const f32x4*>(&b1f[hid]);
#pragma unroll
      for (int b = 0; b < BTW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[b] = fmaf(ww[r], gelu_exact(acc[a][b][4 * g + r] + bb[r]), part[b]);
    }
#pragma unroll
  for (int b = 0; b < BTW; ++b) {
    part[b] += swap_halves(part[b]);
    if (half == 0) red[wh][32 * (wt * BTW + b) + l32] = part[b];
  }
  __syncthreads();
  for (int t = tid; t < BT; t += kScoreWaves * 64) {
    if (tok0 + t < n) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < T::WH; ++w) s += red[w][t];
      scores[tok0 + t] = s + b2;
    }
  }
}

template <int H, int BTW>
static tg_status launch_score_bf16(int n, int d_model, const void* x, int64_t ldx, const void* w1,
                                   const float* b1, const void* w2, float b2, float* scores,
                                   hipStream_t stream) {
  constexpr int BT = ScoreTile<H, BTW>::BT;
  const int grid = (n + BT - 1) / BT;
  hipLaunchKernelGGL((score_bf16_kernel<H, BTW>), dim3(grid), dim3(kScoreWaves * 64), 0, stream, n,
                     d_model, static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(w1),
                     b1, static_cast<const uint16_t*>(w2), b2, scores);
  TG_CHECK_LAUNCH();
  return TG_OK;
}


// ---------------------------------------------------------------------------------
// bf16 path, d_hidden 256: the same tile (all 256 hidden units x BT tokens per
// workgroup, C^T = W1 . X^T on 32x32x16 MFMA) fed through an NS-stage LDS ring by
// DMA (global_load_lds, 16 bytes per lane).  A stage holds a 64-wide k-chunk: every
// row segment is one whole 128-byte line, and up to NS - 1 chunks are in flight while
// one is consumed.  X is read exactly once, so its DMAs carry the non-temporal cache
// policy (W1's, re-read by every workgroup, do not): 163 -> 154 us at 131072 tokens,
// 45 -> 43 us at 32768 and 28.5 -> 24.8 us at 16384, the same scores.  The DMA is issued
// from inline asm so that the compiler does not
// make the operand reads wait for it; the kernel waits for exactly the chunk it
// needs (s_waitcnt vmcnt) and publishes it with one barrier per chunk.  Rows are
// 128 bytes; their 16-byte chunks are XOR-swizzled by (row >> 1) & 7, which makes
// the b128 operand reads bank-conflict free and keeps each lane's operand address
// fixed for the whole loop (rows 32 i + l32 share the swizzle of l32).
// ---------------------------------------------------------------------------------
constexpr int kRingKC = 64;                 // k elements per stage
constexpr int kRingRow = kRingKC * 2;       // bytes per row per stage
__device__ __forceinline__ int ring_swz(int row) { return (row >> 1) & 7; }

// WH waves split the 256 hidden units (AT 32-unit tiles each), the other kScoreWaves / WH
// split the tokens (BTW 32-token tiles each).
template <int BTW, int NS, int WH_ = 2>
struct RingTile {
  static constexpr int H = 256, WH = WH_, AT = H / 32 / WH, WT = kScoreWaves / WH, BT = 32 * BTW * WT;
  static constexpr int WB = H * kRingRow, XB = BT * kRingRow, STAGE = WB + XB;
  static constexpr int WI = WB / 1024 / kScoreWaves, XI = XB / 1024 / kScoreWaves;   // DMAs per wave per stage
  static_assert(WI >= 1 && XI >= 1, "stage split over the waves");
};

template <int BTW, int NS, int WH>
__global__ __launch_bounds__(kScoreWaves * 64, 1) void score_ring_kernel(
    int n, int d_model, const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ w1,
    const float* __restrict__ b1, const uint16_t* __restrict__ w2, float b2, float* __restrict__ scores) {
  using T = RingTile<BTW, NS, WH>;
  constexpr int H = T::H, BT = T::BT, AT = T::AT, WT = T::WT;
  __shared__ __attribute__((aligned(16))) char ring[NS * T::STAGE];
  __shared__ __attribute__((aligned(16))) float w2f[H];
  __shared__ __attribute__((aligned(16))) float b1f[H];
  __shared__ float red[T::WH][BT];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)ring;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int wh = wave / WT, wt = wave % WT;
  const int tok0 = blockIdx.x * BT;

  for (int i = tid; i < H; i += kScoreWaves * 64) {
    w2f[i] = bf16_to_f32(w2[i]);
    b1f[i] = b1 ? b1[i] : 0.f;
  }

  // DMA j of this wave fills rows 8 (I wave + j) + lane/8 of the W (or X) stage; the lane
  // writes physical chunk lane%8 of its row, which holds logical chunk (lane%8) ^ swz(row).
  // Token rows past the end re-read the last token (their scores are never written).
  uint32_t wo[T::WI], wm[T::WI], xo[T::XI], xm[T::XI];
#pragma unroll
  for (int j = 0; j < T::WI; ++j) {
    const int r = 8 * (T::WI * wave + j) + lane / 8;
    wo[j] = (uint32_t)((r * d_model + 8 * ((lane % 8) ^ ring_swz(r))) * 2);
    wm[j] = (uint32_t)((T::WI * wave + j) * 1024);
  }
#pragma unroll
  for (int j = 0; j < T::XI; ++j) {
    const int r = 8 * (T::XI * wave + j) + lane / 8;
    const int64_t rt = min(tok0 + r, n - 1) - tok0;
    xo[j] = (uint32_t)((rt * ldx + 8 * ((lane % 8) ^ ring_swz(r))) * 2);
    xm[j] = (uint32_t)(T::WB + (T::XI * wave + j) * 1024);
  }
  const char* wg = reinterpret_cast<const char*>(w1);
  const char* xg = reinterpret_cast<const char*>(x) + (int64_t)tok0 * ldx * 2;
  auto issue = [&](int c, int slot) {
#pragma unroll
    for (int j = 0; j < T::WI; ++j) dma_lds16(wo[j], wg + c * kRingRow, lds0 + slot * T::STAGE + wm[j]);
#pragma unroll
    for (int j = 0; j < T::XI; ++j) dma_lds16_nt(xo[j], xg + c * kRingRow, lds0 + slot * T::STAGE + xm[j]);
  };

  // operand byte address of k-step ks for row l32 (plus 32-row tile offsets)
  uint32_t oa[kRingKC / 16];
#pragma unroll
  for (int ks = 0; ks < kRingKC / 16; ++ks) oa[ks] = (uint32_t)(l32 * kRingRow + 16 * ((2 * ks + half) ^ ring_swz(l32)));

  f32x16 acc[AT][BTW];
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BTW; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int nch = d_model / kRingKC;
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
    const char* st = ring + slot * T::STAGE;
    // operands of k-step ks + 1 are read before the products of k-step ks (two register sets),
    // scheduling fences keeping them there
    constexpr int NKS = kRingKC / 16;
    bf16x8 af[2][AT], bfr[2][BTW];
    auto load = [&](int ks, int buf) {
#pragma unroll
      for (int a = 0; a < AT; ++a)
        af[buf][a] = *reinterpret_cast<const bf16x8*>(st + oa[ks] + 32 * kRingRow * (wh * AT + a));
#pragma unroll
      for (int b = 0; b < BTW; ++b)
        bfr[buf][b] = *reinterpret_cast<const bf16x8*>(st + T::WB + oa[ks] + 32 * kRingRow * (wt * BTW + b));
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

  // epilogue: lane holds token 32 (wt BTW + b) + l32 and hidden units
  // 32 (wh AT + a) + 8 g + 4 half + r of tile (a, b)
  float part[BTW];
#pragma unroll
  for (int b = 0; b < BTW; ++b) part[b] = 0.f;
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int hid = 32 * (wh * AT + a) + 8 * g + 4 * half;
      const f32x4 ww = *reinterpret_cast<const f32x4*>(&w2f[hid]);
      const f32x4 bb = *reinterpret_cast<const f32x4*>(&b1f[hid]);
#pragma unroll
      for (int b = 0; b < BTW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[b] = fmaf(ww[r], gelu_exact(acc[a][b][4 * g + r] + bb[r]), part[b]);
    }
#pragma unroll
  for (int b = 0; b < BTW; ++b) {
    part[b] += swap_halves(part[b]);
    if (half == 0) red[wh][32 * (wt * BTW + b) + l32] = part[b];
  }
  __syncthreads();
  for (int t = tid; t < BT; t += kScoreWaves * 64) {
    if (tok0 + t < n) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < T::WH; ++w) s += red[w][t];
      scores[tok0 + t] = s + b2;
    }
  }
}

template <int BTW, int NS, int WH = 2>
static tg_status launch_score_ring(int n, int d_model, const void* x, int64_t ldx, const void* w1, const float* b1,
                                   const void* w2, float b2, float* scores, hipStream_t stream) {
  constexpr int BT = RingTile<BTW, NS, WH>::BT;
  const int grid = (n + BT - 1) / BT;
  hipLaunchKernelGGL((score_ring_kernel<BTW, NS, WH>), dim3(grid), dim3(kScoreWaves * 64), 0, stream, n, d_model,
                     static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(w1), b1,
                     static_cast<const uint16_t*>(w2), b2, scores);
  TG_CHECK_LAUNCH();
  return TG_OK;
}

}  // namespace tg

extern "C" tg_status tg_gate_score(int32_t dtype, int64_t n, int32_t d_model, int32_t d_hidden,
                                   const void* x, int64_t ldx, const void* w1, const float* b1,
                                   const void* w2, float b2, float* scores, void* stream) {
  using namespace tg;
  if (dtype != TG_F32 && dtype != TG_BF16) return TG_ERR_INVALID_ARG;
  if (!x || !w1 || !w2 || !scores) return TG_ERR_INVALID_ARG;
  if (n <= 0 || n > INT32_MAX || d_model <= 0 || d_hidden <= 0 || ldx < d_model) return TG_ERR_INVALID_ARG;
  if (!std::isfinite(b2)) return TG_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == TG_F32) {
    if (d_hidden > 256) return TG_ERR_UNSUPPORTED;
    const int grid = static_cast<int>((n + kF32Toks - 1) / kF32Toks);
    hipLaunchKernelGGL(score_f32_kernel, dim3(grid), dim3(256), 0, st, static_cast<int>(n), d_model,
                       d_hidden, static_cast<const float*>(x), ldx, static_cast<const float*>(w1), b1,
                       static_cast<const float*>(w2), b2, scores);
    TG_CHECK_LAUNCH();
    return TG_OK;
  }
  if (d_model % kScoreKC != 0 || ldx % 8 != 0) return TG_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w1)) & 15u) return TG_ERR_UNSUPPORTED;
  const int nn = static_cast<int>(n);
  // d_hidden 256: DMA ring; 256-token tiles (two stages) once there are enough of them to
  // fill the chip, which halves the W1 re-reads per token, else 128-token tiles (three
  // stages), and 64-token tiles (4 waves along the hidden units) below 32768 tokens, where
  // 128-token tiles leave CUs idle.  The row offsets of one tile must fit 32 bits.
  // 64/128/192: register-staged tiles.
  const bool big = n >= 65536, small = n < 32768;
  switch (d_hidden) {
    case 64:
      return launch_score_bf16<64, 1>(nn, d_model, x, ldx, w1, b1, w2, b2, scores, st);
    case 128:
      return launch_score_bf16<128, 1>(nn, d_model, x, ldx, w1, b1, w2, b2, scores, st);
    case 192:
      return launch_score_bf16<192, 1>(nn, d_model, x, ldx, w1, b1, w2, b2, scores, st);
    case 256:
      if ((int64_t)ldx * 2 * 256 > INT32_MAX || (int64_t)d_model * 2 * 256 > INT32_MAX) return TG_ERR_UNSUPPORTED;
      if (big) return launch_score_ring<2, 2>(nn, d_model, x, ldx, w1, b1, w2, b2, scores, st);
      if (small) return launch_score_ring<1, 3, 4>(nn, d_model, x, ldx, w1, b1, w2, b2, scores, st);
      return launch_score_ring<1, 3>(nn, d_model, x, ldx, w1, b1, w2, b2, scores, st);
    default:
      return TG_ERR_UNSUPPORTED;
  }
}
