// Gradient of the token-gated attention.
//
// The gate's top-K is not differentiable; TokenGate turns each kept token's score
// into a bias on the attention logits so that the scorer receives a gradient, and
// trains a per-head gain and a temperature with it (aiproducthub.cn "斯坦福伯克利
// TokenGate 预填充提速11.3倍", section 事件详情; aisight.pl "TokenGate: Stanford i
// Berkeley ...", section "Jak to dziala"; news.chathome.org TokenGate article, section
// "トークンゲート付きアテンションとは").  With logit[i,j] = q_i.k_j / (sqrt(d) tau) +
// gain[h] s[j] on the visible keys, P the row softmax and dO the output gradient:
//     dP = dO V^T,  D_i = dO_i . O_i,  dZ = P (dP - D)            (logit gradient)
//     dQ = dZ K / (sqrt(d) tau),  dK = dZ^T Q / (sqrt(d) tau),  dV = P^T dO
//     ds[j] = sum_h gain[h] sum_i dZ_h[i,j],  dgain[h] = sum_j s[j] sum_i dZ_h[i,j]
//     dtau = -(1/tau) sum dZ . (q.k / (sqrt(d) tau))
// P is recomputed from the forward's row log-sum-exp: P = exp2(c2 q.k + g2 s - lse2)
// with c2 = log2(e) / (sqrt(d) tau), g2 = gain log2(e), lse2 = lse log2(e); the
// product q.k is exact in float32 from the bf16 operands and the scale is applied in
// float32.
//
// Kernels (bf16 MFMA 32x32x16, float32 accumulation), the streamed tiles fed by DMA
// (global_load_lds) into double-buffered, XOR-swizzled LDS: the next tile is in
// flight while the current one is consumed, one barrier per tile.
//  * prep: D[h, i] = dO_i . O_i and lse2[h, i], head-major so a tile's values are
//    contiguous;
//  * dq:  the forward's shape -- a wave owns 32 queries of one head with Q^T and dO^T
//         as fixed B operands in registers; 64-key K/V tiles stream through LDS; per
//         32 keys, S^T = K Q^T and dP^T = V dO^T give dZ^T in registers (lane =
//         query), and dQ^T += K^T dZ^T reads K^T from the tile with ds_read_b64_tr_b16;
//  * dkv: the transpose, on 16x16x32 MFMA -- a workgroup (8 waves, two per SIMD) owns
//         128 keys of one key/value head and a wave 16 of them, with K and V as fixed B
//         operands in registers and the dK / dV accumulators beside them (about 210
//         registers with the compiler's prefetching, which still lets two waves share
//         a SIMD and hide each other's latencies);
//         32-query Q / dO tiles of every head of the group stream through a 3-stage LDS
//         ring; S = Q K^T and dP = dO V^T give P and dZ (lane = key), dV^T += dO^T P and
//         dK^T += Q^T dZ read dO^T and Q^T from the tiles by transposing LDS reads.  The
//         key-side sums (ds, dgain, dtau) accumulate per lane and leave as
//         per-wave partials;
//  * reduce: sums the partials of ds (over key/value heads), dgain and dtau in a fixed
//         order, so results are deterministic.
// Every gradient element is written by exactly one workgroup: no float atomics.  Both
// gradient kernels apply the visibility mask only on tiles where a key can follow a query
// or a row lies past the end, and address every LDS operand by a per-lane offset formed
// once plus an immediate (their tile loops are unrolled over the LDS buffers): the vector
// work per tile is otherwise comparable to the MFMA work.
#include <type_traits>

#include "tg_common.h"

namespace tg {

constexpr int kDqWaves = 4;                      // dq workgroup
constexpr int kDqKeys = 64;                      // keys per dq tile
constexpr int kDkvWaves = 8;                     // dkv workgroup (two waves per SIMD)
constexpr int kDkvKeys = 16 * kDkvWaves;         // keys per dkv workgroup, 16 per wave
constexpr int kDkvRows = 32;                     // queries per dkv tile
constexpr int kDkvStages = 3;                    // dkv tiles in flight or in use

typedef short bs16x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// XOR swizzle of the 16-byte chunks of a tile row (row = key or query in the tile)
template <int D> __device__ __forceinline__ int bwd_swz(int r);
template <> __device__ __forceinline__ int bwd_swz<128>(int r) { return r & 15; }
template <> __device__ __forceinline__ int bwd_swz<64>(int r) { return (r >> 1) & 7; }

// DMA of `rows` rows of D bf16 (row stride ld elements, first row `first`, rows past
// `m` re-read row m - 1) into a swizzled LDS tile at byte address `dst`.  A DMA
// instruction moves 1 KiB = 1024 / (2 D) rows; instruction I of the tile goes to wave
// I % waves.  Lane L writes physical chunk L % CPR of row RPI I + L / CPR, which holds
// logical chunk (L % CPR) ^ swz(row).
template <int D>
__device__ __forceinline__ void bwd_dma_tile(uint32_t dst, const uint16_t* __restrict__ src, int64_t ld, int first,
                                             int m, int rows, int wave, int waves, int lane) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int n_inst = rows / RPI;
  const char* base = reinterpret_cast<const char*>(src + (int64_t)first * ld);
  for (int I = wave; I < n_inst; I += waves) {
    const int r = RPI * I + lane / CPR, p = lane % CPR;
    const int rr = min(first + r, m - 1) - first;
    const uint32_t off = (uint32_t)(((int64_t)rr * ld + 8 * (p ^ bwd_swz<D>(r))) * 2);
    dma_lds16(off, base, dst + I * 1024);
  }
}

// The same DMA for a tile with no row past m: instruction I = I0 + waves j reads rows RPI I ..,
// whose swizzle repeats every 16 rows, so one per-lane offset (tile_dma_off, formed once per
// kernel) serves every instruction of the wave, the rows stepping through the scalar base.
template <int D>
__device__ __forceinline__ uint32_t tile_dma_off(int64_t ld, int I0, int lane) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int r = RPI * I0 + lane / CPR;
  return (uint32_t)(((int64_t)r * ld + 8 * ((lane % CPR) ^ bwd_swz<D>(r))) * 2);
}
template <int D>
__device__ __forceinline__ void bwd_dma_tile_full(uint32_t dst, const uint16_t* __restrict__ src, int64_t ld, int first,
                                                  int rows, int I0, int waves, uint32_t off) {
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  static_assert((RPI * 4) % 16 == 0, "the swizzle repeats across a wave's instructions");
  const int n_inst = rows / RPI;
  const char* base = reinterpret_cast<const char*>(src + (int64_t)first * ld);
  for (int I = I0; I < n_inst; I += waves)
    dma_lds16(off, base + (int64_t)(RPI * (I - I0)) * ld * 2, dst + I * 1024);
}

// Operand reads at a precomputed per-lane byte offset from a tile's LDS base: the offsets of
// the swizzled layouts depend only on the lane and the k-step or d tile, so they are formed
// once per kernel and every read is one base + offset address (plus an immediate).
__device__ __forceinline__ bf16x8 lds_row(const char* base, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}
__device__ __forceinline__ u32x2 lds_tr(const char* base, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) bs16x4*)(base + off)));
}

// bf16 B operand of the 16-row k-step s2 from a 32x32 accumulator
__device__ __forceinline__ bf16x8 pack_acc(const f32x16& a, int s2) {
  u32x4 w;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) w[e2] = pack_bf16x2(a[8 * s2 + 2 * e2], a[8 * s2 + 2 * e2 + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// ---------------------------------------------------------------------------------
// D[h, i] = dO[i, h, :] . O[i, h, :] and lse2[h, i] = lse[i, h] log2(e), head-major
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(int m, int hq, const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        const float* __restrict__ lse, float* __restrict__ dsum_t,
                                                        float* __restrict__ lse2_t) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;   // = row * hq + head
  if (r >= (int64_t)m * hq) return;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + r * D + 8 * c);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + r * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_to_f32(a[e] & 0xffffu), bf16_to_f32(b[e] & 0xffffu), acc);
      acc = fmaf(bf16_to_f32(a[e] >> 16), bf16_to_f32(b[e] >> 16), acc);
    }
  }
  const int64_t row = r / hq, head = r % hq;
  dsum_t[head * m + row] = acc;
  lse2_t[head * m + row] = lse[r] * kLog2e;
}

// ---------------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------------
template <int D>
struct DqLds {
  static constexpr int TILE = kDqKeys * D * 2;                 // bytes of one K or V tile
  static constexpr int K0 = 0, V0 = TILE, S0 = 2 * TILE, P0 = S0 + kDqKeys * 4, BUF = P0 + kDqKeys * 4;
  static constexpr int BYTES = 2 * BUF;
};

template <int D, int HPW>
__global__ __launch_bounds__(kDqWaves * 64, 2) void bwd_dq_kernel(
    int m, int hq, int hkv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos, const float* __restrict__ s_kept,
    const float* __restrict__ gain, const float* __restrict__ lse, const float* __restrict__ dsum_t,
    const uint16_t* __restrict__ dout, float c2, float c_nat, uint16_t* __restrict__ dq, int n_qtiles) {
  using L = DqLds<D>;
  constexpr int ROWS = 32 * kDqWaves / HPW;
  __shared__ __attribute__((aligned(1024))) char lds[L::BYTES];
  const uint32_t lds0 = lds_addr(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int group = hq / hkv;
  const int slots_per_kv = group / HPW;
  const int units = hkv * slots_per_kv;
  const int unit = blockIdx.x % units;
  const int qt = n_qtiles - 1 - blockIdx.x / units;             // longest first
  const int kvh = unit / slots_per_kv;
  const int head = kvh * group + (unit % slots_per_kv) * HPW + wave % HPW;
  const int q0 = qt * ROWS + (wave / HPW) * 32;
  const int row = q0 + l32;
  const bool wave_live = q0 < m;
  const int wave_last = min(m - 1, q0 + 31);
  const bool live_row = row < m;

  // fixed B operands: Q and dO, lane = query row
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (live_row) {
      qf[s] = *reinterpret_cast<const bf16x8*>(q + ((int64_t)row * hq + head) * D + 16 * s + 8 * half);
      df[s] = *reinterpret_cast<const bf16x8*>(dout + ((int64_t)row * hq + head) * D + 16 * s + 8 * half);
    } else {
      qf[s] = bf16x8{};
      df[s] = bf16x8{};
    }
  }
  const float nlse2 = live_row ? -lse[(int64_t)row * hq + head] * kLog2e : 0.f;
  const float dval = live_row ? dsum_t[(int64_t)head * m + row] : 0.f;
  const int32_t qpos = live_row ? (pos ? pos[row] : row) : INT32_MIN;
  const float g2 = s_kept ? gain[head] * kLog2e : 0.f;

  f32x16 dqa[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[u][i] = 0.f;

  // byte offsets within a 32-key half tile: K / V row l32, 16-wide k-step s, lane half h
  // (A operand of S^T and dP^T), and K^T for d tile u (A operand of dQ^T): lane half h
  // receives keys {4h..4h+3} (g8 = 0) and {8+4h..8+4h+3} (g8 = 1) of each 16-key step, the
  // order in which the 32x32 accumulator's registers leave them, at d = 32u + (lane & 31)
  uint32_t rowo[D / 16], tro[D / 32][2];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) rowo[s] = (uint32_t)(2 * (l32 * D + 8 * ((2 * s + half) ^ bwd_swz<D>(l32))));
  {
    const int gi = lane & 15, gg = lane >> 4;
    const int row_lane = 4 * half + (gi >> 2);
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int g8 = 0; g8 < 2; ++g8) {
        const int row = 8 * g8 + row_lane;
        const int dcol = 32 * u + 16 * (gg & 1) + 4 * (gi & 3);
        tro[u][g8] = (uint32_t)(2 * (row * D + 8 * ((dcol >> 3) ^ bwd_swz<D>(row)) + (dcol & 7)));
      }
  }

  const int rows_end = min(m, (qt + 1) * ROWS);
  const int n_tiles = (rows_end + kDqKeys - 1) / kDqKeys;
  const uint16_t* kh = k + (int64_t)kvh * D;
  const uint16_t* vh = v + (int64_t)kvh * D;
  const int64_t ld = (int64_t)hkv * D;

  const int iv0 = (wave + 2) % kDqWaves;
  const uint32_t offk = tile_dma_off<D>(ld, wave, lane), offv = tile_dma_off<D>(ld, iv0, lane);
  auto issue = [&](int t) {
    const int kb = t * kDqKeys;
    const uint32_t buf = lds0 + (t & 1) * L::BUF;
    if (kb + kDqKeys <= m) {
      bwd_dma_tile_full<D>(buf + L::K0, kh, ld, kb, kDqKeys, wave, kDqWaves, offk);
      bwd_dma_tile_full<D>(buf + L::V0, vh, ld, kb, kDqKeys, iv0, kDqWaves, offv);
    } else {
      bwd_dma_tile<D>(buf + L::K0, kh, ld, kb, m, kDqKeys, wave, kDqWaves, lane);
      bwd_dma_tile<D>(buf + L::V0, vh, ld, kb, m, kDqKeys, iv0, kDqWaves, lane);
    }
    const uint32_t off = (uint32_t)((min(kb + lane, m - 1) - kb) * 4);
    if (wave == 0 && s_kept) dma_lds4(off, s_kept + kb, buf + L::S0);
    if (wave == 1 && pos) dma_lds4(off, pos + kb, buf + L::P0);
  };

  if (n_tiles > 0) issue(0);
  // 32 keys of tile t (half h2 of its 64) from LDS buffer BUF = t mod 2; BUF and h2 are
  // compile-time constants, so every operand address is a per-lane offset plus an immediate
  auto half_tile = [&](int kb, auto bufc, auto h2c) {
    constexpr int BUF = decltype(bufc)::value, h2 = decltype(h2c)::value;
    const int kb2 = kb + 32 * h2;
    const char* buf = lds + BUF * L::BUF;
    const float* s_t = reinterpret_cast<const float*>(buf + L::S0);
    const int32_t* p_t = reinterpret_cast<const int32_t*>(buf + L::P0);
    const char* kh2 = buf + L::K0 + h2 * 32 * D * 2;   // this half's 32 keys
    const char* vh2 = buf + L::V0 + h2 * 32 * D * 2;
    f32x16 sa, da;
#pragma unroll
    for (int i = 0; i < 16; ++i) { sa[i] = 0.f; da[i] = 0.f; }
    // products n = 2 s + (0: S^T from K, 1: dP^T from V), in that order; each operand is read
    // RING - 1 products ahead in a ring, scheduling fences keeping the reads there
    constexpr int NP = 2 * (D / 16), RING = 3;
    auto opnd = [&](int n) { return lds_row((n & 1) ? vh2 : kh2, rowo[n >> 1]); };
    bf16x8 ring[RING];
#pragma unroll
    for (int n = 0; n < RING - 1; ++n) ring[n] = opnd(n);
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      if (n + RING - 1 < NP) ring[(n + RING - 1) % RING] = opnd(n + RING - 1);
      if (n & 1) da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % RING], df[n >> 1], da, 0, 0, 0);
      else sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % RING], qf[n >> 1], sa, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // register e holds key kb2 + 8 (e/4) + 4 half + e%4, query = this lane's row.  The mask
    // is needed only where a key may follow a query (positions rise with the index) or a key
    // or query lies past the end; elsewhere every key is visible (uniform over the wave).
    const bool masked = kb2 + 31 > q0 || kb2 + 32 > m || q0 + 32 > m;
    auto dz = [&](auto maskc) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = 32 * h2 + 8 * g + 4 * half;
        f32x4 sv = {0.f, 0.f, 0.f, 0.f};
        if (s_kept) sv = *reinterpret_cast<const f32x4*>(&s_t[j0]);
        i32x4 kp = {};
        if (decltype(maskc)::value) {
          if (pos) kp = *reinterpret_cast<const i32x4*>(&p_t[j0]);
          else kp = i32x4{kb + j0, kb + j0 + 1, kb + j0 + 2, kb + j0 + 3};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          const bool vis = !decltype(maskc)::value || (kp[r] <= qpos && kb + j0 + r < m);
          const float p = vis ? __builtin_amdgcn_exp2f(fmaf(sa[e], c2, fmaf(g2, sv[r], nlse2))) : 0.f;
          da[e] = p * (da[e] - dval);   // da now holds dZ
        }
      }
    };
    if (masked) dz(std::true_type{});
    else dz(std::false_type{});
    const bf16x8 z0 = pack_acc(da, 0), z1 = pack_acc(da, 1);
    // dQ products n = 2 u + s2 (keys 16 s2 .. 16 s2 + 15 of the half), K^T operands read
    // RING - 1 products ahead
    auto kt_opnd = [&](int n) {
      const int u = n >> 1, s2 = n & 1;
      const u32x2 p0 = lds_tr(kh2 + s2 * 16 * D * 2, tro[u][0]);
      const u32x2 p1 = lds_tr(kh2 + s2 * 16 * D * 2, tro[u][1]);
      const u32x4 a4 = {p0[0], p0[1], p1[0], p1[1]};
      return __builtin_bit_cast(bf16x8, a4);
    };
    constexpr int NQ = 2 * (D / 32);
#pragma unroll
    for (int n = 0; n < RING - 1; ++n) ring[n] = kt_opnd(n);
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      if (n + RING - 1 < NQ) ring[(n + RING - 1) % RING] = kt_opnd(n + RING - 1);
      dqa[n >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % RING], (n & 1) ? z1 : z0, dqa[n >> 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](int t, auto bufc) {
    const int kb = t * kDqKeys;
    dma_wait_all();
    __syncthreads();   // tile t visible to every wave; tile t - 1's buffer free
    if (t + 1 < n_tiles) issue(t + 1);
    if (!wave_live || kb > wave_last) return;
    half_tile(kb, bufc, std::integral_constant<int, 0>{});
    if (kb + 32 <= wave_last) half_tile(kb, bufc, std::integral_constant<int, 1>{});
  };
  static_assert(kDqKeys == 64, "two 32-key halves per tile");
  for (int t0 = 0; t0 < n_tiles; t0 += 2) {
    step(t0, std::integral_constant<int, 0>{});
    if (t0 + 1 < n_tiles) step(t0 + 1, std::integral_constant<int, 1>{});
  }
  if (live_row) {
    uint16_t* orow = dq + ((int64_t)row * hq + head) * D;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * u + 8 * g + 4 * half;
        const u32x2 pk = {pack_bf16x2(dqa[u][4 * g] * c_nat, dqa[u][4 * g + 1] * c_nat),
                          pack_bf16x2(dqa[u][4 * g + 2] * c_nat, dqa[u][4 * g + 3] * c_nat)};
        *reinterpret_cast<u32x2*>(orow + d0) = pk;
      }
  }
}

// ---------------------------------------------------------------------------------
// dK, dV and the key-side partial sums (v_mfma_f32_16x16x32_bf16: A 16 rows x 32 k and
// B 32 k x 16 columns hold row / column lane % 16 and k = 8 (lane / 16) + 0..7; the
// 16x16 result holds column lane % 16 and rows 4 (lane / 16) + 0..3)
// ---------------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 pack8(const f32x4_t& a, const f32x4_t& b) {
  const u32x4 w = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
  return __builtin_bit_cast(bf16x8, w);
}

template <int D>
struct DkvLds {
  static constexpr int TILE = kDkvRows * D * 2;                // bytes of one Q or dO tile
  static constexpr int Q0 = 0, O0 = TILE, ST0 = 2 * TILE;      // stats: lse2[32] | D[32] | pos[32]
  static constexpr int BUF = ST0 + 3 * kDkvRows * 4 + 128;     // (+ the unused upper half of the pos DMA)
  static constexpr int BYTES = kDkvStages * BUF;
};

template <int D>
__global__ __launch_bounds__(kDkvWaves * 64, 1) void bwd_dkv_kernel(
    int m, int hq, int hkv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos, const float* __restrict__ s_kept,
    const float* __restrict__ gain, const float* __restrict__ stats, int64_t dsum_off, const uint16_t* __restrict__ dout,
    float c2, float c_nat, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ ds_part,
    float* __restrict__ dgain_part, float* __restrict__ dtau_part, int n_kblocks) {
  using L = DkvLds<D>;
  constexpr int KS = D / 32;                      // 32-wide k-steps over d
  constexpr int DT = D / 16;                      // 16-wide d tiles of dK / dV
  __shared__ __attribute__((aligned(1024))) char lds[L::BYTES];
  const uint32_t lds0 = lds_addr(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, l16 = lane & 15;
  const int group = hq / hkv;
  const int kvh = blockIdx.x % hkv;
  const int kblk = blockIdx.x / hkv;              // longest (earliest keys) first
  const int kb0 = kblk * kDkvKeys;
  const int kw0 = kb0 + 16 * wave;                // this wave's first key
  const int key = kw0 + l16;
  const bool live_key = key < m;
  const int kc = min(key, m - 1);
  const int32_t kpos = live_key ? (pos ? pos[kc] : kc) : INT32_MAX;
  const float sk = s_kept ? s_kept[kc] : 0.f;

  // fixed B operands: K and V of this lane's key, d = 32 s + 8 G + 0..7
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kf[s] = *reinterpret_cast<const bf16x8*>(k + ((int64_t)kc * hkv + kvh) * D + 32 * s + 8 * grp);
    vf[s] = *reinterpret_cast<const bf16x8*>(v + ((int64_t)kc * hkv + kvh) * D + 32 * s + 8 * grp);
  }

  f32x4_t dka[DT], dva[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) { dka[t][i] = 0.f; dva[t][i] = 0.f; }
  float ds_acc = 0.f, dtau_acc = 0.f;

  // byte offsets within a Q or dO tile: row l16, 32-wide k-step s, lane group G (A operand
  // of S and dP), and the transposed read for d tile t2 (A operand of dK^T and dV^T): lane
  // group G receives rows {4G..4G+3} and, 16 rows further, {16+4G..16+4G+3}, the rows a
  // 16x16 result leaves in its two row blocks, at d = 16 t2 + (lane & 15)
  uint32_t rowo[KS], tro[DT];
#pragma unroll
  for (int s = 0; s < KS; ++s) rowo[s] = (uint32_t)(2 * (l16 * D + 8 * ((4 * s + grp) ^ bwd_swz<D>(l16))));
#pragma unroll
  for (int t2 = 0; t2 < DT; ++t2) {
    const int row = 4 * grp + (l16 >> 2);
    const int dcol = 16 * t2 + 4 * (l16 & 3);
    tro[t2] = (uint32_t)(2 * (row * D + 8 * ((dcol >> 3) ^ bwd_swz<D>(row)) + (dcol & 7)));
  }
  constexpr uint32_t kBlk16 = 16 * D * 2;         // bytes of 16 rows

  const int first_tile = kb0 / kDkvRows;          // queries before the first key see none of them
  const int n_qt = (m + kDkvRows - 1) / kDkvRows;
  const int per_head = n_qt - first_tile;
  const int n_it = group * per_head;
  const int64_t ld = (int64_t)hq * D;
  // DMAs this wave issues per tile (its share of the Q and dO rows, plus the statistics)
  constexpr int PER16 = 2 * (kDkvRows * D * 2 / 1024) / kDkvWaves;
  static_assert(PER16 >= 1 && (2 * (kDkvRows * D * 2 / 1024)) % kDkvWaves == 0, "tile DMAs split evenly");
  const bool extra = wave == 0 || (wave == 1 && pos);

  // this wave's Q and dO pieces of a whole tile: instruction I of bwd_dma_tile (at most one
  // per wave and matrix), its per-lane byte offset formed once; ragged tiles clamp per call
  constexpr int CPR = D / 8, RPI = 64 / CPR, NI = kDkvRows / RPI;
  static_assert(NI <= kDkvWaves, "one DMA per wave and matrix");
  const int iq = wave, io = (wave + kDkvWaves / 2) % kDkvWaves;
  auto piece_off = [&](int I) {
    const int r = RPI * I + lane / CPR;
    return (uint32_t)(((int64_t)r * ld + 8 * ((lane % CPR) ^ bwd_swz<D>(r))) * 2);
  };
  const uint32_t offq = piece_off(iq), offo = piece_off(io);
  // tiles in issue order: it = hh per_head + (t - first_tile); counters advanced one tile at a
  // time instead of dividing by per_head
  auto advance = [&](int& hh, int& t) {
    if (++t == n_qt) {
      t = first_tile;
      ++hh;
    }
  };
  auto issue = [&](int it, int hh, int t) {
    const int head = kvh * group + hh, qb = t * kDkvRows;
    const uint32_t buf = lds0 + (it % kDkvStages) * L::BUF;
    if (qb + kDkvRows <= m) {
      const char* qg = reinterpret_cast<const char*>(q + (int64_t)head * D + (int64_t)qb * ld);
      const char* og = reinterpret_cast<const char*>(dout + (int64_t)head * D + (int64_t)qb * ld);
      if (iq < NI) dma_lds16(offq, qg, buf + L::Q0 + iq * 1024);
      if (io < NI) dma_lds16(offo, og, buf + L::O0 + io * 1024);
    } else {
      bwd_dma_tile<D>(buf + L::Q0, q + (int64_t)head * D, ld, qb, m, kDkvRows, wave, kDkvWaves, lane);
      bwd_dma_tile<D>(buf + L::O0, dout + (int64_t)head * D, ld, qb, m, kDkvRows, (wave + kDkvWaves / 2) % kDkvWaves,
                      kDkvWaves, lane);
    }
    const int qi = min(qb + (lane & 31), m - 1);
    if (wave == 0) {   // lanes 0..31: lse2[head][qi], lanes 32..63: D[head][qi]
      const uint32_t off = (uint32_t)(((int64_t)head * m + qi) * 4 + (lane >= 32 ? dsum_off : 0));
      dma_lds4(off, stats, buf + L::ST0);
    }
    if (wave == 1 && pos) dma_lds4((uint32_t)(qi * 4), pos, buf + L::ST0 + 2 * kDkvRows * 4);
  };

  int ihh = 0, it_t = first_tile;   // the next tile to issue
  for (int i = 0; i < kDkvStages - 1; ++i)
    if (i < n_it) {
      issue(i, ihh, it_t);
      advance(ihh, it_t);
    }
  int shh = 0, st_t = first_tile;   // the next tile to compute
  float col = 0.f;   // this lane's part of the sum over queries of dZ, current head
  // one query tile; ST = it mod kDkvStages is a compile-time constant, so the tile's LDS base
  // and every operand address within it are a per-lane offset plus an immediate
  auto step = [&](int it, auto stc) {
    constexpr int ST = decltype(stc)::value;
    const int hh = shh, t = st_t;
    advance(shh, st_t);
    const int head = kvh * group + hh, qb = t * kDkvRows;
    // tile it has landed once the DMAs of the later tiles already issued are all that remain
    const int later = min(kDkvStages - 2, n_it - 1 - it);
    if (later == 1) {
      if (extra) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PER16 + 1) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PER16) : "memory");
    } else {
      dma_wait_all();
    }
    __syncthreads();   // tile it visible to every wave; the buffer of tile it - 1 is free
    if (it + kDkvStages - 1 < n_it) {
      issue(it + kDkvStages - 1, ihh, it_t);
      advance(ihh, it_t);
    }
    if (qb + kDkvRows - 1 >= kw0 && kw0 < m) {   // some query of the tile sees these keys
      const char* buf = lds + ST * L::BUF;   // ST = it mod kDkvStages, a constant here
      const uint16_t* q_t = reinterpret_cast<const uint16_t*>(buf + L::Q0);
      const uint16_t* o_t = reinterpret_cast<const uint16_t*>(buf + L::O0);
      const float* lse_t = reinterpret_cast<const float*>(buf + L::ST0);
      const float* d_t = lse_t + kDkvRows;
      const int32_t* p_t = reinterpret_cast<const int32_t*>(d_t + kDkvRows);
      const float bias2 = s_kept ? gain[head] * kLog2e * sk : 0.f;
      // S = Q K^T and dP = dO V^T for the tile's two 16-query blocks
      f32x4_t sa[2], da[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) { sa[b][i] = 0.f; da[b][i] = 0.f; }
      const char* qc = reinterpret_cast<const char*>(q_t);
      const char* oc = reinterpret_cast<const char*>(o_t);
      // transposed A operand over the tile's 32 rows: rows 4G.. of each 16-row block, d tile t2
      auto tr_a = [&](const char* tile, int t2) {
        const u32x2 p0 = lds_tr(tile, tro[t2]), p1 = lds_tr(tile + kBlk16, tro[t2]);
        const u32x4 a4 = {p0[0], p0[1], p1[0], p1[1]};
        return __builtin_bit_cast(bf16x8, a4);
      };
      // products n = 4 s + 2 b + (0: S from Q, 1: dP from dO), in that order; each operand is read
      // three products ahead (a ring of four), scheduling fences keeping the reads there
      constexpr int NP = 4 * KS, RING = 5;
      auto opnd = [&](int n) { return lds_row(((n & 1) ? oc : qc) + ((n >> 1) & 1) * kBlk16, rowo[n >> 2]); };
      bf16x8 ring[RING];
#pragma unroll
      for (int n = 0; n < RING - 1; ++n) ring[n] = opnd(n);
      // the rows' statistics (lse in base-2 units, D) are read with the first operands
      f32x4_t lvs[2], dvs[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        lvs[b] = *reinterpret_cast<const f32x4_t*>(&lse_t[16 * b + 4 * grp]);
        dvs[b] = *reinterpret_cast<const f32x4_t*>(&d_t[16 * b + 4 * grp]);
      }
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        const int sk_ = n >> 2, b = (n >> 1) & 1;
        if (n + RING - 1 < NP) ring[(n + RING - 1) % RING] = opnd(n + RING - 1);
        if (n & 1) da[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[n % RING], vf[sk_], da[b], 0, 0, 0);
        else sa[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[n % RING], kf[sk_], sa[b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);   // one read and one product per slot, in this order
      }
      // register i of block b holds query qb + 16 b + 4 G + i, key = this lane's.  The mask is
      // needed only where a query may precede a key of this wave or a key or query lies past
      // the end; elsewhere every pair is visible (uniform over the wave).
      const bool masked = qb < kw0 + 15 || qb + kDkvRows > m || kw0 + 16 > m;
      f32x4_t p[2];
      auto probs = [&](auto maskc) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int i0 = 16 * b + 4 * grp;
          const f32x4_t lv = lvs[b];
          i32x4 qp = {};
          if (decltype(maskc)::value) {
            if (pos) qp = *reinterpret_cast<const i32x4*>(&p_t[i0]);
            else qp = i32x4{qb + i0, qb + i0 + 1, qb + i0 + 2, qb + i0 + 3};
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool vis = !decltype(maskc)::value || (kpos <= qp[i] && qb + i0 + i < m);
            p[b][i] = vis ? __builtin_amdgcn_exp2f(fmaf(sa[b][i], c2, bias2 - lv[i])) : 0.f;
          }
        }
      };
      if (masked) probs(std::true_type{});
      else probs(std::false_type{});
      const bf16x8 pb = pack8(p[0], p[1]);
      // dV products t2 = 0 .. DT-1 then dK products: operands (transposed dO, then Q) read three
      // products ahead in a ring of four, across the two
      bf16x8 tring[RING];
      auto topnd = [&](int n) { return n < DT ? tr_a(oc, n) : tr_a(qc, n - DT); };
#pragma unroll
      for (int n = 0; n < RING - 1; ++n) tring[n] = topnd(n);
#pragma unroll
      for (int t2 = 0; t2 < DT; ++t2) {
        if (t2 + RING - 1 < 2 * DT) tring[(t2 + RING - 1) % RING] = topnd(t2 + RING - 1);
        dva[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tring[t2 % RING], pb, dva[t2], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const f32x4_t dv4 = dvs[b];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z = p[b][i] * (da[b][i] - dv4[i]);
          col += z;
          dtau_acc = fmaf(z, sa[b][i], dtau_acc);
          da[b][i] = z;   // da now holds dZ
        }
      }
      const bf16x8 zb = pack8(da[0], da[1]);
#pragma unroll
      for (int t2 = 0; t2 < DT; ++t2) {
        const int n = DT + t2;
        if (n + RING - 1 < 2 * DT) tring[(n + RING - 1) % RING] = topnd(n + RING - 1);
        dka[t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tring[n % RING], zb, dka[t2], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (t == n_qt - 1) {
      // this head's key-side sums: the four lane groups hold parts of the same key's column
      col += __shfl_xor(col, 16, 64);
      col += __shfl_xor(col, 32, 64);
      ds_acc = fmaf(s_kept ? gain[head] : 0.f, col, ds_acc);
      float gsum = (grp == 0 && live_key) ? sk * col : 0.f;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) gsum += __shfl_xor(gsum, o, 64);
      if (lane == 0) dgain_part[((int64_t)head * n_kblocks + kblk) * kDkvWaves + wave] = gsum;
      col = 0.f;
    }
    };
  static_assert(kDkvStages == 3, "the tile loop is unrolled over the three stages");
  for (int it0 = 0; it0 < n_it; it0 += kDkvStages) {
    step(it0, std::integral_constant<int, 0>{});
    if (it0 + 1 < n_it) step(it0 + 1, std::integral_constant<int, 1>{});
    if (it0 + 2 < n_it) step(it0 + 2, std::integral_constant<int, 2>{});
  }
  if (live_key) {
    if (grp == 0) ds_part[(int64_t)kvh * m + key] = ds_acc;
    uint16_t* krow = dk + ((int64_t)key * hkv + kvh) * D;
    uint16_t* vrow = dv + ((int64_t)key * hkv + kvh) * D;
#pragma unroll
    for (int t2 = 0; t2 < DT; ++t2) {
      const int d0 = 16 * t2 + 4 * grp;
      const u32x2 kk = {pack_bf16x2(dka[t2][0] * c_nat, dka[t2][1] * c_nat),
                        pack_bf16x2(dka[t2][2] * c_nat, dka[t2][3] * c_nat)};
      const u32x2 vv = {pack_bf16x2(dva[t2][0], dva[t2][1]), pack_bf16x2(dva[t2][2], dva[t2][3])};
      *reinterpret_cast<u32x2*>(krow + d0) = kk;
      *reinterpret_cast<u32x2*>(vrow + d0) = vv;
    }
  }
  float tsum = live_key ? dtau_acc : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tsum += __shfl_xor(tsum, o, 64);
  if (lane == 0) dtau_part[(int64_t)blockIdx.x * kDkvWaves + wave] = tsum;
}

// ---------------------------------------------------------------------------------
// Fixed-order sums of the partials.  Blocks 0 .. ceil(m/256)-1 sum ds over the
// key/value heads, the next hq blocks dgain (one head each), the last block dtau.
// Each sum's order is fixed by the launch shape alone, so results are bitwise
// reproducible.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_reduce_kernel(int m, int hq, int hkv, int n_kblocks, int n_dkv_blocks,
                                                          const float* __restrict__ ds_part,
                                                          const float* __restrict__ dgain_part,
                                                          const float* __restrict__ dtau_part, float dtau_scale,
                                                          float* __restrict__ ds, float* __restrict__ dgain,
                                                          float* __restrict__ dtau) {
  __shared__ float red[4];
  const int n_ds_blocks = (m + 255) / 256;
  if ((int)blockIdx.x < n_ds_blocks) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (ds && j < m) {
      float acc = 0.f;
      for (int g = 0; g < hkv; ++g) acc += ds_part[(int64_t)g * m + j];
      ds[j] = acc;
    }
    return;
  }
  const int b = (int)blockIdx.x - n_ds_blocks;
  const bool is_gain = b < hq;
  if (is_gain ? !dgain : !dtau) return;   // uniform over the block
  const float* src = is_gain ? dgain_part + (int64_t)b * n_kblocks * kDkvWaves : dtau_part;
  const int n = (is_gain ? n_kblocks : n_dkv_blocks) * kDkvWaves;
  // four independent partial sums per thread, so that four loads are in flight at once
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  int i = threadIdx.x;
  for (; i + 768 < n; i += 1024) {
    a0 += src[i];
    a1 += src[i + 256];
    a2 += src[i + 512];
    a3 += src[i + 768];
  }
  for (; i < n; i += 256) a0 += src[i];
  float acc = (a0 + a1) + (a2 + a3);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    if (is_gain) dgain[b] = tot;
    else *dtau = tot * dtau_scale;
  }
}

struct BwdLayout {
  size_t lse2, dsum, ds_part, dgain_part, dtau_part, bytes;
  BwdLayout(int64_t m, int64_t hq, int64_t hkv) {
    const int64_t nkb = (m + kDkvKeys - 1) / kDkvKeys;
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    lse2 = 0;                                    // [hq][m]
    dsum = up(lse2 + (size_t)m * hq * 4);        // [hq][m]
    ds_part = up(dsum + (size_t)m * hq * 4);     // [hkv][m]
    dgain_part = up(ds_part + (size_t)hkv * m * 4);
    dtau_part = up(dgain_part + (size_t)hq * nkb * kDkvWaves * 4);
    bytes = up(dtau_part + (size_t)hkv * nkb * kDkvWaves * 4);
  }
};

template <int D, int HPW>
static void launch_bwd_dq(int m, int hq, int hkv, const void* q, const void* k, const void* v, const int32_t* pos,
                          const float* s_kept, const float* gain, const float* lse, const float* dsum_t,
                          const void* dout, float c2, float c_nat, void* dq, hipStream_t st) {
  constexpr int ROWS = 32 * kDqWaves / HPW;
  const int n_qtiles = (m + ROWS - 1) / ROWS;
  const int grid = n_qtiles * (hq / HPW);
  hipLaunchKernelGGL((bwd_dq_kernel<D, HPW>), dim3(grid), dim3(kDqWaves * 64), 0, st, m, hq, hkv,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), pos, s_kept, gain, lse, dsum_t,
                     static_cast<const uint16_t*>(dout), c2, c_nat, static_cast<uint16_t*>(dq), n_qtiles);
}

template <int D>
static tg_status attention_backward(int m, int hq, int hkv, const void* q, const void* k, const void* v,
                                    const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                    const void* out, const float* lse, const void* dout, void* dq, void* dk,
                                    void* dv, float* ds, float* dgain, float* dtau, char* ws, hipStream_t st) {
  const BwdLayout L(m, hq, hkv);
  float* lse2_t = reinterpret_cast<float*>(ws + L.lse2);
  float* dsum_t = reinterpret_cast<float*>(ws + L.dsum);
  float* ds_part = reinterpret_cast<float*>(ws + L.ds_part);
  float* dgain_part = reinterpret_cast<float*>(ws + L.dgain_part);
  float* dtau_part = reinterpret_cast<float*>(ws + L.dtau_part);
  const double sd = std::sqrt((double)D) * (double)tau;
  const float c2 = static_cast<float>(1.4426950408889634 / sd);   // base-2 logit per unit q.k
  const float c_nat = static_cast<float>(1.0 / sd);

  const int64_t rows = (int64_t)m * hq;
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, m, hq,
                     static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), lse, dsum_t, lse2_t);
  const int group = hq / hkv;
  if (group % 4 == 0)
    launch_bwd_dq<D, 4>(m, hq, hkv, q, k, v, pos, s_kept, gain, lse, dsum_t, dout, c2, c_nat, dq, st);
  else if (group % 2 == 0)
    launch_bwd_dq<D, 2>(m, hq, hkv, q, k, v, pos, s_kept, gain, lse, dsum_t, dout, c2, c_nat, dq, st);
  else
    launch_bwd_dq<D, 1>(m, hq, hkv, q, k, v, pos, s_kept, gain, lse, dsum_t, dout, c2, c_nat, dq, st);
  const int n_kblocks = (m + kDkvKeys - 1) / kDkvKeys;
  const int n_dkv = n_kblocks * hkv;
  hipLaunchKernelGGL((bwd_dkv_kernel<D>), dim3(n_dkv), dim3(kDkvWaves * 64), 0, st, m, hq, hkv,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), pos, s_kept, gain, lse2_t,
                     (int64_t)(L.dsum - L.lse2), static_cast<const uint16_t*>(dout), c2, c_nat,
                     static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), ds_part, dgain_part, dtau_part,
                     n_kblocks);
  // dtau = -(1/tau) sum dZ (q.k / (sqrt(d) tau)); the kernel summed dZ q.k
  const float dtau_scale = static_cast<float>(-1.0 / (sd * (double)tau));
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((m + 255) / 256 + hq + 1), dim3(256), 0, st, m, hq, hkv, n_kblocks, n_dkv,
                     ds_part, dgain_part, dtau_part, dtau_scale, ds, dgain, dtau);
  TG_CHECK_LAUNCH();
  return TG_OK;
}

}  // namespace tg

extern "C" size_t tg_gated_attention_backward_workspace_bytes(int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                                              int32_t head_dim) {
  if (m < 0 || m > INT32_MAX || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0) return 0;
  return tg::BwdLayout(m, n_q_heads, n_kv_heads).bytes;
}

extern "C" tg_status tg_gated_attention_backward(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                                 int32_t head_dim, const void* q, const void* k, const void* v,
                                                 const int32_t* pos, const float* s_kept, const float* gain,
                                                 float tau, const void* out, const float* lse, const void* dout,
                                                 void* dq, void* dk, void* dv, float* ds_kept, float* dgain,
                                                 float* dtau, void* workspace, size_t workspace_bytes,
                                                 void* stream) {
  using namespace tg;
  if (dtype != TG_F32 && dtype != TG_BF16) return TG_ERR_INVALID_ARG;
  if (m < 0 || m > INT32_MAX || n_q_heads <= 0 || n_kv_heads <= 0) return TG_ERR_INVALID_ARG;
  if (n_q_heads % n_kv_heads != 0) return TG_ERR_INVALID_ARG;
  if ((s_kept == nullptr) != (gain == nullptr)) return TG_ERR_INVALID_ARG;
  if ((s_kept == nullptr) != (ds_kept == nullptr) || (gain == nullptr) != (dgain == nullptr)) return TG_ERR_INVALID_ARG;
  if (!std::isfinite(tau) || !(tau > 0.f)) return TG_ERR_INVALID_ARG;
  if (dtype != TG_BF16 || (head_dim != 64 && head_dim != 128)) return TG_ERR_UNSUPPORTED;
  // the dK/dV kernel's DMA reaches the [Hq][m] float statistics through 32-bit byte offsets
  if (m * n_q_heads >= (int64_t(1) << 29)) return TG_ERR_UNSUPPORTED;
  if (m == 0) return TG_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return TG_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return TG_ERR_INVALID_ARG;
  if (workspace_bytes < BwdLayout(m, n_q_heads, n_kv_heads).bytes) return TG_ERR_WORKSPACE;
#ifdef TG_DEBUG
  if (const tg_status s = debug_check_positions(pos, m, stream); s != TG_OK) return s;
#endif
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out) |
                          reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                          reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
  if (align & 15u) return TG_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int mm = static_cast<int>(m);
  char* ws = static_cast<char*>(workspace);
  return head_dim == 128
             ? attention_backward<128>(mm, n_q_heads, n_kv_heads, q, k, v, pos, s_kept, gain, tau, out, lse, dout,
                                       dq, dk, dv, ds_kept, dgain, dtau, ws, st)
             : attention_backward<64>(mm, n_q_heads, n_kv_heads, q, k, v, pos, s_kept, gain, tau, out, lse, dout,
                                      dq, dk, dv, ds_kept, dgain, dtau, ws, st);
}
