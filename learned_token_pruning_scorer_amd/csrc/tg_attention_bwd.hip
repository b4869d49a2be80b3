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
// P is recomputed from the forward's row log-sum-exp.
//
// Kernels (bf16 MFMA 32x32x16, float32 accumulation):
//  * dot: D[i,h] = dO_i . O_i;
//  * dq:  the forward's shape -- a wave owns 32 queries of one head with Q^T and dO^T
//         as fixed B operands; 32-key K/V tiles stream through LDS; S^T = K Q'^T and
//         dP^T = V dO^T give dZ^T in registers (lane = query), and dQ^T += K^T dZ^T
//         reads K^T from the tile with ds_read_b64_tr_b16 exactly as the forward reads V^T;
//  * dkv: the transpose -- a wave owns 32 keys of one key/value head; the workgroup's
//         K' and V rows stay in LDS as the waves' fixed B operands; 32-query Q/dO tiles of
//         every head of the group stream through LDS; S = Q K'^T and dP = dO V^T give
//         dZ in registers (lane = key), dV^T += dO^T P and dK^T += Q^T dZ read dO^T and
//         Q^T from the tiles by transposing LDS reads.  The key-side sums (ds, dgain,
//         dtau) accumulate per lane and are reduced at the end;
//  * reduce: sums the per-workgroup partials of ds (over key/value heads), dgain and
//         dtau in a fixed order, so results are deterministic.
// Every gradient element is written by exactly one workgroup: no float atomics.
#include "tg_common.h"

namespace tg {

constexpr int kBwdWaves = 4;                     // dq workgroup
constexpr int kDkvWaves = 8;                     // dkv workgroup
constexpr int kBwdTile = 32;                     // keys (dq) or queries (dkv) per LDS tile
constexpr int kDkvKeys = 32 * kDkvWaves;         // keys per dkv workgroup
constexpr float kLn2 = 0.69314718055994531f;

typedef short bs16x4 __attribute__((ext_vector_type(4)));

// XOR swizzle of the 16-byte chunks of a tile row (row = key or query in the tile)
template <int D> __device__ __forceinline__ int bwd_swz(int r);
template <> __device__ __forceinline__ int bwd_swz<128>(int r) { return r & 15; }
template <> __device__ __forceinline__ int bwd_swz<64>(int r) { return (r >> 1) & 7; }

// Copies `rows` rows of D bf16 (row stride `ld` elements) into a swizzled LDS tile;
// rows past `valid` repeat the last valid row (their results are masked).
// With a scale, each element is multiplied by it (in float32) and rounded back to bf16.
template <int D>
__device__ __forceinline__ void bwd_load_tile(uint16_t* tile, const uint16_t* __restrict__ src, int64_t ld,
                                              int first, int valid, int rows, float scale = 1.0f,
                                              bool scaled = false) {
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  for (int p = threadIdx.x; p < rows * CPR; p += blockDim.x) {
    const int r = p / CPR, c = p % CPR;
    const int rr = min(first + r, valid - 1);
    u32x4 v = *reinterpret_cast<const u32x4*>(src + (int64_t)rr * ld + 8 * c);
    if (scaled) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = pack_bf16x2(bf16_to_f32(v[e] & 0xffffu) * scale, bf16_to_f32(v[e] >> 16) * scale);
    }
    *reinterpret_cast<u32x4*>(&tile[r * D + 8 * (c ^ bwd_swz<D>(r))]) = v;
  }
}

// A-operand (row) read: row r of a swizzled tile, 16-wide k-step s, lane half h
template <int D>
__device__ __forceinline__ bf16x8 bwd_row(const uint16_t* tile, int r, int s, int half) {
  return *reinterpret_cast<const bf16x8*>(&tile[r * D + 8 * ((2 * s + half) ^ bwd_swz<D>(r))]);
}

// Transposed A operand over the tile's rows for a 16-row k-step s2 and d tile u: lane half
// h receives rows {4h..4h+3, 8+4h..8+4h+3} (+16 s2), the order in which a 32x32
// accumulator's registers leave them, at d = 32u + (lane & 31)
template <int D>
__device__ __forceinline__ bf16x8 bwd_tr(const uint16_t* tile, int s2, int u, int lane) {
  const int half = lane >> 5, gi = lane & 15, gg = lane >> 4;
  const int row_lane = 4 * half + (gi >> 2);
  const int dcol = 32 * u + 16 * (gg & 1) + 4 * (gi & 3);
  u32x2 part[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 16 * s2 + 8 * r + row_lane;
    const int off = row * D + 8 * ((dcol >> 3) ^ bwd_swz<D>(row)) + (dcol & 7);
    part[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                            (__attribute__((address_space(3))) bs16x4*)(&tile[off])));
  }
  const u32x4 a4 = {part[0][0], part[0][1], part[1][0], part[1][1]};
  return __builtin_bit_cast(bf16x8, a4);
}

// bf16 B operand of the 16-row k-step s2 from a 32x32 accumulator
__device__ __forceinline__ bf16x8 pack_acc(const f32x16& a, int s2) {
  u32x4 w;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) w[e2] = pack_bf16x2(a[8 * s2 + 2 * e2], a[8 * s2 + 2 * e2 + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// ---------------------------------------------------------------------------------
// D[i, h] = dO[i, h, :] . O[i, h, :]
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(int rows, const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout, float* __restrict__ dsum) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + (int64_t)r * D + 8 * c);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + (int64_t)r * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_to_f32(a[e] & 0xffffu), bf16_to_f32(b[e] & 0xffffu), acc);
      acc = fmaf(bf16_to_f32(a[e] >> 16), bf16_to_f32(b[e] >> 16), acc);
    }
  }
  dsum[r] = acc;
}

// ---------------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------------
template <int D, int HPW>
__global__ __launch_bounds__(kBwdWaves * 64, 2) void bwd_dq_kernel(
    int m, int hq, int hkv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos, const float* __restrict__ s_kept,
    const float* __restrict__ gain, const float* __restrict__ lse, const float* __restrict__ dsum,
    const uint16_t* __restrict__ dout, float c2, float c_nat, uint16_t* __restrict__ dq, int n_qtiles) {
  constexpr int ROWS = 32 * kBwdWaves / HPW;
  __shared__ __attribute__((aligned(16))) uint16_t k_t[kBwdTile * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_t[kBwdTile * D];
  __shared__ __attribute__((aligned(16))) float s_t[kBwdTile];
  __shared__ __attribute__((aligned(16))) int32_t p_t[kBwdTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int group = hq / hkv;
  const int slots_per_kv = group / HPW;
  const int units = hkv * slots_per_kv;
  const int unit = blockIdx.x % units;
  const int qt = n_qtiles - 1 - blockIdx.x / units;
  const int kvh = unit / slots_per_kv;
  const int head = kvh * group + (unit % slots_per_kv) * HPW + wave % HPW;
  const int q0 = qt * ROWS + (wave / HPW) * 32;
  const int row = q0 + l32;
  const bool wave_live = q0 < m;
  const int wave_last = min(m - 1, q0 + 31);
  const bool live_row = row < m;

  // fixed B operands: Q' = c2 Q (base-2 logits) and dO, lane = query row
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (live_row) {
      const bf16x8 raw = *reinterpret_cast<const bf16x8*>(q + ((int64_t)row * hq + head) * D + 16 * s + 8 * half);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<__bf16>(static_cast<float>(raw[e]) * c2);
      df[s] = *reinterpret_cast<const bf16x8*>(dout + ((int64_t)row * hq + head) * D + 16 * s + 8 * half);
    } else {
      qf[s] = bf16x8{};
      df[s] = bf16x8{};
    }
  }
  const float lse2 = live_row ? lse[(int64_t)row * hq + head] * kLog2e : 0.f;
  const float dval = live_row ? dsum[(int64_t)row * hq + head] : 0.f;
  const int32_t qpos = live_row ? (pos ? pos[row] : row) : INT32_MIN;
  const float g2 = s_kept ? gain[head] * kLog2e : 0.f;

  f32x16 dqa[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[u][i] = 0.f;

  const int rows_end = min(m, (qt + 1) * ROWS);
  const int n_tiles = (rows_end + kBwdTile - 1) / kBwdTile;
  for (int t = 0; t < n_tiles; ++t) {
    const int kb = t * kBwdTile;
    __syncthreads();   // the previous tile is no longer read
    bwd_load_tile<D>(k_t, k + (int64_t)kvh * D, (int64_t)hkv * D, kb, m, kBwdTile);
    bwd_load_tile<D>(v_t, v + (int64_t)kvh * D, (int64_t)hkv * D, kb, m, kBwdTile);
    if (tid < kBwdTile) {
      const int key = kb + tid, kc = min(key, m - 1);
      s_t[tid] = s_kept ? s_kept[kc] : 0.f;
      p_t[tid] = key < m ? (pos ? pos[kc] : kc) : INT32_MAX;
    }
    __syncthreads();
    if (!(wave_live && kb <= wave_last)) continue;
    f32x16 sa, da;
#pragma unroll
    for (int i = 0; i < 16; ++i) { sa[i] = 0.f; da[i] = 0.f; }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_row<D>(k_t, l32, s, half), qf[s], sa, 0, 0, 0);
      da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_row<D>(v_t, l32, s, half), df[s], da, 0, 0, 0);
    }
    // register e holds key j = 8 (e/4) + 4 half + e%4 of the tile, query = this lane's row
    f32x16 dz;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j0 = 8 * g + 4 * half;
      const f32x4 sv = *reinterpret_cast<const f32x4*>(&s_t[j0]);
      typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
      const i32x4 kp = *reinterpret_cast<const i32x4*>(&p_t[j0]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * g + r;
        const float p = kp[r] <= qpos ? __builtin_amdgcn_exp2f(sa[e] + g2 * sv[r] - lse2) : 0.f;
        dz[e] = p * (da[e] - dval);
      }
    }
    const bf16x8 z0 = pack_acc(dz, 0), z1 = pack_acc(dz, 1);
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      dqa[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(k_t, 0, u, lane), z0, dqa[u], 0, 0, 0);
      dqa[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(k_t, 1, u, lane), z1, dqa[u], 0, 0, 0);
    }
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
// dK, dV and the key-side partial sums
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kDkvWaves * 64, 1) void bwd_dkv_kernel(
    int m, int hq, int hkv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos, const float* __restrict__ s_kept,
    const float* __restrict__ gain, const float* __restrict__ lse, const float* __restrict__ dsum,
    const uint16_t* __restrict__ dout, float c2, float c_nat, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ ds_part, float* __restrict__ dgain_part, float* __restrict__ dtau_part, int n_kblocks) {
  __shared__ __attribute__((aligned(16))) uint16_t k_b[kDkvKeys * D];     // this workgroup's K' = c2 K rows
  __shared__ __attribute__((aligned(16))) uint16_t v_b[kDkvKeys * D];     // and V rows
  __shared__ __attribute__((aligned(16))) uint16_t q_t[kBwdTile * D];
  __shared__ __attribute__((aligned(16))) uint16_t o_t[kBwdTile * D];     // dO tile
  __shared__ __attribute__((aligned(16))) float lse_t[kBwdTile];
  __shared__ __attribute__((aligned(16))) float d_t[kBwdTile];
  __shared__ __attribute__((aligned(16))) int32_t p_t[kBwdTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int group = hq / hkv;
  const int kvh = blockIdx.x % hkv;
  const int kblk = blockIdx.x / hkv;              // longest (earliest keys) first
  const int kb0 = kblk * kDkvKeys;
  const int kw0 = kb0 + 32 * wave;                // this wave's first key
  const int key = kw0 + l32;
  const bool live_key = key < m;
  const int kc = min(key, m - 1);
  const int32_t kpos = live_key ? (pos ? pos[kc] : kc) : INT32_MAX;
  const float sk = s_kept ? s_kept[kc] : 0.f;

  // the workgroup's keys: K' = c2 K and V, read by each wave as its fixed B operands
  bwd_load_tile<D>(k_b, k + (int64_t)kvh * D, (int64_t)hkv * D, kb0, m, kDkvKeys, c2, true);
  bwd_load_tile<D>(v_b, v + (int64_t)kvh * D, (int64_t)hkv * D, kb0, m, kDkvKeys);

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dka[u][i] = 0.f; dva[u][i] = 0.f; }
  float ds_acc = 0.f, dtau_acc = 0.f;

  const int first_tile = kb0 / kBwdTile;          // queries before the first key see none of them
  const int n_tiles = (m + kBwdTile - 1) / kBwdTile;
  for (int hh = 0; hh < group; ++hh) {
    const int head = kvh * group + hh;
    const float g2 = s_kept ? gain[head] * kLog2e : 0.f;
    const float bias2 = g2 * sk;
    float col = 0.f;   // sum over queries of dZ for this lane's key and this head
    for (int t = first_tile; t < n_tiles; ++t) {
      const int qb = t * kBwdTile;
      __syncthreads();   // the previous tile is no longer read
      bwd_load_tile<D>(q_t, q + (int64_t)head * D, (int64_t)hq * D, qb, m, kBwdTile);
      bwd_load_tile<D>(o_t, dout + (int64_t)head * D, (int64_t)hq * D, qb, m, kBwdTile);
      if (tid < kBwdTile) {
        const int qi = qb + tid, qc = min(qi, m - 1);
        lse_t[tid] = lse[(int64_t)qc * hq + head] * kLog2e;
        d_t[tid] = dsum[(int64_t)qc * hq + head];
        p_t[tid] = qi < m ? (pos ? pos[qc] : qc) : INT32_MIN;
      }
      __syncthreads();
      if (qb + kBwdTile - 1 < kw0 || kw0 >= m) continue;   // no query of the tile sees these keys
      f32x16 sa, da;
#pragma unroll
      for (int i = 0; i < 16; ++i) { sa[i] = 0.f; da[i] = 0.f; }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_row<D>(q_t, l32, s, half),
                                                     bwd_row<D>(k_b, 32 * wave + l32, s, half), sa, 0, 0, 0);
        da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_row<D>(o_t, l32, s, half),
                                                     bwd_row<D>(v_b, 32 * wave + l32, s, half), da, 0, 0, 0);
        if (s % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // bounds the operand reads in flight
      }
      // register e holds query i = 8 (e/4) + 4 half + e%4 of the tile, key = this lane's.
      // P is finished and fed to dV before dZ is formed, so the two never share registers.
      typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
      f32x16 p;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i0 = 8 * g + 4 * half;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&lse_t[i0]);
        const i32x4 qp = *reinterpret_cast<const i32x4*>(&p_t[i0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          p[e] = kpos <= qp[r] ? __builtin_amdgcn_exp2f(sa[e] + bias2 - lv[r]) : 0.f;
        }
      }
      {
        const bf16x8 p0 = pack_acc(p, 0), p1 = pack_acc(p, 1);
#pragma unroll
        for (int u = 0; u < D / 32; ++u) {
          dva[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(o_t, 0, u, lane), p0, dva[u], 0, 0, 0);
          dva[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(o_t, 1, u, lane), p1, dva[u], 0, 0, 0);
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(&d_t[8 * g + 4 * half]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          const float z = p[e] * (da[e] - dv4[r]);
          col += z;
          dtau_acc = fmaf(z, sa[e], dtau_acc);
          da[e] = z;   // da now holds dZ
        }
      }
      const bf16x8 z0 = pack_acc(da, 0), z1 = pack_acc(da, 1);
#pragma unroll
      for (int u = 0; u < D / 32; ++u) {
        dka[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(q_t, 0, u, lane), z0, dka[u], 0, 0, 0);
        dka[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bwd_tr<D>(q_t, 1, u, lane), z1, dka[u], 0, 0, 0);
      }
    }
    // this head's key-side sums: both lane halves hold parts of the same key's column
    col += swap_halves(col);
    ds_acc = fmaf(s_kept ? gain[head] : 0.f, col, ds_acc);
    float gsum = (half == 0 && live_key) ? sk * col : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) gsum += __shfl_xor(gsum, o, 64);
    if (lane == 0) dgain_part[((int64_t)head * n_kblocks + kblk) * kDkvWaves + wave] = gsum;
  }
  if (live_key) {
    if (half == 0) ds_part[(int64_t)kvh * m + key] = ds_acc;
    uint16_t* krow = dk + ((int64_t)key * hkv + kvh) * D;
    uint16_t* vrow = dv + ((int64_t)key * hkv + kvh) * D;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * u + 8 * g + 4 * half;
        const u32x2 kk = {pack_bf16x2(dka[u][4 * g] * c_nat, dka[u][4 * g + 1] * c_nat),
                          pack_bf16x2(dka[u][4 * g + 2] * c_nat, dka[u][4 * g + 3] * c_nat)};
        const u32x2 vv = {pack_bf16x2(dva[u][4 * g], dva[u][4 * g + 1]),
                          pack_bf16x2(dva[u][4 * g + 2], dva[u][4 * g + 3])};
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
// fixed-order sums of the partials
// ---------------------------------------------------------------------------------
// Blocks 0 .. ceil(m/256)-1 sum ds over the key/value heads; the last block sums dgain
// (one wave per head) and dtau (the whole block).  Each sum's order is fixed by the
// launch shape alone, so results are bitwise reproducible.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(int m, int hq, int hkv, int n_kblocks, int n_dkv_blocks,
                                                          const float* __restrict__ ds_part,
                                                          const float* __restrict__ dgain_part,
                                                          const float* __restrict__ dtau_part, float dtau_scale,
                                                          float* __restrict__ ds, float* __restrict__ dgain,
                                                          float* __restrict__ dtau) {
  __shared__ float red[256];
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per_head = n_kblocks * kDkvWaves;
  if (dgain)
    for (int h = wave; h < hq; h += 4) {
      float acc = 0.f;
      for (int i = lane; i < per_head; i += 64) acc += dgain_part[(int64_t)h * per_head + i];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (lane == 0) dgain[h] = acc;
    }
  if (dtau) {
    float acc = 0.f;
    for (int i = threadIdx.x; i < n_dkv_blocks * kDkvWaves; i += 256) acc += dtau_part[i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
      __syncthreads();
    }
    if (threadIdx.x == 0) *dtau = red[0] * dtau_scale;
  }
}

struct BwdLayout {
  size_t dsum, ds_part, dgain_part, dtau_part, bytes;
  BwdLayout(int64_t m, int64_t hq, int64_t hkv) {
    const int64_t nkb = (m + kDkvKeys - 1) / kDkvKeys;
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    dsum = 0;
    ds_part = up(dsum + (size_t)m * hq * 4);
    dgain_part = up(ds_part + (size_t)hkv * m * 4);
    dtau_part = up(dgain_part + (size_t)hq * nkb * kDkvWaves * 4);
    bytes = up(dtau_part + (size_t)hkv * nkb * kDkvWaves * 4);
  }
};

template <int D, int HPW>
static void launch_bwd_dq(int m, int hq, int hkv, const void* q, const void* k, const void* v, const int32_t* pos,
                          const float* s_kept, const float* gain, const float* lse, const float* dsum,
                          const void* dout, float c2, float c_nat, void* dq, hipStream_t st) {
  constexpr int ROWS = 32 * kBwdWaves / HPW;
  const int n_qtiles = (m + ROWS - 1) / ROWS;
  const int grid = n_qtiles * (hq / HPW);
  hipLaunchKernelGGL((bwd_dq_kernel<D, HPW>), dim3(grid), dim3(kBwdWaves * 64), 0, st, m, hq, hkv,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), pos, s_kept, gain, lse, dsum,
                     static_cast<const uint16_t*>(dout), c2, c_nat, static_cast<uint16_t*>(dq), n_qtiles);
}

template <int D>
static tg_status attention_backward(int m, int hq, int hkv, const void* q, const void* k, const void* v,
                                    const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                    const void* out, const float* lse, const void* dout, void* dq, void* dk,
                                    void* dv, float* ds, float* dgain, float* dtau, char* ws, hipStream_t st) {
  const BwdLayout L(m, hq, hkv);
  float* dsum = reinterpret_cast<float*>(ws + L.dsum);
  float* ds_part = reinterpret_cast<float*>(ws + L.ds_part);
  float* dgain_part = reinterpret_cast<float*>(ws + L.dgain_part);
  float* dtau_part = reinterpret_cast<float*>(ws + L.dtau_part);
  const double sd = std::sqrt((double)D) * (double)tau;
  const float c2 = static_cast<float>(1.4426950408889634 / sd);   // base-2 logit per unit q.k
  const float c_nat = static_cast<float>(1.0 / sd);

  const int rows = m * hq;
  hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3((rows + 255) / 256), dim3(256), 0, st, rows,
                     static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), dsum);
  const int group = hq / hkv;
  if (group % 4 == 0)
    launch_bwd_dq<D, 4>(m, hq, hkv, q, k, v, pos, s_kept, gain, lse, dsum, dout, c2, c_nat, dq, st);
  else if (group % 2 == 0)
    launch_bwd_dq<D, 2>(m, hq, hkv, q, k, v, pos, s_kept, gain, lse, dsum, dout, c2, c_nat, dq, st);
  else
    launch_bwd_dq<D, 1>(m, hq, hkv, q, k, v, pos, s_kept, gain, lse, dsum, dout, c2, c_nat, dq, st);
  const int n_kblocks = (m + kDkvKeys - 1) / kDkvKeys;
  const int n_dkv = n_kblocks * hkv;
  hipLaunchKernelGGL((bwd_dkv_kernel<D>), dim3(n_dkv), dim3(kDkvWaves * 64), 0, st, m, hq, hkv,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), pos, s_kept, gain, lse, dsum,
                     static_cast<const uint16_t*>(dout), c2, c_nat, static_cast<uint16_t*>(dk),
                     static_cast<uint16_t*>(dv), ds_part, dgain_part, dtau_part, n_kblocks);
  // dtau = -(1/tau) sum dZ . (q.k / (sqrt(d) tau)); the kernel summed dZ . (c2 q.k)
  const float dtau_scale = static_cast<float>(-kLn2 / (double)tau);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((m + 255) / 256 + 1), dim3(256), 0, st, m, hq, hkv, n_kblocks, n_dkv,
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
  if (m * n_q_heads > INT32_MAX) return TG_ERR_UNSUPPORTED;   // row indices are 32-bit
  if (m == 0) return TG_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return TG_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return TG_ERR_INVALID_ARG;
  if (workspace_bytes < BwdLayout(m, n_q_heads, n_kv_heads).bytes) return TG_ERR_WORKSPACE;
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
