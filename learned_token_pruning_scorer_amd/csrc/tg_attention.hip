// Token-gated attention over the kept tokens.
//
// Each kept token's gate score becomes a bias on the attention logits of the
// layers above the gate, weighted by a learnable per-head gain, and a learnable
// temperature corrects for every query seeing fewer keys (aiproducthub.cn
// "斯坦福伯克利TokenGate 预填充提速11.3倍", section 事件详情; aisight.pl "TokenGate:
// Stanford i Berkeley ...", section "Jak to dziala"; news.chathome.org TokenGate
// article, section "トークンゲート付きアテンションとは").  Adopted form:
//     logit[i,j] = q_i . k_j / (sqrt(d) tau) + gain[h] s_kept[j],   pos[j] <= pos[i]
//
// bf16 kernel (flash attention for CDNA4, wave64):
//  * a workgroup = 4 waves = 32 query rows x 4 (row-block, head) slots; the heads of
//    one workgroup share a key/value head (grouped-query attention), so each K/V
//    tile staged in LDS serves every wave;
//  * K and V tiles of 64 keys go from HBM straight into LDS (global_load_lds, 16
//    bytes per lane: no staging registers, no VALU), double-buffered, with the next
//    tile in flight while the current one is consumed.  Both keep the natural
//    [key][d] layout with the 16-byte chunks of each row XOR-swizzled by the row,
//    chosen so that the operand reads below are bank-conflict free;
//  * scores are computed transposed, S^T = K . Q^T, on v_mfma_f32_32x32x16_bf16: a
//    lane then owns ONE query and 16 keys per 32x32 tile, so the row max / row sum
//    are in-register plus one exchange between the two lane halves;
//  * the key bias enters through the MFMA accumulator: S^T starts from
//    gain[h] s_kept[j] sqrt(d) tau (the bias in q.k units, staged per tile in LDS),
//    so S = q.k + that and the base-2 logit is S * log2(e)/(sqrt(d) tau) -- one FMA
//    with the running max folded in gives the exponent;
//  * lazy rescaling: the running max (and with it O and the row sum) is only moved
//    when a tile's max exceeds it by more than 8 in the base-2 exponent, so P stays
//    below 2^8 and most tiles skip the O rescale;
//  * P^T stays in registers as the B operand of O^T = V^T . P^T; its row sums come
//    from v_dot2_f32_bf16 on the packed bf16 P that the MFMA consumes.  The V^T
//    operand is read from the [key][d] tile with ds_read_b64_tr_b16: each 16-lane
//    group addresses 4 keys x 16 d and lane L receives the 4 keys at d0 + L.  The
//    32x32 accumulator layout leaves each lane half with keys {4h..4h+3,
//    8+4h..8+4h+3} of every 16-key step, which is what two such reads deliver;
//  * workgroups are numbered longest-first (the causal triangle's last query
//    tiles first), and consecutive workgroup ids map to different key/value heads,
//    which the dispatcher spreads round-robin over the 8 XCDs, so each XCD's L2
//    holds the K/V of one head.
#include "tg_common.h"

namespace tg {

constexpr int kAttnWaves = 4;
constexpr int kBN = 64;   // keys per tile

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void gbl_void_t;

// 16 bytes per lane from global memory straight into LDS (lane l -> lds + 16 l; the
// LDS address must be wave-uniform).  The explicit global address-space cast is needed
// for the host compilation pass to accept the call.
__device__ __forceinline__ void lds_load16(const void* gptr, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)const_cast<void*>(gptr), (lds_void_t*)lds, 16, 0, 0);
}


// XOR swizzles of the 16-byte chunks of a tile row (row = key within the tile).
template <int D> struct TileSwz;
template <> struct TileSwz<128> {   // 256-byte rows: every row starts at bank 0
  static __device__ __forceinline__ int k(int r) { return r & 15; }
  static __device__ __forceinline__ int v(int r) { return (r & 3) << 2; }
};
template <> struct TileSwz<64> {    // 128-byte rows: consecutive rows alternate bank halves
  static __device__ __forceinline__ int k(int r) { return (r >> 1) & 7; }
  static __device__ __forceinline__ int v(int r) { return ((r >> 1) & 1) << 2; }
};

template <int D, int HPW>
struct AttnCfg {
  static constexpr int ROWS = 32 * kAttnWaves / HPW;    // query rows per workgroup
  static constexpr int CPR = D / 8;                      // 16-byte chunks per K/V row
  static constexpr int ROWS_PER_LOAD = 64 / CPR;         // rows one wave-wide 1 KiB load covers
  static constexpr int LOADS_PER_WAVE = kBN * CPR / 64 / kAttnWaves;
  static_assert(LOADS_PER_WAVE >= 1, "tile loads");
};

template <int D, int HPW>
__global__ __launch_bounds__(kAttnWaves * 64, 2) void attn_bf16_kernel(
    int m, int hq, int hkv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos, const float* __restrict__ s_kept,
    const float* __restrict__ gain, float c_scale, float bias_scale, float rescale_thr,
    uint16_t* __restrict__ out, int n_qtiles) {
  using C = AttnCfg<D, HPW>;
  using Swz = TileSwz<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][kBN * D];
  __shared__ __attribute__((aligned(16))) float bias_lds[2][HPW][kBN];
  __shared__ __attribute__((aligned(16))) int32_t kpos_lds[2][kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  // workgroup -> (key/value head, head slot, query tile), longest tiles first
  const int group = hq / hkv;
  const int slots_per_kv = group / HPW;
  const int units = hkv * slots_per_kv;
  const int unit = blockIdx.x % units;
  const int qt = n_qtiles - 1 - blockIdx.x / units;
  const int kvh = unit / slots_per_kv;
  const int head0 = kvh * group + (unit % slots_per_kv) * HPW;
  const int hh = wave % HPW;
  const int head = head0 + hh;
  const int q0 = qt * C::ROWS + (wave / HPW) * 32;   // this wave's first query row
  const int row = q0 + l32;
  const bool wave_live = q0 < m;
  const int wave_last = min(m - 1, q0 + 31);         // last valid row of this wave

  // Q fragments: B operand of S^T, lane holds Q[row][16s + 8*half .. +7]
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (row < m)
      qf[s] = *reinterpret_cast<const bf16x8*>(q + ((int64_t)row * hq + head) * D + 16 * s + 8 * half);
    else
      qf[s] = bf16x8{};
  }
  const int32_t qpos = row < m ? (pos ? pos[row] : row) : INT32_MAX;
  const bool use_bias = s_kept != nullptr;
  float hgain[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) hgain[j] = use_bias ? gain[head0 + j] * bias_scale : 0.f;

  // ---- tile loads: K and V global -> LDS directly; bias and positions via registers ----
  // Wave w's load i covers tile rows ROWS_PER_LOAD*(w*LOADS_PER_WAVE + i) + lane/CPR; lane
  // writes physical chunk lane%CPR of its row, i.e. logical chunk (lane%CPR) ^ swizzle(row).
  // Keys past the end are clamped to the last row: the loads stay in bounds, and their
  // position INT32_MAX masks them out (P = 0 exactly).
  int ld_row[C::LOADS_PER_WAVE], ld_kc[C::LOADS_PER_WAVE], ld_vc[C::LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
    const int r = C::ROWS_PER_LOAD * (wave * C::LOADS_PER_WAVE + i) + lane / C::CPR;
    ld_row[i] = r;
    ld_kc[i] = (lane % C::CPR) ^ Swz::k(r);
    ld_vc[i] = (lane % C::CPR) ^ Swz::v(r);
  }
  float sreg = 0.f;
  int32_t preg = INT32_MAX;
  auto issue_tile = [&](int t, int buf) {
    const int kb = t * kBN;
#pragma unroll
    for (int i = 0; i < C::LOADS_PER_WAVE; ++i) {
      const int key = min(kb + ld_row[i], m - 1);
      const int64_t rowoff = ((int64_t)key * hkv + kvh) * D;
      const int slot = (wave * C::LOADS_PER_WAVE + i) * 512;   // 512 bf16 = 1 KiB per wave load
      lds_load16(k + rowoff + 8 * ld_kc[i], &k_lds[buf][slot]);
      lds_load16(v + rowoff + 8 * ld_vc[i], &v_lds[buf][slot]);
    }
    if (tid < kBN) {
      const int key = kb + tid;
      const int kc = min(key, m - 1);
      sreg = use_bias ? s_kept[kc] : 0.f;
      const int32_t pk = pos ? pos[kc] : kc;
      preg = key < m ? pk : INT32_MAX;
    }
  };
  auto finish_tile = [&](int buf) {   // after the tile's loads have completed
    if (tid < kBN) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) bias_lds[buf][j][tid] = sreg * hgain[j];
      kpos_lds[buf][tid] = preg;
    }
  };

  // V^T operand addressing (ds_read_b64_tr_b16): 16-lane group g = lane/16 covers
  // d = 32u + 16(g%2) + (0..15); its lane i addresses key 16*s2 + (8r) + 4*half + i/4 and
  // d columns 32u + 16(g%2) + 4(i%4) .. +3 (half a 16-byte chunk).
  const int gi = lane & 15, gg = lane >> 4;
  const int vkey_lane = 4 * half + (gi >> 2);          // key offset within a 16-key step (r = 0)
  const int vd_lane = 16 * (gg & 1) + 4 * (gi & 3);   // d offset within a 32-wide d tile

  f32x16 oacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[u][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f, neg_mc = 0.f;

  const int rows_end = min(m, (qt + 1) * C::ROWS);
  const int n_tiles = (rows_end + kBN - 1) / kBN;
  issue_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  finish_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int kb = t * kBN;
    if (t + 1 < n_tiles) issue_tile(t + 1, buf ^ 1);   // buf^1 was last read before the previous barrier
    const uint16_t* kt_lds = k_lds[buf];
    const uint16_t* vt_lds = v_lds[buf];

    if (wave_live && kb <= wave_last) {
      // S^T tile: keys kb + 32*kt + (8*g + 4*half + r) for register 4g+r, query = row.
      // The accumulator starts at the key bias (q.k units), so S = q.k + bias.
      f32x16 sacc[2];
      if (use_bias) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 bb = *reinterpret_cast<const f32x4*>(&bias_lds[buf][hh][32 * kt + 8 * g + 4 * half]);
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[kt][4 * g + r] = bb[r];
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int r = 32 * kt + l32;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kt_lds[r * D + 8 * ((2 * s + half) ^ Swz::k(r))]);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kt], 0, 0, 0);
        }
      }
      if ((kb + kBN - 1 > q0) || (kb + kBN > m)) {   // tile straddles the causal edge or the end
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int kk = 32 * kt + 8 * g + 4 * half;
            typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
            const i32x4 kp = *reinterpret_cast<const i32x4*>(&kpos_lds[buf][kk]);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (kp[r] > qpos) sacc[kt][4 * g + r] = -INFINITY;
          }
      }
      float mt = sacc[0][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kt][i]);
      mt = pair_max(mt);
      // lazy rescale: move the running max only when this tile exceeds it by > 2^8
      if (__ballot(mt > m_run + rescale_thr)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c_scale);
        m_run = m_new;
        neg_mc = -m_new * c_scale;
        l_run *= alpha;
#pragma unroll
        for (int u = 0; u < D / 32; ++u)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[u][i] *= alpha;
      }
      // P = exp2(S c - m c), packed to bf16 as the B operand of the P.V step: step s2
      // covers keys 16*s2 .. +15; element e of lane half h is key 16*s2 + (e < 4 ? 4h + e :
      // 8 + 4h + e - 4) = register 8*(s2%2) + e of tile s2/2
      bf16x8 pf[4];
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        u32x4 w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[s2 >> 1][8 * (s2 & 1) + 2 * e2], c_scale, neg_mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[s2 >> 1][8 * (s2 & 1) + 2 * e2 + 1], c_scale, neg_mc));
          // (bit-cast a scalar, not the vector element: clang folds the latter to element 0)
          const uint32_t pk = pack_bf16x2(p0, p1);
          w[e2] = pk;
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, l_run, false);
        }
        pf[s2] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int u = 0; u < D / 32; ++u) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          u32x2 part[2];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int key = 16 * s2 + 8 * r + vkey_lane;
            const int dcol = 32 * u + vd_lane;
            const int off = key * D + 8 * ((dcol >> 3) ^ Swz::v(key)) + (dcol & 7);
            part[r] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(&vt_lds[off])));
          }
          const u32x4 a4 = {part[0][0], part[0][1], part[1][0], part[1][1]};
          oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), pf[s2], oacc[u], 0, 0, 0);
        }
      }
    }
    if (t + 1 < n_tiles) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's share of tile t+1 has landed
      finish_tile(buf ^ 1);
    }
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);   // wave-uniform exchange
  if (row < m) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = out + ((int64_t)row * hq + head) * D;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * u + 8 * g + 4 * half;
        u32x2 pk = {pack_bf16x2(oacc[u][4 * g] * inv, oacc[u][4 * g + 1] * inv),
                    pack_bf16x2(oacc[u][4 * g + 2] * inv, oacc[u][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = pk;
      }
  }
}

// ---------------------------------------------------------------------------------
// float32 path: one thread per (query row, head); K/V tiles of 32 keys in LDS.
// ---------------------------------------------------------------------------------
constexpr int kF32Rows = 64;
constexpr int kF32Keys = 32;

template <int D>
__global__ __launch_bounds__(kF32Rows) void attn_f32_kernel(int m, int hq, int hkv, const float* __restrict__ q,
                                                            const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            const int32_t* __restrict__ pos,
                                                            const float* __restrict__ s_kept,
                                                            const float* __restrict__ gain, float c_scale,
                                                            float* __restrict__ out) {
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  __shared__ float bs[kF32Keys];
  __shared__ int32_t ps[kF32Keys];
  const int head = blockIdx.y;
  const int kvh = head / (hq / hkv);
  const int row = blockIdx.x * kF32Rows + threadIdx.x;
  const bool live = row < m;
  float qv[D], ov[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = live ? q[((int64_t)row * hq + head) * D + c] : 0.f;
    ov[c] = 0.f;
  }
  const int32_t qpos = live ? (pos ? pos[row] : row) : INT32_MAX;
  const float hg = s_kept ? gain[head] * kLog2e : 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int rows_end = min(m, (int)(blockIdx.x + 1) * kF32Rows);
  for (int kb = 0; kb < rows_end; kb += kF32Keys) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kF32Keys * D; idx += kF32Rows) {
      const int r = idx / D, c = idx % D;
      const int key = kb + r;
      ks[r][c] = key < m ? k[((int64_t)key * hkv + kvh) * D + c] : 0.f;
      vs[r][c] = key < m ? v[((int64_t)key * hkv + kvh) * D + c] : 0.f;
    }
    if (threadIdx.x < kF32Keys) {
      const int key = kb + threadIdx.x;
      bs[threadIdx.x] = (s_kept && key < m) ? s_kept[key] * hg : 0.f;
      ps[threadIdx.x] = key < m ? (pos ? pos[key] : key) : INT32_MAX;
    }
    __syncthreads();
    if (!live) continue;
    for (int r = 0; r < kF32Keys; ++r) {
      if (ps[r] > qpos) continue;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], ks[r][c], dot);
      const float t = fmaf(dot, c_scale, bs[r]);
      const float m_new = fmaxf(m_run, t);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      const float p = __builtin_amdgcn_exp2f(t - m_new);
      l_run = fmaf(l_run, alpha, p);
#pragma unroll
      for (int c = 0; c < D; ++c) ov[c] = fmaf(ov[c], alpha, p * vs[r][c]);
      m_run = m_new;
    }
  }
  if (live) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int c = 0; c < D; ++c) out[((int64_t)row * hq + head) * D + c] = ov[c] * inv;
  }
}

template <int D, int HPW>
static tg_status launch_attn_bf16(int m, int hq, int hkv, const void* q, const void* k, const void* v,
                                  const int32_t* pos, const float* s_kept, const float* gain, float c_scale,
                                  float bias_scale, void* out, hipStream_t st) {
  using C = AttnCfg<D, HPW>;
  const int n_qtiles = (m + C::ROWS - 1) / C::ROWS;
  const int64_t grid = (int64_t)n_qtiles * (hq / HPW);
  if (grid > INT32_MAX) return TG_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((attn_bf16_kernel<D, HPW>), dim3((unsigned)grid), dim3(kAttnWaves * 64), 0, st, m, hq, hkv,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), pos, s_kept, gain, c_scale, bias_scale,
                     8.0f / c_scale, static_cast<uint16_t*>(out), n_qtiles);
  TG_CHECK_LAUNCH();
  return TG_OK;
}

template <int D>
static tg_status dispatch_attn_bf16(int m, int hq, int hkv, const void* q, const void* k, const void* v,
                                    const int32_t* pos, const float* s_kept, const float* gain, float c_scale,
                                    float bias_scale, void* out, hipStream_t st) {
  const int group = hq / hkv;
  if (group % 4 == 0)
    return launch_attn_bf16<D, 4>(m, hq, hkv, q, k, v, pos, s_kept, gain, c_scale, bias_scale, out, st);
  if (group % 2 == 0)
    return launch_attn_bf16<D, 2>(m, hq, hkv, q, k, v, pos, s_kept, gain, c_scale, bias_scale, out, st);
  return launch_attn_bf16<D, 1>(m, hq, hkv, q, k, v, pos, s_kept, gain, c_scale, bias_scale, out, st);
}

}  // namespace tg

extern "C" tg_status tg_gated_attention(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t head_dim, const void* q, const void* k, const void* v,
                                        const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                        void* out, void* stream) {
  using namespace tg;
  if (dtype != TG_F32 && dtype != TG_BF16) return TG_ERR_INVALID_ARG;
  if (m < 0 || m > INT32_MAX || n_q_heads <= 0 || n_kv_heads <= 0) return TG_ERR_INVALID_ARG;
  if (n_q_heads % n_kv_heads != 0) return TG_ERR_INVALID_ARG;
  if ((s_kept == nullptr) != (gain == nullptr)) return TG_ERR_INVALID_ARG;
  if (!std::isfinite(tau) || !(tau > 0.f)) return TG_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return TG_ERR_UNSUPPORTED;
  if (m == 0) return TG_OK;
  if (!q || !k || !v || !out) return TG_ERR_INVALID_ARG;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if (align & 15u) return TG_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float c_scale = static_cast<float>(1.4426950408889634 / (std::sqrt((double)head_dim) * (double)tau));
  const float bias_scale = static_cast<float>(std::sqrt((double)head_dim) * (double)tau);   // bias in q.k units
  const int mm = static_cast<int>(m);
  if (dtype == TG_BF16) {
    return head_dim == 128
               ? dispatch_attn_bf16<128>(mm, n_q_heads, n_kv_heads, q, k, v, pos, s_kept, gain, c_scale,
                                         bias_scale, out, st)
               : dispatch_attn_bf16<64>(mm, n_q_heads, n_kv_heads, q, k, v, pos, s_kept, gain, c_scale,
                                        bias_scale, out, st);
  }
  const dim3 grid((mm + kF32Rows - 1) / kF32Rows, n_q_heads);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kF32Rows), 0, st, mm, n_q_heads, n_kv_heads,
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                       pos, s_kept, gain, c_scale, static_cast<float*>(out));
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kF32Rows), 0, st, mm, n_q_heads, n_kv_heads,
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                       pos, s_kept, gain, c_scale, static_cast<float*>(out));
  TG_CHECK_LAUNCH();
  return TG_OK;
}
