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
// bf16 kernel (flash attention for CDNA4, wave64).  On this part the softmax's vector
// work per tile is about as long as the tile's MFMA work, and a wave issues one
// instruction at a time, so the kernel is built to issue as few instructions per
// tile as it can:
//  * a workgroup = 4 waves = 32 query rows x 4 (row-block, head) slots; the heads of
//    one workgroup share a key/value head (grouped-query attention), so each K/V
//    tile staged in LDS serves every wave; two workgroups share a CU;
//  * K and V tiles of 64 keys go from HBM straight into LDS by DMA (global_load_lds,
//    16 bytes per lane), double-buffered, issued from inline asm so that the
//    compiler does not make later LDS reads wait for them; the global address is a
//    scalar base advanced per tile plus per-lane offsets computed once (only the
//    ragged last tile recomputes clamped ones);
//  * 16-byte chunks of each K/V row are XOR-swizzled by the row so that the operand
//    reads are bank-conflict free; every operand read is a per-lane address fixed
//    for the whole loop plus an immediate offset (the loop is unrolled by two so
//    the buffer index is a constant);
//  * scores are computed transposed, S^T = K . Q^T, on v_mfma_f32_32x32x16_bf16: a
//    lane owns ONE query and 16 keys per 32x32 tile, so row max / row sum are
//    in-register plus one exchange between the two lane halves;
//  * Q is pre-scaled by log2(e)/(sqrt(d) tau), and one extra 16-wide MFMA k-step per
//    32 keys adds both the key bias and minus the running max: key rows carry
//    [s_hi, s_hi, s_lo, s_lo, 1, 0..] (the kept score split into two bf16 parts),
//    query columns [cG_hi, cG_lo, cG_hi, cG_lo, -m, 0..] with cG = gain[h] in base-2
//    units.  The accumulator then holds the base-2 logit minus the running max, and
//    P = exp2(S) needs no further vector arithmetic;
//  * lazy rescaling: the running max (kept bf16-exact) moves only when a tile's max
//    exceeds it by more than 8 in the base-2 exponent, so P stays below 2^8 and most
//    tiles skip the O rescale;
//  * operand reads are issued ahead of the work that waits on them: the first two
//    k-steps' K operands before the next tile's DMA, every later k-step's two k-steps
//    before its products, the V^T operands of the first 16 keys (every d tile) before
//    the softmax, each next 16 keys' while the current ones' products run;
//  * the softmax and the P . V products alternate per 16 keys: the exponentials of
//    keys 16 (s + 1) .. 16 s + 31 are issued while the four O tiles' products of the
//    previous 16 keys run (each O tile still accumulates the keys in order);
//  * a wave raises its issue priority (s_setprio) for the vector phase of a tile (mask,
//    max, exponentials and packing, with the P . V products interleaved) and drops it
//    for the S products, so that of the two waves sharing a SIMD the one in its softmax
//    goes first while the other's MFMAs run (about 5% on the 128k workload);
//  * P^T stays in registers as the B operand of O^T = V^T . P^T; its row sums come
//    from v_dot2_f32_bf16 on the packed bf16 P that the MFMA consumes.  The V^T
//    operand is read from the [key][d] tile with ds_read_b64_tr_b16: each 16-lane
//    group addresses 4 keys x 16 d and lane L receives the 4 keys at d0 + L;
//  * workgroups are numbered longest-first (the causal triangle's last query tiles
//    first), and consecutive workgroup ids map to different key/value heads, which
//    the dispatcher spreads round-robin over the 8 XCDs, so each XCD's L2 holds the
//    K/V of one head.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "tg_common.h"

namespace tg {

constexpr int kAttnWaves = 4;
constexpr int kBN = 64;   // keys per tile

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Global -> LDS DMA issued from inline asm: the compiler does not track these, so it
// does not serialise later LDS reads behind them; the kernel waits for them itself
// (wait_dma) before the barrier that publishes a tile.  M0 (the LDS destination,
// wave-uniform) is saved and restored around the issue; the global address is a
// 64-bit scalar base plus a 32-bit per-lane offset.  dma16x2 issues a K and a V piece
// whose LDS destinations are one wave-uniform base plus compile-time byte offsets KM and
// VM, added into M0 inside the asm: the base is then the only LDS address the loop keeps
// in a scalar register (precomputed destinations, one per piece and buffer, outgrow the
// scalar file and are spilled to vector lanes, costing a v_readlane per DMA).
template <uint32_t KM, uint32_t VM>
__device__ __forceinline__ void dma16x2(uint32_t m0base, uint32_t ko, const void* kb, uint32_t vo, const void* vb) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %4\n\t"
               "s_add_u32 m0, %1, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %7\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "s"(m0base), "n"(KM), "v"(ko), "s"(kb), "n"(VM), "v"(vo), "s"(vb) : "memory", "scc");
}
// f(integral_constant<int, I>) for I = 0 .. N-1, each I a compile-time constant
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, uint32_t m0v) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(save) : "s"(m0v), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// XOR swizzles of the 16-byte chunks of a tile row (row = key within the tile).  The
// K swizzle depends only on the row's low bits, so it is the same for rows r and r + 32
// and a lane's K operand address is fixed for the whole loop; the V^T reads see keys
// 4h..4h+3 (+8, +16 s2) in a lane, whose swizzle is likewise fixed per lane.
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
  static constexpr int ROWS = 32 * kAttnWaves / HPW;
  static constexpr int CPR = D / 8;
  static constexpr int ROWS_PER_LOAD = 64 / CPR;
  static constexpr int LPW = kBN * CPR / 64 / kAttnWaves;   // wave loads per tile (per K or V)
  static constexpr int TILE = kBN * D * 2;              // bytes of one K or V tile
  // LDS layout (bytes)
  static constexpr int K0 = 0, V0 = 2 * TILE, SB = 4 * TILE, PB = SB + 2 * kBN * 4, BYTES = PB + 2 * kBN * 4;
};

// Key split: query tile qt's key tiles are cut into runs of `tiles`; run j (grid y) walks
// tiles [j tiles, (j + 1) tiles).  Query tiles with more than one run (qt >= qt0) write
// partial states: part_o [qt - qt0][j][row in tile][head][D], the run's normalised output
// row O_j / l_j in float32, and part_ml (same index) = [m_j, l_j] in float32; tiles = 0
// means no split.
struct AttnSplit {
  int tiles, qt0, jmax;
  float* part_o;
  float* part_ml;
};

// KS key groups per workgroup: group g (waves 4g .. 4g+3, each with its own double-buffered
// K/V region of LDS) walks key tiles t_begin + g, t_begin + g + KS, ...; at the end the
// groups' softmax states are combined through LDS.  RUNS: the query tile's keys are cut into
// runs over grid y (AttnSplit).  KS = 1 without runs is the plain kernel.
template <int D, int HPW, bool BIAS, int KS, bool RUNS>
__global__ __launch_bounds__(kAttnWaves * 64 * KS, 2 / KS) void attn_bf16_kernel(
    int m, int hq, int hkv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ pos, const float* __restrict__ s_kept,
    const float* __restrict__ gain, float c_scale, float bias_scale, float rescale_thr,
    uint16_t* __restrict__ out, float* __restrict__ lse, int n_qtiles, AttnSplit sp) {
  using C = AttnCfg<D, HPW>;
  using S = TileSwz<D>;
  __shared__ __attribute__((aligned(16))) char lds_all[C::BYTES * KS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6) % kAttnWaves;
  const int grp = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6) / kAttnWaves;
  const int half = lane >> 5, l32 = lane & 31;
  char* const lds = lds_all + grp * C::BYTES;   // this key group's buffers
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)lds;

  const int group = hq / hkv;
  const int slots_per_kv = group / HPW;
  const int units = hkv * slots_per_kv;
  const int unit = blockIdx.x % units;
  const int qt = n_qtiles - 1 - blockIdx.x / units;
  const int kvh = unit / slots_per_kv;
  const int head0 = kvh * group + (unit % slots_per_kv) * HPW;
  const int head = head0 + wave % HPW;
  const int q0 = qt * C::ROWS + (wave / HPW) * 32;
  const int row = q0 + l32;
  const bool wave_live = q0 < m;
  const int wave_last = min(m - 1, q0 + 31);

  // key tiles this workgroup walks: all of the query tile's, or one split of them
  const int rows_end = min(m, (qt + 1) * C::ROWS);
  const int n_tiles = (rows_end + kBN - 1) / kBN;
  int t_begin = 0, t_end = n_tiles;
  bool to_part = false;
  if (RUNS) {
    t_begin = blockIdx.y * sp.tiles;
    if (t_begin >= n_tiles) return;   // this query tile has fewer splits (uniform over the workgroup)
    t_end = min(n_tiles, t_begin + sp.tiles);
    to_part = n_tiles > sp.tiles;
  }

  // ---- DMA: per-lane byte offsets relative to the tile's first key (constant across tiles) ----
  const int64_t key_stride = (int64_t)hkv * D * 2;   // bytes between consecutive keys
  uint32_t koff[C::LPW], voff[C::LPW];
  int lrow[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int r = C::ROWS_PER_LOAD * (wave * C::LPW + i) + lane / C::CPR;
    lrow[i] = r;
    koff[i] = (uint32_t)(r * key_stride) + 16 * ((lane % C::CPR) ^ S::k(r));
    voff[i] = (uint32_t)(r * key_stride) + 16 * ((lane % C::CPR) ^ S::v(r));
  }
  const char* kbase = reinterpret_cast<const char*>(k) + (int64_t)kvh * D * 2;
  const char* vbase = reinterpret_cast<const char*>(v) + (int64_t)kvh * D * 2;
  const uint32_t ldsw = lds0 + (uint32_t)(wave * C::LPW * 1024);   // this wave's pieces of a tile
  auto issue_tile = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kb = t * kBN;
    const char* kt_g = kbase + kb * key_stride;
    const char* vt_g = vbase + kb * key_stride;
    if (kb + kBN <= m) {
      static_for<C::LPW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        dma16x2<C::K0 + buf * C::TILE + 1024 * i, C::V0 + buf * C::TILE + 1024 * i>(ldsw, koff[i], kt_g, voff[i], vt_g);
      });
    } else {   // ragged last tile: keys past the end are clamped to the last key
      static_for<C::LPW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int64_t shift = (int64_t)(min(kb + lrow[i], m - 1) - (kb + lrow[i])) * key_stride;
        dma16x2<C::K0 + buf * C::TILE + 1024 * i, C::V0 + buf * C::TILE + 1024 * i>(
            ldsw, (uint32_t)(koff[i] + shift), kt_g, (uint32_t)(voff[i] + shift), vt_g);
      });
    }
    const uint32_t soff = 4u * (uint32_t)(min(kb + lane, m - 1) - kb);
    if (BIAS && wave == 0) dma4(soff, s_kept + kb, lds0 + C::SB + buf * kBN * 4);
    if (wave == 1) {
      if (pos) dma4(soff, pos + kb, lds0 + C::PB + buf * kBN * 4);
      else reinterpret_cast<int32_t*>(lds + C::PB + buf * kBN * 4)[lane] = min(kb + lane, m - 1);
    }
  };
  // the first K/V tile is in flight while Q is loaded and scaled
  if (t_begin + grp < t_end) issue_tile(t_begin + grp, std::integral_constant<int, 0>{});

  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (row < m) {
      const bf16x8 raw = *reinterpret_cast<const bf16x8*>(q + ((int64_t)row * hq + head) * D + 16 * s + 8 * half);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<__bf16>(static_cast<float>(raw[e]) * c_scale);
    } else {
      qf[s] = bf16x8{};
    }
  }
  const int32_t qpos = row < m ? (pos ? pos[row] : row) : INT32_MAX;
  // extra k-step, B operand (lane half 0): [cG_hi, cG_lo, cG_hi, cG_lo, -m, 0, 0, 0] with
  // G = gain sqrt(d) tau (so c G s = gain s in base-2 logit units) and m the running max
  __bf16 cg_hi = static_cast<__bf16>(0.f), cg_lo = static_cast<__bf16>(0.f);
  if (BIAS) {
    const float cG = gain[head] * bias_scale * c_scale;
    cg_hi = static_cast<__bf16>(cG);
    cg_lo = static_cast<__bf16>(cG - static_cast<float>(cg_hi));
  }
  auto make_qext = [&](float mrun) {
    bf16x8 e = bf16x8{};
    if (half == 0) { e[0] = cg_hi; e[1] = cg_lo; e[2] = cg_hi; e[3] = cg_lo; e[4] = static_cast<__bf16>(-mrun); }
    return e;
  };


  // ---- LDS operand addresses (bytes, buffer 0); other buffers/steps are immediate offsets ----
  uint32_t ka[D / 16];   // K A-operand: row l32 (+32 kt), chunk (2s + half) ^ swz
#pragma unroll
  for (int s = 0; s < D / 16; ++s) ka[s] = (uint32_t)(l32 * D * 2 + 16 * ((2 * s + half) ^ S::k(l32)));
  const int gi = lane & 15, gg = lane >> 4;
  const int vkey_lane = 4 * half + (gi >> 2);
  const int vd_lane = 16 * (gg & 1) + 4 * (gi & 3);
  uint32_t va[D / 32];   // V^T operand via ds_read_b64_tr_b16: key vkey_lane (+16 s2 + 8 r), d tile u
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    const int dcol = 32 * u + vd_lane;
    va[u] = (uint32_t)(vkey_lane * D * 2 + 2 * (8 * ((dcol >> 3) ^ S::v(vkey_lane)) + (dcol & 7)));
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[u][i] = 0.f;
  float m_run = 0.f, l_run = 0.f, l_run2 = 0.f;   // m_run: bf16-exact running max (base-2 units)
  bf16x8 qext = make_qext(0.f);

  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  // this group's tiles: tg0 + KS j for j = 0, 1, ... below t_end; every group runs the
  // same number of iterations (and barriers), skipping the tiles past the end
  const int tg0 = t_begin + grp;
  const int n_iter = (t_end - t_begin + KS - 1) / KS;
  auto tt = [&](int j) { return tg0 + KS * j; };

  // bias k-step A operand [s_hi, s_hi, s_lo, s_lo, 1, 0, 0, 0]: the constant upper half stays
  // in registers, each tile writes the lower half
  u32x4 ebias = {0u, 0u, 0x3f80u, 0u};
  constexpr int KPRE = 2;
  auto read_k = [&](int s, int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    return *reinterpret_cast<const bf16x8*>(lds + ka[s] + (C::K0 + buf * C::TILE + kt * 32 * D * 2));
  };
  auto tile = [&](int t, auto bufc, const bf16x8 (&kpre)[KPRE][2]) {
    constexpr int buf = decltype(bufc)::value;
    const int kb = t * kBN;
    if (!(wave_live && kb <= wave_last)) return;
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
    __builtin_amdgcn_s_setprio(0);   // MFMA phase: yield issue slots to a wave in its softmax
    // the tile's key scores (bias k-step) are read first, under the S products
    float sr[2] = {0.f, 0.f};
    if (BIAS) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        sr[kt] = *reinterpret_cast<const float*>(lds + 4 * l32 + (C::SB + buf * kBN * 4 + kt * 128));
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // K operands in a ring of three k-steps, each read two k-steps before its products; the
    // scheduling groups stop the compiler from sinking the reads next to their use
    bf16x8 kr[3][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) { kr[0][kt] = kpre[0][kt]; kr[1][kt] = kpre[1][kt]; }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (s + 2 < D / 16) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) kr[(s + 2) % 3][kt] = read_k(s + 2, kt, bufc);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[s % 3][kt], qf[s], sacc[kt], 0, 0, 0);
      if (s + 2 < D / 16) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // then two MFMAs
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      uint32_t hh = 0, ll = 0;
      if (BIAS) {   // the score as two bf16 parts, each in both halves of a word
        hh = pack_bf16x2(sr[kt], sr[kt]);
        ll = pack_bf16x2(sr[kt] - __uint_as_float(hh & 0xffff0000u), sr[kt] - __uint_as_float(hh & 0xffff0000u));
      }
      // 1.0 at k = 4.  The upper lane half holds k = 8..15, where the B operand is zero, so its
      // (finite) values add nothing and need no masking.
      ebias[0] = hh;
      ebias[1] = ll;
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ebias), qext, sacc[kt], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(2);   // vector phase (mask, max, exp, pack) goes first
    if ((kb + kBN - 1 > q0) || (kb + kBN > m)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int kk = 32 * kt + 8 * g + 4 * half;
          typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
          const i32x4 kp = *reinterpret_cast<const i32x4*>(lds + C::PB + buf * kBN * 4 + 4 * kk);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kp[r] > qpos || kb + kk + r >= m) sacc[kt][4 * g + r] = -INFINITY;
        }
    }
    // a serial chain of three-input maxima (v_max3_f32): 16 instructions for 32 values
    float mt = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), sacc[0][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mt = fmaxf(fmaxf(mt, sacc[0][i]), sacc[0][i + 1]);
    mt = fmaxf(fmaxf(mt, sacc[0][15]), sacc[1][0]);
#pragma unroll
    for (int i = 1; i < 15; i += 2) mt = fmaxf(fmaxf(mt, sacc[1][i]), sacc[1][i + 1]);
    mt = fmaxf(mt, sacc[1][15]);
    // V^T operands (ds_read_b64_tr_b16) of d tile u and keys 16 s2 .. 16 s2 + 15
    auto read_vt = [&](int u, int s2) {
      u32x2 part[2];
#pragma unroll
      for (int r = 0; r < 2; ++r)
        part[r] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(lds + va[u] + (C::V0 + buf * C::TILE + (16 * s2 + 8 * r) * D * 2))));
      return u32x4{part[0][0], part[0][1], part[1][0], part[1][1]};
    };
    u32x4 vcur[D / 32];   // the first 16 keys' operands: read now, consumed after the softmax
#pragma unroll
    for (int u = 0; u < D / 32; ++u) vcur[u] = read_vt(u, 0);
    mt = pair_max(mt);   // tile max of S - m (base-2 units)
    // first tile: adopt its max; later: move the max only when exceeded by > 2^8
    if (t == tg0 || __ballot(mt > rescale_thr)) {
      const float m_new = static_cast<float>(static_cast<__bf16>(m_run + (t == tg0 ? mt : fmaxf(mt, 0.f))));
      const float delta = m_new - m_run;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      m_run = m_new;
      qext = make_qext(m_run);
      l_run *= alpha;
      l_run2 *= alpha;
#pragma unroll
      for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[u][i] *= alpha;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] -= delta;
    }
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      u32x4 w;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float p0 = __builtin_amdgcn_exp2f(sacc[s2 >> 1][8 * (s2 & 1) + 2 * e2]);
        const float p1 = __builtin_amdgcn_exp2f(sacc[s2 >> 1][8 * (s2 & 1) + 2 * e2 + 1]);
        const uint32_t pk = pack_bf16x2(p0, p1);
        w[e2] = pk;
        if (e2 & 1) l_run2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, l_run2, false);
        else l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, l_run, false);
      }
      const bf16x8 pf = __builtin_bit_cast(bf16x8, w);
      u32x4 vnext[D / 32];
      if (s2 < 3) {
#pragma unroll
        for (int u = 0; u < D / 32; ++u) vnext[u] = read_vt(u, s2 + 1);
      }
#pragma unroll
      for (int u = 0; u < D / 32; ++u)
        oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vcur[u]), pf, oacc[u], 0, 0, 0);
      if (s2 < 3) {
#pragma unroll
        for (int u = 0; u < D / 32; ++u) vcur[u] = vnext[u];
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  wait_dma();
  __syncthreads();
  for (int j = 0; j < n_iter; j += 2) {
    {
      bf16x8 kp[KPRE][2];
#pragma unroll
      for (int s = 0; s < KPRE; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) kp[s][kt] = read_k(s, kt, std::integral_constant<int, 0>{});
      if (tt(j + 1) < t_end) issue_tile(tt(j + 1), std::integral_constant<int, 1>{});
      if (KS == 1 || tt(j) < t_end) tile(tt(j), std::integral_constant<int, 0>{}, kp);
    }
    wait_dma();
    __syncthreads();
    if (j + 1 < n_iter) {
      bf16x8 kp[KPRE][2];
#pragma unroll
      for (int s = 0; s < KPRE; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) kp[s][kt] = read_k(s, kt, std::integral_constant<int, 1>{});
      if (tt(j + 2) < t_end) issue_tile(tt(j + 2), std::integral_constant<int, 0>{});
      if (KS == 1 || tt(j + 1) < t_end) tile(tt(j + 1), std::integral_constant<int, 1>{}, kp);
      wait_dma();
      __syncthreads();
    }
  }

  if (KS > 1) {
    // the groups' states (running max, row sum, unnormalised O) meet in group 0; every tile
    // is done (the loop ended on a barrier), so the K/V buffers are free.  A group that saw
    // no key of a row has l = 0 and contributes nothing.
    constexpr int NO = D / 32 * 16;
    float* xs = reinterpret_cast<float*>(lds_all) + wave * ((NO + 2) * 64);
    const float l_own = pair_sum(l_run + l_run2);
    if (grp == 1) {
#pragma unroll
      for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[(16 * u + i) * 64 + lane] = oacc[u][i];
      xs[NO * 64 + lane] = m_run;
      xs[(NO + 1) * 64 + lane] = l_own;
    }
    __syncthreads();
    if (grp != 0) return;
    const float m1 = xs[NO * 64 + lane], l1 = xs[(NO + 1) * 64 + lane];
    const float mn = l1 > 0.f ? (l_own > 0.f ? fmaxf(m_run, m1) : m1) : m_run;
    const float a0 = l_own > 0.f ? __builtin_amdgcn_exp2f(m_run - mn) : 0.f;
    const float a1 = l1 > 0.f ? __builtin_amdgcn_exp2f(m1 - mn) : 0.f;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[u][i] = fmaf(a0, oacc[u][i], a1 * xs[(16 * u + i) * 64 + lane]);
    // l_run + l_run2 is summed over the lane pair below: keep the combined row sum in one half
    l_run = half == 0 ? fmaf(a0, l_own, a1 * l1) : 0.f;
    l_run2 = 0.f;
    m_run = mn;
  }

  const float l_tot = pair_sum(l_run + l_run2);
  if (RUNS && to_part) {
    // one run of a query tile: the run's normalised output row (float32), its running max
    // (base-2 units) and row sum go to the workspace; attn_merge_kernel combines the runs.
    // A wave that saw no key of this run leaves l = 0, which the merge skips.
    if (row < m) {
      const int64_t prow =
          ((int64_t)((qt - sp.qt0) * sp.jmax + (int)blockIdx.y) * C::ROWS + (row - qt * C::ROWS)) * hq + head;
      float* po = sp.part_o + prow * D;
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
      for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * u + 8 * g + 4 * half;
          f32x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = oacc[u][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(po + d0) = o4;
        }
      if (half == 0) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 ml = {m_run, l_tot};
        *reinterpret_cast<f32x2*>(sp.part_ml + prow * 2) = ml;
      }
    }
    return;
  }
  if (row < m) {
    const float inv = 1.0f / l_tot;
    // natural-log log-sum-exp of the row's logits: (m + log2(l)) in base-2 units, times ln 2
    if (lse && half == 0) lse[(int64_t)row * hq + head] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
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

// Combines the runs of the query tiles that were split: for a row and head with run
// states (m_j, l_j, Y_j = O_j / l_j) (m_j in base-2 units),
//     M = max_j m_j,  w_j = 2^(m_j - M) l_j,  out = sum_j w_j Y_j / sum_j w_j,
// over the runs with l_j > 0, in run order.  D / 4 threads per (row, head), each owning 4
// consecutive elements; consecutive threads cover consecutive heads of a row, so reads
// and writes are contiguous.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(int m, int hq, int rows, int row0, AttnSplit sp,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int TPR = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = gid / TPR;
  const int d0 = 4 * (int)(gid % TPR);
  const int row = row0 + (int)(pair / hq);
  const int head = (int)(pair % hq);
  if (row >= m) return;
  const int qt = row / rows;
  const int n_tiles = (min(m, (qt + 1) * rows) + kBN - 1) / kBN;
  const int nj = (n_tiles + sp.tiles - 1) / sp.tiles;
  const int64_t base = ((int64_t)(qt - sp.qt0) * sp.jmax * rows + (row - qt * rows)) * hq + head;
  const int64_t jstride = (int64_t)rows * hq;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  // runs are read JC at a time, every load of a group issued before any is used
  constexpr int JC = 8;
  float mx = -INFINITY;
  for (int j0 = 0; j0 < nj; j0 += JC) {
    f32x2 ml[JC];
#pragma unroll
    for (int c = 0; c < JC; ++c)
      ml[c] = j0 + c < nj ? *reinterpret_cast<const f32x2*>(sp.part_ml + (base + (j0 + c) * jstride) * 2)
                          : f32x2{0.f, 0.f};
#pragma unroll
    for (int c = 0; c < JC; ++c)
      if (ml[c][1] > 0.f) mx = fmaxf(mx, ml[c][0]);
  }
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nj; j0 += JC) {
    f32x2 ml[JC];
    f32x4 y[JC];
#pragma unroll
    for (int c = 0; c < JC; ++c) {
      const int64_t pr = base + (j0 + c) * jstride;
      ml[c] = j0 + c < nj ? *reinterpret_cast<const f32x2*>(sp.part_ml + pr * 2) : f32x2{0.f, 0.f};
      y[c] = j0 + c < nj ? *reinterpret_cast<const f32x4*>(sp.part_o + pr * D + d0) : f32x4{};
    }
#pragma unroll
    for (int c = 0; c < JC; ++c) {
      if (!(ml[c][1] > 0.f)) continue;
      const float w = __builtin_amdgcn_exp2f(ml[c][0] - mx) * ml[c][1];
      l += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, y[c][e], acc[e]);
    }
  }
  const float inv = 1.0f / l;
  const u32x2 pk = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2*>(out + ((int64_t)row * hq + head) * D + d0) = pk;
  if (lse && d0 == 0) lse[(int64_t)row * hq + head] = (mx + __log2f(l)) * 0.69314718055994531f;
}

// Launch plan of the bf16 kernel: heads per workgroup, rows per query tile, key groups per
// workgroup and the key split.  Measured on the workloads' shapes (Hq/Hkv = 16/8, d = 128):
// below a few thousand kept rows the grid cannot fill the GPU with two workgroups per CU,
// and the launch is as long as the longest query tile's walk over its keys; two key groups
// per workgroup halve that walk with no extra traffic (-12% at 1088 rows, -19% at 2112,
// -11% at 4160; +10% at 8256, where the grid is full).  With few head slots per query tile
// (Hq / heads-per-workgroup < 4) even that leaves most CUs idle, and runs of key tiles spread
// over workgroups and merged pay instead (one K/V head, 8256 rows: 169 -> 73 us).
constexpr int kAttnKeyGroupMaxGrid = 768;
constexpr int kAttnMaxSplitQtiles = 4096;

struct AttnPlan {
  int hpw, rows, n_qtiles, ks, tiles, qt0, jmax;
  size_t part_o_bytes, part_ml_bytes;
};

// split_tiles: 0 = automatic, < 0 = never split, > 0 = key tiles per run (one key group).
static AttnPlan plan_attn(int m, int hq, int hkv, int head_dim, int split_tiles) {
  AttnPlan p{};
  const int group = hq / hkv;
  p.hpw = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  p.rows = 32 * kAttnWaves / p.hpw;
  p.n_qtiles = (m + p.rows - 1) / p.rows;
  const int units = hq / p.hpw;
  const int64_t grid = (int64_t)p.n_qtiles * units;
  auto n_tiles = [&](int qt) { return (int)((std::min<int64_t>(m, (int64_t)(qt + 1) * p.rows) + kBN - 1) / kBN); };
  p.ks = 1;
  int tiles = 0;
  if (split_tiles > 0) {
    tiles = split_tiles;
  } else if (grid <= kAttnKeyGroupMaxGrid) {
    if (split_tiles < 0 || units >= 4) {
      p.ks = 2;
    } else if (p.n_qtiles <= kAttnMaxSplitQtiles) {
      int64_t work = 0;
      for (int qt = 0; qt < p.n_qtiles; ++qt) work += n_tiles(qt);
      work *= units;
      tiles = (int)std::max<int64_t>(8, (work + 255) / 256);
    }
  }
  if (m <= 0 || tiles == 0 || p.n_qtiles > kAttnMaxSplitQtiles) return p;
  const int nt_max = n_tiles(p.n_qtiles - 1);
  if (tiles >= nt_max) {   // one run per query tile: as without runs
    p.ks = grid <= kAttnKeyGroupMaxGrid ? 2 : 1;
    return p;
  }
  p.tiles = tiles;
  p.jmax = (nt_max + tiles - 1) / tiles;
  p.qt0 = 0;
  while (n_tiles(p.qt0) <= tiles) ++p.qt0;
  const size_t prow = (size_t)(p.n_qtiles - p.qt0) * p.jmax * p.rows * hq;
  p.part_o_bytes = (prow * head_dim * 4 + 255) & ~size_t(255);
  p.part_ml_bytes = (prow * 2 * 4 + 255) & ~size_t(255);
  return p;
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

template <int D, int HPW, bool BIAS, int KS, bool RUNS>
static void launch_attn_kernel(int m, int hq, int hkv, const void* q, const void* k, const void* v,
                               const int32_t* pos, const float* s_kept, const float* gain, float c_scale,
                               float bias_scale, void* out, float* lse, const AttnPlan& p, const AttnSplit& sp,
                               dim3 grid, hipStream_t st) {
  constexpr float kRescaleThreshold = 8.0f;   // base-2 exponent headroom of P
  hipLaunchKernelGGL((attn_bf16_kernel<D, HPW, BIAS, KS, RUNS>), grid, dim3(kAttnWaves * 64 * KS), 0, st, m, hq, hkv,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), pos, s_kept, gain, c_scale, bias_scale, kRescaleThreshold,
                     static_cast<uint16_t*>(out), lse, p.n_qtiles, sp);
}

template <int D, int HPW>
static tg_status launch_attn_bf16(int m, int hq, int hkv, const void* q, const void* k, const void* v,
                                  const int32_t* pos, const float* s_kept, const float* gain, float c_scale,
                                  float bias_scale, void* out, float* lse, const AttnPlan& p, const AttnSplit& sp,
                                  hipStream_t st) {
  const int64_t gx = (int64_t)p.n_qtiles * (hq / HPW);
  const int gy = p.tiles > 0 ? p.jmax : 1;
  if (gx > INT32_MAX) return TG_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)gx, gy);
  // instances: one key group (plain), one key group with runs, two key groups (no runs)
#define TG_ATTN_LAUNCH(BIAS, KS, RUNS)                                                                         \
  launch_attn_kernel<D, HPW, BIAS, KS, RUNS>(m, hq, hkv, q, k, v, pos, s_kept, gain, c_scale, bias_scale, out, lse, \
                                             p, sp, grid, st)
  if (s_kept) {
    if (p.tiles > 0) TG_ATTN_LAUNCH(true, 1, true);
    else if (p.ks == 2) TG_ATTN_LAUNCH(true, 2, false);
    else TG_ATTN_LAUNCH(true, 1, false);
  } else {
    if (p.tiles > 0) TG_ATTN_LAUNCH(false, 1, true);
    else if (p.ks == 2) TG_ATTN_LAUNCH(false, 2, false);
    else TG_ATTN_LAUNCH(false, 1, false);
  }
#undef TG_ATTN_LAUNCH
  TG_CHECK_LAUNCH();
  if (p.tiles > 0) {
    const int row0 = p.qt0 * p.rows;
    const int64_t threads = (int64_t)(m - row0) * hq * (D / 4);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX) return TG_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(attn_merge_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, m, hq, p.rows, row0, sp,
                       static_cast<uint16_t*>(out), lse);
    TG_CHECK_LAUNCH();
  }
  return TG_OK;
}

template <int D>
static tg_status dispatch_attn_bf16(int m, int hq, int hkv, const void* q, const void* k, const void* v,
                                    const int32_t* pos, const float* s_kept, const float* gain, float c_scale,
                                    float bias_scale, void* out, float* lse, const AttnPlan& p,
                                    const AttnSplit& sp, hipStream_t st) {
  if (p.hpw == 4)
    return launch_attn_bf16<D, 4>(m, hq, hkv, q, k, v, pos, s_kept, gain, c_scale, bias_scale, out, lse, p, sp, st);
  if (p.hpw == 2)
    return launch_attn_bf16<D, 2>(m, hq, hkv, q, k, v, pos, s_kept, gain, c_scale, bias_scale, out, lse, p, sp, st);
  return launch_attn_bf16<D, 1>(m, hq, hkv, q, k, v, pos, s_kept, gain, c_scale, bias_scale, out, lse, p, sp, st);
}

}  // namespace tg

namespace tg {

static tg_status gated_attention(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                 const void* q, const void* k, const void* v, const int32_t* pos,
                                 const float* s_kept, const float* gain, float tau, void* out, float* lse,
                                 int32_t split_tiles, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != TG_F32 && dtype != TG_BF16) return TG_ERR_INVALID_ARG;
  if (m < 0 || m > INT32_MAX || n_q_heads <= 0 || n_kv_heads <= 0) return TG_ERR_INVALID_ARG;
  if (n_q_heads % n_kv_heads != 0) return TG_ERR_INVALID_ARG;
  if ((s_kept == nullptr) != (gain == nullptr)) return TG_ERR_INVALID_ARG;
  if (!std::isfinite(tau) || !(tau > 0.f)) return TG_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return TG_ERR_UNSUPPORTED;
  if (lse && dtype != TG_BF16) return TG_ERR_UNSUPPORTED;
  if (m == 0) return TG_OK;
  if (!q || !k || !v || !out) return TG_ERR_INVALID_ARG;
#ifdef TG_DEBUG
  if (const tg_status s = debug_check_positions(pos, m, stream); s != TG_OK) return s;
#endif
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if (align & 15u) return TG_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float c_scale = static_cast<float>(1.4426950408889634 / (std::sqrt((double)head_dim) * (double)tau));
  const float bias_scale = static_cast<float>(std::sqrt((double)head_dim) * (double)tau);   // bias in q.k units
  const int mm = static_cast<int>(m);
  if (dtype == TG_BF16) {
    const AttnPlan p = plan_attn(mm, n_q_heads, n_kv_heads, head_dim, split_tiles);
    AttnSplit sp{p.tiles, p.qt0, p.jmax, nullptr, nullptr};
    if (p.tiles > 0) {
      if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return TG_ERR_INVALID_ARG;
      if (workspace_bytes < p.part_o_bytes + p.part_ml_bytes) return TG_ERR_WORKSPACE;
      sp.part_o = static_cast<float*>(workspace);
      sp.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.part_o_bytes);
    }
    return head_dim == 128
               ? dispatch_attn_bf16<128>(mm, n_q_heads, n_kv_heads, q, k, v, pos, s_kept, gain, c_scale,
                                         bias_scale, out, lse, p, sp, st)
               : dispatch_attn_bf16<64>(mm, n_q_heads, n_kv_heads, q, k, v, pos, s_kept, gain, c_scale,
                                        bias_scale, out, lse, p, sp, st);
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

}  // namespace tg

extern "C" tg_status tg_gated_attention(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t head_dim, const void* q, const void* k, const void* v,
                                        const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                        void* out, void* stream) {
  return tg::gated_attention(dtype, m, n_q_heads, n_kv_heads, head_dim, q, k, v, pos, s_kept, gain, tau, out,
                             nullptr, -1, nullptr, 0, stream);
}

extern "C" tg_status tg_gated_attention_lse(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                            int32_t head_dim, const void* q, const void* k, const void* v,
                                            const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                            void* out, float* lse, void* stream) {
  if (!lse && m > 0) return TG_ERR_INVALID_ARG;
  return tg::gated_attention(dtype, m, n_q_heads, n_kv_heads, head_dim, q, k, v, pos, s_kept, gain, tau, out, lse,
                             -1, nullptr, 0, stream);
}

extern "C" size_t tg_gated_attention_split_workspace_bytes(int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                                           int32_t head_dim, int32_t split_tiles) {
  if (m <= 0 || m > INT32_MAX || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  const tg::AttnPlan p = tg::plan_attn(static_cast<int>(m), n_q_heads, n_kv_heads, head_dim, split_tiles);
  return p.part_o_bytes + p.part_ml_bytes;
}

extern "C" tg_status tg_gated_attention_split(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                              int32_t head_dim, const void* q, const void* k, const void* v,
                                              const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                              void* out, float* lse, int32_t split_tiles, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  return tg::gated_attention(dtype, m, n_q_heads, n_kv_heads, head_dim, q, k, v, pos, s_kept, gain, tau, out, lse,
                             split_tiles, workspace, workspace_bytes, stream);
}
