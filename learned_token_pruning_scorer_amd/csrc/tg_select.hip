// Document-only top-K selection with exact ties, compacted in position order.
//
// TokenGate keeps the K best-scoring tokens of the prunable document and never
// prunes the question (aiproducthub.cn "斯坦福伯克利TokenGate 预填充提速11.3倍",
// section 事件详情; aisight.pl "TokenGate: Stanford i Berkeley ...", section
// "Jak to dziala").
//
// One launch does the whole selection.  At most 64 workgroups each own a
// contiguous chunk of positions (held in registers as keys); they are all
// resident at once and meet at counted grid barriers between phases.  A barrier
// is one device-scope atomic per workgroup plus polling -- no cache write-back
// fence: every value that crosses workgroups (histogram bins, chunk counts) is
// itself a device-scope atomic, and each thread drains its own atomics before
// its workgroup arrives.  The wait is bounded, so a grid that is not fully
// resident (the device shared with other work) cannot hang; a timeout is flagged
// in the workspace.  Phases:
//   1-3. radix select over the order-preserving uint32 score keys, three digits
//        (bits 31..21, 20..10, 9..0): each workgroup histograms its chunk's
//        document keys that carry the prefix fixed so far into LDS, merges the
//        non-zero bins into a global histogram with atomics, and after the barrier
//        every workgroup scans that histogram from the top to fix the next digit.
//        The result is the threshold key T (the K-th largest document key) and
//        need_eq, how many keys equal to T are kept;
//   4.   compaction: position i is kept iff it lies outside the document, or its
//        key > T, or key == T and fewer than need_eq equal keys precede it.  Its
//        output slot is base_before(i) + min(eq_before(i), need_eq), from two
//        prefix counts (positions kept outright, document keys equal to T); the
//        per-workgroup totals are exchanged at one more barrier.
// Ties therefore go to the lowest positions and the output is ascending.
//
// Several budgets in one launch (one gate serves every budget: aiproducthub.cn, section
// 事件详情; aisight.pl, section "Wyniki"): the first digit's histogram is shared; the
// later digits, the threshold and the compaction run per budget at the same barriers,
// each budget writing its own kept list.
//
// Random selector (the pages' random-K ablation: aiproducthub.cn, section 事件详情;
// news.chathome.org, section "ベンチマーク"): the same selection on keys drawn per
// position from SplitMix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom Number
// Generators", OOPSLA 2014): the key of position i is the high half of the i-th output of
// the stream seeded with `seed`.  The K largest of independent uniform keys form a
// uniformly random K-subset of the document.
#include <atomic>

#include "tg_common.h"

namespace tg {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelMaxBlocks = 64;             // barrier cost grows with the number of workgroups
constexpr int kSelPosPerBlock = 1024;         // target chunk per workgroup (measured: 16384 positions
                                              // take 15.6 us in 16 chunks, 17.3 us in 8)
constexpr int kSelRegKeys = 4;                // keys per thread kept in registers across phases
constexpr int kSelMaxBins = 2048;
constexpr int kSelMaxBudgets = 8;
constexpr uint32_t kSpinLimit = 1u << 22;     // bounded barrier wait (never reached when co-resident)

struct SelState {       // head of the workspace (64 bytes)
  uint32_t barrier;     // barrier arrivals of the current call (reset by the last workgroup out)
  uint32_t exit;        // workgroups finished
  uint32_t timeout;     // set if a barrier wait ever gave up
  uint32_t pad[13];
};

struct SelLayout {
  static constexpr size_t state = 0;
  static constexpr size_t hist0 = 64;                                         // [2048] first digit, shared
  static constexpr size_t hist1 = hist0 + 2048 * 4;                           // [budget][2048]
  static constexpr size_t hist2 = hist1 + kSelMaxBudgets * 2048 * 4;          // [budget][1024]
  static constexpr size_t counts = hist2 + kSelMaxBudgets * 1024 * 4;         // [block][budget][2]
  static constexpr size_t bytes = (counts + kSelMaxBlocks * kSelMaxBudgets * 2 * 4 + 255) & ~size_t(255);
};

// Budgets of one launch.  mode 0: keep no document token; 1: keep the whole document;
// 2: select k_eff = min(k, D) of it.  Budget b's kept list starts at kept + out_off[b].
struct SelBudgets {
  int nk;
  int mode[kSelMaxBudgets];
  uint32_t k_eff[kSelMaxBudgets];
  uint32_t m[kSelMaxBudgets];
  int64_t out_off[kSelMaxBudgets];
};

// Where the keys come from: the scores, or SplitMix64 outputs of (seed, position).
struct SelKeys {
  const float* scores;
  uint64_t seed;
  int random;
};

__device__ __forceinline__ uint32_t random_key(uint64_t seed, int i) {
  uint64_t z = seed + static_cast<uint64_t>(i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return static_cast<uint32_t>(z >> 32);
}

__device__ __forceinline__ uint32_t key_at(const SelKeys& src, int i) {
  return src.random ? random_key(src.seed, i) : score_key(src.scores[i]);
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this thread's own outstanding memory operations (the device-scope
// atomics it issued) have completed.
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// All workgroups of the grid wait here until `target` arrivals have been counted.
__device__ __forceinline__ void grid_barrier(SelState* st, uint32_t target) {
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&st->barrier, 1u);
    uint32_t spins = 0;
    while (ld_agent(&st->barrier) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {             // only if the grid is not fully resident; never hang
        atomicOr(&st->timeout, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Exclusive scan of one value per thread over the workgroup; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* sh /*[kSelWaves]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  uint32_t wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t s = sh[w];
    wbase += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* sh /*[kSelWaves]*/) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) tot += sh[w];
  __syncthreads();
  return tot;
}

// NKM: the most budgets one instantiation handles (1 for the single-budget calls).
template <int NKM>
__global__ __launch_bounds__(kSelThreads) void sel_fused_kernel(SelKeys src, int n, int doc_begin, int doc_end,
                                                                SelBudgets bud, int chunk, char* ws,
                                                                int32_t* __restrict__ kept) {
  __shared__ uint32_t lh[NKM * kSelMaxBins];
  __shared__ uint32_t sh[kSelWaves];
  __shared__ uint32_t sh_prefix, sh_rank;
  SelState* st = reinterpret_cast<SelState*>(ws + SelLayout::state);
  uint32_t* hist0 = reinterpret_cast<uint32_t*>(ws + SelLayout::hist0);
  uint32_t* hist1 = reinterpret_cast<uint32_t*>(ws + SelLayout::hist1);
  uint32_t* hist2 = reinterpret_cast<uint32_t*>(ws + SelLayout::hist2);
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + SelLayout::counts);
  const int tid = threadIdx.x;
  const uint32_t G = gridDim.x;
  const int c0 = blockIdx.x * chunk;
  const int c1 = min(n, c0 + chunk);
  const int nk = NKM == 1 ? 1 : bud.nk;

  // The chunk's keys: position c0 + tid + 512*r is keys[r], kept in registers when the
  // chunk fits (up to 64 x 512 x 4 = 131072 positions); larger chunks recompute them.
  const bool in_regs = c1 - c0 <= kSelThreads * kSelRegKeys;
  uint32_t keys[kSelRegKeys];
#pragma unroll
  for (int r = 0; r < kSelRegKeys; ++r) {
    const int i = c0 + tid + r * kSelThreads;
    keys[r] = (in_regs && i < c1) ? key_at(src, i) : 0u;
  }
  // f(i, key) for every position of the chunk held by this thread
  auto for_chunk = [&](auto&& f) {
    if (in_regs) {
#pragma unroll
      for (int r = 0; r < kSelRegKeys; ++r) {
        const int i = c0 + tid + r * kSelThreads;
        if (i < c1) f(i, keys[r]);
      }
    } else {
      for (int i = c0 + tid; i < c1; i += kSelThreads) f(i, key_at(src, i));
    }
  };

  // per budget: digit prefix fixed so far and rank still to find; at the end, the
  // threshold key T and the number of keys equal to T that are kept
  uint32_t prefix[NKM], rank[NKM];
  bool any_select = false;
#pragma unroll
  for (int b = 0; b < NKM; ++b) {
    prefix[b] = 0u;
    rank[b] = b < nk ? bud.k_eff[b] : 0u;
    any_select |= b < nk && bud.mode[b] == 2;
  }
  uint32_t barriers = 0;
  if (any_select) {
#pragma unroll 1
    for (int p = 0; p < 3; ++p) {
      const int shift = p == 0 ? 21 : (p == 1 ? 10 : 0);
      const int bits = p == 2 ? 10 : 11;
      const uint32_t bins = 1u << bits;
      const int nh = p == 0 ? 1 : nk;   // the first digit's histogram serves every budget
      uint32_t* hist = p == 0 ? hist0 : (p == 1 ? hist1 : hist2);
      for (uint32_t i = tid; i < nh * bins; i += kSelThreads) lh[i] = 0u;
      __syncthreads();
      for_chunk([&](int i, uint32_t key) {
        if (i < doc_begin || i >= doc_end) return;
        if (p == 0) {
          atomicAdd(&lh[key >> shift], 1u);
        } else {
#pragma unroll
          for (int b = 0; b < NKM; ++b)
            if (b < nk && bud.mode[b] == 2 && (key >> (shift + bits)) == prefix[b])
              atomicAdd(&lh[b * bins + ((key >> shift) & (bins - 1))], 1u);
        }
      });
      __syncthreads();
      for (uint32_t i = tid; i < nh * bins; i += kSelThreads)
        if (lh[i]) atomicAdd(&hist[i], lh[i]);
      grid_barrier(st, ++barriers * G);
      // every workgroup finished reading the previous digit's histograms before this barrier
      if (p == 1 && blockIdx.x == 0)
        for (uint32_t i = tid; i < 2048u; i += kSelThreads) hist0[i] = 0u;
      if (p == 2 && blockIdx.x == 0)
        for (uint32_t i = tid; i < nk * 2048u; i += kSelThreads) hist1[i] = 0u;
#pragma unroll
      for (int b = 0; b < NKM; ++b) {   // uniform
        if (!(b < nk && bud.mode[b] == 2)) continue;
        const uint32_t* hb = hist + (p == 0 ? 0u : b * bins);
        // walk the bins from the top (largest keys) to the one holding the rank-th key
        const uint32_t per = bins / kSelThreads;   // 4 or 2
        uint32_t c[4] = {0u, 0u, 0u, 0u};
        uint32_t local = 0u;
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
          if (q < per) {
            c[q] = ld_agent(&hb[bins - 1 - (tid * per + q)]);
            local += c[q];
          }
        }
        uint32_t total;
        uint32_t above = block_excl_scan(local, &total, sh);
        if (above < rank[b] && rank[b] <= above + local) {
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q) {
            if (q < per) {
              if (rank[b] <= above + c[q]) {
                sh_prefix = (prefix[b] << bits) | (bins - 1 - (tid * per + q));
                sh_rank = rank[b] - above;
                break;
              }
              above += c[q];
            }
          }
        }
        __syncthreads();
        prefix[b] = sh_prefix;
        rank[b] = sh_rank;
        __syncthreads();   // sh_prefix / sh_rank are reused by the next budget
      }
    }
  }
  uint32_t T[NKM], need[NKM];
#pragma unroll
  for (int b = 0; b < NKM; ++b) {
    const int md = b < nk ? bud.mode[b] : 0;
    T[b] = md == 2 ? prefix[b] : (md == 1 ? 0u : 0xffffffffu);   // mode 0: no key reaches 0xffffffff
    need[b] = md == 2 ? rank[b] : (md == 1 ? 0xffffffffu : 0u);
  }

  // ---- compaction ----
  // flags of a position: fb = kept outright (outside the document, or key > T); fe = key == T
  auto flags = [&](uint32_t Tb, int i, uint32_t key, uint32_t* fb, uint32_t* fe) {
    const bool doc = i >= doc_begin && i < doc_end;
    *fb = (!doc || key > Tb) ? 1u : 0u;
    *fe = (doc && key == Tb) ? 1u : 0u;
  };
#pragma unroll
  for (int b = 0; b < NKM; ++b) {
    if (b >= nk) continue;
    uint32_t nb = 0u, ne = 0u;
    for_chunk([&](int i, uint32_t key) {
      uint32_t fb, fe;
      flags(T[b], i, key, &fb, &fe);
      nb += fb;
      ne += fe;
    });
    nb = block_sum(nb, sh);
    ne = block_sum(ne, sh);
    if (tid == 0) {
      st_agent(&counts[2 * (blockIdx.x * kSelMaxBudgets + b)], nb);
      st_agent(&counts[2 * (blockIdx.x * kSelMaxBudgets + b) + 1], ne);
    }
  }
  grid_barrier(st, ++barriers * G);
  if (any_select && blockIdx.x == 0)
    for (int i = tid; i < nk * 1024; i += kSelThreads) hist2[i] = 0u;
#pragma unroll
  for (int b = 0; b < NKM; ++b) {
    if (b >= nk) continue;
    uint32_t pb = 0u, pe = 0u;
    for (uint32_t w = tid; w < blockIdx.x; w += kSelThreads) {
      pb += ld_agent(&counts[2 * (w * kSelMaxBudgets + b)]);
      pe += ld_agent(&counts[2 * (w * kSelMaxBudgets + b) + 1]);
    }
    uint32_t base_before = block_sum(pb, sh);
    uint32_t eq_before = block_sum(pe, sh);
    int32_t* out = kept + bud.out_off[b];
    const uint32_t mb = bud.m[b];
    // one round of 512 positions: scan the flags and write the kept positions
    auto round = [&](int i, uint32_t key) {
      uint32_t fb = 0u, fe = 0u;
      if (i < c1) flags(T[b], i, key, &fb, &fe);
      uint32_t tot;   // both counts in one scan: each is <= kSelThreads
      const uint32_t ex = block_excl_scan(fb | (fe << 16), &tot, sh);
      const uint32_t bb = base_before + (ex & 0xffffu), eb = eq_before + (ex >> 16);
      const uint32_t slot = bb + min(eb, need[b]);
      if ((fb || (fe && eb < need[b])) && slot < mb) out[slot] = i;   // slot < m always holds
      base_before += tot & 0xffffu;
      eq_before += tot >> 16;
    };
    if (in_regs) {
#pragma unroll
      for (int r = 0; r < kSelRegKeys; ++r)
        if (c0 + r * kSelThreads < c1) round(c0 + tid + r * kSelThreads, keys[r]);   // uniform condition
    } else {
      for (int r0 = c0; r0 < c1; r0 += kSelThreads) {
        const int i = r0 + tid;
        round(i, i < c1 ? key_at(src, i) : 0u);
      }
    }
  }
  // the last workgroup out resets the barrier counters for the next call
  __syncthreads();
  if (tid == 0 && atomicAdd(&st->exit, 1u) == G - 1) {
    st->barrier = 0u;
    st->exit = 0u;
  }
}

// Workgroups of sel_fused_kernel that fit on `device` at once (cached).
static int coresident_blocks(int device) {
  static std::atomic<int> cache[64];
  if (device < 0 || device >= 64) return 0;
  int v = cache[device].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sel_fused_kernel<kSelMaxBudgets>, kSelThreads, 0) !=
      hipSuccess)
    return 0;
  v = cus * per_cu;
  cache[device].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace tg

extern "C" int64_t tg_num_kept(int64_t n, int64_t doc_begin, int64_t doc_end, int64_t k) {
  if (n < 0 || k < 0 || doc_begin < 0 || doc_begin > doc_end || doc_end > n) return -1;
  const int64_t d = doc_end - doc_begin;
  return (n - d) + (k < d ? k : d);
}

extern "C" size_t tg_select_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  return tg::SelLayout::bytes;
}

namespace tg {

// Validates a span and budgets, plans the grid and launches one selection.
static tg_status launch_select(int64_t n, const SelKeys& src, int64_t doc_begin, int64_t doc_end, const int64_t* ks,
                               int nk, int32_t* kept_idx, void* workspace, size_t workspace_bytes, void* stream) {
  if (n <= 0 || n > INT32_MAX || nk < 1 || nk > kSelMaxBudgets || !ks) return TG_ERR_INVALID_ARG;
  SelBudgets bud{};
  bud.nk = nk;
  int64_t total = 0;
  const int64_t d = doc_end - doc_begin;
  for (int b = 0; b < nk; ++b) {
    const int64_t mb = tg_num_kept(n, doc_begin, doc_end, ks[b]);
    if (mb < 0) return TG_ERR_INVALID_ARG;
    const int64_t k_eff = ks[b] < d ? ks[b] : d;
    bud.mode[b] = k_eff == 0 ? 0 : (k_eff == d ? 1 : 2);
    bud.k_eff[b] = static_cast<uint32_t>(k_eff);
    bud.m[b] = static_cast<uint32_t>(mb);
    bud.out_off[b] = total;
    total += mb;
  }
  if (total == 0) return TG_OK;   // nothing kept, nothing to write
  if ((!src.random && !src.scores) || !kept_idx || !workspace) return TG_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return TG_ERR_INVALID_ARG;
  if (workspace_bytes < SelLayout::bytes) return TG_ERR_WORKSPACE;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return TG_ERR_HIP;
  const int cap = coresident_blocks(device);
  if (cap <= 0) return TG_ERR_HIP;
  int64_t grid = (n + kSelPosPerBlock - 1) / kSelPosPerBlock;
  grid = grid < 1 ? 1 : grid;
  grid = grid > kSelMaxBlocks ? kSelMaxBlocks : grid;
  grid = grid > cap ? cap : grid;
  int64_t chunk = (n + grid - 1) / grid;
  chunk = (chunk + kSelThreads - 1) / kSelThreads * kSelThreads;
  grid = (n + chunk - 1) / chunk;
  if (nk == 1)
    hipLaunchKernelGGL(sel_fused_kernel<1>, dim3(static_cast<unsigned>(grid)), dim3(kSelThreads), 0,
                       static_cast<hipStream_t>(stream), src, static_cast<int>(n), static_cast<int>(doc_begin),
                       static_cast<int>(doc_end), bud, static_cast<int>(chunk), static_cast<char*>(workspace),
                       kept_idx);
  else
    hipLaunchKernelGGL(sel_fused_kernel<kSelMaxBudgets>, dim3(static_cast<unsigned>(grid)), dim3(kSelThreads), 0,
                       static_cast<hipStream_t>(stream), src, static_cast<int>(n), static_cast<int>(doc_begin),
                       static_cast<int>(doc_end), bud, static_cast<int>(chunk), static_cast<char*>(workspace),
                       kept_idx);
  TG_CHECK_LAUNCH();
  return TG_OK;
}

}  // namespace tg

extern "C" tg_status tg_select_topk(int64_t n, const float* scores, int64_t doc_begin, int64_t doc_end,
                                    int64_t k, int32_t* kept_idx, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const tg::SelKeys src{scores, 0ull, 0};
  return tg::launch_select(n, src, doc_begin, doc_end, &k, 1, kept_idx, workspace, workspace_bytes, stream);
}

extern "C" tg_status tg_select_topk_multi(int64_t n, const float* scores, int64_t doc_begin, int64_t doc_end,
                                          const int64_t* ks, int32_t n_budgets, int32_t* kept_idx, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  const tg::SelKeys src{scores, 0ull, 0};
  return tg::launch_select(n, src, doc_begin, doc_end, ks, n_budgets, kept_idx, workspace, workspace_bytes, stream);
}

extern "C" tg_status tg_select_random(int64_t n, int64_t doc_begin, int64_t doc_end, int64_t k, uint64_t seed,
                                      int32_t* kept_idx, void* workspace, size_t workspace_bytes, void* stream) {
  const tg::SelKeys src{nullptr, seed, 1};
  return tg::launch_select(n, src, doc_begin, doc_end, &k, 1, kept_idx, workspace, workspace_bytes, stream);
}
