// Document-only top-K selection with exact ties, compacted in position order.
//
// TokenGate keeps the K best-scoring tokens of the prunable document and never
// prunes the question (aiproducthub.cn "斯坦福伯克利TokenGate 预填充提速11.3倍",
// section 事件详情; aisight.pl "TokenGate: Stanford i Berkeley ...", section
// "Jak to dziala").  Kept positions are listed in ascending order; ties go to the
// lower position; keys are the order-preserving uint32 images of the scores.
//
// Both kernels here run as one launch whose workgroups are all resident at once and
// meet at counted grid barriers: one device-scope atomic per workgroup plus polling,
// no cache write-back fence, because every value that crosses workgroups is itself
// a device-scope atomic or atomic store, and each thread drains its own before its
// workgroup arrives.  Every wait is bounded: a wait that gives up (a grid that is not
// fully resident because the device is shared) sets the workspace's sticky failure
// word, its workgroup stops, and every later selection on that workspace exits at
// once until the caller zero-fills it again (tg_select_check reports the word).
//
// sel_gather_kernel -- one budget with the gather of the kept rows fused in
// (tg_select_gather, tg_select_gather_noalloc).  At most 64 selection workgroups of 256
// threads each own a chunk of positions, their keys held in registers; the rest of a
// grid of up to 512 workgroups are helpers that only copy rows.  Two barriers among the
// selection workgroups:
//   1. each workgroup histograms its document keys over the top 8 bits (coarse) and
//      the top 14 bits (fine) in LDS and merges the non-zero bins into global
//      histograms;  [barrier]
//   2. every workgroup scans the coarse histogram, then the 64 fine bins under the
//      coarse bin that holds the K-th largest key: the fine bin fb and the rank left
//      inside it.  Positions outside the document or with a fine bin above fb are kept
//      for sure; those in fb are candidates.  Each workgroup publishes its count of
//      sure positions and appends its candidates (key, position) to a global list;
//      [barrier]
//   3. every workgroup loads the candidates (a few hundred at 128k positions) and
//      resolves the exact threshold key T and the number need_eq of keys equal to T
//      that are kept with two 9-bit radix passes in LDS; from the candidates and the
//      sure counts it knows every chunk's kept count, so its own output slots follow
//      without another exchange: position i is kept iff it is sure, or a candidate
//      with key > T, or key == T with fewer than need_eq equal keys before it, and its
//      slot is (kept-outright positions before i) + min(equal keys before i, need_eq);
//   4. the gather: chunk w's owner publishes its first output slot and slot count on
//      its flag line, and the owner and its helpers (the team of chunk w) copy those
//      rows, each a share of them, after waiting for the flag.
// If the threshold's fine bin holds more candidates than fit in LDS (heavy ties),
// steps 2-3 fall back to two more radix passes over global histograms and one more
// exchange of per-chunk counts (three more barriers), with the same result.
//
// sel_fused_kernel -- one budget (tg_select_topk; faster than the kernel above when the
// gather runs as its own launch), several budgets in one launch (tg_select_topk_multi)
// and the random selector (tg_select_random).  At most 64 workgroups of 512 threads; radix
// select over three digits (bits 31..21, 20..10, 9..0), each a histogram merged with
// atomics and a barrier, then the counts of kept-outright and equal-to-T positions
// are exchanged at one more barrier and every workgroup compacts its chunk.  The
// first digit's histogram serves every budget (one gate serves every budget:
// aiproducthub.cn, section 事件详情; aisight.pl, section "Wyniki"); the later digits,
// the threshold and the compaction run per budget at the same barriers.
//
// Random selector (the pages' random-K ablation: aiproducthub.cn, section 事件详情;
// news.chathome.org, section "ベンチマーク"): the same selection on keys drawn per
// position from SplitMix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom Number
// Generators", OOPSLA 2014): the key of position i is the high half of the i-th output of
// the stream seeded with `seed`.  The K largest of independent uniform keys form a
// uniformly random K-subset of the document.
#include <atomic>
#include <cstddef>
#include <mutex>

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
constexpr uint32_t kSpinGiveUp = 0xffffffffu; // spin_limit word: every wait gives up at once

struct SelState {       // head of the workspace (64 bytes); the byte offsets are part of the ABI
  uint32_t barrier;     // 0: barrier arrivals of the current call (reset by the last workgroup out)
  uint32_t exit;        // 4: workgroups finished
  uint32_t fail;        // 8: sticky: set when a wait gave up; selections then exit at once
  uint32_t spin_limit;  // 12: 0 = default bound on each wait; kSpinGiveUp = give up at once
  uint32_t ncand;       // 16: candidates appended (sel_gather_kernel)
  uint32_t pad[11];
};
static_assert(sizeof(SelState) == 64, "workspace head");

struct SelLayout {     // sel_fused_kernel's regions
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

// Bound on one wait, from the workspace's spin_limit word (0: kSpinLimit polls).
__device__ __forceinline__ uint32_t spin_bound(const SelState* st) {
  const uint32_t v = ld_agent(&st->spin_limit);
  return v == 0u ? kSpinLimit : v;
}

// Polls *p until it reaches `target`; false if the bound ran out first.
__device__ __forceinline__ bool wait_at_least(const uint32_t* p, uint32_t target, uint32_t limit) {
  if (limit == kSpinGiveUp) return false;
  uint32_t spins = 0;
  while (ld_agent(p) < target) {
    if (++spins > limit) return false;   // only if the grid is not fully resident; never hang
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// All workgroups of the grid wait here until `target` arrivals have been counted.  Returns
// false in every thread of the workgroup if the wait gave up (the failure word is then set
// and the workgroup must stop).  *flag is a word of LDS.
__device__ __forceinline__ bool grid_barrier(SelState* st, uint32_t target, uint32_t limit, uint32_t* flag) {
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&st->barrier, 1u);
    const bool ok = wait_at_least(&st->barrier, target, limit);
    if (!ok) atomicOr(&st->fail, 1u);
    *flag = ok ? 1u : 0u;
  }
  __syncthreads();
  return *flag != 0u;
}

// True in every thread if the workspace's failure word is clear (read once, by thread 0).
__device__ __forceinline__ bool workspace_ok(SelState* st, uint32_t* flag) {
  if (threadIdx.x == 0) *flag = ld_agent(&st->fail) == 0u ? 1u : 0u;
  __syncthreads();
  const bool ok = *flag != 0u;
  __syncthreads();
  return ok;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row moves (no LDS round
// trips): shifts of 1, 2, 4, 8 inside each row of 16 lanes, then the last lane of row r
// is broadcast into row r + 1 (rows 1, 3) and lane 31 into rows 2, 3.  A lane whose DPP
// source does not exist adds 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive scan of one value per thread over a workgroup of NT threads; *total gets
// the sum.  sh: NT / 64 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_n(uint32_t v, uint32_t* total, uint32_t* sh) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  uint32_t wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t s = sh[w];
    wbase += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum_n(uint32_t v, uint32_t* sh) {
  constexpr int NW = NT / 64;
  v = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot += sh[w];
  __syncthreads();
  return tot;
}

__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* sh) {
  return block_excl_scan_n<kSelThreads>(v, total, sh);
}
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* sh) { return block_sum_n<kSelThreads>(v, sh); }

// NKM: the most budgets one instantiation handles (1 for the single-budget calls).
template <int NKM>
__global__ __launch_bounds__(kSelThreads) void sel_fused_kernel(SelKeys src, int n, int doc_begin, int doc_end,
                                                                SelBudgets bud, int chunk, char* ws,
                                                                int32_t* __restrict__ kept) {
  __shared__ uint32_t lh[NKM * kSelMaxBins];
  __shared__ uint32_t sh[kSelWaves];
  __shared__ uint32_t sh_prefix, sh_rank, sh_count, sh_flag;
  SelState* st = reinterpret_cast<SelState*>(ws + SelLayout::state);
  if (!workspace_ok(st, &sh_flag)) return;   // an earlier call on this workspace gave up
  const uint32_t limit = spin_bound(st);
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
  // expect: the keys the next digit's histogram must hold (the document, then the
  // chosen bin's count); a histogram that sums to anything else was not zero at the start
  uint32_t prefix[NKM], rank[NKM], expect[NKM];
  bool any_select = false;
#pragma unroll
  for (int b = 0; b < NKM; ++b) {
    prefix[b] = 0u;
    expect[b] = static_cast<uint32_t>(doc_end - doc_begin);
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
      if (!grid_barrier(st, ++barriers * G, limit, &sh_flag)) return;
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
        if (total != expect[b]) {   // same value in every workgroup: all of them give up
          if (tid == 0) atomicOr(&st->fail, 1u);
          return;
        }
        if (above < rank[b] && rank[b] <= above + local) {
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q) {
            if (q < per) {
              if (rank[b] <= above + c[q]) {
                sh_prefix = (prefix[b] << bits) | (bins - 1 - (tid * per + q));
                sh_rank = rank[b] - above;
                sh_count = c[q];
                break;
              }
              above += c[q];
            }
          }
        }
        __syncthreads();
        prefix[b] = sh_prefix;
        rank[b] = sh_rank;
        expect[b] = sh_count;
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
  if (!grid_barrier(st, ++barriers * G, limit, &sh_flag)) return;
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

// ---------------------------------------------------------------------------------
// sel_gather_kernel: one budget, two barriers, the row gather fused in
// ---------------------------------------------------------------------------------
constexpr int kSgThreads = 256;
constexpr int kSgMaxBlocks = 64;              // selection workgroups (chunks); barrier cost grows with them
constexpr int kSgMaxGrid = 512;               // selection workgroups plus their gather helpers
constexpr int kSgRegKeys = 8;                 // keys per thread in registers (chunks up to 2048 positions)
constexpr int kSgTeamWords = 32;              // per-chunk flag line: ready, first slot, slot count (128 B)
constexpr int kSgCoarse = 256;                // bins of key >> 24
constexpr int kSgFine = 16384;                // bins of key >> 18
constexpr int kSgFineShift = 18, kSgCoarseShift = 24;
constexpr int kSgFinePerCoarse = kSgFine / kSgCoarse;
constexpr int kSgCap = 4096;                  // candidates resolved in LDS
constexpr int kSgDigit = 512;                 // 9-bit digits of the last 18 key bits
constexpr int kSgCopyUnroll = 16;             // 16-byte pieces in flight per thread in the gather

struct SgLayout {   // after sel_fused_kernel's regions, so one workspace serves both kernels
  static constexpr size_t coarse = SelLayout::bytes;                  // [256]  zero between calls
  static constexpr size_t fine = coarse + kSgCoarse * 4;               // [16384] zero between calls
  static constexpr size_t digit_a = fine + kSgFine * 4;                // [512]  zero between calls
  static constexpr size_t digit_b = digit_a + kSgDigit * 4;            // [512]  zero between calls
  static constexpr size_t team = digit_b + kSgDigit * 4;               // [64][32] ready flags: zero between calls
  static constexpr size_t sure = team + kSgMaxBlocks * kSgTeamWords * 4;   // [64] per-chunk counts
  static constexpr size_t gt = sure + kSgMaxBlocks * 4;                // [64]
  static constexpr size_t eq = gt + kSgMaxBlocks * 4;                  // [64]
  static constexpr size_t ckey = eq + kSgMaxBlocks * 4;                // [4096] candidates
  static constexpr size_t cpos = ckey + kSgCap * 4;                    // [4096]
  static constexpr size_t bytes = (cpos + kSgCap * 4 + 255) & ~size_t(255);
};

struct SgArgs {
  const float* scores;
  int n, doc_begin, doc_end;
  int mode;              // 0: no document position kept; 1: every one; 2: the k_eff best
  uint32_t k_eff;
  int chunk;             // positions per selection workgroup (a multiple of kSgThreads)
  int nsel;              // selection workgroups (chunks); the grid is nsel x team
  int vec;               // scores 16-byte aligned: 8 consecutive positions load as two vectors
  uint32_t* status;      // NULL, or a word set to 1 when a wait gives up (allocation-free calls)
  int m;                 // kept positions
  char* ws;
  int32_t* kept;
  float* s_kept;         // may be NULL
  const char* x;         // NULL: selection only
  char* xk;
  int64_t ldx_b, ldo_b;  // row strides in bytes
  int row_b;             // bytes copied per row
  int unit;              // copy unit in bytes: 16, 4 or 2
};

// Clears `words` words at p, and *status if given (the allocation-free entry point's
// scratch and its caller's status word).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, uint32_t words,
                                                         uint32_t* __restrict__ status) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i < words) p[i] = 0u;
  if (status && i == 0) *status = 0u;
}

template <typename U>
__device__ __forceinline__ void copy_rows(const SgArgs& a, const int32_t* lrow, int64_t s0, int nrows) {
  constexpr int UB = sizeof(U);
  const int per_row = a.row_b / UB;
  const int total = nrows * per_row;
  for (int p0 = 0; p0 < total; p0 += kSgThreads * kSgCopyUnroll) {
    U v[kSgCopyUnroll];
#pragma unroll
    for (int u = 0; u < kSgCopyUnroll; ++u) {
      const int p = p0 + threadIdx.x + u * kSgThreads;
      if (p < total) {
        const int r = p / per_row, c = p - r * per_row;
        if (lrow[r] >= 0) v[u] = *reinterpret_cast<const U*>(a.x + (int64_t)lrow[r] * a.ldx_b + (int64_t)c * UB);
      }
    }
#pragma unroll
    for (int u = 0; u < kSgCopyUnroll; ++u) {
      const int p = p0 + threadIdx.x + u * kSgThreads;
      if (p < total) {
        const int r = p / per_row, c = p - r * per_row;
        if (lrow[r] >= 0) *reinterpret_cast<U*>(a.xk + (s0 + r) * a.ldo_b + (int64_t)c * UB) = v[u];
      }
    }
  }
}

__global__ __launch_bounds__(kSgThreads, 2) void sel_gather_kernel(SgArgs a) {
  constexpr int NT = kSgThreads;
  static_assert(NT == kSgCoarse && 2 * NT == kSgDigit && NT >= kSgMaxBlocks, "one coarse bin per thread");
  __shared__ __attribute__((aligned(16))) uint32_t lbuf[kSgFine];   // fine histogram; later candidates
  __shared__ uint32_t lcoarse[kSgCoarse];
  __shared__ uint32_t lfb[kSgMaxBlocks + 1], leq[kSgMaxBlocks + 1], lgt[kSgMaxBlocks];
  __shared__ int32_t lrow[NT];
  __shared__ uint32_t sh[NT / 64];
  __shared__ uint32_t bc[8];
  __shared__ uint32_t sh_flag;

  SelState* st = reinterpret_cast<SelState*>(a.ws);
  uint32_t* gcoarse = reinterpret_cast<uint32_t*>(a.ws + SgLayout::coarse);
  uint32_t* gfine = reinterpret_cast<uint32_t*>(a.ws + SgLayout::fine);
  uint32_t* gda = reinterpret_cast<uint32_t*>(a.ws + SgLayout::digit_a);
  uint32_t* gdb = reinterpret_cast<uint32_t*>(a.ws + SgLayout::digit_b);
  uint32_t* gteam = reinterpret_cast<uint32_t*>(a.ws + SgLayout::team);
  uint32_t* gsure = reinterpret_cast<uint32_t*>(a.ws + SgLayout::sure);
  uint32_t* ggt = reinterpret_cast<uint32_t*>(a.ws + SgLayout::gt);
  uint32_t* geq = reinterpret_cast<uint32_t*>(a.ws + SgLayout::eq);
  uint32_t* gckey = reinterpret_cast<uint32_t*>(a.ws + SgLayout::ckey);
  uint32_t* gcpos = reinterpret_cast<uint32_t*>(a.ws + SgLayout::cpos);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.nsel;                    // selection workgroups = chunks
  const int w = blockIdx.x % G;            // this workgroup's chunk
  const int share = blockIdx.x / G;        // 0: selects chunk w and copies the first share of its rows
  const int team = gridDim.x / G;          // workgroups copying chunk w's rows (1 without the gather)
  // a wait that gives up also marks the caller's status word, if there is one
  auto fail_out = [&a]() {
    if (threadIdx.x == 0 && a.status) st_agent(a.status, 1u);
  };
  if (!workspace_ok(st, &sh_flag)) {   // an earlier call on this workspace gave up
    fail_out();
    return;
  }
  const uint32_t limit = spin_bound(st);
  uint32_t* flag_line = gteam + w * kSgTeamWords;   // [0] ready, [1] first slot, [2] slots

  if (share == 0) {
    uint32_t nbar = 0;
    // this chunk, in blocks of NT * per positions: thread tid owns the `per` consecutive
    // positions blk + per * tid + r of each block (per = 8 for chunks of 2048 or more, else
    // chunk / NT).  A chunk of one block keeps its score bits in registers (raw[r]);
    // larger chunks re-read them at every pass.
    const int c0 = w * a.chunk, c1 = min(a.n, c0 + a.chunk);
    const int per = min(a.chunk / NT, kSgRegKeys);
    const int blk = NT * per;
    const bool in_regs = a.chunk <= blk;
    uint32_t raw[kSgRegKeys];
    auto load_block = [&a, tid, per, c1](int b0, uint32_t (&dst)[kSgRegKeys]) {
      const int i0 = b0 + per * tid;
      if (per == kSgRegKeys && a.vec && i0 + kSgRegKeys <= c1) {   // two 16-byte loads
        const u32x4 lo = *reinterpret_cast<const u32x4*>(a.scores + i0);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(a.scores + i0 + 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r] = lo[r], dst[r + 4] = hi[r];
      } else {
#pragma unroll
        for (int r = 0; r < kSgRegKeys; ++r)
          dst[r] = (r < per && i0 + r < c1) ? __float_as_uint(a.scores[i0 + r]) : 0u;
      }
    };
    if (in_regs) load_block(c0, raw);
    // f(position, score bits) for every position of the chunk held by this thread
    auto for_chunk = [&raw, &load_block, in_regs, c0, c1, per, blk, tid](auto&& f) {
      if (in_regs) {
#pragma unroll
        for (int r = 0; r < kSgRegKeys; ++r) {
          const int i = c0 + per * tid + r;
          if (r < per && i < c1) f(i, raw[r]);
        }
      } else {
        for (int b0 = c0; b0 < c1; b0 += blk) {
          uint32_t bits[kSgRegKeys];
          load_block(b0, bits);
#pragma unroll
          for (int r = 0; r < kSgRegKeys; ++r) {
            const int i = b0 + per * tid + r;
            if (r < per && i < c1) f(i, bits[r]);
          }
        }
      }
    };
    const int doc_begin = a.doc_begin, doc_end = a.doc_end;
    auto is_doc = [doc_begin, doc_end](int i) { return i >= doc_begin && i < doc_end; };
    auto key_of = [](uint32_t bits) { return score_key(__uint_as_float(bits)); };

    uint32_t fb = 0u;            // fine bin of the threshold key (mode 2)
    uint32_t T = 0xffffffffu;    // threshold key; kept: key > T, or key == T within need_eq
    uint32_t need = 0u;

    if (a.mode == 2) {
      // ---- 1. coarse and fine histograms of the document keys ----
      lcoarse[tid] = 0u;
      __syncthreads();
      for_chunk([&](int i, uint32_t b) {
        if (is_doc(i)) atomicAdd(&lcoarse[key_of(b) >> kSgCoarseShift], 1u);
      });
      __syncthreads();
      // only the fine bins under occupied coarse bins are used: each wave zeroes (and later
      // merges) the 64 fine bins of each occupied coarse bin among its 64, one per lane
      const uint64_t occ = __ballot(lcoarse[tid] != 0u);
      for (uint64_t o = occ; o; o &= o - 1) lbuf[(wave * 64 + __builtin_ctzll(o)) * kSgFinePerCoarse + lane] = 0u;
      __syncthreads();
      for_chunk([&](int i, uint32_t b) {
        if (is_doc(i)) atomicAdd(&lbuf[key_of(b) >> kSgFineShift], 1u);
      });
      __syncthreads();
      if (lcoarse[tid]) atomicAdd(&gcoarse[tid], lcoarse[tid]);
      for (uint64_t o = occ; o; o &= o - 1) {
        const int f = (wave * 64 + __builtin_ctzll(o)) * kSgFinePerCoarse + lane;
        const uint32_t v = lbuf[f];
        if (v) atomicAdd(&gfine[f], v);
      }
      if (!grid_barrier(st, ++nbar * G, limit, &sh_flag)) {
        fail_out();
        return;
      }

      // ---- 2. the fine bin holding the k_eff-th largest key, and the rank inside it ----
      uint32_t rank = a.k_eff;   // 0 < k_eff < D
      {
        const uint32_t cv = ld_agent(&gcoarse[kSgCoarse - 1 - tid]);   // bins from the top
        uint32_t tot;
        const uint32_t above = block_excl_scan_n<NT>(cv, &tot, sh);
        if (tot != (uint32_t)(a.doc_end - a.doc_begin)) {   // the workspace was not zero: give up
          if (tid == 0) atomicOr(&st->fail, 1u);
          fail_out();
          return;
        }
        if (above < rank && rank <= above + cv) {
          bc[1] = kSgCoarse - 1 - tid;
          bc[2] = rank - above;
        }
        __syncthreads();
        const uint32_t cb = bc[1], rc = bc[2];
        if (tid < 64) {   // one wave scans the 64 fine bins under cb from the top
          const uint32_t f = cb * kSgFinePerCoarse + (kSgFinePerCoarse - 1 - tid);
          const uint32_t fv = ld_agent(&gfine[f]);
          const uint32_t incl = wave_incl_scan(fv);
          if (incl - fv < rc && rc <= incl) {
            bc[3] = f;
            bc[4] = rc - (incl - fv);
            bc[5] = fv;
          }
        }
        __syncthreads();
        fb = bc[3];
        rank = bc[4];
      }
      const uint32_t ncand = bc[5];   // document keys in bin fb (all of them candidates)
      const bool fits = ncand <= (uint32_t)kSgCap;

      // sure positions of this chunk, and its candidates appended to the global list
      uint32_t ns = 0u, nc = 0u;
      for_chunk([&](int i, uint32_t b) {
        const uint32_t f = key_of(b) >> kSgFineShift;
        const bool doc = is_doc(i);
        ns += (!doc || f > fb) ? 1u : 0u;
        nc += (doc && f == fb) ? 1u : 0u;
      });
      uint32_t slot, nc_tot;
      if (a.chunk < 65536) {   // both counts in one scan (each is at most the chunk)
        uint32_t both;
        slot = block_excl_scan_n<NT>(ns | (nc << 16), &both, sh) >> 16;
        ns = both & 0xffffu;
        nc_tot = both >> 16;
      } else {
        ns = block_sum_n<NT>(ns, sh);
        slot = block_excl_scan_n<NT>(nc, &nc_tot, sh);
      }
      if (tid == 0) {
        st_agent(&gsure[w], ns);
        if (fits && nc_tot) bc[6] = atomicAdd(&st->ncand, nc_tot);
      }
      __syncthreads();
      if (fits && nc_tot) {
        slot += bc[6];
        for_chunk([&](int i, uint32_t b) {
          const uint32_t key = key_of(b);
          if (is_doc(i) && (key >> kSgFineShift) == fb) {
            if (slot < (uint32_t)kSgCap) {   // always holds: the candidates are the keys in bin fb
              st_agent(&gckey[slot], key);
              st_agent(&gcpos[slot], (uint32_t)i);
            }
            ++slot;
          }
        });
      }
      if (!grid_barrier(st, ++nbar * G, limit, &sh_flag)) {
        fail_out();
        return;
      }
      // every selection workgroup has read the histograms: clear them for the next call
      for (int i = w * (kSgFine / G) + tid; i < (w + 1) * (kSgFine / G); i += NT) st_agent(&gfine[i], 0u);
      if (w == G - 1)
        for (int i = (kSgFine / G) * G + tid; i < kSgFine; i += NT) st_agent(&gfine[i], 0u);
      if (w == 0) {
        st_agent(&gcoarse[tid], 0u);
        if (tid == 0) st_agent(&st->ncand, 0u);
      }

      // ---- 3. exact threshold T, need_eq, and every chunk's counts ----
      if (tid < G) lgt[tid] = 0u, leq[tid] = 0u;
      if (fits) {
        uint32_t* lk = lbuf;
        uint32_t* lp = lbuf + kSgCap;
        uint32_t* lh = lbuf + 2 * kSgCap;
        for (int j = tid; j < (int)ncand; j += NT) {
          lk[j] = ld_agent(&gckey[j]);
          lp[j] = ld_agent(&gcpos[j]);
        }
        __syncthreads();
        if (wave == 0) {   // one wave resolves the last 18 bits: two 9-bit passes, no block barriers
          uint32_t prefix = fb, rk = rank;
          for (int pass = 0; pass < 2; ++pass) {   // bits 17..9, then 8..0
            const int shift = pass == 0 ? 9 : 0;
            for (int b = lane; b < kSgDigit; b += 64) lh[b] = 0u;
            for (int j = lane; j < (int)ncand; j += 64)
              if ((lk[j] >> (shift + 9)) == prefix) atomicAdd(&lh[(lk[j] >> shift) & (kSgDigit - 1)], 1u);
            // lane l holds bins 511 - 8 l .. 504 - 8 l, from the top
            uint32_t h[8], sum = 0u;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              h[q] = lh[kSgDigit - 1 - 8 * lane - q];
              sum += h[q];
            }
            const uint32_t incl = wave_incl_scan(sum);
            uint32_t ab = incl - sum, digit = 0u, r2 = 0u;
            const bool here = ab < rk && rk <= incl;
            if (here) {
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                if (digit == 0u && rk <= ab + h[q]) {
                  digit = (uint32_t)(kSgDigit - 1 - 8 * lane - q) | 0x80000000u;
                  r2 = rk - ab;
                }
                ab += h[q];
              }
            }
            const int src = __builtin_ctzll(__ballot(here));
            digit = __shfl(digit, src, 64) & 0x7fffffffu;
            rk = __shfl(r2, src, 64);
            prefix = (prefix << 9) | digit;
          }
          if (lane == 0) {
            bc[1] = prefix;
            bc[2] = rk;
          }
        }
        __syncthreads();
        T = bc[1];
        need = bc[2];
        for (int j = tid; j < (int)ncand; j += NT) {
          const int ch = (int)(lp[j] / (uint32_t)a.chunk);
          if (ch < G) {   // always holds: candidates are positions of this call
            if (lk[j] > T) atomicAdd(&lgt[ch], 1u);
            else if (lk[j] == T) atomicAdd(&leq[ch], 1u);
          }
        }
      } else {
        // heavy ties in bin fb: the last 18 bits by two radix passes over global histograms
        uint32_t prefix = fb;
        for (int pass = 0; pass < 2; ++pass) {
          const int shift = pass == 0 ? 9 : 0;
          uint32_t* gd = pass == 0 ? gda : gdb;
          uint32_t* lh = lbuf;
          lh[tid] = 0u;
          lh[tid + NT] = 0u;
          __syncthreads();
          for_chunk([&](int i, uint32_t b) {
            const uint32_t key = key_of(b);
            if (is_doc(i) && (key >> (shift + 9)) == prefix) atomicAdd(&lh[(key >> shift) & (kSgDigit - 1)], 1u);
          });
          __syncthreads();
          if (lh[tid]) atomicAdd(&gd[tid], lh[tid]);
          if (lh[tid + NT]) atomicAdd(&gd[tid + NT], lh[tid + NT]);
          if (!grid_barrier(st, ++nbar * G, limit, &sh_flag)) {
        fail_out();
        return;
      }
          if (pass == 1 && w == 0) {   // digit a was read by everyone before this barrier
            st_agent(&gda[tid], 0u);
            st_agent(&gda[tid + NT], 0u);
          }
          const uint32_t b0 = kSgDigit - 1 - 2 * tid, b1 = b0 - 1;
          const uint32_t h0 = ld_agent(&gd[b0]), h1 = ld_agent(&gd[b1]);
          uint32_t tot;
          const uint32_t ab = block_excl_scan_n<NT>(h0 + h1, &tot, sh);
          if (ab < rank && rank <= ab + h0) {
            bc[1] = b0;
            bc[2] = rank - ab;
          } else if (ab + h0 < rank && rank <= ab + h0 + h1) {
            bc[1] = b1;
            bc[2] = rank - ab - h0;
          }
          __syncthreads();
          prefix = (prefix << 9) | bc[1];
          rank = bc[2];
          __syncthreads();
        }
        T = prefix;
        need = rank;
        uint32_t ngt = 0u, neq = 0u;
        for_chunk([&](int i, uint32_t b) {
          const uint32_t key = key_of(b);
          const bool c = is_doc(i) && (key >> kSgFineShift) == fb;
          ngt += (c && key > T) ? 1u : 0u;
          neq += (c && key == T) ? 1u : 0u;
        });
        ngt = block_sum_n<NT>(ngt, sh);
        neq = block_sum_n<NT>(neq, sh);
        if (tid == 0) {
          st_agent(&ggt[w], ngt);
          st_agent(&geq[w], neq);
        }
        if (!grid_barrier(st, ++nbar * G, limit, &sh_flag)) {
        fail_out();
        return;
      }
        if (w == 0) {   // digit b was read by everyone before this barrier
          st_agent(&gdb[tid], 0u);
          st_agent(&gdb[tid + NT], 0u);
        }
        if (tid < G) lgt[tid] = ld_agent(&ggt[tid]), leq[tid] = ld_agent(&geq[tid]);
      }
      if (tid < G) lfb[tid] = ld_agent(&gsure[tid]);
      __syncthreads();
    } else {
      // nothing to rank: every chunk's count follows from the span
      if (tid < G) {
        const int d0 = tid * a.chunk, d1 = min(a.n, d0 + a.chunk);
        const int in_doc = max(0, min(d1, a.doc_end) - max(d0, a.doc_begin));
        lfb[tid] = (uint32_t)(a.mode == 1 ? d1 - d0 : (d1 - d0) - in_doc);
        lgt[tid] = 0u;
        leq[tid] = 0u;
      }
      __syncthreads();
    }

    // ---- 4. slots: exclusive prefixes over the chunks of the kept-outright count (sure +
    //         candidates above T) and of the count of keys equal to T ----
    {
      const uint32_t f0 = tid < G ? lfb[tid] + lgt[tid] : 0u, e0 = tid < G ? leq[tid] : 0u;
      uint32_t ftot, etot;
      const uint32_t fx = block_excl_scan_n<NT>(f0, &ftot, sh);
      const uint32_t ex = block_excl_scan_n<NT>(e0, &etot, sh);
      if (tid < G) lfb[tid] = fx, leq[tid] = ex;
      if (tid == 0) lfb[G] = ftot, leq[G] = etot;
      __syncthreads();
    }
    // write this chunk's kept positions (and their scores) to their slots: per block, one
    // scan of the per-thread counts, then each thread walks its positions in order
    uint32_t fbb = lfb[w], eqb = leq[w];
    const bool gather = a.x != nullptr;
    auto compact_block = [&](int b0, const uint32_t (&bits)[kSgRegKeys]) {
      uint32_t fo = 0u, fe = 0u, cnt = 0u;   // flags as bit masks over r, and the two counts
#pragma unroll
      for (int r = 0; r < kSgRegKeys; ++r) {
        const int i = b0 + per * tid + r;
        if (r < per && i < c1) {
          const uint32_t key = key_of(bits[r]);
          const bool doc = is_doc(i);
          bool o = false, e = false;
          if (!doc || a.mode == 1) o = true;
          else if (a.mode == 2) {
            const uint32_t f = key >> kSgFineShift;
            o = f > fb || (f == fb && key > T);
            e = f == fb && key == T;
          }
          fo |= (o ? 1u : 0u) << r;
          fe |= (e ? 1u : 0u) << r;
          cnt += (o ? 1u : 0u) + (e ? 0x10000u : 0u);
        }
      }
      uint32_t tot;   // both counts in one scan: each is <= NT * per <= 2048
      const uint32_t ex = block_excl_scan_n<NT>(cnt, &tot, sh);
      uint32_t bb = fbb + (ex & 0xffffu), eb = eqb + (ex >> 16);
#pragma unroll
      for (int r = 0; r < kSgRegKeys; ++r) {
        const bool o = (fo >> r) & 1u, e = (fe >> r) & 1u;
        if (o || (e && eb < need)) {
          const uint32_t sl = bb + min(eb, need);
          const int i = b0 + per * tid + r;
          if (sl < (uint32_t)a.m) {   // always holds
            if (gather) st_agent(reinterpret_cast<uint32_t*>(a.kept) + sl, (uint32_t)i);
            else a.kept[sl] = i;
            if (a.s_kept) a.s_kept[sl] = __uint_as_float(bits[r]);
          }
        }
        bb += o ? 1u : 0u;
        eb += e ? 1u : 0u;
      }
      fbb += tot & 0xffffu;
      eqb += tot >> 16;
    };
    if (in_regs) {
      compact_block(c0, raw);
    } else {
      for (int b0 = c0; b0 < c1; b0 += blk) {
        uint32_t bits[kSgRegKeys];
        load_block(b0, bits);
        compact_block(b0, bits);
      }
    }
    if (gather) {   // publish this chunk's slots to its team: first slot and count, then ready
      const uint32_t first = lfb[w] + min(leq[w], need);
      const uint32_t end = lfb[w + 1] + min(leq[w + 1], need);
      drain_vmem();
      __syncthreads();
      if (tid == 0) {
        st_agent(&flag_line[1], first);
        st_agent(&flag_line[2], end - first);
        drain_vmem();
        st_agent(&flag_line[0], 1u);
        bc[0] = first;
        bc[1] = end - first;
      }
      __syncthreads();
    }
  } else {
    // a helper: wait for this chunk's selection workgroup to publish its slots
    if (tid == 0) {
      uint32_t ok = 1u, spins = 0;
      if (limit == kSpinGiveUp) ok = 0u;
      while (ok && ld_agent(&flag_line[0]) == 0u) {
        if (++spins > limit) ok = 0u;
        __builtin_amdgcn_s_sleep(8);
      }
      if (ok) {
        bc[0] = ld_agent(&flag_line[1]);
        bc[1] = ld_agent(&flag_line[2]);
      } else {
        atomicOr(&st->fail, 1u);
      }
      sh_flag = ok;
    }
    __syncthreads();
    if (!sh_flag) {
      fail_out();
      return;
    }
  }

  // ---- 5. the gather: this workgroup's share of chunk w's slots ----
  if (a.x != nullptr) {
    const int64_t first = bc[0], cnt = bc[1];
    const int64_t s0 = first + cnt * share / team, s1 = first + cnt * (share + 1) / team;
    for (int64_t r0 = s0; r0 < s1; r0 += NT) {
      const int nr = (int)min<int64_t>(NT, s1 - r0);
      if (tid < nr) {
        const uint32_t src = ld_agent(reinterpret_cast<const uint32_t*>(a.kept) + r0 + tid);
        lrow[tid] = src < (uint32_t)a.n ? (int32_t)src : -1;   // always in range: written by this call
      }
      __syncthreads();
      if (a.unit == 16) copy_rows<u32x4>(a, lrow, r0, nr);
      else if (a.unit == 4) copy_rows<uint32_t>(a, lrow, r0, nr);
      else copy_rows<uint16_t>(a, lrow, r0, nr);
      __syncthreads();
    }
  }

  // ---- the last workgroup out resets the counters and ready flags for the next call ----
  __syncthreads();
  if (tid == 0) sh_flag = atomicAdd(&st->exit, 1u) == gridDim.x - 1u ? 1u : 0u;
  __syncthreads();
  if (sh_flag) {
    if (a.x != nullptr && tid < G) st_agent(&gteam[tid * kSgTeamWords], 0u);
    if (tid == 0) {
      st_agent(&st->barrier, 0u);
      st_agent(&st->exit, 0u);
    }
  }
}

// Workgroups of `kernel` (NT threads) that fit on `device` at once (cached per slot).
template <int SLOT>
static int coresident_blocks(int device, const void* kernel, int nt) {
  static std::atomic<int> cache[64];
  if (device < 0 || device >= 64) return 0;
  int v = cache[device].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nt, 0) != hipSuccess) return 0;
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
  return tg::SgLayout::bytes;
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
  if (workspace_bytes < SgLayout::bytes) return TG_ERR_WORKSPACE;   // the documented size: one workspace serves every selection
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return TG_ERR_HIP;
  const int cap = coresident_blocks<0>(device, reinterpret_cast<const void*>(sel_fused_kernel<kSelMaxBudgets>),
                                       kSelThreads);
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

// One budget, with the gather of the kept rows when x is given (sel_gather_kernel).
static void* scratch_address(int device);

// use_scratch: the allocation-free variant: the workspace is this device's static scratch
// array, cleared on the stream before the selection (its contents are whatever the last
// call left, which may have given up).
static tg_status launch_select_gather(int64_t n, const float* scores, int64_t doc_begin, int64_t doc_end, int64_t k,
                                      int32_t* kept_idx, float* s_kept, int32_t dtype, int32_t d_model, const void* x,
                                      int64_t ldx, void* x_kept, int64_t ld_out, void* workspace,
                                      size_t workspace_bytes, void* stream, bool use_scratch = false,
                                      uint32_t* status = nullptr) {
  if (n <= 0 || n > INT32_MAX || k < 0) return TG_ERR_INVALID_ARG;
  const int64_t m = tg_num_kept(n, doc_begin, doc_end, k);
  if (m < 0) return TG_ERR_INVALID_ARG;
  SgArgs a{};
  if (x) {
    if (dtype != TG_F32 && dtype != TG_BF16) return TG_ERR_INVALID_ARG;
    if (d_model <= 0 || ldx < d_model || ld_out < d_model || !x_kept) return TG_ERR_INVALID_ARG;
    const int esz = dtype == TG_BF16 ? 2 : 4;
    a.x = static_cast<const char*>(x);
    a.xk = static_cast<char*>(x_kept);
    a.ldx_b = ldx * esz;
    a.ldo_b = ld_out * esz;
    a.row_b = d_model * esz;
    const uintptr_t align = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_kept) |
                            static_cast<uintptr_t>(a.ldx_b) | static_cast<uintptr_t>(a.ldo_b) |
                            static_cast<uintptr_t>(a.row_b);
    a.unit = (align & 15u) == 0 ? 16 : ((align & 3u) == 0 ? 4 : 2);
  }
  if (m == 0) return TG_OK;   // nothing kept, nothing to write
  if (!scores || !kept_idx || (!workspace && !use_scratch)) return TG_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return TG_ERR_INVALID_ARG;
  if (!use_scratch && workspace_bytes < SgLayout::bytes) return TG_ERR_WORKSPACE;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return TG_ERR_HIP;
  if (use_scratch) {
    workspace = scratch_address(device);
    if (!workspace) return TG_ERR_HIP;
  }
  const int cap = coresident_blocks<1>(device, reinterpret_cast<const void*>(sel_gather_kernel), kSgThreads);
  if (cap <= 0) return TG_ERR_HIP;
  int64_t nsel = (n + kSgThreads - 1) / kSgThreads;
  nsel = nsel > kSgMaxBlocks ? kSgMaxBlocks : nsel;
  nsel = nsel > cap ? cap : nsel;
  int64_t chunk = (n + nsel - 1) / nsel;
  chunk = (chunk + kSgThreads - 1) / kSgThreads * kSgThreads;
  nsel = (n + chunk - 1) / chunk;
  // with the gather, each chunk's rows are copied by a team of workgroups (the selection
  // workgroup and helpers), all resident together
  int64_t team = 1;
  if (x) {
    const int64_t room = (cap < kSgMaxGrid ? cap : kSgMaxGrid) / nsel;
    const int64_t want = (m + nsel * 4 - 1) / (nsel * 4);   // at least ~4 rows per workgroup
    team = room < want ? room : want;
    team = team < 1 ? 1 : team;
  }
  const int64_t grid = nsel * team;
  const int64_t d = doc_end - doc_begin;
  const int64_t k_eff = k < d ? k : d;
  a.scores = scores;
  a.vec = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0 ? 1 : 0;
  a.n = static_cast<int>(n);
  a.doc_begin = static_cast<int>(doc_begin);
  a.doc_end = static_cast<int>(doc_end);
  a.mode = k_eff == 0 ? 0 : (k_eff == d ? 1 : 2);
  a.k_eff = static_cast<uint32_t>(k_eff);
  a.chunk = static_cast<int>(chunk);
  a.nsel = static_cast<int>(nsel);
  a.m = static_cast<int>(m);
  a.ws = static_cast<char*>(workspace);
  a.kept = kept_idx;
  a.s_kept = s_kept;
  a.status = status;
  if (use_scratch) {
    const uint32_t words = static_cast<uint32_t>(SgLayout::bytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t*>(workspace), words, status);
    TG_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(sel_gather_kernel, dim3(static_cast<unsigned>(grid)), dim3(kSgThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  TG_CHECK_LAUNCH();
  return TG_OK;
}

// ---------------------------------------------------------------------------------
// Allocation-free selection + gather: the workspace is a static device array, one per
// device, held by the library until the process ends.
// ---------------------------------------------------------------------------------
constexpr size_t kScratchBytes = SgLayout::bytes;   // 217 KiB: the selection's layout does not depend on n
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on `device` (the current device), looked up once per device
// with that device current; NULL if the runtime cannot give it.
static void* scratch_address(int device) {
  static std::mutex mu;
  static void* addr[64] = {};
  if (device < 0 || device >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[device] = p;
  }
  return addr[device];
}

}  // namespace tg

extern "C" tg_status tg_select_topk(int64_t n, const float* scores, int64_t doc_begin, int64_t doc_end,
                                    int64_t k, int32_t* kept_idx, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  // the three-digit kernel: measured faster for the selection alone than sel_gather_kernel
  const tg::SelKeys src{scores, 0ull, 0};
  return tg::launch_select(n, src, doc_begin, doc_end, &k, 1, kept_idx, workspace, workspace_bytes, stream);
}

extern "C" tg_status tg_select_gather(int32_t dtype, int64_t n, int32_t d_model, const float* scores,
                                      int64_t doc_begin, int64_t doc_end, int64_t k, const void* x, int64_t ldx,
                                      int32_t* kept_idx, void* x_kept, int64_t ld_out, float* s_kept,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !s_kept) return TG_ERR_INVALID_ARG;
  return tg::launch_select_gather(n, scores, doc_begin, doc_end, k, kept_idx, s_kept, dtype, d_model, x, ldx, x_kept,
                                  ld_out, workspace, workspace_bytes, stream);
}

extern "C" tg_status tg_select_gather_noalloc(int32_t dtype, int64_t n, int32_t d_model, const float* scores,
                                              int64_t doc_begin, int64_t doc_end, int64_t k, const void* x,
                                              int64_t ldx, int32_t* kept_idx, void* x_kept, int64_t ld_out,
                                              float* s_kept, int32_t* status, void* stream) {
  if (!x || !s_kept) return TG_ERR_INVALID_ARG;
  // the scratch array has the selection's fixed layout, whatever n is: never exceeded
  if (tg_select_workspace_bytes(n) > tg::kScratchBytes) return TG_ERR_WORKSPACE;
  return tg::launch_select_gather(n, scores, doc_begin, doc_end, k, kept_idx, s_kept, dtype, d_model, x, ldx, x_kept,
                                  ld_out, nullptr, 0, stream, true, reinterpret_cast<uint32_t*>(status));
}

extern "C" tg_status tg_select_check(const void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < sizeof(tg::SelState)) return TG_ERR_INVALID_ARG;
  uint32_t fail = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&fail, static_cast<const char*>(workspace) + offsetof(tg::SelState, fail), sizeof(fail),
                     hipMemcpyDeviceToHost, st) != hipSuccess)
    return TG_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return TG_ERR_HIP;
  return fail ? TG_ERR_INCOMPLETE : TG_OK;
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
