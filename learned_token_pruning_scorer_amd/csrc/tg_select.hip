// Document-only top-K selection with exact ties, compacted in position order.
//
// TokenGate keeps the K best-scoring tokens of the prunable document and never
// prunes the question (aiproducthub.cn "斯坦福伯克利TokenGate 预填充提速11.3倍",
// section 事件详情; aisight.pl "TokenGate: Stanford i Berkeley ...", section
// "Jak to dziala").
//
// Scores are mapped to order-preserving uint32 keys.  A radix select over three
// digits (bits 31..20, 19..8, 7..0) finds the threshold key T, the K-th largest
// document key, and `need_eq`, how many keys equal to T are kept.  Each digit pass
// builds a workgroup-local LDS histogram, adds it to a global histogram with
// atomics, and the last workgroup to finish (a done-counter) scans the global
// histogram to pick the digit and clears it again.  Compaction then needs, for
// every position i, two prefix counts: `base` (positions kept outright: outside
// the document, or key > T) and `eq` (document keys equal to T).  Position i is
// kept iff base(i) or (eq(i) and eq_before(i) < need_eq), and its output slot is
// base_before(i) + min(eq_before(i), need_eq).  Ties thus go to the lowest
// positions, and the output is ascending by construction.
#include "tg_common.h"

namespace tg {

constexpr int kSelThreads = 256;
constexpr int kHistBins01 = 4096;   // digits of passes 0 and 1 (12 bits)
constexpr int kHistBins2 = 256;     // digit of pass 2 (8 bits)
constexpr int kCmpPerThread = 4;
constexpr int kCmpChunk = kSelThreads * kCmpPerThread;   // positions per compaction block
constexpr int kHistMaxBlocks = 256;

struct SelState {         // head of the workspace (64 bytes)
  uint32_t done[4];       // per-pass done counters (always 0 between calls)
  uint32_t prefix;        // key bits fixed so far
  uint32_t rank;          // 1-based rank still wanted among keys with that prefix
  uint32_t pad[10];
};

struct SelLayout {
  size_t state = 0;
  size_t hist0 = 64;
  size_t hist1 = hist0 + kHistBins01 * 4;
  size_t hist2 = hist1 + kHistBins01 * 4;
  size_t counts = hist2 + kHistBins2 * 4;
  size_t bytes(int64_t n) const {
    const int64_t blocks = (n + kCmpChunk - 1) / kCmpChunk;
    const size_t end = counts + (size_t)blocks * 2 * sizeof(uint32_t);
    return (end + 255) & ~size_t(255);
  }
};

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide exclusive scan of one uint32 per thread (kSelThreads threads); returns
// the exclusive prefix and writes the block total to *total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* sh /*[4]*/) {
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
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const uint32_t s = sh[w];
    wbase += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

// One radix digit pass over the document keys.
template <int PASS>
__global__ __launch_bounds__(kSelThreads) void sel_hist_kernel(const float* __restrict__ scores,
                                                               int doc_begin, int doc_len,
                                                               uint32_t k_eff, SelState* st,
                                                               uint32_t* hist) {
  constexpr int BINS = PASS == 2 ? kHistBins2 : kHistBins01;
  __shared__ uint32_t lh[BINS];
  __shared__ uint32_t sh_scan[4];
  __shared__ int sh_last;
  const int tid = threadIdx.x;
  for (int i = tid; i < BINS; i += kSelThreads) lh[i] = 0;
  __syncthreads();
  const uint32_t prefix = PASS == 0 ? 0u : st->prefix;
  for (int i = blockIdx.x * kSelThreads + tid; i < doc_len; i += gridDim.x * kSelThreads) {
    const uint32_t key = score_key(scores[doc_begin + i]);
    if (PASS == 0) {
      atomicAdd(&lh[key >> 20], 1u);
    } else if (PASS == 1) {
      if ((key >> 20) == prefix) atomicAdd(&lh[(key >> 8) & 0xfffu], 1u);
    } else {
      if ((key >> 8) == prefix) atomicAdd(&lh[key & 0xffu], 1u);
    }
  }
  __syncthreads();
  for (int i = tid; i < BINS; i += kSelThreads)
    if (lh[i]) atomicAdd(&hist[i], lh[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) sh_last = (atomicAdd(&st->done[PASS], 1u) == gridDim.x - 1);
  __syncthreads();
  if (!sh_last) return;
  __threadfence();

  // Last block: walk the bins from the top (largest keys) down to the one that
  // holds the rank-th largest key among those with the current prefix.
  const uint32_t rank = PASS == 0 ? k_eff : st->rank;
  constexpr int PER = BINS / kSelThreads;
  uint32_t c[PER];
  uint32_t local = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    c[p] = ld_agent(&hist[BINS - 1 - (tid * PER + p)]);
    local += c[p];
  }
  uint32_t total;
  uint32_t above = block_excl_scan(local, &total, sh_scan);
  if (above < rank && rank <= above + local) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      if (rank <= above + c[p]) {
        const uint32_t bin = BINS - 1 - (tid * PER + p);
        st->prefix = PASS == 0 ? bin : (PASS == 1 ? (prefix << 12) | bin : (prefix << 8) | bin);
        st->rank = rank - above;
        break;
      }
      above += c[p];
    }
  }
  for (int i = tid; i < BINS; i += kSelThreads) hist[i] = 0u;
  if (tid == 0) st->done[PASS] = 0u;
}

// Selection outcome as (threshold key, quota of keys equal to it).
//   mode 0: keep no document token; mode 1: keep the whole document; mode 2: from the passes.
__device__ __forceinline__ void sel_threshold(int mode, const SelState* st, uint32_t* T, uint32_t* need) {
  if (mode == 0) { *T = 0xffffffffu; *need = 0u; }          // no key reaches 0xffffffff
  else if (mode == 1) { *T = 0u; *need = 0xffffffffu; }     // every key >= 0 = T, no quota
  else { *T = st->prefix; *need = st->rank; }
}

__device__ __forceinline__ void cmp_flags(const float* scores, int i, int n, int doc_begin, int doc_end,
                                          uint32_t T, uint32_t* base, uint32_t* eq) {
  *base = 0u; *eq = 0u;
  if (i >= n) return;
  if (i < doc_begin || i >= doc_end) { *base = 1u; return; }
  const uint32_t key = score_key(scores[i]);
  *base = key > T;
  *eq = key == T;
}

__global__ __launch_bounds__(kSelThreads) void sel_count_kernel(const float* __restrict__ scores, int n,
                                                                int doc_begin, int doc_end, int mode,
                                                                const SelState* st, uint32_t* counts) {
  __shared__ uint32_t sh[2][4];
  uint32_t T, need;
  sel_threshold(mode, st, &T, &need);
  const int i0 = blockIdx.x * kCmpChunk + threadIdx.x * kCmpPerThread;
  uint32_t nb = 0, ne = 0;
#pragma unroll
  for (int r = 0; r < kCmpPerThread; ++r) {
    uint32_t b, e;
    cmp_flags(scores, i0 + r, n, doc_begin, doc_end, T, &b, &e);
    nb += b; ne += e;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    nb += __shfl_xor(nb, o, 64);
    ne += __shfl_xor(ne, o, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { sh[0][wave] = nb; sh[1][wave] = ne; }
  __syncthreads();
  if (threadIdx.x == 0) {
    counts[2 * blockIdx.x] = sh[0][0] + sh[0][1] + sh[0][2] + sh[0][3];
    counts[2 * blockIdx.x + 1] = sh[1][0] + sh[1][1] + sh[1][2] + sh[1][3];
  }
}

__global__ __launch_bounds__(kSelThreads) void sel_write_kernel(const float* __restrict__ scores, int n,
                                                                int doc_begin, int doc_end, int mode,
                                                                const SelState* st,
                                                                const uint32_t* __restrict__ counts,
                                                                int32_t* __restrict__ kept, uint32_t m) {
  __shared__ uint32_t sh_scan[4];
  __shared__ uint32_t sh_red[2][4];
  uint32_t T, need;
  sel_threshold(mode, st, &T, &need);
  // offsets of this block: sums of the counts of all earlier blocks
  uint32_t pb = 0, pe = 0;
  for (int b = threadIdx.x; b < (int)blockIdx.x; b += kSelThreads) {
    pb += counts[2 * b];
    pe += counts[2 * b + 1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    pb += __shfl_xor(pb, o, 64);
    pe += __shfl_xor(pe, o, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { sh_red[0][wave] = pb; sh_red[1][wave] = pe; }
  __syncthreads();
  const uint32_t block_base = sh_red[0][0] + sh_red[0][1] + sh_red[0][2] + sh_red[0][3];
  const uint32_t block_eq = sh_red[1][0] + sh_red[1][1] + sh_red[1][2] + sh_red[1][3];

  const int i0 = blockIdx.x * kCmpChunk + threadIdx.x * kCmpPerThread;
  uint32_t fb[kCmpPerThread], fe[kCmpPerThread], nb = 0, ne = 0;
#pragma unroll
  for (int r = 0; r < kCmpPerThread; ++r) {
    cmp_flags(scores, i0 + r, n, doc_begin, doc_end, T, &fb[r], &fe[r]);
    nb += fb[r]; ne += fe[r];
  }
  // pack both counts in one 32-bit scan: each is <= kCmpChunk (< 2^16)
  uint32_t tot;
  const uint32_t ex = block_excl_scan(nb | (ne << 16), &tot, sh_scan);
  uint32_t base_before = block_base + (ex & 0xffffu);
  uint32_t eq_before = block_eq + (ex >> 16);
#pragma unroll
  for (int r = 0; r < kCmpPerThread; ++r) {
    const bool keep = fb[r] || (fe[r] && eq_before < need);
    const uint32_t slot = base_before + min(eq_before, need);
    if (keep && slot < m) kept[slot] = i0 + r;   // slot < m always holds; the guard is defensive
    base_before += fb[r];
    eq_before += fe[r];
  }
}

}  // namespace tg

extern "C" int64_t tg_num_kept(int64_t n, int64_t doc_begin, int64_t doc_end, int64_t k) {
  if (n < 0 || k < 0 || doc_begin < 0 || doc_begin > doc_end || doc_end > n) return -1;
  const int64_t d = doc_end - doc_begin;
  return (n - d) + (k < d ? k : d);
}

extern "C" size_t tg_select_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  return tg::SelLayout().bytes(n);
}

extern "C" tg_status tg_select_topk(int64_t n, const float* scores, int64_t doc_begin, int64_t doc_end,
                                    int64_t k, int32_t* kept_idx, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  using namespace tg;
  if (n <= 0 || n > INT32_MAX || tg_num_kept(n, doc_begin, doc_end, k) < 0) return TG_ERR_INVALID_ARG;
  if (tg_num_kept(n, doc_begin, doc_end, k) == 0) return TG_OK;   // nothing kept, nothing to write
  if (!scores || !kept_idx || !workspace) return TG_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return TG_ERR_INVALID_ARG;
  const SelLayout L;
  if (workspace_bytes < L.bytes(n)) return TG_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  SelState* state = reinterpret_cast<SelState*>(ws + L.state);
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + L.counts);
  const int nn = static_cast<int>(n), db = static_cast<int>(doc_begin), de = static_cast<int>(doc_end);
  const int64_t d = doc_end - doc_begin;
  const int64_t k_eff = k < d ? k : d;
  int mode;
  if (k_eff == 0) {
    mode = 0;
  } else if (k_eff == d) {
    mode = 1;
  } else {
    mode = 2;
    const int want = static_cast<int>((d + kSelThreads * 8 - 1) / (kSelThreads * 8));
    const int grid = want < 1 ? 1 : (want > kHistMaxBlocks ? kHistMaxBlocks : want);
    const int dl = static_cast<int>(d);
    const uint32_t ke = static_cast<uint32_t>(k_eff);
    hipLaunchKernelGGL(sel_hist_kernel<0>, dim3(grid), dim3(kSelThreads), 0, st, scores, db, dl, ke, state,
                       reinterpret_cast<uint32_t*>(ws + L.hist0));
    TG_CHECK_LAUNCH();
    hipLaunchKernelGGL(sel_hist_kernel<1>, dim3(grid), dim3(kSelThreads), 0, st, scores, db, dl, ke, state,
                       reinterpret_cast<uint32_t*>(ws + L.hist1));
    TG_CHECK_LAUNCH();
    hipLaunchKernelGGL(sel_hist_kernel<2>, dim3(grid), dim3(kSelThreads), 0, st, scores, db, dl, ke, state,
                       reinterpret_cast<uint32_t*>(ws + L.hist2));
    TG_CHECK_LAUNCH();
  }
  const int cblocks = static_cast<int>((n + kCmpChunk - 1) / kCmpChunk);
  hipLaunchKernelGGL(sel_count_kernel, dim3(cblocks), dim3(kSelThreads), 0, st, scores, nn, db, de, mode,
                     state, counts);
  TG_CHECK_LAUNCH();
  const uint32_t m = static_cast<uint32_t>(tg_num_kept(n, doc_begin, doc_end, k));
  hipLaunchKernelGGL(sel_write_kernel, dim3(cblocks), dim3(kSelThreads), 0, st, scores, nn, db, de, mode,
                     state, counts, kept_idx, m);
  TG_CHECK_LAUNCH();
  return TG_OK;
}
