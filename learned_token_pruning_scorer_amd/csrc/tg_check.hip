// Precondition check of the gated attention: the kept tokens' original positions must be
// strictly increasing (the order tg_select_topk writes them in), because the attention
// masks on positions and skips key tiles that lie wholly after a query tile, which is
// exact only then (aiproducthub.cn "斯坦福伯克利TokenGate 预填充提速11.3倍", section 事件详情:
// kept tokens keep their order; the causal mask is on original positions).
//
// tg_check_positions counts the violations with one workgroup (no cross-workgroup
// exchange, so no counter has to start at zero).  A library built with TG_DEBUG runs the
// same count inside the attention entry points, on a static device word, synchronises the
// stream and rejects a bad `pos` with TG_ERR_INVALID_ARG before launching anything.
#include <mutex>

#include "tg_common.h"

namespace tg {

constexpr int kCheckThreads = 1024;

// *violations = number of i in [1, m) with pos[i] <= pos[i - 1], plus the number of
// negative positions.
__global__ __launch_bounds__(kCheckThreads) void check_positions_kernel(const int32_t* __restrict__ pos, int64_t m,
                                                                       int32_t* __restrict__ violations) {
  __shared__ int32_t part[kCheckThreads / 64];
  int32_t bad = 0;
  for (int64_t i = threadIdx.x; i < m; i += kCheckThreads) {
    const int32_t p = pos[i];
    bad += (p < 0) ? 1 : 0;
    if (i > 0) bad += (p <= pos[i - 1]) ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bad += __shfl_xor(bad, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t tot = 0;
#pragma unroll
    for (int w = 0; w < kCheckThreads / 64; ++w) tot += part[w];
    *violations = tot;
  }
}

static tg_status launch_check(const int32_t* pos, int64_t m, int32_t* violations, hipStream_t stream) {
  hipLaunchKernelGGL(check_positions_kernel, dim3(1), dim3(kCheckThreads), 0, stream, pos, m, violations);
  TG_CHECK_LAUNCH();
  return TG_OK;
}

#ifdef TG_DEBUG
// the debug build's result word, one per device (no allocation)
static __device__ int32_t debug_violations;

tg_status debug_check_positions(const int32_t* pos, int64_t m, void* stream) {
  if (!pos || m <= 1) return TG_OK;
  static std::mutex mu;
  static void* addr[64] = {};
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= 64) return TG_ERR_HIP;
  void* word = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device] && hipGetSymbolAddress(&addr[device], HIP_SYMBOL(debug_violations)) != hipSuccess)
      return TG_ERR_HIP;
    word = addr[device];
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const tg_status s = launch_check(pos, m, static_cast<int32_t*>(word), st);
  if (s != TG_OK) return s;
  int32_t bad = 0;
  if (hipMemcpyAsync(&bad, word, sizeof(bad), hipMemcpyDeviceToHost, st) != hipSuccess) return TG_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return TG_ERR_HIP;
  return bad == 0 ? TG_OK : TG_ERR_INVALID_ARG;
}
#endif

}  // namespace tg

extern "C" tg_status tg_check_positions(const int32_t* pos, int64_t m, int32_t* violations, void* stream) {
  if (m < 0 || !violations || (m > 0 && !pos)) return TG_ERR_INVALID_ARG;
  return tg::launch_check(pos, m, violations, static_cast<hipStream_t>(stream));
}

extern "C" int32_t tg_debug_build(void) {
#ifdef TG_DEBUG
  return 1;
#else
  return 0;
#endif
}
