// Gather of the kept rows: layers above the gate see only the kept tokens and no
// KV entry is made for a pruned one (aiproducthub.cn "斯坦福伯克利TokenGate
// 预填充提速11.3倍", section 事件详情; aisight.pl "TokenGate: Stanford i Berkeley ...",
// section "Jak to dziala").
//
// x_kept[r, :] = x[kept[r], :] and s_kept[r] = scores[kept[r]].  Pure data movement:
// each workgroup copies ROWS rows with 16-byte vector loads issued together before
// the stores, so one 4 KiB row (d_model 2048, bf16) is one load per thread.  8 rows per
// workgroup from 8192 rows on (half the workgroups, twice the bytes in flight per thread;
// at M = 8256 the 4-row grid, 2064 workgroups of 256 threads, is 16 more than the chip
// holds at once), 4 below, where more workgroups spread the rows over more CUs.
#include "tg_common.h"

namespace tg {

constexpr int kGatherThreads = 256;
constexpr int kGatherManyRows = 8192;   // from here on, 8 rows per workgroup

template <int ROWS>
__global__ __launch_bounds__(kGatherThreads) void gather_vec16_kernel(
    const char* __restrict__ x, int64_t ldx_bytes, int n, const int32_t* __restrict__ kept, int m,
    char* __restrict__ out, int64_t ldo_bytes, int pieces, const float* __restrict__ scores,
    float* __restrict__ s_kept) {
  const int r0 = blockIdx.x * ROWS;
  int src[ROWS];
  bool live[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    src[r] = (r0 + r < m) ? kept[r0 + r] : 0;
    live[r] = r0 + r < m && src[r] >= 0 && src[r] < n;   // out-of-range indices are skipped
  }
  for (int p = threadIdx.x; p < pieces; p += kGatherThreads) {
    u32x4 v[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      if (live[r]) v[r] = *reinterpret_cast<const u32x4*>(x + (int64_t)src[r] * ldx_bytes + 16 * (int64_t)p);
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      if (live[r]) *reinterpret_cast<u32x4*>(out + (int64_t)(r0 + r) * ldo_bytes + 16 * (int64_t)p) = v[r];
  }
  if (scores && threadIdx.x < ROWS && live[threadIdx.x])
    s_kept[r0 + threadIdx.x] = scores[src[threadIdx.x]];
}

// Any width / alignment: element-wise copy (2- or 4-byte elements).
template <typename E>
__global__ __launch_bounds__(kGatherThreads) void gather_elem_kernel(
    const E* __restrict__ x, int64_t ldx, int n, const int32_t* __restrict__ kept, int m, E* __restrict__ out,
    int64_t ldo, int width, const float* __restrict__ scores, float* __restrict__ s_kept) {
  const int r = blockIdx.x;
  if (r >= m) return;
  const int src = kept[r];
  if (src < 0 || src >= n) return;   // out-of-range indices are skipped
  for (int c = threadIdx.x; c < width; c += kGatherThreads) out[(int64_t)r * ldo + c] = x[(int64_t)src * ldx + c];
  if (scores && threadIdx.x == 0) s_kept[r] = scores[src];
}

}  // namespace tg

extern "C" tg_status tg_gather_kept(int32_t dtype, int64_t n, int32_t d_model, const void* x, int64_t ldx,
                                    const int32_t* kept_idx, int64_t m, void* x_kept, int64_t ld_out,
                                    const float* scores, float* s_kept, void* stream) {
  using namespace tg;
  if (dtype != TG_F32 && dtype != TG_BF16) return TG_ERR_INVALID_ARG;
  if (n <= 0 || n > INT32_MAX || m < 0 || m > INT32_MAX || d_model <= 0) return TG_ERR_INVALID_ARG;
  if (ldx < d_model || ld_out < d_model) return TG_ERR_INVALID_ARG;
  if ((scores == nullptr) != (s_kept == nullptr)) return TG_ERR_INVALID_ARG;
  if (m == 0) return TG_OK;
  if (!x || !kept_idx || !x_kept) return TG_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int esz = dtype == TG_BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)d_model * esz;
  const uintptr_t align = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_kept) |
                          static_cast<uintptr_t>(ldx * esz) | static_cast<uintptr_t>(ld_out * esz) |
                          static_cast<uintptr_t>(row_bytes);
  const int mm = static_cast<int>(m);
  if ((align & 15u) == 0) {
    const bool many = mm >= kGatherManyRows;
    const int rows = many ? 8 : 4;
    const int grid = (mm + rows - 1) / rows;
    hipLaunchKernelGGL(many ? gather_vec16_kernel<8> : gather_vec16_kernel<4>, dim3(grid), dim3(kGatherThreads), 0,
                       st, static_cast<const char*>(x), ldx * esz, static_cast<int>(n), kept_idx, mm,
                       static_cast<char*>(x_kept), ld_out * esz, static_cast<int>(row_bytes / 16), scores, s_kept);
  } else if (esz == 2) {
    hipLaunchKernelGGL(gather_elem_kernel<uint16_t>, dim3(mm), dim3(kGatherThreads), 0, st,
                       static_cast<const uint16_t*>(x), ldx, static_cast<int>(n), kept_idx, mm, static_cast<uint16_t*>(x_kept),
                       ld_out, d_model, scores, s_kept);
  } else {
    hipLaunchKernelGGL(gather_elem_kernel<uint32_t>, dim3(mm), dim3(kGatherThreads), 0, st,
                       static_cast<const uint32_t*>(x), ldx, static_cast<int>(n), kept_idx, mm, static_cast<uint32_t*>(x_kept),
                       ld_out, d_model, scores, s_kept);
  }
  TG_CHECK_LAUNCH();
  return TG_OK;
}
