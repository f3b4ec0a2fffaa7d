// S5: weighted combine plus the sigmoid-gated shared expert.
//
// [Strata] "路由以后，专家怎样分工？": the outputs that belong to one token are
// matched up, each is multiplied by its router weight, they are summed, and the
// gated shared-expert contribution is added.  "少算这些专家，会付出什么代价？": the
// output is the shared contribution plus sum_i w_i E_i(x), with no
// renormalisation.  Gather form: each token reads its k expert rows through
// inv_perm, so no atomics are used and the fp32 summation order (slot 0..k-1,
// then the shared row) is fixed; the result is rounded once to bf16 (R2).
#include "moe_common.hpp"

namespace moe {
#ifdef MOE_STAGE_TIMING
STAGE_TIMES_DEFINE(moe_debug_stage_times_combine)
#endif
namespace {

// grid (T, ceil(H / (8 kCombineThreads))); kCombineThreads threads x 8
// consecutive columns.  Two dependent rounds of loads: the slot indices,
// weights, sigma and the shared row first, then every routed row of the token
// at once (kCombineSlots per pass).  Workgroups of one wavefront spread a
// token's row loads over several CUs.
constexpr int kCombineSlots = 16;
#ifndef MOE_COMBINE_THREADS
#define MOE_COMBINE_THREADS 64
#endif
constexpr int kCombineThreads = MOE_COMBINE_THREADS;

__global__ __launch_bounds__(kCombineThreads) void k_combine(const uint16_t* __restrict__ yr, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, const float* __restrict__ sigma,
                                                 int T, int H, int k, uint16_t* __restrict__ y) {
  STAGE_STAMP(2, 0);
  const int t = blockIdx.x;
  const int col = (blockIdx.y * kCombineThreads + threadIdx.x) * 8;
  if (col >= H) return;
  const float st = sigma[t];
  const uint4 vs = *reinterpret_cast<const uint4*>(yr + ((int64_t)T * k + t) * H + col);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += kCombineSlots) {
    int p[kCombineSlots];
    float wj[kCombineSlots];
#pragma unroll
    for (int u = 0; u < kCombineSlots; u++) {
      const int j = min(j0 + u, k - 1);
      p[u] = inv[(int64_t)t * k + j];
      wj[u] = (j0 + u < k) ? w[(int64_t)t * k + j] : 0.0f;
    }
    uint4 v[kCombineSlots];
#pragma unroll
    for (int u = 0; u < kCombineSlots; u++)
      v[u] = *reinterpret_cast<const uint4*>(yr + (int64_t)max(p[u], 0) * H + col);
#pragma unroll
    for (int u = 0; u < kCombineSlots; u++) {
      if (j0 + u >= k || p[u] < 0) continue;
      const uint32_t uu[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] = fmaf(wj[u], bf16_bits_to_f32(uu[i] & 0xFFFFu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj[u], bf16_bits_to_f32(uu[i] >> 16), acc[2 * i + 1]);
      }
    }
  }
  STAGE_STAMP(2, 1);
  const uint32_t u[4] = {vs.x, vs.y, vs.z, vs.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float a = fmaf(st, bf16_bits_to_f32(u[i] & 0xFFFFu), acc[2 * i]);
    const float b = fmaf(st, bf16_bits_to_f32(u[i] >> 16), acc[2 * i + 1]);
    o[i] = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
  }
  *reinterpret_cast<uint4*>(y + (int64_t)t * H + col) = make_uint4(o[0], o[1], o[2], o[3]);
  STAGE_STAMP(2, 2);
}

}  // namespace

hipError_t launch_combine(const moe_dims& d, const uint16_t* y_rows, const int32_t* inv_perm, const float* w,
                          const float* sigma, uint16_t* y, hipStream_t s) {
  dim3 grid((unsigned)d.T, (unsigned)((d.H + 8 * kCombineThreads - 1) / (8 * kCombineThreads)));
  hipLaunchKernelGGL(k_combine, grid, dim3(kCombineThreads), 0, s, y_rows, inv_perm, w, sigma, d.T, d.H, d.k, y);
  return hipGetLastError();
}

}  // namespace moe
