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
namespace {

// grid (T, ceil(H / 2048)); 256 threads x 8 consecutive columns.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ yr, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, const float* __restrict__ sigma,
                                                 int T, int H, int k, uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (col >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // batches of 8 slots: indices and weights, then the rows, then the math in slot order
  for (int j0 = 0; j0 < k; j0 += 8) {
    int p[8];
    float wj[8];
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      p[u] = (j0 + u < k) ? inv[(int64_t)t * k + j0 + u] : -1;
      wj[u] = (j0 + u < k) ? w[(int64_t)t * k + j0 + u] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; u++)
      v[u] = (p[u] >= 0) ? *reinterpret_cast<const uint4*>(yr + (int64_t)p[u] * H + col) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; u++) {
      if (p[u] < 0) continue;
      const uint32_t uu[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] = fmaf(wj[u], bf16_bits_to_f32(uu[i] & 0xFFFFu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj[u], bf16_bits_to_f32(uu[i] >> 16), acc[2 * i + 1]);
      }
    }
  }
  const float st = sigma[t];
  const uint4 v = *reinterpret_cast<const uint4*>(yr + ((int64_t)T * k + t) * H + col);
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float a = fmaf(st, bf16_bits_to_f32(u[i] & 0xFFFFu), acc[2 * i]);
    const float b = fmaf(st, bf16_bits_to_f32(u[i] >> 16), acc[2 * i + 1]);
    o[i] = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
  }
  *reinterpret_cast<uint4*>(y + (int64_t)t * H + col) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_combine(const moe_dims& d, const uint16_t* y_rows, const int32_t* inv_perm, const float* w,
                          const float* sigma, uint16_t* y, hipStream_t s) {
  dim3 grid((unsigned)d.T, (unsigned)((d.H + 2047) / 2048));
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, y_rows, inv_perm, w, sigma, d.T, d.H, d.k, y);
  return hipGetLastError();
}

}  // namespace moe
