// S1 + S2: router logits, wavefront top-k, renormalised softmax, shared gate.
//
// [Strata] "显存里缓存的是什么？": the router decides which experts a token uses
// and the merge weight of each expert output; "还有一条会改变输出的路径" ranks a
// token's experts.  The k-way selection runs one wavefront per token: every lane
// keeps E/64 logits in registers as order-preserving integer keys, and k rounds
// of a wave-wide arg-max (logit descending, expert index ascending: a DPP max
// of the keys, then a ballot for the lowest index holding it) retire one winner
// each (topk_wave.hpp).
#include <math.h>

#include "moe_common.hpp"
#include "topk_wave.hpp"

namespace moe {
#ifdef MOE_STAGE_TIMING
STAGE_TIMES_DEFINE(moe_debug_stage_times_route)
#endif
namespace {

constexpr int kRtTok = 64;  // router GEMM tile: tokens
constexpr int kRtExp = 64;  // router GEMM tile: experts
constexpr int kRtK = 16;    // router GEMM K step

// logits[t][e] = sum_h x[t][h] * W[h][e] in fp32, h ascending (deterministic).
// 256 threads, each 4 tokens x 4 experts.
__global__ __launch_bounds__(256) void k_router_matrix(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ w, float* __restrict__ logits,
                                                       int T, int H, int E) {
  __shared__ float xs[kRtK][kRtTok + 4];
  __shared__ float ws[kRtK][kRtExp + 4];
  const int t0 = blockIdx.x * kRtTok, e0 = blockIdx.y * kRtExp;
  const int tid = threadIdx.x;
  const int tr = (tid / 16) * 4, er = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int h0 = 0; h0 < H; h0 += kRtK) {
    for (int i = tid; i < kRtK * kRtTok; i += 256) {
      const int tt = i / kRtK, hh = i % kRtK;
      const int t = t0 + tt;
      xs[hh][tt] = (t < T) ? bf16_bits_to_f32(x[(int64_t)t * H + h0 + hh]) : 0.0f;
    }
    for (int i = tid; i < kRtK * kRtExp; i += 256) {
      const int hh = i / kRtExp, ee = i % kRtExp;
      const int e = e0 + ee;
      ws[hh][ee] = (e < E) ? w[(int64_t)(h0 + hh) * E + e] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < kRtK; hh++) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        a[i] = xs[hh][tr + i];
        b[i] = ws[hh][er + i];
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int t = t0 + tr + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = e0 + er + j;
      if (e < E) logits[(int64_t)t * E + e] = acc[i][j];
    }
  }
}

// One wavefront per token; 4 tokens per 256-thread block.
template <int NPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const uint16_t* __restrict__ x,
                                              const float* __restrict__ w_sg, int T, int H, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ wout,
                                              float* __restrict__ sigma) {
  extern __shared__ unsigned char smem[];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  uint32_t* win_k = reinterpret_cast<uint32_t*>(smem) + wave * k;                       // [4][k]
  int* win_i = reinterpret_cast<int*>(smem + 4 * k * sizeof(uint32_t)) + wave * k;     // [4][k]
  STAGE_STAMP(0, 0);
  if (t >= T) return;
  topk_wave<NPL>(logits, x, w_sg, t, H, E, k, ids, wout, sigma, win_k, win_i);
  STAGE_STAMP(0, 4);
}

}  // namespace

hipError_t launch_router_matrix(const moe_dims& d, const uint16_t* x, const float* w_router, float* logits,
                                hipStream_t s) {
  dim3 grid((d.T + kRtTok - 1) / kRtTok, (d.E + kRtExp - 1) / kRtExp);
  hipLaunchKernelGGL(k_router_matrix, grid, dim3(256), 0, s, x, w_router, logits, d.T, d.H, d.E);
  return hipGetLastError();
}

hipError_t launch_topk(const moe_dims& d, const float* logits, const uint16_t* x, const float* w_sg, int32_t* ids,
                       float* w, float* sigma, hipStream_t s) {
  const size_t shmem = (size_t)4 * d.k * (sizeof(uint32_t) + sizeof(int));
  const dim3 g((d.T + 3) / 4), b(256);
  const int npl = (d.E + 63) / 64;
  if (npl <= 1) hipLaunchKernelGGL(k_topk<1>, g, b, shmem, s, logits, x, w_sg, d.T, d.H, d.E, d.k, ids, w, sigma);
  else if (npl <= 2) hipLaunchKernelGGL(k_topk<2>, g, b, shmem, s, logits, x, w_sg, d.T, d.H, d.E, d.k, ids, w, sigma);
  else if (npl <= 4) hipLaunchKernelGGL(k_topk<4>, g, b, shmem, s, logits, x, w_sg, d.T, d.H, d.E, d.k, ids, w, sigma);
  else if (npl <= 8) hipLaunchKernelGGL(k_topk<8>, g, b, shmem, s, logits, x, w_sg, d.T, d.H, d.E, d.k, ids, w, sigma);
  else hipLaunchKernelGGL(k_topk<16>, g, b, shmem, s, logits, x, w_sg, d.T, d.H, d.E, d.k, ids, w, sigma);
  return hipGetLastError();
}

}  // namespace moe
