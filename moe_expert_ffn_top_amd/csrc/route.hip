// S1 + S2: router logits, wavefront top-k, renormalised softmax, shared gate.
//
// [Strata] "显存里缓存的是什么？": the router decides which experts a token uses
// and the merge weight of each expert output; "还有一条会改变输出的路径" ranks a
// token's experts.  The k-way selection runs one wavefront per token: every lane
// keeps E/64 logits in registers and k rounds of a wave-wide arg-max (logit
// descending, expert index ascending) retire one winner each.
#include <math.h>

#include "moe_common.hpp"

namespace moe {
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

constexpr int kMaxPerLane = 16;  // E <= 1024 = 64 lanes x 16

__device__ inline bool better(float va, int ia, float vb, int ib) { return va > vb || (va == vb && ia < ib); }

// One wavefront per token; 4 tokens per 256-thread block.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const uint16_t* __restrict__ x,
                                              const float* __restrict__ w_sg, int T, int H, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ wout,
                                              float* __restrict__ sigma) {
  extern __shared__ unsigned char smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  float* win_v = reinterpret_cast<float*>(smem) + wave * k;                       // [4][k]
  int* win_i = reinterpret_cast<int*>(smem + 4 * k * sizeof(float)) + wave * k;   // [4][k]
  if (t >= T) return;

  float v[kMaxPerLane];
  uint32_t alive = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; i++) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? logits[(int64_t)t * E + e] : 0.0f;
    if (e < E) alive |= 1u << i;
  }
  for (int j = 0; j < k; j++) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; i++) {
      const int e = lane + 64 * i;
      if (((alive >> i) & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    // wave-wide arg-max; every lane ends with the winner
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) alive &= ~(1u << (bi >> 6));
    if (lane == 0) {
      win_v[j] = bv;
      win_i[j] = bi;
    }
  }
  // shared gate: z = x[t] . w_sg.  Lane l takes 8-value chunks l, l+64, ...;
  // loads of 4 chunks are issued before their math; then a fixed xor tree.
  float z = 0.0f;
  const int nch = H / 8;
  const uint16_t* xr = x + (int64_t)t * H;
  for (int c0 = 0; c0 < nch; c0 += 4 * 64) {
    uint4 xv[4];
    float4 wv[4][2];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int c = c0 + u * 64 + lane;
      xv[u] = make_uint4(0, 0, 0, 0);
      wv[u][0] = wv[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < nch) {
        xv[u] = *reinterpret_cast<const uint4*>(xr + 8 * c);
        wv[u][0] = *reinterpret_cast<const float4*>(w_sg + 8 * c);
        wv[u][1] = *reinterpret_cast<const float4*>(w_sg + 8 * c + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const uint32_t xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
      const float ws[8] = {wv[u][0].x, wv[u][0].y, wv[u][0].z, wv[u][0].w,
                           wv[u][1].x, wv[u][1].y, wv[u][1].z, wv[u][1].w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        z = fmaf(bf16_bits_to_f32(xs[i] & 0xFFFFu), ws[2 * i], z);
        z = fmaf(bf16_bits_to_f32(xs[i] >> 16), ws[2 * i + 1], z);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
  // lane 0 wrote the winners above and is the only reader: no barrier needed
  if (lane == 0) {
    const float l0 = win_v[0];
    float den = 0.0f;
    for (int j = 0; j < k; j++) den += expf(win_v[j] - l0);
    for (int j = 0; j < k; j++) {
      ids[(int64_t)t * k + j] = win_i[j];
      wout[(int64_t)t * k + j] = expf(win_v[j] - l0) / den;
    }
    sigma[t] = 1.0f / (1.0f + expf(-z));
  }
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
  const size_t shmem = (size_t)4 * d.k * (sizeof(float) + sizeof(int));
  hipLaunchKernelGGL(k_topk, dim3((d.T + 3) / 4), dim3(256), shmem, s, logits, x, w_sg, d.T, d.H, d.E, d.k, ids, w,
                     sigma);
  return hipGetLastError();
}

}  // namespace moe
