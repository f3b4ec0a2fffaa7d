// S1 + S2: router logits, wavefront top-k, renormalised softmax, shared gate.
//
// [Strata] "显存里缓存的是什么？": the router decides which experts a token uses
// and the merge weight of each expert output; "还有一条会改变输出的路径" ranks a
// token's experts.  The k-way selection runs one wavefront per token: every lane
// keeps E/64 logits in registers as order-preserving integer keys, and k rounds
// of a wave-wide arg-max (logit descending, expert index ascending; two DPP
// reductions, the largest key then the lowest index holding it) retire one
// winner each.
#include <math.h>

#include "moe_common.hpp"

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

// Order-preserving map of a finite fp32 to uint32 (a larger float gets a larger
// key).  -0 is first made +0: the two zeros compare equal and must tie.
__device__ inline uint32_t f32_key(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_f32(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// DPP lane exchange (lanes a row mask leaves out keep their own value).
template <int CTRL, int ROWMASK = 0xF>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK = 0xF>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
// Wave-wide max: within quads (xor 1, xor 2), half rows and rows, then the row
// broadcasts fold rows 0..3 into lane 63, which every lane reads back.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
  v = max(v, dpp_u32<0x142, 0xA>(v));
  v = max(v, dpp_u32<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// fixed-order (deterministic) wave sum
__device__ inline float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  v += dpp_f32<0x142, 0xA>(v);
  v += dpp_f32<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One wavefront per token; 4 tokens per 256-thread block.  NPL = logits per
// lane (E <= 64 * NPL); lane l holds experts l, l + 64, ...
template <int NPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const uint16_t* __restrict__ x,
                                              const float* __restrict__ w_sg, int T, int H, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ wout,
                                              float* __restrict__ sigma) {
  extern __shared__ unsigned char smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  uint32_t* win_k = reinterpret_cast<uint32_t*>(smem) + wave * k;                       // [4][k]
  int* win_i = reinterpret_cast<int*>(smem + 4 * k * sizeof(uint32_t)) + wave * k;     // [4][k]
  STAGE_STAMP(0, 0);
  if (t >= T) return;

  // every load this wave needs is issued up front: the logits, and the first
  // four 8-value chunks per lane of x[t] and w_sg for the shared gate
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; i++) v[i] = logits[(int64_t)t * E + min(lane + 64 * i, E - 1)];
  const int nch = H / 8;
  const uint16_t* xr = x + (int64_t)t * H;
  uint4 xv[4];
  float4 wv[4][2];
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int cc = min(u * 64 + lane, nch - 1);
    xv[u] = *reinterpret_cast<const uint4*>(xr + 8 * cc);
    wv[u][0] = *reinterpret_cast<const float4*>(w_sg + 8 * cc);
    wv[u][1] = *reinterpret_cast<const float4*>(w_sg + 8 * cc + 4);
  }
  uint32_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; i++) key[i] = (lane + 64 * i < E) ? f32_key(v[i]) : 0u;  // 0: no entry (NaN keys only)
  STAGE_STAMP(0, 1);
  // k rounds: each takes the largest key, the lowest expert index among equal
  // keys, and retires it
  for (int j = 0; j < k; j++) {
    uint32_t kb = key[0];
#pragma unroll
    for (int i = 1; i < NPL; i++) kb = max(kb, key[i]);
    const uint32_t M = wave_max_u32(kb);
    // the lowest expert index holding M: per register slot i a ballot of the
    // lanes, searched from the highest slot down so the lowest i wins
    uint32_t I = 0;
#pragma unroll
    for (int i = NPL - 1; i >= 0; i--) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(key[i] == M);
      I = m ? (uint32_t)(64 * i + __builtin_ctzll(m)) : I;
    }
#pragma unroll
    for (int i = 0; i < NPL; i++) key[i] = ((uint32_t)(lane + 64 * i) == I) ? 0u : key[i];
    if (lane == 0) {
      win_k[j] = M;
      win_i[j] = (int)I;
    }
  }
  STAGE_STAMP(0, 2);
  // shared gate: z = x[t] . w_sg, lane-strided chunks, then a fixed-order sum
  float z = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const float m = (u * 64 + lane < nch) ? 1.0f : 0.0f;
    const uint32_t xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
    const float ws[8] = {wv[u][0].x, wv[u][0].y, wv[u][0].z, wv[u][0].w,
                         wv[u][1].x, wv[u][1].y, wv[u][1].z, wv[u][1].w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      z = fmaf(m * bf16_bits_to_f32(xs[i] & 0xFFFFu), ws[2 * i], z);
      z = fmaf(m * bf16_bits_to_f32(xs[i] >> 16), ws[2 * i + 1], z);
    }
  }
  for (int c = 256 + lane; c < nch; c += 64) {  // H > 2048
    const uint4 xq = *reinterpret_cast<const uint4*>(xr + 8 * c);
    const float4 w0 = *reinterpret_cast<const float4*>(w_sg + 8 * c);
    const float4 w1 = *reinterpret_cast<const float4*>(w_sg + 8 * c + 4);
    const uint32_t xs[4] = {xq.x, xq.y, xq.z, xq.w};
    const float ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      z = fmaf(bf16_bits_to_f32(xs[i] & 0xFFFFu), ws[2 * i], z);
      z = fmaf(bf16_bits_to_f32(xs[i] >> 16), ws[2 * i + 1], z);
    }
  }
  z = wave_sum_f32(z);
  STAGE_STAMP(0, 3);
  // renormalised softmax over the k winners; lane l takes slots l, l + 64, ...
  // (lane 0 wrote the winners; a wavefront's LDS accesses stay in order)
  __builtin_amdgcn_wave_barrier();
  const float l0 = key_f32(win_k[0]);
  float part = 0.0f;
  for (int j = lane; j < k; j += 64) part += expf(key_f32(win_k[j]) - l0);
  const float den = wave_sum_f32(part);
  for (int j = lane; j < k; j += 64) {
    ids[(int64_t)t * k + j] = win_i[j];
    wout[(int64_t)t * k + j] = expf(key_f32(win_k[j]) - l0) / den;
  }
  if (lane == 0) sigma[t] = 1.0f / (1.0f + expf(-z));
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
