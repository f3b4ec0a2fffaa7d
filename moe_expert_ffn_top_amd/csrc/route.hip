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

// Router logits on MFMA.  x is bf16 (exact in a bf16 MFMA operand); each fp32
// weight w is split exactly into three bf16 parts, w = hi + mid + lo
// (hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid: each residual has
// at most 16, then 8 significant bits).  Every product x * part is exact in
// fp32, so the only rounding is the fp32 accumulation of the MFMAs, over
// 3 * H / 32 partial sums per logit instead of H fused multiply-adds.
// Workgroup tile: 128 tokens x 128 experts, 64 values of H per step; four
// wavefronts, each 64 tokens x 64 experts.  x rows are staged as they are;
// the weights are split and transposed into [expert][h] tiles, two h values
// per 32-bit store.  VEC: E % 4 == 0 (weight rows read as float4).
constexpr int kRmTok = 128, kRmExp = 128, kRmK = 64, kRmRow = kRmK + 16;  // 160-byte LDS rows

template <bool VEC>
__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                     float* __restrict__ logits, int T, int H, int E) {
  __shared__ __align__(16) uint16_t As[2][kRmTok * kRmRow];
  __shared__ __align__(16) uint16_t Bs[2][3][kRmExp * kRmRow];
  const int t0 = blockIdx.x * kRmTok, e0 = blockIdx.y * kRmExp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 15, q = lane >> 4;
  // staging: x -> row ar, values 32 ah .. 32 ah + 31 of the step; W -> rows
  // 2 hp, 2 hp + 1 of the step, experts 16 eb .. 16 eb + 15
  const int ar = tid >> 1, ah = tid & 1;
  const int hp = tid & 31, eb = tid >> 5;
  const bool arow_in = t0 + ar < T;
  const uint16_t* xrow = x + (int64_t)min(t0 + ar, T - 1) * H + 32 * ah;
  uint4 xa[4];
  float wv[2][16];
  auto gload = [&](int h0) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      xa[i] = (h0 + 32 * ah < H) ? *reinterpret_cast<const uint4*>(xrow + h0 + 8 * i) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < 2; rr++) {
      const int h = h0 + 2 * hp + rr;
      const float* wp = w + (int64_t)min(h, H - 1) * E + e0 + 16 * eb;
      if (VEC && h < H && e0 + 16 * eb + 16 <= E) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float4 v = *reinterpret_cast<const float4*>(wp + 4 * i);
          wv[rr][4 * i] = v.x; wv[rr][4 * i + 1] = v.y; wv[rr][4 * i + 2] = v.z; wv[rr][4 * i + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; j++) wv[rr][j] = (h < H && e0 + 16 * eb + j < E) ? wp[j] : 0.0f;
      }
    }
  };
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  auto pack2 = [](float a, float b) {
    union {
      bf16x2 v;
      uint32_t u;
    } c;
    c.v = bf16x2{(__bf16)a, (__bf16)b};
    return c.u;
  };
  auto store = [&](int buf) {
    uint4* ad = reinterpret_cast<uint4*>(&As[buf][ar * kRmRow + 32 * ah]);
#pragma unroll
    for (int i = 0; i < 4; i++) ad[i] = arow_in ? xa[i] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const float a = wv[0][j], b = wv[1][j];
      const uint32_t hi = pack2(a, b);
      const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xFFFF0000u);
      const uint32_t mid = pack2(ra, rb);
      const float sa = ra - __uint_as_float(mid << 16), sb = rb - __uint_as_float(mid & 0xFFFF0000u);
      const uint32_t lo = pack2(sa, sb);
      const int off = (16 * eb + j) * kRmRow + 2 * hp;
      *reinterpret_cast<uint32_t*>(&Bs[buf][0][off]) = hi;
      *reinterpret_cast<uint32_t*>(&Bs[buf][1][off]) = mid;
      *reinterpret_cast<uint32_t*>(&Bs[buf][2][off]) = lo;
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  gload(0);
  store(0);
  __syncthreads();
  const int nsteps = (H + kRmK - 1) / kRmK;
  for (int st = 0; st < nsteps; st++) {
    const int buf = st & 1;
    if (st + 1 < nsteps) gload((st + 1) * kRmK);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      bf16x8 fa[4];
#pragma unroll
      for (int rb = 0; rb < 4; rb++)
        fa[rb] = *reinterpret_cast<const bf16x8*>(&As[buf][(64 * wm + 16 * rb + r) * kRmRow + 32 * ks + 8 * q]);
#pragma unroll
      for (int part = 0; part < 3; part++) {
        bf16x8 fb[4];
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
          fb[cb] = *reinterpret_cast<const bf16x8*>(
              &Bs[buf][part][(64 * wn + 16 * cb + r) * kRmRow + 32 * ks + 8 * q]);
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
#pragma unroll
          for (int cb = 0; cb < 4; cb++) acc[rb][cb] = mfma16x16x32(fa[rb], fb[cb], acc[rb][cb]);
      }
    }
    if (st + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }
  // D[i][j] of block (rb, cb): lane j + 16 (i / 4), element i % 4
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
#pragma unroll
    for (int e4 = 0; e4 < 4; e4++) {
      const int t = t0 + 64 * wm + 16 * rb + 4 * q + e4;
      if (t >= T) continue;
#pragma unroll
      for (int cb = 0; cb < 4; cb++) {
        const int e = e0 + 64 * wn + 16 * cb + r;
        if (e < E) logits[(int64_t)t * E + e] = acc[rb][cb][e4];
      }
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
  dim3 grid((d.T + kRmTok - 1) / kRmTok, (d.E + kRmExp - 1) / kRmExp);
  if (d.E % 4 == 0)
    hipLaunchKernelGGL(k_router_mfma<true>, grid, dim3(256), 0, s, x, w_router, logits, d.T, d.H, d.E);
  else
    hipLaunchKernelGGL(k_router_mfma<false>, grid, dim3(256), 0, s, x, w_router, logits, d.T, d.H, d.E);
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
