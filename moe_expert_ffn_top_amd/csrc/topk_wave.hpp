// Top-k selection and renormalised softmax of one token by one wavefront,
// shared by the top-k kernel and the fused route + group kernel (which
// selects through a threshold, topk_threshold, and falls back on the rounds).
//
// [Strata] "还有一条会改变输出的路径": a token's experts are ranked; the merge
// weights are the softmax of the chosen logits ("显存里缓存的是什么？").  Every lane
// keeps E/64 logits as order-preserving integer keys; k rounds of a wave-wide
// arg-max (logit descending, expert index ascending) retire one winner each.
#pragma once

#include "moe_common.hpp"

namespace moe {

// Order-preserving map of a finite fp32 to uint32 (a larger float gets a larger
// key).  -0 is first made +0: the two zeros compare equal and must tie.
__device__ __forceinline__ uint32_t f32_key(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// DPP lane exchange (lanes a row mask leaves out keep their own value).
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
// Wave-wide max: within quads (xor 1, xor 2), half rows and rows, then the row
// broadcasts fold rows 0..3 into lane 63, which every lane reads back.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
  v = max(v, dpp_u32<0x142, 0xA>(v));
  v = max(v, dpp_u32<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// fixed-order (deterministic) wave sum
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  v += dpp_f32<0x142, 0xA>(v);
  v += dpp_f32<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The shared gate's inputs of token t held by one lane: its first four
// 8-value chunks of x[t] and of w_sg (loads issued early so their latency
// overlaps the top-k rounds).
struct GateIn {
  uint4 xv[4];
  float4 wv[4][2];
};

__device__ __forceinline__ void gate_load(GateIn& g, const uint16_t* __restrict__ x, const float* __restrict__ w_sg, int t,
                                 int H) {
  const int lane = threadIdx.x & 63;
  const int nch = H / 8;
  const uint16_t* xr = x + (int64_t)t * H;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int cc = min(u * 64 + lane, nch - 1);
    g.xv[u] = *reinterpret_cast<const uint4*>(xr + 8 * cc);
    g.wv[u][0] = *reinterpret_cast<const float4*>(w_sg + 8 * cc);
    g.wv[u][1] = *reinterpret_cast<const float4*>(w_sg + 8 * cc + 4);
  }
}

// z = x[t] . w_sg: lane-strided chunks, then a fixed-order wave sum.
__device__ __forceinline__ float gate_dot(const GateIn& g, const uint16_t* __restrict__ x, const float* __restrict__ w_sg,
                                 int t, int H) {
  const int lane = threadIdx.x & 63;
  const int nch = H / 8;
  const uint16_t* xr = x + (int64_t)t * H;
  float z = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const float m = (u * 64 + lane < nch) ? 1.0f : 0.0f;
    const uint32_t xs[4] = {g.xv[u].x, g.xv[u].y, g.xv[u].z, g.xv[u].w};
    const float ws[8] = {g.wv[u][0].x, g.wv[u][0].y, g.wv[u][0].z, g.wv[u][0].w,
                         g.wv[u][1].x, g.wv[u][1].y, g.wv[u][1].z, g.wv[u][1].w};
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
  return wave_sum_f32(z);
}

// This lane's keys of experts e0 + lane + 64 i (i < NPL), 0 past e1.
template <int NPL>
__device__ __forceinline__ void load_keys(uint32_t* key, const float* __restrict__ logits, int t, int E, int e0, int e1) {
  const int lane = threadIdx.x & 63;
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; i++) v[i] = logits[(int64_t)t * E + min(e0 + lane + 64 * i, e1 - 1)];
#pragma unroll
  for (int i = 0; i < NPL; i++) key[i] = (e0 + lane + 64 * i < e1) ? f32_key(v[i]) : 0u;  // 0: no entry
}

// kk rounds over the wave's keys (experts e0 + lane + 64 i): each takes the
// largest key, the lowest expert index among equal keys, and retires it;
// lane 0 writes round j's key and expert to win_k[j], win_i[j].  kk must not
// exceed the number of entries.
template <int NPL>
__device__ __forceinline__ void topk_rounds(uint32_t* key, int e0, int kk, uint32_t* win_k, int* win_i) {
  const int lane = threadIdx.x & 63;
  for (int j = 0; j < kk; j++) {
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
      win_i[j] = e0 + (int)I;
    }
  }
}

// Renormalised softmax over the k winners (win_k / win_i in slot order, in
// LDS, written by this wavefront or before a barrier); lane l takes slots l,
// l + 64, ...; z is the shared gate's dot product.
// DEV: the weights and sigma are stored device-coherently (written through to
// memory), for workgroups on other XCDs of the same launch to read.
template <bool DEV = false>
__device__ __forceinline__ void topk_finish(const uint32_t* win_k, const int* win_i, int t, int k, float z,
                                   int32_t* __restrict__ ids, float* __restrict__ wout, float* __restrict__ sigma) {
  const int lane = threadIdx.x & 63;
  __builtin_amdgcn_wave_barrier();
  const float l0 = key_f32(win_k[0]);
  float part = 0.0f;
  for (int j = lane; j < k; j += 64) part += expf(key_f32(win_k[j]) - l0);
  const float den = wave_sum_f32(part);
  for (int j = lane; j < k; j += 64) {
    ids[(int64_t)t * k + j] = win_i[j];
    store_maybe_dev<DEV>(wout + (int64_t)t * k + j, expf(key_f32(win_k[j]) - l0) / den);
  }
  if (lane == 0) store_maybe_dev<DEV>(sigma + t, 1.0f / (1.0f + expf(-z)));
}

// Token t by the calling wavefront.  NPL = logits per lane (E <= 64 * NPL);
// lane l holds experts l, l + 64, ...  win_k / win_i: LDS arrays of k entries
// that receive the winners' keys and expert indices in slot order (lane 0
// writes them); ids / wout / sigma receive the token's outputs.
template <int NPL>
__device__ __forceinline__ void topk_wave(const float* __restrict__ logits, const uint16_t* __restrict__ x,
                                 const float* __restrict__ w_sg, int t, int H, int E, int k,
                                 int32_t* __restrict__ ids, float* __restrict__ wout, float* __restrict__ sigma,
                                 uint32_t* win_k, int* win_i) {
  // every load this wave needs is issued up front: the logits, and the first
  // four 8-value chunks per lane of x[t] and w_sg for the shared gate
  uint32_t key[NPL];
  load_keys<NPL>(key, logits, t, E, 0, E);
  GateIn g;
  gate_load(g, x, w_sg, t, H);
  topk_rounds<NPL>(key, 0, k, win_k, win_i);
  const float z = gate_dot(g, x, w_sg, t, H);
  topk_finish(win_k, win_i, t, k, z, ids, wout, sigma);
}

// Top-k of one token by the calling wavefront through a threshold: tau = the
// k-th largest of the 64 lane maxima with its low 16 bits cleared (a radix
// select over the top 16 bits of one value per lane, ballot and popcount).
// The k largest keys are all >= tau: the k lanes whose maxima reach tau hold k
// distinct keys >= tau.  A lower tau only admits more candidates, and the 16
// bits kept (sign, exponent, 7 mantissa bits) already leave few keys of
// continuous logits between tau and the k-th key.  The keys >= tau (usually a
// little over k) are compacted into cand (LDS, 64 entries of this wavefront,
// 16-byte aligned) and ranked exactly under (key descending, expert
// ascending): each candidate counts those that outrank it, two per broadcast
// LDS read, as 64-bit (key, ~expert) compares.  The winners land in win_k /
// win_i in slot order.  More than 64 such keys, or k > 64: the arg-max rounds
// instead.  Same winners, same order either way.
template <int NPL>
__device__ __forceinline__ void topk_threshold(uint32_t* key, int k, uint32_t* win_k, int* win_i, uint2* cand) {
  const int lane = threadIdx.x & 63;
  if (k > 64) {
    topk_rounds<NPL>(key, 0, k, win_k, win_i);
    return;
  }
  uint32_t lm = key[0];
#pragma unroll
  for (int i = 1; i < NPL; i++) lm = max(lm, key[i]);
  uint32_t tau = 0;
  for (int b = 31; b >= 16; b--) {
    const uint32_t c = tau | (1u << b);
    if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(lm >= c)) >= k) tau = c;
  }
  uint64_t m[NPL];
  int n = 0;
#pragma unroll
  for (int i = 0; i < NPL; i++) {
    m[i] = __builtin_amdgcn_ballot_w64(key[i] >= tau && key[i] != 0u);
    n += __builtin_popcountll(m[i]);
  }
  if (n > 64) {
    topk_rounds<NPL>(key, 0, k, win_k, win_i);
    return;
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < NPL; i++) {
    const uint32_t lo = (uint32_t)m[i], hi = (uint32_t)(m[i] >> 32);
    const int below = (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
    if ((m[i] >> lane) & 1ull) cand[base + below] = make_uint2(key[i], (uint32_t)(lane + 64 * i));
    base += __builtin_popcountll(m[i]);
  }
  __builtin_amdgcn_wave_barrier();
  const uint2 me = lane < n ? cand[lane] : make_uint2(0u, 0u);
  // (key, ~expert) as one 64-bit value: larger means ranked earlier
  const uint64_t pm = ((uint64_t)me.x << 32) | (uint32_t)~me.y;
  const uint4* c4 = reinterpret_cast<const uint4*>(cand);
  int rank = 0;
#pragma unroll 4
  for (int j = 0; j < n; j += 2) {   // two candidates per read; a last odd one masked
    const uint4 v = c4[j >> 1];
    rank += (((uint64_t)v.x << 32) | (uint32_t)~v.y) > pm ? 1 : 0;
    rank += (j + 1 < n && (((uint64_t)v.z << 32) | (uint32_t)~v.w) > pm) ? 1 : 0;
  }
  if (lane < n && rank < k) {
    win_k[rank] = me.x;
    win_i[rank] = (int)me.y;
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace moe
