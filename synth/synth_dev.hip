// Seeded synthetic inputs, device implementation (gfx950).
//
// Implements the recipe in synth_recipe.md, independently of synth_host.c; a
// GPU test compares the two byte for byte.  Built with -ffp-contract=off so
// every fp32 operation rounds once.  Used to fill the multi-GB expert pools
// that would take minutes to generate on the host.  It encodes random weights
// only and holds none of the MoE layer's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "blob_pos.h"

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t rng(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGolden); }

__host__ __device__ inline uint64_t make_key(uint64_t seed, uint64_t kind, uint64_t cfg, uint64_t a, uint64_t b,
                                             uint64_t c) {
  return mix64(mix64(seed) ^ (kind << 60) ^ (cfg << 52) ^ (a << 32) ^ (b << 8) ^ c);
}

__device__ inline uint32_t sum16(uint64_t r) {
  return (uint32_t)(r & 0xFFFF) + (uint32_t)((r >> 16) & 0xFFFF) + (uint32_t)((r >> 32) & 0xFFFF) +
         (uint32_t)(r >> 48);
}

__device__ inline float normal_dev(uint64_t key, uint64_t i) {
  uint32_t s = sum16(rng(key, 3 * i)) + sum16(rng(key, 3 * i + 1)) + sum16(rng(key, 3 * i + 2));
  return __fmul_rn((float)((int32_t)s - 393210), 1.0f / 65536.0f);
}

__device__ inline uint8_t e4m3_encode(float v) {
  if (!(v > 0.0f)) return 0;
  if (v < 0.015625f) return (uint8_t)rintf(__fmul_rn(v, 512.0f));
  uint32_t u = __float_as_uint(v);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
  int32_t b = (int32_t)r - 960;
  if (b > 0x7E) b = 0x7E;
  return (uint8_t)b;
}

__device__ inline float e4m3_value(uint8_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return __fmul_rn((float)m, 1.0f / 512.0f);
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

__device__ inline uint8_t e2m1_encode(float q) {
  float a = fabsf(q);
  uint8_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  if (c != 0 && q < 0.0f) c |= 8;
  return c;
}

__host__ __device__ inline float global_scale(uint64_t seed, int cfg, int layer, int expert, int matrix) {
  uint64_t r = rng(make_key(seed, 2, cfg, layer, expert, matrix), 0);
  float f = 1.0f + (float)(r >> 56) * (1.0f / 256.0f);
  float base = 0.12f / 2688.0f;
  return base * f;
}

struct BlobGeom {
  uint64_t off_codes[3];
  uint64_t off_scales[3];
  uint64_t off_globals;
  uint64_t slot_stride;
  int H, I;
};

// One thread per 16-value block of the 3 matrices of expert blockIdx.y of layer `layer`.
__global__ void k_pool_layer(uint64_t seed, int cfg, int layer, const int32_t* __restrict__ slot_row,
                             int64_t n_slots, BlobGeom g, uint8_t* __restrict__ pool) {
  const int expert = blockIdx.y;
  const int32_t slot = slot_row[expert];
  if (slot < 0 || slot >= n_slots) return;
  uint8_t* blob = pool + (uint64_t)slot * g.slot_stride;
  const uint64_t nb_gu = (uint64_t)g.I * (g.H / 16);  // blocks in gate (and in up)
  const uint64_t nb_all = 3 * nb_gu;                  // down has H*I/16 blocks too
  const uint64_t gb = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gb < 3) {
    const float G = global_scale(seed, cfg, layer, expert, (int)gb);
    *reinterpret_cast<float*>(blob + g.off_globals + 4 * gb) = G;
  }
  if (gb >= nb_all) return;
  const int m = (int)(gb / nb_gu);
  const uint64_t lb = gb - (uint64_t)m * nb_gu;
  const int K = m < 2 ? g.H : g.I;
  const int nbr = K / 16;
  const uint64_t n = lb / nbr;
  const int b = (int)(lb % nbr);
  const uint64_t key = make_key(seed, 1, cfg, layer, expert, m);
  const float G = global_scale(seed, cfg, layer, expert, m);
  const float t6 = __fmul_rn(6.0f, G);
  float w[16];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const uint64_t i = n * (uint64_t)K + (uint64_t)(16 * b + j);
    w[j] = __fmul_rn(0.02f, normal_dev(key, i));
    amax = fmaxf(amax, fabsf(w[j]));
  }
  const uint8_t sb = e4m3_encode(__fdiv_rn(amax, t6));
  blob[g.off_scales[m] + synth_scale_pos(n, b, K)] = sb;
  uint32_t lo = 0, hi = 0;
  if (sb != 0) {
    const float d = __fmul_rn(e4m3_value(sb), G);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t c = (uint32_t)e2m1_encode(__fdiv_rn(w[2 * j], d)) |
                         ((uint32_t)e2m1_encode(__fdiv_rn(w[2 * j + 1], d)) << 4);
      if (j < 4) lo |= c << (8 * j);
      else hi |= c << (8 * (j - 4));
    }
  }
  uint2 v;
  v.x = lo;
  v.y = hi;
  *reinterpret_cast<uint2*>(blob + g.off_codes[m] + synth_code_pos(n, b, K)) = v;
}

// MX recipe (synth_recipe.md): one thread per 32-value block.
__global__ void k_pool_layer_mx(uint64_t seed, int cfg, int layer, const int32_t* __restrict__ slot_row,
                                int64_t n_slots, BlobGeom g, uint8_t* __restrict__ pool) {
  const int expert = blockIdx.y;
  const int32_t slot = slot_row[expert];
  if (slot < 0 || slot >= n_slots) return;
  uint8_t* blob = pool + (uint64_t)slot * g.slot_stride;
  const uint64_t nb_gu = (uint64_t)g.I * (g.H / 32);
  const uint64_t gb = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gb >= 3 * nb_gu) return;
  const int m = (int)(gb / nb_gu);
  const uint64_t lb = gb - (uint64_t)m * nb_gu;
  const int K = m < 2 ? g.H : g.I;
  const int nbr = K / 32;
  const uint64_t n = lb / nbr;
  const int b = (int)(lb % nbr);
  const uint64_t key = make_key(seed, 1, cfg, layer, expert, m);
  float w[32];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; j++) {
    const uint64_t i = n * (uint64_t)K + (uint64_t)(32 * b + j);
    w[j] = __fmul_rn(0.02f, normal_dev(key, i));
    amax = fmaxf(amax, fabsf(w[j]));
  }
  const uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFFu;
  const uint8_t sb = ef >= 2 ? (uint8_t)(ef - 2) : 0;
  blob[g.off_scales[m] + synth_mx_scale_pos(n, b, K)] = sb;
  const float inv = __uint_as_float((uint32_t)(254 - sb) << 23);
#pragma unroll
  for (int h = 0; h < 2; h++) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t c = (uint32_t)e2m1_encode(__fmul_rn(w[16 * h + 2 * j], inv)) |
                         ((uint32_t)e2m1_encode(__fmul_rn(w[16 * h + 2 * j + 1], inv)) << 4);
      if (j < 4) lo |= c << (8 * j);
      else hi |= c << (8 * (j - 4));
    }
    uint2 v;
    v.x = lo;
    v.y = hi;
    *reinterpret_cast<uint2*>(blob + g.off_codes[m] + synth_code_pos(n, 2 * b + h, K)) = v;
  }
}

__global__ void k_x(uint64_t key, int64_t n, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t u = __float_as_uint(normal_dev(key, (uint64_t)i));
  out[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void k_w(uint64_t key, int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = __fmul_rn(0.02f, normal_dev(key, (uint64_t)i));
}

}  // namespace

extern "C" {

// Fill the blobs of every (layer, expert) of `layers` [layer0, layer0+n_layers)
// whose slot (slot_table_dev[layer][expert], a device int32 [L][E1] table) is in
// [0, n_slots).  pool is a device buffer of n_slots * slot_stride bytes.
// Returns 0, or a hipError_t.
int synth_dev_pool(uint64_t seed, int cfg, int layer0, int n_layers, int E1, int H, int I,
                   const int32_t* slot_table_dev, int64_t n_slots, const uint64_t* off_codes,
                   const uint64_t* off_scales, uint64_t off_globals, uint64_t slot_stride, void* pool,
                   hipStream_t stream) {
  BlobGeom g;
  for (int m = 0; m < 3; m++) {
    g.off_codes[m] = off_codes[m];
    g.off_scales[m] = off_scales[m];
  }
  g.off_globals = off_globals;
  g.slot_stride = slot_stride;
  g.H = H;
  g.I = I;
  const uint64_t nb_all = 3ull * (uint64_t)I * (uint64_t)(H / 16);
  dim3 grid((unsigned)((nb_all + 255) / 256), (unsigned)E1);
  for (int l = layer0; l < layer0 + n_layers; l++) {
    hipLaunchKernelGGL(k_pool_layer, grid, dim3(256), 0, stream, seed, cfg, l, slot_table_dev + (int64_t)l * E1,
                       n_slots, g, static_cast<uint8_t*>(pool));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

// As synth_dev_pool, with MX blobs (no globals).
int synth_dev_pool_mx(uint64_t seed, int cfg, int layer0, int n_layers, int E1, int H, int I,
                      const int32_t* slot_table_dev, int64_t n_slots, const uint64_t* off_codes,
                      const uint64_t* off_scales, uint64_t slot_stride, void* pool, hipStream_t stream) {
  BlobGeom g;
  for (int m = 0; m < 3; m++) {
    g.off_codes[m] = off_codes[m];
    g.off_scales[m] = off_scales[m];
  }
  g.off_globals = 0;
  g.slot_stride = slot_stride;
  g.H = H;
  g.I = I;
  const uint64_t nb_all = 3ull * (uint64_t)I * (uint64_t)(H / 32);
  dim3 grid((unsigned)((nb_all + 255) / 256), (unsigned)E1);
  for (int l = layer0; l < layer0 + n_layers; l++) {
    hipLaunchKernelGGL(k_pool_layer_mx, grid, dim3(256), 0, stream, seed, cfg, l, slot_table_dev + (int64_t)l * E1,
                       n_slots, g, static_cast<uint8_t*>(pool));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

int synth_dev_x(uint64_t seed, int cfg, int layer, int step, int T, int H, uint16_t* out, hipStream_t stream) {
  const int64_t n = (int64_t)T * H;
  hipLaunchKernelGGL(k_x, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     make_key(seed, 3, cfg, layer, step, 0), n, out);
  return (int)hipGetLastError();
}

int synth_dev_w_router(uint64_t seed, int cfg, int layer, int H, int E, float* out, hipStream_t stream) {
  const int64_t n = (int64_t)H * E;
  hipLaunchKernelGGL(k_w, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     make_key(seed, 4, cfg, layer, 0, 0), n, out);
  return (int)hipGetLastError();
}

int synth_dev_w_shared_gate(uint64_t seed, int cfg, int layer, int H, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_w, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, stream,
                     make_key(seed, 5, cfg, layer, 0, 0), (int64_t)H, out);
  return (int)hipGetLastError();
}

}  // extern "C"
