// Measurement probes: the HBM read rate and the dense MFMA rates this GPU
// reaches, measured beside the published peaks that the rooflines divide by.
//
// k_probe_read streams a buffer once: each wavefront instruction reads one
// contiguous KiB (16 B per lane), eight KiB per wavefront per loop trip, the
// access pattern of the weight-streaming FFN at its best.  The loaded words
// are folded into one value that is stored only if it equals a constant the
// fill never produces, so the loads cannot be dropped and nothing is written.
//
// k_probe_mfma issues back-to-back MFMAs on register operands, four
// independent accumulators per wavefront, and stores each lane's sum at the
// end: kind 0 = v_mfma_f32_32x32x16_bf16 (the bf16 contractions of the
// grouped GEMM), kind 1 = the scaled 16x16x128 MFMA with fp8 (E4M3) A and
// fp4 (E2M1) B operands (what the MX grouped GEMM issues), kind 2 = the same
// with fp8 on both sides.
//
// k_probe_scaled_mfma runs one v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 A,
// E2M1 B, C = 0) per wavefront on operands given lane by lane, or, with split,
// the pair the MX grouped GEMM issues for gate/up (split_e4m3: big codes, then
// small codes into the same accumulator): the instruction's own arithmetic,
// held against exact sums by the tests.
#include <hip/hip_runtime.h>

#include "moe_common.hpp"

namespace moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kReadChunk = 8192;   // bytes per wavefront per loop trip
constexpr uint32_t kNever = 0x9e3779b9u;

__global__ __launch_bounds__(256) void k_probe_read(const uint4* __restrict__ p, uint64_t n_chunks,
                                                    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint64_t w = (static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const uint64_t nw = (static_cast<uint64_t>(gridDim.x) * blockDim.x) >> 6;
  uint32_t acc = 0;
  for (uint64_t c = w; c < n_chunks; c += nw) {
    const uint4* b = p + c * (kReadChunk / 16);
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = b[i * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; i++) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (acc == kNever) sink[0] = acc;
}

template <int KIND>
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float* __restrict__ sink) {
  const int t = threadIdx.x & 63;   // operands depend on the lane only: every wavefront computes the same
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      a[e] = static_cast<__bf16>(static_cast<float>((t + e) & 7) * 0.125f);
      b[e] = static_cast<__bf16>(static_cast<float>((t * 3 + e) & 7) * 0.0625f);
    }
    for (int i = 0; i < iters; i++) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc3, 0, 0, 0);
    }
  } else {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      a[e] = 0x38303830 ^ ((t + e) & 0x07070707);    // small E4M3 values
      b[e] = (KIND == 1 ? 0x23232323 : 0x30383038) ^ ((t * 5 + e) & 0x01010101);
    }
    constexpr int kFmtB = KIND == 1 ? 4 : 0;   // 4 = E2M1, 0 = E4M3
    const int s = 127;                          // E8M0 scale 2^0
    for (int i = 0; i < iters; i++) {
      c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, 0, kFmtB, 0, s, 0, s);
      c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c1, 0, kFmtB, 0, s, 0, s);
      c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c2, 0, kFmtB, 0, s, 0, s);
      c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c3, 0, kFmtB, 0, s, 0, s);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int e = 0; e < 16; e++) r += acc0[e] + acc1[e] + acc2[e] + acc3[e];
#pragma unroll
  for (int e = 0; e < 4; e++) r += c0[e] + c1[e] + c2[e] + c3[e];
  sink[static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = r;
}

template <bool SPLIT>
__global__ __launch_bounds__(64) void k_probe_scaled_mfma(const int32_t* __restrict__ a, const int32_t* __restrict__ b,
                                                          const int32_t* __restrict__ sa,
                                                          const int32_t* __restrict__ sb, float* __restrict__ d) {
  const uint64_t l = static_cast<uint64_t>(blockIdx.x) * 64 + threadIdx.x;
  i32x8 av, bv = {};
#pragma unroll
  for (int i = 0; i < 8; i++) av[i] = a[8 * l + i];
#pragma unroll
  for (int i = 0; i < 4; i++) bv[i] = b[4 * l + i];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (SPLIT) {
    i32x8 big, small;
    split_e4m3(av, big, small);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(big, bv, acc, 0, 4, 0, sa[l], 0, sb[l]);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(small, bv, acc, 0, 4, 0, sa[l], 0, sb[l]);
  } else {
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 4, 0, sa[l], 0, sb[l]);
  }
#pragma unroll
  for (int e = 0; e < 4; e++) d[4 * l + e] = acc[e];
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_probe_hbm_read(const void* buf, uint64_t bytes, int32_t grid, uint32_t* sink, moe_stream_t stream) {
  if (!buf || !sink) return moe::record_error(MOE_ERR_ARG, "buf and sink are required");
  if (bytes == 0 || bytes % moe::kReadChunk)
    return moe::record_error(MOE_ERR_ARG, "bytes must be a positive multiple of 8192");
  if (reinterpret_cast<uintptr_t>(buf) & 15) return moe::record_error(MOE_ERR_ALIGN, "buf must be 16-byte aligned");
  if (grid < 1 || grid > (1 << 20)) return moe::record_error(MOE_ERR_ARG, "grid must be in [1, 2^20]");
  hipLaunchKernelGGL(moe::k_probe_read, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), bytes / moe::kReadChunk, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return moe::record_error(MOE_ERR_HIP, hipGetErrorString(e));
  return MOE_OK;
}

int moe_probe_mfma(int32_t kind, int32_t grid, int32_t iters, float* sink, moe_stream_t stream) {
  if (!sink) return moe::record_error(MOE_ERR_ARG, "sink is required");
  if (kind < 0 || kind > 2) return moe::record_error(MOE_ERR_ARG, "kind must be 0, 1 or 2");
  if (grid < 1 || grid > (1 << 16) || iters < 1 || iters > (1 << 20))
    return moe::record_error(MOE_ERR_ARG, "grid must be in [1, 2^16] and iters in [1, 2^20]");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (kind == 0) hipLaunchKernelGGL(moe::k_probe_mfma<0>, dim3(grid), dim3(256), 0, s, iters, sink);
  if (kind == 1) hipLaunchKernelGGL(moe::k_probe_mfma<1>, dim3(grid), dim3(256), 0, s, iters, sink);
  if (kind == 2) hipLaunchKernelGGL(moe::k_probe_mfma<2>, dim3(grid), dim3(256), 0, s, iters, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return moe::record_error(MOE_ERR_HIP, hipGetErrorString(e));
  return MOE_OK;
}

int moe_probe_scaled_mfma(const int32_t* a, const int32_t* b, const int32_t* sa, const int32_t* sb, int32_t n,
                          int32_t split, float* d, moe_stream_t stream) {
  if (!a || !b || !sa || !sb || !d) return moe::record_error(MOE_ERR_ARG, "a, b, sa, sb and d are required");
  if (n < 1 || n > (1 << 16)) return moe::record_error(MOE_ERR_ARG, "n must be in [1, 2^16]");
  if (split != 0 && split != 1) return moe::record_error(MOE_ERR_ARG, "split must be 0 or 1");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (split) hipLaunchKernelGGL(moe::k_probe_scaled_mfma<true>, dim3(n), dim3(64), 0, s, a, b, sa, sb, d);
  else hipLaunchKernelGGL(moe::k_probe_scaled_mfma<false>, dim3(n), dim3(64), 0, s, a, b, sa, sb, d);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return moe::record_error(MOE_ERR_HIP, hipGetErrorString(e));
  return MOE_OK;
}

}  // extern "C"
