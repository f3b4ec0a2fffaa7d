// MXFP8 quantisation of bf16 activations (OCP MX: E4M3FN codes, one E8M0
// scale per 32 consecutive values), shared by the MX kernels and by the
// route + group kernel that quantises x for the MX FFN in its own launch.
// [FreeToken] 2.1 (natively MXFP4 experts); the format is read as OCP MX.
#pragma once

#include "moe_common.hpp"

namespace moe {

// Two fp32 values of a block with E8M0 byte sb as OCP E4M3FN bytes (lo in
// byte 0, hi in byte 1): v / 2^(sb - 127) is exact (ldexp), clamped to
// +-448 (the saturation), then v_cvt_scalef32_pk_fp8_f32 with scale 1 rounds
// to the nearest E4M3 value, ties to even, subnormals included (it returns
// NaN above the range instead of saturating, hence the clamp).
__device__ __forceinline__ uint32_t e4m3_pair(float lo, float hi, int sb) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const float a = __builtin_amdgcn_fmed3f(ldexpf(lo, 127 - sb), -448.f, 448.f);
  const float b = __builtin_amdgcn_fmed3f(ldexpf(hi, 127 - sb), -448.f, 448.f);
  const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, a, b, 1.0f, false);
  return (uint32_t)(uint16_t)r[0];
}

// The E8M0 byte of a block with largest magnitude m (m >= 0, fp32): the shared
// exponent floor(log2 m) - 8, clamped below at -127 (zero and tiny blocks), is
// the biased fp32 exponent field minus 127 + 8.
__device__ __forceinline__ int e8m0_of_amax(float m) { return max((int)(__float_as_uint(m) >> 23) - 8, 0); }

// Eight consecutive bf16 values (one uint4) of a 32-value block whose other
// 24 values are held by the other three lanes of this lane's DPP quad (every
// lane of the quad calls this together): the block's E8M0 byte from its
// largest magnitude, each value's E4M3 code, and back the bf16 value the code
// stands for, e4m3(code) * 2^(sb - 127), exact in bf16 (both have at most 4
// significant bits; values below 2^-133 would round, far below any
// activation here).
__device__ __forceinline__ uint4 mx_quant8_bf16(const uint4 w) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  float f[8];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(ww[i] << 16);
    f[2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
    m = fmaxf(m, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
  }
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  const int sb = e8m0_of_amax(m);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t c2 = e4m3_pair(f[2 * i], f[2 * i + 1], sb);
    const float v0 = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)c2, 0), sb - 127);
    const float v1 = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)c2, 1), sb - 127);
    o[i] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);  // exact: the low halves are zero
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace moe
