// S4: block-FP4 expert FFNs on MFMA.
//
// [Strata] "路由以后，专家怎样分工？" and "CPU 怎样把剩下的专家算完？": an expert computes
// gate/up, the activation, re-encodes the intermediate for the next kernel
// (here bf16, rounding point R1), then the down projection (bf16 output, R3).
// [PLE] "NVFP4 code 和 scale 如何反量化": value = E2M1 code x E4M3 block scale x fp32
// global; [PLE] also keeps weights packed across the slow path and dequantises
// on the consumer, which is what these kernels do: codes are decoded in
// registers and never written back.
//
// Tile kernel: one workgroup = 4 wavefronts = one tile of <= 16 rows of one
// group x 16 output units; the wavefronts split the reduction axis K and sum
// their partials through LDS.  Lane (c = lane % 16, q = lane / 16) owns output
// unit c and, in each step, the 32-value chunk q of a 128-value K slice: it
// loads 16 bytes of codes (32 E2M1 values) plus their 2 E4M3 scales, and the
// 32 matching activations of token row c.  The four v_mfma_f32_16x16x32_bf16
// of a step consume these chunks; A and B walk K in the same permuted order, so
// the sum is unchanged.  Exact dequantisation: code x scale has <= 6
// significant bits, so the bf16 B operand is exact; products are exact in fp32.
#include <math.h>

#include "moe_common.hpp"

namespace moe {
namespace {

constexpr int kSplitK = 4;  // wavefronts per workgroup, each a quarter of K

struct FfnArgs {
  FfnGeom g;
  const uint16_t* x;
  const int32_t* perm;
  const int4* tiles;
  const int32_t* n_tiles;
  uint16_t* h;
  uint16_t* y;
  int32_t T, H, I, E, k;
};

__device__ inline const uint16_t* row_input(const FfnArgs& a, int g, int p, bool routed_x) {
  // gate/up read token rows of x; down reads rows of h
  if (!routed_x) return a.h + (int64_t)p * a.I;
  const int t = (g < a.E) ? a.perm[p] / a.k : p - a.T * a.k;
  return a.x + (int64_t)t * a.H;
}

// One 128-value K step for NMAT weight matrices sharing the A operand.
template <int NMAT>
__device__ inline void kstep(const uint16_t* arow, const uint8_t* const* codes, const uint8_t* const* scales, int ch,
                             bool valid, f32x4* acc) {
  uint4 w[NMAT];
  uint32_t sc[NMAT];
  uint4 xa[4];
#pragma unroll
  for (int mtx = 0; mtx < NMAT; mtx++) {
    w[mtx] = make_uint4(0, 0, 0, 0);
    sc[mtx] = 0;
  }
#pragma unroll
  for (int i = 0; i < 4; i++) xa[i] = make_uint4(0, 0, 0, 0);
  if (valid) {
#pragma unroll
    for (int mtx = 0; mtx < NMAT; mtx++) {
      w[mtx] = *reinterpret_cast<const uint4*>(codes[mtx] + (int64_t)ch * 16);
      sc[mtx] = *reinterpret_cast<const uint16_t*>(scales[mtx] + (int64_t)ch * 2);
    }
    if (arow) {
      const uint4* xp = reinterpret_cast<const uint4*>(arow + (int64_t)ch * 32);
#pragma unroll
      for (int i = 0; i < 4; i++) xa[i] = xp[i];
    }
  }
#pragma unroll
  for (int mtx = 0; mtx < NMAT; mtx++) {
    const float s0 = e4m3_to_f32<0>(sc[mtx]);
    const float s1 = e4m3_to_f32<1>(sc[mtx]);
    acc[mtx] = mfma16x16x32(as_bf16x8(xa[0]), dequant8(w[mtx].x, s0), acc[mtx]);
    acc[mtx] = mfma16x16x32(as_bf16x8(xa[1]), dequant8(w[mtx].y, s0), acc[mtx]);
    acc[mtx] = mfma16x16x32(as_bf16x8(xa[2]), dequant8(w[mtx].z, s1), acc[mtx]);
    acc[mtx] = mfma16x16x32(as_bf16x8(xa[3]), dequant8(w[mtx].w, s1), acc[mtx]);
  }
}

// GATEUP: matrices gate and up over K = H, output h (I units).
// !GATEUP: matrix down over K = I, output y (H units).
template <bool GATEUP>
__global__ __launch_bounds__(256) void k_ffn_tile(FfnArgs a) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  const int tile = blockIdx.x;
  if (tile >= *a.n_tiles) return;
  const int4 td = a.tiles[tile];
  const int g = td.x, p0 = td.y, n = td.z, slot = td.w;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, q = lane >> 4;
  const int K = GATEUP ? a.H : a.I;
  const int units = GATEUP ? a.I : a.H;
  const int unit = blockIdx.y * 16 + c;
  uint16_t* out = GATEUP ? a.h : a.y;

  if (slot < 0 || slot >= a.g.n_slots) {  // not resident: zero rows (flagged by the grouping)
    if (wave == 0) {
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = 4 * q + r;
        if (m < n) out[(int64_t)(p0 + m) * units + unit] = 0;
      }
    }
    return;
  }
  const uint8_t* blob = a.g.pool + (uint64_t)slot * a.g.slot_stride;
  const uint8_t* codes[NMAT];
  const uint8_t* scales[NMAT];
#pragma unroll
  for (int mtx = 0; mtx < NMAT; mtx++) {
    const int m = GATEUP ? mtx : 2;
    codes[mtx] = blob + a.g.off_codes[m] + (int64_t)unit * (K / 2);
    scales[mtx] = blob + a.g.off_scales[m] + (int64_t)unit * (K / 16);
  }
  const uint16_t* arow = (c < n) ? row_input(a, g, p0 + c, GATEUP) : nullptr;

  f32x4 acc[NMAT];
#pragma unroll
  for (int mtx = 0; mtx < NMAT; mtx++) acc[mtx] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nc = K / 32;
  const int wc = (nc + kSplitK - 1) / kSplitK;
  const int c0 = wave * wc, c1 = min(nc, c0 + wc);
  for (int ch0 = c0; ch0 < c1; ch0 += 4) {
    const int ch = ch0 + q;
    kstep<NMAT>(arow, codes, scales, ch, ch < c1, acc);
  }

  __shared__ f32x4 red[kSplitK][NMAT][64];
#pragma unroll
  for (int mtx = 0; mtx < NMAT; mtx++) red[wave][mtx][lane] = acc[mtx];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mtx = 0; mtx < NMAT; mtx++) {
    f32x4 s = red[0][mtx][lane];
#pragma unroll
    for (int w = 1; w < kSplitK; w++) s += red[w][mtx][lane];
    acc[mtx] = s;
  }
  const float* glob = reinterpret_cast<const float*>(blob + a.g.off_globals);
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int m = 4 * q + r;  // D[m][c] of the 16x16 tile
    if (m >= n) continue;
    float v;
    if (GATEUP) {
      const float gv = glob[0] * acc[0][r];
      const float uv = glob[1] * acc[1][r];
      v = gv / (1.0f + expf(-gv)) * uv;
    } else {
      v = glob[2] * acc[0][r];
    }
    out[(int64_t)(p0 + m) * units + unit] = f32_to_bf16_rne(v);
  }
}

}  // namespace

hipError_t launch_ffn(const moe_dims& d, const uint16_t* x, const FfnGeom& g, const int32_t* perm, uint16_t* h,
                      uint16_t* y_rows, int32_t* dev_status, void* ws, hipStream_t s) {
  (void)dev_status;
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  FfnArgs a;
  a.g = g;
  a.x = x;
  a.perm = perm;
  a.tiles = reinterpret_cast<const int4*>(base + wl.off_tiles);
  a.n_tiles = reinterpret_cast<const int32_t*>(base + wl.off_meta);
  a.h = h;
  a.y = y_rows;
  a.T = d.T;
  a.H = d.H;
  a.I = d.I;
  a.E = d.E;
  a.k = d.k;
  hipLaunchKernelGGL(k_ffn_tile<true>, dim3((unsigned)wl.max_tiles, (unsigned)(d.I / 16)), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_ffn_tile<false>, dim3((unsigned)wl.max_tiles, (unsigned)(d.H / 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
