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
// Tile kernel.  One workgroup = 4 wavefronts = one sub-tile of <= RT rows of
// one group x (16 * 4 / SPLITK) output units.
//  - A operand: the sub-tile's input rows (x rows through perm for gate/up, h
//    rows for down) are staged once into LDS as f16, each row scaled by a power
//    of two 2^-e_r chosen from its largest |value| (e_r = exponent - 14).  A
//    bf16 value has 8 significant bits and f16 has 11, so the staged values are
//    exact except below 2^-29 of the row's largest value (then f16-subnormal,
//    error < 2^-40 of that value); the output is multiplied by 2^e_r again.
//  - B operand: lane (c = lane % 16, q = lane / 16) owns output unit c; per
//    128-value K step it loads 16 code bytes (32 E2M1 values, chunk q) and the
//    2 E4M3 scales covering them.  v_cvt_scalef32_pk_f16_fp4 gives the codes
//    as exact f16, v_pk_mul_f16 multiplies by the scale: code x scale has at
//    most 6 significant bits and lies in [2^-10, 2688], so B is exact in f16.
//    The products in v_mfma_f32_16x16x32_f16 are exact in fp32.
//  - Each wavefront streams its units' weights over its share of K with a
//    software pipeline of DEPTH steps in flight; SPLITK wavefronts of a unit
//    block split K and add their partials through LDS.
// MFMA rows beyond the sub-tile read a valid row (clamped) and are discarded.
#include <math.h>

#include "moe_common.hpp"

namespace moe {
namespace {

#ifndef MOE_FFN_DEPTH
#define MOE_FFN_DEPTH 8
#endif
#ifndef MOE_FFN_LDS_BUDGET
#define MOE_FFN_LDS_BUDGET 66560
#endif
#ifndef MOE_FFN_WAVE_STEPS
#define MOE_FFN_WAVE_STEPS 4
#endif
constexpr int kWaves = 4;                 // wavefronts per workgroup
constexpr int kDepth = MOE_FFN_DEPTH;     // most 128-value K steps of weights in flight per wavefront
constexpr int kApad = 8;                  // f16 padding per staged row (spreads rows over LDS banks)

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#ifdef MOE_FFN_TIMING
// Tuning builds only: per-wavefront wall-clock stamps of the FFN phases.
__device__ unsigned long long g_ffn_times[1 << 18][5];
#define FFN_STAMP(i)                                                                           \
  do {                                                                                         \
    if ((threadIdx.x & 63) == 0) {                                                             \
      const unsigned w = ((((blockIdx.y * gridDim.x + blockIdx.x) * 4u + (threadIdx.x >> 6)) & ((1u << 17) - 1)) | (GATEUP ? 0u : (1u << 17))); \
      g_ffn_times[w][i] = wall_clock64();                                                     \
    }                                                                                          \
  } while (0)
#else
#define FFN_STAMP(i) \
  do {               \
  } while (0)
#endif

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

__device__ inline const uint16_t* row_input(const FfnArgs& a, int g, int p, bool gateup) {
  if (!gateup) return a.h + (int64_t)p * a.I;  // down reads rows of h
  const int t = (g < a.E) ? a.perm[p] / a.k : p - a.T * a.k;
  return a.x + (int64_t)t * a.H;               // gate/up read token rows of x
}

// Weights of one 128-value K step of one lane.
template <int NMAT>
struct BFrag {
  uint4 w[NMAT];
  uint32_t sc[NMAT];
};

// Unconditional loads (no branch around them, so the compiler's wait counts
// stay exact); a chunk past the end re-reads the last valid chunk and is
// zeroed at compute time through its scale.
template <int NMAT>
__device__ inline void b_load(BFrag<NMAT>& f, const uint8_t* const* codes, const uint8_t* const* scales,
                              const int* sodd, int ch) {
#pragma unroll
  for (int m = 0; m < NMAT; m++) {
    f.w[m] = *reinterpret_cast<const uint4*>(codes[m] + (int64_t)ch * 16);
    // the aligned dword holding this chunk's two scale bytes (a 16-bit value
    // carried around the loop would be re-extended at its head, stalling it).
    // The two bytes start at an even address, so they never straddle dwords;
    // the aligned-down read stays inside the blob (scale rows are followed by
    // further scale rows or the globals).
    // (offset arithmetic only: the pointer keeps its global address space)
    const int64_t off = (int64_t)ch * 2 - 2 * ((sodd[m] + ch) & 1);
    f.sc[m] = *reinterpret_cast<const uint32_t*>(scales[m] + off);
  }
}

// 8 E2M1 codes of word w times the f16 scale held in both halves of s2.
__device__ inline f16x8 dequant8_f16(uint32_t w, f16x2 s2) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// sodd[m]: bit 1 of the scale row's address, so that the chunk's two scale
// bytes are the high half of the loaded dword iff (sodd[m] + ch) is odd.
template <int NMAT>
__device__ inline void b_mma(const BFrag<NMAT>& f, const _Float16* arow, int ch, const int* sodd, bool valid,
                             f32x4* acc) {
  f16x8 a[4];
#pragma unroll
  for (int i = 0; i < 4; i++) a[i] = *reinterpret_cast<const f16x8*>(arow + 8 * i);
#pragma unroll
  for (int m = 0; m < NMAT; m++) {
    const uint32_t sw = valid ? (f.sc[m] >> (16 * ((sodd[m] + ch) & 1))) : 0u;
    const f16x2 sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);  // E4M3 -> f16, exact
    const f16x2 s0 = f16x2{sp[0], sp[0]}, s1 = f16x2{sp[1], sp[1]};
    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], dequant8_f16(f.w[m].x, s0), acc[m], 0, 0, 0);
    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], dequant8_f16(f.w[m].y, s0), acc[m], 0, 0, 0);
    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2], dequant8_f16(f.w[m].z, s1), acc[m], 0, 0, 0);
    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[3], dequant8_f16(f.w[m].w, s1), acc[m], 0, 0, 0);
  }
}

// Stage rows [0, nrows) of the sub-tile into LDS as scaled f16; rexp[r] gets e_r.
// Wavefront w copies rows w, w+4, ... and reduces each row's largest |value|
// with a fixed xor tree (no atomics: same-address LDS atomics serialise).
template <bool GATEUP>
__device__ void stage_a(const FfnArgs& a, int g, int p0, int nrows, int K, _Float16* As, int* rexp) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int pitch = K + kApad;
  uint16_t* raw = reinterpret_cast<uint16_t*>(As);
  const int cpr = K / 8;  // 16-byte chunks per row
  for (int r = wave; r < nrows; r += kWaves) {
    const uint16_t* src = row_input(a, g, p0 + r, GATEUP);
    uint32_t m = 0;
    for (int j0 = 0; j0 < cpr; j0 += 4 * 64) {  // four chunks per lane in flight
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int j = j0 + 64 * u + lane;
        v[u] = j < cpr ? *reinterpret_cast<const uint4*>(src + 8 * j) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int j = j0 + 64 * u + lane;
        if (j < cpr) *reinterpret_cast<uint4*>(raw + r * pitch + 8 * j) = v[u];
        const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int t = 0; t < 4; t++) m = max(m, max(w4[t] & 0x7FFFu, (w4[t] >> 16) & 0x7FFFu));
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (lane == 0) {  // largest |bf16| bits -> shift e_r (row of zeros: 0)
      const int be = (int)(m >> 7) & 0xFF;
      rexp[r] = be == 0 ? 0 : max(-100, min(113, be - 127 - 14));
    }
  }
  __syncthreads();
  for (int i = tid; i < nrows * cpr; i += blockDim.x) {
    const int r = i / cpr, j = i - r * cpr;
    const float sc = __uint_as_float((uint32_t)(127 - rexp[r]) << 23);  // 2^-e_r
    uint4* cell = reinterpret_cast<uint4*>(raw + r * pitch + 8 * j);
    const uint4 v = *cell;
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const f16x2 hv = f16x2{(_Float16)(bf16_bits_to_f32(u[t] & 0xFFFFu) * sc),
                             (_Float16)(bf16_bits_to_f32(u[t] >> 16) * sc)};
      o[t] = __builtin_bit_cast(uint32_t, hv);
    }
    *cell = make_uint4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();
}

// GATEUP: matrices gate and up over K = H, output h (I units).
// !GATEUP: matrix down over K = I, output y (H units).
template <bool GATEUP, int SPLITK, int RT, int DEPTH>
__global__ __launch_bounds__(256) void k_ffn_tile(FfnArgs a) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int UB = kWaves / SPLITK;  // unit blocks per workgroup
  constexpr int NSUB = 16 / RT;        // sub-tiles per tile
  const int tile = blockIdx.x / NSUB, sub = blockIdx.x % NSUB;
  FFN_STAMP(0);
  if (tile >= *a.n_tiles) return;
  const int4 td = a.tiles[tile];
  const int g = td.x, slot = td.w;
  const int p0 = td.y + sub * RT, n = min(RT, td.z - sub * RT);
  if (n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ub = wave / SPLITK, kpart = wave % SPLITK;
  const int c = lane & 15, q = lane >> 4;
  const int K = GATEUP ? a.H : a.I;
  const int units = GATEUP ? a.I : a.H;
  const int unit = (blockIdx.y * UB + ub) * 16 + c;
  uint16_t* out = GATEUP ? a.h : a.y;

  if (slot < 0 || slot >= a.g.n_slots) {  // not resident: zero rows (flagged by the grouping)
    if (kpart == 0) {
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
  int sodd[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; m++) {
    const int mi = GATEUP ? m : 2;
    codes[m] = blob + a.g.off_codes[mi] + (int64_t)unit * (K / 2);
    scales[m] = blob + a.g.off_scales[mi] + (int64_t)unit * (K / 16);
    sodd[m] = (int)((reinterpret_cast<uintptr_t>(scales[m]) >> 1) & 1);
  }
  const int nc = K / 32;  // 32-value chunks along K
  const int wc = (nc + SPLITK - 1) / SPLITK;
  int c0 = kpart * wc, c1 = min(nc, c0 + wc);
  const int nsteps = (c1 - c0 + 3) / 4;
  if (nsteps <= 0) c0 = c1 = 0;  // an empty K share still needs valid addresses

  // weights of the first DEPTH steps are requested before the A staging
  BFrag<NMAT> f[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; d++) b_load<NMAT>(f[d], codes, scales, sodd, min(c0 + 4 * d + q, c1 - 1));

  extern __shared__ __align__(16) unsigned char smem[];
  int* rexp = reinterpret_cast<int*>(smem);
  _Float16* As = reinterpret_cast<_Float16*>(smem + 64);
  FFN_STAMP(1);
  stage_a<GATEUP>(a, g, p0, n, K, As, rexp);
  FFN_STAMP(2);

  const _Float16* arow = As + min(c, n - 1) * (K + kApad);
  f32x4 acc[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; m++) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsteps; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; d++) {
      const int chr = c0 + 4 * (s0 + d) + q;  // this lane's chunk (may be past the end)
      const int chc = min(chr, c1 - 1);
      b_mma<NMAT>(f[d], arow + chc * 32, chc, sodd, chr < c1, acc);
      b_load<NMAT>(f[d], codes, scales, sodd, min(chr + 4 * DEPTH, c1 - 1));
      // keep steps in program order: the scheduler must not pull the next
      // step's math (and its wait on loads) up into this one
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  FFN_STAMP(3);
  if (SPLITK > 1) {
    f32x4* red = reinterpret_cast<f32x4*>(smem + 64 + (size_t)RT * (K + kApad) * 2);
#pragma unroll
    for (int m = 0; m < NMAT; m++) red[(wave * NMAT + m) * 64 + lane] = acc[m];
    __syncthreads();
    if (kpart != 0) return;
#pragma unroll
    for (int m = 0; m < NMAT; m++) {
      f32x4 sum = red[(wave * NMAT + m) * 64 + lane];
#pragma unroll
      for (int w = 1; w < SPLITK; w++) sum += red[((wave + w) * NMAT + m) * 64 + lane];
      acc[m] = sum;
    }
  }
  const float* glob = reinterpret_cast<const float*>(blob + a.g.off_globals);
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int m = 4 * q + r;  // D[m][c] of the 16x16 tile
    if (m >= n) continue;
    const float rs = __uint_as_float((uint32_t)(127 + rexp[m]) << 23);  // 2^e_m
    float v;
    if (GATEUP) {
      const float gv = glob[0] * (acc[0][r] * rs);
      const float uv = glob[1] * (acc[1][r] * rs);
      v = gv / (1.0f + expf(-gv)) * uv;
    } else {
      v = glob[2] * (acc[0][r] * rs);
    }
    out[(int64_t)(p0 + m) * units + unit] = f32_to_bf16_rne(v);
  }
  FFN_STAMP(4);
}

// LDS budget for the staged rows: RT rows per sub-tile, as many as fit in the
// budget (65 KiB: two workgroups share a CU).
int pick_rt(int K) {
  int rt = 16;
  while (rt > 1 && (size_t)rt * (K + kApad) * 2 > MOE_FFN_LDS_BUDGET) rt /= 2;
  return rt;
}

// K split so that a wavefront streams about 4 steps (each 2 KiB of gate+up
// codes per lane group): every weight byte of a decode layer is then
// requested in the first round, and more waves per SIMD hide latency.
int pick_splitk(int K, int units) {
  const int steps = (K + 127) / 128;
  int s = 1;
  while (s < kWaves && steps > MOE_FFN_WAVE_STEPS * s) s *= 2;
  while (s < kWaves && (units / 16) % (kWaves / s) != 0) s *= 2;
  return s;
}

template <bool GATEUP, int SK, int RT, int DEPTH>
hipError_t launch_one(const FfnArgs& a, int64_t max_tiles, int K, int units, hipStream_t s) {
  const size_t lds = 64 + (size_t)RT * (K + kApad) * 2 + (SK > 1 ? (size_t)kWaves * (GATEUP ? 2 : 1) * 64 * 16 : 0);
  const dim3 grid((unsigned)(max_tiles * (16 / RT)), (unsigned)(units / 16 / (kWaves / SK)));
  hipLaunchKernelGGL((k_ffn_tile<GATEUP, SK, RT, DEPTH>), grid, dim3(kWaves * 64), lds, s, a);
  return hipGetLastError();
}

template <bool GATEUP, int SK, int DEPTH>
hipError_t launch_rt(const FfnArgs& a, int64_t max_tiles, int K, int units, hipStream_t s) {
  switch (pick_rt(K)) {
    case 16: return launch_one<GATEUP, SK, 16, DEPTH>(a, max_tiles, K, units, s);
    case 8: return launch_one<GATEUP, SK, 8, DEPTH>(a, max_tiles, K, units, s);
    case 4: return launch_one<GATEUP, SK, 4, DEPTH>(a, max_tiles, K, units, s);
    default: return launch_one<GATEUP, SK, 2, DEPTH>(a, max_tiles, K, units, s);
  }
}

// Steps in flight: the wavefront's step count rounded up to 2, 4 or kDepth.
template <bool GATEUP, int SK>
hipError_t launch_depth(const FfnArgs& a, int64_t max_tiles, int K, int units, hipStream_t s) {
  const int steps = ((K / 32 + SK - 1) / SK + 3) / 4;
  if (steps <= 2) return launch_rt<GATEUP, SK, 2>(a, max_tiles, K, units, s);
  if (steps <= 4) return launch_rt<GATEUP, SK, 4>(a, max_tiles, K, units, s);
  return launch_rt<GATEUP, SK, kDepth>(a, max_tiles, K, units, s);
}

template <bool GATEUP>
hipError_t launch_stage(const FfnArgs& a, int64_t max_tiles, int K, int units, hipStream_t s) {
  switch (pick_splitk(K, units)) {
    case 1: return launch_depth<GATEUP, 1>(a, max_tiles, K, units, s);
    case 2: return launch_depth<GATEUP, 2>(a, max_tiles, K, units, s);
    default: return launch_depth<GATEUP, 4>(a, max_tiles, K, units, s);
  }
}

}  // namespace

#ifdef MOE_FFN_TIMING
extern "C" void* moe_debug_ffn_times(void) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_ffn_times)) != hipSuccess) return nullptr;
  return p;
}
#endif

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
  hipError_t e = launch_stage<true>(a, wl.max_tiles, d.H, d.I, s);
  if (e != hipSuccess) return e;
  return launch_stage<false>(a, wl.max_tiles, d.I, d.H, s);
}

}  // namespace moe
