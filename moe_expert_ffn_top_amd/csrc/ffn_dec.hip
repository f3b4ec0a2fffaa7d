// S4 for decode-sized groups: persistent bf16-MFMA expert FFN.
//
// [Strata] "路由以后，专家怎样分工？": in decode a window holds a few tokens, so a
// group has few rows and the expert's weight bytes dominate; the time goes
// into reading them ([FreeToken] 2.2: decode is a stream of small, latency-
// sensitive expert reads).  This kernel is built for that regime:
//  - A persistent grid (sized to stay resident) walks a list of work items
//    (tile of <= 16 rows, block of output units); each workgroup requests the
//    weights of its next item before it computes the current one, so the
//    dependent-load chains of an item (tile descriptor -> slot -> weights)
//    overlap the previous item's math.
//  - A operand: bf16 rows read straight from x (through perm) or h, exact.
//  - B operand: lane (c = lane % 16, q = lane / 16) owns output unit c and per
//    128-value K step loads 16 code bytes (32 E2M1 values, chunk q) and their
//    two E4M3 scales; codes are decoded with v_cvt_scalef32_pk_f32_fp4 and
//    multiplied by the scale in fp32 (exact: <= 6 significant bits), then
//    packed to bf16 (exact).  v_mfma_f32_16x16x32_bf16 sums exact products in
//    fp32.
//  - SPLITK wavefronts of a unit block split K; partials meet in LDS.
// MFMA rows beyond a tile's n read a real row and their outputs are discarded.
#include <math.h>

#include "moe_common.hpp"

namespace moe {
namespace {

// Data that no kernel of this launch writes (tile descriptors, token tables,
// the weight pool) is read through the constant address space: a load from it
// at a wavefront-uniform address always becomes a scalar load, which is counted
// apart from the vector loads in flight.
template <typename T>
using cptr = const __attribute__((address_space(4))) T*;
using i32x4 = int __attribute__((ext_vector_type(4)));

template <typename T>
__device__ inline cptr<T> as_const(const T* p) {
  return (cptr<T>)p;
}

#ifdef MOE_DEC_TIMING
// Tuning builds only: per-wavefront wall-clock stamps (start, first item's
// descriptor ready, first weights arrived, end of items 1..4, end).
__device__ unsigned long long g_dec_times[1 << 17][8];
#define DEC_STAMP(i)                                                                              \
  do {                                                                                            \
    if ((threadIdx.x & 63) == 0) {                                                                \
      const unsigned w = (((blockIdx.x * 4u + (threadIdx.x >> 6)) & ((1u << 16) - 1)) | (GATEUP ? 0u : (1u << 16))); \
      g_dec_times[w][i] = wall_clock64();                                                         \
    }                                                                                             \
  } while (0)
#else
#define DEC_STAMP(i) \
  do {               \
  } while (0)
#endif

#ifndef MOE_DEC_CONTIG
#define MOE_DEC_CONTIG 0
#endif
#ifndef MOE_DEC_ABUF
#define MOE_DEC_ABUF 1
#endif

struct DecArgs {
  uint64_t slot_stride;
  int64_t n_slots;
  uint64_t off_codes[3];
  uint64_t off_scales[3];
  uint64_t off_globals;
  int32_t H, I;
  int32_t n_ug;     // unit-block groups (workgroup items) per tile
  int32_t a_bytes;  // bytes of x (T * H * 2), the gate/up A buffer
};

// One lane's loads for one 128-value K step.
template <int NMAT>
struct Step {
  uint4 w[NMAT];
  uint32_t sc[NMAT];
};

// Per-wavefront view of one work item.
template <int NMAT>
struct Item {
  const uint8_t* codes[NMAT];
  const uint8_t* scales[NMAT];
  int sodd[NMAT];
  const uint16_t* arow;  // this lane's input row (padding rows repeat row 0)
  __amdgpu_buffer_rsrc_t arsrc;  // A rows as a buffer: padding lanes read out of range (zeros, no traffic)
  uint32_t aoff;                 // this lane's row start in arsrc (bytes)
  float g0, g1;          // fp32 global scales (gate, up) or (down, -)
  int p0, n, unit;
  bool live;      // an item exists
  bool resident;  // its slot is inside the pool
};

// Everything here is read-only for the kernel and reached through restrict
// pointers at uniform addresses, so the compiler uses scalar loads: they are
// counted apart from the vector loads of the weights in flight, and waiting on
// them never drains the weight pipeline.
template <bool GATEUP>
__device__ inline Item<GATEUP ? 2 : 1> make_item(const DecArgs& a, int item, int n_items, int ub, int c,
                                                  const int4* __restrict__ tiles,
                                                  const int32_t* __restrict__ tile_tok,
                                                  const uint8_t* __restrict__ pool,
                                                  const uint16_t* __restrict__ ain) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  Item<NMAT> it;
  const int K = GATEUP ? a.H : a.I;
  it.live = false;
  it.resident = false;
  it.arow = ain;
  it.arsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ain), (short)0, 0, 0x00020000);
  it.aoff = 0x80000000u;
  it.g0 = it.g1 = 0.f;
  it.p0 = it.n = it.unit = 0;
#pragma unroll
  for (int m = 0; m < NMAT; m++) {
    it.codes[m] = pool;
    it.scales[m] = pool;
    it.sodd[m] = 0;
  }
  if (item >= n_items) return it;
  const int tile = item / a.n_ug, ug = item - tile * a.n_ug;
  const i32x4 td = as_const(reinterpret_cast<const i32x4*>(tiles))[tile];
  const int ubw = (GATEUP ? a.I : a.H) / 16 / a.n_ug;  // unit blocks per item
  it.live = true;
  it.p0 = td.y;
  it.n = td.z;
  it.unit = (ug * ubw + ub) * 16 + c;
  // this lane's input row; MFMA rows beyond n repeat row 0 (outputs discarded)
  if (GATEUP) {
    // one 64-byte scalar load of the tile's 16 tokens, then a per-lane pick
    cptr<i32x4> tt = as_const(reinterpret_cast<const i32x4*>(tile_tok + (int64_t)tile * 16));
    const i32x4 q0 = tt[0], q1 = tt[1], q2 = tt[2], q3 = tt[3];
    const int tok[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                         q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
    // the chain starts from a constant so that no select has two loads as
    // operands (the code generator would fold that into a per-lane load)
    int t = 0;
#pragma unroll
    for (int j = 0; j < 16; j++) t = (c == j) ? tok[j] : t;
    it.arow = ain + (int64_t)t * a.H;
    it.arsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ain), (short)0, a.a_bytes, 0x00020000);
    it.aoff = c < it.n ? (uint32_t)t * (uint32_t)a.H * 2u : 0x80000000u;
  } else {
    it.arow = ain + (int64_t)(it.p0 + min(c, it.n - 1)) * a.I;
    // the buffer holds exactly the tile's rows, so lanes c >= n fall outside it
    it.arsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ain + (int64_t)it.p0 * a.I), (short)0,
                                                 it.n * a.I * 2, 0x00020000);
    it.aoff = (uint32_t)c * (uint32_t)a.I * 2u;
  }
  it.resident = td.w >= 0 && td.w < a.n_slots;
  if (!it.resident) return it;
  const uint8_t* blob = pool + (uint64_t)td.w * a.slot_stride;
#pragma unroll
  for (int m = 0; m < NMAT; m++) {
    const int mi = GATEUP ? m : 2;
    it.codes[m] = blob + a.off_codes[mi] + (int64_t)it.unit * (K / 2);
    it.scales[m] = blob + a.off_scales[mi] + (int64_t)it.unit * (K / 16);
    it.sodd[m] = (int)((reinterpret_cast<uintptr_t>(it.scales[m]) >> 1) & 1);
  }
  cptr<float> glob = as_const(reinterpret_cast<const float*>(blob + a.off_globals));
  it.g0 = glob[GATEUP ? 0 : 2];
  it.g1 = GATEUP ? glob[1] : 0.f;
  return it;
}

// Unconditional, address-clamped weight loads (exact wait counts): see the
// header of ffn.hip.  The scale dword is the aligned one holding the chunk's
// two bytes.
template <int NMAT>
__device__ inline void load_step(Step<NMAT>& s, const Item<NMAT>& it, int ch) {
#pragma unroll
  for (int m = 0; m < NMAT; m++) {
    s.w[m] = *reinterpret_cast<const uint4*>(it.codes[m] + (int64_t)ch * 16);
    const int64_t off = (int64_t)ch * 2 - 2 * ((it.sodd[m] + ch) & 1);
    s.sc[m] = *reinterpret_cast<const uint32_t*>(it.scales[m] + off);
  }
}

template <int NMAT>
__device__ inline void load_a(uint4* xa, const Item<NMAT>& it, int ch) {
#if MOE_DEC_ABUF
  using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(it.arsrc, it.aoff + (uint32_t)ch * 64u + 16u * i, 0, 0);
    xa[i] = uint4{v.x, v.y, v.z, v.w};
  }
#else
  const uint4* p = reinterpret_cast<const uint4*>(it.arow + (int64_t)ch * 32);
#pragma unroll
  for (int i = 0; i < 4; i++) xa[i] = p[i];
#endif
}

template <int NMAT>
__device__ inline void mma_step(const Step<NMAT>& s, const uint4* xa, const Item<NMAT>& it, int ch, bool valid,
                                f32x4* acc) {
#pragma unroll
  for (int m = 0; m < NMAT; m++) {
    const uint32_t sw = valid ? (s.sc[m] >> (16 * ((it.sodd[m] + ch) & 1))) : 0u;
    const float s0 = e4m3_to_f32<0>(sw), s1 = e4m3_to_f32<1>(sw);
    acc[m] = mfma16x16x32(as_bf16x8(xa[0]), dequant8(s.w[m].x, s0), acc[m]);
    acc[m] = mfma16x16x32(as_bf16x8(xa[1]), dequant8(s.w[m].y, s0), acc[m]);
    acc[m] = mfma16x16x32(as_bf16x8(xa[2]), dequant8(s.w[m].z, s1), acc[m]);
    acc[m] = mfma16x16x32(as_bf16x8(xa[3]), dequant8(s.w[m].w, s1), acc[m]);
  }
}

// S: 128-value steps per wavefront and item (<= 4).  UBW unit blocks per item;
// SPLITK * UBW == 4 wavefronts.
template <bool GATEUP, int SPLITK, int S>
__global__ __launch_bounds__(256) void k_ffn_dec(DecArgs a, const int4* __restrict__ tiles,
                                                 const int32_t* __restrict__ tile_tok,
                                                 const int32_t* __restrict__ n_tiles,
                                                 const uint8_t* __restrict__ pool, const uint16_t* __restrict__ ain,
                                                 uint16_t* __restrict__ out) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ub = wave / SPLITK, kpart = wave % SPLITK;
  const int c = lane & 15, q = lane >> 4;
  const int K = GATEUP ? a.H : a.I;
  const int units = GATEUP ? a.I : a.H;
  const int n_items = *as_const(n_tiles) * a.n_ug;
  const int nc = K / 32;
  const int wc = (nc + SPLITK - 1) / SPLITK;
  const int c0 = min(kpart * wc, nc - 1), c1 = min(nc, kpart * wc + wc);  // this wave's chunks [c0, c1)
  const bool kempty = kpart * wc >= nc;

  __shared__ f32x4 red[4][NMAT][64];
  // chunk of step s for this lane
#if MOE_DEC_CONTIG
#define DEC_CH(s) (c0 + q * S + (s))
#else
#define DEC_CH(s) (c0 + 4 * (s) + q)
#endif

  DEC_STAMP(0);
  int item = blockIdx.x;
  Item<NMAT> cur = make_item<GATEUP>(a, item, n_items, ub, c, tiles, tile_tok, pool, ain);
  if (!cur.live) return;
  DEC_STAMP(1);
#ifdef MOE_DEC_TIMING
  int n_done = 0;
#endif
  // A fragments of every step of the current item stay in registers.  Once
  // step s is computed, its registers (weights and A) are refilled with the
  // next item's step s, so both stream one item ahead and every wait is on
  // loads issued a whole item earlier.
  uint4 xa[S][4];
#pragma unroll
  for (int s = 0; s < S; s++) load_a(xa[s], cur, min(DEC_CH(s), c1 - 1));
  Step<NMAT> fb[S];
#pragma unroll
  for (int s = 0; s < S; s++) load_step<NMAT>(fb[s], cur, min(DEC_CH(s), c1 - 1));

  while (cur.live) {
    const int nitem = item + gridDim.x;
    const Item<NMAT> nxt = make_item<GATEUP>(a, nitem, n_items, ub, c, tiles, tile_tok, pool, ain);
    f32x4 acc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; m++) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S; s++) {
      const int chr = DEC_CH(s);
      const int chc = min(chr, c1 - 1);
      mma_step<NMAT>(fb[s], xa[s], cur, chc, !kempty && chr < c1 && cur.resident, acc);
#ifdef MOE_DEC_TIMING
      if (s == 0 && n_done == 0) {
        __builtin_amdgcn_sched_barrier(0);
        DEC_STAMP(2);
      }
#endif
      // this step's registers now carry the next item's step s
      load_step<NMAT>(fb[s], nxt, min(DEC_CH(s), c1 - 1));
      load_a(xa[s], nxt, min(DEC_CH(s), c1 - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    // split-K partials meet in LDS; kpart 0 finishes the unit block
    if (SPLITK > 1) {
#pragma unroll
      for (int m = 0; m < NMAT; m++) red[wave][m][lane] = acc[m];
      __syncthreads();
      if (kpart == 0) {
#pragma unroll
        for (int m = 0; m < NMAT; m++) {
          f32x4 sum = red[wave][m][lane];
#pragma unroll
          for (int w = 1; w < SPLITK; w++) sum += red[wave + w][m][lane];
          acc[m] = sum;
        }
      }
      __syncthreads();
    }
    if (kpart == 0) {
      const float g0 = cur.g0, g1 = cur.g1;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = 4 * q + r;  // D[m][c]
        if (m >= cur.n) continue;
        float v = 0.f;
        if (cur.resident) {
          if (GATEUP) {
            const float gv = g0 * acc[0][r];
            const float uv = g1 * acc[NMAT - 1][r];
            v = gv / (1.0f + expf(-gv)) * uv;
          } else {
            v = g0 * acc[0][r];
          }
        }
        out[(int64_t)(cur.p0 + m) * units + cur.unit] = f32_to_bf16_rne(v);
      }
    }
    item = nitem;
    cur = nxt;
#ifdef MOE_DEC_TIMING
    n_done++;
    if (n_done <= 4) DEC_STAMP(2 + n_done);
#endif
  }
  DEC_STAMP(7);
}

// steps per wave = ceil(K / 128 / SPLITK) <= 4 for K <= 2048 with SPLITK 4;
// larger K uses more steps through the templated S.
struct DecPtrs {
  const int4* tiles;
  const int32_t* tile_tok;
  const int32_t* n_tiles;
  const uint8_t* pool;
  const uint16_t* ain;
  uint16_t* out;
};

template <bool GATEUP, int SK>
hipError_t launch_s(const DecArgs& a, const DecPtrs& p, int K, int grid, hipStream_t st) {
  const int steps = ((K / 32 + SK - 1) / SK + 3) / 4;
  const dim3 g(grid), b(256);
#define MOE_DEC_LAUNCH(S_)                                                                                     \
  hipLaunchKernelGGL((k_ffn_dec<GATEUP, SK, S_>), g, b, 0, st, a, p.tiles, p.tile_tok, p.n_tiles, p.pool, p.ain, \
                     p.out)
  if (steps <= 1) MOE_DEC_LAUNCH(1);
  else if (steps <= 2) MOE_DEC_LAUNCH(2);
  else if (steps <= 4) MOE_DEC_LAUNCH(4);
  else MOE_DEC_LAUNCH(8);
#undef MOE_DEC_LAUNCH
  return hipGetLastError();
}

}  // namespace

#ifndef MOE_DEC_WGS_PER_CU
#define MOE_DEC_WGS_PER_CU 2
#endif

// Decode-path FFN: both stages, persistent grids of (CUs x MOE_DEC_WGS_PER_CU)
// workgroups (fewer when there is less work than that).
hipError_t launch_ffn_dec(const moe_dims& d, const uint16_t* x, const FfnGeom& g, const int32_t* perm, uint16_t* h,
                          uint16_t* y_rows, void* ws, int n_cu, hipStream_t s) {
  (void)perm;
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  DecArgs a;
  a.slot_stride = g.slot_stride;
  a.n_slots = g.n_slots;
  for (int m = 0; m < 3; m++) {
    a.off_codes[m] = g.off_codes[m];
    a.off_scales[m] = g.off_scales[m];
  }
  a.off_globals = g.off_globals;
  a.H = d.H;
  a.I = d.I;
  a.a_bytes = (int32_t)((int64_t)d.T * d.H * 2);
  DecPtrs ptrs;
  ptrs.tiles = reinterpret_cast<const int4*>(base + wl.off_tiles);
  ptrs.tile_tok = reinterpret_cast<const int32_t*>(base + wl.off_tile_tok);
  ptrs.n_tiles = reinterpret_cast<const int32_t*>(base + wl.off_meta);
  ptrs.pool = g.pool;
  const int64_t cap = (int64_t)n_cu * MOE_DEC_WGS_PER_CU;
  for (int stage = 0; stage < 2; stage++) {
    const bool gu = stage == 0;
    const int K = gu ? d.H : d.I, units = gu ? d.I : d.H;
    const int steps = (K + 127) / 128;
    // split K four ways when a unit block has more than 4 steps, else give
    // each wavefront its own unit block
    const int sk = steps > 4 ? 4 : 1;
    const int ubw = 4 / sk;
    if ((units / 16) % ubw != 0) {  // unit blocks must fill whole items
      a.n_ug = units / 16;           // one block per item, split K four ways
    } else {
      a.n_ug = units / 16 / ubw;
    }
    const int sk_used = ((units / 16) % ubw != 0) ? 4 : sk;
    const int64_t items = wl.max_tiles * a.n_ug;
    const int grid = (int)(items < cap ? items : cap);
    ptrs.ain = gu ? x : h;
    ptrs.out = gu ? h : y_rows;
    hipError_t e;
    if (gu) e = sk_used == 4 ? launch_s<true, 4>(a, ptrs, K, grid, s) : launch_s<true, 1>(a, ptrs, K, grid, s);
    else e = sk_used == 4 ? launch_s<false, 4>(a, ptrs, K, grid, s) : launch_s<false, 1>(a, ptrs, K, grid, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

#ifdef MOE_DEC_TIMING
extern "C" void* moe_debug_dec_times(void) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_dec_times)) != hipSuccess) return nullptr;
  return p;
}
#endif

}  // namespace moe
