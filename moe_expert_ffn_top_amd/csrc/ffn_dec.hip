// S4 for decode-sized groups: persistent bf16-MFMA expert FFN.
//
// [Strata] "路由以后，专家怎样分工？": in decode a window holds a few tokens, so a
// group has few rows and the expert's weight bytes dominate; the time goes
// into reading them ([FreeToken] 2.2: decode is a stream of small, latency-
// sensitive expert reads).  This kernel is built for that regime:
//  - A persistent grid (sized to stay resident) walks a list of work units
//    (tile of <= 16 rows, block of output units, K round); each workgroup
//    requests the weights of its next unit before it computes the current one,
//    so the dependent-load chains of a unit (tile descriptor -> slot ->
//    weights) overlap the previous unit's math.
//  - A operand: bf16 rows of x (gathered through the tile's token table) or of
//    h, read exactly, through buffer loads: lanes of the MFMA rows beyond the
//    tile's n rows address past the end of the buffer and get zeros without
//    any memory traffic.
//  - B operand: lane (c = lane % 16, q = lane / 16) owns output unit c of each
//    of its unit blocks and, in a K round of S steps, the S consecutive
//    32-value chunks S q .. S q + S - 1 of the wavefront's share.  The blob
//    stores a chunk of a 16-row block as 256 contiguous bytes, so one step's
//    16-byte code loads cover four such runs.  When the share is whole
//    512-value groups (S = 4), a lane's 8 scale bytes of a round are adjacent
//    in the blob and come in one load per unit; otherwise each step loads the
//    dword holding its chunk's two scales.  Codes are decoded with
//    v_cvt_scalef32_pk_f32_fp4 and multiplied by the scale in fp32 (exact:
//    <= 6 significant bits), then packed to bf16 (exact).
//    v_mfma_f32_16x16x32_bf16 sums exact products in fp32.
//  - A wavefront runs U unit blocks (and, for gate/up, both matrices) against
//    the same A registers, so one unit carries U times the weight bytes for
//    the registers of one A fragment.
//  - SPLITK wavefronts of a unit block split K; partials meet in LDS.  A
//    wavefront's share of K is covered in K rounds of S steps.
//  - MX blobs ([FreeToken] 2.1: natively MXFP4 experts, read as OCP MX): one
//    E8M0 scale 2^(b - 127) per 32-value chunk, the four of a 128-value group
//    in one dword per row, and no global scales.  The A rows are then the
//    bf16 values of MXFP8(x) and MXFP8(h) (exact in bf16), so the products
//    stay exact and the sums fp32, as on the NVFP4 path.
#include <hip/hip_ext.h>
#include <math.h>

#include "moe_common.hpp"

// resident workgroups per CU for the persistent grid, per stage
#ifndef MOE_DEC_WGS_GU
#define MOE_DEC_WGS_GU 2
#endif
#ifndef MOE_DEC_WGS_DN
#define MOE_DEC_WGS_DN 2
#endif
// unit blocks per wavefront and steps per K round, per stage
#ifndef MOE_DEC_U_GU
#define MOE_DEC_U_GU 1
#endif
#ifndef MOE_DEC_MAXS_GU
#define MOE_DEC_MAXS_GU 4
#endif
#ifndef MOE_DEC_U_DN
#define MOE_DEC_U_DN 2
#endif
#ifndef MOE_DEC_MAXS_DN
#define MOE_DEC_MAXS_DN 4
#endif

namespace moe {
namespace {

#ifdef MOE_DEC_TIMING
// Tuning builds only: per-wavefront wall-clock stamps (start, first unit's
// descriptor ready, first weights arrived, end of units 1..4, end).
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

// Blob offsets and the slot stride fit 32 bits (a blob is at most 27 * 16384^2
// / 16 bytes); narrow fields keep the kernel's scalar registers free.
struct DecArgs {
  uint32_t slot_stride;
  int32_t n_slots;
  uint32_t off_codes[3];
  uint32_t off_scales[3];
  uint32_t off_globals;
  int32_t H, I;
  int32_t n_ug;       // items (unit-block groups) per tile
  int32_t n_kr;       // K rounds per item
  int32_t max_tiles;  // entries of the tile list
  int32_t a_bytes;    // bytes of x (T * H * 2), the gate/up A buffer
};

// One lane's loads for one 128-value K step of NS weight streams.
template <int NS>
struct Step {
  uint4 w[NS];
  uint32_t sc[NS];
};

// Per-wavefront view of one item.  Stream m is matrix m % NMAT of unit block
// m / NMAT.  codes[m]: this lane's row of chunk 0 of the unit block; scales[m]:
// the block's scales (plus, with whole groups, this lane's 8 bytes of group 0).
template <int NS>
struct Item {
  const uint8_t* codes[NS];
  const uint8_t* scales[NS];
  __amdgpu_buffer_rsrc_t arsrc;  // A rows as a buffer
  uint32_t aoff;                 // this lane's row start in arsrc (bytes; past the end for padding rows)
  float g0, g1;                  // fp32 global scales (gate, up) or (down, -)
  int p0, n, unit;               // first row, rows, this lane's unit in its first unit block
  bool live;                     // the item exists
  bool resident;                 // it exists and its slot is inside the pool
};

// The raw descriptor of an item: its tile entry (the same 16 bytes in every
// lane) and, for gate/up, this lane's token from the tile's token table.  Both
// are vector loads issued two work units ahead of their use: the in-order wait
// for them then only covers loads that are a whole unit old.  The tile index
// is clamped, so the load does not wait for the item count; the item is masked
// when it is derived.
struct Desc {
  int4 td;
  int tok;
  int item;
};

template <bool GATEUP>
__device__ inline Desc load_desc(const DecArgs& a, int item, int c, const int4* __restrict__ tiles,
                                 const int32_t* __restrict__ tile_tok) {
  Desc d;
  const int tile = min(item / a.n_ug, a.max_tiles - 1);
  d.td = tiles[tile];
  d.tok = GATEUP ? tile_tok[(int64_t)tile * 16 + c] : 0;
  d.item = item;
  return d;
}

template <bool GATEUP, int U, bool FS, bool MX>
__device__ inline Item<(GATEUP ? 2 : 1) * U> make_item(const DecArgs& a, const Desc& d, int n_items, int wub, int c,
                                                        const uint8_t* __restrict__ pool,
                                                        const uint16_t* __restrict__ ain) {
  constexpr int NMAT = GATEUP ? 2 : 1, NS = NMAT * U;
  Item<NS> it;
  const int K = GATEUP ? a.H : a.I;
  const int item = d.item;
  const int tile_u = item / a.n_ug, ug = item - tile_u * a.n_ug;
  // the tile entry is the same in every lane
  const int p0 = __builtin_amdgcn_readfirstlane(d.td.y);
  const int tn = __builtin_amdgcn_readfirstlane(d.td.z);
  const int slot = __builtin_amdgcn_readfirstlane(d.td.w);
  const int ubw = (GATEUP ? a.I : a.H) / 16 / a.n_ug;  // unit blocks per item
  const int q = (threadIdx.x & 63) >> 4;
  it.live = item < n_items;
  it.p0 = p0;
  it.n = it.live ? tn : 0;
  it.unit = (ug * ubw + wub) * 16 + c;
  if (GATEUP) {
    it.arsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ain), (short)0, a.a_bytes, 0x00020000);
    it.aoff = c < it.n ? (uint32_t)d.tok * (uint32_t)a.H * 2u : 0x80000000u;
  } else {
    // the buffer holds exactly the tile's rows, so lanes c >= n fall outside it
    it.arsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ain + (it.live ? (int64_t)p0 * a.I : 0)),
                                                 (short)0, it.n * a.I * 2, 0x00020000);
    it.aoff = (uint32_t)c * (uint32_t)a.I * 2u;
  }
  it.resident = it.live && slot >= 0 && slot < a.n_slots;
  const uint8_t* blob = pool + (it.resident ? (uint64_t)slot * (uint64_t)a.slot_stride : 0);
#pragma unroll
  for (int m = 0; m < NS; m++) {
    const int mi = GATEUP ? (m % NMAT) : 2;
    const int unit = it.unit + (m / NMAT) * 16;
    // the lane's row in its 16-row block (blob tiling in moe_common.hpp)
    const int64_t ub = unit >> 4;
    it.codes[m] = it.resident ? blob + a.off_codes[mi] + ub * (8 * K) + c * 16 : pool;
    if (MX)  // the row's dword of group g at 64 g + 4 c of its block's K/2 bytes
      it.scales[m] = it.resident ? blob + a.off_scales[mi] + ub * (K / 2) + c * 4 : pool;
    else
      it.scales[m] = it.resident ? blob + a.off_scales[mi] + ub * K + (FS ? c * 32 + q * 8 : 0) : pool;
  }
  if (MX) {  // no globals (off_globals is the end of the blob)
    it.g0 = it.resident ? 1.f : 0.f;
    it.g1 = (GATEUP && it.resident) ? 1.f : 0.f;
  } else {
    cptr<float> glob = as_const(reinterpret_cast<const float*>(blob + a.off_globals));
    it.g0 = it.resident ? glob[GATEUP ? 0 : 2] : 0.f;
    it.g1 = (GATEUP && it.resident) ? glob[1] : 0.f;
  }
  return it;
}

// Unconditional, address-clamped weight loads (exact wait counts): invalid
// chunks are zeroed through their scale.  Without whole groups (FS false) the
// scale dword is the aligned one holding the chunk's two bytes.
template <int NS, bool FS, bool MX>
__device__ inline void load_step(Step<NS>& s, const Item<NS>& it, int ch, int nc, int c) {
#pragma unroll
  for (int m = 0; m < NS; m++) {
    s.w[m] = *reinterpret_cast<const uint4*>(it.codes[m] + (int64_t)ch * 256);
    if (MX) s.sc[m] = *reinterpret_cast<const uint32_t*>(it.scales[m] + 64 * (ch >> 2));
    else if (!FS) s.sc[m] = *reinterpret_cast<const uint32_t*>(it.scales[m] + (blob_sc_off(ch, nc, c) & ~3));
  }
}

// With whole groups: this lane's 8 scale bytes (its 4 chunks) of group grp.
template <int NS>
__device__ inline void load_sc(uint2* sc, const Item<NS>& it, int grp) {
#pragma unroll
  for (int m = 0; m < NS; m++) sc[m] = *reinterpret_cast<const uint2*>(it.scales[m] + (int64_t)grp * 512);
}

template <int NS>
__device__ inline void load_a(uint4* xa, const Item<NS>& it, int ch) {
  using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(it.arsrc, it.aoff + (uint32_t)ch * 64u + 16u * i, 0, 0);
    xa[i] = uint4{v.x, v.y, v.z, v.w};
  }
}

// sc[m]: the step's two E4M3 scales of stream m in the low 16 bits, or (MX)
// its E8M0 byte in the low 8
template <int NS, bool MX>
__device__ inline void mma_step(const Step<NS>& s, const uint4* xa, const uint32_t* sc, bool valid, f32x4* acc) {
#pragma unroll
  for (int m = 0; m < NS; m++) {
    const uint32_t sw = valid ? sc[m] : 0u;
    float s0, s1;
    if (MX) {
      // 2^(b - 127); b = 0 is the subnormal 2^-127
      const uint32_t b = sw & 0xFFu;
      s0 = s1 = valid ? __uint_as_float(b ? b << 23 : 0x00400000u) : 0.f;
    } else {
      s0 = e4m3_to_f32<0>(sw);
      s1 = e4m3_to_f32<1>(sw);
    }
    acc[m] = mfma16x16x32(as_bf16x8(xa[0]), dequant8(s.w[m].x, s0), acc[m]);
    acc[m] = mfma16x16x32(as_bf16x8(xa[1]), dequant8(s.w[m].y, s0), acc[m]);
    acc[m] = mfma16x16x32(as_bf16x8(xa[2]), dequant8(s.w[m].z, s1), acc[m]);
    acc[m] = mfma16x16x32(as_bf16x8(xa[3]), dequant8(s.w[m].w, s1), acc[m]);
  }
}

// S: 128-value steps per wavefront and K round; U unit blocks per wavefront;
// SPLITK wavefronts per unit block (4 / SPLITK unit-block groups per item);
// FS: every K round of every wavefront is one whole 512-value group (S = 4).
template <bool GATEUP, int SPLITK, int S, int U, bool FS, bool MX>
__global__ __launch_bounds__(256) void k_ffn_dec(DecArgs a, const int4* __restrict__ tiles,
                                                 const int32_t* __restrict__ tile_tok,
                                                 const int32_t* __restrict__ n_tiles,
                                                 const uint8_t* __restrict__ pool, const uint16_t* __restrict__ ain,
                                                 uint16_t* __restrict__ out) {
  constexpr int NMAT = GATEUP ? 2 : 1, NS = NMAT * U;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wub = (wave / SPLITK) * U, kpart = wave % SPLITK;  // first unit block of this wave in the item
  const int c = lane & 15, q = lane >> 4;
  const int K = GATEUP ? a.H : a.I;
  const int units = GATEUP ? a.I : a.H;
  const int n_items = *as_const(n_tiles) * a.n_ug;
  const int nkr = a.n_kr;
  const int nc = K / 32;
  const int wc = (nc + SPLITK - 1) / SPLITK;
  const int c0 = min(kpart * wc, nc - 1), c1 = min(nc, kpart * wc + wc);  // this wave's chunks [c0, c1)
  const bool kempty = kpart * wc >= nc;

  __shared__ f32x4 red[SPLITK > 1 ? 4 : 1][NS][64];
  // chunk of step s in K round r for this lane, and (FS) the round's group
#define DEC_CH(r, s) (c0 + (r) * (4 * S) + S * q + (s))
#define DEC_GRP(r) ((c0 + (r) * (4 * S)) >> 4)

  DEC_STAMP(0);
  // work units u = 0, 1, ...: item blockIdx.x + (u / nkr) * gridDim.x, K round u % nkr
  const int G = gridDim.x;
  int item = blockIdx.x, kr = 0;
  Item<NS> cur =
      make_item<GATEUP, U, FS, MX>(a, load_desc<GATEUP>(a, item, c, tiles, tile_tok), n_items, wub, c, pool, ain);
  if (!cur.live) return;
  // descriptor of unit 1
  Desc dn = load_desc<GATEUP>(a, nkr > 1 ? item : item + G, c, tiles, tile_tok);
  int kr2 = nkr > 2 ? 2 : (nkr == 2 ? 0 : 0);   // K round of unit 2
  int item2 = nkr > 2 ? item : (nkr == 2 ? item + G : item + 2 * G);
  DEC_STAMP(1);
#ifdef MOE_DEC_TIMING
  int n_done = 0;
#endif
  // A fragments of every step of the current unit stay in registers.  Once
  // step s is computed, its registers (weights and A) are refilled with the
  // next unit's step s, so both stream one unit ahead and every wait is on
  // loads issued a whole unit earlier.
  uint4 xa[S][4];
#pragma unroll
  for (int s = 0; s < S; s++) load_a(xa[s], cur, min(DEC_CH(0, s), c1 - 1));
  Step<NS> fb[S];
  uint2 scn[NS];  // FS: the scales of the next unit to compute
  if (FS) load_sc<NS>(scn, cur, DEC_GRP(0));
#pragma unroll
  for (int s = 0; s < S; s++) load_step<NS, FS, MX>(fb[s], cur, min(DEC_CH(0, s), c1 - 1), nc, c);
  f32x4 acc[NS];

  while (cur.live) {
    const bool last_round = kr + 1 == nkr;
    const int nkr_next = last_round ? 0 : kr + 1;
    // the next unit (derived from the descriptor fetched a unit ago; the same
    // item again when it is a further K round), then the descriptor of the
    // unit after it
    const Item<NS> nxt = make_item<GATEUP, U, FS, MX>(a, dn, n_items, wub, c, pool, ain);
    __builtin_amdgcn_sched_barrier(0);
    dn = load_desc<GATEUP>(a, item2, c, tiles, tile_tok);
    kr2 = kr2 + 1 == nkr ? 0 : kr2 + 1;
    item2 = kr2 == 0 ? item2 + G : item2;
    __builtin_amdgcn_sched_barrier(0);
    if (kr == 0) {
#pragma unroll
      for (int m = 0; m < NS; m++) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // (FS) this unit's scales; scn is refilled with the next unit's at step 0
    uint2 scc[NS];
#pragma unroll
    for (int m = 0; m < NS; m++) scc[m] = scn[m];
#pragma unroll
    for (int s = 0; s < S; s++) {
      const int chr = DEC_CH(kr, s);
      const int chc = min(chr, c1 - 1);
      uint32_t sw[NS];
#pragma unroll
      for (int m = 0; m < NS; m++)
        sw[m] = MX   ? (fb[s].sc[m] >> (8 * (chc & 3)))
                : FS ? ((s < 2 ? scc[m].x : scc[m].y) >> (16 * (s & 1)))
                     : (fb[s].sc[m] >> (16 * ((blob_sc_off(chc, nc, c) >> 1) & 1)));
      mma_step<NS, MX>(fb[s], xa[s], sw, !kempty && chr < c1 && cur.resident, acc);
#ifdef MOE_DEC_TIMING
      if (s == 0 && n_done == 0) {
        __builtin_amdgcn_sched_barrier(0);
        DEC_STAMP(2);
      }
#endif
      // this step's registers now carry the next unit's step s
      const int chn = min(DEC_CH(nkr_next, s), c1 - 1);
      load_step<NS, FS, MX>(fb[s], nxt, chn, nc, c);
      if (FS && s == 0) load_sc<NS>(scn, nxt, DEC_GRP(nkr_next));
      load_a(xa[s], nxt, chn);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (last_round) {
      // split-K partials meet in LDS; kpart 0 finishes the unit blocks
      if (SPLITK > 1) {
#pragma unroll
        for (int m = 0; m < NS; m++) red[wave][m][lane] = acc[m];
        __syncthreads();
        if (kpart == 0) {
#pragma unroll
          for (int m = 0; m < NS; m++) {
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
        for (int u = 0; u < U; u++) {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int m = 4 * q + r;  // D[m][c]
            if (m >= cur.n) continue;
            float v;
            if (GATEUP) {
              const float gv = g0 * acc[u * NMAT][r];
              const float uv = g1 * acc[u * NMAT + NMAT - 1][r];
              v = gv / (1.0f + expf(-gv)) * uv;
            } else {
              v = g0 * acc[u][r];
            }
            out[(int64_t)(cur.p0 + m) * units + cur.unit + 16 * u] = f32_to_bf16_rne(v);
          }
        }
      }
#ifdef MOE_DEC_TIMING
      n_done++;
      if (n_done <= 4) DEC_STAMP(2 + n_done);
#endif
    }
    item = last_round ? item + G : item;
    kr = nkr_next;
    cur = nxt;
  }
  DEC_STAMP(7);
#undef DEC_CH
#undef DEC_GRP
}

struct DecPtrs {
  const int4* tiles;
  const int32_t* tile_tok;
  const int32_t* n_tiles;
  const uint8_t* pool;
  const uint16_t* ain;
  uint16_t* out;
};

// ev0 / ev1: when either is set, the launch goes through hipExtLaunchKernelGGL
// and the device records them at the kernel's start and end.
struct DecLaunch {
  int grid;
  hipStream_t st;
  hipEvent_t ev0, ev1;
};

template <bool GATEUP, int SK, int S, int U, bool FS, bool MX>
hipError_t launch_k(const DecArgs& a, const DecPtrs& p, const DecLaunch& l) {
  if (l.ev0 || l.ev1)
    hipExtLaunchKernelGGL((k_ffn_dec<GATEUP, SK, S, U, FS, MX>), dim3(l.grid), dim3(256), 0, l.st, l.ev0, l.ev1, 0,
                          a, p.tiles, p.tile_tok, p.n_tiles, p.pool, p.ain, p.out);
  else
    hipLaunchKernelGGL((k_ffn_dec<GATEUP, SK, S, U, FS, MX>), dim3(l.grid), dim3(256), 0, l.st, a, p.tiles,
                       p.tile_tok, p.n_tiles, p.pool, p.ain, p.out);
  return hipGetLastError();
}

// S = 4 with every wavefront's share of K made of whole 512-value groups
// (K a multiple of 512 SK) takes the per-unit scale loads
template <bool GATEUP, int SK, int U, bool MX>
hipError_t launch_s(const DecArgs& a, const DecPtrs& p, int S, const DecLaunch& l) {
  if (S <= 1) return launch_k<GATEUP, SK, 1, U, false, MX>(a, p, l);
  if (S <= 2) return launch_k<GATEUP, SK, 2, U, false, MX>(a, p, l);
  constexpr int S4 = (GATEUP ? MOE_DEC_MAXS_GU : MOE_DEC_MAXS_DN) >= 4 ? 4 : 2;
  const int K = GATEUP ? a.H : a.I;
  if (!MX && S4 == 4 && K % (512 * SK) == 0) return launch_k<GATEUP, SK, S4, U, S4 == 4, MX>(a, p, l);
  return launch_k<GATEUP, SK, S4, U, false, MX>(a, p, l);
}

template <bool GATEUP, bool MX>
hipError_t launch_su(const DecArgs& a, const DecPtrs& p, int sk, int S, int U, const DecLaunch& l) {
  if (sk == 4) return U == 2 ? launch_s<GATEUP, 4, 2, MX>(a, p, S, l) : launch_s<GATEUP, 4, 1, MX>(a, p, S, l);
  return U == 2 ? launch_s<GATEUP, 1, 2, MX>(a, p, S, l) : launch_s<GATEUP, 1, 1, MX>(a, p, S, l);
}

}  // namespace

// Decode-path FFN: both stages, persistent grids of (CUs x MOE_DEC_WGS_GU or
// MOE_DEC_WGS_DN) workgroups (fewer when there is less work than that).
hipError_t launch_ffn_dec(const moe_dims& d, const uint16_t* x, const FfnGeom& g, const int32_t* perm, uint16_t* h,
                          uint16_t* y_rows, void* ws, int n_cu, int stages, hipEvent_t ev_start, hipEvent_t ev_stop,
                          hipStream_t s, bool mx, const uint16_t* down_in) {
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
  a.max_tiles = (int32_t)wl.max_tiles;
  a.a_bytes = (int32_t)((int64_t)d.T * d.H * 2);
  DecPtrs ptrs;
  ptrs.tiles = reinterpret_cast<const int4*>(base + wl.off_tiles);
  ptrs.tile_tok = reinterpret_cast<const int32_t*>(base + wl.off_tile_tok);
  ptrs.n_tiles = reinterpret_cast<const int32_t*>(base + wl.off_meta);
  ptrs.pool = g.pool;
  for (int stage = 0; stage < 2; stage++) {
    if (!((stages >> stage) & 1)) continue;
    const bool gu = stage == 0;
    const int64_t cap = (int64_t)n_cu * (gu ? MOE_DEC_WGS_GU : MOE_DEC_WGS_DN);
    const int K = gu ? d.H : d.I, units = gu ? d.I : d.H;
    const int ublocks = units / 16;
    const int steps = (K + 127) / 128;
    // split K four ways when a unit block has more than 4 steps, else give
    // each wavefront its own unit blocks; steps beyond MOE_DEC_MAXS per
    // wavefront run as further K rounds
    const int maxs = gu ? MOE_DEC_MAXS_GU : MOE_DEC_MAXS_DN;
    int sk = steps > 4 ? 4 : 1;
    int U = (gu ? MOE_DEC_U_GU : MOE_DEC_U_DN) > 1 ? 2 : 1;
    if (ublocks % ((4 / sk) * U) != 0) U = 1;
    if (ublocks % ((4 / sk) * U) != 0) sk = 4;  // one unit block per item, K split four ways
    const int wsteps = (steps + sk - 1) / sk;
    const int S = wsteps <= 1 ? 1 : (wsteps <= 2 || maxs <= 2) ? 2 : 4;
    a.n_kr = (wsteps + S - 1) / S;
    a.n_ug = ublocks / ((4 / sk) * U);
    const int64_t items = (int64_t)wl.max_tiles * a.n_ug;
    const int grid = (int)(items < cap ? items : cap);
    ptrs.ain = gu ? x : (down_in ? down_in : h);
    ptrs.out = gu ? h : y_rows;
    // the start event goes with the first stage launched, the stop event with the last
    const bool first = gu || !(stages & 1), last = !gu || !(stages & 2);
    const DecLaunch l{grid, s, first ? ev_start : nullptr, last ? ev_stop : nullptr};
    const hipError_t e = mx ? (gu ? launch_su<true, true>(a, ptrs, sk, S, U, l) : launch_su<false, true>(a, ptrs, sk, S, U, l))
                            : (gu ? launch_su<true, false>(a, ptrs, sk, S, U, l)
                                  : launch_su<false, false>(a, ptrs, sk, S, U, l));
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
