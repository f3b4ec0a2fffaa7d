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
//
// Both stages in one launch (k_ffn_dec_fused; [FreeToken] 3.5: one step's
// control flow stays on the device).  The down projection of a tile needs the
// whole of its h rows, which the tile's gate/up items (other workgroups,
// possibly on other XCDs) write.  Each workgroup first issues the weight
// loads of its first down unit, which do not depend on h, then walks its
// gate/up items; at the end of that walk every wavefront that stored h rows
// waits for its stores to complete and adds one to each of its items' tile
// counters.  A down unit waits (bounded; one polling wavefront per
// workgroup) until its tile's counter is full, then reads h.  Each counter
// has a 256-byte line of its own.  Stores and loads of h go
// through the device-coherent path (sc1: written through to memory, read
// past the XCD-private caches), so no cache-wide write-back or invalidation
// is needed.  Optionally the same launch also combines (S5): the wavefront
// that completes the last down item of a column block marks it, and its
// workgroup combines that block for every token of the window once its own
// down items are done.
#include <hip/hip_ext.h>
#include <math.h>

#include <atomic>
#include <type_traits>
#include <mutex>

#include "moe_common.hpp"
#include "route_small.hpp"

// resident workgroups per CU for the persistent grid, per stage
#ifndef MOE_DEC_WGS_GU
#define MOE_DEC_WGS_GU 2
#endif
#ifndef MOE_DEC_WGS_DN
#define MOE_DEC_WGS_DN 2
#endif
// and for the fused launch
#ifndef MOE_DEC_WGS_FUSED
#define MOE_DEC_WGS_FUSED 2
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
// polls of a tile counter before a fused launch gives up on it (each poll is
// a device-coherent load plus a short sleep: about 0.1-0.2 s in all)
#ifndef MOE_DEC_SPIN_LIMIT
#define MOE_DEC_SPIN_LIMIT (1 << 18)
#endif

namespace moe {
namespace {

// cache policy of buffer loads and stores: sc1 = coherent at device scope
constexpr int kAuxPlain = 0;
constexpr int kAuxDevice = 16;

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

// Routing in the gate/up launch (moe_route_group_ffn): with logits set, every
// workgroup routes and groups the window itself (route_small.hpp) into LDS and
// walks that work list; workgroup 0 then stores every output of
// moe_route_group (the down stage and the combine read them).
struct RouteArgs {
  const float* logits;      // [T][E]; null: the work list comes from memory
  const float* w_sg;        // [H]
  const int32_t* slot_row;  // the layer's row of the slot table, E + 1 entries
  int32_t T, k, E;
  int32_t n_slots;          // the slot table's bound (status bits), as for moe_route_group
  int32_t* ids;
  float* w;
  float* sigma;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  int32_t* group_slot;
  int32_t* status;
  int32_t* meta;
  int4* tiles;
  int32_t* tile_tok;
  int32_t* sync;
  int64_t n_sync;
};
constexpr int kRouteMaxTiles = kSortF + 1;   // routed groups, then the shared group's one tile (T <= 16)

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
  int tile, ug;                  // tile and unit-block group of the item
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

// TilesP / TokP: pointers into memory, or (the routing launch) into LDS, so
// that the reads are LDS reads there and never flat ones (which the wait
// counters would have to treat as both).
using lds_int4_p = const __attribute__((address_space(3))) int4*;
using lds_int_p = const __attribute__((address_space(3))) int*;
__device__ inline int4 tile_at(const int4* __restrict__ tiles, int i) { return tiles[i]; }
__device__ inline int4 tile_at(lds_int4_p tiles, int i) {
  const lds_int_p q = (lds_int_p)(tiles + i);
  return make_int4(q[0], q[1], q[2], q[3]);
}

template <bool GATEUP, class TilesP, class TokP>
__device__ inline Desc load_desc(const DecArgs& a, int item, int c, TilesP tiles, TokP tile_tok) {
  Desc d;
  const int tile = min(item / a.n_ug, a.max_tiles - 1);
  d.td = tile_at(tiles, tile);
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
  it.tile = tile_u;
  it.ug = ug;
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

// AUX: the cache policy (sc1 for A rows that other workgroups of the launch wrote)
template <int NS, int AUX>
__device__ inline void load_a(uint4* xa, const Item<NS>& it, int ch) {
  using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(it.arsrc, it.aoff + (uint32_t)ch * 64u + 16u * i, 0, AUX);
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

// ---- synchronisation of the fused launch ------------------------------------
// The counters live in the workspace (ws_layout: sync), kSyncStride words
// apart, zeroed by every grouping kernel and by the last workgroup of every
// fused launch.  Counter i is the word sync[i * kSyncStride]:
//   0                    workgroups of the launch that have finished
//   1 + t                wavefront stores of tile t's h rows done
//   1 + max_tiles + b    wavefront stores of column block b's Y rows done
struct FusedCtx {
  int32_t* sync;
  int32_t* status;
  int32_t max_tiles;
  int32_t gu_target;  // h-row publications that complete a tile
  int32_t dn_target;  // Y-row publications that complete a column block (x n_tiles)
  int32_t spin_limit;
  // (k_layer_dec) the ready flag and the counters workgroup 0 zeroes first
  uint64_t* flag;
  int32_t n_zero;
  // combine (S5) arguments; inv_perm null: no combine in this launch
  const int32_t* inv_perm;
  const float* w;
  const float* sigma;
  uint16_t* y;
  int32_t T, k, H, cols;  // cols: output columns per down item
};

__device__ inline int32_t* counter(const FusedCtx& fc, int i) { return fc.sync + (int64_t)i * kSyncStride; }

// The calling wavefront's h or Y stores have completed (written through to
// the device-coherent level); then one lane counts them.
__device__ inline int publish(int32_t* ctr) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int old = 0;
  if ((threadIdx.x & 63) == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_amdgcn_readfirstlane(old);
}

// Wait (bounded) until *ctr >= target: wavefront 0 polls, the workgroup
// meets it at a barrier (every wavefront of the workgroup calls this).  On
// time-out MOE_DEV_SYNC_TIMEOUT is set and the workgroup goes on: its results
// are then undefined, but every wave still ends.
__device__ inline void wait_count(const int32_t* ctr, int target, const FusedCtx& fc) {
  if ((threadIdx.x >> 6) == 0) {
    int spins = 0;
    while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) <
           target) {
      if (++spins > fc.spin_limit) {
        if ((threadIdx.x & 63) == 0) atomicOr(fc.status, MOE_DEV_SYNC_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
  }
  __syncthreads();
  asm volatile("" ::: "memory");
}

// bf16 store of element idx of rows (a wavefront-uniform base holding
// `bytes` bytes) with a cache policy
template <int AUX>
__device__ inline void store_bf16(uint16_t* rows, int bytes, int idx, uint16_t v) {
  if (AUX == kAuxPlain) {
    rows[idx] = v;
  } else {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(rows, (short)0, bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b16(v, r, 2 * idx, 0, AUX);
  }
}

// S5 for the column blocks marked in mask (bit b: columns [b cols, b cols +
// cols)), for every token, by the whole workgroup, in exactly k_combine's
// arithmetic: y = bf16(sum_j w_j Y[inv(t, j)] + sigma Y_sh), fp32 fused
// multiply-adds in slot order, then the shared row.  pw / sg: inv_perm, w
// and sigma (written before the launch), staged in LDS at the launch's
// start; the Y rows (written by other workgroups of this launch) are read
// with device-coherent loads, all of a column pair's at once.
__device__ inline void combine_blocks(const uint16_t* __restrict__ yr, const FusedCtx& fc, const uint32_t* mask,
                                      const int2* pw, const float* sg) {
  const int nb = fc.H / fc.cols, nw = (nb + 31) / 32;
  bool any = false;
  for (int i = 0; i < nw; i++) any |= mask[i] != 0;
  if (!any) return;
  const int Tk = fc.T * fc.k;
  const int pairs = fc.cols / 2;
  for (int wi = 0; wi < nw; wi++) {
    uint32_t m = mask[wi];
    while (m) {
      const int b = 32 * wi + __builtin_ctz(m);
      m &= m - 1;
      for (int o = threadIdx.x; o < fc.T * pairs; o += blockDim.x) {
        const int t = o / pairs, col = b * fc.cols + 2 * (o - t * pairs);
        int p[kFusedCombineMaxK];
        float wj[kFusedCombineMaxK];
        uint32_t v[kFusedCombineMaxK];
#pragma unroll
        for (int j = 0; j < kFusedCombineMaxK; j++) {
          const int2 e = pw[t * fc.k + min(j, fc.k - 1)];
          p[j] = j < fc.k ? e.x : -1;
          wj[j] = __int_as_float(e.y);
        }
#pragma unroll
        for (int j = 0; j < kFusedCombineMaxK; j++)
          v[j] = __hip_atomic_load(reinterpret_cast<const uint32_t*>(yr + (int64_t)max(p[j], 0) * fc.H + col),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t vs =
            __hip_atomic_load(reinterpret_cast<const uint32_t*>(yr + ((int64_t)Tk + t) * fc.H + col),
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < kFusedCombineMaxK; j++) {
          if (p[j] < 0) continue;
          a0 = fmaf(wj[j], bf16_bits_to_f32(v[j] & 0xFFFFu), a0);
          a1 = fmaf(wj[j], bf16_bits_to_f32(v[j] >> 16), a1);
        }
        const float st = sg[t];
        const float b0 = fmaf(st, bf16_bits_to_f32(vs & 0xFFFFu), a0);
        const float b1 = fmaf(st, bf16_bits_to_f32(vs >> 16), a1);
        *reinterpret_cast<uint32_t*>(fc.y + (int64_t)t * fc.H + col) =
            (uint32_t)f32_to_bf16_rne(b0) | ((uint32_t)f32_to_bf16_rne(b1) << 16);
      }
    }
  }
}

// ---- one stage's walk over its work units -----------------------------------
// Geometry of the calling wavefront in a stage.
template <bool GATEUP, int SPLITK, int S, int U>
struct Geo {
  int wave, lane, wub, kpart, c, q, K, units, nc, wc, c0, c1;
  bool kempty;
  __device__ inline Geo(const DecArgs& a) {
    wave = threadIdx.x >> 6;
    lane = threadIdx.x & 63;
    wub = (wave / SPLITK) * U;  // first unit block of this wave in the item
    kpart = wave % SPLITK;
    c = lane & 15;
    q = lane >> 4;
    K = GATEUP ? a.H : a.I;
    units = GATEUP ? a.I : a.H;
    nc = K / 32;
    wc = (nc + SPLITK - 1) / SPLITK;
    c0 = min(kpart * wc, nc - 1);  // this wave's chunks [c0, c1)
    c1 = min(nc, kpart * wc + wc);
    kempty = kpart * wc >= nc;
  }
  // chunk of step s in K round r for this lane, and (FS) the round's group
  __device__ inline int ch(int r, int s) const { return c0 + r * (4 * S) + S * q + s; }
  __device__ inline int grp(int r) const { return (c0 + r * (4 * S)) >> 4; }
};

// The first unit of a stage, with its weight loads issued: a caller can issue
// them long before the stage runs (the fused launch issues its first down
// unit's before its gate/up items).
// Loads are counted in issue order (vmcnt), so a caller that starts two
// stages issues both first descriptors before either start: a start then
// waits only on loads issued before its own.
template <bool GATEUP, int SPLITK, int S, int U, bool FS, bool MX>
struct Start {
  static constexpr int NS = (GATEUP ? 2 : 1) * U;
  Item<NS> cur;
  Step<NS> fb[S];
  uint2 scn[NS];
  uint4 xa[S][4];  // A rows of the first unit (when they are loaded at the start)
  Desc dn;         // descriptor of the second unit
};

// The first unit (descriptor d0): its weights, its A rows when LOAD_A, then
// the second unit's descriptor.  stride: item step of the walk.
template <bool GATEUP, int SPLITK, int S, int U, bool FS, bool MX, bool LOAD_A, class TilesP, class TokP>
__device__ inline void stage_start(Start<GATEUP, SPLITK, S, U, FS, MX>& st, const DecArgs& a, const Desc& d0,
                                   int n_items, int stride, TilesP tiles, TokP tile_tok,
                                   const uint8_t* __restrict__ pool,
                                   const uint16_t* __restrict__ ain) {
  constexpr int NS = (GATEUP ? 2 : 1) * U;
  const Geo<GATEUP, SPLITK, S, U> g(a);
  st.cur = make_item<GATEUP, U, FS, MX>(a, d0, n_items, g.wub, g.c, pool, ain);
  if (FS) load_sc<NS>(st.scn, st.cur, g.grp(0));
#pragma unroll
  for (int s = 0; s < S; s++) load_step<NS, FS, MX>(st.fb[s], st.cur, min(g.ch(0, s), g.c1 - 1), g.nc, g.c);
  if (LOAD_A) {
#pragma unroll
    for (int s = 0; s < S; s++) load_a<NS, kAuxPlain>(st.xa[s], st.cur, min(g.ch(0, s), g.c1 - 1));
  }
  st.dn = load_desc<GATEUP>(a, a.n_kr > 1 ? d0.item : d0.item + stride, g.c, tiles, tile_tok);
}

// Policy of a stage's walk:
//   AAUX    cache policy of the A-row loads
//   OAUX    cache policy of the output stores
//   WAIT    before a unit's A rows are read, wait for its tile's h (fused down)
//   PUB     (down) after an item's stores, publish them to the column
//           block's counter; the wavefront that completes a column block
//           marks it in comb_mask (LDS) for its workgroup to combine
template <int AAUX, int OAUX, bool WAIT, bool PUB>
struct Policy {
  static constexpr int kAAux = AAUX, kOAux = OAUX;
  static constexpr bool kWait = WAIT, kPub = PUB;
};
using PlainStage = Policy<kAuxPlain, kAuxPlain, false, false>;

// Walks work units u = 0, 1, ...: item first_item + (u / nkr) * stride, K round
// u % nkr, starting from st (its weight loads already issued).
template <bool GATEUP, int SPLITK, int S, int U, bool FS, bool MX, class P, class TilesP, class TokP>
__device__ inline void stage_walk(Start<GATEUP, SPLITK, S, U, FS, MX>& st, const DecArgs& a, int stride,
                                  int n_items, TilesP tiles, TokP tile_tok,
                                  const uint8_t* __restrict__ pool, const uint16_t* __restrict__ ain,
                                  uint16_t* __restrict__ out, const FusedCtx* fc, f32x4 (*red)[(GATEUP ? 2 : 1) * U][64],
                                  uint32_t* comb_mask = nullptr) {
  constexpr int NMAT = GATEUP ? 2 : 1, NS = NMAT * U;
  const Geo<GATEUP, SPLITK, S, U> g(a);
  const int c = g.c, q = g.q, nc = g.nc, c1 = g.c1;
  const int nkr = a.n_kr;
  Item<NS> cur = st.cur;
  if (!cur.live) return;
  int item = cur.tile * a.n_ug + cur.ug, kr = 0;
  Desc dn = st.dn;  // descriptor of unit 1
  int kr2 = nkr > 2 ? 2 : 0;  // K round of unit 2
  int item2 = nkr > 2 ? item : (nkr == 2 ? item + stride : item + 2 * stride);
  // A fragments of every step of the current unit stay in registers.  Once
  // step s is computed, its registers (weights and A) are refilled with the
  // next unit's step s, so both stream one unit ahead and every wait is on
  // loads issued a whole unit earlier.  With WAIT the A rows of a unit are
  // requested only once its tile is complete: the first unit's here, every
  // next unit's at the end of the unit before it.
  uint4 (*xa)[4] = st.xa;
  if (P::kWait) {
    wait_count(counter(*fc, 1 + cur.tile), fc->gu_target, *fc);
#pragma unroll
    for (int s = 0; s < S; s++) load_a<NS, P::kAAux>(xa[s], cur, min(g.ch(0, s), c1 - 1));
  }
  Step<NS>* fb = st.fb;
  uint2 scn[NS];  // FS: the scales of the next unit to compute
#pragma unroll
  for (int m = 0; m < NS; m++) scn[m] = st.scn[m];
  f32x4 acc[NS];

  while (cur.live) {
    const bool last_round = kr + 1 == nkr;
    const int nkr_next = last_round ? 0 : kr + 1;
    // the next unit (derived from the descriptor fetched a unit ago; the same
    // item again when it is a further K round), then the descriptor of the
    // unit after it
    const Item<NS> nxt = make_item<GATEUP, U, FS, MX>(a, dn, n_items, g.wub, c, pool, ain);
    __builtin_amdgcn_sched_barrier(0);
    dn = load_desc<GATEUP>(a, item2, c, tiles, tile_tok);
    kr2 = kr2 + 1 == nkr ? 0 : kr2 + 1;
    item2 = kr2 == 0 ? item2 + stride : item2;
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
      const int chr = g.ch(kr, s);
      const int chc = min(chr, c1 - 1);
      uint32_t sw[NS];
#pragma unroll
      for (int m = 0; m < NS; m++)
        sw[m] = MX   ? (fb[s].sc[m] >> (8 * (chc & 3)))
                : FS ? ((s < 2 ? scc[m].x : scc[m].y) >> (16 * (s & 1)))
                     : (fb[s].sc[m] >> (16 * ((blob_sc_off(chc, nc, c) >> 1) & 1)));
      mma_step<NS, MX>(fb[s], xa[s], sw, !g.kempty && chr < c1 && cur.resident, acc);
      // this step's registers now carry the next unit's step s
      const int chn = min(g.ch(nkr_next, s), c1 - 1);
      load_step<NS, FS, MX>(fb[s], nxt, chn, nc, c);
      if (FS && s == 0) load_sc<NS>(scn, nxt, g.grp(nkr_next));
      if (!P::kWait) load_a<NS, P::kAAux>(xa[s], nxt, chn);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (last_round) {
      // split-K partials meet in LDS; kpart 0 finishes the unit blocks
      if (SPLITK > 1) {
#pragma unroll
        for (int m = 0; m < NS; m++) red[g.wave][m][g.lane] = acc[m];
        __syncthreads();
        if (g.kpart == 0) {
#pragma unroll
          for (int m = 0; m < NS; m++) {
            f32x4 sum = red[g.wave][m][g.lane];
#pragma unroll
            for (int w = 1; w < SPLITK; w++) sum += red[g.wave + w][m][g.lane];
            acc[m] = sum;
          }
        }
        __syncthreads();
      }
      if (g.kpart == 0) {
        const float g0 = cur.g0, g1 = cur.g1;
        uint16_t* orows = out + (int64_t)cur.p0 * g.units;  // the tile's rows
        const int obytes = cur.n * g.units * 2;
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
            store_bf16<P::kOAux>(orows, obytes, m * g.units + cur.unit + 16 * u, f32_to_bf16_rne(v));
          }
        }
        if (P::kPub) {
          // the wavefront that completes the column block combines it
          const int old = publish(counter(*fc, 1 + fc->max_tiles + cur.ug));
          const int n_tiles = n_items / a.n_ug;
          if (old == fc->dn_target * n_tiles - 1 && g.lane == 0)
            atomicOr(&comb_mask[cur.ug >> 5], 1u << (cur.ug & 31));
        }
      }
    }
    if (P::kWait && nxt.live) {
      // the next unit's A rows, once its tile is complete
      if (nxt.tile != cur.tile || last_round) wait_count(counter(*fc, 1 + nxt.tile), fc->gu_target, *fc);
#pragma unroll
      for (int s = 0; s < S; s++) load_a<NS, P::kAAux>(xa[s], nxt, min(g.ch(nkr_next, s), c1 - 1));
    }
    item = last_round ? item + stride : item;
    kr = nkr_next;
    cur = nxt;
  }
}

// One stage as its own launch (stages split, and the MX path).
// ROUTE (gate/up on NVFP4 blobs, RouteArgs r): every workgroup first routes
// and groups the window itself (T <= 16, T k <= 256, E <= 1024) into LDS, the
// same in each.  Workgroup 0 then stores the routing outputs and ends;
// workgroups 1 .. G walk the items with the work list from LDS (item i goes to
// workgroup 1 + i mod (G - 1)), so no item waits on those stores and the walk
// holds none of the output pointers.
struct RouteLds {
  SmallRouteLds<4> L;
  int4 tiles[kRouteMaxTiles];
  int32_t tok[kRouteMaxTiles * kTileRows];
  int32_t n[2];
};
struct NoRouteLds {
  int32_t unused;
};

// The arguments that a workgroup's first loads depend on lead the list (the
// routing's logits and slot row, the work list and its bounds): the library
// is built to preload leading kernel arguments into scalar registers at
// dispatch, so those loads do not wait for a load of the argument block.
template <bool GATEUP, int SPLITK, int S, int U, bool FS, bool MX, int RNPL>
__global__ __launch_bounds__(256) void k_ffn_dec(const float* __restrict__ r_logits,
                                                 const int32_t* __restrict__ r_slot_row, int32_t r_T, int32_t r_E,
                                                 int32_t r_k, const int4* __restrict__ tiles,
                                                 const int32_t* __restrict__ n_tiles, int32_t n_ug, int32_t max_tiles,
                                                 DecArgs a, const int32_t* __restrict__ tile_tok,
                                                 const uint8_t* __restrict__ pool, const uint16_t* __restrict__ ain,
                                                 uint16_t* __restrict__ out, RouteArgs r) {
  constexpr bool ROUTE = RNPL > 0;   // RNPL: logits per lane of the routing (E <= 64 RNPL)
  // the leading copies of these fields (the same values)
  a.n_ug = n_ug;
  a.max_tiles = max_tiles;
  r.logits = r_logits;
  r.slot_row = r_slot_row;
  r.T = r_T;
  r.E = r_E;
  r.k = r_k;
  static_assert(!ROUTE || (GATEUP && !MX), "routing runs in the NVFP4 gate/up launch");
  constexpr int NS = (GATEUP ? 2 : 1) * U;
  __shared__ f32x4 red[SPLITK > 1 ? 4 : 1][NS][64];
  __shared__ std::conditional_t<ROUTE, RouteLds, NoRouteLds> rl;
  int n_items, first = blockIdx.x, stride = gridDim.x;
  if constexpr (ROUTE) {
    const int wave = threadIdx.x >> 6;
    const int F = r.T * r.k;
    small_route_topk<(RNPL > 0 ? RNPL : 1), 4, false>(rl.L, r.logits, ain, r.w_sg, r.T, a.H, r.E, r.k, r.slot_row);
    __syncthreads();
    // the walkers' work list straight from the sorting wavefronts' registers
    const SortedRow row = small_route_sort_rows<4>(rl.L, F, r.E);
    if (blockIdx.x != 0 && wave < sort_waves(F))
      small_route_tiles<4>(rl.L, row, r.T, r.k, r.E, rl.tiles, rl.tok, rl.n, nullptr, nullptr, wave == 0, false);
    __syncthreads();
    if (blockIdx.x == 0) {
      // the shared gates here, not beside the top-k: their registers would
      // stay live through the other workgroups' walks otherwise
      small_route_gate<4>(rl.L, ain, r.w_sg, r.T, a.H);
      small_route_store<4>(rl.L, r.T, r.k, r.E, r.n_slots, r.ids, r.w, r.sigma, r.offsets, r.perm, r.inv_perm,
                           r.group_slot, r.status, r.meta, r.tiles, r.tile_tok, nullptr, r.sync, r.n_sync);
      return;
    }
    n_items = rl.n[0] * a.n_ug;
    first -= 1;
    stride -= 1;
  } else {
    n_items = *as_const(n_tiles) * a.n_ug;
  }
  auto walk = [&](auto tl, auto tt) __attribute__((always_inline)) {
    Start<GATEUP, SPLITK, S, U, FS, MX> st;
    const Desc d0 = load_desc<GATEUP>(a, first, threadIdx.x & 15, tl, tt);
    stage_start<GATEUP, SPLITK, S, U, FS, MX, true>(st, a, d0, n_items, stride, tl, tt, pool, ain);
    stage_walk<GATEUP, SPLITK, S, U, FS, MX, PlainStage>(st, a, stride, n_items, tl, tt, pool, ain, out, nullptr,
                                                         red);
  };
  if constexpr (ROUTE)
    walk((lds_int4_p)rl.tiles, (lds_int_p)rl.tok);
  else
    walk(tiles, tile_tok);
}

// The down projection and the combine in one launch, by column block (S4 down
// + S5; [Strata] "路由以后，专家怎样分工？": a token's expert outputs are
// weighted and summed once all have arrived).  Workgroup P b + e (P parts)
// computes the Y rows of the tiles t = e, e + P, ... for the 16 output units
// of column block b (K = I = 512: one round of four 32-value chunks per
// lane); its wavefronts take those tiles in turn (t = e + P w + P W i), each
// issuing a batch of tiles' weight loads at once and their h rows one tile
// ahead.  Measured on the 48-layer decode window, one tile per wavefront and
// batch, 16 wavefronts and two parts were fastest: many short independent
// streams per CU.  The Y rows are stored device-coherently; the workgroup then
// counts itself on the block's counter (zeroed by the grouping that wrote the
// work list), and the last of the P combines the block for every token in
// k_combine's arithmetic and zeroes the counter again.  Nothing waits, so the
// grid need not be resident as a whole.
#ifndef MOE_DC_TILES
#define MOE_DC_TILES 1
#endif
#ifndef MOE_DC_PARTS
#define MOE_DC_PARTS 2
#endif
#ifndef MOE_DC_WAVES
#define MOE_DC_WAVES 16
#endif
constexpr int kDcTiles = MOE_DC_TILES;   // tiles per wavefront per batch
constexpr int kDcWaves = MOE_DC_WAVES;   // wavefronts per workgroup
constexpr int kDcParts = MOE_DC_PARTS;   // workgroups per column block
constexpr int kDcMaxT = 16;       // tokens of a window
constexpr int kDcMaskWords = 32;  // column blocks / 32 (H <= 16384)
__global__ __launch_bounds__(64 * kDcWaves, kDcParts > 2 ? 2 : 1) void k_down_comb(const int4* __restrict__ tiles, const int32_t* __restrict__ n_tiles_p,
                                                   DecArgs a, const uint8_t* __restrict__ pool,
                                                   const uint16_t* __restrict__ h, uint16_t* __restrict__ y_rows,
                                                   FusedCtx fc) {
  __shared__ int2 pw[kSortF];         // (inv_perm, w) of each (token, slot) entry
  __shared__ float sg[kDcMaxT];       // sigma of each token
  __shared__ uint32_t mask[kDcMaskWords];
  __shared__ int second;
  const int cb = blockIdx.x / kDcParts, part = blockIdx.x % kDcParts;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
  const int nt = *as_const(n_tiles_p);
  const int n_items = nt * a.n_ug;
  // wavefront w takes tiles part + P w + P W i (P parts, W wavefronts), kDcTiles at a time
  for (int j0 = 0; part + kDcParts * wave + kDcParts * kDcWaves * kDcTiles * j0 < nt; j0++) {
    Item<1> it[kDcTiles];
    Step<1> fb[kDcTiles][4];
    uint2 sc[kDcTiles];
#pragma unroll
    for (int m = 0; m < kDcTiles; m++) {
      const int t = part + kDcParts * wave + kDcParts * kDcWaves * (kDcTiles * j0 + m);
      Desc dd;
      dd.td = tiles[min(t, a.max_tiles - 1)];
      dd.tok = 0;
      dd.item = t * a.n_ug + cb;
      it[m] = make_item<false, 1, true, false>(a, dd, n_items, 0, c, pool, h);
      load_sc<1>(&sc[m], it[m], 0);
#pragma unroll
      for (int st = 0; st < 4; st++) load_step<1, true, false>(fb[m][st], it[m], 4 * q + st, 16, c);
    }
    uint4 xa[2][4][4];
#pragma unroll
    for (int st = 0; st < 4; st++) load_a<1, kAuxPlain>(xa[0][st], it[0], 4 * q + st);
#pragma unroll
    for (int m = 0; m < kDcTiles; m++) {
      if (m + 1 < kDcTiles) {
#pragma unroll
        for (int st = 0; st < 4; st++) load_a<1, kAuxPlain>(xa[(m + 1) & 1][st], it[m + 1], 4 * q + st);
      }
      f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int st = 0; st < 4; st++) {
        const uint32_t sw = (st < 2 ? sc[m].x : sc[m].y) >> (16 * (st & 1));
        mma_step<1, false>(fb[m][st], xa[m & 1][st], &sw, it[m].resident, acc);
      }
      if (it[m].live) {
        uint16_t* orows = y_rows + (int64_t)it[m].p0 * a.H;
        const int obytes = it[m].n * a.H * 2;
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int row = 4 * q + r;  // D[row][c]
          if (row < it[m].n)
            store_bf16<kAuxDevice>(orows, obytes, row * a.H + it[m].unit, f32_to_bf16_rne(it[m].g0 * acc[0][r]));
        }
      }
    }
  }
  // the routing's outputs for the combine (written before the launch)
  const int F = fc.T * fc.k;
  for (int i = threadIdx.x; i < F; i += blockDim.x) pw[i] = make_int2(fc.inv_perm[i], __float_as_int(fc.w[i]));
  for (int i = threadIdx.x; i < fc.T; i += blockDim.x) sg[i] = fc.sigma[i];
  for (int i = threadIdx.x; i < (fc.H / 16 + 31) / 32; i += blockDim.x) mask[i] = i == (cb >> 5) ? 1u << (cb & 31) : 0u;
  // every Y store of this workgroup has completed (written through to the
  // device-coherent level) before it is counted
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t* ctr = counter(fc, 1 + fc.max_tiles + cb);
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    second = old == kDcParts - 1;
    if (old == kDcParts - 1) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (second) combine_blocks(y_rows, fc, mask, pw, sg);
}

// Gate/up items of the fused launch: with R = ceil(n / G) rounds, the first
// nf = n - (R - 1) G workgroups take R items each, the others R - 1.  The R-item
// workgroups take the last R nf items (strided by nf, so each round covers
// consecutive items), so only the tiles of those items finish a round late;
// the others take items [0, n - R nf), strided by G - nf.
struct GuWalk {
  int first, stride, limit;
};
__device__ inline GuWalk gu_walk(int n, int G, int b) {
  const int R = (n + G - 1) / G;
  const int nf = n - (R - 1) * G;
  if (R == 0) return GuWalk{0, 1, 0};
  if (b < nf) return GuWalk{n - R * nf + b, nf, n};
  return GuWalk{b - nf, G - nf, n - R * nf};
}

// Both stages in one launch.  Gate/up items as gu_walk gives them; down items
// to G - 1 - b, G - 1 - b + G, ... (the workgroups that take the late tiles'
// gate/up items take the late tiles' first down items, so these wait on no
// other late work).  The grid must be resident as a whole (the launcher sizes
// it by the occupancy), so a down item's wait only ever waits on gate/up
// work of running workgroups.
template <int GSK, int GS, int GU, bool GFS, int DSK, int DS, int DU, bool DFS, bool COMB>
__global__ __launch_bounds__(256) void k_ffn_dec_fused(DecArgs ag, DecArgs ad, const int4* __restrict__ tiles,
                                                       const int32_t* __restrict__ tile_tok,
                                                       const int32_t* __restrict__ n_tiles_p,
                                                       const uint8_t* __restrict__ pool,
                                                       const uint16_t* __restrict__ x, uint16_t* __restrict__ h,
                                                       uint16_t* __restrict__ y_rows, FusedCtx fc) {
  constexpr int GNS = 2 * GU, DNS = DU;
  constexpr int RW = (GSK > 1 || DSK > 1) ? 4 : 1, RNS = GNS > DNS ? GNS : DNS;
  __shared__ f32x4 red[RW][RNS][64];
  __shared__ int last_wg;
  // column blocks this workgroup combines, and the staged combine inputs
  __shared__ uint32_t comb_mask[COMB ? kMaxExperts / 32 : 1];
  __shared__ int2 comb_pw[COMB ? kFusedCombineMaxT * kFusedCombineMaxK : 1];
  __shared__ float comb_sg[COMB ? kFusedCombineMaxT : 1];
  if (COMB)
    for (int i = threadIdx.x; i < kMaxExperts / 32; i += blockDim.x) comb_mask[i] = 0;
  const int n_tiles = *as_const(n_tiles_p);
  const int n_gu = n_tiles * ag.n_ug, n_dn = n_tiles * ad.n_ug;
  const int G = gridDim.x, b = blockIdx.x;
  // both first descriptors; gate/up's first unit (weights, A rows, next
  // descriptor); then the first down unit's weights (they do not depend on h)
  const int c = threadIdx.x & 15;
  const GuWalk gw = gu_walk(n_gu, G, b);
  const Desc gd0 = load_desc<true>(ag, gw.first, c, tiles, tile_tok);
  const Desc dd0 = load_desc<false>(ad, G - 1 - b, c, tiles, tile_tok);
  // (combine) this thread's share of inv_perm, w and sigma, staged in LDS
  // after the starts: off the launch's critical tail
  constexpr int kPwPer = kFusedCombineMaxT * kFusedCombineMaxK / 256;
  int2 cpw[COMB ? kPwPer : 1];
  float csg = 0.f;
  const int Tk = fc.T * fc.k;
  if (COMB) {
#pragma unroll
    for (int r = 0; r < kPwPer; r++) {
      const int i = min((int)threadIdx.x + 256 * r, Tk - 1);
      cpw[r] = make_int2(fc.inv_perm[i], __float_as_int(fc.w[i]));
    }
    csg = fc.sigma[min((int)threadIdx.x, fc.T - 1)];
  }
  Start<true, GSK, GS, GU, GFS, false> sg;
  stage_start<true, GSK, GS, GU, GFS, false, true>(sg, ag, gd0, gw.limit, gw.stride, tiles, tile_tok, pool, x);
  Start<false, DSK, DS, DU, DFS, false> sd;
  stage_start<false, DSK, DS, DU, DFS, false, false>(sd, ad, dd0, n_dn, G, tiles, tile_tok, pool, h);
  if (COMB) {
#pragma unroll
    for (int r = 0; r < kPwPer; r++)
      if ((int)threadIdx.x + 256 * r < Tk) comb_pw[threadIdx.x + 256 * r] = cpw[r];
    if ((int)threadIdx.x < fc.T) comb_sg[threadIdx.x] = csg;
  }
  stage_walk<true, GSK, GS, GU, GFS, false, Policy<kAuxPlain, kAuxDevice, false, false>>(
      sg, ag, gw.stride, gw.limit, tiles, tile_tok, pool, x, h, &fc, reinterpret_cast<f32x4(*)[GNS][64]>(red));
  // every wavefront that stored h rows: once its stores are complete, one
  // count for each of its gate/up items' tiles.  Published together at the
  // end of the gate/up walk: one wait for the stores instead of one per item
  // (no down item of this workgroup could start earlier anyway).
  if ((threadIdx.x >> 6) % GSK == 0 && gw.first < gw.limit) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if ((threadIdx.x & 63) == 0)
      for (int it = gw.first; it < gw.limit; it += gw.stride)
        __hip_atomic_fetch_add(counter(fc, 1 + it / ag.n_ug), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  stage_walk<false, DSK, DS, DU, DFS, false,
             Policy<kAuxDevice, COMB ? kAuxDevice : kAuxPlain, true, COMB>>(
      sd, ad, G, n_dn, tiles, tile_tok, pool, h, y_rows, &fc, reinterpret_cast<f32x4(*)[DNS][64]>(red), comb_mask);
  if (COMB) {
    __syncthreads();
    combine_blocks(y_rows, fc, comb_mask, comb_pw, comb_sg);
  }
  // the last workgroup to finish zeroes the counters for the next launch
  __syncthreads();
  if (threadIdx.x == 0)
    last_wg = __hip_atomic_fetch_add(counter(fc, 0), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1;
  __syncthreads();
  if (last_wg) {
    const int nb = COMB ? fc.H / fc.cols : 0;
    for (int i = threadIdx.x; i < n_tiles; i += blockDim.x) *counter(fc, 1 + i) = 0;
    for (int i = threadIdx.x; i < nb; i += blockDim.x) *counter(fc, 1 + fc.max_tiles + i) = 0;
    if (threadIdx.x == 0) *counter(fc, 0) = 0;
  }
}

// ---- route, group, both FFN stages and the combine in one launch ----------
// (moe_route_group_ffn_combine; [FreeToken] 3.5: a decode step's control flow
// stays on the device.)  Every workgroup first routes and groups the window
// into its own LDS (as the routing gate/up launch does), so the weight stream
// starts without a descriptor chain through memory.  Workgroup 0 then zeroes
// this launch's counters, stores every routing output (the combine's inputs
// device-coherently) and, once those stores have completed, sets the ready
// flag to kLayerReady; it walks down items only.  Workgroups 1 .. G - 1 issue
// their first down unit's weights, walk the gate/up items (gu_walk over G - 1
// walkers, h stored device-coherently), and wait for the flag before their
// first counter access, so every count of the launch lands on zeroed
// counters even in a workspace fresh from the allocator (the flag holds the
// value only between workgroup 0's stores and the launch's end).  From there
// on the down stage and the combine run as in k_ffn_dec_fused, the combine's
// inputs (inv_perm, weights, sigma) read back from memory into LDS.
constexpr uint64_t kLayerReady = 0x4d6f454c61796572ull;

template <int GSK, int GS, int GU, bool GFS, int DSK, int DS, int DU, bool DFS, int RNPL>
__global__ __launch_bounds__(256) void k_layer_dec(DecArgs ag, DecArgs ad, const uint8_t* __restrict__ pool,
                                                   const uint16_t* __restrict__ x, uint16_t* __restrict__ h,
                                                   uint16_t* __restrict__ y_rows, FusedCtx fc, RouteArgs r) {
  constexpr int GNS = 2 * GU, DNS = DU;
  constexpr int RW = (GSK > 1 || DSK > 1) ? 4 : 1, RNS = GNS > DNS ? GNS : DNS;
  __shared__ f32x4 red[RW][RNS][64];
  __shared__ RouteLds rl;
  __shared__ int last_wg;
  __shared__ uint32_t comb_mask[kMaxExperts / 32];
  __shared__ int2 comb_pw[kSortF];
  __shared__ float comb_sg[16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, c = tid & 15;
  const int G = gridDim.x, b = blockIdx.x;
  const int F = r.T * r.k;
  for (int i = tid; i < kMaxExperts / 32; i += blockDim.x) comb_mask[i] = 0;
  small_route_topk<RNPL, 4, false>(rl.L, r.logits, x, r.w_sg, r.T, ag.H, r.E, r.k, r.slot_row);
  __syncthreads();
  const SortedRow row = small_route_sort_rows<4>(rl.L, F, r.E);
  if (wave < sort_waves(F))
    small_route_tiles<4>(rl.L, row, r.T, r.k, r.E, rl.tiles, rl.tok, rl.n, nullptr, nullptr, wave == 0, false);
  __syncthreads();
  const lds_int4_p tiles = (lds_int4_p)rl.tiles;
  const lds_int_p tok = (lds_int_p)rl.tok;
  const int n_tiles = rl.n[0];
  const int n_gu = n_tiles * ag.n_ug, n_dn = n_tiles * ad.n_ug;
  const Desc dd0 = load_desc<false>(ad, G - 1 - b, c, tiles, tok);
  Start<false, DSK, DS, DU, DFS, false> sd;
  GuWalk gw{0, 1, 0};
  if (b == 0) {
    stage_start<false, DSK, DS, DU, DFS, false, false>(sd, ad, dd0, n_dn, G, tiles, tok, pool, h);
    for (int i = tid; i < fc.n_zero; i += blockDim.x)
      __hip_atomic_store(counter(fc, i), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    small_route_gate<4>(rl.L, x, r.w_sg, r.T, ag.H);
    small_route_store<4, true>(rl.L, r.T, r.k, r.E, r.n_slots, r.ids, r.w, r.sigma, r.offsets, r.perm, r.inv_perm,
                               r.group_slot, r.status, r.meta, r.tiles, r.tile_tok, nullptr, nullptr, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) __hip_atomic_store(fc.flag, kLayerReady, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    gw = gu_walk(n_gu, G - 1, b - 1);
    const Desc gd0 = load_desc<true>(ag, gw.first, c, tiles, tok);
    Start<true, GSK, GS, GU, GFS, false> sg;
    stage_start<true, GSK, GS, GU, GFS, false, true>(sg, ag, gd0, gw.limit, gw.stride, tiles, tok, pool, x);
    stage_start<false, DSK, DS, DU, DFS, false, false>(sd, ad, dd0, n_dn, G, tiles, tok, pool, h);
    stage_walk<true, GSK, GS, GU, GFS, false, Policy<kAuxPlain, kAuxDevice, false, false>>(
        sg, ag, gw.stride, gw.limit, tiles, tok, pool, x, h, &fc, reinterpret_cast<f32x4(*)[GNS][64]>(red));
  }
  // the ready flag (bounded wait by wavefront 0; its first poll is issued
  // after this wavefront's h stores, so one wait covers both)
  if (wave == 0) {
    int spins = 0;
    for (;;) {
      const uint64_t v = __hip_atomic_load(fc.flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
      if ((((uint64_t)hi << 32) | lo) == kLayerReady) break;
      if (++spins > fc.spin_limit) {
        if (lane == 0) atomicOr(fc.status, MOE_DEV_SYNC_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
  }
  __syncthreads();
  // every wavefront that stored h rows: one count for each of its gate/up
  // items' tiles, once its stores have completed
  if (b > 0 && wave % GSK == 0 && gw.first < gw.limit) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0)
      for (int it = gw.first; it < gw.limit; it += gw.stride)
        __hip_atomic_fetch_add(counter(fc, 1 + it / ag.n_ug), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the combine's inputs, written by workgroup 0 before the flag
  if (wave > 0) {
    for (int i = tid - 64; i < F; i += 192)
      comb_pw[i] = make_int2(__hip_atomic_load(r.inv_perm + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                             __float_as_int(__hip_atomic_load(r.w + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
    if (tid - 64 < r.T)
      comb_sg[tid - 64] = __hip_atomic_load(r.sigma + (tid - 64), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  stage_walk<false, DSK, DS, DU, DFS, false, Policy<kAuxDevice, kAuxDevice, true, true>>(
      sd, ad, G, n_dn, tiles, tok, pool, h, y_rows, &fc, reinterpret_cast<f32x4(*)[DNS][64]>(red), comb_mask);
  __syncthreads();
  combine_blocks(y_rows, fc, comb_mask, comb_pw, comb_sg);
  // the last workgroup to finish zeroes the counters and clears the flag
  __syncthreads();
  if (tid == 0)
    last_wg = __hip_atomic_fetch_add(counter(fc, 0), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1;
  __syncthreads();
  if (last_wg) {
    const int nb = fc.H / fc.cols;
    for (int i = tid; i < n_tiles; i += blockDim.x) *counter(fc, 1 + i) = 0;
    for (int i = tid; i < nb; i += blockDim.x) *counter(fc, 1 + fc.max_tiles + i) = 0;
    if (tid == 0) {
      *counter(fc, 0) = 0;
      *fc.flag = 0;
    }
  }
}

struct DecPtrs {
  const int4* tiles;
  const int32_t* tile_tok;
  const int32_t* n_tiles;
  const uint8_t* pool;
  const uint16_t* ain;
  uint16_t* out;
  RouteArgs route;  // gate/up only; logits null otherwise
};

// ev0 / ev1: when either is set, the launch goes through hipExtLaunchKernelGGL
// and the device records them at the kernel's start and end.
struct DecLaunch {
  int grid;
  hipStream_t st;
  hipEvent_t ev0, ev1;
};

template <bool GATEUP, int SK, int S, int U, bool FS, bool MX, int RNPL>
hipError_t launch_kr(const DecArgs& a, const DecPtrs& p, const DecLaunch& l) {
  const RouteArgs& r = p.route;
  if (l.ev0 || l.ev1)
    hipExtLaunchKernelGGL((k_ffn_dec<GATEUP, SK, S, U, FS, MX, RNPL>), dim3(l.grid), dim3(256), 0, l.st, l.ev0,
                          l.ev1, 0, r.logits, r.slot_row, r.T, r.E, r.k, p.tiles, p.n_tiles, a.n_ug, a.max_tiles, a,
                          p.tile_tok, p.pool, p.ain, p.out, r);
  else
    hipLaunchKernelGGL((k_ffn_dec<GATEUP, SK, S, U, FS, MX, RNPL>), dim3(l.grid), dim3(256), 0, l.st, r.logits,
                       r.slot_row, r.T, r.E, r.k, p.tiles, p.n_tiles, a.n_ug, a.max_tiles, a, p.tile_tok, p.pool,
                       p.ain, p.out, r);
  return hipGetLastError();
}

template <bool GATEUP, int SK, int S, int U, bool FS, bool MX>
hipError_t launch_k(const DecArgs& a, const DecPtrs& p, const DecLaunch& l) {
  if constexpr (GATEUP && !MX)
    if (p.route.logits)
      return p.route.E <= 512 ? launch_kr<GATEUP, SK, S, U, FS, MX, 8>(a, p, l)
                              : launch_kr<GATEUP, SK, S, U, FS, MX, 16>(a, p, l);
  return launch_kr<GATEUP, SK, S, U, FS, MX, 0>(a, p, l);
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

// A stage's split: K four ways when a unit block has more than 4 steps, else
// each wavefront its own unit blocks; steps beyond MOE_DEC_MAXS per wavefront
// run as further K rounds.  FS: every wavefront's share is whole 512-value
// groups with S = 4.
struct Split {
  int sk, U, S, n_kr, n_ug;
  bool fs;
};

Split stage_split(const moe_dims& d, bool gu, bool mx) {
  Split sp;
  const int K = gu ? d.H : d.I, units = gu ? d.I : d.H;
  const int ublocks = units / 16;
  const int steps = (K + 127) / 128;
  const int maxs = gu ? MOE_DEC_MAXS_GU : MOE_DEC_MAXS_DN;
  sp.sk = steps > 4 ? 4 : 1;
  sp.U = (gu ? MOE_DEC_U_GU : MOE_DEC_U_DN) > 1 ? 2 : 1;
  if (ublocks % ((4 / sp.sk) * sp.U) != 0) sp.U = 1;
  if (ublocks % ((4 / sp.sk) * sp.U) != 0) sp.sk = 4;  // one unit block per item, K split four ways
  const int wsteps = (steps + sp.sk - 1) / sp.sk;
  sp.S = wsteps <= 1 ? 1 : (wsteps <= 2 || maxs <= 2) ? 2 : 4;
  sp.n_kr = (wsteps + sp.S - 1) / sp.S;
  sp.n_ug = ublocks / ((4 / sp.sk) * sp.U);
  sp.fs = !mx && sp.S == 4 && maxs >= 4 && K % (512 * sp.sk) == 0;
  return sp;
}

DecArgs dec_args(const moe_dims& d, const FfnGeom& g, const WsLayout& wl, const Split& sp) {
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
  a.n_kr = sp.n_kr;
  a.n_ug = sp.n_ug;
  return a;
}

// ---- the fused launch: the splits it is built for ---------------------------
// (gate/up split, down split) pairs with an instantiation; other shapes run
// the two stages as two launches.
struct FusedKey {
  int gsk, gs, gu, gfs, dsk, ds, du, dfs;
};
constexpr FusedKey kFused[] = {
    {4, 4, 1, 1, 1, 4, 2, 1},  // H 2048, I 512 (the 48-layer 512-expert decode)
    {4, 4, 1, 1, 4, 4, 2, 1},  // H 4096, I 2048 (the 43-layer 256-expert decode)
    {1, 4, 1, 1, 1, 2, 2, 0},  // H 512, I 256
};

using FusedFn = void (*)(DecArgs, DecArgs, const int4*, const int32_t*, const int32_t*, const uint8_t*,
                         const uint16_t*, uint16_t*, uint16_t*, FusedCtx);

template <int I>
FusedFn fused_fn(bool comb) {
  constexpr FusedKey f = kFused[I];
  return comb ? k_ffn_dec_fused<f.gsk, f.gs, f.gu, (bool)f.gfs, f.dsk, f.ds, f.du, (bool)f.dfs, true>
              : k_ffn_dec_fused<f.gsk, f.gs, f.gu, (bool)f.gfs, f.dsk, f.ds, f.du, (bool)f.dfs, false>;
}

FusedFn find_fused(const Split& g, const Split& dn, bool comb) {
  auto match = [&](const FusedKey& f) {
    return f.gsk == g.sk && f.gs == g.S && f.gu == g.U && f.gfs == (int)g.fs && f.dsk == dn.sk && f.ds == dn.S &&
           f.du == dn.U && f.dfs == (int)dn.fs;
  };
  if (match(kFused[0])) return fused_fn<0>(comb);
  if (match(kFused[1])) return fused_fn<1>(comb);
  if (match(kFused[2])) return fused_fn<2>(comb);
  return nullptr;
}

// The fused launch's wait parameters: the poll limit, and a count added to
// every tile's target.  Tests set them (moe_debug_set_fused_wait) to force a
// wait to time out while every wavefront still ends: with an added count the
// target is never reached and each wait gives up after the poll limit.
std::atomic<int> g_spin_limit{MOE_DEC_SPIN_LIMIT};
std::atomic<int> g_extra_target{0};

// The routed one-launch layer (k_layer_dec) for the same splits; RNPL as for
// the routing gate/up launch (8 logits per lane up to E = 512, 16 above).
using LayerFn = void (*)(DecArgs, DecArgs, const uint8_t*, const uint16_t*, uint16_t*, uint16_t*, FusedCtx,
                         RouteArgs);

template <int I>
LayerFn layer_fn(int E) {
  constexpr FusedKey f = kFused[I];
  return E <= 512 ? k_layer_dec<f.gsk, f.gs, f.gu, (bool)f.gfs, f.dsk, f.ds, f.du, (bool)f.dfs, 8>
                  : k_layer_dec<f.gsk, f.gs, f.gu, (bool)f.gfs, f.dsk, f.ds, f.du, (bool)f.dfs, 16>;
}

LayerFn find_layer(const Split& g, const Split& dn, int E) {
  auto match = [&](const FusedKey& f) {
    return f.gsk == g.sk && f.gs == g.S && f.gu == g.U && f.gfs == (int)g.fs && f.dsk == dn.sk && f.ds == dn.S &&
           f.du == dn.U && f.dfs == (int)dn.fs;
  };
  if (match(kFused[0])) return layer_fn<0>(E);
  if (match(kFused[1])) return layer_fn<1>(E);
  if (match(kFused[2])) return layer_fn<2>(E);
  return nullptr;
}

// workgroups of fn resident per CU (queried once per kernel)
int fused_occupancy(const void* fn) {
  static std::mutex mu;
  static const void* keys[8];
  static int vals[8];
  static int n = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; i++)
    if (keys[i] == fn) return vals[i];
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) !=
      hipSuccess)
    per_cu = 0;
  if (n < 8) {
    keys[n] = fn;
    vals[n] = per_cu;
    n++;
  }
  return per_cu;
}

}  // namespace

namespace {

// The stages of the decode-path FFN, one launch each; route (gate/up only):
// the window's routing in that launch.
hipError_t launch_dec_stages(const moe_dims& d, const uint16_t* x, const FfnGeom& g, uint16_t* h, uint16_t* y_rows,
                             void* ws, int n_cu, int stages, hipEvent_t ev_start, hipEvent_t ev_stop, hipStream_t s,
                             bool mx, const uint16_t* down_in, const RouteArgs* route) {
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  DecPtrs ptrs;
  ptrs.tiles = reinterpret_cast<const int4*>(base + wl.off_tiles);
  ptrs.tile_tok = reinterpret_cast<const int32_t*>(base + wl.off_tile_tok);
  ptrs.n_tiles = reinterpret_cast<const int32_t*>(base + wl.off_meta);
  ptrs.pool = g.pool;
  for (int stage = 0; stage < 2; stage++) {
    if (!((stages >> stage) & 1)) continue;
    const bool gu = stage == 0;
    const int64_t cap = (int64_t)n_cu * (gu ? MOE_DEC_WGS_GU : MOE_DEC_WGS_DN);
    const Split sp = stage_split(d, gu, mx);
    DecArgs a = dec_args(d, g, wl, sp);
    // a routing launch's work list is in LDS: at most kRouteMaxTiles entries
    if (gu && route && a.max_tiles > kRouteMaxTiles) a.max_tiles = kRouteMaxTiles;
    const int64_t items = (int64_t)a.max_tiles * a.n_ug;
    // a routing launch has one more workgroup, which only stores the routing;
    // the grid stays within the resident cap (a workgroup beyond it would
    // start only when another ends)
    const int64_t want = items + ((gu && route) ? 1 : 0);
    const int grid = (int)(want < cap ? want : cap);
    ptrs.ain = gu ? x : (down_in ? down_in : h);
    ptrs.out = gu ? h : y_rows;
    ptrs.route = RouteArgs{};
    if (gu && route) ptrs.route = *route;
    // the start event goes with the first stage launched, the stop event with the last
    const bool first = gu || !(stages & 1), last = !gu || !(stages & 2);
    const DecLaunch l{grid, s, first ? ev_start : nullptr, last ? ev_stop : nullptr};
    const hipError_t e = mx ? (gu ? launch_su<true, true>(a, ptrs, sp.sk, sp.S, sp.U, l)
                                  : launch_su<false, true>(a, ptrs, sp.sk, sp.S, sp.U, l))
                            : (gu ? launch_su<true, false>(a, ptrs, sp.sk, sp.S, sp.U, l)
                                  : launch_su<false, false>(a, ptrs, sp.sk, sp.S, sp.U, l));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// Decode-path FFN: both stages, persistent grids of (CUs x MOE_DEC_WGS_GU or
// MOE_DEC_WGS_DN) workgroups (fewer when there is less work than that).
hipError_t launch_ffn_dec(const moe_dims& d, const uint16_t* x, const FfnGeom& g, const int32_t* perm, uint16_t* h,
                          uint16_t* y_rows, void* ws, int n_cu, int stages, hipEvent_t ev_start, hipEvent_t ev_stop,
                          hipStream_t s, bool mx, const uint16_t* down_in) {
  (void)perm;
  return launch_dec_stages(d, x, g, h, y_rows, ws, n_cu, stages, ev_start, ev_stop, s, mx, down_in, nullptr);
}

bool route_ffn_fusable(const moe_dims& d) {
  return !use_gemm(d) && d.T <= 16 && (int64_t)d.T * d.k <= kSortF && d.E <= kMaxExperts;
}

hipError_t launch_route_ffn_dec(const moe_dims& d, int32_t layer, const float* logits, const uint16_t* x,
                                const float* w_sg, const int32_t* slot_table, int32_t n_slots, int32_t* ids,
                                float* w, float* sigma, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                int32_t* group_slot, int32_t* dev_status, const FfnGeom& g, uint16_t* h,
                                uint16_t* y_rows, void* ws, int n_cu, int stages, hipEvent_t ev_start,
                                hipEvent_t ev_stop, hipStream_t s) {
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  RouteArgs r;
  r.logits = logits;
  r.w_sg = w_sg;
  r.slot_row = slot_table + (int64_t)layer * (d.E + 1);
  r.T = d.T;
  r.k = d.k;
  r.E = d.E;
  r.n_slots = n_slots;
  r.ids = ids;
  r.w = w;
  r.sigma = sigma;
  r.offsets = offsets;
  r.perm = perm;
  r.inv_perm = inv_perm;
  r.group_slot = group_slot;
  r.status = dev_status;
  r.meta = reinterpret_cast<int32_t*>(base + wl.off_meta);
  r.tiles = reinterpret_cast<int4*>(base + wl.off_tiles);
  r.tile_tok = reinterpret_cast<int32_t*>(base + wl.off_tile_tok);
  r.sync = reinterpret_cast<int32_t*>(base + wl.off_sync);
  r.n_sync = wl.n_sync;
  return launch_dec_stages(d, x, g, h, y_rows, ws, n_cu, stages | 1, ev_start, ev_stop, s, false, nullptr, &r);
}

bool ffn_dec_fusable(const moe_dims& d, bool combine) {
  if (use_gemm(d)) return false;
  if (combine && (d.T > kFusedCombineMaxT || d.k > kFusedCombineMaxK)) return false;
  return find_fused(stage_split(d, true, false), stage_split(d, false, false), combine) != nullptr;
}

hipError_t launch_ffn_dec_fused(const moe_dims& d, const uint16_t* x, const FfnGeom& g, uint16_t* h,
                                uint16_t* y_rows, int32_t* dev_status, void* ws, int n_cu, hipEvent_t ev_start,
                                hipEvent_t ev_stop, hipStream_t s, const int32_t* inv_perm, const float* w,
                                const float* sigma, uint16_t* y) {
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const Split sg = stage_split(d, true, false), sdn = stage_split(d, false, false);
  const bool comb = inv_perm != nullptr;
  const FusedFn fn = find_fused(sg, sdn, comb);
  if (!fn) return hipErrorInvalidConfiguration;
  const DecArgs ag = dec_args(d, g, wl, sg), ad = dec_args(d, g, wl, sdn);
  const int per_cu = fused_occupancy(reinterpret_cast<const void*>(fn));
  if (per_cu <= 0) return hipErrorInvalidConfiguration;
  const int64_t cap = (int64_t)n_cu * (per_cu < MOE_DEC_WGS_FUSED ? per_cu : MOE_DEC_WGS_FUSED);
  const int64_t items = (int64_t)wl.max_tiles * (ag.n_ug > ad.n_ug ? ag.n_ug : ad.n_ug);
  const int grid = (int)(items < cap ? items : cap);
  FusedCtx fc;
  fc.sync = reinterpret_cast<int32_t*>(base + wl.off_sync);
  fc.status = dev_status;
  fc.max_tiles = (int32_t)wl.max_tiles;
  // every storing wavefront of every gate/up item of a tile
  fc.gu_target = ag.n_ug * (4 / sg.sk) + g_extra_target.load(std::memory_order_relaxed);
  fc.dn_target = 4 / sdn.sk;  // storing wavefronts of a down item
  fc.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  fc.flag = nullptr;
  fc.n_zero = 0;
  fc.inv_perm = inv_perm;
  fc.w = w;
  fc.sigma = sigma;
  fc.y = y;
  fc.T = d.T;
  fc.k = d.k;
  fc.H = d.H;
  fc.cols = d.H / ad.n_ug;
  const int4* tiles = reinterpret_cast<const int4*>(base + wl.off_tiles);
  const int32_t* tile_tok = reinterpret_cast<const int32_t*>(base + wl.off_tile_tok);
  const int32_t* n_tiles = reinterpret_cast<const int32_t*>(base + wl.off_meta);
  const uint8_t* pool = g.pool;
  void* args[] = {(void*)&ag, (void*)&ad, (void*)&tiles, (void*)&tile_tok, (void*)&n_tiles, (void*)&pool,
                  (void*)&x, (void*)&h, (void*)&y_rows, (void*)&fc};
  if (ev_start || ev_stop)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(256), args, 0, s, ev_start, ev_stop,
                              0);
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(256), args, 0, s);
}

bool down_combine_fusable(const moe_dims& d) {
  return !use_gemm(d) && d.I == 512 && d.T <= kDcMaxT && d.k <= kFusedCombineMaxK && (int64_t)d.T * d.k <= kSortF &&
         d.H % 16 == 0 && d.H / 16 <= 32 * kDcMaskWords;
}

hipError_t launch_down_combine(const moe_dims& d, const FfnGeom& g, const uint16_t* h, uint16_t* y_rows, void* ws,
                               hipEvent_t ev_start, hipEvent_t ev_stop, hipStream_t s, const int32_t* inv_perm,
                               const float* w, const float* sigma, uint16_t* y) {
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  DecArgs a = dec_args(d, g, wl, stage_split(d, false, false));
  a.n_ug = d.H / 16;  // an item is one tile by one 16-unit column block
  a.n_kr = 1;
  FusedCtx fc = {};
  fc.sync = reinterpret_cast<int32_t*>(base + wl.off_sync);
  fc.max_tiles = (int32_t)wl.max_tiles;
  fc.inv_perm = inv_perm;
  fc.w = w;
  fc.sigma = sigma;
  fc.y = y;
  fc.T = d.T;
  fc.k = d.k;
  fc.H = d.H;
  fc.cols = 16;
  const int4* tiles = reinterpret_cast<const int4*>(base + wl.off_tiles);
  const int32_t* n_tiles = reinterpret_cast<const int32_t*>(base + wl.off_meta);
  const dim3 grid((unsigned)(kDcParts * (d.H / 16))), block(64 * kDcWaves);
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(k_down_comb, grid, block, 0, s, ev_start, ev_stop, 0, tiles, n_tiles, a, g.pool, h, y_rows,
                          fc);
  else
    hipLaunchKernelGGL(k_down_comb, grid, block, 0, s, tiles, n_tiles, a, g.pool, h, y_rows, fc);
  return hipGetLastError();
}

bool route_ffn_combine_fusable(const moe_dims& d) {
  return route_ffn_fusable(d) && d.T <= 16 && d.k <= kFusedCombineMaxK &&
         find_layer(stage_split(d, true, false), stage_split(d, false, false), d.E) != nullptr;
}

hipError_t launch_route_ffn_combine_dec(const moe_dims& d, int32_t layer, const float* logits, const uint16_t* x,
                                        const float* w_sg, const int32_t* slot_table, int32_t n_slots, int32_t* ids,
                                        float* w, float* sigma, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                        int32_t* group_slot, int32_t* dev_status, const FfnGeom& g, uint16_t* h,
                                        uint16_t* y_rows, uint16_t* y, void* ws, int n_cu, hipEvent_t ev_start,
                                        hipEvent_t ev_stop, hipStream_t s) {
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const Split sg = stage_split(d, true, false), sdn = stage_split(d, false, false);
  const LayerFn fn = find_layer(sg, sdn, d.E);
  if (!fn) return hipErrorInvalidConfiguration;
  DecArgs ag = dec_args(d, g, wl, sg), ad = dec_args(d, g, wl, sdn);
  // the work list is in LDS: at most kRouteMaxTiles entries
  if (ag.max_tiles > kRouteMaxTiles) ag.max_tiles = kRouteMaxTiles;
  ad.max_tiles = ag.max_tiles;
  const int per_cu = fused_occupancy(reinterpret_cast<const void*>(fn));
  if (per_cu <= 0) return hipErrorInvalidConfiguration;
  // the whole grid is resident (the waits only ever wait on running
  // workgroups): workgroup 0 plus the walkers
  const int64_t cap = (int64_t)n_cu * (per_cu < MOE_DEC_WGS_FUSED ? per_cu : MOE_DEC_WGS_FUSED);
  const int64_t items = (int64_t)ag.max_tiles * (ag.n_ug > ad.n_ug ? ag.n_ug : ad.n_ug) + 1;
  const int grid = (int)(items < cap ? items : cap);
  if (grid < 2) return hipErrorInvalidConfiguration;
  int32_t* sync = reinterpret_cast<int32_t*>(base + wl.off_sync);
  FusedCtx fc;
  fc.sync = sync;
  fc.status = dev_status;
  fc.max_tiles = (int32_t)wl.max_tiles;
  fc.gu_target = ag.n_ug * (4 / sg.sk) + g_extra_target.load(std::memory_order_relaxed);
  fc.dn_target = 4 / sdn.sk;
  fc.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  fc.flag = reinterpret_cast<uint64_t*>(sync + (wl.n_sync - 1) * kSyncStride);
  fc.n_zero = (int32_t)(wl.n_sync - 1);
  fc.inv_perm = inv_perm;
  fc.w = w;
  fc.sigma = sigma;
  fc.y = y;
  fc.T = d.T;
  fc.k = d.k;
  fc.H = d.H;
  fc.cols = d.H / ad.n_ug;
  RouteArgs r;
  r.logits = logits;
  r.w_sg = w_sg;
  r.slot_row = slot_table + (int64_t)layer * (d.E + 1);
  r.T = d.T;
  r.k = d.k;
  r.E = d.E;
  r.n_slots = n_slots;
  r.ids = ids;
  r.w = w;
  r.sigma = sigma;
  r.offsets = offsets;
  r.perm = perm;
  r.inv_perm = inv_perm;
  r.group_slot = group_slot;
  r.status = dev_status;
  r.meta = reinterpret_cast<int32_t*>(base + wl.off_meta);
  r.tiles = reinterpret_cast<int4*>(base + wl.off_tiles);
  r.tile_tok = reinterpret_cast<int32_t*>(base + wl.off_tile_tok);
  r.sync = nullptr;
  r.n_sync = 0;
  const uint8_t* pool = g.pool;
  void* args[] = {(void*)&ag, (void*)&ad, (void*)&pool, (void*)&x, (void*)&h, (void*)&y_rows, (void*)&fc, (void*)&r};
  if (ev_start || ev_stop)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(256), args, 0, s, ev_start, ev_stop,
                              0);
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(256), args, 0, s);
}

}  // namespace moe

// Test hook (declared in include/moe.h for the tests only): the fused FFN launch's
// poll limit and a count added to its tile targets; (-1, 0) restores the
// defaults.  Affects launches enqueued afterwards, from every thread.
extern "C" void moe_debug_set_fused_wait(int spin_limit, int extra_target) {
  moe::g_spin_limit.store(spin_limit < 0 ? MOE_DEC_SPIN_LIMIT : spin_limit);
  moe::g_extra_target.store(extra_target < 0 ? 0 : extra_target);
}
