// S4 for prefill-sized groups: grouped GEMM over chunks of <= 256 rows.
//
// [Strata] "路由以后，专家怎样分工？": the rows routed to one expert form one
// group, so the expert's weights can be read once for all of them; with a few
// hundred rows per group the FFN is a dense contraction and belongs on MFMA.
//  - Work: (chunk of <= 256 rows of one group, tile of output columns).  The
//    grouping kernels list the chunks; blocks map to (chunk, tile) so that all
//    tiles of one chunk run on the same XCD and share the chunk's A rows in
//    that XCD's L2.
//  - A workgroup has two roles, ROLES wavefronts of each per SIMD (gate/up
//    two: 1024 threads; down one: 512).  The producer wavefronts do all
//    global loads and stage each 64-value K step into LDS (double buffered):
//    the chunk's A rows (bf16 rows of x gathered through perm, or rows of h)
//    and the B tile, 128 columns of weights (gate/up: 64 units of each
//    matrix; down: 128 units) decoded from E2M1 codes times their E4M3 scale
//    in fp32 (exact: <= 6 significant bits) and packed to bf16 (exact).  Their
//    loads run three steps ahead in four register stages.  The consumer
//    wavefronts only read fragments and issue MFMAs.  Each barrier interval
//    then costs the longer of the two roles, not their sum, and the
//    producers' staging overlaps the MFMAs on each SIMD; with two producers
//    per SIMD each stages half as much per step (one A row half, a quarter
//    of a B column), and their load, decode and store latencies overlap.
//  - Consumer (row group wm, column part ch) owns four 16-row blocks
//    (interleaved over the SIMDs) by 128 / ROLES columns of the 256 x 128
//    output (gate/up: the gate and up blocks of the same units) and
//    accumulates exact bf16 products in fp32 with v_mfma_f32_16x16x32_bf16;
//    row blocks past the chunk's rows are skipped.  The global scales and the
//    activation are applied in the epilogue.
#include <hip/hip_ext.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "moe_common.hpp"

namespace moe {
namespace {

constexpr int GM = kChunkRows;   // rows per workgroup
constexpr int GC = 128;          // output columns per workgroup
constexpr int GK = 64;           // K per step
constexpr int LROW = GK + 16;    // bf16 per LDS row: 160-byte rows keep the 16-byte fragment reads of 16 rows conflict-free (144 does not)
// Wavefronts of each role per SIMD, per stage (1 or 2).  Gate/up (K = H,
// long items) runs two of each; down (K = I, eight steps an item) one.
#ifndef MOE_GEMM_ROLES_GU
#define MOE_GEMM_ROLES_GU 2
#endif
#ifndef MOE_GEMM_ROLES_DN
#define MOE_GEMM_ROLES_DN 1
#endif
template <int ROLES>
struct Shape {
  static constexpr int NCW = 4 * ROLES, NPW = NCW;    // consumer and producer wavefronts
  static constexpr int GT = 64 * (NCW + NPW);         // threads per workgroup
  static constexpr int AR = 2 * GM / (64 * NPW);      // A rows per producer thread (each its half of the step's 64 values)
  static constexpr int BQ = 64 * NPW / GC;            // producer threads per B column and step (2: 32 values each; 4: 16)
  static constexpr int NCB = 8 * 4 / NCW;             // 16-column blocks per consumer wavefront
};
constexpr int NST = 4;           // producer register stages

template <typename T>
using cptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ inline cptr<T> as_const(const T* p) {
  return (cptr<T>)p;
}

struct GemmArgs {
  uint32_t slot_stride;
  int32_t n_slots;
  uint32_t off_codes[3];
  uint32_t off_scales[3];
  uint32_t off_globals;
  int32_t H, I, k, Tk;  // Tk = T * k: routed rows; rows from Tk on are the shared group's
  int32_t n_ut;         // column tiles per chunk
  int32_t nk;           // K steps
};

// An empty instruction that reads v: the value counts as used on this path.
__device__ inline void touch(const uint4& v) { asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w)); }
__device__ inline void touch(const uint2& v) { asm volatile("" ::"v"(v.x), "v"(v.y)); }

// A producer thread's B values of one step into LDS: 32 codes (two scale
// blocks) or 16 codes (one), times their scales, as bf16
__device__ inline void stage_b(bf16x8* bd, const uint4& c, uint32_t sw) {
  const float s0 = e4m3_to_f32<0>(sw), s1 = e4m3_to_f32<1>(sw);
  bd[0] = dequant8(c.x, s0);
  bd[1] = dequant8(c.y, s0);
  bd[2] = dequant8(c.z, s1);
  bd[3] = dequant8(c.w, s1);
}
__device__ inline void stage_b(bf16x8* bd, const uint2& c, uint32_t sw) {
  const float s0 = e4m3_to_f32<0>(sw);
  bd[0] = dequant8(c.x, s0);
  bd[1] = dequant8(c.y, s0);
}

// Two floats as a bf16 pair (round to nearest even), lo in the low half.
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// One producer thread's global loads for one K step: 32 A values of each of
// two rows, and 32 weight codes with the aligned dword holding their two
// scales.
template <int BQ>
struct Codes;
template <>
struct Codes<2> {
  using type = uint4;  // 32 codes
};
template <>
struct Codes<4> {
  using type = uint2;  // 16 codes
};
template <int AR, int BQ>
struct Stage {
  uint4 a[AR][4];
  typename Codes<BQ>::type c;
  uint32_t sc;   // the dword holding the scale byte(s)
  uint32_t ssh;  // their bit offset in it
};

template <bool GATEUP, int ROLES>
__global__ __launch_bounds__(Shape<ROLES>::GT) void k_ffn_gemm(GemmArgs a, const int4* __restrict__ chunks,
                                                 const int32_t* __restrict__ meta, const int32_t* __restrict__ perm,
                                                 const uint8_t* __restrict__ pool, const uint16_t* __restrict__ ain,
                                                 uint16_t* __restrict__ out) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  using S_ = Shape<ROLES>;
  constexpr int NCW = S_::NCW, GT = S_::GT, AR = S_::AR, BQ = S_::BQ, NCB = S_::NCB;
  using Stage = moe::Stage<AR, BQ>;
  constexpr int UPW = GC / NMAT;  // units per workgroup
  const int K = GATEUP ? a.H : a.I;
  const int units = GATEUP ? a.I : a.H;
  // Work items are (chunk, column tile) pairs: item i is tile (i / 8) % n_ut
  // of chunk ((i / 8) / n_ut) * 8 + i % 8.  Blocks are dealt to the 8 XCDs
  // round-robin and the grid is a multiple of 8, so the items block b walks
  // (b, b + gridDim.x, ...) all run on XCD b % 8, where the tiles of their
  // chunks share its L2.  Their chunks grow along the walk: the first one
  // past the chunk count ends it.
  const int n_chunks = *as_const(meta + 1);
  using i32x4 = int __attribute__((ext_vector_type(4)));
  auto item_chunk = [&](int i) { return ((i >> 3) / a.n_ut) * 8 + (i & 7); };
  auto item_desc = [&](int i) { return as_const(reinterpret_cast<const i32x4*>(chunks))[item_chunk(i)]; };
  auto item_u0 = [&](int i) { return ((i >> 3) % a.n_ut) * UPW; };
  int item = blockIdx.x;
  if (item_chunk(item) >= n_chunks) return;

  __shared__ __align__(16) uint16_t As[2][GM * LROW];
  __shared__ __align__(16) uint16_t Bs[2][GC * LROW];

  // the output tile, staged for the epilogue in the A buffers
  constexpr int OC = GATEUP ? GC / 2 : GC;  // output columns of the tile
  constexpr int OSTR = OC + 8;              // uint16 per row: 16-byte pad, rows stay 16-byte aligned
  static_assert(GM * OSTR <= 2 * GM * LROW, "output tile fits the A buffers");
  uint16_t* os = &As[0][0];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the step loop runs a multiple of 4 steps (the producers' register ring);
  // steps past the end stage zeros
  const int nk4 = (a.nk + 3) & ~3;

  // epilogue, part 2 (all eight wavefronts, once the consumers have written
  // the tile): it leaves in 16-byte row segments (units come in multiples of
  // 16); the second barrier frees the A buffers for the next item
  constexpr int SEGS = OC / 8;
  auto copy_out = [&](int p0, int n, int u0) __attribute__((always_inline)) {
    __syncthreads();
#pragma unroll 4
    for (int i = tid; i < n * SEGS; i += GT) {
      const int row = i / SEGS, sg = i % SEGS;
      const int unit = u0 + 8 * sg;
      if (unit < units)
        *reinterpret_cast<uint4*>(out + (int64_t)(p0 + row) * units + unit) =
            *reinterpret_cast<const uint4*>(&os[row * OSTR + 8 * sg]);
    }
    __syncthreads();
  };

  if (wave >= NCW) {
    // ---------------- producer ----------------
    const int t = tid - 64 * NCW;
    // A staging: rows ar and ar + 128, K half ah (32 values each).  Rows beyond
    // n load the last row (unbranched loads keep the wait counts exact) but are
    // not written to LDS unless their 16-row block is live (their outputs are
    // dropped)
    const int ah = t & 1;
    int ar[AR];
#pragma unroll
    for (int h = 0; h < AR; h++) ar[h] = (t >> 1) + (GM / AR) * h;
    // B staging: column bc, K part bh of the step (a half of 32 values, or a
    // quarter of 16)
    const int bc = t / BQ, bh = t % BQ;
    const int bmat = GATEUP ? bc / UPW : 2;
    const int nc = K / 32, nfull = nc >> 4;
    // the item's sources, set by setup()
    bool alive[AR];
    const uint16_t* asrc[AR];
    bool bvalid;
    uint32_t sfull, stail;
    const uint8_t* crow;
    const uint8_t* sblk;
    auto setup = [&](int it) __attribute__((always_inline)) {
      const i32x4 cd = item_desc(it);
      const int p0 = cd.y, n = cd.z, slot = cd.w;
      const bool resident = slot >= 0 && slot < a.n_slots;
      const uint8_t* blob = pool + (resident ? (uint64_t)slot * (uint64_t)a.slot_stride : 0);
      const int arow16 = (n + 15) & ~15;
#pragma unroll
      for (int h = 0; h < AR; h++) {
        alive[h] = ar[h] < arow16;
        const int p = p0 + min(ar[h], n - 1);
        const int64_t arow = GATEUP ? (int64_t)(p < a.Tk ? perm[p] / a.k : p - a.Tk) : (int64_t)p;
        asrc[h] = ain + arow * K;
      }
      const int bunit = item_u0(it) + bc % UPW;
      bvalid = resident && bunit < units;
      const int bunit_c = min(bunit, units - 1);
      // a non-resident group reads the pool's first bytes (valid memory) and
      // is zeroed through its scales
      // (blob tiling in moe_common.hpp: chunk j of the column at crow + 256 j,
      // its scales at sblk + blob_sc_off(j, nc, br))
      const int br = bunit_c & 15;
      // this row's offset in a scale group: 32 bytes per row in whole groups,
      // 2 (nc % 16) in the last one when it is shorter
      sfull = (uint32_t)br * 32u;
      stail = (uint32_t)br * 2u * (uint32_t)(nc & 15);
      crow = bvalid ? blob + a.off_codes[bmat] + (int64_t)(bunit_c >> 4) * (8 * K) + br * 16 : pool;
      sblk = bvalid ? blob + a.off_scales[bmat] + (int64_t)(bunit_c >> 4) * K : pool;
    };

    // Every load stays inside its row: the K offset is clamped to the last
    // 32 values, which only a half step beyond K (K % 64 == 32) needs; that
    // half is zeroed when staged.
    auto gload = [&](Stage& st, int s) {
      const int sc_ = min(s, a.nk - 1);
      const int ko = min(sc_ * GK + ah * 32, K - 32);
#pragma unroll
      for (int h = 0; h < AR; h++) {
        const uint4* ap = reinterpret_cast<const uint4*>(asrc[h] + ko);
#pragma unroll
        for (int i = 0; i < 4; i++) st.a[h][i] = ap[i];
      }
      // chunk j (32 values) of the column; a quarter thread takes half of it
      const int j = min(2 * sc_ + bh / (BQ / 2), nc - 1);
      const int hq = BQ == 4 ? (bh & 1) : 0;
      st.c = *reinterpret_cast<const typename Codes<BQ>::type*>(crow + (int64_t)j * 256 + 8 * hq);
      // the scale byte(s) of these values, from the aligned dword holding
      // them; the shift waits for the stage, so no wait is forced here
      // (blob_sc_off(j, nc, br) without a multiply in the loop)
      const uint32_t so =
          (uint32_t)(j >> 4) * 512u + ((j >> 4) < nfull ? sfull : stail) + 2u * (uint32_t)(j & 15) + (uint32_t)hq;
      st.sc = *reinterpret_cast<const uint32_t*>(sblk + (so & ~3u));
      st.ssh = 8u * (so & (BQ == 4 ? 3u : 2u));
    };
    auto stage = [&](const Stage& st, int buf, int s) {
      // every loaded register is read here on every path (the stores below are
      // branched): a load whose value only some paths read leaves the compiler
      // unsure it has landed, and it then waits for all loads before reusing
      // the register
#pragma unroll
      for (int h = 0; h < AR; h++)
#pragma unroll
        for (int i = 0; i < 4; i++) touch(st.a[h][i]);
      touch(st.c);
      asm volatile("" ::"v"(st.sc));
      const bool kval = s * GK + ah * 32 < K;
#pragma unroll
      for (int h = 0; h < AR; h++) {
        uint4* ad = reinterpret_cast<uint4*>(&As[buf][ar[h] * LROW + ah * 32]);
        if (alive[h]) {
#pragma unroll
          for (int i = 0; i < 4; i++) ad[i] = kval ? st.a[h][i] : make_uint4(0, 0, 0, 0);
        }
      }
      const uint32_t sw = (bvalid && s * GK + (bh / (BQ / 2)) * 32 < K) ? st.sc >> st.ssh : 0u;
      stage_b(reinterpret_cast<bf16x8*>(&Bs[buf][bc * LROW + bh * (64 / BQ)]), st.c, sw);
    };

    // half-step h loads step h + 3 into stage (h + 3) % 4 and stages step h + 1
    // (loaded two half-steps earlier) into LDS buffer (h + 1) % 2, while the
    // consumers compute step h from buffer h % 2
    // (four named stages, NST of them: an array of them is not kept in registers)
    Stage st0, st1, st2, st3;
    setup(item);
    gload(st0, 0);
    gload(st1, 1);
    gload(st2, 2);
    for (;;) {
      const i32x4 cd = item_desc(item);
      stage(st0, 0, 0);
      __syncthreads();
      for (int s = 0; s < nk4; s += 4) {
        gload(st3, s + 3);
        stage(st1, 1, s + 1);
        __syncthreads();
        gload(st0, s + 4);
        stage(st2, 0, s + 2);
        __syncthreads();
        gload(st1, s + 5);
        stage(st3, 1, s + 3);
        __syncthreads();
        gload(st2, s + 6);
        stage(st0, 0, s + 4);
        __syncthreads();
      }
      // the next item's first three steps load while the consumers finish this
      // one (after the last item they reload its own, harmlessly)
      const int nxt = item + (int)gridDim.x;
      const bool more = item_chunk(nxt) < n_chunks;
      if (more) setup(nxt);
      gload(st0, 0);
      gload(st1, 1);
      gload(st2, 2);
      copy_out(cd.y, cd.z, item_u0(item));
      if (!more) break;
      item = nxt;
    }
  } else {

  // ---------------- consumer ----------------
  for (;;) {
  const i32x4 cd = item_desc(item);
  const int p0 = cd.y, n = cd.z, slot = cd.w;
  const bool resident = slot >= 0 && slot < a.n_slots;
  const uint8_t* blob = pool + (resident ? (uint64_t)slot * (uint64_t)a.slot_stride : 0);
  // the global scales, fetched now as a vector load: it has the whole loop to
  // land (a scalar load would share the LDS wait counter)
  int zero_v;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero_v));
  const float4 gsc = *reinterpret_cast<const float4*>(blob + a.off_globals + zero_v);
  // row group wm (16-row blocks wm, wm + 4, ...) and column part ch: NCB of
  // the tile's eight 16-column blocks (gate/up: the gate blocks and the up
  // blocks of the same units)
  const int wm = wave & 3, ch = wave >> 2;
  const int r = lane & 15, q = lane >> 4;
  auto col_block = [&](int lc) {
    return GATEUP ? (lc < NCB / 2 ? ch * (NCB / 2) + lc : 4 + ch * (NCB / 2) + lc - NCB / 2) : ch * NCB + lc;
  };

  // Row block rb of this wavefront is rows 64 rb + 16 wm .. + 15: the four
  // SIMDs take turns over 16-row blocks, so a chunk of n < 256 rows leaves them
  // evenly loaded, and the blocks at or past n are skipped.  The consumer is
  // instantiated per count of live blocks (NRB), each with its own
  // accumulators, so no accumulator is merged across code paths.
  // The wavefront's eight 16-column blocks of the B tile: gate/up pairs the
  // gate block cb with the up block cb + 4 (same units).
  auto consume = [&](auto nrb_c) __attribute__((always_inline)) {
    constexpr int NRB = decltype(nrb_c)::value;
    f32x4 acc[NRB][NCB];
#pragma unroll
    for (int i = 0; i < NRB; i++)
#pragma unroll
      for (int j = 0; j < NCB; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        bf16x8 fa[NRB], fb[NCB];
#pragma unroll
        for (int rb = 0; rb < NRB; rb++)
          fa[rb] = *reinterpret_cast<const bf16x8*>(&As[buf][(64 * rb + 16 * wm + r) * LROW + 32 * ks + 8 * q]);
#pragma unroll
        for (int cb = 0; cb < NCB; cb++)
          fb[cb] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(16 * col_block(cb) + r) * LROW + 32 * ks + 8 * q]);
#pragma unroll
        for (int rb = 0; rb < NRB; rb++)
#pragma unroll
          for (int cb = 0; cb < NCB; cb++) acc[rb][cb] = mfma16x16x32(fa[rb], fb[cb], acc[rb][cb]);
      }
    };
    // one barrier per step, as the producers have
    __syncthreads();
    for (int s = 0; s < nk4; s += 2) {
      compute(0);
      __syncthreads();
      compute(1);
      __syncthreads();
    }
    // epilogue, part 1: D[i][j] of block (rb, cb) is in lane j + 16 (i / 4),
    // element i % 4, so a lane holds rows 4q .. 4q + 3 of column r.  Adjacent
    // lanes swap two of their four bf16 results (one DPP move): the even lane
    // then holds rows 4q and 4q + 2, the odd lane rows 4q + 1 and 4q + 3, each
    // as a pair of columns, written to the output tile in LDS (the A buffers,
    // free after the last step's barrier).
    const float g0 = resident ? (GATEUP ? gsc.x : gsc.z) : 0.f;
    const float g1 = (GATEUP && resident) ? gsc.y : 0.f;
    const bool odd = r & 1;
    // byte selectors over {recv: bytes 4..7, mine: bytes 0..3}, low column
    // first: the even lane's words are (mine, recv), the odd lane's (recv, mine)
    const uint32_t sel0 = odd ? 0x01000504u : 0x05040100u;  // the low halves: rows 4q / 4q + 1
    const uint32_t sel1 = odd ? 0x03020706u : 0x07060302u;  // the high halves: rows 4q + 2 / 4q + 3
#pragma unroll
    for (int rb = 0; rb < NRB; rb++) {
#pragma unroll
      for (int oc = 0; oc < OC / 16 / (NCW / 4); oc++) {
        float v[4];
#pragma unroll
        for (int e4 = 0; e4 < 4; e4++) {
          if (GATEUP) {
            // silu(g) u = g u / (1 + e^-g): v_exp_f32 and v_rcp_f32 (errors of
            // a few fp32 ulp, far below the bf16 rounding of h)
            const float gv = g0 * acc[rb][oc][e4];
            const float uv = g1 * acc[rb][oc + NCB / 2][e4];
            v[e4] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          } else {
            v[e4] = g0 * acc[rb][oc][e4];
          }
        }
        // pa: rows 4q, 4q + 2 of this lane's column; pb: rows 4q + 1, 4q + 3.
        // The lane sends its partner the pair the partner keeps (the even lane
        // keeps pa), then merges the received halves with its own: one byte
        // permute whose selector depends only on the lane's parity.
        const uint32_t pa = pack_bf16(v[0], v[2]), pb = pack_bf16(v[1], v[3]);
        const uint32_t send = odd ? pa : pb, mine = odd ? pb : pa;
        const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
        const uint32_t w0 = __builtin_amdgcn_perm(recv, mine, sel0);
        const uint32_t w1 = __builtin_amdgcn_perm(recv, mine, sel1);
        const int row = 64 * rb + 16 * wm + 4 * q + (odd ? 1 : 0);
        const int col = 16 * (ch * (OC / 16 / (NCW / 4)) + oc) + (r & ~1);
        *reinterpret_cast<uint32_t*>(&os[row * OSTR + col]) = w0;
        *reinterpret_cast<uint32_t*>(&os[(row + 2) * OSTR + col]) = w1;
      }
    }
  };
  switch (max(0, min(4, (n - 16 * wm + 63) >> 6))) {
    case 4: consume(std::integral_constant<int, 4>{}); break;
    case 3: consume(std::integral_constant<int, 3>{}); break;
    case 2: consume(std::integral_constant<int, 2>{}); break;
    case 1: consume(std::integral_constant<int, 1>{}); break;
    default:  // no live rows: the barriers only
      __syncthreads();
      for (int s = 0; s < nk4; s += 2) {
        __syncthreads();
        __syncthreads();
      }
  }
  copy_out(p0, n, item_u0(item));
  item += (int)gridDim.x;
  if (item_chunk(item) >= n_chunks) break;
  }
  }
}

}  // namespace

hipError_t launch_ffn_gemm(const moe_dims& d, const uint16_t* x, const FfnGeom& g, const int32_t* perm, uint16_t* h,
                           uint16_t* y_rows, void* ws, int n_cu, int stages, hipEvent_t ev_start, hipEvent_t ev_stop,
                           hipStream_t s) {
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  GemmArgs a;
  a.slot_stride = (uint32_t)g.slot_stride;
  a.n_slots = (int32_t)g.n_slots;
  for (int m = 0; m < 3; m++) {
    a.off_codes[m] = (uint32_t)g.off_codes[m];
    a.off_scales[m] = (uint32_t)g.off_scales[m];
  }
  a.off_globals = (uint32_t)g.off_globals;
  a.H = d.H;
  a.I = d.I;
  a.k = d.k;
  a.Tk = d.T * d.k;
  const int4* chunks = reinterpret_cast<const int4*>(base + wl.off_chunks);
  const int32_t* meta = reinterpret_cast<const int32_t*>(base + wl.off_meta);
  for (int stage = 0; stage < 2; stage++) {
    if (!((stages >> stage) & 1)) continue;
    const bool gu = stage == 0;
    const int K = gu ? d.H : d.I, units = gu ? d.I : d.H;
    const int upw = GC / (gu ? 2 : 1);
    a.n_ut = (units + upw - 1) / upw;
    a.nk = (K + GK - 1) / GK;
    // persistent: one workgroup per CU (the LDS holds one), a multiple of 8
    const int64_t items = (wl.max_chunks + 7) / 8 * 8 * a.n_ut;
    const dim3 grid((unsigned)std::min<int64_t>(items, (int64_t)(n_cu + 7) / 8 * 8));
    const dim3 block(gu ? Shape<MOE_GEMM_ROLES_GU>::GT : Shape<MOE_GEMM_ROLES_DN>::GT);
    const bool first = gu || !(stages & 1), last = !gu || !(stages & 2);
    hipEvent_t e0 = first ? ev_start : nullptr, e1 = last ? ev_stop : nullptr;
    const uint16_t* ain = gu ? x : h;
    uint16_t* out = gu ? h : y_rows;
    auto* kern = gu ? k_ffn_gemm<true, MOE_GEMM_ROLES_GU> : k_ffn_gemm<false, MOE_GEMM_ROLES_DN>;
    if (e0 || e1)
      hipExtLaunchKernelGGL(kern, grid, block, 0, s, e0, e1, 0, a, chunks, meta, perm, g.pool, ain, out);
    else
      hipLaunchKernelGGL(kern, grid, block, 0, s, a, chunks, meta, perm, g.pool, ain, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
