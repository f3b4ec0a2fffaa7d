// S4, MX variant: the grouped-GEMM expert FFN with MXFP4 weights and MXFP8
// activations on CDNA4's scaled MFMA.
//
// [FreeToken] notes that the DeepSeek-V4-Flash experts are natively MXFP4.  The
// format is read as OCP Microscaling:
//  - 32 values along K share one E8M0 scale 2^(b - 127);
//  - weight elements are E2M1 codes, with no global scale;
//  - activations meet the weights as MXFP8: E4M3 elements, shared exponent
//    floor(log2 amax) - 8, round to nearest even, saturating at 448.
// v_mfma_scale_f32_16x16x128_f8f6f4 takes both operands in these formats with
// their E8M0 scales, so nothing is dequantised: weight codes travel from HBM
// through LDS to the matrix cores exactly as stored.
//
//  - k_quant_mx: bf16 rows -> E4M3 codes and E8M0 scales (x, once per token).
//  - k_ffn_mx<GATEUP>: the same work split as the bf16 grouped GEMM: (chunk of
//    <= 256 rows of one group, 128-column tile), with the tiles of one chunk on
//    one XCD.
//    - Four producer wavefronts move each 128-value K step into one of three
//      LDS buffers, two steps ahead, with LDS DMA (global_load_lds: lane l's
//      bytes land at the wave's LDS base + size * l).  The source addresses
//      are chosen so that LDS holds the MFMA operands in lane order:
//        B   the 128 K values of a 16-column block are 1 KB of contiguous blob
//            bytes (four 32-column chunks of its 16 rows).  Lane c + 16 q holds
//            column c, K 32q .. 32q + 31: the scaled MFMA's FP4 operand.
//        A   16-row blocks of 2 KB, row r's 128 bytes at 128 r, its 16-byte
//            chunk c at slot c ^ (r & 7) (a swizzle that keeps the fragment
//            reads of 16 rows conflict-free).  One DMA instruction moves 8
//            whole rows (8 lanes each, one 128-byte line per row).  The FP8
//            operand of lane (r, q) is chunks q and 4 + q of row r.
//        scales  per step one dword per B column holding the step's four E8M0
//            bytes; the A rows' scales come every four steps, 16 bytes per
//            row, into a two-slot ring (one gathered 16-byte load per row
//            instead of four 4-byte ones).  Lane (r, q) shifts byte q of its
//            dword down (the MFMA reads byte 0).
//    - Four consumer wavefronts read fragments (64 lanes x 16 contiguous bytes,
//      conflict-free): a step's eight B fragments first, then row block by row
//      block its A fragment, and issue two scaled MFMAs per (16-row block,
//      16-column block) per step: the instruction truncates small products
//      inside each run of 8 (split_e4m3), so the A codes are cut into those of
//      magnitude >= 2 and the rest and each part is summed whole.  g, u and
//      the down projection are then the exact sums up to fp32 addition, as the
//      roundings that follow (h to bf16 and MXFP8, Y to bf16) require.
//  - Gate/up epilogue: h = bf16(silu(g) u), as in the bf16 path, and h quantised
//    to MXFP8.  A 32-unit block of one row lies in two 16-column blocks of one
//    16-lane row, so its amax is an in-lane max plus four DPP max steps.  It
//    writes h (bf16), its codes and its scales.
//  - Down epilogue: Y = bf16(acc).
#include <hip/hip_ext.h>
#include <math.h>

#include <type_traits>

#include "moe_common.hpp"
#include "mx_quant.hpp"

namespace moe {
namespace {

constexpr int XM = kChunkRows;  // rows per workgroup
constexpr int XC = 128;         // output columns per workgroup
constexpr int XK = 128;         // K per step: one scaled MFMA
constexpr int XT = 512;         // 4 consumer + 4 producer wavefronts
constexpr int NBUF = 3;
// one LDS buffer
constexpr int A_OFF = 0;                       // FP8 A, operand order: 16 row blocks x 2 KB
constexpr int B_OFF = A_OFF + XM * XK;         // FP4 B, operand order: 8 column blocks x 1 KB
constexpr int BS_OFF = B_OFF + XC * XK / 2;    // B scales: a dword per column
constexpr int BUF_BYTES = BS_OFF + XC * 4;     // 41472
// A scales of four steps: [row][4 dwords], two slots
constexpr int ASG_OFF = NBUF * BUF_BYTES;
constexpr int ASG_SLOT = XM * 16;
constexpr int LDS_BYTES = ASG_OFF + 2 * ASG_SLOT;  // 132608
// epilogue tiles (in the buffers, free after the last step)
constexpr int QSTR = 80;  // bytes per row of the code tile: rows 4 apart land 16 banks apart

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <typename T>
using cptr = const __attribute__((address_space(4))) T*;

struct MxArgs {
  uint32_t slot_stride;
  int32_t n_slots;
  uint32_t off_codes[3];
  uint32_t off_scales[3];
  int32_t H, I, k, Tk;  // Tk = T * k: routed rows; rows from Tk on are the shared group's
  int32_t n_ut;         // column tiles per chunk
  int32_t nk;           // K steps
  int32_t as_stride;    // bytes per row of the A scales (a multiple of 16)
  int32_t hs_stride;    // bytes per row of the h scales written by gate/up
};

// One LDS DMA instruction: lane l's 16 (4) bytes at src land at LDS byte
// lds + 16 l (4 l).  Opaque to the compiler, which would otherwise treat every
// later LDS access as possibly aliasing it and wait for all loads in flight;
// the producers wait for it explicitly (wait_vm) before the barrier that
// precedes its use.  It counts in vmcnt, which the compiler does not see, so
// the compiler's own waits only get more conservative.
__device__ inline void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
__device__ inline void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding)
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// max over the 16 lanes of a DPP row (lanes 16 q .. 16 q + 15)
__device__ inline float row16_max(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));   // quad [1,0,3,2]
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));   // quad [2,3,0,1]
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x140, 0xF, 0xF, false)));  // row_mirror
  return m;
}

// Two floats as a bf16 pair (round to nearest even), lo in the low half.
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float bf16_round(float v) { return (float)(__bf16)v; }

// x [rows][K] bf16 -> codes [rows][K] E4M3 and scales [rows][stride] E8M0
// (K/32 of them per row).  Thread t takes 8 consecutive values (tpr = K/8
// threads per row); the four threads of a 32-value block are one DPP quad
// (K % 32 == 0, so quads never straddle rows).
__global__ __launch_bounds__(256) void k_quant_mx(const uint16_t* __restrict__ x, int64_t n8, int32_t tpr,
                                                  int32_t stride, uint8_t* __restrict__ q,
                                                  uint8_t* __restrict__ sc) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;  // whole quads leave together (n8 % 4 == 0)
  const uint4 w = reinterpret_cast<const uint4*>(x)[t];
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
  const uint2 out = make_uint2(e4m3_pair(f[0], f[1], sb) | (e4m3_pair(f[2], f[3], sb) << 16),
                               e4m3_pair(f[4], f[5], sb) | (e4m3_pair(f[6], f[7], sb) << 16));
  reinterpret_cast<uint2*>(q)[t] = out;
  if ((t & 3) == 0) sc[(t / tpr) * stride + (t % tpr) / 4] = (uint8_t)sb;
}

// The same quantisation, written back as the bf16 values it stands for
// (mx_quant8_bf16).
__global__ __launch_bounds__(256) void k_quant_mx_bf16(const uint16_t* __restrict__ x, int64_t n8,
                                                       uint16_t* __restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;  // whole quads leave together (n8 % 4 == 0)
  reinterpret_cast<uint4*>(y)[t] = mx_quant8_bf16(reinterpret_cast<const uint4*>(x)[t]);
}

template <bool GATEUP>
__global__ __launch_bounds__(XT) void k_ffn_mx(MxArgs a, const int4* __restrict__ chunks,
                                               const int32_t* __restrict__ meta, const int32_t* __restrict__ perm,
                                               const uint8_t* __restrict__ pool, const uint8_t* __restrict__ aq,
                                               const uint8_t* __restrict__ as, uint16_t* __restrict__ out,
                                               uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  constexpr int UPW = GATEUP ? XC / 2 : XC;  // units per work item
  constexpr int OC = GATEUP ? XC / 2 : XC;   // output columns of the tile
  constexpr int OSTR = OC + 8;               // uint16 per row of the h / Y tile
  // the epilogue's tiles sit in buffers 1 and 2, so that the next item's
  // first step can land in buffer 0 meanwhile
  static_assert(XM * OSTR * 2 + (GATEUP ? XM * QSTR + XM * 2 : 0) <= 2 * BUF_BYTES, "epilogue tiles fit");
  const int K = GATEUP ? a.H : a.I;
  const int units = GATEUP ? a.I : a.H;

  __shared__ __align__(16) uint8_t smem[LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  uint16_t* os = reinterpret_cast<uint16_t*>(smem + BUF_BYTES);
  uint8_t* qs = smem + BUF_BYTES + XM * OSTR * 2;  // gate/up: code tile [XM][QSTR]
  uint8_t* ss = qs + XM * QSTR;                    // gate/up: scale tile [XM][2]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;

  // Persistent: workgroup w takes work items w, w + P, w + 2 P, ... (P, the
  // grid, a multiple of 8).  Item i is column tile (i >> 3) % n_ut of chunk
  // ((i >> 3) / n_ut) * 8 + i % 8: workgroups are dealt to the XCDs round-
  // robin, so item i runs on XCD i % 8 and the tiles of one chunk run at once
  // on one XCD, sharing its A rows in that XCD's L2.  Chunks grow with i, so a
  // workgroup's first inactive item ends its walk.
  const int n_chunks = *(cptr<int32_t>)(meta + 1);
  const int P = gridDim.x;
  auto item_chunk = [&](int i) { return ((i >> 3) / a.n_ut) * 8 + (i & 7); };
  struct ItemInfo {
    int p0, n, u0;
    bool resident;
    const uint8_t* blob;
  };
  // a non-resident group reads the pool's first bytes (valid memory); its
  // outputs are zero (selected, so no scale byte read there matters)
  auto info = [&](int i) __attribute__((always_inline)) {
    const i32x4 cd = ((cptr<i32x4>)chunks)[item_chunk(i)];
    ItemInfo it;
    it.p0 = cd.y;
    it.n = cd.z;
    it.resident = cd.w >= 0 && cd.w < a.n_slots;
    it.blob = pool + (it.resident ? (uint64_t)cd.w * (uint64_t)a.slot_stride : 0);
    it.u0 = ((i >> 3) % a.n_ut) * UPW;
    return it;
  };
  // epilogue, part 2 (all eight wavefronts): the tiles leave in 16-byte row
  // segments
  auto copy_out = [&](const ItemInfo& it) __attribute__((always_inline)) {
    constexpr int SEGS = OC / 8;
#pragma unroll 4
    for (int i = tid; i < it.n * SEGS; i += XT) {
      const int row = i / SEGS, sg = i % SEGS;
      *reinterpret_cast<uint4*>(out + (int64_t)(it.p0 + row) * units + it.u0 + 8 * sg) =
          *reinterpret_cast<const uint4*>(&os[row * OSTR + 8 * sg]);
    }
    if (GATEUP) {
      for (int i = tid; i < it.n * 4; i += XT) {
        const int row = i >> 2, sg = i & 3;
        *reinterpret_cast<uint4*>(hq + (int64_t)(it.p0 + row) * units + it.u0 + 16 * sg) =
            *reinterpret_cast<const uint4*>(&qs[row * QSTR + 16 * sg]);
      }
      for (int row = tid; row < it.n; row += XT)
        *reinterpret_cast<uint16_t*>(hs + (int64_t)(it.p0 + row) * a.hs_stride + it.u0 / 32) =
            *reinterpret_cast<const uint16_t*>(&ss[row * 2]);
    }
  };

  int item = blockIdx.x;
  if (item_chunk(item) >= n_chunks) return;

  if (wave >= 4) {
    // ---------------- producer ----------------
    const int pw = wave - 4;
    // this wavefront's source addresses for one item; A rows past n load row
    // n - 1 (their outputs are dropped)
    struct PAddr {
      const uint8_t* asrc[4];
      const uint8_t* asrc2[4];
      const uint8_t* ssrc;
      const uint8_t* bsrc[2];
      const uint8_t* bssrc;
      int na;  // live A blocks of this wavefront: pw + 4 i, i < na
    };
    auto paddr = [&](const ItemInfo& it) __attribute__((always_inline)) {
      PAddr pa;
      auto arow = [&](int row) -> int64_t {
        const int p = it.p0 + min(row, it.n - 1);
        return GATEUP ? (int64_t)(p < a.Tk ? perm[p] / a.k : p - a.Tk) : (int64_t)p;
      };
      // lane l of the block's half hf moves row 8 hf + l / 8, slot l % 8
      // (chunk (l % 8) ^ (row & 7)); asrc[i] is the lane's row of half 0,
      // asrc2[i] of half 1
      const int sl = lane & 7, rr = lane >> 3;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        pa.asrc[i] = aq + arow(16 * (pw + 4 * i) + rr) * K + 16 * (sl ^ rr);
        pa.asrc2[i] = aq + arow(16 * (pw + 4 * i) + 8 + rr) * K + 16 * (sl ^ rr);  // (8 + rr) & 7 == rr
      }
      pa.ssrc = as + arow(64 * pw + lane) * a.as_stride;
      // B: column blocks 2 pw and 2 pw + 1 (gate/up: blocks 0..3 gate, 4..7
      // up, the same units)
      auto bunit = [&](int cb) { return it.u0 + 16 * (GATEUP ? (cb & 3) : cb); };
      auto bmat = [&](int cb) { return GATEUP ? (cb >> 2) : 2; };
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int cb = 2 * pw + j;
        pa.bsrc[j] =
            (it.resident ? it.blob + a.off_codes[bmat(cb)] + (int64_t)(bunit(cb) >> 4) * (8 * K) : pool) + 16 * lane;
      }
      // B scales (wavefronts 0 and 1): column 64 pw + lane
      const int scol = (64 * pw + lane) & (XC - 1), scb = scol >> 4;
      pa.bssrc = (it.resident ? it.blob + a.off_scales[bmat(scb)] + (int64_t)(bunit(scb) >> 4) * (K / 2) : pool) +
                 4 * (scol & 15);
      pa.na = max(0, min(4, (((it.n + 15) >> 4) - pw + 3) >> 2));
      return pa;
    };
    // the DMA instructions of step s into buffer bi: 2 na (A) + 2 (B) + 1
    // (B scales, wavefronts 0 and 1) + 1 every fourth step (A scales)
    auto issue = [&](const PAddr& pa, int s, int bi) __attribute__((always_inline)) {
      const uint32_t buf = lds0 + (uint32_t)(bi * BUF_BYTES);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (i < pa.na) {
          const uint32_t d = buf + A_OFF + (uint32_t)(pw + 4 * i) * 2048u;
          dma16(pa.asrc[i] + XK * s, __builtin_amdgcn_readfirstlane(d));
          dma16(pa.asrc2[i] + XK * s, __builtin_amdgcn_readfirstlane(d + 1024u));
        }
      }
#pragma unroll
      for (int j = 0; j < 2; j++)
        dma16(pa.bsrc[j] + 1024 * s, __builtin_amdgcn_readfirstlane(buf + B_OFF + (uint32_t)(2 * pw + j) * 1024u));
      if (pw < 2) dma4(pa.bssrc + 64 * s, __builtin_amdgcn_readfirstlane(buf + BS_OFF + 256u * (uint32_t)pw));
      if ((s & 3) == 0)  // the A scales of steps s .. s + 3 (the row's 16 bytes from 4 s)
        dma16(pa.ssrc + 4 * s, __builtin_amdgcn_readfirstlane(lds0 + ASG_OFF + (uint32_t)(((s >> 2) & 1) * ASG_SLOT) +
                                                             1024u * (uint32_t)pw));
    };

    ItemInfo cur = info(item);
    PAddr pa = paddr(cur);
    bool pre0 = false;  // step 0 of the current item already issued
    for (;;) {
      auto run = [&](auto na_c) __attribute__((always_inline)) {
        constexpr int NA = decltype(na_c)::value;
        constexpr int N = 2 * NA + 2;
        // the step before step s has landed once at most step s's
        // instructions (and none older) are in flight
        auto wait_next = [&](int s) __attribute__((always_inline)) {
          const bool g = (s & 3) == 0;
          if (pw < 2) {
            if (g) wait_vm<N + 2>();
            else wait_vm<N + 1>();
          } else {
            if (g) wait_vm<N + 1>();
            else wait_vm<N>();
          }
        };
        if (!pre0) issue(pa, 0, 0);
        if (a.nk > 1) {
          issue(pa, 1, 1);
          wait_next(1);
        } else {
          wait_vm<0>();
        }
        __syncthreads();
        int bi = 2;  // buffer of step s + 2
        for (int s = 0; s < a.nk; s++) {
          // buffer (s + 2) % 3 was last read in step s - 1, which every
          // consumer finished before the barrier just passed; so was the
          // A-scale slot of step s + 2 (last read in step s - 6)
          if (s + 2 < a.nk) {
            issue(pa, s + 2, bi);
            bi = bi == 2 ? 0 : bi + 1;
            wait_next(s + 2);
          } else {
            wait_vm<0>();
          }
          __syncthreads();
        }
      };
      switch (pa.na) {
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        default: run(std::integral_constant<int, 0>{}); break;
      }
      // every consumer is past the last step: buffer 0 and both A-scale slots
      // are free, so the next item's first step goes out now, while the
      // consumers run the epilogue in buffers 1 and 2
      const int nxt = item + P;
      const bool more = item_chunk(nxt) < n_chunks;
      const ItemInfo done = cur;
      if (more) {
        cur = info(nxt);
        pa = paddr(cur);
        issue(pa, 0, 0);
        pre0 = true;
      }
      __syncthreads();
      copy_out(done);
      __syncthreads();
      if (!more) break;
      item = nxt;
    }
  } else {
    // ---------------- consumer ----------------
    const int wm = wave;
    for (;;) {
      const ItemInfo it = info(item);
      const int nb = (it.n + 15) >> 4;  // live 16-row blocks; block rbk belongs to wavefront pair rbk % 4

      // Row block rb of this wavefront is block 4 rb + wm (rows 64 rb + 16 wm
      // .. + 15); the consumer is instantiated per count of live blocks (NRB).
      auto consume = [&](auto nrb_c) __attribute__((always_inline)) {
        constexpr int NRB = decltype(nrb_c)::value;
        f32x4 acc[NRB][8];
#pragma unroll
        for (int i = 0; i < NRB; i++)
#pragma unroll
          for (int j = 0; j < 8; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
        int bi = 0;
        for (int s = 0; s < a.nk; s++) {
          const uint8_t* bb = smem + bi * BUF_BYTES;
          i32x8 fb[8];
          int sb[8];
#pragma unroll
          for (int cb = 0; cb < 8; cb++) {
            const i32x4 f = *reinterpret_cast<const i32x4*>(bb + B_OFF + cb * 1024 + 16 * lane);
            fb[cb] = i32x8{f.x, f.y, f.z, f.w, 0, 0, 0, 0};
            sb[cb] = (int)(*reinterpret_cast<const uint32_t*>(bb + BS_OFF + (16 * cb + r) * 4) >> (8 * q));
          }
#pragma unroll
          for (int rb = 0; rb < NRB; rb++) {
            const int rbk = 4 * rb + wm;
            const uint8_t* rowp = bb + A_OFF + rbk * 2048 + 128 * r;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(rowp + 16 * (q ^ (r & 7)));
            const i32x4 hi = *reinterpret_cast<const i32x4*>(rowp + 16 * ((4 + q) ^ (r & 7)));
            const i32x8 fa = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const int sa = (int)(*reinterpret_cast<const uint32_t*>(smem + ASG_OFF + ((s >> 2) & 1) * ASG_SLOT +
                                                                   (16 * rbk + r) * 16 + 4 * (s & 3)) >> (8 * q));
            // both products feed a rounding that the oracle takes on the exact
            // sum (h: bf16 then MXFP8; Y: bf16), so each is summed whole: two
            // MFMAs, the big and the small codes of A
            i32x8 big, small;
            split_e4m3(fa, big, small);
#pragma unroll
            for (int cb = 0; cb < 8; cb++)
              acc[rb][cb] =
                  __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(big, fb[cb], acc[rb][cb], 0, 4, 0, sa, 0, sb[cb]);
#pragma unroll
            for (int cb = 0; cb < 8; cb++)
              acc[rb][cb] =
                  __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(small, fb[cb], acc[rb][cb], 0, 4, 0, sa, 0, sb[cb]);
          }
          // a wavefront issues in order, so the split of row block rb + 1 would
          // leave the matrix core idle if it ran as one block between the MFMAs
          // of rb and rb + 1: interleave up to four VALU instructions after each
          // MFMA instead
#pragma unroll
          for (int i = 0; i < NRB * 16; i++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to four VALU
          }
          bi = bi == 2 ? 0 : bi + 1;
          __syncthreads();
        }
        // epilogue, part 1: D[i][j] of block (rb, cb) is in lane j + 16 (i / 4),
        // element i % 4: a lane holds rows 4q .. 4q + 3 of column r.  The bf16
        // results leave through the tile in LDS as in the bf16 GEMM: adjacent
        // lanes swap half their pairs (one DPP move) and write column pairs.
        const bool odd = r & 1;
        const uint32_t sel0 = odd ? 0x01000504u : 0x05040100u;
        const uint32_t sel1 = odd ? 0x03020706u : 0x07060302u;
#pragma unroll
        for (int rb = 0; rb < NRB; rb++) {
          const int row0 = 16 * (4 * rb + wm) + 4 * q;
          float v[OC / 16][4];
#pragma unroll
          for (int oc = 0; oc < OC / 16; oc++)
#pragma unroll
            for (int e4 = 0; e4 < 4; e4++) {
              float t;
              if (GATEUP) {
                const float gv = acc[rb][oc][e4], uv = acc[rb][oc + 4][e4];
                t = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
              } else {
                t = acc[rb][oc][e4];
              }
              v[oc][e4] = bf16_round(it.resident ? t : 0.f);
            }
#pragma unroll
          for (int oc = 0; oc < OC / 16; oc++) {
            const uint32_t pa = pack_bf16(v[oc][0], v[oc][2]), pb = pack_bf16(v[oc][1], v[oc][3]);
            const uint32_t send = odd ? pa : pb, mine = odd ? pb : pa;
            const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);
            const int row = row0 + (odd ? 1 : 0);
            const int col = 16 * oc + (r & ~1);
            *reinterpret_cast<uint32_t*>(&os[row * OSTR + col]) = __builtin_amdgcn_perm(recv, mine, sel0);
            *reinterpret_cast<uint32_t*>(&os[(row + 2) * OSTR + col]) = __builtin_amdgcn_perm(recv, mine, sel1);
          }
          if (GATEUP) {
            // h at the MXFP8 rounding point: the 32-unit block p of row row0 +
            // e4 is column blocks 2p, 2p + 1 of the 16 lanes of this lane row
#pragma unroll
            for (int e4 = 0; e4 < 4; e4++)
#pragma unroll
              for (int p = 0; p < 2; p++) {
                const float m = row16_max(fmaxf(fabsf(v[2 * p][e4]), fabsf(v[2 * p + 1][e4])));
                const int sb = e8m0_of_amax(m);
                const int row = row0 + e4;
                const uint32_t c2 = e4m3_pair(v[2 * p][e4], v[2 * p + 1][e4], sb);
                qs[row * QSTR + 32 * p + r] = (uint8_t)c2;
                qs[row * QSTR + 32 * p + 16 + r] = (uint8_t)(c2 >> 8);
                if (r == 0) ss[row * 2 + p] = (uint8_t)sb;
              }
          }
        }
      };
      switch (max(0, min(4, (nb - wm + 3) >> 2))) {
        case 4: consume(std::integral_constant<int, 4>{}); break;
        case 3: consume(std::integral_constant<int, 3>{}); break;
        case 2: consume(std::integral_constant<int, 2>{}); break;
        case 1: consume(std::integral_constant<int, 1>{}); break;
        default:  // no live rows: the barriers only
          __syncthreads();
          for (int s = 0; s < a.nk; s++) __syncthreads();
      }
      __syncthreads();
      copy_out(it);
      __syncthreads();
      item += P;
      if (item_chunk(item) >= n_chunks) break;
    }
  }
}

}  // namespace

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                           int32_t scale_stride, hipEvent_t ev_start, hipStream_t s) {
  const int64_t n8 = rows * (K / 8);
  if (n8 == 0) return hipSuccess;
  const dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  const int32_t tpr = K / 8;
  if (ev_start)
    hipExtLaunchKernelGGL(k_quant_mx, grid, block, 0, s, ev_start, nullptr, 0, x, n8, tpr, scale_stride, codes, scales);
  else
    hipLaunchKernelGGL(k_quant_mx, grid, block, 0, s, x, n8, tpr, scale_stride, codes, scales);
  return hipGetLastError();
}

hipError_t launch_ffn_dec_mx(const moe_dims& d, const uint16_t* x, const FfnGeom& g, const int32_t* perm, uint16_t* h,
                             uint16_t* y_rows, void* ws, void* mx_ws, int n_cu, int stages, hipEvent_t ev_start,
                             hipEvent_t ev_stop, hipStream_t s, bool x_ready) {
  const MxWsLayout ml = mx_ws_layout(d);
  uint16_t* xb = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(mx_ws) + ml.off_xb);
  uint16_t* hb = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(mx_ws) + ml.off_hb);
  for (int stage = 0; stage < 2; stage++) {
    if (!((stages >> stage) & 1)) continue;
    const bool gu = stage == 0;
    const bool first = gu || !(stages & 1), last = !gu || !(stages & 2);
    // the quantisation first, then the FFN kernel, which the events bracket
    // (x_ready: the route + group launch already wrote x's into the workspace)
    const int64_t rows = gu ? d.T : (int64_t)d.T * d.k + d.T;
    const int64_t n8 = rows * ((gu ? d.H : d.I) / 8);
    if (n8 > 0 && !(gu && x_ready))
      hipLaunchKernelGGL(k_quant_mx_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, gu ? x : h, n8,
                         gu ? xb : hb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_ffn_dec(d, xb, g, perm, h, y_rows, ws, n_cu, gu ? 1 : 2, first ? ev_start : nullptr,
                       last ? ev_stop : nullptr, s, true, hb);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_ffn_mx(const moe_dims& d, const uint16_t* x, const FfnGeom& g, const int32_t* perm, uint16_t* h,
                         uint16_t* y_rows, void* ws, void* mx_ws, int n_cu, int stages, hipEvent_t ev_start,
                         hipEvent_t ev_stop, hipStream_t s) {
  const WsLayout wl = ws_layout(d);
  const MxWsLayout ml = mx_ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* mb = static_cast<uint8_t*>(mx_ws);
  MxArgs a;
  a.slot_stride = (uint32_t)g.slot_stride;
  a.n_slots = (int32_t)g.n_slots;
  for (int m = 0; m < 3; m++) {
    a.off_codes[m] = (uint32_t)g.off_codes[m];
    a.off_scales[m] = (uint32_t)g.off_scales[m];
  }
  a.H = d.H;
  a.I = d.I;
  a.k = d.k;
  a.Tk = d.T * d.k;
  const int4* chunks = reinterpret_cast<const int4*>(base + wl.off_chunks);
  const int32_t* meta = reinterpret_cast<const int32_t*>(base + wl.off_meta);
  uint8_t *xq = mb + ml.off_xq, *xs = mb + ml.off_xs, *hq = mb + ml.off_hq, *hs = mb + ml.off_hs;
  for (int stage = 0; stage < 2; stage++) {
    if (!((stages >> stage) & 1)) continue;
    const bool gu = stage == 0;
    const bool first = gu || !(stages & 1), last = !gu || !(stages & 2);
    hipEvent_t e0 = first ? ev_start : nullptr, e1 = last ? ev_stop : nullptr;
    if (gu) {  // the events bracket the GEMMs alone
      const hipError_t e = launch_quant_mx(x, d.T, d.H, xq, xs, ml.xs_stride, nullptr, s);
      if (e != hipSuccess) return e;
    }
    const int K = gu ? d.H : d.I, units = gu ? d.I : d.H;
    a.n_ut = units / (gu ? XC / 2 : XC);
    a.nk = K / XK;
    a.as_stride = gu ? ml.xs_stride : ml.hs_stride;
    a.hs_stride = ml.hs_stride;
    // persistent grid: one workgroup per CU (a multiple of 8), at most one per item
    const int64_t items = (wl.max_chunks + 7) / 8 * 8 * a.n_ut;
    const int64_t cap = ((int64_t)n_cu + 7) / 8 * 8;
    const dim3 grid((unsigned)(items < cap ? items : cap)), block(XT);
    const uint8_t* aq = gu ? xq : hq;
    const uint8_t* as = gu ? xs : hs;
    uint16_t* out = gu ? h : y_rows;
    if (e0 || e1) {
      if (gu)
        hipExtLaunchKernelGGL(k_ffn_mx<true>, grid, block, 0, s, e0, e1, 0, a, chunks, meta, perm, g.pool, aq, as,
                              out, hq, hs);
      else
        hipExtLaunchKernelGGL(k_ffn_mx<false>, grid, block, 0, s, e0, e1, 0, a, chunks, meta, perm, g.pool, aq, as,
                              out, (uint8_t*)nullptr, (uint8_t*)nullptr);
    } else {
      if (gu)
        hipLaunchKernelGGL(k_ffn_mx<true>, grid, block, 0, s, a, chunks, meta, perm, g.pool, aq, as, out, hq, hs);
      else
        hipLaunchKernelGGL(k_ffn_mx<false>, grid, block, 0, s, a, chunks, meta, perm, g.pool, aq, as, out,
                           (uint8_t*)nullptr, (uint8_t*)nullptr);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
