// S3: grouping of (token, slot) rows by expert through the slot table.
//
// [Strata] "路由以后，专家怎样分工？": within one layer and window, the tokens that
// picked the same expert form one group that records their inputs and output
// positions, so the expert's weights are read once for the whole group.
// [Strata] "哪些专家能长期留在显存？": the residency table maps (layer, expert) to a
// slot, or to a special not-resident value.  [FreeToken] 4: the logical ->
// physical rewrite stays on the device, with fixed launch shapes and
// device-side counts, so no host synchronisation is needed.
//
// Up to 256 (token, slot) entries (decode): one fused single-block kernel.
// Otherwise a stable counting sort in three fixed-shape kernels:
//   count   per kCntBlk-entry block, LDS histogram of expert ids (order-free atomics)
//   scan    one block: per-expert prefix over blocks, exclusive scan over experts,
//           slot rewrite, and the FFN work list
//   scatter per 256-entry block: an entry's row is its group's first row, plus
//           the entries of its expert in earlier counting blocks (the scan),
//           in earlier 256-entry parts of its own counting block (an LDS
//           histogram) and earlier in its own part (counted over the ids
//           staged in LDS), so a row depends only on the ids (deterministic).
#include "moe_common.hpp"
#include "mx_quant.hpp"
#include "route_small.hpp"
#include "topk_wave.hpp"

#include <type_traits>

namespace moe {
#ifdef MOE_STAGE_TIMING
STAGE_TIMES_DEFINE(moe_debug_stage_times_group)
#endif
namespace {

constexpr int kBlk = 256;

constexpr int kParts = kCntBlk / kBlk;  // 256-entry parts per counting block

// With the tail-skip rule (skip_rank > 0) also each expert's lowest slot rank
// in the block, into mrk [ncb][E] (k where the block has none).
__global__ __launch_bounds__(kBlk) void k_count(const int32_t* __restrict__ ids, int64_t F, int E, int k,
                                                int skip_rank, int32_t* __restrict__ cnt, int32_t* __restrict__ mrk,
                                                int32_t* __restrict__ status) {
  __shared__ int32_t hist[1024];
  __shared__ int32_t mr[1024];
  int ev[kParts];
#pragma unroll
  for (int j = 0; j < kParts; j++) {
    const int64_t f = (int64_t)blockIdx.x * kCntBlk + j * kBlk + threadIdx.x;
    ev[j] = f < F ? ids[f] : 0;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    hist[e] = 0;
    mr[e] = k;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kParts; j++) {
    const int64_t f = (int64_t)blockIdx.x * kCntBlk + j * kBlk + threadIdx.x;
    if (f < F) {
      if (ev[j] >= 0 && ev[j] < E) {
        atomicAdd(&hist[ev[j]], 1);
        if (skip_rank > 0) atomicMin(&mr[ev[j]], (int)(f % k));
      } else {
        atomicOr(status, MOE_DEV_BAD_EXPERT_ID);
      }
    }
  }
  __syncthreads();
  if (skip_rank > 0)
    for (int e = threadIdx.x; e < E; e += blockDim.x) mrk[(int64_t)blockIdx.x * E + e] = mr[e];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Thread e (< E) holds count = rows of expert e.  Writes offsets, group_slot,
// residency status and the FFN work list (the tile lists, or with `chunks`
// the chunk list); returns this expert's first row.
// `slot` is slot_table[layer][e] for thread e < E and `ss` the shared expert's
// slot; the caller loads both at its start, so their latency overlaps its own.
// `chunks` (or null): the grouped-GEMM work list, written in place of the
// tile lists when the FFN will run as a GEMM; *tbase_out is then not set.
// Tail-skip (skip_rank > 0): thread e's expert, when it is not resident and
// minrank (its lowest slot rank in the window) is skip_rank or more, is
// skipped: its rows are zero like any non-resident group's, it sets
// MOE_DEV_TAIL_SKIPPED instead of MOE_DEV_NOT_RESIDENT, and *n_skipped (if
// set) receives the number of skipped experts.
__device__ int scan_and_tiles(int count, int T, int k, int E, int slot, int ss, int32_t n_slots,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ group_slot,
                              int32_t* __restrict__ status, int32_t* __restrict__ meta, int4* __restrict__ tiles,
                              int32_t* __restrict__ tile_tok, int32_t* __restrict__ tile_base, int4* __restrict__ chunks,
                              int* lds17, int* tbase_out = nullptr, int minrank = 0, int skip_rank = 0,
                              int32_t* __restrict__ n_skipped = nullptr) {
  const int e = threadIdx.x;
  int total = 0;
  const int off = block_exclusive_scan(count, lds17, &total);
  const int64_t Tk = (int64_t)T * k;
  const bool skipped = skip_rank > 0 && e < E && count > 0 && slot < 0 && minrank >= skip_rank;
  if (e < E) {
    offsets[e] = off;
    group_slot[e] = slot;
    if (count > 0 && slot < 0) atomicOr(status, skipped ? MOE_DEV_TAIL_SKIPPED : MOE_DEV_NOT_RESIDENT);
    if (count > 0 && slot >= n_slots) atomicOr(status, MOE_DEV_BAD_SLOT);
  }
  if (n_skipped) {  // uniform: every thread of the block takes this branch or none does
    int ns = 0;
    block_exclusive_scan(skipped ? 1 : 0, lds17, &ns);
    if (threadIdx.x == 0) *n_skipped = ns;
  }
  if (e == 0) {
    offsets[E] = total;
    offsets[E + 1] = (int32_t)(Tk + T);
    group_slot[E] = ss;
    if (ss < 0) atomicOr(status, MOE_DEV_NOT_RESIDENT);
    if (ss >= n_slots) atomicOr(status, MOE_DEV_BAD_SLOT);
  }
  if (!chunks) {  // uniform: every thread of the block takes this branch or none does
    // FFN tiles of kTileRows rows: routed groups in expert order, then the shared group
    const int nt = (count + kTileRows - 1) / kTileRows;
    int nt_total = 0;
    const int tbase = block_exclusive_scan(nt, lds17, &nt_total);
    if (e < E) tile_base[e] = tbase;
    if (tbase_out) *tbase_out = tbase;
    for (int i = 0; i < nt; i++) {
      const int n = min(kTileRows, count - i * kTileRows);
      tiles[tbase + i] = make_int4(e, off + i * kTileRows, n, slot);
    }
    const int nts = (T + kTileRows - 1) / kTileRows;
    for (int i = threadIdx.x; i < nts; i += blockDim.x)
      tiles[nt_total + i] =
          make_int4(E, (int32_t)(Tk + (int64_t)i * kTileRows), min(kTileRows, T - i * kTileRows), ss);
    for (int i = threadIdx.x; i < nts * kTileRows; i += blockDim.x) {  // shared rows: token = row - T*k
      const int tl = i / kTileRows, r = i % kTileRows;
      const int n = min(kTileRows, T - tl * kTileRows);
      tile_tok[(int64_t)(nt_total + tl) * kTileRows + r] = tl * kTileRows + (r < n ? r : 0);
    }
    if (threadIdx.x == 0) meta[0] = nt_total + nts;
  } else {
    // grouped-GEMM chunks of kChunkRows rows, in the same order
    const int nck = (count + kChunkRows - 1) / kChunkRows;
    int nck_total = 0;
    const int cbase = block_exclusive_scan(nck, lds17, &nck_total);
    for (int i = 0; i < nck; i++)
      chunks[cbase + i] = make_int4(e, off + i * kChunkRows, min(kChunkRows, count - i * kChunkRows), slot);
    const int ncs = (T + kChunkRows - 1) / kChunkRows;
    for (int i = threadIdx.x; i < ncs; i += blockDim.x)
      chunks[nck_total + i] =
          make_int4(E, (int32_t)(Tk + (int64_t)i * kChunkRows), min(kChunkRows, T - i * kChunkRows), ss);
    if (threadIdx.x == 0) meta[1] = nck_total + ncs;
  }
  return off;
}

// One block over the ncb x E counts.  V adjacent experts per thread (V = 4
// when E % 4 == 0: one int4 per row of counts), EV = E2 / V expert groups
// (E2 = E rounded up to a power of two) and P = 1024 / EV parts: thread
// (eq = tid % EV, part = tid / EV) owns rows [part nbp, part nbp + nbp) of
// experts eq V .. eq V + V - 1.  Rows go in batches of kBatch loads; the first
// batch stays in registers for the second pass, so a part of at most kBatch
// rows is read once.
template <int V>
__global__ __launch_bounds__(1024) void k_scan(int64_t ncb, int T, int k, int E, int layer,
                                               const int32_t* __restrict__ slot_table, int32_t n_slots,
                                               int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ group_slot, int32_t* __restrict__ status,
                                               int32_t* __restrict__ meta, int4* __restrict__ tiles,
                                               int32_t* __restrict__ tile_tok, int32_t* __restrict__ tile_base,
                                               int4* __restrict__ chunks, int skip_rank,
                                               const int32_t* __restrict__ mrk, int32_t* __restrict__ n_skipped,
                                               int32_t* __restrict__ sync, int64_t n_sync) {
  using vec = typename std::conditional<V == 4, int4, int>::type;
  zero_sync(sync, n_sync);
  constexpr int kBatch = 16;
  __shared__ int lds[17];
  __shared__ int32_t part_sum[1024 * V];  // [part][eq][V] = [part][expert]
  const int tid = threadIdx.x;
  const int E2 = E <= 1 ? 1 : 1 << (32 - __builtin_clz(E - 1));
  const int EV = E2 / V > 0 ? E2 / V : 1;
  const int P = 1024 / EV;
  const int eq = tid % EV, part = tid / EV;
  const int64_t nbp = (ncb + P - 1) / P;
  const int64_t b0 = min<int64_t>(ncb, part * nbp), b1 = min<int64_t>(ncb, b0 + nbp);
  const int slot = tid < E ? slot_table[(int64_t)layer * (E + 1) + tid] : -1;
  const int ss = slot_table[(int64_t)layer * (E + 1) + E];
  // with V = 4, E % 4 == 0: a live group has all four experts
  const int64_t nrow = eq * V < E ? b1 - b0 : 0;
  vec* col = reinterpret_cast<vec*>(cnt) + (int64_t)b0 * (E / V) + eq;
  const int64_t rs = E / V;  // row stride in vec
  int32_t mine[V] = {};
  auto add = [&](const vec& c) {
    if constexpr (V == 4) {
      mine[0] += c.x; mine[1] += c.y; mine[2] += c.z; mine[3] += c.w;
    } else {
      mine[0] += c;
    }
  };
  vec first[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; i++) first[i] = i < nrow ? col[i * rs] : vec{};
#pragma unroll
  for (int i = 0; i < kBatch; i++) add(first[i]);
  for (int64_t b = kBatch; b < nrow; b += kBatch) {
    vec c[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; i++) c[i] = b + i < nrow ? col[(b + i) * rs] : vec{};
#pragma unroll
    for (int i = 0; i < kBatch; i++) add(c[i]);
  }
#pragma unroll
  for (int i = 0; i < V; i++) part_sum[tid * V + i] = mine[i];
  __syncthreads();
  // exclusive prefix of the earlier parts, and expert tid's total
  int32_t run[V] = {};
  for (int pp = 0; pp < part; pp++)
#pragma unroll
    for (int i = 0; i < V; i++) run[i] += part_sum[(pp * EV + eq) * V + i];
  int count = 0;
  if (tid < E)
    for (int pp = 0; pp < P; pp++) count += part_sum[pp * EV * V + tid];
  // the counts become each row's exclusive prefix within its expert
  auto step = [&](vec& c) {
    if constexpr (V == 4) {
      const int4 v = c;
      c = make_int4(run[0], run[1], run[2], run[3]);
      run[0] += v.x; run[1] += v.y; run[2] += v.z; run[3] += v.w;
    } else {
      const int v = c;
      c = run[0];
      run[0] += v;
    }
  };
#pragma unroll
  for (int i = 0; i < kBatch; i++) {
    step(first[i]);
    if (i < nrow) col[i * rs] = first[i];
  }
  for (int64_t b = kBatch; b < nrow; b += kBatch) {
    vec c[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; i++) c[i] = b + i < nrow ? col[(b + i) * rs] : vec{};
#pragma unroll
    for (int i = 0; i < kBatch; i++) {
      step(c[i]);
      if (b + i < nrow) col[(b + i) * rs] = c[i];
    }
  }
  // tail-skip: expert tid's lowest slot rank over the counting blocks
  int minrank = k;
  if (skip_rank > 0 && tid < E)
    for (int64_t b = 0; b < ncb; b++) minrank = min(minrank, mrk[b * E + tid]);
  scan_and_tiles(count, T, k, E, slot, ss, n_slots, offsets, group_slot, status, meta, tiles, tile_tok, tile_base,
                 chunks, lds, nullptr, minrank, skip_rank, n_skipped);
}

// Token of routed row p (flat index f) into its tile's row table; the first
// row of a tile also fills the padding rows of a partial tile.
// tile_base and offsets may be LDS or global copies.
__device__ inline void note_tile_row(int32_t* __restrict__ tile_tok, const int32_t* tile_base,
                                     const int32_t* offsets, int e, int p, int f, int k, int count) {
  const int rel = p - offsets[e];
  const int tl = tile_base[e] + rel / kTileRows, r = rel % kTileRows;
  const int t = f / k;
  tile_tok[(int64_t)tl * kTileRows + r] = t;
  if (r == 0) {
    const int n = min(kTileRows, count - rel);
    for (int rr = n; rr < kTileRows; rr++) tile_tok[(int64_t)tl * kTileRows + rr] = t;
  }
}

// Whole grouping in one 1024-thread block for F = T*k <= kSmallF entries: the
// rank of an entry is the number of earlier entries with the same expert,
// counted directly over the ids staged in LDS.
constexpr int kSmallF = 256;

// The grouping of F <= kSmallF entries by one 1024-thread block, once every
// thread's entry e_mine (-1 for none) is staged in sid[] (LDS, entries F..255
// hold -1) and hist[0..E) is zero: counts, offsets, tiles, ranks, perm.
__device__ inline void group_small_tail(int e_mine, int F, int T, int k, int E, int slot, int ss, int32_t n_slots,
                                        int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                        int32_t* __restrict__ inv_perm, int32_t* __restrict__ group_slot,
                                        int32_t* __restrict__ status, int32_t* __restrict__ meta,
                                        int4* __restrict__ tiles, int32_t* __restrict__ tile_tok,
                                        int32_t* __restrict__ tile_base, int4* __restrict__ chunks, int32_t* hist,
                                        int32_t* cntl, int32_t* tbl, const int32_t* sid, int* lds,
                                        int32_t* minr = nullptr, int skip_rank = 0,
                                        int32_t* __restrict__ n_skipped = nullptr) {
  const int tid = threadIdx.x;
  if (e_mine >= 0) {
    atomicAdd(&hist[e_mine], 1);
    if (skip_rank > 0) atomicMin(&minr[e_mine], tid % k);  // minr[e] = k beforehand
  }
  __syncthreads();
  const int count = tid < E ? hist[tid] : 0;
  const int minrank = (skip_rank > 0 && tid < E) ? minr[tid] : k;
  if (tid < E) cntl[tid] = count;
  int tb = 0;
  STAGE_STAMP(1, 2);
  const int off = scan_and_tiles(count, T, k, E, slot, ss, n_slots, offsets, group_slot, status, meta, tiles,
                                 tile_tok, tile_base, chunks, lds, &tb, minrank, skip_rank, n_skipped);
  STAGE_STAMP(1, 3);
  if (tid < E) {
    hist[tid] = off;  // hist now holds each expert's first row
    tbl[tid] = tb;
  }
  __syncthreads();
  STAGE_STAMP(1, 4);
  if (tid < F) {
    if (e_mine < 0) {
      inv_perm[tid] = -1;
    } else {
      // rank = earlier entries with the same expert; 4 staged ids per LDS read,
      // over the wavefront's uniform range of earlier entries
      const int fend = min(F, (tid | 63) + 1);
      int rank = 0;
      const int4* sid4 = reinterpret_cast<const int4*>(sid);
#pragma unroll 4
      for (int f0 = 0; f0 < fend; f0 += 4) {
        const int4 q = sid4[f0 >> 2];
        rank += (f0 + 0 < tid && q.x == e_mine) + (f0 + 1 < tid && q.y == e_mine) +
                (f0 + 2 < tid && q.z == e_mine) + (f0 + 3 < tid && q.w == e_mine);
      }
      const int p = hist[e_mine] + rank;
      perm[p] = tid;
      inv_perm[tid] = p;
      if (!chunks) note_tile_row(tile_tok, tbl, hist, e_mine, p, tid, k, cntl[e_mine]);
    }
  }
  STAGE_STAMP(1, 5);
}

// Whole grouping in one 1024-thread block for F = T*k <= kSmallF entries: the
// rank of an entry is the number of earlier entries with the same expert,
// counted directly over the ids staged in LDS.
__global__ __launch_bounds__(1024) void k_group_small(const int32_t* __restrict__ ids, int F, int T, int k, int E,
                                                      int layer, const int32_t* __restrict__ slot_table,
                                                      int32_t n_slots, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                                      int32_t* __restrict__ group_slot, int32_t* __restrict__ status,
                                                      int32_t* __restrict__ meta, int4* __restrict__ tiles,
                                                      int32_t* __restrict__ tile_tok,
                                                      int32_t* __restrict__ tile_base, int4* __restrict__ chunks,
                                                      int skip_rank, int32_t* __restrict__ n_skipped,
                                                      int32_t* __restrict__ sync, int64_t n_sync) {
  __shared__ int32_t hist[1024];
  __shared__ int32_t cntl[1024];
  __shared__ int32_t tbl[1024];
  __shared__ int32_t minr[1024];
  __shared__ __align__(16) int32_t sid[kSmallF];
  __shared__ int lds[17];
  const int tid = threadIdx.x;
  STAGE_STAMP(1, 0);
  const int slot = tid < E ? slot_table[(int64_t)layer * (E + 1) + tid] : -1;
  const int ss = slot_table[(int64_t)layer * (E + 1) + E];
  zero_sync(sync, n_sync);
  if (tid < E) {
    hist[tid] = 0;
    minr[tid] = k;
  }
  int e_mine = -1;
  if (tid < F) {
    e_mine = ids[tid];
    if (e_mine < 0 || e_mine >= E) {
      atomicOr(status, MOE_DEV_BAD_EXPERT_ID);
      e_mine = -1;
    }
  }
  if (tid < kSmallF) sid[tid] = e_mine;  // -1 beyond F and for bad ids
  __syncthreads();
  STAGE_STAMP(1, 1);
  group_small_tail(e_mine, F, T, k, E, slot, ss, n_slots, offsets, perm, inv_perm, group_slot, status, meta, tiles,
                   tile_tok, tile_base, chunks, hist, cntl, tbl, sid, lds, minr, skip_rank, n_skipped);
}

// Route and group fused for small windows (T <= 16 tokens, T*k <= 256
// entries, drawn logits), one 1024-thread block: the sort path of
// route_small.hpp (threshold top-k per token wavefront, then the grouped order
// by rank counting).  With xq, the same launch also writes the MX FFN's A
// rows, bf16(MXFP8(x)) (mx_quant8_bf16, eight values per thread; the first
// pass's loads are issued before the top-k, so they land meanwhile).
template <int NPL>
__global__ __launch_bounds__(1024) void k_route_group_sort(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, const float* __restrict__ w_sg, int T, int H,
    int E, int k, int layer, const int32_t* __restrict__ slot_table, int32_t n_slots, int32_t* __restrict__ ids,
    float* __restrict__ wout, float* __restrict__ sigma, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ group_slot, int32_t* __restrict__ status,
    int32_t* __restrict__ meta, int4* __restrict__ tiles, int32_t* __restrict__ tile_tok, int4* __restrict__ chunks,
    int32_t* __restrict__ sync, int64_t n_sync, uint16_t* __restrict__ xq) {
  __shared__ SmallRouteLds<16> L;
  STAGE_STAMP(1, 0);
  const int64_t n8 = (int64_t)T * H / 8;  // x's 8-value groups (H % 32 == 0: whole quads)
  uint4 xv0 = make_uint4(0u, 0u, 0u, 0u);
  if (xq && threadIdx.x < n8) xv0 = reinterpret_cast<const uint4*>(x)[threadIdx.x];
  small_route_topk<NPL, 16, true>(L, logits, x, w_sg, T, H, E, k, slot_table + (int64_t)layer * (E + 1));
  __syncthreads();
  STAGE_STAMP(1, 1);
  small_route_sort_rows<16>(L, T * k, E);
  __syncthreads();
  STAGE_STAMP(1, 2);
  small_route_store<16>(L, T, k, E, n_slots, ids, wout, sigma, offsets, perm, inv_perm, group_slot, status, meta,
                        tiles, tile_tok, chunks, sync, n_sync);
  if (xq) {
    for (int64_t g = threadIdx.x; g < n8; g += 1024)
      reinterpret_cast<uint4*>(xq)[g] = mx_quant8_bf16(g < 1024 ? xv0 : reinterpret_cast<const uint4*>(x)[g]);
  }
  STAGE_STAMP(1, 3);
}

// Stable placement of one block of kBlk entries: an entry's rank is the number
// of earlier entries of the block with the same expert, counted over the ids
// staged in LDS (4 per read); its row is offsets[e] + the block's exclusive
// prefix for e (from k_scan) + rank.
__global__ __launch_bounds__(kBlk) void k_scatter(const int32_t* __restrict__ ids, int64_t F, int E, int k,
                                                  const int32_t* __restrict__ cnt, const int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                                  int32_t* __restrict__ tile_tok,
                                                  const int32_t* __restrict__ tile_base) {
  __shared__ __align__(16) int32_t sid[kBlk];
  __shared__ int32_t hist[1024];  // entries per expert in the earlier parts of this counting block
  const int i = threadIdx.x;
  const int64_t f = (int64_t)blockIdx.x * kBlk + i;
  const int part = blockIdx.x % kParts;  // block-uniform
  const int64_t cb = blockIdx.x / kParts;
  // the earlier parts are whole (only the last block can be partial)
  int prev[kParts - 1];
#pragma unroll
  for (int j = 0; j < kParts - 1; j++) prev[j] = j < part ? ids[cb * kCntBlk + j * kBlk + i] : -1;
  const bool in = f < F;
  const int e = in ? ids[f] : -1;
  const bool ok = in && e >= 0 && e < E;
  sid[i] = ok ? e : -1;
  if (part)
    for (int x = i; x < E; x += kBlk) hist[x] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kParts - 1; j++)
    if (prev[j] >= 0 && prev[j] < E) atomicAdd(&hist[prev[j]], 1);
  __syncthreads();
  if (in && !ok) inv_perm[f] = -1;
  if (!ok) return;
  int rank = part ? hist[e] : 0;
  const int4* sid4 = reinterpret_cast<const int4*>(sid);
  for (int j0 = 0; j0 < i; j0 += 4) {
    const int4 v = sid4[j0 >> 2];
    rank += (j0 + 0 < i && v.x == e) + (j0 + 1 < i && v.y == e) + (j0 + 2 < i && v.z == e) + (j0 + 3 < i && v.w == e);
  }
  const int p = offsets[e] + cnt[cb * E + e] + rank;
  perm[p] = (int32_t)f;
  inv_perm[f] = p;
  if (tile_tok) note_tile_row(tile_tok, tile_base, offsets, e, p, (int)f, k, offsets[e + 1] - offsets[e]);
}

}  // namespace

hipError_t launch_group(const moe_dims& d, int32_t layer, const int32_t* ids, const int32_t* slot_table,
                        int32_t n_slots, int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* group_slot,
                        int32_t* dev_status, void* ws, hipStream_t s, int32_t skip_rank, int32_t* n_skipped) {
  const WsLayout wl = ws_layout(d);
  const int64_t F = (int64_t)d.T * d.k;
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + wl.off_cnt);
  int32_t* meta = reinterpret_cast<int32_t*>(base + wl.off_meta);
  int4* tiles = reinterpret_cast<int4*>(base + wl.off_tiles);
  int32_t* tile_tok = reinterpret_cast<int32_t*>(base + wl.off_tile_tok);
  int32_t* tile_base = reinterpret_cast<int32_t*>(base + wl.off_tile_base);
  int4* chunks = use_gemm(d) ? reinterpret_cast<int4*>(base + wl.off_chunks) : nullptr;
  int32_t* sync = reinterpret_cast<int32_t*>(base + wl.off_sync);
  if (F <= kSmallF) {
    hipLaunchKernelGGL(k_group_small, dim3(1), dim3(1024), 0, s, ids, (int)F, d.T, d.k, d.E, layer, slot_table,
                       n_slots, offsets, perm, inv_perm, group_slot, dev_status, meta, tiles, tile_tok, tile_base,
                       chunks, skip_rank, n_skipped, sync, wl.n_sync);
    return hipGetLastError();
  }
  int32_t* mrk = reinterpret_cast<int32_t*>(base + wl.off_mrk);
  hipLaunchKernelGGL(k_count, dim3((unsigned)wl.ncb), dim3(kBlk), 0, s, ids, F, d.E, d.k, skip_rank, cnt, mrk,
                     dev_status);
  auto scan = d.E % 4 == 0 ? k_scan<4> : k_scan<1>;
  hipLaunchKernelGGL(scan, dim3(1), dim3(1024), 0, s, wl.ncb, d.T, d.k, d.E, layer, slot_table, n_slots, cnt,
                     offsets, group_slot, dev_status, meta, tiles, tile_tok, tile_base, chunks, skip_rank, mrk,
                     n_skipped, sync, wl.n_sync);
  hipLaunchKernelGGL(k_scatter, dim3((unsigned)wl.nb), dim3(kBlk), 0, s, ids, F, d.E, d.k, cnt, offsets, perm, inv_perm,
                     chunks ? nullptr : tile_tok, tile_base);
  return hipGetLastError();
}

bool route_group_fusable(const moe_dims& d) { return d.T <= 16 && (int64_t)d.T * d.k <= kSortF; }

hipError_t launch_route_group(const moe_dims& d, int32_t layer, const float* logits, const uint16_t* x,
                              const float* w_sg, const int32_t* slot_table, int32_t n_slots, int32_t* ids, float* w,
                              float* sigma, int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* group_slot,
                              int32_t* dev_status, void* ws, hipStream_t s, uint16_t* xq) {
  const WsLayout wl = ws_layout(d);
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* meta = reinterpret_cast<int32_t*>(base + wl.off_meta);
  int4* tiles = reinterpret_cast<int4*>(base + wl.off_tiles);
  int32_t* tile_tok = reinterpret_cast<int32_t*>(base + wl.off_tile_tok);
  int4* chunks = use_gemm(d) ? reinterpret_cast<int4*>(base + wl.off_chunks) : nullptr;
  int32_t* sync = reinterpret_cast<int32_t*>(base + wl.off_sync);
  const int npl = (d.E + 63) / 64;
  const dim3 g(1), b(1024);
  const int32_t* st = slot_table;
#define MOE_RG_SORT(N)                                                                                             \
  hipLaunchKernelGGL((k_route_group_sort<N>), g, b, 0, s, logits, x, w_sg, d.T, d.H, d.E, d.k, layer, st, n_slots, \
                     ids, w, sigma, offsets, perm, inv_perm, group_slot, dev_status, meta, tiles, tile_tok, chunks,   \
                     sync, wl.n_sync, xq)
#define MOE_RG_NPL(L)                 \
  if (npl <= 1) L(1);                 \
  else if (npl <= 2) L(2);            \
  else if (npl <= 4) L(4);            \
  else if (npl <= 8) L(8);            \
  else L(16);
  MOE_RG_NPL(MOE_RG_SORT)
#undef MOE_RG_NPL
#undef MOE_RG_SORT
  return hipGetLastError();
}

}  // namespace moe
