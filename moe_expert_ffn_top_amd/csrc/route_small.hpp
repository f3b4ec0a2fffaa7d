// Route (S1) and group (S3) of a small window by one workgroup: T <= 16
// tokens, F = T k <= 256 (token, slot) entries, drawn logits.  The pieces are
// shared by the route + group kernel (k_route_group_sort, one 1024-thread
// workgroup) and by the gate/up kernel that routes in its own prologue
// (k_ffn_dec with RouteArgs; every workgroup routes for itself, workgroup 0
// stores the results).
//
// [Strata] "还有一条会改变输出的路径" and "路由以后，专家怎样分工？": a token's k
// largest logits pick its experts (the lower index wins a tie, slot j holds
// the j-th largest); the rows of one expert form one group, ascending token.
//  - small_route_topk: the slot row into LDS; token t by wavefront t mod NW
//    (threshold top-k, topk_threshold), each wavefront's tokens' logits all
//    requested before the first top-k; optionally the shared gate's dot
//    product.
//  - small_route_sort_rows: the grouped order.  Keys (expert, entry) are
//    distinct, so a valid key's row is the count of smaller keys.  Every key
//    is staged in LDS once; a lane then counts the keys below its own with
//    broadcast reads of four keys, sixteen keys per round in flight, and
//    plain vector compares.  F <= 64: wavefront 0 alone; F <= 256: wavefront
//    w holds entries 64 w .. 64 w + 63.  One scatter through LDS gives row p
//    its key; its neighbours' keys and wavefront scans (with the earlier
//    wavefronts' totals through LDS) give each row its group, its group's
//    first row and its rank in the group (one tile per group: a group has at
//    most T <= 16 rows).
//  - small_route_tiles: the FFN work list (tiles and their token tables, or
//    the GEMM's chunks) through generic pointers, so into LDS or memory, from
//    the sorting wavefronts' registers or from the rows the sort left in LDS.
//  - small_route_store: every other output.  No global store comes before the
//    callers' last barrier (a barrier waits for the wavefront's outstanding
//    memory operations, stores included).
#pragma once

#include "moe_common.hpp"
#include "topk_wave.hpp"

namespace moe {

constexpr int kSortF = 256;  // entries of the sort path
constexpr int kSortF1 = 64;  // entries sorted by one wavefront alone

// wavefronts that hold rows of the grouped order (64 rows each)
__host__ __device__ constexpr int sort_waves(int F) { return F <= kSortF1 ? 1 : (F + 63) / 64; }

template <int NW>
struct SmallRouteLds {
  alignas(16) int32_t sid[kSortF];  // the winners' experts [T][k] (entry f = t k + j), -1 beyond F
  uint32_t wink[kSortF];            // the winners' keys
  uint2 cand[NW * 64];              // top-k candidates, 64 per wavefront
  int32_t slots[kMaxExperts + 1];   // slot of each expert, the shared one at E
  float z[16];                      // the shared gate's dot product of each token
  int32_t ge[kSortF];               // group g: its expert (ascending)
  int32_t gp[kSortF];               //          its first row
  int32_t gnv[2];                   // groups, valid rows
  int4 rowi[kSortF];                // row p: (expert, entry, group, rank)
  int2 rowj[kSortF];                // row p: (group's first row, last row of its group)
  alignas(16) uint32_t kin[kSortF]; // the sort's keys by entry (above every valid key from F on)
  uint32_t skey[kSortF];            // the sort's scatter: row p's key
  int32_t wnv[kSortF / 64];         // per sorting wavefront: valid entries,
  int32_t wnf[kSortF / 64];         //   group starts among its rows,
  int32_t wsf[kSortF / 64];         //   its last group start (row << 8 | entry)
};

// Row p of the grouped order, held by lane p of the sorting wavefront.
struct SortedRow {
  int e;        // expert, -1 past the valid rows
  int f;        // entry t k + j
  int grp;      // group
  int rank;     // rank in the group
  int start;    // the group's first row
  int f_first;  // the entry of that row
  bool last;    // last row of the group
  int nd, nv;   // groups, valid rows (the same in every lane)
};

constexpr uint32_t kNoRowKey = 1u << 30;   // above every valid key (expert < 2^10, entry < 2^8)

// The count of keys kin[0 .. F) below key.  kin holds keys above every valid
// one from F up to F rounded up to 4.  The reads are the same address in
// every lane (one broadcast LDS read per four keys), four of them in flight.
__device__ __forceinline__ int count_keys_below(const uint32_t* kin, int F, uint32_t key) {
  const uint4* k4 = reinterpret_cast<const uint4*>(kin);
  const int n4 = (F + 3) >> 2;
  int below = 0, i = 0;
  for (; i + 4 <= n4; i += 4) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) v[u] = k4[i + u];
#pragma unroll
    for (int u = 0; u < 4; u++)
      below += (v[u].x < key ? 1 : 0) + (v[u].y < key ? 1 : 0) + (v[u].z < key ? 1 : 0) + (v[u].w < key ? 1 : 0);
  }
  for (; i < n4; i++) {
    const uint4 v = k4[i];
    below += (v.x < key ? 1 : 0) + (v.y < key ? 1 : 0) + (v.z < key ? 1 : 0) + (v.w < key ? 1 : 0);
  }
  return below;
}

// floor(f / k) for 0 <= f < 2^8 and k >= 1 through rk = 1 / k in fp32: f + 0.5
// lies at least 0.5 / k from a multiple of k, a relative gap of at least 2^-9,
// far above the two roundings' 2^-23.
__device__ __forceinline__ int entry_token(int f, float rk) { return (int)(((float)f + 0.5f) * rk); }

// Inclusive max-scan of one wavefront (values >= 0) with DPP, the pattern of
// wave_inclusive_scan: lanes shifted in from outside a row give 0.
__device__ __forceinline__ int wave_inclusive_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true));   // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true));   // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true));   // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true));   // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// Every wavefront of the NW: the slot row slot_row[0..E] into LDS; tokens
// t = wave, wave + NW, ... < T: the winners into sid / wink (slot order);
// with GATE (one token per wavefront), z[t] = x[t] . w_sg.  The caller then
// meets a barrier.
template <int NPL, int NW, bool GATE>
__device__ __forceinline__ void small_route_topk(SmallRouteLds<NW>& L, const float* __restrict__ logits,
                                        const uint16_t* __restrict__ x, const float* __restrict__ w_sg, int T, int H,
                                        int E, int k, const int32_t* __restrict__ slot_row) {
  constexpr int MAXT = (16 + NW - 1) / NW;   // tokens per wavefront (T <= 16)
  static_assert(!GATE || MAXT == 1, "the shared gate runs beside the top-k only at one token per wavefront");
  const int tid = threadIdx.x, wave = tid >> 6;
  const int F = T * k;
  // the slot row is loaded into registers first and stored after the top-k,
  // so its round trip overlaps the logits' instead of preceding it
  constexpr int SPT = (kMaxExperts + 1 + NW * 64 - 1) / (NW * 64);
  int sl[SPT];
#pragma unroll
  for (int i = 0; i < SPT; i++) {
    const int e = tid + i * NW * 64;
    sl[i] = e <= E ? slot_row[e] : -1;
  }
  for (int f = F + tid; f < kSortF; f += NW * 64) L.sid[f] = -1;
  uint32_t key[MAXT][NPL];
#pragma unroll
  for (int i = 0; i < MAXT; i++)
    if (wave + i * NW < T) load_keys<NPL>(key[i], logits, wave + i * NW, E, 0, E);
  GateIn g;
  if (GATE && wave < T) gate_load(g, x, w_sg, wave, H);
#pragma unroll
  for (int i = 0; i < MAXT; i++) {
    const int t = wave + i * NW;
    if (t < T) topk_threshold<NPL>(key[i], k, L.wink + t * k, L.sid + t * k, L.cand + wave * 64);
  }
  if (GATE && wave < T) {
    const float z = gate_dot(g, x, w_sg, wave, H);
    if ((tid & 63) == 0) L.z[wave] = z;
  }
#pragma unroll
  for (int i = 0; i < SPT; i++) {
    const int e = tid + i * NW * 64;
    if (e <= E) L.slots[e] = sl[i];
  }
}

// z[t] = x[t] . w_sg for tokens t = wave, wave + NW, ... < T (small_route_topk
// without the gate; the same wavefront then finishes the token in
// small_route_store, so no barrier is needed between).
template <int NW>
__device__ __forceinline__ void small_route_gate(SmallRouteLds<NW>& L, const uint16_t* __restrict__ x,
                                        const float* __restrict__ w_sg, int T, int H) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int t = wave; t < T; t += NW) {
    GateIn g;
    gate_load(g, x, w_sg, t, H);
    const float z = gate_dot(g, x, w_sg, t, H);
    if ((tid & 63) == 0) L.z[t] = z;
  }
}

// Wavefront 0 alone, F <= 64, after the barrier that follows small_route_topk:
// the grouped order of the F entries, returned lane by lane and left in rowi /
// rowj / ge / gp / gnv for small_route_store.  An entry whose expert lies
// outside [0, E) (none, for top-k winners) sorts last and is not valid.  Keys
// are distinct, so a valid key's rank (the count of smaller keys; only entries
// below F can be smaller) is its row.
template <int NW>
__device__ __forceinline__ SortedRow small_route_sort1(SmallRouteLds<NW>& L, int F, int E) {
  const int lane = threadIdx.x & 63;
  const int e0 = lane < F ? L.sid[lane] : -1;
  const bool ok = lane < F && e0 >= 0 && e0 < E;
  const uint32_t key = ok ? ((uint32_t)e0 << 6) | (uint32_t)lane : kNoRowKey | (uint32_t)lane;
  const int nv = __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok));
  L.kin[lane] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int below = count_keys_below(L.kin, F, key);
  if (ok) L.skey[below] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const bool valid = lane < nv;
  const uint32_t kp = valid ? L.skey[lane] : 0u;
  const uint32_t kprev = valid && lane > 0 ? L.skey[lane - 1] : 0u;
  const uint32_t knext = lane + 1 < nv ? L.skey[lane + 1] : 0u;
  const int e_r = valid ? (int)(kp >> 6) : -1;
  const int f_r = valid ? (int)(kp & 63u) : 63;
  const bool flag = valid && (lane == 0 || (int)(kprev >> 6) != e_r);
  const bool last = valid && (lane == nv - 1 || (int)(knext >> 6) != e_r);
  const int grp = wave_inclusive_scan(flag ? 1 : 0) - 1;
  // the latest group start at or below this row, with its entry in the low bits
  const int sf = wave_inclusive_max(flag ? (lane << 6) | f_r : 0);
  const int start = sf >> 6;
  const int nd = __builtin_popcountll(__builtin_amdgcn_ballot_w64(flag));
  if (flag) {
    L.ge[grp] = e_r;
    L.gp[grp] = lane;
  }
  L.rowi[lane] = make_int4(e_r, f_r, grp, lane - start);
  L.rowj[lane] = make_int2(start, last ? 1 : 0);
  if (lane == 0) {
    L.gnv[0] = nd;
    L.gnv[1] = nv;
  }
  return SortedRow{e_r, f_r, grp, lane - start, start, sf & 63, last, nd, nv};
}

// Key of entry j with expert e in the many-wavefront sort: (e << 8 | j), or
// above every valid key when e is not an expert (the -1 past F included).
__device__ __forceinline__ uint32_t sort_key_n(int e, int j, int E) {
  return (e >= 0 && e < E) ? ((uint32_t)e << 8) | (uint32_t)j : kNoRowKey | (uint32_t)j;
}

// Every wavefront of the workgroup, 64 < F <= 256 (meets three barriers):
// wavefront w < sort_waves(F) stages the keys of entries 64 w + lane, ranks
// them against all F keys and then holds rows 64 w + lane of the grouped
// order; the others return rows that are not valid.  Outputs as
// small_route_sort1.
template <int NW>
__device__ __forceinline__ SortedRow small_route_sortN(SmallRouteLds<NW>& L, int F, int E) {
  static_assert(NW >= kSortF / 64, "one wavefront per 64 rows");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nws = sort_waves(F);
  const int p = wave * 64 + lane;   // this thread's entry, then its row
  const bool act = wave < nws;
  const uint32_t key = act ? sort_key_n(p < F ? L.sid[p] : -1, p, E) : 0u;
  const bool ok = act && key < kNoRowKey;
  if (act) L.kin[p] = key;
  __syncthreads();
  if (act) {
    const int below = count_keys_below(L.kin, F, key);
    if (ok) L.skey[below] = key;
    const int nvw = __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok));
    if (lane == 0) L.wnv[wave] = nvw;
  }
  __syncthreads();
  int nv = 0;
  for (int w = 0; w < nws; w++) nv += L.wnv[w];
  const bool valid = p < nv;   // (only rows of the sorting wavefronts)
  const uint32_t kp = valid ? L.skey[p] : 0u;
  const uint32_t kprev = valid && p > 0 ? L.skey[p - 1] : 0u;
  const uint32_t knext = p + 1 < nv ? L.skey[p + 1] : 0u;
  const int e_r = valid ? (int)(kp >> 8) : -1;
  const int f_r = valid ? (int)(kp & 255u) : 255;
  const bool flag = valid && (p == 0 || (int)(kprev >> 8) != e_r);
  const bool last = valid && (p == nv - 1 || (int)(knext >> 8) != e_r);
  const int cnt_in = wave_inclusive_scan(flag ? 1 : 0);
  const int sf_in = wave_inclusive_max(flag ? (p << 8) | f_r : 0);
  if (act && lane == 63) {
    L.wnf[wave] = cnt_in;
    L.wsf[wave] = sf_in;
  }
  __syncthreads();
  // the earlier wavefronts' group starts: the count before this one, and the
  // latest start (rows ascend, so the largest packed value)
  int pre = 0, carry = 0, nd = 0;
  for (int w = 0; w < nws; w++) {
    const int nf = L.wnf[w];
    nd += nf;
    if (w < wave) {
      pre += nf;
      carry = max(carry, L.wsf[w]);
    }
  }
  const int grp = pre + cnt_in - 1;
  const int sf = max(sf_in, carry);
  const int start = sf >> 8;
  if (act) {
    if (flag) {
      L.ge[grp] = e_r;
      L.gp[grp] = p;
    }
    L.rowi[p] = make_int4(e_r, f_r, grp, p - start);
    L.rowj[p] = make_int2(start, last ? 1 : 0);
    if (p == 0) {
      L.gnv[0] = nd;
      L.gnv[1] = nv;
    }
  }
  return SortedRow{e_r, f_r, grp, p - start, start, sf & 255, last, nd, nv};
}

// Every wavefront of the workgroup, after the barrier that follows
// small_route_topk: the grouped order (small_route_sort1 or _sortN by F, the
// same in every wavefront).  Wavefronts w < sort_waves(F) return rows
// 64 w + lane; the others rows that are not valid.  The caller then meets a
// barrier before other wavefronts read what the sort left in LDS.
template <int NW>
__device__ __forceinline__ SortedRow small_route_sort_rows(SmallRouteLds<NW>& L, int F, int E) {
  if (F <= kSortF1) {
    if ((threadIdx.x >> 6) == 0) return small_route_sort1<NW>(L, F, E);
    return SortedRow{-1, 63, 0, 0, 0, 0, false, 0, 0};
  }
  return small_route_sortN<NW>(L, F, E);
}

// Row p of the grouped order from what the sort left in LDS (after a barrier).
template <int NW>
__device__ __forceinline__ SortedRow sorted_row_from_lds(const SmallRouteLds<NW>& L, int p) {
  const int4 ri = L.rowi[p];
  const int2 rj = L.rowj[p];
  return SortedRow{ri.x, ri.y, ri.z, ri.w, rj.x, L.rowi[rj.x].y, rj.y != 0, L.gnv[0], L.gnv[1]};
}

// The FFN work list of the grouped rows, one row per thread (the calls for
// rows 0 .. F - 1 together).  Without chunks: tile g of each routed group
// (expert, first row, rows, slot) and its 16-entry token table (with pad,
// rows past n repeat the group's first token; without, they are left as they
// were: a reader that masks rows past n does not need them), then, by the one
// wavefront that passes shared_part, the shared group's tiles and n_tiles =
// their count.  With
// chunks (the grouped GEMM's list): one chunk per routed group, then the
// shared group's, and n_chunks = their count.  Generic pointers: LDS or
// memory.
template <int NW>
__device__ __forceinline__ void small_route_tiles(const SmallRouteLds<NW>& L, const SortedRow& row, int T, int k, int E,
                                         int4* tiles, int32_t* tile_tok, int32_t* n_tiles, int4* chunks,
                                         int32_t* n_chunks, bool shared_part, bool pad = true) {
  const int lane = threadIdx.x & 63;
  const int F = T * k;
  const int e_r = row.e, f_r = row.f, grp = row.grp, rank = row.rank, start = row.start;
  const bool valid = e_r >= 0, last = row.last;
  const int nd = row.nd;
  const int ss = L.slots[E];
  const int se = valid ? L.slots[e_r] : -1;
  if (valid && last && chunks) chunks[grp] = make_int4(e_r, start, rank + 1, se);
  if (!chunks) {
    const float rk = 1.0f / (float)k;
    if (valid) {
      tile_tok[grp * kTileRows + rank] = entry_token(f_r, rk);
      if (last) {
        tiles[grp] = make_int4(e_r, start, rank + 1, se);
        if (pad) {   // rows past n repeat the group's first token
          const int t0 = entry_token(row.f_first, rk);
          for (int r = rank + 1; r < kTileRows; r++) tile_tok[grp * kTileRows + r] = t0;
        }
      }
    }
    // the shared group: tiles after the routed ones, rows in token order
    if (shared_part) {
      const int nts = (T + kTileRows - 1) / kTileRows;
      if (lane < nts) tiles[nd + lane] = make_int4(E, F + lane * kTileRows, min(kTileRows, T - lane * kTileRows), ss);
      for (int i = lane; i < nts * kTileRows; i += 64) {
        const int tl = i / kTileRows, r = i % kTileRows;
        const int n = min(kTileRows, T - tl * kTileRows);
        tile_tok[(nd + tl) * kTileRows + r] = tl * kTileRows + (r < n ? r : 0);
      }
      if (lane == 0) *n_tiles = nd + nts;
    }
  } else if (shared_part && lane == 0) {
    chunks[nd] = make_int4(E, F, T, ss);   // T <= 16 <= kChunkRows
    *n_chunks = nd + 1;
  }
}

// The outputs, after the callers' last barrier, by a workgroup of NW
// wavefronts: expert e's first row (the first group at or above e), its slot
// and the status bits (threads e, e + 64 NW, ...); the rows' perm / inv_perm,
// the groups' bounds and the work list (wavefront NW - 1); the tokens' ids,
// weights and shared gates (wavefront t mod NW; needs z, small_route_topk with
// gate); the fused launch's counters zeroed.  DEV: the weights, sigma and
// inv_perm (the combine's inputs) are stored device-coherently, for the other
// workgroups of a launch that combines.
template <int NW, bool DEV = false>
__device__ __forceinline__ void small_route_store(const SmallRouteLds<NW>& L, int T, int k, int E, int32_t n_slots,
                                         int32_t* __restrict__ ids, float* __restrict__ wout,
                                         float* __restrict__ sigma, int32_t* __restrict__ offsets,
                                         int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                         int32_t* __restrict__ group_slot, int32_t* __restrict__ status,
                                         int32_t* __restrict__ meta, int4* __restrict__ tiles,
                                         int32_t* __restrict__ tile_tok, int4* __restrict__ chunks,
                                         int32_t* __restrict__ sync, int64_t n_sync) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int F = T * k;
  const int nd = L.gnv[0], nv = L.gnv[1];
  for (int e = tid; e < E; e += NW * 64) {
    int lo = 0, hi = nd;   // first g with ge[g] >= e
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (L.ge[mid] < e) lo = mid + 1;
      else hi = mid;
    }
    const int slot = L.slots[e];
    offsets[e] = lo < nd ? L.gp[lo] : nv;
    group_slot[e] = slot;
    if (lo < nd && L.ge[lo] == e) {
      if (slot < 0) atomicOr(status, MOE_DEV_NOT_RESIDENT);
      if (slot >= n_slots) atomicOr(status, MOE_DEV_BAD_SLOT);
    }
  }
  if (wave == NW - 1) {
    for (int p0 = 0; p0 < F; p0 += 64) {
      const int p = p0 + lane;
      const int4 ri = L.rowi[p];
      if (ri.x >= 0) {
        perm[p] = ri.y;
        store_maybe_dev<DEV>(inv_perm + ri.y, p);
      }
      if (p < F) {
        const int e0 = L.sid[p];
        if (e0 < 0 || e0 >= E) store_maybe_dev<DEV>(inv_perm + p, -1);   // (never for top-k winners)
      }
      small_route_tiles<NW>(L, sorted_row_from_lds(L, p), T, k, E, tiles, tile_tok, meta, chunks, meta + 1, p0 == 0);
    }
    if (lane == 0) {
      const int ss = L.slots[E];
      offsets[E] = nv;
      offsets[E + 1] = F + T;
      group_slot[E] = ss;
      if (ss < 0) atomicOr(status, MOE_DEV_NOT_RESIDENT);
      if (ss >= n_slots) atomicOr(status, MOE_DEV_BAD_SLOT);
      if (nv < F) atomicOr(status, MOE_DEV_BAD_EXPERT_ID);
    }
  }
  for (int t = wave; t < T; t += NW) topk_finish<DEV>(L.wink + t * k, L.sid + t * k, t, k, L.z[t], ids, wout, sigma);
  zero_sync(sync, n_sync);
}

}  // namespace moe
