// Partial residency: one LRU cache of (layer, expert) blobs in S device slots.
//
// [FreeToken] 3.3: one LRU over (layer, expert), shared by all layers; a hit
// refreshes the expert's last use, a fill admits a newly chosen expert, and
// eviction removes the least recently used.  [FreeToken] 4: per MoE layer one
// device kernel dedups the routed experts, classifies them against the
// residency table, picks the victims (the least recently used slots, found in
// one pass over the slots, whatever the number of misses) and rewrites the
// table; one fixed-shape kernel then moves the blobs, masked by a device-side
// valid count, with no decision on the host.
//  - k_residency: one 1024-thread block per layer call.  Each thread owns a
//    contiguous run of slots, so no thread reads cache state another thread
//    wrote in this kernel.  The victims are the `take` smallest keys
//    (last use + 1; 0 for a slot never used) among the slots this call does
//    not hit: a four-pass radix select (8 bits a pass, LDS histograms) finds
//    the threshold key, keys equal to it go in slot order, and the victims are
//    ranked by (key, slot).  Misses (ascending expert) take victims in that
//    order.  The clock is a device counter, so a captured graph replays it.
//  - k_fill: a fixed grid copies the listed blobs from device-accessible
//    pinned host memory into their slots in 64 KiB pieces, masked by the
//    count the residency kernel wrote.
#include "moe_common.hpp"

namespace moe {
namespace {

constexpr int kResThreads = 1024;
constexpr uint64_t kFillChunk = 65536;

__global__ __launch_bounds__(kResThreads) void k_residency(const int32_t* __restrict__ ids, int F, int E, int layer,
                                                           int32_t* __restrict__ slot_table,
                                                           int32_t* __restrict__ owner, int32_t* __restrict__ last,
                                                           int S, int n_keys, int32_t* __restrict__ clock,
                                                           int2* __restrict__ fills, int32_t* __restrict__ n_fill,
                                                           int32_t* __restrict__ status) {
  __shared__ int32_t need[kMaxExperts + 1];           // expert e of this layer is needed (E: the shared one)
  __shared__ uint32_t hitmap[kMaxResidencySlots / 32];  // slots this call hits
  __shared__ int32_t hist[256];
  __shared__ int lds17[17];
  __shared__ uint32_t sel[2];                          // a pass's digit and the count below it
  __shared__ int32_t vkey[kMaxExperts + 1], vslot[kMaxExperts + 1], vord[kMaxExperts + 1];
  __shared__ int32_t nvict;
  const int tid = threadIdx.x;
  const int E1 = E + 1;
  const int now = clock[0];
  int32_t* row = slot_table + (int64_t)layer * E1;

  // 1. the experts this window needs: its routed ids (ids outside [0, E) are
  // the grouping's to report) and the shared expert
  for (int e = tid; e < E1; e += kResThreads) need[e] = e == E;
  for (int w = tid; w < (S + 31) / 32; w += kResThreads) hitmap[w] = 0;
  if (tid == 0) nvict = 0;
  __syncthreads();
  for (int f = tid; f < F; f += kResThreads) {
    const int e = ids[f];
    if (e >= 0 && e < E) need[e] = 1;
  }
  __syncthreads();

  // 2. thread t classifies expert t (the last thread also takes expert 1024,
  // so the experts stay in thread order): hits mark their slot, misses are
  // numbered in ascending expert order
  const int e_lo = min(tid, E1), e_hi = min(tid == kResThreads - 1 ? E1 : tid + 1, E1);
  int nmiss = 0;
  for (int e = e_lo; e < e_hi; e++) {
    if (!need[e]) continue;
    const int s = row[e];
    if (s >= S) atomicOr(status, MOE_DEV_BAD_SLOT);  // left as it is
    else if (s >= 0) atomicOr(&hitmap[s >> 5], 1u << (s & 31));
    else nmiss++;
  }
  int m = 0;
  const int mbase = block_exclusive_scan(nmiss, lds17, &m);  // (its barriers also publish hitmap)

  // 3. victims: the `take` least recently used slots this call does not hit
  const int per = (S + kResThreads - 1) / kResThreads;
  const int s0 = min(S, tid * per), s1 = min(S, s0 + per);
  auto cand = [&](int s) { return ((hitmap[s >> 5] >> (s & 31)) & 1u) == 0; };
  auto key = [&](int s) { return (uint32_t)(last[s] + 1); };
  int ncand_mine = 0;
  for (int s = s0; s < s1; s++) ncand_mine += cand(s);
  int ncand = 0;
  block_exclusive_scan(ncand_mine, lds17, &ncand);
  const int take = min(m, ncand);
  if (take < m && tid == 0) atomicOr(status, MOE_DEV_CACHE_FULL);
  // radix select of the take-th smallest key thr; rem = how many keys equal
  // to thr are taken (those below thr all are)
  uint32_t thr = 0, tmask = 0;
  int rem = take;
  if (take > 0) {
    for (int pass = 0; pass < 4; pass++) {
      const int sh = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int s = s0; s < s1; s++) {
        if (!cand(s)) continue;
        const uint32_t k = key(s);
        if ((k & tmask) == thr) atomicAdd(&hist[(k >> sh) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {  // wavefront 0 finds the digit where the running count reaches rem
        int h[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          h[i] = hist[4 * tid + i];
          sum += h[i];
        }
        const int inc = wave_inclusive_scan(sum);
        const uint64_t reach = __builtin_amdgcn_ballot_w64(inc >= rem);
        if (tid == __builtin_ctzll(reach)) {
          int c = inc - sum, b = 0;
          while (b < 3 && c + h[b] < rem) c += h[b++];
          sel[0] = (uint32_t)(4 * tid + b);
          sel[1] = (uint32_t)c;
        }
      }
      __syncthreads();
      thr |= sel[0] << sh;
      tmask |= 255u << sh;
      rem -= (int)sel[1];
      __syncthreads();  // sel is rewritten by the next pass
    }
  }
  // every candidate key below thr, and the first rem equal to it in slot order
  int neq_mine = 0;
  if (take > 0)
    for (int s = s0; s < s1; s++) neq_mine += cand(s) && key(s) == thr;
  int neq = 0;
  int eq_i = block_exclusive_scan(neq_mine, lds17, &neq);
  if (take > 0) {
    for (int s = s0; s < s1; s++) {
      if (!cand(s)) continue;
      const uint32_t k = key(s);
      bool v = k < thr;
      if (k == thr) v = eq_i++ < rem;
      if (v) {
        const int p = atomicAdd(&nvict, 1);
        if (p < take) {  // exactly take victims are found; the test keeps the arrays in bounds regardless
          vkey[p] = (int32_t)k;
          vslot[p] = s;
        }
      }
    }
  }
  __syncthreads();
  // victims in LRU order: rank by (key, slot)
  for (int i = tid; i < take; i += kResThreads) {
    const uint64_t ki = ((uint64_t)(uint32_t)vkey[i] << 32) | (uint32_t)vslot[i];
    int r = 0;
    for (int j = 0; j < take; j++) r += (((uint64_t)(uint32_t)vkey[j] << 32) | (uint32_t)vslot[j]) < ki;
    vord[r] = vslot[i];
  }
  __syncthreads();

  // 4. rewrite: hits refresh their slot; miss i (expert order) takes victim i,
  // whose previous owner leaves the table
  int mi = mbase;
  for (int e = e_lo; e < e_hi; e++) {
    if (!need[e]) continue;
    const int s = row[e];
    if (s >= S) continue;
    if (s >= 0) {
      last[s] = now;
      continue;
    }
    if (mi < take) {
      const int v = vord[mi];
      const int old = owner[v];
      if (old >= 0 && old < n_keys) slot_table[old] = -1;  // flat [L][E+1] index
      const int k = layer * E1 + e;
      owner[v] = k;
      last[v] = now;
      row[e] = v;
      fills[mi] = make_int2(k, v);
    }
    mi++;
  }
  if (tid == 0) {
    clock[0] = now + 1;
    n_fill[0] = take;
  }
}

__global__ __launch_bounds__(256) void k_fill(const int2* __restrict__ fills, const int32_t* __restrict__ n_fill,
                                              const uint8_t* __restrict__ host, int32_t n_keys, int32_t n_slots,
                                              uint64_t stride, uint64_t blob_bytes, int cpb, uint8_t* __restrict__ pool) {
  const int64_t items = (int64_t)n_fill[0] * cpb;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int2 f = fills[it / cpb];
    if (f.x < 0 || f.x >= n_keys || f.y < 0 || f.y >= n_slots) continue;  // not a list this library wrote
    const uint64_t b0 = (uint64_t)(it % cpb) * kFillChunk;
    const uint64_t b1 = b0 + kFillChunk < blob_bytes ? b0 + kFillChunk : blob_bytes;
    const uint8_t* src = host + (uint64_t)f.x * stride;
    uint8_t* dst = pool + (uint64_t)f.y * stride;
    const uint64_t t0 = b0 + ((b1 - b0) & ~uint64_t(15));
    for (uint64_t o = b0 + 16 * threadIdx.x; o < t0; o += 16 * blockDim.x)
      *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(src + o);
    for (uint64_t o = t0 + 4 * threadIdx.x; o < b1; o += 4 * blockDim.x)
      *reinterpret_cast<uint32_t*>(dst + o) = *reinterpret_cast<const uint32_t*>(src + o);
  }
}

}  // namespace

hipError_t launch_residency(const moe_dims& d, int32_t layer, const int32_t* ids, int32_t* slot_table, int32_t* owner,
                            int32_t* last, int32_t n_slots, int32_t* clock, int32_t* fills, int32_t* n_fill,
                            int32_t* dev_status, hipStream_t s) {
  hipLaunchKernelGGL(k_residency, dim3(1), dim3(kResThreads), 0, s, ids, d.T * d.k, d.E, layer, slot_table, owner, last,
                     n_slots, d.L * (d.E + 1), clock, reinterpret_cast<int2*>(fills), n_fill, dev_status);
  return hipGetLastError();
}

hipError_t launch_fill(const moe_dims& d, const uint8_t* host, uint64_t stride, uint64_t blob_bytes, uint8_t* pool,
                       int32_t n_slots, const int32_t* fills, const int32_t* n_fill, hipStream_t s) {
  const int cpb = (int)((blob_bytes + kFillChunk - 1) / kFillChunk);
  hipLaunchKernelGGL(k_fill, dim3(512), dim3(256), 0, s, reinterpret_cast<const int2*>(fills), n_fill, host,
                     d.L * (d.E + 1), n_slots, stride, blob_bytes, cpb, pool);
  return hipGetLastError();
}

}  // namespace moe

// ---- hot/cold swaps -----------------------------------------------------------
// [Strata] "哪些专家能长期留在显存？": each expert's heat accumulates its routing
// counts and decays after every swap round; a swap moves a hot expert's blob
// into a cold expert's slot, and the table names the new owner only once the
// copy is done (stream order: list, fill, publish).
namespace moe {
namespace {

// heat[layer][e] += rows of routed group e (offsets from moe_group)
__global__ __launch_bounds__(256) void k_heat(const int32_t* __restrict__ offsets, int E, int layer,
                                              float* __restrict__ heat) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < E) heat[(int64_t)layer * E + e] += (float)(offsets[e + 1] - offsets[e]);
}

__global__ __launch_bounds__(256) void k_heat_decay(float* __restrict__ heat, int64_t n, float decay) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) heat[i] *= decay;
}

// plan entry i = (layer, hot, cold) -> fill (key of (layer, hot), slot of cold);
// an entry that no longer fits the table (hot resident, cold not) gets key -1
// and is skipped by the fill and the publication.  So does an entry that
// names, in its layer, an expert an earlier entry already names (as hot or as
// cold): two fills into one slot, or one expert moved twice, would leave the
// table pointing at bytes that are not its expert's.
__global__ __launch_bounds__(256) void k_swap_list(const int3* __restrict__ plan, int n_plan, int L, int E,
                                                   int n_slots, const int32_t* __restrict__ table,
                                                   int2* __restrict__ fills, int32_t* __restrict__ n_fill) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) *n_fill = n_plan;
  if (i >= n_plan) return;
  const int3 p = plan[i];
  const int E1 = E + 1;
  bool ok = p.x >= 0 && p.x < L && p.y >= 0 && p.y < E && p.z >= 0 && p.z < E && p.y != p.z;
  for (int j = 0; ok && j < i; j++) {
    const int3 q = plan[j];
    if (q.x == p.x && (q.y == p.y || q.y == p.z || q.z == p.y || q.z == p.z)) ok = false;
  }
  const int hot_slot = ok ? table[p.x * E1 + p.y] : 0, cold_slot = ok ? table[p.x * E1 + p.z] : -1;
  const bool fits = ok && hot_slot < 0 && cold_slot >= 0 && cold_slot < n_slots;
  fills[i] = fits ? make_int2(p.x * E1 + p.y, cold_slot) : make_int2(-1, -1);
}

__global__ __launch_bounds__(256) void k_swap_publish(const int3* __restrict__ plan, int n_plan, int E,
                                                      const int2* __restrict__ fills, int32_t* __restrict__ table) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_plan) return;
  const int2 f = fills[i];
  if (f.x < 0) return;
  const int3 p = plan[i];
  table[p.x * (E + 1) + p.y] = f.y;
  table[p.x * (E + 1) + p.z] = -1;
}

}  // namespace

hipError_t launch_heat(const moe_dims& d, int32_t layer, const int32_t* offsets, float* heat, hipStream_t s) {
  hipLaunchKernelGGL(k_heat, dim3((d.E + 255) / 256), dim3(256), 0, s, offsets, d.E, layer, heat);
  return hipGetLastError();
}

hipError_t launch_heat_decay(const moe_dims& d, float* heat, float decay, hipStream_t s) {
  const int64_t n = (int64_t)d.L * d.E;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_heat_decay, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s, heat, n, decay);
  return hipGetLastError();
}

hipError_t launch_swap_apply(const moe_dims& d, const uint8_t* host, uint64_t stride, uint64_t blob_bytes,
                             uint8_t* pool, int32_t n_slots, int32_t* table, const int32_t* plan, int32_t n_plan,
                             int32_t* fills, int32_t* n_fill, hipStream_t s) {
  const dim3 g((unsigned)((n_plan + 255) / 256 > 0 ? (n_plan + 255) / 256 : 1));
  hipLaunchKernelGGL(k_swap_list, g, dim3(256), 0, s, reinterpret_cast<const int3*>(plan), n_plan, d.L, d.E, n_slots,
                     table, reinterpret_cast<int2*>(fills), n_fill);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_fill(d, host, stride, blob_bytes, pool, n_slots, fills, n_fill, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_swap_publish, g, dim3(256), 0, s, reinterpret_cast<const int3*>(plan), n_plan, d.E,
                     reinterpret_cast<const int2*>(fills), table);
  return hipGetLastError();
}

}  // namespace moe
