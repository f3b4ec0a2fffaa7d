/*
 * moe.h — C ABI of libmoe: one MoE layer's routed-expert computation on an
 * AMD Instinct MI355X (gfx950).
 *
 * The layer computes, for T tokens x[t] of width H:
 *   router logits -> top-k experts and renormalised softmax weights,
 *   grouping of the (token, slot) rows by expert through a resident slot table,
 *   block-FP4 expert FFNs  down( SiLU(gate x) * (up x) ),
 *   combine  y[t] = sum_j w[t,j] * E_{id[t,j]}(x[t]) + sigma(x[t].w_sg) * E_shared(x[t]).
 *
 * Sources (cited by page and section throughout this library):
 *   [Strata]    "strata-expert-paths", hanayo.cn, 2026-10-13 — an engine's MoE
 *               layer walk-through: router, grouping, expert paths, combine,
 *               staging ring, tail-skip.
 *   [FreeToken] "FreeToken 阅读笔记" (FreeToken reading notes), zhongzhuzhou.org,
 *               2026-08-23 — (layer, expert) slot pool, device-resident control
 *               flow, full-layer double buffering.
 *   [PLE]       "02-PLE 如何从 NVMe 送到 GPU" (how PLE rows travel from NVMe to
 *               the GPU), mengman.github.io, 2026-09-10 — the NVFP4 block-FP4
 *               encoding and its packed-row byte count.
 *
 * Conventions for every entry point:
 *   - Ownership: the caller owns every device buffer, pinned host buffer and
 *     stream.  The library never allocates device memory.  It owns only a
 *     ring's opaque struct and its four hipEvent_t.
 *   - Asynchrony: device work is enqueued on the given stream; no entry point
 *     synchronises, and all enqueued work is capturable into a HIP graph.  Grid
 *     shapes depend only on moe_dims, never on data: device-side counts mask
 *     unused blocks.
 *   - Errors: every entry point validates synchronously and returns a
 *     negative MOE_ERR_* code having enqueued nothing; moe_last_error() gives a
 *     human-readable detail for the calling thread.  Anomalies that only the
 *     device can see are OR-ed into the caller's int32 dev_status word
 *     (MOE_DEV_* bits), which the caller reads after its own synchronisation.
 *   - Pointers marked "device" must be device (or managed) memory; all device
 *     pointers must be 16-byte aligned (MOE_ERR_ALIGN otherwise).
 *   - Thread safety: re-entrant; a ring is driven from one host thread.
 *
 * Shapes: 1 <= T <= 2^20, 1 <= k <= E <= 1024, H % 32 == 0, I % 32 == 0,
 * 32 <= H, I <= 16384, T * H * 2 < 2^31 (x addressable with 32-bit byte
 * offsets) and T * (k + 1) < 2^30.
 * The shared expert has the same intermediate size I as a routed expert.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream handle (hipStream_t); NULL means the legacy default stream. */
struct ihipStream_t;
typedef struct ihipStream_t* moe_stream_t;

/* ---- status codes ------------------------------------------------------- */
#define MOE_OK 0
#define MOE_ERR_ARG (-1)        /* NULL pointer where one is required, bad enum/flag */
#define MOE_ERR_SHAPE (-2)      /* dims outside the supported shapes listed above */
#define MOE_ERR_ALIGN (-3)      /* a device pointer is not 16-byte aligned */
#define MOE_ERR_NOT_PINNED (-4) /* host source of a staged copy is not page-locked */
#define MOE_ERR_WORKSPACE (-5)  /* workspace missing or smaller than moe_workspace_bytes */
#define MOE_ERR_HIP (-6)        /* a HIP runtime call or kernel launch failed */
#define MOE_ERR_STATE (-7)      /* ring protocol violated (see moe_stage_h2d) */

/* ---- device status bits (OR-ed into *dev_status by kernels) ------------- */
#define MOE_DEV_BAD_EXPERT_ID 1   /* a topk id outside [0, E): its row is dropped */
#define MOE_DEV_NOT_RESIDENT 2    /* a non-empty group's slot is -1: rows are zero */
#define MOE_DEV_BAD_SLOT 4        /* a slot index >= n_slots: rows are zero */
#define MOE_DEV_TAIL_SKIPPED 8    /* moe_group_tail_skip skipped a group (rows zero) */
#define MOE_DEV_CACHE_FULL 16     /* moe_residency_update had more misses than slots to evict */
#define MOE_DEV_SYNC_TIMEOUT 32   /* a one-launch FFN's wait for another workgroup's rows timed out:
                                     that call's h / y_rows / y are undefined */

const char* moe_status_string(int status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);

/* ---- dimensions --------------------------------------------------------- */
typedef struct moe_dims {
  int32_t T; /* tokens in this call (one chunk / one verification window) */
  int32_t H; /* hidden width */
  int32_t I; /* expert intermediate width (routed and shared) */
  int32_t E; /* routed experts per layer; the shared expert is index E */
  int32_t k; /* experts picked per token */
  int32_t L; /* layers addressed by the slot table (rows of slot_table) */
} moe_dims;

/* ---- expert blob format ([PLE] "NVFP4 code 和 scale 如何反量化" and
 *      "一个 160 维向量在 packed 文件中占 90 字节") --------------------------
 *
 * One blob holds every tensor of one (layer, expert) ([FreeToken] 3, one cache
 * slot per (layer, expert)).  Its three matrices are
 *     m = 0  gate  [I rows][H columns]
 *     m = 1  up    [I rows][H columns]
 *     m = 2  down  [H rows][I columns]
 * (rows are output units; columns are the reduction axis K).
 * Each matrix is stored NVFP4-style:
 *   codes  rows * K/2 bytes.  Logically a row is K/2 bytes: byte c holds
 *          column 2c in its low nibble and column 2c+1 in its high nibble.  A
 *          nibble is an E2M1 code: bit 3 is the sign, bits 0..2 index the
 *          magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *   scales rows * K/16 bytes, OCP FP8 E4M3FN (bias 7, no infinity, 0x7F/0xFF
 *          NaN).  Scale b of a row applies to columns 16b..16b+15.
 *   global one fp32 per matrix.
 * value(r, c) = e2m1(code(r, c)) * e4m3(scale(r, c/16)) * global.
 * Placement (rows and K are multiples of 16 and 32): the rows are tiled in
 * blocks of 16.  Row block n/16 owns 8K code bytes from 8K*(n/16): the
 * 32-column chunk j of its row n%16 is the 16 bytes at 256j + 16(n%16), i.e.
 * logical bytes 16j..16j+15 of the row.  It owns K scale bytes from K*(n/16):
 * the chunks form groups of 16 (512 columns; the last group may hold fewer,
 * c_g = min(16, K/32 - 16g)); group g starts at 512g and holds 2c_g bytes per
 * row, row n%16's at 2c_g*(n%16), scale b at byte b - 32g of them.  One
 * chunk of 16 rows is thus 256 contiguous code bytes, and a row's scales of
 * one group are contiguous.
 * Section order inside a blob: gate codes, up codes, down codes, gate scales,
 * up scales, down scales, then the three fp32 globals (gate, up, down).
 * Every section starts on a 256-byte boundary.  Blobs sit in a pool at
 * pool + slot * slot_stride, slot_stride = blob_bytes rounded up to 4096.
 * Gate codes and up codes are adjacent, so the gate codes section followed by
 * the up codes section reads as one matrix of 2I rows (likewise the scales).
 */
typedef struct moe_blob_layout {
  uint64_t blob_bytes;    /* bytes up to the end of the globals */
  uint64_t slot_stride;   /* blob_bytes rounded up to a multiple of 4096 */
  uint64_t off_codes[3];  /* byte offsets of gate, up, down codes */
  uint64_t off_scales[3]; /* byte offsets of gate, up, down scales */
  uint64_t off_globals;   /* byte offset of float[3] {G_gate, G_up, G_down} */
} moe_blob_layout;

/* Host, pure.  Fills *out for widths (H, I).  MOE_ERR_SHAPE unless H and I are
 * multiples of 32 within [32, 16384]. */
int moe_blob_layout_init(int32_t H, int32_t I, moe_blob_layout* out);

/* Host, pure.  Bytes of device workspace that moe_group and moe_expert_ffn
 * need for dims d (the same buffer is passed to both, group first). */
int moe_workspace_bytes(const moe_dims* d, uint64_t* out_bytes);

/* ---- S1 + S2: router ---------------------------------------------------
 * [Strata] "显存里缓存的是什么？" (the router picks the experts and their merge
 * weights) and "还有一条会改变输出的路径" (experts are ranked per token).
 *
 * Logits: exactly one of w_router / logits_in is non-NULL.
 *   w_router  device fp32 [H][E] row-major: l[t,e] = sum_h x[t,h] * W[h,e],
 *             accumulated in fp32 (rounding point R0: fp32 logits).  Each
 *             W[h,e] is split exactly into three bf16 parts and the products
 *             (exact in fp32) are summed by bf16 MFMAs, so the only rounding
 *             is the fp32 accumulation.
 *   logits_in device fp32 [T][E]: used as given.
 * x            device bf16 bits [T][H] row-major (required: the shared gate reads it).
 * w_shared_gate device fp32 [H], 16-byte aligned:
 *              sigma[t] = 1 / (1 + exp(-sum_h x[t,h] w_sg[h])).
 * logits_out   device fp32 [T][E] or NULL: receives the logits used.
 * topk_ids     device int32 [T][k]: slot j holds the j-th largest logit; ties
 *              go to the lower expert index.
 * topk_w       device fp32 [T][k]: w_j = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0),
 *              i.e. the softmax over all E renormalised to the chosen k.
 * shared_sigma device fp32 [T].
 * Logits must be finite (NaN/inf inputs give unspecified ids).
 */
int moe_route(const moe_dims* d, const uint16_t* x, const float* w_router,
              const float* logits_in, const float* w_shared_gate,
              float* logits_out, int32_t* topk_ids, float* topk_w,
              float* shared_sigma, moe_stream_t stream);

/* ---- S3: grouping ------------------------------------------------------
 * [Strata] "路由以后，专家怎样分工？" (tokens of one layer and window that picked
 * the same expert form one group recording their inputs and output positions)
 * and "哪些专家能长期留在显存？" (the residency table maps (layer, expert) to a
 * slot or to a special not-resident value); [FreeToken] 4 (logical -> physical
 * slot rewrite on the device, no host synchronisation).
 *
 * Row space p: [0, T*k) routed rows grouped by expert (ascending expert, then
 * ascending token inside a group); [T*k, T*k+T) shared-expert rows in token
 * order.  f = t*k + j is the flat (token, slot) index.
 * topk_ids   device int32 [T][k].  Ids outside [0,E) set MOE_DEV_BAD_EXPERT_ID
 *            and are placed in no group (inv_perm -1, no row).
 * slot_table device int32 [L][E+1]; column E is the shared expert; -1 = not
 *            resident.  layer in [0, L).  n_slots bounds valid slot indices.
 * offsets    device int32 [E+2]: routed group e < E is rows
 *            [offsets[e], offsets[e+1]); offsets[E] = number of routed rows
 *            with a valid id (T*k when all are valid); offsets[E+1] = T*k + T.
 *            The shared group is always rows [T*k, T*k+T); rows
 *            [offsets[E], T*k) exist only when ids were dropped and are unused.
 * perm       device int32 [T*k]: p -> f (routed rows only).
 * inv_perm   device int32 [T*k]: f -> p (-1 for a dropped bad id).
 * group_slot device int32 [E+1]: slot_table[layer][e].
 * dev_status device int32 [1]: MOE_DEV_* bits are OR-ed in.
 * ws         device workspace of >= moe_workspace_bytes(d) bytes; it also
 *            carries the work list that moe_expert_ffn reads.
 */
int moe_group(const moe_dims* d, int32_t layer, const int32_t* topk_ids,
              const int32_t* slot_table, int32_t n_slots, int32_t* offsets,
              int32_t* perm, int32_t* inv_perm, int32_t* group_slot,
              int32_t* dev_status, void* ws, uint64_t ws_bytes,
              moe_stream_t stream);

/* ---- Partial residency (a variant): an LRU cache of expert blobs --------
 * [FreeToken] 3.3 (one LRU over (layer, expert) shared by all layers: a hit
 * refreshes the expert's last use, a fill admits a newly chosen expert,
 * eviction removes the least recently used) and 4 (per layer one device
 * kernel classifies the routed experts against the residency table, picks the
 * victims in one pass and rewrites the table; one fixed-shape transfer, masked
 * by a device-side count, moves the blobs; no host decision).
 *
 * The cache is n_slots slots of the pool (slot s at pool + s * slot_stride).
 * Its state lives on the device and belongs to the caller:
 *   slot_table [L][E+1] int32: slot of (layer, expert), or -1;
 *   slot_owner [n_slots] int32: key layer*(E+1)+e of the slot's blob, or -1;
 *   last_use   [n_slots] int32: clock of the slot's last use, -1 if never used;
 *   clock      [1] int32: ticks once per moe_residency_update.
 * Start from slot_table, slot_owner and last_use all -1 and clock 0 (or any
 * state these calls produced).
 *
 * moe_residency_update: for the window topk_ids [T][k] of `layer`, the needed
 * experts are its routed ids in [0, E) and the shared expert.  Hits refresh
 * their slot's last use.  Misses, in ascending expert order, take the least
 * recently used slots this call does not hit (ties: lower slot; never used
 * first); a victim's previous owner becomes -1 in slot_table.  fill_list
 * [E+1][2] int32 receives (key, slot) per placed miss in that order and
 * n_fill [1] their count.  More misses than evictable slots: the first ones
 * are placed, the rest stay -1 and MOE_DEV_CACHE_FULL is set in dev_status.
 * Requires E <= 1024 and n_slots <= 262144.
 *
 * moe_residency_fill: copies the blob of each (key, slot) of fill_list (first
 * *n_fill entries) from host_blobs + key * slot_stride to pool + slot *
 * slot_stride (layout->blob_bytes bytes each).  host_blobs is pinned host
 * memory the device can read (all L*(E+1) blobs, 16-byte aligned), owned by
 * the caller and unchanged until the copy is done.  Fixed grid; entries with
 * a key or slot out of range are skipped.  Run it on the stream of the update
 * and before the FFN that reads the slots: stream order publishes the blobs.
 */
int moe_residency_update(const moe_dims* d, int32_t layer, const int32_t* topk_ids,
                         int32_t* slot_table, int32_t* slot_owner, int32_t* last_use,
                         int32_t n_slots, int32_t* clock, int32_t* fill_list,
                         int32_t* n_fill, int32_t* dev_status, moe_stream_t stream);
int moe_residency_fill(const moe_dims* d, const moe_blob_layout* layout,
                       const void* host_blobs, void* pool, uint64_t pool_bytes,
                       int32_t n_slots, const int32_t* fill_list, const int32_t* n_fill,
                       moe_stream_t stream);

/* ---- Hot/cold swaps (a variant) -----------------------------------------
 * [Strata] "哪些专家能长期留在显存？" (the passages on heat and candidate pairs,
 * and on swaps and publication): each expert's heat accumulates its routing
 * counts and is multiplied by a decay (default 0.7) after every round; per
 * round, inside one layer the hottest experts outside the cache pair with the
 * coldest inside, a pair whose heat gap reaches the threshold (default 1.5)
 * is a candidate, and the candidates go by gap, at most max_swaps (default
 * 96).  A swap copies the hot expert's blob into the cold expert's slot; the
 * table names the new owner only after the copy.
 *
 * moe_heat_update: heat [L][E] fp32 (device) += the row count of each routed
 * group of this layer call, from offsets written by moe_group (ids outside
 * [0, E) have no group and do not count).
 * moe_heat_decay: every entry of heat [L][E] times decay.
 * moe_swap_plan (host, pure): heat [L][E] and slot_table [L][E+1] are HOST
 * copies; writes the round's swaps to plan [max_swaps][3] as (layer, hot
 * expert, cold expert), largest heat gap first, and their number to *n_plan.
 * Pairs form in heat order (ties to the lower expert index), a layer stops at
 * its first pair below the threshold, equal gaps go by (layer, pair index),
 * the shared expert never swaps; comparisons are taken in fp32.
 * moe_swap_apply: plan [n_plan][3] device (from moe_swap_plan); for each entry
 * whose hot expert is still out of the cache and whose cold expert is still
 * in it, copies the hot blob from host_blobs (device-readable pinned memory,
 * as for moe_residency_fill) into the cold expert's slot, then sets the hot
 * expert's table entry to that slot and the cold one's to -1.  An entry that
 * names, in its layer, an expert that an earlier entry of the plan already
 * names (as hot or cold) is skipped.  fill_scratch [n_plan][2] and n_scratch
 * [1]: device scratch.  Everything runs on `stream` in that order; kernels
 * that read the pool must be ordered after it.
 * The swaps rewrite slot_table only.  A table whose slots are also managed by
 * moe_residency_update (slot_owner, last_use) must not be passed here: the
 * LRU state would still name the cold expert as the slot's owner, and a later
 * eviction of that slot would leave the hot expert's entry pointing at another
 * expert's bytes.  Use one of the two policies per table.
 */
int moe_heat_update(const moe_dims* d, int32_t layer, const int32_t* offsets,
                    float* heat, moe_stream_t stream);
int moe_heat_decay(const moe_dims* d, float* heat, float decay, moe_stream_t stream);
int moe_swap_plan(const moe_dims* d, const float* heat, const int32_t* slot_table,
                  float threshold, int32_t max_swaps, int32_t* plan, int32_t* n_plan);
int moe_swap_apply(const moe_dims* d, const moe_blob_layout* layout,
                   const void* host_blobs, void* pool, uint64_t pool_bytes,
                   int32_t n_slots, int32_t* slot_table, const int32_t* plan,
                   int32_t n_plan, int32_t* fill_scratch, int32_t* n_scratch,
                   moe_stream_t stream);

/* ---- S3 with the route tail-skip (a variant) ---------------------------
 * [Strata] "少算这些专家，会付出什么代价？" and the skip-condition passage before it
 * (default threshold 7, ranks from zero; the kept experts' weights are not
 * renormalised).
 *
 * moe_group with one more rule, over the T tokens of this call (the window):
 * a routed expert that is not resident (slot -1) and that every token of the
 * window that picked it ranks at skip_rank or later (slot j >= skip_rank) is
 * skipped.  Its rows are zero as for any non-resident group and moe_combine
 * adds nothing for them, so the output moves by exactly the skipped w_j E_j(x)
 * terms; it sets MOE_DEV_TAIL_SKIPPED instead of MOE_DEV_NOT_RESIDENT.  A
 * non-resident expert that some token ranks earlier still sets
 * MOE_DEV_NOT_RESIDENT.  skip_rank <= 0 (or >= k) skips nothing.
 * n_skipped  device int32 [1] or NULL: receives the number of skipped experts.
 * Every other argument, the validation and the results are moe_group's.
 */
int moe_group_tail_skip(const moe_dims* d, int32_t layer, const int32_t* topk_ids,
                        const int32_t* slot_table, int32_t n_slots, int32_t skip_rank,
                        int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        int32_t* group_slot, int32_t* dev_status, int32_t* n_skipped,
                        void* ws, uint64_t ws_bytes, moe_stream_t stream);

/* ---- S1 + S2 + S3 together ---------------------------------------------
 * moe_route followed by moe_group on the same stream, with exactly their
 * arguments, validation and results (every output bit-identical).  For small
 * windows (T <= 16, T*k <= 256) the top-k and the grouping run in one kernel
 * (after the router GEMM when w_router is given), which saves a launch and the
 * ids' round trip through memory; otherwise the two calls' kernels are
 * launched in turn. */
int moe_route_group(const moe_dims* d, int32_t layer, const uint16_t* x,
                    const float* w_router, const float* logits_in,
                    const float* w_shared_gate, float* logits_out,
                    int32_t* topk_ids, float* topk_w, float* shared_sigma,
                    const int32_t* slot_table, int32_t n_slots, int32_t* offsets,
                    int32_t* perm, int32_t* inv_perm, int32_t* group_slot,
                    int32_t* dev_status, void* ws, uint64_t ws_bytes,
                    moe_stream_t stream);

/* ---- S4: expert FFNs ---------------------------------------------------
 * [Strata] "路由以后，专家怎样分工？" and "CPU 怎样把剩下的专家算完？" (gate/up,
 * activation, the intermediate re-encoded for the next kernel, down).
 * For every row p of group e (routed or shared) with token t:
 *   g = G_gate * sum_c x[t,c] Wg[i,c],  u = G_up * sum_c x[t,c] Wu[i,c]
 *   h[p,i] = bf16_rne( g / (1 + exp(-g)) * u )                 (rounding point R1)
 *   Y[p,n] = bf16_rne( G_down * sum_i h[p,i] Wd[n,i] )          (rounding point R3)
 * with the matrices decoded from the blob at pool + group_slot[e]*slot_stride.
 * Weight codes and scales multiply exactly; sums are fp32.
 * x          device bf16 [T][H].
 * pool       device, pool_bytes long (at least one slot_stride, MOE_ERR_ARG
 *            otherwise); every slot used must lie inside it.
 * h          device bf16 [T*k+T][I] (intermediate, also an output).
 * y_rows     device bf16 [T*k+T][H]: unweighted expert outputs per row.
 * Rows of a group whose slot is -1 or >= pool_bytes/slot_stride are written
 * as zeros and flagged in dev_status.
 * offsets/perm/group_slot/ws: exactly as written by moe_group on the same stream.
 */
int moe_expert_ffn(const moe_dims* d, const uint16_t* x, const void* pool,
                   uint64_t pool_bytes, const moe_blob_layout* layout,
                   const int32_t* offsets, const int32_t* perm,
                   const int32_t* group_slot, uint16_t* h, uint16_t* y_rows,
                   int32_t* dev_status, void* ws, uint64_t ws_bytes,
                   moe_stream_t stream);

/* The two stages of moe_expert_ffn (same definition as above), selectively:
 * stages = 1 runs gate/up and the activation (writes h), 2 runs the down
 * projection (reads h, writes y_rows), 3 runs both and is moe_expert_ffn.  A
 * down stage reads the h written by a gate/up stage with the same inputs
 * earlier on the same stream.  For callers that time the stages apart or put
 * other work between them.
 * ev_start, ev_stop: hipEvent_t handles created by the caller, or NULL.  When
 * set, the device records ev_start when the first launched kernel starts and
 * ev_stop when the last one ends (hipExtLaunchKernelGGL), so their elapsed
 * time is the stages' own duration.  Leave both NULL under graph capture.
 * MOE_ERR_ARG for stages outside 1..3; every other argument as for
 * moe_expert_ffn. */
int moe_expert_ffn_stages(const moe_dims* d, const uint16_t* x, const void* pool,
                          uint64_t pool_bytes, const moe_blob_layout* layout,
                          const int32_t* offsets, const int32_t* perm,
                          const int32_t* group_slot, uint16_t* h, uint16_t* y_rows,
                          int32_t* dev_status, void* ws, uint64_t ws_bytes,
                          int32_t stages, void* ev_start, void* ev_stop,
                          moe_stream_t stream);

/* ---- S4 + S5 together ----------------------------------------------------
 * moe_expert_ffn followed by moe_combine on the same stream, with exactly
 * their arguments, validation and results (h, y_rows and y bit-identical).
 * For decode windows (T <= 64 and k <= 16 on the weight-streaming path, and
 * (H, I) of (2048, 512), (4096, 2048) or (512, 256)) both FFN stages and the
 * combine run as one launch ([FreeToken] 3.5: a step's control flow stays on
 * the device): the down projection of a tile waits, inside the launch, for
 * the workgroups that write its h rows, and the wavefront that completes the
 * last down item of a block of output columns marks that block for its
 * workgroup to combine for every token ([Strata] "路由以后，专家怎样分工？": each
 * token's expert outputs are weighted and summed once all have arrived).
 * The waits are bounded; should one time out (only if the device cannot keep
 * the launch's workgroups resident together, e.g. other work holds its
 * compute units for a long time), MOE_DEV_SYNC_TIMEOUT is set and h, y_rows
 * and y are undefined.  One launch saves two launches' host cost; inside a
 * HIP graph the separate launches overlap their start-up and were measured
 * slightly faster on MI355X.
 * ev_start, ev_stop as for moe_expert_ffn_stages (they bracket the FFN
 * launch, and the combine when it is part of it). */
int moe_expert_ffn_combine(const moe_dims* d, const uint16_t* x, const void* pool,
                           uint64_t pool_bytes, const moe_blob_layout* layout,
                           const int32_t* offsets, const int32_t* perm,
                           const int32_t* group_slot, const int32_t* inv_perm,
                           const float* topk_w, const float* shared_sigma, uint16_t* h,
                           uint16_t* y_rows, uint16_t* y, int32_t* dev_status, void* ws,
                           uint64_t ws_bytes, void* ev_start, void* ev_stop, moe_stream_t stream);

/* ---- S4 down + S5 together ---------------------------------------------
 * moe_expert_ffn_stages (stages 2) followed by moe_combine on the same stream,
 * with exactly their arguments, validation and results (y_rows and y
 * bit-identical).  x: as for moe_expert_ffn_stages (validated, not read); h:
 * the rows a gate/up stage wrote earlier on the same stream, read only.  For
 * decode windows on the weight-streaming path with I = 512, T <= 16 and
 * k <= 16 the two run as one launch ([Strata] "路由以后，专家怎样分工？": a
 * token's expert outputs are weighted and summed once all of them have
 * arrived): two workgroups share each block of 16 output columns, each
 * computing the Y rows of half the tiles for it, and the second of the two to
 * finish combines the block for every token in moe_combine's arithmetic.
 * Nothing in the launch waits.  Each block's counter lives in ws (zeroed by
 * the grouping that wrote ws's work list, and again after each use).
 * Y rows are stored device-coherently (written through) so the combining
 * workgroup reads them across XCDs.  Other shapes run the two launches.
 * ev_start, ev_stop as for moe_expert_ffn_stages. */
int moe_expert_ffn_down_combine(const moe_dims* d, const uint16_t* x, const void* pool,
                                uint64_t pool_bytes, const moe_blob_layout* layout,
                                const int32_t* offsets, const int32_t* perm,
                                const int32_t* group_slot, const int32_t* inv_perm,
                                const float* topk_w, const float* shared_sigma, const uint16_t* h,
                                uint16_t* y_rows, uint16_t* y, int32_t* dev_status, void* ws,
                                uint64_t ws_bytes, void* ev_start, void* ev_stop,
                                moe_stream_t stream);

/* ---- S1 + S2 + S3 + S4 together ---------------------------------------
 * moe_route_group followed by moe_expert_ffn_stages on the same stream, with
 * exactly their arguments, validation and results (every output of both
 * bit-identical); stages is 1 (gate/up) or 3 (gate/up and down).  For decode
 * windows with drawn logits (logits_in, not w_router; T <= 16, T*k <= 256,
 * E <= 1024, T*k < 16 E) the routing runs inside the gate/up launch
 * ([FreeToken] 3.5: a step's control flow stays on the device): every
 * workgroup selects the window's top-k and groups it into its own work list,
 * so the weight stream starts without a routing kernel or a work-list round
 * trip through memory before it, and one more workgroup stores the routing
 * outputs (ids, weights, sigma, offsets, perm, inv_perm, group_slot, status,
 * and the workspace's work list for the down stage).  Otherwise the two
 * calls' kernels are launched in turn.  ev_start, ev_stop bracket the FFN
 * launches, which then include the routing. */
int moe_route_group_ffn(const moe_dims* d, int32_t layer, const uint16_t* x,
                        const float* w_router, const float* logits_in,
                        const float* w_shared_gate, float* logits_out,
                        int32_t* topk_ids, float* topk_w, float* shared_sigma,
                        const int32_t* slot_table, int32_t n_slots, int32_t* offsets,
                        int32_t* perm, int32_t* inv_perm, int32_t* group_slot,
                        const void* pool, uint64_t pool_bytes, const moe_blob_layout* layout,
                        uint16_t* h, uint16_t* y_rows, int32_t* dev_status, void* ws,
                        uint64_t ws_bytes, int32_t stages, void* ev_start, void* ev_stop,
                        moe_stream_t stream);

/* ---- S1 + S2 + S3 + S4 + S5 together ---------------------------------
 * moe_route_group_ffn (stages 3) followed by moe_combine on the same stream,
 * with exactly their arguments, validation and results (every output of the
 * three calls bit-identical, y included).  For decode windows with drawn
 * logits (logits_in, not w_router; T <= 16, T*k <= 256, k <= 16, E <= 1024,
 * T*k < 16 E, and (H, I) of (2048, 512), (4096, 2048) or (512, 256)) the
 * whole layer runs as one launch ([FreeToken] 3.5: a decode step's control
 * flow stays on the device; [Strata] "路由以后，专家怎样分工？": the expert
 * outputs of a token are weighted and summed once all have arrived):
 *  - every workgroup routes and groups the window into its own work list;
 *  - one workgroup zeroes the launch's counters in ws, stores the routing
 *    outputs and then sets a ready flag in ws; the others stream the gate/up
 *    weights and count each tile's h rows once the flag is set;
 *  - the down projection of a tile waits, inside the launch, for its h rows
 *    (its weights were requested before the gate/up walk), and the wavefront
 *    that completes a block of output columns combines that block for every
 *    token.
 * The waits are bounded; should one time out (only if the device cannot keep
 * the launch's workgroups resident together), MOE_DEV_SYNC_TIMEOUT is set and
 * h, y_rows and y are undefined.  ws needs no preparation: the counters are
 * zeroed inside the launch before any is counted, and the flag is cleared
 * again by the launch's last workgroup.  Calls that share one ws must not
 * overlap in time.  Otherwise (other shapes, or w_router) the calls' own
 * launches run in turn.  ev_start, ev_stop bracket the layer's launch (with
 * the routing and the combine in it), or the FFN launches otherwise.
 * MOE_ERR_ARG if y is NULL; every other argument as for moe_route_group_ffn
 * and moe_combine. */
int moe_route_group_ffn_combine(const moe_dims* d, int32_t layer, const uint16_t* x,
                                const float* w_router, const float* logits_in,
                                const float* w_shared_gate, float* logits_out,
                                int32_t* topk_ids, float* topk_w, float* shared_sigma,
                                const int32_t* slot_table, int32_t n_slots, int32_t* offsets,
                                int32_t* perm, int32_t* inv_perm, int32_t* group_slot,
                                const void* pool, uint64_t pool_bytes,
                                const moe_blob_layout* layout, uint16_t* h, uint16_t* y_rows,
                                uint16_t* y, int32_t* dev_status, void* ws, uint64_t ws_bytes,
                                void* ev_start, void* ev_stop, moe_stream_t stream);

/* ---- S4, MX variant: MXFP4 experts on the scaled MFMA ---------------------
 * [FreeToken] notes that the DeepSeek-V4-Flash experts are natively MXFP4; the
 * pages do not define the format, which is read as OCP Microscaling (MX):
 *   E8M0   a scale byte b is 2^(b - 127); 255 is NaN.
 *   MXFP4  32 values along K share one E8M0 scale; elements are E2M1 codes
 *          (nibbles as in the NVFP4 blob); there is no global scale.
 *   MXFP8  32 values share an E8M0 scale X = 2^(floor(log2 amax) - 8), the
 *          exponent clamped to [-127, 127] (a zero block takes -127); each
 *          element is v / X rounded to the nearest E4M3FN value (ties to the
 *          even code), saturating at +-448.
 *
 * MX blob (moe_blob_layout_init_mx): the three matrices' codes exactly as in the
 * NVFP4 blob (same tiling and section order), then their E8M0 scales, rows*K/32
 * bytes per matrix, every section on a 256-byte boundary.  No globals:
 * off_globals == blob_bytes.  Scale placement: each 16-row block owns K/2
 * bytes from (K/2)*(n/16); inside, group g of four 32-value blocks (128
 * columns, one step of the scaled MFMA) takes the 64 bytes from 64g, row
 * n%16's four bytes at 4(n%16), block b at byte b%4 of them.  So the scale of
 * (row n, block b) sits at (K/2)(n/16) + 64(b/4) + 4(n%16) + b%4.
 * Requires H and I multiples of 128 in [128, 16384] (MOE_ERR_SHAPE otherwise).
 */
int moe_blob_layout_init_mx(int32_t H, int32_t I, moe_blob_layout* out);

/* Host, pure.  Bytes of the MX activation workspace that moe_expert_ffn_mx
 * needs for d.  Layout (each section from a 256-byte boundary, in order):
 *   xq [T][H] E4M3 codes of x, xs [T][SX] their E8M0 scales,
 *   hq [T*k+T][I] E4M3 codes of h, hs [T*k+T][SI] their E8M0 scales,
 * where a scale row holds H/32 (I/32) bytes and is padded to SX = H/32 (SI =
 * I/32) rounded up to a multiple of 16 (padding bytes undefined).  After a
 * gate/up stage, hq/hs hold MXFP8(h) for the rows that stage wrote.  That is
 * the layout when T*k >= 16 E (the grouped GEMM).  Below, the FFN streams the
 * weights through bf16 MFMAs instead, and the workspace holds
 *   xb [T][H] bf16, the values of MXFP8(x); hb [T*k+T][I] bf16, those of
 *   MXFP8(h) (written by the down stage before it reads them). */
int moe_mx_workspace_bytes(const moe_dims* d, uint64_t* out_bytes);

/* MXFP8 quantisation (definition above) of bf16 rows x [rows][K] (device,
 * 16-byte aligned; K a positive multiple of 32) into codes [rows][K] (device,
 * 8-byte aligned) and scales [rows][K/32] (device), on stream.  The gate/up
 * stage of moe_expert_ffn_mx applies it to x. */
int moe_quantize_mxfp8(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes,
                       uint8_t* scales, moe_stream_t stream);

/* The expert FFN of S4 on MX blobs:
 *   x^ = MXFP8(x[t])                                               (rounding point RA)
 *   g = sum_c x^[c] Wg[i,c],  u = sum_c x^[c] Wu[i,c]   (Wg, Wu, Wd: MXFP4 values)
 *   h[p,i] = bf16_rne( g / (1 + exp(-g)) * u )                     (R1)
 *   h^ = MXFP8(h[p])                                               (RA)
 *   Y[p,n] = bf16_rne( sum_i h^[i] Wd[n,i] )                       (R3)
 * Products of codes and scales are exact; sums are fp32.  The MX workspace
 * mx_ws (device, 256-byte aligned, at least moe_mx_workspace_bytes; contents
 * as documented there) carries x^ and h^ between the stages.  As for
 * moe_expert_ffn, groups averaging >= 16 rows (T*k >= 16 E) run as a grouped
 * GEMM on the scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, FP8 x FP4 with
 * their E8M0 scales); smaller ones stream the weights through bf16 MFMAs on
 * the bf16 values of x^ and h^ (exact).  layout must equal
 * moe_blob_layout_init_mx(H, I).  stages, ev_start and ev_stop as for
 * moe_expert_ffn_stages, except that the events bracket the GEMM kernels
 * only; the gate/up stage first quantises x (a kernel before them).  Every other
 * argument and the handling of missing slots as for moe_expert_ffn. */
int moe_expert_ffn_mx(const moe_dims* d, const uint16_t* x, const void* pool,
                      uint64_t pool_bytes, const moe_blob_layout* layout,
                      const int32_t* offsets, const int32_t* perm,
                      const int32_t* group_slot, uint16_t* h, uint16_t* y_rows,
                      int32_t* dev_status, void* ws, uint64_t ws_bytes, void* mx_ws,
                      uint64_t mx_ws_bytes, int32_t stages, void* ev_start, void* ev_stop,
                      moe_stream_t stream);

/* ---- S1 + S2 + S3 + S4 together, MX experts --------------------------------
 * moe_route_group followed by moe_expert_ffn_mx on the same stream, with
 * exactly their arguments, validation and results (every output of both
 * bit-identical); stages is 1 (gate/up) or 3 (gate/up and down).  For decode
 * windows (T <= 16, T*k <= 256, T*k < 16 E) the one route + group kernel also
 * writes the MX FFN's A rows into mx_ws (the bf16 values of MXFP8(x);
 * [FreeToken] 2.1, the format read as OCP MX), so the FFN begins with its
 * gate/up kernel: one launch fewer per layer ([FreeToken] 3.5: a step's
 * control flow stays on the device).  Otherwise the two calls' kernels are
 * launched in turn.  ev_start, ev_stop bracket the FFN launches. */
int moe_route_group_ffn_mx(const moe_dims* d, int32_t layer, const uint16_t* x,
                           const float* w_router, const float* logits_in,
                           const float* w_shared_gate, float* logits_out,
                           int32_t* topk_ids, float* topk_w, float* shared_sigma,
                           const int32_t* slot_table, int32_t n_slots, int32_t* offsets,
                           int32_t* perm, int32_t* inv_perm, int32_t* group_slot,
                           const void* pool, uint64_t pool_bytes,
                           const moe_blob_layout* layout, uint16_t* h, uint16_t* y_rows,
                           int32_t* dev_status, void* ws, uint64_t ws_bytes, void* mx_ws,
                           uint64_t mx_ws_bytes, int32_t stages, void* ev_start,
                           void* ev_stop, moe_stream_t stream);

/* moe_expert_ffn_mx for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, hosts that forbid
 * hipMalloc.  Same computation, arguments and results as moe_expert_ffn_mx
 * with stages as there, except that the MX workspace (mx_ws) is not an
 * argument: it is a static device array inside the library, 32 MiB (33554432
 * bytes) per GPU, held from the first call on that GPU until the process
 * ends.  No timing events.
 * Limit: dims whose moe_mx_workspace_bytes exceeds 32 MiB are refused with
 * MOE_ERR_WORKSPACE, having enqueued nothing (e.g. T = 4096 at H = 2048,
 * I = 512, k = 10 fits; T = 8192 does not).
 * Set-up: the first call on a device looks up that device's address of the
 * array (hipGetSymbolAddress, with the device current); make it outside any
 * graph capture.  The call allocates nothing: no hipMalloc, no hipFree.
 * Sharing: every call on one GPU uses that GPU's one array, which keeps the
 * last call's contents.  Calls that overlap on one GPU (two streams, two
 * threads, two captured graphs replayed concurrently) race on it and must be
 * ordered by the caller; a gate/up stage and the down stage that reads its
 * quantised h must not have another call's gate/up stage between them. */
int moe_expert_ffn_mx_noalloc(const moe_dims* d, const uint16_t* x, const void* pool,
                              uint64_t pool_bytes, const moe_blob_layout* layout,
                              const int32_t* offsets, const int32_t* perm,
                              const int32_t* group_slot, uint16_t* h, uint16_t* y_rows,
                              int32_t* dev_status, void* ws, uint64_t ws_bytes, int32_t stages,
                              moe_stream_t stream);

/* ---- S5: combine -------------------------------------------------------
 * [Strata] "路由以后，专家怎样分工？" (each expert output times its router weight,
 * summed, plus the gated shared-expert contribution) and "少算这些专家，会付出
 * 什么代价？" (the output is linear in the weighted expert terms).
 *   y[t] = bf16_rne( sum_{j<k} w[t,j] * Y[inv_perm[t*k+j]] + sigma[t] * Y[T*k+t] )
 * accumulated in fp32 in exactly this order (rounding point R2); no
 * renormalisation.  A slot whose inv_perm is -1 contributes nothing.
 */
int moe_combine(const moe_dims* d, const uint16_t* y_rows,
                const int32_t* inv_perm, const float* topk_w,
                const float* shared_sigma, uint16_t* y, moe_stream_t stream);

/* ---- S6: two-slot staging ring ([Strata] "PCIe 搬运怎样与计算重叠？";
 *      [FreeToken] 3.1 full-layer double buffering) --------------------------
 * Two device slots of slot_bytes each, written by a copy stream and read by a
 * compute stream.  Per slot s the ring holds events copied[s] and used[s]:
 *   moe_stage_h2d: on copy_stream wait used[s] (the last release of s), then
 *     hipMemcpyAsync(slot s <- pinned host src), then record copied[s].
 *     Slots are used alternately 0,1,0,1...; *out_slot receives s.  The source
 *     must be page-locked (MOE_ERR_NOT_PINNED otherwise) and bytes <= slot_bytes.
 *     MOE_ERR_STATE if slot s was staged but not yet released.
 *   moe_ring_acquire: compute stream waits copied[s]; s must be staged.
 *   moe_ring_release: records used[s] on the compute stream after the reads of
 *     s; s must be acquired.  A later stage into s waits for it.
 * A slot's data is valid for reads enqueued on the compute stream between its
 * acquire and its release.
 */
typedef struct moe_ring moe_ring;
int moe_ring_create(void* slot0, void* slot1, uint64_t slot_bytes,
                    moe_stream_t copy_stream, moe_ring** out);
int moe_stage_h2d(moe_ring* ring, const void* pinned_host_src, uint64_t bytes,
                  int32_t* out_slot);
int moe_ring_acquire(moe_ring* ring, int32_t slot, moe_stream_t compute);
int moe_ring_release(moe_ring* ring, int32_t slot, moe_stream_t compute);
int moe_ring_slot_ptr(moe_ring* ring, int32_t slot, void** out);
int moe_ring_destroy(moe_ring* ring);

/* ---- test hook ----------------------------------------------------------------
 * For the tests of moe_expert_ffn_combine's bounded wait only: sets the poll
 * limit of that launch's in-kernel waits and a count added to every tile
 * target (a target that is never reached makes each wait give up after the
 * limit, set MOE_DEV_SYNC_TIMEOUT, and let every wavefront end).  (-1, 0)
 * restores the defaults.  Applies to launches enqueued afterwards, from every
 * thread of the process; not for production use.
 */
void moe_debug_set_fused_wait(int spin_limit, int extra_target);

/* ---- measurement probes ------------------------------------------------------
 * Not part of the layer.  Kernels that measure what this GPU reaches, so a
 * roofline fraction against a published peak can be read beside the measured
 * one ([Strata] "PCIe 搬运怎样与计算重叠？": a claimed rate needs a trace on
 * the device).  Each only enqueues on `stream`; time them with events on it.
 *
 * moe_probe_hbm_read: reads bytes of buf once, 1 KiB per wavefront
 *   instruction, 8 KiB per wavefront per loop trip, over `grid` workgroups of
 *   256 threads.  buf: device, 16-byte aligned, bytes a positive multiple of
 *   8192.  sink: one device uint32 that is written only if the folded words
 *   equal a constant (a guard against the loads being dropped), so its content
 *   is unchanged for ordinary data.  MOE_ERR_ARG / MOE_ERR_ALIGN on bad input.
 * moe_probe_mfma: `grid` workgroups of 4 wavefronts, each wavefront issuing
 *   `iters` x 4 back-to-back MFMAs on register operands.  kind 0:
 *   v_mfma_f32_32x32x16_bf16 (32768 flop each); kind 1: the scaled
 *   16x16x128 MFMA with E4M3 A and E2M1 B (65536 flop each); kind 2: the same
 *   with E4M3 on both sides.  sink: device float[grid * 256], each lane's sum
 *   of its four accumulators.  grid in [1, 2^16], iters in [1, 2^20].
 * moe_probe_scaled_mfma: the arithmetic of the MX grouped GEMM's instruction
 *   ([FreeToken] "FreeToken 阅读笔记" §2.1: the experts are MXFP4), one
 *   v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 A, E2M1 B, C = 0) per wavefront,
 *   n wavefronts; split = 1 issues the gate/up pair instead (A cut into its
 *   codes of magnitude >= 2 and the rest, two MFMAs into one accumulator).
 *   Operands lane by lane, all device int32 arrays, lane l of wavefront w at
 *   index 64 w + l: a [n*64][8] (the lane's 32 E4M3 bytes, little-endian),
 *   b [n*64][4] (32 E2M1 nibbles, low nibble first), sa, sb [n*64] (E8M0 scale
 *   in the low byte).  Lane (i, j) = l % 16, l / 16 holds A row i, K 16 j ..
 *   16 j + 15 and 64 + 16 j .. 64 + 16 j + 15; B column i, K 32 j .. 32 j +
 *   31; the scales of row / column i, K block j (32 j .. 32 j + 31).
 *   d [n*64][4]: D[4 (l / 16) + e][l % 16] at lane l, element e.  n in
 *   [1, 2^16]; split 0 or 1; MOE_ERR_ARG otherwise.
 */
int moe_probe_hbm_read(const void* buf, uint64_t bytes, int32_t grid,
                       uint32_t* sink, moe_stream_t stream);
int moe_probe_mfma(int32_t kind, int32_t grid, int32_t iters, float* sink,
                   moe_stream_t stream);
int moe_probe_scaled_mfma(const int32_t* a, const int32_t* b,
                          const int32_t* sa, const int32_t* sb, int32_t n,
                          int32_t split, float* d, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
