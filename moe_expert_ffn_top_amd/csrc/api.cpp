// libmoe C ABI: argument validation, status codes, launches on the caller's stream.
// Semantics of every entry point are documented in include/moe.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "moe_common.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_width(int32_t v, const char* name) {
  if (v < 32 || v > 16384 || v % 32 != 0)
    return fail(MOE_ERR_SHAPE, "%s = %d: must be a multiple of 32 in [32, 16384]", name, v);
  return MOE_OK;
}

int check_dims(const moe_dims* d) {
  if (!d) return fail(MOE_ERR_ARG, "dims is NULL");
  if (d->T < 1) return fail(MOE_ERR_SHAPE, "T = %d: must be >= 1", d->T);
  if (d->T > (1 << 20)) return fail(MOE_ERR_SHAPE, "T = %d: must be <= 2^20", d->T);
  int r = check_width(d->H, "H");
  if (r) return r;
  if ((r = check_width(d->I, "I"))) return r;
  if (d->E < 1 || d->E > 1024) return fail(MOE_ERR_SHAPE, "E = %d: must be in [1, 1024]", d->E);
  if (d->k < 1 || d->k > d->E) return fail(MOE_ERR_SHAPE, "k = %d: must be in [1, E = %d]", d->k, d->E);
  if (d->L < 1) return fail(MOE_ERR_SHAPE, "L = %d: must be >= 1", d->L);
  if ((int64_t)d->T * (d->k + 1) > INT32_MAX / 2) return fail(MOE_ERR_SHAPE, "T * (k + 1) too large");
  if ((int64_t)d->T * d->H * 2 > INT32_MAX) return fail(MOE_ERR_SHAPE, "T * H * 2 = %lld bytes of x: must be < 2^31",
                                                       (long long)d->T * d->H * 2);
  return MOE_OK;
}

#define REQUIRE(p, align, name)                                                                   \
  do {                                                                                            \
    if (!(p)) return fail(MOE_ERR_ARG, "%s is NULL", name);                                       \
    if (!aligned((p), (align))) return fail(MOE_ERR_ALIGN, "%s is not %d-byte aligned", name, (int)(align)); \
  } while (0)

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace moe {
int record_error(int code, const char* msg) {
  g_last_error = msg;
  return code;
}
}  // namespace moe

extern "C" {

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
    case MOE_ERR_NOT_PINNED: return "MOE_ERR_NOT_PINNED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_STATE: return "MOE_ERR_STATE";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_version(void) { return "libmoe 0.1 (gfx950)"; }

int moe_blob_layout_init(int32_t H, int32_t I, moe_blob_layout* out) {
  if (!out) return fail(MOE_ERR_ARG, "out is NULL");
  int r = check_width(H, "H");
  if (r) return r;
  if ((r = check_width(I, "I"))) return r;
  const uint64_t rows[3] = {(uint64_t)I, (uint64_t)I, (uint64_t)H};
  const uint64_t kk[3] = {(uint64_t)H, (uint64_t)H, (uint64_t)I};
  uint64_t off = 0;
  for (int m = 0; m < 3; m++) {
    out->off_codes[m] = off;
    off = moe::align256(off + rows[m] * kk[m] / 2);
  }
  for (int m = 0; m < 3; m++) {
    out->off_scales[m] = off;
    off = moe::align256(off + rows[m] * kk[m] / 16);
  }
  out->off_globals = off;
  out->blob_bytes = off + 12;
  out->slot_stride = (out->blob_bytes + 4095) & ~uint64_t(4095);
  return ok();
}

int moe_workspace_bytes(const moe_dims* d, uint64_t* out_bytes) {
  int r = check_dims(d);
  if (r) return r;
  if (!out_bytes) return fail(MOE_ERR_ARG, "out_bytes is NULL");
  *out_bytes = moe::ws_layout(*d).total;
  return ok();
}

namespace {

int validate_route(const moe_dims* d, const uint16_t* x, const float* w_router, const float* logits_in,
                   const float* w_shared_gate, float* logits_out, int32_t* topk_ids, float* topk_w,
                   float* shared_sigma) {
  int r = check_dims(d);
  if (r) return r;
  if ((w_router == nullptr) == (logits_in == nullptr))
    return fail(MOE_ERR_ARG, "exactly one of w_router and logits_in must be given");
  if (w_router && !logits_out) return fail(MOE_ERR_ARG, "logits_out is required when w_router is given");
  REQUIRE(x, 16, "x");
  REQUIRE(w_shared_gate, 16, "w_shared_gate");
  REQUIRE(topk_ids, 4, "topk_ids");
  REQUIRE(topk_w, 4, "topk_w");
  REQUIRE(shared_sigma, 4, "shared_sigma");
  if (w_router) REQUIRE(w_router, 16, "w_router");
  if (logits_in) REQUIRE(logits_in, 4, "logits_in");
  if (logits_out) REQUIRE(logits_out, 4, "logits_out");
  return MOE_OK;
}

int validate_group(const moe_dims* d, int32_t layer, const int32_t* topk_ids, const int32_t* slot_table,
                   int32_t n_slots, int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* group_slot,
                   int32_t* dev_status, void* ws, uint64_t ws_bytes) {
  int r = check_dims(d);
  if (r) return r;
  if (layer < 0 || layer >= d->L) return fail(MOE_ERR_ARG, "layer = %d outside [0, L = %d)", layer, d->L);
  if (n_slots < 0) return fail(MOE_ERR_ARG, "n_slots = %d < 0", n_slots);
  REQUIRE(topk_ids, 4, "topk_ids");
  REQUIRE(slot_table, 4, "slot_table");
  REQUIRE(offsets, 4, "offsets");
  REQUIRE(perm, 4, "perm");
  REQUIRE(inv_perm, 4, "inv_perm");
  REQUIRE(group_slot, 4, "group_slot");
  REQUIRE(dev_status, 4, "dev_status");
  REQUIRE(ws, 16, "ws");
  const uint64_t need = moe::ws_layout(*d).total;
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %llu bytes < required %llu", (unsigned long long)ws_bytes,
                (unsigned long long)need);
  return MOE_OK;
}

// The logits copy (logits_in -> logits_out) and, with w_router, the logits GEMM.
int route_logits(const moe_dims* d, const uint16_t* x, const float* w_router, const float* logits_in,
                 float* logits_out, hipStream_t s, const float** lg) {
  *lg = logits_in;
  if (w_router) {
    hipError_t e = moe::launch_router_matrix(*d, x, w_router, logits_out, s);
    if (e != hipSuccess) return hip_status(e, "router logits launch");
    *lg = logits_out;
  } else if (logits_out && logits_out != logits_in) {
    hipError_t e = hipMemcpyAsync(logits_out, logits_in, (size_t)d->T * d->E * sizeof(float),
                                  hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e, "logits copy");
  }
  return MOE_OK;
}

}  // namespace

int moe_route(const moe_dims* d, const uint16_t* x, const float* w_router, const float* logits_in,
              const float* w_shared_gate, float* logits_out, int32_t* topk_ids, float* topk_w, float* shared_sigma,
              moe_stream_t stream) {
  int r = validate_route(d, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w, shared_sigma);
  if (r) return r;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float* lg = nullptr;
  if ((r = route_logits(d, x, w_router, logits_in, logits_out, s, &lg))) return r;
  return hip_status(moe::launch_topk(*d, lg, x, w_shared_gate, topk_ids, topk_w, shared_sigma, s), "top-k launch");
}

int moe_group(const moe_dims* d, int32_t layer, const int32_t* topk_ids, const int32_t* slot_table, int32_t n_slots,
              int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* group_slot, int32_t* dev_status, void* ws,
              uint64_t ws_bytes, moe_stream_t stream) {
  int r = validate_group(d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status, ws,
                         ws_bytes);
  if (r) return r;
  return hip_status(moe::launch_group(*d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot,
                                      dev_status, ws, reinterpret_cast<hipStream_t>(stream)),
                    "group launch");
}

int moe_group_tail_skip(const moe_dims* d, int32_t layer, const int32_t* topk_ids, const int32_t* slot_table,
                        int32_t n_slots, int32_t skip_rank, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        int32_t* group_slot, int32_t* dev_status, int32_t* n_skipped, void* ws, uint64_t ws_bytes,
                        moe_stream_t stream) {
  int r = validate_group(d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status, ws,
                         ws_bytes);
  if (r) return r;
  if (n_skipped) REQUIRE(n_skipped, 4, "n_skipped");
  return hip_status(moe::launch_group(*d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot,
                                      dev_status, ws, reinterpret_cast<hipStream_t>(stream), skip_rank, n_skipped),
                    "group launch");
}

int moe_residency_update(const moe_dims* d, int32_t layer, const int32_t* topk_ids, int32_t* slot_table,
                         int32_t* slot_owner, int32_t* last_use, int32_t n_slots, int32_t* clock, int32_t* fill_list,
                         int32_t* n_fill, int32_t* dev_status, moe_stream_t stream) {
  int r = check_dims(d);
  if (r) return r;
  if (layer < 0 || layer >= d->L) return fail(MOE_ERR_ARG, "layer = %d outside [0, L = %d)", layer, d->L);
  if (n_slots < 1 || n_slots > moe::kMaxResidencySlots)
    return fail(MOE_ERR_ARG, "n_slots = %d outside [1, %d]", n_slots, moe::kMaxResidencySlots);
  REQUIRE(topk_ids, 4, "topk_ids");
  REQUIRE(slot_table, 4, "slot_table");
  REQUIRE(slot_owner, 4, "slot_owner");
  REQUIRE(last_use, 4, "last_use");
  REQUIRE(clock, 4, "clock");
  REQUIRE(fill_list, 8, "fill_list");
  REQUIRE(n_fill, 4, "n_fill");
  REQUIRE(dev_status, 4, "dev_status");
  return hip_status(moe::launch_residency(*d, layer, topk_ids, slot_table, slot_owner, last_use, n_slots, clock,
                                          fill_list, n_fill, dev_status, reinterpret_cast<hipStream_t>(stream)),
                    "residency launch");
}

int moe_residency_fill(const moe_dims* d, const moe_blob_layout* layout, const void* host_blobs, void* pool,
                       uint64_t pool_bytes, int32_t n_slots, const int32_t* fill_list, const int32_t* n_fill,
                       moe_stream_t stream) {
  int r = check_dims(d);
  if (r) return r;
  if (!layout) return fail(MOE_ERR_ARG, "layout is NULL");
  if (n_slots < 1) return fail(MOE_ERR_ARG, "n_slots = %d < 1", n_slots);
  REQUIRE(host_blobs, 16, "host_blobs");
  REQUIRE(pool, 16, "pool");
  REQUIRE(fill_list, 8, "fill_list");
  REQUIRE(n_fill, 4, "n_fill");
  if (pool_bytes < (uint64_t)n_slots * layout->slot_stride)
    return fail(MOE_ERR_ARG, "pool_bytes %llu < n_slots * slot_stride", (unsigned long long)pool_bytes);
  return hip_status(moe::launch_fill(*d, static_cast<const uint8_t*>(host_blobs), layout->slot_stride,
                                     layout->blob_bytes, static_cast<uint8_t*>(pool), n_slots, fill_list, n_fill,
                                     reinterpret_cast<hipStream_t>(stream)),
                    "residency fill launch");
}

int moe_heat_update(const moe_dims* d, int32_t layer, const int32_t* offsets, float* heat, moe_stream_t stream) {
  int r = check_dims(d);
  if (r) return r;
  if (layer < 0 || layer >= d->L) return fail(MOE_ERR_ARG, "layer = %d outside [0, L = %d)", layer, d->L);
  REQUIRE(offsets, 4, "offsets");
  REQUIRE(heat, 4, "heat");
  return hip_status(moe::launch_heat(*d, layer, offsets, heat, reinterpret_cast<hipStream_t>(stream)), "heat launch");
}

int moe_heat_decay(const moe_dims* d, float* heat, float decay, moe_stream_t stream) {
  int r = check_dims(d);
  if (r) return r;
  REQUIRE(heat, 4, "heat");
  return hip_status(moe::launch_heat_decay(*d, heat, decay, reinterpret_cast<hipStream_t>(stream)),
                    "heat decay launch");
}

int moe_swap_plan(const moe_dims* d, const float* heat, const int32_t* slot_table, float threshold,
                  int32_t max_swaps, int32_t* plan, int32_t* n_plan) {
  int r = check_dims(d);
  if (r) return r;
  if (!heat || !slot_table || !n_plan || (!plan && max_swaps > 0)) return fail(MOE_ERR_ARG, "a pointer is NULL");
  if (max_swaps < 0) return fail(MOE_ERR_ARG, "max_swaps = %d < 0", max_swaps);
  *n_plan = moe::plan_swaps(*d, heat, slot_table, threshold, max_swaps, plan);
  return ok();
}

int moe_swap_apply(const moe_dims* d, const moe_blob_layout* layout, const void* host_blobs, void* pool,
                   uint64_t pool_bytes, int32_t n_slots, int32_t* slot_table, const int32_t* plan, int32_t n_plan,
                   int32_t* fill_scratch, int32_t* n_scratch, moe_stream_t stream) {
  int r = check_dims(d);
  if (r) return r;
  if (!layout) return fail(MOE_ERR_ARG, "layout is NULL");
  if (n_slots < 1) return fail(MOE_ERR_ARG, "n_slots = %d < 1", n_slots);
  if (n_plan < 0) return fail(MOE_ERR_ARG, "n_plan = %d < 0", n_plan);
  if (n_plan == 0) return ok();
  REQUIRE(host_blobs, 16, "host_blobs");
  REQUIRE(pool, 16, "pool");
  REQUIRE(slot_table, 4, "slot_table");
  REQUIRE(plan, 4, "plan");
  REQUIRE(fill_scratch, 8, "fill_scratch");
  REQUIRE(n_scratch, 4, "n_scratch");
  if (pool_bytes < (uint64_t)n_slots * layout->slot_stride)
    return fail(MOE_ERR_ARG, "pool_bytes %llu < n_slots * slot_stride", (unsigned long long)pool_bytes);
  return hip_status(moe::launch_swap_apply(*d, static_cast<const uint8_t*>(host_blobs), layout->slot_stride,
                                           layout->blob_bytes, static_cast<uint8_t*>(pool), n_slots, slot_table,
                                           plan, n_plan, fill_scratch, n_scratch,
                                           reinterpret_cast<hipStream_t>(stream)),
                    "swap launch");
}

int moe_route_group(const moe_dims* d, int32_t layer, const uint16_t* x, const float* w_router,
                    const float* logits_in, const float* w_shared_gate, float* logits_out, int32_t* topk_ids,
                    float* topk_w, float* shared_sigma, const int32_t* slot_table, int32_t n_slots,
                    int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* group_slot, int32_t* dev_status,
                    void* ws, uint64_t ws_bytes, moe_stream_t stream) {
  int r = validate_route(d, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w, shared_sigma);
  if (r) return r;
  if ((r = validate_group(d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status,
                          ws, ws_bytes)))
    return r;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float* lg = nullptr;
  if ((r = route_logits(d, x, w_router, logits_in, logits_out, s, &lg))) return r;
  if (moe::route_group_fusable(*d))
    return hip_status(moe::launch_route_group(*d, layer, lg, x, w_shared_gate, slot_table, n_slots, topk_ids, topk_w,
                                              shared_sigma, offsets, perm, inv_perm, group_slot, dev_status, ws, s),
                      "route + group launch");
  if ((r = hip_status(moe::launch_topk(*d, lg, x, w_shared_gate, topk_ids, topk_w, shared_sigma, s),
                      "top-k launch")))
    return r;
  return hip_status(moe::launch_group(*d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot,
                                      dev_status, ws, s),
                    "group launch");
}

int moe_expert_ffn(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                   const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm,
                   const int32_t* group_slot, uint16_t* h, uint16_t* y_rows, int32_t* dev_status, void* ws,
                   uint64_t ws_bytes, moe_stream_t stream) {
  return moe_expert_ffn_stages(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                               ws_bytes, 3, nullptr, nullptr, stream);
}

}  // extern "C"

namespace {

// S4 (stages: 1 gate/up, 2 down, 3 both) and, with y set, S5 after it.  With
// the combine, decode windows whose shapes have an instantiation run the two
// stages and the combine as one launch; otherwise one launch per stage, then
// the combine's own.
// The NVFP4 FFN's arguments (moe_expert_ffn_stages) checked, and its geometry:
// the pool's slots and the device's compute-unit count.
int validate_ffn(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                 const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm, const int32_t* group_slot,
                 uint16_t* h, uint16_t* y_rows, int32_t* dev_status, void* ws, uint64_t ws_bytes, int32_t stages,
                 moe::FfnGeom* g, int* n_cu) {
  if (stages < 1 || stages > 3) return fail(MOE_ERR_ARG, "stages = %d: must be 1 (gate/up), 2 (down) or 3", stages);
  int r = check_dims(d);
  if (r) return r;
  if (!layout) return fail(MOE_ERR_ARG, "layout is NULL");
  moe_blob_layout want;
  if ((r = moe_blob_layout_init(d->H, d->I, &want))) return r;
  if (memcmp(&want, layout, sizeof want) != 0)
    return fail(MOE_ERR_ARG, "layout does not match moe_blob_layout_init(H = %d, I = %d)", d->H, d->I);
  REQUIRE(x, 16, "x");
  REQUIRE(pool, 16, "pool");
  REQUIRE(offsets, 4, "offsets");
  REQUIRE(perm, 4, "perm");
  REQUIRE(group_slot, 4, "group_slot");
  REQUIRE(h, 16, "h");
  REQUIRE(y_rows, 16, "y_rows");
  REQUIRE(dev_status, 4, "dev_status");
  REQUIRE(ws, 16, "ws");
  const uint64_t need = moe::ws_layout(*d).total;
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %llu bytes < required %llu", (unsigned long long)ws_bytes,
                (unsigned long long)need);
  if (pool_bytes < layout->slot_stride)
    return fail(MOE_ERR_ARG, "pool_bytes %llu is smaller than one slot (%llu)", (unsigned long long)pool_bytes,
                (unsigned long long)layout->slot_stride);
  int dev = 0;
  *n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || *n_cu <= 0)
    return fail(MOE_ERR_HIP, "cannot query the device's compute-unit count");
  g->pool = static_cast<const uint8_t*>(pool);
  g->slot_stride = layout->slot_stride;
  g->n_slots = (int64_t)(pool_bytes / layout->slot_stride);
  for (int m = 0; m < 3; m++) {
    g->off_codes[m] = layout->off_codes[m];
    g->off_scales[m] = layout->off_scales[m];
  }
  g->off_globals = layout->off_globals;
  return MOE_OK;
}

// S4 (stages: 1 gate/up, 2 down, 3 both) and, with y set, S5 after it.  With
// the combine, decode windows whose shapes have an instantiation run the two
// stages and the combine as one launch; otherwise one launch per stage, then
// the combine's own.
int expert_ffn(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
               const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm, const int32_t* group_slot,
               uint16_t* h, uint16_t* y_rows, int32_t* dev_status, void* ws, uint64_t ws_bytes, int32_t stages,
               void* ev_start, void* ev_stop, moe_stream_t stream, const int32_t* inv_perm, const float* topk_w,
               const float* shared_sigma, uint16_t* y) {
  moe::FfnGeom g;
  int n_cu = 0;
  int r = validate_ffn(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                       ws_bytes, stages, &g, &n_cu);
  if (r) return r;
  const bool comb = y != nullptr;
  if (comb) {
    REQUIRE(inv_perm, 4, "inv_perm");
    REQUIRE(topk_w, 4, "topk_w");
    REQUIRE(shared_sigma, 4, "shared_sigma");
    REQUIRE(y, 16, "y");
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
  // groups averaging >= kGemmMinRows rows: grouped GEMM over 256-row chunks;
  // otherwise weight streaming over 16-row tiles (the grouping kernels wrote
  // the matching work list)
  // moe_expert_ffn_combine on decode windows: the FFN's two stages and the
  // combine in one launch where the shapes have an instantiation
  if (comb && stages == 3 && !moe::use_gemm(*d) && moe::ffn_dec_fusable(*d, true))
    return hip_status(moe::launch_ffn_dec_fused(*d, x, g, h, y_rows, dev_status, ws, n_cu, e0, e1, st, inv_perm,
                                                topk_w, shared_sigma, y),
                      "expert FFN + combine launch");
  // moe_expert_ffn_down_combine on decode windows: the down stage and the
  // combine in one launch
  if (comb && stages == 2 && moe::down_combine_fusable(*d))
    return hip_status(moe::launch_down_combine(*d, g, h, y_rows, ws, e0, e1, st, inv_perm, topk_w, shared_sigma, y),
                      "down + combine launch");
  if (moe::use_gemm(*d))
    r = hip_status(moe::launch_ffn_gemm(*d, x, g, perm, h, y_rows, ws, n_cu, stages, e0, e1, st), "expert FFN launch");
  else
    r = hip_status(moe::launch_ffn_dec(*d, x, g, perm, h, y_rows, ws, n_cu, stages, e0, e1, st), "expert FFN launch");
  if (r || !comb) return r;
  return hip_status(moe::launch_combine(*d, y_rows, inv_perm, topk_w, shared_sigma, y, st), "combine launch");
}

}  // namespace

extern "C" {

int moe_expert_ffn_stages(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                          const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm,
                          const int32_t* group_slot, uint16_t* h, uint16_t* y_rows, int32_t* dev_status, void* ws,
                          uint64_t ws_bytes, int32_t stages, void* ev_start, void* ev_stop, moe_stream_t stream) {
  return expert_ffn(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws, ws_bytes,
                    stages, ev_start, ev_stop, stream, nullptr, nullptr, nullptr, nullptr);
}

int moe_expert_ffn_combine(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                           const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm,
                           const int32_t* group_slot, const int32_t* inv_perm, const float* topk_w,
                           const float* shared_sigma, uint16_t* h, uint16_t* y_rows, uint16_t* y,
                           int32_t* dev_status, void* ws, uint64_t ws_bytes, void* ev_start, void* ev_stop,
                           moe_stream_t stream) {
  if (!y) return fail(MOE_ERR_ARG, "y is NULL");
  return expert_ffn(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws, ws_bytes, 3,
                    ev_start, ev_stop, stream, inv_perm, topk_w, shared_sigma, y);
}

int moe_expert_ffn_down_combine(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                                const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm,
                                const int32_t* group_slot, const int32_t* inv_perm, const float* topk_w,
                                const float* shared_sigma, const uint16_t* h, uint16_t* y_rows, uint16_t* y,
                                int32_t* dev_status, void* ws, uint64_t ws_bytes, void* ev_start, void* ev_stop,
                                moe_stream_t stream) {
  if (!y) return fail(MOE_ERR_ARG, "y is NULL");
  return expert_ffn(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, const_cast<uint16_t*>(h), y_rows,
                    dev_status, ws, ws_bytes, 2, ev_start, ev_stop, stream, inv_perm, topk_w, shared_sigma, y);
}

int moe_route_group_ffn(const moe_dims* d, int32_t layer, const uint16_t* x, const float* w_router,
                        const float* logits_in, const float* w_shared_gate, float* logits_out, int32_t* topk_ids,
                        float* topk_w, float* shared_sigma, const int32_t* slot_table, int32_t n_slots,
                        int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* group_slot, const void* pool,
                        uint64_t pool_bytes, const moe_blob_layout* layout, uint16_t* h, uint16_t* y_rows,
                        int32_t* dev_status, void* ws, uint64_t ws_bytes, int32_t stages, void* ev_start,
                        void* ev_stop, moe_stream_t stream) {
  if (stages != 1 && stages != 3) return fail(MOE_ERR_ARG, "stages = %d: must be 1 (gate/up) or 3 (both)", stages);
  int r = validate_route(d, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w, shared_sigma);
  if (r) return r;
  if ((r = validate_group(d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status,
                          ws, ws_bytes)))
    return r;
  moe::FfnGeom g;
  int n_cu = 0;
  if ((r = validate_ffn(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                        ws_bytes, stages, &g, &n_cu)))
    return r;
  if (w_router || !moe::route_ffn_fusable(*d)) {
    // the routing in kernels of its own: route + group, then the FFN
    if ((r = moe_route_group(d, layer, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w,
                             shared_sigma, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status, ws,
                             ws_bytes, stream)))
      return r;
    return moe_expert_ffn_stages(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                                 ws_bytes, stages, ev_start, ev_stop, stream);
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float* lg = nullptr;
  if ((r = route_logits(d, x, nullptr, logits_in, logits_out, st, &lg))) return r;
  return hip_status(moe::launch_route_ffn_dec(*d, layer, lg, x, w_shared_gate, slot_table, n_slots, topk_ids, topk_w,
                                              shared_sigma, offsets, perm, inv_perm, group_slot, dev_status, g, h,
                                              y_rows, ws, n_cu, stages, static_cast<hipEvent_t>(ev_start),
                                              static_cast<hipEvent_t>(ev_stop), st),
                    "route + group + expert FFN launch");
}

int moe_route_group_ffn_combine(const moe_dims* d, int32_t layer, const uint16_t* x, const float* w_router,
                                const float* logits_in, const float* w_shared_gate, float* logits_out,
                                int32_t* topk_ids, float* topk_w, float* shared_sigma, const int32_t* slot_table,
                                int32_t n_slots, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                int32_t* group_slot, const void* pool, uint64_t pool_bytes,
                                const moe_blob_layout* layout, uint16_t* h, uint16_t* y_rows, uint16_t* y,
                                int32_t* dev_status, void* ws, uint64_t ws_bytes, void* ev_start, void* ev_stop,
                                moe_stream_t stream) {
  if (!y) return fail(MOE_ERR_ARG, "y is NULL");
  int r = validate_route(d, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w, shared_sigma);
  if (r) return r;
  if ((r = validate_group(d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status,
                          ws, ws_bytes)))
    return r;
  moe::FfnGeom g;
  int n_cu = 0;
  if ((r = validate_ffn(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                        ws_bytes, 3, &g, &n_cu)))
    return r;
  REQUIRE(y, 16, "y");
  if (w_router || !moe::route_ffn_combine_fusable(*d)) {
    // the calls' own launches, in turn
    if ((r = moe_route_group_ffn(d, layer, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w,
                                 shared_sigma, slot_table, n_slots, offsets, perm, inv_perm, group_slot, pool,
                                 pool_bytes, layout, h, y_rows, dev_status, ws, ws_bytes, 3, ev_start, ev_stop,
                                 stream)))
      return r;
    return moe_combine(d, y_rows, inv_perm, topk_w, shared_sigma, y, stream);
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float* lg = nullptr;
  if ((r = route_logits(d, x, nullptr, logits_in, logits_out, st, &lg))) return r;
  return hip_status(moe::launch_route_ffn_combine_dec(*d, layer, lg, x, w_shared_gate, slot_table, n_slots, topk_ids,
                                                      topk_w, shared_sigma, offsets, perm, inv_perm, group_slot,
                                                      dev_status, g, h, y_rows, y, ws, n_cu,
                                                      static_cast<hipEvent_t>(ev_start),
                                                      static_cast<hipEvent_t>(ev_stop), st),
                    "route + group + expert FFN + combine launch");
}

int moe_blob_layout_init_mx(int32_t H, int32_t I, moe_blob_layout* out) {
  if (!out) return fail(MOE_ERR_ARG, "out is NULL");
  if (H < 128 || H > 16384 || H % 128 != 0) return fail(MOE_ERR_SHAPE, "H = %d: must be a multiple of 128 in [128, 16384]", H);
  if (I < 128 || I > 16384 || I % 128 != 0) return fail(MOE_ERR_SHAPE, "I = %d: must be a multiple of 128 in [128, 16384]", I);
  const uint64_t rows[3] = {(uint64_t)I, (uint64_t)I, (uint64_t)H};
  const uint64_t kk[3] = {(uint64_t)H, (uint64_t)H, (uint64_t)I};
  uint64_t off = 0;
  for (int m = 0; m < 3; m++) {
    out->off_codes[m] = off;
    off = moe::align256(off + rows[m] * kk[m] / 2);
  }
  for (int m = 0; m < 3; m++) {
    out->off_scales[m] = off;
    off = moe::align256(off + rows[m] * kk[m] / 32);
  }
  out->off_globals = off;  // no globals: the blob ends here
  out->blob_bytes = off;
  out->slot_stride = (off + 4095) & ~uint64_t(4095);
  return ok();
}

int moe_mx_workspace_bytes(const moe_dims* d, uint64_t* out_bytes) {
  int r = check_dims(d);
  if (r) return r;
  if (!out_bytes) return fail(MOE_ERR_ARG, "out_bytes is NULL");
  *out_bytes = moe::mx_ws_layout(*d).total;
  return ok();
}

int moe_quantize_mxfp8(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                       moe_stream_t stream) {
  if (rows < 0) return fail(MOE_ERR_SHAPE, "rows = %lld: must be >= 0", (long long)rows);
  if (K < 32 || K % 32 != 0) return fail(MOE_ERR_SHAPE, "K = %d: must be a positive multiple of 32", K);
  if (rows * (int64_t)K / 8 > INT32_MAX * 64LL) return fail(MOE_ERR_SHAPE, "rows * K too large");
  REQUIRE(x, 16, "x");
  REQUIRE(codes, 8, "codes");
  REQUIRE(scales, 1, "scales");
  return hip_status(moe::launch_quant_mx(x, rows, K, codes, scales, K / 32, nullptr,
                                         reinterpret_cast<hipStream_t>(stream)),
                    "MXFP8 quantisation launch");
}

}  // extern "C"

namespace {

// moe_expert_ffn_mx; with mx_ws NULL (moe_expert_ffn_mx_noalloc) the MX
// workspace is the library's static scratch, and a size beyond it is refused
// before any HIP call.
// The MX FFN's argument checks (moe_expert_ffn_mx); fills the geometry, the
// CU count and, with static_scratch, *mx_ws with the library's array.
int validate_ffn_mx(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                    const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm,
                    const int32_t* group_slot, uint16_t* h, uint16_t* y_rows, int32_t* dev_status, void* ws,
                    uint64_t ws_bytes, void** mx_ws, uint64_t mx_ws_bytes, int32_t stages, bool static_scratch,
                    moe::FfnGeom* g_out, int* n_cu_out) {
  if (stages < 1 || stages > 3) return fail(MOE_ERR_ARG, "stages = %d: must be 1 (gate/up), 2 (down) or 3", stages);
  int r = check_dims(d);
  if (r) return r;
  if (!layout) return fail(MOE_ERR_ARG, "layout is NULL");
  moe_blob_layout want;
  if ((r = moe_blob_layout_init_mx(d->H, d->I, &want))) return r;
  if (memcmp(&want, layout, sizeof want) != 0)
    return fail(MOE_ERR_ARG, "layout does not match moe_blob_layout_init_mx(H = %d, I = %d)", d->H, d->I);
  REQUIRE(x, 16, "x");
  REQUIRE(pool, 16, "pool");
  REQUIRE(offsets, 4, "offsets");
  REQUIRE(perm, 4, "perm");
  REQUIRE(group_slot, 4, "group_slot");
  REQUIRE(h, 16, "h");
  REQUIRE(y_rows, 16, "y_rows");
  REQUIRE(dev_status, 4, "dev_status");
  REQUIRE(ws, 16, "ws");
  if (!static_scratch) REQUIRE(*mx_ws, 256, "mx_ws");
  const uint64_t need = moe::ws_layout(*d).total;
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %llu bytes < required %llu", (unsigned long long)ws_bytes,
                (unsigned long long)need);
  const uint64_t need_mx = moe::mx_ws_layout(*d).total;
  if (static_scratch && need_mx > moe::kNoAllocScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "these dims need %llu bytes of MX workspace, more than the %llu bytes of the library's static "
                "scratch; use moe_expert_ffn_mx with a caller workspace",
                (unsigned long long)need_mx, (unsigned long long)moe::kNoAllocScratchBytes);
  if (!static_scratch && mx_ws_bytes < need_mx)
    return fail(MOE_ERR_WORKSPACE, "MX workspace %llu bytes < required %llu", (unsigned long long)mx_ws_bytes,
                (unsigned long long)need_mx);
  if (pool_bytes < layout->slot_stride)
    return fail(MOE_ERR_ARG, "pool_bytes %llu is smaller than one slot (%llu)", (unsigned long long)pool_bytes,
                (unsigned long long)layout->slot_stride);
  moe::FfnGeom& g = *g_out;
  g.pool = static_cast<const uint8_t*>(pool);
  g.slot_stride = layout->slot_stride;
  g.n_slots = (int64_t)(pool_bytes / layout->slot_stride);
  for (int m = 0; m < 3; m++) {
    g.off_codes[m] = layout->off_codes[m];
    g.off_scales[m] = layout->off_scales[m];
  }
  g.off_globals = layout->off_globals;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || n_cu <= 0)
    return fail(MOE_ERR_HIP, "cannot query the device's compute-unit count");
  *n_cu_out = n_cu;
  if (static_scratch) {
    const hipError_t e = moe::noalloc_scratch(mx_ws);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  }
  return ok();
}

int expert_ffn_mx(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                  const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm,
                  const int32_t* group_slot, uint16_t* h, uint16_t* y_rows, int32_t* dev_status, void* ws,
                  uint64_t ws_bytes, void* mx_ws, uint64_t mx_ws_bytes, int32_t stages, void* ev_start,
                  void* ev_stop, moe_stream_t stream, bool static_scratch) {
  moe::FfnGeom g;
  int n_cu = 0;
  const int r = validate_ffn_mx(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                                ws_bytes, &mx_ws, mx_ws_bytes, stages, static_scratch, &g, &n_cu);
  if (r) return r;
  const hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (moe::use_gemm(*d))
    return hip_status(moe::launch_ffn_mx(*d, x, g, perm, h, y_rows, ws, mx_ws, n_cu, stages, e0, e1, st),
                      "MX expert FFN launch");
  return hip_status(moe::launch_ffn_dec_mx(*d, x, g, perm, h, y_rows, ws, mx_ws, n_cu, stages, e0, e1, st),
                    "MX expert FFN launch");
}

}  // namespace

extern "C" {

int moe_expert_ffn_mx(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                      const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm,
                      const int32_t* group_slot, uint16_t* h, uint16_t* y_rows, int32_t* dev_status, void* ws,
                      uint64_t ws_bytes, void* mx_ws, uint64_t mx_ws_bytes, int32_t stages, void* ev_start,
                      void* ev_stop, moe_stream_t stream) {
  return expert_ffn_mx(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                       ws_bytes, mx_ws, mx_ws_bytes, stages, ev_start, ev_stop, stream, false);
}

int moe_expert_ffn_mx_noalloc(const moe_dims* d, const uint16_t* x, const void* pool, uint64_t pool_bytes,
                              const moe_blob_layout* layout, const int32_t* offsets, const int32_t* perm,
                              const int32_t* group_slot, uint16_t* h, uint16_t* y_rows, int32_t* dev_status,
                              void* ws, uint64_t ws_bytes, int32_t stages, moe_stream_t stream) {
  return expert_ffn_mx(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                       ws_bytes, nullptr, 0, stages, nullptr, nullptr, stream, true);
}

int moe_route_group_ffn_mx(const moe_dims* d, int32_t layer, const uint16_t* x, const float* w_router,
                           const float* logits_in, const float* w_shared_gate, float* logits_out, int32_t* topk_ids,
                           float* topk_w, float* shared_sigma, const int32_t* slot_table, int32_t n_slots,
                           int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* group_slot, const void* pool,
                           uint64_t pool_bytes, const moe_blob_layout* layout, uint16_t* h, uint16_t* y_rows,
                           int32_t* dev_status, void* ws, uint64_t ws_bytes, void* mx_ws, uint64_t mx_ws_bytes,
                           int32_t stages, void* ev_start, void* ev_stop, moe_stream_t stream) {
  if (stages != 1 && stages != 3) return fail(MOE_ERR_ARG, "stages = %d: must be 1 (gate/up) or 3 (both)", stages);
  int r = validate_route(d, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w, shared_sigma);
  if (r) return r;
  if ((r = validate_group(d, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status,
                          ws, ws_bytes)))
    return r;
  moe::FfnGeom g;
  int n_cu = 0;
  if ((r = validate_ffn_mx(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                           ws_bytes, &mx_ws, mx_ws_bytes, stages, false, &g, &n_cu)))
    return r;
  if (moe::use_gemm(*d) || !moe::route_group_fusable(*d)) {
    // the two calls' kernels in turn
    if ((r = moe_route_group(d, layer, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w,
                             shared_sigma, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status, ws,
                             ws_bytes, stream)))
      return r;
    return moe_expert_ffn_mx(d, x, pool, pool_bytes, layout, offsets, perm, group_slot, h, y_rows, dev_status, ws,
                             ws_bytes, mx_ws, mx_ws_bytes, stages, ev_start, ev_stop, stream);
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float* lg = nullptr;
  if ((r = route_logits(d, x, w_router, logits_in, logits_out, st, &lg))) return r;
  uint16_t* xb = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(mx_ws) + moe::mx_ws_layout(*d).off_xb);
  if ((r = hip_status(moe::launch_route_group(*d, layer, lg, x, w_shared_gate, slot_table, n_slots, topk_ids, topk_w,
                                              shared_sigma, offsets, perm, inv_perm, group_slot, dev_status, ws, st,
                                              xb),
                      "route + group + MXFP8(x) launch")))
    return r;
  return hip_status(moe::launch_ffn_dec_mx(*d, x, g, perm, h, y_rows, ws, mx_ws, n_cu, stages,
                                           static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop), st,
                                           true),
                    "MX expert FFN launch");
}

int moe_combine(const moe_dims* d, const uint16_t* y_rows, const int32_t* inv_perm, const float* topk_w,
                const float* shared_sigma, uint16_t* y, moe_stream_t stream) {
  int r = check_dims(d);
  if (r) return r;
  REQUIRE(y_rows, 16, "y_rows");
  REQUIRE(inv_perm, 4, "inv_perm");
  REQUIRE(topk_w, 4, "topk_w");
  REQUIRE(shared_sigma, 4, "shared_sigma");
  REQUIRE(y, 16, "y");
  return hip_status(moe::launch_combine(*d, y_rows, inv_perm, topk_w, shared_sigma, y,
                                        reinterpret_cast<hipStream_t>(stream)),
                    "combine launch");
}

}  // extern "C"
