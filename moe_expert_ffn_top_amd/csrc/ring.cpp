// S6: two-slot staging ring of layer-sized device slots.
//
// [Strata] "PCIe 搬运怎样与计算重叠？": page-locked weights are submitted as
// asynchronous H2D copies; the copy stream records `copied` and the compute
// stream waits for it before reading a slot; after the slot's data is consumed
// the compute stream records `used`, and the next overwrite of that slot waits
// for it.  [FreeToken] 3.1: two layer-sized buffers, so that layer l+1 streams
// in while layer l computes.  Unpinned sources are rejected rather than
// staged through a host bounce buffer.
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include <string>

#include "moe_common.hpp"

struct moe_ring {
  void* slot[2];
  uint64_t slot_bytes;
  hipStream_t copy;
  hipEvent_t copied[2];
  hipEvent_t used[2];
  bool used_recorded[2];
  int state[2];  // 0 empty, 1 staged, 2 acquired
  int next;
};

namespace {
enum { kEmpty = 0, kStaged = 1, kAcquired = 2 };

int rfail(int code, const std::string& msg) { return moe::record_error(code, msg.c_str()); }
int rhip(hipError_t e, const char* what) {
  if (e != hipSuccess) return rfail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_ring_create(void* slot0, void* slot1, uint64_t slot_bytes, moe_stream_t copy_stream, moe_ring** out) {
  if (!slot0 || !slot1 || !out) return rfail(MOE_ERR_ARG, "slot0, slot1 and out are required");
  if ((reinterpret_cast<uintptr_t>(slot0) | reinterpret_cast<uintptr_t>(slot1)) & 15)
    return rfail(MOE_ERR_ALIGN, "ring slots must be 16-byte aligned");
  if (slot_bytes == 0) return rfail(MOE_ERR_ARG, "slot_bytes is 0");
  moe_ring* r = static_cast<moe_ring*>(calloc(1, sizeof(moe_ring)));
  if (!r) return rfail(MOE_ERR_ARG, "out of host memory");
  r->slot[0] = slot0;
  r->slot[1] = slot1;
  r->slot_bytes = slot_bytes;
  r->copy = reinterpret_cast<hipStream_t>(copy_stream);
  for (int s = 0; s < 2; s++) {
    hipError_t e = hipEventCreateWithFlags(&r->copied[s], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r->used[s], hipEventDisableTiming);
    if (e != hipSuccess) {
      for (int q = 0; q <= s; q++) {
        if (r->copied[q]) (void)hipEventDestroy(r->copied[q]);
        if (r->used[q]) (void)hipEventDestroy(r->used[q]);
      }
      free(r);
      return rhip(e, "hipEventCreate");
    }
  }
  *out = r;
  return MOE_OK;
}

int moe_stage_h2d(moe_ring* r, const void* src, uint64_t bytes, int32_t* out_slot) {
  if (!r || !src || !out_slot) return rfail(MOE_ERR_ARG, "ring, src and out_slot are required");
  if (bytes > r->slot_bytes) return rfail(MOE_ERR_ARG, "bytes exceed the slot size");
  const int s = r->next;
  if (r->state[s] != kEmpty)
    return rfail(MOE_ERR_STATE, "slot " + std::to_string(s) + " still holds data that was not released");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, src);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();  // clear the sticky error of an unknown pointer
    return rfail(MOE_ERR_NOT_PINNED, "source is not page-locked host memory");
  }
  if (r->used_recorded[s] && (e = hipStreamWaitEvent(r->copy, r->used[s], 0)) != hipSuccess)
    return rhip(e, "wait used");
  if ((e = hipMemcpyAsync(r->slot[s], src, bytes, hipMemcpyHostToDevice, r->copy)) != hipSuccess)
    return rhip(e, "hipMemcpyAsync");
  if ((e = hipEventRecord(r->copied[s], r->copy)) != hipSuccess) return rhip(e, "record copied");
  r->state[s] = kStaged;
  r->next = s ^ 1;
  *out_slot = s;
  return MOE_OK;
}

int moe_ring_acquire(moe_ring* r, int32_t s, moe_stream_t compute) {
  if (!r || s < 0 || s > 1) return rfail(MOE_ERR_ARG, "bad ring or slot");
  if (r->state[s] != kStaged) return rfail(MOE_ERR_STATE, "slot was not staged");
  int rc = rhip(hipStreamWaitEvent(reinterpret_cast<hipStream_t>(compute), r->copied[s], 0), "wait copied");
  if (rc) return rc;
  r->state[s] = kAcquired;
  return MOE_OK;
}

int moe_ring_release(moe_ring* r, int32_t s, moe_stream_t compute) {
  if (!r || s < 0 || s > 1) return rfail(MOE_ERR_ARG, "bad ring or slot");
  if (r->state[s] != kAcquired) return rfail(MOE_ERR_STATE, "slot was not acquired");
  int rc = rhip(hipEventRecord(r->used[s], reinterpret_cast<hipStream_t>(compute)), "record used");
  if (rc) return rc;
  r->used_recorded[s] = true;
  r->state[s] = kEmpty;
  return MOE_OK;
}

int moe_ring_slot_ptr(moe_ring* r, int32_t s, void** out) {
  if (!r || s < 0 || s > 1 || !out) return rfail(MOE_ERR_ARG, "bad ring, slot or out");
  *out = r->slot[s];
  return MOE_OK;
}

int moe_ring_destroy(moe_ring* r) {
  if (!r) return rfail(MOE_ERR_ARG, "ring is NULL");
  for (int s = 0; s < 2; s++) {
    (void)hipEventDestroy(r->copied[s]);
    (void)hipEventDestroy(r->used[s]);
  }
  free(r);
  return MOE_OK;
}

}  // extern "C"
