"""MI355X-native routed-expert MoE layer: C-ABI library libmoe (HIP, gfx950) and
its thin Python binding.  The binding raises on import if libmoe.so is not
built; there is no CPU fallback."""
from .binding import (Dims, BlobLayout, MoeError, moe_version, moe_status_string,  # noqa: F401
                      moe_blob_layout_init, moe_workspace_bytes, moe_route, moe_group, moe_expert_ffn,
                      moe_combine, moe_ring_create, moe_stage_h2d, moe_ring_acquire, moe_ring_release,
                      moe_ring_slot_ptr, moe_ring_destroy, LIB_PATH, EXPORTED)
