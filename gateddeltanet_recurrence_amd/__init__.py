"""MI355X (gfx950) GatedDeltaNet operator: Python binding of libgdn.so.

The binding only marshals arguments: it checks that tensors are contiguous,
on the GPU and shaped consistently with each other, fills the C structs of
include/gdn.h and calls the library. Every step of the operator runs in the
HIP kernels of libgdn.so; there is no Python or CPU fallback, and a missing
library raises an error.
"""
from .binding import (  # noqa: F401
    GDNError, LibraryNotBuilt, PLAN_AUTO, PLAN_RECURRENT, PLAN_CHUNK,
    GDN_F32, GDN_F16, GDN_BF16, RULE_GATED_DELTA, RULE_DELTA, RULE_GATED, RULE_LINEAR, GATE_RAW, GATE_NONE, ABI_VERSION,
    STATE_V_MAJOR, STATE_K_MAJOR,
    GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_ALIAS, GDN_ERR_CAPACITY,
    GDN_ERR_WORKSPACE, GDN_ERR_PLAN, GDN_ERR_RULE, GDN_ERR_HIP, GDN_ERR_SCRATCH, GdnParams, GdnTensors,
    lib, library_path, gdn_abi_version, gdn_strerror, gdn_forward, gdn_forward_workspace_bytes,
    gdn_resolve_plan, gdn_replay, gdn_replay_forward, gdn_replay_forward_pooled, capsule_width, make_params,
    CONV_SILU, CONV_NONE, GdnConvParams, GdnConvTensors, gdn_conv_forward, gdn_conv_replay,
    GdnSlots, gdn_forward_pooled, gdn_replay_pooled, gdn_conv_forward_pooled, gdn_conv_replay_pooled,
    gdn_publish_slots, gdn_forward_no_alloc, NO_ALLOC_SCRATCH_BYTES, GdnConvFused, gdn_conv_decode_forward,
)
