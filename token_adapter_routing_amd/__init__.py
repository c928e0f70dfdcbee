"""MI355X (gfx950) per-token adapter routing: Python binding of the HIP library libmolora.so.

The C ABI is declared in include/molora.h; the functions exported here carry the same names
and only marshal arguments.  The library must be built first (``__graft_entry__.build()``);
importing the functions does not load it, calling one does, and a missing library raises.
"""
from .binding import (  # noqa: F401
    BF16, F32, LAYOUT_DIRECT, LAYOUT_INDIRECT, PATH_AUTO, PATH_BLOCK, PATH_GROUPED, PATH_SKINNY, PATH_TILE, PATH_GROUPED_FIXED,
    HotSet, MoloraError, exported_symbols, load_library, LIB_PATH, NOALLOC_SCRATCH_BYTES,
    MOLORA_OK, MOLORA_EINVAL, MOLORA_ENOTSUP, MOLORA_ENOSPC, MOLORA_EHIP,
    molora_apply, molora_apply_multi, molora_apply_path, molora_apply_multi_workspace, molora_apply_workspace, molora_dispatch,
    molora_dispatch_workspace, molora_dispatch_apply_multi, molora_dispatch_apply_multi_workspace,
    molora_hotset_bytes, molora_hotset_destroy, molora_hotset_init, molora_hotset_load, molora_route_topk, molora_route_topk_workspace,
    molora_route_vocab, molora_seqpass_meta, molora_step_vocab, molora_step_vocab_noalloc, molora_step_workspace,
    molora_hotset_init_transposed, molora_backward, molora_backward_workspace,
    molora_route_topk_backward, molora_router_backward, molora_router_backward_workspace,
    XfModel, XF_TARGETS, molora_xf_workspace, molora_xf_forward,
)
