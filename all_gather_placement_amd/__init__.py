"""MI355X (gfx950) layout-aware reduce-scatter and all-gather placement for FSDP parameter groups.

The compute path is the C-ABI library ``libtide.so`` (hand-written HIP kernels); this package only
marshals arguments to it.  Importing the package does not load the library; the first call does,
and fails loudly if it has not been built (``python -m all_gather_placement_amd.build``).
"""
from .tide import (  # noqa: F401
    TIDE_AG_COPY2D,
    TIDE_AG_KERNEL,
    TIDE_AG_SDMA,
    TIDE_CU_EXCLUSIVE_MAX_ITEMS,
    TIDE_LAUNCH_BOUNDED,
    TIDE_LAUNCH_CU_EXCLUSIVE,
    TIDE_LAUNCH_DEFAULT,
    TIDE_LAUNCH_PER_CU_CAP,
    TIDE_MAX_WGS_PER_CU,
    Launch,
    Layout,
    TideError,
    library_path,
    load_library,
    BoundCall,
    tide_ag_place,
    tide_ag_prepare,
    tide_call_destroy,
    tide_call_launch,
    tide_layout_create,
    tide_rs_bf16_to_fp32,
    tide_rs_bf16_to_fp32_noalloc,
    TIDE_NOALLOC_MAX_PTRS,
    tide_rs_launch_shape,
    tide_rs_prepare,
    tide_rs_slots_bf16_to_fp32,
    tide_rs_slots_prepare,
    tide_slot_pack,
    tide_slot_pack_prepare,
)
