"""MI355X (gfx950) single-token MLA decode.

A thin Python binding over ``libmla_decode.so``, whose C ABI is declared in
``include/mla_decode.h``. The binding only marshals torch device tensors into
pointers and sizes; every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is missing or fails to load,
importing this package raises.
"""
from ._lib import (  # noqa: F401
    FLAG_COMBINE_LAUNCH,
    FLAG_FORCE_PERSISTENT,
    FLAG_FORCE_SPLIT,
    FLAG_GRID_SHIFT,
    FLAG_MIXED_LENGTHS,
    FLAG_SPLITS_SHIFT,
    KV_BF16,
    KV_FP8_E4M3,
    KV_MXFP4,
    LIB_PATH,
    NUM_HEADS,
    QK_DIM,
    V_DIM,
    WORKSPACE_COUNTER_BYTES,
    MlaError,
    Q_SCALE_DYNAMIC,
    Q_SCALE_STATIC,
    PlanInfo,
    flags_for,
    mla_decode,
    mla_decode_mtp,
    mla_decode_noalloc,
    mla_decode_mtp_workspace_size,
    mla_decode_paged,
    mla_decode_plan,
    mla_decode_q8,
    mla_decode_q8_workspace_size,
    mla_decode_workspace_size,
    mla_dequant_debug,
    mla_hbm_read_probe,
    mla_quantize_q8_debug,
    mla_source_digest,
    mla_status_string,
    new_workspace,
    prepare_decode,
    prepare_decode_mtp,
    prepare_decode_paged,
    prepare_decode_q8,
)
