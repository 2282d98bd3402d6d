"""DeepSeek-V4 hyper-connection (HC) op for AMD MI355X (gfx950).

The op's kernels are hand-written HIP behind the C ABI in ``include/ds4hc.h``
(``libds4hc.so``); ``binding`` is the ctypes binding with the same names.
``workloads`` draws seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    DS4HC_BF16,
    DS4HC_F32,
    DS4HC_FLAG_DETERMINISTIC,
    DS4HC_FLAG_FORCE_ROWRES,
    DS4HC_FLAG_FORCE_SPLITK,
    DS4HC_FLAG_FORCE_TILE,
    Ds4hcError,
    ds4hc_combine,
    ds4hc_fused,
    ds4hc_partials,
    ds4hc_post,
    ds4hc_post_pre,
    ds4hc_post_pre_workspace_bytes,
    ds4hc_pre,
    ds4hc_sinkhorn,
    ds4hc_workspace_bytes,
    load,
    make_params,
)
