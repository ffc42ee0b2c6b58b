"""DeepSelect row-wise top-k for AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI declared in include/dstopk.h;
this package is the thin Python binding (same names as the C entry points) plus the
build step. torch supplies device memory and streams only.
"""
from ._binding import (BF16, DS_ERR_ALIGNMENT, DS_ERR_DEVICE, DS_ERR_INVALID_ARG, DS_ERR_LAUNCH,  # noqa: F401
                       DS_ERR_UNSUPPORTED, DS_ERR_WORKSPACE, DS_MAX_K, DS_NOALLOC_SCRATCH_BYTES, DS_OK, FP32, LIB_PATH, PRESAMPLE_AUTO,
                       PRESAMPLE_OFF, PRESAMPLE_ON, MERGE_AUTO, MERGE_LISTS, MERGE_SELECT, SCHEDULE_AUTO,
                       SCHEDULE_FREE, SCHEDULE_LOCKSTEP, STATS_DTYPE, OUTPUT_UNSORTED, OUTPUT_INDEX_INT64, SHARE_AUTO, SHARE_OFF, SHARE_ON,
                       DSError, decode_stats, ds_probe_copy, ds_probe_read, ds_status_string, ds_topk, ds_topk_ex,
                       ds_topk_merge, ds_topk_noalloc, ds_topk_plan, ds_topk_slices, ds_topk_workspace_size, dtype_code, header_functions, lib, stats_buffer)
