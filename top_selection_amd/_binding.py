"""ctypes binding of libdstopk.so (include/dstopk.h). Argument marshalling only.

Every step of top-k runs in the HIP kernels behind the C ABI; torch is used here for
device memory and streams only. There is no fallback: if the library is not built or
cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Dict, Optional, Tuple

import numpy as np

BF16 = 0
FP32 = 1

DS_OK = 0
DS_ERR_INVALID_ARG = -1
DS_ERR_UNSUPPORTED = -2
DS_ERR_ALIGNMENT = -3
DS_ERR_WORKSPACE = -4
DS_ERR_LAUNCH = -5
DS_ERR_DEVICE = -6
DS_MAX_K = 4096
DS_NOALLOC_SCRATCH_BYTES = 8 << 20
PRESAMPLE_AUTO, PRESAMPLE_OFF, PRESAMPLE_ON = 0, 1, 2
MERGE_AUTO, MERGE_LISTS, MERGE_SELECT = 0, 1, 2
SCHEDULE_AUTO, SCHEDULE_FREE, SCHEDULE_LOCKSTEP = 0, 1, 2
OUTPUT_UNSORTED, OUTPUT_INDEX_INT64 = 1, 2
SHARE_AUTO, SHARE_OFF, SHARE_ON = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
# DS_LIBRARY names another build of the library (e.g. one with host-side sanitizers)
LIB_PATH = os.environ.get("DS_LIBRARY") or os.path.join(_HERE, "libdstopk.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dstopk.h")


class DSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ds_status_string(status)} ({status})")


class ds_config(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("slack", ctypes.c_int32), ("slices", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("presample", ctypes.c_int32), ("order_group", ctypes.c_int32),
                ("merge", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("depth", ctypes.c_int32), ("output", ctypes.c_int32), ("warmup", ctypes.c_int32),
                ("share", ctypes.c_int32)]


STATS_FIELDS = ["appended", "compactions", "work", "max_len", "reads", "index_sum", "monotone", "slice_lo",
                "slice_len", "block", "slack", "t_total_ns", "t_compact_ns", "t_sync_ns", "t_final_ns", "passes"]
STATS_DTYPE = np.dtype([(f, np.uint64) for f in STATS_FIELDS])

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, i32, u64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64, ctypes.c_int
            cfgp = ctypes.POINTER(ds_config)
            L.ds_topk.argtypes = [vp, i64, i64, i64, ci, ci, u64, vp, vp, vp]
            L.ds_topk.restype = ci
            L.ds_topk_ex.argtypes = [vp, vp, i64, i64, i64, ci, ci, u64, vp, vp, vp, ctypes.c_size_t, cfgp, vp, vp]
            L.ds_topk_ex.restype = ci
            L.ds_topk_noalloc.argtypes = [vp, i64, i64, i64, ci, ci, u64, vp, vp, vp]
            L.ds_topk_noalloc.restype = ci
            L.ds_topk_slices.argtypes = [vp, vp, i64, i64, i64, ci, ci, u64, vp, vp, vp, ctypes.c_size_t, cfgp,
                                         vp, vp]
            L.ds_topk_slices.restype = ci
            L.ds_topk_merge.argtypes = [vp, i64, i64, ci, ci, u64, vp, vp, vp, ctypes.c_size_t, cfgp, vp]
            L.ds_topk_merge.restype = ci
            L.ds_topk_plan.argtypes = [i64, i64, ci, ci, cfgp, cfgp]
            L.ds_topk_plan.restype = ci
            L.ds_topk_workspace_size.argtypes = [i64, i64, ci, ci, cfgp, ctypes.POINTER(ctypes.c_size_t)]
            L.ds_topk_workspace_size.restype = ci
            L.ds_probe_read.argtypes = [vp, i64, vp, vp]
            L.ds_probe_read.restype = ci
            L.ds_probe_sink_words.argtypes = [i64]
            L.ds_probe_sink_words.restype = i64
            L.ds_probe_copy.argtypes = [vp, vp, i64, vp]
            L.ds_probe_copy.restype = ci
            L.ds_status_string.argtypes = [ci]
            L.ds_status_string.restype = ctypes.c_char_p
            _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/dstopk.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(ds_\w+)\s*\(", text, flags=re.M)))


def ds_status_string(status: int) -> str:
    return lib().ds_status_string(int(status)).decode()


def _cfg(cfg: Optional[Dict[str, int]]):
    if cfg is None:
        return None
    c = ds_config(int(cfg.get("block", 0)), int(cfg.get("slack", 0)), int(cfg.get("slices", 0)),
                  int(cfg.get("waves", 0)), int(cfg.get("presample", 0)), int(cfg.get("order_group", 0)),
                  int(cfg.get("merge", 0)), int(cfg.get("schedule", 0)), 0, int(cfg.get("output", 0)),
                  int(cfg.get("warmup", 0)), int(cfg.get("share", 0)))
    return ctypes.pointer(c)


def ds_topk_plan(rows: int, n: int, k: int, dtype: int, cfg: Optional[Dict[str, int]] = None) -> Dict[str, int]:
    out = ds_config()
    st = lib().ds_topk_plan(rows, n, k, dtype, _cfg(cfg), ctypes.byref(out))
    if st != DS_OK:
        raise DSError(st, "ds_topk_plan")
    return {"block": out.block, "slack": out.slack, "slices": out.slices, "waves": out.waves,
            "presample": out.presample, "order_group": out.order_group, "merge": out.merge,
            "schedule": out.schedule, "depth": out.depth, "output": out.output, "warmup": out.warmup,
            "share": out.share}


def ds_topk_workspace_size(rows: int, n: int, k: int, dtype: int, cfg: Optional[Dict[str, int]] = None) -> int:
    b = ctypes.c_size_t(0)
    st = lib().ds_topk_workspace_size(rows, n, k, dtype, _cfg(cfg), ctypes.byref(b))
    if st != DS_OK:
        raise DSError(st, "ds_topk_workspace_size")
    return int(b.value)


# ----------------------------------------------------------------------------- torch-facing calls
def _torch():
    import torch  # noqa: WPS433 (device memory and streams only)
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}; expected torch.bfloat16 or torch.float32")


def _stream_handle(stream, device=None) -> Optional[int]:
    """The hipStream_t of `stream`, or of torch's current stream on `device` (read without
    building a Stream object when torch offers the raw accessor)."""
    if stream is not None:
        return stream.cuda_stream
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        index = device.index if device is not None and device.index is not None else torch.cuda.current_device()
        return raw(index)
    return torch.cuda.current_stream().cuda_stream


def _prep(x, k: int, values: bool, indices: bool, out_vals, out_idx, idx64: bool = False):
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, N]")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if x.shape[0] > 0 and x.stride(1) != 1:
        raise ValueError("rows of x must be contiguous (stride(1) == 1)")
    rows, n = x.shape
    dt = dtype_code(x)
    if values and out_vals is None:
        out_vals = torch.empty((rows, k), dtype=x.dtype, device=x.device)
    idt = torch.int64 if idx64 else torch.int32
    if indices and out_idx is None:
        out_idx = torch.empty((rows, k), dtype=idt, device=x.device)
    for o, want in ((out_vals, x.dtype), (out_idx, idt)):
        if o is not None and (o.dtype != want or not o.is_contiguous() or tuple(o.shape) != (rows, k)):
            raise ValueError("outputs must be contiguous [rows, k] of the input dtype / the index type")
    row_stride = x.stride(0) if rows > 0 else n
    return rows, n, row_stride, dt, out_vals, out_idx


def ds_topk(x, k: int, seed: int = 0, values: bool = True, indices: bool = True, out_vals=None, out_idx=None,
            stream=None) -> Tuple[Optional[object], Optional[object]]:
    """Top-k of every row of the 2-D device tensor x (bf16 or fp32); see include/dstopk.h.

    Returns (values [rows,k] of x's dtype, indices [rows,k] int32), sorted by value
    descending (+0 before -0), ties by smaller index. Enqueued on `stream` (default: the
    current torch stream); no synchronisation.
    """
    rows, n, rs, dt, out_vals, out_idx = _prep(x, k, values, indices, out_vals, out_idx)
    st = lib().ds_topk(x.data_ptr() if rows else None, rows, n, rs, k, dt, seed & 0xFFFFFFFFFFFFFFFF,
                       out_vals.data_ptr() if out_vals is not None else None,
                       out_idx.data_ptr() if out_idx is not None else None, _stream_handle(stream, x.device))
    if st != DS_OK:
        raise DSError(st, "ds_topk")
    return out_vals, out_idx


def ds_topk_noalloc(x, k: int, seed: int = 0, values: bool = True, indices: bool = True, out_vals=None,
                    out_idx=None, stream=None) -> Tuple[Optional[object], Optional[object]]:
    """ds_topk whose workspace is the library's fixed per-GPU device array (no device
    allocation by the library; outputs not given are allocated here by torch). Raises
    DSError(DS_ERR_WORKSPACE) when the plan needs more than DS_NOALLOC_SCRATCH_BYTES."""
    rows, n, rs, dt, out_vals, out_idx = _prep(x, k, values, indices, out_vals, out_idx)
    st = lib().ds_topk_noalloc(x.data_ptr() if rows else None, rows, n, rs, k, dt, seed & 0xFFFFFFFFFFFFFFFF,
                               out_vals.data_ptr() if out_vals is not None else None,
                               out_idx.data_ptr() if out_idx is not None else None, _stream_handle(stream, x.device))
    if st != DS_OK:
        raise DSError(st, "ds_topk_noalloc")
    return out_vals, out_idx


def _idx64(cfg) -> bool:
    return bool(cfg and int(cfg.get("output", 0)) & OUTPUT_INDEX_INT64)


def _lens_ptr(lens, rows: int):
    if lens is None:
        return None
    torch = _torch()
    if not lens.is_cuda or lens.dtype != torch.int32 or not lens.is_contiguous() or lens.numel() != rows:
        raise ValueError("lens must be a contiguous device int32 tensor of one length per row")
    return lens.data_ptr()


def ds_topk_ex(x, k: int, seed: int = 0, workspace=None, cfg: Optional[Dict[str, int]] = None, stats=None,
               values: bool = True, indices: bool = True, out_vals=None, out_idx=None, stream=None, lens=None):
    """ds_topk with a caller workspace (a device tensor), forced config (including the output
    flags), optional stats (a device uint8 tensor of rows*slices*128 bytes) and optional
    per-row lengths (a device int32 tensor [rows]). Allocates nothing itself beyond the
    outputs it is not given."""
    rows, n, rs, dt, out_vals, out_idx = _prep(x, k, values, indices, out_vals, out_idx, _idx64(cfg))
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    st = lib().ds_topk_ex(x.data_ptr() if rows else None, _lens_ptr(lens, rows), rows, n, rs, k, dt,
                          seed & 0xFFFFFFFFFFFFFFFF,
                          out_vals.data_ptr() if out_vals is not None else None,
                          out_idx.data_ptr() if out_idx is not None else None, ws_ptr, ws_bytes, _cfg(cfg),
                          stats.data_ptr() if stats is not None else None, _stream_handle(stream, x.device))
    if st != DS_OK:
        raise DSError(st, "ds_topk_ex")
    return out_vals, out_idx


def ds_topk_slices(x, k: int, seed: int = 0, workspace=None, cfg: Optional[Dict[str, int]] = None, stats=None,
                   out_vals=None, out_idx=None, values: bool = True, indices: bool = True, stream=None, lens=None):
    """First launch of ds_topk_ex (the select kernel); returns the outputs it may fill."""
    rows, n, rs, dt, out_vals, out_idx = _prep(x, k, values, indices, out_vals, out_idx, _idx64(cfg))
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    st = lib().ds_topk_slices(x.data_ptr() if rows else None, _lens_ptr(lens, rows), rows, n, rs, k, dt,
                              seed & 0xFFFFFFFFFFFFFFFF,
                              out_vals.data_ptr() if out_vals is not None else None,
                              out_idx.data_ptr() if out_idx is not None else None, ws_ptr, ws_bytes, _cfg(cfg),
                              stats.data_ptr() if stats is not None else None, _stream_handle(stream, x.device))
    if st != DS_OK:
        raise DSError(st, "ds_topk_slices")
    return out_vals, out_idx


def ds_topk_merge(rows: int, n: int, k: int, dtype: int, seed: int = 0, workspace=None,
                  cfg: Optional[Dict[str, int]] = None, out_vals=None, out_idx=None, stream=None, lens=None):
    """Second launch of ds_topk_ex (the merge kernel) into the given output tensors."""
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    st = lib().ds_topk_merge(_lens_ptr(lens, rows), rows, n, k, dtype, seed & 0xFFFFFFFFFFFFFFFF,
                             out_vals.data_ptr() if out_vals is not None else None,
                             out_idx.data_ptr() if out_idx is not None else None, ws_ptr, ws_bytes, _cfg(cfg),
                             _stream_handle(stream, out_vals.device if out_vals is not None else
                                            (out_idx.device if out_idx is not None else None)))
    if st != DS_OK:
        raise DSError(st, "ds_topk_merge")
    return out_vals, out_idx


def stats_buffer(rows: int, slices: int, device):
    torch = _torch()
    return torch.zeros(rows * slices * STATS_DTYPE.itemsize, dtype=torch.uint8, device=device)


def decode_stats(buf) -> np.ndarray:
    return buf.cpu().numpy().view(STATS_DTYPE)


def ds_probe_read(src, sink=None, stream=None):
    """Stream all bytes of the device tensor src through the scan's 16-byte loads."""
    torch = _torch()
    nbytes = src.numel() * src.element_size()
    words = int(lib().ds_probe_sink_words(nbytes))
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=src.device)
    st = lib().ds_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream_handle(stream, src.device))
    if st != DS_OK:
        raise DSError(st, "ds_probe_read")
    return sink


def ds_probe_copy(dst, src, stream=None):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    st = lib().ds_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream_handle(stream, src.device))
    if st != DS_OK:
        raise DSError(st, "ds_probe_copy")
    return dst
