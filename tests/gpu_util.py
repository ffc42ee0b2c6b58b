"""Helpers shared by the GPU tests: upload numpy inputs, run the HIP path through the
binding, download, and compare with the oracle. Not collected by pytest."""
from __future__ import annotations

import sys

import numpy as np

import top_selection_amd as ts


def say(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def to_device(x: np.ndarray, pad_to: int = 0):
    """numpy [rows, n] (uint16 = bf16 bits, float32) -> torch device tensor, optionally with a
    padded row stride (the view keeps stride(0) = pad_to)."""
    import torch
    rows, n = x.shape
    per16 = 8 if x.dtype == np.uint16 else 4  # rows must start on 16-byte boundaries
    stride = max(-(-n // per16) * per16, pad_to)
    if x.dtype == np.uint16:
        full = np.zeros((rows, stride), np.uint16)
        full[:, :n] = x
        t = torch.from_numpy(full.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        full = np.zeros((rows, stride), np.float32)
        full[:, :n] = x
        t = torch.from_numpy(full).cuda()
    return t[:, :n]


def to_numpy_vals(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run_gpu(x: np.ndarray, k: int, seed: int = 1, cfg=None, values=True, indices=True, pad_to=0, stats=False):
    import torch
    xd = to_device(x, pad_to)
    st = None
    if cfg is None and not stats:
        v, i = ts.ds_topk(xd, k, seed=seed, values=values, indices=indices)
    else:
        rows, n = x.shape
        dt = ts.BF16 if x.dtype == np.uint16 else ts.FP32
        plan = ts.ds_topk_plan(rows, n, k, dt, cfg)
        wsb = ts.ds_topk_workspace_size(rows, n, k, dt, cfg)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None
        sb = ts.stats_buffer(rows, plan["slices"], "cuda") if stats else None
        v, i = ts.ds_topk_ex(xd, k, seed=seed, workspace=ws, cfg=cfg, stats=sb, values=values, indices=indices)
        if stats:
            st = (plan, ts.decode_stats(sb).reshape(rows, plan["slices"]))
    torch.cuda.synchronize()
    vals = to_numpy_vals(v) if v is not None else None
    idx = i.cpu().numpy() if i is not None else None
    return vals, idx, st


def assert_same(x: np.ndarray, k: int, got_vals, got_idx, want_vals, want_idx, label: str) -> None:
    if got_idx is not None:
        bad = np.argwhere(got_idx != want_idx)
        if bad.size:
            r, c = bad[0]
            raise AssertionError(f"{label}: index mismatch at row {r} pos {c}: got {got_idx[r, c]} want "
                                 f"{want_idx[r, c]} ({bad.shape[0]} mismatches)")
    if got_vals is not None:
        a = got_vals.view(np.uint16 if got_vals.dtype == np.uint16 else np.uint32)
        b = want_vals.view(a.dtype)
        bad = np.argwhere(a != b)
        if bad.size:
            r, c = bad[0]
            raise AssertionError(f"{label}: value mismatch at row {r} pos {c} ({bad.shape[0]} mismatches)")
