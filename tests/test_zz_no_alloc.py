"""ds_topk_noalloc (the entry point whose workspace is the library's fixed per-GPU array):
through the C ABI it gives what ds_topk gives, bit for bit, and what the oracle gives, on
calls in a row that reuse the array with different and smaller plans, under graph capture
with other calls between the replays, and it refuses a plan larger than the array."""
import numpy as np
import pytest

import top_selection_amd as ts
from gpu_util import assert_same, say, to_device, to_numpy_vals
from oracle import topk as otk
from workloads import gen

pytestmark = pytest.mark.gpu

# (label, input, k), each input smaller than the one before: a plan near the array's size
# (k = 4096 over 125 rows of 131072: 2 slices' lists and the shared row thresholds, 8193000
# of its 8388608 bytes), indexer rows, then smaller split plans
CASES = [("bf16 125x131072 k4096 (near the array size)", lambda: gen.rows_family("normal", gen.BF16, 83, 125, 131072),
          4096),
         ("indexer rows 48x131072 k512", lambda: gen.WORKLOADS["c2_indexer"].make(rows=48), 512),
         ("fp32 3x300000 k64 ties", lambda: gen.rows_family("ties", gen.FP32, 82, 3, 300000), 64),
         ("bf16 2x140000 k100", lambda: gen.rows_family("normal", gen.BF16, 81, 2, 140000), 100)]


def _dt(x):
    return gen.BF16 if x.dtype == np.uint16 else gen.FP32


def _both(xd, k, seed):
    """(noalloc values, indices), (ds_topk values, indices) on the current stream."""
    a = ts.ds_topk_noalloc(xd, k, seed=seed)
    b = ts.ds_topk(xd, k, seed=seed)
    return a, b


def test_noalloc_matches_ds_topk_and_oracle():
    import torch
    prev = None
    for label, make, k in CASES:
        x = make()
        rows, n = x.shape
        plan = ts.ds_topk_plan(rows, n, k, _dt(x))
        wsb = ts.ds_topk_workspace_size(rows, n, k, _dt(x))
        say(f"[gpu] noalloc {label}: plan slices={plan['slices']} workspace={wsb}")
        assert plan["slices"] > 1 and 0 < wsb <= ts.DS_NOALLOC_SCRATCH_BYTES
        if prev is not None:
            assert wsb < prev[0] and rows * n <= prev[1], "each call uses less of the array than the one before"
        prev = (wsb, rows * n)
        xd = to_device(x)
        (av, ai), (bv, bi) = _both(xd, k, seed=3)
        torch.cuda.synchronize()
        assert torch.equal(ai, bi) and torch.equal(av.view(torch.int16) if av.dtype == torch.bfloat16 else av,
                                                   bv.view(torch.int16) if bv.dtype == torch.bfloat16 else bv)
        wv, wi = otk.topk(x, k)
        assert_same(x, k, to_numpy_vals(av), ai.cpu().numpy(), wv, wi, f"noalloc {label}")


def test_noalloc_graph_replays_with_calls_between():
    """A captured pair of calls (large, then smaller) replays to the eager results, with
    eager calls on another input overwriting the array between replays."""
    import torch
    xs = [gen.WORKLOADS["c2_indexer"].make(), gen.rows_family("normal", gen.BF16, 84, 2, 140000)]
    ks = [512, 100]
    xds = [to_device(x) for x in xs]
    other = to_device(gen.rows_family("normal", gen.BF16, 85, 32, 131072))
    want = [otk.topk(x, k) for x, k in zip(xs, ks)]
    outs = [(torch.empty((x.shape[0], k), dtype=torch.bfloat16, device="cuda"),
             torch.empty((x.shape[0], k), dtype=torch.int32, device="cuda")) for x, k in zip(xs, ks)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for xd, k, (v, i) in zip(xds, ks, outs):  # one eager call first, as before any capture
            ts.ds_topk_noalloc(xd, k, seed=7, out_vals=v, out_idx=i, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for xd, k, (v, i) in zip(xds, ks, outs):
            ts.ds_topk_noalloc(xd, k, seed=7, out_vals=v, out_idx=i, stream=s)
    for rep in range(3):
        say(f"[gpu] noalloc graph replay {rep}")
        for v, i in outs:
            v.zero_()
            i.fill_(-1)
        ts.ds_topk_noalloc(other, 2048)  # eager work that overwrites the array
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, k, (v, i), (wv, wi) in zip(xs, ks, outs, want):
            assert_same(x, k, to_numpy_vals(v), i.cpu().numpy(), wv, wi, f"noalloc replay {rep}")


def test_noalloc_refuses_a_plan_beyond_the_array():
    import torch
    rows, n, k = 130, 131072, 4096
    wsb = ts.ds_topk_workspace_size(rows, n, k, ts.BF16)
    assert wsb > ts.DS_NOALLOC_SCRATCH_BYTES
    xd = torch.zeros((rows, n), dtype=torch.bfloat16, device="cuda")
    v = torch.full((rows, k), 7, dtype=torch.bfloat16, device="cuda")
    i = torch.full((rows, k), -5, dtype=torch.int32, device="cuda")
    with pytest.raises(ts.DSError) as e:
        ts.ds_topk_noalloc(xd, k, out_vals=v, out_idx=i)
    assert e.value.status == ts.DS_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((i == -5).all()) and bool((v == 7).all()), "a refused call enqueues nothing"
    vv, ii = ts.ds_topk(xd, k)  # ds_topk still serves it from its cache
    torch.cuda.synchronize()
    assert bool((ii[0] == torch.arange(k, device="cuda", dtype=torch.int32)).all())
