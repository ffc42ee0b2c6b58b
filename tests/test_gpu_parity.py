"""Bit-exact parity of the HIP path with the CPU oracle (values and indices, tolerance 0).

Every call goes through the C ABI (the ctypes binding). Inputs are the seeded workload
recipes (reduced row counts, then the full sizes in the launch configuration the
benchmark times) plus edge families and a fuzz sweep; the expected values come from the
oracle only.
"""
import numpy as np
import pytest

import top_selection_amd as ts
from gpu_util import assert_same, run_gpu, say
from oracle import model
from oracle import topk as otk
from workloads import gen

pytestmark = pytest.mark.gpu


def _check(x, k, label, seed=1, cfg=None, values=True, indices=True, pad_to=0, stats=False, want=None):
    say(f"[gpu] {label}: rows={x.shape[0]} n={x.shape[1]} k={k} dtype={x.dtype} cfg={cfg} seed={seed}")
    gv, gi, _ = run_gpu(x, k, seed=seed, cfg=cfg, values=values, indices=indices, pad_to=pad_to, stats=stats)
    wv, wi = otk.topk(x, k) if want is None else want
    assert_same(x, k, gv, gi, wv if values else None, wi if indices else None, label)


SEEDS = (1, 2, 3)  # block-order seeds: the result must not depend on the order (design note, "Algorithm")


def _check_seeds(x, k, label, **kw):
    want = otk.topk(x, k)
    for seed in SEEDS:
        _check(x, k, f"{label} seed={seed}", seed=seed, want=want, **kw)


def test_smoke_small():
    x = gen.WORKLOADS["c1_small"].make(rows=2, n=4096)
    _check(x, 64, "smoke")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_c1_small_forced_blocks(seed):
    w = gen.WORKLOADS["c1_small"]
    x = w.make()
    _check(x, 512, "c1", seed=seed, cfg={"block": 1024, "slack": 1024, "slices": 1})
    _check(x, 512, "c1-auto", seed=seed)


@pytest.mark.parametrize("slices", [0, 1, 3, 8])
def test_c2_indexer_rows(slices):
    x = gen.WORKLOADS["c2_indexer"].make(rows=6)
    _check(x, 512, f"c2 slices={slices}", cfg=None if slices == 0 else {"slices": slices})


@pytest.mark.parametrize("slices", [0, 1, 2])
def test_c3_sampler_rows(slices):
    x = gen.WORKLOADS["c3_sampler"].make(rows=5)
    _check(x, 512, f"c3 slices={slices}", cfg=None if slices == 0 else {"slices": slices})


@pytest.mark.parametrize("k", [512, 4096])
def test_c4_long_full(k):
    x = gen.WORKLOADS["c4_long"].make()
    _check_seeds(x, k, f"c4 k={k}")


def test_c5_reduced():
    x = gen.WORKLOADS["c5_giant"].make(n=1 << 22)
    _check(x, 32, "c5-reduced", indices=False)
    _check(x, 32, "c5-reduced-idx")


@pytest.mark.parametrize("name", ["c2_indexer", "c3_sampler"])
def test_full_size_bench_shapes(name):
    w = gen.WORKLOADS[name]
    x = w.make()
    _check_seeds(x, w.ks[0], f"{name}-full")


def test_c5_full_size():
    w = gen.WORKLOADS["c5_giant"]
    x = w.make()
    _check_seeds(x, 32, "c5-full", indices=False)


FAMILIES = ["normal", "ascending", "descending", "constant", "ties", "specials", "tiny", "neg"]


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("family", FAMILIES)
def test_edge_families(family, dtype):
    for n, k in [(1, 1), (7, 3), (513, 512), (3000, 1), (3000, 3000), (20000, 4096), (70001, 777)]:
        x = gen.rows_family(family, dtype, 5, 3, n)
        _check(x, k, f"{family}")


def test_strided_rows_and_output_modes():
    x = gen.rows_family("ties", gen.FP32, 9, 4, 9000)
    _check(x, 100, "strided", pad_to=9004)
    xb = gen.rows_family("normal", gen.BF16, 9, 4, 9000)
    _check(xb, 100, "strided-bf16", pad_to=9016)
    _check(xb, 100, "values-only", indices=False)
    _check(xb, 100, "indices-only", values=False)


def test_fuzz():
    g = np.random.default_rng(2024)
    for t in range(60):
        dtype = gen.BF16 if g.random() < 0.5 else gen.FP32
        rows = int(g.integers(1, 17))
        n = int(np.exp(g.uniform(0, np.log(300000))))
        k = int(g.integers(1, min(4096, n) + 1))
        fam = FAMILIES[int(g.integers(0, len(FAMILIES)))]
        x = gen.rows_family(fam, dtype, int(g.integers(0, 1 << 30)), rows, n)
        cfg = None
        if g.random() < 0.4:
            maxs = max(1, n // 2048)
            cfg = {"slices": int(g.integers(1, min(maxs, 32) + 1))}
        try:
            _check(x, k, f"fuzz#{t} {fam}", seed=int(g.integers(0, 1 << 40)), cfg=cfg)
        except ts.DSError as e:
            assert e.status == ts.DS_ERR_UNSUPPORTED and cfg is not None, str(e)


@pytest.mark.parametrize("mode", ["design-note", "default-lockstep", "free", "warm-up", "warm-up-free"])
@pytest.mark.parametrize("dtype,n,k,block,slack,slices", [
    (gen.BF16, 50000, 100, 1024, 333, 3),
    (gen.FP32, 129280, 512, 1024, 1024, 1),
    (gen.BF16, 262144, 512, 1024, 1024, 1),
    (gen.FP32, 70000, 64, 2048, 100, 4),
    (gen.BF16, 131072, 512, 0, 0, 4),   # the indexer shape's plan: 4 blocks per slice
    (gen.FP32, 129280, 512, 0, 0, 1),   # the sampler shape's plan: 16 blocks, groups of two
    (gen.FP32, 200000, 32, 0, 0, 2),    # small k: blocks of 16384 (16 waves x 4 chunks)
    (gen.BF16, 200000, 16, 0, 0, 1),    # small k, bf16: blocks of 16384 (16 waves x 2 chunks)
])
def test_counters_match_model(mode, dtype, n, k, block, slack, slices):
    """Under the lockstep schedule the kernel's A, R, W, max buffer length and read checksums
    equal the CPU model's under the same Feistel block order, B, B2 and slicing: with the
    design note's start and order (no presampled threshold, a random order of single
    blocks) forced, and with the plan's own presampled start and order groups. Under the
    free-running schedule the counters depend on how the waves interleave, so only what the
    design note's notes and analysis fix is checked: every element read once, T
    non-decreasing, W = A + k R, R B2 <= A and the buffer bound k + B2 + B - 1. With a
    warm-up window of two blocks (its forced compaction may come before k + B2 entries, so
    R B2 <= A is not claimed) the lockstep counters again equal the model's."""
    x = gen.rows_family("normal", dtype, 17, 9, n)  # 8 rows dealt to the XCDs, 1 in plain order
    x[1] = gen.rows_family("ascending", dtype, 18, 1, n)[0]
    free = mode in ("free", "warm-up-free")
    # no shared row threshold: with it the counters depend on how the slices interleave
    cfg = {"slices": slices, "schedule": ts.SCHEDULE_FREE if free else ts.SCHEDULE_LOCKSTEP, "share": ts.SHARE_OFF}
    if mode.startswith("warm-up"):
        cfg["warmup"] = 2
    if block:
        cfg.update(block=block, slack=slack)
    if mode == "design-note":
        cfg.update(presample=ts.PRESAMPLE_OFF, order_group=1)
    seed = 99
    say(f"[gpu] counters: n={n} k={k} cfg={cfg}")
    gv, gi, (plan, st) = run_gpu(x, k, seed=seed, cfg=cfg, stats=True)
    wv, wi = otk.topk(x, k)
    assert_same(x, k, gv, gi, wv, wi, "counters-run")
    pw = plan["waves"] if plan["presample"] == ts.PRESAMPLE_ON else None
    if mode == "design-note":
        assert pw is None and plan["order_group"] == 1
    warm = plan["warmup"]
    assert warm == (2 if mode.startswith("warm-up") else 0) and (pw is None or not warm)
    B, B2 = plan["block"], plan["slack"]
    for r in range(x.shape[0]):
        per = -(-n // plan["slices"])
        slice_len = -(-per // B) * B  # the planner's slice length
        if not free:
            _, mst = model.deepselect_row(x[r], k, B, B2, "feistel", seed=seed, row_id=r,
                                          slice_len=slice_len, group=plan["order_group"], presample_waves=pw,
                                          presample_depth=plan["depth"], warmup=warm)
            assert len(mst) == plan["slices"]
        for s in range(plan["slices"]):
            g = st[r, s]
            lo = s * slice_len
            ln = min(slice_len, n - lo)
            assert int(g["slice_lo"]) == lo and int(g["slice_len"]) == ln
            assert int(g["reads"]) == ln
            assert int(g["index_sum"]) == ln * lo + ln * (ln - 1) // 2
            assert int(g["monotone"]) == 1
            a, rr, w, ml = int(g["appended"]), int(g["compactions"]), int(g["work"]), int(g["max_len"])
            assert w == a + k * rr and ml <= k + B2 + B - 1
            assert warm or rr * B2 <= a
            if not free:
                ms = mst[s]
                assert (a, rr, w, ml) == (ms.A, ms.R, ms.W, ms.max_len), (r, s)


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
def test_split_rows_reuse_and_graph_replays(dtype):
    """Split rows (sorted slice lists merged by the list-merge kernel): repeated calls on one
    workspace, replays of a captured graph with eager work in between, and other plans on the
    same workspace (the merge kernel, a two-level list merge) all give the oracle's result;
    the workspace's contents on entry never matter."""
    import torch
    from gpu_util import to_device, to_numpy_vals
    rows, n, k, cfg = 6, 60000, 300, {"slices": 4}
    x = gen.rows_family("normal", dtype, 31, rows, n)
    wv, wi = otk.topk(x, k)
    xd = to_device(x)
    wsb = ts.ds_topk_workspace_size(rows, n, k, dtype, cfg)
    assert wsb == rows * ((cfg["slices"] * k + 1) // 2 * 2) * 8
    ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device="cuda")
    vals = torch.empty((rows, k), dtype=xd.dtype, device="cuda")
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")

    def check(label):
        torch.cuda.synchronize()
        assert_same(x, k, to_numpy_vals(vals), idx.cpu().numpy(), wv, wi, label)

    for rep in range(3):
        say(f"[gpu] split rows eager call {rep}")
        idx.fill_(-1)
        ts.ds_topk_ex(xd, k, seed=rep, workspace=ws, cfg=cfg, out_vals=vals, out_idx=idx)
        check(f"eager#{rep}")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ts.ds_topk_ex(xd, k, seed=7, workspace=ws, cfg=cfg, out_vals=vals, out_idx=idx)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ts.ds_topk_ex(xd, k, seed=7, workspace=ws, cfg=cfg, out_vals=vals, out_idx=idx, stream=s)
    for rep in range(3):
        say(f"[gpu] split rows graph replay {rep}")
        idx.fill_(-1)
        vals.zero_()
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        check(f"replay#{rep}")
    for label, xo, ko, co in [("other-lists", gen.rows_family("ties", dtype, 32, 3, 40000), 100, {"slices": 2}),
                              ("merge-kernel", gen.rows_family("normal", dtype, 33, 2, 16384), 64,
                               {"block": 1024, "slices": 16, "merge": ts.MERGE_SELECT}),
                              ("list-levels", gen.rows_family("normal", dtype, 34, 2, 40 * 1024 - 500), 16,
                               {"block": 1024, "slices": 40})]:
        say(f"[gpu] split rows workspace reuse: {label}")
        assert ts.ds_topk_workspace_size(xo.shape[0], xo.shape[1], ko, dtype, co) <= wsb
        gv, gi = ts.ds_topk_ex(to_device(xo), ko, seed=3, workspace=ws, cfg=co)
        torch.cuda.synchronize()
        ov, oi = otk.topk(xo, ko)
        assert_same(xo, ko, to_numpy_vals(gv), gi.cpu().numpy(), ov, oi, label)
    idx.fill_(-1)
    ts.ds_topk_ex(xd, k, seed=5, workspace=ws, cfg=cfg, out_vals=vals, out_idx=idx)
    check("after-other-plans")


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("family", ["normal", "ascending", "ties", "constant", "specials"])
def test_presample_on_and_off(dtype, family):
    """A presampled first threshold never drops a top-k element: both starts give the oracle's
    result; on i.i.d. rows the presampled start appends far fewer elements."""
    rows, n, k = 4, 65536, 512
    x = gen.rows_family(family, dtype, 41, rows, n)
    wv, wi = otk.topk(x, k)
    res = {}
    for mode in (ts.PRESAMPLE_OFF, ts.PRESAMPLE_ON):
        cfg = {"slices": 1, "presample": mode}
        assert ts.ds_topk_plan(rows, n, k, dtype, cfg)["presample"] == mode
        say(f"[gpu] presample={mode} {family} dtype={dtype}")
        gv, gi, (plan, st) = run_gpu(x, k, seed=5, cfg=cfg, stats=True)
        assert_same(x, k, gv, gi, wv, wi, f"presample={mode} {family}")
        res[mode] = st
    for r in range(rows):
        assert int(res[ts.PRESAMPLE_ON][r, 0]["reads"]) == n
        if family == "normal":
            assert 2 * int(res[ts.PRESAMPLE_ON][r, 0]["appended"]) < int(res[ts.PRESAMPLE_OFF][r, 0]["appended"])


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("group", [1, 2, 4])
def test_order_groups(dtype, group):
    """A random order over groups of G consecutive blocks gives the same result for every G,
    including streams whose last group is partial (its missing blocks read nothing)."""
    rows, k = 3, 256
    for n in (6 * 8192 + 100, 13 * 8192, 3 * 8192 - 5):
        for fam in ("normal", "ascending"):
            x = gen.rows_family(fam, dtype, 51, rows, n)
            cfg = {"slices": 1, "block": 8192, "order_group": group}
            assert ts.ds_topk_plan(rows, n, k, dtype, cfg)["order_group"] == group
            _check(x, k, f"group={group} n={n} {fam}", seed=9, cfg=cfg)


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("family,rows,n,k,slices,block", [
    ("normal", 3, 40 * 1024 - 500, 64, 40, 1024),    # two levels (7, 6); the last group has 5 lists
    ("ties", 3, 40 * 1024 - 500, 64, 40, 1024),
    ("normal", 2, 43 * 1024 - 1000, 512, 43, 1024),  # last slice 24 < k elements, alone in its group
    ("ascending", 2, 43 * 1024 - 1000, 512, 43, 1024),
    ("normal", 2, 40 * 1024 - 5, 1, 40, 1024),       # k = 1
    ("normal", 2, 200000, 4096, 5, 0),               # k = 4096: two levels (3, 2)
    ("ties", 2, 200000, 4096, 5, 0),
    ("normal", 4, 32 * 8192 - 1000, 300, 32, 0),     # two levels (6, 6)
    ("normal", 4, 16 * 8192 - 1000, 300, 16, 0),     # one level of 16 lists
])
def test_list_merge_levels(dtype, family, rows, n, k, slices, block):
    """The list merge's levels (groups, a ragged last group, short padded lists, k = 1 and
    4096) and the merge kernel on the same split give the oracle's result."""
    x = gen.rows_family(family, dtype, 51, rows, n)
    base = {"slices": slices}
    if block:
        base["block"] = block
    for merge in (ts.MERGE_LISTS, ts.MERGE_SELECT):
        cfg = dict(base, merge=merge)
        assert ts.ds_topk_plan(rows, n, k, dtype, cfg)["merge"] == merge
        _check(x, k, f"{family} merge={merge}", seed=5, cfg=cfg)


def test_list_merge_values_only_many_slices():
    """A values-only giant row cut into 256 slices: two list-merge levels with sixteen lists
    per workgroup (k = 32)."""
    x = gen.WORKLOADS["c5_giant"].make(n=1 << 22)
    cfg = {"slices": 256}
    plan = ts.ds_topk_plan(1, 1 << 22, 32, gen.FP32, cfg)
    assert plan["merge"] == ts.MERGE_LISTS and plan["slices"] == 256
    _check(x, 32, "values-only 256 slices", cfg=cfg, indices=False)
    _check(x, 32, "values+indices 256 slices", cfg=cfg)


def test_list_merge_many_rows():
    """More split rows than one list-merge launch covers (65528 rows per launch, rows dealt to
    the XCDs in eights and the last rows in plain order): rows on both sides of the launch
    boundary, the last rows and a random sample equal the oracle."""
    rows, n, k = 65535 + 101, 2048, 16
    x = gen.rows_family("normal", gen.BF16, 71, rows, n)
    cfg = {"slices": 2, "block": 1024}
    plan = ts.ds_topk_plan(rows, n, k, gen.BF16, cfg)
    assert plan["slices"] == 2 and plan["merge"] == ts.MERGE_LISTS
    say(f"[gpu] many rows: rows={rows} n={n} k={k} cfg={cfg}")
    gv, gi, _ = run_gpu(x, k, cfg=cfg)
    rng = np.random.default_rng(5)
    pick = sorted(set(range(8)) | set(range(65520, 65544)) | set(range(rows - 12, rows)) |
                  set(rng.choice(rows, 40, replace=False).tolist()))
    wv, wi = otk.topk(x[pick], k)
    assert_same(x[pick], k, gv[pick], gi[pick], wv, wi, "many rows")


def test_two_streams_share_nothing():
    """ds_topk on two streams at once, both on split rows: each stream has its own cached
    workspace, so both results equal the oracle's."""
    import torch
    from gpu_util import to_device, to_numpy_vals
    xa = gen.WORKLOADS["c2_indexer"].make(rows=8)
    xb = gen.rows_family("ascending", gen.BF16, 77, 8, 131072)
    assert ts.ds_topk_plan(8, 131072, 512, gen.BF16)["slices"] > 1
    da, db = to_device(xa), to_device(xb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"[gpu] two streams, round {rep}")
        with torch.cuda.stream(sa):
            va, ia = ts.ds_topk(da, 512, seed=rep, stream=sa)
        with torch.cuda.stream(sb):
            vb, ib = ts.ds_topk(db, 512, seed=rep + 10, stream=sb)
        outs.append((va, ia, vb, ib))
    torch.cuda.synchronize()
    wa, wia = otk.topk(xa, 512)
    wb, wib = otk.topk(xb, 512)
    for va, ia, vb, ib in outs:
        assert_same(xa, 512, to_numpy_vals(va), ia.cpu().numpy(), wa, wia, "stream a")
        assert_same(xb, 512, to_numpy_vals(vb), ib.cpu().numpy(), wb, wib, "stream b")


def test_cache_growth_refused_under_capture():
    """Under stream capture ds_topk does not allocate: a call that would grow the stream's
    cached workspace returns DS_ERR_WORKSPACE, and one that fits is captured and replays
    correctly."""
    import torch
    from gpu_util import to_device, to_numpy_vals
    s = torch.cuda.Stream()
    small = gen.WORKLOADS["c2_indexer"].make(rows=2)
    big = gen.WORKLOADS["c2_indexer"].make(rows=16)
    ds, db = to_device(small), to_device(big)
    with torch.cuda.stream(s):
        ts.ds_topk(ds, 512, stream=s)  # the stream's cache now fits two rows
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    vals = torch.empty((2, 512), dtype=ds.dtype, device="cuda")
    idx = torch.empty((2, 512), dtype=torch.int32, device="cuda")
    with torch.cuda.graph(g, stream=s):
        with pytest.raises(ts.DSError) as e:
            ts.ds_topk(db, 512, stream=s)
        ts.ds_topk(ds, 512, out_vals=vals, out_idx=idx, stream=s)
    assert e.value.status == ts.DS_ERR_WORKSPACE
    wv, wi = otk.topk(small, 512)
    for rep in range(3):
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(small, 512, to_numpy_vals(vals), idx.cpu().numpy(), wv, wi, f"replay {rep}")


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("schedule", [ts.SCHEDULE_FREE, ts.SCHEDULE_LOCKSTEP])
def test_partial_block_first_without_threshold(dtype, schedule):
    """All-negative rows whose first block read is the partial last block, with no threshold
    yet (presample off): the zero padding the hardware returns past the row's end must never
    be appended (a +0 would outrank every real element). Block orders are picked on the CPU
    (the model's Feistel order is the kernel's) so that the partial block comes first."""
    B = 16384
    n = 5 * B + 3392
    rows = 8
    x = gen.rows_family("neg", dtype, 91, rows, n)
    m = -(-n // B)
    seed = next(s for s in range(1000)
                if all(int(model.block_order("feistel", m, s, r, 0)[0]) == m - 1 for r in range(2)))
    cfg = {"slices": 1, "block": B, "presample": ts.PRESAMPLE_OFF, "order_group": 1, "schedule": schedule}
    _check(x, 64, f"partial-first seed={seed}", seed=seed, cfg=cfg)
    _check(x, 64, f"partial-first stats seed={seed}", seed=seed, cfg=cfg, stats=True)


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("warmup", [1, 3])
@pytest.mark.parametrize("family", ["normal", "ascending", "ties", "specials"])
def test_warmup_window(dtype, warmup, family):
    """The warm-up window (the plan's own schedule, split and whole rows) gives the oracle's
    result; the plan reports the window and turns the presampled start off."""
    x = gen.rows_family(family, dtype, 31, 6, 150000)
    for cfg in ({"warmup": warmup}, {"warmup": warmup, "slices": 1}, {"warmup": warmup, "block": 1024}):
        plan = ts.ds_topk_plan(6, 150000, 700, dtype, cfg)
        assert plan["warmup"] == warmup and plan["presample"] == ts.PRESAMPLE_OFF
        _check(x, 700, f"warm-up {family} {cfg}", seed=warmup, cfg=cfg)
