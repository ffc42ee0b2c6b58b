"""Pins for the instrumented CPU model of DeepSelect and for the bound evaluator.

* model result == sorting oracle, over shapes, block sizes, orders, slices and input kinds;
* the invariants the design note states (buffer bound, read-once, monotone threshold) and
  the proof's identities (W = A + k R, R B2 <= A), on every run;
* the block-order experiment printed in the tutorial chapter (section 2.3): the
  deterministic sequential rows reproduce exactly, the random rows in magnitude;
* Table 2 (section 3.7), Table 4 (section 1.3) and the ~78k figure (section 6.3);
* the boxed bound E[W] <= (1+k/B2) L H_m, estimated over seeds at every workload shape;
* the Feistel block order is a bijection.
"""
import math
import os

import numpy as np
import pytest

from oracle import model
from oracle import topk as otk
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_invariants(st, n, k, B, B2):
    assert st.max_len <= k + B2 + B - 1                     # len < k+B2 before the block, +B at most
    assert st.reads is not None and np.all(st.reads == 1)  # every element read exactly once
    assert st.W == st.A + k * st.R                          # each in-loop call carries k into the next call
    assert st.R * B2 <= st.A                                # each in-loop call removes at least B2
    assert st.W == sum(st.call_sizes)
    assert all(c >= k + B2 for c in st.call_sizes[:-1])     # in-loop calls fire at k+B2
    assert st.call_sizes[-1] >= min(k, n)                   # nothing is dropped before the first call
    key = [(t.v, t.pos, -t.j) for t in st.thresholds]
    assert key == sorted(key)                               # T never decreases


CASES = [
    # (family, dtype, N, k, B, B2)
    ("normal", gen.BF16, 5000, 64, 256, 256),
    ("normal", gen.FP32, 4097, 1, 64, 1),
    ("ties", gen.BF16, 20000, 64, 128, 128),
    ("ties", gen.FP32, 7000, 300, 512, 200),
    ("specials", gen.FP32, 3000, 100, 100, 50),
    ("specials", gen.BF16, 3000, 2999, 128, 64),
    ("ascending", gen.BF16, 9000, 128, 256, 512),
    ("descending", gen.FP32, 9000, 128, 256, 128),
    ("constant", gen.BF16, 2000, 500, 64, 64),
    ("tiny", gen.BF16, 4000, 77, 100, 33),
    ("neg", gen.FP32, 2500, 2500, 1024, 1024),
    ("normal", gen.FP32, 300, 20, 1024, 1024),               # N < B: a single partial block
]


@pytest.mark.parametrize("family,dtype,n,k,B,B2", CASES)
@pytest.mark.parametrize("order", ["feistel", "uniform", "sequential"])
def test_model_matches_oracle(family, dtype, n, k, B, B2, order):
    x = gen.rows_family(family, dtype, 29, 3, n)
    _, want = otk.topk(x, k)
    for r in range(x.shape[0]):
        got, stats = model.deepselect_row(x[r], k, B, B2, order, seed=r + 1, row_id=r)
        assert got.tolist() == want[r].tolist()
        assert len(stats) == 1
        _check_invariants(stats[0], n, k, B, B2)


@pytest.mark.parametrize("slice_blocks", [1, 2, 5])
@pytest.mark.parametrize("family", ["normal", "ties", "ascending"])
def test_split_rows_match_oracle(slice_blocks, family):
    n, k, B, B2 = 10000, 200, 256, 256
    x = gen.rows_family(family, gen.BF16, 31, 2, n)
    _, want = otk.topk(x, k)
    for r in range(2):
        got, stats = model.deepselect_row(x[r], k, B, B2, "feistel", seed=9, row_id=r, slice_len=slice_blocks * B)
        assert got.tolist() == want[r].tolist()
        assert len(stats) == -(-n // (slice_blocks * B))
        for st in stats:
            _check_invariants(st, st.reads.size, k, B, B2)


def test_value_only_threshold_is_wrong_on_ties():
    """The composite threshold is needed: a value-only strict filter drops tied elements with
    smaller indices (so the plain reading of the pseudocode loses the tie rule)."""
    n, k, B, B2 = 20000, 64, 128, 128
    x = gen.rows_family("ties", gen.FP32, 3, 1, n)
    v = x[0].astype(np.float64)
    order = model.block_order("feistel", -(-n // B), seed=1)
    cand, thr = np.zeros(0, np.int64), None
    for b in order:
        js = np.arange(b * B, min((b + 1) * B, n))
        keep = js if thr is None else js[v[js] > thr]
        cand = np.concatenate([cand, keep])
        if cand.size >= k + B2:
            cand = cand[np.lexsort((cand, -v[cand]))[:k]]
            thr = v[cand].min()
    cand = cand[np.lexsort((cand, -v[cand]))[:k]]
    _, want = otk.topk(x, k)
    assert sorted(cand.tolist()) != sorted(want[0].tolist())
    got, _ = model.deepselect_row(x[0], k, B, B2, "feistel", seed=1)
    assert got.tolist() == want[0].tolist()


def _read_table():
    rows = []
    with open(os.path.join(GOLDEN, "block_order_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            inp, order, A, R, W, wn, ok = line.split()
            rows.append((inp, order, int(A), int(R), int(W), float(wn), ok == "True"))
    return rows


def _table_input(kind, n, seed=0):
    g = np.random.default_rng(seed)
    if kind == "random":
        return g.permutation(n).astype(np.float32)
    if kind == "ascending":
        return np.arange(n, dtype=np.float32)
    if kind == "descending":
        return np.arange(n, dtype=np.float32)[::-1].copy()
    raise ValueError(kind)


def test_block_order_table():
    n, k, B, B2 = 262144, 512, 1024, 1024
    table = _read_table()
    for inp, order, A, R, W, wn, ok in table:
        assert W == A + k * R                        # every printed row satisfies W = A + kR
        assert abs(W / n - wn) < 0.0006
        if inp == "staircase":
            continue                                 # undefined on the page
        x = _table_input(inp, n)
        want = np.argsort(-x, kind="stable")[:k]
        fam = "sequential" if order == "sequential" else "uniform"
        got, (st,) = model.deepselect_row(x, k, B, B2, fam, seed=12345)
        assert got.tolist() == want.tolist()
        if order == "sequential" and inp in ("ascending", "descending"):
            assert (st.A, st.R, st.W) == (A, R, W)  # deterministic: exact reproduction
        else:
            assert 0.02 < st.W / n < 0.06            # random order: W/N of a few percent
            assert 0.5 * A < st.A < 2.0 * A


def test_complexity_tables():
    k, B, B2 = 512, 1024, 1024
    with open(os.path.join(GOLDEN, "complexity_table2.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            n, bound, asym, klog, ratio = line.split()
            n = int(n)
            b = model.expected_work_bound(n, k, B, B2)
            a = model.asymptotic_work(n, k, B, B2)
            assert round(b) == int(bound)
            assert round(a) == int(asym)
            assert round(model.klogn(n, k)) == int(klog)
            assert round(b / a, 2) == float(ratio)
    facts = {}
    with open(os.path.join(GOLDEN, "cost_model.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, val = line.split()
            facts[name] = int(val)
    n = 1 << 20
    assert n == facts["table4_read"]
    assert n * int(math.log2(k)) == facts["table4_sort_model"]
    assert abs(model.expected_work_bound(n, k, 1024, 1024) - facts["bound_n1m_b1024"]) < 100
    assert abs(model.expected_work_bound(n, k, 8192, 4096) - facts["bound_n1m_b8192_b4096"]) < 500
    assert abs(model.harmonic(128) - 5.433147) < 1e-6


def test_feistel_is_bijection():
    for m in list(range(1, 1100)) + [2047, 2048, 2049, 4095, 4096, 65535, 65537, 100003, 262143, 262144]:
        p = model.feistel_order(m, seed=m * 7 + 1, row=m % 5, slice_=m % 3)
        assert p.size == m
        assert np.array_equal(np.sort(p), np.arange(m))


# workload shapes for the bound check: (name, N, k, B, B2, families, seeds)
BOUND_SHAPES = [
    ("c1_small", 32768, 512, 1024, 1024, ("normal", "ascending"), 200),
    ("c2_indexer", 131072, 512, 1024, 1024, ("indexer", "ascending"), 200),
    ("c3_sampler", 129280, 512, 1024, 1024, ("sampler", "ascending"), 200),
    ("c4_long", 1048576, 512, 1024, 1024, ("normal", "ascending", "quantised"), 40),
    ("c4_long_k4096", 1048576, 4096, 4096, 4096, ("normal", "ascending"), 40),
    ("c5_slice", 1 << 18, 32, 1024, 1024, ("grid",), 200),
]


def _bound_row(kind, n):
    if kind == "normal":
        return gen.rows_normal_bf16(77, 1, n)[0]
    if kind == "ascending":
        return gen.rows_long_bf16(78, 5, n)[4]
    if kind == "indexer":
        return gen.rows_indexer_bf16(79, 1, n)[0]
    if kind == "sampler":
        return gen.rows_sampler_f32(80, 1, n)[0]
    if kind == "quantised":
        return gen.rows_long_bf16(81, 4, n)[3]
    if kind == "grid":
        return gen.rows_grid_f32(82, 1, n)[0]
    raise ValueError(kind)


def _work_only(v, pos, n, k, B, B2, order):
    _, st = model.deepselect_range(v, pos, 0, n, k, B, B2, order)
    return st.W


@pytest.mark.parametrize("shape", BOUND_SHAPES, ids=[s[0] for s in BOUND_SHAPES])
def test_expected_work_bound(shape):
    name, n, k, B, B2, kinds, seeds = shape
    bound = model.expected_work_bound(n, k, B, B2)
    m = -(-n // B)
    for kind in kinds:
        row = _bound_row(kind, n)
        v = model.widen(row)
        pos = (~np.signbit(v)).astype(np.int64)
        for fam in ("uniform", "feistel"):
            ws = [_work_only(v, pos, n, k, B, B2, model.block_order(fam, m, seed=s, row=s % 7))
                  for s in range(seeds)]
            mean = float(np.mean(ws))
            half = 1.96 * float(np.std(ws)) / math.sqrt(len(ws))
            assert mean + half <= bound, (name, kind, fam, mean, half, bound)
