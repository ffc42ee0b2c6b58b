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


# The plans the library ships for the workloads (one slice each): (name, slice length, k, B,
# B2, G, presample waves or None, blocks covered by the presample, rows, seeds). A grouped
# order reads G consecutive blocks in turn, so the bound's analysis applies to super-blocks of
# G*B elements: m = ceil(N / (G*B)) and L = k + G*B + B2.
SHIPPED_PLANS = [
    ("indexer_slice", 32768, 512, 8192, 4096, 1, 16, 4, ("indexer", "ascending"), 60),
    ("sampler_row", 129280, 512, 8192, 4096, 2, 16, 4, ("sampler", "sampler_ascending"), 30),
    ("long_k4096_slice", 32768, 4096, 4096, 4096, 2, None, 4, ("normal", "ascending"), 60),
    ("giant_slice", 1 << 20, 32, 16384, 1024, 2, 16, 2, ("grid", "grid_ascending"), 80),
]


def _shipped_row(kind, n):
    if kind == "sampler_ascending":
        return np.sort(gen.rows_sampler_f32(80, 1, n)[0])
    if kind == "grid_ascending":
        return np.sort(gen.rows_grid_f32(82, 1, n)[0])
    return _bound_row(kind, n)


def grouped_bound(n, k, B, B2, G):
    """The boxed bound with the block replaced by a group of G blocks."""
    m = -(-n // (G * B))
    return (1.0 + k / B2) * (k + G * B + B2) * model.harmonic(m)


def test_grouped_bound_reduces_to_the_boxed_bound():
    for n, k, B, B2 in [(32768, 512, 1024, 1024), (1 << 20, 4096, 4096, 4096), (129280, 512, 8192, 4096)]:
        assert grouped_bound(n, k, B, B2, 1) == model.expected_work_bound(n, k, B, B2)


@pytest.mark.parametrize("plan", SHIPPED_PLANS, ids=[p[0] for p in SHIPPED_PLANS])
def test_expected_work_bound_at_shipped_plans(plan):
    """Mean W over block-order seeds (95% upper confidence) stays under the bound at the plans
    the library runs: its B and B2, its order groups and its presampled start."""
    name, n, k, B, B2, G, waves, depth, kinds, seeds = plan
    bound = grouped_bound(n, k, B, B2, G)
    for kind in kinds:
        row = _shipped_row(kind, n)
        ws = []
        for s in range(seeds):
            _, st = model.deepselect_row(row, k, B, B2, "feistel", seed=s + 1, row_id=s % 5, group=G,
                                         presample_waves=waves, presample_depth=depth)
            assert len(st) == 1
            ws.append(st[0].W)
        mean = float(np.mean(ws))
        half = 1.96 * float(np.std(ws)) / math.sqrt(len(ws))
        assert mean + half <= bound, (name, kind, mean, half, bound)


# ----------------------------------------------------------------------------- grouped order, presample
def test_keys_follow_numeric_order():
    """keys_of orders values as numbers do, with +0 above -0 (bf16 and fp32, specials too)."""
    for dtype in (gen.BF16, gen.FP32):
        x = np.concatenate([gen.rows_family(f, dtype, 61, 1, 4000)[0] for f in ("normal", "specials", "tiny", "neg")])
        keys = model.keys_of(x).astype(np.int64)
        v = model.widen(x)
        pos = (~np.signbit(v)).astype(np.int64)
        by_key = np.argsort(keys, kind="stable")
        by_value = np.lexsort((pos, v))  # value ascending, -0 before +0
        assert np.array_equal(keys[by_key], keys[by_value])
        same = (v[:, None] == v[None, :]) & (pos[:, None] == pos[None, :])
        assert np.array_equal(same[:200, :200], (keys[:200, None] == keys[None, :200]))
    one, mone = np.array([0x3F80], np.uint16), np.array([0xBF80], np.uint16)  # bf16 +1.0, -1.0
    assert int(model.keys_of(one)[0]) == 0xBF80 and int(model.keys_of(mone)[0]) == 0x407F
    z = np.array([0.0, -0.0], np.float32)
    assert model.keys_of(z).tolist() == [0x80000000, 0x7FFFFFFF]


@pytest.mark.parametrize("m,group", [(1, 2), (7, 2), (8, 2), (16, 2), (13, 4), (5, 1)])
def test_grouped_order_structure(m, group):
    order = model.grouped_order(m, group, seed=9, row=3, slice_=1)
    assert sorted(order.tolist()) == list(range(m))
    groups = model.feistel_order(-(-m // group), 9, 3, 1)
    want = [g * group + j for g in groups for j in range(group) if g * group + j < m]
    assert order.tolist() == want
    if group == 1:
        assert order.tolist() == model.feistel_order(m, 9, 3, 1).tolist()


def _brute_t0(blocks, k, waves, vec, bits):
    """T0 by its definition, with an explicit search per wave: the largest value whose low
    (bits - 16) bits are zero that at least ceil(k/waves) lane maxima reach."""
    lane_max = {}
    for kb in blocks:
        for o, key in enumerate(kb.tolist()):
            lane = ((o // (64 * vec)) % waves, (o % (64 * vec)) // vec)
            lane_max[lane] = max(lane_max.get(lane, 0), key)
    j = -(-k // waves)
    out = []
    for w in range(waves):
        maxima = [lane_max.get((w, l), 0) for l in range(64)]
        best = 0
        for top16 in range(1 << 16):
            v = top16 << (bits - 16)
            if sum(mx >= v for mx in maxima) >= j:
                best = v
            else:
                break
        out.append(best)
    return min(out)


@pytest.mark.parametrize("dtype,waves,k,nblocks", [(gen.BF16, 2, 100, 1), (gen.BF16, 2, 128, 2),
                                                    (gen.FP32, 4, 256, 1), (gen.FP32, 4, 7, 2)])
@pytest.mark.parametrize("family", ["normal", "ties", "neg"])
def test_presample_key(dtype, waves, k, nblocks, family):
    """T0 equals its definition (a brute-force search per wave) and at least k of the
    sampled elements reach it, so it never exceeds their k-th largest key."""
    vec = 8 if dtype == gen.BF16 else 4
    bits = 16 if dtype == gen.BF16 else 32
    B = waves * 64 * vec
    x = gen.rows_family(family, dtype, 63, 1, nblocks * B)[0]
    keys = model.keys_of(x)
    blocks = [keys[b * B:(b + 1) * B] for b in range(nblocks)]
    t0 = model.presample_key(blocks, k, model.Presample(waves, vec, bits))
    if family != "ties" or dtype == gen.BF16:  # the brute force walks 2^16 candidates at most
        assert t0 == _brute_t0(blocks, k, waves, vec, bits)
    assert int((keys >= np.uint64(t0)).sum()) >= k
    assert t0 <= int(np.sort(keys)[::-1][k - 1])


@pytest.mark.parametrize("family", ["normal", "ascending", "ties", "specials"])
@pytest.mark.parametrize("dtype,n,k,B,slice_len,group,depth", [
    (gen.BF16, 20000, 100, 1024, None, 2, 4),   # 20 blocks, the first four presampled
    (gen.BF16, 6000, 128, 1024, None, 1, 2),    # 6 blocks: the first two presampled
    (gen.FP32, 9000, 200, 1024, 4096, 2, 4),    # slices of 4 blocks, groups of two
    (gen.FP32, 3000, 50, 1024, None, 4, 4),     # a short last group
])
def test_model_grouped_presampled_matches_oracle(family, dtype, n, k, B, slice_len, group, depth):
    """The grouped order and the presampled start keep the result exact and the design
    note's invariants; on i.i.d. rows the presampled start appends fewer elements."""
    waves = 2 if dtype == gen.BF16 else 4
    x = gen.rows_family(family, dtype, 65, 2, n)
    _, want = otk.topk(x, k)
    for r in range(x.shape[0]):
        got, stats = model.deepselect_row(x[r], k, B, 256, seed=r + 3, row_id=r, slice_len=slice_len, group=group,
                                          presample_waves=waves, presample_depth=depth)
        assert got.tolist() == want[r].tolist()
        for st in stats:
            _check_invariants(st, n, k, B, 256)
        if family == "normal":
            _, plain = model.deepselect_row(x[r], k, B, 256, seed=r + 3, row_id=r, slice_len=slice_len, group=group)
            assert sum(s.A for s in stats) < sum(s.A for s in plain)


@pytest.mark.parametrize("m,group,depth", [(6, 1, 4), (7, 2, 4), (5, 2, 4), (1, 2, 4), (9, 4, 2), (3, 4, 4)])
def test_first_positions_follow_the_grouped_order(m, group, depth):
    """The presampled blocks are the first positions of the processing order, the padding of
    a short last group left out (the grouped order lists the same blocks in the same order)."""
    firsts = model.first_positions(m, group, depth, 5, 1, 0)
    order = model.grouped_order(m, group, 5, 1, 0) if group > 1 else model.feistel_order(m, 5, 1, 0)
    assert firsts == [int(b) for b in order[:len(firsts)]]
    assert len(firsts) <= depth and all(0 <= b < m for b in firsts)
    if group > 1:
        ng = -(-m // group)
        drawn = model.feistel_order(ng, 5, 1, 0)[:-(-depth // group)]
        if m % group == 0 or ng - 1 not in drawn.tolist():
            assert len(firsts) == min(depth, m)  # padding only comes from a short last group
    else:
        assert len(firsts) == min(depth, m)


# ----------------------------------------------------------------------------- warm-up window
@pytest.mark.parametrize("family", ["normal", "ascending", "descending", "ties", "specials"])
@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("warmup", [1, 2, 5])
def test_warmup_window_matches_oracle(family, dtype, warmup):
    x = gen.rows_family(family, dtype, 21, 3, 20000)
    for r in range(3):
        got, st = model.deepselect_row(x[r], 300, 1024, 2048, "feistel", seed=r + 4, row_id=r, warmup=warmup)
        _, want = otk.topk(x[r:r + 1], 300)
        assert got.tolist() == want[0].tolist()
        s = st[0]
        assert s.W == s.A + 300 * s.R and s.max_len <= 300 + 2048 + 1024 - 1
        assert (s.reads == 1).all()


def test_warmup_threshold_is_the_windows_kth_element():
    """After a window of w blocks (w*B > k, below the k + B2 trigger) the first threshold is
    the k-th best element of those w blocks, found here by the sorting oracle."""
    x = gen.rows_family("normal", gen.FP32, 22, 1, 40 * 1024)[0]
    k, B, B2 = 700, 1024, 8192
    for w in (1, 2, 3, 6):
        order = model.block_order("feistel", 40, seed=w, row=0)
        _, st = model.deepselect_range(model.widen(x), (~np.signbit(model.widen(x))).astype(np.int64), 0, x.size,
                                       k, B, B2, order, warmup=w)
        blocks = np.concatenate([np.arange(int(b) * B, int(b) * B + B) for b in order[:w]])
        if w * B <= k:
            assert not st.thresholds or st.call_sizes[0] >= k + B2
            continue
        _, idx = otk.topk(x[None, blocks], k)
        kth = int(blocks[idx[0, -1]])
        assert st.thresholds[0].j == kth and st.call_sizes[0] == w * B


@pytest.mark.parametrize("kind", ["normal", "ascending"])
def test_warmup_work_against_the_bound(kind):
    """A and W with a warm-up window, over block-order seeds, against the boxed bound (the
    window only adds a compaction at a fixed point of the order) and against the run without
    a window on the same orders (i.i.d. rows: the window appends fewer elements)."""
    n, k, B, B2 = 131072, 512, 1024, 4096
    row = _bound_row(kind, n)
    bound = model.expected_work_bound(n, k, B, B2)
    a0, a1, w1 = [], [], []
    for s in range(40):
        _, st0 = model.deepselect_row(row, k, B, B2, "feistel", seed=s + 1, row_id=s % 3)
        _, st1 = model.deepselect_row(row, k, B, B2, "feistel", seed=s + 1, row_id=s % 3, warmup=1)
        a0.append(st0[0].A)
        a1.append(st1[0].A)
        w1.append(st1[0].W)
    mean = float(np.mean(w1))
    half = 1.96 * float(np.std(w1)) / math.sqrt(len(w1))
    assert mean + half <= bound, (kind, mean, half, bound)
    if kind == "normal":
        assert np.mean(a1) < np.mean(a0)


# ----------------------------------------------------------------------------- shared row threshold
@pytest.mark.parametrize("family", ["normal", "ascending", "descending", "ties", "specials", "neg"])
@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
def test_shared_threshold_matches_oracle(family, dtype):
    """Slices that publish their thresholds to the row and filter with the row's still give
    the oracle's top-k (every published value ranks at or below the row's k-th element)."""
    x = gen.rows_family(family, dtype, 23, 2, 40000)
    for r in range(2):
        for slice_len, presample in ((4096, None), (8192, 16), (12288, 16)):
            got, st = model.deepselect_row(x[r], 500, 1024, 1024, "feistel", seed=r + 9, row_id=r,
                                           slice_len=slice_len, presample_waves=presample, share=True)
            _, want = otk.topk(x[r:r + 1], 500)
            assert got.tolist() == want[0].tolist(), (family, dtype, r, slice_len)
            for s in st:
                assert s.W == s.A + 500 * s.R and s.max_len <= 500 + 1024 + 1024 - 1


def test_shared_threshold_cuts_work_on_a_descending_row():
    """A descending row split in eight: with the first slice's thresholds shared, the later
    slices append a fraction of what they append alone."""
    x = gen.rows_family("descending", gen.FP32, 24, 1, 65536)[0]
    plain = model.deepselect_row(x, 512, 1024, 1024, "feistel", seed=3, slice_len=8192)[1]
    shared = model.deepselect_row(x, 512, 1024, 1024, "feistel", seed=3, slice_len=8192, share=True)[1]
    a_plain = sum(s.A for s in plain[1:])
    a_shared = sum(s.A for s in shared[1:])
    assert shared[0].A == plain[0].A and a_shared < 0.25 * a_plain, (a_shared, a_plain)
