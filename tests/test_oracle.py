"""Pins for the sorting oracle: brute force, special cases and a library sort.

None of these checks re-states the oracle's comparator: brute force counts ranks with a
tuple key, the special cases have closed-form answers, and numpy's lexsort is a library
routine with its own encoding of the order.
"""
import itertools

import numpy as np
import pytest

from oracle import brute
from oracle import topk as otk
from workloads import gen

ALPHABET = [-np.inf, -1.0, -0.0, 0.0, 1.0, 2.0, np.inf]


def _as_dtype(vals, dtype):
    a = np.asarray(vals, np.float32)
    return gen.bf16_bits_from_f32(a) if dtype == gen.BF16 else a


def _widen(x):
    return gen.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_exhaustive_alphabet_vs_brute(dtype, n):
    rows = np.array(list(itertools.product(ALPHABET, repeat=n)), np.float32)
    x = _as_dtype(rows, dtype)
    xv = _widen(x)
    for k in range(1, n + 1):
        vals, idx = otk.topk(x, k)
        for r in range(x.shape[0]):
            want = brute.brute_topk(list(xv[r]), k)
            assert idx[r].tolist() == want, (rows[r], k)
            assert np.array_equal(vals[r], x[r, want])


def test_batch_brute_agrees_with_row_brute():
    """The vectorised rank count against the per-row one, on every 4-element alphabet row."""
    rows = np.array(list(itertools.product(ALPHABET, repeat=4)), np.float64)
    order = brute.brute_order_batch(rows)
    for r in range(0, rows.shape[0], 7):
        assert order[r].tolist() == brute.brute_topk(list(rows[r]), 4)


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
@pytest.mark.parametrize("n", [5, 6, 7])
def test_exhaustive_alphabet_vs_batch_brute(dtype, n):
    """Every row of n <= 7 elements over the 7-value alphabet (signed zeros, infinities,
    ties), every k: the oracle's output equals the rank count's."""
    rows = np.array(list(itertools.product(ALPHABET, repeat=n)), np.float32)
    x = _as_dtype(rows, dtype)
    order = np.concatenate([brute.brute_order_batch(_widen(x[i:i + 65536])) for i in range(0, x.shape[0], 65536)])
    for k in range(1, n + 1):
        vals, idx = otk.topk(x, k)
        assert np.array_equal(idx, order[:, :k]), k
        assert np.array_equal(vals, np.take_along_axis(x, order[:, :k], axis=1)), k


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
def test_random_tiny_ties_vs_brute(dtype):
    g = np.random.default_rng(7)
    for trial in range(300):
        n = int(g.integers(1, 40))
        k = int(g.integers(1, n + 1))
        vals = np.array(ALPHABET + [0.5, -0.5, 3.0], np.float32)[g.integers(0, 10, size=n)]
        x = _as_dtype(vals[None, :], dtype)
        v, i = otk.topk(x, k)
        want = brute.brute_topk(list(_widen(x)[0]), k)
        assert i[0].tolist() == want
        assert np.array_equal(v[0], x[0, want])


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
def test_special_cases(dtype):
    n = 1000
    # constant row: the first k indices
    x = _as_dtype(np.full((1, n), 1.5, np.float32), dtype)
    _, i = otk.topk(x, 37)
    assert i[0].tolist() == list(range(37))
    # strictly increasing row (integers, exact in bf16 too): the last k indices, largest first
    m = 250
    x = _as_dtype(np.arange(m, dtype=np.float32)[None, :] - 125.0, dtype)
    _, i = otk.topk(x, 10)
    assert i[0].tolist() == list(range(m - 1, m - 11, -1))
    # k == N on a row without zeros: the stable descending sort
    g = np.random.default_rng(3)
    f = g.integers(1, 20, size=n).astype(np.float32) * np.where(g.random(n) < 0.5, -1, 1).astype(np.float32)
    x = _as_dtype(f[None, :], dtype)
    _, i = otk.topk(x, n)
    assert i[0].tolist() == np.argsort(-_widen(x)[0], kind="stable").tolist()
    # k == 1: the first position of the maximum
    _, i = otk.topk(x, 1)
    assert i[0, 0] == int(np.argmax(_widen(x)[0]))
    # +0 ranks before -0, whatever their positions
    x = _as_dtype(np.array([[-0.0, -1.0, 0.0, -0.0, 0.0]], np.float32), dtype)
    _, i = otk.topk(x, 5)
    assert i[0].tolist() == [2, 4, 0, 3, 1]


def _lexsort_topk(x, k):
    v = _widen(x)
    out = np.empty((x.shape[0], k), np.int64)
    for r in range(x.shape[0]):
        pos = (~np.signbit(v[r])).astype(np.int64)
        out[r] = np.lexsort((np.arange(v.shape[1]), -pos, -v[r]))[:k]
    return out


@pytest.mark.parametrize("family", ["normal", "ties", "specials", "tiny", "neg", "ascending"])
@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
def test_medium_vs_library_sort(family, dtype):
    x = gen.rows_family(family, dtype, 11, 6, 20000)
    for k in (1, 64, 512, 4096):
        vals, idx = otk.topk(x, k)
        want = _lexsort_topk(x, k)
        assert np.array_equal(idx, want)
        assert np.array_equal(vals, np.take_along_axis(x, want, 1))


def test_chunked_long_row_vs_library_sort():
    # one row longer than 2^20 with several threads takes the chunk-sort + merge path
    x = gen.rows_grid_f32(5, 1, (1 << 20) + 12345, bits=12)  # heavy ties
    vals, idx = otk.topk(x, 300, threads=8)
    want = _lexsort_topk(x, 300)
    assert np.array_equal(idx, want)
    assert np.array_equal(vals, np.take_along_axis(x, want, 1))


def test_values_only_and_rejects():
    x = gen.rows_family("normal", gen.FP32, 1, 3, 100)
    v, i = otk.topk(x, 5, indices=False)
    assert i is None and v.shape == (3, 5)
    with pytest.raises(ValueError):
        otk.topk(x, 101)
    with pytest.raises(ValueError):
        otk.topk(x, 0)


@pytest.mark.parametrize("dtype", [gen.BF16, gen.FP32])
def test_ragged_rows_vs_brute(dtype):
    """Ragged rows: each row's first L elements against the rank count with k' = min(k, L);
    the positions past a short row's length are padding (index -1, value bits all ones)."""
    g = np.random.default_rng(11)
    rows, n, k = 40, 30, 9
    vals = np.array(ALPHABET + [0.5, -0.5, 3.0], np.float32)[g.integers(0, 10, size=(rows, n))]
    x = _as_dtype(vals, dtype)
    lens = g.integers(-3, n + 4, size=rows)
    lens[:4] = [0, 1, k, n]
    v, i = otk.topk_ragged(x, lens, k)
    pad = otk.padding_value(x.dtype)
    for r in range(rows):
        L = min(max(int(lens[r]), 0), n)
        kk = min(k, L)
        want = brute.brute_topk(list(_widen(x)[r, :L]), kk) if kk else []
        assert i[r, :kk].tolist() == want
        assert np.array_equal(v[r, :kk], x[r, want])
        assert (i[r, kk:] == -1).all()
        assert (v[r, kk:].view(pad.dtype) == pad).all() if dtype == gen.BF16 else \
            (v[r, kk:].view(np.uint32) == 0xFFFFFFFF).all()


def test_ragged_full_lengths_equal_plain_topk():
    x = gen.rows_family("normal", gen.FP32, 12, 6, 5000)
    v, i = otk.topk_ragged(x, np.full(6, 5000), 100)
    wv, wi = otk.topk(x, 100)
    assert np.array_equal(i, wi) and np.array_equal(v.view(np.uint32), wv.view(np.uint32))
