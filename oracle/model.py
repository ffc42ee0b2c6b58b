"""Instrumented CPU model of DeepSelect. TEST INFRASTRUCTURE ONLY.

Follows the DeepSelect design note ("Algorithm", the DeepSelectTopk pseudocode, and
"Expected Upper Bound on the Total Elements Processed by RadixSelectTopK"), restated in
the tutorial chapter (sections 2.2-2.4 and 3). Names follow the pages: ``B`` block size,
``B2`` compaction slack, ``T`` the threshold, ``A`` appended count, ``R`` in-loop
compactions, ``W`` the summed input sizes of all RadixSelectTopK calls, ``m`` the number
of blocks, ``L = k + B + B2``, ``H_m`` the m-th harmonic number.

Readings (where the pages leave a step open):

* Ties. The pages assume distinct elements. Here every element is the pair
  (value, index) under one total order: larger value first, +0 before -0, then smaller
  index first. The threshold is such a pair and "x > T" is the strict comparison in this
  order, so all pairs are distinct and the pseudocode applies as written.
* Initial threshold -inf means "accept everything" until the first compaction.
* RadixSelectTopK(c, k) returns exactly the k best pairs of c. The pages allow "radix
  select, or another top-k algorithm"; the model uses a library sort (numpy lexsort) for
  that step, which is exact. The internal order of the kept set is irrelevant.
* The compaction test runs once after each whole block (the pseudocode's placement).

Block orders: ``sequential`` (identity), ``uniform`` (numpy permutation from a seed, the
hypothesis of the bound) and ``feistel``, the keyed bijection the GPU kernels use, written
here from its specification:

  mix64(z)      = splitmix64 finaliser: z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
                  z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31   (mod 2^64)
  lowbias32(x)  = x ^= x>>16; x *= 0x7FEB352D; x ^= x>>15; x *= 0x846CA68B; x ^= x>>16 (mod 2^32)
  hs  = mix64(seed)
  key_r = low 32 bits of mix64(hs XOR (row<<33 | slice<<2 | r)), r = 0..3
  width: the smallest even b >= 2 with 2^b >= m; half = b/2; mask = 2^half - 1
  round (L, R) -> (R, L ^ (lowbias32(R ^ key_r) & mask)), four rounds, value (L<<half)|R
  pi(i) = first value < m on the cycle i -> F(i) -> F(F(i)) ... (cycle walking); m = 1 -> 0.

Two switchable departures of the GPU kernels from the design note are modelled too (both
leave the result unchanged, only the counts):

* grouped order: the Feistel bijection is drawn over ceil(m/G) groups of G consecutive
  blocks, and the blocks of a group are read in turn (positions past the last block are
  skipped);
* presampled start: instead of "accept everything", the first block read, when it is
  whole, sets T0 = the smallest over the workgroup's waves of each wave's j-th largest
  lane maximum (j = ceil(k / waves)), with the low (key bits - 16) key bits cleared; every
  element with key >= T0 is appended until the first compaction. A lane's maximum is over
  its elements of every whole block among the first `depth` positions of the order (the
  blocks the kernel has requested before it filters anything; lane l of wave w holds, in
  every 16-byte chunk c of a block with c mod waves = w, the elements at l*vec ..
  l*vec+vec-1; vec = 16 / element bytes). With groups of G blocks, position d is block
  G*g(d // G) + d mod G of the group order g, and positions past the last block are empty.
  Keys are the order-preserving unsigned images of the raw bits: sign bit clear -> set the
  sign bit, sign bit set -> invert every bit.

Slices (the split-row path): slice s of a row covers [s*Ls, min((s+1)*Ls, N)) for a slice
length Ls that is a multiple of B; each slice runs the method on its own elements with its
own block order (row, slice) and keeps its k best (or all, if fewer); the row's answer is
the k best of the union of the slices' survivors.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

_M64 = (1 << 64) - 1


# ----------------------------------------------------------------------------- values
def widen(row: np.ndarray) -> np.ndarray:
    """Exact float64 values of a row given as bf16 bits (uint16) or float32."""
    if row.dtype == np.uint16:
        return (row.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if row.dtype == np.float32:
        return row.astype(np.float64)
    raise ValueError("row must be uint16 (bf16 bits) or float32")


@dataclasses.dataclass(frozen=True)
class Pair:
    """One element of the total order: value, positive-zero flag, index."""
    v: float
    pos: int  # 1 when the sign bit is clear (only decides between +0 and -0)
    j: int


def _beats(v: np.ndarray, pos: np.ndarray, j: np.ndarray, t: Pair) -> np.ndarray:
    """Elementwise: does (v, pos, j) rank strictly before the pair t?"""
    return (v > t.v) | ((v == t.v) & ((pos > t.pos) | ((pos == t.pos) & (j < t.j))))


def _order(v: np.ndarray, pos: np.ndarray, j: np.ndarray) -> np.ndarray:
    """Positions that sort the pairs best first (value desc, +0 before -0, index asc)."""
    return np.lexsort((j, -pos, -v))


# ----------------------------------------------------------------------------- block orders
def mix64(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def _lowbias32(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.uint64) & np.uint64(0xFFFFFFFF)
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(0x7FEB352D)) & np.uint64(0xFFFFFFFF)
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(0x846CA68B)) & np.uint64(0xFFFFFFFF)
    x ^= x >> np.uint64(16)
    return x


def feistel_keys(seed: int, row: int, slice_: int) -> List[int]:
    hs = mix64(seed)
    return [mix64(hs ^ ((row << 33) | (slice_ << 2) | r)) & 0xFFFFFFFF for r in range(4)]


def _feistel_width(m: int) -> int:
    b = 2
    while (1 << b) < m:
        b += 2
    return b


def feistel_order(m: int, seed: int, row: int = 0, slice_: int = 0) -> np.ndarray:
    """Block ids in processing order under the keyed Feistel bijection with cycle walking."""
    if m <= 1:
        return np.zeros(m, np.int64)
    keys = feistel_keys(seed, row, slice_)
    half = _feistel_width(m) // 2
    mask = np.uint64((1 << half) - 1)

    def f(x: np.ndarray) -> np.ndarray:
        left, right = x >> np.uint64(half), x & mask
        for kr in keys:
            left, right = right, left ^ (_lowbias32(right ^ np.uint64(kr)) & mask)
        return (left << np.uint64(half)) | right

    y = f(np.arange(m, dtype=np.uint64))
    bad = y >= np.uint64(m)
    while bad.any():
        y[bad] = f(y[bad])
        bad = y >= np.uint64(m)
    return y.astype(np.int64)


def block_order(family: str, m: int, seed: int = 0, row: int = 0, slice_: int = 0) -> np.ndarray:
    if family == "sequential":
        return np.arange(m, dtype=np.int64)
    if family == "uniform":
        return np.random.Generator(np.random.PCG64(seed)).permutation(m).astype(np.int64)
    if family == "feistel":
        return feistel_order(m, seed, row, slice_)
    raise ValueError(f"unknown block order family {family!r}")


def grouped_order(m: int, group: int, seed: int, row: int = 0, slice_: int = 0) -> np.ndarray:
    """Blocks in processing order when the random order is over groups of `group`
    consecutive blocks: group g = feistel(i) contributes blocks g*group .. g*group+group-1."""
    if group == 1:
        return feistel_order(m, seed, row, slice_)
    groups = feistel_order(-(-m // group), seed, row, slice_)
    out = [int(g) * group + j for g in groups for j in range(group) if int(g) * group + j < m]
    return np.asarray(out, np.int64)


# ----------------------------------------------------------------------------- keys, presample
def keys_of(row: np.ndarray) -> np.ndarray:
    """Order-preserving unsigned keys of a row given as bf16 bits (uint16) or float32."""
    if row.dtype == np.uint16:
        b, sign, mask = row.astype(np.uint64), 0x8000, 0xFFFF
    elif row.dtype == np.float32:
        b, sign, mask = row.view(np.uint32).astype(np.uint64), 0x80000000, 0xFFFFFFFF
    else:
        raise ValueError("row must be uint16 (bf16 bits) or float32")
    neg = (b & np.uint64(sign)) != 0
    return np.where(neg, (~b) & np.uint64(mask), b | np.uint64(sign)).astype(np.uint64)


@dataclasses.dataclass(frozen=True)
class Presample:
    """The kernel shape the presampled start depends on."""
    waves: int
    vec: int       # elements per lane per 16-byte chunk (8 bf16, 4 fp32)
    key_bits: int  # 16 (bf16) or 32 (fp32)


def presample_key(block_keys: List[np.ndarray], k: int, ps: Presample) -> int:
    """T0 from whole blocks' keys (each array one block, in element order)."""
    chunk = 64 * ps.vec
    lane_max = np.zeros((ps.waves, 64), np.uint64)
    for kb in block_keys:
        o = np.arange(kb.size)
        np.maximum.at(lane_max, ((o // chunk) % ps.waves, (o % chunk) // ps.vec), kb)
    j = -(-k // ps.waves)
    assert 1 <= j <= 64, "the presampled start needs k <= 64 * waves"
    shift = np.uint64(ps.key_bits - 16)
    per_wave = [(np.sort(lane_max[w])[::-1][j - 1] >> shift) << shift for w in range(ps.waves)]
    return int(min(per_wave))


# ----------------------------------------------------------------------------- the method
@dataclasses.dataclass
class RunStats:
    A: int = 0                      # elements appended to the candidate buffer
    R: int = 0                      # in-loop RadixSelectTopK calls
    W: int = 0                      # summed input sizes of all RadixSelectTopK calls (final included)
    max_len: int = 0                # largest buffer length seen (after a block's appends)
    call_sizes: List[int] = dataclasses.field(default_factory=list)  # inputs of every call, final last
    thresholds: List[Pair] = dataclasses.field(default_factory=list)  # T after each in-loop call
    reads: Optional[np.ndarray] = None  # times each element of the input range was read


def radix_select_topk(v: np.ndarray, pos: np.ndarray, j: np.ndarray, cand: np.ndarray, k: int) -> np.ndarray:
    """The k best candidates (positions into v); all of them when there are at most k."""
    if cand.size <= k:
        return cand
    o = _order(v[cand], pos[cand], j[cand])
    return cand[o[:k]]


def deepselect_range(v: np.ndarray, pos: np.ndarray, lo: int, hi: int, k: int, B: int, B2: int,
                     order: np.ndarray, keys: Optional[np.ndarray] = None,
                     presample: Optional[Presample] = None,
                     firsts: Optional[List[int]] = None, warmup: int = 0,
                     shared: Optional[List[int]] = None) -> Tuple[np.ndarray, RunStats]:
    """DeepSelectTopk over the elements [lo, hi) of a row (indices stay row-relative).

    ``order`` lists the blocks of the range in processing order (block b covers
    [lo + b*B, min(lo + (b+1)*B, hi))). With ``presample`` (and the row's ``keys``) the run
    starts from the presampled threshold when the first block read is whole; ``firsts`` are
    the blocks at the first positions of the order whose whole blocks the threshold covers.
    With ``warmup`` = w > 0 (the warm-up window of TileLang tutorial chapter 37, section
    5.2(1)) the buffer is also compacted right after the w-th block of the order when it
    holds more than k entries, so that T is the k-th best of the window's elements.
    With ``shared`` (a one-element list: the row's published threshold as a composite
    key << 32 | (~index & 0xFFFFFFFF), 0 for none; needs ``keys``) the range shares its
    threshold with the row's other ranges (the cluster split of the design note,
    "Implementation"): it reads the row's at its start, and whenever its own threshold is set
    (T0, a compaction) it publishes it with a maximum and reads back the row's; it appends
    only elements ranking above the larger of the two. Returns the kept positions (at most k, unordered) and the run's counts.
    """
    n = hi - lo
    assert n >= 1 and k >= 1 and B >= 1 and B2 >= 1
    m = -(-n // B)
    assert sorted(order.tolist()) == list(range(m)), "block order must be a permutation"
    st = RunStats(reads=np.zeros(n, np.int64))
    jall = np.arange(v.size, dtype=np.int64)
    cand = np.zeros(0, np.int64)
    thr: Optional[Pair] = None  # None: the threshold is -inf, every element is accepted
    t0: Optional[int] = None    # presampled start: keep key >= t0 until the first compaction

    def whole(b: int) -> bool:
        return lo + (b + 1) * B <= hi

    adopted = shared[0] if shared is not None else 0  # the row's threshold as last read (sharing)

    def publish(c: int) -> None:
        nonlocal adopted
        if shared is not None:
            shared[0] = max(shared[0], c)
            adopted = shared[0]

    if presample is not None and whole(int(order[0])):
        covered = [b for b in (firsts or [int(order[0])]) if whole(b)]
        t0 = presample_key([keys[lo + b * B:lo + (b + 1) * B] for b in covered], k, presample)
        publish(t0 << 32)  # index ~0: ties with T0 rank above it
    for position, b in enumerate(order):
        blo, bhi = lo + int(b) * B, min(lo + (int(b) + 1) * B, hi)
        js = np.arange(blo, bhi, dtype=np.int64)
        st.reads[blo - lo:bhi - lo] += 1
        if thr is not None:
            keep = js[_beats(v[js], pos[js], js, thr)]
        elif t0 is not None:
            keep = js[keys[js] >= np.uint64(t0)]
        else:
            keep = js
        if adopted:
            comp = (keys[keep].astype(np.uint64) << np.uint64(32)) | (~keep.astype(np.uint64) & np.uint64(0xFFFFFFFF))
            keep = keep[comp > np.uint64(adopted)]
        cand = np.concatenate([cand, keep])
        st.A += int(keep.size)
        st.max_len = max(st.max_len, int(cand.size))
        if cand.size >= k + B2 or (warmup > 0 and position + 1 == warmup and cand.size > k):
            st.W += int(cand.size)
            st.R += 1
            st.call_sizes.append(int(cand.size))
            cand = radix_select_topk(v, pos, jall, cand, k)
            worst = cand[_order(v[cand], pos[cand], cand)[-1]]
            thr = Pair(float(v[worst]), int(pos[worst]), int(worst))
            st.thresholds.append(thr)
            if shared is not None:
                publish((int(keys[worst]) << 32) | (~int(worst) & 0xFFFFFFFF))
    st.W += int(cand.size)
    st.call_sizes.append(int(cand.size))
    return radix_select_topk(v, pos, jall, cand, k), st


def sort_output(v: np.ndarray, pos: np.ndarray, kept: np.ndarray) -> np.ndarray:
    return kept[_order(v[kept], pos[kept], kept)]


def first_positions(m: int, group: int, depth: int, seed: int, row_id: int, slice_: int,
                    family: str = "feistel") -> List[int]:
    """Blocks at the first ``depth`` positions of the order (empty positions left out)."""
    if group == 1:
        return [int(b) for b in block_order(family, m, seed, row_id, slice_)[:depth]]
    g = feistel_order(-(-m // group), seed, row_id, slice_)
    out = []
    for d in range(min(depth, g.size * group)):
        b = int(g[d // group]) * group + d % group
        if b < m:
            out.append(b)
    return out


def deepselect_row(row: np.ndarray, k: int, B: int, B2: int, family: str = "feistel", seed: int = 0,
                   row_id: int = 0, slice_len: Optional[int] = None, group: int = 1,
                   presample_waves: Optional[int] = None,
                   presample_depth: int = 4, warmup: int = 0,
                   share: bool = False) -> Tuple[np.ndarray, List[RunStats]]:
    """DeepSelect on one row (bf16 bits or float32), optionally split into slices.

    ``group`` > 1 draws the Feistel order over groups of blocks; ``presample_waves`` (the
    workgroup's waves) turns on the presampled start, over the whole blocks among the first
    ``presample_depth`` positions of the order; ``warmup`` > 0 adds the warm-up window's
    compaction after that many blocks; ``share`` runs the slices one after another with a
    shared row threshold (one order of events the concurrent slices can take). Returns the
    top-k indices in output order and the per-slice counts.
    """
    v = widen(row)
    pos = (~np.signbit(v)).astype(np.int64)
    n = v.size
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= N")
    if slice_len is None:
        slice_len = -(-n // B) * B
    assert slice_len % B == 0 and slice_len >= B
    keys, ps = None, None
    if presample_waves is not None or share:
        keys = keys_of(row)
    if presample_waves is not None:
        bf16 = row.dtype == np.uint16
        ps = Presample(presample_waves, 8 if bf16 else 4, 16 if bf16 else 32)
    if group != 1 and family != "feistel":
        raise ValueError("grouped orders are Feistel orders")
    stats = []
    kept_all = []
    row_shared = [0]
    for s, lo in enumerate(range(0, n, slice_len)):
        hi = min(lo + slice_len, n)
        m = -(-(hi - lo) // B)
        order = grouped_order(m, group, seed, row_id, s) if group != 1 else block_order(family, m, seed, row_id, s)
        firsts = first_positions(m, group, presample_depth, seed, row_id, s, family)
        kept, st = deepselect_range(v, pos, lo, hi, k, B, B2, order, keys, ps, firsts, warmup,
                                    row_shared if share else None)
        stats.append(st)
        kept_all.append(kept)
    union = np.concatenate(kept_all)
    final = radix_select_topk(v, pos, np.arange(n, dtype=np.int64), union, k)
    return sort_output(v, pos, final), stats


# ----------------------------------------------------------------------------- the bound
def harmonic(m: int) -> float:
    return math.fsum(1.0 / i for i in range(1, m + 1))


def expected_work_bound(n: int, k: int, B: int, B2: int) -> float:
    """(1 + k/B2) * L * H_m with L = k+B+B2 and m = ceil(N/B) (the boxed bound)."""
    m = -(-n // B)
    return (1.0 + k / B2) * (k + B + B2) * harmonic(m)


def asymptotic_work(n: int, k: int, B: int, B2: int) -> float:
    """(1 + k/B2) * (k+B+B2) * ln(N/B), the bound with H_m replaced by its logarithm."""
    return (1.0 + k / B2) * (k + B + B2) * math.log(n / B)


def klogn(n: int, k: int) -> float:
    return k * math.log(n / k)
