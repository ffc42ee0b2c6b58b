"""Seeded synthetic inputs for row-wise top-k.

This module only draws numbers. It contains none of the selection arithmetic, so the
oracle side and the GPU side can both take their inputs from here without sharing
any of the method's code.

Every generator is deterministic in (seed, rows, N). Each row gets its own stream from
``numpy.random.SeedSequence(seed).spawn(rows)`` so a row's content does not depend on
how many rows are drawn. bf16 data is carried as ``uint16`` bit patterns; fp32 data
as ``float32``.

Workload families (the shapes come from the two places the DeepSelect pages put top-k:
the DSA Lightning Indexer scoring ~1M context tokens in bf16 with k=512, and the
sampler over a ~128K vocabulary in fp32):

* ``c1_small``   4 x 32768 bf16, N(0,1), k=512, block sizes forced to B=B2=1024.
* ``c2_indexer`` 64 x 131072 bf16, N(0,1) plus +3 on 2 % of positions, k=512.
* ``c3_sampler`` 256 x 129280 fp32, 4*N(0,1) plus a Zipf(s=1.1) log-probability bias
  laid over a random vocabulary permutation, k=512.
* ``c4_long``    8 x 1048576 bf16, rows 0-2 N(0,1), row 3 quantised to 256 levels,
  rows 4-7 N(0,1) sorted ascending; k in {512, 4096}.
* ``c5_giant``   1 x 268435456 fp32, uniform on the 2^-24 grid in [0,1), k=32, values only.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional

import numpy as np

BF16 = 0
FP32 = 1
DTYPE_NAMES = {BF16: "bf16", FP32: "fp32"}
ELEM_BYTES = {BF16: 2, FP32: 4}


# ----------------------------------------------------------------------------- bf16 bits
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs never hold NaN here, so the plain carry-propagating form is exact.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly (the bf16 bits are the high half)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _row_rngs(seed: int, rows: int) -> List[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(rows)]


# ----------------------------------------------------------------------------- recipes
def rows_normal_bf16(seed: int, rows: int, n: int) -> np.ndarray:
    out = np.empty((rows, n), np.uint16)
    for r, g in enumerate(_row_rngs(seed, rows)):
        out[r] = bf16_bits_from_f32(g.standard_normal(n, dtype=np.float32))
    return out


def rows_indexer_bf16(seed: int, rows: int, n: int, frac: float = 0.02, boost: float = 3.0) -> np.ndarray:
    """Indexer scores: N(0,1) plus +boost on round(frac*n) positions drawn without replacement."""
    out = np.empty((rows, n), np.uint16)
    cnt = int(round(frac * n))
    for r, g in enumerate(_row_rngs(seed, rows)):
        z = g.standard_normal(n, dtype=np.float32)
        pos = g.choice(n, size=cnt, replace=False)
        z[pos] = z[pos] + np.float32(boost)
        out[r] = bf16_bits_from_f32(z)
    return out


def rows_sampler_f32(seed: int, rows: int, n: int, s: float = 1.1, scale: float = 4.0) -> np.ndarray:
    """Sampler logits: scale*N(0,1) + log of a Zipf(s) law over a per-row random vocabulary order.

    The bias of the token at popularity rank i (0-based) is -s*ln(i+1); the token that gets
    rank i is drawn by a uniform permutation. Computed in float64, rounded once to float32.
    """
    out = np.empty((rows, n), np.float32)
    ranks = np.arange(n, dtype=np.float64)
    bias_by_rank = -s * np.log(ranks + 1.0)
    for r, g in enumerate(_row_rngs(seed, rows)):
        z = g.standard_normal(n)
        perm = g.permutation(n)
        bias = np.empty(n, np.float64)
        bias[perm] = bias_by_rank
        out[r] = (scale * z + bias).astype(np.float32)
    return out


def _quantised_row(g: np.random.Generator, n: int) -> np.ndarray:
    z = g.standard_normal(n, dtype=np.float32).astype(np.float64)
    q = np.clip(np.floor(32.0 * z) + 128.0, 0.0, 255.0)
    return bf16_bits_from_f32(((2.0 * q - 255.0) / 64.0).astype(np.float32))


def rows_long_bf16(seed: int, rows: int, n: int) -> np.ndarray:
    """Long-context mix, by row index modulo 8: 0-2 N(0,1); 3 quantised to 256 levels
    (heavy ties); 4-7 N(0,1) sorted ascending (large values at the end of the row)."""
    out = np.empty((rows, n), np.uint16)
    for r, g in enumerate(_row_rngs(seed, rows)):
        role = r % 8
        if role == 3:
            out[r] = _quantised_row(g, n)
        elif role >= 4:
            out[r] = bf16_bits_from_f32(np.sort(g.standard_normal(n, dtype=np.float32)))
        else:
            out[r] = bf16_bits_from_f32(g.standard_normal(n, dtype=np.float32))
    return out


def rows_grid_f32(seed: int, rows: int, n: int, bits: int = 24) -> np.ndarray:
    """Uniform [0,1) on the 2^-bits grid: integers in [0, 2^bits) times 2^-bits (exact)."""
    out = np.empty((rows, n), np.float32)
    for r, g in enumerate(_row_rngs(seed, rows)):
        u = g.integers(0, 1 << bits, size=n, dtype=np.uint32)
        out[r] = u.astype(np.float32) * np.float32(2.0 ** -bits)
    return out


# ----------------------------------------------------------------------------- edge families
SPECIAL_F32 = np.array([-np.inf, -2.0, -1.0, -0.0, 0.0, 1.0, 2.0, np.inf], np.float32)


def rows_family(family: str, dtype: int, seed: int, rows: int, n: int) -> np.ndarray:
    """Edge-case families used by the fuzz and edge tests.

    normal, ascending, descending, constant, ties (8 levels), specials (+-0, +-inf, small
    alphabet), tiny (bf16 subnormals and values near zero), neg (all negative).
    """
    rs = _row_rngs(seed, rows)
    f = np.empty((rows, n), np.float32)
    for r, g in enumerate(rs):
        if family == "normal":
            v = g.standard_normal(n, dtype=np.float32)
        elif family == "ascending":
            v = np.sort(g.standard_normal(n, dtype=np.float32))
        elif family == "descending":
            v = np.sort(g.standard_normal(n, dtype=np.float32))[::-1]
        elif family == "constant":
            v = np.full(n, np.float32(g.integers(-3, 4)), np.float32)
        elif family == "ties":
            v = g.integers(-4, 4, size=n).astype(np.float32) * np.float32(0.5)
        elif family == "specials":
            v = SPECIAL_F32[g.integers(0, len(SPECIAL_F32), size=n)]
        elif family == "tiny":
            # bit patterns with a zero exponent field: subnormals of both signs and +-0
            mant = g.integers(0, 1 << 7, size=n).astype(np.uint32) << np.uint32(16)
            sign = g.integers(0, 2, size=n).astype(np.uint32) << np.uint32(31)
            v = (mant | sign).view(np.float32)
        elif family == "neg":
            v = -np.abs(g.standard_normal(n, dtype=np.float32)) - np.float32(0.25)
        else:
            raise ValueError(f"unknown family {family!r}")
        f[r] = v
    return bf16_bits_from_f32(f) if dtype == BF16 else f


# ----------------------------------------------------------------------------- named workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    n: int
    dtype: int
    ks: tuple
    seed: int
    values_only: bool
    forced_B: Optional[int]
    forced_B2: Optional[int]
    recipe: Callable[[int, int, int], np.ndarray]
    description: str

    def make(self, rows: Optional[int] = None, n: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
        return self.recipe(self.seed if seed is None else seed, self.rows if rows is None else rows,
                           self.n if n is None else n)

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    def input_bytes(self, rows: Optional[int] = None, n: Optional[int] = None) -> int:
        return (self.rows if rows is None else rows) * (self.n if n is None else n) * self.elem_bytes


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("c1_small", 4, 32768, BF16, (512,), 101, False, 1024, 1024, rows_normal_bf16,
                 "4 rows x 32768 bf16 N(0,1), k=512, B=B2=1024"),
        Workload("c2_indexer", 64, 131072, BF16, (512,), 102, False, None, None, rows_indexer_bf16,
                 "DSA indexer: 64 query rows x 131072 context scores bf16, N(0,1) with 2% boosted by +3, k=512"),
        Workload("c3_sampler", 256, 129280, FP32, (512,), 103, False, None, None, rows_sampler_f32,
                 "sampler: 256 rows x 129280 vocab fp32, 4*N(0,1) + Zipf(1.1) log-bias, k=512"),
        Workload("c4_long", 8, 1048576, BF16, (512, 4096), 104, False, None, None, rows_long_bf16,
                 "long context: 8 rows x 1048576 bf16, iid / 256-level quantised / ascending rows, k in {512,4096}"),
        Workload("c5_giant", 1, 268435456, FP32, (32,), 105, True, None, None, rows_grid_f32,
                 "1-D giant row: 268435456 fp32 uniform on the 2^-24 grid, k=32, values only"),
    ]
}
