"""Seeded synthetic inputs for the cross-entropy workloads.

This module only draws random numbers and stores them in the dtypes the
library reads: float32, float16, and bfloat16 (kept as uint16 bit patterns in
NumPy, since NumPy has no bfloat16).  It holds none of the loss arithmetic, so
both the HIP path and the float64 oracle can consume what it produces.

Every generator is seeded with ``numpy.random.default_rng([workload, stream])``.
The pages draw standard-normal logits and uniform integer targets from seed 0
("fast.cross_entropy VJP returns wrong gradients for large non-contiguous
inputs on Metal", To Reproduce; "fast.cross_entropy silently skips rows",
Test and reproduction); the workloads below keep those distributions.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"
DTYPES = (F32, F16, BF16)
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}


def rng(workload: int, stream: int = 0) -> np.random.Generator:
    return np.random.default_rng([workload, stream])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bit patterns, rounding to nearest even.

    NaN inputs map to a quiet NaN; infinities and signed zeros are kept.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = ((u[nan] >> 16).astype(np.uint16)) | np.uint16(0x0040)
    return rounded


def encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 draws in ``dtype`` (bf16 as uint16 bits), rounding to nearest even."""
    if dtype == F32:
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def normal_f32(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def uniform_targets(g: np.random.Generator, shape, V: int) -> np.ndarray:
    return g.integers(0, V, size=shape, dtype=np.int32)


@dataclass
class CEBatch:
    """A row batch: ``logits`` is [rows, V] storage (bf16 as uint16 bits)."""

    logits: np.ndarray
    targets: np.ndarray
    g: np.ndarray
    dtype: str
    notes: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.logits.shape[0]

    @property
    def V(self) -> int:
        return self.logits.shape[-1]


def normal_rows(rows: int, V: int, dtype: str, workload: int, stream: int = 0) -> CEBatch:
    """[rows, V] standard-normal logits, uniform targets in [0, V), g = 1."""
    g = rng(workload, stream)
    x = normal_f32(g, (rows, V))
    y = uniform_targets(g, (rows,), V)
    return CEBatch(encode(x, dtype), y, np.ones(rows, np.float32), dtype)


def prob_targets(rows: int, V: int, dtype: str, workload: int, stream: int = 0, normalised_rows: int = None):
    """[rows, V] probability targets stored in ``dtype``: U[0, 1) entries, the first
    ``normalised_rows`` rows (default all) divided by their sums, the rest left
    unnormalised."""
    g = rng(workload, stream)
    t = g.uniform(0.0, 1.0, size=(rows, V))
    k = rows if normalised_rows is None else normalised_rows
    t[:k] /= t[:k].sum(axis=1, keepdims=True)
    return encode(t.astype(np.float32), dtype)


# --- small-V rows: 1,048,576 x 8 fp32 --------------------------------------

def small_v_rows(rows: int = 1 << 20, V: int = 8) -> CEBatch:
    return normal_rows(rows, V, F32, workload=1)


# --- numerics stress: 65,536 x 1024 with offsets, -inf rows, twins ---------

OFFSETS = {F32: (0.0, 1e4, 1e6, 1e8), F16: (0.0, 1e4)}
EQUAL_VALUES = {F32: (1.0, 1e4, 1e6, 1e8, 1e36), F16: (1.0, 1e4)}
GAP_OFFSETS = {F32: (0.0, 1e4, 1e6, 1e8), F16: (0.0, 1e4)}


@dataclass
class StressBatch(CEBatch):
    """Rows tagged by kind; ``twin_of[i] = j`` means row i = row j minus its offset."""

    kind: np.ndarray = None
    offset: np.ndarray = None
    twin_pairs: np.ndarray = None  # [k, 2]: (offset row, de-offset twin row)
    equal_rows: np.ndarray = None  # rows [v, v, -inf, ...] with target 0
    equal_values: tuple = ()


KIND_NORMAL, KIND_HALF_NEGINF, KIND_ONLY_TARGET, KIND_TARGET_NEGINF, KIND_TWIN, KIND_EQUAL = range(6)


def numerics_stress(dtype: str, rows: int = 65536, V: int = 1024, n_twins: int = 256,
                    n_each_neginf: int = 64) -> StressBatch:
    """The numerics-stress batch.

    * Every row is N(0,1) plus one offset per row, drawn from OFFSETS[dtype].
      float16 cannot store 1e6 or 1e8 (its largest finite value is 65504), so
      its offsets come from {0, 1e4}.
    * ``n_twins`` rows hold an offset row minus its offset, computed in
      float64 from the stored values and checked to be exact in ``dtype``.
    * Three groups of ``n_each_neginf`` rows hold -inf entries: half of the
      non-target entries, all non-target entries, or only the target entry.
    * One row per equal-logit value v holds [v, v, -inf, ...] with target 0.
    """
    if dtype not in OFFSETS:
        raise ValueError("numerics stress is defined for f32 and f16")
    np_t = np.float32 if dtype == F32 else np.float16
    g = rng(2, 0 if dtype == F32 else 1)
    x = normal_f32(g, (rows, V)).astype(np.float64)
    y = uniform_targets(g, (rows,), V)
    offs = np.asarray(OFFSETS[dtype], np.float64)
    off = offs[g.integers(0, len(offs), size=rows)]
    kind = np.full(rows, KIND_NORMAL, np.int8)
    store = (x + off[:, None]).astype(np_t)

    # special rows live at fixed, spread-out positions
    perm = g.permutation(rows)
    cur = 0

    def take(n):
        nonlocal cur
        sel = np.sort(perm[cur:cur + n])
        cur += n
        return sel

    ninf = np_t(-np.inf)
    half_rows = take(n_each_neginf)
    for r in half_rows:
        mask = g.random(V) < 0.5
        mask[y[r]] = False
        store[r, mask] = ninf
    kind[half_rows] = KIND_HALF_NEGINF
    only_rows = take(n_each_neginf)
    for r in only_rows:
        t = store[r, y[r]]
        store[r, :] = ninf
        store[r, y[r]] = t
    kind[only_rows] = KIND_ONLY_TARGET
    tneg_rows = take(n_each_neginf)
    store[tneg_rows, y[tneg_rows]] = ninf
    kind[tneg_rows] = KIND_TARGET_NEGINF

    vals = EQUAL_VALUES[dtype]
    eq_rows = take(len(vals))
    for r, v in zip(eq_rows, vals):
        store[r, :] = ninf
        store[r, 0] = np_t(v)
        store[r, 1] = np_t(v)
        y[r] = 0
        off[r] = 0.0
    kind[eq_rows] = KIND_EQUAL

    # de-offset twins of normal rows with a nonzero offset; the twin rows are reserved
    # first so that no row serves as both a source and a twin
    dst = take(n_twins)
    kind[dst] = KIND_TWIN
    cand = np.flatnonzero((kind == KIND_NORMAL) & (off != 0.0))
    src = np.sort(g.choice(cand, size=n_twins, replace=False))
    for s_row, d_row in zip(src, dst):
        tw = store[s_row].astype(np.float64) - off[s_row]
        tw_t = tw.astype(np_t)
        assert np.array_equal(tw_t.astype(np.float64), tw), "twin not exact"
        store[d_row] = tw_t
        y[d_row] = y[s_row]
        off[d_row] = 0.0
    kind[dst] = KIND_TWIN
    b = StressBatch(np.ascontiguousarray(store), y, np.ones(rows, np.float32), dtype)
    b.kind, b.offset = kind, off.astype(np.float32)
    b.twin_pairs = np.stack([src, dst], axis=1)
    b.equal_rows, b.equal_values = eq_rows, vals
    return b


def equal_pairs(dtype: str) -> CEBatch:
    """Rows [v, v] with target 0 for each equal-logit value (V = 2, separate launch)."""
    np_t = np.float32 if dtype == F32 else np.float16
    vals = EQUAL_VALUES[dtype]
    x = np.array([[v, v] for v in vals], np.float64).astype(np_t)
    return CEBatch(x, np.zeros(len(vals), np.int32), np.ones(len(vals), np.float32), dtype,
                   notes={"values": vals})


def gap_pairs(dtype: str) -> CEBatch:
    """Rows [2 + c, -1 + c] with target 0 for each shared offset c (V = 2)."""
    np_t = np.float32 if dtype == F32 else np.float16
    offs = GAP_OFFSETS[dtype]
    x = np.array([[2.0 + c, -1.0 + c] for c in offs], np.float64).astype(np_t)
    return CEBatch(x, np.zeros(len(offs), np.int32), np.ones(len(offs), np.float32), dtype,
                   notes={"offsets": offs})


# --- non-contiguous view: B=10, L=119, V=32768 fp32 -------------------------

def strided_view_source(B: int = 10, L: int = 119, V: int = 32768):
    """Full [B, L, V] float32 logits and [B, L] int32 targets.

    The workload reads the view ``x[:, :-1]`` and the targets ``y[:, 1:]``
    (next-token alignment); ``shifted_targets`` makes the latter contiguous.
    """
    g = rng(3)
    x = normal_f32(g, (B, L, V))
    y = uniform_targets(g, (B, L), V)
    return x, y


def shifted_targets(y: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(y[:, 1:]).reshape(-1)


# --- large vocabulary and huge row counts ----------------------------------

def large_vocab(rows: int, V: int, dtype: str = BF16) -> CEBatch:
    return normal_rows(rows, V, dtype, workload=4, stream=V)


HUGE_ROWS = (1 << 27) + (1 << 20)


def huge_rows(rows: int = HUGE_ROWS, V: int = 8) -> CEBatch:
    """fp32 [rows, 8]; past 2**32 threads when every row gets 32 threads."""
    return normal_rows(rows, V, F32, workload=5)


# --- fused linear cross-entropy ---------------------------------------------

def linear_ce(N: int, D: int, V: int, seed_stream: int = 0, w_scale: float | None = None):
    """H ~ N(0,1) [N, D] and W ~ N(0, 1/D) [V, D], both bf16 bits; targets U[0, V).

    "N(0, 1/D)" is read as variance 1/D (standard deviation D**-0.5), which
    keeps the logits H.W^T near N(0,1) like the other workloads.
    """
    g = rng(6, seed_stream)
    H = f32_to_bf16_bits(normal_f32(g, (N, D)))
    scale = D ** -0.5 if w_scale is None else w_scale
    W = np.empty((V, D), np.uint16)
    step = max(1, (1 << 24) // max(D, 1))
    for v0 in range(0, V, step):
        v1 = min(V, v0 + step)
        W[v0:v1] = f32_to_bf16_bits(normal_f32(g, (v1 - v0, D), scale))
    y = uniform_targets(g, (N,), V)
    return H, W, y


# --- KL divergence: student and teacher logits --------------------------------

def kl_pair(rows: int, V: int, dtype: str, scale: float = 4.0, workload: int = 20, stream: int = 0):
    """(q, p, g): student and teacher logits [rows, V] ~ N(0, 1) * scale, stored in dtype,
    and g = 1.  "One barrier short", Run it yourself, draws both at scale 4 with V = 151,936."""
    gen = rng(workload, stream)
    q = encode(normal_f32(gen, (rows, V), scale), dtype)
    p = encode(normal_f32(gen, (rows, V), scale), dtype)
    return q, p, np.ones(rows, np.float32)


def with_row_offsets(x: np.ndarray, dtype: str, offsets, workload: int, stream: int = 0):
    """Stored logits ``x`` [rows, V] plus one offset per row drawn uniformly from
    ``offsets``, added in float64 to the stored values and stored again in ``dtype``.
    Returns (stored rows, the offset of each row).  "Shift by the max in cross_entropy",
    Proposed changes: results must not depend on a shared offset of a row's logits."""
    gen = rng(workload, stream)
    off = np.asarray(offsets, np.float64)[gen.integers(0, len(offsets), size=x.shape[0])]
    if dtype == BF16:
        base = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        base = x.astype(np.float64)
    return encode((base + off[:, None]).astype(np.float32), dtype), off
