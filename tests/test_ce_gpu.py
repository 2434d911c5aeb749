"""GPU parity of ce_forward and ce_vjp against the float64 oracle.

Every test calls the HIP library through its C ABI (softmax_cross_entropy_amd.abi)
and compares with oracle/ on the same seeded inputs, using the tolerance rules in
tests/gpu_util.py.
"""

import math

import numpy as np
import pytest
import torch

from oracle import ce as oce
from softmax_cross_entropy_amd import abi, inputs
from tests import golden_io
from tests.gpu_util import TORCH_DT, check_grad, check_loss, check_lse, decode, from_dev, to_dev

pytestmark = pytest.mark.gpu

LOG2 = math.log(2.0)
LANES = [0, 1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]


def run(b, lanes=0, g=None, view=None):
    """GPU forward + VJP of a CEBatch; returns host arrays (loss, lse, dlogits storage)."""
    x = to_dev(b.logits, b.dtype) if view is None else view
    t = torch.from_numpy(b.targets).cuda()
    gg = torch.from_numpy(b.g if g is None else g).cuda()
    loss, lse = abi.ce_forward(x, t, lanes_per_row=lanes)
    d = abi.ce_vjp(x, t, lse, gg, lanes_per_row=lanes)
    torch.cuda.synchronize()
    return from_dev(loss), from_dev(lse), from_dev(d)


def full_check(b, lanes=0, rows=None):
    loss, lse, d = run(b, lanes)
    z = decode(b.logits if rows is None else b.logits[rows], b.dtype)
    sel = slice(None) if rows is None else rows
    rl, rm, rls = oce.forward(z, b.targets[sel])
    check_loss(loss[sel], rl, b.dtype)
    check_lse(lse[sel], rm, rls, b.dtype)
    check_grad(d[sel], oce.grad(z, b.targets[sel], b.g[sel], rm, rls), b.dtype)
    return loss, lse, d


# --- 1,048,576 rows x 8 classes, fp32 ----------------------------------------

@pytest.mark.parametrize("lanes", [0, -1, 1, 2, 8, 64])
def test_small_vocab_rows(lanes):
    b = inputs.small_v_rows()
    full_check(b, lanes)


# --- numerics stress: offsets, -inf rows, de-offset twins, equal logits -------

@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_numerics_stress(dtype):
    b = inputs.numerics_stress(dtype)
    loss, lse, d = full_check(b)
    # twins: invariance to the shared offset, on the GPU's own outputs
    src, dst = b.twin_pairs[:, 0], b.twin_pairs[:, 1]
    check_loss(loss[dst], loss[src].astype(np.float64), dtype, "twin loss")
    gd = decode(d, dtype)
    check_grad(d[dst], gd[src], dtype, "twin dlogits")
    # padded equal-logit rows [v, v, -inf, ...] give log 2 and (-1/2, 1/2)
    check_loss(loss[b.equal_rows], np.full(len(b.equal_rows), LOG2), dtype, "equal rows")
    expect = np.zeros((len(b.equal_rows), b.V))
    expect[:, 0], expect[:, 1] = -0.5, 0.5
    check_grad(d[b.equal_rows], expect, dtype, "equal rows dlogits")
    assert np.all(loss[b.kind == inputs.KIND_ONLY_TARGET] == 0.0)
    assert np.all(loss[b.kind == inputs.KIND_TARGET_NEGINF] == np.inf)
    rows = np.isin(b.kind, [inputs.KIND_NORMAL, inputs.KIND_TWIN, inputs.KIND_HALF_NEGINF])
    tol = 1e-5 if dtype == "f32" else 4 * 2.0 ** -11
    assert np.max(np.abs(gd[rows].sum(axis=1))) <= tol


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("lanes", [0, 1, 2])
def test_equal_and_gap_pairs(dtype, lanes):
    """Separate V = 2 launches: [v, v] -> log 2 up to 1e36; [2 + c, -1 + c] as stored."""
    eq = inputs.equal_pairs(dtype)
    loss, lse, d = run(eq, lanes)
    check_loss(loss, np.full(eq.rows, LOG2), dtype, "equal pairs")
    check_grad(d, np.tile([-0.5, 0.5], (eq.rows, 1)), dtype, "equal pairs dlogits")
    gp = inputs.gap_pairs(dtype)
    loss, lse, d = full_check(gp, lanes)
    for c, l, z in zip(gp.notes["offsets"], loss, decode(gp.logits, dtype)):
        expect = math.log1p(math.exp(-3.0)) if z[0] - z[1] == 3.0 else LOG2
        assert abs(l - expect) <= 1e-5 * (1 if dtype == "f32" else 10)


# --- non-contiguous view x[:, :-1] of [10, 119, 32768] fp32 -------------------

def test_strided_view_interleaved_calls():
    gold = golden_io.read("strided_view_grad_norm.txt")
    x, y = inputs.strided_view_source(gold["B"], gold["L"], gold["V"])
    yv = inputs.shifted_targets(y)
    X = torch.from_numpy(x).cuda()
    view = X[:, :-1]  # read in place: 10 blocks of 118 rows, batch stride 119 * V
    assert not view.is_contiguous()
    t = torch.from_numpy(yv).cuda()
    g = torch.ones(len(yv), dtype=torch.float32, device="cuda")
    z = decode(np.ascontiguousarray(x[:, :-1]).reshape(-1, gold["V"]), "f32")
    rl, rm, rls = oce.forward(z, yv)
    rd = oce.grad(z, yv, np.ones(len(yv)), rm, rls)
    ref_norm = float(np.sqrt(np.sum(rd * rd)))
    outs = []
    for call in range(3):
        loss, lse = abi.ce_forward(view, t)
        d = abi.ce_vjp(view, t, lse, g)
        loss2, _ = abi.ce_forward(view, t)  # a plain forward between gradient calls
        torch.cuda.synchronize()
        outs.append((from_dev(loss), from_dev(lse), from_dev(d), from_dev(loss2)))
    for loss, lse, d, loss2 in outs:
        check_loss(loss, rl, "f32")
        check_lse(lse, rm, rls, "f32")
        check_grad(d.reshape(-1, gold["V"]), rd, "f32")
        norm = float(np.sqrt(np.sum(d.astype(np.float64) ** 2)))
        assert abs(norm - ref_norm) <= 1e-6 * ref_norm
        assert abs(round(norm, 3) - gold["grad_norm"]) <= 1e-3
        # bitwise identical across calls
        for a, b_ in zip((loss, lse, d, loss2), outs[0]):
            assert np.array_equal(a.view(np.uint32), b_.view(np.uint32))
    # the contiguous copy gives the same bits; the source tensor is untouched
    c = view.contiguous()
    lc, sc = abi.ce_forward(c, t)
    dc = abi.ce_vjp(c, t, sc, g)
    assert np.array_equal(from_dev(lc).view(np.uint32), outs[0][0].view(np.uint32))
    assert np.array_equal(from_dev(dc).view(np.uint32), outs[0][2].view(np.uint32))
    assert np.array_equal(from_dev(X), x)


def test_strided_view_in_place_vjp():
    x, y = inputs.strided_view_source(4, 9, 4096)
    yv = inputs.shifted_targets(y)
    X = torch.from_numpy(x).cuda()
    view = X[:, :-1]
    t = torch.from_numpy(yv).cuda()
    g = torch.linspace(-2, 2, len(yv), dtype=torch.float32, device="cuda")
    loss, lse = abi.ce_forward(view, t)
    expect = abi.ce_vjp(view, t, lse, g)
    out = abi.ce_vjp(view, t, lse, g, dlogits=view)  # overwrite the logits in place
    torch.cuda.synchronize()
    assert out.data_ptr() == view.data_ptr()
    assert np.array_equal(from_dev(view), from_dev(expect))
    # the excluded last position of each sequence is untouched
    assert np.array_equal(from_dev(X[:, -1]), x[:, -1])


# --- large vocabulary, bf16 ---------------------------------------------------

@pytest.mark.parametrize("rows,V", [(2048, 151936), (8192, 32000)])
def test_large_vocab_bf16(rows, V):
    b = inputs.large_vocab(rows, V)
    loss, lse, d = run(b)
    rl, rm, rls = oce.forward_stored(b.logits, "bf16", b.targets, chunk=256)
    check_loss(loss, rl, "bf16")
    check_lse(lse, rm, rls, "bf16")
    # every row of the gradient, in chunks of 256 rows
    for r0 in range(0, rows, 256):
        r1 = min(rows, r0 + 256)
        z = decode(b.logits[r0:r1], "bf16")
        check_grad(d[r0:r1], oce.grad(z, b.targets[r0:r1], b.g[r0:r1], rm[r0:r1], rls[r0:r1]), "bf16",
                   f"dlogits rows {r0}-{r1}")
        gd = decode(d[r0:r1], "bf16")
        assert np.max(np.abs(gd.sum(axis=1))) <= 2.0 ** -8 * 4


def test_vocab_row_repeat_is_bitwise_stable():
    """128 x 151,936 fp32: matches the oracle, then 10 more calls are bit-identical
    ("One barrier short", The fix: the regression test's shape and repeat count)."""
    b = inputs.normal_rows(128, 151936, "f32", workload=7)
    for lanes in (0, 256, 1024):
        loss, lse, d = full_check(b, lanes)
        for _ in range(10):
            l2, s2, d2 = run(b, lanes)
            assert np.array_equal(l2.view(np.uint32), loss.view(np.uint32))
            assert np.array_equal(s2.view(np.uint32), lse.view(np.uint32))
            assert np.array_equal(d2.view(np.uint32), d.view(np.uint32))


# --- 2^27 + 2^20 rows x 8 classes: past 2^32 threads at 32 threads per row -----

def test_huge_row_count():
    gold = golden_io.read("huge_rows.txt")
    n = gold["rows_fail"]
    assert n * gold["threads_per_row"] > 2 ** 32
    b = inputs.huge_rows(n, gold["classes"])
    x = to_dev(b.logits, "f32")
    t = torch.from_numpy(b.targets).cuda()
    loss = torch.full((n,), float("nan"), device="cuda")
    lse = torch.full((n, 2), float("nan"), device="cuda")
    abi.ce_forward(x, t, loss=loss, lse=lse)
    g = torch.ones(n, dtype=torch.float32, device="cuda")
    d = torch.full_like(x, float("nan"))
    abi.ce_vjp(x, t, lse, g, dlogits=d)
    torch.cuda.synchronize()
    # every row written (the buffers started as NaN)
    assert not torch.isnan(loss).any().item()
    assert not torch.isnan(d).any().item()
    assert (loss >= 0).all().item()
    # the oracle on boundary windows and a strided sample, including the first row the
    # wrapped grid dropped
    first = gold["first_wrong_row_when_wrapped"]
    rows = np.unique(np.concatenate([
        np.arange(0, 64), np.arange(first - 64, first + 64), np.arange(2 ** 27 - 64, 2 ** 27 + 64),
        np.arange(n - 64, n), np.arange(0, n, 997)]))
    z = decode(b.logits[rows], "f32")
    rl, rm, rls = oce.forward(z, b.targets[rows])
    idx = torch.from_numpy(rows).cuda()
    check_loss(from_dev(loss[idx]), rl, "f32")
    check_lse(from_dev(lse[idx]), rm, rls, "f32")
    err = check_grad(from_dev(d[idx]), oce.grad(z, b.targets[rows], b.g[rows], rm, rls), "f32")
    assert err <= gold["wrong_threshold"]


# --- boundary sizes, alignment, both layouts ----------------------------------

SIZES = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000,
         1023, 1024, 1025, 4095, 4097]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_boundary_sizes_all_lane_counts(dtype):
    for V in SIZES:
        b = inputs.normal_rows(67, V, dtype, workload=8, stream=V)
        z = decode(b.logits, dtype)
        rl, rm, rls = oce.forward(z, b.targets)
        rd = oce.grad(z, b.targets, b.g, rm, rls)
        for lanes in LANES:
            loss, lse, d = run(b, lanes)
            check_loss(loss, rl, dtype, f"loss V={V} lanes={lanes}")
            check_lse(lse, rm, rls, dtype)
            check_grad(d, rd, dtype, f"dlogits V={V} lanes={lanes}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shift", [1, 3])
def test_misaligned_rows(dtype, shift):
    """Views starting off a 16-byte boundary take the scalar head/tail path."""
    for V in (5, 64, 1000, 4099):
        b = inputs.normal_rows(33, V + shift + 2, dtype, workload=9, stream=V)
        full = to_dev(b.logits, dtype)
        view = full[:, shift:shift + V]
        zs = decode(b.logits[:, shift:shift + V], dtype)
        y = b.targets % V
        t = torch.from_numpy(y).cuda()
        rl, rm, rls = oce.forward(zs, y)
        rd = oce.grad(zs, y, b.g, rm, rls)
        for lanes in (0, 1, 16, 256):
            loss, lse = abi.ce_forward(view, t, lanes_per_row=lanes)
            d = abi.ce_vjp(view, t, lse, torch.from_numpy(b.g).cuda(), lanes_per_row=lanes)
            # an output whose 16-byte phase differs from the input's
            out = torch.empty(33, V + 1, dtype=TORCH_DT[dtype], device="cuda")[:, 1:]
            d2 = abi.ce_vjp(view, t, lse, torch.from_numpy(b.g).cuda(), dlogits=out, lanes_per_row=lanes)
            torch.cuda.synchronize()
            check_loss(from_dev(loss), rl, dtype)
            check_grad(from_dev(d), rd, dtype)
            check_grad(from_dev(d2), rd, dtype)


# --- chunked VJP layout: rows of at least 2048 16-byte vectors ---------------

CHUNK_ELEMS = {"f32": 2048, "f16": 4096, "bf16": 4096}  # 512 vectors of 16 bytes
CHUNK_V = {"f32": [8189, 10243, 16384], "f16": [16377], "bf16": [16377, 20483, 32768]}


def edge_targets(V, dtype):
    """Targets at both row ends and within 8 elements of every chunk edge, so that for
    any 16-byte phase of the row start some target falls in the unaligned head, the
    tail, and the first and last vector of each chunk."""
    c = CHUNK_ELEMS[dtype]
    pos = [0, 1, 2, 3, V - 1, V - 2, V - 3, V - 4]
    pos += [k * c + d for k in range(1, V // c + 1) for d in range(-8, 9)]
    return np.array(sorted({q for q in pos if 0 <= q < V}), np.int32)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_chunked_vjp_edges(dtype):
    """The default VJP layout for long rows against the oracle and, bit for bit, against
    one workgroup per row: contiguous rows, views starting 1 and 3 elements off a
    16-byte boundary, and an output in another 16-byte phase than the input."""
    for V in CHUNK_V[dtype]:
        y = edge_targets(V, dtype)
        n = len(y)
        for shift in (0, 1, 3):
            b = inputs.normal_rows(n, V + shift + 2, dtype, workload=30, stream=V + shift)
            full = to_dev(b.logits, dtype)
            view = full[:, shift:shift + V]
            z = decode(b.logits[:, shift:shift + V], dtype)
            g = np.linspace(-1.5, 2.0, n).astype(np.float32)
            rl, rm, rls = oce.forward(z, y)
            rd = oce.grad(z, y, g, rm, rls)
            t = torch.from_numpy(y).cuda()
            gd = torch.from_numpy(g).cuda()
            loss, lse = abi.ce_forward(view, t)
            d = abi.ce_vjp(view, t, lse, gd)
            rows = abi.ce_vjp(view, t, lse, gd, lanes_per_row=1024)
            out = torch.empty(n, V + 1, dtype=TORCH_DT[dtype], device="cuda")[:, 1:]
            d2 = abi.ce_vjp(view, t, lse, gd, dlogits=out)
            torch.cuda.synchronize()
            check_loss(from_dev(loss), rl, dtype)
            check_grad(from_dev(d), rd, dtype, f"dlogits V={V} shift={shift}")
            check_grad(from_dev(d2), rd, dtype, f"dlogits (other phase) V={V} shift={shift}")
            assert np.array_equal(from_dev(d), from_dev(rows))
            assert np.array_equal(from_dev(d2), from_dev(rows))


def test_chunked_vjp_in_place_strided():
    """In place on a [B, L - 1, V] view with V past the chunking threshold."""
    x, y = inputs.strided_view_source(3, 7, 9001)
    yv = inputs.shifted_targets(y)
    X = torch.from_numpy(x).cuda()
    view = X[:, :-1]
    t = torch.from_numpy(yv).cuda()
    g = torch.linspace(-2, 2, len(yv), dtype=torch.float32, device="cuda")
    loss, lse = abi.ce_forward(view, t)
    expect = abi.ce_vjp(view, t, lse, g, lanes_per_row=1024)
    abi.ce_vjp(view, t, lse, g, dlogits=view)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(view), from_dev(expect))
    assert np.array_equal(from_dev(X[:, -1]), x[:, -1])
    z = decode(np.ascontiguousarray(x[:, :-1]).reshape(-1, 9001), "f32")
    rl, rm, rls = oce.forward(z, yv)
    check_grad(from_dev(view).reshape(-1, 9001), oce.grad(z, yv, from_dev(g), rm, rls), "f32")


def test_degenerate_rows():
    """Out-of-range targets, all -inf, +inf and NaN entries: NaN loss and gradient rows."""
    V = 300
    x = np.random.default_rng(5).standard_normal((8, V)).astype(np.float32)
    y = np.array([0, -1, V, 7, 1, 2, 3, 4], np.int32)
    x[3] = -np.inf
    x[4, 10] = np.inf
    x[5, 11] = np.nan
    x[6, :] = -np.inf
    x[6, 3] = 2.5  # only the target finite: loss 0
    x[7, 4] = -np.inf  # target -inf: loss +inf
    b = inputs.CEBatch(x, y, np.full(8, 1.5, np.float32), "f32")
    for lanes in (0, 1, 64, 256):
        loss, lse, d = run(b, lanes)
        assert np.all(np.isnan(loss[1:6])) and np.all(np.isnan(d[1:6]))
        assert loss[6] == 0.0 and np.all(d[6] == 0.0)
        assert loss[7] == np.inf and d[7, 4] == -1.5 and np.all(np.isfinite(d[7]))
        z = decode(x[[0, 7]], "f32")
        check_grad(d[[0, 7]], oce.grad(z, y[[0, 7]], b.g[[0, 7]]), "f32")


def test_empty_batch():
    x = torch.empty(0, 128, device="cuda")
    t = torch.empty(0, dtype=torch.int32, device="cuda")
    loss, lse = abi.ce_forward(x, t)
    d = abi.ce_vjp(x, t, lse, torch.empty(0, device="cuda"))
    assert loss.numel() == 0 and d.shape == (0, 128)


def test_rejects_output_aliasing_input():
    x = torch.randn(16, 64, device="cuda")
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    loss, lse = abi.ce_forward(x, t)
    with pytest.raises(abi.CEError) as e:
        abi.ce_vjp(x[:, :32], t, lse, torch.ones(16, device="cuda"), dlogits=x[:, 32:])
    assert e.value.status == -7
