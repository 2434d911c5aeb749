"""GPU: seeded random views against the float64 oracle: ce_forward and ce_vjp, and
ce_forward_vjp on the same views; kl_forward, kl_vjp, js_forward and js_vjp; the options
calls with index and probability targets.

Each case draws a dtype, a vocabulary size (log-uniform up to 70,000, so it lands in
every layout: one lane per row, lanes per row, a workgroup per row, the chunked VJP),
and a strided [B, L, V] view cut out of a wider padded buffer: a slice of its rows
([:, :-1] or [:, 1:]) and a column offset, so rows start at any element alignment.
Logits are N(0, s^2) with a random scale s; targets are uniform; g is U[0.25, 2).
Tolerances are the stated ones (tests/gpu_util.py), with the target elements' cancellation
allowance: at scale 20 a short row's target probability can round to 1 in float32.
"""

import numpy as np
import pytest
import torch

from oracle import ce as oce
from softmax_cross_entropy_amd import abi, inputs
from tests.gpu_util import check_grad, check_lse, check_loss, from_dev, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]


def draw(seed):
    g = np.random.default_rng([777, seed])
    dtype = DTYPES[int(g.integers(3))]
    V = int(np.exp(g.uniform(0.0, np.log(70000))))
    B = int(g.integers(1, 5))
    L = int(g.integers(2, 60))
    pad = int(g.integers(0, 10))        # extra columns per stored row
    off = int(g.integers(0, pad + 1))   # the view's first column
    cut = int(g.integers(3))            # 0: all rows, 1: [:, :-1], 2: [:, 1:]
    scale = float(np.exp(g.uniform(np.log(0.1), np.log(20.0))))
    store = inputs.encode(inputs.normal_f32(g, (B, L, V + pad), scale), dtype)
    rows = {0: slice(0, L), 1: slice(0, L - 1), 2: slice(1, L)}[cut]
    view = store[:, rows, off:off + V]
    n = view.shape[0] * view.shape[1]
    y = inputs.uniform_targets(g, (n,), V)
    gr = g.uniform(0.25, 2.0, n).astype(np.float32)
    return dtype, V, store, rows, off, view, y, gr


@pytest.mark.parametrize("seed", range(40))
def test_random_view(seed):
    dtype, V, store, rows, off, view, y, gr = draw(seed)
    dev = to_dev(store, dtype)
    x = dev[:, rows, off:off + V]
    t = torch.from_numpy(y).cuda()
    loss, lse = abi.ce_forward(x, t)
    d = abi.ce_vjp(x, t, lse, torch.from_numpy(gr).cuda())
    torch.cuda.synchronize()
    z = oce.decode(np.ascontiguousarray(view).reshape(-1, V), dtype)
    rl, rm, rls = oce.forward(z, y)
    rd = oce.grad(z, y, gr.astype(np.float64), rm, rls)
    check_loss(loss.cpu().numpy(), rl, dtype)
    check_lse(lse.cpu().numpy(), rm, rls, dtype)
    check_grad(from_dev(d).reshape(-1, V), rd, dtype, targets=y, g=gr)
    # the same in one kernel: its dlogits equal ce_vjp's for the lse it writes
    fl, fs, fd = abi.ce_forward_vjp(x, t, torch.from_numpy(gr).cuda())
    torch.cuda.synchronize()
    check_loss(fl.cpu().numpy(), rl, dtype, "ce_forward_vjp loss")
    check_lse(fs.cpu().numpy(), rm, rls, dtype)
    check_grad(from_dev(fd).reshape(-1, V), rd, dtype, "ce_forward_vjp dlogits", targets=y, g=gr)
    print(f"seed {seed}: {dtype} V={V} view {tuple(x.shape)} strides {tuple(x.stride())}")


# --- the KL and Jensen-Shannon pairs and the options on random views --------------------
#
# Student and teacher views are cut from two differently padded buffers (their row strides
# and first columns differ), the fp32 and fp16 rows carry independent per-row offsets
# (fp32 up to 1e4, fp16 up to 1e2: the offset cancellation cases), and the options draw a
# smoothing from {0, 0.1, 0.5}, an ignore_index on some rows and a reduction.

OFFSETS = {"f32": [0.0, 1e2, 1e4], "f16": [0.0, 1e2], "bf16": [0.0]}


def view_of(g, dtype, B, L, V, rows, scale):
    """(device view [B, len(rows), V], its decoded float64 rows) of a padded random store
    whose rows carry random per-row offsets."""
    pad = int(g.integers(0, 10))
    off = int(g.integers(0, pad + 1))
    x = inputs.normal_f32(g, (B, L, V + pad), scale).astype(np.float64)
    x += g.choice(OFFSETS[dtype], size=(B, L, 1))
    store = inputs.encode(x.astype(np.float32), dtype)
    dev = to_dev(store, dtype)[:, rows, off:off + V]
    z = oce.decode(np.ascontiguousarray(store[:, rows, off:off + V]).reshape(-1, V), dtype)
    return dev, z


def draw_pair(seed):
    g = np.random.default_rng([778, seed])
    dtype = DTYPES[int(g.integers(3))]
    V = int(np.exp(g.uniform(0.0, np.log(40000))))
    B, L = int(g.integers(1, 4)), int(g.integers(2, 40))
    rows = [slice(0, L), slice(0, L - 1), slice(1, L)][int(g.integers(3))]
    scale = float(np.exp(g.uniform(np.log(0.1), np.log(20.0 if dtype != "f16" else 8.0))))
    q, zq = view_of(g, dtype, B, L, V, rows, scale)
    p, zp = view_of(g, dtype, B, L, V, rows, scale)
    gr = g.uniform(0.25, 2.0, zq.shape[0]).astype(np.float32)
    return g, dtype, V, q, p, zq, zp, gr


@pytest.mark.parametrize("seed", range(24))
def test_random_view_kl_js(seed):
    from oracle import js as ojs
    from oracle import kl as okl
    from tests.test_js_gpu import check_dq as js_check_dq, check_val
    from tests.test_kl_gpu import check_dq as kl_check_dq, check_kl
    _, dtype, V, q, p, zq, zp, gr = draw_pair(seed)
    gd = torch.from_numpy(gr).cuda()
    kl, lq, lp = abi.kl_forward(q, p)
    dq = abi.kl_vjp(q, p, lq, lp, gd)
    js, jq, jp, hq = abi.js_forward(q, p)
    dj = abi.js_vjp(q, p, jq, jp, hq, gd)
    torch.cuda.synchronize()
    rk, mq, _, mp, _ = okl.forward(zq, zp)
    check_kl(kl.cpu().numpy(), rk, dtype)
    assert np.array_equal(lq.cpu().numpy()[:, 0], mq) and np.array_equal(lp.cpu().numpy()[:, 0], mp)
    kl_check_dq(from_dev(dq).reshape(-1, V), zq, zp, gr, dtype)
    rj, _, _, _, _, rH = ojs.forward(zq, zp)
    check_val(js.cpu().numpy(), rj, dtype, "js")
    check_val(hq.cpu().numpy(), rH, dtype, "hq")
    js_check_dq(from_dev(dj).reshape(-1, V), zq, zp, gr, dtype)
    print(f"seed {seed}: {dtype} V={V} views {tuple(q.shape)} strides {tuple(q.stride())} / {tuple(p.stride())}")


@pytest.mark.parametrize("seed", range(24))
def test_random_view_options(seed):
    from oracle import ce_options as oco
    from tests.test_ce_options_gpu import check_opt_grad, check_rows, check_total
    g, dtype, V, x, t_view, z, zt_raw, gr = draw_pair(seed)
    n = z.shape[0]
    eps = float(g.choice([0.0, 0.1, 0.5]))
    red = str(g.choice(["none", "sum", "mean"]))
    # index targets, some rows ignored
    y = inputs.uniform_targets(g, (n,), V)
    y[g.random(n) < 0.2] = -100
    gi_up = gr if red == "none" else np.array([1.75], np.float32)
    loss, lse, total, count = abi.ce_forward_ex(x, torch.from_numpy(y).cuda(), eps, -100, red)
    d = abi.ce_vjp_ex(x, torch.from_numpy(y).cuda(), lse, torch.from_numpy(gi_up).cuda(), eps, -100, red,
                      count=count)
    torch.cuda.synchronize()
    rl, rm, rls, rt, rc = oco.forward_index(z, y, eps, -100, red)
    check_rows(loss.cpu().numpy(), rl, dtype, f"index loss eps={eps} red={red}")
    fin = np.isfinite(rm)
    assert np.array_equal(lse.cpu().numpy()[fin, 0], rm[fin])
    w, counted = oco.index_weights(y, V, eps, -100)
    if red != "none":
        assert int(count.item()) == rc
        check_total(float(total.item()), rl, counted, red, dtype, rc)
    gv = gi_up if red == "none" else gi_up[0]
    gi = oco.row_upstream(gv, counted, red, rc)
    check_opt_grad(from_dev(d).reshape(n, V), oco.grad_index(z, y, gv, eps, -100, red), z, w, gi, dtype,
                   f"index dlogits eps={eps} red={red}")
    # probability targets: the second view's softmax-free magnitudes, made non-negative
    pt = np.abs(zt_raw - zt_raw.mean(axis=1, keepdims=True))
    pt = pt / np.maximum(pt.sum(axis=1, keepdims=True), 1e-30)
    ts = inputs.encode(pt.astype(np.float32), dtype).reshape(x.shape)
    td = to_dev(ts, dtype)
    zt = oce.decode(ts.reshape(n, V), dtype)
    gg = gr if red == "none" else np.array([1.25], np.float32)
    loss, lse, wsum, total, count = abi.ce_forward_probs(x, td, eps, red)
    d = abi.ce_vjp_probs(x, td, lse, wsum, torch.from_numpy(gg).cuda(), eps, red, count=count)
    torch.cuda.synchronize()
    rl, rm, rls, rW, rt, rc = oco.forward_probs(z, zt, eps, red)
    check_rows(loss.cpu().numpy(), rl, dtype, f"probs loss eps={eps} red={red}")
    counted = np.ones(n, bool)
    if red != "none":
        assert int(count.item()) == n
        check_total(float(total.item()), rl, counted, red, dtype, n)
    gi = oco.row_upstream(gg if red == "none" else gg[0], counted, red, n)
    check_opt_grad(from_dev(d).reshape(n, V), oco.grad_probs(z, zt, gg if red == "none" else gg[0], eps, red), z,
                   oco.prob_weights(zt, eps), gi, dtype, f"probs dlogits eps={eps} red={red}")
    print(f"seed {seed}: {dtype} V={V} eps={eps} red={red} view {tuple(x.shape)} strides {tuple(x.stride())}")
