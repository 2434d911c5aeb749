"""GPU: a step of the library's calls captured in a HIP graph replays to the eager bits.

The kernels allocate nothing and issue no memset, so a caller can capture them.  One step
(cross-entropy forward and VJP, lce_forward and lce_backward in both chunk layouts, KL and
Jensen-Shannon forward and VJP, the options with a mean through both the workspace and the
allocation-free forward) is captured through torch.cuda.CUDAGraph after a warm-up, then replayed several
times; before each replay the graph's outputs are cleared and the eager step runs again,
and every replay must match the eager results bit for bit.
"""

import numpy as np
import pytest
import torch

from softmax_cross_entropy_amd import abi, inputs
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def test_captured_step_replays_match_eager():
    b = inputs.normal_rows(128, 5000, "bf16", workload=80)
    x = to_dev(b.logits, "bf16")
    t = torch.from_numpy(b.targets).cuda()
    yi = b.targets.copy()
    yi[::9] = -100
    ti = torch.from_numpy(yi).cuda()
    g = torch.from_numpy(np.linspace(0.5, 1.5, 128).astype(np.float32)).cuda()
    g1 = torch.tensor([1.5], device="cuda")
    h, w, y = inputs.linear_ce(256, 128, 3000, seed_stream=3)
    H, W, Y = to_dev(h, "bf16"), to_dev(w, "bf16"), torch.from_numpy(y).cuda()
    q_np, p_np, _ = inputs.kl_pair(48, 3000, "f32", workload=81)
    q, p = to_dev(q_np, "f32"), to_dev(p_np, "f32")
    gk = torch.from_numpy(np.linspace(1.0, 2.0, 48).astype(np.float32)).cuda()
    gl = torch.from_numpy(np.linspace(0.25, 2.0, 256).astype(np.float32)).cuda()
    # lce_backward in one chunk over a vocabulary wider than the 8192-column chunk
    h2, w2, y2 = inputs.linear_ce(64, 64, 9000, seed_stream=4)
    H2, W2, Y2 = to_dev(h2, "bf16"), to_dev(w2, "bf16"), torch.from_numpy(y2).cuda()
    _, lse2 = abi.lce_forward(H2, W2, Y2)
    g2 = torch.from_numpy(np.linspace(0.5, 1.5, 64).astype(np.float32)).cuda()
    na_loss = torch.empty(128, device="cuda")
    na_lse = torch.empty(128, 2, device="cuda")
    na_tot = torch.empty(1, device="cuda")
    na_cnt = torch.empty(1, dtype=torch.int64, device="cuda")

    def step():
        loss, lse = abi.ce_forward(x, t)
        d = abi.ce_vjp(x, t, lse, g)
        ll, llse = abi.lce_forward(H, W, Y)
        kl, lq, lp = abi.kl_forward(q, p)
        dq = abi.kl_vjp(q, p, lq, lp, gk)
        l2, s2, tot, cnt = abi.ce_forward_ex(x, ti, 0.1, -100, "mean")
        d2 = abi.ce_vjp_ex(x, ti, s2, g1, 0.1, -100, "mean", count=cnt)
        dH, dW = abi.lce_backward(H, W, Y, llse, gl)
        dH2, dW2 = abi.lce_backward(H2, W2, Y2, lse2, g2, one_pass=True)
        js, jq, jp, jh = abi.js_forward(q, p)
        jd = abi.js_vjp(q, p, jq, jp, jh, gk)
        abi.ce_forward_ex_noalloc(x, ti, 0.5, -100, "sum", na_loss, na_lse, na_tot, na_cnt)
        return [loss, lse, d, ll, llse, kl, dq, l2, tot, cnt, d2, dH, dW, dH2, dW2, js, jd, na_loss, na_lse, na_tot,
                na_cnt]

    eager = [o.clone() for o in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    torch.cuda.synchronize()
    for _ in range(4):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b_) for a, b_ in zip(outs, eager))
        again = step()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b_) for a, b_ in zip(again, eager))
