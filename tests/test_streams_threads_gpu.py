"""GPU: the calls run on the caller's stream, and concurrent host threads get the same bits.

Every entry point enqueues its work on the stream it is given (torch's current stream in
the binding) and keeps no global mutable state but a per-device CU count (and the
address of the allocation-free call's per-GPU array).  ctypes releases the GIL during a
call, so two Python threads enter the library concurrently here.  Results are
deterministic, so everything is compared bit for bit with the default-stream results.
"""

import threading

import numpy as np
import pytest
import torch

from softmax_cross_entropy_amd import abi, inputs
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def make_case(seed):
    b = inputs.normal_rows(64, 5000, "bf16", workload=70, stream=seed)
    h, w, y = inputs.linear_ce(96, 64, 1000, seed_stream=seed)
    q, p, _ = inputs.kl_pair(32, 3000, "f32", workload=71, stream=seed)
    return {
        "x": to_dev(b.logits, "bf16"), "t": torch.from_numpy(b.targets).cuda(),
        "g": torch.from_numpy(np.linspace(0.5, 1.5, 64).astype(np.float32)).cuda(),
        "H": to_dev(h, "bf16"), "W": to_dev(w, "bf16"), "y": torch.from_numpy(y).cuda(),
        "gl": torch.from_numpy(np.linspace(0.25, 2.0, 96).astype(np.float32)).cuda(),
        "q": to_dev(q, "f32"), "p": to_dev(p, "f32"),
        "gk": torch.from_numpy(np.linspace(1.0, 2.0, 32).astype(np.float32)).cuda(),
    }


def run_all(c):
    loss, lse = abi.ce_forward(c["x"], c["t"])
    d = abi.ce_vjp(c["x"], c["t"], lse, c["g"])
    ll, llse = abi.lce_forward(c["H"], c["W"], c["y"])
    dH, dW = abi.lce_backward(c["H"], c["W"], c["y"], llse, c["gl"])
    kl, lq, lp = abi.kl_forward(c["q"], c["p"])
    dq = abi.kl_vjp(c["q"], c["p"], lq, lp, c["gk"])
    return [loss, lse, d, ll, llse, dH, dW, kl, dq]


def same(a, b):
    return all(torch.equal(u, v) for u, v in zip(a, b))


def test_side_stream_gives_the_default_stream_bits():
    c = make_case(0)
    ref = run_all(c)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = run_all(c)
    s.synchronize()
    assert same(ref, got)


def test_two_host_threads_on_their_own_streams():
    cases = [make_case(1), make_case(2)]
    refs = [run_all(c) for c in cases]
    torch.cuda.synchronize()
    out = [None, None]
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            res = []
            with torch.cuda.stream(s):
                for _ in range(5):
                    res.append(run_all(cases[k]))
            s.synchronize()
            out[k] = res
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for k in range(2):
        assert out[k] is not None
        for res in out[k]:
            assert same(refs[k], res)
