"""The C ABI without a GPU: the library loads, exports what the header declares, and
rejects invalid arguments on the host with the documented status before any launch.

Pointers below are fake addresses that are never dereferenced: every call here fails
validation first, or, with valid arguments, the device lookup (no GPU is visible where
this module runs).
"""

import ctypes
import os
import re

import pytest
import torch

from softmax_cross_entropy_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ce_mi355x.h")
TESTING_HEADER = os.path.join(ROOT, "include", "ce_mi355x_testing.h")

OK, NULL, SHAPE, DTYPE, LAYOUT, WORKSPACE, LAUNCH, ALIAS, DEVICE, OPTION = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9

# The pointers are fake device addresses, so a call that passes validation must not reach a
# GPU: the module runs only where none is visible, and such calls stop at the device lookup
# with CE_ERR_DEVICE.
pytestmark = [pytest.mark.skipif(not os.path.exists(abi.LIB_PATH), reason="library not built"),
              pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake device addresses: host only")]


def declared_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text)))


def test_exports_every_declared_symbol():
    names = declared_functions(HEADER)
    testing = declared_functions(TESTING_HEADER)
    assert set(names) == set(abi.EXPORTS)
    assert set(testing) == set(abi.TESTING_EXPORTS)
    assert not set(names) & set(testing)
    L = ctypes.CDLL(abi.LIB_PATH)
    for n in names + testing:
        assert hasattr(L, n), n


def test_product_header_declares_no_tuning_knob():
    """The product header's calls pick their own row-to-lane mapping; the calls that take
    one from the caller live in the testing header only."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    assert "lanes_per_row" not in text
    assert all(n.endswith("_lanes") for n in declared_functions(TESTING_HEADER))


def test_status_strings():
    for code, name in abi.STATUS.items():
        assert abi.status_string(code).startswith(name)
    assert "unknown" in abi.status_string(-99)


A = 1 << 20  # fake, 256-byte aligned device addresses, far apart
P_LOGITS, P_T, P_LOSS, P_LSE, P_G, P_OUT, P_W, P_WS = (ctypes.c_void_p(A * k) for k in range(1, 9))


def lay(rows, rs, bs=None):
    return abi.CELayout(rows, rs, rs * rows if bs is None else bs)


def fwd(logits=P_LOGITS, layout=None, dt=0, t=P_T, n=16, V=8, loss=P_LOSS, lse=P_LSE, lanes=0):
    layout = layout or lay(n, V)
    return abi.lib().ce_forward_lanes(logits, layout, dt, t, n, V, loss, lse, lanes, None)


def vjp(logits=P_LOGITS, layout=None, dt=0, t=P_T, lse=P_LSE, g=P_G, n=16, V=8, out=P_OUT, olayout=None, lanes=0):
    layout = layout or lay(n, V)
    olayout = olayout or lay(n, V)
    return abi.lib().ce_vjp_lanes(logits, layout, dt, t, lse, g, n, V, out, olayout, lanes, None)


def test_forward_rejects_bad_arguments():
    assert fwd(logits=None) == NULL
    assert fwd(t=None) == NULL
    assert fwd(loss=None) == NULL
    assert fwd(lse=None) == NULL
    assert fwd(V=0) == SHAPE
    assert fwd(V=-3) == SHAPE
    assert fwd(V=1 << 31) == SHAPE
    assert fwd(n=-1) == SHAPE
    assert fwd(dt=3) == DTYPE
    assert fwd(dt=-1) == DTYPE
    assert fwd(lanes=3) == SHAPE
    assert fwd(lanes=2048) == SHAPE
    assert fwd(lanes=-2) == SHAPE
    assert fwd(layout=abi.CELayout(0, 8, 0)) == LAYOUT
    assert fwd(layout=abi.CELayout(16, -8, 0)) == LAYOUT
    assert fwd(logits=ctypes.c_void_p(A + 2)) == LAYOUT  # fp32 logits not 4-byte aligned
    assert fwd(lse=ctypes.c_void_p(5 * A + 4)) == LAYOUT  # lse pairs need 8 bytes
    assert fwd(loss=ctypes.c_void_p(3 * A + 2)) == LAYOUT


def test_forward_rejects_aliasing_outputs():
    assert fwd(loss=ctypes.c_void_p(A + 64)) == ALIAS  # loss inside the logits
    assert fwd(lse=ctypes.c_void_p(2 * A)) == ALIAS  # lse on the targets
    assert fwd(lse=ctypes.c_void_p(3 * A + 32)) == ALIAS  # lse over loss


def test_zero_rows_is_a_noop():
    assert fwd(n=0, logits=None, t=None, loss=None, lse=None) == OK
    assert vjp(n=0, logits=None, t=None, lse=None, g=None, out=None) == OK
    assert abi.lib().lce_forward(None, None, None, 0, 64, 100, None, None, None, 0, None) == OK


def test_vjp_rejects_bad_arguments():
    assert vjp(out=None) == NULL
    assert vjp(g=None) == NULL
    assert vjp(lse=None) == NULL
    assert vjp(V=0) == SHAPE
    assert vjp(dt=7) == DTYPE
    assert vjp(olayout=abi.CELayout(16, 4, 64)) == LAYOUT  # output rows overlap
    assert vjp(olayout=abi.CELayout(4, 8, 16)) == LAYOUT  # output batches overlap
    assert vjp(out=ctypes.c_void_p(6 * A + 2)) == LAYOUT


def test_vjp_aliasing():
    # the output may be the input only with an identical layout
    assert vjp(out=ctypes.c_void_p(A + 64)) == ALIAS
    assert vjp(out=P_LOGITS, olayout=lay(16, 16, 256), layout=lay(16, 8, 128)) == ALIAS
    assert vjp(out=ctypes.c_void_p(5 * A)) == ALIAS  # output over g
    assert vjp(out=ctypes.c_void_p(4 * A - 16)) == ALIAS  # output runs into lse


def fvj(logits=P_LOGITS, layout=None, dt=0, t=P_T, g=P_G, n=16, V=8, loss=P_LOSS, lse=P_LSE, out=P_OUT,
        olayout=None, lanes=0):
    layout = layout or lay(n, V)
    olayout = olayout or lay(n, V)
    return abi.lib().ce_forward_vjp_lanes(logits, layout, dt, t, g, n, V, loss, lse, out, olayout, lanes, None)


def test_forward_vjp_rejects_bad_arguments():
    for k in ("logits", "t", "g", "loss", "lse", "out"):
        assert fvj(**{k: None}) == NULL, k
    assert fvj(V=0) == SHAPE
    assert fvj(V=1 << 31) == SHAPE
    assert fvj(n=-1) == SHAPE
    assert fvj(lanes=3) == SHAPE
    assert fvj(dt=3) == DTYPE
    assert fvj(olayout=abi.CELayout(16, 4, 64)) == LAYOUT  # output rows overlap
    assert fvj(g=ctypes.c_void_p(5 * A + 2)) == LAYOUT
    assert fvj(lse=ctypes.c_void_p(4 * A + 4)) == LAYOUT
    assert fvj(n=0, logits=None, t=None, g=None, loss=None, lse=None, out=None) == OK


def test_forward_vjp_aliasing():
    assert fvj(out=ctypes.c_void_p(A + 64)) == ALIAS  # dlogits overlap the logits
    assert fvj(out=P_LOGITS, olayout=lay(16, 16, 256), layout=lay(16, 8, 128)) == ALIAS
    assert fvj(loss=ctypes.c_void_p(A + 64)) == ALIAS  # loss inside the logits
    assert fvj(lse=ctypes.c_void_p(5 * A)) == ALIAS  # lse over g
    assert fvj(out=ctypes.c_void_p(2 * A - 16)) == ALIAS  # dlogits run into the targets
    assert fvj(loss=ctypes.c_void_p(6 * A + 64)) == ALIAS  # loss inside dlogits
    assert fvj(lse=ctypes.c_void_p(3 * A + 32)) == ALIAS  # lse over loss


def lce(H=P_LOGITS, W=P_W, t=P_T, N=32, D=64, V=1000, loss=P_LOSS, lse=P_LSE, ws=P_WS, wsb=None):
    if wsb is None:
        wsb = abi.lce_workspace_size(N, D, V)
    return abi.lib().lce_forward(H, W, t, N, D, V, loss, lse, ws, wsb, None)


def test_lce_rejects_bad_arguments():
    assert abi.lce_workspace_size(32, 64, 1000) > 0
    assert abi.lce_workspace_size(32, 60, 1000) == 0
    assert lce(D=60) == SHAPE
    assert lce(D=0) == SHAPE
    assert lce(V=0) == SHAPE
    assert lce(N=-1) == SHAPE
    assert lce(H=None) == NULL
    assert lce(W=None) == NULL
    assert lce(ws=None) == WORKSPACE
    assert lce(wsb=abi.lce_workspace_size(32, 64, 1000) - 1) == WORKSPACE
    assert lce(H=ctypes.c_void_p(A + 8)) == LAYOUT
    assert lce(ws=ctypes.c_void_p(8 * A + 64)) == LAYOUT
    assert lce(loss=ctypes.c_void_p(2 * A - 64)) == ALIAS  # loss inside W's range? no: inside H..W
    assert lce(ws=ctypes.c_void_p(7 * A + 256)) == ALIAS  # workspace inside W


def test_lce_tile_grid_bound():
    """One workgroup of 256 work-items per 256 x 256 tile, in super-blocks of 4 x 8 tiles
    (N of 1024 rows by 2048 columns) and whole rounds of 8 super-blocks: a dispatch holds
    under 2^32 work-items, so a call takes at most 65535 rounds (524,280 super-blocks).  N = 8192 (8 super-block
    rows) by V = 2048 x 65535 is the largest such shape; one more row is rejected."""
    V = 2048 * 65535
    assert abi.lce_workspace_size(8192, 8, V) > 0
    assert abi.lce_workspace_size(8193, 8, V) == 0
    assert abi.lce_workspace_size(8193, 8, 2048 * 58253) > 0   # 9 x 58253 = 524277 super-blocks
    assert abi.lce_workspace_size(8193, 8, 2048 * 58254) == 0
    assert lce(N=8193, D=8, V=V, wsb=1 << 50) == SHAPE
    # the backward's two products share one launch: N x D and 8192 x D.  At N = 2^22
    # (4096 super-block rows) and D = 2048 k they take 512 k + k rounds: k <= 127.
    assert abi.lce_backward_workspace_size(1 << 22, 2048 * 127, 1000) > 0
    assert abi.lce_backward_workspace_size(1 << 22, 2048 * 128, 1000) == 0
    assert abi.lce_backward_workspace_size_one_pass(1 << 22, 2048 * 128, 1000) == 0
    assert lbw(N=1 << 22, D=2048 * 128, wsb=1 << 50) == SHAPE
    # one chunk over N = 2^22 rows by V = 2^22 columns would need 4096 x 2048 super-blocks:
    # that call keeps chunks of 8192 columns
    n, v = 1 << 22, 1 << 22
    assert abi.lce_backward_workspace_size_one_pass(n, 8, v) == abi.lce_backward_workspace_size(n, 8, v) > 0
    assert abi.lce_backward_workspace_size_one_pass(1 << 12, 8, v) > abi.lce_backward_workspace_size(1 << 12, 8, v)


P_DH, P_DW = ctypes.c_void_p(A * 200), ctypes.c_void_p(A * 210)  # clear of the workspace


def lbw(H=P_LOGITS, W=P_W, t=P_T, lse=P_LSE, g=P_G, N=32, D=64, V=1000, dH=P_DH, dW=P_DW, ws=P_WS, wsb=None):
    if wsb is None:
        wsb = abi.lce_backward_workspace_size(N, D, V)
    return abi.lib().lce_backward(H, W, t, lse, g, N, D, V, dH, dW, ws, wsb, None)


def test_lce_backward_rejects_bad_arguments():
    need = abi.lce_backward_workspace_size(32, 64, 1000)
    # a chunk of V rounded up to 256 columns (1024) when V is below the chunk width:
    # dZ chunk [32][1024] and its transpose [1024][32]; H^T [64][32]; W chunk^T [64][1024]
    assert need == 2 * 32 * 1024 * 2 + 64 * 32 * 2 + 64 * 1024 * 2
    # N = 33: the transposed buffers' rows are padded to 40 tokens, each buffer to 256 bytes
    a256 = lambda x: (x + 255) // 256 * 256
    assert abi.lce_backward_workspace_size(33, 64, 1000) == (a256(33 * 1024 * 2) + a256(1024 * 40 * 2) +
                                                             a256(64 * 40 * 2) + a256(64 * 1024 * 2))
    assert abi.lce_backward_workspace_size(32, 60, 1000) == 0
    assert abi.lce_backward_workspace_size((1 << 22) + 1, 64, 1000) == 0
    assert abi.lce_backward_workspace_size(1 << 22, 64, 1000) > 0
    assert lbw(D=60) == SHAPE
    assert lbw(D=0) == SHAPE
    assert lbw(V=0) == SHAPE
    assert lbw(N=-1) == SHAPE
    assert lbw(N=1 << 31, wsb=1 << 40) == SHAPE
    assert lbw(N=(1 << 22) + 1, wsb=1 << 40) == SHAPE
    assert lbw(D=(1 << 22) + 8) == SHAPE
    for name in ("H", "W", "t", "lse", "g", "dH", "dW"):
        assert lbw(**{name: None}) == NULL, name
    assert lbw(ws=None) == WORKSPACE
    assert lbw(wsb=need - 1) == WORKSPACE
    assert lbw(H=ctypes.c_void_p(A + 8)) == LAYOUT
    assert lbw(dH=ctypes.c_void_p(200 * A + 4)) == LAYOUT   # dH and dW take 16-byte stores
    assert lbw(dW=ctypes.c_void_p(210 * A + 8)) == LAYOUT
    assert lbw(lse=ctypes.c_void_p(4 * A + 4)) == LAYOUT
    assert lbw(ws=ctypes.c_void_p(8 * A + 64)) == LAYOUT
    assert lbw(dW=ctypes.c_void_p(7 * A + 1024)) == ALIAS   # dW inside W
    assert lbw(dH=ctypes.c_void_p(8 * A + 4096)) == ALIAS   # dH inside the workspace
    assert lbw(dH=ctypes.c_void_p(210 * A + 4096)) == ALIAS  # dH inside dW
    assert lbw(dW=ctypes.c_void_p(5 * A)) == ALIAS          # dW over g


def test_lce_backward_one_pass_workspace():
    """The workspace of one chunk over the whole vocabulary, and the call's overlap check
    against the part of the workspace it uses."""
    a256 = lambda x: (x + 255) // 256 * 256
    size = lambda C, N=32, D=8, n8=32: a256(N * C * 2) + a256(C * n8 * 2) + a256(D * n8 * 2) + a256(D * C * 2)
    N, D, V = 32, 8, 9000
    chunked, one = abi.lce_backward_workspace_size(N, D, V), abi.lce_backward_workspace_size_one_pass(N, D, V)
    assert chunked == size(8192) and one == size(9216)   # 9000 columns rounded up to 256
    assert abi.lce_backward_workspace_size_one_pass(33, 64, 20000) == (a256(33 * 20224 * 2) + a256(20224 * 40 * 2) +
                                                                       a256(64 * 40 * 2) + a256(64 * 20224 * 2))
    # a vocabulary of one chunk already, or above 2^22 columns: the chunked size
    assert abi.lce_backward_workspace_size_one_pass(32, 64, 1000) == abi.lce_backward_workspace_size(32, 64, 1000)
    big = (1 << 22) + 1
    assert abi.lce_backward_workspace_size_one_pass(32, 64, big) == abi.lce_backward_workspace_size(32, 64, big)
    assert abi.lce_backward_workspace_size_one_pass(32, 64, 1 << 22) > abi.lce_backward_workspace_size(32, 64, 1 << 22)
    assert abi.lce_backward_workspace_size_one_pass(32, 60, 1000) == 0
    assert abi.lce_backward_workspace_size_one_pass((1 << 22) + 1, 64, 1000) == 0
    # dH just past the chunked layout but inside the one-chunk layout: an overlap only when
    # the workspace is large enough for one chunk
    dH = ctypes.c_void_p(8 * A + chunked + 256)
    assert lbw(N=N, D=D, V=V, dH=dH, wsb=chunked) == DEVICE
    assert lbw(N=N, D=D, V=V, dH=dH, wsb=one) == ALIAS
    assert lbw(N=N, D=D, V=V, dH=dH, wsb=one - 1) == DEVICE


def test_lce_backward_empty_batch_needs_only_w_and_dw():
    """N == 0 still writes dW (= 0); H, targets, lse, g, dH and the workspace may be NULL."""
    st = lbw(H=None, t=None, lse=None, g=None, dH=None, ws=None, N=0, wsb=0)
    assert st == DEVICE
    assert lbw(N=0, dW=None) == NULL


P_P, P_KL, P_LQ, P_LP, P_DQ = (ctypes.c_void_p(A * k) for k in (300, 310, 320, 330, 340))


def klf(q=P_LOGITS, ql=None, p=P_P, pl=None, dt=0, n=16, V=8, kl=P_KL, lq=P_LQ, lp=P_LP, lanes=0):
    return abi.lib().kl_forward_lanes(q, ql or lay(n, V), p, pl or lay(n, V), dt, n, V, kl, lq, lp, lanes, None)


def klv(q=P_LOGITS, ql=None, p=P_P, pl=None, dt=0, lq=P_LQ, lp=P_LP, g=P_G, n=16, V=8, dq=P_DQ, dl=None, lanes=0):
    return abi.lib().kl_vjp_lanes(q, ql or lay(n, V), p, pl or lay(n, V), dt, lq, lp, g, n, V, dq, dl or lay(n, V),
                                  lanes, None)


def test_kl_rejects_bad_arguments():
    assert klf(dt=3) == DTYPE and klv(dt=-1) == DTYPE
    assert klf(V=0) == SHAPE and klf(n=-1) == SHAPE
    assert klf(lanes=-1) == SHAPE and klv(lanes=3) == SHAPE and klf(lanes=2048) == SHAPE
    assert klf(n=0, q=None) == OK and klv(n=0, dq=None) == OK
    for name in ("q", "p", "kl", "lq", "lp"):
        assert klf(**{name: None}) == NULL, name
    for name in ("q", "p", "lq", "lp", "g", "dq"):
        assert klv(**{name: None}) == NULL, name
    assert klf(p=ctypes.c_void_p(300 * A + 2)) == LAYOUT  # fp32 p not 4-byte aligned
    assert klf(lq=ctypes.c_void_p(320 * A + 4)) == LAYOUT
    assert klv(dl=abi.CELayout(16, 4, 64)) == LAYOUT  # output rows overlap
    assert klf(kl=ctypes.c_void_p(300 * A + 16)) == ALIAS  # kl inside p
    assert klf(lp=ctypes.c_void_p(310 * A)) == ALIAS  # lse_p over kl
    assert klv(dq=ctypes.c_void_p(300 * A)) == ALIAS  # dq over p
    assert klv(dq=ctypes.c_void_p(A + 64)) == ALIAS  # dq overlapping q, not in place
    assert klv(dq=ctypes.c_void_p(5 * A)) == ALIAS  # dq over g
    assert klv(dq=P_LOGITS) == DEVICE  # in place, identical layout


P_HQ = ctypes.c_void_p(A * 350)


def jsf(q=P_LOGITS, dt=0, p=P_P, n=16, V=8, js=P_KL, lq=P_LQ, lp=P_LP, hq=P_HQ, lanes=0):
    return abi.lib().js_forward_lanes(q, lay(n, V), p, lay(n, V), dt, n, V, js, lq, lp, hq, lanes, None)


def jsv(q=P_LOGITS, dt=0, p=P_P, lq=P_LQ, lp=P_LP, hq=P_HQ, g=P_G, n=16, V=8, dq=P_DQ, lanes=0):
    return abi.lib().js_vjp_lanes(q, lay(n, V), p, lay(n, V), dt, lq, lp, hq, g, n, V, dq, lay(n, V), lanes, None)


def test_js_rejects_bad_arguments():
    assert jsf(dt=3) == DTYPE and jsv(dt=-1) == DTYPE
    assert jsf(V=0) == SHAPE and jsv(n=-1) == SHAPE and jsf(lanes=3) == SHAPE
    assert jsf(n=0, q=None) == OK and jsv(n=0, dq=None) == OK
    for name in ("q", "p", "js", "lq", "lp", "hq"):
        assert jsf(**{name: None}) == NULL, name
    for name in ("q", "p", "lq", "lp", "hq", "g", "dq"):
        assert jsv(**{name: None}) == NULL, name
    assert jsf(hq=ctypes.c_void_p(350 * A + 2)) == LAYOUT
    assert jsf(hq=P_KL) == ALIAS and jsf(hq=P_P) == ALIAS
    assert jsv(dq=P_HQ) == ALIAS and jsv(dq=P_P) == ALIAS
    assert jsv(dq=P_LOGITS) == DEVICE


P_TOT, P_CNT, P_RWS, P_PR, P_WSUM, P_GR = (ctypes.c_void_p(A * k) for k in (400, 401, 402, 410, 420, 421))
WSB = 1 << 14


def opts(eps=0.1, ign=None, red="mean"):
    return abi.options(eps, ign, red)


def fex(logits=P_LOGITS, dt=0, t=P_T, n=16, V=8, o=None, loss=P_LOSS, lse=P_LSE, tot=P_TOT, cnt=P_CNT, ws=P_RWS,
        wsb=WSB):
    return abi.lib().ce_forward_ex(logits, lay(n, V), dt, t, n, V, o or opts(), loss, lse, tot, cnt, ws, wsb, None)


def vex(logits=P_LOGITS, dt=0, t=P_T, lse=P_LSE, g=P_GR, n=16, V=8, o=None, cnt=P_CNT, d=P_OUT, dl=None):
    return abi.lib().ce_vjp_ex(logits, lay(n, V), dt, t, lse, g, n, V, o or opts(), cnt, d, dl or lay(n, V), None)


def fpr(logits=P_LOGITS, dt=0, pr=P_PR, n=16, V=8, o=None, loss=P_LOSS, lse=P_LSE, ws_=P_WSUM, tot=P_TOT,
        cnt=P_CNT, ws=P_RWS, wsb=WSB):
    return abi.lib().ce_forward_probs(logits, lay(n, V), dt, pr, lay(n, V), n, V, o or opts(), loss, lse, ws_, tot,
                                      cnt, ws, wsb, None)


def vpr(logits=P_LOGITS, dt=0, pr=P_PR, lse=P_LSE, ws_=P_WSUM, g=P_GR, n=16, V=8, o=None, cnt=P_CNT, d=P_OUT):
    return abi.lib().ce_vjp_probs(logits, lay(n, V), dt, pr, lay(n, V), lse, ws_, g, n, V, o or opts(), cnt, d,
                                  lay(n, V), None)


def test_reduce_workspace_size():
    assert abi.ce_reduce_workspace_size() == WSB


def test_options_reject_bad_arguments():
    for f in (fex, vex, fpr, vpr):
        assert f(o=opts(eps=-0.01)) == OPTION and f(o=opts(eps=1.5)) == OPTION
        assert f(o=opts(eps=float("nan"))) == OPTION and f(o=abi.options(0.1, None, 3)) == OPTION
        assert f(dt=5) == DTYPE and f(V=0) == SHAPE and f(n=-1) == SHAPE
    # ignore_index has no meaning for probability targets
    assert fpr(o=opts(ign=-100)) == OPTION and vpr(o=opts(ign=-100)) == OPTION
    # a reduction needs its outputs and the workspace
    assert fex(tot=None) == NULL and fex(cnt=None) == NULL and fex(ws=None) == NULL
    assert fex(wsb=WSB - 1) == WORKSPACE
    assert fex(cnt=ctypes.c_void_p(400 * A + 4)) == LAYOUT
    assert fex(o=opts(red="none"), tot=None, cnt=None, ws=None, wsb=0) == DEVICE
    for name in ("logits", "t", "loss", "lse"):
        assert fex(**{name: None}) == NULL, name
    assert fpr(pr=None) == NULL and fpr(ws_=None) == NULL
    assert vex(cnt=None) == NULL and vex(o=opts(red="sum"), cnt=None) == DEVICE
    assert vpr(ws_=None) == NULL and vpr(pr=None) == NULL
    # aliasing among the outputs and with the inputs
    assert fex(tot=P_LOSS) == ALIAS and fex(ws=ctypes.c_void_p(A + 8)) == ALIAS and fex(cnt=P_RWS) == ALIAS
    assert fpr(ws_=P_PR) == ALIAS and fpr(loss=P_WSUM) == ALIAS
    assert vex(d=P_GR) == ALIAS and vex(d=P_CNT) == ALIAS and vpr(d=P_PR) == ALIAS and vpr(d=P_WSUM) == ALIAS
    assert vex(d=P_LOGITS) == DEVICE  # in place
    # an empty batch with a reduction still writes total and count; without one it is a no-op
    assert fex(n=0, logits=None, t=None, loss=None, lse=None) == DEVICE
    assert fex(n=0, tot=P_RWS) == ALIAS
    assert fex(n=0, logits=None, o=opts(red="none"), tot=None, cnt=None, ws=None) == OK
    assert vex(n=0, logits=None, d=None) == OK and vpr(n=0, pr=None, d=None) == OK


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES", None) is not None or os.path.exists("/dev/kfd"),
                    reason="only meaningful without a GPU")
def test_valid_call_without_device_reports_device_error():
    assert fwd() == DEVICE
    assert vjp() == DEVICE
    assert fvj() == DEVICE
    assert fvj(out=P_LOGITS) == DEVICE  # in place with the same layout is allowed
    assert lce() == DEVICE
    assert lbw() == DEVICE
    assert lbw(H=None, t=None, lse=None, g=None, dH=None, ws=None, N=0, wsb=0) == DEVICE
    assert klf() == DEVICE
    assert klv() == DEVICE
    assert fex() == DEVICE and vex() == DEVICE and fpr() == DEVICE and vpr() == DEVICE
    assert jsf() == DEVICE and jsv() == DEVICE
    assert fex(n=0, logits=None, t=None, loss=None, lse=None) == DEVICE
