"""The C ABI's host checks under random views (no GPU needed).

ce_vjp writes dlogits through a caller-given strided view.  The host check may reject a
view that would in fact be fine (it is conservative), but it must never accept an output
view whose rows share an element, and it must never accept a dlogits view that overlaps
an input.  A plain Python model enumerates the element offsets of small views and decides
both questions exactly; the library's answer (LAYOUT or ALIAS, against any other status)
must agree with it wherever the model says "unsafe".  Pointers are fake addresses that
fail validation or, once accepted, stop at the device check: nothing is dereferenced.
"""

import ctypes
import os

import pytest
import torch
from hypothesis import given, settings, strategies as st

from softmax_cross_entropy_amd import abi

# The pointers are fake device addresses, so a call that passes validation must not reach a
# GPU: the module runs only where none is visible, and such calls stop at the device lookup
# with CE_ERR_DEVICE.
pytestmark = [pytest.mark.skipif(not os.path.exists(abi.LIB_PATH), reason="library not built"),
              pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake device addresses: host only")]

OK, LAYOUT, ALIAS, DEVICE = 0, -4, -7, -8
ES = 4  # fp32
BASE = 1 << 40  # fake device addresses, far from each other and 256-byte aligned


def offsets(n, V, rpb, rs, bs):
    """Element offsets of every (row, column) of the view."""
    return [(r // rpb) * bs + (r % rpb) * rs + c for r in range(n) for c in range(V)]


def rows_disjoint(n, V, rpb, rs, bs):
    offs = offsets(n, V, rpb, rs, bs)
    return len(set(offs)) == len(offs)


def call_vjp(n, V, out_lay, out_ptr, in_lay=None, in_ptr=BASE):
    in_lay = in_lay or abi.CELayout(n, V, n * V)
    vp = ctypes.c_void_p
    return abi.lib().ce_vjp_lanes(vp(in_ptr), in_lay, 0, vp(BASE + (1 << 36)), vp(BASE + (2 << 36)),
                                  vp(BASE + (3 << 36)), n, V, vp(out_ptr), out_lay, 0, None)


views = st.tuples(st.integers(1, 24), st.integers(1, 12), st.integers(1, 8), st.integers(0, 40),
                  st.integers(0, 300))


@settings(max_examples=400, deadline=None)
@given(views)
def test_accepted_output_views_never_share_an_element(v):
    n, V, rpb, rs, bs = v
    st_ = call_vjp(n, V, abi.CELayout(rpb, rs, bs), BASE + (8 << 36))
    assert st_ in (OK, DEVICE, LAYOUT), st_
    if st_ != LAYOUT:
        assert rows_disjoint(n, V, rpb, rs, bs), f"accepted an output view whose rows overlap: {v}"


@settings(max_examples=400, deadline=None)
@given(st.integers(1, 24), st.integers(1, 12), st.integers(-2000, 2000))
def test_dlogits_overlapping_the_logits_is_refused(n, V, shift_elems):
    """dlogits as a contiguous view placed shift_elems elements after the logits: exactly the
    in-place case (shift 0) may pass; any other overlap must be refused."""
    lay = abi.CELayout(n, V, n * V)
    out = BASE + shift_elems * ES
    st_ = call_vjp(n, V, lay, out)
    a_lo, a_hi = BASE, BASE + n * V * ES
    b_lo, b_hi = out, out + n * V * ES
    overlap = a_lo < b_hi and b_lo < a_hi
    if shift_elems == 0:
        assert st_ == DEVICE, st_           # in place, same layout
    elif overlap:
        assert st_ in (ALIAS, LAYOUT), (st_, shift_elems)
    else:
        assert st_ == DEVICE, (st_, shift_elems)
