"""Helpers for the GPU parity tests: host<->device transfers and the tolerance rules.

Tolerances (stated once, used by every GPU test):
* float32 logits: |loss - ref| <= 1e-5 and |dlogits - ref| <= 1e-5 per element.
* float16 / bfloat16 logits: |loss - ref| <= 1e-3 |ref| + 1e-5 (loss is float32,
  accumulated in float32; the absolute floor covers losses near 0, where a float32
  sum 1 + eps cannot hold eps < 6e-8), and every dlogits element within
  max(1e-3 |ref|, one ulp of the 16-bit type at |ref|): an output rounded to 16 bits
  already carries up to half an ulp of error, and for bfloat16 one ulp is 2^-7
  relative, so 1e-3 relative alone is unattainable by any 16-bit output.
* lse: the row maximum m must equal the oracle's exactly (it is a stored logit);
  log s follows the loss rule.
* The target element g (p_y - 1) is formed from a float32 p_y.  Where p_y is within
  float32's spacing of 1 the difference cancels: the float32 p_y is within 2^-23 of the
  exact one, so that element carries up to |g| 2^-23 of absolute error however it is
  rounded afterwards (with g = 1 and logits [0, -40] the exact value is -4e-18 and any
  float32 computation gives 0).  Checks that pass the targets and g add |g| 2^-22 to the
  target element's tolerance, 2^-22 covering the exponential's own rounding; every other
  element keeps the rule above.
"""

import numpy as np
import torch

from oracle import ce as oce

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
NP_STORE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def to_dev(x: np.ndarray, dtype: str = None) -> torch.Tensor:
    """Host storage array -> device tensor (bf16 given as uint16 bits)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host storage array (bf16 returned as uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    return oce.decode(x, dtype)


def ulp16(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the 16-bit type at |ref| (subnormal spacing near zero)."""
    a = np.abs(ref)
    if dtype == "f16":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
        return 2.0 ** (e - 10)
    if dtype == "bf16":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
        return 2.0 ** (e - 7)
    raise ValueError(dtype)


def check_loss(got, ref, dtype, what="loss", finite_only=False):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf]), f"{what}: infinities differ"
    ok = ~nan_ref & ~inf
    err = np.abs(got[ok] - ref[ok])
    tol = 1e-5 if dtype == "f32" else 1e-3 * np.abs(ref[ok]) + 1e-5
    bad = err > tol
    if bad.any():
        i = np.flatnonzero(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {ok.sum()} values off; first at {np.flatnonzero(ok)[i]}: "
                             f"got {got[ok][i]!r} ref {ref[ok][i]!r}")
    return float(err.max()) if err.size else 0.0


def target_slack(shape, targets, g) -> np.ndarray:
    """|g| 2^-22 at each row's target column (rows with a target in range), 0 elsewhere."""
    slack = np.zeros(shape)
    y = np.asarray(targets, np.int64).reshape(-1)
    r = np.flatnonzero((y >= 0) & (y < shape[1]))
    slack[r, y[r]] = np.abs(np.asarray(g, np.float64).reshape(-1)[r]) * 2.0 ** -22
    return slack


def check_grad(got_store, ref, dtype, what="dlogits", targets=None, g=None):
    """got_store: device output as host storage; ref: float64 oracle gradient.  With the
    targets and g, the target elements get the cancellation allowance |g| 2^-22."""
    got = decode(got_store, dtype)
    ref = np.asarray(ref, np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    ok = ~nan_ref
    err = np.abs(got[ok] - ref[ok])
    if dtype == "f32":
        tol = np.full(err.shape, 1e-5)
    else:
        tol = np.maximum(1e-3 * np.abs(ref[ok]), ulp16(ref[ok], dtype))
    if targets is not None:
        tol = tol + target_slack(ref.shape, targets, g)[ok]
    bad = err > tol
    if bad.any():
        idx = np.argwhere(ok)[np.flatnonzero(bad)[0]]
        raise AssertionError(f"{what}: {bad.sum()} of {ok.sum()} elements off; first at {tuple(idx)}: "
                             f"got {got[tuple(idx)]!r} ref {ref[tuple(idx)]!r}")
    return float(err.max()) if err.size else 0.0


def check_lse(lse_got, m_ref, ls_ref, dtype, rows=None):
    lse_got = np.asarray(lse_got, np.float64)
    m_ref = np.asarray(m_ref, np.float64)
    ok = np.isfinite(m_ref) & np.isfinite(ls_ref)
    assert np.array_equal(lse_got[ok, 0], m_ref[ok]), "lse: row maximum differs"
    check_loss(lse_got[ok, 1], ls_ref[ok], dtype, "log s")
