"""CPU model of the exponent shift that keeps bfloat16 gradients in the subnormal range.

The kernels form a bf16 gradient g p as (g 2^-S) (2^S p), with 2^S p from the hardware
base-2 exponential, which returns 0 for results below 2^-126 (the smallest normal
float32), and S = clamp(floor(log2 |g|) + 9 + extra, 0, 120), where 2^extra bounds a
further factor on p.  This model replays that arithmetic in float32 (numpy keeps float32
subnormals, as the kernels' float32 mode does) and checks that the bf16 result is within
one bf16 ulp of the exact product for upstream gradients across float32's whole range and
probabilities across [2^-160, 1], and that S = 0 (no shift) fails on the same grid, so the
check has teeth.
"""

import numpy as np

from softmax_cross_entropy_amd.inputs import f32_to_bf16_bits

F32 = np.float32


def exp2_hw(u):
    """2^u rounded to float32, flushed to 0 below 2^-126."""
    r = np.exp2(np.asarray(u, np.float64)).astype(F32)
    return np.where(r < F32(2.0 ** -126), F32(0.0), r)


def out_shift(g, extra=0):
    _, e = np.frexp(np.asarray(g, F32))  # floor(log2 |g|) + 1; 0 for g = 0
    e = np.where(np.isfinite(g), e, 0)
    return np.clip(e + 8 + extra, 0, 120)


def bf16_value(x32):
    bits = f32_to_bf16_bits(np.asarray(x32, F32)).astype(np.uint32) << 16
    return bits.view(F32).astype(np.float64)


def ulp_bf16(a):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** -126))) - 7)


def model(g, u, extra=0, shift=True):
    """bf16 of g 2^u (u = log2 p) the kernels' way; `extra` widens S only."""
    S = out_shift(g, extra) if shift else np.zeros(np.shape(g), np.int64)
    c = (S.astype(np.float64)).astype(F32)          # S - log2 s with log2 s = 0 here
    us = (np.asarray(u, np.float64) + c).astype(F32)  # the exponent's fused multiply-add
    ps = exp2_hw(us)
    gs = np.ldexp(np.asarray(g, F32), -S).astype(F32)
    return bf16_value(gs * ps)


def grid():
    gen = np.random.default_rng(5)
    g = np.concatenate([
        np.exp2(gen.uniform(-149, 127, 4000)) * gen.choice([-1, 1], 4000),
        [1.0, -1.0, 0.75, 2.0 ** -118, 2.0 ** -117, 2.0 ** -9, 2.0 ** 91, 2.0 ** 92, 2.0 ** 100, 2.0 ** 110,
         3 * 2.0 ** -140]]).astype(F32)
    u = np.concatenate([-gen.uniform(0, 160, 400), -np.arange(120, 150, 0.25), [0.0, -1.0]])
    u = u.astype(F32).astype(np.float64)
    return np.meshgrid(g, u, indexing="ij")


def test_shifted_product_is_within_one_bf16_ulp():
    G, U = grid()
    exact = G.astype(np.float64) * np.exp2(U)
    finite = np.abs(exact) < 2.0 ** 127
    got = model(G, U)
    err = np.abs(got - exact)
    bad = finite & (err > ulp_bf16(exact))
    assert not bad.any(), (G[bad][:3], U[bad][:3], got[bad][:3], exact[bad][:3])
    # the grid does reach the subnormal range
    assert np.count_nonzero(finite & (np.abs(exact) > 2.0 ** -134) & (np.abs(exact) < 2.0 ** -126)) > 1000


def test_a_larger_factor_is_covered_by_extra():
    # JS multiplies 2^S Q by a factor below 2^7 in size before g: extra = 8 covers it
    G, U = grid()
    f = F32(100.0)
    S = out_shift(G, 8)
    ps = exp2_hw((U + S).astype(F32))
    with np.errstate(over="ignore"):
        got = bf16_value(np.ldexp(G, -S).astype(F32) * (ps * f))
    exact = G.astype(np.float64) * np.exp2(U) * 100.0
    finite = np.abs(exact) < 2.0 ** 127
    assert not (finite & (np.abs(got - exact) > ulp_bf16(exact))).any()


def test_no_shift_loses_the_subnormal_range():
    G, U = grid()
    exact = G.astype(np.float64) * np.exp2(U)
    finite = np.abs(exact) < 2.0 ** 127
    got = model(G, U, shift=False)
    bad = finite & (np.abs(got - exact) > ulp_bf16(exact))
    assert bad.any()
    # what it loses is exactly the products whose p lies below the exponential's range:
    # bf16 subnormals, and for |g| > 1 normal values too
    assert np.all(U[bad] < -126)
    assert np.any(np.abs(exact[bad]) >= 2.0 ** -126)
