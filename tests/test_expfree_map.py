"""The exp-free P_hat mapping (HIFA4_PHAT_EXPFREE) against E2M1 rounding of 2^u (CPU only).

HiFA4 (arXiv 2607.04302, Abstract): with P-Reordering the normalizer and the PV product both
use the 4-bit P_hat, so only its codes are needed.  The kernel's exp-free mode computes, from
u = t - e (t = S c - m, e the block exponent), the value 2^floor(u) * (1 + r(f)) with
f = u - floor(u) and the cubic r(f) = f (a + f (b + g f)), and rounds that to E2M1.  This file
re-derives the cubic from the E2M1 grid (the fractions at which 2^u crosses a rounding boundary)
and checks, in fp32 arithmetic emulated with numpy, that the mapping gives the code of 2^u
itself: exactly at points away from a boundary, and on all but a few ulps' worth of a dense
sweep.  Exact codes come from the midpoint rule, itself checked against the oracle's encoder.
"""
import numpy as np

import oracle

# the kernel's coefficients (hifa4_device.hpp, expcast_e2m1)
KA, KB, KG = np.float32(0.6950093980189241), np.float32(0.22919986977314274), np.float32(0.07502727831798092)

# E2M1 rounding boundaries of non-negative values, with the side a tie goes to (even code)
BOUNDS = [(0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False)]


def e2m1_code(x):
    """Magnitude code 0..7 of RNE to E2M1 (ties to the even code, saturating at 6)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.zeros(x.shape, dtype=np.int64)
    for b, tie_up in BOUNDS:
        c += (x >= b) if tie_up else (x > b)
    return c


def f32_fma(a, b, c):
    return (np.float64(a) * np.float64(b) + np.float64(c)).astype(np.float32)


def expcast(u):
    u = np.asarray(u, dtype=np.float32)
    k = np.floor(u)
    f = (u - k).astype(np.float32)
    m = f32_fma(f, f32_fma(f, f32_fma(f, KG, KB), KA), np.float32(1.0))
    return np.ldexp(m.astype(np.float64), k.astype(np.int64))


def test_midpoint_rule_matches_oracle_encoder():
    xs = np.concatenate([np.linspace(0, 7, 2801), [b for b, _ in BOUNDS]])
    got = e2m1_code(xs)
    ref = np.array([oracle.e2m1_encode(float(x)) for x in xs])
    assert np.array_equal(got, ref)


def test_cubic_hits_the_boundary_fractions():
    """r(f) = 2^f - 1 at the three fractions where 2^u meets a boundary; r(0) = 0; increasing."""
    fr = np.log2([1.25, 1.5, 1.75])
    m = np.stack([fr, fr ** 2, fr ** 3], axis=1)
    a, b, g = np.linalg.solve(m, 2.0 ** fr - 1.0)
    assert np.allclose([a, b, g], [KA, KB, KG], rtol=1e-7)
    f = np.linspace(0.0, 1.0, 20001)
    r = f * (a + f * (b + g * f))
    assert np.all(np.diff(r) > 0)
    assert np.max(np.abs(r - (2.0 ** f - 1.0))) < 1e-3  # a stand-in for 2^f, exact only where it matters


def test_codes_equal_those_of_exp2_away_from_boundaries():
    rng = np.random.default_rng(11)
    u = rng.uniform(-12.0, 3.0, size=400000).astype(np.float32)
    exact = e2m1_code(np.exp2(u.astype(np.float64)))
    got = e2m1_code(expcast(u))
    # distance of 2^u to the nearest boundary, relative
    x = np.exp2(u.astype(np.float64))
    near = np.zeros(u.shape, dtype=bool)
    for b, _ in BOUNDS:
        near |= np.abs(x / b - 1.0) < 2e-6
    assert np.array_equal(got[~near], exact[~near])
    assert np.mean(got == exact) > 1 - 1e-5


def test_dense_sweep_and_edges():
    # every 64th fp32 value in [-130, 3): masked keys clamp to -126 and give code 0
    lo = np.float32(-130.0).view(np.uint32)
    neg = np.arange(np.float32(-1e-30).view(np.uint32), lo, 64, dtype=np.uint32).view(np.float32)
    pos = np.arange(0, np.float32(3.0).view(np.uint32), 64, dtype=np.uint32).view(np.float32)
    u = np.maximum(np.concatenate([neg, pos]), np.float32(-126.0))
    agree = np.mean(e2m1_code(expcast(u)) == e2m1_code(np.exp2(u.astype(np.float64))))
    assert agree > 1 - 1e-6
    # the boundaries themselves: u = -2 is the 0/0.5 tie (code 0), u = log2 of a boundary
    # +- 1e-5 lands on the right side
    assert e2m1_code(expcast(np.float32(-2.0)))[()] == 0
    for b, _ in BOUNDS:
        lb = np.log2(b)
        for du, side in ((-1e-5, 0), (1e-5, 1)):
            uu = np.float32(lb + du)
            assert e2m1_code(expcast(uu))[()] == e2m1_code(np.exp2(np.float64(uu)))[()]
    assert e2m1_code(expcast(np.float32(-126.0)))[()] == 0
