"""Pins for the oracle's RoPE step (CPU only).

The HiFA4 abstract (arXiv 2607.04302) applies Smooth-QK to K after RoPE, so a
decode-time cache append rotates each new K row before smoothing and
quantizing it.  The pages do not define RoPE; the oracle takes the rotate-half
form (channel j < d/2 paired with j + d/2) with caller-supplied fp32 cosine
and sine tables.  Pinned here by:

* closed forms: the zero angle leaves a row unchanged, a quarter turn maps
  (a, b) to (-b, a) and a half turn to (-a, -b), all bit for bit;
* the input generator's own double-precision RoPE (written separately in C):
  rotating the generator's unrotated noise must land within the binary16
  rounding of both sides on the generator's rotated noise, at every position;
* invariants: pair norms are preserved, and rotating a sequence in pieces
  (positions offset by pos0) equals rotating it whole, bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth


def _noise(seed, B, H, N, d, theta=0.0, pos0=0):
    return synth.tensor(seed, B, H, N, d, theta, pos0=pos0)


def test_zero_angle_is_identity():
    x = _noise(11, 2, 3, 5, 64)
    cos, sin = synth.rope_table(1e4, 64, 5)
    cos[:] = 1.0
    sin[:] = 0.0
    r = oracle.rope_f16(x, cos, sin)
    assert np.array_equal(r.view(np.uint16), x.view(np.uint16))
    # the real table has angle 0 at position 0
    cos, sin = synth.rope_table(1e4, 64, 5)
    r = oracle.rope_f16(x, cos, sin)
    assert np.array_equal(r[:, :, 0].view(np.uint16), x[:, :, 0].view(np.uint16))


@pytest.mark.parametrize("c,s,sa,sb", [(0.0, 1.0, None, None), (-1.0, 0.0, -1, -1)])
def test_quarter_and_half_turn(c, s, sa, sb):
    d = 128
    x = _noise(12, 1, 2, 7, d)
    cos = np.full((7, d // 2), c, dtype=np.float32)
    sin = np.full((7, d // 2), s, dtype=np.float32)
    r = oracle.rope_f16(x, cos, sin).astype(np.float32)
    a, b = x[..., : d // 2].astype(np.float32), x[..., d // 2:].astype(np.float32)
    if sa is None:  # quarter turn: (a, b) -> (-b, a)
        want = np.concatenate([-b, a], axis=-1)
    else:           # half turn: (a, b) -> (-a, -b)
        want = np.concatenate([-a, -b], axis=-1)
    assert np.array_equal(r + 0.0, want + 0.0)


@pytest.mark.parametrize("theta,d,pos0", [(1e6, 128, 0), (1e4, 256, 3000), (5e5, 64, 8185)])
def test_matches_generator_rope(theta, d, pos0):
    """synth.tensor(theta) rotates exact noise in double, then rounds once; the oracle
    rotates the binary16-rounded noise in fp32 and rounds again.  Both describe the same
    rotation, so they differ by the input's binary16 rounding plus one output ulp."""
    B, H, N = 2, 2, 24
    raw = _noise(21, B, H, N, d, 0.0, pos0)
    ref = _noise(21, B, H, N, d, theta, pos0).astype(np.float64)
    cos, sin = synth.rope_table(theta, d, pos0 + N)
    got = oracle.rope_f16(raw, cos, sin, pos0=pos0).astype(np.float64)
    a = np.abs(raw.astype(np.float64))
    pair = np.concatenate([a[..., : d // 2] + a[..., d // 2:]] * 2, axis=-1)
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    tol = pair * 2.0 ** -10 + 2 * ulp + 2.0 ** -24
    assert np.all(np.abs(got - ref) <= tol)
    # a swapped sine sign or a wrong pairing is far outside that bound
    bad = np.concatenate([got[..., d // 2:], got[..., : d // 2]], axis=-1)
    assert np.mean(np.abs(bad - ref) > tol) > 0.5


def test_pair_norm_preserved():
    d = 128
    x = _noise(31, 1, 4, 64, d, 0.0)
    cos, sin = synth.rope_table(1e6, d, 4096)
    r = oracle.rope_f16(x, cos, sin, pos0=4000).astype(np.float64)
    x = x.astype(np.float64)
    n0 = x[..., : d // 2] ** 2 + x[..., d // 2:] ** 2
    n1 = r[..., : d // 2] ** 2 + r[..., d // 2:] ** 2
    assert np.all(np.abs(np.sqrt(n1) - np.sqrt(n0)) <= np.sqrt(n0) * 2.0 ** -9 + 2.0 ** -20)


def test_pieces_equal_whole():
    d, N = 64, 77
    x = _noise(41, 2, 2, N, d)
    cos, sin = synth.rope_table(1e4, d, N)
    whole = oracle.rope_f16(x, cos, sin)
    for a, b in ((0, 1), (1, 33), (33, 64), (64, 77)):
        part = oracle.rope_f16(np.ascontiguousarray(x[:, :, a:b]), cos, sin, pos0=a)
        assert np.array_equal(part.view(np.uint16), whole[:, :, a:b].view(np.uint16))


def test_table_too_short_is_rejected():
    x = _noise(51, 1, 1, 4, 64)
    cos, sin = synth.rope_table(1e4, 64, 5)
    with pytest.raises(ValueError):
        oracle.rope_f16(x, cos, sin, pos0=2)
