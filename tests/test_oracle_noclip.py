"""Pins for the no-clipping block-exponent rule (CPU only).

The default MX rule floor(log2 amax) - 2 saturates blocks whose amax * 2^-e lands in [6, 8);
the no-clipping rule takes the smallest e with amax * 2^-e <= 6 (the ablation of the scale
choice for the undefined HIF4 format of HiFA4, arXiv 2607.04302, Abstract).  Checked against
the hand table tests/golden/mx_noclip_table.txt and against the defining inequalities over
random blocks; the P_hat exponent (taken from t, P = 2^t) against the same inequalities in the
log domain; and whole tensors against element-by-element decoding.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_noclip_table.txt")
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _rows(kind):
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#") and line.split()[0] == kind:
            out.append(line.split()[1:])
    return out


def test_noclip_hand_blocks():
    rows = _rows("noclip_block")
    assert len(rows) >= 12
    for amax_s, sc_s, code_s in rows:
        amax = float(amax_s)
        blk = np.array([amax, amax / 3, -amax / 7, 0.0] + [amax / 5] * 28, dtype=np.float32)
        codes, sc = oracle.mx_block(blk, oracle.RULE_NOCLIP)
        assert sc == int(sc_s) and codes[0] == int(code_s), (amax_s, sc, codes[0])


def test_noclip_hand_elements():
    rows = _rows("noclip_elem")
    assert len(rows) >= 5
    for amax_s, x_s, code_s in rows:
        blk = np.zeros(32, dtype=np.float32)
        blk[0], blk[9] = float(amax_s), float(x_s)
        codes, _ = oracle.mx_block(blk, oracle.RULE_NOCLIP)
        assert codes[9] == int(code_s), (amax_s, x_s, codes[9])


def test_phat_exponent_hand_table():
    rows = _rows("phat")
    assert len(rows) >= 12
    for t_s, rule_s, e_s in rows:
        assert oracle.phat_exponent(float(t_s), int(rule_s)) == int(e_s), (t_s, rule_s)


def test_block_exponent_inequalities_random():
    """Over random block maxima spanning 2^-100 .. 2^100: the default rule puts amax * 2^-e in
    [4, 8); the no-clipping rule puts it in (3, 6] and is the smallest such e."""
    rng = np.random.default_rng(11)
    amax = (2.0 ** rng.uniform(-100, 100, 4000)).astype(np.float32)
    for a in amax:
        blk = np.zeros(32, dtype=np.float32)
        blk[5] = -a
        e0 = oracle.mx_exponent(blk, oracle.RULE_OCP)
        e1 = oracle.mx_exponent(blk, oracle.RULE_NOCLIP)
        s0 = float(a) * 2.0 ** -e0
        s1 = float(a) * 2.0 ** -e1
        assert 4.0 <= s0 < 8.0
        assert 3.0 < s1 <= 6.0 and float(a) * 2.0 ** -(e1 - 1) > 6.0
        assert e1 - e0 in (0, 1)
        codes, _ = oracle.mx_block(blk, oracle.RULE_NOCLIP)
        assert E2M1[codes[5] & 7] >= 3.0 and codes[5] & 8  # never saturated, sign kept


def test_phat_exponent_inequalities_random():
    """P_hat's exponent from t: rule 0 gives 2^(t - e) in [4, 8); rule 1 gives the smallest e
    with 2^(t - e) <= 6, up to the single fp32 rounding of t - log2(3/2) at the boundary."""
    rng = np.random.default_rng(12)
    ts = rng.uniform(-120, 1, 20000).astype(np.float32)
    tol = 2.0 ** -20
    for t in ts:
        e0 = oracle.phat_exponent(float(t), 0)
        e1 = oracle.phat_exponent(float(t), 1)
        assert 4.0 <= 2.0 ** (float(t) - e0) < 8.0
        assert 2.0 ** (float(t) - e1) <= 6.0 * (1 + tol)
        assert 2.0 ** (float(t) - (e1 - 1)) > 6.0 * (1 - tol)


@pytest.mark.parametrize("rule", [0, 1])
def test_tensor_quantizers_follow_the_rule(rule):
    """Row and token quantization of a whole tensor equal block-by-block mx_block calls."""
    x = synth.tensor(synth.seed_of(77, 1), 1, 2, 70, 64)
    x[0, 1, 3, :32] = np.float16(1.75)  # a block the default rule would saturate
    codes, scales = oracle.quantize_rows(x, 2, None, rule)
    vc, vs = oracle.quantize_v(x, rule)
    for h in range(2):
        for n in (0, 3, 69):
            for b in range(2):
                c, s = oracle.mx_block(x[0, h, n, 32 * b:32 * b + 32].astype(np.float32), rule)
                assert scales[0, h, n, b] == s
                assert np.array_equal(oracle.unpack_nibbles(codes[0, h, n, 16 * b:16 * b + 16]), c)
        for j in (0, 31, 63):
            blk = np.zeros(32, dtype=np.float32)
            blk[:32] = x[0, h, 32:64, j].astype(np.float32)
            c, s = oracle.mx_block(blk, rule)
            assert vs[0, h, j, 1] == s
            assert np.array_equal(oracle.unpack_nibbles(vc[0, h, j, 16:32]), c)
    assert scales[0, 1, 3, 0] == (126 if rule else 125)
