"""Pins for the oracle's number formats (CPU only).

* E2M1 / MX block encoding against the hand table in tests/golden/e2m1_mx_table.txt,
  worked from the format definition (HiFA4, arXiv 2607.04302, Abstract names the
  4-bit block-scaled operands; the MXFP4 substitute is defined in that fixture).
* binary16 rounding against numpy's own IEEE conversion (an independent library
  routine) over every binary16 pattern and over a dense float32 sweep.
* Tensor quantization layouts (nibble order, token padding, V transposition,
  Smooth-QK multiply) against brute-force element-by-element decoding.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_mx_table.txt")


def _table():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def test_hand_table_elements():
    n = 0
    for r in _table():
        if r[0] != "element":
            continue
        x = float(r[1])
        assert oracle.e2m1_encode(x) == int(r[2]), r
        n += 1
    assert n >= 20


def test_hand_table_blocks():
    n = 0
    for r in _table():
        if r[0] != "block":
            continue
        amax = float(r[1])
        blk = np.array([amax, amax / 3, -amax / 7, 0.0] + [amax / 5] * 28, dtype=np.float32)
        codes, sc = oracle.mx_block(blk)
        assert sc == int(r[2]), r
        assert codes[0] == int(r[3]), r
        if amax == 0:
            assert not (codes & 7).any()  # zeros keep their sign (code 8 is -0)
        n += 1
    assert n >= 8


def test_e2m1_decode_table():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.e2m1_decode(c)
        assert abs(v) == mags[c & 7]
        assert np.signbit(v) == bool(c & 8)
    # decode(encode(v)) == v for every representable value
    for c in range(16):
        v = oracle.e2m1_decode(c)
        assert oracle.e2m1_decode(oracle.e2m1_encode(v)) == v


def test_e2m1_sweep_nearest_and_monotone():
    """Every input maps to a nearest grid value; ties only at midpoints; monotone."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    xs = np.linspace(0, 7.5, 3001)
    prev = -1
    for x in xs:
        c = oracle.e2m1_encode(float(x))
        v = grid[c & 7]
        dist = abs(min(x, 6.0) - v)
        assert dist <= np.min(np.abs(min(x, 6.0) - grid)) + 1e-12
        assert (c & 7) >= prev
        prev = c & 7


def test_fp16_all_patterns_roundtrip():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.f32_from_f16_array(pats)
    ref = pats.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(f[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.all(np.isnan(f[nan]))
    back = oracle.f16_from_f32_array(f)
    assert np.array_equal(back[~nan], pats[~nan])


def test_fp16_rne_matches_numpy():
    rng = np.random.default_rng(7)
    # dense sweep of bit patterns across the whole binary16 range and beyond
    bits = rng.integers(0x2F000000, 0x47FFFFFF, size=400000, dtype=np.uint32)
    x = bits.view(np.float32)
    x = np.concatenate([x, -x, np.array([65504, 65519.99, 65520, 2.0**-24, 2.0**-25,
                                         2.0**-25 * 1.0000001, 3 * 2.0**-26, 1e-30, 0.0,
                                         -0.0, np.inf, -np.inf], dtype=np.float32)])
    got = oracle.f16_from_f32_array(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_mx_exponent_cases():
    assert oracle.mx_exponent(np.zeros(32)) == -127
    assert oracle.mx_exponent(np.full(32, 2.0**-140, dtype=np.float32)) == -127  # clamp
    assert oracle.mx_exponent(np.array([1.0])) == -2
    assert oracle.mx_exponent(np.array([-7.9])) == 0
    assert oracle.mx_exponent(np.array([3e38], dtype=np.float32)) == 125


def _decode_rows(codes, scales):
    """[..., n/2] nibbles + [..., n/32] scales -> float64 [..., n] (brute force)."""
    nib = oracle.unpack_nibbles(codes).astype(np.int64)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    val = mags[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sc = np.repeat(scales.astype(np.int64) - 127, 32, axis=-1)
    return val * np.exp2(sc.astype(np.float64))


def test_quantize_rows_layout_and_error():
    w = synth.qwen3_8b(B=1, Hq=4, Hkv=2, N=200, d=128, n_cal=64)
    s, inv = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    qc, qs = oracle.quantize_rows(w.q, w.Hkv, s)
    assert qc.shape == (1, 4, 256, 64) and qs.shape == (1, 4, 256, 4)
    assert not qc[:, :, 200:].any() and not qs[:, :, 200:].any()  # padding rows are zero
    deq = _decode_rows(qc[:, :, :200], qs[:, :, :200])
    x = w.q.astype(np.float32) * np.repeat(s, 2, axis=0)[None, :, None, :]  # head h uses s[h // 2]
    # error bound from the format: half the widest grid gap (2 * 2^e between 4 and 6)
    # for unclipped values, and up to 2 * 2^e for values clipped from [6, 8) * 2^e
    blk_max = np.abs(x).reshape(1, 4, 200, 4, 32).max(-1)
    e = np.floor(np.log2(blk_max)) - 2
    step = np.repeat(np.exp2(e), 32, axis=-1).reshape(x.shape)
    err = np.abs(deq - x)
    clipped = np.abs(x) > 6 * step
    assert np.all(err[~clipped] <= step[~clipped])
    assert np.all(err[clipped] <= 2 * step[clipped])
    # nibble order: element 2i in the low nibble
    c0 = oracle.mx_block(x[0, 0, 0, :32])[0]
    assert np.array_equal(oracle.unpack_nibbles(qc[0, 0, 0, :16]), c0)


def test_quantize_v_layout():
    v = synth.tensor(synth.seed_of(99, 3), 1, 2, 70, 64)
    vc, vs = oracle.quantize_v(v)
    assert vc.shape == (1, 2, 64, 64) and vs.shape == (1, 2, 64, 4)
    for h in range(2):
        for j in (0, 5, 63):
            for beta in range(4):
                blk = np.zeros(32, dtype=np.float32)
                n1 = min(70, 32 * beta + 32)
                if n1 > 32 * beta:
                    blk[:n1 - 32 * beta] = v[0, h, 32 * beta:n1, j].astype(np.float32)
                c, sc = oracle.mx_block(blk)
                assert vs[0, h, j, beta] == sc
                assert np.array_equal(oracle.unpack_nibbles(vc[0, h, j, 16 * beta:16 * beta + 16]), c)
    assert not vc[..., 48:].any()  # tokens 96.. are pure padding (blocks 3) -> zero
    assert not vs[..., 3].any()


def test_calibrate_alpha_half_is_sqrt_ratio():
    """The single-head workload fixes s_j = sqrt(max|K_j| / max|Q_j|) for alpha = 0.5."""
    w = synth.single_head()
    s, inv = oracle.calibrate(w.q_cal, w.k_cal, 0.5)
    q = np.abs(w.q.astype(np.float64)).max(axis=(0, 2))[0]
    k = np.abs(w.k.astype(np.float64)).max(axis=(0, 2))[0]
    ref = np.sqrt(k / q)
    assert np.allclose(s[0], ref, rtol=2 ** -23, atol=0)
    assert np.allclose(inv[0] * s[0], 1.0, rtol=2 ** -22)
    # outlier channels get the largest scales (difficulty moves from K to Q)
    top = set(np.argsort(s[0])[-4:].tolist())
    assert top == {3, 17, 64, 101}


def test_calibrate_gqa_groups_and_alpha():
    w = synth.qwen3_8b(B=1, Hq=8, Hkv=2, N=64, d=64, n_cal=96)
    s, _ = oracle.calibrate(w.q_cal, w.k_cal, 0.25)
    qg = np.abs(w.q_cal.astype(np.float64)).reshape(1, 2, 4, 96, 64).max(axis=(0, 2, 3))
    kg = np.abs(w.k_cal.astype(np.float64)).max(axis=(0, 2))
    ref = kg ** 0.25 / qg ** 0.75
    assert np.allclose(s, ref, rtol=2 ** -22)
