"""Bit-level pin of the oracle's split-KV merge (C11) and of the Smooth-QK rule at alpha != 1/2.

Split-KV merge.  With one tile per chunk (num_splits = number of tiles) every chunk starts
from the empty state (m = -inf, l = 0, O = 0), so its state after its only tile has a closed
form with no recurrence (HiFA4 Abstract: 4-bit P_hat from an FP16 running max, normalizer
summed from P_hat with P-Reordering or from P without it, FP16 state):
    m_k = fp16(fp32(c * max S)),  t = fma(S, c, -m_k),  P = fp32(2^t),
    P_hat per 32 keys with e = floor(max t) - 2,  l_k = fp16(fp32(sum P_hat or sum P)),
    O_k = fp32(sum_j P_hat_j V_hat_j).
The chunks are then merged in chunk order:
    M = max m_k,  w_k = fp32(2^(m_k - M)),  L = sum fp32(w_k l_k) (fp32, in order),
    A = sum fp32(w_k O_k) (fp32, in order),  out = fp16(A / fp16(L)).
This file computes all of it in numpy -- its own E2M1 decoding, an exactly rounded fp32 fma
from rational arithmetic, its own ties-to-even E2M1 rounding -- and requires the oracle's
output to be identical bit for bit.  It also shows that the test can tell: dropping the
fp16 rounding of L, or dealing the tiles to chunks in another partition, changes the bits.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # magnitudes of codes 0..7


def dequant_rows(codes, scales):
    """Row-layout MX values [..., N][d] from codes [..., N][d/2] and scales [..., N][d/32]."""
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1)
    val = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sc = np.exp2(scales.astype(np.float64) - 127.0)
    return val * np.repeat(sc, 32, axis=-1)


def dequant_v(codes, scales):
    """Token-blocked V values [..., d][Npad] from codes [..., d][Npad/2], scales [..., d][Npad/32]."""
    return dequant_rows(codes, scales)


def f32_round(x: Fraction) -> np.float32:
    """Round an exact rational to binary32, nearest with ties to even (subnormals kept)."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # a in [2^e, 2^(e+1)); quantum 2^(e-23), or 2^-149 below the normal range
    q = max(e, -126) - 23
    scaled = a / (Fraction(2) ** q)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(n) * 2.0 ** q)


def fmaf(a, b, c) -> np.float32:
    """fp32(a * b + c) with one rounding, the operands being fp32 values."""
    return f32_round(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def f16(x) -> np.float32:
    """binary16 round-to-nearest-even of an fp32 value, as fp32."""
    return np.float32(np.float16(np.float32(x)))


def e2m1_rne_value(x: float) -> float:
    """Magnitude of the nearest E2M1 value to x >= 0, ties to the even code, saturating at 6."""
    mids = (E2M1[:-1] + E2M1[1:]) / 2
    k = int(np.searchsorted(mids, x, side="left"))  # mids strictly below x
    if k < 7 and x == mids[k] and k % 2 == 1:
        k += 1
    return float(E2M1[k])


def one_tile_state(qv, kv, vv, keys, c, reorder, rule=0):
    """State (m, l, O) of one row after the single tile of `keys` (valid keys only), from the
    empty state.  rule 1 takes P_hat's block exponent as the smallest e with
    2^(t_max - e) <= 6 = 2^(2 + log2 1.5), from one fp32 subtraction t_max - fp32(log2 1.5)."""
    if len(keys) == 0:
        return np.float32(-np.inf), np.float32(0.0), np.zeros(vv.shape[0], np.float32)
    S = [f32_round(sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv, kv[j])),
                       Fraction(0))) for j in keys]
    smax = max(S)
    m = f16(np.float32(c) * np.float32(smax))
    t = [fmaf(s, c, -m) for s in S]
    P = [np.float32(np.exp2(np.float64(x))) for x in t]
    P = [p if p >= np.finfo(np.float32).tiny else np.float32(0.0) for p in P]
    Ph = [0.0] * len(keys)
    for b0 in range(0, len(keys), 32):
        # keys of a tile start on a 32-key boundary, so list blocks are the MX blocks
        blk = range(b0, min(b0 + 32, len(keys)))
        tmax = max(t[i] for i in blk)
        if rule == 1:
            u = np.float32(tmax - np.float32(np.log2(1.5)))
            e = max(-127, min(127, int(np.ceil(u)) - 2))
        else:
            e = max(-127, min(127, int(np.floor(tmax)) - 2))
        for i in blk:
            Ph[i] = e2m1_rne_value(float(P[i]) * 2.0 ** -e) * 2.0 ** e
    rs = 0.0
    for i in range(len(keys)):
        rs += Ph[i] if reorder else float(P[i])
    l = f16(np.float32(rs))
    acc = np.zeros(vv.shape[0], np.float64)
    for i, j in enumerate(keys):
        acc = acc + Ph[i] * vv[:, j]  # key order, one double rounding per step
    return m, l, acc.astype(np.float32)


def merge(states, round_L=True):
    M = max(s[0] for s in states)
    w = [np.float32(0.0) if s[0] == -np.inf else np.float32(np.exp2(np.float64(s[0]) - np.float64(M)))
         for s in states]
    L = np.float32(0.0)
    for wk, s in zip(w, states):
        L = np.float32(L + np.float32(wk * s[1]))
    lf = f16(L) if round_L else L
    A = np.zeros_like(states[0][2])
    for wk, s in zip(w, states):
        A = (A + (wk * s[2]).astype(np.float32)).astype(np.float32)
    return np.float16((A / lf).astype(np.float32))


def split_reference(w, q4, k4, v4, kv_tile, chunk_tiles, reorder, round_L=True, rule=0):
    """Rows of a single-head workload through chunks of `chunk_tiles` tiles each, where each
    chunk must be one tile (the closed form above)."""
    assert chunk_tiles == 1
    d = w.d
    qd = dequant_rows(*q4)[0, 0]
    kd = dequant_rows(*k4)[0, 0]
    vd = dequant_v(*v4)[0, 0]
    c = np.float32(1.4426950408889634073599246810019 / np.sqrt(np.float64(d)))
    T = -(-w.N_kv // kv_tile)
    out = np.zeros((w.N_q, d), np.float16)
    for i in range(w.N_q):
        last = i + w.N_kv - w.N_q if w.causal else w.N_kv - 1
        states = []
        for t in range(T):
            keys = [j for j in range(t * kv_tile, min((t + 1) * kv_tile, w.N_kv)) if j <= last]
            states.append(one_tile_state(qd[i], kd, vd, keys, c, reorder, rule))
        out[i] = merge(states, round_L)
    return out


@pytest.fixture(scope="module")
def small():
    # one head, 6 query rows, 200 keys (4 tiles of 64, the last one ragged), d = 64
    w = synth.qwen3_8b(B=1, Hq=1, Hkv=1, N=6, N_kv=200, d=64, n_cal=32)
    s, inv = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    return w, oracle.quantize_rows(w.q, 1, s), oracle.quantize_rows(w.k, 1, inv), oracle.quantize_v(w.v)


@pytest.mark.parametrize("reorder,causal", [(1, False), (0, False), (1, True)])
def test_split_merge_bitwise_one_tile_chunks(small, reorder, causal):
    w, q4, k4, v4 = small
    w.causal = causal
    T = 4
    ref = split_reference(w, q4, k4, v4, 64, 1, reorder)
    got = oracle.attn(1, 1, 1, w.N_q, w.N_kv, w.d, causal=causal, reorder=reorder, kv_tile=64,
                      num_splits=T, q4=q4, k4=k4, v4=v4)["out"]
    assert np.array_equal(got.reshape(w.N_q, w.d), ref.view(np.uint16))


def test_split_merge_bitwise_noclip_rule():
    """The same closed form with every block exponent (Q, K, V and P_hat) from the
    no-clipping rule, against the oracle run with that rule; and the rule matters here: the
    default rule gives different bits on these inputs."""
    w = synth.qwen3_8b(B=1, Hq=1, Hkv=1, N=6, N_kv=200, d=64, n_cal=32)
    s, inv = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    q4 = oracle.quantize_rows(w.q, 1, s, oracle.RULE_NOCLIP)
    k4 = oracle.quantize_rows(w.k, 1, inv, oracle.RULE_NOCLIP)
    v4 = oracle.quantize_v(w.v, oracle.RULE_NOCLIP)
    w.causal = False
    ref = split_reference(w, q4, k4, v4, 64, 1, 1, rule=1)
    got = oracle.attn(1, 1, 1, w.N_q, w.N_kv, w.d, causal=False, reorder=1, kv_tile=64,
                      num_splits=4, q4=q4, k4=k4, v4=v4, scale_rule=1)["out"]
    assert np.array_equal(got.reshape(w.N_q, w.d), ref.view(np.uint16))
    other = oracle.attn(1, 1, 1, w.N_q, w.N_kv, w.d, causal=False, reorder=1, kv_tile=64,
                        num_splits=4, q4=q4, k4=k4, v4=v4, scale_rule=0)["out"]
    assert not np.array_equal(got, other)


def test_split_merge_pin_detects_mistakes(small):
    """The same inputs through a merge without the fp16 rounding of L, and through another
    chunk partition, give different bits: the bitwise test above constrains both."""
    w, q4, k4, v4 = small
    w.causal = False
    got = oracle.attn(1, 1, 1, w.N_q, w.N_kv, w.d, causal=False, reorder=1, kv_tile=64,
                      num_splits=4, q4=q4, k4=k4, v4=v4)["out"].reshape(w.N_q, w.d)
    no_round = split_reference(w, q4, k4, v4, 64, 1, 1, round_L=False)
    assert not np.array_equal(got, no_round.view(np.uint16))
    two_chunks = oracle.attn(1, 1, 1, w.N_q, w.N_kv, w.d, causal=False, reorder=1, kv_tile=64,
                             num_splits=2, q4=q4, k4=k4, v4=v4)["out"].reshape(w.N_q, w.d)
    assert not np.array_equal(got, two_chunks)


def test_fmaf_and_f32_round_helpers():
    # a tie at binary32 precision: 1 + 2^-24 rounds to 1 (even), 1 + 3*2^-24 to 1 + 2^-22
    assert f32_round(Fraction(1) + Fraction(1, 2 ** 24)) == np.float32(1.0)
    assert f32_round(Fraction(1) + Fraction(3, 2 ** 24)) == np.float32(1.0 + 2.0 ** -22)
    # smallest subnormal, and a value just above half of it
    assert f32_round(Fraction(1, 2 ** 149)) == np.float32(2.0 ** -149)
    assert f32_round(Fraction(1, 2 ** 150) + Fraction(1, 2 ** 200)) == np.float32(2.0 ** -149)
    # the product term is kept exact before the single rounding
    a = np.float32(1.0 + 2.0 ** -12)
    assert fmaf(a, a, np.float32(-1.0)) == np.float32(2.0 ** -11 + 2.0 ** -24)
    assert np.float32(a * a) - np.float32(1.0) != np.float32(2.0 ** -11 + 2.0 ** -24)


# ---------------------------------------------------------------------------
# Smooth-QK calibration at strengths other than 1/2: channel maxima chosen so that
# s = kmax^alpha / qmax^(1 - alpha) is an exact small number.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("alpha,kmax,qmax,expect", [
    (0.25, 16.0, 1.0, 2.0), (0.25, 1.0, 16.0, 0.125), (0.25, 81.0, 1.0, 3.0),
    (0.25, 16.0, 16.0, 0.25), (0.75, 16.0, 16.0, 4.0), (0.75, 1.0, 16.0, 0.5),
    (1.0, 6.0, 100.0, 6.0), (0.0, 100.0, 8.0, 0.125), (0.5, 9.0, 4.0, 1.5)])
def test_calibrate_closed_form_alphas(alpha, kmax, qmax, expect):
    q = np.full((1, 2, 4, 32), np.float16(0.5), dtype=np.float16)
    k = np.full((1, 1, 4, 32), np.float16(0.5), dtype=np.float16)
    q[0, 1, 2, 7] = np.float16(-qmax)   # the Q maximum of channel 7 sits in the second head
    k[0, 0, 3, 7] = np.float16(kmax)
    s, inv = oracle.calibrate(q, k, alpha)
    assert s[0, 7] == np.float32(expect)
    assert inv[0, 7] == np.float32(1.0 / expect)
    # the other channels see kmax = qmax = 0.5
    assert s[0, 0] == np.float32(0.5 ** alpha / 0.5 ** (1 - alpha))
