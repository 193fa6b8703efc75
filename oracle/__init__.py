"""ctypes binding of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and the two
share no code.  The arithmetic lives in ``hifa4_oracle.cpp``; this file only
marshals numpy arrays.

Method: HiFA4 (arXiv 2607.04302), Abstract.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

TOKEN_PAD = 128  # token dimension of every 4-bit layout is padded to a multiple of this


def padded(n: int) -> int:
    return -(-n // TOKEN_PAD) * TOKEN_PAD


def cpu_share() -> int:
    """Host threads the oracle uses when none are given: the CPUs this process may run on,
    at most 16 (the host share one GPU gets on a shared box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build(force: bool = False) -> str:
    """Compile liboracle.so with g++ (no fast-math, no FP contraction)."""
    src = os.path.join(_HERE, "hifa4_oracle.cpp")
    hdr = os.path.join(_HERE, "hifa4_oracle.h")
    newest = max(os.path.getmtime(src), os.path.getmtime(hdr))
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < newest:
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
                               "-ffp-contract=off", "-fno-fast-math", src, "-o", tmp])
        os.replace(tmp, _SO)
    return _SO


class AttnParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("N_q", ctypes.c_int64), ("N_kv", ctypes.c_int64), ("d", ctypes.c_int64),
        ("Npad_q", ctypes.c_int64), ("Npad_kv", ctypes.c_int64),
        ("causal", ctypes.c_int), ("reorder", ctypes.c_int),
        ("kv_tile", ctypes.c_int), ("num_splits", ctypes.c_int),
        ("quantized", ctypes.c_int), ("state_fp16", ctypes.c_int),
        ("q_codes", ctypes.c_void_p), ("q_scales", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("q_f32", ctypes.c_void_p), ("k_f32", ctypes.c_void_p), ("v_f32", ctypes.c_void_p),
        ("out_f16", ctypes.c_void_p), ("out_f32", ctypes.c_void_p),
        ("phat_codes", ctypes.c_void_p), ("phat_scales", ctypes.c_void_p),
        ("sum_p", ctypes.c_void_p), ("sum_phat", ctypes.c_void_p),
        ("m_out", ctypes.c_void_p), ("l_out", ctypes.c_void_p),
        ("rows", ctypes.c_void_p), ("n_rows", ctypes.c_int64),
        ("threads", ctypes.c_int), ("scale_rule", ctypes.c_int),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        i64, vp, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.orc_f16_from_f32.argtypes = [ctypes.c_float]
        lib.orc_f16_from_f32.restype = ctypes.c_uint16
        lib.orc_f32_from_f16.argtypes = [ctypes.c_uint16]
        lib.orc_f32_from_f16.restype = ctypes.c_float
        lib.orc_e2m1_encode.argtypes = [ctypes.c_float]
        lib.orc_e2m1_encode.restype = ctypes.c_int
        lib.orc_e2m1_decode.argtypes = [ctypes.c_int]
        lib.orc_e2m1_decode.restype = ctypes.c_float
        lib.orc_mx_exponent.argtypes = [vp, ctypes.c_int, ctypes.c_int]
        lib.orc_mx_exponent.restype = ctypes.c_int
        lib.orc_mx_block.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int]
        lib.orc_phat_exponent.argtypes = [ctypes.c_float, ctypes.c_int]
        lib.orc_phat_exponent.restype = ctypes.c_int
        lib.orc_calibrate.argtypes = [vp, vp, i64, i64, i64, i64, i64, dbl, vp, vp]
        lib.orc_quantize_rows.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, vp, vp, ctypes.c_int]
        lib.orc_quantize_v.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, ctypes.c_int]
        lib.orc_attn.argtypes = [ctypes.POINTER(AttnParams)]
        lib.orc_attn.restype = ctypes.c_int
        lib.orc_attn_exact.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                       vp, i64, vp, ctypes.c_int]
        lib.orc_attn_exact.restype = ctypes.c_int
        lib.orc_inexact_count.restype = ctypes.c_int64
        lib.orc_f16_from_f32_array.argtypes = [vp, i64, vp]
        lib.orc_f32_from_f16_array.argtypes = [vp, i64, vp]
        lib.orc_score.argtypes = [vp, vp, vp, vp, i64]
        lib.orc_score.restype = ctypes.c_float
        lib.orc_rope_f16.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, i64, vp]
        lib.orc_rope_f16.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p).value


def _f16bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    assert x.dtype == np.uint16
    return x


# ---- scalar pieces --------------------------------------------------------

def f16_from_f32(x: float) -> int:
    return _load().orc_f16_from_f32(float(x))


def f32_from_f16(h: int) -> float:
    return _load().orc_f32_from_f16(int(h))


def f16_from_f32_array(x: np.ndarray) -> np.ndarray:
    xa = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(xa.shape, dtype=np.uint16)
    _load().orc_f16_from_f32_array(_p(xa), xa.size, _p(out))
    return out


def f32_from_f16_array(h: np.ndarray) -> np.ndarray:
    ha = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.zeros(ha.shape, dtype=np.float32)
    _load().orc_f32_from_f16_array(_p(ha), ha.size, _p(out))
    return out


def score(q_codes, q_scales, k_codes, k_scales, d: int) -> float:
    arrs = [np.ascontiguousarray(a, dtype=np.uint8) for a in (q_codes, q_scales, k_codes, k_scales)]
    return _load().orc_score(*[_p(a) for a in arrs], d)


def e2m1_encode(x: float) -> int:
    return _load().orc_e2m1_encode(float(x))


def e2m1_decode(code: int) -> float:
    return _load().orc_e2m1_decode(int(code))


# block-exponent rules: the OCP MX rule (saturates blocks whose amax * 2^-e lands in
# [6, 8)) and the no-clipping rule (smallest e with amax * 2^-e <= 6)
RULE_OCP, RULE_NOCLIP = 0, 1


def mx_block(x, rule: int = RULE_OCP) -> tuple:
    """Quantize <= 32 values: (codes uint8[n], scale byte)."""
    xa = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(len(xa), dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint8)
    _load().orc_mx_block(_p(xa), len(xa), _p(codes), _p(sc), int(rule))
    return codes, int(sc[0])


def mx_exponent(x, rule: int = RULE_OCP) -> int:
    xa = np.ascontiguousarray(x, dtype=np.float32)
    return _load().orc_mx_exponent(_p(xa), len(xa), int(rule))


def phat_exponent(tmax: float, rule: int = RULE_OCP) -> int:
    """Block exponent of P_hat from the block's largest t (P = 2^t)."""
    return _load().orc_phat_exponent(float(tmax), int(rule))


# ---- tensors --------------------------------------------------------------

def calibrate(q_cal: np.ndarray, k_cal: np.ndarray, alpha: float):
    B, Hq, N, d = q_cal.shape
    Hkv = k_cal.shape[1]
    s = np.zeros((Hkv, d), dtype=np.float32)
    inv = np.zeros((Hkv, d), dtype=np.float32)
    _load().orc_calibrate(_p(_f16bits(q_cal)), _p(_f16bits(k_cal)), B, Hq, Hkv, N, d,
                          float(alpha), _p(s), _p(inv))
    return s, inv


def quantize_rows(x: np.ndarray, Hkv: int, mult: Optional[np.ndarray] = None,
                  rule: int = RULE_OCP):
    """[B][H][N][d] f16 -> (codes [B][H][Npad][d/2], scales [B][H][Npad][d/32])."""
    B, H, N, d = x.shape
    Np = padded(N)
    codes = np.zeros((B, H, Np, d // 2), dtype=np.uint8)
    scales = np.zeros((B, H, Np, d // 32), dtype=np.uint8)
    m = None if mult is None else np.ascontiguousarray(mult, dtype=np.float32)
    _load().orc_quantize_rows(_p(_f16bits(x)), B, H, Hkv, N, Np, d, _p(m), _p(codes), _p(scales),
                              int(rule))
    return codes, scales


def quantize_v(v: np.ndarray, rule: int = RULE_OCP):
    """[B][H][N][d] f16 -> (codes [B][H][d][Npad/2], scales [B][H][d][Npad/32])."""
    B, H, N, d = v.shape
    Np = padded(N)
    codes = np.zeros((B, H, d, Np // 2), dtype=np.uint8)
    scales = np.zeros((B, H, d, Np // 32), dtype=np.uint8)
    _load().orc_quantize_v(_p(_f16bits(v)), B, H, N, Np, d, _p(codes), _p(scales), int(rule))
    return codes, scales


def rope_f16(x: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray, pos0: int = 0) -> np.ndarray:
    """Rotate-half RoPE of binary16 rows [B][H][N][d] at positions pos0.. with fp32 tables
    [n_rope][d/2]; binary16 result (one fp32 rounding per product and per sum)."""
    B, H, N, d = x.shape
    c = np.ascontiguousarray(cos_t, dtype=np.float32)
    s = np.ascontiguousarray(sin_t, dtype=np.float32)
    assert c.shape == s.shape and c.shape[1] == d // 2
    out = np.zeros((B, H, N, d), dtype=np.uint16)
    rc = _load().orc_rope_f16(_p(_f16bits(x)), B, H, N, d, pos0, _p(c), _p(s), c.shape[0],
                              _p(out))
    if rc != 0:
        raise ValueError("orc_rope_f16: bad sizes")
    return out.view(np.float16)


def attn(B, Hq, Hkv, N_q, N_kv, d, *, causal, reorder, kv_tile=64, num_splits=1,
         q4=None, k4=None, v4=None, q_f32=None, k_f32=None, v_f32=None, state_fp16=True,
         rows: Optional[np.ndarray] = None, want_phat=False, want_sums=False, want_f32=False,
         want_state=False, threads: int = 0, npad_kv: Optional[int] = None,
         scale_rule: int = RULE_OCP) -> dict:
    """Run the oracle forward.  q4/k4/v4 are (codes, scales) pairs (quantized mode) or
    q_f32/k_f32/v_f32 real tensors (quant-off mode).  Outputs are indexed by the
    position in `rows` (flat ids (b*Hq + h)*N_q + i) or by the flat id when rows is None."""
    quantized = q4 is not None
    Npq, Npk = padded(N_q), (padded(N_kv) if npad_kv is None else npad_kv)
    n = B * Hq * N_q if rows is None else len(rows)
    res = {"out": np.zeros((n, d), dtype=np.uint16)}
    P = AttnParams()
    P.B, P.Hq, P.Hkv, P.N_q, P.N_kv, P.d = B, Hq, Hkv, N_q, N_kv, d
    P.Npad_q, P.Npad_kv = Npq, Npk
    P.causal, P.reorder, P.kv_tile, P.num_splits = int(causal), int(reorder), kv_tile, num_splits
    P.quantized, P.state_fp16 = int(quantized), int(state_fp16)
    keep = []
    if quantized:
        arrs = [np.ascontiguousarray(a) for a in (q4[0], q4[1], k4[0], k4[1], v4[0], v4[1])]
        keep += arrs
        (P.q_codes, P.q_scales, P.k_codes, P.k_scales, P.v_codes, P.v_scales) = [_p(a) for a in arrs]
    else:
        arrs = [np.ascontiguousarray(a, dtype=np.float32) for a in (q_f32, k_f32, v_f32)]
        keep += arrs
        P.q_f32, P.k_f32, P.v_f32 = [_p(a) for a in arrs]
    P.out_f16 = _p(res["out"])
    if want_f32:
        res["out_f32"] = np.zeros((n, d), dtype=np.float32)
        P.out_f32 = _p(res["out_f32"])
    if want_phat:
        res["phat_codes"] = np.zeros((n, Npk // 2), dtype=np.uint8)
        res["phat_scales"] = np.zeros((n, Npk // 32), dtype=np.uint8)
        P.phat_codes, P.phat_scales = _p(res["phat_codes"]), _p(res["phat_scales"])
    T = -(-N_kv // kv_tile)
    if want_sums:
        res["sum_p"] = np.full((n, T), np.nan)
        res["sum_phat"] = np.full((n, T), np.nan)
        P.sum_p, P.sum_phat = _p(res["sum_p"]), _p(res["sum_phat"])
    if want_state:
        res["m"] = np.zeros(n, dtype=np.float32)
        res["l"] = np.zeros(n, dtype=np.float32)
        P.m_out, P.l_out = _p(res["m"]), _p(res["l"])
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        keep.append(r)
        P.rows, P.n_rows = _p(r), len(r)
    P.threads = threads if threads > 0 else cpu_share()
    P.scale_rule = int(scale_rule)
    rc = _load().orc_attn(ctypes.byref(P))
    if rc != 0:
        raise ValueError(f"orc_attn failed with {rc}")
    return res


def attn_exact(q, k, v, causal: bool, rows: Optional[np.ndarray] = None, threads: int = 0):
    """fp64 softmax(QK^T/sqrt(d))V on binary16 inputs; [n_rows][d] float64."""
    B, Hq, N_q, d = q.shape
    Hkv, N_kv = k.shape[1], k.shape[2]
    n = B * Hq * N_q if rows is None else len(rows)
    out = np.zeros((n, d), dtype=np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    rc = _load().orc_attn_exact(_p(_f16bits(q)), _p(_f16bits(k)), _p(_f16bits(v)), B, Hq, Hkv,
                                N_q, N_kv, d, int(causal), _p(r), 0 if r is None else len(r),
                                _p(out), threads if threads > 0 else cpu_share())
    if rc != 0:
        raise ValueError(f"orc_attn_exact failed with {rc}")
    return out


def inexact_count() -> int:
    return _load().orc_inexact_count()


def reset_inexact() -> None:
    _load().orc_reset_inexact()


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """uint8 [..., n/2] -> uint8 [..., n] codes (element 2i from the low nibble)."""
    lo = codes & 0x0F
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


def f16_to_f32_array(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
