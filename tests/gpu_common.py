"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np

import oracle

# Acceptance bounds: >= 99.9 % identical 4-bit codes; output error relative to each
# row's max |O_oracle| at most 1e-2 (max) and 1e-3 (mean).
CODE_MATCH = 0.999
ERR_MAX = 1e-2
ERR_MEAN = 1e-3


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.float16:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def codes_equal(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-nibble equality of packed E2M1 codes, with +0 (code 0) == -0 (code 8)."""
    na, nb = oracle.unpack_nibbles(a), oracle.unpack_nibbles(b)
    za = (na & 7) == 0
    zb = (nb & 7) == 0
    return (na == nb) | (za & zb)


def code_match_fraction(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.mean(codes_equal(a, b)))


def out_error(got_f16: np.ndarray, ref_f16: np.ndarray):
    """(max, mean) of |got - ref| / max_row |ref| over rows of the last axis."""
    g = got_f16.astype(np.float32).reshape(-1, got_f16.shape[-1]).astype(np.float64)
    r = ref_f16.astype(np.float32).reshape(-1, ref_f16.shape[-1]).astype(np.float64)
    rowmax = np.abs(r).max(axis=1, keepdims=True)
    rowmax[rowmax == 0] = 1.0
    e = np.abs(g - r) / rowmax
    return float(e.max()), float(e.mean())


def oracle_quant(w, s=None, inv=None):
    q4 = oracle.quantize_rows(w.q, w.Hkv, s)
    k4 = oracle.quantize_rows(w.k, w.Hkv, inv)
    v4 = oracle.quantize_v(w.v)
    return q4, k4, v4


def mx4_to_dev(pair):
    import bit_flashattention_amd as hf
    return hf.MX4(to_dev(pair[0]), to_dev(pair[1]))


def operand_key(k: int) -> int:
    """Token of a 32-token block stored at nibble k in the library's V_hat layout:
    the bits (k4 k3 k2 k1 k0) of k name token (k3 k2 k4 k1 k0)."""
    return (((k >> 3) & 1) << 4) | (((k >> 2) & 1) << 3) | ((k >> 4) << 2) | (k & 3)


OPERAND_ORDER = np.array([operand_key(k) for k in range(32)])


def tile_v(pair):
    """Canonical V_hat ([B][H][d][Npad/2] codes, [B][H][d][Npad/32] scales) -> the
    library's tiled token layout ([B][H][Npad/64][d][32], [B][H][Npad/64][d][2]) with
    each 32-token block's nibbles in operand order.  A pure re-arrangement of 4-bit
    codes: no value changes."""
    codes, scales = pair
    B, H, d, nb = codes.shape
    t = nb // 32
    nib = oracle.unpack_nibbles(codes).reshape(B, H, d, -1, 32)[..., OPERAND_ORDER]
    nib = nib.reshape(B, H, d, -1, 16, 2).astype(np.uint8)
    codes = (nib[..., 0] | (nib[..., 1] << 4)).reshape(B, H, d, nb)
    c = np.ascontiguousarray(codes.reshape(B, H, d, t, 32).transpose(0, 1, 3, 2, 4))
    s = np.ascontiguousarray(scales.reshape(B, H, d, t, 2).transpose(0, 1, 3, 2, 4))
    return c, s


def v_to_dev(pair):
    return mx4_to_dev(tile_v(pair))
