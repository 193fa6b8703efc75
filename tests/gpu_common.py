"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import json
import os

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


def valid_keys(flat_rows: np.ndarray, N_q: int, N_kv: int, causal: bool) -> np.ndarray:
    """Number of keys each query row attends to: keys j < N_kv and, when causal,
    j <= i + N_kv - N_q (bottom-right alignment), for flat rows (b*Hq + h)*N_q + i."""
    i = np.asarray(flat_rows, dtype=np.int64) % N_q
    if not causal:
        return np.full(i.shape, N_kv, dtype=np.int64)
    return np.minimum(i + N_kv - N_q + 1, N_kv)


def phat_match(got_codes, got_scales, ref_codes, ref_scales, nvalid, chunk=4096):
    """P_hat agreement over the entries that carry information: codes of the keys a row
    attends to (j < nvalid[row]) and scale bytes of the 32-key blocks holding at least one
    such key.  Keys past a row's last valid key are zero on both sides by construction and
    are left out, so the fractions are over real codes only.
    Returns (code fraction, scale fraction, codes compared, blocks compared)."""
    n = got_codes.shape[0]
    gc = got_codes.reshape(n, -1)
    rc = ref_codes.reshape(n, -1)
    gs = got_scales.reshape(n, -1)
    rs = ref_scales.reshape(n, -1)
    nvalid = np.asarray(nvalid, dtype=np.int64).reshape(n)
    keys = np.arange(gc.shape[1] * 2, dtype=np.int64)
    blocks = np.arange(gs.shape[1], dtype=np.int64)
    code_eq = code_n = blk_eq = blk_n = 0
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        nv = nvalid[r0:r1, None]
        km = keys[None, :] < nv
        bm = 32 * blocks[None, :] < nv
        eq = codes_equal(gc[r0:r1], rc[r0:r1])
        code_eq += int(np.count_nonzero(eq & km))
        code_n += int(np.count_nonzero(km))
        blk_eq += int(np.count_nonzero((gs[r0:r1] == rs[r0:r1]) & bm))
        blk_n += int(np.count_nonzero(bm))
    cf = code_eq / code_n if code_n else 1.0
    sf = blk_eq / blk_n if blk_n else 1.0
    return cf, sf, code_n, blk_n


def record(case: str, **fields):
    """Print one parity record and, when HIFA4_PARITY_RECORD names a file, append it there
    as a JSON line (the GPU runs keep these as the record of the measured fractions)."""
    rec = {"case": case, **{k: (float(v) if isinstance(v, (np.floating, float)) else
                                 int(v) if isinstance(v, (np.integer,)) else v)
                             for k, v in fields.items()}}
    line = json.dumps(rec, sort_keys=False)
    print("  " + line, flush=True)
    path = os.environ.get("HIFA4_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
    return rec


def out_error(got_f16: np.ndarray, ref_f16: np.ndarray):
    """(max, mean) of |got - ref| / max_row |ref| over rows of the last axis."""
    g = got_f16.astype(np.float32).reshape(-1, got_f16.shape[-1]).astype(np.float64)
    r = ref_f16.astype(np.float32).reshape(-1, ref_f16.shape[-1]).astype(np.float64)
    rowmax = np.abs(r).max(axis=1, keepdims=True)
    rowmax[rowmax == 0] = 1.0
    e = np.abs(g - r) / rowmax
    return float(e.max()), float(e.mean())


def oracle_quant(w, s=None, inv=None, rule=0):
    q4 = oracle.quantize_rows(w.q, w.Hkv, s, rule)
    k4 = oracle.quantize_rows(w.k, w.Hkv, inv, rule)
    v4 = oracle.quantize_v(w.v, rule)
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


def check_attn(case: str, got_out, ref, nvalid, phat=None, **fields):
    """Assert the acceptance bars on one attention result and record the measured figures:
    output error (relative to each row's max |O_oracle|) and, when a P_hat dump is given as
    (codes, scales) host arrays, code and scale agreement over valid keys only."""
    emax, emean = out_error(got_out, ref["out"].view(np.float16))
    rec = dict(fields, rows=int(np.asarray(nvalid).size), err_max=emax, err_mean=emean)
    if phat is not None:
        cf, sf, nc, nb = phat_match(phat[0], phat[1], ref["phat_codes"], ref["phat_scales"],
                                    nvalid)
        rec.update(phat_code_match=cf, phat_scale_match=sf, phat_codes=nc, phat_blocks=nb)
    record(case, **rec)
    msg = f"{case}: {rec}"
    assert emax <= ERR_MAX and emean <= ERR_MEAN, msg
    if phat is not None:
        assert rec["phat_code_match"] >= CODE_MATCH and rec["phat_scale_match"] >= CODE_MATCH, msg
    return rec
