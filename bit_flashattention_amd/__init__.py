"""Python binding of libhifa4 (the MI355X 4-bit FlashAttention library).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/hifa4.h``.  PyTorch supplies
device memory and the current stream.  There is no CPU fallback: if the
library is not built, importing a function raises.

The operation is the HiFA4 attention operator (arXiv 2607.04302, Abstract):
4-bit QK^T and PV GEMMs with an FP16 online-softmax state, Smooth-QK and
P-Reordering; the 4-bit format is MXFP4 (E2M1 + E8M0 per 32).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhifa4.so")
TOKEN_PAD = 128
MAX_NKV = 32768

OK, EINVAL, EUNSUPPORTED, ENODEV, EHIP, ENOSPACE = range(6)
# block-exponent rules (hifa4.h): the OCP MX rule, and the smallest exponent that clips nothing
SCALE_OCP, SCALE_NOCLIP = 0, 1
# how P_hat's codes are made (hifa4.h): from 2^t by the hardware exponential, or exp-free from t
PHAT_EXP2, PHAT_EXPFREE = 0, 1

_lib = None


class HiFA4Error(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status}: {message}")
        self.status = status


class AttnArgs(ctypes.Structure):
    """Mirror of hifa4_attn_args."""
    _fields_ = [
        ("q_codes", ctypes.c_void_p), ("q_scales", ctypes.c_void_p),
        ("q_f16", ctypes.c_void_p), ("s", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("out_f16", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("kv_tile", ctypes.c_int), ("num_splits", ctypes.c_int),
        ("phat_codes", ctypes.c_void_p), ("phat_scales", ctypes.c_void_p),
        ("kv_capacity", ctypes.c_int64), ("scale_rule", ctypes.c_int),
        ("phat_mode", ctypes.c_int),
    ]


EXPORTS = (
    "hifa4_version", "hifa4_status_str", "hifa4_last_error", "hifa4_mx4_bytes",
    "hifa4_calibrate_smooth", "hifa4_quantize_qkv", "hifa4_attn_workspace_bytes",
    "hifa4_attn_fwd", "hifa4_attn_fwd_noalloc", "hifa4_kv_append", "hifa4_v_layout",
)


def load(path: str = LIB_PATH):
    """Load libhifa4.so (raises OSError if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run `python -m bit_flashattention_amd.build`")
    lib = ctypes.CDLL(path)
    i64, vp, sz, ci, cf = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    lib.hifa4_version.restype = ci
    lib.hifa4_status_str.argtypes = [ci]
    lib.hifa4_status_str.restype = ctypes.c_char_p
    lib.hifa4_last_error.restype = ctypes.c_char_p
    lib.hifa4_mx4_bytes.argtypes = [ci, i64, i64, i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.hifa4_mx4_bytes.restype = ci
    lib.hifa4_calibrate_smooth.argtypes = [vp, vp, i64, i64, i64, i64, i64, cf, vp, vp, vp]
    lib.hifa4_calibrate_smooth.restype = ci
    lib.hifa4_quantize_qkv.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, vp, vp,
                                       vp, vp, vp, vp, vp, vp, ci, vp]
    lib.hifa4_quantize_qkv.restype = ci
    lib.hifa4_attn_workspace_bytes.argtypes = [i64, i64, i64, i64, ci, ctypes.POINTER(sz)]
    lib.hifa4_attn_workspace_bytes.restype = ci
    lib.hifa4_attn_fwd.argtypes = [i64, i64, i64, i64, i64, i64, ci, ci, ci,
                                   ctypes.POINTER(AttnArgs), vp]
    lib.hifa4_attn_fwd.restype = ci
    lib.hifa4_attn_fwd_noalloc.argtypes = [i64, i64, i64, i64, i64, i64, ci, ci, ci,
                                           ctypes.POINTER(AttnArgs), vp]
    lib.hifa4_attn_fwd_noalloc.restype = ci
    lib.hifa4_kv_append.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, vp, vp, i64, ci, vp,
                                    vp, vp, vp, vp, vp, ci, vp]
    lib.hifa4_kv_append.restype = ci
    lib.hifa4_v_layout.argtypes = [ci, vp, vp, vp, vp, i64, i64, i64, i64, vp]
    lib.hifa4_v_layout.restype = ci
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != OK:
        msg = load().hifa4_last_error().decode(errors="replace")
        raise HiFA4Error(status, where, msg)


def padded(n: int) -> int:
    return -(-n // TOKEN_PAD) * TOKEN_PAD


# ---------------------------------------------------------------------------
# Raw C-ABI calls (same names as the C functions; integers are device pointers)
# ---------------------------------------------------------------------------

def hifa4_mx4_bytes(v_layout: int, B: int, H: int, N: int, d: int):
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().hifa4_mx4_bytes(v_layout, B, H, N, d, ctypes.byref(cb), ctypes.byref(sb)),
           "hifa4_mx4_bytes")
    return cb.value, sb.value


def hifa4_attn_workspace_bytes(B: int, Hq: int, N_q: int, d: int, num_splits: int) -> int:
    n = ctypes.c_size_t()
    _check(load().hifa4_attn_workspace_bytes(B, Hq, N_q, d, num_splits, ctypes.byref(n)),
           "hifa4_attn_workspace_bytes")
    return n.value


def hifa4_calibrate_smooth(q_cal, k_cal, B, Hq, Hkv, N_cal, d, alpha, s_out, inv_s_out, stream):
    _check(load().hifa4_calibrate_smooth(q_cal, k_cal, B, Hq, Hkv, N_cal, d, float(alpha),
                                         s_out, inv_s_out, stream), "hifa4_calibrate_smooth")


def hifa4_quantize_qkv(q, k, v, B, Hq, Hkv, N_q, N_kv, d, smooth, s, inv_s, q_codes, q_scales,
                       k_codes, k_scales, v_codes, v_scales, scale_rule, stream):
    _check(load().hifa4_quantize_qkv(q, k, v, B, Hq, Hkv, N_q, N_kv, d, int(smooth), s, inv_s,
                                     q_codes, q_scales, k_codes, k_scales, v_codes, v_scales,
                                     int(scale_rule), stream), "hifa4_quantize_qkv")


def hifa4_attn_fwd(B, Hq, Hkv, N_q, N_kv, d, causal, smooth, reorder, args: AttnArgs, stream):
    _check(load().hifa4_attn_fwd(B, Hq, Hkv, N_q, N_kv, d, int(causal), int(smooth), int(reorder),
                                 ctypes.byref(args), stream), "hifa4_attn_fwd")


def hifa4_attn_fwd_noalloc(B, Hq, Hkv, N_q, N_kv, d, causal, smooth, reorder, args: AttnArgs,
                           stream):
    _check(load().hifa4_attn_fwd_noalloc(B, Hq, Hkv, N_q, N_kv, d, int(causal), int(smooth),
                                         int(reorder), ctypes.byref(args), stream),
           "hifa4_attn_fwd_noalloc")


def hifa4_kv_append(k_new, v_new, B, Hkv, T, d, pos, kv_capacity, rope_cos, rope_sin, rope_rows,
                    smooth, inv_s, k_codes, k_scales, v_codes, v_scales, v_stage, scale_rule,
                    stream):
    st = (_lib or load()).hifa4_kv_append(k_new, v_new, B, Hkv, T, d, pos, kv_capacity, rope_cos,
                                          rope_sin, rope_rows, int(smooth), inv_s, k_codes,
                                          k_scales, v_codes, v_scales, v_stage, int(scale_rule),
                                          stream)
    if st != OK:
        _check(st, "hifa4_kv_append")


def hifa4_v_layout(to_tiled, codes_in, scales_in, codes_out, scales_out, B, H, N, d, stream):
    _check(load().hifa4_v_layout(int(to_tiled), codes_in, scales_in, codes_out, scales_out, B, H, N,
                                 d, stream), "hifa4_v_layout")


# ---------------------------------------------------------------------------
# torch-tensor conveniences (allocation with torch, then the same C calls)
# ---------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    """Raw HIP stream handle: the given torch stream's, else torch's current stream on the
    current device (read without building a torch.cuda.Stream object, which costs more host
    time than a short kernel launch)."""
    if stream is not None:
        return stream.cuda_stream
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is None:  # a torch without the raw accessor: the public (slower) path
        return torch.cuda.current_stream().cuda_stream
    if not torch.cuda.is_initialized():
        torch.cuda.init()
    return raw(torch._C._cuda_getDevice())


@dataclass
class MX4:
    """A 4-bit tensor: uint8 codes (two E2M1 per byte) + uint8 E8M0 scales."""
    codes: "object"
    scales: "object"


def empty_mx4(v_layout: bool, B: int, H: int, N: int, d: int, device="cuda") -> MX4:
    import torch
    npad = padded(N)
    if v_layout:  # tiled token layout: [B][H][Npad/64][d][32] codes, [..][d][2] scales
        return MX4(torch.empty((B, H, npad // 64, d, 32), dtype=torch.uint8, device=device),
                   torch.empty((B, H, npad // 64, d, 2), dtype=torch.uint8, device=device))
    return MX4(torch.empty((B, H, npad, d // 2), dtype=torch.uint8, device=device),
               torch.empty((B, H, npad, d // 32), dtype=torch.uint8, device=device))


def v_layout(v4: MX4, to_tiled: bool, stream=None) -> MX4:
    """V_hat converted between the canonical token-blocked layout (codes [B][H][d][Npad/2],
    scales [B][H][d][Npad/32]) and the tiled layout the attention kernels read (codes
    [B][H][Npad/64][d][32], scales [B][H][Npad/64][d][2]): hifa4_v_layout.  to_tiled=True
    takes a canonical tensor, False a tiled one; returns a new MX4 in the other layout."""
    import torch
    c = v4.codes
    if to_tiled:
        B, H, d, half = c.shape
        npad = 2 * half
    else:
        B, H, nt, d, _ = c.shape
        npad = 64 * nt
    if to_tiled:
        out = empty_mx4(True, B, H, npad, d, device=c.device)
    else:
        out = MX4(torch.empty((B, H, d, npad // 2), dtype=torch.uint8, device=c.device),
                  torch.empty((B, H, d, npad // 32), dtype=torch.uint8, device=c.device))
    hifa4_v_layout(to_tiled, _ptr(v4.codes), _ptr(v4.scales), _ptr(out.codes), _ptr(out.scales), B, H,
                   npad, d, _stream(stream))
    return out


def calibrate_smooth(q_cal, k_cal, alpha: float, stream=None):
    """Smooth-QK scales (s, inv_s) [Hkv][d] fp32 from binary16 calibration tensors."""
    import torch
    B, Hq, N, d = q_cal.shape
    Hkv = k_cal.shape[1]
    s = torch.empty((Hkv, d), dtype=torch.float32, device=q_cal.device)
    inv = torch.empty_like(s)
    hifa4_calibrate_smooth(_ptr(q_cal.contiguous()), _ptr(k_cal.contiguous()), B, Hq, Hkv, N, d,
                           alpha, _ptr(s), _ptr(inv), _stream(stream))
    return s, inv


def quantize_qkv(q=None, k=None, v=None, *, Hkv: int, smooth: bool = False, s=None, inv_s=None,
                 out=None, scale_rule: int = SCALE_OCP, stream=None):
    """Smooth-QK + MXFP4 quantization.  Returns (q4, k4, v4) (None for skipped inputs).
    `out` may pass preallocated (q4, k4, v4) MX4 buffers."""
    ref = next(t for t in (q, k, v) if t is not None)
    B, d = ref.shape[0], ref.shape[3]
    Hq = q.shape[1] if q is not None else Hkv
    N_q = q.shape[2] if q is not None else 0
    N_kv = (k if k is not None else v).shape[2] if (k is not None or v is not None) else 0
    if out is None:
        q4 = empty_mx4(False, B, Hq, N_q, d, ref.device) if q is not None else None
        k4 = empty_mx4(False, B, Hkv, N_kv, d, ref.device) if k is not None else None
        v4 = empty_mx4(True, B, Hkv, N_kv, d, ref.device) if v is not None else None
    else:
        q4, k4, v4 = out
    hifa4_quantize_qkv(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N_q, N_kv, d, smooth,
                       _ptr(s), _ptr(inv_s),
                       _ptr(q4.codes) if q4 else None, _ptr(q4.scales) if q4 else None,
                       _ptr(k4.codes) if k4 else None, _ptr(k4.scales) if k4 else None,
                       _ptr(v4.codes) if v4 else None, _ptr(v4.scales) if v4 else None,
                       scale_rule, _stream(stream))
    return q4, k4, v4


def make_args(q4: Optional[MX4], k4: MX4, v4: MX4, out, *, q_f16=None, s=None, workspace=None,
              num_splits: int = 1, kv_tile: int = 64, phat: Optional[MX4] = None,
              kv_capacity: int = 0, scale_rule: int = SCALE_OCP,
              phat_mode: int = PHAT_EXP2) -> AttnArgs:
    a = AttnArgs()
    a.q_codes = _ptr(q4.codes) if q4 else None
    a.q_scales = _ptr(q4.scales) if q4 else None
    a.q_f16 = _ptr(q_f16)
    a.s = _ptr(s)
    a.k_codes, a.k_scales = _ptr(k4.codes), _ptr(k4.scales)
    a.v_codes, a.v_scales = _ptr(v4.codes), _ptr(v4.scales)
    a.out_f16 = _ptr(out)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.kv_tile = kv_tile
    a.num_splits = num_splits
    a.phat_codes = _ptr(phat.codes) if phat else None
    a.phat_scales = _ptr(phat.scales) if phat else None
    a.kv_capacity = kv_capacity
    a.scale_rule = scale_rule
    a.phat_mode = phat_mode
    return a


def attn_fwd(q4: Optional[MX4], k4: MX4, v4: MX4, *, B: int, Hq: int, Hkv: int, N_q: int,
             N_kv: int, d: int, causal: bool, smooth: bool, reorder: bool, q_f16=None, s=None,
             num_splits: int = 1, kv_tile: int = 64, out=None, workspace=None,
             phat: Optional[MX4] = None, kv_capacity: int = 0, scale_rule: int = SCALE_OCP,
             phat_mode: int = PHAT_EXP2, stream=None):
    """4-bit attention forward; returns out [B][Hq][N_q][d] binary16.  kv_capacity: token
    rows of the K/V buffers when they are a cache larger than N_kv (0: padded N_kv)."""
    import torch
    dev = k4.codes.device
    if out is None:
        out = torch.empty((B, Hq, N_q, d), dtype=torch.float16, device=dev)
    if workspace is None:
        nbytes = hifa4_attn_workspace_bytes(B, Hq, N_q, d, num_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    args = make_args(q4, k4, v4, out, q_f16=q_f16, s=s, workspace=workspace,
                     num_splits=num_splits, kv_tile=kv_tile, phat=phat, kv_capacity=kv_capacity,
                     scale_rule=scale_rule, phat_mode=phat_mode)
    hifa4_attn_fwd(B, Hq, Hkv, N_q, N_kv, d, causal, smooth, reorder, args, _stream(stream))
    return out


def attn_fwd_noalloc(q4: Optional[MX4], k4: MX4, v4: MX4, *, B: int, Hq: int, Hkv: int,
                     N_q: int, N_kv: int, d: int, causal: bool, smooth: bool, reorder: bool,
                     out, q_f16=None, s=None, num_splits: int = 1, kv_tile: int = 64,
                     phat: Optional[MX4] = None, kv_capacity: int = 0,
                     scale_rule: int = SCALE_OCP, phat_mode: int = PHAT_EXP2, stream=None):
    """attn_fwd through the entry point that allocates nothing: the caller passes `out`, and
    the split-KV partial states use the library's static device scratch."""
    args = make_args(q4, k4, v4, out, q_f16=q_f16, s=s, workspace=None, num_splits=num_splits,
                     kv_tile=kv_tile, phat=phat, kv_capacity=kv_capacity, scale_rule=scale_rule,
                     phat_mode=phat_mode)
    hifa4_attn_fwd_noalloc(B, Hq, Hkv, N_q, N_kv, d, causal, smooth, reorder, args,
                           _stream(stream))
    return out


@dataclass
class KVCache:
    """A 4-bit KV cache of `capacity` token rows per (sequence, KV head): K in the row layout,
    V in the tiled token layout, and the binary16 staging rows of the V block still filling."""
    k4: MX4
    v4: MX4
    v_stage: "object"
    capacity: int


def empty_kv_cache(B: int, Hkv: int, capacity: int, d: int, device="cuda") -> KVCache:
    """Zeroed cache (positions never appended read as zero codes with scale byte 0)."""
    import torch
    if capacity % TOKEN_PAD:
        raise ValueError(f"capacity must be a multiple of {TOKEN_PAD}")
    k4 = empty_mx4(False, B, Hkv, capacity, d, device)
    v4 = empty_mx4(True, B, Hkv, capacity, d, device)
    for t in (k4.codes, k4.scales, v4.codes, v4.scales):
        t.zero_()
    stage = torch.zeros((B, Hkv, 32, d), dtype=torch.float16, device=device)
    return KVCache(k4, v4, stage, capacity)


def kv_append(cache: KVCache, k_new=None, v_new=None, *, pos: int, rope_cos=None, rope_sin=None,
              smooth: bool = False, inv_s=None, scale_rule: int = SCALE_OCP,
              stream=None) -> None:
    """Append tokens [pos, pos + T) ([B][Hkv][T][d] binary16; K before RoPE) to the cache."""
    # written out inline: at one token per sequence this call is host-bound, and every
    # Python-level step here costs a measurable part of the kernel's own time
    ref = k_new if k_new is not None else v_new
    B, Hkv, T, d = ref.shape
    if rope_cos is None:
        rows, cos_p, sin_p = 0, None, _ptr(rope_sin)
    else:
        rows, cos_p, sin_p = rope_cos.shape[0], rope_cos.data_ptr(), _ptr(rope_sin)
    k4, v4 = cache.k4, cache.v4
    hifa4_kv_append(None if k_new is None else k_new.data_ptr(),
                    None if v_new is None else v_new.data_ptr(), B, Hkv, T, d, pos, cache.capacity,
                    cos_p, sin_p, rows, smooth, None if inv_s is None else inv_s.data_ptr(),
                    k4.codes.data_ptr(), k4.scales.data_ptr(), v4.codes.data_ptr(),
                    v4.scales.data_ptr(), cache.v_stage.data_ptr(), scale_rule, _stream(stream))
