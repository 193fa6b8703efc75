"""Seeded synthetic inputs for the 4-bit attention workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds none of the attention method's arithmetic: it draws
Gaussian noise (counter-based SplitMix64 + Box-Muller, implemented in
``synth.c``), applies RoPE, per-channel outlier multipliers and mean offsets,
and rounds once to binary16.  The post-RoPE placement of the outliers mirrors
the HiFA4 abstract (arXiv 2607.04302, "Abstract"), which applies its
per-channel rescale to Q and K after RoPE.

Workloads (sizes from the benchmark configurations; every tensor is BHSD):

* ``single_head``   B=1, H=1, N=256, d=128, non-causal, K channels {3,17,64,101} x10.
* ``qwen3_8b``      B=1, Hq=32, Hkv=8, N=4096, d=128, causal, RoPE 1e6,
                    8 K outlier channels x12 per KV head + offsets ~ N(0, 2).
* ``gemma2_9b``     B=1, Hq=16, Hkv=8, N=4096, d=256, causal, RoPE 1e4,
                    8 K outlier channels x6 per KV head.
* ``llama_batched`` B=8, Hq=32, Hkv=8, N=2048, d=128, causal, RoPE 5e5,
                    4 K outlier channels x4 per KV head.
* ``decode``        B=64, Hq=32, Hkv=8, d=128, one query per sequence, KV length
                    8192 built with the ``qwen3_8b`` recipe.
* ``kv_append``     the decode cache's shape (B=64, Hkv=8, d=128, 8192 tokens) with K
                    drawn before RoPE, plus RoPE tables (theta 1e6), for cache appends.

Each workload accepts shape overrides so that tests can build scaled-down
instances with the same structure.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream tags: seed = (workload_id << 32) | tag
TAG_Q, TAG_K, TAG_V, TAG_QCAL, TAG_KCAL, TAG_OUTLIER, TAG_OFFSET, TAG_QUERY = range(1, 9)


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (plain C, pthreads)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-ffp-contract=off", src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.synth_normal_f64.argtypes = [u64, u64, i64, vp]
        lib.synth_uniform_f64.argtypes = [u64, u64, i64, vp]
        lib.synth_raw_u64.argtypes = [u64, u64, i64, vp]
        lib.synth_f16_from_f64.argtypes = [dbl]
        lib.synth_f16_from_f64.restype = ctypes.c_uint16
        lib.synth_tensor_f16.argtypes = [u64, i64, i64, i64, i64, i64, dbl, vp, vp, vp, ctypes.c_int]
        lib.synth_tensor_f16.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def seed_of(workload_id: int, tag: int) -> int:
    return ((workload_id & 0xFFFFFFFF) << 32) | tag


def normal(seed: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal_f64(seed, first, n, _ptr(out))
    return out


def uniform(seed: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(seed, first, n, _ptr(out))
    return out


def raw_u64(seed: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_raw_u64(seed, first, n, _ptr(out))
    return out


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def tensor(seed: int, B: int, H: int, N: int, d: int, theta: float = 0.0,
           mult: Optional[np.ndarray] = None, offset: Optional[np.ndarray] = None,
           pos0: int = 0) -> np.ndarray:
    """[B][H][N][d] float16: RoPE_theta(N(0,1) noise) * mult[h][j] + offset[h][j]."""
    out = np.empty((B, H, N, d), dtype=np.float16)
    m = None if mult is None else np.ascontiguousarray(mult, dtype=np.float64).reshape(H, d)
    o = None if offset is None else np.ascontiguousarray(offset, dtype=np.float64).reshape(H, d)
    rc = _load().synth_tensor_f16(seed, B, H, N, d, pos0, float(theta), _ptr(m), _ptr(o),
                                  out.ctypes.data_as(ctypes.c_void_p), threads())
    if rc != 0:
        raise ValueError("synth_tensor_f16: bad shape")
    return out


def outlier_channels(seed: int, H: int, d: int, count: int) -> np.ndarray:
    """[H][count] distinct channel indices per head (smallest `count` keys of a u64 stream)."""
    out = np.empty((H, count), dtype=np.int64)
    for h in range(H):
        keys = raw_u64(seed, d, first=h * d)
        out[h] = np.sort(np.argsort(keys, kind="stable")[:count])
    return out


@dataclass
class Workload:
    """One seeded synthetic attention problem (all tensors float16, BHSD)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    N_q: int
    N_kv: int
    d: int
    causal: bool
    smooth: bool
    alpha: float
    kv_tile: int
    num_splits: int
    reorders: tuple
    q: np.ndarray = field(repr=False, default=None)
    k: np.ndarray = field(repr=False, default=None)
    v: np.ndarray = field(repr=False, default=None)
    q_cal: Optional[np.ndarray] = field(repr=False, default=None)
    k_cal: Optional[np.ndarray] = field(repr=False, default=None)

    @property
    def flops(self) -> float:
        """4 * N_q * N_kv * d * Hq * B, halved when causal (ones column not counted)."""
        f = 4.0 * self.N_q * self.N_kv * self.d * self.Hq * self.B
        return f / 2 if self.causal else f

    @property
    def kv_bytes(self) -> int:
        """B * Hkv * N_kv * (d + d/16): 4-bit codes of K and V plus one scale byte per 32."""
        return self.B * self.Hkv * self.N_kv * (self.d + self.d // 16)


def _head_structure(wid: int, Hkv: int, d: int, n_out: int, factor: float, offset_var: float):
    mult = np.ones((Hkv, d), dtype=np.float64)
    if n_out:
        ch = outlier_channels(seed_of(wid, TAG_OUTLIER), Hkv, d, n_out)
        for g in range(Hkv):
            mult[g, ch[g]] = factor
    off = None
    if offset_var > 0:
        off = np.sqrt(offset_var) * normal(seed_of(wid, TAG_OFFSET), Hkv * d).reshape(Hkv, d)
    return mult, off


def _prefill(name, wid, B, Hq, Hkv, N, d, theta, n_out, factor, offset_var, alpha, reorders,
             kv_tile=64, n_cal=512, N_kv=None):
    N_kv = N if N_kv is None else N_kv
    mult, off = _head_structure(wid, Hkv, d, n_out, factor, offset_var)
    q = tensor(seed_of(wid, TAG_Q), B, Hq, N, d, theta)
    k = tensor(seed_of(wid, TAG_K), B, Hkv, N_kv, d, theta, mult, off)
    v = tensor(seed_of(wid, TAG_V), B, Hkv, N_kv, d)
    w = Workload(name, B, Hq, Hkv, N, N_kv, d, True, alpha is not None, alpha or 0.0,
                 kv_tile, 1, reorders, q, k, v)
    if alpha is not None:
        w.q_cal = tensor(seed_of(wid, TAG_QCAL), 1, Hq, n_cal, d, theta)
        w.k_cal = tensor(seed_of(wid, TAG_KCAL), 1, Hkv, n_cal, d, theta, mult, off)
    return w


def single_head(N: int = 256, d: int = 128, kv_tile: int = 64) -> Workload:
    """B=1, H=1, N queries x N keys, d=128, non-causal; K channels {3,17,64,101} x10;
    Smooth-QK scales from the same tensors (alpha 0.5)."""
    wid = 1
    mult = np.ones((1, d))
    for j in (3, 17, 64, 101):
        if j < d:
            mult[0, j] = 10.0
    q = tensor(seed_of(wid, TAG_Q), 1, 1, N, d)
    k = tensor(seed_of(wid, TAG_K), 1, 1, N, d, 0.0, mult)
    v = tensor(seed_of(wid, TAG_V), 1, 1, N, d)
    w = Workload("single_head", 1, 1, 1, N, N, d, False, True, 0.5, kv_tile, 1, (1,), q, k, v)
    w.q_cal, w.k_cal = q, k
    return w


def qwen3_8b(B=1, Hq=32, Hkv=8, N=4096, d=128, kv_tile=64, n_cal=512, N_kv=None) -> Workload:
    return _prefill("qwen3_8b_prefill", 2, B, Hq, Hkv, N, d, 1e6, 8, 12.0, 2.0, 0.5, (1, 0),
                    kv_tile, n_cal, N_kv)


def gemma2_9b(B=1, Hq=16, Hkv=8, N=4096, d=256, kv_tile=64, n_cal=512, N_kv=None) -> Workload:
    return _prefill("gemma2_9b_prefill", 3, B, Hq, Hkv, N, d, 1e4, 8, 6.0, 0.0, 0.25, (1,),
                    kv_tile, n_cal, N_kv)


def llama_batched(B=8, Hq=32, Hkv=8, N=2048, d=128, kv_tile=64, N_kv=None) -> Workload:
    return _prefill("llama_batched_prefill", 4, B, Hq, Hkv, N, d, 5e5, 4, 4.0, 0.0, None, (1, 0),
                    kv_tile, 512, N_kv)


def decode(B=64, Hq=32, Hkv=8, N_kv=8192, d=128, num_splits=16, kv_tile=64,
           n_cal=512) -> Workload:
    """One query per sequence against a KV cache built with the qwen3_8b recipe
    (RoPE 1e6 over positions 0..N_kv-1, 8 x12 outlier channels + offsets)."""
    wid = 5
    mult, off = _head_structure(wid, Hkv, d, 8, 12.0, 2.0)
    q = tensor(seed_of(wid, TAG_QUERY), B, Hq, 1, d)
    k = tensor(seed_of(wid, TAG_K), B, Hkv, N_kv, d, 1e6, mult, off)
    v = tensor(seed_of(wid, TAG_V), B, Hkv, N_kv, d)
    w = Workload("decode", B, Hq, Hkv, 1, N_kv, d, False, True, 0.5, kv_tile, num_splits, (1,),
                 q, k, v)
    w.q_cal = tensor(seed_of(wid, TAG_QCAL), 1, Hq, n_cal, d, 1e6)
    w.k_cal = tensor(seed_of(wid, TAG_KCAL), 1, Hkv, n_cal, d, 1e6, mult, off)
    return w


def rope_table(theta: float, d: int, n_pos: int, pos0: int = 0):
    """RoPE cosine and sine tables [n_pos][d/2] fp32 for positions pos0 .. pos0+n_pos-1:
    angle (pos0 + p) * theta^(-2j/d), evaluated in double and rounded once to fp32 (the
    same angles ``tensor`` rotates by)."""
    j = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * j / float(d))
    ang = (pos0 + np.arange(n_pos, dtype=np.float64))[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclass
class AppendWorkload:
    """A decode-time KV-cache append problem: binary16 K (before RoPE) and V of N tokens per
    (sequence, KV head), RoPE tables for positions 0..N-1, Smooth-QK calibration tensors.
    A test or benchmark appends tokens [pos, pos + T) of these tensors to a 4-bit cache."""
    name: str
    B: int
    Hkv: int
    Hq: int
    N: int
    d: int
    theta: float
    alpha: float
    k_raw: np.ndarray = field(repr=False, default=None)
    v: np.ndarray = field(repr=False, default=None)
    cos: np.ndarray = field(repr=False, default=None)
    sin: np.ndarray = field(repr=False, default=None)
    q_cal: Optional[np.ndarray] = field(repr=False, default=None)
    k_cal: Optional[np.ndarray] = field(repr=False, default=None)


def kv_append(B=64, Hkv=8, Hq=32, N=8192, d=128, n_cal=512) -> AppendWorkload:
    """Decode-shaped cache (B=64, Hkv=8, d=128, RoPE theta 1e6, the decode workload's 8 x12
    outlier channels and offsets), here drawn before RoPE: the append applies RoPE itself."""
    wid = 6
    mult, off = _head_structure(wid, Hkv, d, 8, 12.0, 2.0)
    k_raw = tensor(seed_of(wid, TAG_K), B, Hkv, N, d, 0.0, mult, off)
    v = tensor(seed_of(wid, TAG_V), B, Hkv, N, d)
    cos, sin = rope_table(1e6, d, N)
    w = AppendWorkload("kv_append", B, Hkv, Hq, N, d, 1e6, 0.5, k_raw, v, cos, sin)
    w.q_cal = tensor(seed_of(wid, TAG_QCAL), 1, Hq, n_cal, d, 1e6)
    w.k_cal = tensor(seed_of(wid, TAG_KCAL), 1, Hkv, n_cal, d, 1e6, mult, off)
    return w


WORKLOADS = {
    "single_head": single_head,
    "qwen3_8b": qwen3_8b,
    "gemma2_9b": gemma2_9b,
    "llama_batched": llama_batched,
    "decode": decode,
}
