"""GPU parity of the no-clipping block-exponent rule (scale_rule = HIFA4_SCALE_NOCLIP).

Every 4-bit block the library writes or computes -- Q_hat, K_hat, V_hat from the quantize
pass, a query quantized inside the attention kernels, the KV-cache append, and P_hat inside
the attention -- takes the smallest exponent that clips nothing instead of the OCP MX rule.
Against the oracle run with the same rule: identical Q/K/V codes and scale bytes, >= 99.9 %
identical P_hat codes and scale bytes over valid keys, output error <= 1e-2 max and <= 1e-3
mean relative to each row's max |O_oracle|.  Each case also checks that the rule takes
effect (some P_hat scale bytes differ from the default rule's).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import (check_attn, codes_equal, mx4_to_dev, oracle_quant, tile_v, to_dev,
                        to_host, v_to_dev, valid_keys)

pytestmark = pytest.mark.gpu
NOCLIP = 1


@pytest.fixture(scope="module")
def hf():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible HIP device")
    import bit_flashattention_amd as m
    m.load()
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,kw", [
    ("qwen3_8b", dict(B=1, Hq=8, Hkv=2, N=300, d=128, n_cal=96)),
    ("gemma2_9b", dict(B=1, Hq=4, Hkv=2, N=130, d=256, n_cal=64)),
    ("llama_batched", dict(B=2, Hq=4, Hkv=2, N=257, d=64)),
])
def test_quantize_noclip_matches_oracle(hf, name, kw):
    print(f"[noclip quantize] {name} {kw}", flush=True)
    w = synth.WORKLOADS[name](**kw)
    # blocks whose largest magnitude has a mantissa above 1.5 (the default rule saturates them)
    w.q[0, 0, 5, :] = np.float16(1.75)
    w.k[0, 1, 7, 32:64] = np.float16(-3.5)
    w.v[0, 0, 40:72, 3] = np.float16(7.0)
    s = inv = s_ref = inv_ref = None
    if w.smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
        s, inv = to_dev(s_ref), to_dev(inv_ref)
    q4, k4, v4 = hf.quantize_qkv(to_dev(w.q), to_dev(w.k), to_dev(w.v), Hkv=w.Hkv,
                                 smooth=w.smooth, s=s, inv_s=inv, scale_rule=NOCLIP)
    _sync()
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref, rule=NOCLIP)
    for got, ref in ((q4, rq), (k4, rk), (v4, tile_v(rv))):
        assert np.all(codes_equal(to_host(got.codes), ref[0]))
        assert np.array_equal(to_host(got.scales), ref[1])
    # the rule took effect: the default rule's scale bytes differ somewhere
    assert not np.array_equal(oracle_quant(w, s_ref, inv_ref, rule=0)[0][1], rq[1])


PREFILL = [
    # name, overrides, reorder, kv_tile, raw_q
    ("qwen3_8b", dict(B=1, Hq=4, Hkv=1, N=512, d=128, n_cal=128), 1, 128, False),
    ("qwen3_8b", dict(B=1, Hq=2, Hkv=2, N=200, N_kv=330, d=128, n_cal=64), 0, 64, True),
    ("gemma2_9b", dict(B=1, Hq=2, Hkv=1, N=384, d=256, n_cal=128), 1, 64, False),
    ("llama_batched", dict(B=2, Hq=4, Hkv=2, N=257, d=64), 1, 128, True),
]


@pytest.mark.parametrize("name,kw,reorder,kv_tile,raw_q", PREFILL)
def test_prefill_noclip_matches_oracle(hf, name, kw, reorder, kv_tile, raw_q):
    import torch
    print(f"[noclip prefill] {name} {kw} reorder={reorder} kv_tile={kv_tile} raw_q={raw_q}",
          flush=True)
    w = synth.WORKLOADS[name](**kw)
    s_ref = inv_ref = None
    if w.smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref, rule=NOCLIP)
    npk = oracle.padded(w.N_kv)
    phat = hf.MX4(torch.zeros((w.B, w.Hq, w.N_q, npk // 2), dtype=torch.uint8, device="cuda"),
                  torch.zeros((w.B, w.Hq, w.N_q, npk // 32), dtype=torch.uint8, device="cuda"))
    qarg = dict(q_f16=to_dev(w.q), s=None if s_ref is None else to_dev(s_ref)) if raw_q else {}
    out = hf.attn_fwd(None if raw_q else mx4_to_dev(rq), mx4_to_dev(rk), v_to_dev(rv), B=w.B,
                      Hq=w.Hq, Hkv=w.Hkv, N_q=w.N_q, N_kv=w.N_kv, d=w.d, causal=w.causal,
                      smooth=w.smooth, reorder=reorder, phat=phat, kv_tile=kv_tile,
                      scale_rule=NOCLIP, **qarg)
    _sync()
    ref = oracle.attn(w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, causal=w.causal, reorder=reorder,
                      kv_tile=kv_tile, q4=rq, k4=rk, v4=rv, want_phat=True, scale_rule=NOCLIP)
    got = to_host(out).reshape(-1, w.d)
    n = len(got)
    ps = to_host(phat.scales).reshape(n, -1)
    check_attn(f"noclip prefill {name} {kw} reorder={reorder} kv_tile={kv_tile} raw_q={raw_q}",
               got, ref, valid_keys(np.arange(n), w.N_q, w.N_kv, w.causal),
               phat=(to_host(phat.codes).reshape(n, -1), ps))
    ref0 = oracle.attn(w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, causal=w.causal, reorder=reorder,
                       kv_tile=kv_tile, q4=rq, k4=rk, v4=rv, want_phat=True, scale_rule=0)
    assert not np.array_equal(ps, ref0["phat_scales"])


@pytest.mark.parametrize("kw", [
    dict(B=16, Hq=32, Hkv=8, N_kv=700, d=128, num_splits=5, kv_tile=64),   # fused decode kernel
    dict(B=2, Hq=8, Hkv=2, N_kv=1000, d=128, num_splits=4, kv_tile=128),   # split + merge kernels
])
def test_decode_noclip_matches_oracle(hf, kw):
    import torch
    print(f"[noclip decode] {kw}", flush=True)
    kw = dict(kw)
    C, kt = kw.pop("num_splits"), kw.pop("kv_tile")
    w = synth.decode(n_cal=128, **kw)
    s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref, rule=NOCLIP)
    npk = oracle.padded(w.N_kv)
    phat = hf.MX4(torch.zeros((w.B, w.Hq, 1, npk // 2), dtype=torch.uint8, device="cuda"),
                  torch.zeros((w.B, w.Hq, 1, npk // 32), dtype=torch.uint8, device="cuda"))
    out = hf.attn_fwd(None, mx4_to_dev(rk), v_to_dev(rv), B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=1,
                      N_kv=w.N_kv, d=w.d, causal=False, smooth=True, reorder=True,
                      q_f16=to_dev(w.q), s=to_dev(s_ref), num_splits=C, phat=phat, kv_tile=kt,
                      scale_rule=NOCLIP)
    _sync()
    ref = oracle.attn(w.B, w.Hq, w.Hkv, 1, w.N_kv, w.d, causal=False, reorder=1, num_splits=C,
                      kv_tile=kt, q4=rq, k4=rk, v4=rv, want_phat=True, scale_rule=NOCLIP)
    got = to_host(out).reshape(-1, w.d)
    n = len(got)
    check_attn(f"noclip decode {kw} splits={C} kv_tile={kt}", got, ref,
               valid_keys(np.arange(n), 1, w.N_kv, False),
               phat=(to_host(phat.codes).reshape(n, -1), to_host(phat.scales).reshape(n, -1)))


def test_append_noclip_matches_oracle(hf):
    """Appends (RoPE + Smooth-QK + 4-bit K rows, re-quantized V blocks) with the rule leave the
    cache that quantizing the whole post-RoPE sequence with the rule gives."""
    ts = [1, 30, 1, 33, 64, 2]
    w = synth.kv_append(B=2, Hkv=2, Hq=4, N=sum(ts), d=128, n_cal=64)
    w.v[0, 1, 10, :] = np.float16(1.75)  # blocks the default rule would saturate
    s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    cache = hf.empty_kv_cache(w.B, w.Hkv, 256, w.d)
    k_all, v_all = to_dev(w.k_raw), to_dev(w.v)
    cos, sin, inv = to_dev(w.cos), to_dev(w.sin), to_dev(inv_ref)
    pos = 0
    for t in ts:
        hf.kv_append(cache, k_all[:, :, pos:pos + t].contiguous(), v_all[:, :, pos:pos + t].contiguous(),
                     pos=pos, rope_cos=cos, rope_sin=sin, smooth=True, inv_s=inv, scale_rule=NOCLIP)
        pos += t
    _sync()
    k = oracle.rope_f16(np.ascontiguousarray(w.k_raw[:, :, :pos]), w.cos, w.sin)
    k4 = oracle.quantize_rows(np.ascontiguousarray(k), w.Hkv, inv_ref, NOCLIP)
    v4 = tile_v(oracle.quantize_v(np.ascontiguousarray(w.v[:, :, :pos]), NOCLIP))
    npad = k4[0].shape[2]
    assert codes_equal(to_host(cache.k4.codes)[:, :, :npad], k4[0]).all()
    assert np.array_equal(to_host(cache.k4.scales)[:, :, :npad], k4[1])
    assert codes_equal(to_host(cache.v4.codes)[:, :, :npad // 64], v4[0]).all()
    assert np.array_equal(to_host(cache.v4.scales)[:, :, :npad // 64], v4[1])
