"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: 100 % identical Q/K/V codes and scales (deterministic quantizer; +0 and
-0 compare equal), >= 99.9 % identical P_hat codes and scale bytes counted over
the keys each row attends to (and the 32-key blocks holding them), output error
<= 1e-2 max and <= 1e-3 mean relative to each row's max |O_oracle|.  Inputs are the seeded
synthetic workloads (scaled-down shapes with the benchmark's structure, plus
ragged and degenerate cases).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import (ERR_MAX, ERR_MEAN, check_attn, codes_equal, mx4_to_dev, oracle_quant,
                        out_error, tile_v, to_dev, to_host, v_to_dev, valid_keys)

pytestmark = pytest.mark.gpu


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


# ---------------------------------------------------------------------------
# calibration + quantization
# ---------------------------------------------------------------------------

QUANT_CASES = [
    ("single_head", dict()),
    ("qwen3_8b", dict(B=1, Hq=8, Hkv=2, N=300, d=128, n_cal=200)),
    ("gemma2_9b", dict(B=1, Hq=4, Hkv=2, N=130, d=256, n_cal=96)),
    ("llama_batched", dict(B=2, Hq=4, Hkv=2, N=257, d=128)),
    ("qwen3_8b", dict(B=2, Hq=2, Hkv=1, N=33, d=64, n_cal=40)),
]


@pytest.mark.parametrize("name,kw", QUANT_CASES)
def test_calibrate_and_quantize_match_oracle(hf, name, kw):
    print(f"[quantize] {name} {kw}", flush=True)
    w = synth.WORKLOADS[name](**kw)
    if w.smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
        s, inv = hf.calibrate_smooth(to_dev(w.q_cal), to_dev(w.k_cal), w.alpha)
        assert np.array_equal(to_host(s), s_ref)
        assert np.array_equal(to_host(inv), inv_ref)
    else:
        s_ref = inv_ref = s = inv = None
    q4, k4, v4 = hf.quantize_qkv(to_dev(w.q), to_dev(w.k), to_dev(w.v), Hkv=w.Hkv,
                                 smooth=w.smooth, s=s, inv_s=inv)
    _sync()
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref)
    for got, ref in ((q4, rq), (k4, rk), (v4, tile_v(rv))):
        assert np.all(codes_equal(to_host(got.codes), ref[0]))
        assert np.array_equal(to_host(got.scales), ref[1])


@pytest.mark.parametrize("B,Hq,Hkv,N,d,alpha", [(1, 32, 8, 512, 128, 0.5), (2, 6, 2, 77, 96, 0.25),
                                                 (3, 4, 4, 300, 256, 0.5), (1, 8, 1, 5000, 64, 1.0)])
def test_calibrate_shapes(hf, B, Hq, Hkv, N, d, alpha):
    """Calibration maxima over batches, GQA groups, a channel count that is not a multiple of
    64 and more rows than one workgroup takes; zero channels give s = 1."""
    q = synth.tensor(101, B, Hq, N, d)
    k = synth.tensor(102, B, Hkv, N, d)
    q[:, :, :, 3] = 0          # zero in Q only
    k[:, :, :, 5] = 0          # zero in K only
    q[:, :, :, d - 1] = 0      # zero in both
    k[:, :, :, d - 1] = 0
    k[:, :, N - 1, 7] = np.float16(-300.0)  # the maximum on the last K row
    s, inv = hf.calibrate_smooth(to_dev(q), to_dev(k), alpha)
    s_ref, inv_ref = oracle.calibrate(q, k, alpha)
    assert np.array_equal(to_host(s), s_ref) and np.array_equal(to_host(inv), inv_ref)
    assert np.all(s_ref[:, [3, 5, d - 1]] == 1.0)


def test_quantize_edge_values(hf):
    """Zero blocks, subnormal binary16, saturating and tiny blocks."""
    import torch
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((1, 2, 64, 128)) * 3).astype(np.float16)
    x[0, 0, 0, :32] = 0                                   # all-zero block -> scale byte 0
    x[0, 0, 1, :32] = np.float16(2.0 ** -24)              # subnormal binary16 block
    x[0, 0, 2, :32] = np.float16(-0.0)
    x[0, 0, 3, 32:64] = np.float16(60000.0)               # large
    x[0, 1, 5, :] = np.float16(7.9)                        # clip [6, 8) * 2^e -> 6
    x[0, 1, 6, 64:96] = np.linspace(-1, 1, 32).astype(np.float16)
    s = np.ones((1, 128), dtype=np.float32)
    s[0, :32] = 2.0 ** -120                                # drives products subnormal in fp32
    inv = (1.0 / s).astype(np.float32)
    q4, k4, _ = hf.quantize_qkv(to_dev(x), to_dev(x[:, :1]), None, Hkv=1, smooth=True,
                                s=to_dev(s), inv_s=to_dev(inv))
    _sync()
    rq = oracle.quantize_rows(x, 1, s)
    rk = oracle.quantize_rows(x[:, :1], 1, inv)
    assert np.all(codes_equal(to_host(q4.codes), rq[0]))
    assert np.array_equal(to_host(q4.scales), rq[1])
    assert np.all(codes_equal(to_host(k4.codes), rk[0]))
    assert np.array_equal(to_host(k4.scales), rk[1])
    v = x.copy()
    _, _, v4 = hf.quantize_qkv(None, None, to_dev(v), Hkv=2)
    _sync()
    rv = tile_v(oracle.quantize_v(v))
    assert np.all(codes_equal(to_host(v4.codes), rv[0]))
    assert np.array_equal(to_host(v4.scales), rv[1])


@pytest.mark.parametrize("B,H,N,d", [(2, 3, 200, 128), (1, 2, 64, 64), (1, 1, 300, 256)])
def test_v_layout_conversion(hf, B, H, N, d):
    """hifa4_v_layout against the oracle's canonical V_hat: canonical -> tiled equals the
    test-side re-arrangement (tile_v) byte for byte, tiled -> canonical gives the oracle's
    bytes back, and the quantize pass's own tiled V_hat converts to the oracle's canonical
    V_hat (codes with +-0 equal, scales identical)."""
    print(f"[v_layout] B={B} H={H} N={N} d={d}", flush=True)
    rng = np.random.default_rng(N + d)
    v = (rng.standard_normal((B, H, N, d)) * 2).astype(np.float16)
    canon = oracle.quantize_v(v)
    c4 = hf.MX4(to_dev(canon[0]), to_dev(canon[1]))
    t4 = hf.v_layout(c4, to_tiled=True)
    _sync()
    ref_t = tile_v(canon)
    assert np.array_equal(to_host(t4.codes), ref_t[0])
    assert np.array_equal(to_host(t4.scales), ref_t[1])
    back = hf.v_layout(t4, to_tiled=False)
    _sync()
    assert np.array_equal(to_host(back.codes), canon[0])
    assert np.array_equal(to_host(back.scales), canon[1])
    _, _, v4 = hf.quantize_qkv(None, None, to_dev(v), Hkv=H)
    cq = hf.v_layout(v4, to_tiled=False)
    _sync()
    assert np.all(codes_equal(to_host(cq.codes), canon[0]))
    assert np.array_equal(to_host(cq.scales), canon[1])


# ---------------------------------------------------------------------------
# attention forward
# ---------------------------------------------------------------------------

ATTN_CASES = [
    # name, overrides, reorder, kv_tile
    ("single_head", dict(), 1, 64),
    ("single_head", dict(), 0, 64),
    ("single_head", dict(), 1, 128),
    ("qwen3_8b", dict(B=1, Hq=4, Hkv=1, N=512, d=128, n_cal=128), 1, 64),
    ("qwen3_8b", dict(B=1, Hq=4, Hkv=1, N=512, d=128, n_cal=128), 0, 64),
    ("qwen3_8b", dict(B=1, Hq=4, Hkv=1, N=512, d=128, n_cal=128), 1, 128),
    ("qwen3_8b", dict(B=1, Hq=4, Hkv=1, N=512, d=128, n_cal=128), 0, 128),
    ("qwen3_8b", dict(B=1, Hq=2, Hkv=2, N=200, N_kv=330, d=128, n_cal=64), 1, 64),  # ragged
    ("qwen3_8b", dict(B=1, Hq=2, Hkv=2, N=200, N_kv=330, d=128, n_cal=64), 1, 128),
    ("gemma2_9b", dict(B=1, Hq=2, Hkv=1, N=384, d=256, n_cal=128), 1, 64),
    ("gemma2_9b", dict(B=1, Hq=2, Hkv=1, N=384, d=256, n_cal=128), 1, 128),
    ("gemma2_9b", dict(B=1, Hq=4, Hkv=2, N=200, N_kv=330, d=256, n_cal=64), 0, 128),  # ragged
    ("llama_batched", dict(B=2, Hq=4, Hkv=2, N=257, d=128), 1, 64),
    ("llama_batched", dict(B=2, Hq=4, Hkv=2, N=257, d=128), 0, 128),
    ("qwen3_8b", dict(B=1, Hq=8, Hkv=1, N=130, d=64, n_cal=64), 1, 64),
    ("qwen3_8b", dict(B=1, Hq=8, Hkv=1, N=130, d=64, n_cal=64), 0, 128),
    # non-causal with N_q != N_kv: fewer queries than keys, and more (ragged tails on both)
    ("qwen3_8b", dict(B=1, Hq=4, Hkv=2, N=200, N_kv=330, d=128, n_cal=64, causal=False), 1, 128),
    ("llama_batched", dict(B=2, Hq=4, Hkv=1, N=300, N_kv=100, d=64, causal=False), 0, 64),
    ("gemma2_9b", dict(B=1, Hq=2, Hkv=2, N=97, N_kv=161, d=256, n_cal=64, causal=False), 1, 128),
]


def _prefill_case(hf, w, reorder, dump=True, kv_tile=64):
    import torch
    if w.smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    else:
        s_ref = inv_ref = None
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref)
    q4, k4, v4 = mx4_to_dev(rq), mx4_to_dev(rk), v_to_dev(rv)
    phat = None
    npk = oracle.padded(w.N_kv)
    if dump:
        phat = hf.MX4(torch.zeros((w.B, w.Hq, w.N_q, npk // 2), dtype=torch.uint8, device="cuda"),
                      torch.zeros((w.B, w.Hq, w.N_q, npk // 32), dtype=torch.uint8, device="cuda"))
    out = hf.attn_fwd(q4, k4, v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=w.N_q, N_kv=w.N_kv, d=w.d,
                      causal=w.causal, smooth=w.smooth, reorder=reorder, phat=phat,
                      kv_tile=kv_tile)
    _sync()
    ref = oracle.attn(w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, causal=w.causal, reorder=reorder,
                      kv_tile=kv_tile, q4=rq, k4=rk, v4=rv, want_phat=dump)
    return out, phat, ref


@pytest.mark.parametrize("name,kw,reorder,kv_tile", ATTN_CASES)
def test_prefill_matches_oracle(hf, name, kw, reorder, kv_tile):
    print(f"[prefill] {name} {kw} reorder={reorder} kv_tile={kv_tile}", flush=True)
    kw = dict(kw)
    causal = kw.pop("causal", None)
    w = synth.WORKLOADS[name](**kw)
    if name == "single_head":
        w.causal = False
    if causal is not None:
        w.causal = causal
    out, phat, ref = _prefill_case(hf, w, reorder, kv_tile=kv_tile)
    got = to_host(out).reshape(-1, w.d)
    n = len(got)
    nv = valid_keys(np.arange(n), w.N_q, w.N_kv, w.causal)
    check_attn(f"prefill {name} {kw} causal={w.causal} reorder={reorder} kv_tile={kv_tile}", got,
               ref, nv, phat=(to_host(phat.codes).reshape(n, -1), to_host(phat.scales).reshape(n, -1)))


RAW_Q_CASES = [
    # name, overrides, reorder, kv_tile (query rows per KV head > 32: the prefill kernel)
    ("qwen3_8b", dict(B=1, Hq=8, Hkv=2, N=300, d=128, n_cal=96), 1, 128),
    ("qwen3_8b", dict(B=2, Hq=4, Hkv=2, N=77, N_kv=200, d=128, n_cal=64), 0, 64),  # ragged
    ("gemma2_9b", dict(B=1, Hq=2, Hkv=1, N=160, d=256, n_cal=64), 1, 64),
    ("gemma2_9b", dict(B=1, Hq=2, Hkv=1, N=160, d=256, n_cal=64), 1, 128),
    ("qwen3_8b", dict(B=1, Hq=8, Hkv=1, N=130, d=64, n_cal=64), 1, 128),
    ("llama_batched", dict(B=2, Hq=4, Hkv=2, N=100, d=128), 1, 128),            # no Smooth-QK
]


@pytest.mark.parametrize("name,kw,reorder,kv_tile", RAW_Q_CASES)
def test_prefill_raw_query_matches_oracle(hf, name, kw, reorder, kv_tile):
    """Binary16 Q given to the prefill kernel, smoothed and quantized there: the same
    P_hat and output as the oracle on the oracle's own Q_hat."""
    import torch
    print(f"[prefill raw q] {name} {kw} reorder={reorder} kv_tile={kv_tile}", flush=True)
    w = synth.WORKLOADS[name](**kw)
    if w.smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    else:
        s_ref = inv_ref = None
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref)
    k4, v4 = mx4_to_dev(rk), v_to_dev(rv)
    npk = oracle.padded(w.N_kv)
    phat = hf.MX4(torch.zeros((w.B, w.Hq, w.N_q, npk // 2), dtype=torch.uint8, device="cuda"),
                  torch.zeros((w.B, w.Hq, w.N_q, npk // 32), dtype=torch.uint8, device="cuda"))
    out = hf.attn_fwd(None, k4, v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=w.N_q, N_kv=w.N_kv, d=w.d,
                      causal=w.causal, smooth=w.smooth, reorder=reorder, phat=phat,
                      kv_tile=kv_tile, q_f16=to_dev(w.q),
                      s=None if s_ref is None else to_dev(s_ref))
    _sync()
    ref = oracle.attn(w.B, w.Hq, w.Hkv, w.N_q, w.N_kv, w.d, causal=w.causal, reorder=reorder,
                      kv_tile=kv_tile, q4=rq, k4=rk, v4=rv, want_phat=True)
    got = to_host(out).reshape(-1, w.d)
    n = len(got)
    check_attn(f"prefill raw q {name} {kw} reorder={reorder} kv_tile={kv_tile}", got, ref,
               valid_keys(np.arange(n), w.N_q, w.N_kv, w.causal),
               phat=(to_host(phat.codes).reshape(n, -1), to_host(phat.scales).reshape(n, -1)))
    # the same launch with pre-quantized Q gives the same output bit for bit
    q4d, _, _ = hf.quantize_qkv(to_dev(w.q), None, None, Hkv=w.Hkv, smooth=w.smooth,
                                s=None if s_ref is None else to_dev(s_ref))
    out2 = hf.attn_fwd(q4d, k4, v4, B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=w.N_q, N_kv=w.N_kv, d=w.d,
                       causal=w.causal, smooth=w.smooth, reorder=reorder, kv_tile=kv_tile)
    _sync()
    assert np.array_equal(to_host(out2).view(np.uint16), to_host(out).view(np.uint16))


def test_prefill_deterministic(hf):
    w = synth.qwen3_8b(B=1, Hq=4, Hkv=1, N=256, d=128, n_cal=64)
    a, _, _ = _prefill_case(hf, w, 1, dump=False)
    b, _, _ = _prefill_case(hf, w, 1, dump=False)
    assert np.array_equal(to_host(a).view(np.uint16), to_host(b).view(np.uint16))


def _degenerate_scores(w, kind, seed):
    """Make a workload's score distribution degenerate (the binary16 tensors only; the
    calibration batch is left as it is).
    flat:  Q = 0, so every score is 0, every P is 1 and every P_hat block has the same
           exponent (P_hat = 1 exactly, the row sum is the number of valid keys).
    spiky: the K rows of about 5 % of the keys are scaled by 100, so those keys' scores
           exceed the rest of their row by hundreds of log2 units: most P underflow below
           2^-126 (taken as 0), P_hat block exponents reach their clamp at -127, the running
           max jumps by large steps and alpha underflows to 0."""
    if kind == "flat":
        w.q = np.zeros_like(w.q)
    else:
        rng = np.random.default_rng(seed)
        k = w.k.astype(np.float32)
        k[:, :, rng.random(k.shape[2]) < 0.05, :] *= 100.0
        assert np.abs(k).max() < 60000.0
        w.k = k.astype(np.float16)
    return w


@pytest.mark.parametrize("kind", ["flat", "spiky"])
@pytest.mark.parametrize("reorder,kv_tile,d", [(1, 64, 128), (1, 128, 128), (0, 128, 128), (1, 128, 256)])
def test_prefill_degenerate_scores(hf, kind, reorder, kv_tile, d):
    """Prefill on degenerate score distributions (causal, ragged): every P_hat code and
    scale against the oracle, output within the bars."""
    print(f"[degenerate prefill] {kind} reorder={reorder} kv_tile={kv_tile} d={d}", flush=True)
    w = _degenerate_scores(synth.qwen3_8b(B=1, Hq=4, Hkv=2, N=300, N_kv=333, d=d, n_cal=64), kind, 3)
    out, phat, ref = _prefill_case(hf, w, reorder, kv_tile=kv_tile)
    got = to_host(out).reshape(-1, w.d)
    n = len(got)
    check_attn(f"degenerate {kind} prefill reorder={reorder} kv_tile={kv_tile} d={d}", got, ref,
               valid_keys(np.arange(n), w.N_q, w.N_kv, w.causal),
               phat=(to_host(phat.codes).reshape(n, -1), to_host(phat.scales).reshape(n, -1)))


@pytest.mark.parametrize("kind", ["flat", "spiky"])
@pytest.mark.parametrize("B,Hkv,C", [(1, 2, 24), (16, 8, 5)])
def test_decode_degenerate_scores(hf, kind, B, Hkv, C):
    """Split-KV decode (split and merge kernels at B = 1, the fused kernel at 128 KV heads)
    on degenerate score distributions, binary16 query quantized in the kernel."""
    import torch
    print(f"[degenerate decode] {kind} B={B} Hkv={Hkv} splits={C}", flush=True)
    w = _degenerate_scores(synth.decode(B=B, Hq=4 * Hkv, Hkv=Hkv, N_kv=1500, d=128, n_cal=64), kind, 4)
    s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rk = oracle.quantize_rows(w.k, w.Hkv, inv_ref)
    rv = oracle.quantize_v(w.v)
    rq = oracle.quantize_rows(w.q, w.Hkv, s_ref)
    npk = oracle.padded(w.N_kv)
    phat = hf.MX4(torch.zeros((w.B, w.Hq, 1, npk // 2), dtype=torch.uint8, device="cuda"),
                  torch.zeros((w.B, w.Hq, 1, npk // 32), dtype=torch.uint8, device="cuda"))
    out = hf.attn_fwd(None, mx4_to_dev(rk), v_to_dev(rv), B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=1,
                      N_kv=w.N_kv, d=w.d, causal=False, smooth=True, reorder=True,
                      q_f16=to_dev(w.q), s=to_dev(s_ref), num_splits=C, phat=phat, kv_tile=64)
    _sync()
    ref = oracle.attn(w.B, w.Hq, w.Hkv, 1, w.N_kv, w.d, causal=False, reorder=1, num_splits=C,
                      kv_tile=64, q4=rq, k4=rk, v4=rv, want_phat=True)
    got = to_host(out).reshape(-1, w.d)
    n = len(got)
    check_attn(f"degenerate {kind} decode B={B} Hkv={Hkv} splits={C}", got, ref,
               valid_keys(np.arange(n), 1, w.N_kv, False),
               phat=(to_host(phat.codes).reshape(n, -1), to_host(phat.scales).reshape(n, -1)))


def test_v_ones_gives_one(hf):
    """P-Reordering on the GPU: V = 1 yields output 1 up to the FP16 normalizer."""
    import torch
    w = synth.qwen3_8b(B=1, Hq=2, Hkv=1, N=256, d=128, n_cal=64)
    w.v = np.ones_like(w.v)
    out, _, _ = _prefill_case(hf, w, 1, dump=False)
    o = to_host(out).astype(np.float32)
    assert np.abs(o - 1).max() <= 4 * 2.0 ** -11 + 2.0 ** -11


DECODE_CASES = [
    dict(B=2, Hq=8, Hkv=2, N_kv=1000, d=128, num_splits=4, kv_tile=64),
    dict(B=2, Hq=8, Hkv=2, N_kv=1000, d=128, num_splits=4, kv_tile=128),
    dict(B=3, Hq=32, Hkv=8, N_kv=512, d=128, num_splits=1, kv_tile=64),
    dict(B=2, Hq=4, Hkv=4, N_kv=700, d=64, num_splits=3, kv_tile=64),
    dict(B=1, Hq=8, Hkv=1, N_kv=4096, d=256, num_splits=16, kv_tile=64),
    # at least 128 (b, g) pairs: the fused decode kernel (partials merged in LDS)
    dict(B=16, Hq=32, Hkv=8, N_kv=700, d=128, num_splits=5, kv_tile=64),
    dict(B=32, Hq=16, Hkv=4, N_kv=520, d=256, num_splits=3, kv_tile=64),
    dict(B=64, Hq=8, Hkv=2, N_kv=300, d=64, num_splits=2, kv_tile=128),
    # one sequence, many chunks: the merge kernel over more chunks than channels
    dict(B=1, Hq=4, Hkv=1, N_kv=8192, d=64, num_splits=128, kv_tile=64),
    dict(B=1, Hq=8, Hkv=2, N_kv=16384, d=128, num_splits=64, kv_tile=128),
    # more chunks than the merge stages at once (128): a second, ragged batch, and
    # chunks past the last tile (256 tiles dealt 2 per chunk to 200 chunks)
    dict(B=1, Hq=4, Hkv=1, N_kv=16384, d=128, num_splits=200, kv_tile=64),
]


@pytest.mark.parametrize("kw", DECODE_CASES)
def test_decode_split_matches_oracle(hf, kw):
    import torch
    print(f"[decode] {kw}", flush=True)
    kw = dict(kw)
    C = kw.pop("num_splits")
    kt = kw.pop("kv_tile")
    w = synth.decode(n_cal=128, **kw)
    s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rk = oracle.quantize_rows(w.k, w.Hkv, inv_ref)
    rv = oracle.quantize_v(w.v)
    rq = oracle.quantize_rows(w.q, w.Hkv, s_ref)
    npk = oracle.padded(w.N_kv)
    phat = hf.MX4(torch.zeros((w.B, w.Hq, 1, npk // 2), dtype=torch.uint8, device="cuda"),
                  torch.zeros((w.B, w.Hq, 1, npk // 32), dtype=torch.uint8, device="cuda"))
    out = hf.attn_fwd(None, mx4_to_dev(rk), v_to_dev(rv), B=w.B, Hq=w.Hq, Hkv=w.Hkv, N_q=1,
                      N_kv=w.N_kv, d=w.d, causal=False, smooth=True, reorder=True,
                      q_f16=to_dev(w.q), s=to_dev(s_ref), num_splits=C, phat=phat, kv_tile=kt)
    _sync()
    ref = oracle.attn(w.B, w.Hq, w.Hkv, 1, w.N_kv, w.d, causal=False, reorder=1, num_splits=C,
                      kv_tile=kt, q4=rq, k4=rk, v4=rv, want_phat=True)
    got = to_host(out).reshape(-1, w.d)
    n = len(got)
    check_attn(f"decode {kw} splits={C} kv_tile={kt}", got, ref,
               valid_keys(np.arange(n), 1, w.N_kv, False),
               phat=(to_host(phat.codes).reshape(n, -1), to_host(phat.scales).reshape(n, -1)))


def test_split_path_with_prequantized_q_and_causal(hf):
    """Split-KV with pre-quantized Q, several query rows (G * N_q <= 32) and a causal mask."""
    w = synth.qwen3_8b(B=2, Hq=8, Hkv=2, N=4, N_kv=700, d=128, n_cal=64)
    s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref)
    out = hf.attn_fwd(mx4_to_dev(rq), mx4_to_dev(rk), v_to_dev(rv), B=2, Hq=8, Hkv=2, N_q=4,
                      N_kv=700, d=128, causal=True, smooth=True, reorder=False, num_splits=5)
    _sync()
    ref = oracle.attn(2, 8, 2, 4, 700, 128, causal=True, reorder=0, num_splits=5, q4=rq, k4=rk,
                      v4=rv)
    emax, emean = out_error(to_host(out).reshape(-1, 128), ref["out"].view(np.float16))
    assert emax <= ERR_MAX and emean <= ERR_MEAN


# Split-KV with 128-key tiles (the split kernel and the merge kernel, fewer than 128 KV heads in
# the batch): reorder off, a causal mask over several query rows, d = 64, Smooth-QK off, 16 and
# 24 query columns, no merge (one chunk), one tile per chunk, and merges of 64 chunks (one batch
# of loads) and 65 (the batched path).
# (B, Hq, Hkv, N_q, N_kv, d, causal, reorder, raw_q, smooth, num_splits)
SPLIT_CASES = [
    (2, 8, 2, 1, 1000, 128, False, True, True, True, 4),
    (2, 8, 2, 1, 1000, 128, False, False, True, True, 4),
    (1, 4, 2, 1, 700, 64, False, True, True, True, 3),
    (2, 8, 2, 4, 700, 128, True, False, False, True, 5),
    (2, 8, 2, 4, 700, 128, True, True, False, True, 5),
    (1, 16, 2, 2, 515, 64, True, True, True, False, 2),
    (1, 16, 2, 3, 515, 128, False, True, True, True, 2),
    (1, 8, 2, 1, 128, 128, False, True, True, True, 1),
    (3, 4, 1, 1, 4096, 128, False, True, True, True, 1),
    (1, 4, 1, 1, 8192, 64, False, False, True, True, 64),
    (1, 4, 1, 1, 8320, 128, False, True, True, True, 65),
]


@pytest.mark.parametrize("B,Hq,Hkv,N_q,N_kv,d,causal,reorder,raw_q,smooth,C", SPLIT_CASES)
def test_split_cases_match_oracle(hf, B, Hq, Hkv, N_q, N_kv, d, causal, reorder, raw_q, smooth, C):
    import torch
    print(f"[split] B={B} Hq={Hq} Hkv={Hkv} N_q={N_q} N_kv={N_kv} d={d} causal={causal} "
          f"reorder={reorder} raw_q={raw_q} smooth={smooth} C={C}", flush=True)
    w = synth.qwen3_8b(B=B, Hq=Hq, Hkv=Hkv, N=N_q, N_kv=N_kv, d=d, n_cal=64)
    s_ref = inv_ref = None
    if smooth:
        s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref)
    npk = oracle.padded(N_kv)
    phat = hf.MX4(torch.zeros((B, Hq, N_q, npk // 2), dtype=torch.uint8, device="cuda"),
                  torch.zeros((B, Hq, N_q, npk // 32), dtype=torch.uint8, device="cuda"))
    qarg = dict(q_f16=to_dev(w.q), s=to_dev(s_ref) if smooth else None) if raw_q else {}
    out = hf.attn_fwd(None if raw_q else mx4_to_dev(rq), mx4_to_dev(rk), v_to_dev(rv), B=B, Hq=Hq,
                      Hkv=Hkv, N_q=N_q, N_kv=N_kv, d=d, causal=causal, smooth=smooth,
                      reorder=reorder, num_splits=C, phat=phat, kv_tile=128, **qarg)
    _sync()
    ref = oracle.attn(B, Hq, Hkv, N_q, N_kv, d, causal=causal, reorder=int(reorder), num_splits=C,
                      kv_tile=128, q4=rq, k4=rk, v4=rv, want_phat=True)
    got = to_host(out).reshape(-1, d)
    n = len(got)
    check_attn(f"split B={B} Hq={Hq} Hkv={Hkv} N_q={N_q} N_kv={N_kv} d={d} causal={causal} "
               f"reorder={reorder} raw_q={raw_q} smooth={smooth} C={C}", got, ref,
               valid_keys(np.arange(n), N_q, N_kv, causal),
               phat=(to_host(phat.codes).reshape(n, -1), to_host(phat.scales).reshape(n, -1)))


def test_empty_and_single_key(hf):
    import torch
    w = synth.qwen3_8b(B=1, Hq=2, Hkv=1, N=3, N_kv=1, d=128, n_cal=32)
    rq, rk, rv = oracle_quant(w)
    out = hf.attn_fwd(mx4_to_dev(rq), mx4_to_dev(rk), v_to_dev(rv), B=1, Hq=2, Hkv=1, N_q=3,
                      N_kv=1, d=128, causal=False, smooth=False, reorder=True)
    _sync()
    ref = oracle.attn(1, 2, 1, 3, 1, 128, causal=False, reorder=1, q4=rq, k4=rk, v4=rv)
    assert np.array_equal(to_host(out).reshape(-1, 128).view(np.uint16), ref["out"])
    # N_q = 0: a successful no-op
    empty = torch.empty((1, 2, 0, 128), dtype=torch.float16, device="cuda")
    hf.attn_fwd(mx4_to_dev(rq), mx4_to_dev(rk), v_to_dev(rv), B=1, Hq=2, Hkv=1, N_q=0,
                N_kv=1, d=128, causal=False, smooth=False, reorder=True, out=empty)
    _sync()


def test_maximum_kv_length(hf):
    """N_kv = 32768, the largest length the FP16 normalizer allows (l <= 1.5 N_kv < 65504):
    causal prefill over the whole length on sampled rows (the last row attends to every key)
    and a split-KV decode step over it."""
    import torch
    n = hf.MAX_NKV
    w = synth.qwen3_8b(B=1, Hq=2, Hkv=1, N=n, d=128, n_cal=128)
    print(f"[max N_kv] N={n}", flush=True)
    s_ref, inv_ref = oracle.calibrate(w.q_cal, w.k_cal, w.alpha)
    rq, rk, rv = oracle_quant(w, s_ref, inv_ref)
    k4, v4 = mx4_to_dev(rk), v_to_dev(rv)
    out = hf.attn_fwd(mx4_to_dev(rq), k4, v4, B=1, Hq=2, Hkv=1, N_q=n, N_kv=n, d=128,
                      causal=True, smooth=True, reorder=True, kv_tile=128)
    _sync()
    rng = np.random.default_rng(32768)
    rows = np.unique(np.concatenate([rng.choice(2 * n, 40, replace=False), [n - 1, 2 * n - 1]]))
    ref = oracle.attn(1, 2, 1, n, n, 128, causal=True, reorder=1, kv_tile=128, q4=rq, k4=rk,
                      v4=rv, rows=rows.astype(np.int64))
    idx = torch.from_numpy(rows).cuda()
    emax, emean = out_error(to_host(out.reshape(-1, 128)[idx]), ref["out"].view(np.float16))
    print(f"  prefill rows {len(rows)}: err max {emax:.2e} mean {emean:.2e}", flush=True)
    assert emax <= ERR_MAX and emean <= ERR_MEAN
    # decode: one query per head against all 32768 keys, 16 splits
    q1 = np.ascontiguousarray(w.q[:, :, -1:])
    rq1 = oracle.quantize_rows(q1, 1, s_ref)
    out1 = hf.attn_fwd(None, k4, v4, B=1, Hq=2, Hkv=1, N_q=1, N_kv=n, d=128, causal=False,
                       smooth=True, reorder=True, q_f16=to_dev(q1), s=to_dev(s_ref),
                       num_splits=16)
    _sync()
    ref1 = oracle.attn(1, 2, 1, 1, n, 128, causal=False, reorder=1, num_splits=16, kv_tile=64,
                       q4=rq1, k4=rk, v4=rv)
    emax, emean = out_error(to_host(out1).reshape(-1, 128), ref1["out"].view(np.float16))
    print(f"  decode: err max {emax:.2e} mean {emean:.2e}", flush=True)
    assert emax <= ERR_MAX and emean <= ERR_MEAN
