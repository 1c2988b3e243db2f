"""GPU parity of the RTN control (per-token asymmetric INT3 / INT4 keys with an
fp16 scale and zero-point, V in fp16; the simpler baseline of the EdgeLLM-Nano
page) through the C ABI against the float64 oracle in oracle/rtn.py.

Bars: records bit-exact (both sides decide scale, zero-point and codes in
float64 from the same fp16 values); logits within the fp32 accumulation bound
(d + 4) * 2^-24 * sum_c |q_c| |k-hat_c| (times 2); attention outputs within
1e-3 max-abs, the bar of the PGKQ decode.  Decode parity runs on the oracle's
packed records so that it is independent of the encoder.
"""

import numpy as np
import pytest
import torch

from oracle import rtn
from synth import CONFIGS, make_inputs

from gpu_cases import k_tensor, q_tensor, to_dev, v_cache, value_capacity

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from compressed_cache_decode_pgkq_amd import _lib
    _lib.lib()


def _api():
    import compressed_cache_decode_pgkq_amd as api
    return api


_INPUTS = {}


def _inputs(name, **over):
    key = (name, tuple(sorted(over.items())))
    if key not in _INPUTS:
        cfg = CONFIGS[name].with_(**over)
        _INPUTS[key] = (cfg, make_inputs(cfg))
    return _INPUTS[key]


SMALL = {
    "d64_f32": ("nano_b64_t512", dict(n_seq=2)),
    "d128_f16": ("gqa_b16_t32k", dict(n_seq=2, n_tokens=1000)),
}


def _gpu_records(K, bits, cap, off=0, codes=None):
    api = _api()
    out = api.pgkq_rtn_encode(k_tensor(K), bits, codes=codes, capacity=cap, token_offset=off)
    torch.cuda.synchronize()
    return out


def _oracle_out(q, K, V, bits, scale=None):
    out, _ = rtn.decode_cache(q, K, V, bits, scale)
    return out


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("name", list(SMALL))
def test_rtn_encode_bit_exact(name, bits):
    base, over = SMALL[name]
    cfg, inp = _inputs(base, **over)
    K = inp["K"]
    cap = K.shape[2] + 5
    got = _gpu_records(K, bits, cap).cpu().numpy()
    want = rtn.pack_cache(K.astype(np.float64), bits, cap)
    assert got.shape == want.shape
    diff = np.flatnonzero(got != want)
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8]}"


@pytest.mark.parametrize("bits", [3, 4])
def test_rtn_encode_degenerate_keys(bits):
    """Constant keys (zero range -> scale 1), exact ramps, signed-zero extremes,
    ties at half steps and minima that fp16 rounds upward."""
    rng = np.random.default_rng(5)
    d = 64
    K = rng.standard_normal((1, 1, 64, d)).astype(np.float32)
    K[0, 0, 0] = 2.5                                    # constant
    K[0, 0, 1] = 0.0                                    # all zeros
    K[0, 0, 2] = -0.0                                   # all negative zeros
    K[0, 0, 3] = np.float32(-1.25) + np.float32(0.375) * (np.arange(d) % (1 << bits))  # ramp
    K[0, 0, 4] = 0.0
    K[0, 0, 4, :8] = [0.0, 0.5, 1.5, 2.5, 3.5, 14.5, 15.0, 7.5]  # ties at scale 1 (INT4)
    K[0, 0, 5] = np.linspace(0, 1, d, dtype=np.float32)
    K[0, 0, 5, 0] = np.float32(1e-3 + 2 ** -22)         # fp16(min) > min -> clamped code 0
    K[0, 0, 6, 7] = 3e4                                 # wide range
    K[0, 0, 7] = np.float32(1e-6) * rng.standard_normal(d).astype(np.float32)  # fp16 subnormals
    cap = 64
    got = _gpu_records(K, bits, cap).cpu().numpy()
    want = rtn.pack_cache(K.astype(np.float64), bits, cap)
    assert np.array_equal(got, want)


def test_rtn_encode_appends_at_token_offset():
    cfg, inp = _inputs("nano_b64_t512", n_seq=2)
    K = inp["K"]
    T = K.shape[2]
    cap = T + 16
    whole = _gpu_records(K, 4, cap).cpu().numpy()
    api = _api()
    codes = torch.zeros((K.shape[0], K.shape[1], cap * rtn.record_bytes(64, 4)), dtype=torch.uint8,
                        device="cuda:0")
    api.pgkq_rtn_encode(k_tensor(np.ascontiguousarray(K[:, :, :300])), 4, codes=codes, capacity=cap)
    api.pgkq_rtn_encode(k_tensor(np.ascontiguousarray(K[:, :, 300:])), 4, codes=codes, capacity=cap,
                        token_offset=300)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), whole)


def _check_decode(K, V, q, q_dtype, bits, n_splits=0, T=None, cap=None):
    """GPU decode on the oracle's packed records vs the oracle decode."""
    api = _api()
    T = K.shape[2] if T is None else T
    cap = value_capacity(T) if cap is None else cap
    K = K[:, :, :T].astype(np.float64)
    recs = rtn.pack_cache(K, bits, cap)
    out = api.pgkq_rtn_decode_attn(q_tensor(q, q_dtype), to_dev(recs), v_cache(V[:, :, :T], cap), bits,
                                   n_tokens=T, n_splits=n_splits)
    torch.cuda.synchronize()
    want = _oracle_out(q, K, V[:, :, :T], bits)
    err = float(np.abs(out.cpu().numpy() - want).max())
    assert err <= OUT_TOL, (bits, n_splits, T, err)
    return err


@pytest.mark.parametrize("n_splits", [1, 0, 7, 64])
@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("name", list(SMALL))
def test_rtn_decode_matches_oracle(name, bits, n_splits):
    base, over = SMALL[name]
    cfg, inp = _inputs(base, **over)
    _check_decode(inp["K"], inp["V"], inp["q"], cfg.q_dtype, bits, n_splits)


def _logit_bound(q, codes, scale, zp):
    khat = rtn.dequantize(codes, scale, zp)
    d = khat.shape[-1]
    return 2 * (d + 4) * 2.0 ** -24 * (np.abs(khat) @ np.abs(q)) + 1e-30


@pytest.mark.parametrize("bits", [3, 4])
def test_rtn_logits_within_fp32_bound(bits):
    api = _api()
    cfg, inp = _inputs("gqa_b16_t32k", n_seq=2, n_tokens=1000)
    K = inp["K"].astype(np.float64)
    q = inp["q"]
    n_seq, n_kv, T, d = K.shape
    recs = rtn.pack_cache(K, bits, T)
    lg = api.pgkq_rtn_logits(q_tensor(q, cfg.q_dtype), to_dev(recs), n_kv, T, bits).cpu().numpy()
    G = cfg.n_q // n_kv
    worst = 0.0
    for b in range(n_seq):
        for h in range(n_kv):
            codes, scale, zp = rtn.quantize(K[b, h], bits)
            for g in range(G):
                qq = q[b, h * G + g].astype(np.float64)
                want = rtn.logits(qq, codes, scale, zp)
                bound = _logit_bound(qq, codes, scale, zp)
                r = np.abs(lg[b, h * G + g] - want) / bound
                worst = max(worst, float(r.max()))
    assert worst <= 1.0, worst


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_rtn_group_sizes(group):
    cfg, inp = _inputs("gqa_b16_t32k", n_seq=1, n_tokens=600, n_q=8 * group)
    _check_decode(inp["K"], inp["V"], inp["q"], cfg.q_dtype, 4)


@pytest.mark.parametrize("T", [1, 63, 65, 777])
def test_rtn_ragged_lengths(T):
    cfg, inp = _inputs("gqa_b16_t32k", n_seq=1, n_tokens=1000)
    for ns in (0, 3, 9):
        _check_decode(inp["K"], inp["V"], inp["q"], cfg.q_dtype, 3, ns, T=T, cap=1024)


def test_rtn_long_stream_wave_partitions():
    """One sequence, few streams: the automatic split runs one partition per
    wavefront (the long-context launch shape)."""
    cfg, inp = _inputs("gqa_b1_t131k", n_tokens=6000)
    _check_decode(inp["K"], inp["V"], inp["q"], cfg.q_dtype, 4, 0)
    _check_decode(inp["K"], inp["V"], inp["q"], cfg.q_dtype, 4, 48)


def test_rtn_empty_cache_gives_zeros():
    api = _api()
    out = torch.full((1, 4, 64), 7.0, device="cuda:0")
    recs = torch.zeros((1, 4, 32 * 36), dtype=torch.uint8, device="cuda:0")
    V = torch.zeros((1, 4, 32, 64), dtype=torch.float16, device="cuda:0")
    q = torch.ones((1, 4, 64), dtype=torch.float32, device="cuda:0")
    api.pgkq_rtn_decode_attn(q, recs, V, 4, n_tokens=0, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


@pytest.mark.parametrize("mutation", ["swap_scale_zp", "code_plus_one", "drop_zero_point"])
def test_rtn_negative_controls_break_parity(mutation):
    """A planted mistake in the oracle's records (CPU side) must fail the logit
    bar: the comparison can tell."""
    api = _api()
    cfg, inp = _inputs("nano_b64_t512", n_seq=1)
    K = inp["K"][:, :2].astype(np.float64)
    q = inp["q"][:, :2]
    n_seq, n_kv, T, d = K.shape
    codes, scale, zp = rtn.quantize(K[0, 0], 4)
    if mutation == "swap_scale_zp":
        scale, zp = zp, scale
    elif mutation == "code_plus_one":
        codes = np.minimum(codes + 1, 15)
    else:
        zp = np.zeros_like(zp)
    recs = rtn.pack_cache(K, 4, T)
    rtn.pack_stream(codes, scale, zp, 4, T, 0, recs[0, 0])
    lg = api.pgkq_rtn_logits(q_tensor(q, cfg.q_dtype), to_dev(recs), n_kv, T, 4).cpu().numpy()
    good_codes, good_scale, good_zp = rtn.quantize(K[0, 0], 4)
    qq = q[0, 0].astype(np.float64)
    want = rtn.logits(qq, good_codes, good_scale, good_zp)
    r = np.abs(lg[0, 0] - want) / _logit_bound(qq, good_codes, good_scale, good_zp)
    assert r.max() > 1.0
    # the untouched stream still passes
    c1, s1, z1 = rtn.quantize(K[0, 1], 4)
    q1 = q[0, 1].astype(np.float64)
    r1 = np.abs(lg[0, 1] - rtn.logits(q1, c1, s1, z1)) / _logit_bound(q1, c1, s1, z1)
    assert r1.max() <= 1.0


def test_rtn_end_to_end_encode_then_decode():
    """GPU encode, then GPU decode of those records, against the oracle."""
    api = _api()
    cfg, inp = _inputs("gqa_b16_t32k", n_seq=2, n_tokens=1000)
    K, V, q = inp["K"], inp["V"], inp["q"]
    cap = value_capacity(K.shape[2])
    recs = _gpu_records(K, 3, cap)
    out = api.pgkq_rtn_decode_attn(q_tensor(q, cfg.q_dtype), recs, v_cache(V, cap), 3,
                                   n_tokens=K.shape[2])
    torch.cuda.synchronize()
    want = _oracle_out(q, K.astype(np.float64), V, 3)
    assert float(np.abs(out.cpu().numpy() - want).max()) <= OUT_TOL
