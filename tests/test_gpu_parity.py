"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Bars (stated for the method): codes bit-exact except decision-boundary cases
(classified in parity_util, fewer than 1e-5 of all code fields); logits within
2e-3 * ||q|| * ||k|| absolute; attention outputs within 1e-3 max-abs.
Decode parity runs on identical code buffers (packed by the oracle) so that an
encoder boundary case cannot leak into the decoder comparison.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attn, layout
from synth import CONFIGS

from gpu_cases import (OUT_TOL, Case, check_decode, code_counts, gpu_encode, k_tensor, lib_params,
                       q_tensor, to_dev, v_cache, value_capacity)
from parity_util import assert_code_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from compressed_cache_decode_pgkq_amd import _lib
    _lib.lib()  # the HIP library must be built; no fallback exists


def _api():
    import compressed_cache_decode_pgkq_amd as api
    return api


SMALL = {
    "nano_t128": (CONFIGS["nano_t128"], {}),
    "nano_b64_t512": (CONFIGS["nano_b64_t512"].with_(n_seq=3), {}),
    "nano_b64_t512_b4": (CONFIGS["nano_b64_t512_b4"].with_(n_seq=3), {}),
    "gqa_b16_t32k": (CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_tokens=1000), {}),
    "gqa_b16_t32k_encode": (CONFIGS["gqa_b16_t32k_encode"].with_(n_seq=2, n_tokens=700), {"reorder": True}),
    "gqa_b1_t131k": (CONFIGS["gqa_b1_t131k"].with_(n_tokens=3000), {}),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_encode_codes_match_oracle(name):
    cfg, kw = SMALL[name]
    case = Case(cfg, **kw)
    got = gpu_encode(case)
    counts = code_counts(case, got)
    print(name, counts)
    assert_code_parity(counts)
    if counts["mismatch"] == 0:
        assert np.array_equal(got, case.oracle_codes())


def test_encode_without_hadamard():
    case = Case(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=500), hadamard=False)
    counts = code_counts(case, gpu_encode(case))
    print(counts)
    assert_code_parity(counts)


def test_encode_appends_at_token_offset():
    api = _api()
    cfg = CONFIGS["nano_b64_t512"].with_(n_seq=2, n_tokens=200)
    case = Case(cfg, capacity=256)
    dev = case.dev_inputs()
    p = lib_params(case.p)
    codes = torch.zeros((2, cfg.n_kv, case.cap * layout.record_bytes(case.p)), dtype=torch.uint8,
                        device="cuda:0")
    # two appends: tokens [0, 77) then [77, 200)
    for t0, t1 in ((0, 77), (77, 200)):
        api.pgkq_encode(p, k_tensor(case.K[:, :, t0:t1]), dev["signs"], dev["perm"], dev["codebook"],
                        dev["S"], codes=codes, capacity=case.cap, token_offset=t0)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    assert np.array_equal(got, case.oracle_codes())


@pytest.mark.parametrize("name", ["nano_t128", "nano_b64_t512", "gqa_b16_t32k_encode"])
def test_calibrate_matches_oracle(name):
    api = _api()
    cfg, kw = SMALL[name]
    reorder = kw.get("reorder", False)
    case = Case(cfg, **kw)
    sumsq, perm, cb = api.pgkq_calibrate(lib_params(case.p), k_tensor(case.K), reorder=reorder)
    torch.cuda.synchronize()
    np.testing.assert_allclose(sumsq.cpu().numpy(), case.sumsq, rtol=1e-12)
    if reorder:
        assert np.array_equal(perm.cpu().numpy().view(np.uint16), case.perm.astype(np.uint16))
    got = cb.cpu().numpy()
    ulp = np.abs(np.spacing(case.cb.astype(np.float32)))
    fin = np.isfinite(case.cb)
    assert np.all(np.abs(got[fin] - case.cb[fin]) <= ulp[fin])
    assert np.all(np.isinf(got[~fin]))


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("n_splits", [1, 0, 7, 12, 256])  # 12, 256: one partition per wavefront
def test_decode_matches_oracle_on_identical_codes(name, n_splits):
    cfg, kw = SMALL[name]
    check_decode(Case(cfg, **kw), n_splits=n_splits)


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_decode_group_sizes(group):
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_kv=2, n_q=2 * group, n_tokens=600)
    check_decode(Case(cfg), n_splits=0)


@pytest.mark.parametrize("qd", ["f32", "f16", "bf16"])
def test_decode_query_dtypes(qd):
    case = Case(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=400))
    q = case.q.astype(np.float16).astype(np.float32) if qd == "f16" else case.q
    check_decode(case, q_override=q, q_dtype=qd)


@pytest.mark.parametrize("T", [1, 2, 63, 65, 257, 1000])
def test_decode_ragged_lengths(T):
    case = Case(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=1000), n_tokens=T, capacity=1024)
    check_decode(case, n_splits=0)
    check_decode(case, n_splits=3)
    check_decode(case, n_splits=9)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129, 200])
@pytest.mark.parametrize("variant", ["b3_qjl_g1", "b3_qjl_g2", "b4_g1"])
def test_decode_ragged_lengths_d64(T, variant):
    """head_dim 64: one workgroup per stream (two wavefronts, the query prepared
    in the scan; the first chunk requested before the preparation computes,
    ragged tiles masked at use) and split launches, on every tail shape."""
    base = CONFIGS["nano_t128"].with_(n_tokens=200)
    if variant == "b3_qjl_g2":
        base = base.with_(n_kv=12, n_q=24)
    elif variant == "b4_g1":
        base = base.with_(b_main=4, b_angle=3, qjl_m=0)
    # spare value slots hold NaN: a ragged tile's tail must be masked, not weighted by 0
    case = Case(base, n_tokens=T, capacity=224, v_spare=np.nan)
    check_decode(case, n_splits=0)
    check_decode(case, n_splits=1)
    check_decode(case, n_splits=3)


def test_decode_empty_cache_gives_zeros():
    api = _api()
    case = Case(CONFIGS["nano_t128"], n_tokens=0, capacity=128)
    dev = case.dev_inputs()
    out = torch.full((1, 24, 64), 7.0, device="cuda:0")
    api.pgkq_decode_attn(lib_params(case.p), q_tensor(case.q, "f32"),
                         torch.zeros((1, 24, 128 * 30), dtype=torch.uint8, device="cuda:0"),
                         dev["V"], dev["signs"], None, dev["codebook"], dev["S"], n_tokens=0, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


@pytest.mark.parametrize("hadamard", [True, False])
@pytest.mark.parametrize("qjl", [True, False])
def test_ablation_grid_hadamard_by_qjl(hadamard, qjl):
    """The 2x2 of the ablation paragraph (Hadamard on/off x QJL on/off, b_main = 3):
    every cell encodes bit-exactly and decodes within the bars."""
    cfg = CONFIGS["nano_b64_t512"].with_(n_seq=2, qjl_m=64 if qjl else 0)
    case = Case(cfg, hadamard=hadamard)
    counts = code_counts(case, gpu_encode(case))
    print(hadamard, qjl, counts)
    assert_code_parity(counts)
    check_decode(case)


def test_decode_without_hadamard():
    case = Case(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=500), hadamard=False)
    check_decode(case)


def test_end_to_end_calibrate_encode_decode():
    """GPU calibrate -> encode -> decode against oracle calibrate -> encode -> decode."""
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k_encode"].with_(n_seq=2, n_tokens=900)
    case = Case(cfg, reorder=True)
    p = lib_params(case.p)
    Kt = k_tensor(case.K)
    sumsq, perm, cb = api.pgkq_calibrate(p, Kt, reorder=True)
    dev = case.dev_inputs()
    codes = api.pgkq_encode(p, Kt, dev["signs"], perm, cb, dev["S"], capacity=case.cap)
    out = api.pgkq_decode_attn(p, q_tensor(case.q, cfg.q_dtype), codes, dev["V"], dev["signs"], perm,
                               cb, dev["S"], n_tokens=case.T)
    torch.cuda.synchronize()
    ref, _ = case.oracle_decode()
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    print("end-to-end max-abs", err)
    assert err <= OUT_TOL


def _fp16_check(cfg, n_splits=0, T=None, cap=None):
    from synth import make_inputs
    api = _api()
    inp = make_inputs(cfg)
    T = cfg.n_tokens if T is None else T
    cap = value_capacity(T) if cap is None else cap
    n_seq, n_kv = cfg.n_seq, cfg.n_kv
    d = cfg.head_dim
    K16 = inp["K"][:, :, :T].astype(np.float16)
    V16 = inp["V"][:, :, :T]
    Kp = np.zeros((n_seq, n_kv, cap, d), np.float16)
    Kp[:, :, :T] = K16
    out = api.pgkq_fp16_decode_attn(q_tensor(inp["q"], cfg.q_dtype), to_dev(Kp), v_cache(V16, cap),
                                    n_tokens=T, n_splits=n_splits)
    torch.cuda.synchronize()
    ref, _ = attn.fp16_attention(inp["q"], K16, V16)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    print("fp16 comparator max-abs", cfg.name, n_splits, T, err)
    assert err <= OUT_TOL


@pytest.mark.parametrize("n_splits", [0, 1, 5, 40])
@pytest.mark.parametrize("name", ["nano_b64_t512", "gqa_b16_t32k"])
def test_fp16_comparator_matches_oracle(name, n_splits):
    cfg, _ = SMALL[name]
    _fp16_check(cfg, n_splits)


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_fp16_comparator_group_sizes(d, group):
    base = CONFIGS["nano_b64_t512"] if d == 64 else CONFIGS["gqa_b16_t32k"]
    cfg = base.with_(n_seq=1, n_kv=4, n_q=4 * group, n_tokens=700)
    _fp16_check(cfg, 0)
    _fp16_check(cfg, 6)


@pytest.mark.parametrize("T", [1, 63, 65, 777])
def test_fp16_comparator_ragged(T):
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=1000)
    for ns in (0, 3, 9):
        _fp16_check(cfg, ns, T=T, cap=1024)


def test_fp16_comparator_long_stream_wave_partitions():
    _fp16_check(CONFIGS["gqa_b1_t131k"].with_(n_tokens=6000), 0)


# ------------------------------------------------------------------ negative controls
# A planted mistake lives in the oracle's data, on the CPU: the parity check
# must notice it (the broken-cache control of the LCDF harness, applied here).

def _decode_err(case, codes_np, tables=None, signs=None):
    api = _api()
    dev = case.dev_inputs()
    p = lib_params(case.p)
    out = api.pgkq_decode_attn(p, q_tensor(case.q, case.cfg.q_dtype), to_dev(case.oracle_codes()),
                               dev["V"], dev["signs"], dev["perm"], dev["codebook"], dev["S"],
                               n_tokens=case.T)
    torch.cuda.synchronize()
    n_seq, n_kv = case.K.shape[:2]
    fields = [[layout.unpack_stream(codes_np[b, h], case.p, case.cap, case.T) for h in range(n_kv)]
              for b in range(n_seq)]
    ref, _ = attn.decode_cache(case.q, fields, case.V, tables or case.tables, case.S,
                               case.signs if signs is None else signs, case.perm_arg, case.p)
    return float(np.max(np.abs(out.cpu().numpy() - ref)))


@pytest.mark.parametrize("mutation", ["radius_code", "sign_words", "rht_signs", "codebook"])
def test_negative_controls_break_parity(mutation):
    case = Case(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=256))
    good = case.oracle_codes()
    assert _decode_err(case, good) <= OUT_TOL
    bad = good.copy()
    tables = None
    signs = None
    cap = case.cap
    NC = layout.code_words(case.p)
    words = bad[0, 0, : layout.n_words(case.p) * 4 * cap].view(np.uint32).reshape(-1, cap)
    if mutation == "radius_code":
        # move the heaviest-weight token's first radius code by one level
        words[0, :] ^= 0x1
    elif mutation == "sign_words":
        words[NC:, :] = 0
    elif mutation == "rht_signs":
        signs = case.signs.copy()
        signs[0, :8] *= -1
    elif mutation == "codebook":
        tables = [(lv[::-1].copy(), th) for lv, th in case.tables]
    err = _decode_err(case, bad, tables=tables, signs=signs)
    print(mutation, err)
    assert err > OUT_TOL
