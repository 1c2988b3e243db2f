"""Parity at the measured workloads' full sizes, in the launch configuration the
benchmark times: the GPU runs the whole cache, the oracle checks sampled
streams one by one (its codes for those streams are written into the GPU code
buffer so that decode parity runs on identical codes)."""

import numpy as np
import pytest
import torch

from oracle import attn, calibrate, codebook, encode, layout
from synth import CONFIGS, make_inputs

from gpu_cases import k_tensor, lib_params, params_of, q_tensor, to_dev, untile_values, v_cache
from parity_util import assert_code_parity, classify, codebook_array, merge_counts

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _api():
    import compressed_cache_decode_pgkq_amd as api
    return api


def _oracle_tables(K, cfg, reorder):
    n_seq, n_kv, T, d = K.shape
    c, t = codebook.lloyd_max_beta(d, cfg.b_main)
    tables, perms, sums = [], [], []
    for h in range(n_kv):
        ss = np.zeros(d)
        for b in range(n_seq):
            ss += calibrate.channel_sumsq(K[b, h])
        sums.append(ss)
        tables.append(codebook.scaled_table(c, t, calibrate.head_scale(ss, n_seq * T), d))
        perms.append(calibrate.reorder_perm(ss) if reorder else None)
    return tables, perms, np.stack(sums)


def _run_full(cfg, samples, n_splits):
    api = _api()
    p = params_of(cfg)
    lp = lib_params(p)
    inp = make_inputs(cfg)
    K, V, q, signs, S = inp["K"], inp["V"], inp["q"], inp["signs"], inp["S"]
    cap = cfg.n_tokens
    tables, _, _ = _oracle_tables(K, cfg, reorder=False)
    cb = codebook_array(tables)
    dsigns, dcb, dS = to_dev(signs), to_dev(cb), to_dev(S)
    Kt = k_tensor(K)
    codes = api.pgkq_encode(lp, Kt, dsigns, None, dcb, dS, capacity=cap)
    torch.cuda.synchronize()
    del Kt
    counts = {}
    for (b, h) in samples:
        f = encode.encode_keys(K[b, h], signs[h], None, tables[h][0], tables[h][1], S[h], p)
        got = layout.unpack_stream(codes[b, h].cpu().numpy(), p, cap, cfg.n_tokens)
        merge_counts(counts, classify(f, got, tables[h][1], S[h], p))
        codes[b, h] = torch.from_numpy(layout.pack_stream(f, p, cap)).to(codes.device)
        inp.setdefault("fields", {})[(b, h)] = f
    print(cfg.name, "encode", counts)
    assert_code_parity(counts)
    out = api.pgkq_decode_attn(lp, q_tensor(q, cfg.q_dtype), codes, v_cache(V, cap), dsigns, None, dcb,
                               dS, n_splits=n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = cfg.n_q // cfg.n_kv
    worst = 0.0
    for (b, h) in samples:
        f = inp["fields"][(b, h)]
        for g in range(G):
            hq = h * G + g
            s = attn.analytic_logits(q[b, hq], f, tables[h][0], S[h], signs[h], None, p)
            ref = attn.attend(s, V[b, h], 1.0 / np.sqrt(cfg.head_dim))
            worst = max(worst, float(np.max(np.abs(out[b, hq] - ref))))
    print(cfg.name, "decode max-abs", worst)
    assert worst <= OUT_TOL
    assert np.all(np.isfinite(out))


def test_c3_full_size_sampled():
    _run_full(CONFIGS["gqa_b16_t32k"], [(0, 0), (7, 3), (15, 7)], n_splits=CONFIGS["gqa_b16_t32k"].n_splits)


def test_c5_full_size_sampled():
    _run_full(CONFIGS["gqa_b1_t131k"], [(0, 0), (0, 5)], n_splits=CONFIGS["gqa_b1_t131k"].n_splits)


@pytest.mark.parametrize("name", ["nano_b64_t512", "nano_b64_t512_b4"])
def test_c2_full_size_every_stream(name):
    cfg = CONFIGS[name]
    n_streams = [(b, h) for b in range(cfg.n_seq) for h in range(cfg.n_kv)]
    _run_full(cfg, n_streams[:: 97] + [n_streams[-1]], n_splits=0)


def test_c4_full_size_calibrate_and_encode_sampled():
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k_encode"]
    p = params_of(cfg)
    lp = lib_params(p)
    inp = make_inputs(cfg, with_values=False)
    K, signs, S = inp["K"], inp["signs"], inp["S"]
    tables, perms, sums = _oracle_tables(K, cfg, reorder=True)
    Kt = k_tensor(K)
    sumsq, perm, cb = api.pgkq_calibrate(lp, Kt, reorder=True)
    codes = api.pgkq_encode(lp, Kt, to_dev(signs), perm, cb, to_dev(S), capacity=cfg.n_tokens)
    torch.cuda.synchronize()
    np.testing.assert_allclose(sumsq.cpu().numpy(), sums, rtol=1e-12)
    gperm = perm.cpu().numpy().view(np.uint16)
    for h in range(cfg.n_kv):
        assert np.array_equal(gperm[h], perms[h])
    gcb = cb.cpu().numpy()
    ocb = codebook_array(tables)
    fin = np.isfinite(ocb)
    assert np.all(np.abs(gcb[fin] - ocb[fin]) <= np.abs(np.spacing(ocb[fin])))
    counts = {}
    for (b, h) in [(0, 0), (5, 2), (15, 7)]:
        f = encode.encode_keys(K[b, h], signs[h], perms[h], tables[h][0], tables[h][1], S[h], p)
        got = layout.unpack_stream(codes[b, h].cpu().numpy(), p, cfg.n_tokens, cfg.n_tokens)
        merge_counts(counts, classify(f, got, tables[h][1], S[h], p))
    print("bulk encode", counts)
    assert_code_parity(counts)


def test_c2_fp16_comparator_full_size():
    api = _api()
    cfg = CONFIGS["nano_b64_t512"]
    inp = make_inputs(cfg)
    K16 = inp["K"].astype(np.float16)
    out = api.pgkq_fp16_decode_attn(q_tensor(inp["q"], cfg.q_dtype), to_dev(K16),
                                    v_cache(inp["V"], cfg.n_tokens))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    worst = 0.0
    for b in (0, 31, 63):
        ref, _ = attn.fp16_attention(inp["q"][b:b + 1], K16[b:b + 1], inp["V"][b:b + 1])
        worst = max(worst, float(np.max(np.abs(out[b] - ref[0]))))
    print("fp16 comparator max-abs", worst)
    assert worst <= OUT_TOL


# ------------------------------------------------------------------ controls and the next rows at full size

def _c3_inputs():
    cfg = CONFIGS["gqa_b16_t32k"]
    return cfg, make_inputs(cfg)


@pytest.mark.parametrize("bits", [4, 3])
def test_c3_rtn_control_full_size_sampled(bits):
    """RTN INT4 / INT3 keys on the full 32k-token GQA cache, 8 splits (the launch
    the benchmark's controls time): GPU-encoded records bit-exact on sampled
    streams, outputs of their query heads within 1e-3."""
    from oracle import rtn
    api = _api()
    cfg, inp = _c3_inputs()
    K, V, q = inp["K"], inp["V"], inp["q"]
    codes = api.pgkq_rtn_encode(k_tensor(K), bits)
    out = api.pgkq_rtn_decode_attn(q_tensor(q, cfg.q_dtype), codes, v_cache(V, cfg.n_tokens), bits,
                                   n_splits=cfg.n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = cfg.n_q // cfg.n_kv
    worst = 0.0
    for (b, h) in [(0, 0), (9, 4), (15, 7)]:
        c, s, z = rtn.quantize(K[b, h].astype(np.float64), bits)
        want = rtn.pack_stream(c, s, z, bits, cfg.n_tokens)
        assert np.array_equal(codes[b, h].cpu().numpy(), want)
        khat = rtn.dequantize(c, s, z)
        for g in range(G):
            hq = h * G + g
            ref = attn.attend(khat @ q[b, hq].astype(np.float64), V[b, h], 1.0 / np.sqrt(cfg.head_dim))
            worst = max(worst, float(np.abs(out[b, hq] - ref).max()))
    print("rtn", bits, "max-abs", worst)
    assert worst <= OUT_TOL and np.isfinite(out).all()


def test_c3_fp16_comparator_full_size_sampled():
    api = _api()
    cfg, inp = _c3_inputs()
    K16, V, q = inp["K"].astype(np.float16), inp["V"], inp["q"]
    out = api.pgkq_fp16_decode_attn(q_tensor(q, cfg.q_dtype), to_dev(K16), v_cache(V, cfg.n_tokens),
                                    n_splits=cfg.n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    worst = 0.0
    for (b, h) in [(0, 0), (15, 7)]:
        ref, _ = attn.fp16_attention(q[b:b + 1, h * 4:h * 4 + 4], K16[b:b + 1, h:h + 1],
                                     V[b:b + 1, h:h + 1])
        worst = max(worst, float(np.abs(out[b, h * 4:h * 4 + 4] - ref[0]).max()))
    print("fp16 32k-token cache max-abs", worst)
    assert worst <= OUT_TOL


def test_c3_pgkq_kv_full_size_sampled():
    """PGKQ-KV (k3v3, QJL on both) on the full 32k-token cache: value records of
    sampled streams within the code bar, their outputs within 1e-3 (decoded on
    the oracle's records for those streams)."""
    from oracle import kv
    from synth.inputs import value_projection
    api = _api()
    cfg, inp = _c3_inputs()
    K, V, q, signs, S = inp["K"], inp["V"], inp["q"], inp["signs"], inp["S"]
    Sv = value_projection(cfg)
    p = params_of(cfg)
    pv = kv.value_params(cfg.head_dim, cfg.b_main, cfg.qjl_m)
    cap = cfg.n_tokens
    tables, _, _ = _oracle_tables(K, cfg, reorder=False)
    vtables = kv.value_tables(V.astype(np.float64), cfg.b_main)
    dsigns = to_dev(signs)
    ck = api.pgkq_encode(lib_params(p), k_tensor(K), dsigns, None, to_dev(codebook_array(tables)),
                         to_dev(S), capacity=cap)
    cv = api.pgkq_encode(lib_params(pv), k_tensor(V), dsigns, None, to_dev(codebook_array(vtables)),
                         to_dev(Sv), capacity=cap)
    torch.cuda.synchronize()
    counts, kf, vf = {}, {}, {}
    samples = [(0, 0), (15, 7)]
    for (b, h) in samples:
        kf[(b, h)] = encode.encode_keys(K[b, h], signs[h], None, tables[h][0], tables[h][1], S[h], p)
        vf[(b, h)] = kv.encode_values(V[b, h].astype(np.float64), vtables[h][0], vtables[h][1],
                                      Sv[h], pv)
        got = layout.unpack_stream(cv[b, h].cpu().numpy(), pv, cap, cap)
        merge_counts(counts, classify(vf[(b, h)], got, vtables[h][1], Sv[h], pv))
        ck[b, h] = torch.from_numpy(layout.pack_stream(kf[(b, h)], p, cap)).to(ck.device)
        cv[b, h] = torch.from_numpy(layout.pack_stream(vf[(b, h)], pv, cap)).to(cv.device)
    print("kv value encode", counts)
    assert_code_parity(counts)
    out = api.pgkq_kv_decode_attn(lib_params(p), lib_params(pv), q_tensor(q, cfg.q_dtype), ck, cv,
                                  cfg.n_kv, cap, dsigns, None, to_dev(codebook_array(tables)),
                                  to_dev(S), to_dev(codebook_array(vtables)), to_dev(Sv),
                                  n_splits=cfg.n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = cfg.n_q // cfg.n_kv
    worst = 0.0
    for (b, h) in samples:
        Vh = kv.dequantize_values(vf[(b, h)], vtables[h][0], Sv[h], pv)
        for g in range(G):
            hq = h * G + g
            s = attn.analytic_logits(q[b, hq], kf[(b, h)], tables[h][0], S[h], signs[h], None, p)
            ref = attn.softmax_weights(s, 1.0 / np.sqrt(cfg.head_dim)) @ Vh
            worst = max(worst, float(np.abs(out[b, hq] - ref).max()))
    print("kv decode max-abs", worst)
    assert worst <= OUT_TOL and np.isfinite(out).all()


def test_c3_decode_step_full_size_sampled():
    """The decode step on the full cache: the last slot re-appended inside the
    decode call; its records and the sampled outputs match the oracle."""
    api = _api()
    cfg, inp = _c3_inputs()
    K, V, q, signs, S = inp["K"], inp["V"], inp["q"], inp["signs"], inp["S"]
    p = params_of(cfg)
    T = cap = cfg.n_tokens
    tables, _, _ = _oracle_tables(K, cfg, reorder=False)
    dsigns, dcb, dS = to_dev(signs), to_dev(codebook_array(tables)), to_dev(S)
    codes = api.pgkq_encode(lib_params(p), k_tensor(K[:, :, :T - 1]), dsigns, None, dcb, dS,
                            capacity=cap)
    Vz = V.copy()
    Vz[:, :, T - 1] = 0
    Vd = v_cache(Vz, cap)
    del Vz
    out = api.pgkq_decode_step(lib_params(p), q_tensor(q, cfg.q_dtype),
                               k_tensor(np.ascontiguousarray(K[:, :, T - 1])),
                               to_dev(np.ascontiguousarray(V[:, :, T - 1])), codes, Vd, T - 1,
                               dsigns, None, dcb, dS, n_splits=cfg.n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.array_equal(untile_values(Vd.cpu().numpy()), V)
    G = cfg.n_q // cfg.n_kv
    counts, worst = {}, 0.0
    for (b, h) in [(0, 0), (15, 7)]:
        f = encode.encode_keys(K[b, h], signs[h], None, tables[h][0], tables[h][1], S[h], p)
        got = layout.unpack_stream(codes[b, h].cpu().numpy(), p, cap, T)
        merge_counts(counts, classify(f, got, tables[h][1], S[h], p))
        for g in range(G):
            hq = h * G + g
            s = attn.analytic_logits(q[b, hq], f, tables[h][0], S[h], signs[h], None, p)
            ref = attn.attend(s, V[b, h], 1.0 / np.sqrt(cfg.head_dim))
            worst = max(worst, float(np.abs(out[b, hq] - ref).max()))
    print("step encode", counts, "decode max-abs", worst)
    assert_code_parity(counts)
    assert worst <= OUT_TOL
