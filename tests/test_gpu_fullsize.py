"""Parity at the measured workloads' full sizes, in the launch configuration the
benchmark times: the GPU runs the whole cache, the oracle checks sampled
streams one by one (its codes for those streams are written into the GPU code
buffer so that decode parity runs on identical codes)."""

import numpy as np
import pytest
import torch

from oracle import attn, calibrate, codebook, encode, layout
from synth import CONFIGS, make_inputs

from gpu_cases import k_tensor, lib_params, params_of, q_tensor, to_dev
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
    out = api.pgkq_decode_attn(lp, q_tensor(q, cfg.q_dtype), codes, to_dev(V), dsigns, None, dcb, dS,
                               n_splits=n_splits)
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
    _run_full(CONFIGS["c3"], [(0, 0), (7, 3), (15, 7)], n_splits=CONFIGS["c3"].n_splits)


def test_c5_full_size_sampled():
    _run_full(CONFIGS["c5"], [(0, 0), (0, 5)], n_splits=CONFIGS["c5"].n_splits)


@pytest.mark.parametrize("name", ["c2a", "c2b"])
def test_c2_full_size_every_stream(name):
    cfg = CONFIGS[name]
    n_streams = [(b, h) for b in range(cfg.n_seq) for h in range(cfg.n_kv)]
    _run_full(cfg, n_streams[:: 97] + [n_streams[-1]], n_splits=0)


def test_c4_full_size_calibrate_and_encode_sampled():
    api = _api()
    cfg = CONFIGS["c4"]
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
    print("c4 encode", counts)
    assert_code_parity(counts)


def test_c2_fp16_comparator_full_size():
    api = _api()
    cfg = CONFIGS["c2a"]
    inp = make_inputs(cfg)
    K16 = inp["K"].astype(np.float16)
    out = api.pgkq_fp16_decode_attn(q_tensor(inp["q"], cfg.q_dtype), to_dev(K16), to_dev(inp["V"]))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    worst = 0.0
    for b in (0, 31, 63):
        ref, _ = attn.fp16_attention(inp["q"][b:b + 1], K16[b:b + 1], inp["V"][b:b + 1])
        worst = max(worst, float(np.max(np.abs(out[b] - ref[0]))))
    print("fp16 comparator max-abs", worst)
    assert worst <= OUT_TOL
