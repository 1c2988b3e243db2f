"""Parity at the measured workloads' full sizes, in the launch configuration the
benchmark times: the GPU runs the whole cache and the oracle checks EVERY
(sequence, kv-head) stream of it, one stream per worker thread (NumPy and BLAS
release the GIL).  For decode parity the oracle's codes are written into the
GPU code buffer, so that decode runs on identical codes."""

import concurrent.futures as cf
import functools
import os

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

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


def _pmap(fn, items):
    """fn over items on the host cores (at most 16 threads, one BLAS thread each)."""
    workers = max(1, min(len(os.sched_getaffinity(0)), 16))
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def _all_streams(cfg):
    return [(b, h) for b in range(cfg.n_seq) for h in range(cfg.n_kv)]


def _small(f):
    """The stored fields of an oracle encoding (its diagnostics are large)."""
    return {"rc": f.rc.astype(np.uint8), "ac": f.ac.astype(np.uint8), "bits": f.bits, "nu": f.nu}


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


def _run_full(cfg, n_splits, streams=None):
    """GPU encode + decode of the whole cache; every stream's codes classified
    against the oracle's, then decode on the oracle's codes compared for every
    query head of every stream."""
    api = _api()
    p = params_of(cfg)
    lp = lib_params(p)
    inp = _inputs(cfg.name)
    K, V, q, signs, S = inp["K"], inp["V"], inp["q"], inp["signs"], inp["S"]
    cap = T = cfg.n_tokens
    streams = _all_streams(cfg) if streams is None else streams
    tables, _, _ = _oracle_tables(K, cfg, reorder=False)
    cb = codebook_array(tables)
    dsigns, dcb, dS = to_dev(signs), to_dev(cb), to_dev(S)
    Kt = k_tensor(K)
    codes = api.pgkq_encode(lp, Kt, dsigns, None, dcb, dS, capacity=cap)
    torch.cuda.synchronize()
    del Kt
    got_all = codes.cpu().numpy()
    ours = got_all.copy()

    def enc(bh):
        b, h = bh
        f = encode.encode_keys(K[b, h], signs[h], None, tables[h][0], tables[h][1], S[h], p)
        got = layout.unpack_stream(got_all[b, h], p, cap, T)
        cnt = classify(f, got, tables[h][1], S[h], p)
        layout.pack_stream(f, p, cap, 0, ours[b, h])
        return cnt, _small(f)

    res = _pmap(enc, streams)
    counts = {}
    for cnt, _ in res:
        merge_counts(counts, cnt)
    print(cfg.name, f"encode, {len(streams)} streams", counts)
    assert_code_parity(counts)
    codes.copy_(torch.from_numpy(ours))
    del got_all, ours
    out = api.pgkq_decode_attn(lp, q_tensor(q, cfg.q_dtype), codes, v_cache(V, cap), dsigns, None, dcb,
                               dS, n_splits=n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))
    G = cfg.n_q // cfg.n_kv

    def dec(i):
        (b, h), (_, f) = streams[i], res[i]
        w = 0.0
        for g in range(G):
            hq = h * G + g
            s = attn.analytic_logits(q[b, hq], f, tables[h][0], S[h], signs[h], None, p)
            ref = attn.attend(s, V[b, h], 1.0 / np.sqrt(cfg.head_dim))
            w = max(w, float(np.max(np.abs(out[b, hq] - ref))))
        return w

    worst = max(_pmap(dec, range(len(streams))))
    print(cfg.name, f"decode max-abs over {len(streams) * G} query heads", worst)
    assert worst <= OUT_TOL


@functools.lru_cache(maxsize=4)
def _inputs(name):
    return make_inputs(CONFIGS[name])


def test_c3_full_size_every_stream():
    _run_full(CONFIGS["gqa_b16_t32k"], n_splits=CONFIGS["gqa_b16_t32k"].n_splits)


def test_c5_full_size_every_stream():
    _run_full(CONFIGS["gqa_b1_t131k"], n_splits=CONFIGS["gqa_b1_t131k"].n_splits)


@pytest.mark.parametrize("name", ["nano_b64_t512", "nano_b64_t512_b4"])
def test_c2_full_size_every_stream(name):
    _run_full(CONFIGS[name], n_splits=0)


def test_c4_full_size_calibrate_and_encode_every_stream():
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k_encode"]
    p = params_of(cfg)
    lp = lib_params(p)
    inp = _inputs("gqa_b16_t32k")   # the same keys (the bulk encode is the 32k-token cache)
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
    got_all = codes.cpu().numpy()

    def enc(bh):
        b, h = bh
        f = encode.encode_keys(K[b, h], signs[h], perms[h], tables[h][0], tables[h][1], S[h], p)
        got = layout.unpack_stream(got_all[b, h], p, cfg.n_tokens, cfg.n_tokens)
        return classify(f, got, tables[h][1], S[h], p)

    counts = {}
    for cnt in _pmap(enc, _all_streams(cfg)):
        merge_counts(counts, cnt)
    print("bulk encode, every stream", counts)
    assert_code_parity(counts)


def test_c2_fp16_comparator_full_size():
    api = _api()
    cfg = CONFIGS["nano_b64_t512"]
    inp = _inputs(cfg.name)
    K16 = inp["K"].astype(np.float16)
    out = api.pgkq_fp16_decode_attn(q_tensor(inp["q"], cfg.q_dtype), to_dev(K16),
                                    v_cache(inp["V"], cfg.n_tokens))
    torch.cuda.synchronize()
    out = out.cpu().numpy()

    def one(b):
        ref, _ = attn.fp16_attention(inp["q"][b:b + 1], K16[b:b + 1], inp["V"][b:b + 1])
        return float(np.max(np.abs(out[b] - ref[0])))

    worst = max(_pmap(one, range(cfg.n_seq)))
    print("fp16 comparator max-abs, every sequence", worst)
    assert worst <= OUT_TOL


# ------------------------------------------------------------------ controls and the next rows at full size

def _c3_inputs():
    return CONFIGS["gqa_b16_t32k"], _inputs("gqa_b16_t32k")


@pytest.mark.parametrize("bits", [4, 3])
def test_c3_rtn_control_full_size_every_stream(bits):
    """RTN INT4 / INT3 keys on the full 32k-token GQA cache, 8 splits (the launch
    the benchmark's controls time): GPU-encoded records bit-exact on every
    stream, every query head's output within 1e-3."""
    from oracle import rtn
    api = _api()
    cfg, inp = _c3_inputs()
    K, V, q = inp["K"], inp["V"], inp["q"]
    codes = api.pgkq_rtn_encode(k_tensor(K), bits)
    out = api.pgkq_rtn_decode_attn(q_tensor(q, cfg.q_dtype), codes, v_cache(V, cfg.n_tokens), bits,
                                   n_splits=cfg.n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    got_all = codes.cpu().numpy()
    G = cfg.n_q // cfg.n_kv

    def one(bh):
        b, h = bh
        c, s, z = rtn.quantize(K[b, h].astype(np.float64), bits)
        same = np.array_equal(got_all[b, h], rtn.pack_stream(c, s, z, bits, cfg.n_tokens))
        khat = rtn.dequantize(c, s, z)
        w = 0.0
        for g in range(G):
            hq = h * G + g
            ref = attn.attend(khat @ q[b, hq].astype(np.float64), V[b, h], 1.0 / np.sqrt(cfg.head_dim))
            w = max(w, float(np.abs(out[b, hq] - ref).max()))
        return same, w

    res = _pmap(one, _all_streams(cfg))
    worst = max(w for _, w in res)
    print("rtn", bits, "records equal on", sum(s for s, _ in res), "of", len(res), "streams; max-abs", worst)
    assert all(s for s, _ in res)
    assert worst <= OUT_TOL and np.isfinite(out).all()


def test_c3_fp16_comparator_full_size_every_stream():
    api = _api()
    cfg, inp = _c3_inputs()
    K16, V, q = inp["K"].astype(np.float16), inp["V"], inp["q"]
    out = api.pgkq_fp16_decode_attn(q_tensor(q, cfg.q_dtype), to_dev(K16), v_cache(V, cfg.n_tokens),
                                    n_splits=cfg.n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = cfg.n_q // cfg.n_kv

    def one(bh):
        b, h = bh
        ref, _ = attn.fp16_attention(q[b:b + 1, h * G:(h + 1) * G], K16[b:b + 1, h:h + 1],
                                     V[b:b + 1, h:h + 1])
        return float(np.abs(out[b, h * G:(h + 1) * G] - ref[0]).max())

    worst = max(_pmap(one, _all_streams(cfg)))
    print("fp16 32k-token cache max-abs, every stream", worst)
    assert worst <= OUT_TOL


def test_c3_pgkq_kv_full_size_every_stream():
    """PGKQ-KV (k3v3, QJL on both) on the full 32k-token cache: value records of
    every stream within the code bar, every output within 1e-3 (decoded on the
    oracle's key and value records)."""
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
    got_v = cv.cpu().numpy()
    ours_k = np.zeros_like(got_v, shape=tuple(ck.shape))
    ours_v = got_v.copy()
    streams = _all_streams(cfg)

    def enc(bh):
        b, h = bh
        kf = encode.encode_keys(K[b, h], signs[h], None, tables[h][0], tables[h][1], S[h], p)
        vf = kv.encode_values(V[b, h].astype(np.float64), vtables[h][0], vtables[h][1], Sv[h], pv)
        got = layout.unpack_stream(got_v[b, h], pv, cap, cap)
        cnt = classify(vf, got, vtables[h][1], Sv[h], pv)
        layout.pack_stream(kf, p, cap, 0, ours_k[b, h])
        layout.pack_stream(vf, pv, cap, 0, ours_v[b, h])
        return cnt, _small(kf), _small(vf)

    res = _pmap(enc, streams)
    counts = {}
    for cnt, _, _ in res:
        merge_counts(counts, cnt)
    print("kv value encode, every stream", counts)
    assert_code_parity(counts)
    ck.copy_(torch.from_numpy(ours_k))
    cv.copy_(torch.from_numpy(ours_v))
    del got_v, ours_k, ours_v
    out = api.pgkq_kv_decode_attn(lib_params(p), lib_params(pv), q_tensor(q, cfg.q_dtype), ck, cv,
                                  cfg.n_kv, cap, dsigns, None, to_dev(codebook_array(tables)),
                                  to_dev(S), to_dev(codebook_array(vtables)), to_dev(Sv),
                                  n_splits=cfg.n_splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    G = cfg.n_q // cfg.n_kv

    def dec(i):
        (b, h), (_, kf, vf) = streams[i], res[i]
        Vh = kv.dequantize_values(vf, vtables[h][0], Sv[h], pv)
        w = 0.0
        for g in range(G):
            hq = h * G + g
            s = attn.analytic_logits(q[b, hq], kf, tables[h][0], S[h], signs[h], None, p)
            ref = attn.softmax_weights(s, 1.0 / np.sqrt(cfg.head_dim)) @ Vh
            w = max(w, float(np.abs(out[b, hq] - ref).max()))
        return w

    worst = max(_pmap(dec, range(len(streams))))
    print("kv decode max-abs, every stream", worst)
    assert worst <= OUT_TOL and np.isfinite(out).all()


def test_c3_decode_step_full_size_every_stream():
    """The decode step on the full cache: the last slot appended inside the
    decode call; the records of every stream and every output match the oracle."""
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
    del Vd
    got_all = codes.cpu().numpy()
    G = cfg.n_q // cfg.n_kv

    def one(bh):
        b, h = bh
        f = encode.encode_keys(K[b, h], signs[h], None, tables[h][0], tables[h][1], S[h], p)
        got = layout.unpack_stream(got_all[b, h], p, cap, T)
        cnt = classify(f, got, tables[h][1], S[h], p)
        polar_same = bool(np.array_equal(got["rc"], f.rc) and np.array_equal(got["ac"], f.ac))
        w = 0.0
        if cnt["mismatch"] == 0:
            for g in range(G):
                hq = h * G + g
                s = attn.analytic_logits(q[b, hq], f, tables[h][0], S[h], signs[h], None, p)
                ref = attn.attend(s, V[b, h], 1.0 / np.sqrt(cfg.head_dim))
                w = max(w, float(np.abs(out[b, hq] - ref).max()))
        return cnt, w, polar_same

    res = _pmap(one, _all_streams(cfg))
    counts = {}
    for cnt, _, _ in res:
        merge_counts(counts, cnt)
    worst = max(w for _, w, _ in res)
    checked = sum(1 for cnt, _, _ in res if cnt["mismatch"] == 0)
    print("step encode, every stream", counts, f"decode max-abs {worst} over {checked} streams "
          "with identical codes")
    assert_code_parity(counts)
    # streams whose records hold a boundary case are compared through their codes only
    assert checked >= len(res) - counts["mismatch"]
    assert worst <= OUT_TOL
