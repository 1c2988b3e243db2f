"""GPU parity at the largest streams and batches the C ABI accepts.

The scans address one stream's codes and value rows with 32-bit byte offsets
(buffer resources), so the library rejects a stream whose codes or values
would pass 4 GiB.  These tests run the largest accepted streams and check the
tokens at the start, across the 2 GiB mark and at the very end:

* decode attention over one stream of 16 777 184 tokens (d128, b3/2 + QJL,
  4 query heads): its value rows end 32 bytes short of the largest accepted
  range (capacity x 256 bytes, 32-token tiles);
* the logit hook over one stream of 58 040 098 tokens (d128, b4/3 + QJL,
  74-byte records): its codes end within 16 bytes of the largest accepted
  range;
* decode attention over 65 535 sequences, the most a grid dimension holds
  (the sequence index is one of the scan's grid dimensions), at one and at
  three splits per stream.

In the first two, every key is one of two fixed keys ("cold" everywhere, "hot" in three 64-token
blocks: at the start, across 2^31 bytes of the stream, at the end), so the
oracle needs only those two keys: their codes (compared word by word at the
hot blocks and at random cold tokens), their logits, and the attention output
in closed form.  With hot tokens h and cold tokens c (N_c of them, all with
value row v_c) the weights are exp(z_h), exp(z_c) with z = logit / sqrt(d):
    out = (N_c e^{z_c} v_c + e^{z_h} sum_{t hot} v_t) / (N_c e^{z_c} + N_h e^{z_h}).
The value rows of the hot tokens are all different, so a hot token read from
the wrong place changes the output.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attn, calibrate, codebook, encode, layout
from oracle.encode import Params

from gpu_cases import DEV, LOGIT_TOL, OUT_TOL

pytestmark = pytest.mark.gpu

D = 128
MAX_RANGE = 0xFFFFFFF0   # largest byte range of one stream the library accepts


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from compressed_cache_decode_pgkq_amd import _lib
    _lib.lib()


def _two_keys(p: Params, q, n_cold, n_hot, seed):
    """The cold and hot keys (fp16), the shared per-head inputs, the oracle's
    table for this cache and the oracle fields of the two keys."""
    rng = np.random.default_rng(seed)
    signs = np.where(rng.random(D) < 0.5, -1, 1).astype(np.int8)
    S = rng.standard_normal((p.qjl_m, D)).astype(np.float32) if p.qjl_m else None
    k_cold = (0.7 * rng.standard_normal(D)).astype(np.float16)
    u = q.sum(axis=0)
    k_hot = (12.0 * u / np.linalg.norm(u)).astype(np.float16)
    # the head scale of this cache (n_cold copies of one key, n_hot of the other)
    sumsq = (n_cold * k_cold.astype(np.float64) ** 2 + n_hot * k_hot.astype(np.float64) ** 2)
    c, t = codebook.lloyd_max_beta(D, p.b_main)
    lv, th = codebook.scaled_table(c, t, calibrate.head_scale(sumsq, n_cold + n_hot), D)
    f = encode.encode_keys(np.stack([k_cold, k_hot]), signs, None, lv, th, S, p)
    return signs, S, k_cold, k_hot, (lv, th), f


def _oracle_words(p: Params, f):
    """Code words and norm bits of the two keys, packed as a 2-slot stream."""
    buf = layout.pack_stream(f, p, 2)
    W = layout.n_words(p)
    words = buf[: W * 4 * 2].view(np.uint32).reshape(W, 2)
    nu = buf[W * 4 * 2: W * 4 * 2 + 4].view(np.uint16) if p.qjl_m else None
    return words, nu


def _device_words(codes, p: Params, cap, tokens):
    """Code words [W, len(tokens)] and norm bits of `tokens` of a device stream."""
    W = layout.n_words(p)
    flat = codes.view(-1)
    idx = torch.as_tensor(tokens, device=DEV, dtype=torch.int64)
    words = []
    for w in range(W):
        b0 = 4 * (w * cap + idx)
        words.append(torch.stack([flat[b0 + k] for k in range(4)], dim=1).cpu().numpy())
    words = np.stack(words).astype(np.uint32)
    words = words[..., 0] | (words[..., 1] << 8) | (words[..., 2] << 16) | (words[..., 3] << 24)
    nu = None
    if p.qjl_m:
        b0 = 4 * W * cap + 2 * idx
        nb = torch.stack([flat[b0], flat[b0 + 1]], dim=1).cpu().numpy().astype(np.uint16)
        nu = nb[:, 0] | (nb[:, 1] << 8)
    return words, nu


def _hot_blocks(T):
    mid = (1 << 31) // 256          # the token whose value tile starts 2 GiB into the stream
    return [np.arange(0, 64), np.arange(mid - 32, mid + 32), np.arange(T - 64, T)]


def _check_codes(codes, p, cap, hot, T, f, seed):
    ow, onu = _oracle_words(p, f)
    rng = np.random.default_rng(seed + 1)
    cold = rng.choice(np.setdiff1d(np.arange(T - 200000, T), hot), 256, replace=False)
    cold = np.concatenate([cold, rng.integers(64, T // 2, 256)])
    cold = np.setdiff1d(cold, hot)
    for toks, col in ((hot, 1), (cold, 0)):
        gw, gnu = _device_words(codes, p, cap, toks)
        assert np.array_equal(gw, np.repeat(ow[:, col:col + 1], len(toks), axis=1)), col
        if p.qjl_m:
            assert np.all(gnu == onu[col]), col


def test_decode_at_the_largest_value_stream():
    import compressed_cache_decode_pgkq_amd as api
    p = Params(D, 3, 2, D, True)
    T = MAX_RANGE // (D * 2) // 32 * 32            # 16 777 184 tokens, capacity = T
    assert T * D * 2 <= MAX_RANGE < (T + 32) * D * 2
    rng = np.random.default_rng(5150)
    q = rng.standard_normal((4, D)).astype(np.float32)
    hot = np.concatenate(_hot_blocks(T))
    n_hot = len(hot)
    signs, S, k_cold, k_hot, (lv, th), f = _two_keys(p, q, T - n_hot, n_hot, 5151)
    print(f"T {T}, hot tokens {n_hot}", flush=True)

    lp = api.PgkqParams(D, 3, 2, D, 1)
    hot_t = torch.as_tensor(hot, device=DEV)
    K = torch.as_tensor(k_cold, device=DEV).view(1, 1, 1, D).expand(1, 1, T, D).contiguous()
    K[0, 0, hot_t] = torch.as_tensor(k_hot, device=DEV)
    cb = torch.as_tensor(codebook.pack_table(lv, th)[None].astype(np.float32), device=DEV)
    d_signs = torch.as_tensor(signs[None], device=DEV)
    d_S = torch.as_tensor(S[None], device=DEV)
    codes = api.pgkq_encode(lp, K, d_signs, None, cb, d_S, capacity=T)
    del K
    torch.cuda.synchronize()
    _check_codes(codes, p, T, hot, T, f, 5152)

    # value rows: v_c everywhere, a different row for every hot token
    v_cold = rng.standard_normal(D).astype(np.float16)
    v_hot = rng.standard_normal((n_hot, D)).astype(np.float16)
    rows = torch.as_tensor(v_cold, device=DEV).view(1, 1, 1, D).expand(1, 1, T, D).contiguous()
    rows[0, 0, hot_t] = torch.as_tensor(v_hot, device=DEV)
    Vt = api.pgkq_pack_values(rows, capacity=T)
    del rows

    # closed form from the oracle's logits of the two keys
    lg = np.stack([attn.analytic_logits(q[g], f, lv, S, signs, None, p) for g in range(4)])  # [4, 2]
    z = lg / math.sqrt(D)
    zm = z.max(axis=1, keepdims=True)
    wc, wh = np.exp(z[:, 0:1] - zm), np.exp(z[:, 1:2] - zm)
    num = (T - n_hot) * wc * v_cold.astype(np.float64)[None] + wh * v_hot.astype(np.float64).sum(0)[None]
    ref = num / ((T - n_hot) * wc + n_hot * wh)
    print("hot share per head", (n_hot * wh / ((T - n_hot) * wc + n_hot * wh)).ravel(), flush=True)

    dq = torch.as_tensor(q[None], device=DEV)
    # the automatic plan, and a requested single split (cut into 2^18-token
    # splits, so that no lane sums more than 1024 of these equal terms)
    for ns in (0, 1):
        out = api.pgkq_decode_attn(lp, dq, codes, Vt, d_signs, None, cb, d_S, n_tokens=T,
                                   n_splits=ns)
        torch.cuda.synchronize()
        err = float(np.max(np.abs(out.cpu().numpy()[0] - ref)))
        print(f"n_splits {ns}: max-abs {err:.2e}", flush=True)
        assert err <= OUT_TOL and math.isfinite(err)


def test_logits_at_the_largest_code_stream():
    import compressed_cache_decode_pgkq_amd as api
    p = Params(D, 4, 3, D, True)
    rb = layout.record_bytes(p)                         # 74 bytes
    T = MAX_RANGE // rb // 2 * 2                         # 58 040 098 tokens (even: QJL)
    assert T * rb <= MAX_RANGE < (T + 2) * rb
    rng = np.random.default_rng(6160)
    q = rng.standard_normal((4, D)).astype(np.float32)
    hot = np.concatenate([np.arange(0, 64), np.arange(T // 2 - 32, T // 2 + 32), np.arange(T - 64, T)])
    signs, S, k_cold, k_hot, (lv, th), f = _two_keys(p, q, T - len(hot), len(hot), 6161)
    print(f"T {T}, codes {T * rb / 2**30:.3f} GiB", flush=True)

    lp = api.PgkqParams(D, 4, 3, D, 1)
    hot_t = torch.as_tensor(hot, device=DEV)
    K = torch.as_tensor(k_cold, device=DEV).view(1, 1, 1, D).expand(1, 1, T, D).contiguous()
    K[0, 0, hot_t] = torch.as_tensor(k_hot, device=DEV)
    cb = torch.as_tensor(codebook.pack_table(lv, th)[None].astype(np.float32), device=DEV)
    d_signs = torch.as_tensor(signs[None], device=DEV)
    d_S = torch.as_tensor(S[None], device=DEV)
    codes = api.pgkq_encode(lp, K, d_signs, None, cb, d_S, capacity=T)
    del K
    torch.cuda.synchronize()
    _check_codes(codes, p, T, hot, T, f, 6162)

    dq = torch.as_tensor(q[None], device=DEV)
    lg = api.pgkq_estimate_logits(lp, dq, codes, 1, T, d_signs, None, cb, d_S, n_tokens=T)
    torch.cuda.synchronize()
    ref = np.stack([attn.analytic_logits(q[g], f, lv, S, signs, None, p) for g in range(4)])  # [4, 2]
    qn = np.linalg.norm(q.astype(np.float64), axis=1)
    kn = np.array([np.linalg.norm(k_cold.astype(np.float64)), np.linalg.norm(k_hot.astype(np.float64))])
    cold = np.setdiff1d(np.random.default_rng(6163).integers(0, T, 4096), hot)
    for toks, col in ((hot, 1), (cold, 0)):
        got = lg[0][:, torch.as_tensor(toks, device=DEV)].cpu().numpy()     # [4, n]
        err = np.abs(got - ref[:, col:col + 1]) / (qn[:, None] * kn[col])
        print(f"{'hot' if col else 'cold'}: max error {err.max():.2e} of ||q|| ||k||", flush=True)
        assert err.max() <= LOGIT_TOL



@pytest.mark.parametrize("T,n_splits", [(40, 0), (200, 3)])
def test_decode_with_the_most_sequences(T, n_splits):
    """65 535 sequences (a grid dimension at its limit) of one kv-head with two
    query heads, d64, b3/2 + QJL: the scan's grid is (kv-head, sequence,
    split), the preparation's (sequence, query head).  One workgroup per
    stream at 40 tokens, three splits at 200.  Codes and outputs of 96 sampled
    sequences (the first two, the last two and random ones) against the
    oracle."""
    import compressed_cache_decode_pgkq_amd as api
    from parity_util import assert_code_parity, classify, merge_counts
    n_seq, n_kv, n_q, d = 65535, 1, 2, 64
    p = Params(d, 3, 2, d, True)
    rng = np.random.default_rng(7170 + T)
    scale = np.exp(0.5 * rng.standard_normal(d)).astype(np.float32)
    K = rng.standard_normal((n_seq, n_kv, T, d), dtype=np.float32)
    K *= scale
    V = rng.standard_normal((n_seq, n_kv, T, d), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((n_seq, n_q, d), dtype=np.float32)
    signs = np.where(rng.random((n_kv, d)) < 0.5, -1, 1).astype(np.int8)
    S = rng.standard_normal((n_kv, d, d), dtype=np.float32)
    sumsq = np.zeros(d)
    for b0 in range(0, n_seq, 4096):
        sumsq += calibrate.channel_sumsq(K[b0:b0 + 4096, 0])
    c, t = codebook.lloyd_max_beta(d, 3)
    lv, th = codebook.scaled_table(c, t, calibrate.head_scale(sumsq, n_seq * T), d)
    cb = codebook.pack_table(lv, th)[None].astype(np.float32)
    print(f"T {T}, splits {n_splits}: inputs ready", flush=True)

    lp = api.PgkqParams(d, 3, 2, d, 1)
    d_signs, d_S, d_cb = (torch.as_tensor(x, device=DEV) for x in (signs, S, cb))
    cap = -(-T // 32) * 32
    dK = torch.as_tensor(K, device=DEV)
    codes = api.pgkq_encode(lp, dK, d_signs, None, d_cb, d_S, capacity=cap)
    del dK
    Vt = api.pgkq_pack_values(torch.as_tensor(V, device=DEV), capacity=cap)
    out = api.pgkq_decode_attn(lp, torch.as_tensor(q, device=DEV), codes, Vt, d_signs, None, d_cb,
                               d_S, n_tokens=T, n_splits=n_splits)
    torch.cuda.synchronize()

    pick = np.unique(np.concatenate([[0, 1, n_seq - 2, n_seq - 1],
                                     rng.choice(n_seq, 92, replace=False)]))
    pick_t = torch.as_tensor(pick, device=DEV)
    f = encode.encode_cache(K[pick], signs, None, [(lv, th)], S, p)
    counts = {}
    got_codes = codes[pick_t].cpu().numpy()
    for i in range(len(pick)):
        u = layout.unpack_stream(got_codes[i, 0], p, cap, T)
        merge_counts(counts, classify(f[i][0], u, th, S[0], p))
    ref, _ = attn.decode_cache(q[pick], f, V[pick], [(lv, th)], S, signs, None, p)
    err = float(np.max(np.abs(out[pick_t].cpu().numpy() - ref)))
    print(f"T {T}, splits {n_splits}: {counts}, max-abs {err:.2e}", flush=True)
    assert_code_parity(counts)
    assert err <= OUT_TOL and math.isfinite(err)
