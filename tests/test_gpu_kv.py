"""GPU parity of PGKQ-KV (values coded by the key encoder without the
transform, decoded in the code domain) through the C ABI against oracle/kv.py.

Bars: the value records written by pgkq_encode obey the code-parity bar
(bit-exact except G15 boundary cases); decode outputs within 1e-3 max-abs of
the oracle's softmax-weighted explicit reconstruction.  Decode parity runs on
the oracle's packed key and value records.
"""

import numpy as np
import pytest
import torch

from oracle import kv, layout
from synth import CONFIGS
from synth.inputs import value_projection

from gpu_cases import Case, k_tensor, lib_params, q_tensor, to_dev
from parity_util import assert_code_parity, classify, codebook_array, merge_counts

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


class KVCase:
    """Key side from Case; value side coded by the oracle with its own table and
    projection."""

    def __init__(self, cfg, bm_v, n_tokens=None, capacity=None, **kw):
        self.k = Case(cfg, n_tokens=n_tokens, capacity=capacity, **kw)
        k = self.k
        self.cfg = cfg
        d = cfg.head_dim
        self.pv = kv.value_params(d, bm_v, cfg.qjl_m)
        self.Sv = value_projection(cfg) if cfg.qjl_m else None
        V = k.V if k.T > 0 else np.zeros((k.V.shape[0], k.V.shape[1], 1, d), np.float16)
        self.v_tables = kv.value_tables(V.astype(np.float64), bm_v)
        n_seq, n_kv = k.K.shape[:2]
        self.v_fields = [[kv.encode_values(k.V[b, h].astype(np.float64), self.v_tables[h][0],
                                           self.v_tables[h][1],
                                           None if self.Sv is None else self.Sv[h], self.pv)
                          for h in range(n_kv)] for b in range(n_seq)]

    def oracle_v_codes(self):
        k = self.k
        n_seq, n_kv = k.K.shape[:2]
        out = np.zeros((n_seq, n_kv, k.cap * layout.record_bytes(self.pv)), dtype=np.uint8)
        for b in range(n_seq):
            for h in range(n_kv):
                layout.pack_stream(self.v_fields[b][h], self.pv, k.cap, 0, out[b, h])
        return out

    def oracle_out(self):
        k = self.k
        out, _ = kv.decode_kv(k.q, k.oracle_fields(), self.v_fields, k.tables, self.v_tables, k.S,
                              self.Sv, k.signs, k.perm_arg, k.p, self.pv)
        return out

    def gpu_decode(self, n_splits=0, codes_v=None):
        api = _api()
        k = self.k
        dev = k.dev_inputs()
        n_seq, n_kv = k.K.shape[:2]
        cv = to_dev(self.oracle_v_codes()) if codes_v is None else codes_v
        out = api.pgkq_kv_decode_attn(
            lib_params(k.p), lib_params(self.pv), q_tensor(k.q, self.cfg.q_dtype),
            to_dev(k.oracle_codes()), cv, n_kv, k.cap, dev["signs"], dev["perm"], dev["codebook"],
            dev["S"], to_dev(codebook_array(self.v_tables)),
            to_dev(self.Sv) if self.Sv is not None else None, n_tokens=k.T, n_splits=n_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy()


KV_CASES = {
    "k3v3_d64_nanogpt": (CONFIGS["nano_t128"], 3, {}),
    "k3v3_d64_b2": (CONFIGS["nano_b64_t512"].with_(n_seq=2), 3, {}),
    "k3v3_d128_gqa": (CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_tokens=1000), 3, {}),
    "k2v2_d128": (CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=700, b_main=2, b_angle=1), 2, {}),
    "k4v4_d128_long": (CONFIGS["gqa_b1_t131k"].with_(n_tokens=3000), 4, {}),
    "k3v2_d128": (CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=700), 2, {}),
    "k4v2_d128": (CONFIGS["gqa_b1_t131k"].with_(n_tokens=900), 2, {}),
    "k4v4_d64_noqjl": (CONFIGS["nano_b64_t512_b4"].with_(n_seq=2), 4, {}),
    "k3v3_reorder": (CONFIGS["gqa_b16_t32k_encode"].with_(n_seq=1, n_tokens=600), 3, {"reorder": True}),
}


@pytest.mark.parametrize("name", list(KV_CASES))
def test_kv_decode_matches_oracle(name):
    cfg, bm_v, kw = KV_CASES[name]
    case = KVCase(cfg, bm_v, **kw)
    want = case.oracle_out()
    for ns in (0, 1, 7):
        err = float(np.abs(case.gpu_decode(ns) - want).max())
        print(name, ns, err)
        assert err <= OUT_TOL, (name, ns, err)


@pytest.mark.parametrize("name", ["k3v3_d64_b2", "k3v3_d128_gqa", "k4v4_d128_long", "k4v4_d64_noqjl"])
def test_kv_value_encode_matches_oracle(name):
    """pgkq_encode on V with the value parameters (no transform) writes the value
    records the oracle defines (code-parity bar), and decoding them gives the
    oracle output."""
    api = _api()
    cfg, bm_v, kw = KV_CASES[name]
    case = KVCase(cfg, bm_v, **kw)
    k = case.k
    dev = k.dev_inputs()
    cv = api.pgkq_encode(lib_params(case.pv), k_tensor(k.V), dev["signs"], None,
                         to_dev(codebook_array(case.v_tables)),
                         to_dev(case.Sv) if case.Sv is not None else None, capacity=k.cap)
    torch.cuda.synchronize()
    got = cv.cpu().numpy()
    counts = {}
    n_seq, n_kv = k.K.shape[:2]
    for b in range(n_seq):
        for h in range(n_kv):
            u = layout.unpack_stream(got[b, h], case.pv, k.cap, k.T)
            merge_counts(counts, classify(case.v_fields[b][h], u, case.v_tables[h][1],
                                          None if case.Sv is None else case.Sv[h], case.pv))
    print(name, counts)
    assert_code_parity(counts)
    err = float(np.abs(case.gpu_decode(0, codes_v=cv) - case.oracle_out()).max())
    assert err <= OUT_TOL, err


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_kv_group_sizes(group):
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_kv=4, n_q=4 * group, n_tokens=500)
    case = KVCase(cfg, 3)
    err = float(np.abs(case.gpu_decode(0) - case.oracle_out()).max())
    assert err <= OUT_TOL, err


@pytest.mark.parametrize("base,bm_v", [("nano_b64_t512", 3), ("nano_b64_t512_b4", 4),
                                       ("gqa_b16_t32k", 2), ("gqa_b1_t131k", 4)])
def test_kv_eight_heads_per_kv_head(base, bm_v):
    """8 query heads per kv-head: a lane holds 4 value channels instead of 8
    (d64 and d128, with and without the sketch, value widths 2 to 4), several
    splits and a ragged length."""
    cfg = CONFIGS[base].with_(n_seq=1, n_kv=2, n_q=16, n_tokens=450)
    case = KVCase(cfg, bm_v)
    want = case.oracle_out()
    for ns in (0, 1, 5):
        err = float(np.abs(case.gpu_decode(ns) - want).max())
        assert err <= OUT_TOL, (base, bm_v, ns, err)


@pytest.mark.parametrize("T", [1, 63, 65, 777])
def test_kv_ragged_lengths(T):
    case = KVCase(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=1000), 3, n_tokens=T, capacity=1024)
    want = case.oracle_out()
    for ns in (0, 3, 9):
        err = float(np.abs(case.gpu_decode(ns) - want).max())
        assert err <= OUT_TOL, (T, ns, err)


def test_kv_garbage_beyond_the_cache_is_ignored():
    """Slots past n_tokens may hold any bits (a norm that reads as NaN or inf
    included): they carry no weight."""
    case = KVCase(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=1000), 3, n_tokens=700, capacity=1024)
    cv = case.oracle_v_codes()
    rng = np.random.default_rng(0)
    k = case.k
    rb = layout.record_bytes(case.pv)
    words = cv.reshape(cv.shape[0], cv.shape[1], -1)
    W = layout.n_words(case.pv)
    for b in range(cv.shape[0]):
        for h in range(cv.shape[1]):
            w = words[b, h][: W * 4 * k.cap].view(np.uint32).reshape(W, k.cap)
            w[:, 700:] = rng.integers(0, 2 ** 32, size=(W, k.cap - 700), dtype=np.uint32)
            nu = words[b, h][W * 4 * k.cap:].view(np.uint16)
            nu[700:] = 0x7E00  # NaN
    assert rb * k.cap == words.shape[-1]
    out = case.gpu_decode(0, codes_v=to_dev(cv))
    assert np.isfinite(out).all()
    assert float(np.abs(out - case.oracle_out()).max()) <= OUT_TOL
