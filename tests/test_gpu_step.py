"""GPU parity of the decode step (pgkq_decode_step): the new token's key is
encoded into the cache and its value copied inside the decode call, then
attention runs over the grown cache.  Checked against the oracle with the
codebook calibrated once on the whole key sequence (the table of a live cache
does not move while it grows):

* the appended record obeys the code-parity bar (bit-exact except G15
  boundary cases), as does every earlier record;
* the appended value row equals v_new exactly;
* the output matches the oracle's decode over the grown cache within 1e-3.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import attn, layout
from synth import CONFIGS

from gpu_cases import Case, k_tensor, lib_params, q_tensor, to_dev, untile_values, v_cache, value_capacity
from parity_util import assert_code_parity, classify, merge_counts

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


def _prefix(f, t):
    return dataclasses.replace(f, **{k.name: getattr(f, k.name)[:t] for k in dataclasses.fields(f)})


def _oracle_out(case, t):
    f = case.oracle_fields()
    n_seq, n_kv = case.K.shape[:2]
    fp = [[_prefix(f[b][h], t) for h in range(n_kv)] for b in range(n_seq)]
    out, _ = attn.decode_cache(case.q, fp, case.V[:, :, :t], case.tables, case.S, case.signs,
                               case.perm_arg, case.p)
    return out


def _counts(case, got, t):
    f = case.oracle_fields()
    counts = {}
    n_seq, n_kv = case.K.shape[:2]
    for b in range(n_seq):
        for h in range(n_kv):
            u = layout.unpack_stream(got[b, h], case.p, case.cap, t)
            merge_counts(counts, classify(_prefix(f[b][h], t), u, case.tables[h][1],
                                          None if case.S is None else case.S[h], case.p))
    return counts


STEP_CASES = {
    "d64_qjl_f32": (CONFIGS["nano_b64_t512"].with_(n_seq=2, n_tokens=300), {}),
    "d64_noqjl": (CONFIGS["nano_b64_t512_b4"].with_(n_seq=2, n_tokens=300), {}),
    "d128_qjl_f16": (CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_tokens=700), {}),
    "d128_reorder": (CONFIGS["gqa_b16_t32k_encode"].with_(n_seq=1, n_tokens=500), {"reorder": True}),
    "d128_b4": (CONFIGS["gqa_b1_t131k"].with_(n_tokens=900), {}),
    "no_hadamard": (CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=400), {"hadamard": False}),
    # the preparation launch is a (sequence, row) grid: the appending
    # workgroups take the first n_kv rows of each sequence, the query
    # preparation the n_q rows after them; group sizes 1, 2 and 8, and more
    # than two sequences so that the sequence axis of that grid is exercised
    "d128_g2": (CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_kv=4, n_q=8, n_tokens=200), {}),
    "d128_g8": (CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_kv=2, n_q=16, n_tokens=300), {}),
    "d128_g1_5seq": (CONFIGS["gqa_b16_t32k"].with_(n_seq=5, n_kv=3, n_q=3, n_tokens=150), {}),
    "d64_g4_3seq": (CONFIGS["nano_b64_t512"].with_(n_seq=3, n_kv=2, n_q=8, n_tokens=100), {}),
}


@pytest.mark.parametrize("name", list(STEP_CASES))
def test_decode_step_appends_then_attends(name):
    cfg, kw = STEP_CASES[name]
    api = _api()
    case = Case(cfg, capacity=value_capacity(cfg.n_tokens + 1), **kw)
    T = case.T
    dev = case.dev_inputs()
    p = lib_params(case.p)
    n_seq, n_kv, _, d = case.K.shape
    codes = torch.zeros((n_seq, n_kv, case.cap * layout.record_bytes(case.p)), dtype=torch.uint8,
                        device="cuda:0")
    api.pgkq_encode(p, k_tensor(case.K[:, :, :T - 1]), dev["signs"], dev["perm"], dev["codebook"],
                    dev["S"], codes=codes, capacity=case.cap)
    Vz = case.V.copy()
    Vz[:, :, T - 1:] = 0
    Vd = v_cache(Vz, case.cap)
    k_new = k_tensor(np.ascontiguousarray(case.K[:, :, T - 1]))
    v_new = to_dev(np.ascontiguousarray(case.V[:, :, T - 1]))
    out = api.pgkq_decode_step(p, q_tensor(case.q, cfg.q_dtype), k_new, v_new, codes, Vd, T - 1,
                               dev["signs"], dev["perm"], dev["codebook"], dev["S"])
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    counts = _counts(case, got, T)
    print(name, counts)
    assert_code_parity(counts)
    rows = untile_values(Vd.cpu().numpy())
    assert np.array_equal(rows[:, :, T - 1], v_new.cpu().numpy())
    assert not rows[:, :, T:].any()                    # nothing beyond the slot
    err = float(np.abs(out.cpu().numpy() - _oracle_out(case, T)).max())
    assert err <= OUT_TOL, err


def test_decode_step_loop_matches_oracle_every_step():
    """Six consecutive steps on one cache: after each, the output equals the
    oracle's decode over the cache grown so far (auto and fixed splits)."""
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=506)
    case = Case(cfg, capacity=512)
    dev = case.dev_inputs()
    p = lib_params(case.p)
    n_seq, n_kv, _, d = case.K.shape
    T0 = 500
    codes = torch.zeros((n_seq, n_kv, case.cap * layout.record_bytes(case.p)), dtype=torch.uint8,
                        device="cuda:0")
    api.pgkq_encode(p, k_tensor(case.K[:, :, :T0]), dev["signs"], dev["perm"], dev["codebook"],
                    dev["S"], codes=codes, capacity=case.cap)
    Vz = case.V.copy()
    Vz[:, :, T0:] = 0
    Vd = v_cache(Vz, case.cap)
    q = q_tensor(case.q, cfg.q_dtype)
    for i, t in enumerate(range(T0, case.T)):
        out = api.pgkq_decode_step(p, q, k_tensor(np.ascontiguousarray(case.K[:, :, t])),
                                   to_dev(np.ascontiguousarray(case.V[:, :, t])), codes, Vd, t,
                                   dev["signs"], dev["perm"], dev["codebook"], dev["S"],
                                   n_splits=(0, 3)[i % 2])
        torch.cuda.synchronize()
        err = float(np.abs(out.cpu().numpy() - _oracle_out(case, t + 1)).max())
        assert err <= OUT_TOL, (t, err)
    assert_code_parity(_counts(case, codes.cpu().numpy(), case.T))


def test_decode_step_equals_encode_then_decode_when_codes_agree():
    """Where the appended record equals the bulk encoder's, the step's output is
    the output of pgkq_encode + pgkq_decode_attn on the same cache, bit for bit."""
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_tokens=333)
    case = Case(cfg, capacity=352)
    dev = case.dev_inputs()
    p = lib_params(case.p)
    n_seq, n_kv, T, d = case.K.shape
    rb = layout.record_bytes(case.p)
    full = api.pgkq_encode(p, k_tensor(case.K), dev["signs"], dev["perm"], dev["codebook"],
                           dev["S"], capacity=case.cap)
    codes = torch.zeros((n_seq, n_kv, case.cap * rb), dtype=torch.uint8, device="cuda:0")
    api.pgkq_encode(p, k_tensor(case.K[:, :, :T - 1]), dev["signs"], dev["perm"], dev["codebook"],
                    dev["S"], codes=codes, capacity=case.cap)
    Vd = dev["V"].clone()
    q = q_tensor(case.q, cfg.q_dtype)
    out_step = api.pgkq_decode_step(p, q, k_tensor(np.ascontiguousarray(case.K[:, :, T - 1])),
                                    to_dev(np.ascontiguousarray(case.V[:, :, T - 1])), codes, Vd,
                                    T - 1, dev["signs"], dev["perm"], dev["codebook"], dev["S"],
                                    n_splits=2)
    out_ref = api.pgkq_decode_attn(p, q, full, dev["V"], dev["signs"], dev["perm"], dev["codebook"],
                                   dev["S"], n_tokens=T, n_splits=2)
    torch.cuda.synchronize()
    if torch.equal(codes, full):
        assert torch.equal(out_step, out_ref)
    else:  # a boundary case decided differently by the two encoders: within the bar
        assert float((out_step - out_ref).abs().max()) <= OUT_TOL
