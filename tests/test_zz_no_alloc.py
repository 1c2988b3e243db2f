"""pgkq_decode_attn_noalloc (the decode entry point for callers that cannot
allocate) against pgkq_decode_attn: two calls in a row on one GPU, the second
on a smaller cache, both through the C ABI.  The two entry points run the same
kernels on the same inputs, so the outputs must agree bit for bit; both are
also held to the oracle's bar (outputs within 1e-3)."""

import numpy as np
import pytest
import torch

from synth import CONFIGS

from gpu_cases import OUT_TOL, Case, Guarded, lib_params, q_tensor, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from compressed_cache_decode_pgkq_amd import _lib
    _lib.lib()


def test_noalloc_decode_equals_decode_attn_on_two_calls():
    import compressed_cache_decode_pgkq_amd as api
    cases = [
        (Case(CONFIGS["gqa_b16_t32k"].with_(n_seq=3, n_tokens=1500)), 0),
        (Case(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_kv=2, n_q=8, n_tokens=300)), 3),
    ]
    for case, n_splits in cases:
        dev = case.dev_inputs()
        p = lib_params(case.p)
        q = q_tensor(case.q, case.cfg.q_dtype)
        codes = to_dev(case.oracle_codes())
        n_seq, n_q, d = case.q.shape
        ref = api.pgkq_decode_attn(p, q, codes, dev["V"], dev["signs"], dev["perm"], dev["codebook"],
                                   dev["S"], n_tokens=case.T, n_splits=n_splits)
        out = Guarded((n_seq, n_q, d), torch.float32)
        api.pgkq_decode_attn_noalloc(p, q, codes, dev["V"], dev["signs"], dev["perm"],
                                     dev["codebook"], dev["S"], out.t, n_tokens=case.T,
                                     n_splits=n_splits)
        torch.cuda.synchronize()
        out.check("out")
        assert torch.equal(out.t, ref), float((out.t - ref).abs().max())
        oracle, _ = case.oracle_decode()
        err = float(np.max(np.abs(out.t.cpu().numpy() - oracle)))
        print(f"n_seq {n_seq} T {case.T} splits {n_splits}: max-abs vs oracle {err:.2e}")
        assert err <= OUT_TOL
