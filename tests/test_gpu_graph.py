"""The decode entry points under HIP graph capture.

The library only enqueues kernels on the caller's stream (no allocation,
memset or synchronization inside a call, workspaces come from the caller), so
a serving loop can capture a decode call into a graph and replay it.  Each
case captures one call, then replays the graph several times with eager work
and synchronizations in between; every replay must equal the eager call on
the same inputs bit for bit, also after a query was overwritten in place
(the graph reads the current contents of its buffers).  Covered: the PGKQ
decode (split and single-workgroup launches), the fused append + decode step,
the PGKQ-KV decode and the FP16-cache comparator.
"""

import numpy as np
import pytest
import torch

from synth import CONFIGS

from gpu_cases import Case, k_tensor, lib_params, q_tensor, to_dev, v_cache, value_capacity
from parity_util import codebook_array

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from compressed_cache_decode_pgkq_amd import _lib
    _lib.lib()


def _api():
    import compressed_cache_decode_pgkq_amd as api
    return api


def _capture(call):
    """call() once on a side stream (warm-up), then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def _replays_match(g, out, want, n=4):
    for _ in range(n):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want)


@pytest.mark.parametrize("name,n_splits", [("gqa_b16_t32k", 3), ("gqa_b16_t32k", 0), ("nano_b64_t512", 0)])
def test_decode_attn_replays_in_a_graph(name, n_splits):
    """Split launch (preparation, scan, merge) and the single-workgroup launch
    whose scan prepares the query itself."""
    api = _api()
    cfg = CONFIGS[name].with_(n_seq=2, n_tokens=700)
    case = Case(cfg)
    dev = case.dev_inputs()
    codes = to_dev(case.oracle_codes())
    p = lib_params(case.p)
    q = q_tensor(case.q, cfg.q_dtype)
    n_seq, n_q, d = q.shape
    ws = torch.empty(api.pgkq_decode_workspace_bytes(p, n_seq, n_q, cfg.n_kv, case.T, n_splits),
                     dtype=torch.uint8, device=q.device)
    out_e = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    out_g = torch.empty_like(out_e)

    def call(out):
        api.pgkq_decode_attn(p, q, codes, dev["V"], dev["signs"], dev["perm"], dev["codebook"],
                             dev["S"], n_tokens=case.T, n_splits=n_splits, out=out, workspace=ws)

    call(out_e)
    torch.cuda.synchronize()
    g = _capture(lambda: call(out_g))
    _replays_match(g, out_g, out_e)
    # a new query written into the captured buffer
    q.copy_(torch.flip(q, dims=[1]))
    call(out_e)
    torch.cuda.synchronize()
    _replays_match(g, out_g, out_e)


def test_decode_step_replays_in_a_graph():
    """The fused append + decode: every replay rewrites the same slot with the
    same token and attends over the grown cache."""
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_tokens=701)
    full = Case(cfg)
    T = 700
    case = Case(cfg, n_tokens=T, capacity=full.cap)
    dev = case.dev_inputs()
    codes = to_dev(case.oracle_codes())
    p = lib_params(case.p)
    q = q_tensor(case.q, cfg.q_dtype)
    k_new = k_tensor(full.K[:, :, T].copy())
    v_new = to_dev(full.V[:, :, T].copy().astype("float16"))
    n_seq, n_q, d = q.shape
    ws = torch.empty(api.pgkq_decode_workspace_bytes(p, n_seq, n_q, cfg.n_kv, T + 1, 0),
                     dtype=torch.uint8, device=q.device)
    out_e = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    out_g = torch.empty_like(out_e)

    def call(out):
        api.pgkq_decode_step(p, q, k_new, v_new, codes, dev["V"], T, dev["signs"], dev["perm"],
                             dev["codebook"], dev["S"], out=out, workspace=ws)

    call(out_e)
    torch.cuda.synchronize()
    g = _capture(lambda: call(out_g))
    _replays_match(g, out_g, out_e)


@pytest.mark.parametrize("n_q,n_splits", [(32, 3), (64, 3), (32, 0)])
def test_kv_decode_replays_in_a_graph(n_q, n_splits):
    """PGKQ-KV (values coded too): 4 query heads per kv-head (sketch sums on
    the matrix cores) and 8 (sketch sums on the vector ALU)."""
    from test_gpu_kv import KVCase
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_tokens=700, n_q=n_q)
    case = KVCase(cfg, 3)
    k = case.k
    dev = k.dev_inputs()
    ck = to_dev(k.oracle_codes())
    cv = to_dev(case.oracle_v_codes())
    pk, pv = lib_params(k.p), lib_params(case.pv)
    q = q_tensor(k.q, cfg.q_dtype)
    n_seq, _, d = q.shape
    cbv = to_dev(codebook_array(case.v_tables))
    Sv = to_dev(case.Sv)
    ws = torch.empty(api.pgkq_kv_decode_workspace_bytes(pk, pv, n_seq, n_q, cfg.n_kv, k.T, n_splits),
                     dtype=torch.uint8, device=q.device)
    out_e = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    out_g = torch.empty_like(out_e)

    def call(out):
        api.pgkq_kv_decode_attn(pk, pv, q, ck, cv, cfg.n_kv, k.cap, dev["signs"], dev["perm"],
                                dev["codebook"], dev["S"], cbv, Sv, n_tokens=k.T, n_splits=n_splits,
                                out=out, workspace=ws)

    call(out_e)
    torch.cuda.synchronize()
    g = _capture(lambda: call(out_g))
    _replays_match(g, out_g, out_e)


@pytest.mark.parametrize("n_splits", [3, 0])
def test_fp16_decode_replays_in_a_graph(n_splits):
    """The FP16-cache comparator."""
    from synth import make_inputs
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=2, n_tokens=700)
    inp = make_inputs(cfg)
    T = cfg.n_tokens
    cap = value_capacity(T)
    n_seq, n_kv, d = cfg.n_seq, cfg.n_kv, cfg.head_dim
    Kp = np.zeros((n_seq, n_kv, cap, d), np.float16)
    Kp[:, :, :T] = inp["K"][:, :, :T].astype(np.float16)
    K16 = to_dev(Kp)
    V16 = v_cache(inp["V"][:, :, :T], cap)
    q = q_tensor(inp["q"], cfg.q_dtype)
    n_q = q.shape[1]
    ws = torch.empty(api.pgkq_fp16_decode_workspace_bytes(d, n_seq, n_q, n_kv, T, n_splits),
                     dtype=torch.uint8, device=q.device)
    out_e = torch.empty((n_seq, n_q, d), dtype=torch.float32, device=q.device)
    out_g = torch.empty_like(out_e)

    def call(out):
        api.pgkq_fp16_decode_attn(q, K16, V16, n_tokens=T, n_splits=n_splits, out=out, workspace=ws)

    call(out_e)
    torch.cuda.synchronize()
    g = _capture(lambda: call(out_g))
    _replays_match(g, out_g, out_e)
