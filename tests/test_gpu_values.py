"""The fp16 value cache in 32-token tiles.

* pgkq_pack_values / pgkq_unpack_values against the layout written out in
  NumPy (tests/gpu_cases.tile_values), byte for byte, including partial
  8-token groups at both ends of the written slot range and the slots outside
  it staying untouched;
* slots at or beyond n_tokens may hold any bits (NaN, infinities): the decode
  paths that read fp16 values (PGKQ, RTN control, FP16 comparator) give the
  oracle's output regardless, for ragged lengths inside a tile.
"""

import numpy as np
import pytest
import torch

from oracle import attn, rtn
from synth import CONFIGS, make_inputs

from gpu_cases import (Case, lib_params, q_tensor, tile_values, to_dev, untile_values,
                       value_capacity)

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


@pytest.mark.parametrize("d", [64, 128, 16, 80])
@pytest.mark.parametrize("T,cap,off", [(100, 128, 0), (1, 32, 0), (37, 96, 5), (64, 64, 0),
                                       (21, 64, 43), (0, 32, 3)])
def test_pack_unpack_match_the_layout(d, T, cap, off):
    api = _api()
    rng = np.random.default_rng(d * 1000 + T)
    rows = rng.standard_normal((2, 3, T, d)).astype(np.float16)
    sentinel = rng.standard_normal((2, 3, cap, d)).astype(np.float16)  # rows of the old contents
    cache = to_dev(tile_values(sentinel, cap))
    api.pgkq_pack_values(to_dev(rows), cache=cache, slot_offset=off)
    torch.cuda.synchronize()
    want_rows = sentinel.copy()
    want_rows[:, :, off:off + T] = rows
    got = cache.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), tile_values(want_rows, cap).view(np.uint16))
    back = api.pgkq_unpack_values(cache, n_tokens=T, slot_offset=off)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy().view(np.uint16), rows.view(np.uint16))
    assert np.array_equal(untile_values(got)[:, :, off:off + T], rows)


def test_pack_values_full_cache_of_the_decode_workload_sampled():
    """Packing the 32k-token cache of the benchmark workload (16 x 8 streams):
    sampled streams equal the NumPy layout."""
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k"]
    inp = make_inputs(cfg)
    V = inp["V"]
    Vt = api.pgkq_pack_values(to_dev(V))
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (7, 3), (15, 7)]:
        want = tile_values(V[b:b + 1, h:h + 1], cfg.n_tokens)
        assert np.array_equal(Vt[b:b + 1, h:h + 1].cpu().numpy(), want)


def _poison_tail(cache, T):
    """Slots [T, cap) of every stream of a tiled cache set to NaN / +inf / -inf
    bit patterns."""
    rows = untile_values(cache)
    n = rows.shape[2] - T
    pattern = np.array([0x7E00, 0x7C00, 0xFC00, 0xFFFF], dtype=np.uint16)
    rows[:, :, T:] = np.resize(pattern, rows[:, :, T:].size).reshape(rows[:, :, T:].shape).view(np.float16)
    assert n >= 0
    return tile_values(rows, rows.shape[2])


@pytest.mark.parametrize("T", [1, 33, 63, 250])
def test_pgkq_decode_ignores_garbage_past_the_cache(T):
    api = _api()
    case = Case(CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=256), n_tokens=T, capacity=256)
    dev = case.dev_inputs()
    Vbad = to_dev(_poison_tail(dev["V"].cpu().numpy(), T))
    want, _ = case.oracle_decode()
    for ns in (0, 3):
        out = api.pgkq_decode_attn(lib_params(case.p), q_tensor(case.q, case.cfg.q_dtype),
                                   to_dev(case.oracle_codes()), Vbad, dev["signs"], dev["perm"],
                                   dev["codebook"], dev["S"], n_tokens=T, n_splits=ns)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.isfinite(o).all()
        assert float(np.abs(o - want).max()) <= OUT_TOL


@pytest.mark.parametrize("T", [5, 70])
def test_rtn_and_fp16_decode_ignore_garbage_past_the_cache(T):
    api = _api()
    cfg = CONFIGS["gqa_b16_t32k"].with_(n_seq=1, n_tokens=128)
    inp = make_inputs(cfg)
    K, V, q = inp["K"][:, :, :T], inp["V"][:, :, :T], inp["q"]
    cap = value_capacity(T)
    Vbad = to_dev(_poison_tail(tile_values(V, cap), T))
    # RTN INT4 keys
    recs = rtn.pack_cache(K.astype(np.float64), 4, cap)
    out = api.pgkq_rtn_decode_attn(q_tensor(q, cfg.q_dtype), to_dev(recs), Vbad, 4, n_tokens=T)
    torch.cuda.synchronize()
    want, _ = rtn.decode_cache(q, K.astype(np.float64), V, 4)
    assert np.isfinite(out.cpu().numpy()).all()
    assert float(np.abs(out.cpu().numpy() - want).max()) <= OUT_TOL
    # fp16 keys
    K16 = np.zeros((1, cfg.n_kv, cap, cfg.head_dim), np.float16)
    K16[:, :, :T] = K
    out = api.pgkq_fp16_decode_attn(q_tensor(q, cfg.q_dtype), to_dev(K16), Vbad, n_tokens=T)
    torch.cuda.synchronize()
    ref, _ = attn.fp16_attention(q, K.astype(np.float16), V)
    assert np.isfinite(out.cpu().numpy()).all()
    assert float(np.abs(out.cpu().numpy() - ref).max()) <= OUT_TOL
