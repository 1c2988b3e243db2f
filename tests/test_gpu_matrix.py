"""GPU parity over every parameter combination the C ABI accepts.

pgkq_encode, pgkq_decode_attn and pgkq_estimate_logits accept head_dim 64 or
128, b_main 2, 3 or 4 (b_angle = b_main - 1, "PGKQ pipeline" step (3) of the
EdgeLLM-Nano paper page), QJL on or off and the Hadamard transform on or off
(the 2x2 of "Ablations for PGKQ"), keys in fp32 or fp16, and 1, 2, 4 or 8
query heads per kv-head.  Each combination is its own kernel instance (LDS
table layout, lanes per key, lookup grouping), so each is compared with the
oracle here on a small ragged case:

* encode (d x b_main x QJL x key dtype x Hadamard, 48 cases, half of them with
  the channel reorder): codes under the boundary classifier;
* decode (d x b_main x QJL x group x Hadamard, 48 cases, each with the
  automatic split and with one workgroup per stream, which for groups up to 2
  is the path where the scan prepares the query itself): outputs within 1e-3
  and logits within 2e-3 ||q|| ||k||, with guard bands around the outputs and
  workspaces.
"""

import itertools

import numpy as np
import pytest
import torch

from synth import CONFIGS

from gpu_cases import Case, check_decode, code_counts, gpu_encode
from parity_util import assert_code_parity

pytestmark = pytest.mark.gpu

T_SMALL = 333          # five 64-token tiles and a ragged tail


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    from compressed_cache_decode_pgkq_amd import _lib
    _lib.lib()


def _cfg(d, bm, qjl, group=1, k_dtype=None):
    base = CONFIGS["nano_b64_t512"] if d == 64 else CONFIGS["gqa_b16_t32k"]
    return base.with_(n_seq=2, n_kv=2, n_q=2 * group, n_tokens=T_SMALL, b_main=bm,
                      b_angle=bm - 1, qjl_m=d if qjl else 0,
                      k_dtype=k_dtype or base.k_dtype)


ENCODE = list(itertools.product([64, 128], [2, 3, 4], [True, False], ["f32", "f16"], [True, False]))


@pytest.mark.parametrize("d,bm,qjl,kd,had", ENCODE,
                         ids=[f"d{d}-b{b}-{'qjl' if q else 'noqjl'}-{k}-{'ht' if h else 'id'}"
                              for d, b, q, k, h in ENCODE])
def test_encode_every_accepted_combination(d, bm, qjl, kd, had):
    reorder = (bm + (kd == "f16")) % 2 == 0
    case = Case(_cfg(d, bm, qjl, k_dtype=kd), hadamard=had, reorder=reorder)
    got = gpu_encode(case)
    counts = code_counts(case, got)
    print(d, bm, qjl, kd, had, reorder, counts)
    assert_code_parity(counts)
    if counts["mismatch"] == 0:
        assert np.array_equal(got, case.oracle_codes())


DECODE = list(itertools.product([64, 128], [2, 3, 4], [True, False], [1, 2, 4, 8], [True, False]))


@pytest.mark.parametrize("d,bm,qjl,group,had", DECODE,
                         ids=[f"d{d}-b{b}-{'qjl' if q else 'noqjl'}-g{g}-{'ht' if h else 'id'}"
                              for d, b, q, g, h in DECODE])
def test_decode_every_accepted_combination(d, bm, qjl, group, had):
    case = Case(_cfg(d, bm, qjl, group=group), hadamard=had)
    check_decode(case, n_splits=0)
    check_decode(case, n_splits=1)
