"""Edge cases of the code decisions on the GPU: pairs exactly on radius
thresholds and on angle-cell edges, signed zeros, the zero pair, subnormal and
very large components (residual norm saturating in fp16).

With the transform off (the ablation setting) a key's pairs reach the polar
step unchanged, so exact edge inputs can be built.  The GPU codes are checked
against the decision rules the readings state, evaluated here in exact
rational arithmetic:
  radius : code = #{j : T_j < r}, i.e. T_j^2 < x^2 + y^2 (a tie takes the
           lower code), T_j the fp32 thresholds;
  angle  : 2^b cells of width 2 pi / 2^b from -pi, half-open [e_k, e_k+1)
           counter-clockwise; theta = pi counts as -pi; the zero pair counts as
           theta = 0.  For b <= 3 every edge direction is a multiple of pi/4,
           so membership is decided by exact cross-product signs.
The float64 oracle takes the same decisions through atan2 and hypot; on these
adversarial inputs any disagreement with it must be a decision-boundary case.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codebook, encode, layout
from oracle.encode import Params

from gpu_cases import k_tensor, lib_params, to_dev
from parity_util import classify, codebook_array

pytestmark = pytest.mark.gpu

# directions of the 9 octant edges -pi + k pi/4, k = 0..8, scaled to integers
_EDGES = [(-1, 0), (-1, -1), (0, -1), (1, -1), (1, 0), (1, 1), (0, 1), (-1, 1), (-1, 0)]


def _cross(u, x, y):
    return u[0] * y - u[1] * x


def exact_octant(x: float, y: float) -> int:
    X, Y = Fraction(x), Fraction(y)
    if X == 0 and Y == 0:
        return 4  # theta = 0
    for k in range(8):
        if _cross(_EDGES[k], X, Y) >= 0 and _cross(_EDGES[k + 1], X, Y) < 0:
            return k
    raise AssertionError("no cell")


def exact_radius_code(x: float, y: float, thresholds32) -> int:
    r2 = Fraction(x) ** 2 + Fraction(y) ** 2
    return sum(1 for t in np.asarray(thresholds32, np.float32) if Fraction(float(t)) ** 2 < r2)


def _edge_pairs(thresholds32):
    f32 = np.float32
    pairs = [(0.0, 0.0), (1.0, 0.0), (0.0, 1.0), (-1.0, 0.0), (0.0, -1.0),
             (1.5, 1.5), (-1.5, 1.5), (-1.5, -1.5), (1.5, -1.5),
             (-0.0, 0.0), (0.0, -0.0), (-0.0, -0.0), (-2.0, -0.0), (-2.0, 0.0), (-0.0, 3.0),
             (1e-40, 0.0), (0.0, -1e-40), (-1e-40, 1e-40), (3e4, 3e4), (-6e4, 1.0), (1e6, -1e6)]
    for t in np.asarray(thresholds32, np.float32):
        up = float(np.nextafter(f32(t), f32(np.inf)))
        dn = float(np.nextafter(f32(t), f32(0)))
        pairs += [(float(t), 0.0), (0.0, -float(t)), (up, 0.0), (dn, 0.0), (-float(t), -0.0)]
    return pairs


@pytest.mark.parametrize("b_main,qjl", [(3, 64), (2, 0), (4, 64)])
def test_encode_edge_pairs_follow_the_stated_rules(b_main, qjl):
    import compressed_cache_decode_pgkq_amd as api
    d = 64
    p = Params(d, b_main, b_main - 1, qjl, False)
    c, t = codebook.lloyd_max_beta(d, b_main)
    lv, th = codebook.scaled_table(c, t, 2.0, d)
    pairs = _edge_pairs(th)
    n = d // 2
    n_keys = (len(pairs) + n - 1) // n + 1
    rng = np.random.default_rng(b_main)
    # every edge pair once, the rest of the slots random; plus one key of
    # random pairs and one all-zero key
    flat = pairs + [tuple(rng.standard_normal(2)) for _ in range(n_keys * n - len(pairs))]
    K = np.array(flat, dtype=np.float32).reshape(n_keys, d)
    K = np.concatenate([K, np.zeros((1, d), np.float32)])
    N = K.shape[0]
    S = rng.standard_normal((qjl, d)).astype(np.float32) if qjl else None
    signs = np.ones((1, d), np.int8)
    cap = N + (N & 1)
    codes = api.pgkq_encode(lib_params(p), k_tensor(K[None, None]), to_dev(signs), None,
                            to_dev(codebook_array([(lv, th)])), to_dev(S[None]) if qjl else None,
                            capacity=cap)
    torch.cuda.synchronize()
    got = layout.unpack_stream(codes[0, 0].cpu().numpy(), p, cap, N)
    bad = []
    for tkn in range(N):
        for i in range(n):
            x, y = float(K[tkn, 2 * i]), float(K[tkn, 2 * i + 1])
            rc = exact_radius_code(x, y, th)
            ac = exact_octant(x, y) >> (3 - p.b_angle)
            if got["rc"][tkn, i] != rc or got["ac"][tkn, i] != ac:
                bad.append((x, y, rc, ac, int(got["rc"][tkn, i]), int(got["ac"][tkn, i])))
    assert not bad, bad[:10]
    # the oracle (atan2 / hypot in float64) agrees up to boundary cases
    f = encode.encode_keys(K, signs[0], None, lv, th, S, p)
    res = classify(f, got, th, S, p)
    print(res)
    assert res["unexplained"] == 0, res
    # saturated residual norms stay finite: fp16 maximum, not infinity
    if qjl:
        assert np.all(np.isfinite(got["nu"].astype(np.float32)))
