"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: values
printed on the EdgeLLM-Nano paper page (tests/golden/), closed forms, textbook
special cases, independent numerical routes (quadrature, brute force, a fast
transform written only for this test) and statistical laws.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.integrate as integrate
import scipy.optimize as optimize
import scipy.stats as stats

from oracle import accounting, attn, calibrate, codebook, encode, layout, rht, rtn
from oracle.encode import Params

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- P1 accounting

def test_p1_printed_byte_example():
    g = _golden("pages_accounting.json")["kv_example_128_tokens"]
    lh = g["n_layers"] * g["n_heads"]
    rb = layout.record_bytes(Params(g["head_dim"], g["b_main"], g["b_angle"], g["qjl_m"]))
    assert rb == 30
    assert accounting.key_record_bytes(g["head_dim"], g["b_main"], g["b_angle"], g["qjl_m"]) == 30
    cb = accounting.cache_bytes(lh, g["n_tokens"], g["head_dim"], g["b_main"], g["b_angle"], g["qjl_m"])
    assert cb["k"] == 92160
    assert cb["kv"] == g["pgkq_kv_bytes"]
    assert accounting.fp16_cache_bytes(lh, g["n_tokens"], g["head_dim"]) == g["fp16_kv_bytes"]
    assert round(g["fp16_kv_bytes"] / cb["kv"], 2) == g["reduction"]
    assert accounting.key_bits_per_element(g["head_dim"], g["b_main"], g["b_angle"], g["qjl_m"]) \
        == g["key_bits_per_element"]


def test_p1_bit_budget_and_ablation():
    g = _golden("pages_accounting.json")
    bb, ab = g["bit_budget"], g["ablation"]
    kb = accounting.key_bits_per_element(64, 3, 2, 64)
    assert kb == bb["key_bits_per_element"]
    avg = accounting.occupied_average_bpe(kb, 16.0, bb["ctx"], bb["occupied"])
    assert round(avg, 2) == bb["k_only_average_bpe"]
    assert accounting.key_bits_per_element(64, 3, 2, 0) == ab["without_qjl"]
    assert accounting.qjl_bits_per_element(64, 64) == ab["qjl_cost"]
    assert accounting.polar_bits_per_element(3, 2) + accounting.qjl_bits_per_element(64, 64) \
        == ab["with_qjl"]


def test_p1_rtn_and_pgkq_kv():
    g = _golden("pages_accounting.json")
    assert accounting.rtn_bits_per_element(3, 64) == g["rtn"]["int3_bpe"]
    assert accounting.rtn_bits_per_element(4, 64) == g["rtn"]["int4_bpe"]
    kv = g["pgkq_kv"]
    k2 = accounting.key_bits_per_element(64, 2, 1, 64)
    k4 = accounting.key_bits_per_element(64, 4, 3, 64)
    assert round(accounting.occupied_average_bpe(k2, k2), 2) == kv["k2v2_bpe"]
    assert round(accounting.occupied_average_bpe(k4, k4), 2) == kv["k4v4_bpe"]
    # K and V both at 30 B per token-head over the 128-token, 24-head example
    assert 2 * accounting.cache_bytes(24, 128, 64, 3, 2, 64, v_fp16=False)["k"] == kv["kv_bytes"]


def test_p1_record_sizes_of_the_measured_configs():
    assert layout.record_bytes(Params(64, 4, 3, 0)) == 28
    assert layout.record_bytes(Params(128, 3, 2, 128)) == 58
    assert layout.record_bytes(Params(128, 4, 3, 128)) == 74


# ------------------------------------------------------------------ P2 transform

def _fwht_reference(x):
    """Iterative butterfly Walsh-Hadamard transform (natural order), test-only."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(*y.shape[:-3], d)
        h *= 2
    return y


@pytest.mark.parametrize("d", [4, 8, 64, 128])
def test_p2_hadamard_invariants(d):
    H = rht.sylvester(d)
    assert np.array_equal(H @ H.T, d * np.eye(d))
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    popc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(H, (-1.0) ** popc)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, d))
    signs = rng.choice([-1, 1], size=d)
    perm = rng.permutation(d)
    kt = rht.forward(x, signs, perm)
    fast = _fwht_reference(x[:, perm] * signs) / math.sqrt(d)
    np.testing.assert_allclose(kt, fast, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(kt, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    q = rng.standard_normal(d)
    qt = rht.forward(q, signs, perm)
    np.testing.assert_allclose(kt @ qt, x @ q, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rht.inverse(kt, signs, perm), x, atol=1e-12)


def test_p2_fp16_inputs_transform_exactly():
    # for fp16 keys every partial sum of the dense product is exact in float64,
    # so the transform equals an exact rational computation
    from fractions import Fraction
    rng = np.random.default_rng(2)
    d = 16
    x = (rng.standard_normal(d) * np.exp(rng.standard_normal(d))).astype(np.float16)
    signs = rng.choice([-1, 1], size=d)
    H = rht.sylvester(d)
    got = rht.forward(x, signs) * math.sqrt(d)
    for i in range(d):
        exact = sum(Fraction(float(H[i, j])) * Fraction(float(x[j])) * signs[j] for j in range(d))
        assert Fraction(float(got[i])) == exact or abs(float(exact) - got[i]) <= 1e-15 * abs(float(exact))


# ------------------------------------------------------------------ P3 the prior

@pytest.mark.parametrize("d", [16, 64, 128])
def test_p3_pair_energy_follows_beta_prior(d):
    rng = np.random.default_rng(3 + d)
    n = d // 2
    k = rng.standard_normal((100000, d))
    signs = rng.choice([-1, 1], size=d)
    kt = rht.forward(k, signs)
    u = (kt[:, 0] ** 2 + kt[:, 1] ** 2) / np.sum(kt * kt, axis=1)
    res = stats.kstest(u, "beta", args=(1, n - 1))
    assert res.pvalue > 1e-3
    rho = np.sqrt(u * n)
    res2 = stats.kstest(rho, lambda r: codebook.rho_cdf(r, n))
    assert res2.pvalue > 1e-3


# ------------------------------------------------------------------ P4 codebook

@pytest.mark.parametrize("n", [2, 8, 32, 64])
def test_p4_density_cdf_and_moment_by_quadrature(n):
    top = math.sqrt(n)
    tot, _ = integrate.quad(lambda r: codebook.rho_pdf(r, n), 0, top, epsabs=1e-14, epsrel=1e-13)
    assert abs(tot - 1.0) < 1e-11
    e2, _ = integrate.quad(lambda r: r * r * codebook.rho_pdf(r, n), 0, top, epsabs=1e-14, epsrel=1e-13)
    assert abs(e2 - 1.0) < 1e-11
    for fa, fb in [(0.0, 0.2), (0.2, 0.5), (0.5, 0.8), (0.8, 1.0)]:
        a, b = fa * top, fb * top
        P, _ = integrate.quad(lambda r: codebook.rho_pdf(r, n), a, b, epsabs=1e-15, epsrel=1e-13)
        M, _ = integrate.quad(lambda r: r * codebook.rho_pdf(r, n), a, b, epsabs=1e-15, epsrel=1e-13)
        assert abs(codebook.partial_mass(a, b, n) - P) < 1e-12
        assert abs(codebook.partial_moment(a, b, n) - M) < 1e-12


@pytest.mark.parametrize("d,b", [(64, 3), (64, 4), (128, 3), (128, 4), (64, 2), (16, 2)])
def test_p4_lloyd_max_fixed_point(d, b):
    n = d // 2
    c, t, hist = codebook.lloyd_max_beta(d, b, history=True)
    L = 1 << b
    assert len(c) == L and len(t) == L - 1
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(t, 0.5 * (c[:-1] + c[1:]))
    edges = np.concatenate([[0.0], t, [math.sqrt(n)]])
    # centroid condition, by quadrature rather than by the closed form
    for j in range(L):
        P, _ = integrate.quad(lambda r: codebook.rho_pdf(r, n), edges[j], edges[j + 1],
                              epsabs=1e-15, epsrel=1e-13)
        M, _ = integrate.quad(lambda r: r * codebook.rho_pdf(r, n), edges[j], edges[j + 1],
                              epsabs=1e-15, epsrel=1e-13)
        assert abs(M / P - c[j]) < 1e-10
    h = np.array(hist)
    assert np.all(np.diff(h) <= 1e-14)  # non-increasing up to float64 rounding
    # uniqueness (log-concave density): an unrelated start reaches the same table
    c2, _ = codebook.lloyd_max_beta(d, b, init=np.linspace(0.05, 2.5, L))
    np.testing.assert_allclose(c2, c, atol=1e-9)


def test_p4_monte_carlo_distortion():
    rng = np.random.default_rng(44)
    d, b = 64, 3
    n = d // 2
    c, t = codebook.lloyd_max_beta(d, b)
    u = rng.beta(1, n - 1, size=4_000_000)
    rho = np.sqrt(n * u)
    idx = np.searchsorted(t, rho, side="left")
    err2 = (rho - c[idx]) ** 2
    D = codebook.distortion(c, t, n)
    sem = err2.std() / math.sqrt(err2.size)
    assert abs(err2.mean() - D) < 4 * sem


def test_p4_two_level_special_case_closed_form():
    # d = 4 (n = 2): u ~ Beta(1, 1) so f(rho) = rho on [0, sqrt 2].  Cells [0, t]
    # and [t, sqrt 2] have centroids 2t/3 and (2/3)(2 sqrt 2 - t^3)/(2 - t^2).
    top = math.sqrt(2.0)

    def g(tt):
        c0 = 2 * tt / 3
        c1 = (2.0 / 3.0) * (top ** 3 - tt ** 3) / (2 - tt ** 2)
        return 0.5 * (c0 + c1) - tt

    ts = optimize.brentq(g, 0.1, 1.4, xtol=1e-15)
    c, t = codebook.lloyd_max_beta(4, 1)
    assert abs(t[0] - ts) < 1e-11
    assert abs(c[0] - 2 * ts / 3) < 1e-11


def test_p4_rayleigh_limit():
    # as n grows rho tends to Rayleigh with E rho^2 = 1, f(rho) = 2 rho exp(-rho^2)
    def ray_lm(L):
        cdf = lambda r: 1 - math.exp(-r * r)
        mom = lambda a, b: integrate.quad(lambda r: 2 * r * r * math.exp(-r * r), a, b,
                                          epsabs=1e-15, epsrel=1e-13)[0]
        c = np.array([math.sqrt(-math.log(1 - (j + 0.5) / L)) for j in range(L)])
        for _ in range(20000):
            t = 0.5 * (c[:-1] + c[1:])
            e = np.concatenate([[0.0], t, [12.0]])
            cn = np.array([mom(e[j], e[j + 1]) / (cdf(e[j + 1]) - cdf(e[j])) for j in range(L)])
            if np.max(np.abs(cn - c)) < 1e-12:
                return cn
            c = cn
        return c

    lim = ray_lm(8)
    errs = [np.max(np.abs(codebook.lloyd_max_beta(d, 3)[0] - lim)) for d in (64, 128, 1024)]
    assert errs[0] > errs[1] > errs[2]
    # the Beta(1, n-1) prior approaches the Rayleigh law at rate 1/n, so does the table
    assert errs[2] < 1e-2
    assert 4.0 < errs[1] / errs[2] < 16.0


def test_p4_scaled_table_is_fp32_rounding_of_product():
    c, t = codebook.lloyd_max_beta(128, 3)
    s = 23.456789
    lv, th = codebook.scaled_table(c, t, s, 128)
    assert lv.dtype == np.float32 and th.dtype == np.float32
    sig = s / 8.0
    for j in range(8):
        assert lv[j] == np.float32(c[j] * sig)
    rec = codebook.pack_table(lv, th)
    assert rec.shape == (16,) and np.isinf(rec[-1])
    lv2, th2 = codebook.unpack_table(rec, 3)
    assert np.array_equal(lv2, lv) and np.array_equal(th2, th)


# ------------------------------------------------------- radius unit of the per-head table
# The table is built in rho units, rho = (r / ||k||) sqrt(d/2), and scaled into
# radius units by the head scale.  For keys of one fixed norm c the calibrated
# head scale is c, so the radius of a pair after the transform, r = rho c /
# sqrt(d/2), follows the Beta-prior law in those units exactly.  The checks
# below draw such keys, take the table the oracle builds for them
# (channel_sumsq -> head_scale -> scaled_table) and test physical statements
# about the sampled radii: the mass below every threshold, the centroid of every
# cell, and a KS test of the radii against the law implied by the table.


def _fixed_norm_radii(d, n_keys, seed, norm=3.7):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((n_keys, d))
    K = norm * g / np.linalg.norm(g, axis=1, keepdims=True)
    signs = rng.choice([-1, 1], size=d)
    kt = rht.forward(K, signs)
    # one pair per key (the pair index cycles), so the radii are independent
    i = np.arange(n_keys) % (d // 2)
    r = np.hypot(kt[np.arange(n_keys), 2 * i], kt[np.arange(n_keys), 2 * i + 1])
    return K, r


def _table_fits_radii(levels32, thresholds32, c, t, r, n):
    """(ok, details): the absolute table agrees with the sampled radii under the
    Beta-prior law within 5 standard errors at every threshold and cell, and the
    radii pass a KS test against the law in the table's own unit."""
    lv = np.asarray(levels32, dtype=np.float64)
    th = np.asarray(thresholds32, dtype=np.float64)
    N = r.size
    fails = []
    for j in range(len(th)):
        p = float(codebook.rho_cdf(t[j], n))
        frac = float(np.mean(r <= th[j]))
        se = math.sqrt(p * (1 - p) / N)
        if abs(frac - p) > 5 * se:
            fails.append(("mass", j, frac, p))
    cell = np.searchsorted(th, r, side="left")  # #{T_j < r}
    for j in range(len(lv)):
        rr = r[cell == j]
        if rr.size < 100:
            fails.append(("empty", j, rr.size))
            continue
        se = rr.std() / math.sqrt(rr.size)
        if abs(rr.mean() - lv[j]) > 5 * se:
            fails.append(("centroid", j, rr.mean(), lv[j], se))
    unit = lv[-1] / c[-1]
    ks = stats.kstest(r / unit, lambda x: codebook.rho_cdf(x, n))
    if ks.pvalue <= 1e-3:
        fails.append(("ks", ks.pvalue))
    return not fails, fails


@pytest.mark.parametrize("d", [64, 128])
def test_radius_unit_of_scaled_table_matches_the_prior(d):
    n = d // 2
    K, r = _fixed_norm_radii(d, 200_000, seed=1000 + d)
    c, t = codebook.lloyd_max_beta(d, 3)
    s_h = calibrate.head_scale(calibrate.channel_sumsq(K), K.shape[0])
    assert abs(s_h - 3.7) < 1e-12
    lv, th = codebook.scaled_table(c, t, s_h, d)
    ok, why = _table_fits_radii(lv, th, c, t, r, n)
    assert ok, why


@pytest.mark.parametrize("d", [64, 128])
def test_radius_unit_check_rejects_other_scalings(d):
    """The check above has the power to catch a wrong radius unit: s_h / sqrt(d)
    and s_h sqrt(d/2) in place of s_h / sqrt(d/2) both fail it."""
    n = d // 2
    K, r = _fixed_norm_radii(d, 200_000, seed=2000 + d)
    c, t = codebook.lloyd_max_beta(d, 3)
    s_h = calibrate.head_scale(calibrate.channel_sumsq(K), K.shape[0])
    # scaled_table divides by sqrt(d/2); feed it the head scale that yields the wrong unit
    for wrong in (s_h / math.sqrt(2.0), s_h * n):
        lv, th = codebook.scaled_table(c, t, wrong, d)
        ok, _ = _table_fits_radii(lv, th, c, t, r, n)
        assert not ok


def test_gqa_head_mapping_of_decode_cache_by_hand():
    """8 query heads over 2 kv-heads: heads 0-3 read kv-head 0 and heads 4-7 read
    kv-head 1 (query 3 -> kv 0, query 4 -> kv 1), each checked against attention
    computed explicitly on that kv-head's dequantized keys."""
    rng = np.random.default_rng(77)
    d, T = 16, 30
    p = Params(d, 3, 2, d)
    kv_of = [0, 0, 0, 0, 1, 1, 1, 1]
    K = rng.standard_normal((1, 2, T, d)) * np.array([1.0, 3.0])[None, :, None, None]
    V = rng.standard_normal((1, 2, T, d)) + np.array([-5.0, 5.0])[None, :, None, None]
    q = rng.standard_normal((1, 8, d))
    signs = rng.choice([-1, 1], size=(2, d))
    S = rng.standard_normal((2, d, d)).astype(np.float32)
    c, t = codebook.lloyd_max_beta(d, 3)
    tables = []
    for h in range(2):
        ss = calibrate.channel_sumsq(K[0, h])
        tables.append(codebook.scaled_table(c, t, calibrate.head_scale(ss, T), d))
    fields = encode.encode_cache(K, signs, None, tables, S, p)
    out, lg = attn.decode_cache(q, fields, V, tables, S, signs, None, p)
    for hq in range(8):
        h = kv_of[hq]
        Khat = attn.dequantize_keys(fields[0][h], tables[h][0], S[h], signs[h], None, p)
        s = Khat @ q[0, hq]
        w = np.exp((s - s.max()) / math.sqrt(d))
        ref = (w / w.sum()) @ V[0, h]
        np.testing.assert_allclose(lg[0, hq], s, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(out[0, hq], ref, rtol=1e-11, atol=1e-11)
    # the value means of the two kv-heads differ by 10: a wrong mapping cannot pass
    assert np.all(out[0, :4].mean(axis=1) < -2) and np.all(out[0, 4:].mean(axis=1) > 2)


# ------------------------------------------------------------ calibrate (step 0)

def test_reorder_hand_examples():
    assert calibrate.reorder_perm([1.0, 4.0, 9.0, 16.0]).tolist() == [3, 0, 2, 1]
    assert calibrate.reorder_perm([2.0, 2.0, 1.0, 1.0]).tolist() == [0, 3, 1, 2]
    assert calibrate.reorder_perm([5.0, 1.0, 3.0, 2.0, 4.0, 0.5, 7.0, 6.0]).tolist() == \
        [6, 5, 7, 1, 0, 3, 4, 2]
    k = np.array([[1.0, 2.0], [3.0, -4.0]])
    np.testing.assert_array_equal(calibrate.channel_sumsq(k), [10.0, 20.0])
    assert abs(calibrate.head_scale([10.0, 20.0], 2) - math.sqrt(15.0)) < 1e-15


# ------------------------------------------------------------------ codes

def test_angle_code_hand_values():
    pi = math.pi
    th = np.array([0.1, -0.1, 3.0, -3.0, pi, -pi, pi / 2 + 0.01, -pi / 2 + 0.01, pi / 2 - 0.01])
    assert encode.angle_code(th, 2).tolist() == [2, 1, 3, 0, 0, 0, 3, 1, 2]
    assert encode.angle_code(th, 1).tolist() == [1, 0, 1, 0, 0, 0, 1, 0, 1]
    th3 = np.array([-pi + 0.1, -3 * pi / 4 + 0.1, -pi / 2 + 0.1, -pi / 4 + 0.1, 0.1,
                    pi / 4 + 0.1, pi / 2 + 0.1, 3 * pi / 4 + 0.1])
    assert encode.angle_code(th3, 3).tolist() == list(range(8))
    c2 = encode.angle_centers(2)
    np.testing.assert_allclose(c2, [-3 * pi / 4, -pi / 4, pi / 4, 3 * pi / 4], atol=1e-15)
    # mid-rise: every center lies in its own cell, 2^b distinct directions
    for b in (1, 2, 3):
        c = encode.angle_centers(b)
        assert encode.angle_code(c, b).tolist() == list(range(1 << b))


def test_radius_code_hand_values():
    th = np.array([1.0, 2.0, 3.0], dtype=np.float32)
    r = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 3.5, 0.0])
    assert encode.radius_code(r, th).tolist() == [0, 0, 1, 1, 2, 3, 0]


def test_fp16_residual_norm_rounding():
    # nearest, ties to even; beyond the range saturates
    one = 1.0
    ulp = 2.0 ** -10
    v = np.array([one + ulp / 2, one + 1.5 * ulp, one + ulp / 2 + 1e-12, 70000.0, 65519.0])
    h = encode.to_fp16_saturating(v)
    assert h[0] == np.float16(1.0)
    assert float(h[1]) == one + 2 * ulp
    assert float(h[2]) == one + ulp
    assert float(h[3]) == 65504.0 and float(h[4]) == 65504.0


# ------------------------------------------------------------------ P5 identity

@pytest.mark.parametrize("d", [4, 8, 16])
@pytest.mark.parametrize("bm,ba", [(1, 1), (2, 1), (3, 2), (3, 3)])
@pytest.mark.parametrize("qjl", [False, True])
def test_p5_analytic_logit_equals_dequantize_then_dot(d, bm, ba, qjl):
    rng = np.random.default_rng(d * 100 + bm * 10 + ba + 7 * qjl)
    p = Params(d, bm, ba, d if qjl else 0)
    K = rng.standard_normal((40, d)) * np.exp(0.5 * rng.standard_normal(d))
    signs = rng.choice([-1, 1], size=d)
    perm = rng.permutation(d)
    c, t = codebook.lloyd_max_beta(d, bm)
    ss = calibrate.channel_sumsq(K)
    lv, th = codebook.scaled_table(c, t, calibrate.head_scale(ss, K.shape[0]), d)
    S = rng.standard_normal((d, d)).astype(np.float32)
    f = encode.encode_keys(K, signs, perm, lv, th, S, p)
    q = rng.standard_normal(d)
    s = attn.analytic_logits(q, f, lv, S, signs, perm, p)
    Khat = attn.dequantize_keys(f, lv, S, signs, perm, p)
    ref = Khat @ q
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ------------------------------------------------------------------ P6 QJL

def test_p6_qjl_unbiased_with_closed_form_variance():
    rng = np.random.default_rng(66)
    d = m = 16
    qt = rng.standard_normal(d)
    eps = rng.standard_normal(d) * 0.3
    en = float(np.linalg.norm(eps))
    R = 100000
    S = rng.standard_normal((R, m, d)).astype(np.float32)
    z = np.empty(R)
    for r in range(R):
        Sr = S[r].astype(np.float64)
        bits = (Sr @ eps >= 0)[None, :]
        z[r] = attn.qjl_term(qt, S[r], bits, np.array([en]), m)[0]
    target = float(qt @ eps)
    V = ((math.pi / 2) * (qt @ qt) * en * en - target * target) / m
    assert abs(z.mean() - target) < 4 * math.sqrt(V / R)
    assert abs(z.var() / V - 1.0) < 0.05


def test_p6_qjl_term_tracks_the_true_residual_product():
    # on encoded keys the QJL term estimates <q~, eps~>: positive slope near 1
    rng = np.random.default_rng(67)
    d = 64
    p = Params(d, 3, 2, d)
    K = rng.standard_normal((20000, d)) * np.exp(0.5 * rng.standard_normal(d))
    signs = rng.choice([-1, 1], size=d)
    c, t = codebook.lloyd_max_beta(d, 3)
    lv, th = codebook.scaled_table(c, t, calibrate.head_scale(calibrate.channel_sumsq(K), len(K)), d)
    S = rng.standard_normal((d, d)).astype(np.float32)
    f = encode.encode_keys(K, signs, None, lv, th, S, p)
    q = rng.standard_normal(d)
    qt = attn.query_transform(q, signs, None, p)
    truth = f.eps @ qt
    est = attn.qjl_term(qt, S, f.bits, f.nu, d)
    slope = float(np.dot(est, truth) / np.dot(truth, truth))
    assert 0.8 < slope < 1.2
    # and the residual really is the part of <q, k> the polar codes miss
    polar = attn.analytic_logits(q, encode.Fields(f.rc, f.ac, np.zeros((len(K), 0), bool),
                                                  np.zeros(len(K), np.float16), None, None, None,
                                                  None, None, None),
                                 lv, None, signs, None, Params(d, 3, 2, 0))
    np.testing.assert_allclose(polar + truth, K @ q, rtol=1e-10, atol=1e-9)


# ------------------------------------------------------------------ P7 special case

@pytest.mark.parametrize("bm,ba", [(3, 2), (4, 3), (2, 1)])
def test_p7_points_on_the_grid_reconstruct_exactly(bm, ba):
    d = 16
    n = d // 2
    p = Params(d, bm, ba, d, hadamard=False)
    rng = np.random.default_rng(70 + bm)
    c, t = codebook.lloyd_max_beta(d, bm)
    lv, th = codebook.scaled_table(c, t, 3.0, d)
    cen = encode.angle_centers(ba)
    rc = rng.integers(0, 1 << bm, size=(30, n))
    ac = rng.integers(0, 1 << ba, size=(30, n))
    kt = np.empty((30, d))
    kt[:, 0::2] = lv.astype(np.float64)[rc] * np.cos(cen[ac])
    kt[:, 1::2] = lv.astype(np.float64)[rc] * np.sin(cen[ac])
    S = rng.standard_normal((d, d)).astype(np.float32)
    f = encode.encode_keys(kt, np.ones(d), None, lv, th, S, p)
    assert np.array_equal(f.rc, rc) and np.array_equal(f.ac, ac)
    assert np.all(f.eps == 0) and np.all(f.nu == 0) and np.all(f.bits)
    q = rng.standard_normal(d)
    s = attn.analytic_logits(q, f, lv, S, np.ones(d), None, p)
    np.testing.assert_allclose(s, kt @ q, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ P8 brute force

@pytest.mark.parametrize("d", [4, 8])
@pytest.mark.parametrize("bm,ba", [(1, 1), (2, 2), (3, 3), (3, 1)])
def test_p8_scalar_quantizers_are_nearest(d, bm, ba):
    rng = np.random.default_rng(80 + d + bm + ba)
    p = Params(d, bm, ba, 0)
    K = rng.standard_normal((500, d))
    c, t = codebook.lloyd_max_beta(d, bm)
    lv, th = codebook.scaled_table(c, t, math.sqrt(d), d)
    f = encode.encode_keys(K, rng.choice([-1, 1], size=d), None, lv, th, None, p)
    lv64 = lv.astype(np.float64)
    dist = np.abs(f.r[..., None] - lv64)
    assert np.array_equal(np.argmin(dist, axis=-1), f.rc)
    cen = encode.angle_centers(ba)
    dth = np.abs(np.angle(np.exp(1j * (f.theta[..., None] - cen))))
    assert np.array_equal(np.argmin(dth, axis=-1), f.ac)


# ------------------------------------------------------------------ P9 softmax

def test_p9_split_merge_and_uniform_weights():
    rng = np.random.default_rng(9)
    s = rng.standard_normal(1000) * 5
    V = rng.standard_normal((1000, 8))
    full = attn.attend(s, V, 0.3)
    for P in (1, 2, 7, 64, 1000):
        np.testing.assert_allclose(attn.split_attend(s, V, 0.3, P), full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(attn.attend(np.full(1000, 2.5), V, 0.7), V.mean(axis=0),
                               rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ P10 FP16 comparator

def test_p10_fp16_attention_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(10)
    q = rng.standard_normal((2, 8, 64)).astype(np.float32)
    K = rng.standard_normal((2, 2, 50, 64)).astype(np.float16)
    V = rng.standard_normal((2, 2, 50, 64)).astype(np.float16)
    out, _ = attn.fp16_attention(q, K, V)
    tq = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    tk = torch.from_numpy(K.astype(np.float64)).repeat_interleave(4, dim=1)
    tv = torch.from_numpy(V.astype(np.float64)).repeat_interleave(4, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ P12 fidelity trend

def test_p12_logit_error_falls_with_radius_bits():
    rng = np.random.default_rng(12)
    d = 64
    K = rng.standard_normal((4000, d)) * np.exp(0.5 * rng.standard_normal(d))
    signs = rng.choice([-1, 1], size=d)
    S = rng.standard_normal((d, d)).astype(np.float32)
    q = rng.standard_normal(d)
    exact = K @ q
    ss = calibrate.channel_sumsq(K)
    scale = calibrate.head_scale(ss, K.shape[0])
    errs = []
    for bm in (2, 3, 4):
        p = Params(d, bm, bm - 1, d)
        c, t = codebook.lloyd_max_beta(d, bm)
        lv, th = codebook.scaled_table(c, t, scale, d)
        f = encode.encode_keys(K, signs, None, lv, th, S, p)
        s = attn.analytic_logits(q, f, lv, S, signs, None, p)
        errs.append(float(np.sqrt(np.mean((s - exact) ** 2))))
    assert errs[0] > errs[1] > errs[2]


# ------------------------------------------------------------------ layout

def test_layout_hand_packed_words():
    # d = 64, b_main = 3, b_angle = 2: 5-bit joint codes rc | ac << 3, 32 pairs
    # -> 160 code bits = 5 words, then 2 sign words, then the fp16 norm row
    p = Params(64, 3, 2, 64)
    n = 32
    rc = np.zeros((1, n), dtype=np.int64)
    ac = np.zeros((1, n), dtype=np.int64)
    rc[0, 1] = 1                  # code 1 at stream bit 5
    rc[0, 6], ac[0, 6] = 7, 3     # code 31 at stream bits 30..34 (crosses a word)
    ac[0, 31] = 1                 # code 8 at stream bits 155..159 -> bit 158
    f = encode.Fields(rc=rc, ac=ac, bits=(np.arange(64)[None, :] % 3 == 0),
                      nu=np.array([1.5], dtype=np.float16),
                      kt=None, r=None, theta=None, eps=None, eps_norm=None, u=None)
    buf = layout.pack_stream(f, p, capacity=4, token_offset=1)
    assert buf.nbytes == 4 * 30
    words = buf[: 7 * 16].view(np.uint32).reshape(7, 4)
    assert words[:5, 1].tolist() == [0xC0000020, 0x7, 0, 0, 0x40000000]
    exp = [sum(1 << (j % 32) for j in range(32 * w, 32 * w + 32) if j % 3 == 0) for w in range(2)]
    assert words[5, 1] == exp[0] and words[6, 1] == exp[1]
    assert np.all(words[:, 0] == 0) and np.all(words[:, 2:] == 0)
    norms = buf[7 * 16:].view(np.float16)
    assert float(norms[1]) == 1.5 and norms[0] == 0
    u = layout.unpack_stream(buf, p, 4, 1, token_offset=1)
    assert np.array_equal(u["rc"], f.rc) and np.array_equal(u["ac"], f.ac)
    assert np.array_equal(u["bits"], f.bits) and u["nu"][0] == f.nu[0]


@pytest.mark.parametrize("prm", [(64, 3, 2, 64), (64, 4, 3, 0), (128, 3, 2, 128), (128, 4, 3, 128)])
def test_layout_round_trip(prm):
    p = Params(*prm)
    rng = np.random.default_rng(sum(prm))
    T = 77
    f = encode.Fields(
        rc=rng.integers(0, 1 << p.b_main, size=(T, p.n_pairs)),
        ac=rng.integers(0, 1 << p.b_angle, size=(T, p.n_pairs)),
        bits=rng.integers(0, 2, size=(T, p.qjl_m)).astype(bool),
        nu=rng.random(T).astype(np.float16) if p.qjl_m else np.zeros(T, np.float16),
        kt=None, r=None, theta=None, eps=None, eps_norm=None, u=None)
    buf = layout.pack_stream(f, p, capacity=96, token_offset=5)
    assert buf.nbytes == 96 * layout.record_bytes(p)
    u = layout.unpack_stream(buf, p, 96, T, token_offset=5)
    for k in ("rc", "ac", "bits", "nu"):
        assert np.array_equal(u[k], getattr(f, k))


# ------------------------------------------------------------------ RTN control

def test_rtn_reconstruction_error_bound():
    rng = np.random.default_rng(13)
    K = rng.standard_normal((200, 64)) * 3
    for bits in (3, 4):
        codes, scale, zp = rtn.quantize(K, bits)
        assert codes.min() >= 0 and codes.max() <= (1 << bits) - 1
        err = np.abs(rtn.dequantize(codes, scale, zp) - K)
        # half a step plus the fp16 rounding of the scale and zero-point
        bound = 0.5 * scale.astype(np.float64)[:, None] * 1.01 + \
            (1 << bits) * np.abs(scale.astype(np.float64))[:, None] * 2 ** -11 + \
            np.abs(zp.astype(np.float64))[:, None] * 2 ** -11
        assert np.all(err <= bound)


def test_rtn_record_is_the_printed_bit_budget():
    """Record bytes * 8 / d reproduce the 3.50 / 4.50 bits per element printed for
    INT3 / INT4 RTN at d = 64 ('Comparison to simpler baselines')."""
    g = json.load(open(os.path.join(GOLDEN, "pages_accounting.json")))["rtn"]
    assert rtn.record_bytes(64, 3) * 8 / 64 == g["int3_bpe"]
    assert rtn.record_bytes(64, 4) * 8 / 64 == g["int4_bpe"]


@pytest.mark.parametrize("d,bits", [(64, 3), (64, 4), (128, 3), (128, 4)])
def test_rtn_packing_matches_bit_string(d, bits):
    """Words of the packed stream against an independent construction: the codes
    written as one LSB-first bit string, cut into 32-bit words."""
    rng = np.random.default_rng(d * 10 + bits)
    N, cap, off = 5, 9, 3
    codes = rng.integers(0, 1 << bits, size=(N, d))
    scale = rng.uniform(0.01, 2, N).astype(np.float16)
    zp = rng.uniform(-5, 5, N).astype(np.float16)
    buf = rtn.pack_stream(codes, scale, zp, bits, cap, token_offset=off)
    words = buf.view(np.uint32).reshape(-1, cap)
    nc = d * bits // 32
    assert words.shape[0] == nc + 1
    for t in range(N):
        bitstr = "".join(format(int(c), f"0{bits}b")[::-1] for c in codes[t])
        assert len(bitstr) == 32 * nc
        for w in range(nc):
            assert int(bitstr[32 * w:32 * w + 32][::-1], 2) == words[w, off + t]
        sz = int(words[nc, off + t])
        assert sz & 0xFFFF == int(scale[t].view(np.uint16))
        assert sz >> 16 == int(zp[t].view(np.uint16))
    assert not words[:, :off].any() and not words[:, off + N:].any()
    c2, s2, z2 = rtn.unpack_stream(buf, d, bits, cap, N, token_offset=off)
    assert np.array_equal(c2, codes) and np.array_equal(s2.view(np.uint16), scale.view(np.uint16))
    assert np.array_equal(z2.view(np.uint16), zp.view(np.uint16))


@pytest.mark.parametrize("bits", [3, 4])
def test_rtn_ramp_is_exact(bits):
    """A ramp lo + j * step over 2^b levels with an fp16-exact step is its own
    quantization: zero-point lo, scale step, codes j, exact reconstruction."""
    L = 1 << bits
    lo, step = -1.25, 0.375
    K = (lo + step * (np.arange(64) % L)).reshape(1, 64)
    codes, scale, zp = rtn.quantize(K, bits)
    assert float(zp[0]) == lo and float(scale[0]) == step
    assert np.array_equal(codes[0], np.arange(64) % L)
    assert np.array_equal(rtn.dequantize(codes, scale, zp), K)


def test_rtn_rounds_half_to_even_and_handles_degenerate_keys():
    # range 15 -> scale 1 at INT4: half-way values go to the even code
    k = np.zeros(64)
    k[:8] = [0.0, 0.5, 1.5, 2.5, 3.5, 14.5, 15.0, 7.5]
    codes, scale, zp = rtn.quantize(k[None], 4)
    assert float(scale[0]) == 1.0 and float(zp[0]) == 0.0
    assert list(codes[0, :8]) == [0, 0, 2, 2, 4, 14, 15, 8]
    # a constant key: zero range -> scale 1, every code 0, exact reconstruction
    c = np.full((1, 64), -3.0)
    codes, scale, zp = rtn.quantize(c, 3)
    assert float(scale[0]) == 1.0 and not codes.any()
    assert np.array_equal(rtn.dequantize(codes, scale, zp), c)
    # -0 and +0 extremes give the +0 zero-point
    z = np.zeros((1, 64))
    z[0, 5] = -0.0
    _, _, zp = rtn.quantize(z, 3)
    assert zp[0].view(np.uint16) == 0
    # a minimum that fp16 rounds upward is clamped to code 0, not -1
    m = np.linspace(0, 1, 64)
    m[0] = 1e-3 + 2 ** -22  # fp16(m0) > m0
    codes, _, zp = rtn.quantize(m[None], 4)
    assert float(zp[0]) > m[0] and codes[0, 0] == 0


def test_rtn_logits_converge_to_exact_with_bits():
    """The RTN logit error shrinks about 2x per extra bit (uniform step)."""
    rng = np.random.default_rng(3)
    K = rng.standard_normal((300, 64))
    q = rng.standard_normal(64)
    errs = []
    for bits in (3, 4, 6, 8):
        codes, scale, zp = rtn.quantize(K, bits)
        errs.append(np.abs(rtn.logits(q, codes, scale, zp) - K @ q).mean())
    assert errs[0] > errs[1] > errs[2] > errs[3]
    assert 1.5 < errs[0] / errs[1] < 2.8
    assert 10 < errs[1] / errs[3] < 24


# ------------------------------------------------------------------ PGKQ-KV (values coded)

def test_kv_grid_values_reconstruct_exactly():
    """Without the transform, a value whose pairs sit on (level_j, centre_a) points
    reconstructs exactly: codes (j, a), residual 0, nu 0, QJL term 0."""
    from oracle import kv
    d, bm = 16, 3
    pv = kv.value_params(d, bm, d)
    c, t = codebook.lloyd_max_beta(d, bm)
    lv, th = codebook.scaled_table(c, t, 2.0, d)
    cen = encode.angle_centers(pv.b_angle)
    rng = np.random.default_rng(4)
    js = rng.integers(0, 1 << bm, size=(5, d // 2))
    ac = rng.integers(0, 1 << pv.b_angle, size=(5, d // 2))
    lv64 = lv.astype(np.float64)
    V = np.zeros((5, d))
    V[:, 0::2] = lv64[js] * np.cos(cen[ac])
    V[:, 1::2] = lv64[js] * np.sin(cen[ac])
    S = rng.standard_normal((d, d)).astype(np.float32)
    f = kv.encode_values(V, lv, th, S, pv)
    assert np.array_equal(f.rc, js) and np.array_equal(f.ac, ac)
    assert np.all(f.nu == 0)
    np.testing.assert_allclose(kv.dequantize_values(f, lv, S, pv), V, rtol=0, atol=1e-12)


def test_kv_code_domain_output_equals_explicit_reconstruction():
    """The decoder's form (weighted pair reconstructions, then one S^T product of
    the weighted signed norms) equals p @ V-hat."""
    from oracle import kv
    rng = np.random.default_rng(8)
    for d, bm, m in ((16, 2, 16), (64, 3, 64), (128, 4, 128), (64, 3, 0)):
        pv = kv.value_params(d, bm, m)
        V = rng.standard_normal((40, d)) * np.exp(0.5 * rng.standard_normal(d))
        tab = kv.value_tables(V[None, None], bm)[0]
        S = rng.standard_normal((m, d)).astype(np.float32) if m else None
        f = kv.encode_values(V, tab[0], tab[1], S, pv)
        p = rng.dirichlet(np.ones(40))
        want = p @ kv.dequantize_values(f, tab[0], S, pv)
        np.testing.assert_allclose(kv.code_domain_output(p, f, tab[0], S, pv), want,
                                   rtol=1e-12, atol=1e-12)


def test_kv_qjl_residual_estimate_is_unbiased():
    """Over independent Gaussian projections, kappa ||eps|| S^T sign(S eps) has mean
    eps (each coordinate within 4 standard errors) and per-coordinate variance
    (pi/2) ||eps||^2 / m - eps_c^2 / m (the closed form of the vector estimator)."""
    from oracle import attn as A
    rng = np.random.default_rng(21)
    d = m = 16
    eps = rng.standard_normal(d)
    R = 40000
    S = rng.standard_normal((R, m, d))
    u = np.einsum("rmd,d->rm", S, eps)
    est = A.kappa(m) * np.linalg.norm(eps) * np.einsum("rm,rmd->rd", np.where(u >= 0, 1.0, -1.0), S)
    mean = est.mean(axis=0)
    var_cf = (math.pi / 2) * (eps @ eps) / m - eps ** 2 / m
    se = np.sqrt(var_cf / R)
    assert np.all(np.abs(mean - eps) <= 4 * se)
    np.testing.assert_allclose(est.var(axis=0), var_cf, rtol=0.05)


def test_kv_decode_error_shrinks_with_bits():
    """PGKQ-KV output error against exact attention falls from b = 2 to 4 (values
    coded; keys coded with the same bit width)."""
    from oracle import kv
    rng = np.random.default_rng(30)
    d, T = 64, 256
    K = rng.standard_normal((1, 1, T, d)) * np.exp(0.5 * rng.standard_normal(d))
    V = rng.standard_normal((1, 1, T, d))
    q = rng.standard_normal((1, 1, d))
    signs = np.where(rng.integers(0, 2, (1, d)) > 0, 1.0, -1.0)
    Sk = rng.standard_normal((1, d, d)).astype(np.float32)
    Sv = rng.standard_normal((1, d, d)).astype(np.float32)
    p_exact = attn.softmax_weights(K[0, 0] @ q[0, 0], 1 / math.sqrt(d))
    exact = p_exact @ V[0, 0]
    errs = []
    for bm in (2, 3, 4):
        pk = Params(d, bm, bm - 1, d)
        pv = kv.value_params(d, bm, d)
        c, t = codebook.lloyd_max_beta(d, bm)
        kt = [codebook.scaled_table(c, t, calibrate.head_scale(calibrate.channel_sumsq(K[0, 0]), T), d)]
        vt = kv.value_tables(V, bm)
        kf = [[encode.encode_keys(K[0, 0], signs[0], None, kt[0][0], kt[0][1], Sk[0], pk)]]
        vf = [[kv.encode_values(V[0, 0], vt[0][0], vt[0][1], Sv[0], pv)]]
        out, _ = kv.decode_kv(q, kf, vf, kt, vt, Sk, Sv, signs, None, pk, pv)
        errs.append(np.abs(out[0, 0] - exact).max())
    assert errs[0] > errs[1] > errs[2]


# ------------------------------------------------------------------ empirical refit (PGKQ-KV')

def test_empirical_lloyd_max_recovers_a_discrete_distribution():
    """Samples on exactly L distinct values, equally often: the fixed point puts
    one level on each value (each cell holds one value; zero error)."""
    vals = np.array([0.3, 0.7, 1.1, 1.2, 2.0, 2.05, 3.5, 4.0])
    x = np.repeat(vals, 50)
    c, t, hist = codebook.lloyd_max_empirical(np.random.default_rng(1).permutation(x), 3,
                                              history=True)
    np.testing.assert_allclose(c, vals, rtol=0, atol=1e-15)
    assert hist[-1] < 1e-28


def test_empirical_lloyd_max_fixed_point_and_monotone_error():
    rng = np.random.default_rng(7)
    x = np.abs(rng.standard_normal(5000)) * 1.3
    c, t, hist = codebook.lloyd_max_empirical(x, 3, history=True)
    cells = np.sum(t[None, :] < x[:, None], axis=1)
    for j in range(8):  # every level is its cell's mean, thresholds are midpoints
        np.testing.assert_allclose(c[j], x[cells == j].mean(), rtol=1e-14)
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=0)
    assert all(b <= a + 1e-15 for a, b in zip(hist, hist[1:]))


def test_empirical_lloyd_max_on_prior_samples_approaches_the_beta_table():
    """Fitted to the prior's own quantiles at (i + 1/2)/N (a stratified sample of
    the Beta radius law), the empirical table tends to the analytic one as N
    grows."""
    d, b = 64, 3
    c_ref, _ = codebook.lloyd_max_beta(d, b)
    errs = []
    for N in (20000, 100000):
        x = codebook.rho_quantile((np.arange(N) + 0.5) / N, d // 2)
        c_emp, _ = codebook.lloyd_max_empirical(x, b)
        errs.append(float(np.max(np.abs(c_emp - c_ref))))
    assert errs[1] < 1e-3 and errs[1] < 0.5 * errs[0], errs
