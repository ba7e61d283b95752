"""Pins of the CPU oracle against things other than itself.

Every test here checks the oracle against a value printed on the pages, a
closed form, a textbook table, an independent quadrature or brute force, so
that a plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong constant) fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
from scipy import integrate, linalg, special

from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- signs ----

def test_splitmix64_matches_published_outputs():
    want = [int(v, 16) for v in _golden_lines("splitmix64_seed0.txt")]
    assert O.splitmix64(0, len(want)) == want


def test_rotation_signs_use_top_bit_and_are_balanced():
    z = O.splitmix64(7, 64)
    s = O.rotation_signs(7, 64)
    assert all((zz >> 63 == 0) == (ss == 1) for zz, ss in zip(z, s))
    tot = np.concatenate([O.rotation_signs(seed, D) for seed in range(200)]).astype(float)
    # 25600 fair +/-1 draws: |mean| < 4 sigma
    assert abs(tot.mean()) < 4.0 / math.sqrt(tot.size)
    # different seeds give different sign vectors
    assert not np.array_equal(O.rotation_signs(42, D), O.rotation_signs(43, D))


# -------------------------------------------------------------- hadamard ---

def _fwht_bruteforce(x):
    """The butterfly transform with strides h = 1, 2, 4, ... written as plain
    loops (the algorithm of the deep-dive blog's Step 1 listing)."""
    x = [float(v) for v in x]
    d = len(x)
    h = 1
    while h < d:
        for i in range(0, d, 2 * h):
            for j in range(i, i + h):
                a, b = x[j], x[j + h]
                x[j], x[j + h] = a + b, a - b
        h *= 2
    return np.array(x)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_equals_library_and_butterflies(d):
    H = O.hadamard(d)
    assert np.array_equal(H, linalg.hadamard(d).astype(float))
    assert np.array_equal(H @ H.T, d * np.eye(d))
    rng = np.random.default_rng(d)
    for _ in range(3):
        x = rng.integers(-50, 50, size=d).astype(float)
        assert np.array_equal(H @ x, _fwht_bruteforce(x))


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        O.hadamard(12)


# -------------------------------------------------------------- rotation ---

def test_rotation_is_sign_flip_then_fwht_then_scale():
    for seed in (0, 42, 12345):
        R = O.rotation_matrix(seed, D)
        s = O.rotation_signs(seed, D)
        x = np.random.default_rng(seed).standard_normal(D)
        want = _fwht_bruteforce(x * s) / math.sqrt(D)
        np.testing.assert_allclose(R @ x, want, rtol=0, atol=1e-12)
        # and not the other order (D applied after H): the test can tell them apart
        other = _fwht_bruteforce(x) * s / math.sqrt(D)
        assert np.max(np.abs(R @ x - other)) > 1e-3


def test_rotation_is_orthogonal_and_preserves_geometry():
    R = O.rotation_matrix(42, D)
    np.testing.assert_allclose(R @ R.T, np.eye(D), atol=1e-13)
    rng = np.random.default_rng(1)
    x, y = rng.standard_normal((2, D)) * 10
    assert abs(np.linalg.norm(R @ x) - np.linalg.norm(x)) < 1e-12 * np.linalg.norm(x)
    assert abs((R @ x) @ (R @ y) - x @ y) < 1e-11


def test_rotation_spreads_a_spike_flat():
    # an outlier concentrated in one coordinate comes out with every
    # coordinate of magnitude |a|/sqrt(d) (the blog's RHT-effect example,
    # quantitatively)
    R = O.rotation_matrix(42, D)
    for i in (0, 5, 127):
        e = np.zeros(D)
        e[i] = 45.3
        np.testing.assert_allclose(np.abs(R @ e), 45.3 / math.sqrt(D), rtol=1e-14)


# -------------------------------------------------------------- codebook ---

def test_density_is_normalised_with_variance_one_over_d():
    for d in (8, 128):
        # 400-node Gauss-Legendre on [-1, 1] (exact for polynomials of degree
        # < 800, and f_d is smooth enough for 1e-13)
        x, w = np.polynomial.legendre.leggauss(400)
        tot = np.sum(w * O.coord_density(x, d))
        var = np.sum(w * x * x * O.coord_density(x, d))
        assert abs(tot - 1) < 1e-12
        assert abs(var - 1.0 / d) < 1e-12


def test_density_matches_sphere_marginal_by_monte_carlo():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((200000, 16))
    u = g / np.linalg.norm(g, axis=1, keepdims=True)
    hist, edges = np.histogram(u[:, 0], bins=20, range=(-1, 1), density=True)
    mids = 0.5 * (edges[1:] + edges[:-1])
    np.testing.assert_allclose(hist, O.coord_density(mids, 16), atol=0.03)


@pytest.mark.parametrize("d", [16, 128])
def test_cdf_and_moments_agree_with_quadrature(d):
    pts = [(-0.9, -0.3), (-0.2, 0.05), (0.0, 0.1), (0.12, 0.6), (-1.0, 1.0)]
    for a, b in pts:
        p = integrate.quad(lambda x: O.coord_density(x, d), a, b, epsabs=1e-15)[0]
        m1 = integrate.quad(lambda x: x * O.coord_density(x, d), a, b, epsabs=1e-15)[0]
        m2 = integrate.quad(lambda x: x * x * O.coord_density(x, d), a, b, epsabs=1e-15)[0]
        assert abs((O.coord_cdf(b, d) - O.coord_cdf(a, d)) - p) < 1e-12
        assert abs(O.coord_partial_mean(a, b, d) - m1) < 1e-13
        assert abs(O.coord_partial_second_moment(a, b, d) - m2) < 1e-13


def test_one_bit_codebook_closed_form():
    # b = 1: c = +/- E|X| = +/- Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)),
    # unit-vector distortion 1 - d c^2
    c, t = O.lloyd_max(D, 1)
    closed = math.exp(special.gammaln(D / 2) - special.gammaln((D + 1) / 2)) / math.sqrt(math.pi)
    assert abs(closed - 0.0706615727) < 1e-10
    np.testing.assert_allclose(c, [-closed, closed], rtol=1e-13)
    assert t[0] == 0.0
    assert abs(D * O.codebook_distortion(D, 1) - (1 - D * closed ** 2)) < 1e-12
    assert abs(1 - D * closed ** 2 - 0.3608886) < 1e-7


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_satisfies_lloyd_conditions_by_quadrature(bits):
    c, t = O.lloyd_max(D, bits)
    np.testing.assert_array_equal(c, -c[::-1])            # symmetric
    assert np.all(np.diff(c) > 0)
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for i in range(len(c)):
        a, b = edges[i], edges[i + 1]
        p = integrate.quad(lambda x: O.coord_density(x, D), a, b, epsabs=1e-16, limit=200)[0]
        m = integrate.quad(lambda x: x * O.coord_density(x, D), a, b, epsabs=1e-16, limit=200)[0]
        assert abs(m / p - c[i]) < 1e-10 * max(1.0, abs(c[i]))


def test_codebook_gaussian_limit_matches_max_1960():
    rows = _golden_lines("max1960_gaussian.txt")
    d = 65536
    for row in rows:
        lv, outs, ths, mse = [p.strip() for p in row.split("|")]
        bits = int(lv).bit_length() - 1
        c, t = O.lloyd_max(d, bits, tol=1e-10)
        half = len(c) // 2
        np.testing.assert_allclose(math.sqrt(d) * c[half:], [float(v) for v in outs.split()], atol=1.5e-3)
        if ths != "-":
            np.testing.assert_allclose(math.sqrt(d) * t[half:], [float(v) for v in ths.split()], atol=1.5e-3)
        assert abs(d * O.codebook_distortion(d, bits, c) - float(mse)) < 1e-3 * float(mse) + 1e-5


def test_distortion_falls_about_4x_per_bit_and_is_above_octopus():
    dist = {b: D * O.codebook_distortion(D, b) for b in (1, 2, 3, 4)}
    for b in (2, 3, 4):
        ratio = dist[b - 1] / dist[b]
        assert 2.9 < ratio < 4.0, (b, ratio)
    # the related triplet codec claims lower MSE at equal bits; a per-coordinate
    # rotation codec should therefore not be below its printed values
    for row in _golden_lines("octopus_synthetic_mse.txt"):
        b, mse = row.split()
        assert dist[int(b)] >= float(mse)


def test_distortion_matches_monte_carlo_and_finite_d_shift_from_gaussian():
    rng = np.random.default_rng(11)
    g = rng.standard_normal((20000, D))
    y = (g / np.linalg.norm(g, axis=1, keepdims=True)).ravel()
    for bits in (2, 4):
        c, _ = O.lloyd_max(D, bits)
        q = c[np.argmin((y[:, None] - c) ** 2, axis=1)]
        e = (y - q) ** 2
        mc, se = e.mean(), e.std() / math.sqrt(e.size)
        assert abs(mc - O.codebook_distortion(D, bits)) < 4 * se


def test_codebook_fp32_rounding_and_midpoints():
    for bits in (2, 3, 4):
        c, _ = O.lloyd_max(D, bits)
        c32, t32 = O.codebook_fp32(D, bits)
        assert np.array_equal(c32, c.astype(np.float32).astype(np.float64))
        assert np.array_equal(c32, -c32[::-1])
        assert t32[len(t32) // 2] == 0.0
        assert np.all((t32 > c32[:-1]) & (t32 < c32[1:]))
        assert np.all(np.abs(t32 - 0.5 * (c32[:-1] + c32[1:])) <= np.abs(np.spacing(np.float32(t32))).astype(float))


# ---------------------------------------------------------------- encode ---

def _brute_nearest(y, c):
    out = []
    for v in y:
        best, bi = None, None
        for i, ci in enumerate(c):
            dd = (v - ci) ** 2
            if best is None or dd < best:
                best, bi = dd, i
        out.append(bi)
    return np.array(out)


def test_encode_nearest_codeword_by_brute_force_and_threshold_count():
    c32, t32 = O.codebook_fp32(D, 3)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((20, D))
    enc = O.encode(x, 42, c32)
    for i in range(3):
        assert np.array_equal(enc["idx"][i], _brute_nearest(enc["y"][i], c32))
    # threshold counting gives the same codes away from exact ties
    cnt = np.sum(enc["y"][..., None] > t32, axis=-1)
    assert np.array_equal(cnt, enc["idx"])


def test_encode_split_norm_and_direction():
    c32, _ = O.codebook_fp32(D, 4)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, D)) * 3
    enc = O.encode(x, 42, c32)
    np.testing.assert_allclose(enc["gamma"], np.linalg.norm(x, axis=1), rtol=1e-15)
    np.testing.assert_allclose(np.linalg.norm(enc["y"], axis=1), 1.0, rtol=1e-14)
    # positive scaling changes only the norm
    enc2 = O.encode(7.5 * x, 42, c32)
    assert np.array_equal(enc2["idx"], enc["idx"])
    np.testing.assert_allclose(enc2["gamma"], 7.5 * enc["gamma"], rtol=1e-14)


def test_encode_zero_vector_and_ties_go_low():
    for bits in (2, 3, 4):
        c32, _ = O.codebook_fp32(D, bits)
        enc = O.encode(np.zeros((1, D)), 42, c32)
        assert enc["gamma"][0] == 0 and float(enc["gamma16"][0]) == 0.0
        assert np.all(enc["idx"] == (1 << (bits - 1)) - 1)
    # two equal spikes cancel exactly on half of the rotated coordinates:
    # y_j = 0 there, a tie between the two middle centroids -> lower index
    c32, _ = O.codebook_fp32(D, 4)
    x = np.zeros(D)
    s = O.rotation_signs(42, D)
    x[0], x[1] = 1.0 * s[0], 1.0 * s[1]
    enc = O.encode(x[None], 42, c32)
    zero = enc["y"][0] == 0.0
    assert zero.sum() == D // 2
    assert np.all(enc["idx"][0][zero] == 7)


def test_encode_spike_lands_on_the_centroid_nearest_one_over_sqrt_d():
    for bits in (2, 3, 4):
        c32, _ = O.codebook_fp32(D, bits)
        x = np.zeros((1, D))
        x[0, 17] = -45.3
        enc = O.encode(x, 42, c32)
        v = 1.0 / math.sqrt(D)
        pos = int(np.argmin((c32 - v) ** 2))
        neg = int(np.argmin((c32 + v) ** 2))
        assert set(np.unique(enc["idx"])) <= {pos, neg}


def test_fp16_norm_rounding_and_saturation():
    vals = np.array([0.0, 1.0, 2049.0, 2051.0, 65504.0, 65519.0, 70000.0, 1e30])
    want = np.array([0.0, 1.0, 2048.0, 2052.0, 65504.0, 65504.0, 65504.0, 65504.0])
    assert np.array_equal(O.fp16_norm(vals).astype(np.float64), want)


def test_fp16_sat_rounds_to_nearest_even_and_saturates_both_signs():
    # fp16 has 11 significant bits: 2049 is a tie between 2048 and 2050 (even
    # mantissa 2048); 65520 is the tie between 65504 and the overflow, which
    # round-to-nearest-even would send to infinity: saturation keeps 65504.
    vals = np.array([0.0, -0.0, 1.5, -2049.0, 2051.0, 65504.0, 65519.0, 65520.0, 1e6, -65520.0, -1e30, 6e-8])
    want = np.array([0.0, -0.0, 1.5, -2048.0, 2052.0, 65504.0, 65504.0, 65504.0, 65504.0, -65504.0, -65504.0,
                     5.960464477539063e-08])
    got = O.fp16_sat(vals)
    assert got.dtype == np.float16
    assert np.array_equal(got.astype(np.float64), want)
    assert np.signbit(got[1]) and not np.signbit(got[0])
    assert np.all(np.isfinite(got))


def test_isotropic_reconstruction_mse_equals_codebook_distortion():
    # R fixed and orthogonal maps Haar-uniform directions to Haar-uniform
    # directions, so E||u - u_hat||^2 = d * D_b exactly in expectation
    rng = np.random.default_rng(8)
    g = rng.standard_normal((6000, D))
    u = g / np.linalg.norm(g, axis=1, keepdims=True)
    for bits in (2, 3, 4):
        c32, _ = O.codebook_fp32(D, bits)
        enc = O.encode(u, 42, c32)
        uh = O.reconstruct(enc["idx"], np.ones(len(u)), 42, c32)
        e = np.sum((u - uh) ** 2, axis=1)
        want = D * O.codebook_distortion(D, bits, c32)
        assert abs(e.mean() - want) < 4 * e.std() / math.sqrt(e.size)


def test_reconstruct_uses_the_transpose_rotation():
    # <q, x_hat> == gamma16 <R q, c[idx]>: the rotated-frame identity
    c32, _ = O.codebook_fp32(D, 4)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, D))
    q = rng.standard_normal(D)
    enc = O.encode(x, 42, c32)
    xh = O.reconstruct(enc["idx"], enc["gamma16"], 42, c32)
    R = O.rotation_matrix(42, D)
    lhs = xh @ q
    rhs = enc["gamma16"].astype(float) * (c32[enc["idx"]] @ (R @ q))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    # exact y instead of c[idx] gives back x (up to the fp16 norm)
    xr = enc["gamma"][:, None] * (enc["y"] @ R)
    np.testing.assert_allclose(xr, x, atol=1e-12)


# ------------------------------------------------------------ bit budget ---

def test_bits_per_vector_match_the_pages():
    for row in _golden_lines("pages_bit_budget.txt"):
        d, b, total, ratio = row.split()
        d, b, total, ratio = int(d), int(b), int(total), float(ratio)
        if b == 16:
            assert d * b == total
            continue
        assert O.bits_per_vector(d, b) == total
        assert abs(2048 / total - ratio) < 0.05
    assert O.bits_per_vector(128, 2, qjl=True) == 128 * 2 + 16 + 128 + 16


def test_layout_v1_block_sizes():
    assert O.LayoutV1(128, 8, 4, 4, False, 1).block_bytes == 16 * (528 + 528) // 8
    assert O.LayoutV1(128, 8, 3, 3, False, 1).block_bytes == 16 * (400 + 400) // 8
    assert O.LayoutV1(128, 1, 2, 0, True, 1).block_bytes == 832


def test_pack_codes_bit_order():
    # code j at bits [j*b, j*b+b), LSB first, little-endian bytes
    assert O.pack_codes([1, 2, 3, 4], 4) == bytes([0x21, 0x43])
    assert O.pack_codes([7, 0, 0, 0, 0, 0, 0, 5], 3) == bytes([0x07, 0x00, 0xA0])
    assert O.pack_codes([3, 0, 1, 2], 2) == bytes([0b10010011])
    rng = np.random.default_rng(2)
    for b in (1, 2, 3, 4):
        codes = rng.integers(0, 1 << b, size=D)
        rec = O.pack_codes(codes, b)
        assert len(rec) == D * b // 8
        assert np.array_equal(O.unpack_codes(rec, b, D), codes)


def test_cache_round_trip():
    lay = O.LayoutV1(128, 3, 3, 2, True, 5)
    pool = bytearray(lay.pool_bytes)
    rng = np.random.default_rng(4)
    items = {}
    for slot in (0, 17, 31, 79):
        for h in range(3):
            it = dict(k_idx=rng.integers(0, 8, D), k_g16=np.float16(rng.random()),
                      v_idx=rng.integers(0, 4, D), v_g16=np.float16(rng.random()),
                      qjl_bits=rng.integers(0, 2, D), rho16=np.float16(rng.random()))
            O.write_cache(pool, lay, slot, h, **it)
            items[(slot, h)] = it
    for (slot, h), it in items.items():
        got = O.read_cache(pool, lay, slot, h)
        for k, v in it.items():
            assert np.array_equal(np.asarray(got[k]), np.asarray(v)), k


# ------------------------------------------------------------------- QJL ---

def test_qjl_constant_is_unbiased_for_a_gaussian_sketch():
    # textbook: for g ~ N(0, I), E[sign(g.r) (g.w)] = sqrt(2/pi) <r, w> / ||r||
    rng = np.random.default_rng(12)
    r = rng.standard_normal(D)
    w = r + 0.5 * rng.standard_normal(D)
    n = 100000
    G = rng.standard_normal((n, D))
    est = O.SQRT_HALF_PI * np.linalg.norm(r) * np.sign(G @ r) * (G @ w)
    assert abs(est.mean() - r @ w) < 4 * est.std() / math.sqrt(n)


def test_qjl_removes_the_inner_product_bias_for_aligned_queries():
    # q = u (aligned): the MSE-only estimate <y, c[idx]> is biased by about
    # -d * D_b; adding the QJL estimate of <y, r> should remove >= 90% of it.
    rng = np.random.default_rng(13)
    for bits in (2, 3):
        c32, _ = O.codebook_fp32(D, bits)
        errs_mse, errs_qjl = [], []
        for trial in range(40):
            g = rng.standard_normal((250, D))
            u = g / np.linalg.norm(g, axis=1, keepdims=True)
            enc = O.encode(u, 1000 + trial, c32)
            y = enc["y"]
            base = np.sum(y * c32[enc["idx"]], axis=1)
            sk = O.qjl_encode(y, enc["idx"], c32, 5000 + trial)
            corr = O.qjl_dot_estimate(sk["bits"], sk["rho16"], y, 5000 + trial)
            errs_mse.append(base - 1.0)
            errs_qjl.append(base + corr - 1.0)
        bm = np.mean(np.concatenate(errs_mse))
        bq = np.mean(np.concatenate(errs_qjl))
        assert abs(bm + D * O.codebook_distortion(D, bits, c32)) < 0.05 * abs(bm)
        assert abs(bq) < 0.10 * abs(bm), (bits, bm, bq)


def test_qjl_mean_error_over_1e5_correlated_pairs_is_near_zero():
    # q = u + isotropic noise of the same length: <q, u> = 1 on average, so
    # the MSE-only estimate carries the -d * D_b bias (many standard errors
    # at 10^5 pairs) and the QJL estimate has to cancel it.  (With q drawn
    # independently of u both estimates have mean zero, which pins nothing.)
    rng = np.random.default_rng(14)
    c32, _ = O.codebook_fp32(D, 2)
    e_mse, e_qjl = [], []
    for trial in range(10):
        g = rng.standard_normal((10000, D))
        u = g / np.linalg.norm(g, axis=1, keepdims=True)
        q = u + rng.standard_normal((10000, D)) / math.sqrt(D)
        enc = O.encode(u, 77 + trial, c32)
        R = O.rotation_matrix(77 + trial, D)
        qr = q @ R.T
        sk = O.qjl_encode(enc["y"], enc["idx"], c32, 300 + trial)
        base = np.sum(qr * c32[enc["idx"]], axis=1)
        corr = O.qjl_dot_estimate(sk["bits"], sk["rho16"], qr, 300 + trial)
        truth = np.sum(q * u, axis=1)
        e_mse.append(base - truth)
        e_qjl.append(base + corr - truth)
    em, eq = np.concatenate(e_mse), np.concatenate(e_qjl)
    assert eq.size == 100000
    se_m, se_q = em.std() / math.sqrt(em.size), eq.std() / math.sqrt(eq.size)
    bias = -D * O.codebook_distortion(D, 2, c32)
    assert abs(em.mean() - bias) < 4 * se_m + 0.05 * abs(bias)       # the bias is there ...
    assert abs(em.mean()) > 20 * se_m
    assert abs(eq.mean()) < 0.10 * abs(em.mean())                     # ... and QJL removes it
    assert abs(eq.mean()) < 4 * se_q + 0.02 * abs(bias)


def test_qjl_logits_remove_the_score_bias_in_the_original_frame():
    # logits(q, khat, qjl=...) in the original frame, with the key's own
    # direction as the query (scaled by a), keys of widely varying norms and
    # fresh rotation seeds per trial.  Truth: tau * a * gamma.  MSE-only
    # scores are biased by about -tau * a * gamma * d * D_b; the QJL term
    # must remove >= 90% of it.  Sketching q instead of R q, dropping gamma16
    # or tau, or flipping the term's sign all leave (or grow) the bias.
    rng = np.random.default_rng(19)
    tau = 1.0 / math.sqrt(D)
    for bits in (2, 3, 4):
        c32, _ = O.codebook_fp32(D, bits)
        rel_mse, rel_qjl = [], []
        for trial in range(30):
            n = 120
            g = rng.standard_normal((n, D))
            u = g / np.linalg.norm(g, axis=1, keepdims=True)
            gam = np.exp(rng.uniform(math.log(0.3), math.log(60.0), n))
            x = u * gam[:, None]
            seed, seed_q = 2000 + trial, 7000 + trial
            enc = O.encode(x, seed, c32)
            sk = O.qjl_encode(enc["y"], enc["idx"], c32, seed_q)
            khat = O.reconstruct(enc["idx"], enc["gamma16"], seed, c32)
            qd = dict(bits=sk["bits"], rho16=sk["rho16"], gamma16=enc["gamma16"], seed=seed, seed_qjl=seed_q)
            for t in range(0, n, 6):            # a query per sampled key, scored against that key
                a = 2.5
                q = a * u[t]
                truth = tau * a * np.float64(enc["gamma16"][t])
                s0 = O.logits(q, khat[t:t + 1])[0]
                s1 = O.logits(q, khat[t:t + 1], qjl={k: (v[t:t + 1] if isinstance(v, np.ndarray) else v)
                                                      for k, v in qd.items()})[0]
                rel_mse.append((s0 - truth) / truth)
                rel_qjl.append((s1 - truth) / truth)
        bm, bq = float(np.mean(rel_mse)), float(np.mean(rel_qjl))
        assert abs(bm + D * O.codebook_distortion(D, bits, c32)) < 0.1 * abs(bm), (bits, bm)
        assert abs(bq) < 0.10 * abs(bm), (bits, bm, bq)


def test_qjl_sign_bits_and_zero_residual():
    c32, _ = O.codebook_fp32(D, 4)
    y = c32[np.arange(D) % 16][None, :]     # y exactly on centroids -> r = 0
    sk = O.qjl_encode(y, (np.arange(D) % 16)[None, :], c32, 9)
    assert sk["rho"][0] == 0 and np.all(sk["bits"] == 0)   # sign of 0 is +


# ------------------------------------------------------- logits/attention --

def test_logit_scale_and_frames():
    c32, _ = O.codebook_fp32(D, 4)
    rng = np.random.default_rng(15)
    x = rng.standard_normal((6, D))
    q = rng.standard_normal(D)
    enc = O.encode(x, 42, c32)
    xh = O.reconstruct(enc["idx"], enc["gamma16"], 42, c32)
    s = O.logits(q, xh)
    np.testing.assert_allclose(s, (xh @ q) / math.sqrt(D), rtol=1e-15)
    np.testing.assert_allclose(O.logits(q, xh, scale=0.5), 0.5 * (xh @ q), rtol=1e-15)


def test_attention_special_cases():
    rng = np.random.default_rng(16)
    q = rng.standard_normal(D)
    V = rng.standard_normal((9, D))
    # identical keys -> uniform weights -> mean of values
    K = np.tile(rng.standard_normal(D), (9, 1))
    o, _ = O.attention(q, K, V)
    np.testing.assert_allclose(o, V.mean(axis=0), atol=1e-14)
    # one key far ahead -> its value (scores of several thousand: the softmax
    # must subtract the maximum to stay finite)
    K = rng.standard_normal((9, D))
    K[4] = 5000.0 * q / np.linalg.norm(q)
    o, _ = O.attention(q, K, V)
    np.testing.assert_allclose(o, V[4], atol=1e-12)
    # single token
    o, _ = O.attention(q, K[:1], V[:1])
    np.testing.assert_allclose(o, V[0], atol=1e-15)
    # adding the same vector a*q/|q|^2 to all keys shifts all scores equally
    K = rng.standard_normal((9, D))
    o1, s1 = O.attention(q, K, V)
    o2, s2 = O.attention(q, K + 3.0 * q / (q @ q), V)
    np.testing.assert_allclose(s2 - s1, 3.0 / math.sqrt(D), atol=1e-12)
    np.testing.assert_allclose(o2, o1, atol=1e-12)


def test_attention_without_quantisation_is_textbook():
    # feeding exact keys/values reduces the oracle to softmax(q K^T/sqrt d) V
    rng = np.random.default_rng(17)
    q = rng.standard_normal(D)
    K = rng.standard_normal((50, D))
    V = rng.standard_normal((50, D))
    o, s = O.attention(q, K, V)
    p = special.softmax(K @ q / math.sqrt(D))
    np.testing.assert_allclose(o, p @ V, atol=1e-13)


def test_vectorised_unpacker_equals_per_token_spec():
    rng = np.random.default_rng(21)
    for bk, bv, qjl in ((4, 4, False), (3, 3, True), (2, 0, True)):
        lay = O.LayoutV1(128, 2, bk, bv, qjl, 3)
        pool = bytearray(rng.integers(0, 256, lay.pool_bytes, dtype=np.uint8).tobytes())
        vec = O.unpack_pool(pool, lay)
        for slot in (0, 5, 16, 47):
            for h in range(2):
                one = O.read_cache(pool, lay, slot, h)
                b, r = divmod(slot, 16)
                for k, v in one.items():
                    np.testing.assert_array_equal(np.asarray(vec[k][b, h, r]), np.asarray(v), err_msg=k)
        sub = O.unpack_pool(pool, lay, blocks=[2, 0])
        np.testing.assert_array_equal(sub["k_idx"][0], vec["k_idx"][2])


# ---------------------------------------------------------------------------
# Min/max comparison codec ([P4] Step 3 compress_value / decompress_value)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_minmax_arithmetic_progression_closed_form(bits):
    # rotated coordinates a + (b - a) j / 127 in a shuffled order: lo = a,
    # scale = (b - a) / (2^bits - 1), code of step j = round(j (2^bits-1)/127)
    # (127 is prime, so no step lands on a rounding tie)
    rng = np.random.default_rng(bits)
    a, b = -0.7, 1.3
    j = rng.permutation(128)
    y = a + (b - a) * j / 127.0
    x = y @ O.rotation_matrix(5, 128)           # R x = y
    enc = O.minmax_encode(x, 5, bits)
    levels = (1 << bits) - 1
    assert np.allclose(enc["y"], y, atol=1e-13)
    assert abs(enc["zero"] - a) < 1e-13 and abs(enc["scale"] - (b - a) / levels) < 1e-13
    assert np.array_equal(enc["codes"], np.rint(j * levels / 127.0).astype(np.int64))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_minmax_endpoints_and_error_bound(bits):
    rng = np.random.default_rng(10 + bits)
    x = rng.standard_normal((500, 128)) * rng.lognormal(size=(500, 1))
    enc = O.minmax_encode(x, 42, bits)
    levels = (1 << bits) - 1
    rows = np.arange(500)
    assert np.all(enc["codes"][rows, enc["y"].argmin(-1)] == 0)
    assert np.all(enc["codes"][rows, enc["y"].argmax(-1)] == levels)
    # with the exact scale and zero point every coordinate is within half a step
    yq = enc["codes"] * enc["scale"][:, None] + enc["zero"][:, None]
    assert np.all(np.abs(yq - enc["y"]) <= enc["scale"][:, None] / 2 * (1 + 1e-12))
    # decoding from the fp16 parameters adds at most their rounding errors
    xh = O.minmax_decode(enc["codes"], enc["scale16"], enc["zero16"], 42)
    yh = xh @ O.rotation_matrix(42, 128).T
    bound = (enc["scale"] / 2 + levels * np.abs(enc["scale16"].astype(np.float64) - enc["scale"])
             + np.abs(enc["zero16"].astype(np.float64) - enc["zero"]))
    assert np.all(np.abs(yh - enc["y"]) <= bound[:, None] * (1 + 1e-9))


def test_minmax_uniform_data_mse_is_step_squared_over_12():
    # i.i.d. U(-1, 1) rotated coordinates: a uniform quantiser's error is
    # uniform on half a step, mean square scale^2 / 12 (exact parameters)
    rng = np.random.default_rng(21)
    y = rng.uniform(-1, 1, size=(4000, 128))
    x = y @ O.rotation_matrix(3, 128)
    enc = O.minmax_encode(x, 3, 4)
    err = enc["codes"] * enc["scale"][:, None] + enc["zero"][:, None] - enc["y"]
    ratio = np.mean(err ** 2) / np.mean(enc["scale"] ** 2 / 12)
    assert abs(ratio - 1) < 0.02, ratio


def test_minmax_zero_vector():
    enc = O.minmax_encode(np.zeros((2, 128)), 42, 3)
    assert np.all(enc["codes"] == 0) and np.all(enc["scale16"] == 0) and np.all(enc["zero16"] == 0)
    assert np.all(O.minmax_decode(enc["codes"], enc["scale16"], enc["zero16"], 42) == 0)


def test_minmax_against_lloyd_max_on_gaussian_vectors():
    # The comparison the codec is built for.  Lloyd-Max is MSE-optimal for the
    # coordinate marginal (and spends 16 bits per vector on the norm, against
    # 32 for scale + zero point), so at every bit width its relative error on
    # N(0, I) vectors must be the lower one.
    rng = np.random.default_rng(33)
    x = rng.standard_normal((3000, 128))
    for bits in (2, 3, 4):
        c32, _ = O.codebook_fp32(128, bits)
        e = O.encode(x, 42, c32)
        xl = O.reconstruct(e["idx"], e["gamma16"], 42, c32)
        m = O.minmax_encode(x, 42, bits)
        xm = O.minmax_decode(m["codes"], m["scale16"], m["zero16"], 42)
        n2 = np.sum(x * x, axis=1)
        mse_l = np.mean(np.sum((x - xl) ** 2, axis=1) / n2)
        mse_m = np.mean(np.sum((x - xm) ** 2, axis=1) / n2)
        assert mse_l < mse_m, (bits, mse_l, mse_m)


# --------------------------------------------------------- triplet codec ----

def _unit_sphere(n, rng):
    g = rng.standard_normal((n, 3))
    return g / np.linalg.norm(g, axis=1, keepdims=True)


def test_oct_map_fixed_points_and_round_trip():
    pts = np.array([[0, 0, 1], [1, 0, 0], [0, 1, 0], [-1, 0, 0], [0, -1, 0]], float)
    xi, eta = O.oct_map(pts)
    np.testing.assert_allclose(np.stack([xi, eta], 1), [[0, 0], [1, 0], [0, 1], [-1, 0], [0, -1]], atol=1e-15)
    xi, eta = O.oct_map(np.array([[0.0, 0.0, -1.0]]))
    assert abs(xi[0]) == 1.0 and abs(eta[0]) == 1.0          # south pole: a corner
    # the diagonal direction of the first octant's equator lands mid-edge
    xi, eta = O.oct_map(np.array([[1.0, 1.0, 0.0]]) / math.sqrt(2))
    np.testing.assert_allclose([xi[0], eta[0]], [0.5, 0.5], atol=1e-15)
    n = _unit_sphere(5000, np.random.default_rng(3))
    xi, eta = O.oct_map(n)
    assert np.all(np.abs(xi) <= 1) and np.all(np.abs(eta) <= 1)
    np.testing.assert_allclose(O.oct_unmap(xi, eta), n, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(O.oct_unmap(*np.random.default_rng(4).uniform(-1, 1, (2, 999))),
                                              axis=1), 1.0, atol=1e-14)


def test_oct_unmap_is_equal_area():
    # the sphere (area 4 pi) over the square (area 4): the area element of the
    # inverse map is pi everywhere, measured by central differences
    rng = np.random.default_rng(5)
    p = rng.uniform(-0.98, 0.98, (400, 2))
    s = np.abs(p).sum(1)
    keep = (np.abs(s - 1) > 0.01) & (np.abs(p[:, 0]) > 0.01) & (np.abs(p[:, 1]) > 0.01)
    p = p[keep]
    h = 1e-6
    dx = (O.oct_unmap(p[:, 0] + h, p[:, 1]) - O.oct_unmap(p[:, 0] - h, p[:, 1])) / (2 * h)
    dy = (O.oct_unmap(p[:, 0], p[:, 1] + h) - O.oct_unmap(p[:, 0], p[:, 1] - h)) / (2 * h)
    np.testing.assert_allclose(np.linalg.norm(np.cross(dx, dy), axis=1), math.pi, rtol=1e-6)


def test_uniform_directions_map_to_uniform_square_so_the_uniform_codebook_is_lloyd_max():
    # triplets of uniform unit vectors in R^128 have isotropic directions, and
    # through the map xi and eta come out uniform on [-1, 1]
    rng = np.random.default_rng(6)
    g = rng.standard_normal((4000, D))
    t = (g / np.linalg.norm(g, axis=1, keepdims=True))[:, :126].reshape(-1, 3)
    xi, eta = O.oct_map(t / np.linalg.norm(t, axis=1, keepdims=True))
    from scipy import stats
    for v in (xi, eta):
        assert stats.kstest(v, "uniform", args=(-1, 2)).pvalue > 1e-3
    # uniform density: every centroid is the mean of its cell
    for bd in (3, 4, 5):
        c = O.octo_dir_codebook(bd)
        edges = np.concatenate(([-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
        np.testing.assert_allclose(c, 0.5 * (edges[:-1] + edges[1:]), atol=1e-15)
        assert np.all(np.diff(edges) > 0) and len(c) == 1 << bd


def test_rho_codebook_is_lloyd_max_by_quadrature_and_monte_carlo():
    from scipy import stats
    be = (D - 3) / 2.0
    dens = lambda r: 2 * r * stats.beta.pdf(r * r, 1.5, be)
    m2, _ = integrate.quad(lambda r: r * r * dens(r), 0, 1)
    assert abs(m2 - 3.0 / D) < 1e-10                        # E[rho^2] = 3/d
    for bits in (1, 2, 3):
        c, t = O.rho_lloyd_max(D, bits)
        edges = np.concatenate(([0.0], t, [1.0]))
        for i in range(len(c)):
            num, _ = integrate.quad(lambda r: r * dens(r), edges[i], edges[i + 1], epsabs=1e-14)
            den, _ = integrate.quad(dens, edges[i], edges[i + 1], epsabs=1e-14)
            assert abs(num / den - c[i]) < 1e-9
    rng = np.random.default_rng(8)
    g = rng.standard_normal((20000, D))
    rho = np.linalg.norm((g / np.linalg.norm(g, axis=1, keepdims=True))[:, :3], axis=1)
    c, _ = O.rho_lloyd_max(D, 3)
    cells = np.searchsorted(0.5 * (c[:-1] + c[1:]), rho)
    for i in range(8):
        sel = rho[cells == i]
        assert abs(sel.mean() - c[i]) < 5 * sel.std() / math.sqrt(len(sel)) + 1e-4


def test_triplet_joint_rounding_reaches_brute_force_and_beats_independent_rounding():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((60, D))
    for b in (2, 3):
        dirs, crho = O.octo_codebooks(D, b)
        e = O.octo_encode(x, 7, b, dirs, crho)
        t = e["t"]
        best = np.full(t.shape[:2], np.inf)
        for a in range(dirs.shape[0]):
            for c in range(dirs.shape[1]):
                for k in range(len(crho)):
                    best = np.minimum(best, np.sum((t - crho[k] * dirs[a, c]) ** 2, axis=-1))
        assert np.all(e["err"] >= best - 1e-15)
        assert np.mean(e["err"] <= best + 1e-15) > 0.99
        np.testing.assert_allclose(O.octo_triplet_error(t, e["a"], e["c"], e["k"], dirs, crho), e["err"], atol=1e-15)
        # independent rounding: nearest xi, eta, rho separately
        rho = np.linalg.norm(t, axis=-1)
        xi, eta = O.oct_map(t / rho[..., None])
        nd = dirs.shape[0]
        ja = np.clip(np.floor((xi + 1) * nd / 2).astype(int), 0, nd - 1)
        jc = np.clip(np.floor((eta + 1) * nd / 2).astype(int), 0, nd - 1)
        jk = np.argmin((rho[..., None] - crho) ** 2, axis=-1)
        ind = O.octo_triplet_error(t, ja, jc, jk, dirs, crho)
        assert np.all(e["err"] <= ind + 1e-15) and np.mean(e["err"] < ind - 1e-12) > 0.05


def test_triplet_codes_are_a_fixed_point_of_the_triplet_stage():
    # a triplet built from codes (a, c, k) encodes back to (a, c, k) with no
    # error: pins the a-major table index (xi first), the norm scaling and
    # the candidate window around the nearest cell
    rng = np.random.default_rng(10)
    for b in (2, 3, 4):
        dirs, crho = O.octo_codebooks(D, b)
        nd = dirs.shape[0]
        a, c, k = rng.integers(0, nd, 500), rng.integers(0, nd, 500), rng.integers(0, len(crho), 500)
        e = O.octo_encode_triplets(crho[k][:, None] * dirs[a, c], b, dirs, crho)
        np.testing.assert_array_equal(e["a"], a)
        np.testing.assert_array_equal(e["c"], c)
        np.testing.assert_array_equal(e["k"], k)
        assert np.all(e["err"] < 1e-12)


def test_triplet_codec_matches_the_pages_synthetic_results():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((8000, D))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    mse_page = {int(r.split()[0]): float(r.split()[1]) for r in _golden_lines("octopus_synthetic_mse.txt")}
    cos_page = {int(r.split()[0]): float(r.split()[1]) for r in _golden_lines("octopus_synthetic_cos.txt")}
    lm = {b: D * O.codebook_distortion(D, b) for b in (2, 3, 4)}
    for b in (2, 3, 4):
        dirs, crho = O.octo_codebooks(D, b)
        e = O.octo_encode(x, 7, b, dirs, crho)
        xh = O.octo_decode(e["a"], e["c"], e["k"], e["gamma"], 7, D, dirs, crho) / e["gamma"][:, None]
        mse = np.mean(np.sum((xh - u) ** 2, 1))
        cos = np.mean(np.sum(xh * u, 1) / np.linalg.norm(xh, axis=1))
        assert abs(mse - mse_page[b]) < 0.12 * mse_page[b], (b, mse)
        assert abs(cos - cos_page[b]) < 0.005, (b, cos)
        assert mse < lm[b]                               # below the per-coordinate codec


def test_triplet_codec_inner_product_error_matches_the_pages():
    """The pages' "IP" figures, read as mean |<q, k> - <q, k_hat>| over
    Gaussian q, k in d = 128 (golden file header): OCTOPUS at 2 / 3 / 4 bits
    and OCTOPUS-QJL (the residual sketch of octo_qjl_encode, estimate as in
    logits(..., qjl=...)) at 2 bits, each within 7%.  A sketch of the wrong
    residual, of q instead of R q, or one that drops gamma or rho would not
    bring the 2-bit error down by the page's quarter."""
    rows = [r.split() for r in _golden_lines("octopus_synthetic_ip.txt")]
    page = {(r[0], int(r[1])): float(r[2]) for r in rows}
    rng = np.random.default_rng(21)
    n = 4000
    x = rng.standard_normal((n, D))
    q = rng.standard_normal((n, D))
    exact = np.sum(q * x, 1)
    for b in (2, 3, 4):
        dirs, crho = O.octo_codebooks(D, b)
        e = O.octo_qjl_encode(x, 7, 99, b, dirs, crho)
        xh = O.octo_decode(e["a"], e["c"], e["k"], e["gamma16"], 7, D, dirs, crho)
        ip = np.mean(np.abs(exact - np.sum(q * xh, 1)))
        assert abs(ip - page[("octopus", b)]) < 0.07 * page[("octopus", b)], (b, ip)
        if b == 2:
            tau = 1.0 / math.sqrt(D)
            s = np.array([O.logits(q[i], xh[i:i + 1], qjl={"bits": e["qjl_bits"][i:i + 1], "rho16": e["qjl_rho16"][i:i + 1],
                                                            "gamma16": e["gamma16"][i:i + 1], "seed": 7, "seed_qjl": 99})[0]
                          for i in range(n)]) / tau
            ipq = np.mean(np.abs(exact - s))
            assert abs(ipq - page[("octopus_qjl", 2)]) < 0.07 * page[("octopus_qjl", 2)], ipq
            assert ipq < 0.8 * ip


def test_triplet_qjl_sketch_removes_the_inner_product_bias():
    """With the query along the key (q = x), <q, k_hat> falls short of
    <q, k> = |x|^2 by about |x|^2 * MSE (the reconstruction is shorter than
    the key); the residual sketch's estimate is unbiased, so OCTOPUS-QJL
    removes at least 90% of that bias at every width."""
    rng = np.random.default_rng(22)
    n = 3000
    x = rng.standard_normal((n, D))
    for b in (2, 3, 4):
        dirs, crho = O.octo_codebooks(D, b)
        e = O.octo_qjl_encode(x, 5, 77, b, dirs, crho)
        xh = O.octo_decode(e["a"], e["c"], e["k"], e["gamma16"], 5, D, dirs, crho)
        exact = np.sum(x * x, 1)
        plain = np.sum(x * xh, 1)
        R = O.rotation_matrix(5, D)
        est = O.qjl_dot_estimate(e["qjl_bits"], e["qjl_rho16"], x @ R.T, 77)
        corrected = plain + e["gamma16"].astype(np.float64) * est
        bias, bias_q = np.mean((plain - exact) / exact), np.mean((corrected - exact) / exact)
        assert bias < -0.004, (b, bias)     # about -MSE: -0.09, -0.026, -0.007
        assert abs(bias_q) < 0.1 * abs(bias), (b, bias, bias_q)


def test_triplet_qjl_residual_is_what_the_codes_leave_out():
    """r = y - y_hat exactly: y_hat + r rebuilds the rotated unit direction,
    |r|^2 is the triplet codec's squared error, and the sketch bits are the
    signs of R' r (brute force on a few vectors)."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((6, D)) * rng.uniform(0.1, 10, (6, 1))
    b = 3
    dirs, crho = O.octo_codebooks(D, b)
    e = O.octo_qjl_encode(x, 3, 4, b, dirs, crho)
    R, Rq = O.rotation_matrix(3, D), O.rotation_matrix(4, D)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = u @ R.T
    for i in range(6):
        yh = np.concatenate([crho[e["k"][i, j]] * dirs[e["a"][i, j], e["c"][i, j]] for j in range(O.octo_triplets(D))])[:D]
        r = y[i] - yh
        np.testing.assert_allclose(e["qjl_rho"][i], np.linalg.norm(r), rtol=1e-12)
        np.testing.assert_array_equal(e["qjl_bits"][i], (Rq @ r < 0).astype(np.uint8))
        xh = O.octo_decode(e["a"][i], e["c"][i], e["k"][i], 1.0, 3, D, dirs, crho)
        np.testing.assert_allclose(np.sum((u[i] - xh) ** 2), e["qjl_rho"][i] ** 2, rtol=1e-9)


def test_triplet_records_place_fields_lsb_first():
    b = 2                       # fields of 3 + 3 + 1 = 7 bits
    nt = O.octo_triplets(D)
    a = np.zeros(nt, int); c = np.zeros(nt, int); k = np.zeros(nt, int)
    a[0], c[0], k[0] = 5, 3, 1          # 101 | 011 << 3 | 1 << 6 = 0b1011101
    a[1], k[1] = 7, 1                   # bits 7..13: 0b1000111
    rec = O.octo_pack(a, c, k, b, D)
    assert rec.shape == (O.octo_record_bytes(D, b),) == (40,)
    assert rec[0] == 0b11011101 and rec[1] == 0b00100011
    assert np.all(rec[2:] == 0)
    assert [O.octo_record_bytes(D, b) for b in (2, 3, 4)] == [40, 56, 72]
    rng = np.random.default_rng(13)
    for b in (2, 3, 4):
        bd, bn = O.octo_bits(b)
        codes = [rng.integers(0, 1 << w, (4, nt)) for w in (bd, bd, bn)]
        back = O.octo_unpack(O.octo_pack(*codes, b, D), b, D)
        for u, v in zip(codes, back):
            np.testing.assert_array_equal(u, v)
