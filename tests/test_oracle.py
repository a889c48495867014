"""Pins of the CPU oracle against values fixed outside it: published test vectors,
textbook tables, closed forms, invariants and brute force on small inputs."""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import attention, codebook, quantize, rng, rotation
from tq_synth import random_unit_vectors

D = 128


# ---------------------------------------------------------------- generator --

def test_splitmix64_published_vectors(golden):
    for row in golden("splitmix64_vectors.txt"):
        seed, outs = int(row[0]), [int(x) for x in row[1:]]
        got = [int(v) for v in rng.splitmix64(seed, len(outs))]
        assert got == outs


def test_uniforms_open_interval_and_top_bits():
    z = rng.splitmix64(7, 1000)
    u = rng.uniforms(7, 1000)
    assert np.all(u > 0) and np.all(u <= 1)
    # u is the top 53 bits of each output plus one half, scaled by 2**-53
    k = (z >> np.uint64(11))
    small = k < np.uint64(1 << 52)
    assert np.array_equal(u[small] * 2.0**53 - 0.5, k[small].astype(np.float64))
    assert np.all(np.abs(u * 2.0**53 - k.astype(np.float64)) <= 1.0)


def test_box_muller_is_standard_normal():
    x = rng.normals(123, 400_000)
    assert abs(x.mean()) < 4 / math.sqrt(len(x))
    assert abs(x.var() - 1) < 4 * math.sqrt(2 / len(x))
    assert stats.kstest(x, "norm").pvalue > 1e-3
    # pairs: z0^2 + z1^2 = -2 ln u1 (the radius of the pair)
    u = rng.uniforms(123, 4)
    assert np.allclose(x[0] ** 2 + x[1] ** 2, -2 * np.log(u[0]), rtol=1e-12)


# ----------------------------------------------------------------- rotation --

def test_rotation_orthogonal_fp32():
    P = rotation.haar_rotation(42, D)
    assert np.abs(P.T @ P - np.eye(D)).max() <= 1e-5
    assert np.abs(P @ P.T - np.eye(D)).max() <= 1e-5


def test_rotation_is_q_of_seeded_gaussian_with_positive_r_diagonal():
    G = rotation.gaussian_matrix(42, D)
    P = rotation.haar_rotation_f64(42, D)
    R = P.T @ G
    assert np.abs(np.tril(R, -1)).max() < 1e-10
    assert np.all(np.diag(R) > 0)


def test_rotation_deterministic_and_seed_dependent():
    a = rotation.haar_rotation(42, D).astype(np.float32).tobytes()
    b = rotation.haar_rotation(42, D).astype(np.float32).tobytes()
    c = rotation.haar_rotation(43, D).astype(np.float32).tobytes()
    assert a == b and a != c


def test_rotation_entries_mean_zero_variance_one_over_d():
    P = rotation.haar_rotation(42, D)
    e = P.ravel()
    n = e.size
    assert abs(e.mean()) < 4 * math.sqrt(1 / D / n)
    # rows are unit vectors, so the mean square is exactly 1/d
    assert abs(np.mean(e * e) - 1 / D) < 1e-9
    # entries of a Haar matrix are close to N(0, 1/d): chi-square of the normalised entries
    z = e * math.sqrt(D)
    counts, edges = np.histogram(z, bins=np.linspace(-3, 3, 13))
    expected = n * np.diff(stats.norm.cdf(edges))
    chi2 = np.sum((counts - expected) ** 2 / expected)
    assert chi2 < stats.chi2.ppf(0.999, len(counts) - 1)


def test_haar_first_column_uniform_on_sphere():
    # Pi e1 over many seeds: each coordinate has variance 1/d and Pi e1 . e1 has
    # mean 0 (a sign bias would show if the sign fix were missing or wrong).
    vals = np.array([rotation.haar_rotation_f64(s, 16)[:, 0] for s in range(1500)])
    assert abs(vals[:, 0].mean()) < 4 * math.sqrt(1 / 16 / 1500)
    assert abs(np.mean(vals ** 2) - 1 / 16) < 0.01 / 16 * 4


def test_qjl_projection_gaussian():
    S = rotation.qjl_projection(4242, D)
    assert stats.kstest(S.ravel(), "norm").pvalue > 1e-3
    assert np.array_equal(S, rotation.gaussian_matrix(4242, D).astype(np.float32).astype(np.float64))


# ----------------------------------------------------------------- codebook --

def _max_table(golden):
    tab = {}
    for row in golden("lloyd_max_gaussian_max1960.txt"):
        tab[(int(row[0]), row[1])] = [float(x) for x in row[2:]]
    return tab


def test_one_bit_closed_form():
    c, _, _ = codebook.lloyd_max_gaussian(1)
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-13)
    assert abs(codebook.mse_fixed_point(c) - (1 - 2 / math.pi)) < 1e-13


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960(golden, bits):
    tab = _max_table(golden)
    L = 1 << bits
    c, _, _ = codebook.lloyd_max_gaussian(bits)
    pos = c[L // 2:]
    assert np.allclose(pos, tab[(L, "output")], atol=1.1e-3)
    mse = codebook.mse_fixed_point(c)
    assert abs(mse - tab[(L, "mse")][0]) / mse < 1e-3
    if (L, "threshold") in tab:
        _, t = codebook.canonical(bits)
        assert np.allclose(t[len(t) // 2:], tab[(L, "threshold")], atol=1.1e-3)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_fixed_point_symmetric(bits):
    c, it, delta = codebook.lloyd_max_gaussian(bits)
    assert delta < 1e-14
    assert codebook.lloyd_residual(c) < 1e-12
    assert np.array_equal(c, -c[::-1])
    assert np.all(np.diff(c) > 0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_canonical_codebook_fp16_exact_midpoints(bits):
    c16, t = codebook.canonical(bits)
    assert np.array_equal(c16.astype(np.float16).astype(np.float64), c16)
    assert np.array_equal(t.astype(np.float32).astype(np.float64), t)
    mid = (c16[:-1] + c16[1:]) / 2
    assert np.array_equal(t, mid)
    assert t[len(t) // 2] == 0.0 and not np.signbit(t[len(t) // 2])
    c, _, _ = codebook.lloyd_max_gaussian(bits)
    assert np.abs(c16 - c).max() <= np.abs(c).max() * 2.0**-11
    # rounding barely moves the MSE
    assert abs(codebook.expected_sq_error(c16, t) - codebook.mse_fixed_point(c)) < 1e-6


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_expected_sq_error_matches_monte_carlo(bits):
    c16, t = codebook.canonical(bits)
    x = np.random.default_rng(5).standard_normal(2_000_000)
    idx = np.searchsorted(t, x, side="right")
    err = (x - c16[idx]) ** 2
    closed = codebook.expected_sq_error(c16, t)
    assert abs(err.mean() - closed) < 4 * err.std() / math.sqrt(len(x))


# ------------------------------------------------- sphere-exact codebook --

def test_sphere_codebook_d3_is_the_uniform_quantizer():
    """d = 3: one coordinate of a uniform point on the 2-sphere is uniform on
    [-1, 1] (Archimedes), whose Lloyd-Max quantizer splits [-1, 1] into L equal
    cells with centroids at their middles; MSE (standard units, z = u sqrt 3)
    is 3 (2/L)^2 / 12 = 1/L^2."""
    for bits in (1, 2, 3):
        L = 1 << bits
        c, _, _ = codebook.lloyd_max_sphere(bits, 3)
        want = (-1.0 + (2 * np.arange(L) + 1) / L) * math.sqrt(3)
        assert np.allclose(c, want, atol=1e-12)
        assert abs(codebook.mse_fixed_point_sphere(c, 3) - 1.0 / L ** 2) < 1e-12


def test_sphere_codebook_one_bit_closed_form():
    """1 bit: the centroids are +-sqrt(d) E|u| = +-sqrt(d) Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2));
    d = 5 gives 3 sqrt(5) / 8 (density 3/4 (1 - u^2))."""
    c, _, _ = codebook.lloyd_max_sphere(1, 5)
    assert abs(c[1] - 3 * math.sqrt(5) / 8) < 1e-12
    for d in (16, 128, 1000):
        c, _, _ = codebook.lloyd_max_sphere(1, d)
        e = math.sqrt(d) * math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
        assert abs(c[1] - e) < 1e-12 and abs(c[0] + e) < 1e-12


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sphere_codebook_tends_to_gaussian(bits):
    """As d grows, sqrt(d) u tends to N(0, 1) and the codebooks agree, the gap
    shrinking like 1/d."""
    g, _, _ = codebook.lloyd_max_gaussian(bits)
    gap = [np.abs(codebook.lloyd_max_sphere(bits, d, tol=1e-11)[0] - g).max() for d in (1000, 10000)]
    assert gap[1] < 1e-3
    assert 8 < gap[0] / gap[1] < 12


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sphere_codebook_fixed_point_and_monte_carlo(bits):
    """d = 128: centroids are the conditional means of their cells under
    sampled sphere coordinates, and the fixed-point MSE matches the sampled
    quantization error; the sphere codebook's MSE is below the Gaussian one's on
    the same sphere data."""
    c, _, _ = codebook.lloyd_max_sphere(bits, D)
    assert np.allclose(c, -c[::-1], atol=0)
    X = random_unit_vectors(30000, D, 77 + bits)
    z = (X * math.sqrt(D)).ravel()
    t = (c[:-1] + c[1:]) / 2
    idx = np.searchsorted(t, z, side="right")
    for i in range(len(c)):
        sel = z[idx == i]
        assert abs(sel.mean() - c[i]) < 5 * sel.std() / math.sqrt(len(sel)) + 1e-9, i
    err = (z - c[idx]) ** 2
    assert abs(err.mean() - codebook.mse_fixed_point_sphere(c, D)) < 4 * err.std() / math.sqrt(len(z))
    g, _, _ = codebook.lloyd_max_gaussian(bits)
    tg = (g[:-1] + g[1:]) / 2
    err_g = (z - g[np.searchsorted(tg, z, side="right")]) ** 2
    assert codebook.mse_fixed_point_sphere(c, D) < err_g.mean() + 4 * err_g.std() / math.sqrt(len(z))


def test_sphere_canonical_fp16_exact_midpoints():
    for bits in (2, 3, 4):
        c16, t = codebook.canonical_sphere(bits, D)
        assert np.array_equal(c16, c16.astype(np.float16).astype(np.float64))
        assert np.all(np.diff(c16) > 0)
        mid = (c16[:-1] + c16[1:]) / 2
        mid[len(mid) // 2] = 0.0
        assert np.array_equal(t, mid)


# --------------------------------------------------- randomized Hadamard --

def test_hadamard_recursion_equals_popcount_form():
    for d in (1, 2, 8, 128):
        h = rotation.sylvester_hadamard(d)
        i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
        pc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
        assert np.array_equal(h, np.where(pc % 2 == 0, 1.0, -1.0))
        assert np.array_equal(h @ h.T, d * np.eye(d))


def test_hadamard_rotation_orthogonal_signs_from_generator():
    P = rotation.hadamard_rotation(42, D)
    assert np.abs(P.T @ P - np.eye(D)).max() <= 1e-6
    assert np.all(np.abs(np.abs(P) - np.float32(1 / math.sqrt(D))) == 0)
    # column j carries sign s_j: the top bit of SplitMix64 output j + 1
    z = rng.splitmix64(42, D)
    s = np.where(z >= np.uint64(1 << 63), -1.0, 1.0)
    assert np.array_equal(np.sign(P[0]), s)            # row 0 of H is all ones
    assert 40 < np.sum(s > 0) < 88                     # both signs present, roughly balanced
    assert not np.array_equal(rotation.hadamard_rotation(43, D), P)


# ----------------------------------------------------------------- quantize --

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_threshold_rule_is_nearest_centroid(bits):
    c16, t = codebook.canonical(bits)
    u = np.random.default_rng(bits).standard_normal((1000, D)) / math.sqrt(D)
    codes = quantize.codes_from_unit(u, t, D)
    cu = c16 / math.sqrt(D)
    nearest = np.argmin(np.abs(u[..., None] - cu), axis=-1)
    assert np.array_equal(codes, nearest)


def test_threshold_rule_ties_and_zero():
    c16, t = codebook.canonical(3)
    s = math.sqrt(D)
    u = np.array([[t[0] / s, t[3] / s, -0.0, 0.0, np.nextafter(t[3] / s, -1)] + [0.0] * (D - 5)])
    codes = quantize.codes_from_unit(u, t, D)[0]
    assert list(codes[:5]) == [1, 4, 4, 4, 3]
    q = quantize.quantize_head(np.zeros((2, D)), np.eye(D), c16, t)
    assert np.all(q["codes"] == 4) and np.all(q["norm"] == 0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_boundary_distance_geometry(bits):
    """The decision-boundary distance that decides which code mismatches the
    parity tests exempt (coordinates within 1e-6, unit domain, of a threshold).
    Fixed by geometry, not by the function's own formula: a coordinate placed
    exactly on threshold t_i / sqrt(d) is at distance 0; one moved by +-5e-7 is
    at 5e-7 (inside the band) on either side; one moved by +-2e-6 is outside;
    the midpoint of two adjacent thresholds is half their gap from both; far
    below the lowest or above the highest threshold the distance is to that
    outermost threshold. A missing sqrt(d), an absolute value on the wrong
    side or a distance to the wrong threshold fails one of these."""
    band = 1e-6
    _, t = codebook.canonical(bits)
    s = math.sqrt(D)
    for i, ti in enumerate(t):
        tu = ti / s
        for delta, want, inside in ((0.0, 0.0, True), (5e-7, 5e-7, True), (-5e-7, 5e-7, True),
                                    (2e-6, 2e-6, False), (-2e-6, 2e-6, False)):
            u = np.zeros((1, D))
            u[0, 7] = tu + delta
            got = quantize.boundary_distance(u, t, D)[0, 7]
            assert abs(got - want) < 1e-12, (bits, i, delta, got)
            assert (got < band) == inside, (bits, i, delta)
        if i + 1 < len(t):
            mid = (t[i] + t[i + 1]) / (2 * s)
            gap = (t[i + 1] - t[i]) / (2 * s)
            got = quantize.boundary_distance(np.full((1, 3), mid), t, D)
            assert np.allclose(got, gap, rtol=0, atol=1e-15)
            assert gap > 10 * band
    # outside the outermost thresholds: distance to that threshold
    lo, hi = t[0] / s, t[-1] / s
    got = quantize.boundary_distance(np.array([[lo - 0.25, hi + 0.5]]), t, D)[0]
    assert np.allclose(got, [0.25, 0.5], rtol=0, atol=1e-12)
    # a coordinate inside the band of threshold i is coded either side of it by
    # an arbitrarily small perturbation; one outside every band is not
    u = np.array([[t[0] / s - 4e-7, t[0] / s + 4e-7, t[0] / s + 3e-6]])
    d = quantize.boundary_distance(u, t, D)[0]
    codes = quantize.codes_from_unit(u, t, D)[0]
    assert d[0] < band and d[1] < band and d[2] > band
    assert codes[0] == 0 and codes[1] == 1 and codes[2] == 1


@pytest.mark.parametrize("bits,cos_lo,cos_hi,mse_rel", [
    (2, 0.9395, 0.9420, 0.03), (3, 0.9822, 0.9840, 0.03), (4, 0.9948, 0.9960, 0.04)])
def test_cosine_on_random_unit_vectors(bits, cos_lo, cos_hi, mse_rel):
    """Haar-rotated unit vectors at d=128: coordinate MSE close to the Gaussian
    Lloyd-Max value (sphere coordinates are slightly lighter-tailed) and the
    reconstruction cosine per bit width."""
    c16, t = codebook.canonical(bits)
    P = rotation.haar_rotation(42, D)
    X = random_unit_vectors(4000, D, 11 + bits)
    q = quantize.quantize_head(X, P, c16, t)
    xh = attention.dequantize_head(q["codes"], q["norm"], P, c16, D)
    cos = attention.cosine(X, xh).mean()
    assert cos_lo < cos < cos_hi
    mse = np.mean((q["u"] * math.sqrt(D) - c16[q["codes"]]) ** 2)
    assert abs(mse - codebook.expected_sq_error(c16, t)) / mse < mse_rel


def test_two_bit_cosine_matches_page_value(golden):
    page = {(r[0], int(r[1])): float(r[2]) for r in golden("page_claims.txt")}
    c16, t = codebook.canonical(2)
    P = rotation.haar_rotation(42, D)
    X = random_unit_vectors(4000, D, 77)
    q = quantize.quantize_head(X, P, c16, t)
    cos = attention.cosine(X, attention.dequantize_head(q["codes"], q["norm"], P, c16, D)).mean()
    assert abs(cos - page[("value_cosine", 2)]) < 0.005


# ------------------------------------------------------------------ packing --

def _expand(words):
    if words[-1].startswith("x"):
        return [int(w, 16) for w in words[:-1]] * int(words[-1][1:])
    return [int(w, 16) for w in words]


def test_packing_worked_words(golden):
    j = np.arange(D)
    for row in golden("packing_worked_words.txt"):
        layout, bits, pattern, words = row[0], int(row[1]), row[2], _expand(row[3:])
        if layout == "key":
            codes = {"j_mod_8": j % 8, "all_4": np.full(D, 4), "j_mod_4": j % 4, "j_mod_16": j % 16}[pattern]
            got = quantize.pack_keys(codes[None, :], bits)[0]
        else:
            tok = np.arange(8)
            codes = {"token_index": tok, "token_index_mod_4": tok % 4}[pattern]
            got = quantize.pack_values(np.repeat(codes[:, None], D, axis=1), bits)[0]
        assert [int(w) for w in got] == words, (layout, bits, pattern)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_roundtrip(bits):
    g = np.random.default_rng(bits)
    codes = g.integers(0, 1 << bits, size=(64, D))
    assert np.array_equal(quantize.unpack_keys(quantize.pack_keys(codes, bits), bits, D), codes)
    assert np.array_equal(quantize.unpack_values(quantize.pack_values(codes, bits), bits, D), codes)
    # both layouts spend d*bits/8 bytes per token
    assert quantize.pack_keys(codes, bits).nbytes == quantize.pack_values(codes, bits).nbytes == 64 * D * bits // 8


def test_value_layout_single_bit_positions():
    # token 8*blk + i, coordinate j, bits b  ->  block stream bit b*(8j+i)
    bits = 3
    codes = np.zeros((16, D), dtype=np.int64)
    codes[8 + 5, 77] = 1
    w = quantize.pack_values(codes, bits)
    pos = bits * (8 * 77 + 5)
    expect = np.zeros_like(w)
    expect[1, pos // 32] = 1 << (pos % 32)
    assert np.array_equal(w, expect)


# ---------------------------------------------------------------------- QJL --

def test_qjl_estimator_unbiased_with_closed_form_variance():
    """Over random Gaussian projections S, sqrt(pi/2)/d * |r| * (S y) . sign(S r)
    has mean y . r and variance (pi/2 |r|^2 |y|^2 - (y . r)^2) / d."""
    g = np.random.default_rng(9)
    y = g.standard_normal(D)
    r = 0.3 * g.standard_normal(D) / math.sqrt(D)
    M = 10000
    est = np.empty(M)
    for c in range(0, M, 500):
        S = g.standard_normal((500, D, D))
        Sy = S @ y
        sg = np.where(S @ r >= 0, 1.0, -1.0)
        est[c:c + 500] = math.sqrt(math.pi / 2) / D * np.linalg.norm(r) * np.sum(Sy * sg, axis=1)
    mean_true = y @ r
    var_true = (math.pi / 2 * (r @ r) * (y @ y) - mean_true ** 2) / D
    assert abs(est.mean() - mean_true) < 4 * math.sqrt(var_true / M)
    assert abs(est.var() / var_true - 1) < 0.06


def test_oracle_qjl_score_matches_estimator_definition():
    """The oracle's rotated-domain QJL score term equals the estimator written
    against the unrotated query (y = Pi q, residual r)."""
    c16, t = codebook.canonical(2)
    P = rotation.haar_rotation(42, D)
    S = rotation.qjl_projection(4242, D)
    g = np.random.default_rng(3)
    X = g.standard_normal((50, D))
    q = g.standard_normal((3, D))
    k = quantize.quantize_head(X, P, c16, t, S=S)
    s = attention.rotated_scores(q, k["codes"], k["norm"], P, c16, D, 1.0, k["signs"], k["gamma"], S)
    y = q @ P.T
    mse_part = y @ (c16[k["codes"]] / math.sqrt(D)).T
    sg = np.where(k["z"] >= 0, 1.0, -1.0)
    qjl_part = (y @ S.T) @ sg.T * (k["gamma"].astype(np.float64) * math.sqrt(math.pi / 2) / D)
    assert np.allclose(s, (mse_part + qjl_part) * k["norm"].astype(np.float64), rtol=1e-12, atol=1e-12)


def test_qjl_keys_unbiased_scores_mse_keys_shrunk():
    """QJL keys: slope of estimated vs true scores is 1; MSE-only 3-bit keys shrink
    scores by about 1 - MSE (the estimate is biased toward zero)."""
    P = rotation.haar_rotation(42, D)
    S = rotation.qjl_projection(4242, D)
    g = np.random.default_rng(4)
    X = g.standard_normal((6000, D))
    q = g.standard_normal((4, D))
    true = q @ X.T
    c2, t2 = codebook.canonical(2)
    k = quantize.quantize_head(X, P, c2, t2, S=S)
    est = attention.rotated_scores(q, k["codes"], k["norm"], P, c2, D, 1.0, k["signs"], k["gamma"], S)
    slope = np.sum(est * true) / np.sum(true * true)
    c3, t3 = codebook.canonical(3)
    k3 = quantize.quantize_head(X, P, c3, t3)
    est3 = attention.rotated_scores(q, k3["codes"], k3["norm"], P, c3, D, 1.0)
    slope3 = np.sum(est3 * true) / np.sum(true * true)
    assert abs(slope - 1) < 0.02
    assert abs(slope3 - (1 - codebook.expected_sq_error(c3, t3))) < 0.01


# ---------------------------------------------------------------- attention --

def _head_case(bits_k=3, bits_v=3, T=300, G=4, qjl=False, seed=0):
    g = np.random.default_rng(seed)
    P = rotation.haar_rotation(42, D)
    S = rotation.qjl_projection(4242, D) if qjl else None
    ck, tk = codebook.canonical(bits_k)
    cv, tv = codebook.canonical(bits_v)
    K = g.standard_normal((T, D)) * 3
    V = g.standard_normal((T, D))
    q = g.standard_normal((G, D))
    k = quantize.quantize_head(K, P, ck, tk, S=S)
    v = quantize.quantize_head(V, P, cv, tv)
    return P, S, ck, cv, K, V, q, k, v


@pytest.mark.parametrize("qjl", [False, True])
def test_rotated_domain_equals_textbook(qjl):
    P, S, ck, cv, K, V, q, k, v = _head_case(bits_k=2 if qjl else 3, qjl=qjl)
    Kh = attention.dequantize_head(k["codes"], k["norm"], P, ck, D,
                                   k.get("signs"), k.get("gamma"), S)
    Vh = attention.dequantize_head(v["codes"], v["norm"], P, cv, D)
    scale = 1 / math.sqrt(D)
    a = attention.attend_textbook(q, Kh, Vh, scale)
    b = attention.attend_rotated(q, k, v, P, P, ck, cv, D, scale, S=S)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_textbook_matches_pure_python_loop():
    P, S, ck, cv, K, V, q, k, v = _head_case(T=20, G=2)
    Kh = attention.dequantize_head(k["codes"], k["norm"], P, ck, D)
    Vh = attention.dequantize_head(v["codes"], v["norm"], P, cv, D)
    scale = 1 / math.sqrt(D)
    out = attention.attend_textbook(q, Kh, Vh, scale)
    for h in range(2):
        s = [scale * sum(q[h, j] * Kh[t, j] for j in range(D)) for t in range(20)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        o = [sum(e[t] / z * Vh[t, j] for t in range(20)) for j in range(D)]
        assert np.allclose(out[h], o, rtol=1e-12, atol=1e-14)
    assert np.allclose(attention.softmax(np.array([[1.0, 2.0, -3.0]])), special.softmax([1.0, 2.0, -3.0]))


def test_chunk_causal_against_textbook_mask():
    """The chunked causal attention equals textbook attention over the
    dequantized cache with the causal mask written out (query i sees keys
    0 .. ctx - M + i), and M = 1 is the decode."""
    rs = np.random.default_rng(21)
    T, M, G = 90, 6, 3
    c16, t = codebook.canonical(3)
    P = rotation.haar_rotation(42, D)
    K = rs.standard_normal((T, D))
    V = rs.standard_normal((T, D))
    kq = quantize.quantize_head(K, P, c16, t)
    vq = quantize.quantize_head(V, P, c16, t)
    Kh = attention.dequantize_head(kq["codes"], kq["norm"], P, c16, D)
    Vh = attention.dequantize_head(vq["codes"], vq["norm"], P, c16, D)
    q = rs.standard_normal((M, G, D))
    sc = 1 / math.sqrt(D)
    for ctx in (T, 50, M, 3):
        got = attention.attend_chunk_causal(q, kq, vq, P, P, c16, c16, D, sc, ctx)
        for i in range(M):
            n = max(ctx - M + i + 1, 0)
            for g in range(G):
                if n == 0:
                    assert np.all(got[i, g] == 0)
                    continue
                s = (Kh[:n] @ q[i, g]) * sc
                w = np.exp(s - s.max())
                assert np.allclose(got[i, g], (w / w.sum()) @ Vh[:n], atol=1e-12)
    one = attention.attend_chunk_causal(q[:1], kq, vq, P, P, c16, c16, D, sc, T)
    assert np.allclose(one[0], attention.attend_rotated(q[0], kq, vq, P, P, c16, c16, D, sc), atol=0)


def test_single_token_returns_its_value():
    P, S, ck, cv, K, V, q, k, v = _head_case(T=1)
    Vh = attention.dequantize_head(v["codes"], v["norm"], P, cv, D)
    o = attention.attend_rotated(q, k, v, P, P, ck, cv, D, 1 / math.sqrt(D))
    assert np.allclose(o, np.repeat(Vh, q.shape[0], axis=0), rtol=1e-12, atol=1e-14)


def test_identical_keys_average_values():
    P, S, ck, cv, K, V, q, k, v = _head_case(T=50)
    k = {"codes": np.repeat(k["codes"][:1], 50, axis=0), "norm": np.repeat(k["norm"][:1], 50)}
    Vh = attention.dequantize_head(v["codes"], v["norm"], P, cv, D)
    o = attention.attend_rotated(q, k, v, P, P, ck, cv, D, 1 / math.sqrt(D))
    assert np.allclose(o, np.repeat(Vh.mean(axis=0, keepdims=True), q.shape[0], axis=0), rtol=1e-10, atol=1e-13)


def test_ctx_len_truncates_and_zero_context_gives_zero():
    P, S, ck, cv, K, V, q, k, v = _head_case(T=100)
    sc = 1 / math.sqrt(D)
    a = attention.attend_rotated(q, k, v, P, P, ck, cv, D, sc, ctx_len=37)
    kk = {key: val[:37] for key, val in k.items() if key in ("codes", "norm")}
    vv = {key: val[:37] for key, val in v.items() if key in ("codes", "norm")}
    b = attention.attend_rotated(q, kk, vv, P, P, ck, cv, D, sc)
    assert np.array_equal(a, b)
    assert np.all(attention.attend_rotated(q, k, v, P, P, ck, cv, D, sc, ctx_len=0) == 0)


@pytest.mark.parametrize("bounds", [[(0, 300)], [(0, 32), (32, 64), (64, 300)],
                                    [(0, 100), (100, 100), (100, 299), (299, 300)]])
def test_split_merge_equals_one_pass(bounds):
    P, S, ck, cv, K, V, q, k, v = _head_case(T=300)
    sc = 1 / math.sqrt(D)
    s = attention.rotated_scores(q, k["codes"], k["norm"], P, ck, D, sc)
    vr = v["norm"].astype(np.float64)[:, None] * cv[v["codes"]] / math.sqrt(D)
    o_rot = attention.merge_partials(attention.split_partials(s, vr, bounds))
    one = attention.softmax(s) @ vr
    assert np.abs(o_rot - one).max() <= 1e-12 * np.abs(one).max()


# ------------------------------------------------- head dimensions 64, 256 --
# The method is stated for any d; these pins hold the oracle at the two other
# head dimensions the library takes.

HEAD_DIMS = (64, 256)


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_rotations_other_head_dims(d):
    P = rotation.haar_rotation_f64(42, d)
    assert np.abs(P.T @ P - np.eye(d)).max() <= 1e-12
    R = P.T @ rotation.gaussian_matrix(42, d)
    assert np.abs(np.tril(R, -1)).max() < 1e-10 and np.all(np.diag(R) > 0)
    H = rotation.hadamard_rotation(42, d)
    assert np.abs(H.T @ H - np.eye(d)).max() <= 1e-6
    assert np.all(np.abs(np.abs(H) - np.float32(1 / math.sqrt(d))) == 0)
    z = rng.splitmix64(42, d)
    assert np.array_equal(np.sign(H[0]), np.where(z >= np.uint64(1 << 63), -1.0, 1.0))


def _sphere_law_sq_error(c, t, d):
    """E[(sqrt(d) u - c[cell(u)])^2] for u one coordinate of a uniform unit vector
    in d dimensions, density proportional to (1 - u^2)^((d-3)/2) on [-1, 1]:
    E[d u^2] = 1, so the error is 1 - 2 sum c_i m_i + sum c_i^2 P_i with P_i the
    cell's probability and m_i = sqrt(d) E[u; cell i] (the incomplete beta law
    and the first moment in closed form)."""
    a = (d - 1) / 2.0
    k = (d - 3) / 2.0
    sd = math.sqrt(d)
    edges = np.concatenate([[-1.0], np.asarray(t) / sd, [1.0]])
    P = np.diff(special.betainc(a, a, (1.0 + edges) / 2.0))
    g = np.exp((k + 1.0) * np.log(np.maximum(1.0 - edges ** 2, 1e-300)) - special.betaln(0.5, k + 1.0))
    m = sd * (g[:-1] - g[1:]) / (2.0 * (k + 1.0))
    return 1.0 - 2.0 * float(np.sum(c * m)) + float(np.sum(c ** 2 * P))


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_error_matches_sphere_law(d, bits):
    """Haar-rotated unit vectors in d dimensions: the mean squared error of the
    scaled coordinates against their centroids equals the closed form under the
    exact law of one sphere coordinate (within 4 standard errors of the sample),
    which tells d = 64 from the Gaussian limit and from d = 128."""
    c16, t = codebook.canonical(bits)
    P = rotation.haar_rotation(42, d)
    X = random_unit_vectors(4000, d, 11 + bits)
    q = quantize.quantize_head(X, P, c16, t)
    err = (q["u"] * math.sqrt(d) - c16[q["codes"]]) ** 2
    per_vec = err.mean(axis=1)
    want = _sphere_law_sq_error(c16, t, d)
    assert abs(per_vec.mean() - want) <= 4 * per_vec.std() / math.sqrt(len(per_vec))
    if d == 64:
        other = _sphere_law_sq_error(c16, t, 4096)   # close to the Gaussian limit
        assert abs(other - want) > 6 * per_vec.std() / math.sqrt(len(per_vec))


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_roundtrip_other_head_dims(d, bits):
    g = np.random.default_rng(bits + d)
    codes = g.integers(0, 1 << bits, size=(24, d))
    assert np.array_equal(quantize.unpack_keys(quantize.pack_keys(codes, bits), bits, d), codes)
    assert np.array_equal(quantize.unpack_values(quantize.pack_values(codes, bits), bits, d), codes)
    assert quantize.pack_keys(codes, bits).nbytes == quantize.pack_values(codes, bits).nbytes == 24 * d * bits // 8


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_value_layout_single_bit_other_head_dims(d):
    bits = 3
    j = d - 3
    codes = np.zeros((16, d), dtype=np.int64)
    codes[8 + 5, j] = 1
    w = quantize.pack_values(codes, bits)
    pos = bits * (8 * j + 5)
    expect = np.zeros_like(w)
    expect[1, pos // 32] = 1 << (pos % 32)
    assert np.array_equal(w, expect)
    kc = np.zeros((1, d), dtype=np.int64)
    kc[0, j] = 5   # key layout: code j at bits [3j, 3j + 3)
    kw = quantize.pack_keys(kc, bits)[0]
    got = sum(int(x) << (32 * i) for i, x in enumerate(kw))
    assert got == 5 << (bits * j)


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_rotated_domain_equals_textbook_other_head_dims(d):
    g = np.random.default_rng(d)
    P = rotation.haar_rotation(42, d)
    ck, tk = codebook.canonical(4)
    cv, tv = codebook.canonical(2)
    k = quantize.quantize_head(g.standard_normal((200, d)) * 3, P, ck, tk)
    v = quantize.quantize_head(g.standard_normal((200, d)), P, cv, tv)
    q = g.standard_normal((5, d))
    Kh = attention.dequantize_head(k["codes"], k["norm"], P, ck, d)
    Vh = attention.dequantize_head(v["codes"], v["norm"], P, cv, d)
    scale = 1 / math.sqrt(d)
    a = attention.attend_textbook(q, Kh, Vh, scale)
    b = attention.attend_rotated(q, k, v, P, P, ck, cv, d, scale)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()
    # one token: its value; identical keys: the mean value
    one = attention.attend_rotated(q, {"codes": k["codes"][:1], "norm": k["norm"][:1]},
                                   {"codes": v["codes"][:1], "norm": v["norm"][:1]}, P, P, ck, cv, d, scale)
    assert np.allclose(one, np.repeat(Vh[:1], 5, axis=0), rtol=1e-12, atol=1e-14)


def test_package_imports_only_numpy_scipy():
    import sys
    assert "decode_attention_tq_amd" not in oracle.__dict__
    for m in (rng, rotation, codebook, quantize, attention):
        src = open(m.__file__).read()
        assert "decode_attention_tq_amd" not in src and "torch" not in src
