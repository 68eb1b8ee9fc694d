"""Pins of the CPU oracle against facts fixed outside the oracle itself:
published known-answer vectors, closed forms, textbook tables, the pages'
bounds and claims, brute force and Monte Carlo.  CPU only."""
import math
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import tq_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# --------------------------------------------------------------------- RNG
def test_philox_known_answers():
    for r in _rows("philox4x32_10_kat.txt"):
        v = [int(x, 16) for x in r]
        out = o.philox4x32_10(np.array(v[:4], np.uint32), np.array(v[4:6], np.uint32))
        assert [int(x) for x in out] == v[6:]


def test_philox_normals_law():
    z = o.philox_normals(12345, o.STREAM_ROTATION, 200000)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # streams and seeds give different numbers
    assert not np.allclose(z[:8], o.philox_normals(12345, o.STREAM_SKETCH, 8))
    assert not np.allclose(z[:8], o.philox_normals(12346, o.STREAM_ROTATION, 8))


# ---------------------------------------------------------------- rotation
@pytest.mark.parametrize("d", [8, 128])
def test_haar_orthogonal(d):
    p = o.haar_rotation(d, 7)
    assert np.max(np.abs(p.T @ p - np.eye(d))) < 1e-12
    assert abs(abs(np.linalg.det(p)) - 1) < 1e-10
    p32 = p.astype(np.float32).astype(np.float64)
    assert np.max(np.abs(p32.T @ p32 - np.eye(d))) < 1e-6


def test_haar_entries_and_rotated_coordinate_law():
    d = 64
    ent, coords = [], []
    u = np.zeros(d)
    u[0], u[5] = 0.6, 0.8
    for s in range(60):
        p = o.haar_rotation(d, 1000 + s)
        ent.append(p.ravel() * math.sqrt(d))
        coords.append(p @ u)
    ent = np.concatenate(ent)
    assert abs(ent.mean()) < 0.01 and abs(ent.var() - 1) < 0.02
    # coordinates of Pi u follow the Beta law of the paper review's "Method"
    al = (d - 1) / 2
    cdf = lambda t: special.betainc(al, al, (np.clip(t, -1, 1) + 1) / 2)
    assert stats.kstest(np.concatenate(coords), cdf).pvalue > 1e-3


def test_sylvester_hadamard_closed_form():
    # order 4 written out (Sylvester's construction), and H H^T = d I with
    # entry (i, j) = (-1)^popcount(i & j) at every order up to 256
    h4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], float)
    assert np.array_equal(o.sylvester_hadamard(4), h4)
    for d in (1, 2, 8, 64, 256):
        h = o.sylvester_hadamard(d)
        assert np.array_equal(h @ h.T, d * np.eye(d))
        i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
        par = np.vectorize(lambda v: bin(v).count("1") & 1)(i & j)
        assert np.array_equal(h, np.where(par == 1, -1.0, 1.0))
    with pytest.raises(ValueError):
        o.sylvester_hadamard(96)


def test_hadamard_rotation_orthogonal_and_sign_averaged_law():
    d = 128
    p = o.hadamard_rotation(d, 7)
    assert np.max(np.abs(p @ p.T - np.eye(d))) < 1e-13
    assert np.allclose(np.abs(p), 1 / math.sqrt(d))
    # the signs act on the input: for a fixed x, averaging over the signs
    # gives E[y_i^2] = ||x||^2 / d for every i (a sign layer on the output
    # instead would leave y_i^2 = (H x)_i^2 / d, far from flat for this x)
    x = np.zeros(d)
    x[0], x[1], x[9] = 0.6, 0.48, 0.64
    ys = np.stack([o.hadamard_rotation(d, 500 + s) @ x for s in range(400)])
    m2 = (ys ** 2).mean(axis=0)
    assert np.max(np.abs(m2 * d - 1)) < 0.35 and abs(m2.mean() * d - 1) < 1e-12
    s = o.rademacher_signs(4096, 3)
    assert set(np.unique(s)) == {-1.0, 1.0} and abs(s.mean()) < 4 / math.sqrt(4096)


def test_hadamard_codec_mse_near_codebook():
    # a randomized Hadamard rotation spreads a generic vector like the Haar
    # rotation: the empirical distortion stays near the Beta codebook's D
    d, b = 128, 2
    codec = o.turboquant_codec(d, b, "mse", rot_seed=11, rotation="hadamard")
    x = np.random.default_rng(2).normal(size=(20000, d))
    enc = o.encode(codec, x, round_norms=False)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    err = np.sum((u - o.reconstruct(codec, enc) / enc.nx[:, None]) ** 2, axis=1)
    D = codec.extra["lloyd_max"].mse * d
    assert abs(err.mean() - D) < 0.03 * D


# --------------------------------------------------------------- codebooks
def _density(d):
    z = math.exp(special.betaln(0.5, (d - 1) / 2))
    return lambda t: (1 - t * t) ** ((d - 3) / 2) / z


@pytest.mark.parametrize("d", [8, 128, 1536])
def test_beta_one_bit_closed_form(d):
    # +-E|T| with E|T| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)); total MSE 1 - d E|T|^2
    e = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    lm = o.beta_codebook(d, 1)
    # lgamma near 770 carries ~1e-13 absolute error, so ~1e-12 relative here
    assert np.allclose(lm.centroids, [-e, e], rtol=1e-11, atol=0)
    assert lm.boundaries[0] == 0.0
    assert abs(lm.mse * d - (1 - d * e * e)) < 1e-10


def test_beta_one_bit_values():
    # numeric values of the closed form at the dims used here
    for d, c, dm in ((8, 0.291026, 0.32243), (128, 0.0706616, 0.36089), (1536, 0.0203618, 0.36317)):
        lm = o.beta_codebook(d, 1)
        assert abs(lm.centroids[1] - c) < 1e-6 and abs(lm.mse * d - dm) < 1e-5


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_beta_d3_is_uniform_quantizer(bits):
    # d = 3: the law is uniform on [-1, 1], whose optimum quantizer is the
    # uniform one; total MSE 4^-b equals the lower bound exactly.
    lm = o.beta_codebook(3, bits)
    L = 1 << bits
    assert np.allclose(lm.centroids, -1 + (2 * np.arange(L) + 1) / L, atol=1e-9)
    assert abs(lm.mse * 3 - 4.0 ** -bits) < 1e-12


def test_gaussian_lloyd_max_matches_max_1960():
    for r in _rows("lloyd_max_gaussian_max1960.txt"):
        L = int(r[0])
        pos = [float(x) for x in r[1:-1]]
        lm = o.gaussian_codebook(int(math.log2(L)))
        assert np.allclose(lm.centroids[L // 2:], pos, rtol=0, atol=6e-4)
        assert abs(lm.mse - float(r[-1])) < 6e-5


def test_beta_tends_to_gaussian():
    for b in (1, 2, 3):
        g = o.gaussian_codebook(b)
        lm = o.beta_codebook(1536, b)
        assert np.allclose(lm.centroids * math.sqrt(1536), g.centroids, rtol=2e-3)
        assert abs(lm.mse * 1536 / g.mse - 1) < 2e-3


@pytest.mark.parametrize("d,bits", [(8, 2), (8, 3), (128, 2), (128, 4), (1536, 3)])
def test_lloyd_max_fixed_point_by_quadrature(d, bits):
    # Independent of the closed forms: adaptive quadrature of the density.
    f = _density(d)
    lm = o.beta_codebook(d, bits)
    edges = np.concatenate([[-1.0], lm.boundaries, [1.0]])
    s = 1 / math.sqrt(d)
    tot = 0.0
    for k in range(len(lm.centroids)):
        a, b = max(edges[k], -40 * s), min(edges[k + 1], 40 * s)
        pts = [x for x in (0.0,) if a < x < b]
        p = integrate.quad(f, a, b, epsabs=1e-15, epsrel=1e-13, limit=200, points=pts or None)[0]
        m1 = integrate.quad(lambda t: t * f(t), a, b, epsabs=1e-16, epsrel=1e-13, limit=200,
                            points=pts or None)[0]
        assert abs(m1 / p - lm.centroids[k]) < 1e-10 * max(1.0, s)
        tot += p
    assert abs(tot - 1) < 1e-10
    assert np.allclose(lm.boundaries, 0.5 * (lm.centroids[1:] + lm.centroids[:-1]), atol=1e-15)
    assert np.array_equal(lm.centroids, -lm.centroids[::-1])
    var = integrate.quad(lambda t: t * t * f(t), -1, 1, epsabs=1e-16, epsrel=1e-12, limit=400,
                         points=[0.0])[0]
    assert abs(var - 1 / d) < 1e-10


@pytest.mark.parametrize("d", [8, 128, 1536])
def test_mse_falls_with_bits_and_stays_within_bounds(d):
    # Paper review, "Validation"/"Results": total MSE of a unit vector at b bits
    # per coordinate lies between the lower bound 4^-b and (sqrt(3) pi / 2) 4^-b.
    prev = math.inf
    for b in range(1, 6):
        D = o.beta_codebook(d, b).mse * d
        assert D < prev
        assert 4.0 ** -b <= D <= math.sqrt(3) * math.pi / 2 * 4.0 ** -b
        prev = D


def test_loops_match_their_definitions():
    # The oracle's loop library against the definitions spelled out in Python
    # on tiny inputs: every output of dot_rows is the sum of the products of
    # one row of each operand (a swapped or transposed operand, a dropped
    # term or a stride slip changes some entry), and count_le counts the
    # boundaries at or below the value (ties included).
    rng = np.random.default_rng(17)
    a = rng.normal(size=(5, 7))
    b = rng.normal(size=(3, 7))
    c = o.dot_rows(a, b)
    assert c.shape == (5, 3)
    for i in range(5):
        for j in range(3):
            ref = 0.0
            for t in range(7):
                ref += a[i, t] * b[j, t]
            assert abs(c[i, j] - ref) <= 1e-13
    assert o.dot_rows(np.zeros((0, 4)), np.ones((2, 4))).shape == (0, 2)
    t = np.array([-0.5, 0.0, 0.25, 1.0])
    y = np.array([-1.0, -0.5, -0.1, 0.0, 0.1, 0.25, 0.9, 1.0, 2.0])
    assert o.count_le(t, y).tolist() == [sum(1 for tk in t if tk <= v) for v in y] == [0, 1, 1, 2, 2, 3, 3, 4, 4]


def test_quantize_matches_brute_force_d8():
    codec = o.turboquant_codec(8, 3, "mse", rot_seed=5)
    rng = np.random.default_rng(0)
    y = rng.normal(size=(5000, 8)) / math.sqrt(8)
    idx = o.quantize(codec, y, 0)
    c = codec.centroids[0][0]
    brute = np.argmin(np.abs(y[:, :, None] - c[None, None, :]), axis=2)
    dist = o.boundary_distance(codec, y)
    ok = dist > 1e-12
    assert np.array_equal(idx[ok], brute[ok])


def _perdim_codec(d, bits_of_dim, seed):
    """A codec whose dims carry different bit counts (and so different
    boundaries): Beta-law Lloyd-Max books of each dim's width, scaled per dim."""
    base = o.turboquant_codec(d, 2, "mse", rot_seed=seed)
    rng = np.random.default_rng(seed)
    scale = rng.uniform(0.5, 2.0, size=d)
    cents = [o._f32(o.beta_codebook(d, int(b)).centroids * scale[i]) for i, b in enumerate(bits_of_dim)]
    bnds = [o._f32(o.beta_codebook(d, int(b)).boundaries * scale[i]) for i, b in enumerate(bits_of_dim)]
    return o.Codec(d, "mse", np.asarray(bits_of_dim), 0, "row", base.rot, None, [cents], [bnds], False)


@pytest.mark.parametrize("uniform", [True, False])
def test_boundary_distance_planted_points(uniform):
    # Values fixed by construction: a point on a boundary is at distance 0,
    # one nudged by delta from it at delta, a midpoint between neighbouring
    # boundaries at half their gap, a point past the outermost boundary at its
    # offset; each dim measured against its own boundaries.
    d = 8
    codec = o.turboquant_codec(d, 3, "mse", rot_seed=3) if uniform else \
        _perdim_codec(d, [1, 2, 3, 4, 5, 3, 2, 1], 4)
    rows, want = [], []
    for i in range(d):
        t = codec.boundaries[0][0 if uniform else i]
        gaps = np.diff(t)
        half = 0.5 * (gaps.min() if len(gaps) else 1.0)
        delta = 1e-3 * half
        cases = [(t[0], 0.0), (t[-1], 0.0), (t[0] - delta, delta), (t[-1] + 3 * delta, 3 * delta),
                 (t[len(t) // 2] + delta, delta), (t[-1] + 0.25, 0.25)]
        if len(t) > 1:
            cases.append((0.5 * (t[0] + t[1]), 0.5 * (t[1] - t[0])))
        for val, dist in cases:
            y = np.full(d, 0.5 * (t[0] + t[-1]) if len(t) > 1 else t[0] + 0.5)
            y[i] = val
            rows.append(y)
            want.append((i, dist))
    got = o.boundary_distance(codec, np.array(rows))
    for r, (i, dist) in enumerate(want):
        assert abs(got[r, i] - dist) <= 1e-15 + 1e-12 * abs(dist), (r, i, got[r, i], dist)


@pytest.mark.parametrize("uniform", [True, False])
def test_boundary_distance_is_the_code_stability_radius(uniform):
    # The comparison rules excuse a code flip only within the band around a
    # boundary; that rests on boundary_distance being exactly how far a value
    # can move before its code changes.  Moving by (1 - eps) of the distance
    # either way keeps every code; moving by (1 + eps) of it changes the code
    # in at least one of the two directions.
    d = 128
    codec = o.turboquant_codec(d, 4, "mse", rot_seed=7) if uniform else \
        _perdim_codec(d, np.random.default_rng(9).integers(1, 6, size=d), 8)
    rng = np.random.default_rng(5)
    y = rng.normal(size=(400, d)) / math.sqrt(d)
    idx = o.quantize(codec, y, 0)
    dist = o.boundary_distance(codec, y)
    ok = dist > 1e-9
    for eps, changes in ((1e-6, False), (1e-6, True)):
        f = 1 - eps if not changes else 1 + eps
        up = o.quantize(codec, y + f * dist, 0) != idx
        dn = o.quantize(codec, y - f * dist, 0) != idx
        if changes:
            assert np.all((up | dn)[ok])
        else:
            assert not np.any((up | dn)[ok])


def test_mse_prod_crossover():
    # Paper review, figure "Inner-product distortion vs bit-width": the
    # unbiased prod variant has the lower inner-product error at low bit
    # widths, the mse variant beyond about 3 bits.  Measured here on the
    # self inner product <x, x_hat> of unit vectors (the case where the mse
    # variant's bias is largest), averaged over 12 rotations and sketches:
    # prod wins at b = 2 and 3, mse at b = 4 and 5.  A dropped or mis-scaled
    # QJL term makes prod biased and loses at every b.
    d, npairs = 128, 64
    rng = np.random.default_rng(21)
    err = {}
    for mode in ("mse", "prod"):
        for b in (2, 3, 4, 5):
            e = []
            for seed in range(12):
                codec = o.turboquant_codec(d, b, mode, rot_seed=3000 + seed, sketch_seed=4000 + seed)
                x = rng.normal(size=(npairs, d))
                x /= np.linalg.norm(x, axis=1, keepdims=True)
                enc = o.encode(codec, x, round_norms=False)
                s = np.diag(o.score(codec, x, enc))
                e.append(np.mean((s - 1.0) ** 2))
            err[mode, b] = float(np.mean(e))
    assert err["prod", 2] < err["mse", 2] and err["prod", 3] < err["mse", 3], err
    assert err["mse", 4] < err["prod", 4] and err["mse", 5] < err["prod", 5], err


def test_residual_sketch_of_own_codes_is_encode():
    # The QJL stage recomputed from a vector's own codes gives its stored
    # signs and n_r; from other codes it gives the residual of those codes.
    d = 128
    codec = o.turboquant_codec(d, 3, "prod", rot_seed=31, sketch_seed=32)
    x = np.random.default_rng(6).normal(size=(50, d))
    enc = o.encode(codec, x, round_norms=False)
    nr, z = o.residual_sketch(codec, enc.y, enc.idx)
    assert np.array_equal(z >= 0, enc.signs) and np.allclose(nr, enc.nr, rtol=0, atol=0)
    other = enc.idx.copy()
    other[:, 0] = 1 - other[:, 0] % 2 + 2 * (other[:, 0] // 2)   # flip the low bit of dim 0
    nr2, z2 = o.residual_sketch(codec, enc.y, other)
    c = codec.centroids[0][0]
    r2 = enc.y - c[other]
    assert np.allclose(nr2, np.linalg.norm(r2, axis=1), rtol=1e-14)
    assert np.allclose(z2, r2 @ codec.sketch.T, rtol=1e-12, atol=1e-14)


def test_empirical_mse_matches_codebook():
    d, b = 128, 2
    codec = o.turboquant_codec(d, b, "mse", rot_seed=11)
    x = np.random.default_rng(1).normal(size=(20000, d))
    enc = o.encode(codec, x, round_norms=False)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    err = np.sum((u - o.reconstruct(codec, enc) / enc.nx[:, None]) ** 2, axis=1)
    D = codec.extra["lloyd_max"].mse * d
    assert abs(err.mean() - D) < 4 * err.std() / math.sqrt(len(err)) + 2e-6


# ------------------------------------------------------------------ scoring
def test_two_scoring_paths_agree():
    d = 128
    codec = o.turboquant_codec(d, 3, "prod", rot_seed=13, sketch_seed=14)
    rng = np.random.default_rng(2)
    x, q = rng.normal(size=(300, d)), rng.normal(size=(7, d))
    enc = o.encode(codec, x)
    s1 = o.score(codec, q, enc)
    s2 = o.score_via_reconstruction(codec, q, enc)
    assert np.max(np.abs(s1 - s2)) < 1e-12 * np.max(np.abs(s1))


def _prod_mc(d, m_codec, x, q, seeds):
    vals = []
    for s in seeds:
        codec = m_codec(s)
        enc = o.encode(codec, x[None], round_norms=False)
        vals.append(o.score(codec, q[None], enc)[0, 0])
    return np.array(vals), codec, enc


def test_prod_estimator_unbiased_over_sketch():
    # Paper review, "Results": the prod variant is exactly unbiased.  Fixed x, q
    # and Pi; the mean over independent sketches S must equal <q, x>.
    d = 64
    rng = np.random.default_rng(3)
    x, q = rng.normal(size=d), rng.normal(size=d)
    codec0 = o.turboquant_codec(d, 3, "prod", rot_seed=21, sketch_seed=0)

    def mk(s):
        c = o.Codec(**{**codec0.__dict__})
        c.sketch = o.stored_sketch(d, 5000 + s)
        return c

    v, codec, enc = _prod_mc(d, mk, x, q, range(3000))
    se = v.std(ddof=1) / math.sqrt(len(v))
    assert abs(v.mean() - q @ x) < 4 * se
    # variance of the QJL term: (n_r^2/m) ((pi/2) |q'|^2 - <q', r_hat>^2) n_x^2
    qr = codec.rot[0] @ q
    y = enc.y[0]
    r = y - o.dequantize(codec, enc.idx, 0)[0]
    nr = np.linalg.norm(r)
    var = (nr ** 2 / d) * ((math.pi / 2) * qr @ qr - (qr @ (r / nr)) ** 2) * float(enc.nx[0]) ** 2
    assert abs(v.var(ddof=1) / var - 1) < 0.1


def test_fp16_sketch_rounding_bias_is_bounded():
    # The stored sketch is the Gaussian draw rounded to fp32 and then to fp16
    # (a reading of the pages, which fix no precision).  The QJL estimator
    # n_r sqrt(pi/2)/m sum_j <s_j, q'> sign<s_j, r> is exactly unbiased for
    # Gaussian rows s_j (paper review, "Results").  Per row, the paired
    # difference between the rounded and the exact sketch bounds the mean
    # shift the rounding causes: it stays below 2^-10 |q'| |r| (the spread of
    # the estimator over one 64-row sketch is about 0.16 |q'| |r|).  Entry by
    # entry the rounding is to nearest: within half an fp16 ulp, 2^-11
    # relative (truncation would reach 2^-10), or 2^-25 absolute below the
    # fp16 normal range.
    m = 64
    rng = np.random.default_rng(41)
    q, r = rng.normal(size=m), rng.normal(size=m)
    c = math.sqrt(math.pi / 2) * np.linalg.norm(r)
    est, diff = [], []
    for s in range(1000):
        g = o.gaussian_sketch(m, 9000 + s)
        st = o.stored_sketch(m, 9000 + s)
        assert np.all(np.abs(st - g) <= np.maximum(np.abs(g) * 2.0 ** -11, 2.0 ** -25))
        e_g = c * (g @ q) * np.where(g @ r >= 0, 1.0, -1.0)
        e_s = c * (st @ q) * np.where(st @ r >= 0, 1.0, -1.0)
        est.append(e_g)
        diff.append(e_s - e_g)
    est, diff = np.concatenate(est), np.concatenate(diff)
    se_est = est.std(ddof=1) / math.sqrt(len(est))
    assert abs(est.mean() - q @ r) < 4 * se_est          # the exact sketch is unbiased
    se = diff.std(ddof=1) / math.sqrt(len(diff))
    bound = 2.0 ** -10 * np.linalg.norm(q) * np.linalg.norm(r)
    assert 4 * se < bound                                # the check resolves the bound
    assert abs(diff.mean()) + 4 * se < bound


def test_mse_inner_product_is_biased():
    # Paper review, "Problem": mse-optimal quantizers give biased inner products.
    # At 1 bit and large d the mean of <q, x_hat> over random rotations is
    # (2/pi) <q, x> (derived: E|T| sqrt(2/pi) sqrt(d) -> 2/pi).
    d = 128
    rng = np.random.default_rng(4)
    x, q = rng.normal(size=d), rng.normal(size=d)
    q = q + 2 * x
    lm = o.beta_codebook(d, 1)
    ratios = []
    for s in range(300):
        c = o.Codec(d, "mse", np.full(d, 1), 0, "row", o._f32(o.haar_rotation(d, 9000 + s))[None],
                    None, [[o._f32(lm.centroids)] * d], [[o._f32(lm.boundaries)] * d])
        enc = o.encode(c, x[None], round_norms=False)
        ratios.append(o.score(c, q[None], enc)[0, 0] / (q @ x))
    assert abs(np.mean(ratios) - 2 / math.pi) < 0.02


def test_scores_converge_with_bits():
    d = 128
    rng = np.random.default_rng(5)
    x, q = rng.normal(size=(400, d)), rng.normal(size=(5, d))
    errs = []
    for b in (2, 3, 4, 5):
        c = o.turboquant_codec(d, b, "mse", rot_seed=31)
        errs.append(np.abs(o.score(c, q, o.encode(c, x)) - q @ x.T).mean())
    assert all(a > b for a, b in zip(errs, errs[1:]))


def test_zero_vector_scores_zero():
    codec = o.turboquant_codec(128, 3, "prod", rot_seed=1, sketch_seed=2)
    enc = o.encode(codec, np.zeros((1, 128)))
    assert float(enc.nx[0]) == 0.0
    assert o.score(codec, np.ones((1, 128)), enc)[0, 0] == 0.0


# ----------------------------------------------------------------- layout
@pytest.mark.parametrize("layout", ["row", "col"])
def test_layout_worked_example(layout):
    codec = o.Codec(8, "mse", np.full(8, 2), 0, layout, np.eye(8)[None], None,
                    [[np.zeros(4)] * 8], [[np.zeros(3)] * 8])
    idx = np.array([[0, 1, 2, 3, 3, 2, 1, 0], [3] * 8])
    enc = o.Encoded(idx, None, np.array([1.0, 2.0], np.float16), None, None, None)
    buf = o.pack(codec, enc)
    rows = {tuple(r[:2]): [int(v, 16) for v in r[2:]] for r in _rows("record_layout_example.txt")}
    assert len(buf) == 256
    if layout == "row":
        assert list(buf[:4]) == rows[("row", "code0")]
        assert list(buf[128:132]) == rows[("row", "nx")]
    else:
        fields = buf[:128].reshape(8, 16)
        assert list(fields[:, 0]) == rows[("col", "dim_byte0")]
        assert not fields[:, 1:].any()
        assert list(buf[128:132]) == rows[("col", "nx")]
    back = o.unpack(codec, buf, 2)
    assert np.array_equal(back.idx, idx)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("n", [1, 64, 100])
def test_pack_roundtrip(layout, n):
    rng = np.random.default_rng(n)
    codec = o.turboquant_codec(128, 3, "prod", rot_seed=3, sketch_seed=4, layout=layout)
    enc = o.encode(codec, rng.normal(size=(n, 128)))
    back = o.unpack(codec, o.pack(codec, enc), n)
    assert np.array_equal(back.idx, enc.idx) and np.array_equal(back.signs, enc.signs)
    assert np.array_equal(back.nx, enc.nx) and np.array_equal(back.nr, enc.nr)
    assert len(o.pack(codec, enc)) == ((n + 63) // 64) * o.tile_bytes(codec)


def test_record_sizes():
    k = o.turboquant_codec(128, 3, "prod", rot_seed=1, sketch_seed=2)
    v = o.turboquant_codec(128, 4, "mse", rot_seed=1, layout="col")
    assert o.tile_bytes(k) == 64 * 52 and o.tile_bytes(v) == 64 * 66


# -------------------------------------------------------------- attention
def test_attention_is_softmax_over_reconstructions():
    d, hq, hkv, T = 128, 8, 2, 200
    rng = np.random.default_rng(6)
    kc = o.turboquant_codec(d, 3, "prod", rot_seed=41, sketch_seed=42)
    vc = o.turboquant_codec(d, 4, "mse", rot_seed=41, layout="col")
    K, V = rng.normal(size=(hkv, T, d)), rng.normal(size=(hkv, T, d))
    q = rng.normal(size=(hq, d))
    ke = [o.encode(kc, K[h]) for h in range(hkv)]
    ve = [o.encode(vc, V[h]) for h in range(hkv)]
    scale = 1 / math.sqrt(d)
    out = o.decode_attention(kc, vc, q, ke, ve, scale)
    for h in range(hq):
        g = h // (hq // hkv)
        kh = o.reconstruct(kc, ke[g])
        w = special.softmax(scale * (kh @ q[h]))
        assert np.allclose(out[h], w @ o.reconstruct(vc, ve[g]), atol=1e-12)


def test_attention_equal_logits_give_mean_value():
    d = 128
    kc = o.turboquant_codec(d, 3, "prod", rot_seed=1, sketch_seed=2)
    vc = o.turboquant_codec(d, 4, "mse", rot_seed=1, layout="col")
    rng = np.random.default_rng(7)
    K = np.repeat(rng.normal(size=(1, d)), 50, axis=0)
    V = rng.normal(size=(50, d))
    out = o.decode_attention(kc, vc, rng.normal(size=(1, d)), [o.encode(kc, K)],
                             [o.encode(vc, V)], 0.1)
    assert np.allclose(out[0], o.reconstruct(vc, o.encode(vc, V)).mean(0), atol=1e-12)


# ------------------------------------------------------------------ top-k
def test_topk_brute_force_and_ties():
    s = np.array([[0.5, 0.9, 0.9, 0.1, 0.7]])
    v, i = o.topk(s, 3)
    assert i.tolist() == [[1, 2, 4]] and v.tolist() == [[0.9, 0.9, 0.7]]
    rng = np.random.default_rng(8)
    s = rng.normal(size=(4, 1000))
    v, i = o.topk(s, 10)
    for r in range(4):
        assert set(i[r]) == set(np.argsort(-s[r])[:10])


# ----------------------------------------------------------- SpectralQuant
def test_eigenbasis_and_spectrum():
    import synth
    law = synth.KVLaw(2, 128, 405)
    calib = np.stack([law.sample(h, 2048, __import__("torch").Generator().manual_seed(h), "cpu")
                      .float().numpy() for h in range(2)]).astype(np.float64)
    for h in range(2):
        lam, rows = o.eigenbasis(calib[h])
        xc = calib[h] - calib[h].mean(0)
        cov = xc.T @ xc / xc.shape[0]
        assert np.max(np.abs(rows @ rows.T - np.eye(128))) < 1e-12
        assert np.max(np.abs(cov @ rows.T - rows.T * lam[None, :])) < 1e-9 * lam[0]
        assert np.all(np.diff(lam) <= 0)
        frac = lam[:4].sum() / lam.sum()
        # about 80% of the variance in 4 of 128 eigendirections (SpectralQuant thread, tweet 2)
        assert 0.75 < frac < 0.95


def test_water_fill_is_optimal_by_brute_force():
    # the greedy allocation minimises sum lambda_i D(b_i) exactly (D convex):
    # check against every allocation of small cases
    import itertools
    D = {b: o.gaussian_codebook(b).mse for b in range(1, 6)}
    rng = np.random.default_rng(5)
    for d, total in ((3, 7), (4, 12), (4, 9), (5, 11)):
        for _ in range(6):
            lam = np.sort(rng.gamma(0.7, size=d))[::-1]
            got = o.water_fill(lam, total)
            assert got.sum() == total and got.min() >= 1 and got.max() <= 5
            best = min(sum(lam[i] * D[b[i]] for i in range(d))
                       for b in itertools.product(range(1, 6), repeat=d) if sum(b) == total)
            assert sum(lam[i] * D[got[i]] for i in range(d)) <= best * (1 + 1e-12)


def test_water_fill_special_cases():
    # equal variances share the bits evenly (the surplus to the lower dims);
    # a larger variance never gets fewer bits; the budget bounds are enforced
    assert np.array_equal(o.water_fill([1.0] * 8, 20), [3, 3, 3, 3, 2, 2, 2, 2])
    lam = np.array([0.5, 0.1, 0.04, 0.04] + [0.2 / 124] * 124)
    bits = o.water_fill(lam, 136)
    assert list(bits[:4]) == [5, 3, 2, 2] and np.all(bits[4:] == 1)  # the [SQ] tweet-6 map
    r = np.random.default_rng(6).gamma(0.5, size=64)
    b = o.water_fill(r, 150)
    order = np.argsort(-r, kind="stable")
    assert np.all(np.diff(b[order]) <= 0)
    with pytest.raises(ValueError):
        o.water_fill([1.0] * 4, 3)


def test_selective_qjl_unbiased_on_signal_dims():
    # QJL on the first m=4 rotated dims only (SpectralQuant thread, tweet 5): the
    # sign term estimates <q'_{0..3}, r_{0..3}> without bias over random S.
    d, m = 128, 4
    rng = np.random.default_rng(9)
    calib = rng.normal(size=(1, 512, d)) * np.linspace(3, 0.1, d)[None, None, :]
    bitmap = [5, 3, 2, 2] + [1] * (d - 4)
    base = o.spectralquant_codec(calib, bitmap, m, sketch_seed=1)
    x, q = calib[0, 7], rng.normal(size=d)
    vals = []
    for s in range(4000):
        c = o.Codec(**{**base.__dict__})
        c.sketch = o.stored_sketch(m, 777 + s)
        enc = o.encode(c, x[None], round_norms=False)
        qr, qs = o.prepare_query(c, q[None])
        vals.append(float(enc.nr[0]) * o.QJL_CONST / m * (qs[0] @ np.where(enc.signs[0], 1, -1)))
    r = enc.y[0, :m] - o.dequantize(c, enc.idx, 0)[0, :m]
    target = qr[0, :m] @ r
    vals = np.array(vals)
    assert abs(vals.mean() - target) < 4 * vals.std(ddof=1) / math.sqrt(len(vals))


# --------------------------------------------------- outlier-channel split
def _split(mode="prod", bits=(3, 2), heads=1, seed=11):
    rng = np.random.default_rng(seed)
    ch = np.stack([rng.permutation(128)[:32] for _ in range(heads)])
    return o.outlier_split_codec(128, ch, bits[0], bits[1], mode, rot_seed=40 + seed, sketch_seed=50 + seed)


def test_split_layout_worked_example():
    sc = _split()
    group, coord = o.split_stored_order(128, 32)
    rows = _rows("split_layout_example.txt")
    for r in rows:
        if r[0] == "order":
            i, g, c = int(r[1]), int(r[2]), int(r[3])
            assert (group[i], coord[i]) == (g, c)
    enc_o = o.Encoded(np.full((1, 32), 3), np.ones((1, 32), bool), np.array([2.0], np.float16),
                      np.array([0.25], np.float16), None, None)
    enc_r = o.Encoded(np.zeros((1, 96), np.int64), np.zeros((1, 96), bool), np.array([1.0], np.float16),
                      np.array([0.5], np.float16), None, None)
    buf = o.split_pack(sc, o.SplitEncoded(enc_o, enc_r))
    for r in rows:
        if r[0] == "bytes":
            off, want = int(r[1]), [int(v, 16) for v in r[2:]]
            assert list(buf[off:off + len(want)]) == want, off
        if r[0] == "tile":
            assert len(buf) == int(r[1]) == o.split_tile_bytes(sc)
    back = o.split_unpack(sc, buf, 1)
    assert np.array_equal(back.o.idx, enc_o.idx) and np.array_equal(back.r.signs, enc_r.signs)


@pytest.mark.parametrize("n", [1, 64, 130])
def test_split_pack_roundtrip(n):
    sc = _split()
    x = np.random.default_rng(n).normal(size=(n, 128))
    enc = o.split_encode(sc, x)
    back = o.split_unpack(sc, o.split_pack(sc, enc), n)
    for a, b in ((enc.o, back.o), (enc.r, back.r)):
        assert np.array_equal(a.idx, b.idx) and np.array_equal(a.signs, b.signs)
        assert np.array_equal(a.nx, b.nx) and np.array_equal(a.nr, b.nr)


def test_split_estimator_unbiased_over_sketches():
    # Each instance's prod estimate is unbiased over its sketch (paper review,
    # "Results"), so the sum over the two channel groups is unbiased for
    # <q, x>, and with independent sketches its variance is the sum of the two
    # QJL variances (n_r^2 / m_g)((pi/2)|q'_g|^2 - <q'_g, r_g/|r_g|>^2) n_x,g^2,
    # each with its own sketch size m_g.
    rng = np.random.default_rng(7)
    x, q = rng.normal(size=128), rng.normal(size=128)
    x[[3, 77]] *= 10.0
    sc0 = _split(seed=3)
    vals = []
    for s in range(2000):
        sc = o.SplitCodec(**{**sc0.__dict__})
        sc.inst_o = o.Codec(**{**sc0.inst_o.__dict__})
        sc.inst_r = o.Codec(**{**sc0.inst_r.__dict__})
        sc.inst_o.sketch = o.stored_sketch(32, 7000 + s)
        sc.inst_r.sketch = o.stored_sketch(96, 9000 + s)
        enc = o.split_encode(sc, x[None], round_norms=False)
        vals.append(o.split_score(sc, q[None], enc)[0, 0])
    vals = np.array(vals)
    se = vals.std(ddof=1) / math.sqrt(len(vals))
    assert abs(vals.mean() - q @ x) < 4 * se
    var = 0.0
    enc = o.split_encode(sc0, x[None], round_norms=False)
    for inst, part, chans in ((sc0.inst_o, enc.o, sc0.outlier[0]), (sc0.inst_r, enc.r, sc0.regular[0])):
        qr = inst.rot[0] @ q[chans]
        r = part.y[0] - o.dequantize(inst, part.idx, 0)[0]
        nr = np.linalg.norm(r)
        var += (nr ** 2 / inst.m) * ((math.pi / 2) * qr @ qr - (qr @ (r / nr)) ** 2) * float(part.nx[0]) ** 2
    assert abs(vals.var(ddof=1) / var - 1) < 0.12


def test_split_distortion_is_per_group():
    # Each group is normalised by its own norm, so its relative distortion is
    # the Lloyd-Max error of its own instance, d_g * D_g(b_g) (paper review,
    # "Method"), whatever the scale of the other group.
    sc = _split(mode="mse", bits=(4, 2), seed=5)
    rng = np.random.default_rng(9)
    x = rng.normal(size=(3000, 128))
    x[:, sc.outlier[0]] *= 30.0
    xh = o.split_reconstruct(sc, o.split_encode(sc, x, round_norms=False))
    for chans, inst in ((sc.outlier[0], sc.inst_o), (sc.regular[0], sc.inst_r)):
        err = np.sum((x[:, chans] - xh[:, chans]) ** 2, axis=1) / np.sum(x[:, chans] ** 2, axis=1)
        want = inst.d * inst.extra["lloyd_max"].mse
        assert abs(err.mean() / want - 1) < 0.05


def test_split_stored_form_gives_same_scores():
    # The library holds a split codec as one codec in stored order (rotation
    # rows placed on the channels, block-diagonal sketch, per-dim codebooks,
    # per-group norms and QJL factors sqrt(pi/2)/m_g).  Scoring through that
    # form, written out here from the layout rule, must give the two-instance
    # scores.
    for heads in (1, 2):
        sc = _split(heads=heads, seed=20 + heads)
        st = o.split_stored_codec(sc)
        group = st.extra["group"]
        rng = np.random.default_rng(heads)
        x, q = rng.normal(size=(40, 128)), rng.normal(size=(3, 128))
        for h in range(heads):
            enc = o.split_encode(sc, x, head=h)
            ref = o.split_score(sc, q, enc, head=h)
            flat = o._split_stored_encoded(sc, enc)
            qr = q @ st.rot[h].T
            qs = qr @ st.sketch.T
            chat = np.stack([np.array([st.centroids[h][i][flat.idx[t, i]] for i in range(128)])
                             for t in range(40)])
            pm = np.where(flat.signs, 1.0, -1.0)
            got = np.zeros_like(ref)
            for gsel, part in ((1, enc.o), (0, enc.r)):
                cols = group == gsel
                kap = math.sqrt(math.pi / 2) / cols.sum()
                code = qr[:, cols] @ chat[:, cols].T
                qjl = (qs[:, cols] @ pm[:, cols].T) * (part.nr.astype(np.float64) * kap)[None]
                got += (code + qjl) * part.nx.astype(np.float64)[None]
            assert np.allclose(got, ref, rtol=1e-10, atol=1e-10)
            # the stored rotation is orthogonal and the stored sketch block-diagonal
            assert np.max(np.abs(st.rot[h] @ st.rot[h].T - np.eye(128))) < 1e-5
            assert not st.sketch[np.ix_(group == 1, group == 0)].any()



def test_split_col_layout_worked_example():
    # Col records of 2.5-bit split values (32 outlier channels at 3 index
    # bits, 96 at 2), worked by hand from the layout: a token group's code
    # words are ordered by lane block n (coordinates 16 vb + n, vb = 0..7),
    # so within group 0 stored coordinate 0 (outlier, 3 bytes) sits at byte
    # 0, stored coordinate 16 (regular, 2 bytes) at byte 3, stored coordinate
    # 1 (outlier) at byte 20 (block 0: 4 x 3 + 4 x 2 bytes), stored coordinate
    # 8 (regular: block 8 starts after 8 blocks of 20 bytes) at byte 160; a
    # group is 8 x 20 + 8 x 16 = 288 bytes, so group 1 starts at 288.
    # Stored coordinate i = 32 blk + r is outlier coordinate 8 blk + r when
    # r < 8, else regular coordinate 24 blk + r - 8.
    sc = o.outlier_split_codec(128, np.arange(32) * 4, 3, 2, "mse", rot_seed=1, layout="col")
    n = 16
    io = np.zeros((n, 32), np.int64)
    ir = np.zeros((n, 96), np.int64)
    io[:8, 0] = [1, 2, 3, 4, 5, 6, 7, 0]     # stored 0, tokens 0..7
    ir[:8, 8] = [3, 0, 1, 2, 3, 0, 1, 2]     # stored 16 = regular 8
    io[:8, 1] = 5                            # stored 1
    ir[:8, 0] = [1, 1, 1, 1, 0, 0, 0, 0]     # stored 8 = regular 0
    io[8:, 0] = 7                            # stored 0, tokens 8..15 (group 1)
    enc = o.SplitEncoded(o.Encoded(io, None, np.full(n, 2.0, np.float16), None, None, None),
                         o.Encoded(ir, None, np.full(n, 0.5, np.float16), None, None, None))
    buf = o.split_pack(sc, enc)
    assert o.split_tile_bytes(sc) == 2560 and len(buf) == 2560
    # 1 + 2<<3 + 3<<6 + 4<<9 + 5<<12 + 6<<15 + 7<<18 = 0x1F58D1
    assert buf[0:3].tolist() == [0xD1, 0x58, 0x1F]
    # 3 + 0<<2 + 1<<4 + 2<<6 + 3<<8 + 0<<10 + 1<<12 + 2<<14 = 0x9393
    assert buf[3:5].tolist() == [0x93, 0x93]
    # eight 5s at 3 bits: 0b101 repeated = 0xB6DB6D
    assert buf[20:23].tolist() == [0x6D, 0xDB, 0xB6]
    # 1, 1, 1, 1, 0, 0, 0, 0 at 2 bits = 0x0055
    assert buf[160:162].tolist() == [0x55, 0x00]
    # group 1, stored 0: eight 7s = 0xFFFFFF
    assert buf[288:291].tolist() == [0xFF, 0xFF, 0xFF]
    assert np.count_nonzero(buf[:2304]) == 3 + 2 + 3 + 1 + 3
    # norms: regular n_x then the outlier n_x, fp16
    assert np.array_equal(buf[2304:2304 + 2 * n].view(np.float16), np.full(n, 0.5, np.float16))
    assert np.array_equal(buf[2432:2432 + 2 * n].view(np.float16), np.full(n, 2.0, np.float16))
    back = o.split_unpack(sc, buf, n)
    assert np.array_equal(back.o.idx, io) and np.array_equal(back.r.idx, ir)
