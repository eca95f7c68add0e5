"""Pins of the fp64 oracle to things other than itself.

Each check below would fail for a plausible slip in the oracle: a wrong
codebook scale or level, a transposed or re-ordered transform, a wrong sign,
a dropped norm, an off-by-one code, a wrong bit order, a wrong GQA mapping, a
wrong softmax scale, a k-means update error.  Independent routes used:
closed forms, the published Gaussian Lloyd-Max table (tests/golden), numerical
quadrature (scipy), scipy's Sylvester Hadamard matrix, numpy bit unpacking,
torch's scaled-dot-product attention on dequantized keys, scikit-learn's Lloyd
k-means, and brute-force nearest-level / nearest-centroid search.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.stats

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "max1960_gaussian_lloyd_max.txt")


def _max_table():
    tab = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            tab[(int(parts[0]), parts[1])] = [p for p in parts[2:]]
    return tab


def _tol(s: str) -> float:
    # half a unit in the last printed digit, plus slack for known last-digit errors in the table
    dec = len(s.split(".")[1]) if "." in s else 0
    return 0.5 * 10.0 ** (-dec) + 1.5e-4


# ----------------------------------------------------------------------------------------------
# Codebook
# ----------------------------------------------------------------------------------------------

def test_lloyd_max_b1_closed_form(oracle_mod):
    c, t, it = oracle_mod.lloyd_max_unit(1)
    assert it > 0
    assert c[1] == pytest.approx(math.sqrt(2.0 / math.pi), abs=1e-12)
    assert c[0] == -c[1]
    assert t[0] == 0.0


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960_table(oracle_mod, b):
    L = 1 << b
    tab = _max_table()
    c, t, it = oracle_mod.lloyd_max_unit(b)
    assert it > 0
    pos_levels = c[L // 2:]
    pos_thr = t[L // 2 - 1:]
    for got, s in zip(pos_levels, tab[(L, "levels")]):
        assert abs(got - float(s)) <= _tol(s), (b, got, s)
    for got, s in zip(pos_thr, tab[(L, "thresholds")]):
        assert abs(got - float(s)) <= _tol(s), (b, got, s)
    mse = oracle_mod.quantizer_mse_unit(b, c, t)
    assert mse == pytest.approx(float(tab[(L, "mse")][0]), rel=1e-3)


def test_lloyd_max_b2_values_given_for_the_method(oracle_mod):
    c, _, _ = oracle_mod.lloyd_max_unit(2)
    assert c[2] == pytest.approx(0.4528, abs=5e-5)
    assert c[3] == pytest.approx(1.5104, abs=5e-5)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_lloyd_max_fixed_point_by_quadrature(oracle_mod, b):
    """Every level is the conditional mean of its cell (scipy quadrature, independent of erfc)."""
    L = 1 << b
    c, t, _ = oracle_mod.lloyd_max_unit(b)
    edges = [-np.inf] + list(t) + [np.inf]
    pdf = scipy.stats.norm.pdf
    for j in range(L):
        mass = scipy.integrate.quad(pdf, edges[j], edges[j + 1], epsabs=1e-14, epsrel=1e-13)[0]
        mom = scipy.integrate.quad(lambda x: x * pdf(x), edges[j], edges[j + 1], epsabs=1e-14, epsrel=1e-13)[0]
        assert mom / mass == pytest.approx(c[j], abs=1e-10)
    # thresholds are midpoints, levels strictly increasing and odd-symmetric
    np.testing.assert_allclose(t, 0.5 * (c[1:] + c[:-1]), rtol=0, atol=1e-15)
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(c, -c[::-1])


@pytest.mark.parametrize("b", [2, 3, 4])
def test_lloyd_max_is_a_local_minimum_of_mse(oracle_mod, b):
    """Perturbing any single level (thresholds re-derived) raises the quadrature MSE."""
    c, t, _ = oracle_mod.lloyd_max_unit(b)

    def mse_quad(levels):
        thr = 0.5 * (levels[1:] + levels[:-1])
        edges = [-np.inf] + list(thr) + [np.inf]
        tot = 0.0
        for j, cj in enumerate(levels):
            tot += scipy.integrate.quad(lambda x: (x - cj) ** 2 * scipy.stats.norm.pdf(x),
                                        edges[j], edges[j + 1], epsabs=1e-14)[0]
        return tot

    base = mse_quad(c)
    assert base == pytest.approx(oracle_mod.quantizer_mse_unit(b, c, t), rel=1e-9)
    for j in range(len(c)):
        for eps in (1e-3, -1e-3):
            p = c.copy()
            p[j] += eps
            assert mse_quad(p) > base


@pytest.mark.parametrize("d,b", [(16, 2), (64, 4), (128, 3), (128, 1)])
def test_codebook_is_unit_quantizer_over_sqrt_d(oracle_mod, d, b):
    c, t, _ = oracle_mod.lloyd_max_unit(b)
    lv, th = oracle_mod.codebook(d, b)
    np.testing.assert_allclose(lv, c / math.sqrt(d), rtol=1e-15)
    np.testing.assert_allclose(th, t / math.sqrt(d), rtol=1e-15)


def test_rotated_coordinates_have_variance_one_over_d(oracle_mod):
    """The premise of the fixed codebook: coordinates of H D k/|k| spread like N(0, 1/d)."""
    d = 64
    rng = np.random.default_rng(5)
    k = rng.standard_normal((2000, d)) * rng.lognormal(0, 1, size=d)  # outlier channels
    s = W.signs(W.LONGCTX)
    lv, th = oracle_mod.codebook(d, 4)
    _, _, y, _ = oracle_mod.encode_keys(th, s, k, 4)
    assert np.mean(y ** 2) == pytest.approx(1.0 / d, rel=1e-12)  # exact: |y| = 1
    # the rotation pulls outlier channels towards the Gaussian shape
    kurt = np.mean(y ** 4) / np.mean(y ** 2) ** 2
    raw = k / np.linalg.norm(k, axis=1, keepdims=True)
    kurt_raw = np.mean(raw ** 4) / np.mean(raw ** 2) ** 2
    assert abs(kurt - 3.0) < 1.0 < abs(kurt_raw - 3.0)
    # isotropic keys: a coordinate of a uniform unit vector has kurtosis 3d/(d+2) (closed form)
    k_iso = rng.standard_normal((20000, d))
    _, _, y_iso, _ = oracle_mod.encode_keys(th, s, k_iso, 4)
    kurt_iso = np.mean(y_iso ** 4) / np.mean(y_iso ** 2) ** 2
    assert kurt_iso == pytest.approx(3.0 * d / (d + 2), rel=0.02)


# ----------------------------------------------------------------------------------------------
# Transform
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
def test_hadamard_is_sylvester_and_orthogonal(oracle_mod, d):
    H = oracle_mod.hadamard(d)
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(d) / math.sqrt(d))
    np.testing.assert_allclose(H @ H.T, np.eye(d), atol=1e-13)


@pytest.mark.parametrize("d", [16, 64, 128])
def test_rotation_preserves_inner_products(oracle_mod, d):
    rng = np.random.default_rng(d)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    qr = oracle_mod.rotate_query(s, q)
    kr = oracle_mod.rotate_query(s, k)
    assert qr @ kr == pytest.approx(q @ k, rel=1e-12, abs=1e-12)
    assert np.linalg.norm(qr) == pytest.approx(np.linalg.norm(q), rel=1e-13)
    # the sign pattern acts before H: compare with an independent construction
    Hs = scipy.linalg.hadamard(d) / math.sqrt(d)
    np.testing.assert_allclose(qr, Hs @ (s * q), atol=1e-12)
    assert not np.allclose(qr, s * (Hs @ q))


# ----------------------------------------------------------------------------------------------
# Write path
# ----------------------------------------------------------------------------------------------

def _independent_codes(keys, signs, levels, d):
    """Nearest level of each rotated coordinate, via scipy's Hadamard and argmin."""
    Hs = scipy.linalg.hadamard(d) / math.sqrt(d)
    k = np.asarray(keys, dtype=np.float64).reshape(-1, d)
    u = k / np.linalg.norm(k, axis=1, keepdims=True)
    y = (u * signs) @ Hs.T
    idx = np.argmin(np.abs(y[..., None] - np.asarray(levels)[None, None, :]), axis=-1)
    return idx, y


@pytest.mark.parametrize("d,b", [(16, 2), (16, 1), (32, 3), (64, 4), (128, 4), (128, 3)])
def test_encode_codes_equal_nearest_level(oracle_mod, d, b):
    rng = np.random.default_rng(100 + d + b)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    keys = rng.standard_normal((300, d)) * rng.lognormal(0, 1, size=(300, 1))
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, y, tie = oracle_mod.encode_keys(th, s, keys, b)
    idx, y_ind = _independent_codes(keys, s, lv, d)
    np.testing.assert_allclose(y, y_ind, atol=1e-13)
    np.testing.assert_allclose(norms, np.linalg.norm(keys, axis=1), rtol=1e-14)
    got = oracle_mod.unpack_codes(codes, d, b)
    np.testing.assert_array_equal(got, idx)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), 1.0, rtol=1e-13)


@pytest.mark.parametrize("d,b", [(16, 2), (32, 3), (64, 4), (64, 1)])
def test_code_packing_is_lsb_first_bitstream(oracle_mod, d, b):
    rng = np.random.default_rng(7)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    keys = rng.standard_normal((50, d))
    lv, th = oracle_mod.codebook(d, b)
    codes, _, _, _ = oracle_mod.encode_keys(th, s, keys, b)
    idx, _ = _independent_codes(keys, s, lv, d)
    assert codes.shape == (50, d * b // 8)
    bits = np.unpackbits(codes, axis=1, bitorder="little").reshape(50, d, b)
    rebuilt = (bits * (1 << np.arange(b))).sum(axis=-1)
    np.testing.assert_array_equal(rebuilt, idx)


def test_code_packing_hand_example(oracle_mod):
    """d=16, b=4: a key equal to the sign-pattern-weighted first Hadamard row has y = e_0."""
    d, b = 16, 4
    s = np.array([1, -1] * 8, dtype=np.int8)
    Hs = scipy.linalg.hadamard(d) / math.sqrt(d)
    k = s * Hs[0] * 3.0  # H D k / |k| = e_0
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, y, _ = oracle_mod.encode_keys(th, s, k[None, :], b)
    assert norms[0] == pytest.approx(3.0)
    np.testing.assert_allclose(y[0], np.eye(d)[0], atol=1e-15)
    # y_0 = 1 > every threshold -> code 15; every other y_i = 0 -> code 8 (the middle threshold is 0)
    expected = np.array([0x8F] + [0x88] * 7, dtype=np.uint8)
    np.testing.assert_array_equal(codes[0], expected)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_encode_negated_key_mirrors_codes(oracle_mod, b):
    d = 64
    rng = np.random.default_rng(b)
    s = W.signs(W.LONGCTX)
    keys = rng.standard_normal((200, d))
    lv, th = oracle_mod.codebook(d, b)
    cp, npos, _, tie = oracle_mod.encode_keys(th, s, keys, b)
    cn, nneg, _, _ = oracle_mod.encode_keys(th, s, -keys, b)
    ip = oracle_mod.unpack_codes(cp, d, b)
    ineg = oracle_mod.unpack_codes(cn, d, b)
    L = 1 << b
    ok = ~tie
    np.testing.assert_array_equal(ineg[ok], (L - 1 - ip)[ok])
    np.testing.assert_array_equal(npos, nneg)


def test_encode_zero_key(oracle_mod):
    d, b = 64, 4
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, y, _ = oracle_mod.encode_keys(th, W.signs(W.LONGCTX), np.zeros((2, d)), b)
    assert np.all(norms == 0)
    assert np.all(oracle_mod.unpack_codes(codes, d, b) == 8)


def test_encode_non_finite_keys(oracle_mod):
    """Reading for keys the pages leave undefined: an infinite or NaN element leaves no unit vector, so the
    key gets the zero key's codes (L/2 everywhere: the middle threshold of the symmetric codebook is 0 and a
    value on a threshold takes the upper code) and its norm as its sum of squares gives it."""
    d = 64
    for b in (1, 2, 3, 4):
        lv, th = oracle_mod.codebook(d, b)
        keys = np.random.default_rng(b).standard_normal((5, d))
        keys[0, 3] = np.inf
        keys[1, 7] = -np.inf
        keys[2, 0] = np.nan
        keys[3, 1], keys[3, 2] = np.inf, np.nan
        keys[4, :] = 0.0
        codes, norms, _, _ = oracle_mod.encode_keys(th, W.signs(W.LONGCTX), keys, b)
        idx = oracle_mod.unpack_codes(codes, d, b)
        assert np.all(idx == (1 << b) // 2), b
        assert norms[0] == np.inf and norms[1] == np.inf
        assert np.isnan(norms[2]) and np.isnan(norms[3])
        assert norms[4] == 0.0


@pytest.mark.parametrize("scale_exp", [-140, -100, 100, 120])
def test_encode_codes_are_scale_invariant_at_extreme_scales(oracle_mod, scale_exp):
    """y = H D k / |k| does not depend on the key's scale: keys scaled by a power of two (exact in fp64) far
    outside fp32's comfortable range (elements near 1e-42 or 1e38, sums of squares far beyond fp32) keep
    the brute-force nearest-level codes of the unscaled keys, and their norms scale exactly."""
    d, b = 128, 4
    rng = np.random.default_rng(5)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    keys = rng.standard_normal((64, d))
    lv, th = oracle_mod.codebook(d, b)
    c0, n0, _, tie = oracle_mod.encode_keys(th, s, keys, b)
    c1, n1, _, _ = oracle_mod.encode_keys(th, s, np.ldexp(keys, scale_exp), b)
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(n1, np.ldexp(n0, scale_exp))
    idx, _ = _independent_codes(keys, s, lv, d)
    np.testing.assert_array_equal(oracle_mod.unpack_codes(c1, d, b)[~tie], idx[~tie])


def test_encode_tie_band_flags(oracle_mod):
    d, b = 16, 2
    s = np.ones(d, dtype=np.int8)
    Hs = scipy.linalg.hadamard(d) / math.sqrt(d)
    lv, th = oracle_mod.codebook(d, b)
    y = np.zeros(d)
    y[0] = th[2] + 5e-7  # inside the band
    y[1] = th[2] + 5e-6  # outside
    y[2] = math.sqrt(max(0.0, 1.0 - y[0] ** 2 - y[1] ** 2))
    k = Hs.T @ y  # H is symmetric and orthogonal, D = I
    _, _, yo, tie = oracle_mod.encode_keys(th, s, k[None, :], b)
    assert tie[0, 0] and not tie[0, 1]
    assert yo[0, 0] == pytest.approx(y[0], abs=1e-15)


# ----------------------------------------------------------------------------------------------
# Read path
# ----------------------------------------------------------------------------------------------

def _dequant_original_domain(codes, norms, signs, levels, d, b, oracle_mod):
    """k_hat = |k| D H^T c_hat: the inverse transform, computed independently (used only in tests)."""
    idx = oracle_mod.unpack_codes(codes, d, b)
    chat = np.asarray(levels)[idx]
    Hs = scipy.linalg.hadamard(d) / math.sqrt(d)
    return norms[..., None] * ((chat @ Hs) * signs)


@pytest.mark.parametrize("d,b", [(16, 2), (64, 4), (128, 3)])
def test_lut_scores_equal_bruteforce_dequant(oracle_mod, d, b):
    rng = np.random.default_rng(11 * d + b)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    B, Hq, Hkv, T = 2, 4, 2, 37
    q = rng.standard_normal((B, Hq, d))
    keys = rng.standard_normal((B, Hkv, T, d)) * 2.0
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, keys, b)
    sc = oracle_mod.scores(lv, s, q, codes, norms)
    # route 1: rotated domain, q' . c_hat (BJ-style brute force)
    idx = oracle_mod.unpack_codes(codes, d, b)
    Hs = scipy.linalg.hadamard(d) / math.sqrt(d)
    qrot = (q * s) @ Hs.T
    G = Hq // Hkv
    for h in range(Hq):
        chat = np.asarray(lv)[idx[:, h // G]]  # [B, T, d]
        ref = norms[:, h // G] * np.einsum("bd,btd->bt", qrot[:, h], chat)
        np.testing.assert_allclose(sc[:, h], ref, rtol=1e-12, atol=1e-12)
    # route 2: original domain, q . k_hat with the inverse transform
    khat = _dequant_original_domain(codes, norms, s, lv, d, b, oracle_mod)
    for h in range(Hq):
        ref = np.einsum("bd,btd->bt", q[:, h], khat[:, h // G])
        np.testing.assert_allclose(sc[:, h], ref, rtol=1e-11, atol=1e-11)


def test_lut_entries(oracle_mod):
    lv, _ = oracle_mod.codebook(16, 2)
    qr = np.arange(16, dtype=np.float64) - 7.5
    lut = oracle_mod.build_lut(lv, qr)
    assert lut.shape == (16, 4)
    np.testing.assert_array_equal(lut, np.multiply.outer(qr, lv))


def test_b1_score_closed_form(oracle_mod):
    d = 64
    rng = np.random.default_rng(3)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    q = rng.standard_normal((1, 1, d))
    keys = rng.standard_normal((1, 1, 20, d))
    lv, th = oracle_mod.codebook(d, 1)
    codes, norms, y, _ = oracle_mod.encode_keys(th, s, keys, 1)
    sc = oracle_mod.scores(lv, s, q, codes, norms)
    qr = oracle_mod.rotate_query(s, q[0, 0])
    sgn = np.where(y[0, 0] >= 0, 1.0, -1.0)
    ref = norms[0, 0] * math.sqrt(2 / math.pi) / math.sqrt(d) * (sgn @ qr)
    np.testing.assert_allclose(sc[0, 0], ref, rtol=1e-12)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_score_error_matches_quantizer_distortion(oracle_mod, b):
    """E[(s - q.k)^2] ~= |q|^2 |k|^2 MSE_b / d: pins the codebook scale and the norm factor."""
    d = 64
    rng = np.random.default_rng(20 + b)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    T = 4000
    q = rng.standard_normal((1, 1, d))
    keys = rng.standard_normal((1, 1, T, d)) * rng.lognormal(0, 0.5, size=(1, 1, T, 1))
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, keys, b)
    sc = oracle_mod.scores(lv, s, q, codes, norms)[0, 0]
    exact = keys[0, 0] @ q[0, 0]
    c, t, _ = oracle_mod.lloyd_max_unit(b)
    mse = oracle_mod.quantizer_mse_unit(b, c, t)
    pred = np.mean(norms[0, 0] ** 2) * np.sum(q ** 2) * mse / d
    assert np.mean((sc - exact) ** 2) == pytest.approx(pred, rel=0.25)


def test_softmax_rows_sum_to_one(oracle_mod):
    rng = np.random.default_rng(1)
    for n in (1, 7, 1000):
        p = oracle_mod.softmax_row(rng.standard_normal(n) * 30, 0.125)
        assert p.sum() == pytest.approx(1.0, abs=1e-12)
        assert np.all(p >= 0)


def _torch_sdpa(q, k, v, scale, G):
    import torch
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[:, :, None, :]  # [B, Hq, 1, d]
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64)).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[:, :, 0, :].numpy()


@pytest.mark.parametrize("d,b,G", [(16, 2, 1), (64, 4, 8), (128, 3, 4)])
def test_decode_attn_equals_sdpa_on_dequantized_keys(oracle_mod, d, b, G):
    rng = np.random.default_rng(d * b + G)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    B, Hkv, T = 2, 2, 50
    Hq = Hkv * G
    q = rng.standard_normal((B, Hq, d)) * 3
    keys = rng.standard_normal((B, Hkv, T, d)) * 2
    v = rng.standard_normal((B, Hkv, T, d))
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, keys, b)
    scale = 1.0 / math.sqrt(d)
    out = oracle_mod.decode_attn(lv, s, q, codes, norms, v, scale)
    khat = _dequant_original_domain(codes, norms, s, lv, d, b, oracle_mod)
    ref = _torch_sdpa(q, khat, v, scale, G)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_decode_attn_special_cases(oracle_mod):
    d, b = 64, 4
    rng = np.random.default_rng(9)
    s = W.signs(W.LONGCTX)
    B, Hkv, T = 1, 1, 40
    keys = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, keys, b)
    # zero query: uniform attention -> mean of V
    out = oracle_mod.decode_attn(lv, s, np.zeros((1, 1, d)), codes, norms, v, 0.125)
    np.testing.assert_allclose(out[0, 0], v[0, 0].mean(axis=0), atol=1e-14)
    # one key with a huge norm aligned with q dominates -> output = its value row
    norms2 = norms.copy()
    norms2[0, 0, 17] = 1e6
    q = oracle_mod_rotate_back(oracle_mod, s, lv, codes[0, 0, 17], d, b)
    out = oracle_mod.decode_attn(lv, s, q[None, None, :], codes, norms2, v, 1.0)
    np.testing.assert_allclose(out[0, 0], v[0, 0, 17], atol=1e-12)


def oracle_mod_rotate_back(oracle_mod, s, lv, code_row, d, b):
    """A query whose score against this code row is maximal: D H^T c_hat."""
    idx = oracle_mod.unpack_codes(code_row[None, :], d, b)[0]
    Hs = scipy.linalg.hadamard(d) / math.sqrt(d)
    return (np.asarray(lv)[idx] @ Hs) * s


def test_seq_lens_truncate_and_empty(oracle_mod):
    d, b = 16, 2
    rng = np.random.default_rng(4)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    B, Hq, Hkv, T = 3, 2, 1, 30
    q = rng.standard_normal((B, Hq, d))
    keys = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, keys, b)
    lens = np.array([30, 0, 11], dtype=np.int32)
    out = oracle_mod.decode_attn(lv, s, q, codes, norms, v, 0.25, seq_lens=lens)
    assert np.all(out[1] == 0)
    sub = oracle_mod.decode_attn(lv, s, q[2:3], codes[2:3, :, :11], norms[2:3, :, :11], v[2:3, :, :11], 0.25)
    np.testing.assert_allclose(out[2], sub[0], rtol=1e-14)
    full = oracle_mod.decode_attn(lv, s, q, codes, norms, v, 0.25)
    np.testing.assert_array_equal(out[0], full[0])
    sc = oracle_mod.scores(lv, s, q, codes, norms, seq_lens=lens)
    assert np.all(np.isneginf(sc[1])) and np.all(np.isneginf(sc[2, :, 11:])) and np.all(np.isfinite(sc[2, :, :11]))


# ----------------------------------------------------------------------------------------------
# Product quantization
# ----------------------------------------------------------------------------------------------

def test_kmeans_objective_never_increases(oracle_mod):
    rng = np.random.default_rng(0)
    train = rng.standard_normal((2000, 8))
    init = rng.permutation(2000)[:64]
    cent, obj = oracle_mod.kmeans(train, 64, 10, init)
    assert np.all(np.diff(obj) <= 1e-12)
    assert obj[-1] < obj[0]


def test_kmeans_all_points_as_centroids_is_exact(oracle_mod):
    rng = np.random.default_rng(1)
    train = rng.standard_normal((50, 4))
    cent, obj = oracle_mod.kmeans(train, 50, 3, np.arange(50))
    assert obj[-1] == 0.0
    np.testing.assert_array_equal(cent, train)


def test_kmeans_matches_sklearn_lloyd(oracle_mod):
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(2)
    train = rng.standard_normal((3000, 8))
    init_rows = rng.permutation(3000)[:32]
    iters = 10
    cent, _ = oracle_mod.kmeans(train, 32, iters, init_rows)
    km = KMeans(n_clusters=32, init=train[init_rows], n_init=1, max_iter=iters, tol=0.0,
                algorithm="lloyd").fit(train)
    # sklearn ends with the centroid update of its last iteration; so does the oracle
    np.testing.assert_allclose(cent, km.cluster_centers_, rtol=1e-9, atol=1e-9)


def test_kmeans_scalar_subspaces(oracle_mod):
    """m = d: one-dimensional k-means; the nearest-centroid cells are intervals between midpoints."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4000, 1))
    cent, _ = oracle_mod.kmeans(x, 8, 50, rng.permutation(4000)[:8])
    cs = np.sort(cent[:, 0])
    # at a converged 1-D k-means, each centroid is the mean of the points between its midpoints
    edges = np.concatenate([[-np.inf], 0.5 * (cs[1:] + cs[:-1]), [np.inf]])
    for j in range(8):
        sel = (x[:, 0] >= edges[j]) & (x[:, 0] < edges[j + 1])
        assert x[sel, 0].mean() == pytest.approx(cs[j], abs=2e-3)


def test_pq_encode_nearest_centroid(oracle_mod):
    rng = np.random.default_rng(8)
    d, m, K = 64, 8, 256
    cent = rng.standard_normal((m, K, d // m))
    keys = rng.standard_normal((100, d))
    codes, gap = oracle_mod.pq_encode(cent, keys)
    for s in range(m):
        sub = keys[:, s * 8:(s + 1) * 8]
        dist = ((sub[:, None, :] - cent[s][None, :, :]) ** 2).sum(-1)
        np.testing.assert_array_equal(codes[:, s], np.argmin(dist, axis=1))
        sd = np.sort(dist, axis=1)
        np.testing.assert_allclose(gap[:, s], sd[:, 1] - sd[:, 0], rtol=1e-9, atol=1e-12)


def test_pq_scores_and_attention_equal_dequantized(oracle_mod):
    rng = np.random.default_rng(10)
    d, m, K = 64, 8, 16
    B, H, T = 2, 3, 40
    cent = rng.standard_normal((H, m, K, d // m))
    q = rng.standard_normal((B, H, d))
    keys = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, d))
    codes = np.zeros((B, H, T, m), dtype=np.uint8)
    for h in range(H):
        codes[:, h] = oracle_mod.pq_encode(cent[h], keys[:, h])[0]
    sc = oracle_mod.pq_scores(cent, q, codes)
    khat = np.zeros((B, H, T, d))
    for h in range(H):
        for s in range(m):
            khat[:, h, :, s * 8:(s + 1) * 8] = cent[h, s][codes[:, h, :, s]]
    np.testing.assert_allclose(sc, np.einsum("bhd,bhtd->bht", q, khat), rtol=1e-12, atol=1e-12)
    out = oracle_mod.pq_decode_attn(cent, q, codes, v, 0.125)
    np.testing.assert_allclose(out, _torch_sdpa(q, khat, v, 0.125, 1), rtol=1e-10, atol=1e-12)


def test_pq_4bit_codes_pack_two_subspaces_per_byte(oracle_mod):
    """With K <= 16 centroids the code of subspace s sits in nibble s of the row (even subspaces low):
    byte j = idx[2j] | idx[2j+1] << 4 with idx the brute-force nearest centroids; scores and attention read
    the same indices as the one-byte layout."""
    rng = np.random.default_rng(12)
    d, m, K = 64, 4, 16
    B, H, T = 2, 2, 30
    cent = rng.standard_normal((H, m, K, d // m))
    keys = rng.standard_normal((B, H, T, d))
    q = rng.standard_normal((B, H, d))
    v = rng.standard_normal((B, H, T, d))
    c8 = np.zeros((B, H, T, m), dtype=np.uint8)
    c4 = np.zeros((B, H, T, m // 2), dtype=np.uint8)
    for h in range(H):
        c8[:, h] = oracle_mod.pq_encode(cent[h], keys[:, h])[0]
        c4[:, h] = oracle_mod.pq_encode(cent[h], keys[:, h], bits=4)[0]
    for s in range(m):
        sub = keys[..., s * 16:(s + 1) * 16]
        dist = ((sub[..., None, :] - cent[None, :, s, None, :, :]) ** 2).sum(-1)  # [B, H, T, K]
        np.testing.assert_array_equal(c8[..., s], np.argmin(dist, axis=-1))
    np.testing.assert_array_equal(c4, c8[..., 0::2] | (c8[..., 1::2] << 4))
    np.testing.assert_array_equal(oracle_mod.pq_scores(cent, q, c4, bits=4), oracle_mod.pq_scores(cent, q, c8))
    np.testing.assert_array_equal(oracle_mod.pq_decode_attn(cent, q, c4, v, 0.125, bits=4),
                                  oracle_mod.pq_decode_attn(cent, q, c8, v, 0.125))


# ----------------------------------------------------------------------------------------------
# Workload generators: seeded and reproducible per batch slice
# ----------------------------------------------------------------------------------------------

def test_workloads_are_deterministic_and_sliceable():
    sh = W.scaled(W.LONGCTX, B=3, T=100)
    a = W.keys(sh)
    b = W.keys(sh, batches=[2])
    np.testing.assert_array_equal(a[2], b[0])
    np.testing.assert_array_equal(W.values(sh), W.values(sh))
    s = W.signs(sh)
    assert set(np.unique(s)) <= {-1, 1}
    assert a.dtype == np.float16


# ------------------------------------------------------------------------------------------------
# Sign-pattern selection (AXELRAM key points / abstract: a one-time, gradient-free choice among
# candidate sign patterns on a few calibration samples; ranked here by attention-output error)
# ------------------------------------------------------------------------------------------------

def _signsel_case(seed, d=16, b=2, n=2, G=2, Hkv=2, T=40, C=6):
    rng = np.random.default_rng(seed)
    Hq = Hkv * G
    cands = (rng.integers(0, 2, (C, d)) * 2 - 1).astype(np.int8)
    chan = np.exp(rng.standard_normal((Hkv, d)))  # heterogeneous channel norms
    q = rng.standard_normal((n, Hq, d)) * 2
    keys = rng.standard_normal((n, Hkv, T, d)) * chan[None, :, None, :]
    v = rng.standard_normal((n, Hkv, T, d))
    return cands, q, keys, v, G


def test_exact_attn_equals_torch_sdpa(oracle_mod):
    cands, q, keys, v, G = _signsel_case(1, d=32, G=4)
    scale = 1.0 / math.sqrt(32)
    np.testing.assert_allclose(oracle_mod.exact_attn(q, keys, v, scale), _torch_sdpa(q, keys, v, scale, G),
                               rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("d,b", [(16, 2), (64, 4)])
def test_sign_errors_by_an_independent_route(oracle_mod, d, b):
    """Each candidate's error recomputed from the inverse-transform dequantization (scipy's Hadamard) and
    torch's attention on the dequantized and on the exact keys; the selection is the first minimum."""
    cands, q, keys, v, G = _signsel_case(7 * d + b, d=d, b=b)
    scale = 1.0 / math.sqrt(d)
    lv, th = oracle_mod.codebook(d, b)
    errors, best = oracle_mod.sign_errors(lv, th, cands, q, keys, v, scale)
    o = _torch_sdpa(q, keys, v, scale, G)
    for c in range(len(cands)):
        codes, norms, _, _ = oracle_mod.encode_keys(th, cands[c], keys, b)
        norms32 = norms.astype(np.float32).astype(np.float64)  # the cache stores fp32 norms
        khat = _dequant_original_domain(codes, norms32, cands[c], lv, d, b, oracle_mod)
        oh = _torch_sdpa(q, khat, v, scale, G)
        ref = np.sum((oh - o) ** 2) / np.sum(o ** 2)
        np.testing.assert_allclose(errors[c], ref, rtol=1e-9)
    assert best == int(np.argmin(errors))
    assert np.all(errors > 0) and np.all(errors < 1)


def test_sign_errors_unchanged_by_negating_the_pattern(oracle_mod):
    """-D mirrors every code and the symmetric codebook mirrors every level, so the dequantized keys, the
    scores and the error are exactly those of D; the tie goes to the lower index."""
    cands, q, keys, v, G = _signsel_case(3, d=64, b=3, C=3)
    cands = np.stack([cands[0], -cands[0], cands[1], -cands[1]])
    lv, th = oracle_mod.codebook(64, 3)
    errors, best = oracle_mod.sign_errors(lv, th, cands, q, keys, v, 0.125)
    assert errors[0] == errors[1] and errors[2] == errors[3]
    assert best in (0, 2)
    single, b1 = oracle_mod.sign_errors(lv, th, cands[1:2], q, keys, v, 0.125)
    assert b1 == 0 and single[0] == errors[1]


# ----------------------------------------------------------------------------------------------
# Values quantized with the key codec
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("d,b", [(16, 1), (64, 4), (128, 3), (256, 2)])
def test_dequant_equals_inverse_transform_by_scipy(oracle_mod, d, b):
    rng = np.random.default_rng(5 * d + b)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    v = rng.standard_normal((3, 11, d)) * rng.lognormal(0, 1, size=(3, 11, 1))
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, v, b)
    got = oracle_mod.dequant(lv, s, codes, norms)
    ref = _dequant_original_domain(codes, norms, s, lv, d, b, oracle_mod)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_dequant_distortion_matches_the_quantizer(oracle_mod, b):
    """E|v/|v| - v_hat/|v||^2 ~= MSE_b of the unit Lloyd-Max quantizer (d coordinates of variance 1/d),
    and the reconstruction is unbiased in direction: E<u, u_hat> ~= 1 - MSE_b (centroid condition)."""
    d = 128
    rng = np.random.default_rng(40 + b)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    v = rng.standard_normal((3000, d)) * 3.0
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, v, b)
    vh = oracle_mod.dequant(lv, s, codes, norms)
    u = v / norms[:, None]
    uh = vh / norms[:, None]
    c, t, _ = oracle_mod.lloyd_max_unit(b)
    mse = oracle_mod.quantizer_mse_unit(b, c, t)
    assert np.mean(np.sum((u - uh) ** 2, axis=1)) == pytest.approx(mse, rel=0.05)
    assert np.mean(np.sum(u * uh, axis=1)) == pytest.approx(1.0 - mse, rel=0.01)


@pytest.mark.parametrize("d,b,G", [(16, 2, 1), (64, 4, 8), (128, 3, 4)])
def test_decode_attn_qv_equals_sdpa_on_dequantized_keys_and_values(oracle_mod, d, b, G):
    rng = np.random.default_rng(7 * d + b + G)
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    B, Hkv, T = 2, 2, 45
    Hq = Hkv * G
    q = rng.standard_normal((B, Hq, d)) * 3
    keys = rng.standard_normal((B, Hkv, T, d)) * 2
    v = rng.standard_normal((B, Hkv, T, d)) * rng.lognormal(0, 1, size=(1, Hkv, 1, d))
    lv, th = oracle_mod.codebook(d, b)
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, keys, b)
    vcodes, vnorms, _, _ = oracle_mod.encode_keys(th, s, v, b)
    scale = 1.0 / math.sqrt(d)
    lens = [T, 17]
    out = oracle_mod.decode_attn_qv(lv, s, q, codes, norms, vcodes, vnorms, scale, seq_lens=lens)
    khat = _dequant_original_domain(codes, norms, s, lv, d, b, oracle_mod)
    vhat = _dequant_original_domain(vcodes, vnorms, s, lv, d, b, oracle_mod)
    for bi, n in enumerate(lens):
        ref = _torch_sdpa(q[bi:bi + 1], khat[bi:bi + 1, :, :n], vhat[bi:bi + 1, :, :n], scale, G)
        np.testing.assert_allclose(out[bi:bi + 1], ref, rtol=1e-10, atol=1e-12)


def test_decode_attn_qv_special_cases(oracle_mod):
    """One value row repeated at every position: the output is that row's reconstruction whatever the
    scores; an empty sequence gives zeros; a zero value row reconstructs to zero."""
    d, b = 64, 4
    rng = np.random.default_rng(12)
    s = W.signs(W.LONGCTX)
    lv, th = oracle_mod.codebook(d, b)
    T = 30
    q = rng.standard_normal((2, 2, d)) * 5
    keys = rng.standard_normal((2, 1, T, d)) * 3
    row = rng.standard_normal(d) * 2
    v = np.broadcast_to(row, (2, 1, T, d)).copy()
    v[1] = 0.0
    codes, norms, _, _ = oracle_mod.encode_keys(th, s, keys, b)
    vcodes, vnorms, _, _ = oracle_mod.encode_keys(th, s, v, b)
    out = oracle_mod.decode_attn_qv(lv, s, q, codes, norms, vcodes, vnorms, 0.125, seq_lens=[T, T])
    rc, rn, _, _ = oracle_mod.encode_keys(th, s, row[None, :], b)
    rhat = oracle_mod.dequant(lv, s, rc, rn)[0]
    np.testing.assert_allclose(out[0], np.broadcast_to(rhat, (2, d)), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(out[1], 0.0)
    out0 = oracle_mod.decode_attn_qv(lv, s, q, codes, norms, vcodes, vnorms, 0.125, seq_lens=[0, 5])
    np.testing.assert_array_equal(out0[0], 0.0)


# ---------------------------------------------------------------------------------------------------------
# Power-of-two key codec (shift-accumulate attention page, English abstract)
# ---------------------------------------------------------------------------------------------------------

POT_CASES = [(b, m) for b in (2, 3, 4) for m in (0, 1)]


@pytest.mark.parametrize("b,mant", POT_CASES)
def test_pot_magnitudes_are_powers_of_two_or_one_extra_term(oracle_mod, b, mant):
    """Every magnitude is 2^-r (plain code) or, with the mantissa term, 2^-r or 2^-r + 2^-(r+1); the set
    descends from 1, so alpha = max|k| leaves every shift non-negative; midpoints sit between neighbours."""
    mags, thr = oracle_mod.pot_levels(b, mant)
    assert len(mags) == 1 << (b - 1) and mags[0] == 1.0
    assert np.all(np.diff(mags) < 0)
    for x in mags:
        r = -math.floor(math.log2(x))
        rest = x - 2.0 ** -r
        assert rest == 0.0 or (mant == 1 and rest == 2.0 ** -(r + 1)), x
    np.testing.assert_array_equal(thr, (mags[:-1] + mags[1:]) / 2)


def test_pot_hand_packed_example(oracle_mod):
    """A key worked by hand (plain 4-bit code: sign in bit 3, index j in bits 0..2, magnitude 2^-j, scale 4):
    x = |k|/4 = 1, .5, .25, .15, .1, 0, .8, .7, .75 (a midpoint: the larger magnitude), .375 (a midpoint),
    .0125, .0025, .0625, .03125, .015625, 1 -> j = 0,1,2,3,3,7,0,1,0,1,6,7,4,5,6,0 with the signs of k;
    codes 0,9,2,3,11,7,0,9,0,1,14,7,4,13,6,8 packed two per byte, low nibble first."""
    k = np.array([4.0, -2.0, 1.0, 0.6, -0.4, 0.0, 3.2, -2.8, 3.0, 1.5, -0.05, 0.01, 0.25, -0.125, 0.0625, -4.0])
    codes, scales, tie = oracle_mod.pot_encode(k[None, :], 4, 0)
    assert scales[0] == 4.0
    assert list(codes[0]) == [0x90, 0x32, 0x7B, 0x90, 0x10, 0x7E, 0xD4, 0x86]
    assert tie[0, 8] and tie[0, 9] and tie.sum() == 2
    khat = 4.0 * np.array([1, -.5, .25, .125, -.125, 2 ** -7, 1, -.5, 1, .5, -2 ** -6, 2 ** -7, 2 ** -4, -2 ** -5,
                           2 ** -6, -1])
    np.testing.assert_array_equal(oracle_mod.pot_dequant(codes, scales, 16, 4, 0)[0], khat)
    s = oracle_mod.pot_scores(np.ones((1, 1, 16)), codes[None, None], scales[None, None], 4, 0)
    assert s[0, 0, 0] == 7.1875 == khat.sum()
    # the same key with the mantissa term: magnitudes 1, 3/4, 1/2, 3/8, 1/4, 3/16, 1/8, 3/32
    c1, _, _ = oracle_mod.pot_encode(k[None, :], 4, 1)
    j1 = oracle_mod.unpack_codes(c1, 16, 4)[0]
    # x = .8, .7 and .75 now take 3/4 (j = 1); .15 takes 1/8 (j = 6: |.15 - .125| < |.15 - .1875|); .1 and
    # everything smaller take 3/32 (j = 7), the smallest magnitude
    assert list(j1 & 7) == [0, 2, 4, 6, 7, 7, 1, 1, 1, 3, 7, 7, 7, 7, 7, 0]
    assert list(j1 >> 3) == [0, 1, 0, 0, 1, 0, 0, 1, 0, 0, 1, 0, 0, 1, 0, 1]


@pytest.mark.parametrize("b,mant", POT_CASES)
def test_pot_encode_is_the_nearest_magnitude(oracle_mod, b, mant):
    """Brute force: the decoded index is argmin_j | |k_i|/alpha - mag_j | (ties to the larger magnitude),
    the sign bit is k_i < 0, alpha = max |k_i|."""
    rng = np.random.default_rng(100 + 10 * b + mant)
    k = rng.standard_normal((300, 32)) * np.exp(rng.standard_normal((300, 1)))
    k = k.astype(np.float16).astype(np.float64)
    codes, scales, tie = oracle_mod.pot_encode(k, b, mant)
    np.testing.assert_array_equal(scales, np.abs(k).max(axis=1))
    mags, _ = oracle_mod.pot_levels(b, mant)
    idx = oracle_mod.unpack_codes(codes, 32, b)
    j, sgn = idx & ((1 << (b - 1)) - 1), idx >> (b - 1)
    x = np.abs(k) / scales[:, None]
    ref = np.argmin(np.abs(x[..., None] - mags), axis=-1)
    np.testing.assert_array_equal(j[~tie], ref[~tie])
    np.testing.assert_array_equal(sgn, (k < 0).astype(sgn.dtype))


@pytest.mark.parametrize("b,mant,bound", [(4, 0, 1 / 3), (4, 1, 1 / 5), (3, 0, 1 / 3), (3, 1, 1 / 5)])
def test_pot_relative_error_closed_form(oracle_mod, b, mant, bound):
    """Nearest power of two in value is off by at most 1/3 of the element (at 3/4 of an octave), and the
    mantissa term brings that to 1/5 (at 5/8); both bounds are reached, at every scale in range."""
    mags, _ = oracle_mod.pot_levels(b, mant)
    x = np.geomspace(mags[-1], 1.0, 40001)
    key = np.concatenate([[1.0], x])  # alpha = 1
    rows = key[: (len(key) // 16) * 16].reshape(-1, 16)
    rows[:, 0] = 1.0
    codes, scales, _ = oracle_mod.pot_encode(rows, b, mant)
    khat = oracle_mod.pot_dequant(codes, scales, 16, b, mant)
    rel = np.abs(khat - rows) / rows
    assert rel.max() <= bound + 1e-12
    assert rel.max() >= bound - 1e-3


def test_pot_scale_invariance_and_sign_mirror(oracle_mod):
    rng = np.random.default_rng(7)
    k = rng.standard_normal((50, 64))
    k[3, :5] = 0.0
    c0, s0, _ = oracle_mod.pot_encode(k, 4, 1)
    for e in (-3, 1, 5):
        c, s, _ = oracle_mod.pot_encode(k * 2.0 ** e, 4, 1)
        np.testing.assert_array_equal(c, c0)
        np.testing.assert_array_equal(s, s0 * 2.0 ** e)
    cn, sn, _ = oracle_mod.pot_encode(-k, 4, 1)
    np.testing.assert_array_equal(sn, s0)
    i0, i1 = oracle_mod.unpack_codes(c0, 64, 4), oracle_mod.unpack_codes(cn, 64, 4)
    np.testing.assert_array_equal(i1 & 7, i0 & 7)
    np.testing.assert_array_equal(i1 >> 3, np.where(k != 0, 1 - (i0 >> 3), 0))


def test_pot_zero_key(oracle_mod):
    k = np.zeros((1, 1, 1, 16))
    codes, scales, _ = oracle_mod.pot_encode(k, 4, 0)
    assert scales.item() == 0.0 and not codes.any()
    s = oracle_mod.pot_scores(np.ones((1, 1, 16)), codes, scales, 4, 0)
    assert s.item() == 0.0


@pytest.mark.parametrize("d,b,mant,G", [(16, 2, 0, 1), (64, 4, 0, 8), (64, 4, 1, 4), (128, 3, 1, 2)])
def test_pot_scores_and_attention_equal_dequantized(oracle_mod, d, b, mant, G):
    """Shift-and-add scores equal q . k_hat (a matrix product on the dequantized keys, GQA by repetition),
    and the attention equals torch SDPA on the dequantized keys."""
    rng = np.random.default_rng(d + b + mant + G)
    B, Hkv, T = 2, 2, 37
    Hq = Hkv * G
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d)) * np.exp(0.5 * rng.standard_normal((B, Hkv, T, 1)))
    v = rng.standard_normal((B, Hkv, T, d))
    codes, scales, _ = oracle_mod.pot_encode(k, b, mant)
    khat = oracle_mod.pot_dequant(codes, scales, d, b, mant)
    s = oracle_mod.pot_scores(q, codes, scales, b, mant)
    ref = np.matmul(q[:, :, None, :], np.repeat(khat, G, axis=1).transpose(0, 1, 3, 2))[:, :, 0, :]
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)
    scale = 1.0 / math.sqrt(d)
    out = oracle_mod.pot_decode_attn(q, codes, scales, v, b, mant, scale)
    np.testing.assert_allclose(out, _torch_sdpa(q, khat, v, scale, G), rtol=1e-10, atol=1e-12)
    lens = [T, 5]
    s2 = oracle_mod.pot_scores(q, codes, scales, b, mant, seq_lens=lens)
    assert np.all(np.isneginf(s2[1, :, 5:])) and np.array_equal(s2[1, :, :5], s[1, :, :5])


def test_pot_iso_bit_accuracy_on_long_context_keys(oracle_mod):
    """At 4 bits per element on the long-context keys (Gaussian within a key, LogNormal(0, 0.5) key scales),
    the mantissa term cuts the RMS score error well below the plain power-of-two code (the page reports
    about half), and the rotated Lloyd-Max code is more accurate than both."""
    sh = W.LONGCTX
    q = W.queries(sh)[[0]].astype(np.float64)
    k = W.keys(sh, batches=[0], T=512).astype(np.float64)
    s_ex = np.einsum("bhd,bhtd->bht", q, np.repeat(k, sh.Hq // sh.Hkv, axis=1))

    def rms(s):
        return math.sqrt(((s - s_ex) ** 2).mean() / (s_ex ** 2).mean())

    e = {}
    for m in (0, 1):
        c, a, _ = oracle_mod.pot_encode(k, 4, m)
        e[m] = rms(oracle_mod.pot_scores(q, c, a, 4, m))
    lv, th = oracle_mod.codebook(sh.d, 4)
    sg = W.signs(sh)
    c, n, _, _ = oracle_mod.encode_keys(th, sg, k, 4)
    e_h = rms(oracle_mod.scores(lv, sg, q, c, n))
    print("score rel RMS error: plain %.4f, mantissa %.4f, Hadamard/Lloyd-Max %.4f" % (e[0], e[1], e_h))
    assert e[1] < 0.75 * e[0]
    assert e_h < e[1]
