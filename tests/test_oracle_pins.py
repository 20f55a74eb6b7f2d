"""Pins of the CPU oracle against facts the pages and the mathematics fix.

None of these re-types an oracle formula: each compares the oracle with an
independent construction (Sylvester recursion, numerical quadrature, published
tables, brute-force search, hand-derived bit patterns, closed forms of tiny
attention problems, the pages' own data-driven Lloyd algorithm).
"""

import math

import numpy as np
import pytest
from scipy import integrate

import oracle as O
from tests.conftest import read_golden

SIGMA = 1.0 / math.sqrt(128)


# ----------------------------------------------------------------- Hadamard / rotation

def test_hadamard_orthogonal_exact():
    h = O.hadamard_matrix(128)
    assert np.array_equal(h @ h.T, 128.0 * np.eye(128))


def test_hadamard_equals_sylvester_recursion():
    h = np.array([[1.0]])
    while h.shape[0] < 128:
        h = np.block([[h, h], [h, -h]])
    assert np.array_equal(O.hadamard_matrix(128), h)


def test_hadamard_special_vectors():
    h = O.hadamard_matrix(128)
    ones = np.ones(128)
    e0 = np.zeros(128); e0[0] = 1
    assert np.array_equal(h @ e0, ones)
    assert np.array_equal(h @ ones, 128 * e0)


def test_sign_vector_bit_order():
    s = O.sign_vector([1, 0, 0, 0x80000000])
    assert s[0] == -1 and s[127] == -1
    assert np.all(s[1:127] == 1)
    s = O.sign_vector([0, 0x10, 0, 0])
    assert s[36] == -1 and np.sum(s == -1) == 1


def test_rotation_applies_signs_before_hadamard():
    """rotate(e_k) must be s_k * H[:, k] / sqrt(d) (D first, then H)."""
    words = np.array([0x80000001, 0x1234, 0, 0xFFFFFFFF], np.uint32)
    s = O.sign_vector(words)
    h = O.hadamard_matrix()
    for k in (0, 1, 5, 31, 44, 127):
        e = np.zeros(128); e[k] = 1
        np.testing.assert_allclose(O.rotate(e[None], s)[0], s[k] * h[:, k] / math.sqrt(128), atol=1e-15)


def test_rotation_norm_and_inverse():
    rng = np.random.default_rng(1)
    u = rng.standard_normal((64, 128))
    s = O.sign_vector(rng.integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32))
    y = O.rotate(u, s)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(u, axis=1), rtol=1e-13)
    np.testing.assert_allclose(O.unrotate(y, s), u, atol=1e-12)


def test_rotation_flattens_a_spike():
    """A single-coordinate outlier spreads to magnitude 1/sqrt(d) on every coordinate."""
    s = O.sign_vector([0xDEADBEEF, 0, 7, 9])
    e = np.zeros(128); e[17] = 1
    np.testing.assert_allclose(np.abs(O.rotate(e[None], s)[0]), np.full(128, 1 / math.sqrt(128)), rtol=1e-14)


# ----------------------------------------------------------------- Lloyd-Max codebook

def test_one_bit_closed_form():
    c = O.gaussian_lloyd_max(2, SIGMA)
    np.testing.assert_allclose(c, [-SIGMA * math.sqrt(2 / math.pi), SIGMA * math.sqrt(2 / math.pi)], rtol=1e-13)
    # distortion of the sign quantizer: sigma^2 (1 - 2/pi)
    assert abs(O.codebook_mse(c, np.array([0.0]), SIGMA) - SIGMA ** 2 * (1 - 2 / math.pi)) < 1e-15


@pytest.mark.parametrize("row", read_golden("lloyd_max_gaussian.txt"), ids=lambda r: r[0])
def test_published_gaussian_table(row):
    levels = int(row[0])
    outs = [float(v) for v in row[1].split()]
    bnds = [float(v) for v in row[2].split()] if row[2] else []
    mse = float(row[3]) if row[3] else None
    c = O.gaussian_lloyd_max(levels, 1.0)
    pos = c[levels // 2:]
    # the 1960 table is printed to four significant digits; allow 1.5 units of
    # the last printed digit (rounding plus a possible last-digit slip)
    for got, want in zip(pos, outs):
        assert abs(got - want) <= 1.5 * 10 ** (math.floor(math.log10(want)) - 3), (got, want)
    b = 0.5 * (c[:-1] + c[1:])
    for got, want in zip(b[levels // 2:], bnds):
        assert abs(got - want) <= 1.5 * 10 ** (math.floor(math.log10(want)) - 3), (got, want)
    if mse is None:
        return
    got_mse = O.codebook_mse(c, b, 1.0)
    assert abs(got_mse - mse) <= 1.5 * 10 ** (math.floor(math.log10(mse)) - 3), (got_mse, mse)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_centroid_condition_by_quadrature(bits):
    """Each centre is the conditional mean of its cell, by numerical integration."""
    c = O.gaussian_lloyd_max(1 << bits, 1.0)
    b = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    for j in range(len(c)):
        lo, hi = max(b[j], -12.0), min(b[j + 1], 12.0)
        m0 = integrate.quad(pdf, lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
        m1 = integrate.quad(lambda x: x * pdf(x), lo, hi, epsabs=0, epsrel=1e-13, limit=200)[0]
        assert abs(m1 / m0 - c[j]) < 1e-9


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_by_quadrature(bits):
    cb = O.build_codebook(bits)
    b = np.concatenate(([-np.inf], cb.boundaries, [np.inf]))
    pdf = lambda x: math.exp(-0.5 * (x / SIGMA) ** 2) / (SIGMA * math.sqrt(2 * math.pi))
    tot = 0.0
    for j in range(cb.n_levels):
        lo, hi = max(b[j], -12 * SIGMA), min(b[j + 1], 12 * SIGMA)
        cj = cb.centroids[j]
        tot += integrate.quad(lambda x: (x - cj) ** 2 * pdf(x), lo, hi, epsabs=0, epsrel=1e-12, limit=200)[0]
    assert abs(tot - cb.mse) < 1e-10 * SIGMA ** 2 + 1e-9 * cb.mse


@pytest.mark.parametrize("bits", [2, 3])
def test_data_driven_lloyd_matches_density_form(bits):
    """The pages' assign/mean/repeat loop on Gaussian samples lands on the analytic centres."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(400_000) * SIGMA
    c_data = O.lloyd_max_from_samples(x, 1 << bits)
    c_ana = O.gaussian_lloyd_max(1 << bits, SIGMA)
    assert np.max(np.abs(c_data - c_ana)) < 0.01 * SIGMA


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_stored_codebook_format(bits):
    cb = O.build_codebook(bits)
    c = cb.centroids
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])
    assert np.array_equal(c.astype(np.float16).astype(np.float64), c)            # float16-exact
    assert np.array_equal(cb.boundaries.astype(np.float32).astype(np.float64), cb.boundaries)  # float32-exact
    assert np.array_equal(cb.boundaries, (c[:-1] + c[1:]) / 2)
    # rounding to float16 moves a centre by at most half a float16 ulp
    ulp = np.spacing(np.abs(cb.centroids_f64).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(c - cb.centroids_f64) <= 0.5 * ulp)


# ----------------------------------------------------------------- encode / pack

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encode_is_nearest_centroid(bits):
    cb = O.build_codebook(bits)
    rng = np.random.default_rng(bits)
    y = rng.standard_normal(200_000) * SIGMA * 1.5
    got = O.encode(y, cb.boundaries)
    brute = np.argmin(np.abs(y[:, None] - cb.centroids[None, :]), axis=1)
    far = ~O.near_boundary_mask(y, cb.boundaries, 1e-12)
    assert np.array_equal(got[far], brute[far])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encode_ties_and_extremes(bits):
    cb = O.build_codebook(bits)
    L = cb.n_levels
    b = cb.boundaries
    assert list(O.encode(b, b)) == list(range(L - 1))                      # tie -> lower code
    assert list(O.encode(np.nextafter(b, np.inf), b)) == list(range(1, L))
    assert O.encode(np.array([0.0]), b)[0] == L // 2 - 1
    assert O.encode(np.array([-1.0, 1.0]), b).tolist() == [0, L - 1]


def test_zero_vector_quantizes_to_middle_code():
    cb = O.build_codebook(3)
    n, codes, y = O.quantize_vectors(np.zeros((1, 128), np.float16), np.ones(128), cb)
    assert n[0] == 0 and np.all(y == 0) and np.all(codes == 3)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_non_finite_vector_stored_as_zero_direction(bits):
    """R14: an inf or NaN element leaves no direction: the codes are the zero
    vector's (the middle code 2^(b-1) - 1, where y = 0 falls), the norm is inf, or
    NaN when an element is NaN; finite rows in the same call are unaffected."""
    cb = O.build_codebook(bits)
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((5, 128)).astype(np.float16)
    x[0, 7] = np.inf
    x[1, 100] = -np.inf
    x[2, 3] = np.nan
    x[3, :] = np.inf
    s = O.sign_vector(rng.integers(0, 2**32, size=4, dtype=np.uint64).astype(np.uint32))
    n, codes, y = O.quantize_vectors(x, s, cb)
    mid = (1 << (bits - 1)) - 1
    assert np.all(codes[:4] == mid) and np.all(y[:4] == 0)
    assert np.isposinf(n[0]) and np.isposinf(n[1]) and np.isnan(n[2]) and np.isposinf(n[3])
    n4, c4, _ = O.quantize_vectors(x[4:], s, cb)
    assert np.array_equal(codes[4:], c4) and n[4] == n4[0] and np.isfinite(n[4])
    # the zero vector takes the same codes (R3, R5)
    _, cz, _ = O.quantize_vectors(np.zeros((1, 128), np.float16), s, cb)
    assert np.array_equal(cz[0], codes[0])


@pytest.mark.parametrize("row", read_golden("pack_patterns.txt"), ids=lambda r: r[0] + ":" + r[1])
def test_pack_hand_patterns(row):
    bits = int(row[0])
    prefix = [int(v) for v in row[1].split()]
    want = bytes(int(v, 16) for v in row[2].split())
    codes = np.array((prefix * (128 // len(prefix) + 1))[:128], np.uint8)
    packed = O.pack_codes(codes, bits)
    assert packed.shape == (16 * bits,)
    assert bytes(packed[: len(want)]) == want
    assert np.array_equal(O.unpack_codes(packed, bits), codes)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_roundtrip_random(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(50, 128)).astype(np.uint8)
    assert np.array_equal(O.unpack_codes(O.pack_codes(codes, bits), bits), codes)


@pytest.mark.parametrize("row", read_golden("bits_per_value.txt"), ids=lambda r: r[0])
def test_bits_per_value_matches_pages(row):
    bits, bpv, ratio = int(row[0]), float(row[1]), float(row[2])
    assert O.bits_per_value(bits) == bpv
    assert (16 * bits + 4) * 8 / 128 == bpv       # bytes stored per 128-block
    assert round(16 / bpv, 1) == ratio


# ----------------------------------------------------------------- dequantize

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequantize_error_matches_codebook_mse(bits):
    """Relative error of Gaussian vectors ~ MSE_b / sigma^2 (rotated coordinates ~ N(0, 1/128))."""
    cb = O.build_codebook(bits)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4000, 128)).astype(np.float16)
    s = O.sign_vector([0x0F0F0F0F, 0x33333333, 0x55555555, 0x00FF00FF])
    n, codes, _ = O.quantize_vectors(x, s, cb)
    xh = O.dequantize_vectors(n, codes, s, cb)
    xf = x.astype(np.float64)
    rel = np.sum((xf - xh) ** 2) / np.sum(xf ** 2)
    want = cb.mse / SIGMA ** 2
    assert 0.9 * want < rel < 1.05 * want, (rel, want)


def test_dequantize_recovers_sign_and_scale():
    """Scaling the input scales the output; flipping it flips the output (antisymmetric codebook)."""
    cb = O.build_codebook(4)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 128)).astype(np.float16)
    s = O.sign_vector([1, 2, 3, 4])
    n, c, _ = O.quantize_vectors(x, s, cb)
    n2, c2, _ = O.quantize_vectors((-x) * np.float16(4), s, cb)
    far = ~O.near_boundary_mask(O.rotate(x.astype(np.float64) / np.linalg.norm(x.astype(np.float64), axis=1)[:, None], s), cb.boundaries)
    assert np.array_equal(c2[far], (cb.n_levels - 1 - c)[far])
    np.testing.assert_allclose(n2, 4 * n, rtol=1e-7)


# ----------------------------------------------------------------- attention

def _cache_from(xs, bits, signs, block_size=4, shuffle=None):
    """Quantize xs [T, H, 128] into an oracle cache with the given page order."""
    T, H, _ = xs.shape
    nb = -(-T // block_size)
    order = np.arange(nb) if shuffle is None else shuffle
    cb = O.build_codebook(bits)
    c = O.new_cache(bits, H, block_size, nb, signs, cb)
    t = np.arange(T)
    slots = order[t // block_size] * block_size + t % block_size
    O.cache_write(c, xs, slots)
    return c, order


def test_score_in_rotated_domain_equals_plain_dot():
    """[llama-tq]: Q.K can be computed against K codes in the Hadamard domain."""
    cb = O.build_codebook(4)
    rng = np.random.default_rng(5)
    s = O.sign_vector([9, 8, 7, 6])
    k = rng.standard_normal((32, 128)).astype(np.float16)
    q = rng.standard_normal(128)
    n, codes, _ = O.quantize_vectors(k, s, cb)
    plain = O.dequantize_vectors(n, codes, s, cb) @ q
    rotated = n.astype(np.float64) * (cb.centroids[codes] @ O.rotate(q[None], s)[0])
    np.testing.assert_allclose(rotated, plain, rtol=1e-12, atol=1e-12)


def test_attention_single_token_returns_value():
    rng = np.random.default_rng(2)
    xs = rng.standard_normal((1, 1, 128)).astype(np.float16)
    kc, _ = _cache_from(xs, 4, [[1, 2, 3, 4]])
    vc, _ = _cache_from(xs[::-1] * np.float16(2), 3, [[5, 6, 7, 8]])
    q = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    out = O.decode_attention(q, kc, vc, [1], np.array([[0]]), 1)
    np.testing.assert_allclose(out[0, 0, 0], O.cache_read(vc, np.array([0]), 0)[0], rtol=1e-14)


def test_attention_two_tokens_closed_form():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((2, 1, 128)).astype(np.float16)
    v = rng.standard_normal((2, 1, 128)).astype(np.float16)
    kc, _ = _cache_from(k, 4, [[3, 1, 4, 1]])
    vc, _ = _cache_from(v, 4, [[5, 9, 2, 6]])
    q = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    kh = O.cache_read(kc, np.array([0, 1]), 0)
    vh = O.cache_read(vc, np.array([0, 1]), 0)
    qq = q[0, 0, 0].astype(np.float64)
    s0, s1 = kh @ qq / math.sqrt(128)
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    want = p0 * vh[0] + (1 - p0) * vh[1]
    out = O.decode_attention(q, kc, vc, [2], np.array([[0]]), 1)          # scale 0 -> 1/sqrt(128)
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=1e-12, atol=1e-14)
    out2 = O.decode_attention(q, kc, vc, [2], np.array([[0]]), 1, scale=0.5)
    s0, s1 = kh @ qq * 0.5
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(out2[0, 0, 0], p0 * vh[0] + (1 - p0) * vh[1], rtol=1e-12, atol=1e-14)


def test_attention_uniform_cases_give_mean_value():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((7, 1, 128)).astype(np.float16)
    kc, _ = _cache_from(np.repeat(rng.standard_normal((1, 1, 128)), 7, 0).astype(np.float16), 4, [[1, 1, 1, 1]])
    vc, _ = _cache_from(v, 3, [[2, 2, 2, 2]])
    vh = O.cache_read(vc, np.arange(7), 0)
    q = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    out = O.decode_attention(q, kc, vc, [7], np.array([[0, 1]]), 1)
    np.testing.assert_allclose(out[0, 0, 0], vh.mean(0), rtol=1e-12, atol=1e-14)
    kc2, _ = _cache_from(rng.standard_normal((7, 1, 128)).astype(np.float16), 4, [[1, 1, 1, 1]])
    out0 = O.decode_attention(np.zeros_like(q), kc2, vc, [7], np.array([[0, 1]]), 1)
    np.testing.assert_allclose(out0[0, 0, 0], vh.mean(0), rtol=1e-12, atol=1e-14)


def test_attention_weights_by_pairwise_form():
    """Brute force: p_t = 1 / sum_u exp(s_u - s_t), a different route to the softmax."""
    rng = np.random.default_rng(8)
    T = 13
    k = rng.standard_normal((T, 1, 128)).astype(np.float16)
    v = rng.standard_normal((T, 1, 128)).astype(np.float16)
    kc, order = _cache_from(k, 3, [[11, 22, 33, 44]], block_size=4, shuffle=np.array([2, 0, 3, 1]))
    vc, _ = _cache_from(v, 2, [[55, 66, 77, 88]], block_size=4, shuffle=np.array([2, 0, 3, 1]))
    q = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    slots = O.slots_for_sequence(order, 4, T)
    kh, vh = O.cache_read(kc, slots, 0), O.cache_read(vc, slots, 0)
    s = kh @ q[0, 0, 0].astype(np.float64) / math.sqrt(128)
    p = np.array([1.0 / sum(math.exp(su - st) for su in s) for st in s])
    out = O.decode_attention(q, kc, vc, [T], order[None], 1)
    np.testing.assert_allclose(out[0, 0, 0], p @ vh, rtol=1e-12, atol=1e-14)


def test_page_order_does_not_change_result():
    rng = np.random.default_rng(9)
    T = 10
    k = rng.standard_normal((T, 1, 128)).astype(np.float16)
    v = rng.standard_normal((T, 1, 128)).astype(np.float16)
    q = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    outs = []
    for perm in (np.arange(3), np.array([1, 2, 0])):
        kc, order = _cache_from(k, 4, [[1, 2, 3, 4]], block_size=4, shuffle=perm)
        vc, _ = _cache_from(v, 3, [[4, 3, 2, 1]], block_size=4, shuffle=perm)
        outs.append(O.decode_attention(q, kc, vc, [T], order[None], 1))
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-14)


def test_causal_multi_token_equals_truncated_single_token():
    rng = np.random.default_rng(10)
    T, nq = 9, 3
    k = rng.standard_normal((T, 1, 128)).astype(np.float16)
    v = rng.standard_normal((T, 1, 128)).astype(np.float16)
    kc, order = _cache_from(k, 4, [[1, 2, 3, 4]], block_size=4)
    vc, _ = _cache_from(v, 4, [[4, 3, 2, 1]], block_size=4)
    q = rng.standard_normal((1, nq, 1, 128)).astype(np.float16)
    out = O.decode_attention(q, kc, vc, [T], order[None], nq)
    for j in range(nq):
        single = O.decode_attention(q[:, j:j + 1], kc, vc, [T - nq + j + 1], order[None], 1)
        np.testing.assert_allclose(out[0, j, 0], single[0, 0, 0], rtol=1e-14)
    # a row that sees no token outputs zeros
    z = O.decode_attention(q, kc, vc, [1], order[None], nq)
    assert np.all(z[0, :2] == 0) and np.any(z[0, 2] != 0)


def test_gqa_maps_query_head_to_kv_head_by_division():
    rng = np.random.default_rng(12)
    T, hkv, g = 6, 2, 3
    k = rng.standard_normal((T, hkv, 128)).astype(np.float16)
    v = rng.standard_normal((T, hkv, 128)).astype(np.float16)
    kc, order = _cache_from(k, 4, [[1, 2, 3, 4], [5, 6, 7, 8]], block_size=8)
    vc, _ = _cache_from(v, 3, [[8, 7, 6, 5], [4, 3, 2, 1]], block_size=8)
    q = rng.standard_normal((1, 1, hkv * g, 128)).astype(np.float16)
    out = O.decode_attention(q, kc, vc, [T], order[None], 1)
    slots = O.slots_for_sequence(order, 8, T)
    for h in range(hkv * g):
        kv = h // g
        kh, vh = O.cache_read(kc, slots, kv), O.cache_read(vc, slots, kv)
        s = kh @ q[0, 0, h].astype(np.float64) / math.sqrt(128)
        p = np.exp(s - s.max()); p /= p.sum()
        np.testing.assert_allclose(out[0, 0, h], p @ vh, rtol=1e-12, atol=1e-14)


def test_sparse_v_semantics():
    """[TQ+ article]: V of low-weight positions is skipped and treated as zero."""
    rng = np.random.default_rng(13)
    T = 40
    k = rng.standard_normal((T, 1, 128)).astype(np.float16) * np.float16(3)
    v = rng.standard_normal((T, 1, 128)).astype(np.float16)
    kc, order = _cache_from(k, 4, [[1, 2, 3, 4]], block_size=8)
    vc, _ = _cache_from(v, 2, [[4, 3, 2, 1]], block_size=8)
    q = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    tbl = order[None]
    dense, w = O.decode_attention(q, kc, vc, [T], tbl, 1, return_weights=True)
    p = w[(0, 0, 0)]
    vh = O.cache_read(vc, O.slots_for_sequence(order, 8, T), 0)
    assert np.array_equal(O.decode_attention(q, kc, vc, [T], tbl, 1, tau=0.0), dense)
    assert np.all(O.decode_attention(q, kc, vc, [T], tbl, 1, tau=1.01) == 0)
    tau = float(np.sort(p)[T // 2]) * 1.0000001
    sp = O.decode_attention(q, kc, vc, [T], tbl, 1, tau=tau)
    want = np.zeros(128)
    for t in range(T):                       # enumeration, no renormalisation
        if p[t] >= tau:
            want += p[t] * vh[t]
    np.testing.assert_allclose(sp[0, 0, 0], want, rtol=1e-12, atol=1e-14)
    skipped = p < tau
    bound = np.sum(p[skipped] * np.linalg.norm(vh[skipped], axis=1))
    assert np.linalg.norm(sp[0, 0, 0] - dense[0, 0, 0]) <= bound * (1 + 1e-12)


# ----------------------------------------------------------- data-fitted codebook

def _cluster_vectors(n_vec, levels, rng, jitter=0.01):
    """Float16 vectors whose rotated coordinates fall in len(levels) well separated
    clusters, 128 / len(levels) coordinates per cluster; also the cluster label of
    each coordinate."""
    k = len(levels)
    base = np.repeat(np.asarray(levels, dtype=np.float64), 128 // k)
    s = O.sign_vector([0x12345678, 0x9ABCDEF0, 0x0F1E2D3C, 0x4B5A6978])
    xs, labels = [], []
    for _ in range(n_vec):
        perm = rng.permutation(128)
        y = base[perm] * (1.0 + jitter * rng.standard_normal(128))
        y /= np.linalg.norm(y)
        xs.append(O.unrotate(y[None, :], s)[0] * 3.0)
        labels.append(np.repeat(np.arange(k), 128 // k)[perm])
    x16 = np.asarray(xs).astype(np.float16)
    return x16, np.asarray(labels), s


def test_fit_codebook_lands_on_cluster_means():
    """Well separated clusters: the fixed point of assign/mean is the clusters' means."""
    rng = np.random.default_rng(11)
    x16, labels, s = _cluster_vectors(64, [-3.0, -1.0, 1.0, 3.0], rng)
    sw = [0x12345678, 0x9ABCDEF0, 0x0F1E2D3C, 0x4B5A6978]
    cb, c64, _ = O.fit_codebook(2, x16[:, None, :], [sw])
    # the same samples, grouped by the cluster they were drawn from
    x = x16.astype(np.float64)
    y = O.rotate(x / np.linalg.norm(x, axis=1, keepdims=True), s)
    means = np.array([y[labels == j].mean() for j in range(4)])
    assert np.allclose(c64, means, rtol=0, atol=1e-12)
    assert np.array_equal(cb.centroids, means.astype(np.float16).astype(np.float64))
    assert np.array_equal(cb.boundaries, (cb.centroids[:-1] + cb.centroids[1:]) / 2)


@pytest.mark.parametrize("bits", [2, 3])
def test_fit_codebook_lloyd_conditions_and_descent(bits):
    """On heavy-tailed data: every centre is the mean of its cell, and the fit is no
    worse on its samples than the Gaussian codebook it starts from."""
    rng = np.random.default_rng(20 + bits)
    x = rng.laplace(size=(256, 2, 128)) * np.where(rng.random((256, 2, 128)) < 0.01, 30.0, 1.0)
    sw = rng.integers(0, 2 ** 32, size=(2, 4), dtype=np.uint64).astype(np.uint32)
    cb, c64, y = O.fit_codebook(bits, x.astype(np.float16), sw)
    b64 = (c64[:-1] + c64[1:]) / 2
    cell = O.encode(y, b64)
    for j in range(1 << bits):
        assert abs(c64[j] - y[cell == j].mean()) < 1e-15
    init = O.build_codebook(bits)
    mse_init = np.mean((y - init.centroids[O.encode(y, init.boundaries)]) ** 2)
    mse_fit = np.mean((y - c64[cell]) ** 2)
    assert mse_fit <= mse_init * (1 + 1e-12)
    assert cb.mse == pytest.approx(np.mean((y - cb.centroids[O.encode(y, cb.boundaries)]) ** 2), rel=1e-12)


def test_fit_codebook_skips_zero_vectors():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 1, 128)).astype(np.float16)
    sw = [[1, 2, 3, 4]]
    a, _, _ = O.fit_codebook(3, x, sw)
    b, _, _ = O.fit_codebook(3, np.concatenate([x, np.zeros((9, 1, 128), np.float16)]), sw)
    assert np.array_equal(a.centroids, b.centroids)


# --------------------------------------------------------------- float16 K side

def test_float16_side_roundtrip_and_attention():
    """R11: a float16 side stores the row's bytes and reads them back exactly; with a
    float16 K side, attention is softmax(scale q . k) over the visible positions
    against the dequantized V, written out here directly."""
    rng = np.random.default_rng(3)
    n_kv, bs, n_tok, G = 2, 16, 37, 3
    k = (rng.standard_normal((n_tok, n_kv, 128)) * 4).astype(np.float16)
    v = rng.standard_normal((n_tok, n_kv, 128)).astype(np.float16)
    sv = rng.integers(0, 2 ** 32, size=(n_kv, 4), dtype=np.uint64).astype(np.uint32)
    kc = O.new_cache(O.FP16, n_kv, bs, 4, np.zeros((n_kv, 4), np.uint32), None)
    vc = O.new_cache(3, n_kv, bs, 4, sv, O.build_codebook(3))
    table = np.array([[2, 0, 3]], np.int32)
    slots = O.slots_for_sequence(table[0], bs, n_tok)
    O.cache_write(kc, k, slots)
    O.cache_write(vc, v, slots)
    for h in range(n_kv):
        assert np.array_equal(O.cache_read(kc, slots, h), k[:, h].astype(np.float64))
    q = rng.standard_normal((1, 2, n_kv * G, 128)).astype(np.float16)
    out = O.decode_attention(q, kc, vc, np.array([n_tok], np.int32), table, 2, 0.0, 0.0)
    for j in range(2):
        for h in range(n_kv * G):
            kv = h // G
            t_vis = n_tok - 2 + j + 1
            s = (q[0, j, h].astype(np.float64) @ k[:t_vis, kv].astype(np.float64).T) / math.sqrt(128)
            p = np.exp(s - s.max())
            p /= p.sum()
            v_hat = O.cache_read(vc, slots[:t_vis], kv)
            assert np.allclose(out[0, j, h], p @ v_hat, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------- heads of several blocks (R12)

@pytest.mark.parametrize("head_dim", [256, 512])
def test_wide_head_is_independent_blocks(head_dim):
    """R12: block i of head j is the 128-slice [128 i, 128 i + 128) quantized on its
    own with sign words signs[j, i]; changing one slice changes only its block."""
    rng = np.random.default_rng(11)
    nb, n_kv, bs, n_tok = head_dim // 128, 3, 8, 13
    x = (rng.standard_normal((n_tok, n_kv, head_dim)) * 3).astype(np.float16)
    sw = rng.integers(0, 2 ** 32, size=(n_kv, nb, 4), dtype=np.uint64).astype(np.uint32)
    cb = O.build_codebook(3)
    c = O.new_cache(3, n_kv, bs, 2, sw, cb, head_dim=head_dim)
    slots = O.slots_for_sequence(np.array([1, 0]), bs, n_tok)
    O.cache_write(c, x, slots)
    for j in range(n_kv):
        got = O.cache_read(c, slots, j)
        assert got.shape == (n_tok, head_dim)
        for i in range(nb):
            s = O.sign_vector(sw[j, i])
            n, codes, _ = O.quantize_vectors(x[:, j, 128 * i:128 * (i + 1)], s, cb)
            want = O.dequantize_vectors(n, codes, s, cb)
            np.testing.assert_array_equal(got[:, 128 * i:128 * (i + 1)], want)
    # locality: a new last block leaves every other block as it was
    x2 = x.copy()
    x2[:, :, head_dim - 128:] = (rng.standard_normal((n_tok, n_kv, 128)) * 7).astype(np.float16)
    c2 = O.new_cache(3, n_kv, bs, 2, sw, cb, head_dim=head_dim)
    O.cache_write(c2, x2, slots)
    for j in range(n_kv):
        a, b = O.cache_read(c, slots, j), O.cache_read(c2, slots, j)
        np.testing.assert_array_equal(a[:, :head_dim - 128], b[:, :head_dim - 128])
        assert not np.array_equal(a[:, head_dim - 128:], b[:, head_dim - 128:])


def test_wide_head_attention_reduces_to_one_block():
    """With q zero outside block 0, 256-wide attention scores equal the 128-wide
    scores of block 0 (same explicit scale); output block 0 is then the 128-wide
    attention over the V block-0 cache and output block 1 the same weights applied
    to the V block-1 cache."""
    rng = np.random.default_rng(12)
    n_kv, G, bs, n_tok = 2, 2, 16, 41
    k = rng.standard_normal((n_tok, n_kv, 256)).astype(np.float16)
    v = rng.standard_normal((n_tok, n_kv, 256)).astype(np.float16)
    sk = rng.integers(0, 2 ** 32, size=(n_kv, 2, 4), dtype=np.uint64).astype(np.uint32)
    sv = rng.integers(0, 2 ** 32, size=(n_kv, 2, 4), dtype=np.uint64).astype(np.uint32)
    cbk, cbv = O.build_codebook(4), O.build_codebook(2)
    table = np.array([[2, 0, 1]], np.int32)
    slots = O.slots_for_sequence(table[0], bs, n_tok)

    def cache(bits, cb, src, sw, hd):
        c = O.new_cache(bits, n_kv, bs, 3, sw, cb, head_dim=hd)
        O.cache_write(c, src, slots)
        return c

    kc, vc = cache(4, cbk, k, sk, 256), cache(2, cbv, v, sv, 256)
    k0 = cache(4, cbk, k[:, :, :128], sk[:, 0], 128)
    v0 = cache(2, cbv, v[:, :, :128], sv[:, 0], 128)
    v1 = cache(2, cbv, v[:, :, 128:], sv[:, 1], 128)
    q = np.zeros((1, 1, n_kv * G, 256), np.float16)
    q[..., :128] = rng.standard_normal((1, 1, n_kv * G, 128)).astype(np.float16)
    lens = np.array([n_tok], np.int32)
    wide = O.decode_attention(q, kc, vc, lens, table, 1, scale=0.3)
    narrow0 = O.decode_attention(q[..., :128], k0, v0, lens, table, 1, scale=0.3)
    narrow1 = O.decode_attention(q[..., :128], k0, v1, lens, table, 1, scale=0.3)
    np.testing.assert_allclose(wide[..., :128], narrow0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(wide[..., 128:], narrow1, rtol=1e-12, atol=1e-13)


def test_wide_head_two_tokens_closed_form_default_scale():
    """Two tokens, head_dim 512: p0 = 1 / (1 + e^(s1 - s0)) with s = q . k_hat / sqrt(512)
    (the default scale is 1/sqrt(head_dim)); the wide float16 side reads back exactly."""
    rng = np.random.default_rng(13)
    k = rng.standard_normal((2, 1, 512)).astype(np.float16)
    v = rng.standard_normal((2, 1, 512)).astype(np.float16)
    kc = O.new_cache(O.FP16, 1, 4, 1, np.zeros((1, 4, 4), np.uint32), None, head_dim=512)
    vc = O.new_cache(4, 1, 4, 1, rng.integers(0, 2 ** 32, size=(4, 4), dtype=np.uint64).astype(np.uint32),
                     O.build_codebook(4), head_dim=512)
    slots = np.array([0, 1])
    O.cache_write(kc, k, slots)
    O.cache_write(vc, v, slots)
    kh = O.cache_read(kc, slots, 0)
    np.testing.assert_array_equal(kh, k[:, 0].astype(np.float64))
    vh = O.cache_read(vc, slots, 0)
    q = rng.standard_normal((1, 1, 1, 512)).astype(np.float16)
    qq = q[0, 0, 0].astype(np.float64)
    s0, s1 = kh @ qq / math.sqrt(512)
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    out = O.decode_attention(q, kc, vc, [2], np.array([[0]]), 1)
    np.testing.assert_allclose(out[0, 0, 0], p0 * vh[0] + (1 - p0) * vh[1], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------- V outlier channels (R13)

def test_select_outlier_channels_brute_force_and_planted():
    """The k channels of largest mean square (ties to the lower index), ascending:
    against a loop over channels, and planted x20 channels are found."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((40, 3, 128)).astype(np.float16)
    x[:, :, 7] = 0
    x[:, :, 9] = 0        # a tie at zero: never among the top
    planted = [[5, 77, 100, 126], [0, 1, 2, 3], [64, 65, 90, 127]]
    for h in range(3):
        x[:, h, planted[h]] *= np.float16(20)
    got = O.select_outlier_channels(x, 4)
    for h in range(3):
        assert list(got[h]) == planted[h]
    got8 = O.select_outlier_channels(x, 8)
    for h in range(3):
        ms = []
        for c in range(128):
            acc = 0.0
            for t in range(40):
                acc += float(x[t, h, c]) ** 2
            ms.append((-acc / 40, c))
        want = sorted(c for _, c in sorted(ms)[:8])
        assert list(got8[h]) == want
    # a tie decided by the lower index
    y = np.ones((2, 1, 128), np.float16)
    assert list(O.select_outlier_channels(y, 3)[0]) == [0, 1, 2]


def test_outlier_side_keeps_channels_and_quantizes_the_rest():
    """R13: the kept channels read back exactly; every other channel equals the plain
    TurboQuant reconstruction of the vector with the kept channels zeroed (its norm
    and rotation see zeros there)."""
    rng = np.random.default_rng(22)
    n_kv, bs, n_tok = 2, 8, 21
    x = rng.standard_normal((n_tok, n_kv, 128)).astype(np.float16)
    idx = np.array([[3, 40, 41, 99, 127], [0, 8, 16, 64, 65]], np.uint8)
    x[:, 0, idx[0]] *= np.float16(30)
    sw = rng.integers(0, 2 ** 32, size=(n_kv, 4), dtype=np.uint64).astype(np.uint32)
    cb = O.build_codebook(3)
    c = O.new_cache(3, n_kv, bs, 4, sw, cb, outlier_channels=idx[:, ::-1])   # any order in, ascending kept
    assert np.array_equal(c.outlier_channels, idx)
    slots = O.slots_for_sequence(np.array([3, 1, 0]), bs, n_tok)
    O.cache_write(c, x, slots)
    for h in range(n_kv):
        got = O.cache_read(c, slots, h)
        np.testing.assert_array_equal(got[:, idx[h]], x[:, h, idx[h]].astype(np.float64))
        z = x[:, h].copy()
        z[:, idx[h]] = 0
        s = O.sign_vector(sw[h])
        n, codes, _ = O.quantize_vectors(z, s, cb)
        want = O.dequantize_vectors(n, codes, s, cb)
        rest = np.setdiff1d(np.arange(128), idx[h])
        np.testing.assert_array_equal(got[:, rest], want[:, rest])


def test_outlier_separation_cuts_the_error_of_planted_outliers():
    """With 4 channels x20 per token, keeping them exactly leaves the quantization
    error of an ordinary N(0,1) vector; without it the outliers dominate the norm
    and the other channels lose most of their resolution."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((400, 1, 128))
    ch = [10, 50, 90, 120]
    x[:, :, ch] *= 20
    x = x.astype(np.float16)
    sw = rng.integers(0, 2 ** 32, size=(1, 4), dtype=np.uint64).astype(np.uint32)
    slots = np.arange(400)
    errs = []
    for idx in (None, O.select_outlier_channels(x, 4)):
        c = O.new_cache(3, 1, 400, 1, sw, O.build_codebook(3), outlier_channels=idx)
        O.cache_write(c, x, slots)
        d = O.cache_read(c, slots, 0) - x[:, 0].astype(np.float64)
        errs.append(np.sum(d * d) / np.sum(x[:, 0].astype(np.float64) ** 2))
    assert errs[1] < errs[0] / 10, errs


def test_outlier_attention_two_tokens_closed_form():
    """Two tokens: at a kept channel the output is p0 v0[c] + p1 v1[c] with the
    exact stored values (p from the K side's closed form)."""
    rng = np.random.default_rng(24)
    k = rng.standard_normal((2, 1, 128)).astype(np.float16)
    v = rng.standard_normal((2, 1, 128)).astype(np.float16)
    v[:, 0, [6, 60]] = np.float16(300)
    kc = O.new_cache(4, 1, 4, 1, [[1, 2, 3, 4]], O.build_codebook(4))
    vc = O.new_cache(2, 1, 4, 1, [[5, 6, 7, 8]], O.build_codebook(2), outlier_channels=[[6, 60]])
    O.cache_write(kc, k, np.array([0, 1]))
    O.cache_write(vc, v, np.array([0, 1]))
    q = rng.standard_normal((1, 1, 1, 128)).astype(np.float16)
    kh = O.cache_read(kc, np.array([0, 1]), 0)
    s0, s1 = kh @ q[0, 0, 0].astype(np.float64) / math.sqrt(128)
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    out = O.decode_attention(q, kc, vc, [2], np.array([[0]]), 1)
    for c in (6, 60):
        np.testing.assert_allclose(out[0, 0, 0, c], p0 * float(v[0, 0, c]) + (1 - p0) * float(v[1, 0, c]),
                                   rtol=1e-13)
