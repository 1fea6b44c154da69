"""Pins that hold the CPU oracle to something other than itself.

Each test names the fact it checks: a published test vector, a closed form,
a textbook special case, brute force on tiny inputs, an invariant, or the
method's own statistical claim (unbiasedness, 1/m variance).  A plausible
mistake in the oracle (dropped term, wrong sign or index, transposed operand,
wrong constant) fails at least one of them.
"""
import math

import numpy as np
import pytest
from scipy import integrate

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- O1 PRNG
def test_splitmix64_published_vector():
    # SplitMix64 from state 0: the first outputs of the reference generator
    # (Steele, Lea & Flood 2014; Vigna's splitmix64.c) are these three words.
    w = O.splitmix64(0, 0, np.arange(3))
    assert [int(x) for x in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    # seed ^ tag keys the stream
    assert int(O.splitmix64(5, 5, [0])[0]) == 0xE220A8397B1DCDAF


def test_gaussian_matrix_is_standard_normal():
    S = O.gaussian_matrix(1024, 1024, seed=7).astype(np.float64).ravel()
    n = S.size
    se = 1 / math.sqrt(n)
    assert abs(S.mean()) < 4 * se
    assert abs(S.var() - 1) < 4 * math.sqrt(2 / n)
    kurt = np.mean(S ** 4) / S.var() ** 2
    assert abs(kurt - 3) < 4 * math.sqrt(24 / n)
    # P(|g| > 1.96) = 0.05 for a standard normal
    frac = np.mean(np.abs(S) > 1.959963984540054)
    assert abs(frac - 0.05) < 4 * math.sqrt(0.05 * 0.95 / n)
    # cos and sin halves of a pair are uncorrelated
    c, s = S[0::2], S[1::2]
    assert abs(np.mean(c * s)) < 4 / math.sqrt(c.size)


def test_rademacher_signs_balanced():
    D = O.rademacher_signs(1 << 16, seed=3)
    assert set(np.unique(D)) == {-1.0, 1.0}
    assert abs(D.mean()) < 4 / math.sqrt(D.size)


# ---------------------------------------------------------------- O2 rotation
@pytest.mark.parametrize("d", [1, 2, 4, 8, 16])
def test_sylvester_equals_walsh_closed_form(d):
    # Brute force: the natural-order Sylvester matrix has H_ij = (-1)^popcount(i & j).
    H = O.sylvester_hadamard(d)
    ref = np.array([[(-1) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
    assert np.array_equal(H, ref)


def test_paley_12_is_hadamard():
    H = O.paley_hadamard_12()
    assert set(np.unique(H)) == {-1, 1}
    assert np.array_equal(H @ H.T, 12 * np.eye(12, dtype=np.int64))


@pytest.mark.parametrize("d", [16, 128, 1536])
def test_rotation_orthogonal_norm_preserving(d):
    R = O.rotation_matrix(d, seed=1234)
    assert np.max(np.abs(R.T @ R - np.eye(d))) < 1e-13
    x = np.random.default_rng(0).standard_normal((5, d))
    assert np.allclose(np.linalg.norm(x @ R.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_rotation_is_hadamard_times_signs():
    d = 128
    R = O.rotation_matrix(d, seed=99)
    D = O.rademacher_signs(d, 99)
    # column j of R = D_j * column j of H / sqrt(d), with H Walsh closed form
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
    assert np.array_equal(R * math.sqrt(d), H * D[None, :])


def test_kron_index_convention_1536():
    H = O.hadamard(1536)
    H12, H128 = O.paley_hadamard_12(), O.sylvester_hadamard(128)
    rng = np.random.default_rng(1)
    for _ in range(200):
        a, b, i, j = rng.integers(0, 12), rng.integers(0, 12), rng.integers(0, 128), rng.integers(0, 128)
        assert H[a * 128 + i, b * 128 + j] == H12[a, b] * H128[i, j]


# ---------------------------------------------------------------- density / Lloyd-Max
@pytest.mark.parametrize("d", [16, 128, 1536])
def test_density_normalised_and_second_moment(d):
    f = lambda x: float(O.sphere_coordinate_density(x, d))
    s = 6 / math.sqrt(d)
    tot = integrate.quad(f, -1, 1, points=[-s, 0, s], limit=200)[0]
    m2 = integrate.quad(lambda x: x * x * f(x), -1, 1, points=[-s, 0, s], limit=200)[0]
    assert abs(tot - 1) < 1e-10
    assert abs(m2 * d - 1) < 1e-9      # E[X^2] = 1/d for a coordinate of a unit vector


@pytest.mark.parametrize("d", [128, 1536])
def test_cdf_and_moment_match_quadrature(d):
    f = lambda x: float(O.sphere_coordinate_density(x, d))
    for t in np.array([-2.0, -0.7, 0.0, 0.3, 1.1, 2.5]) / math.sqrt(d):
        ref = integrate.quad(f, -1, t, limit=400, points=[0.0] if t > 0 else None)[0]
        assert abs(float(O.sphere_coordinate_cdf(t, d)) - ref) < 1e-10
    lo, hi = -0.4 / math.sqrt(d), 1.3 / math.sqrt(d)
    ref = integrate.quad(lambda x: x * f(x), lo, hi)[0]
    assert abs(float(O.sphere_coordinate_first_moment(lo, hi, d)) - ref) < 1e-12


@pytest.mark.parametrize("d", [128, 1536])
def test_lloyd_max_one_bit_closed_form(d):
    # b = 1: c = E|X| = Γ(d/2) / (√π Γ((d+1)/2)),  D = 1 - d c²
    c, t, _ = O.lloyd_max(d, 1)
    ref = math.exp(math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d + 1) / 2))
    assert abs(c[1] - ref) < 1e-11 * ref and abs(c[0] + ref) < 1e-11 * ref
    assert t[0] == 0.0
    if d == 128:
        assert abs(ref - 0.070661572738) < 1e-11
        assert abs((1 - d * ref * ref) - 0.360888594) < 1e-8


# Max (1960), "Quantizing for minimum distortion", optimum quantizer for the
# unit Gaussian: output levels and mean squared error for N = 2, 4, 8 levels.
MAX_1960 = {1: ([0.7979], 0.3634), 2: ([0.4528, 1.510], 0.1175), 3: ([0.2451, 0.7560, 1.344, 2.152], 0.03454)}


@pytest.mark.parametrize("b", [1, 2, 3])
def test_lloyd_max_gaussian_limit_matches_max_1960(b):
    d = 1 << 16   # the sphere law tends to N(0, 1/d); sqrt(d)*c tends to Max's levels
    c, t, _ = O.lloyd_max(d, b)
    levels, mse = MAX_1960[b]
    got = c[len(c) // 2:] * math.sqrt(d)
    assert np.allclose(got, levels, atol=1.5e-3)
    D = _distortion_by_quadrature(c, t, d)
    assert abs(D - mse) < 2e-4


def _distortion_by_quadrature(c, t, d):
    f = lambda x: float(O.sphere_coordinate_density(x, d))
    edges = np.concatenate([[-1.0], t, [1.0]])
    tot = 0.0
    for k in range(len(c)):
        lo, hi = edges[k], edges[k + 1]
        # integrate on a window that holds all the mass (|x| < 12/sqrt(d)) to keep quad accurate
        w = 12 / math.sqrt(d)
        lo, hi = max(lo, -w), min(hi, w)
        tot += integrate.quad(lambda x: (x - c[k]) ** 2 * f(x), lo, hi, limit=200)[0]
    return tot * d


@pytest.mark.parametrize("d,b", [(128, 2), (128, 3), (1536, 2), (1536, 3)])
def test_lloyd_max_fixed_point_and_bound(d, b):
    c, t, _ = O.lloyd_max(d, b)
    f = lambda x: float(O.sphere_coordinate_density(x, d))
    edges = np.concatenate([[-1.0], t, [1.0]])
    w = 14 / math.sqrt(d)
    for k in range(len(c)):   # centroid condition, checked by quadrature
        lo, hi = max(edges[k], -w), min(edges[k + 1], w)
        m0 = integrate.quad(f, lo, hi, limit=200, epsabs=1e-15)[0]
        m1 = integrate.quad(lambda x: x * f(x), lo, hi, limit=200, epsabs=1e-16)[0]
        assert abs(m1 / m0 - c[k]) * math.sqrt(d) < 1e-9
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-17)   # nearest neighbour
    assert np.array_equal(c, -c[::-1])                                    # symmetric
    D = _distortion_by_quadrature(c, t, d)
    # information-theoretic lower bound D_MSE >= 4^-b (深度拆解 第六部分)
    assert D >= 4.0 ** -b
    assert D < {2: 0.12, 3: 0.036}[b]


def test_walsh_expansion_symmetric_codebook_has_only_odd_terms():
    for b in (2, 3):
        c, _, _ = O.lloyd_max(128, b)
        coef = O.walsh_plane_coefficients(c)
        for S, v in coef.items():
            if len(S) % 2 == 0:
                assert abs(v) < 1e-16
        # reconstruct
        for idx in range(1 << b):
            acc = 0.0
            for S, v in coef.items():
                s = 1.0
                for i in S:
                    s *= 2 * ((idx >> i) & 1) - 1
                acc += v * s
            assert abs(acc - c[idx]) < 1e-15


# ---------------------------------------------------------------- packing / storage
def test_packing_bit_positions():
    d, b = 128, 3
    idx = np.zeros((1, d), dtype=np.int64)
    idx[0, 37] = 0b101
    codes = O.pack_planes(idx, b)
    assert codes.shape == (1, 12)
    expect = np.zeros(12, dtype=np.uint32)
    expect[0 * 4 + 1] = 1 << 5     # plane 0, word 37//32 = 1, bit 5
    expect[2 * 4 + 1] = 1 << 5     # plane 2
    assert np.array_equal(codes[0], expect)
    rnd = np.random.default_rng(0).integers(0, 8, size=(7, d))
    assert np.array_equal(O.unpack_planes(O.pack_planes(rnd, b), b, d), rnd)
    bits = np.random.default_rng(1).integers(0, 2, size=(3, 256))
    assert np.array_equal(O.unpack_bits(O.pack_bits(bits), 256), bits)


@pytest.mark.parametrize("bits,ratio", [(3, 16 / 3), (4, 4.0)])
def test_storage_ratio_vs_fp16(bits, ratio):
    cd = O.make_codec(128, bits)
    payload = 4 * (cd.code_words + cd.sign_words)
    assert payload == 128 * bits // 8            # d * B_t / 8 bytes
    assert (2 * 128) / payload == pytest.approx(ratio, rel=0, abs=1e-15)
    assert cd.record_bytes == payload + 8         # + fp32 ν and γ


# ---------------------------------------------------------------- O4 encode
@pytest.fixture(scope="module")
def codec3():
    return O.make_codec(128, 3, seed=1234)


@pytest.fixture(scope="module")
def codec4():
    return O.make_codec(128, 4, seed=1234)


@pytest.mark.parametrize("which", ["codec3", "codec4"])
def test_encode_mc_distortion_equals_codebook_distortion(which, request):
    # Gaussian x: x/||x|| is uniform on the sphere, so after any fixed rotation
    # each coordinate follows the sphere law and E||u - Rᵀ ĉ||² = d·E(X - Q(X))².
    cd = request.getfixturevalue(which)
    x = np.random.default_rng(5).standard_normal((100_000, cd.d))
    enc = O.encode(cd, x)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    chat = cd.c32.astype(np.float64)[enc["idx"]]
    err = np.sum((u - chat @ cd.R) ** 2, axis=1)
    D = _distortion_by_quadrature(cd.c32.astype(np.float64), cd.t32.astype(np.float64), cd.d)
    se = err.std() / math.sqrt(err.size)
    assert abs(err.mean() - D) < 3.5 * se
    assert np.allclose(enc["rnorm"] ** 2, err, rtol=2e-6)
    assert np.allclose(enc["norm"], np.linalg.norm(x, axis=1).astype(np.float32), rtol=0)


@pytest.mark.parametrize("which", ["codec3", "codec4"])
def test_encode_basis_vector_worked_case(which, request):
    # x = e_k: y_j = D_k H_jk / sqrt(d), so every |y_j| = 1/sqrt(d); every code
    # sits in the cell holding ±1/sqrt(d) and γ = |1 - sqrt(d) c_level|.
    cd = request.getfixturevalue(which)
    d = cd.d
    k = 17
    x = np.zeros((1, d)); x[0, k] = 3.0
    enc = O.encode(cd, x)
    t = cd.t32.astype(np.float64) * math.sqrt(d)
    level = int(np.sum(t < 1.0))                 # cell of +1/sqrt(d)
    H = np.array([(-1) ** bin(j & k).count("1") for j in range(d)])
    sign = cd.D[k] * H
    expect_idx = np.where(sign > 0, level, (1 << cd.b) - 1 - level)
    assert np.array_equal(enc["idx"][0], expect_idx)
    c_lvl = float(cd.c32[level]) * math.sqrt(d)
    assert abs(float(enc["rnorm"][0]) - abs(1 - c_lvl)) < 1e-6
    assert float(enc["norm"][0]) == 3.0


def test_encode_zero_vector(codec3):
    enc = O.encode(codec3, np.zeros((2, 128)))
    assert np.all(enc["norm"] == 0)
    # y = 0: idx = #{t < 0} (ties low)
    assert np.all(enc["idx"] == np.sum(codec3.t32 < 0))
    q = np.random.default_rng(0).standard_normal((3, 128))
    assert np.all(O.score(codec3, q, enc) == 0)
    assert np.all(O.dequantize(codec3, enc) == 0)


def test_encode_ties_go_low(codec3):
    # a coordinate exactly on a boundary takes the lower code
    cd = codec3
    y = np.zeros(128); y[0] = float(cd.t32[2]); y[1] = -0.2
    y /= np.linalg.norm(y)
    # y[0] is no longer on the boundary after normalisation; check the rule directly
    t = cd.t32.astype(np.float64)
    v = np.array([t[2], np.nextafter(np.float32(t[2]), np.float32(1))], dtype=np.float64)
    idx = np.sum(t[None, :] < v[:, None], axis=1)
    assert list(idx) == [2, 3]


# ---------------------------------------------------------------- QJL estimator
def test_qjl_estimator_unbiased_and_variance_closed_form():
    # Fix q', r; draw S fresh (independent rows of one seeded stream); the
    # estimator sqrt(pi/2)/m ||r|| <S q', sign(S r)> is unbiased with variance
    # ((pi/2) ||r||² ||q'||² - <q', r>²) / m   (深度拆解 第六部分: unbiased, 1/m).
    d = m = 32
    rng = np.random.default_rng(11)
    qv = rng.standard_normal(d)
    r = rng.standard_normal(d) * 0.3 + 0.2 * qv
    gamma = np.linalg.norm(r)
    n_trials = 100_000
    kappa = O.qjl_constant(m)
    ests = []
    per = 20_000
    for blk in range(n_trials // per):
        S = O.gaussian_matrix(per * m, d, seed=777 + blk).astype(np.float64).reshape(per, m, d)
        p = S @ qv
        z = S @ r
        tau = np.where(z >= 0, 1.0, -1.0)
        ests.append(kappa * gamma * np.sum(p * tau, axis=1))
    e = np.concatenate(ests)
    truth = qv @ r
    var_cf = ((math.pi / 2) * gamma ** 2 * (qv @ qv) - truth ** 2) / m
    se = math.sqrt(var_cf / e.size)
    assert abs(e.mean() - truth) < 3 * se
    # sample variance within a 99.9% chi-square band (normal approx of its SE)
    assert abs(e.var() / var_cf - 1) < 3.3 * math.sqrt(2 / (e.size - 1)) * 1.5


def test_score_end_to_end_unbiased_over_qjl_matrix():
    # For a fixed rotation, E_S[ℓ] = ν <q', ŷ + r> = <q, x>: the full score is
    # unbiased over the QJL matrix; a wrong constant or sign in the QJL term
    # breaks this.
    d = 32
    base = O.make_codec(d, 3, seed=5)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, d)) * 2.0
    q = rng.standard_normal((1, d))
    vals = []
    for s in range(4000):
        cd = O.Codec(d=d, bits=3, m=d, seed=s, D=base.D, R=base.R,
                     S=O.gaussian_matrix(d, d, seed=10_000 + s),
                     centroids=base.centroids, bounds=base.bounds, iters=base.iters)
        vals.append(float(O.score(cd, q, O.encode(cd, x))[0, 0]))
    vals = np.array(vals)
    se = vals.std() / math.sqrt(vals.size)
    assert abs(vals.mean() - float((q @ x.T)[0, 0])) < 3.5 * se


def test_inner_product_distortion_lower_bound(codec3):
    # D_prod >= (||q||²/d) 4^-b for unit keys (深度拆解 第六部分)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((20_000, 128))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    q = rng.standard_normal(128)
    enc = O.encode(codec3, x)
    err = (O.score(codec3, q, enc)[0] - x @ q) ** 2
    assert err.mean() >= (q @ q / 128) * 4.0 ** -codec3.b


# ---------------------------------------------------------------- O5 score invariants
def test_score_invariants(codec3):
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((300, 128))
    enc = O.encode(codec3, keys)
    q1, q2 = rng.standard_normal((2, 128))
    s1, s2 = O.score(codec3, q1, enc)[0], O.score(codec3, q2, enc)[0]
    s12 = O.score(codec3, 2.5 * q1 - 0.5 * q2, enc)[0]
    assert np.allclose(s12, 2.5 * s1 - 0.5 * s2, rtol=1e-12, atol=1e-12)
    assert np.all(O.score(codec3, np.zeros(128), enc) == 0)
    perm = rng.permutation(300)
    enc_p = {k: enc[k][perm] for k in ("codes", "signs", "norm", "rnorm")}
    assert np.array_equal(O.score(codec3, q1, enc_p)[0], s1[perm])
    # scaling the key scales ν only
    enc2 = O.encode(codec3, 4.0 * keys)
    assert np.array_equal(enc2["codes"], enc["codes"]) and np.array_equal(enc2["signs"], enc["signs"])


def test_score_matches_explicit_sum(codec3):
    # one key, one query, the estimator written out term by term
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 128)); q = rng.standard_normal(128)
    enc = O.encode(codec3, x)
    qr = codec3.R @ q
    p = codec3.S.astype(np.float64) @ qr
    idx = enc["idx"][0]
    tau = 2 * O.unpack_bits(enc["signs"], 128)[0] - 1
    mse = sum(qr[j] * float(codec3.c32[idx[j]]) for j in range(128))
    qjl = sum(p[i] * tau[i] for i in range(128))
    ref = float(enc["norm"][0]) * (mse + math.sqrt(math.pi / 2) / 128 * float(enc["rnorm"][0]) * qjl)
    assert abs(O.score(codec3, q, enc)[0, 0] - ref) < 1e-11 * abs(ref) + 1e-12


def test_attn_logits_gqa_layout(codec3):
    rng = np.random.default_rng(6)
    B, Hq, Hk, T, Q = 2, 4, 2, 50, 3
    keys = rng.standard_normal((B * Hk * T, 128))
    enc = O.encode(codec3, keys)
    q = rng.standard_normal((B, Q, Hq, 128))
    out = O.attn_logits(codec3, q, enc, B, Hq, Hk, Q, T)
    b, h, qi = 1, 3, 2
    kh = h // (Hq // Hk)
    rows = slice((b * Hk + kh) * T, (b * Hk + kh + 1) * T)
    ref = O.score(codec3, q[b, qi, h], {k: enc[k][rows] for k in ("codes", "signs", "norm", "rnorm")})[0]
    assert np.allclose(out[b, h, qi], ref, rtol=1e-13, atol=1e-12)


# ---------------------------------------------------------------- O6 attention
def test_decode_attention_two_formulations_agree(codec3):
    rng = np.random.default_rng(9)
    B, Hq, Hk, T = 1, 4, 2, 257
    K = O.encode(codec3, rng.standard_normal((B * Hk * T, 128)))
    V = O.encode(codec3, rng.standard_normal((B * Hk * T, 128)))
    q = rng.standard_normal((B, Hq, 128))
    a = O.decode_attn_materialized(codec3, codec3, q, K, V, B, Hq, Hk, T, 1 / math.sqrt(128))
    b = O.decode_attn_accumulated(codec3, codec3, q, K, V, B, Hq, Hk, T, 1 / math.sqrt(128))
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))


def test_decode_attention_one_hot_and_uniform(codec3, codec4):
    rng = np.random.default_rng(10)
    T = 64
    keys = rng.standard_normal((T, 128))
    q = rng.standard_normal((1, 1, 128))
    K = O.encode(codec3, keys)
    V = O.encode(codec4, rng.standard_normal((T, 128)))
    vhat = O.dequantize(codec4, V)
    # one key with a huge norm dominates the softmax: output = that value
    lg = O.score(codec3, q[0], K)[0]
    j = int(np.argmax(lg))
    K1 = dict(K); K1["norm"] = K["norm"].copy(); K1["norm"][j] *= 1e4
    out = O.decode_attn_accumulated(codec3, codec4, q, K1, V, 1, 1, 1, T, 1.0)
    assert np.allclose(out[0, 0], vhat[j], rtol=1e-12, atol=1e-12)
    # identical keys: uniform weights, output = mean of the values
    Ku = O.encode(codec3, np.repeat(keys[:1], T, axis=0))
    out = O.decode_attn_materialized(codec3, codec4, q, Ku, V, 1, 1, 1, T, 1.0)
    assert np.allclose(out[0, 0], vhat.mean(axis=0), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- MSE-only value codec
@pytest.mark.parametrize("bits", [2, 3])
def test_mse_codec_record_and_codebook(bits):
    # all bits go to the Lloyd-Max code: d*bits/8 code bytes + 4 bytes of ν,
    # and the codebook is the b = bits Lloyd-Max quantizer (Appendix A values
    # at d = 128, scaled by sqrt(d))
    cd = O.make_mse_codec(128, bits)
    assert cd.b == bits and cd.m == 0 and cd.sign_words == 0
    assert cd.record_bytes == 128 * bits // 8 + 4
    expect = {2: [0.452453, 1.505193], 3: [0.244425, 0.753330, 1.336599, 2.131471]}[bits]
    assert np.allclose(cd.centroids[1 << (bits - 1):] * math.sqrt(128), expect, atol=2e-6)
    with pytest.raises(ValueError):
        O.score(cd, np.ones((1, 128)), O.encode(cd, np.ones((1, 128))))


@pytest.mark.parametrize("bits", [2, 3])
def test_mse_codec_distortion_equals_codebook_distortion(bits):
    # v̂ = ν Rᵀ c[idx]: for Gaussian x the mean of ||x/ν - v̂/ν||² is the
    # codebook's distortion d·E(X - Q(X))² (sphere law), with no QJL term
    cd = O.make_mse_codec(128, bits)
    x = np.random.default_rng(31).standard_normal((50_000, 128))
    enc = O.encode(cd, x)
    assert enc["signs"].shape == (x.shape[0], 0)
    vhat = O.dequantize(cd, enc)
    nu = np.linalg.norm(x, axis=1, keepdims=True)
    err = np.sum((x / nu - vhat / nu) ** 2, axis=1)
    D = _distortion_by_quadrature(cd.c32.astype(np.float64), cd.t32.astype(np.float64), 128)
    assert abs(err.mean() - D) < 3.5 * err.std() / math.sqrt(err.size)


@pytest.mark.parametrize("bits", [2, 3])
def test_mse_dequantize_basis_vector_closed_form(bits):
    # x = ν e_k: every |y_j| = 1/sqrt(d), so c[idx] = sqrt(d) c_level · y and
    # v̂ = ν Rᵀ c[idx] = ν sqrt(d) c_level e_k exactly (a transposed R fails this)
    cd = O.make_mse_codec(128, bits)
    x = np.zeros((1, 128)); x[0, 41] = 2.5
    vhat = O.dequantize(cd, O.encode(cd, x))[0]
    t = cd.t32.astype(np.float64) * math.sqrt(128)
    level = int(np.sum(t < 1.0))
    expect = np.zeros(128); expect[41] = 2.5 * math.sqrt(128) * float(cd.c32[level])
    assert np.allclose(vhat, expect, rtol=0, atol=1e-12)
    assert float(cd.c32[level]) * math.sqrt(128) == pytest.approx({2: 1.505193, 3: 0.753330}[bits], abs=2e-6)


def test_decode_attention_mse_values(codec3):
    rng = np.random.default_rng(12)
    B, Hq, Hk, T = 1, 4, 2, 200
    cv = O.make_mse_codec(128, 3)
    K = O.encode(codec3, rng.standard_normal((B * Hk * T, 128)))
    V = O.encode(cv, rng.standard_normal((B * Hk * T, 128)))
    q = rng.standard_normal((B, Hq, 128))
    a = O.decode_attn_materialized(codec3, cv, q, K, V, B, Hq, Hk, T, 1 / math.sqrt(128))
    b = O.decode_attn_accumulated(codec3, cv, q, K, V, B, Hq, Hk, T, 1 / math.sqrt(128))
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
    # one dominant key returns its v̂ = ν Rᵀ c[idx]
    vhat = O.dequantize(cv, V)
    lg = O.score(codec3, q[0, :1], {k: K[k][:T] for k in ("codes", "signs", "norm", "rnorm")})[0]
    j = int(np.argmax(lg))
    K1 = {k: np.array(K[k][:T]) for k in ("codes", "signs", "norm", "rnorm")}
    K1["norm"][j] *= 1e4
    V1 = {k: np.array(V[k][:T]) for k in ("codes", "signs", "norm", "rnorm")}
    out = O.decode_attn_accumulated(codec3, cv, q[:, :1], K1, V1, 1, 1, 1, T, 1.0)
    assert np.allclose(out[0, 0], vhat[j], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- O6b Sparse V
def _sparse_case(codec3, codec4, T, Hq, qscale, seed):
    rng = np.random.default_rng(seed)
    K = O.encode(codec3, rng.standard_normal((T, 128)))
    V = O.encode(codec4, rng.standard_normal((T, 128)))
    q = qscale * rng.standard_normal((1, Hq, 128))
    return K, V, q


def test_sparse_v_gate_zero_is_plain_attention(codec3, codec4):
    K, V, q = _sparse_case(codec3, codec4, 300, 2, 3.0, 21)
    ref = O.decode_attn_materialized(codec3, codec4, q, K, V, 1, 2, 1, 300, 1 / math.sqrt(128))
    out, keep, _ = O.decode_attn_sparse_v(codec3, codec4, q, K, V, 1, 2, 1, 300, 1 / math.sqrt(128), 0.0, 64)
    assert keep.all()
    assert np.array_equal(out, ref)


def test_sparse_v_one_chunk_is_softmax_threshold(codec3, codec4):
    # one chunk over the whole context: the gate is "softmax weight < gate",
    # with the weights from SciPy's softmax of the scaled scores
    from scipy import special
    T, Hq, gate = 300, 2, 1e-3
    K, V, q = _sparse_case(codec3, codec4, T, Hq, 3.0, 22)
    w = special.softmax(O.score(codec3, q[0], K) / math.sqrt(128), axis=-1)
    vhat = O.dequantize(codec4, V)
    out, keep, local = O.decode_attn_sparse_v(codec3, codec4, q, K, V, 1, Hq, 1, T, 1 / math.sqrt(128), gate, T)
    assert np.array_equal(keep[0], w >= gate)
    assert 0.1 < keep.mean() < 0.9                       # the case really gates
    assert not np.array_equal(keep[0, 0], keep[0, 1])    # per head
    assert np.allclose(local[0], w, rtol=1e-12, atol=0)
    ref = (w * keep[0]) @ vhat
    assert np.allclose(out[0], ref, rtol=1e-12, atol=1e-14)


def test_sparse_v_chunked_gate_is_conservative_and_bounded(codec3, codec4):
    from scipy import special
    T, Hq, gate = 1000, 2, 2e-3
    K, V, q = _sparse_case(codec3, codec4, T, Hq, 3.0, 23)
    w = special.softmax(O.score(codec3, q[0], K) / math.sqrt(128), axis=-1)
    vhat = O.dequantize(codec4, V)
    out, keep, local = O.decode_attn_sparse_v(codec3, codec4, q, K, V, 1, Hq, 1, T, 1 / math.sqrt(128), gate, 128)
    assert (~keep).sum() > 100
    assert np.all(local[0] >= w * (1 - 1e-12))           # chunk-local weight bounds the final one
    assert np.all(w[~keep[0]] < gate)                    # every dropped position is below the gate
    full = O.decode_attn_materialized(codec3, codec4, q, K, V, 1, Hq, 1, T, 1 / math.sqrt(128))
    dropped = (w * ~keep[0]) @ np.abs(vhat)              # per-coordinate bound on the dropped mass
    assert np.all(np.abs(full[0] - out[0]) <= dropped * (1 + 1e-9) + 1e-15)
    assert np.all(np.abs(full[0] - out[0]).max(axis=-1) <= gate * (~keep[0]).sum(axis=-1) * np.abs(vhat).max())


def test_sparse_v_gate_uses_the_chunk_maximum(codec3, codec4):
    # chunk 0 holds one dominant key; chunk 1 has no strong key, so its own
    # maximum keeps every one of its positions although their final weights
    # are negligible
    T, gate = 128, 1e-3
    K, V, q = _sparse_case(codec3, codec4, T, 1, 0.01, 24)
    j = int(np.argmax(O.score(codec3, q[0], K)[0, :64]))
    K = dict(K); K["norm"] = K["norm"].copy(); K["norm"][j] *= 1e4
    out, keep, _ = O.decode_attn_sparse_v(codec3, codec4, q, K, V, 1, 1, 1, T, 1.0, gate, 64)
    want = np.zeros(T, dtype=bool); want[j] = True; want[64:] = True
    assert np.array_equal(keep[0, 0], want)
    vhat = O.dequantize(codec4, V)
    assert np.allclose(out[0, 0], vhat[j], rtol=1e-12, atol=1e-12)


def test_sparse_v_plain_rule_is_the_final_weight_threshold(codec3, codec4):
    # the page's rule on its own terms: final softmax weight (SciPy's softmax
    # of the scaled scores) below the gate -> value term dropped, normaliser
    # unchanged; gate 0 is plain attention
    from scipy import special
    T, Hq, gate = 700, 4, 2e-3
    K, V, q = _sparse_case(codec3, codec4, T, Hq, 3.0, 31)
    scale = 1 / math.sqrt(128)
    w = special.softmax(O.score(codec3, q[0], K) * scale, axis=-1)
    vhat = O.dequantize(codec4, V)
    out, keep, wo = O.decode_attn_sparse_v_plain(codec3, codec4, q, K, V, 1, Hq, 2, T // 2, scale, 0.0)
    ref = O.decode_attn_materialized(codec3, codec4, q, K, V, 1, Hq, 2, T // 2, scale)
    assert keep.all() and np.allclose(out, ref, rtol=1e-12, atol=1e-15)
    out, keep, wo = O.decode_attn_sparse_v_plain(codec3, codec4, q, K, V, 1, Hq, 1, T, scale, gate)
    assert np.allclose(wo[0], w, rtol=1e-12, atol=0)
    assert np.array_equal(keep[0], w >= gate)
    assert 0.02 < keep.mean() < 0.9                      # the case really gates
    assert np.allclose(out[0], (w * (w >= gate)) @ vhat, rtol=1e-12, atol=1e-15)


def test_sparse_v_chunked_rule_bounds_the_plain_rule(codec3, codec4):
    # the chunk-local rule of the split kernels keeps a superset of the
    # plain rule's positions, equals it with one chunk over the context, and
    # moves the output by at most the dropped mass of the plain rule
    T, Hq, gate = 2000, 2, 1e-3
    K, V, q = _sparse_case(codec3, codec4, T, Hq, 3.0, 32)
    scale = 1 / math.sqrt(128)
    vhat = O.dequantize(codec4, V)
    plain, keep_p, w = O.decode_attn_sparse_v_plain(codec3, codec4, q, K, V, 1, Hq, 1, T, scale, gate)
    one, keep_1, _ = O.decode_attn_sparse_v(codec3, codec4, q, K, V, 1, Hq, 1, T, scale, gate, T)
    assert np.array_equal(keep_1, keep_p) and np.allclose(one, plain, rtol=1e-12, atol=1e-15)
    for chunk in (128, 256, 1024):
        out, keep_c, _ = O.decode_attn_sparse_v(codec3, codec4, q, K, V, 1, Hq, 1, T, scale, gate, chunk)
        assert np.all(keep_c | ~keep_p)                       # superset
        assert (keep_c & ~keep_p).any()                       # and a strict one here
        extra = (w[0] * (keep_c[0] & ~keep_p[0])) @ np.abs(vhat)
        assert np.allclose(out[0] - plain[0], (w[0] * (keep_c[0] & ~keep_p[0])) @ vhat, rtol=1e-9, atol=1e-15)
        assert np.all(np.abs(out[0] - plain[0]) <= extra * (1 + 1e-9) + 1e-15)
        bound = gate * (~keep_p[0]).sum(axis=-1) * np.abs(vhat).max()
        assert np.all(np.abs(out[0] - plain[0]).max(axis=-1) <= bound)


# ---------------------------------------------------------------- O6c paged cache
def test_paged_rows_closed_form_and_disjoint():
    # one KV head with the identity page table is the contiguous layout
    assert [O.paged_row([[0, 1, 2]], 0, 0, t, 1, 4) for t in range(12)] == list(range(12))
    # two sequences with disjoint pages: every (sequence, head, position) has its own row
    pt = [[3, 0], [1, 2]]
    rows = {O.paged_row(pt, b, kh, t, 2, 8) for b in range(2) for kh in range(2) for t in range(16)}
    assert rows == set(range(4 * 2 * 8))


def test_paged_decode_reduces_to_contiguous_and_ignores_page_order(codec3, codec4):
    rng = np.random.default_rng(41)
    P, T = 16, 40
    K = O.encode(codec3, rng.standard_normal((T, 128)))
    V = O.encode(codec4, rng.standard_normal((T, 128)))
    q = rng.standard_normal((1, 2, 128))
    ref = O.decode_attn_accumulated(codec3, codec4, q, K, V, 1, 2, 1, T, 0.1)
    ident = [[0, 1, 2]]
    assert np.array_equal(O.decode_attn_paged(codec3, codec4, q, K, V, ident, [T], 2, 1, P, 0.1), ref)
    # the same logical cache in shuffled physical pages (with junk in a spare page)
    perm = [4, 1, 3]
    def scatter(R):
        out = {k: np.zeros((5 * P,) + np.asarray(R[k]).shape[1:], dtype=np.asarray(R[k]).dtype) for k in R}
        for k in out:
            out[k][:] = np.asarray(R[k])[rng.integers(0, T, 5 * P)]
            for i, p in enumerate(perm):
                n = min(P, T - i * P)
                out[k][p * P:p * P + n] = np.asarray(R[k])[i * P:i * P + n]
        return out
    Kp, Vp = scatter(K), scatter(V)
    got = O.decode_attn_paged(codec3, codec4, q, Kp, Vp, [perm], [T], 2, 1, P, 0.1)
    assert np.array_equal(got, ref)
    # a shorter context reads only its first positions
    first = lambda R: {k: np.asarray(R[k])[:21] for k in ("codes", "signs", "norm", "rnorm")}
    short = O.decode_attn_accumulated(codec3, codec4, q, first(K), first(V), 1, 2, 1, 21, 0.1)
    assert np.array_equal(O.decode_attn_paged(codec3, codec4, q, Kp, Vp, [perm], [21], 2, 1, P, 0.1), short)
    # an empty context gives zeros
    assert np.all(O.decode_attn_paged(codec3, codec4, q, Kp, Vp, [perm], [0], 2, 1, P, 0.1) == 0)


def test_append_paged_round_trip(codec3):
    # appending token by token into pages, then gathering, equals encoding the rows at once
    rng = np.random.default_rng(42)
    hkv, P, steps = 2, 4, 11
    x = rng.standard_normal((2, hkv, steps, 128))
    pt = np.array([[5, 0, 7, 3], [2, 6, 1, 4]])
    cache = {"codes": np.zeros((8 * hkv * P, codec3.b * 4), np.uint32), "signs": np.zeros((8 * hkv * P, 4), np.uint32),
             "norm": np.zeros(8 * hkv * P, np.float32), "rnorm": np.zeros(8 * hkv * P, np.float32)}
    ctx = np.array([0, 3])
    for t in range(steps):
        O.append_paged(codec3, cache, x[:, :, t:t + 1], ctx, pt, P)
        ctx = ctx + 1
    for b, start in ((0, 0), (1, 3)):
        g = O.gather_paged(cache, pt, b, hkv, start + steps, P)
        want = O.encode(codec3, x[b].reshape(-1, 128))
        for key in ("codes", "signs", "norm", "rnorm"):
            got = np.asarray(g[key]).reshape((hkv, start + steps) + np.asarray(g[key]).shape[1:])[:, start:]
            assert np.array_equal(got.reshape(np.asarray(want[key]).shape), np.asarray(want[key], dtype=got.dtype))


def test_dequantize_unbiased_over_qjl_matrix():
    # E_S[v̂] = v for a fixed rotation
    d = 32
    base = O.make_codec(d, 3, seed=6)
    rng = np.random.default_rng(12)
    x = rng.standard_normal((1, d))
    acc = []
    for s in range(3000):
        cd = O.Codec(d=d, bits=3, m=d, seed=s, D=base.D, R=base.R,
                     S=O.gaussian_matrix(d, d, seed=50_000 + s),
                     centroids=base.centroids, bounds=base.bounds, iters=base.iters)
        acc.append(O.dequantize(cd, O.encode(cd, x))[0])
    acc = np.array(acc)
    se = acc.std(axis=0) / math.sqrt(acc.shape[0])
    assert np.all(np.abs(acc.mean(axis=0) - x[0]) < 4 * se)


# ---------------------------------------------------------------- O7 search
def test_search_topk_matches_brute_force_sort(codec3):
    rng = np.random.default_rng(13)
    db = O.encode(codec3, rng.standard_normal((500, 128)))
    # duplicate a record to create exact ties
    for k in ("codes", "signs", "norm", "rnorm"):
        db[k][7] = db[k][3]
    qs = rng.standard_normal((4, 128))
    idx, sc, full = O.search_topk(codec3, db, qs, 10, chunk=128)
    for qi in range(4):
        order = sorted(range(500), key=lambda i: (-full[qi, i], i))[:10]
        assert list(idx[qi]) == order
        assert np.array_equal(sc[qi], full[qi, order])


# ---------------------------------------------------------------- O8 PolarQuant first stage
def test_polar_transform_worked_cases():
    # d = 4 by hand: level-1 angles of (y0, y1), (y2, y3) in [0, 2π), then the
    # level-2 angle atan2(‖(y2, y3)‖, ‖(y0, y1)‖)
    ang, r = O.polar_transform(np.array([[1.0, 0, 0, 0], [0, 0, 0, 1.0], [-1.0, 0, 0, 0], [0, -1.0, 0, 0],
                                         [3.0, 4.0, 0, 12.0]]))
    two_pi = 2 * math.pi
    assert np.allclose(ang[0], [[0, 0], [0, math.pi / 2], [math.pi, 0], [1.5 * math.pi, 0],
                                [math.atan2(4, 3), math.pi / 2]])
    assert np.allclose(ang[1][:, 0], [0, math.pi / 2, 0, 0, math.atan2(12, 5)])
    assert np.allclose(r, [1, 1, 1, 1, 13])
    assert np.all((ang[0] >= 0) & (ang[0] < two_pi))


def test_polar_angle_laws_match_beta():
    # Monte Carlo: for Gaussian (hence uniform-direction) vectors the level-1
    # angles are uniform and, for level l > 1, sin²θ ~ Beta(n/2, n/2) with
    # n = 2^(l-1) (SciPy's beta distribution as the reference)
    from scipy import stats
    y = np.random.default_rng(61).standard_normal((20000, 64))
    ang, r = O.polar_transform(y)
    assert stats.kstest(ang[0].ravel() / (2 * math.pi), "uniform").pvalue > 1e-3
    for lv in range(2, 7):
        n = 1 << (lv - 1)
        s2 = np.sin(ang[lv - 1][:, 0]) ** 2
        assert stats.kstest(s2, stats.beta(n / 2, n / 2).cdf).pvalue > 1e-3, lv
    assert np.allclose(r, np.linalg.norm(y, axis=1))


def test_polar_density_and_cdf_consistent():
    from scipy import integrate
    for lv in range(2, 8):
        tot, _ = integrate.quad(lambda t: float(O.polar_angle_density(t, lv)), 0, math.pi / 2, points=[math.pi / 4])
        assert abs(tot - 1) < 1e-10
        for t in (0.3, 0.7, 0.8, 1.2):
            part, _ = integrate.quad(lambda u: float(O.polar_angle_density(u, lv)), 0, t, epsabs=1e-14)
            assert abs(part - float(O.polar_angle_cdf(t, lv))) < 1e-9


@pytest.mark.parametrize("b", [1, 2, 3])
def test_polar_lloyd_max_conditions(b):
    from scipy import integrate
    # level 1: the uniform quantizer of the circle
    c, t, _ = O.polar_lloyd_max(1, b)
    L = 1 << b
    assert np.allclose(c, (np.arange(L) + 0.5) * 2 * math.pi / L) and np.allclose(t, np.arange(1, L) * 2 * math.pi / L)
    for lv in (2, 4, 7):
        c, t, _ = O.polar_lloyd_max(lv, b)
        assert np.allclose(c + c[::-1], math.pi / 2, atol=1e-12)           # symmetric about π/4
        assert np.allclose(t, 0.5 * (c[:-1] + c[1:]))                       # nearest neighbour
        edges = np.concatenate([[0], t, [math.pi / 2]])
        f = lambda u: float(O.polar_angle_density(u, lv))
        for k in range(L):                                                  # centroid condition
            m0, _ = integrate.quad(f, edges[k], edges[k + 1], epsabs=0, epsrel=1e-12, limit=200)
            m1, _ = integrate.quad(lambda u: u * f(u), edges[k], edges[k + 1], epsabs=0, epsrel=1e-12, limit=200)
            assert abs(m1 / m0 - c[k]) < 1e-9


def test_polar_reconstruction_closed_form_and_unit_norm():
    pc = O.make_polar_codec(4, 3, seed=7)
    # slots: level-1 angles at 0, 1; the level-2 angle at 2; slot 3 unused
    idx = np.array([[1, 3, 2, 0]])
    y = O.polar_reconstruct(pc.cos32, pc.sin32, [idx[:, 0:2], idx[:, 2:3]])
    a, b0, b1 = pc.centroids[1][2], pc.centroids[0][1], pc.centroids[0][3]
    want = [math.cos(a) * math.cos(b0), math.cos(a) * math.sin(b0), math.sin(a) * math.cos(b1), math.sin(a) * math.sin(b1)]
    assert np.allclose(y[0], want, atol=1e-7)
    assert O.polar_slots(128) == [(0, 64), (64, 96), (96, 112), (112, 120), (120, 124), (124, 126), (126, 127)]
    pc = O.make_polar_codec(128, 3, seed=7)
    rnd = np.random.default_rng(62).integers(0, 4, (50, 128))
    rec = {"codes": O.pack_planes(rnd, 2), "signs": np.zeros((50, 4), np.uint32),
           "norm": np.ones(50, np.float32), "rnorm": np.zeros(50, np.float32)}
    # ν = 1, γ = 0: the reconstruction is Rᵀ ŷ, whose norm is ‖ŷ‖
    assert np.allclose(np.linalg.norm(O.polar_dequantize(pc, rec), axis=1), 1, atol=1e-6)


def test_polar_slots_and_unit_norm_other_head_dims():
    # level l's d/2^l angles sit in [d - d/2^(l-1), d - d/2^l); the last slot is unused
    for d in (64, 256):
        L = int(math.log2(d))
        assert O.polar_slots(d) == [(d - (d >> (l - 1)), d - (d >> l)) for l in range(1, L + 1)]
        pc = O.make_polar_codec(d, 3, seed=7)
        assert pc.levels == L and pc.record_bytes == 4 * (2 * d // 32 + d // 32) + 8
        rnd = np.random.default_rng(d).integers(0, 4, (40, d))
        rec = {"codes": O.pack_planes(rnd, 2), "signs": np.zeros((40, d // 32), np.uint32),
               "norm": np.ones(40, np.float32), "rnorm": np.zeros(40, np.float32)}
        assert np.allclose(np.linalg.norm(O.polar_dequantize(pc, rec), axis=1), 1, atol=1e-6)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_polar_encode_picks_nearest_angle(d):
    pc = O.make_polar_codec(d, 4, seed=7)
    e = O.polar_encode(pc, np.random.default_rng(63).standard_normal((200, d)))
    for lv, (lo, hi) in enumerate(O.polar_slots(d), start=1):
        th = e["angles"][lv - 1]
        c = pc.centroids[lv - 1]
        dist = np.abs(th[:, :, None] - c[None, None, :])
        if lv == 1:
            dist = np.minimum(dist, 2 * math.pi - dist)
        assert np.array_equal(e["idx"][:, lo:hi], np.argmin(dist, axis=2)), lv
    assert np.all(e["idx"][:, d - 1] == 0)


def test_polar_score_unbiased_and_matches_dequantize():
    d = 32
    base = O.make_polar_codec(d, 3, seed=5)
    rng = np.random.default_rng(64)
    x = rng.standard_normal((1, d)) * 2.0
    q = rng.standard_normal((1, d))
    e = O.polar_encode(base, x)
    assert np.allclose(O.polar_score(base, q, e), q @ O.polar_dequantize(base, e).T, rtol=1e-12, atol=1e-12)
    vals = []
    for s in range(4000):
        pc = O.PolarCodec(d=d, bits=3, m=d, seed=s, D=base.D, R=base.R, S=O.gaussian_matrix(d, d, seed=20_000 + s),
                          centroids=base.centroids, bounds=base.bounds, iters=base.iters)
        vals.append(float(O.polar_score(pc, q, O.polar_encode(pc, x))[0, 0]))
    vals = np.array(vals)
    assert abs(vals.mean() - float((q @ x.T)[0, 0])) < 3.5 * vals.std() / math.sqrt(vals.size)


def _dense_attention(qh, khat, vhat, scale):
    """softmax(scale · q k̂ᵀ) v̂ for one KV group, in plain dense fp64 algebra."""
    s = scale * (qh @ khat.T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)) @ vhat


@pytest.mark.parametrize("kpolar,vpolar", [(True, True), (False, True), (True, False)])
def test_polar_decode_attention_is_dense_attention_over_reconstructions(kpolar, vpolar):
    # Either codec with the recursive polar first stage: both formulations of
    # decode attention (materialized v̂, and M/J accumulated in the rotated
    # and QJL domains) equal dense attention over the dequantized keys and
    # values, the logits taken as plain dot products q·k̂ (the score's
    # unbiased form equals ⟨q, k̂⟩ exactly).
    d, batch, hq, hkv, ctx = 32, 2, 4, 2, 9
    ck = O.make_polar_codec(d, 3, seed=21) if kpolar else O.make_codec(d, 3, seed=21)
    cv = O.make_polar_codec(d, 3, seed=22) if vpolar else O.make_codec(d, 3, seed=22)
    rng = np.random.default_rng(8)
    k = rng.standard_normal((batch * hkv * ctx, d)) * 1.5
    v = rng.standard_normal((batch * hkv * ctx, d))
    q = rng.standard_normal((batch, hq, d))
    enc = lambda c, x: O.polar_encode(c, x) if isinstance(c, O.PolarCodec) else O.encode(c, x)
    kr, vr = enc(ck, k), enc(cv, v)
    khat, vhat = O.dequantize(ck, kr), O.dequantize(cv, vr)
    scale = 0.4
    a = O.decode_attn_materialized(ck, cv, q, kr, vr, batch, hq, hkv, ctx, scale)
    b = O.decode_attn_accumulated(ck, cv, q, kr, vr, batch, hq, hkv, ctx, scale)
    G = hq // hkv
    for bi in range(batch):
        for kh in range(hkv):
            rows = slice((bi * hkv + kh) * ctx, (bi * hkv + kh + 1) * ctx)
            hs = slice(kh * G, (kh + 1) * G)
            ref = _dense_attention(q[bi, hs], khat[rows], vhat[rows], scale)
            assert np.allclose(a[bi, hs], ref, rtol=1e-10, atol=1e-12)
            assert np.allclose(b[bi, hs], ref, rtol=1e-10, atol=1e-12)
    # one position: the output is that value's reconstruction, whatever the query
    one = O.decode_attn_accumulated(ck, cv, q[:1, :2], {x: kr[x][:1] for x in ("codes", "signs", "norm", "rnorm")},
                                    {x: vr[x][:1] for x in ("codes", "signs", "norm", "rnorm")}, 1, 2, 1, 1, scale)
    assert np.allclose(one[0], np.repeat(vhat[:1], 2, axis=0), rtol=1e-12, atol=1e-12)
    # the gated oracle at gate 0 is the plain one
    g0, keep, _ = O.decode_attn_sparse_v(ck, cv, q, kr, vr, batch, hq, hkv, ctx, scale, 0.0, 4)
    assert keep.all() and np.allclose(g0, b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- bf16 rounding helper
def _bf16_nearest(x32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to bfloat16 from its definition: of the two
    bfloat16 neighbours of each fp32 value (truncation and the next value
    away from zero; 2^128 stands for the overflow step), take the nearer in
    exact fp64 arithmetic, ties to the even significand, then map 2^128 to
    Inf.  Independent of the bit trick the oracle uses."""
    out = np.empty_like(x32)
    for i, v in enumerate(x32):
        if np.isnan(v) or np.isinf(v):
            out[i] = v
            continue
        u = int(np.float32(v).view(np.uint32))
        sign, mag = u & 0x80000000, u & 0x7FFFFFFF
        lo = mag & 0xFFFF0000
        hi = lo + 0x10000
        a = float(np.uint32(lo).view(np.float32))
        b = 2.0 ** 128 if hi == 0x7F800000 else float(np.uint32(hi).view(np.float32))
        m = abs(float(v))
        if m - a < b - m or (m - a == b - m and (lo >> 16) % 2 == 0):
            r = lo
        else:
            r = hi
        out[i] = np.uint32(sign | r).view(np.float32)
    return out


def test_bf16_round_pinned_to_definition_and_torch():
    torch = pytest.importorskip("torch")
    f = np.float32
    one = 1.0
    cases = [0.0, -0.0, one, -one,
             one + 2.0 ** -8,                 # tie between 1 and 1 + 2^-7: even is 1
             one + 3 * 2.0 ** -8,             # tie: even is 1 + 2^-6
             one + 2.0 ** -8 + 2.0 ** -23,    # just above the tie
             one + 2.0 ** -8 - 2.0 ** -23,    # just below
             -(one + 2.0 ** -8),
             2.0 ** -126, 2.0 ** -130,        # fp32 normal minimum, subnormal
             2.0 ** -133 * 3,                 # bf16 subnormal tie region
             2.0 ** -149, -2.0 ** -149,       # fp32 smallest subnormal
             2.0 ** -140 * 1.5,
             float(np.finfo(np.float32).max),  # rounds up to Inf
             3.3895313892515355e38,           # bfloat16 max, exact
             3.3961775292304958e38,           # just below the overflow tie: stays finite
             float("inf"), float("-inf"), float("nan")]
    rng = np.random.default_rng(5)
    rnd = np.concatenate([rng.standard_normal(4000), rng.standard_normal(2000) * 1e-39, rng.standard_normal(2000) * 1e37,
                          rng.integers(-(2 ** 20), 2 ** 20, 2000) * 2.0 ** -16])  # many exact ties
    x32 = np.array(cases + list(rnd), dtype=np.float64).astype(f)
    got = O.bf16_round(x32)
    want = _bf16_nearest(x32)
    tch = torch.from_numpy(x32.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(x32)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(np.isnan(tch), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    assert np.array_equal(got[~nan].view(np.uint32), tch[~nan].view(np.uint32))
    assert np.isposinf(got[x32 == np.finfo(np.float32).max]).all()
    assert got[4] == 1.0 and got[5] == 1.0 + 2.0 ** -6           # ties to even
    assert np.signbit(got[1]) and got[1] == 0.0                  # -0 stays -0
    # fp64 inputs round to fp32 first (RNE), as torch does for double -> bfloat16
    x64 = np.concatenate([rnd, [1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8 - 2.0 ** -30]])
    g64 = O.bf16_round(x64)
    t64 = torch.from_numpy(x64.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(g64.view(np.uint32), t64.view(np.uint32))
    assert np.array_equal(g64.view(np.uint32), _bf16_nearest(x64.astype(f)).view(np.uint32))


# ---------------------------------------------------------------- O7b value records in 32-row blocks
def _one_bit_record(n, b, row, plane, j):
    """Row records (O4 layout) with a single bit set: plane `plane` (b = the
    sign plane) of coordinate j in row `row`."""
    rec = {"codes": np.zeros((n, 4 * b), np.uint32), "signs": np.zeros((n, 4), np.uint32),
           "norm": np.arange(n, dtype=np.float32), "rnorm": -np.arange(n, dtype=np.float32)}
    if plane < b:
        rec["codes"][row, 4 * plane + j // 32] = np.uint32(1) << np.uint32(j % 32)
    else:
        rec["signs"][row, j // 32] = np.uint32(1) << np.uint32(j % 32)
    return rec


@pytest.mark.parametrize("b,row,plane,j,array,word,bit", [
    # row 9 = 8*1 + 1 (r 1, i 1 -> bit 4*1 + 1); coordinate 17 = 16*1 + 1 (c 1, n 1 -> word 8 + 1);
    # plane 1 of block 0 with b = 2 -> codes word (0*2 + 1)*128 + 9
    (2, 9, 1, 17, "codes", 137, 5),
    # row 63: block 1, tau 31 = 8*3 + 7 -> bit 31; coordinate 127 = 16*7 + 15 -> word 127; sign plane
    (2, 63, 2, 127, "signs", 255, 31),
    # row 32: block 1, tau 0 -> bit 0; coordinate 0 -> word 0; plane 0 of b = 3 -> (1*3 + 0)*128
    (3, 32, 0, 0, "codes", 384, 0),
    # row 2 (i 2, r 0 -> bit 8); coordinate 16 (c 1, n 0 -> word 1); plane 2 of b = 3 -> 2*128 + 1
    (3, 2, 2, 16, "codes", 257, 8),
    # row 24 (r 3, i 0 -> bit 3); coordinate 31 (c 1, n 15 -> word 121); plane 0
    (1, 24, 0, 31, "codes", 121, 3),
])
def test_vblock_single_bits_land_where_the_layout_puts_them(b, row, plane, j, array, word, bit):
    # hand-computed positions of single bits under the block layout
    n = 64
    blk = O.vblock_pack(_one_bit_record(n, b, row, plane, j), b)
    flat = blk[array].reshape(-1)
    assert int(flat[word]) == 1 << bit
    assert np.count_nonzero(blk["codes"]) + np.count_nonzero(blk["signs"]) == 1
    assert np.array_equal(blk["norm"], np.arange(n, dtype=np.float32))


@pytest.mark.parametrize("b,qjl", [(1, True), (2, True), (3, True), (2, False), (3, False)])
def test_vblock_round_trip_and_bit_count(b, qjl):
    # a permutation of the bits: unpack inverts pack, and popcounts agree per block and plane
    rng = np.random.default_rng(b + 10 * qjl)
    n = 96
    rec = {"codes": rng.integers(0, 2 ** 32, (n, 4 * b), dtype=np.uint64).astype(np.uint32),
           "signs": (rng.integers(0, 2 ** 32, (n, 4), dtype=np.uint64).astype(np.uint32) if qjl
                     else np.zeros((n, 0), np.uint32)),
           "norm": rng.random(n).astype(np.float32), "rnorm": rng.random(n).astype(np.float32)}
    blk = O.vblock_pack(rec, b)
    assert blk["codes"].shape == rec["codes"].shape and blk["signs"].shape == rec["signs"].shape
    back = O.vblock_unpack(blk, b)
    for k in rec:
        assert np.array_equal(back[k], rec[k]), k
    pc = lambda a: np.unpackbits(np.ascontiguousarray(a).view(np.uint8)).sum()
    for B_ in range(n // 32):
        for p in range(b):
            assert pc(rec["codes"][32 * B_:32 * B_ + 32, 4 * p:4 * p + 4]) == pc(blk["codes"].reshape(-1)[
                (B_ * b + p) * 128:(B_ * b + p + 1) * 128])
