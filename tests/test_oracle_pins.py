"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code: printed values from the pages
(tests/golden), closed forms, invariants, brute force with NumPy's int64 matmul, and exact
rational arithmetic (tests/exact.py).  None of them needs a GPU.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import exact
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- weight quantization
def test_worked_example_alpha_codes_and_byte():
    g = _golden("worked_example.json")
    w = np.array([g["W"]], np.float32)
    codes, packed, alpha = oracle.quantize_weights(w)
    # alpha printed as 0.6125: the fp32 nearest to it (relative error < 2e-8).
    assert abs(float(alpha) - g["alpha"]) / g["alpha"] < 1e-7
    assert np.float32(alpha).view(np.uint32) == np.float32(0.6125).view(np.uint32)
    # W / alpha printed with 2-3 decimals
    q = w[0] / alpha
    for v, p, d in zip(q, g["w_over_alpha_printed"], g["printed_decimals"]):
        assert abs(float(v) - p) <= 0.5 * 10 ** (-d) + 1e-6
    # round before clip, then clip
    assert [int(v) for v in np.rint(q)] == g["rounded_before_clip"]
    assert codes[0].tolist() == g["codes"]
    assert float((codes == 0).mean()) == g["zero_fraction"]
    assert packed.shape == (1, 1) and int(packed[0, 0]) == g["packed_byte"]


def test_tie_vectors_round_half_even():
    g = _golden("tie_vectors.json")
    for case in g["weights"]:
        w = np.array([case["W"]], np.float32)
        codes, packed, alpha = oracle.quantize_weights(w)
        assert float(alpha) == case["alpha"]
        assert codes[0].tolist() == case["codes"]
        assert int(packed[0, 0]) == case["packed_byte"]


def test_constant_magnitude_gives_sign():
    rs = np.random.default_rng(7)
    for c in (0.02, 1.0, 3.5):
        w = (rs.choice([-1.0, 1.0], size=(8, 16)) * c).astype(np.float32)
        codes, _, alpha = oracle.quantize_weights(w)
        assert float(alpha) == np.float32(c)
        assert np.array_equal(codes, np.sign(w).astype(np.int8))


def test_all_zero_weights_give_zero_codes():
    w = np.zeros((4, 8), np.float32)
    codes, packed, alpha = oracle.quantize_weights(w)
    assert float(alpha) == 0.0
    assert not codes.any()
    assert np.all(packed == 0x55)


def test_codes_match_exact_rational_pipeline():
    for seed in range(3):
        w = (np.random.default_rng(seed).standard_normal((16, 32)) * 0.02).astype(np.float32)
        codes, _, alpha = oracle.quantize_weights(w)
        a = exact.absmean_exact(w)
        assert exact.fr(alpha) == a
        assert np.array_equal(codes, exact.codes_exact(w, a))


def test_codes_are_ternary_and_zero_fraction_matches_gaussian_closed_form():
    w = workloads.weights(1, 1024, 1024)
    codes, _, alpha = oracle.quantize_weights(w)
    assert set(np.unique(codes).tolist()) <= {-1, 0, 1}
    # zero iff |W| < alpha/2 with alpha ~= E|W| = sigma*sqrt(2/pi): P = erf(0.5*sqrt(2/pi)/sqrt(2))
    p0 = math.erf(0.5 * math.sqrt(2 / math.pi) / math.sqrt(2))
    assert abs(p0 - 0.3101) < 1e-4
    assert abs(float((codes == 0).mean()) - p0) < 3e-3
    # and inside the 30-50% the pages quote for the naive demo ([P3] section 4.3)
    assert 0.30 <= float((codes == 0).mean()) <= 0.50
    assert abs(float(alpha) - 0.02 * math.sqrt(2 / math.pi)) < 2e-4


def test_per_row_alpha_matches_per_tensor_on_each_row():
    w = workloads.weights(1, 8, 64)
    rows = oracle.absmean_rows(w)
    for n in range(8):
        assert exact.fr(rows[n]) == exact.absmean_exact(w[n])
        assert np.array_equal(oracle.ternarize_rows(w, rows)[n], oracle.ternarize(w[n], rows[n]))


# ---------------------------------------------------------------- packing
def test_packing_density_closed_forms():
    g = _golden("memory_estimate.json")
    # 2 bits per weight: N*K/4 bytes; 64 weights fill one 128-bit register ([P3] section 5.3)
    codes = np.zeros((1, 64), np.int8)
    assert oracle.pack(codes).nbytes == 16
    n, k = 7, 1024
    assert oracle.pack(np.zeros((n, k), np.int8)).nbytes == n * k // 4
    gib = 1024 ** 3
    p = g["params"]
    assert round(p * 2 / gib, 2) == g["printed_gb"]["fp16"]
    assert round(p * 0.5 / gib, 2) == g["printed_gb"]["int4"]
    bytes_per_weight = oracle.pack(np.zeros((1, 4096), np.int8)).nbytes / 4096
    assert round(p * bytes_per_weight / gib, 2) == g["printed_gb"]["ternary_2bit"]


def test_pack_unpack_roundtrip_and_bad_pattern():
    rs = np.random.default_rng(3)
    codes = rs.integers(-1, 2, size=(5, 36)).astype(np.int8)
    packed = oracle.pack(codes)
    assert np.array_equal(oracle.unpack(packed, 36), codes)
    # brute-force layout: byte b of row n holds k=4b+i at bits 2i
    for nn in range(5):
        for b in range(9):
            expect = sum((int(codes[nn, 4 * b + i]) + 1) << (2 * i) for i in range(4))
            assert packed[nn, b] == expect
    bad = packed.copy()
    bad[2, 3] |= 0b11000000
    with pytest.raises(ValueError):
        oracle.unpack(bad, 36)


# ---------------------------------------------------------------- activation quantization
def test_activation_tie_vector():
    g = _golden("tie_vectors.json")["activations"][0]
    xq, beta = oracle.quantize_act(np.array([g["x"]], np.float32))
    assert float(beta[0]) == g["beta"]
    assert xq[0].tolist() == g["xq"]


def test_activation_matches_exact_rational_pipeline():
    x = workloads.activations_with_outliers(4, 3, 512)
    xq, beta = oracle.quantize_act(x)
    xq_e, beta_e = exact.quantize_act_exact(x)
    assert [exact.fr(b) for b in beta] == beta_e
    assert np.array_equal(xq, xq_e)


def test_activation_invariants_and_error_bound():
    x = workloads.activations_with_outliers(4, 16, 1024)
    xq, beta = oracle.quantize_act(x)
    assert np.abs(xq.astype(np.int32)).max() <= 127
    for m in range(16):
        j = int(np.argmax(np.abs(x[m])))
        assert abs(int(xq[m, j])) == 127 and np.sign(xq[m, j]) == np.sign(x[m, j])
        # beta == max|x| exactly once max|x| >= 0.25 (the 1e-8 guard vanishes in fp32)
        assert beta[m] == np.abs(x[m]).max()
        err = np.abs(x[m].astype(np.float64) - beta[m] * xq[m].astype(np.float64) / 127.0)
        assert err.max() <= beta[m] / 254.0 * (1 + 1e-5)


def test_activation_zero_row():
    xq, beta = oracle.quantize_act(np.zeros((2, 8), np.float32))
    assert beta[0] == np.float32(1e-8)
    assert not xq.any()


# ---------------------------------------------------------------- integer matmul
@pytest.mark.parametrize("m,n,k", [(1, 1, 4), (3, 5, 16), (4, 7, 36), (2, 16, 64)])
def test_matmul_brute_force_against_int64_dense(m, n, k):
    rs = np.random.default_rng(m * 100 + n * 10 + k)
    xq = rs.integers(-127, 128, size=(m, k)).astype(np.int8)
    codes = rs.integers(-1, 2, size=(n, k)).astype(np.int8)
    acc = oracle.ternary_matmul(xq, codes)
    ref = xq.astype(np.int64) @ codes.astype(np.int64).T
    assert np.array_equal(acc, ref)


@pytest.mark.parametrize("k", [4, 8])
def test_matmul_exhaustive_weight_rows(k):
    rows = np.array(np.meshgrid(*[[-1, 0, 1]] * k, indexing="ij")).reshape(k, -1).T
    codes = np.ascontiguousarray(rows.astype(np.int8))
    rs = np.random.default_rng(k)
    xq = rs.integers(-127, 128, size=(3, k)).astype(np.int8)
    acc = oracle.ternary_matmul(xq, codes)
    for m in range(3):
        ref = [sum(int(xq[m, j]) * int(r[j]) for j in range(k)) for r in rows]
        assert acc[m].tolist() == ref


def test_matmul_extreme_magnitude_no_overflow():
    k = 11008
    xq = np.full((1, k), 127, np.int8)
    codes = np.ones((2, k), np.int8)
    codes[1] = -1
    acc = oracle.ternary_matmul(xq, codes)
    assert acc[0].tolist() == [127 * k, -127 * k]


def test_matmul_row_range():
    rs = np.random.default_rng(11)
    xq = rs.integers(-127, 128, size=(2, 32)).astype(np.int8)
    codes = rs.integers(-1, 2, size=(9, 32)).astype(np.int8)
    full = oracle.ternary_matmul(xq, codes)
    part = np.full((2, 9), -7, np.int32)
    oracle.ternary_matmul(xq, codes, 3, 7, out=part)
    assert np.array_equal(part[:, 3:7], full[:, 3:7])
    assert np.all(part[:, :3] == -7) and np.all(part[:, 7:] == -7)


# ---------------------------------------------------------------- dequant epilogue
def test_dequant_scale_unit_and_exact():
    acc = np.array([[0, 1, -5, 3641344]], np.int32)
    y = oracle.dequant(acc, np.array([1.0], np.float32), alpha=127.0)
    assert np.array_equal(y, acc.astype(np.float32))
    rs = np.random.default_rng(5)
    acc = rs.integers(-400000, 400000, size=(3, 6)).astype(np.int32)
    beta = rs.uniform(0.5, 60, size=3).astype(np.float32)
    alpha = np.float32(0.0159)
    y = oracle.dequant(acc, beta, alpha)
    ye = exact.dequant_exact(acc, [exact.fr(b) for b in beta], exact.fr(alpha))
    assert np.array_equal(y, ye)


def test_dequant_bias_and_per_row_alpha():
    acc = np.array([[10, -20, 30]], np.int32)
    beta = np.array([127.0], np.float32)
    ar = np.array([1.0, 2.0, 0.5], np.float32)
    y = oracle.dequant(acc, beta, alpha_rows=ar, bias=np.array([0.5, 0.25, -1.0], np.float32))
    assert y[0].tolist() == [10.5, -39.75, 14.0]


def test_forward_identity_approximates_float_product():
    """[P3] section 2.5: x.W^T ~= (beta*alpha/127) (x_q . W_hat^T).  For Gaussian W the
    approximation has cosine similarity ~0.887 (the pages' 'usually > 0.9' is a soft claim);
    checked as a band, not for parity."""
    w = workloads.weights(1, 512, 1024)
    x = workloads.activations(1, 32, 1024)
    r = oracle.bitlinear(x, w)
    y_fp = x.astype(np.float64) @ w.astype(np.float64).T
    y = r["y"].astype(np.float64).reshape(-1)
    cos = float(y @ y_fp.reshape(-1) / np.linalg.norm(y) / np.linalg.norm(y_fp))
    assert 0.86 < cos < 0.92
    # the integer part is exact: acc equals the int64 product of the quantized operands
    ref = r["xq"].astype(np.int64) @ r["codes"].astype(np.int64).T
    assert np.array_equal(r["acc"], ref)


def test_forward_composes_unpack_matmul_dequant():
    w = workloads.weights(1, 24, 64)
    x = workloads.activations(1, 3, 64)
    r = oracle.bitlinear(x, w)
    acc, y = oracle.forward(r["xq"], r["beta"], r["packed"], 64, r["alpha"])
    assert np.array_equal(acc, r["acc"]) and np.array_equal(y, r["y"])


def _neighbours32(v: float, span: int):
    """fp32 values within ``span`` ulps of fp32(v)."""
    c = np.float32(v)
    out = [c]
    lo = hi = c
    for _ in range(span):
        lo = np.nextafter(lo, np.float32(-np.inf), dtype=np.float32)
        hi = np.nextafter(hi, np.float32(np.inf), dtype=np.float32)
        out += [lo, hi]
    return out


def test_activation_division_order_at_rounding_boundaries():
    """Inputs where fp32(fp32(127*x)/beta) and fp32(x*fp32(127/beta)) round to different
    integers, found with exact arithmetic; the oracle must follow the division order the
    pages' code writes (x * 127.0 / beta)."""
    beta = Fraction(3)
    recip = exact.rne32(Fraction(127) / beta)
    picked = []
    for kk in range(0, 127):
        for v in _neighbours32(float((kk + 0.5) * 3 / 127), 6):
            f = exact.fr(v)
            t_div = exact.rne32(exact.rne32(f * 127) / beta)
            t_rec = exact.rne32(f * recip)
            if exact.round_half_even_int(t_div) != exact.round_half_even_int(t_rec):
                picked.append(v)
    assert len(picked) >= 8
    row = np.array([[3.0] + picked + [-v for v in picked]], np.float32)
    xq, beta_o = oracle.quantize_act(row)
    xq_e, _ = exact.quantize_act_exact(row)
    assert float(beta_o[0]) == 3.0
    assert np.array_equal(xq, xq_e)


def test_ternary_division_order_at_rounding_boundaries():
    """Weights next to alpha/2 where fp32(W/alpha) and fp32(W*fp32(1/alpha)) round to
    different codes, found with exact arithmetic over many alphas; the oracle must divide
    as the pages' code does (weight / alpha)."""
    rs = np.random.default_rng(21)
    pairs = []
    for alpha in rs.uniform(0.005, 0.05, size=300).astype(np.float32):
        a = exact.fr(alpha)
        recip = exact.rne32(1 / a)
        for v in _neighbours32(float(alpha) / 2, 2):
            f = exact.fr(v)
            q_div = exact.round_half_even_int(exact.rne32(f / a))
            q_rec = exact.round_half_even_int(exact.rne32(f * recip))
            if q_div != q_rec:
                pairs.append((v, alpha))
    assert len(pairs) >= 4
    for v, alpha in pairs:
        w = np.array([v, -v], np.float32)
        assert np.array_equal(oracle.ternarize(w, alpha), exact.codes_exact(w, exact.fr(alpha)))


def test_dequant_scale_precision_where_fp32_would_differ():
    """Pairs (alpha, beta) for which a pure-fp32 alpha*beta/127 differs from the fp64 scale
    the pages' code computes (Python floats), found with exact arithmetic."""
    rs = np.random.default_rng(33)
    alpha = np.float32(0.0159)
    a = exact.fr(alpha)
    betas = []
    for b in rs.uniform(1.0, 60.0, size=400).astype(np.float32):
        bb = exact.fr(b)
        s64 = exact.dequant_scale_exact(a, bb)
        s32 = exact.rne32(exact.rne32(a * bb) / 127)
        if s64 != s32:
            betas.append(b)
    assert len(betas) >= 4
    betas = np.array(betas, np.float32)
    acc = np.full((len(betas), 1), 1, np.int32)
    y = oracle.dequant(acc, betas, alpha)
    for i, b in enumerate(betas):
        assert exact.fr(y[i, 0]) == exact.dequant_scale_exact(a, exact.fr(b))
        assert exact.fr(oracle.dequant_scale(alpha, b)) == exact.dequant_scale_exact(a, exact.fr(b))


# ---------------------------------------------------------------- rotation before absmax
# [P3 §6.2]: a randomized Hadamard rotation of x (and the same of W) before absmax.
# Readings R10/R11: blocks of B along K, sign flip first, Sylvester butterflies with
# stride 1, 2, ..., B/2 in fp32, one fp32 multiply by fp32(1/sqrt(B)) last.
def _sylvester(b):
    """Textbook closed form of the Sylvester Hadamard matrix: H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(b)
    bits = np.bitwise_and.outer(i, i)
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def _rotate_dense_f64(x, block, signs):
    """x . diag(d) . blockdiag(H_B / sqrt(B)) in fp64 (matrix form, no butterflies)."""
    m, k = x.shape
    d = np.ones(k) if signs is None else signs.astype(np.float64)
    h = _sylvester(block) / math.sqrt(block)
    xs = x.astype(np.float64) * d
    return (xs.reshape(m, k // block, block) @ h).reshape(m, k)


@pytest.mark.parametrize("block", [1, 2, 4, 8, 16, 32, 64, 256])
def test_hadamard_matches_dense_matrix_within_fp32_bound(block):
    k = 3 * block if block > 1 else 5
    x = workloads.activations_with_outliers(7, 4, k)
    d = workloads.rotation_signs(7, k)
    got = oracle.hadamard_rows(x, block, d).astype(np.float64)
    want = _rotate_dense_f64(x, block, d)
    # log2(B) rounded additions on each path, a rounded scale and a rounded product
    levels = int(round(math.log2(block)))
    mag = np.abs(x.astype(np.float64)).reshape(4, k // block, block).sum(axis=2) / math.sqrt(block)
    bound = np.repeat(mag, block, axis=1) * (levels + 2) * 2.0 ** -24 * 1.001
    assert np.all(np.abs(got - want) <= bound + 1e-30)


@pytest.mark.parametrize("block", [2, 8, 64, 512])
def test_hadamard_rounding_matches_recursive_definition_bitwise(block):
    """H_2n [a; b] = [H_n a + H_n b; H_n a - H_n b] evaluated recursively in fp32 (numpy
    float32 arithmetic), then the fp32 scale: the same roundings as R11 stride order."""
    def rec(v):
        if v.shape[-1] == 1:
            return v
        n = v.shape[-1] // 2
        a, b = rec(v[..., :n]), rec(v[..., n:])
        return np.concatenate([a + b, a - b], axis=-1)

    x = workloads.activations(8, 3, 2 * block)
    v = x.reshape(3, 2, block)
    want = (rec(v) * np.float32(1.0 / math.sqrt(block))).reshape(3, 2 * block).astype(np.float32)
    got = oracle.hadamard_rows(x, block)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("block", [4, 16, 64, 256])
def test_hadamard_is_an_exact_involution_on_small_integers(block):
    """For B a power of 4 the scale is 2^-j, so small integers rotate without rounding and
    H (H x) = x (H symmetric and orthonormal)."""
    g = np.random.default_rng(11)
    x = g.integers(-50, 51, size=(3, 2 * block)).astype(np.float32)
    once = oracle.hadamard_rows(x, block)
    assert np.array_equal(oracle.hadamard_rows(once, block), x)


@pytest.mark.parametrize("block", [2, 16, 128])
def test_hadamard_unit_vectors_give_scaled_rows(block):
    h = _sylvester(block)
    s = np.float32(1.0 / math.sqrt(block))
    for i in (0, 1, block // 2, block - 1):
        e = np.zeros((1, block), np.float32)
        e[0, i] = 4.0
        got = oracle.hadamard_rows(e, block)[0]
        assert np.array_equal(got, (np.float32(4.0) * h[i].astype(np.float32)) * s)


def test_hadamard_constant_block_concentrates_in_first_output():
    x = np.full((1, 64), 3.0, np.float32)
    got = oracle.hadamard_rows(x, 64)[0]
    assert got[0] == np.float32(3.0 * 64 / 8) and not got[1:].any()


def test_hadamard_signs_apply_before_the_transform_and_block_one_is_the_sign_flip():
    x = workloads.activations(9, 2, 96)
    d = workloads.rotation_signs(9, 96)
    flipped = np.where(d < 0, -x, x).astype(np.float32)
    assert np.array_equal(oracle.hadamard_rows(x, 32, d), oracle.hadamard_rows(flipped, 32))
    assert np.array_equal(oracle.hadamard_rows(x, 1, d), flipped)
    assert np.array_equal(oracle.hadamard_rows(x, 1), x)


def test_hadamard_preserves_norms_and_products():
    """R R^T = I: row norms and x . W^T survive the rotation up to fp32 rounding."""
    k, block = 768, 256
    x = workloads.activations_with_outliers(10, 4, k)
    w = workloads.weights(10, 6, k)
    d = workloads.rotation_signs(10, k)
    xr = oracle.hadamard_rows(x, block, d).astype(np.float64)
    wr = oracle.hadamard_rows(w, block, d).astype(np.float64)
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    assert np.allclose((xr ** 2).sum(1), (x64 ** 2).sum(1), rtol=1e-5, atol=0)
    ref = x64 @ w64.T
    scale = np.abs(x64) @ np.abs(w64).T
    assert np.all(np.abs(xr @ wr.T - ref) <= 2e-5 * scale)


def test_hadamard_rejects_bad_blocks():
    x = np.zeros((1, 24), np.float32)
    with pytest.raises(ValueError):
        oracle.hadamard_rows(x, 3)
    with pytest.raises(ValueError):
        oracle.hadamard_rows(x, 16)


def test_rotation_spreads_an_outlier_and_cuts_the_quantization_error():
    """[P3 §6.2]: one large channel inflates beta and crushes the rest to 0; after the
    rotation its energy is spread, beta falls, and the dequantized activations track the
    float ones (and the float product) more closely."""
    k, block = 1024, 256
    x = workloads.activations(12, 8, k) * np.float32(0.05)
    x[:, 17] = np.float32(40.0)
    w = workloads.weights(12, 64, k)
    d = workloads.rotation_signs(12, k)
    xq, beta = oracle.quantize_act(x)
    xq_r, beta_r = oracle.quantize_act_hadamard(x, block, d)
    assert np.all(beta_r < beta / 4)
    x64 = x.astype(np.float64)
    xr64 = oracle.hadamard_rows(x, block, d).astype(np.float64)
    wr64 = oracle.hadamard_rows(w, block, d).astype(np.float64)
    deq = xq * (beta[:, None] / 127.0)
    deq_r = xq_r * (beta_r[:, None] / 127.0)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(deq_r, xr64) < rel(deq, x64) / 4
    ref = x64 @ w.astype(np.float64).T
    assert rel(deq_r @ wr64.T, ref) < rel(deq @ w.astype(np.float64).T, ref) / 4


# ---------------------------------------------------------------- block scales (R12)
# [P1 §2.3, §4.2]: one scale per 128 consecutive weights of a row, shape [C_out, C_in/128].
def _block_weights(seed, n, k):
    """W ~ N(0, 0.02) with a different magnitude per 128-block, so block scales matter."""
    g = np.random.default_rng(seed)
    w = g.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)
    gain = np.exp(g.uniform(np.log(0.05), np.log(5.0), size=(n, k // 128))).astype(np.float32)
    return (w * np.repeat(gain, 128, axis=1)).astype(np.float32)


def test_block_alpha_is_the_exact_mean_of_each_block():
    w = _block_weights(21, 5, 384)
    w[2, 128:256] = 0.0                                              # an all-zero block
    a = oracle.absmean_blocks(w)
    assert a.shape == (5, 3)
    for n in range(5):
        for b in range(3):
            assert exact.fr(a[n, b]) == exact.absmean_exact(w[n, 128 * b:128 * b + 128])
    assert a[2, 1] == 0


def test_block_codes_use_their_own_block_scale():
    w = _block_weights(22, 4, 256)
    w[1, :128] = 0.0
    a = oracle.absmean_blocks(w)
    codes = oracle.ternarize_blocks(w, a)
    for n in range(4):
        for b in range(2):
            blk = slice(128 * b, 128 * b + 128)
            assert np.array_equal(codes[n, blk], exact.codes_exact(w[n, blk], exact.fr(a[n, b])))
    assert not codes[1, :128].any()                                  # alpha = 0 -> codes 0 (R3)
    # a block scale differs from the row scale where magnitudes vary: the codes differ too
    row_codes = oracle.ternarize_rows(w, oracle.absmean_rows(w))
    assert (row_codes != codes).any()


def test_block_sums_brute_force_and_total():
    g = np.random.default_rng(23)
    xq = g.integers(-127, 128, size=(3, 384)).astype(np.int8)
    codes = g.integers(-1, 2, size=(7, 384)).astype(np.int8)
    acc = oracle.ternary_matmul_blocks(xq, codes)
    want = np.einsum("mbk,nbk->mnb", xq.reshape(3, 3, 128).astype(np.int64),
                     codes.reshape(7, 3, 128).astype(np.int64))
    assert np.array_equal(acc, want)
    assert np.array_equal(acc.sum(axis=2), oracle.ternary_matmul(xq, codes))


def test_block_dequant_within_one_rounding_of_the_exact_value():
    g = np.random.default_rng(24)
    m, n, kb = 3, 9, 5
    acc = g.integers(-127 * 128, 127 * 128 + 1, size=(m, n, kb)).astype(np.int32)
    acc[0, 0] = 0
    a = (g.uniform(0.001, 0.05, size=(n, kb))).astype(np.float32)
    a[3, 2] = 0.0
    beta = g.uniform(0.5, 30.0, size=m).astype(np.float32)
    bias = g.standard_normal(n).astype(np.float32)
    y = oracle.dequant_blocks(acc, beta, a)
    yb = oracle.dequant_blocks(acc, beta, a, bias)
    same = 0
    for i in range(m):
        t = exact.fr(beta[i]) / 127
        for j in range(n):
            s = sum((exact.fr(a[j, b]) * int(acc[i, j, b]) for b in range(kb)), Fraction(0))
            want = exact.rne32(s * t)
            got = exact.fr(y[i, j])
            ulp = abs(float(want)) * 2.0 ** -23 if want != 0 else 2.0 ** -149
            assert abs(float(got - want)) <= ulp
            same += got == want
            assert yb[i, j] == np.float32(y[i, j] + bias[j])
    assert y[0, 0] == 0.0
    assert same >= m * n - 1


def test_block_forward_matches_dense_float64_product():
    """y = (x_q . (alpha_b W_hat)^T) beta/127 with the block-scaled weights dequantized."""
    w = _block_weights(25, 6, 512)
    x = workloads.activations(25, 3, 512)
    r = oracle.bitlinear_blocks(x, w)
    wdq = r["codes"].astype(np.float64) * np.repeat(r["alpha_blocks"].astype(np.float64), 128, axis=1)
    ref = (r["xq"].astype(np.float64) @ wdq.T) * (r["beta"].astype(np.float64)[:, None] / 127.0)
    scale = (np.abs(r["xq"].astype(np.float64)) @ np.abs(wdq).T) * (r["beta"].astype(np.float64)[:, None] / 127.0)
    assert np.all(np.abs(r["y"] - ref) <= np.abs(ref) * 2.0 ** -23 + scale * 1e-14)
    acc2, y2 = oracle.forward_blocks(r["xq"], r["beta"], r["packed"], 512, r["alpha_blocks"])
    assert np.array_equal(acc2, r["acc_blocks"]) and np.array_equal(y2, r["y"])


def test_block_scales_track_blockwise_magnitudes_better_than_one_scale():
    """[P1 §2.3]: a scale per 128 weights follows weights whose magnitude changes along K."""
    w = _block_weights(26, 64, 1024)
    x = workloads.activations(26, 4, 1024)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = lambda y: np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel(oracle.bitlinear_blocks(x, w)["y"]) < 0.75 * rel(oracle.bitlinear(x, w)["y"])   # 0.52 vs 0.79


def test_block_functions_reject_k_not_a_multiple_of_128():
    with pytest.raises(ValueError):
        oracle.absmean_blocks(np.zeros((2, 192), np.float32))


# ---------------------------------------------------------------- BitMLP (R13)
# Values of the standard normal CDF (textbook tables give their leading digits): GELU(x) =
# x * Phi(x).  The tail entries reach the range where 1 + erf(x / sqrt 2) has cancelled away
# (x <= -8.3 in fp64) and where GELU is an fp32 subnormal (x = -14).
# `test_phi_table_from_the_series` recomputes every entry from the series of erf.
PHI = {0.5: "0.691462461274013103637704610608", 1.0: "0.841344746068542948585232545632",
       2.0: "0.977249868051820792799717362834", 3.0: "0.998650101968369905473348185232",
       -1.0: "0.158655253931457051414767454368", -2.0: "0.022750131948179207200282637166",
       -4.0: "3.16712418331199212537707567222e-5", -6.0: "9.86587645037698140700864132398e-10",
       -8.0: "6.22096057427178412351599517259e-16", -10.0: "7.61985302416052606597334325160e-24",
       -12.0: "1.77648211207767899769617100185e-33", -14.0: "7.79353681919280025435968183890e-45"}


def _phi_series(x, digits=160):
    """Phi(x) = (1 + erf(x / sqrt 2)) / 2 in decimal arithmetic with `digits` digits, erf from its
    Maclaurin series 2/sqrt(pi) sum_n (-1)^n z^(2n+1) / (n! (2n+1)) and pi from the
    Gauss-Legendre iteration.  The working precision covers the cancellation of the series
    (terms up to e^(z^2), 43 digits at z = 14 / sqrt 2) and of 1 + erf."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = digits
        a, b, t, p = Decimal(1), 1 / Decimal(2).sqrt(), Decimal(1) / 4, Decimal(1)
        for _ in range(12):
            an = (a + b) / 2
            b, t, p, a = (a * b).sqrt(), t - p * (a - an) ** 2, 2 * p, an
        pi = (a + b) ** 2 / (4 * t)
        z = Decimal(x) / Decimal(2).sqrt()
        s, term, n, tiny = Decimal(0), z, 0, Decimal(10) ** (-digits + 10)
        while True:
            add = term / (2 * n + 1)
            s += add
            if n > 8 and abs(add) < tiny:
                break
            n += 1
            term = -term * z * z / n
        return (1 + 2 * s / pi.sqrt()) / 2


def test_phi_table_from_the_series():
    from decimal import Decimal
    for x, v in PHI.items():
        got = _phi_series(x)
        assert abs(got - Decimal(v)) <= Decimal(v) * Decimal("1e-28"), (x, got, v)
    # the leading digits printed in standard normal tables
    assert str(PHI[-6.0]).startswith("9.8658764") and str(PHI[-8.0]).startswith("6.2209605")


def test_gelu_matches_normal_cdf_table():
    from decimal import Decimal
    xs = np.array(sorted(PHI), np.float32)
    g = oracle.gelu(xs)
    for x, v in zip(xs, g):
        want = exact.rne32(Fraction(Decimal(PHI[float(x)])) * exact.fr(x))
        assert exact.fr(v) == want


def test_gelu_tail_is_not_flushed():
    """Below about -5.5 the terms of 1 + erf(x / sqrt 2) cancel in fp64, yet GELU(x) = x Phi(x)
    is a nonzero fp32 number down to x = -14.5.  On 20001 points of [-14, -4] the oracle is
    negative, falls as x falls (GELU decreases left of its minimum at -0.75), and lies within
    two fp32 ulps (or 2^-148 absolute) of x Phi(x) from the asymptotic normal tail
    Phi(x) ~ phi(x)/|x| (1 - 1/x^2 + 3/x^4 - 15/x^6), whose relative error is below the first
    omitted term 105/x^8 (1.6e-3 at x = -4, 6e-6 at x = -8)."""
    import math
    xs = np.linspace(-14.0, -4.0, 20001).astype(np.float32)
    g = oracle.gelu(xs).astype(np.float64)
    assert np.all(g < 0.0)
    x64 = xs.astype(np.float64)
    pdf = np.exp(-0.5 * x64 * x64) / math.sqrt(2.0 * math.pi)
    inv2 = 1.0 / (x64 * x64)
    tail = pdf / np.abs(x64) * (1.0 - inv2 + 3.0 * inv2 ** 2 - 15.0 * inv2 ** 3)
    approx = x64 * tail
    bound = 105.0 * inv2 ** 4 * np.abs(approx) + 2 * np.abs(approx) * 2.0 ** -23 + 2.0 ** -148
    assert np.all(np.abs(g - approx) <= bound)
    # monotone: GELU increases on (-inf, -0.75], so it decreases as x goes down
    assert np.all(np.diff(g) <= 0.0)


def test_gelu_odd_part_identity_and_limits():
    """Phi(x) + Phi(-x) = 1, so GELU(x) - GELU(-x) = x; GELU(0) = 0; GELU(10) = 10."""
    x = np.linspace(-6, 6, 2001).astype(np.float32)
    gp, gm = oracle.gelu(x).astype(np.float64), oracle.gelu(-x).astype(np.float64)
    ulp = np.maximum(np.abs(gp), np.abs(gm)) * 2.0 ** -23
    assert np.all(np.abs(gp - gm - x) <= 2 * ulp + 2.0 ** -149)
    assert oracle.gelu(np.array([0.0, 10.0], np.float32)).tolist() == [0.0, 10.0]
    # the minimum of GELU is about -0.16997 near x = -0.7518
    xs = np.linspace(-1.5, 0.0, 30001).astype(np.float32)
    gs = oracle.gelu(xs)
    assert abs(float(xs[np.argmin(gs)]) + 0.7518) < 2e-3 and abs(float(gs.min()) + 0.16997) < 1e-4


def test_bitmlp_tracks_the_float_mlp():
    """[P3 §6.1]: the BitMLP follows the float MLP it replaces (cosine > 0.75 for Gaussian
    weights of std 0.02 and N(0, 1) inputs)."""
    d, f = 512, 2048
    w1 = workloads.weights(40, f, d)
    w2 = workloads.weights(41, d, f)
    x = workloads.activations(40, 8, d)
    r = oracle.bitmlp(x, w1, w2)
    h = x.astype(np.float64) @ w1.astype(np.float64).T
    from math import erf, sqrt
    ref = (0.5 * h * (1.0 + np.vectorize(erf)(h / sqrt(2.0)))) @ w2.astype(np.float64).T
    cos = (r["y"].astype(np.float64) * ref).sum() / (np.linalg.norm(r["y"]) * np.linalg.norm(ref))
    assert cos > 0.75
    assert np.array_equal(r["g"], oracle.gelu(r["fc1"]["y"]))
    assert np.array_equal(r["fc2"]["xq"], oracle.quantize_act(r["g"])[0])


# ---------------------------------------------------------------- 5 trits per byte (R14)
def test_t5_every_trit_tuple_has_its_own_byte():
    """All 3^5 = 243 code tuples pack to the distinct bytes 0..242, in base-3 order."""
    import itertools
    tuples = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8)[:, ::-1]   # trit 0 fastest
    packed = oracle.pack_t5(tuples.reshape(1, -1)[:, :5 * 243])
    got = packed[0, :243]
    want = np.array([sum((int(c) + 1) * 3 ** i for i, c in enumerate(t)) for t in tuples])
    assert np.array_equal(got, want) and sorted(got.tolist()) == list(range(243))
    assert np.array_equal(oracle.unpack_t5(packed, 5 * 243), tuples.reshape(1, -1))


def test_t5_hand_value_padding_and_density():
    # W_hat = +1, 0, -1, +1, 0 -> c = 2, 1, 0, 2, 1 -> 2 + 3 + 0 + 54 + 81 = 140
    p = oracle.pack_t5(np.array([[1, 0, -1, 1, 0, -1]], np.int8))
    assert p.shape == (1, 16)
    assert p[0, 0] == 140
    assert p[0, 1] == 0 + 3 + 9 + 27 + 81          # weight -1, then four padded weights 0
    assert np.all(p[0, 2:] == 121)                 # bytes with no weight left
    assert oracle.t5_row_bytes(4096) == 832 and oracle.t5_row_bytes(11008) == 2208   # vs 1024, 2752
    assert oracle.t5_row_bytes(80) == 16 and oracle.t5_row_bytes(81) == 32


@pytest.mark.parametrize("k", [1, 4, 5, 79, 80, 81, 203, 4096])
def test_t5_round_trip(k):
    g = np.random.default_rng(k)
    codes = g.integers(-1, 2, size=(3, k)).astype(np.int8)
    assert np.array_equal(oracle.unpack_t5(oracle.pack_t5(codes), k), codes)
    bad = oracle.pack_t5(codes)
    bad[1, 0] = 243
    with pytest.raises(ValueError):
        oracle.unpack_t5(bad, k)


def test_t5_forward_equals_the_2bit_forward():
    """The packing changes bytes, not the product: same acc and y as the 2-bit layout."""
    w = workloads.weights(45, 37, 1000)
    x = workloads.activations(45, 3, 1000)
    codes, packed, alpha = oracle.quantize_weights(w)
    xq, beta = oracle.quantize_act(x)
    acc2, y2 = oracle.forward(xq, beta, packed, 1000, alpha)
    acc5, y5 = oracle.forward_t5(xq, beta, oracle.pack_t5(codes), 1000, alpha)
    assert np.array_equal(acc2, acc5) and np.array_equal(y2, y5)
