"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Bar: packed bytes, x_q, beta and int32 acc bit-exact; alpha within 1e-6 relative (bit-exact
expected) with zero code flips; y within 1e-5 relative (bit-exact expected).  Shapes span
several tiles with ragged tails; the full-size workloads are checked on every output in the
launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest

import oracle
import par_oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bitlinear_matmul_absmean_amd as bl
    return torch, bl


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _to(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _rel_ok(y, ref, tol=1e-5):
    y = y.astype(np.float64)
    ref = ref.astype(np.float64)
    return np.all(np.abs(y - ref) <= tol * np.abs(ref))


# ------------------------------------------------------------------ activation quantization
ACT_CASES = [(1, 1024), (1, 4096), (1, 11008), (3, 28672), (64, 4096), (17, 1000), (2, 6), (5, 4100),
             # one-pass kernel (K <= 32768, K % 4 == 0) with 1..8 float4 per thread, 1024 threads
             # per token, or 256 from 256 tokens with K <= 8192; the two-pass loop beyond
             (1, 32768), (1, 32772), (255, 12), (256, 8192), (300, 4100), (257, 8196), (40, 28676)]


@pytest.mark.parametrize("m,k", ACT_CASES)
def test_quantize_act_parity(dev, m, k):
    torch, bl = dev
    _say(f"quantize_act M={m} K={k}")
    x = workloads.activations_with_outliers(4, m, k)
    xq_o, beta_o = oracle.quantize_act(x)
    xq, beta = bl.bitlinear_quantize_act(_to(torch, x))
    torch.cuda.synchronize()
    assert np.array_equal(beta.cpu().numpy().view(np.uint32), beta_o.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_o)


def test_quantize_act_prefill_full_size(dev):
    torch, bl = dev
    _say("quantize_act prefill M=2048 K=4096 with outliers")
    x = workloads.activations_with_outliers(4, 2048, 4096)
    xq_o, beta_o = oracle.quantize_act(x)
    xq, beta = bl.bitlinear_quantize_act(_to(torch, x))
    torch.cuda.synchronize()
    assert np.array_equal(beta.cpu().numpy(), beta_o)
    assert np.array_equal(xq.cpu().numpy(), xq_o)


def test_quantize_act_ties_and_zero_rows(dev):
    torch, bl = dev
    x = np.zeros((3, 8), np.float32)
    x[0, :6] = [127.0, 0.5, 1.5, -2.5, 2.5, -127.0]
    x[2] = np.linspace(-3, 3, 8, dtype=np.float32)
    xq_o, beta_o = oracle.quantize_act(x)
    xq, beta = bl.bitlinear_quantize_act(_to(torch, x))
    torch.cuda.synchronize()
    assert np.array_equal(beta.cpu().numpy(), beta_o)
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert xq.cpu().numpy()[0, :6].tolist() == [127, 0, 2, -2, 2, -127]


# ------------------------------------------------------------------ weight quantization
W_CASES = [(1024, 1024), (4096, 4096), (11008, 4096), (4096, 11008), (1000, 1028), (3, 4), (7, 12), (65, 64)]


def _flips(w, alpha_gpu, alpha_o, packed_gpu, packed_o, k):
    """Count code mismatches and those that sit within 2 ulp of a rounding boundary."""
    cg = oracle.unpack(packed_gpu, k)
    co = oracle.unpack(packed_o, k)
    bad = np.argwhere(cg != co)
    boundary = 0
    for n, j in bad[:1000]:
        q = np.float32(w[n, j]) / np.float32(alpha_o)
        frac = abs(abs(float(q)) - 0.5)
        if frac <= 2 * np.spacing(np.float32(0.5)) or abs(abs(float(q)) - 1.5) <= 2 * np.spacing(np.float32(1.5)):
            boundary += 1
    return len(bad), boundary


@pytest.mark.parametrize("n,k", W_CASES)
def test_quantize_weights_parity(dev, n, k):
    torch, bl = dev
    _say(f"quantize_weights N={n} K={k}")
    w = workloads.weights(2, n, k)
    _, packed_o, alpha_o = oracle.quantize_weights(w)
    packed, alpha = bl.bitlinear_quantize_weights(_to(torch, w))
    torch.cuda.synchronize()
    a = float(alpha.cpu().numpy()[0])
    assert abs(a - float(alpha_o)) <= 1e-6 * abs(float(alpha_o))
    pg = packed.cpu().numpy()
    flips, boundary = _flips(w, a, alpha_o, pg, packed_o, k)
    assert flips == 0 and boundary == 0, (flips, boundary)
    assert np.array_equal(pg, packed_o)
    assert np.float32(a).view(np.uint32) == np.float32(alpha_o).view(np.uint32)


def test_quantize_weights_special_cases(dev):
    torch, bl = dev
    cases = [np.array([[0.9, -0.3, 0.05, -1.2]], np.float32),           # worked example
             np.array([[3.0, 0.5, -0.5, 0.0]], np.float32),             # ties at .5
             np.zeros((5, 8), np.float32),                              # alpha = 0
             np.full((4, 16), -0.02, np.float32)]                       # constant magnitude
    for w in cases:
        n, k = w.shape
        _, packed_o, alpha_o = oracle.quantize_weights(w)
        packed, alpha = bl.bitlinear_quantize_weights(_to(torch, w))
        torch.cuda.synchronize()
        assert np.array_equal(packed.cpu().numpy(), packed_o), w
        assert alpha.cpu().numpy()[0] == alpha_o
    assert packed_o is not None


@pytest.mark.parametrize("n,k", [(1024, 1024), (11008, 4096), (33, 68)])
def test_quantize_weights_rows_parity(dev, n, k):
    torch, bl = dev
    w = workloads.weights(2, n, k, index=1)
    ar_o = oracle.absmean_rows(w)
    packed_o = oracle.pack(oracle.ternarize_rows(w, ar_o))
    packed, ar = bl.bitlinear_quantize_weights_rows(_to(torch, w))
    torch.cuda.synchronize()
    assert np.array_equal(ar.cpu().numpy(), ar_o)
    assert np.array_equal(packed.cpu().numpy(), packed_o)


# ------------------------------------------------------------------ forward
def _random_operands(m, k, n, seed):
    rs = np.random.default_rng(seed)
    xq = rs.integers(-127, 128, size=(m, k)).astype(np.int8)
    codes = rs.choice(np.array([-1, 0, 1], np.int8), size=(n, k), p=[0.345, 0.31, 0.345])
    beta = rs.uniform(2.0, 60.0, size=m).astype(np.float32)
    alpha = np.float32(rs.uniform(0.015, 0.017))
    return xq, codes, oracle.pack(codes), beta, alpha


FWD_CASES = [
    (1, 64, 1), (1, 1024, 1024), (1, 4096, 100), (2, 4096, 257), (3, 11008, 130), (4, 128, 4096),
    (5, 64, 7), (8, 4096, 300), (16, 1024, 64), (17, 4096, 129), (33, 192, 65), (64, 11008, 70),
    (65, 1024, 130), (128, 256, 256), (130, 4096, 200), (300, 128, 257),
    (64, 4160, 33), (7, 28672, 20), (40, 2048, 300), (16, 16448, 65), (2, 32832, 17), (63, 320, 1000),
    (200, 4160, 130), (129, 192, 300), (1000, 128, 70), (96, 11008, 514),
    # the GEMM's 128-token tiles (more than 128 of them: two rounds, 129 ragged, exactly 256),
    # ragged in M and N; 64-token tiles below (the smaller prefill cases above)
    (1100, 128, 24577), (1030, 256, 2100), (300, 192, 11000), (2048, 640, 4096),
    (1, 100, 33), (6, 4100, 65), (70, 12, 9),      # K % 64 != 0: generic kernel
    # one token, the launch shapes of the decode GEMV (x_q given): 4-wave workgroups for rows of
    # one and of three chunks per lane, 8-wave ones otherwise, one to several rows per wave;
    # ragged N
    (1, 4096, 4096), (1, 4096, 11008), (1, 12288, 4097), (1, 4096, 16385), (1, 16384, 2048),
    (1, 28672, 2100), (1, 8192, 2048),
    # two to four tokens: two on the GEMV (matrices of 2^26 weights or more, or K >= 8192), three
    # and four on the MFMA decode kernel
    (2, 16384, 4100), (4, 8192, 8200), (3, 4096, 16400), (2, 8192, 1000), (2, 11008, 4099), (3, 16384, 4200),
    # batched decode with K % 256 != 0: 16x16x64 tiles with 1/2/4/8 row blocks per workgroup and
    # one or two token blocks, 32x32x32 tiles with 1/2; K % 256 = 64 and K % 128 = 64 tails;
    # ragged N
    (12, 128, 17000), (16, 192, 5000), (9, 4160, 700), (24, 320, 4100),
    (32, 64, 8300), (20, 4352, 300), (48, 192, 8200), (64, 4160, 600), (41, 128, 33),
    # 17-32 tokens on 32x32x32 tiles with one token block (K % 256 != 0, K <= 8192, N >= 8192):
    # 1, 2 and 4 row blocks per workgroup, K % 128 = 64
    (17, 192, 8192), (24, 1088, 9000), (32, 1344, 20000),
    # up to 32 tokens with whole 256-weight sub-steps (K % 256 == 0), two-stage pipeline: one
    # 16-row block per workgroup (N <= 4096), sub-step counts per wave below, at and above two,
    # ragged N and M
    (5, 256, 33), (16, 4096, 4096), (9, 11008, 1000), (12, 8192, 257), (16, 768, 4095),
    (17, 11008, 700), (32, 2048, 4096), (25, 256, 64),
    # ... and 2 to 8 row blocks per workgroup (the fewest that keep the grid within 256
    # workgroups; beyond N = 32768, with more workgroups, 8 for one token block and 7 for two),
    # one and two token blocks; token counts not a multiple of the 4 rows one x_q line load covers
    (8, 256, 9000), (8, 256, 8000), (3, 512, 12001), (12, 256, 16300), (7, 512, 20000),
    (16, 256, 24500), (10, 768, 28672), (5, 256, 40000),
    (24, 512, 8100), (32, 256, 11008), (20, 256, 16001), (28, 256, 17000), (31, 512, 21000),
    (18, 256, 25000), (32, 256, 33000), (24, 4096, 11008), (16, 8192, 10240),
    (29, 512, 40000), (13, 1280, 3000), (19, 2304, 12000), (2, 256, 5000),
    # 33-64 tokens with whole 256-weight sub-steps on at most 768 16-row blocks: three 16-token
    # tiles (33-48 tokens) and four (49-64) with one, two and three row blocks per workgroup, the
    # largest N that takes them and the next one (back to 32x32x32 tiles)
    (33, 256, 100), (48, 512, 4100), (40, 768, 12000), (49, 256, 1000), (64, 512, 8000),
    (57, 1024, 12288), (64, 256, 12289),
    # 33-64 tokens with whole 128-weight sub-steps (K % 128 == 0): one row block per workgroup
    # up to N = 8192, two beyond; sub-step counts not divisible by the eight waves (K = 128:
    # seven waves idle; K = 1152: 9 sub-steps), odd per-wave counts, ragged N and M
    (33, 128, 8193), (64, 1152, 8200), (40, 4096, 300), (64, 11008, 4100), (57, 384, 8191),
    (64, 640, 12345), (35, 2176, 33), (64, 1024, 8192), (48, 256, 30000),
    # 17-64 tokens with whole 256-weight sub-steps on at most 768 16-row blocks (x_q and codes
    # loaded into LDS, codes in weight order): two, three and four 16-token tiles with one, two
    # and three row blocks per workgroup; one sub-step (seven idle waves), sub-step counts not
    # divisible by the eight waves, token counts not a multiple of the four tokens one load
    # instruction covers, ragged N, the largest N of each row-block count and the next one
    (17, 256, 4096), (31, 2304, 4097), (33, 1280, 8192), (47, 512, 8193), (49, 3328, 12288),
    (64, 2816, 12289), (62, 768, 5), (18, 4608, 300), (41, 11008, 1030), (63, 4096, 4099),
    # ... and 4-16 tokens on one 16-token tile: one, two and three row blocks, the largest N of
    # three (768 blocks) and the next one (back to the register-staged kernel)
    (4, 256, 4096), (5, 2304, 4097), (11, 1280, 8192), (16, 512, 12288), (13, 768, 12289),
    (4, 11008, 999), (15, 4096, 63),
    # ... and 33-64 tokens on at most 256 16-row blocks as two 32-token halves of the grid: one
    # and two row blocks per workgroup, a second half of one token, ragged N
    (64, 4096, 4096), (35, 2304, 2049), (33, 11008, 2048), (57, 512, 4000), (48, 1280, 4095),
]


@pytest.mark.parametrize("m,k,n", FWD_CASES)
def test_forward_parity(dev, m, k, n):
    torch, bl = dev
    kern = bl.bitlinear_forward_kernel(m, k, n)
    _say(f"forward M={m} K={k} N={n} kernel={kern}")
    xq, codes, packed, beta, alpha = _random_operands(m, k, n, seed=m * 7919 + k * 31 + n)
    acc_o = oracle.ternary_matmul(xq, codes)
    y_o = oracle.dequant(acc_o, beta, alpha)
    y, acc = bl.bitlinear_forward(_to(torch, xq), _to(torch, beta), _to(torch, packed),
                                  _to(torch, np.array([alpha], np.float32)), acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    yg = y.cpu().numpy()
    assert _rel_ok(yg, y_o)
    assert np.array_equal(yg, y_o)


@pytest.mark.parametrize("m,k,n", [(1, 4096, 64), (12, 1024, 96), (200, 128, 70)])
def test_forward_bias_and_rows(dev, m, k, n):
    torch, bl = dev
    xq, codes, packed, beta, alpha = _random_operands(m, k, n, seed=5)
    rs = np.random.default_rng(9)
    bias = rs.standard_normal(n).astype(np.float32)
    ar = rs.uniform(0.01, 0.02, size=n).astype(np.float32)
    acc_o = oracle.ternary_matmul(xq, codes)
    y_o = oracle.dequant(acc_o, beta, alpha, bias=bias)
    yr_o = oracle.dequant(acc_o, beta, alpha_rows=ar, bias=bias)
    args = (_to(torch, xq), _to(torch, beta), _to(torch, packed))
    y = bl.bitlinear_forward(*args, _to(torch, np.array([alpha], np.float32)), bias=_to(torch, bias))
    yr = bl.bitlinear_forward_rows(*args, _to(torch, ar), bias=_to(torch, bias))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_o)
    assert np.array_equal(yr.cpu().numpy(), yr_o)


# Row ranges longer than one step of the decode GEMV (two register buffers in turn), with
# per-row alpha and a bias, whose loads travel with each step's weight rows: (M, K, N, call).
@pytest.mark.parametrize("m,k,n,call", [(1, 8192, 30000, "forward"), (1, 28672, 5000, "forward"),
                                        (2, 8192, 8200, "forward"), (1, 8192, 30000, "fused")])
def test_forward_rows_bias_multistep(dev, m, k, n, call):
    torch, bl = dev
    _say(f"{call} rows+bias M={m} K={k} N={n}")
    xq, codes, packed, beta, alpha = _random_operands(m, k, n, seed=11)
    rs = np.random.default_rng(12)
    bias = rs.standard_normal(n).astype(np.float32)
    ar = rs.uniform(0.01, 0.02, size=n).astype(np.float32)
    if call == "fused":
        x = workloads.activations(12, m, k)
        xq, beta = oracle.quantize_act(x)
        assert bl.bitlinear_forward_fused_kernel(m, k, n, _to(torch, x)) == "gemv_fused"
    else:
        assert bl.bitlinear_forward_kernel(m, k, n) == "gemv_dot4"
    acc_o = oracle.ternary_matmul(xq, codes)
    yr_o = oracle.dequant(acc_o, beta, alpha_rows=ar, bias=bias)
    y_o = oracle.dequant(acc_o, beta, alpha, bias=bias)
    pk, art, bt = _to(torch, packed), _to(torch, ar), _to(torch, bias)
    if call == "fused":
        yr = bl.bitlinear_forward_fused_rows(_to(torch, x), pk, art, bias=bt)
        y = bl.bitlinear_forward_fused(_to(torch, x), pk, _to(torch, np.array([alpha], np.float32)), bias=bt)
    else:
        args = (_to(torch, xq), _to(torch, beta), pk)
        yr = bl.bitlinear_forward_rows(*args, art, bias=bt)
        y = bl.bitlinear_forward(*args, _to(torch, np.array([alpha], np.float32)), bias=bt)
    torch.cuda.synchronize()
    assert np.array_equal(yr.cpu().numpy(), yr_o)
    assert np.array_equal(y.cpu().numpy(), y_o)


def test_forward_extreme_values(dev):
    """|acc| = 127*K at the largest workload K, and every weight pattern."""
    torch, bl = dev
    k = 28672
    xq = np.full((5, k), 127, np.int8)
    xq[1] = -127
    xq[2, ::2] = -127
    codes = np.ones((6, k), np.int8)
    codes[1] = -1
    codes[2] = 0
    codes[3, 1::2] = -1
    codes[4, ::3] = 0
    codes[5] = np.random.default_rng(1).integers(-1, 2, size=k)
    beta = np.full(5, 127.0, np.float32)
    alpha = np.float32(1.0)
    acc_o = oracle.ternary_matmul(xq, codes)
    for m in (1, 4, 5):
        y, acc = bl.bitlinear_forward(_to(torch, xq[:m]), _to(torch, beta[:m]), _to(torch, oracle.pack(codes)),
                                      _to(torch, np.array([alpha], np.float32)), acc=True)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), acc_o[:m])
    assert acc_o[0, 0] == 127 * k


def test_end_to_end_single_bitlinear(dev):
    """Workload 1: x [1, 1024], W [1024, 1024]: quantize_weights -> quantize_act -> forward."""
    torch, bl = dev
    w = workloads.weights(1, 1024, 1024)
    x = workloads.activations(1, 1, 1024)
    r = oracle.bitlinear(x, w)
    packed, alpha = bl.bitlinear_quantize_weights(_to(torch, w))
    xq, beta = bl.bitlinear_quantize_act(_to(torch, x))
    y, acc = bl.bitlinear_forward(xq, beta, packed, alpha, acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), r["packed"])
    assert np.array_equal(xq.cpu().numpy(), r["xq"])
    assert np.array_equal(acc.cpu().numpy(), r["acc"])
    assert np.array_equal(y.cpu().numpy(), r["y"])


# ------------------------------------------------------------------ full-size workloads, every output
# The decode GEMV, batched-decode and prefill workloads at their full sizes, in the launch
# configuration the benchmark times, compared on every element of acc and y (the oracle runs
# over host threads, output rows split between them).
FULL = [(1, 4096, 4096), (1, 4096, 11008), (1, 11008, 4096),
        (8, 4096, 11008), (8, 11008, 4096), (16, 4096, 11008), (16, 11008, 4096),
        (64, 4096, 11008), (64, 11008, 4096),
        (2048, 4096, 4096), (2048, 4096, 11008)]


@pytest.mark.parametrize("m,k,n", FULL)
def test_full_size(dev, m, k, n):
    torch, bl = dev
    _say(f"full-size M={m} K={k} N={n}")
    w = workloads.weights(3, n, k)
    x = workloads.activations_with_outliers(3, m, k) if m >= 512 else workloads.activations(3, m, k)
    packed, alpha = bl.bitlinear_quantize_weights(_to(torch, w))
    xq, beta = bl.bitlinear_quantize_act(_to(torch, x))
    y, acc = bl.bitlinear_forward(xq, beta, packed, alpha, acc=True)
    torch.cuda.synchronize()
    codes_o, packed_o, alpha_o = oracle.quantize_weights(w)
    xq_o, beta_o = oracle.quantize_act(x)
    assert alpha.cpu().numpy()[0] == alpha_o
    assert np.array_equal(packed.cpu().numpy(), packed_o)
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert np.array_equal(beta.cpu().numpy().view(np.uint32), beta_o.view(np.uint32))
    _say(f"full-size M={m} K={k} N={n}: oracle over {par_oracle.host_threads()} threads")
    acc_o, y_o = par_oracle.forward(xq_o, beta_o, packed_o, k, alpha_o)
    acc_g = acc.cpu().numpy()
    bad = np.argwhere(acc_g != acc_o)
    assert bad.size == 0, (bad[:5], acc_g[tuple(bad[0])], acc_o[tuple(bad[0])])
    y_g = y.cpu().numpy()
    assert _rel_ok(y_g, y_o)
    assert np.array_equal(y_g.view(np.uint32), y_o.view(np.uint32))


def test_repeatable_bitwise(dev):
    torch, bl = dev
    w = workloads.weights(3, 4096, 4096)
    x = workloads.activations(3, 64, 4096)
    wt, xt = _to(torch, w), _to(torch, x)
    outs = []
    for _ in range(3):
        packed, alpha = bl.bitlinear_quantize_weights(wt)
        xq, beta = bl.bitlinear_quantize_act(xt)
        outs.append([t.cpu().numpy().copy() for t in (packed, alpha, xq, beta,
                                                      bl.bitlinear_forward(xq, beta, packed, alpha))])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


# ------------------------------------------------------------------ fused quantize + forward
FUSED_CASES = [(1, 64, 5), (1, 1024, 1024), (1, 4096, 4096), (1, 4096, 11008), (1, 11008, 4096),
               (1, 28672, 1100), (1, 8192, 3000), (1, 32768, 70), (2, 4096, 300), (3, 11008, 130),
               (4, 16384, 257), (4, 192, 4096),
               # several tokens in 8-wave workgroups (N >= 2048): two, three and four tokens
               (2, 8192, 3000), (3, 16384, 2500), (2, 4096, 11008),
               (1, 12288, 4097), (1, 16384, 2048), (1, 28672, 2100), (1, 4096, 16385),
               # one token with the dot products on MFMA: four rows to an MFMA with rows of one and
               # two chunks per lane (four and eight rows per wave), two rows to an MFMA with six
               # rows per wave, double-buffered steps of two rows of three chunks; a row just over
               # one chunk per lane; waves without rows at the end of the grid; ragged N; and four
               # rows of three chunks, which stay on v_dot4
               (1, 8192, 7000), (1, 4096, 7000), (1, 4096, 15000), (1, 8192, 11000), (1, 8192, 15000),
               (1, 11008, 11000), (1, 11008, 13000), (1, 4160, 9000), (1, 8192, 8193), (1, 11008, 7777)]


@pytest.mark.parametrize("m,k,n", FUSED_CASES)
def test_forward_fused_parity(dev, m, k, n):
    torch, bl = dev
    _say(f"forward_fused M={m} K={k} N={n}")
    w = workloads.weights(6, n, k)
    x = workloads.activations_with_outliers(6, m, k)
    codes_o, packed_o, alpha_o = oracle.quantize_weights(w)
    xq_o, beta_o = oracle.quantize_act(x)
    acc_o = oracle.ternary_matmul(xq_o, codes_o)
    y_o = oracle.dequant(acc_o, beta_o, alpha_o)
    xt = _to(torch, x)
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    beta = torch.empty(m, dtype=torch.float32, device="cuda")
    pk, al = _to(torch, packed_o), _to(torch, np.array([alpha_o], np.float32))
    # with x_q and beta given, three or four tokens (two with K > 4096) take the two calls;
    # without them every case here is the one kernel
    two = m >= 3 or (m == 2 and k > 4096)
    assert bl.bitlinear_forward_fused_kernel(m, k, n, xt, pk, xq) == ("quantize_act+forward" if two else "gemv_fused")
    assert bl.bitlinear_forward_fused_kernel(m, k, n, xt, pk) == "gemv_fused"
    y, acc = bl.bitlinear_forward_fused(xt, pk, al, x_q=xq, beta=beta, acc=True)
    y2 = bl.bitlinear_forward_fused(xt, pk, al)          # no exports: one kernel
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert np.array_equal(beta.cpu().numpy(), beta_o)
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    assert np.array_equal(y.cpu().numpy(), y_o)
    assert np.array_equal(y2.cpu().numpy(), y_o)


@pytest.mark.parametrize("m,k,n,off", [(1, 4096, 11008, 16), (1, 4096, 4096, 512), (1, 11008, 4096, 128),
                                       (2, 4096, 3000, 48), (4, 8192, 700, 1008), (1, 32768, 300, 272)])
def test_forward_fused_unaligned_x(dev, m, k, n, off):
    """x at an offset of `off` bytes from a large allocation (16-byte aligned, as the ABI asks,
    but not at a multiple of the 1 KiB the fused kernel's loads cover)."""
    torch, bl = dev
    _say(f"forward_fused unaligned x M={m} K={k} N={n} offset={off}")
    w = workloads.weights(6, n, k, index=5)
    x = workloads.activations_with_outliers(6, m, k, index=5)
    r = oracle.bitlinear(x, w)
    buf = torch.zeros(m * k + 256, dtype=torch.float32, device="cuda")
    start = ((off - buf.data_ptr() % 1024) % 1024) // 4           # x at an address = off mod 1 KiB
    xt = buf[start: start + m * k].view(m, k)
    xt.copy_(_to(torch, x))
    assert xt.data_ptr() % 1024 == off
    pk, al = _to(torch, r["packed"]), _to(torch, np.array([r["alpha"]], np.float32))
    y, acc = bl.bitlinear_forward_fused(xt, pk, al, acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), r["acc"])
    assert np.array_equal(y.cpu().numpy(), r["y"])


@pytest.mark.parametrize("m,k,n", [(5, 4096, 130), (64, 1024, 64), (2, 100, 33), (3, 28672, 40)])
def test_forward_fused_two_call_path(dev, m, k, n):
    torch, bl = dev
    w = workloads.weights(6, n, k, index=2)
    x = workloads.activations(6, m, k, index=2)
    r = oracle.bitlinear(x, w)
    xt = _to(torch, x)
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    beta = torch.empty(m, dtype=torch.float32, device="cuda")
    pk, al = _to(torch, r["packed"]), _to(torch, np.array([r["alpha"]], np.float32))
    assert bl.bitlinear_forward_fused_kernel(m, k, n, xt, pk, xq) == "quantize_act+forward"
    y = bl.bitlinear_forward_fused(xt, pk, al, x_q=xq, beta=beta, bias=None)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), r["xq"])
    assert np.array_equal(y.cpu().numpy(), r["y"])
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear_forward_fused(xt, pk, al)            # needs x_q and beta on this path


# Grouped projections through bitlinear_forward_fused_rows: the packed rows of projections that
# read the same x stacked into one matrix, each projection's own per-tensor alpha repeated over
# its rows.  One launch must give, bit for bit, what the oracle gives for each projection alone.
GROUP_CASES = [
    (1, 4096, (4096, 1024, 1024)),       # q, k, v of an attention block (one kernel)
    (1, 8192, (2816, 2816)),             # gate, up of an MLP
    (1, 1024, (200, 57, 300)),           # ragged groups
    (3, 4096, (1000, 300)),              # M = 3: still one kernel
    (9, 2048, (400, 129)),               # M = 9: the two-call path (forward_rows)
]


@pytest.mark.parametrize("m,k,ns", GROUP_CASES)
def test_forward_fused_rows_grouped(dev, m, k, ns):
    torch, bl = dev
    _say(f"forward_fused_rows grouped M={m} K={k} N={ns}")
    x = workloads.activations(7, m, k)
    xq_o, beta_o = oracle.quantize_act(x)
    packed, alpha_rows, y_ref = [], [], []
    for g, n in enumerate(ns):
        w = workloads.weights(7, n, k, index=g)
        codes_o, packed_o, alpha_o = oracle.quantize_weights(w)
        packed.append(packed_o)
        alpha_rows.append(np.full(n, alpha_o, np.float32))
        y_ref.append(oracle.dequant(oracle.ternary_matmul(xq_o, codes_o), beta_o, alpha_o))
    pk = _to(torch, np.concatenate(packed, axis=0))
    ar = _to(torch, np.concatenate(alpha_rows))
    y_ref = np.concatenate(y_ref, axis=1)
    xt = _to(torch, x)
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    beta = torch.empty(m, dtype=torch.float32, device="cuda")
    y = bl.bitlinear_forward_fused_rows(xt, pk, ar, x_q=xq, beta=beta)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    yg = y.cpu().numpy()
    assert _rel_ok(yg, y_ref)
    assert np.array_equal(yg, y_ref)


@pytest.mark.parametrize("m,k,n", [(1, 4096, 4096), (1, 11008, 300), (2, 1024, 777), (1, 8192, 3000), (1, 11008, 8000)])
def test_forward_fused_rows_per_row_alpha(dev, m, k, n):
    """Per-row alpha [P2 §3.1] quantization followed by the fused per-row forward."""
    torch, bl = dev
    w = workloads.weights(7, n, k, index=9)
    x = workloads.activations(7, m, k, index=9)
    alpha_rows_o = oracle.absmean_rows(w)
    codes_o = oracle.ternarize_rows(w, alpha_rows_o)
    packed_o = oracle.pack(codes_o)
    xq_o, beta_o = oracle.quantize_act(x)
    acc_o = oracle.ternary_matmul(xq_o, codes_o)
    y_o = oracle.dequant(acc_o, beta_o, 0.0, alpha_rows=alpha_rows_o)
    y = bl.bitlinear_forward_fused_rows(_to(torch, x), _to(torch, packed_o), _to(torch, alpha_rows_o))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_o)


# ------------------------------------------------------------------ rotation before absmax [P3 §6.2]
# (M, K, block, with signs): every chunk path (1, 2, 4, 8 chunks of 4096 held in registers,
# and the two-pass path past 8 chunks), ragged last chunks, blocks from 1 to 4096.
HAD_CASES = [(3, 4096, 4096, True), (2, 8192, 2048, True), (2, 11008, 256, True), (1, 12, 4, True),
             (2, 4100, 4, False), (5, 1024, 1024, True), (2, 12352, 64, True), (1, 36, 1, True),
             (2, 28672, 4096, True), (1, 40960, 4096, True), (4, 2048, 2, False), (64, 4096, 4096, True),
             (2, 20480, 1024, True), (3, 6144, 2048, False), (3, 3072, 1024, True), (2500, 1024, 256, True),
             (1030, 2048, 8, False), (6, 2048, 2048, True)]


def _had_inputs(m, k, with_signs, seed=5):
    x = workloads.activations_with_outliers(seed, m, k)
    d = workloads.rotation_signs(seed, k) if with_signs else None
    return x, d


@pytest.mark.parametrize("m,k,block,with_signs", HAD_CASES)
def test_hadamard_rows_parity(dev, m, k, block, with_signs):
    torch, bl = dev
    _say(f"hadamard_rows M={m} K={k} B={block} signs={with_signs}")
    x, d = _had_inputs(m, k, with_signs)
    want = oracle.hadamard_rows(x, block, d)
    got = bl.bitlinear_hadamard_rows(_to(torch, x), block, None if d is None else _to(torch, d))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_hadamard_rows_in_place(dev):
    torch, bl = dev
    x, d = _had_inputs(3, 12288, True, seed=6)
    want = oracle.hadamard_rows(x, 4096, d)
    xt = _to(torch, x)
    out = bl.bitlinear_hadamard_rows(xt, 4096, _to(torch, d), out=xt)
    torch.cuda.synchronize()
    assert out.data_ptr() == xt.data_ptr()
    assert np.array_equal(xt.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("m,k,block,with_signs", HAD_CASES)
def test_quantize_act_hadamard_parity(dev, m, k, block, with_signs):
    torch, bl = dev
    _say(f"quantize_act_hadamard M={m} K={k} B={block} signs={with_signs}")
    x, d = _had_inputs(m, k, with_signs)
    xq_o, beta_o = oracle.quantize_act_hadamard(x, block, d)
    xq, beta = bl.bitlinear_quantize_act_hadamard(_to(torch, x), block, None if d is None else _to(torch, d))
    torch.cuda.synchronize()
    assert np.array_equal(beta.cpu().numpy().view(np.uint32), beta_o.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_o)


@pytest.mark.parametrize("k,block", [(4096, 4096), (1024, 1024), (2048, 2048), (4096, 64)])
def test_quantize_act_hadamard_tiny_and_zero_rows(dev, k, block):
    """Rows whose rotated values are subnormal (all of them, or all but the largest), an
    all-zero row and a single spike: codes and beta still match bit for bit."""
    torch, bl = dev
    _say(f"quantize_act_hadamard tiny rows K={k} B={block}")
    g = np.random.default_rng(3)
    x = np.zeros((5, k), np.float32)
    x[0] = (g.standard_normal(k) * 1e-37).astype(np.float32)          # every rotated value subnormal
    x[1] = (g.standard_normal(k) * 1e-36).astype(np.float32)
    x[1, 7] = np.float32(1.0)                                           # one normal spike
    x[3, k - 1] = np.float32(-3.5)                                      # x[2] stays all zero
    x[4] = (g.standard_normal(k) * 1e-41).astype(np.float32)          # subnormal inputs
    d = workloads.rotation_signs(7, k)
    xq_o, beta_o = oracle.quantize_act_hadamard(x, block, d)
    xq, beta = bl.bitlinear_quantize_act_hadamard(_to(torch, x), block, _to(torch, d))
    torch.cuda.synchronize()
    assert np.array_equal(beta.cpu().numpy().view(np.uint32), beta_o.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_o)


def test_quantize_act_hadamard_prefill_full_size(dev):
    """Prefill activations [2048, 4096] with 0.1% outliers, block 4096: all rows compared."""
    torch, bl = dev
    _say("quantize_act_hadamard M=2048 K=4096 B=4096")
    x = workloads.activations_with_outliers(4, 2048, 4096)
    d = workloads.rotation_signs(4, 4096)
    xq_o, beta_o = oracle.quantize_act_hadamard(x, 4096, d)
    xq, beta = bl.bitlinear_quantize_act_hadamard(_to(torch, x), 4096, _to(torch, d))
    torch.cuda.synchronize()
    assert np.array_equal(beta.cpu().numpy().view(np.uint32), beta_o.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), xq_o)


@pytest.mark.parametrize("m,k,n,block", [(1, 4096, 1024, 4096), (1, 11008, 300, 256), (24, 2048, 200, 2048),
                                         (130, 1024, 96, 512)])
def test_end_to_end_rotated_bitlinear(dev, m, k, n, block):
    """Rotated weights (offline: hadamard_rows then quantize_weights) and rotated activations
    (quantize_act_hadamard) into bitlinear_forward, against the oracle's rotated BitLinear."""
    torch, bl = dev
    _say(f"rotated bitlinear M={m} K={k} N={n} B={block}")
    w = workloads.weights(6, n, k)
    x = workloads.activations_with_outliers(6, m, k)
    d = workloads.rotation_signs(6, k)
    r = oracle.bitlinear_hadamard(x, w, block, d)
    dt = _to(torch, d)
    wr = bl.bitlinear_hadamard_rows(_to(torch, w), block, dt)
    packed, alpha = bl.bitlinear_quantize_weights(wr)
    xq, beta = bl.bitlinear_quantize_act_hadamard(_to(torch, x), block, dt)
    y, acc = bl.bitlinear_forward(xq, beta, packed, alpha, acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), r["packed"])
    assert np.float32(alpha.cpu().numpy()[0]) == r["alpha"]
    assert np.array_equal(xq.cpu().numpy(), r["xq"])
    assert np.array_equal(acc.cpu().numpy(), r["acc"])
    assert _rel_ok(y.cpu().numpy(), r["y"])


# ------------------------------------------------------------------ block scales [P1 §2.3, §4.2]
def _block_w(seed, n, k, zero_block=False):
    g = np.random.default_rng(seed)
    w = g.standard_normal((n, k)).astype(np.float32) * np.float32(0.02)
    gain = np.exp(g.uniform(np.log(0.05), np.log(5.0), size=(n, k // 128))).astype(np.float32)
    w = (w * np.repeat(gain, 128, axis=1)).astype(np.float32)
    if zero_block:
        w[0, :128] = 0.0
    return w


@pytest.mark.parametrize("n,k", [(1024, 1024), (11008, 4096), (4096, 11008), (33, 128), (7, 384), (5, 256)])
def test_quantize_weights_blocks_parity(dev, n, k):
    torch, bl = dev
    _say(f"quantize_weights_blocks N={n} K={k}")
    w = _block_w(31, n, k, zero_block=True)
    _, packed_o, a_o = oracle.quantize_weights_blocks(w)
    packed, a = bl.bitlinear_quantize_weights_blocks(_to(torch, w))
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), a_o.view(np.uint32))
    assert np.array_equal(packed.cpu().numpy(), packed_o)


def _blocks_bound_ok(y, acc_b, alpha_b, beta, y_ref):
    """|y - y_ref| <= one fp32 rounding of y_ref + 2^-40 sum_b |alpha acc| beta/127 (the fp64
    additions in another order), and at least 99% of the outputs bit-identical."""
    t = beta.astype(np.float64)[:, None] / 127.0
    mag = np.einsum("mnb,nb->mn", np.abs(acc_b.astype(np.float64)), np.abs(alpha_b.astype(np.float64))) * t
    ref = y_ref.astype(np.float64)
    ulp = np.maximum(np.abs(ref) * 2.0 ** -23, 2.0 ** -149)
    ok = np.abs(y.astype(np.float64) - ref) <= ulp + mag * 2.0 ** -40
    same = np.mean(y.view(np.uint32) == y_ref.view(np.uint32))
    return bool(ok.all()), same


BLOCK_CASES = [(1, 4096, 4096), (1, 11008, 300), (2, 128, 77), (3, 4096, 1000), (4, 28672, 64), (1, 32768, 40),
               (7, 1024, 333), (64, 2048, 130), (1, 256, 1), (9, 384, 65),
               # more than four tokens: 16x16x64 tiles, one or two token tiles, 1/2/4 row blocks per
               # workgroup, K % 256 == 128 (a lone last block), slices of 32 tokens
               (5, 4096, 4500), (16, 640, 8300), (32, 1152, 5000), (33, 256, 100), (17, 128, 17),
               # the largest K (alpha rows of 257 floats per row in LDS), and three row blocks at a
               # K whose alpha rows take 25 KB of LDS
               (5, 32768, 70), (4, 16384, 8300),
               # the fewest row blocks that keep the grid within 256 workgroups: 3 and 4 with one
               # token tile (4 also beyond 256 workgroups, with 4 x 16 alpha rows at K = 16384),
               # 2 and 3 with two (3 also beyond 256 workgroups)
               (6, 4096, 12000), (8, 1024, 16000), (5, 2048, 20000), (3, 16384, 23000), (7, 512, 30000),
               (24, 128, 6000), (20, 1024, 9000), (32, 640, 15000),
               # 33-127 tokens: three and four slices of 32, the last ragged
               (65, 4224, 4100), (127, 256, 129),
               # K % 256 == 0 from 3 tokens: the buffer-load kernel (codes in weight order, one
               # 128-weight block per pair of MFMAs) in slices of up to 64 tokens, one to four
               # token tiles, one to three row blocks (two at most with three or four tiles, also
               # beyond 256 workgroups), one sub-step (seven idle waves), sub-step counts not
               # divisible by the eight waves, K = 16384 (alpha rows of 129 floats in LDS), ragged
               # N and M; 66 and 100 tokens: a 64-token slice, then 2 tokens on the earlier
               # kernel and 36 on this one
               (8, 256, 4096), (13, 2304, 4097), (17, 1280, 8193), (31, 512, 12288),
               (33, 4096, 300), (47, 768, 4100), (48, 3328, 8192), (49, 256, 4096), (60, 2816, 8193),
               (64, 4096, 12288), (64, 16384, 1000), (66, 1024, 700), (100, 4608, 513),
               (3, 256, 4096), (7, 2304, 8193), (4, 11008, 300),
               # at most 256 16-row blocks from 17 tokens: two halves of the tokens on a second grid
               # dimension, one and two row blocks, one or two tiles per half, a one-token half
               (64, 4096, 4096), (33, 2304, 2049), (20, 1024, 500), (47, 11008, 1000)]


@pytest.mark.parametrize("m,k,n", BLOCK_CASES)
def test_forward_blocks_parity(dev, m, k, n):
    torch, bl = dev
    _say(f"forward_blocks M={m} K={k} N={n}")
    w = _block_w(32, n, k, zero_block=True)
    x = workloads.activations_with_outliers(32, m, k)
    codes, packed, a = oracle.quantize_weights_blocks(w)
    xq, beta = oracle.quantize_act(x)
    bias = workloads.activations(33, 1, n)[0] if m % 2 else None
    acc_b, y_ref = oracle.forward_blocks(xq, beta, packed, k, a, bias=bias)
    y = bl.bitlinear_forward_blocks(_to(torch, xq), _to(torch, beta), _to(torch, packed), _to(torch, a),
                                    bias=None if bias is None else _to(torch, bias))
    torch.cuda.synchronize()
    yv = y.cpu().numpy()
    if bias is None:
        ok, same = _blocks_bound_ok(yv, acc_b, a, beta, y_ref)
    else:
        # one rounding of the pre-bias value (carried through the bias addition) plus the
        # rounding of that addition itself
        y_nb = oracle.dequant_blocks(acc_b, beta, a).astype(np.float64)
        t = beta.astype(np.float64)[:, None] / 127.0
        mag = np.einsum("mnb,nb->mn", np.abs(acc_b.astype(np.float64)), np.abs(a.astype(np.float64))) * t
        ulp = lambda v: np.maximum(np.abs(v) * 2.0 ** -23, 2.0 ** -149)
        ok = bool(np.all(np.abs(yv.astype(np.float64) - y_ref) <= ulp(y_nb) + ulp(y_ref) + mag * 2.0 ** -40))
        same = np.mean(yv.view(np.uint32) == y_ref.view(np.uint32))
    _say(f"  bit-identical fraction {same:.6f}")
    assert ok
    assert same >= 0.99


# 128 tokens and more: the block-scaled GEMM adds alpha * acc per block in fp64 in ascending
# block order, the oracle's order, so y is compared bit for bit.  Cases: one and several 128 x 128
# tiles, ragged M and N, K of one block and odd block counts, with and without bias.
BLOCK_GEMM_CASES = [(128, 128, 100), (200, 256, 129), (128, 4096, 256), (129, 1152, 300), (300, 2048, 1000),
                    (1000, 384, 257), (160, 4224, 4100)]


@pytest.mark.parametrize("m,k,n", BLOCK_GEMM_CASES)
def test_forward_blocks_gemm_bit_exact(dev, m, k, n):
    torch, bl = dev
    _say(f"forward_blocks GEMM M={m} K={k} N={n}")
    w = _block_w(35, n, k, zero_block=True)
    x = workloads.activations_with_outliers(35, m, k)
    _, packed, a = oracle.quantize_weights_blocks(w)
    xq, beta = oracle.quantize_act(x)
    bias = workloads.activations(36, 1, n)[0] if (m + n) % 2 else None
    _, y_ref = oracle.forward_blocks(xq, beta, packed, k, a, bias=bias)
    y = bl.bitlinear_forward_blocks(_to(torch, xq), _to(torch, beta), _to(torch, packed), _to(torch, a),
                                    bias=None if bias is None else _to(torch, bias))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


def test_forward_blocks_prefill_full_size_sampled(dev):
    """M = 2048, K = 4096, N = 11008 with block scales (the prefill workload): every token on 64
    sampled weight rows (first, last and random), bit for bit."""
    torch, bl = dev
    m, k, n = 2048, 4096, 11008
    _say(f"forward_blocks prefill M={m} K={k} N={n}")
    w = _block_w(37, n, k)
    x = workloads.activations_with_outliers(37, m, k)
    packed_t, a_t = bl.bitlinear_quantize_weights_blocks(_to(torch, w))
    xq_t, beta_t = bl.bitlinear_quantize_act(_to(torch, x))
    y = bl.bitlinear_forward_blocks(xq_t, beta_t, packed_t, a_t)
    torch.cuda.synchronize()
    _, packed, a = oracle.quantize_weights_blocks(w)
    xq, beta = oracle.quantize_act(x)
    assert np.array_equal(packed_t.cpu().numpy(), packed)
    assert np.array_equal(a_t.cpu().numpy().view(np.uint32), a.view(np.uint32))
    assert np.array_equal(xq_t.cpu().numpy(), xq)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n),
                                     np.random.default_rng(7).choice(n, 48, replace=False)]))
    _, y_ref = oracle.forward_blocks(xq, beta, np.ascontiguousarray(packed[rows]), k, np.ascontiguousarray(a[rows]))
    assert np.array_equal(y.cpu().numpy()[:, rows].view(np.uint32), y_ref.view(np.uint32))


def test_end_to_end_block_scaled_bitlinear(dev):
    torch, bl = dev
    _say("block-scaled bitlinear M=1 K=4096 N=4096")
    w = _block_w(34, 4096, 4096)
    x = workloads.activations(34, 1, 4096)
    r = oracle.bitlinear_blocks(x, w)
    packed, a = bl.bitlinear_quantize_weights_blocks(_to(torch, w))
    xq, beta = bl.bitlinear_quantize_act(_to(torch, x))
    y = bl.bitlinear_forward_blocks(xq, beta, packed, a)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), r["packed"])
    assert np.array_equal(a.cpu().numpy().view(np.uint32), r["alpha_blocks"].view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), r["xq"])
    ok, same = _blocks_bound_ok(y.cpu().numpy(), r["acc_blocks"], r["alpha_blocks"], r["beta"], r["y"])
    assert ok and same >= 0.99


# ------------------------------------------------------------------ BitMLP [P3 §6.1]
# (M, d_model, d_ff, bias): fc1's GELU epilogue on every kernel path -- fused GEMV (M <= 4),
# 16x16x64 and 32x32x32 batched decode, the MFMA GEMM (its four-wide GELU; ragged d_ff), the
# generic kernel (d % 64 != 0); fc2's quantizer with 256-thread rows (M >= 256).
MLP_CASES = [(1, 1024, 4096, False), (1, 4096, 11008, True), (3, 512, 2048, True), (8, 512, 1024, False),
             (48, 256, 1024, True), (200, 256, 512, False), (5, 100, 36, True),
             (300, 256, 1024, True), (130, 128, 1000, True), (260, 128, 16000, True),
             # 33-64 tokens with K % 128 == 0, two row blocks per workgroup (N >= 8192) in fc1
             (64, 256, 8320, True)]


@pytest.mark.parametrize("m,d,f,with_bias", MLP_CASES)
def test_mlp_forward_parity(dev, m, d, f, with_bias):
    torch, bl = dev
    _say(f"mlp_forward M={m} d_model={d} d_ff={f} bias={with_bias}")
    w1 = workloads.weights(50, f, d)
    w2 = workloads.weights(51, d, f)
    x = workloads.activations_with_outliers(50, m, d)
    b1 = workloads.activations(52, 1, f)[0] * np.float32(0.1) if with_bias else None
    b2 = workloads.activations(53, 1, d)[0] * np.float32(0.1) if with_bias else None
    r = oracle.bitmlp(x, w1, w2, b1, b2)
    p1, a1 = bl.bitlinear_quantize_weights(_to(torch, w1))
    p2, a2 = bl.bitlinear_quantize_weights(_to(torch, w2))
    xq2 = torch.empty((m, f), dtype=torch.int8, device="cuda")
    beta2 = torch.empty(m, dtype=torch.float32, device="cuda")
    y, g = bl.bitlinear_mlp_forward(_to(torch, x), p1, a1, p2, a2,
                                    bias1=None if b1 is None else _to(torch, b1),
                                    bias2=None if b2 is None else _to(torch, b2), x_q2=xq2, beta2=beta2)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy().view(np.uint32), r["g"].view(np.uint32))
    assert np.array_equal(xq2.cpu().numpy(), r["fc2"]["xq"])
    assert np.array_equal(beta2.cpu().numpy().view(np.uint32), r["fc2"]["beta"].view(np.uint32))
    assert _rel_ok(y.cpu().numpy(), r["y"])
    assert np.array_equal(y.cpu().numpy().view(np.uint32), r["y"].view(np.uint32))


def _gelu_probe_values():
    """fp32 inputs for the GELU: every value in [-4.0625, -3.9375] (the edge of the range the
    kernels evaluate without the library erfc), random bit patterns over [-6, 12], the tail
    [-16, -4] (where GELU falls from -1.3e-4 through the fp32 subnormals to -0 near -14.5: every
    128th fp32 of it plus random bit patterns), normal samples, values near 0, denormals, signed
    zeros, infinities and the largest finite values."""
    lo, hi = np.float32(3.9375).view(np.uint32), np.float32(4.0625).view(np.uint32)
    edge = -np.arange(lo, hi + 1, dtype=np.uint32).view(np.float32)
    rng = np.random.default_rng(80)
    pos = rng.integers(0, np.float32(12.0).view(np.uint32), 500_000, dtype=np.uint32).view(np.float32)
    neg = -rng.integers(0, np.float32(6.0).view(np.uint32), 500_000, dtype=np.uint32).view(np.float32)
    t_lo, t_hi = np.float32(4.0).view(np.uint32), np.float32(16.0).view(np.uint32)
    tail = -np.arange(t_lo, t_hi + 1, 128, dtype=np.uint32).view(np.float32)
    tail_r = -rng.integers(t_lo, t_hi + 1, 100_000, dtype=np.uint32).view(np.float32)
    nrm = rng.normal(0.0, 1.0, 200_000).astype(np.float32)
    fmax = np.finfo(np.float32).max
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 3e-45, -3e-45, 1.1754942e-38, -1.1754942e-38, 1e-30, -1e-30,
                        np.inf, -np.inf, fmax, -fmax, 8.0625, 5.5, -5.5, 1.0, -1.0, -6.0, -8.0, -8.3, -10.0,
                        -12.0, -14.0, -14.5, -15.0, -16.0, -38.5, -40.0], np.float32)
    v = np.concatenate([edge, pos, neg, tail, tail_r, nrm, special])
    pad = (-v.size) % 256
    return np.concatenate([v, np.zeros(pad, np.float32)])


# (M, d_ff per call): the one-token fused kernel; the MFMA GEMM's epilogue (four GELUs per
# call), with all values in one call and in calls of 32768.
GELU_VALUE_CASES = [(1, None), (65, None), (130, 32768)]


@pytest.mark.parametrize("m,chunk", GELU_VALUE_CASES)
def test_mlp_gelu_values(dev, m, chunk):
    """GELU against the oracle on about 1.8M chosen inputs, bit for bit.  With x = 0 every
    token's fc1 output is exactly bias1 (acc = 0, so y = 0 * scale + bias), which makes g =
    GELU(bias1) row by row."""
    torch, bl = dev
    h_all = _gelu_probe_values()
    calls = 1 if chunk is None else -(-h_all.size // chunk)
    d = 64
    _say(f"mlp gelu values M={m} d_ff per call={chunk or h_all.size} calls={calls}")
    # pin the premise on a slice with the oracle's fc1: x = 0 gives y == bias (+0 for -0)
    codes = np.zeros((512, d), np.int8)
    xq0, beta0 = oracle.quantize_act(np.zeros((1, d), np.float32))
    _, y0 = oracle.forward(xq0, beta0, oracle.pack(codes), d, np.float32(1.0), bias=h_all[-512:])
    assert np.array_equal(y0[0].view(np.uint32), (h_all[-512:] + np.float32(0.0)).view(np.uint32))
    f = chunk or h_all.size
    x = torch.zeros((m, d), dtype=torch.float32, device="cuda")
    p1 = torch.full((f, d // 4), 0x55, dtype=torch.uint8, device="cuda")   # every code W = 0
    p2 = torch.full((d, f // 4), 0x55, dtype=torch.uint8, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    xq2 = torch.empty((m, f), dtype=torch.int8, device="cuda")      # fc2's quantized input
    beta2 = torch.empty(m, dtype=torch.float32, device="cuda")
    g = torch.empty((m, f), dtype=torch.float32, device="cuda")
    for c in range(calls):
        h = h_all[c * f:(c + 1) * f]
        h = np.concatenate([h, np.zeros(f - h.size, np.float32)])      # the last call's tail: zeros
        bl.bitlinear_mlp_forward(x, p1, one, p2, one, bias1=_to(torch, h), g=g, x_q2=xq2, beta2=beta2)
        torch.cuda.synchronize()
        want = oracle.gelu(h + np.float32(0.0))
        got = g.cpu().numpy()
        nan = np.isnan(want)
        for r in range(m):
            assert np.array_equal(np.isnan(got[r]), nan)
            bad = np.flatnonzero(got[r][~nan].view(np.uint32) != want[~nan].view(np.uint32))
            assert bad.size == 0, (c, r, h[~nan][bad[:5]], got[r][~nan][bad[:5]], want[~nan][bad[:5]])
        if c == 0 and np.isfinite(want).all():
            xq_ref, beta_ref = oracle.quantize_act(want[None, :])
            assert np.array_equal(xq2.cpu().numpy()[0], xq_ref[0])
            assert np.array_equal(beta2.cpu().numpy()[:1].view(np.uint32), beta_ref.view(np.uint32))


def test_binding_rejects_short_buffers(dev):
    """The binding checks every buffer the library reads or writes by size before any launch."""
    torch, bl = dev
    m, k, n = 4, 256, 64
    xq = torch.zeros((m, k), dtype=torch.int8, device="cuda")
    beta = torch.ones(m, dtype=torch.float32, device="cuda")
    wp = torch.full((n, k // 4), 0x55, dtype=torch.uint8, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="bias"):
        bl.bitlinear_forward(xq, beta, wp, one, bias=torch.zeros(n - 1, device="cuda"))
    with pytest.raises(ValueError, match="y"):
        bl.bitlinear_forward(xq, beta, wp, one, y=torch.zeros((m, n - 1), device="cuda"))
    with pytest.raises(ValueError, match="beta"):
        bl.bitlinear_forward(xq, beta[:m - 1], wp, one)
    with pytest.raises(ValueError, match="alpha"):
        bl.bitlinear_forward_rows(xq, beta, wp, torch.ones(n - 1, device="cuda"))
    x = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    w2 = torch.full((k, n // 4), 0x55, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="bias1"):
        bl.bitlinear_mlp_forward(x, wp, one, w2, one, bias1=torch.zeros(n // 2, device="cuda"))
    with pytest.raises(ValueError, match="x_q2"):
        bl.bitlinear_mlp_forward(x, wp, one, w2, one, x_q2=torch.zeros((m, 1), dtype=torch.int8, device="cuda"))
    torch.cuda.synchronize()


# ------------------------------------------------------------------ five codes per byte (R14)
@pytest.mark.parametrize("n,k", [(1024, 1024), (11008, 4096), (4096, 11008), (7, 12), (3, 84), (33, 4100)])
def test_quantize_weights_t5_parity(dev, n, k):
    torch, bl = dev
    _say(f"quantize_weights_t5 N={n} K={k}")
    w = workloads.weights(60, n, k)
    codes, packed2, alpha = oracle.quantize_weights(w)
    want = oracle.pack_t5(codes)
    wt = _to(torch, w)
    t5, a = bl.bitlinear_quantize_weights_t5(wt)
    p2, _ = bl.bitlinear_quantize_weights(wt)
    t5r = bl.bitlinear_repack_t5(p2, k)
    torch.cuda.synchronize()
    assert np.float32(a.cpu().numpy()[0]) == alpha
    assert np.array_equal(t5.cpu().numpy(), want)
    assert np.array_equal(t5r.cpu().numpy(), want)


T5_CASES = [(1, 4096, 4096), (1, 11008, 300), (1, 28672, 64), (2, 100, 33), (3, 4096, 1000), (1, 80, 7),
            (1, 84, 5), (5, 1024, 70), (1, 65536, 8), (1, 4096, 11008), (2, 2000, 9000), (1, 6000, 12000)]


@pytest.mark.parametrize("m,k,n", T5_CASES)
def test_forward_t5_parity(dev, m, k, n):
    torch, bl = dev
    _say(f"forward_t5 M={m} K={k} N={n}")
    w = workloads.weights(61, n, k)
    x = workloads.activations_with_outliers(61, m, k)
    codes, _, alpha = oracle.quantize_weights(w)
    xq, beta = oracle.quantize_act(x)
    bias = workloads.activations(62, 1, n)[0] if m % 2 else None
    _, y_ref = oracle.forward_t5(xq, beta, oracle.pack_t5(codes), k, alpha, bias=bias)
    y = bl.bitlinear_forward_t5(_to(torch, xq), _to(torch, beta), _to(torch, oracle.pack_t5(codes)),
                                _to(torch, np.array([alpha], np.float32)),
                                bias=None if bias is None else _to(torch, bias))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


def test_forward_t5_extremes(dev):
    """All-zero weights (every byte 121), all +1 / all -1 rows with x_q = +-127 (|acc| = 127 K)."""
    torch, bl = dev
    k, n = 8192, 4
    codes = np.zeros((n, k), np.int8)
    codes[1] = 1
    codes[2] = -1
    codes[3, ::3] = 1
    xq = np.full((1, k), 127, np.int8)
    xq[0, 1::2] = -127
    xq[0, :4096] = 127
    beta = np.array([3.0], np.float32)
    alpha = np.float32(0.02)
    _, y_ref = oracle.forward_t5(xq, beta, oracle.pack_t5(codes), k, alpha)
    y = bl.bitlinear_forward_t5(_to(torch, xq), _to(torch, beta), _to(torch, oracle.pack_t5(codes)),
                                _to(torch, np.array([alpha], np.float32)))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


# (M, K, N, block): one launch for a token with K <= 16384, the two-step path otherwise
FUSED_HAD_CASES = [(1, 4096, 4096, 4096), (1, 4096, 11008, 4096), (1, 11008, 4096, 256), (1, 1024, 300, 1024),
                   (1, 16384, 64, 4096), (1, 8192, 1000, 2048), (1, 256, 7, 16), (1, 12288, 33, 4096),
                   (3, 2048, 100, 512), (1, 20480, 40, 4096)]


@pytest.mark.parametrize("m,k,n,block", FUSED_HAD_CASES)
def test_forward_fused_hadamard_parity(dev, m, k, n, block):
    torch, bl = dev
    _say(f"forward_fused_hadamard M={m} K={k} N={n} B={block}")
    w = workloads.weights(70, n, k)
    x = workloads.activations_with_outliers(70, m, k)
    d = workloads.rotation_signs(70, k)
    bias = workloads.activations(71, 1, n)[0] if n % 2 else None
    r = oracle.bitlinear_hadamard(x, w, block, d, bias=bias)
    dt = _to(torch, d)
    packed, alpha = bl.bitlinear_quantize_weights(bl.bitlinear_hadamard_rows(_to(torch, w), block, dt))
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    beta = torch.empty(m, dtype=torch.float32, device="cuda")
    y = bl.bitlinear_forward_fused_hadamard(_to(torch, x), block, dt, packed, alpha,
                                            bias=None if bias is None else _to(torch, bias), x_q=xq, beta=beta)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), r["packed"])
    assert np.array_equal(xq.cpu().numpy(), r["xq"])
    assert np.array_equal(beta.cpu().numpy().view(np.uint32), r["beta"].view(np.uint32))
    assert np.array_equal(y.cpu().numpy().view(np.uint32), r["y"].view(np.uint32))


# without a sign vector (a plain Sylvester rotation): one and two chunks, with and without bias
@pytest.mark.parametrize("k,n,block", [(4096, 301, 4096), (8192, 300, 2048), (12288, 77, 4096)])
def test_forward_fused_hadamard_without_signs(dev, k, n, block):
    torch, bl = dev
    _say(f"forward_fused_hadamard no signs K={k} N={n} B={block}")
    w = workloads.weights(73, n, k)
    x = workloads.activations_with_outliers(73, 1, k)
    bias = workloads.activations(74, 1, n)[0] if n % 2 else None
    r = oracle.bitlinear_hadamard(x, w, block, None, bias=bias)
    packed, alpha = bl.bitlinear_quantize_weights(bl.bitlinear_hadamard_rows(_to(torch, w), block, None))
    y = bl.bitlinear_forward_fused_hadamard(_to(torch, x), block, None, packed, alpha,
                                            bias=None if bias is None else _to(torch, bias))
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), r["packed"])
    assert np.array_equal(y.cpu().numpy().view(np.uint32), r["y"].view(np.uint32))


def test_forward_fused_hadamard_without_outputs(dev):
    """The single-launch path needs no x_q / beta buffers."""
    torch, bl = dev
    k, n, block = 4096, 512, 4096
    w = workloads.weights(72, n, k)
    x = workloads.activations(72, 1, k)
    d = workloads.rotation_signs(72, k)
    r = oracle.bitlinear_hadamard(x, w, block, d)
    dt = _to(torch, d)
    packed, alpha = bl.bitlinear_quantize_weights(bl.bitlinear_hadamard_rows(_to(torch, w), block, dt))
    y = bl.bitlinear_forward_fused_hadamard(_to(torch, x), block, dt, packed, alpha)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), r["y"].view(np.uint32))


# ------------------------------------------------------------------ seeded random shapes
# Shapes drawn around every dispatch boundary (token counts 1-4 on the GEMV, 2-4 on the MFMA
# decode kernel below 2^26 weights, 5-64 on the batched decode tiles, slices of 32 and 64,
# the GEMM from 65 tokens; K multiples of 4, 64 and 128, ragged N), each call against the
# oracle bit for bit (block scales: the bound above).
_RS_TOKENS = [1, 1, 2, 3, 4, 5, 8, 16, 17, 31, 32, 33, 48, 64, 65, 70, 129]


def _rs_shapes(seed, count, k_mult, k_max=2304, n_max=700):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        m = int(g.choice(_RS_TOKENS))
        k = int(g.integers(1, k_max // k_mult + 1)) * k_mult
        n = int(g.integers(1, n_max + 1))
        out.append((m, k, n))
    return out


@pytest.mark.parametrize("m,k,n", _rs_shapes(101, 12, 4) + _rs_shapes(102, 14, 64) + _rs_shapes(103, 8, 128, 4096))
def test_random_shapes_forward(dev, m, k, n):
    torch, bl = dev
    _say(f"random forward M={m} K={k} N={n} kernel={bl.bitlinear_forward_kernel(m, k, n)}")
    xq, codes, packed, beta, alpha = _random_operands(m, k, n, seed=m * 131 + k * 7 + n)
    rs = np.random.default_rng(k + n)
    bias = rs.standard_normal(n).astype(np.float32)
    ar = rs.uniform(0.01, 0.02, size=n).astype(np.float32)
    acc_o = oracle.ternary_matmul(xq, codes)
    args = (_to(torch, xq), _to(torch, beta), _to(torch, packed))
    y, acc = bl.bitlinear_forward(*args, _to(torch, np.array([alpha], np.float32)), acc=True)
    yr = bl.bitlinear_forward_rows(*args, _to(torch, ar), bias=_to(torch, bias))
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    assert np.array_equal(y.cpu().numpy(), oracle.dequant(acc_o, beta, alpha))
    assert np.array_equal(yr.cpu().numpy(), oracle.dequant(acc_o, beta, alpha_rows=ar, bias=bias))


@pytest.mark.parametrize("m,k,n", _rs_shapes(104, 10, 4) + _rs_shapes(105, 10, 64))
def test_random_shapes_fused(dev, m, k, n):
    torch, bl = dev
    x = workloads.activations_with_outliers(m + k, m, k)
    _say(f"random fused M={m} K={k} N={n}")
    _, codes, packed, _, alpha = _random_operands(m, k, n, seed=m * 17 + k + n)
    xq_o, beta_o = oracle.quantize_act(x)
    y_o = oracle.dequant(oracle.ternary_matmul(xq_o, codes), beta_o, alpha)
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    beta = torch.empty(m, dtype=torch.float32, device="cuda")
    y = bl.bitlinear_forward_fused(_to(torch, x), _to(torch, packed), _to(torch, np.array([alpha], np.float32)),
                                   x_q=xq, beta=beta)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_o)
    assert np.array_equal(beta.cpu().numpy().view(np.uint32), beta_o.view(np.uint32))
    assert np.array_equal(y.cpu().numpy(), y_o)


@pytest.mark.parametrize("m,k,n", _rs_shapes(106, 12, 128, 4096))
def test_random_shapes_blocks(dev, m, k, n):
    torch, bl = dev
    _say(f"random blocks M={m} K={k} N={n}")
    w = _block_w(m + n, n, k)
    x = workloads.activations_with_outliers(m + n, m, k)
    _, packed, a = oracle.quantize_weights_blocks(w)
    xq, beta = oracle.quantize_act(x)
    acc_b, y_ref = oracle.forward_blocks(xq, beta, packed, k, a)
    y = bl.bitlinear_forward_blocks(_to(torch, xq), _to(torch, beta), _to(torch, packed), _to(torch, a))
    torch.cuda.synchronize()
    ok, same = _blocks_bound_ok(y.cpu().numpy(), acc_b, a, beta, y_ref)
    assert ok and same >= 0.99


@pytest.mark.parametrize("m,k,n", _rs_shapes(107, 8, 4))
def test_random_shapes_t5(dev, m, k, n):
    torch, bl = dev
    _say(f"random t5 M={m} K={k} N={n}")
    xq, codes, _, beta, alpha = _random_operands(m, k, n, seed=m + k * 3 + n)
    t5 = oracle.pack_t5(codes)
    _, y_ref = oracle.forward_t5(xq, beta, t5, k, alpha)
    y = bl.bitlinear_forward_t5(_to(torch, xq), _to(torch, beta), _to(torch, t5), _to(torch, np.array([alpha], np.float32)))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))
