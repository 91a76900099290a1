"""The library's calls captured in a HIP graph and replayed: every replay must equal the eager
results bit for bit.  Between replays the outputs are overwritten with NaN and the program does
eager work of its own (other library calls on other buffers, synchronizations), so a replay that
skipped or reordered a kernel, or leaned on state left by eager calls, would show.  The library
records no memset nodes and allocates nothing itself; buffers the binding allocates inside the
capture come from the graph's own pool."""
import numpy as np
import pytest

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


def test_graph_replays_match_eager(dev):
    torch, bl = dev
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f32 = dict(dtype=torch.float32, device="cuda")
    # weights
    w_dec = workloads.weights(90, 1000, 4096)            # fused GEMV, one token
    w_gemm = workloads.weights(91, 700, 512)             # MFMA GEMM, 200 tokens
    w_bat = workloads.weights(92, 9000, 1024)            # batched decode MFMA, 24 tokens
    w1, w2 = workloads.weights(93, 1000, 256), workloads.weights(94, 256, 1000)   # BitMLP, 130 tokens
    w_had = workloads.weights(95, 300, 2048)             # rotated projection, one token
    w_blk = workloads.weights(96, 500, 1024)             # block scales, 4 tokens
    w_t5 = workloads.weights(97, 300, 1000)              # five codes per byte, one token
    w_b64 = workloads.weights(100, 9000, 1024)           # batched decode, 64 tokens, whole sub-steps
    w_b16 = workloads.weights(101, 700, 2048)            # batched decode, 12 tokens, one row block per workgroup
    w_bg = workloads.weights(102, 300, 640)              # block-scaled GEMM, 160 tokens
    w_bb = workloads.weights(103, 900, 1024)             # block scales, 40 tokens (x_q and codes through LDS loads)
    p_dec, a_dec = bl.bitlinear_quantize_weights(t(w_dec))
    p_gemm, a_gemm = bl.bitlinear_quantize_weights(t(w_gemm))
    p_bat, a_bat = bl.bitlinear_quantize_weights(t(w_bat))
    p1, a1 = bl.bitlinear_quantize_weights(t(w1))
    p2, a2 = bl.bitlinear_quantize_weights(t(w2))
    signs = t(workloads.rotation_signs(95, 2048))
    p_had, a_had = bl.bitlinear_quantize_weights(bl.bitlinear_hadamard_rows(t(w_had), 2048, signs))
    p_blk, a_blk = bl.bitlinear_quantize_weights_blocks(t(w_blk))
    p_t5, a_t5 = bl.bitlinear_quantize_weights_t5(t(w_t5))
    p_b64, a_b64 = bl.bitlinear_quantize_weights(t(w_b64))
    p_b16, a_b16 = bl.bitlinear_quantize_weights(t(w_b16))
    p_bg, a_bg = bl.bitlinear_quantize_weights_blocks(t(w_bg))
    p_bb, a_bb = bl.bitlinear_quantize_weights_blocks(t(w_bb))
    # activations and static outputs
    x_dec = t(workloads.activations_with_outliers(90, 1, 4096))
    x_gemm = t(workloads.activations_with_outliers(91, 200, 512))
    x_bat = t(workloads.activations_with_outliers(92, 24, 1024))
    x_mlp = t(workloads.activations_with_outliers(93, 130, 256))
    x_had = t(workloads.activations_with_outliers(95, 1, 2048))
    x_blk = t(workloads.activations_with_outliers(96, 4, 1024))
    x_t5 = t(workloads.activations_with_outliers(97, 1, 1000))
    x_b64 = t(workloads.activations_with_outliers(100, 64, 1024))
    x_b16 = t(workloads.activations_with_outliers(101, 12, 2048))
    x_bg = t(workloads.activations_with_outliers(102, 160, 640))
    x_bb = t(workloads.activations_with_outliers(103, 40, 1024))
    bias = t(workloads.activations(98, 1, 9000)[0])
    out = {
        "dec": torch.empty((1, 1000), **f32), "gemm": torch.empty((200, 700), **f32),
        "bat": torch.empty((24, 9000), **f32), "mlp_y": torch.empty((130, 256), **f32),
        "mlp_g": torch.empty((130, 1000), **f32), "had": torch.empty((1, 300), **f32),
        "blk": torch.empty((4, 500), **f32), "t5": torch.empty((1, 300), **f32),
        "b64": torch.empty((64, 9000), **f32), "b16": torch.empty((12, 700), **f32),
        "bg": torch.empty((160, 300), **f32), "bb": torch.empty((40, 900), **f32),
    }
    xq_b64 = torch.empty((64, 1024), dtype=torch.int8, device="cuda")
    b_b64 = torch.empty(64, **f32)
    xq_b16 = torch.empty((12, 2048), dtype=torch.int8, device="cuda")
    b_b16 = torch.empty(12, **f32)
    xq_bg = torch.empty((160, 640), dtype=torch.int8, device="cuda")
    b_bg = torch.empty(160, **f32)
    xq_bb = torch.empty((40, 1024), dtype=torch.int8, device="cuda")
    b_bb = torch.empty(40, **f32)
    xq_gemm = torch.empty((200, 512), dtype=torch.int8, device="cuda")
    b_gemm = torch.empty(200, **f32)
    xq_bat = torch.empty((24, 1024), dtype=torch.int8, device="cuda")
    b_bat = torch.empty(24, **f32)
    xq1 = torch.empty((130, 256), dtype=torch.int8, device="cuda")
    bt1 = torch.empty(130, **f32)
    xq2 = torch.empty((130, 1000), dtype=torch.int8, device="cuda")
    bt2 = torch.empty(130, **f32)
    xq_blk = torch.empty((4, 1024), dtype=torch.int8, device="cuda")
    b_blk = torch.empty(4, **f32)
    xq_t5 = torch.empty((1, 1000), dtype=torch.int8, device="cuda")
    b_t5 = torch.empty(1, **f32)

    def calls():
        bl.bitlinear_forward_fused(x_dec, p_dec, a_dec, y=out["dec"])
        bl.bitlinear_quantize_act(x_gemm, x_q=xq_gemm, beta=b_gemm)
        bl.bitlinear_forward(xq_gemm, b_gemm, p_gemm, a_gemm, bias=bias[:700], y=out["gemm"])
        bl.bitlinear_quantize_act(x_bat, x_q=xq_bat, beta=b_bat)
        bl.bitlinear_forward(xq_bat, b_bat, p_bat, a_bat, bias=bias, y=out["bat"])
        bl.bitlinear_mlp_forward(x_mlp, p1, a1, p2, a2, bias1=bias[:1000], y=out["mlp_y"], g=out["mlp_g"],
                                 x_q1=xq1, beta1=bt1, x_q2=xq2, beta2=bt2)
        bl.bitlinear_forward_fused_hadamard(x_had, 2048, signs, p_had, a_had, y=out["had"])
        bl.bitlinear_quantize_act(x_blk, x_q=xq_blk, beta=b_blk)
        bl.bitlinear_forward_blocks(xq_blk, b_blk, p_blk, a_blk, y=out["blk"])
        bl.bitlinear_quantize_act(x_t5, x_q=xq_t5, beta=b_t5)
        bl.bitlinear_forward_t5(xq_t5, b_t5, p_t5, a_t5, y=out["t5"])
        bl.bitlinear_quantize_act(x_b64, x_q=xq_b64, beta=b_b64)
        bl.bitlinear_forward(xq_b64, b_b64, p_b64, a_b64, bias=bias, y=out["b64"])
        bl.bitlinear_quantize_act(x_b16, x_q=xq_b16, beta=b_b16)
        bl.bitlinear_forward(xq_b16, b_b16, p_b16, a_b16, y=out["b16"])
        bl.bitlinear_quantize_act(x_bg, x_q=xq_bg, beta=b_bg)
        bl.bitlinear_forward_blocks(xq_bg, b_bg, p_bg, a_bg, bias=bias[:300], y=out["bg"])
        bl.bitlinear_quantize_act(x_bb, x_q=xq_bb, beta=b_bb)
        bl.bitlinear_forward_blocks(xq_bb, b_bb, p_bb, a_bb, bias=bias[:900], y=out["bb"])

    _say("graph: eager reference")
    calls()
    torch.cuda.synchronize()
    want = {k: v.cpu().numpy().copy() for k, v in out.items()}
    for k, v in want.items():
        assert np.isfinite(v).all(), k

    _say("graph: capture")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    # eager work between replays: other library calls on buffers of their own
    x_other = t(workloads.activations(99, 200, 512))
    y_other = torch.empty((200, 700), **f32)
    for rep in range(4):
        _say(f"graph: replay {rep}")
        for v in out.values():
            v.fill_(float("nan"))
        bl.bitlinear_forward_fused(x_other, p_gemm, a_gemm, y=y_other, x_q=torch.empty((200, 512), dtype=torch.int8,
                                   device="cuda"), beta=torch.empty(200, **f32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            got = v.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), want[k].view(np.uint32)), (rep, k)
    del graph
