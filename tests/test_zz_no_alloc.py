"""The allocation-free weight quantization (bitlinear_quantize_weights_noalloc, for callers
that cannot allocate device memory) against bitlinear_quantize_weights with its workspace,
through the C ABI: two calls in a row, the second on a smaller tensor, each bit for bit
(packed codes and alpha), and both against the oracle."""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu


def test_noalloc_matches_the_workspace_entry_point():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bitlinear_matmul_absmean_amd as bl
    for i, (n, k) in enumerate([(11008, 4096), (1000, 260)]):
        print(f"quantize_weights_noalloc call {i}: N={n} K={k}", flush=True)
        w = workloads.weights(11, n, k, index=i)
        wt = torch.from_numpy(w).cuda()
        p_ws, a_ws = bl.bitlinear_quantize_weights(wt)
        p_na = torch.full((n, k // 4), 0xFF, dtype=torch.uint8, device="cuda")
        a_na = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        bl.bitlinear_quantize_weights_noalloc(wt, p_na, a_na)
        torch.cuda.synchronize()
        assert np.array_equal(p_na.cpu().numpy(), p_ws.cpu().numpy())
        assert a_na.cpu().numpy().view(np.uint32)[0] == a_ws.cpu().numpy().view(np.uint32)[0]
        _, packed_o, alpha_o = oracle.quantize_weights(w)
        assert np.array_equal(p_na.cpu().numpy(), packed_o)
        assert a_na.cpu().numpy()[0] == alpha_o
