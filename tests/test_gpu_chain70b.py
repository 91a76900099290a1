"""GPU parity for the 70B-class weight stream at M = 1 (80 layers x {q, o: 8192 -> 8192;
k, v: 8192 -> 1024; gate, up: 8192 -> 28672; down: 28672 -> 8192}, [P3 §5.1-§5.2]: every decode
token reads every weight once).

Its 68.5 G codes are drawn directly by a counter-based generator (the float weights cannot be
materialised), on the device for the benchmark (workloads/synth.hip) and in NumPy for the
oracle (workloads/__init__.py): two implementations of one published definition.  Here
  * the device bytes equal the NumPy bytes: sampled rows of every projection of the first and
    the last layer, and every byte of one whole layer;
  * one layer of the chain, as the benchmark runs it, equals the oracle bit for bit: the seven
    fused calls (x per layer and projection), and the grouped form (q/k/v and gate/up stacked
    into one call each, each projection's alpha repeated over its rows, o and down alone).
"""
import sys

import numpy as np
import pytest

import par_oracle
import workloads

pytestmark = pytest.mark.gpu

P = workloads.W5_PROJ
LAYER = 37
GROUPS = ((0, 1, 2), (3,), (4, 5), (6,))


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bitlinear_matmul_absmean_amd as bl
    return torch, bl


@pytest.fixture(scope="module")
def layer_rows():
    """NumPy packed bytes [N, K/4] of every projection of LAYER."""
    th = par_oracle.host_threads()
    return [workloads.stream_packed_rows(LAYER, p, k, np.arange(n), threads=th) for p, (_, k, n) in enumerate(P)]


@pytest.fixture(scope="module")
def layer_dev(dev):
    """Device bytes of LAYER, laid out as the benchmark lays them out: each group's rows in one
    buffer, the projections as row views of it."""
    torch, _ = dev
    views, bufs = {}, []
    for members in GROUPS:
        k = P[members[0]][1]
        rows = sum(P[p][2] for p in members)
        buf = torch.empty((rows, k // 4), dtype=torch.uint8, device="cuda")
        r0 = 0
        for p in members:
            n = P[p][2]
            views[p] = buf[r0:r0 + n]
            workloads.device_stream_packed(views[p], LAYER, p)
            r0 += n
        bufs.append(buf)
    torch.cuda.synchronize()
    return views, bufs


@pytest.mark.parametrize("layer", [0, 79])
def test_device_generator_sampled_rows(dev, layer):
    torch, _ = dev
    rng = np.random.default_rng(layer)
    for p, (name, k, n) in enumerate(P):
        _say(f"70B stream codes layer={layer} proj={name} K={k} N={n}")
        out = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
        workloads.device_stream_packed(out, layer, p)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(4), np.arange(n - 4, n), rng.choice(n, 24, replace=False)]))
        got = out.cpu().numpy()[rows]
        assert np.array_equal(got, workloads.stream_packed_rows(layer, p, k, rows)), name


def test_device_generator_whole_layer(dev, layer_rows, layer_dev):
    views, _ = layer_dev
    for p, (name, k, n) in enumerate(P):
        _say(f"70B stream codes layer={LAYER} proj={name}: every byte")
        assert np.array_equal(views[p].cpu().numpy(), layer_rows[p]), name


def _oracle(x, packed, k, alpha=None, alpha_rows=None):
    import oracle
    xq, beta = oracle.quantize_act(x)
    return par_oracle.forward(xq, beta, packed, k, alpha, alpha_rows=alpha_rows)


def test_chain_layer_fused_calls(dev, layer_rows, layer_dev):
    """The seven calls of one layer, x = stream_activation(layer, projection, K) each."""
    torch, bl = dev
    views, _ = layer_dev
    for p, (name, k, n) in enumerate(P):
        _say(f"70B chain layer={LAYER} fused call {name} K={k} N={n}")
        x = workloads.stream_activation(LAYER, p, k)
        alpha = workloads.stream_alpha(LAYER, p)
        y = bl.bitlinear_forward_fused(torch.from_numpy(x).cuda(), views[p],
                                       torch.tensor([alpha], dtype=torch.float32, device="cuda"))
        torch.cuda.synchronize()
        _, y_o = _oracle(x, layer_rows[p], k, alpha)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_o.view(np.uint32)), name


def test_chain_layer_grouped_calls(dev, layer_rows, layer_dev):
    """The grouped form: q/k/v (x of q) and gate/up (x of gate) in one call each over their
    stacked rows with per-row alpha, o and down alone; outputs split back per projection."""
    torch, bl = dev
    _, bufs = layer_dev
    for members, buf in zip(GROUPS, bufs):
        k = P[members[0]][1]
        names = "/".join(P[p][0] for p in members)
        _say(f"70B chain layer={LAYER} grouped call {names} K={k} N={buf.shape[0]}")
        x = workloads.stream_activation(LAYER, members[0], k)
        ar = np.concatenate([np.full(P[p][2], workloads.stream_alpha(LAYER, p), np.float32) for p in members])
        y = bl.bitlinear_forward_fused_rows(torch.from_numpy(x).cuda(), buf, torch.from_numpy(ar).cuda())
        torch.cuda.synchronize()
        packed = np.concatenate([layer_rows[p] for p in members])
        _, y_o = _oracle(x, packed, k, alpha_rows=ar)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_o.view(np.uint32)), names
        # and each member equals its own per-tensor call on the same x
        r0 = 0
        for p in members:
            n = P[p][2]
            _, y_p = _oracle(x, layer_rows[p], k, workloads.stream_alpha(LAYER, p))
            assert np.array_equal(y_o[:, r0:r0 + n].view(np.uint32), y_p.view(np.uint32)), P[p][0]
            r0 += n
