"""The seeded input generators (no step of the method): the NumPy SplitMix64 stream of the
70B-class codes against a scalar evaluation of its published definition, and the code law."""
import numpy as np

import workloads

M64 = (1 << 64) - 1


def _sm64_scalar(state: int, i: int) -> int:
    """SplitMix64 (Steele, Lea & Flood, OOPSLA 2014), output i of the stream at `state`, on
    Python integers reduced mod 2^64."""
    z = (state + (i + 1) * 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _byte_scalar(z: int) -> int:
    b = 0
    for j in range(4):
        u = (z >> (16 * j)) & 0xFFFF
        c = 1 if u < 20323 else (0 if u < 20323 + 22606 else 2)
        b |= c << (2 * j)
    return b


def test_splitmix64_matches_scalar_definition():
    rng = np.random.default_rng(5)
    for layer, proj in ((0, 0), (37, 4), (79, 6)):
        st = workloads.stream_state(layer, proj)
        idx = np.concatenate([np.arange(8), rng.integers(0, 1 << 40, 200)]).astype(np.int64)
        z = workloads.splitmix64(st, idx)
        assert [int(v) for v in z] == [_sm64_scalar(st, int(i)) for i in idx]


def test_packed_rows_match_scalar_definition():
    layer, proj, k = 3, 6, 28672
    rows = np.array([0, 1, 8191, 4000])
    got = workloads.stream_packed_rows(layer, proj, k, rows)
    st = workloads.stream_state(layer, proj)
    rb = k // 4
    for r_i, r in enumerate(rows):
        for b in (0, 1, 2, rb // 2, rb - 1):
            assert got[r_i, b] == _byte_scalar(_sm64_scalar(st, int(r) * rb + b)), (r, b)


def test_packed_rows_split_and_threads_give_the_same_bytes():
    full = workloads.stream_packed_rows(1, 4, 8192, np.arange(600))
    assert np.array_equal(full, workloads.stream_packed_rows(1, 4, 8192, np.arange(600), threads=4))
    assert np.array_equal(full[[5, 77, 599]], workloads.stream_packed_rows(1, 4, 8192, np.array([5, 77, 599])))


def test_code_law():
    """Codes 00/01/10 with P(0) = 20323 / 65536 = 0.3101 and P(+1) = P(-1) = 0.345; 11 never."""
    p = workloads.stream_packed_rows(2, 0, 8192, np.arange(256))
    c = np.stack([(p >> (2 * j)) & 3 for j in range(4)]).reshape(-1)
    assert not np.any(c == 3)
    f = np.bincount(c, minlength=3) / c.size
    n = c.size
    for got, want in zip(f, (22606 / 65536, 20323 / 65536, 1 - (20323 + 22606) / 65536)):
        assert abs(got - want) < 6 * np.sqrt(want * (1 - want) / n)


def test_stream_activation_and_alpha_are_per_layer_and_projection():
    a = workloads.stream_activation(3, 1, 8192)
    b = workloads.stream_activation(3, 2, 8192)
    assert a.shape == (1, 8192) and a.dtype == np.float32 and not np.array_equal(a, b)
    assert np.array_equal(a, workloads.stream_activation(3, 1, 8192))
    al = [workloads.stream_alpha(layer, p) for layer in range(4) for p in range(7)]
    assert all(0.0150 <= v <= 0.0170 for v in al) and len(set(al)) == len(al)
