"""Seeded synthetic inputs for the BitLinear workloads (shared by tests, bench and smoke).

This module holds no step of the method: it only draws random tensors with the shapes and
distributions of the workloads (float weights W ~ N(0, 0.02), activations x ~ N(0, 1),
optional outliers), and, for the 70B-class weight stream, ternary codes drawn directly
with a counter-based generator (SplitMix64, Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), because 68.5 G float weights cannot be
materialised.  The device implementation of the same generator lives in ``synth.hip``;
this file holds the NumPy one.  Neither implementation calls the other.

Streams are independent ``np.random.default_rng([1580, workload, tensor, index])`` PCG64
generators, so every array is reproducible on its own.
"""
from __future__ import annotations

import numpy as np

SEED = 1580
W_STD = 0.02            # weights ~ N(0, 0.02) (std), as the pages' BitLinear initialises them
X_STD = 1.0             # activations ~ N(0, 1)
OUTLIER_FRACTION = 0.001
OUTLIER_GAIN = 20.0

# Workload shapes (K = in_features, N = out_features).
W1_SHAPE = dict(M=1, K=1024, N=1024)
W2_SHAPES = [(4096, 4096), (4096, 11008), (11008, 4096)]          # 7B decode GEMV (K, N)
W3_MS = [8, 16, 64]
W3_SHAPES = [(4096, 11008), (11008, 4096)]                         # batched decode (K, N)
W4_M = 2048
W4_SHAPES = [(4096, 4096), (4096, 11008)]                          # prefill (K, N)
# 70B-class layer: projection name -> (K, N)
W5_LAYERS = 80
W5_PROJ = [("q", 8192, 8192), ("k", 8192, 1024), ("v", 8192, 1024), ("o", 8192, 8192),
           ("gate", 8192, 28672), ("up", 8192, 28672), ("down", 28672, 8192)]


def rng(workload: int, tensor: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED, workload, tensor, index])


def weights(workload: int, n: int, k: int, index: int = 0) -> np.ndarray:
    """Float weights [N, K] ~ N(0, 0.02), fp32."""
    g = rng(workload, 0, index)
    return (g.standard_normal((n, k), dtype=np.float32) * np.float32(W_STD)).astype(np.float32)


def activations(workload: int, m: int, k: int, index: int = 0) -> np.ndarray:
    """Float activations [M, K] ~ N(0, 1), fp32."""
    g = rng(workload, 1, index)
    return g.standard_normal((m, k), dtype=np.float32)


def activations_with_outliers(workload: int, m: int, k: int, index: int = 0) -> np.ndarray:
    """x ~ N(0, 1) with exactly round(0.001*M*K) entries, chosen uniformly without
    replacement, multiplied by 20 (the prefill workload's outliers)."""
    x = activations(workload, m, k, index)
    g = rng(workload, 2, index)
    count = int(round(OUTLIER_FRACTION * m * k))
    idx = g.choice(m * k, size=count, replace=False)
    flat = x.reshape(-1)
    flat[idx] *= np.float32(OUTLIER_GAIN)
    return x


def rotation_signs(workload: int, k: int, index: int = 0) -> np.ndarray:
    """Random signs d [K] (int8, +1 or -1, each with probability 1/2): the random diagonal of
    a randomized Hadamard rotation, drawn here and passed to both sides as an input."""
    g = rng(workload, 3, index)
    return np.where(g.random(k) < 0.5, -1, 1).astype(np.int8)


# ---------------------------------------------------------------------------------------
# Counter-based ternary codes for the 70B-class weight stream.
#
# SplitMix64 (published definition): with gamma = 0x9E3779B97F4A7C15, output i of a stream
# whose state starts at s is mix(s + (i + 1) * gamma), where
#   mix(z): z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9; z = (z ^ (z >> 27)) * 0x94D049BB133111EB;
#           return z ^ (z >> 31)            (all arithmetic mod 2^64).
# Packed byte i of a projection takes output i and splits it into four 16-bit fields u_j
# (bits 16j..16j+15); field j becomes the 2-bit code at bits 2j..2j+1 of the byte:
#   u < T0            -> 01 (weight 0),  T0 = 20323   (P = 0.3101, the zero fraction that
#                                                       absmean rounding gives Gaussian W)
#   u < T0 + T1       -> 00 (weight -1), T1 = 22606
#   otherwise         -> 10 (weight +1)
# The stream state of (layer, projection) is SEED * 2^40 + (layer * 16 + projection) * 2^32.
# ---------------------------------------------------------------------------------------
SM64_GAMMA = 0x9E3779B97F4A7C15
SM64_M1 = 0xBF58476D1CE4E5B9
SM64_M2 = 0x94D049BB133111EB
CODE_T0 = 20323
CODE_T1 = 22606


def stream_state(layer: int, proj: int) -> int:
    return (SEED << 40) + ((layer * 16 + proj) << 32)


def splitmix64(state: int, index: np.ndarray) -> np.ndarray:
    """Outputs ``index`` (uint64 array) of the SplitMix64 stream starting at ``state``."""
    with np.errstate(over="ignore"):
        z = np.uint64(state) + (index.astype(np.uint64) + np.uint64(1)) * np.uint64(SM64_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(SM64_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(SM64_M2)
        return z ^ (z >> np.uint64(31))


def _packed_bytes(state: int, idx: np.ndarray) -> np.ndarray:
    """Packed bytes at stream indices ``idx``: field j of output idx gives the code at bits 2j,
    (u < T0) -> 01, (u >= T0 + T1) -> 10, else 00."""
    z = splitmix64(state, idx)
    out = np.zeros(idx.shape, np.uint8)
    for j in range(4):
        u = (z >> np.uint64(16 * j)).astype(np.uint16)          # the low 16 bits of the shifted word
        code = (u < CODE_T0).view(np.uint8) + ((u >= CODE_T0 + CODE_T1).view(np.uint8) << np.uint8(1))
        out |= code << np.uint8(2 * j)
    return out


def stream_packed_rows(layer: int, proj: int, k: int, rows: np.ndarray, threads: int = 1) -> np.ndarray:
    """Packed weight bytes [len(rows), K/4] of rows ``rows`` of one 70B-class projection
    (optionally split over ``threads`` host threads; the bytes do not depend on the split)."""
    row_bytes = k // 4
    rows = np.asarray(rows, dtype=np.int64)
    state = stream_state(layer, proj)
    out = np.empty((len(rows), row_bytes), np.uint8)
    span = np.arange(row_bytes, dtype=np.int64)

    def part(r0: int, r1: int):
        idx = (rows[r0:r1, None] * row_bytes + span[None, :]).reshape(-1)
        out[r0:r1] = _packed_bytes(state, idx).reshape(r1 - r0, row_bytes)

    step = max(1, (1 << 20) // row_bytes)                          # about 1 MiB of bytes per piece
    pieces = [(r0, min(r0 + step, len(rows))) for r0 in range(0, len(rows), step)]
    if threads <= 1 or len(pieces) == 1:
        for r0, r1 in pieces:
            part(r0, r1)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda p: part(*p), pieces))
    return out


def stream_alpha(layer: int, proj: int) -> np.float32:
    """Per-(layer, projection) alpha ~ U[0.0150, 0.0170] (around E|N(0, 0.02)| = 0.01596)."""
    return np.float32(rng(5, 3, layer * 16 + proj).uniform(0.0150, 0.0170))


def stream_activation(layer: int, proj: int, k: int) -> np.ndarray:
    """x [1, K] ~ N(0, 1) for one (layer, projection) of the 70B-class stream."""
    return activations(5, 1, k, layer * 16 + proj)


_synth = None


def device_stream_packed(out, layer: int, proj: int, stream=None):
    """Fill the uint8 device tensor ``out`` ([N, K/4]) with the packed codes of one
    70B-class projection, on the device (libsynth.so, same definition as above)."""
    global _synth
    import ctypes
    import os

    import torch
    if _synth is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
        lib = ctypes.CDLL(path)
        lib.synth_ternary_packed.restype = ctypes.c_int
        lib.synth_ternary_packed.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p]
        _synth = lib
    s = torch.cuda.current_stream() if stream is None else stream
    rc = _synth.synth_ternary_packed(out.data_ptr(), out.numel(), stream_state(layer, proj), s.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_ternary_packed failed: hipError {rc}")
    return out
