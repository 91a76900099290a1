"""The oracle's forward with the output rows split over host threads (test helper).

Rows of W are independent in the integer matmul and in the epilogue, so splitting them over
threads changes no result: each thread runs the oracle's own unpack, ternary matmul and
dequant on its slice of rows.  The oracle's ctypes calls release the GIL.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def host_threads(cap: int = 16) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def forward(xq: np.ndarray, beta: np.ndarray, packed: np.ndarray, k: int, alpha=None,
            alpha_rows: np.ndarray | None = None, bias: np.ndarray | None = None, threads: int | None = None):
    """(acc int32 [M, N], y fp32 [M, N]) of oracle.forward, output rows split over threads."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    m = xq.shape[0]
    n = packed.shape[0]
    acc = np.empty((m, n), np.int32)
    y = np.empty((m, n), np.float32)
    threads = threads or host_threads()
    pieces = max(threads * 4, 1)
    bounds = np.unique(np.linspace(0, n, pieces + 1).astype(np.int64))

    def part(i):
        n0, n1 = int(bounds[i]), int(bounds[i + 1])
        ar = None if alpha_rows is None else alpha_rows[n0:n1]
        b = None if bias is None else bias[n0:n1]
        a, yy = oracle.forward(xq, beta, np.ascontiguousarray(packed[n0:n1]), k,
                               0.0 if alpha is None else alpha, bias=b, alpha_rows=ar)
        acc[:, n0:n1] = a
        y[:, n0:n1] = yy

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(part, range(len(bounds) - 1)))
    return acc, y
