"""The oracle's matmul over column blocks on a few host threads.

Test infrastructure only. ``oracle.int4_matmul_ex`` is a ctypes call into the
scalar C oracle, which releases the GIL, so independent column blocks of y run
in parallel threads; each block is the oracle's own result for those weight
rows (no arithmetic is added here). Used where a check compares every output
column of sampled rows of a large case.
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

import oracle

THREADS = max(1, min(8, os.cpu_count() or 1))


def matmul(x, packed, scales, K, group, zeros=None, bias=None, relu=False, threads=THREADS):
    """(y float32 [M, N], bound float64 [M, N]) from the oracle, N split over threads."""
    x = np.ascontiguousarray(x)
    N = packed.shape[0]
    nblk = max(1, min(threads * 4, N // 64))
    edges = np.linspace(0, N, nblk + 1).astype(int)
    y = np.empty((x.shape[0], N), np.float32)
    bound = np.empty((x.shape[0], N), np.float64)

    def run(i):
        a, b = edges[i], edges[i + 1]
        if a == b:
            return
        yb, bb = oracle.int4_matmul_ex(
            x, packed[a:b], scales[a:b], K, group, bias=None if bias is None else bias[a:b],
            relu=relu, with_bound=True, zeros=None if zeros is None else zeros[a:b])
        y[:, a:b] = yb
        bound[:, a:b] = bb

    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, range(nblk)))
    return y, bound
