"""int4_linear_noalloc (the library's own scratch as the workspace) against
int4_linear_ws (a caller workspace) and the oracle, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, each bit for
bit equal to int4_linear_ws on the same arguments (the same kernels and the
same split of K) and within 2e-3 * sum_k |x[m,k] * w_hat| of the oracle; a
call that needs no scratch (one row of x) as well.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests import oracle_threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def say(*a):
    print(*a, flush=True)


def case(M, N, K, g, seed):
    w = np.random.default_rng(seed).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = np.random.default_rng(seed + 1).normal(size=(M, K)).astype(np.float16)
    p, s, _ = oracle.quantize_int4(w, g)
    return x, p, s


def test_noalloc_matches_workspace_entry_point():
    import dequantizing_gemm_amd as dq
    L = dq.lib
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream().cuda_stream
    # (M, N, K, group): four shares (8 MiB of scratch), then a smaller call with
    # eight shares (3 MiB), the skinny kernel's split (four shares, 384 KiB),
    # then one row (no scratch)
    for M, N, K, g in [(128, 4096, 4096, 128), (96, 1024, 8192, 128), (32, 768, 3072, 64), (1, 2048, 4096, 128)]:
        need = dq.linear_workspace_bytes(M, N, K, g)
        say(f"case: noalloc M={M} N={N} K={K} g={g} scratch={need} B")
        x, p, s = case(M, N, K, g, seed=M + N)
        xd, pd, sd = dev(x), dev(p), dev(s)
        y_na = torch.full((M, N), float("nan"), device=DEV)
        rc = L.int4_linear_noalloc(xd.data_ptr(), dq.X_F16, M, pd.data_ptr(), sd.data_ptr(), None, N, K, g,
                                   None, dq.ACT_NONE, y_na.data_ptr(), dq.Y_F32, stream)
        assert rc == 0, L.int4_last_error().decode()
        ws = torch.zeros(max(need, 0), dtype=torch.uint8, device=DEV)
        y_ws = torch.full((M, N), float("nan"), device=DEV)
        rc = L.int4_linear_ws(xd.data_ptr(), dq.X_F16, M, pd.data_ptr(), sd.data_ptr(), None, N, K, g,
                              None, dq.ACT_NONE, y_ws.data_ptr(), dq.Y_F32,
                              ws.data_ptr() if need else None, need, stream)
        assert rc == 0, L.int4_last_error().decode()
        torch.cuda.synchronize()
        a, b = y_na.cpu().numpy(), y_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "noalloc differs from int4_linear_ws"
        rows = np.arange(M) if M <= 64 else np.unique(np.r_[np.arange(16), np.arange(M - 16, M),
                                                            np.random.default_rng(3).choice(M, 32, False)])
        ref, bound = oracle_threads.matmul(x[rows], p, s, K, g)
        err = np.abs(a[rows].astype(np.float64) - ref)
        assert np.all(err <= TOL * bound), "noalloc outside the tolerance"
