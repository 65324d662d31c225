"""The split of K in the many-row kernel (int4_linear with a workspace) on MI355X.

When the grid of output tiles is small, int4_linear_ws cuts K into shares
whose partial tiles meet in the workspace; a second kernel adds them in share
order. Every output must stay within 2e-3 * sum_k |x[m,k] * w_hat| of the
oracle (+ 2^-22 |y| with a bias, + the binary16 rounding for fp16 output),
and two calls must give the same bits whatever the workspace held before.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import oracle_threads
from tests.test_edge_gpu import edge_matrix

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


@pytest.fixture(scope="module")
def dq():
    import dequantizing_gemm_amd as dq
    return dq


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy() if t.dtype == torch.float16 else t.cpu().numpy()


def say(*a):
    print(*a, flush=True)


def rows_of(M):
    if M <= 64:
        return np.arange(M)
    rng = np.random.default_rng(3)
    mid = rng.choice(np.arange(16, M - 16), 32, replace=False)
    return np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M), mid]))


def check(y, x, p, s, K, g, zeros=None, bias=None, relu=False, half_out=False, what=""):
    rows = rows_of(x.shape[0])
    ref, bound = oracle_threads.matmul(x[rows], p, s, K, g, zeros=zeros, bias=bias, relu=relu)
    ref = ref.astype(np.float64)
    allowed = TOL * bound + (2.0 ** -22 * np.abs(ref) if bias is not None else 0.0)
    if half_out:
        allowed = allowed + 2.0 ** -11 * (np.abs(ref) + allowed) + 2.0 ** -25
    err = np.abs(y[rows].astype(np.float64) - ref)
    bad = ~(err <= allowed)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs out of tolerance"


# (M, N, K, group): 32 x 128 tiles with 4 and 8 shares, K = 11008 (shares of
# 44 sub-steps, the last shorter), ragged M and N, group 32 (64 x 128 tiles of
# 32-code sub-steps, 8 shares), a group size decided at run time (1024: shares
# of 16 sub-steps).
SPLIT_CASES = [(128, 4096, 4096, 128), (128, 4096, 11008, 128), (96, 1024, 8192, 128),
               (200, 1030, 4096, 256), (300, 640, 8192, 32), (130, 2048, 4096, 1024),
               (256, 1024, 4096, 128)]


@pytest.mark.parametrize("M,N,K,g", SPLIT_CASES, ids=[f"M{m}-N{n}-K{k}-g{g}" for m, n, k, g in SPLIT_CASES])
def test_split_matches_oracle(dq, M, N, K, g):
    nbytes = dq.linear_workspace_bytes(M, N, K, g)
    assert nbytes > 0, "this shape is meant to split K"
    w = np.random.default_rng(N + K).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = np.random.default_rng(M).normal(size=(M, K)).astype(np.float16)
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd, xd = dev(pr), dev(sr), dev(x)
    ws = dq.linear_workspace(M, N, K, g, device=DEV)
    say(f"case: split M={M} N={N} K={K} g={g} workspace={nbytes} B")
    y1 = host(dq.int4_linear(xd, pd, sd, K, g, workspace=ws))
    ws.fill_(0xA5)                              # any contents will do
    y2 = host(dq.int4_linear(xd, pd, sd, K, g, workspace=ws))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "two calls differ"
    check(y1, x, pr, sr, K, g, what=f"split M={M} N={N} K={K} g={g}")
    y0 = host(dq.int4_linear(xd, pd, sd, K, g))         # the same kernel without the split
    check(y0, x, pr, sr, K, g, what="no split")


def test_split_epilogue_and_half_output(dq):
    M, N, K, g = 128, 4096, 4096, 128
    w = np.random.default_rng(9).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = np.random.default_rng(10).normal(size=(M, K)).astype(np.float16)
    b = np.random.default_rng(11).normal(0, 0.5, N).astype(np.float32)
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd, xd, bd = dev(pr), dev(sr), dev(x), dev(b)
    ws = dq.linear_workspace(M, N, K, g, device=DEV)
    for relu in (False, True):
        for half in (False, True):
            say(f"case: split epilogue relu={relu} fp16 output={half}")
            y = host(dq.int4_linear(xd, pd, sd, K, g, bias=bd, relu=relu,
                                    out_dtype=torch.float16 if half else torch.float32, workspace=ws))
            check(y, x, pr, sr, K, g, bias=b, relu=relu, half_out=half, what=f"relu={relu} half={half}")
            if relu:
                assert np.all(y >= 0)


def test_split_affine(dq):
    M, N, K, g = 128, 4096, 4096, 128
    w = (np.random.default_rng(12).normal(0, 0.02, size=(N, K)) + 0.01).astype(np.float32)
    x = np.random.default_rng(13).normal(size=(M, K)).astype(np.float16)
    pr, sr, zr, _ = oracle.quantize_int4_affine(w, g)
    ws = dq.linear_workspace(M, N, K, g, device=DEV)
    say("case: split affine codes")
    y = host(dq.int4_linear(dev(x), dev(pr), dev(sr), K, g, zeros=dev(zr), workspace=ws))
    check(y, x, pr, sr, K, g, zeros=zr, what="split affine")


def test_split_edge_rows(dq):
    """The edge rows (scale 65504 included, which sends a block through the
    passes that read straight from memory) through a split of K."""
    M, N, K, g = 200, 1030, 4096, 128
    packed, scales = edge_matrix(N, K, g, seed=4)
    x = np.random.default_rng(14).normal(size=(M, K)).astype(np.float16)
    ws = dq.linear_workspace(M, N, K, g, device=DEV)
    assert ws.numel() > 0
    say("case: split edge rows")
    y = host(dq.int4_linear(dev(x), dev(packed), dev(scales), K, g, workspace=ws))
    check(y, x, packed, scales, K, g, what="split edge rows")


def test_small_workspace_runs_unsplit(dq):
    """A workspace smaller than the split wants: the call runs without it, with
    the same bits as int4_linear without a workspace."""
    M, N, K, g = 128, 4096, 4096, 128
    w = np.random.default_rng(15).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = dev(np.random.default_rng(16).normal(size=(M, K)).astype(np.float16))
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd = dev(pr), dev(sr)
    small = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    say("case: split with a workspace too small")
    a = host(dq.int4_linear(x, pd, sd, K, g, workspace=small))
    b = host(dq.int4_linear(x, pd, sd, K, g))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert not host(small).any()


# The skinny kernel's split of K (fewer than 128 groups of 16 weight rows, at
# least 96 K-blocks times 16-row tiles of x per row group): (M, N, K, group).
# Group 32 (128-code K-blocks of four groups) at M = 32 and 17 rows against
# 100 weight rows (4 shares), group 64 (128-code K-blocks of two groups) at 32
# and 40 rows (two and three row tiles), [1024, 8192] at M = 64, ragged M and
# N with a last share shorter than the others (K = 4224: 33 K-blocks in
# shares of 9), group 256 (two K-blocks per group), 33 rows of group 128.
SKINNY_SPLIT_CASES = [(32, 768, 3072, 32), (32, 768, 3072, 64), (40, 768, 3072, 64), (64, 1024, 8192, 128),
                      (17, 100, 4096, 32), (20, 1030, 4224, 64), (24, 2000, 8192, 256), (33, 1000, 4096, 128)]


@pytest.mark.parametrize("M,N,K,g", SKINNY_SPLIT_CASES,
                         ids=[f"M{m}-N{n}-K{k}-g{g}" for m, n, k, g in SKINNY_SPLIT_CASES])
def test_skinny_split_matches_oracle(dq, M, N, K, g):
    nbytes = dq.linear_workspace_bytes(M, N, K, g)
    assert nbytes > 0, "this shape is meant to split K"
    w = np.random.default_rng(N + K + g).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = np.random.default_rng(M + 1).normal(size=(M, K)).astype(np.float16)
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd, xd = dev(pr), dev(sr), dev(x)
    assert dq.matmul_select(xd, pd, sd, K, g) == "skinny"
    ws = dq.linear_workspace(M, N, K, g, device=DEV)
    say(f"case: skinny split M={M} N={N} K={K} g={g} workspace={nbytes} B")
    y1 = host(dq.int4_linear(xd, pd, sd, K, g, workspace=ws))
    ws.fill_(0xA5)
    y2 = host(dq.int4_linear(xd, pd, sd, K, g, workspace=ws))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "two calls differ"
    check(y1, x, pr, sr, K, g, what=f"skinny split M={M} N={N} K={K} g={g}")
    y0 = host(dq.int4_linear(xd, pd, sd, K, g))
    check(y0, x, pr, sr, K, g, what="no split")


def test_skinny_split_epilogue_affine_edge(dq):
    """Bias, ReLU and fp16 output after the share-order reduction; affine
    codes; the edge rows (zero groups, -8 codes, subnormal and 65504 scales)."""
    M, N, K, g = 32, 768, 3072, 64
    w = np.random.default_rng(21).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = np.random.default_rng(22).normal(size=(M, K)).astype(np.float16)
    b = np.random.default_rng(23).normal(0, 0.5, N).astype(np.float32)
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd, xd, bd = dev(pr), dev(sr), dev(x), dev(b)
    ws = dq.linear_workspace(M, N, K, g, device=DEV)
    assert ws.numel() > 0
    for relu in (False, True):
        for half in (False, True):
            say(f"case: skinny split epilogue relu={relu} fp16 output={half}")
            y = host(dq.int4_linear(xd, pd, sd, K, g, bias=bd, relu=relu,
                                    out_dtype=torch.float16 if half else torch.float32, workspace=ws))
            check(y, x, pr, sr, K, g, bias=b, relu=relu, half_out=half, what=f"relu={relu} half={half}")
            if relu:
                assert np.all(y >= 0)
    say("case: skinny split affine codes")
    wa = (np.random.default_rng(24).normal(0, 0.02, size=(N, K)) + 0.01).astype(np.float32)
    pa, sa, za, _ = oracle.quantize_int4_affine(wa, g)
    y = host(dq.int4_linear(xd, dev(pa), dev(sa), K, g, zeros=dev(za), workspace=ws))
    check(y, x, pa, sa, K, g, zeros=za, what="skinny split affine")
    say("case: skinny split edge rows")
    pe, se = edge_matrix(N, K, g, seed=5)
    y = host(dq.int4_linear(xd, dev(pe), dev(se), K, g, workspace=ws))
    check(y, x, pe, se, K, g, what="skinny split edge rows")
