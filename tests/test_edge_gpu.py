"""Edge rows of the method through every binary16 matmul kernel, against the oracle.

The drill page "Implement INT4 group quantization, nibble packing and a
dequantizing matmul" lists, among the topics of its full test suite, a group
of zeros, sign extension of -8 and the matmul against a full dequantization.
Here weight matrices of random N(0, 0.02) rows carry edge rows, and each
kernel variant (forced through int4_matmul_path, so the shapes are chosen to
reach every block layout and group cadence) must give every output of every
edge row within 2e-3 * sum_k |x[m,k] * q[n,k] * scale| of the oracle:

  zero first / middle / last group; a whole zero row; every code -8 with the
  smallest subnormal scale (bits 0x0001, bytes 0x88); groups alternating
  between subnormal scales and a scale of 60000; hand-built bytes 0x88,
  0x08, 0x80, 0xF7, 0x7F; random codes under random subnormal scales; random
  codes under the largest scale 65504; and random codes under scales that are
  zero in some groups (a zero scale contributes nothing, whatever the codes:
  the plain definition sum_g scale_g * (x . q_g)).

Activations are N(0, 1) binary16, and a second draw where some entries are
+-60000, binary16 subnormals or zeros. The affine form (zero points 0 and 15,
zero scales) and the bias/ReLU epilogue with binary32 and binary16 output run
the same rows.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import oracle_threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3
T24 = 2.0 ** -24
H_ULP = 2.0 ** -11
H_SUB = 2.0 ** -25


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


def half_bits(v):
    return int(np.float16(v).view(np.uint16))


EDGE_ROWS = {"zero_first_group": 0, "zero_middle_group": 1, "all_minus8_subnormal": 2,
             "tiny_huge_alternating": 3, "zero_row": 4, "hand_bytes": 5, "subnormal_scales": 6,
             "max_scale": 7, "zero_scale_nonzero_codes": 8}


def edge_matrix(N, K, g, seed):
    """Symmetric codes: (packed, scales float16, row indices). Rows are
    quantized by the oracle, then some are overwritten by hand."""
    assert N >= 12
    rng = np.random.default_rng(seed)
    G = -(-K // g)
    w = rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32)
    w[0, :g] = 0.0
    w[1, (G // 2) * g:(G // 2 + 1) * g] = 0.0
    w[N - 1, (G - 1) * g:] = 0.0
    w[2, :] = np.float32(-8.0 * T24)
    for gi in range(G):
        a, b = gi * g, min(K, (gi + 1) * g)
        if gi % 2 == 0:
            w[3, a:b] = rng.integers(-8, 8, b - a) * np.float32(T24)
        else:
            v = rng.normal(0.0, 1e5, b - a).clip(-4.2e5, 4.2e5)
            v[rng.integers(0, b - a)] = 4.2e5                  # absmax 420000: scale 60000
            w[3, a:b] = v
    w[4, :] = 0.0
    packed, scales, _ = oracle.quantize_int4(w, g)
    s16 = scales.view(np.uint16).copy()
    assert np.all(s16[2] == 0x0001) and np.all(packed[2, :K // 2] == 0x88)
    assert np.all(s16[3, 1::2] == half_bits(60000.0)) and s16[0, 0] == 0 and not packed[0, :g // 2].any()
    B = packed.shape[1]
    packed[5] = np.resize(np.array([0x88, 0x08, 0x80, 0xF7, 0x7F, 0x00, 0x11, 0xFF], np.uint8), B)
    s16[5] = half_bits(0.01)
    packed[6] = rng.integers(0, 256, B, dtype=np.uint8)
    s16[6] = rng.integers(1, 1024, G)                          # subnormal binary16 scales
    packed[7] = rng.integers(0, 256, B, dtype=np.uint8)
    s16[7] = np.where(np.arange(G) % 2 == 0, 0x7BFF, half_bits(0.1))   # 65504 and 0.1
    packed[8] = rng.integers(0, 256, B, dtype=np.uint8)
    s16[8] = rng.integers(0x2000, 0x3000, G)
    s16[8, ::3] = 0x0000
    s16[8, 1::5] = 0x8000                                      # -0.0 is a zero scale too
    return packed, s16.view(np.float16)


def edge_matrix_affine(N, K, g, seed):
    """Affine codes with edge rows: (packed, scales float16, zeros uint8)."""
    rng = np.random.default_rng(seed)
    G = -(-K // g)
    w = rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32) + np.float32(0.01)
    w[0, :g] = 0.0                                             # zero group: scale 0, zp 0
    w[1, :] = np.abs(w[1, :]) + 0.5                            # positive only: zp 0
    w[2, :] = -np.abs(w[2, :]) - 0.5                           # negative only: zp 15
    w[3, :] = 0.0
    packed, scales, zeros, _ = oracle.quantize_int4_affine(w, g)
    s16 = scales.view(np.uint16).copy()
    assert np.all(zeros[1] == 0) and np.all(zeros[2] == 15) and s16[0, 0] == 0
    B = packed.shape[1]
    packed[4] = rng.integers(0, 256, B, dtype=np.uint8)
    s16[4] = rng.integers(1, 1024, G)
    zeros[4] = rng.integers(0, 16, G)
    packed[5] = rng.integers(0, 256, B, dtype=np.uint8)
    s16[5] = rng.integers(0x2000, 0x3000, G)
    s16[5, ::3] = 0
    zeros[5] = rng.integers(0, 16, G)
    packed[6] = 0xFF
    zeros[6] = 0
    s16[6] = 0x7BFF                                            # 15 * 65504 per code
    return packed, s16.view(np.float16), zeros


def activations(M, K, seed, extreme):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(M, K)).astype(np.float32)
    if extreme:
        u = rng.random(size=(M, K))
        x[u < 0.01] = 60000.0 * np.sign(x[u < 0.01])
        sub = (u >= 0.01) & (u < 0.03)
        x[sub] = rng.integers(-1023, 1024, int(sub.sum())) * T24
        x[(u >= 0.03) & (u < 0.08)] = 0.0
    return x.astype(np.float16)


def rows_of(M):
    if M <= 64:
        return np.arange(M)
    rng = np.random.default_rng(3)
    mid = rng.choice(np.arange(16, M - 16), 32, replace=False)
    return np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M), mid]))


def check(y, x, p, s, K, g, zeros=None, bias=None, relu=False, half_out=False, what=""):
    """Every column of the sampled rows of y against the oracle."""
    rows = rows_of(x.shape[0])
    ref, bound = oracle_threads.matmul(x[rows], p, s, K, g, zeros=zeros, bias=bias, relu=relu)
    ref = ref.astype(np.float64)
    yg = y[rows].astype(np.float64)
    allowed = TOL * bound + (2.0 ** -22 * np.abs(ref) if bias is not None else 0.0)
    if half_out:
        # the binary32 result lies within `allowed` of ref; binary16 rounding
        # makes it infinite from 65520 up
        lo, hi = np.abs(ref) - allowed, np.abs(ref) + allowed
        allowed = allowed + H_ULP * (np.abs(ref) + allowed) + H_SUB
        inf_ok = np.isinf(yg) & (np.sign(yg) == np.sign(ref))
        near = np.isfinite(yg) & (np.abs(yg - ref) <= allowed)
        ok = np.where(lo >= 65520.0, inf_ok, np.where(hi < 65520.0, near, inf_ok | near))
    else:
        ok = np.abs(yg - ref) <= allowed
    if not ok.all():
        bad = np.argwhere(~ok)
        m, n = bad[0]
        raise AssertionError(f"{what}: {len(bad)} outputs out of tolerance, first at row {rows[m]} "
                             f"column {n}: gpu {yg[m, n]!r} oracle {ref[m, n]!r} bound {bound[m, n]!r}")
    zero = bound == 0
    assert np.all(yg[zero] == 0.0) if bias is None else True, f"{what}: nonzero y where the bound is 0"


# (N, K, group, M, path): each forced kernel, with the block layouts and group
# cadences it has. gemv M = 1: matrix-core variant unsplit / column-split /
# group 32, the VALU variant (group 96), the whole-row variant (50 MB), the
# 4-row blocks of small matrices with columns split over 3 and 4 wavefronts
# (rows of 6, 11 and 12 column blocks); M = 2 .. 4 with four x rows, also in
# 4-row blocks over 3 wavefronts (rows of 5 and 6 column blocks). skinny:
# staged x slices (M <= 4), direct loads (M = 8, 16), two or four row groups
# per block (N >= 8192 / 16384), eight wavefronts for one row group and rows
# of 32 or more pair-blocks (K = 8192, 11008), two and four 16-row tiles
# (M = 24, 40),
# groups 32 and 64 as K-blocks of four and two groups (M = 5 .. 40, one, two
# and four row groups, rows of a single K-block; K = 64 with group 32 takes
# two-group K-blocks, K = 192 with group 64 one-group K-blocks). tiled: the 128 x 256, 128 x 128, 64 x 128 and 32 x 128 block
# tiles with 1, 2, 4 and 8 sub-steps per group, a group size decided at run
# time (1024), 32-code sub-steps (group 32), ragged N and M tails. generic:
# binary16 x.
PATH_CASES = [
    (300, 1024, 128, 1, "gemv"), (300, 8192, 128, 1, "gemv"), (300, 1024, 32, 1, "gemv"),
    (300, 1536, 96, 1, "gemv"), (12300, 8192, 128, 1, "gemv"), (300, 4096, 512, 1, "gemv"),
    (300, 4096, 256, 2, "gemv"), (300, 8192, 128, 3, "gemv"), (77, 2048, 64, 4, "gemv"),
    (300, 3072, 64, 1, "gemv"), (700, 5632, 128, 1, "gemv"), (2000, 6144, 32, 1, "gemv"),
    (300, 2560, 32, 3, "gemv"), (1000, 3072, 128, 4, "gemv"),
    (300, 2048, 128, 1, "skinny"), (300, 2048, 64, 2, "skinny"), (300, 2048, 256, 4, "skinny"),
    (300, 2048, 128, 8, "skinny"), (300, 1024, 32, 16, "skinny"), (8200, 1024, 128, 8, "skinny"),
    (16400, 1024, 128, 6, "skinny"), (16400, 2304, 256, 12, "skinny"), (8300, 4096, 128, 16, "skinny"),
    (8192, 2048, 128, 10, "skinny"), (300, 8192, 128, 16, "skinny"), (1000, 11008, 128, 5, "skinny"),
    (300, 2048, 128, 24, "skinny"), (300, 2048, 128, 40, "skinny"),
    (300, 1024, 32, 5, "skinny"), (300, 2048, 32, 24, "skinny"), (300, 1024, 32, 40, "skinny"),
    (40, 64, 32, 8, "skinny"), (33, 128, 64, 6, "skinny"), (50, 192, 64, 20, "skinny"),
    (8200, 1024, 32, 8, "skinny"), (16400, 1024, 32, 6, "skinny"),
    (300, 2048, 64, 8, "skinny"), (300, 1024, 64, 24, "skinny"), (300, 2048, 64, 40, "skinny"),
    (8200, 1024, 64, 16, "skinny"), (16400, 2048, 64, 5, "skinny"),
    (4100, 1024, 128, 1280, "tiled"), (4100, 1024, 64, 1300, "tiled"), (4100, 2048, 1024, 1280, "tiled"),
    (2050, 1024, 64, 1280, "tiled"), (2048, 2048, 256, 630, "tiled"),
    (1030, 2048, 512, 100, "tiled"), (640, 4096, 1024, 300, "tiled"), (520, 1024, 32, 200, "tiled"),
    (300, 1024, 128, 37, "tiled"),
    (300, 1024, 128, 3, "generic"),
]


@pytest.mark.parametrize("N,K,g,M,path", PATH_CASES, ids=[f"{p}-N{n}-K{k}-g{g}-M{m}" for n, k, g, m, p in PATH_CASES])
def test_edge_rows_every_kernel(dq, N, K, g, M, path):
    packed, scales = edge_matrix(N, K, g, seed=N + K + g)
    pd, sd = dev(packed), dev(scales)
    for extreme in (False, True):
        x = activations(M, K, seed=M + K, extreme=extreme)
        say(f"case: edge rows {path} N={N} K={K} g={g} M={M} extreme_x={extreme}")
        y = host(dq.int4_matmul_path(dev(x), pd, sd, K, g, path))
        check(y, x, packed, scales, K, g, what=f"{path} N={N} K={K} g={g} M={M} extreme={extreme}")


AFFINE_CASES = [(300, 1024, 128, 1, "gemv"), (12300, 8192, 128, 1, "gemv"), (300, 1536, 96, 1, "gemv"),
                (300, 4096, 128, 4, "gemv"), (300, 3072, 64, 4, "gemv"), (700, 6144, 128, 1, "gemv"),
                (300, 2048, 128, 8, "skinny"), (300, 8192, 128, 12, "skinny"), (300, 2048, 64, 2, "skinny"),
                (300, 1024, 32, 8, "skinny"), (300, 2048, 32, 24, "skinny"), (300, 2048, 64, 16, "skinny"),
                (4100, 1024, 128, 1280, "tiled"), (640, 4096, 1024, 300, "tiled"),
                (520, 1024, 32, 200, "tiled"), (300, 1024, 128, 3, "generic")]


@pytest.mark.parametrize("N,K,g,M,path", AFFINE_CASES, ids=[f"{p}-N{n}-K{k}-g{g}-M{m}" for n, k, g, m, p in AFFINE_CASES])
def test_edge_rows_affine(dq, N, K, g, M, path):
    packed, scales, zeros = edge_matrix_affine(N, K, g, seed=N + K)
    x = activations(M, K, seed=M, extreme=True)
    say(f"case: affine edge rows {path} N={N} K={K} g={g} M={M}")
    y = host(dq.int4_matmul_path(dev(x), dev(packed), dev(scales), K, g, path, zeros=dev(zeros)))
    check(y, x, packed, scales, K, g, zeros=zeros, what=f"affine {path} N={N} K={K} g={g} M={M}")


EPI_CASES = [(300, 1024, 128, 1, "gemv"), (12300, 8192, 128, 1, "gemv"), (300, 4096, 128, 3, "gemv"),
             (300, 2048, 128, 16, "skinny"), (300, 2048, 64, 16, "skinny"), (300, 1024, 32, 24, "skinny"),
             (4100, 1024, 128, 1280, "tiled"), (520, 1024, 32, 200, "tiled"),
             (300, 1024, 128, 3, "generic")]


@pytest.mark.parametrize("N,K,g,M,path", EPI_CASES, ids=[f"{p}-N{n}-K{k}-g{g}-M{m}" for n, k, g, m, p in EPI_CASES])
def test_edge_rows_epilogue(dq, N, K, g, M, path):
    """Bias and ReLU on the edge rows, binary32 output through each kernel and
    binary16 output (int4_linear, the automatic kernel choice) rounded to
    nearest even, infinite where the result passes 65504."""
    packed, scales = edge_matrix(N, K, g, seed=N + K + g)
    x = activations(M, K, seed=M + 7, extreme=False)
    b = np.random.default_rng(N).normal(0, 0.5, N).astype(np.float32)
    pd, sd, xd, bd = dev(packed), dev(scales), dev(x), dev(b)
    for relu in (False, True):
        say(f"case: edge rows epilogue {path} N={N} K={K} g={g} M={M} relu={relu}")
        y = host(dq.int4_matmul_path(xd, pd, sd, K, g, path, bias=bd, relu=relu))
        check(y, x, packed, scales, K, g, bias=b, relu=relu, what=f"epilogue {path} relu={relu}")
        if relu:
            assert np.all(y >= 0) and not np.signbit(y).any()
    yh = host(dq.int4_linear(xd, pd, sd, K, g, bias=bd, relu=True, out_dtype=torch.float16))
    check(yh, x, packed, scales, K, g, bias=b, relu=True, half_out=True, what=f"fp16 output M={M}")


@pytest.mark.parametrize("offset", [1, 2], ids=["scales-2-mod-4", "scales-4-mod-8"])
def test_multi_group_kblocks_unaligned_scales(dq, offset):
    """Groups 32 and 64 at 5 or more rows read each K-block's scales as one
    word (8 bytes for four groups of 32, 4 for two groups); scales at an
    address of 2 mod 4 take one-group K-blocks, at 4 mod 8 two-group ones,
    with and without the split of K (whose shares are then counted in those
    K-blocks). Both against the oracle."""
    for (N, K, M, g) in [(300, 1024, 16, 32), (768, 3072, 32, 32), (300, 1024, 8, 64), (768, 3072, 32, 64)]:
        packed, scales = edge_matrix(N, K, g, seed=N + M)
        G = scales.shape[1]
        buf = torch.zeros(N * G + offset, dtype=torch.float16, device=DEV)
        buf[offset:] = dev(scales).reshape(-1)
        s_odd = buf[offset:].view(N, G)
        assert s_odd.data_ptr() % 8 == 2 * offset
        x = activations(M, K, seed=M + 3, extreme=False)
        xd, pd = dev(x), dev(packed)
        say(f"case: unaligned scales (+{2 * offset} B) N={N} K={K} M={M} g={g}")
        y = host(dq.int4_matmul_path(xd, pd, s_odd, K, g, "skinny"))
        check(y, x, packed, scales, K, g, what=f"unaligned scales N={N} M={M}")
        ws = dq.linear_workspace(M, N, K, g, device=DEV)
        y = host(dq.int4_linear(xd, pd, s_odd, K, g, workspace=ws))
        check(y, x, packed, scales, K, g, what=f"unaligned scales, workspace {ws.numel()} B, N={N} M={M}")
