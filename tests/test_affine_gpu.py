"""Parity of the affine (zero-point) form of the codes with the CPU oracle on
MI355X ("Build a Blockwise INT4 Inference Engine", step 2: per-group scale and
zero point, unsigned codes, value (u - zp) * scale).

Quantize and dequantize must match the oracle byte for byte. The matmul must
satisfy |y_gpu - y_oracle| <= 2e-3 * sum_k |x[m,k] * (u[n,k] - zp) * scale| on
every output, through every kernel. Symmetric codes are affine codes with every
zero point 8 and each nibble's bit 3 flipped: on every kernel the two forms must
give bit-identical results.
"""
import numpy as np
import pytest
import torch

import oracle

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
    return t.cpu().numpy()


def say(*a):
    print(*a, flush=True)


def weights(N, K, seed, shift=0.0):
    """Gaussian rows, a few with a large outlier, shifted so that some groups do
    not straddle zero (the case the zero point exists for)."""
    rng = np.random.default_rng(seed)
    w = rng.normal(size=(N, K)).astype(np.float32) * 0.05 + np.float32(shift)
    w[rng.integers(0, N, 3), rng.integers(0, K, 3)] = 0.6
    return w


def acts(M, K, seed):
    return np.random.default_rng(seed).normal(size=(M, K)).astype(np.float16)


def check(y_gpu, x, p, s, z, K, g, bias=None, relu=False, what=""):
    y_ref, bound = oracle.int4_matmul_ex(x.astype(np.float32), p, s, K, g, bias=bias, relu=relu,
                                         with_bound=True, zeros=z)
    extra = 0.0 if bias is None else 2.0 ** -22 * np.abs(y_ref)
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > TOL * bound + extra
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs outside the bound; worst ratio "
                           f"{float(np.max(err / np.maximum(bound, 1e-300))):.3e}")


# ------------------------------------------------------------- quantize

def test_affine_hand_example_gpu(dq):
    say("case: affine [-1, 0.5, 14, 3] g=4")
    p, s, z, K = dq.quantize_int4_affine(dev(np.array([[-1.0, 0.5, 14.0, 3.0]], np.float32)), 4)
    assert host(p).tolist() == [[0x20, 0x4F]]
    assert float(host(s)[0, 0]) == 1.0 and host(z).tolist() == [[1]]
    wh = host(dq.dequantize_int4(p, s, K, 4, torch.float32, zeros=z))
    assert wh.tolist() == [[-1.0, 1.0, 14.0, 3.0]]


@pytest.mark.parametrize("N,K,g,shift", [(64, 4096, 128, 0.0), (48, 4096, 128, 0.04), (33, 1024, 32, -0.05),
                                         (40, 2048, 64, 0.0), (17, 4096, 256, 0.1), (9, 4096, 512, 0.0),
                                         (256, 8192, 128, 0.02), (5, 1000, 8, 0.0), (6, 520, 16, 0.03)])
def test_quantize_affine_bit_exact(dq, N, K, g, shift):
    say(f"case: quantize_affine N={N} K={K} g={g} shift={shift}")
    w = weights(N, K, N + K, shift)
    p, s, z, _ = dq.quantize_int4_affine(dev(w), g)
    pr, sr, zr, _ = oracle.quantize_int4_affine(w, g)
    assert np.array_equal(host(p), pr)
    assert np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))
    assert np.array_equal(host(z), zr)


@pytest.mark.parametrize("N,K,g", [(7, 301, 1), (9, 33, 3), (5, 250, 5), (6, 200, 96), (4, 100, 1000)])
def test_quantize_affine_ragged(dq, N, K, g):
    say(f"case: quantize_affine ragged N={N} K={K} g={g}")
    for shift in (0.0, 0.07):
        w = weights(N, K, 7 * K + g, shift)
        p, s, z, _ = dq.quantize_int4_affine(dev(w), g)
        pr, sr, zr, _ = oracle.quantize_int4_affine(w, g)
        assert np.array_equal(host(p), pr) and np.array_equal(host(z), zr)
        assert np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))


def test_quantize_affine_ties_and_extremes(dq):
    """Exact half-way codes with odd zero points, zero groups, constant groups,
    subnormal scales and a group beyond the binary16 range of one step."""
    say("case: quantize_affine ties/extremes")
    T = 2.0 ** -24
    w = np.array([[-1.0, 0.5, 14.0, 3.0, -1.0, 2.5, 14.0, -0.5],
                  [0, 0, 0, 0, 3.0, 3.0, 3.0, 3.0],
                  [-3.0, -3.0, -3.0, -3.0, 20 * T, -9 * T, 0, 5 * T],
                  [1e-8, -1e-8, 0, 0, 60000.0, -60000.0, 1.0, 0.0]], np.float32)
    for g in (4, 8):
        p, s, z, _ = dq.quantize_int4_affine(dev(w), g)
        pr, sr, zr, _ = oracle.quantize_int4_affine(w, g)
        assert np.array_equal(host(p), pr) and np.array_equal(host(z), zr), g
        assert np.array_equal(host(s).view(np.uint16), sr.view(np.uint16)), g


# ------------------------------------------------------------- dequantize

@pytest.mark.parametrize("N,K,g,shift", [(64, 4096, 128, 0.03), (7, 301, 1, 0.0), (9, 33, 3, 0.05),
                                         (6, 200, 96, 0.0), (40, 2048, 32, -0.04)])
def test_dequantize_affine_bit_exact(dq, N, K, g, shift):
    say(f"case: dequantize_affine N={N} K={K} g={g}")
    w = weights(N, K, 3 * K + g, shift)
    pr, sr, zr, _ = oracle.quantize_int4_affine(w, g)
    p, s, z = dev(pr), dev(sr), dev(zr)
    for dt, ndt in ((torch.float32, np.float32), (torch.float16, np.float16)):
        got = host(dq.dequantize_int4(p, s, K, g, dt, zeros=z))
        ref = oracle.dequantize_int4(pr, sr, K, g, ndt, zeros=zr)
        assert np.array_equal(got.view(np.uint32 if ndt == np.float32 else np.uint16),
                              ref.view(np.uint32 if ndt == np.float32 else np.uint16)), dt


# ------------------------------------------------------------- matmul

# (N, K, group, M, path): every kernel variant and group cadence.
MM = [
    (300, 4096, 128, 1, "gemv"),      # 4-row MFMA gemv
    (513, 2080, 32, 1, "gemv"),       # MFMA gemv, ragged column blocks
    (301, 8192, 64, 1, "gemv"),       # MFMA gemv, columns split over two wavefronts
    (77, 4096, 96, 1, "gemv"),        # VALU gemv (group not 32 * 2^p)
    (40, 32768, 128, 1, "gemv"),      # VALU gemv, long rows
    (12300, 8224, 32, 1, "gemv"),     # whole-row gemv (>= 48 MB)
    (24577, 4096, 96, 1, "gemv"),     # whole-row gemv, group 96
    (6700, 16384, 256, 1, "gemv"),    # 8 chunks per row: the VALU gemv for affine codes
    (300, 4096, 128, 3, "gemv"),      # MFMA gemv, four x rows in A (rows past M zero)
    (301, 8192, 64, 4, "gemv"),       # ... with the column split
    (513, 2080, 32, 2, "gemv"),       # ... ragged column blocks
    (200, 768, 32, 2, "skinny"),      # staged x, spread order
    (200, 1024, 128, 4, "skinny"),
    (200, 768, 64, 5, "skinny"),      # direct x loads
    (8200, 1024, 64, 9, "skinny"),    # two row groups per block
    (16400, 2048, 128, 7, "skinny"),  # four row groups per block
    (300, 4096, 128, 16, "skinny"),
    (300, 4096, 128, 40, "skinny"),   # four 16-row tiles
    (8200, 1024, 64, 24, "skinny"),   # two tiles, two row groups per block
    (8300, 2304, 256, 12, "skinny"),  # 5 to 16 rows, K split over wavefronts: 9 pair-blocks (3, 2, 2, 2)
    # tiled: 32 x 128, 64 x 128, 128 x 128 and 128 x 256 block tiles over every
    # group cadence (BK 32; a group every 1, 2, 4, 8 sub-steps; decided at run time)
    (200, 1024, 32, 40, "tiled"),
    (4096, 1024, 32, 2048, "tiled"),
    (256, 1024, 64, 300, "tiled"),
    (4096, 1024, 64, 2048, "tiled"),
    (384, 2048, 128, 70, "tiled"),
    (8192, 1024, 128, 512, "tiled"),
    (4096, 1024, 128, 512, "tiled"),
    (260, 2048, 256, 130, "tiled"),
    (4096, 1024, 512, 2048, "tiled"),
    (200, 4096, 1024, 100, "tiled"),
    (4096, 2048, 1024, 2048, "tiled"),
    (70, 301, 5, 3, "generic"),       # odd K, ragged groups
    (64, 512, 128, 8, "generic"),
]


@pytest.mark.parametrize("N,K,g,M,path", MM, ids=[f"{p}-N{N}-K{K}-g{g}-M{M}" for N, K, g, M, p in MM])
def test_matmul_affine(dq, N, K, g, M, path):
    say(f"case: matmul_affine N={N} K={K} g={g} M={M} path={path}")
    w = weights(N, K, N * 7 + K, 0.02)
    pr, sr, zr, _ = oracle.quantize_int4_affine(w, g)
    p, s, z = dev(pr), dev(sr), dev(zr)
    x = acts(M, K, M + K)
    xg = dev(x)
    y = host(dq.int4_matmul_path(xg, p, s, K, g, path, zeros=z))
    rows = np.arange(M) if M <= 64 else np.unique(np.r_[np.arange(16), np.arange(M - 16, M),
                                                        np.random.default_rng(5).choice(M, 32, replace=False)])
    cols = np.arange(N)
    if len(rows) * N * K > 3e8:
        cols = np.unique(np.r_[np.arange(16), np.arange(N - 16, N),
                               np.random.default_rng(6).choice(N, int(3e8 // (len(rows) * K)), replace=False)])
    check(y[np.ix_(rows, cols)], x[rows], pr[cols], sr[cols], zr[cols], K, g, what=path)
    b = np.random.default_rng(9).normal(size=N).astype(np.float32)
    yb = host(dq.int4_matmul_path(xg, p, s, K, g, path, bias=dev(b), relu=True, zeros=z))
    check(yb[np.ix_(rows, cols)], x[rows], pr[cols], sr[cols], zr[cols], K, g, bias=b[cols], relu=True,
          what=path + "+bias+relu")
    assert np.all(yb >= 0)


def test_matmul_affine_fp32_x(dq):
    say("case: matmul_affine fp32 x (generic)")
    N, K, g, M = 96, 1024, 128, 5
    w = weights(N, K, 11, 0.05)
    pr, sr, zr, _ = oracle.quantize_int4_affine(w, g)
    x = np.random.default_rng(12).normal(size=(M, K)).astype(np.float32)
    y = host(dq.int4_matmul(dev(x), dev(pr), dev(sr), K, g, zeros=dev(zr)))
    check(y, x, pr, sr, zr, K, g, what="fp32 x")


# (rows of 8 KB: symmetric codes take the whole-row gemv, affine codes the VALU
# gemv -- two kernels, so not bit-identical; that case is covered above)
SAME_KERNEL = [c for c in MM if not (c[1] > 14336 and c[4] == "gemv" and c[0] * c[1] // 2 >= 48 << 20)]


@pytest.mark.parametrize("N,K,g,M,path", SAME_KERNEL,
                         ids=[f"{p}-N{N}-K{K}-g{g}-M{M}" for N, K, g, M, p in SAME_KERNEL])
def test_symmetric_is_affine_at_zp8(dq, N, K, g, M, path):
    """Flipping bit 3 of every nibble and setting every zero point to 8 turns
    symmetric codes into affine codes of the same values: every kernel must give
    bit-identical outputs for the two (the same exact fp16 codes reach the same
    arithmetic)."""
    say(f"case: zp8 equivalence N={N} K={K} g={g} M={M} path={path}")
    w = weights(N, K, N + 3 * K, 0.0)
    pr, sr, K = oracle.quantize_int4(w, g)
    pa = pr ^ np.uint8(0x88)
    if K % 2:
        pa[:, -1] &= 0x0F
    z8 = np.full(sr.shape, 8, np.uint8)
    xg = dev(acts(M, K, 77))
    ys = host(dq.int4_matmul_path(xg, dev(pr), dev(sr), K, g, path))
    ya = host(dq.int4_matmul_path(xg, dev(pa), dev(sr), K, g, path, zeros=dev(z8)))
    assert np.array_equal(ys.view(np.uint32), ya.view(np.uint32))


def test_affine_auto_path_and_zero_m(dq):
    say("case: matmul_affine auto path, M = 0")
    N, K, g = 128, 2048, 128
    pr, sr, zr, _ = oracle.quantize_int4_affine(weights(N, K, 1, 0.01), g)
    p, s, z = dev(pr), dev(sr), dev(zr)
    for M in (1, 3, 24, 200):
        x = acts(M, K, M)
        check(host(dq.int4_matmul(dev(x), p, s, K, g, zeros=z)), x, pr, sr, zr, K, g, what=f"auto M={M}")
    y = dq.int4_matmul(dev(acts(0, K, 0)).reshape(0, K), p, s, K, g, zeros=z)
    assert tuple(y.shape) == (0, N)


def test_quantize_affine_near_ties(dq):
    """Affine quotients on and within a few ulps of half-integers, with odd and
    even zero points (odd ones flip which way an exact tie rounds): codes and
    zero points bit for bit with the oracle."""
    say("case: quantize_affine near-tie quotients")
    rng = np.random.default_rng(78)
    rows = []
    for (lo, hi) in ((-1.0, 14.0), (-2.0, 13.0), (-7.3, 7.7), (-0.021, 0.138), (-5.5, 9.5)):
        sf = float(np.float16(np.float32(np.float32(hi) - np.float32(lo)) / np.float32(15)))
        for h in np.arange(-6.5, 6.5, 1.0):
            for d in (0.0, 2.0 ** -24, -2.0 ** -24, 2.0 ** -21, -2.0 ** -21, 2.0 ** -18):
                row = [lo, hi]
                for j in range(6):
                    t = h + d * (j + 1) * rng.choice([-1, 1])
                    row.append(float(np.clip(np.float32(t * sf), lo, hi)))
                rows.append(row)
    w = np.array(rows, np.float32)
    p, s, z, K = dq.quantize_int4_affine(dev(w), 8)
    pr, sr, zr, _ = oracle.quantize_int4_affine(w, 8)
    assert np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))
    assert np.array_equal(host(z), zr)
    assert np.array_equal(host(p), pr)
