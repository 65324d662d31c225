"""Parity of the HIP path with the CPU oracle on MI355X.

Quantize, pack and unpack must match the oracle byte for byte; the matmul must
satisfy |y_gpu - y_oracle| <= 2e-3 * sum_k |x[m,k] * q[n,k] * scale| for every
checked output (exact zero where that sum is zero). Inputs are the seeded
synthetic configurations of ``workloads.py`` at their full sizes; where the
oracle cannot compute every output of a large case in seconds, it computes
every column of a fixed sample of 64 rows of y (the first and last 16 and 32
seeded ones between), and the GPU result is compared there.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import oracle_threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


def gemv_takes(M, K, g):
    """Whether the gemv path takes M rows (M = 1 always; 2 .. 4 with K <= 12288
    and group 32 * 2^p)."""
    if M == 1:
        return True
    q, r = divmod(g, 32)
    return 2 <= M <= 4 and K <= 12288 and r == 0 and q & (q - 1) == 0


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


ALL_CASES = [(cfg.key, c) for cfg in workloads.CONFIGS.values() for c in cfg.cases]


@functools.lru_cache(maxsize=2)
def _case_data(key, name):
    case = next(c for (k, c) in ALL_CASES if k == key and c.name == name)
    w = workloads.weights(case)
    p, s, K = oracle.quantize_int4(w, case.group)
    return case, w, p, s


def sample_rows_cols(M, N, K):
    """Rows of y the oracle computes: all of them up to 64, else rows 0-15, the
    last 16 and 32 drawn with seed 3 between them. Every column is checked
    (the oracle runs over column blocks on a few host threads)."""
    rows = np.arange(M)
    if M > 64:
        rng = np.random.default_rng(3)
        mid = rng.choice(np.arange(16, M - 16), 32, replace=False)
        rows = np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M), mid]))
    return rows, np.arange(N)


def check_matmul(y_gpu, x, p, s, K, g, rows=None, cols=None, what=""):
    M, N = y_gpu.shape
    if rows is None or cols is None:
        rows, cols = sample_rows_cols(M, N, K)
    xs = np.ascontiguousarray(x[rows])
    if len(cols) == N:
        y_ref, bound = oracle_threads.matmul(xs, p, s, K, g)
    else:
        y_ref, bound = oracle.int4_matmul(xs, p[cols], s[cols], K, g, with_bound=True)
    yg = y_gpu[np.ix_(rows, cols)].astype(np.float64)
    err = np.abs(yg - y_ref)
    bad = err > TOL * bound
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} outputs outside 2e-3*bound; worst ratio "
        f"{float(np.max(err / np.maximum(bound, 1e-300))):.3e}")
    return float(np.max(err / np.maximum(bound, 1e-300)))


# ---------------------------------------------------------------- page pins

def test_p4_nibble_layout_gpu(dq):
    say("case: drill-page layout [1,-1,7,-7] g=4 and an 8-wide copy at g=8")
    p, s, K = dq.quantize_int4(dev(np.array([[1.0, -1.0, 7.0, -7.0]], np.float32)), 4)
    assert host(p).tolist() == [[0xF1, 0x97]] and float(host(s)[0, 0]) == 1.0
    p, s, K = dq.quantize_int4(dev(np.array([[1.0, -1.0, 7.0, -7.0] * 2], np.float32)), 8)
    assert host(p).tolist() == [[0xF1, 0x97, 0xF1, 0x97]] and float(host(s)[0, 0]) == 1.0


def test_p4_round_trip_gpu(dq):
    """The drill page's visible test "round-trip error stays within half a
    step", on the GPU's codes: per row and group, every weight dequantized
    from the GPU's bytes and scales (by the oracle) lies within (1/2 + 1e-3)
    of the group's step of the original, plus 1e-6."""
    for seed in range(20):
        w = np.random.default_rng(seed).normal(size=(8, 256)).astype(np.float32)
        p, s, K = dq.quantize_int4(dev(w), 128)
        sh = host(s)
        w_hat = oracle.dequantize_int4(host(p), sh, K, 128, np.float32)
        for row in range(8):
            for gi in range(sh.shape[1]):
                cols = slice(gi * 128, (gi + 1) * 128)
                worst = float(np.max(np.abs(w_hat[row, cols].astype(np.float64) - w[row, cols])))
                assert worst <= (0.5 + 1e-3) * float(sh[row, gi]) + 1e-6, (seed, row, gi)


def test_ties_and_clamps_gpu(dq):
    say("case: ties to even, -8 clamp, zero groups, 8-wide and 4-wide groups")
    T = 2.0 ** -24
    w = np.array([[0.5, 2.5, 7.0, -7.0, -0.5, -2.5, 7.0, 1.5],
                  [-9.5 * T, 0, 0, 0, 7.6 * T, 0, 0, 0],
                  [0, 0, 0, 0, 1e-8, -1e-8, 0, 0]], np.float32)
    for g in (4, 8):
        p, s, K = dq.quantize_int4(dev(w), g)
        pr, sr, _ = oracle.quantize_int4(w, g)
        assert np.array_equal(host(p), pr) and np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))
    p, _, _ = dq.quantize_int4(dev(w), 4)
    assert host(p)[0].tolist() == [0x20, 0x97, 0xE0, 0x27]


# ---------------------------------------------------- quantize / unpack parity

@pytest.mark.parametrize("key,case", ALL_CASES, ids=[f"{k}-{c.name}" for k, c in ALL_CASES])
def test_quantize_unpack_bit_exact(dq, key, case):
    say(f"case: quantize+unpack {key} {case.name} [{case.N},{case.K}] g={case.group}")
    _, w, p_ref, s_ref = _case_data(key, case.name)
    wd = dev(w)
    p, s, K = dq.quantize_int4(wd, case.group)
    ph, sh = host(p), host(s)
    assert np.array_equal(sh.view(np.uint16), s_ref.view(np.uint16)), "scales differ"
    assert np.array_equal(ph, p_ref), f"packed differs at {np.argwhere(ph != p_ref)[:3].tolist()}"
    q = host(dq.unpack_int4(p, K))
    assert np.array_equal(q, oracle.unpack_int4(p_ref, K))
    if case.edge_rows:
        assert np.all(sh.view(np.uint16)[7] == 0x0001)
        assert np.all(ph[7, :-1] == 0x88) and ph[7, -1] == 0x08
        assert sh.view(np.uint16)[5, 0] == 0 and np.all(ph[5, :64] == 0)
        assert np.all(q[7] == -8)
    del wd


@pytest.mark.parametrize("N,K,g", [(7, 301, 1), (9, 33, 3), (5, 250, 5), (6, 200, 96),
                                   (4, 777, 100), (3, 2048, 1024), (17, 64, 8), (33, 4104, 512),
                                   (2, 9, 16), (1, 1, 1)])
def test_quantize_ragged_groups(dq, N, K, g):
    say(f"case: quantize ragged N={N} K={K} g={g}")
    w = np.random.default_rng(N * K + g).normal(0, 0.3, size=(N, K)).astype(np.float32)
    w[0, : min(g, K)] = 0.0
    p, s, KK = dq.quantize_int4(dev(w), g)
    pr, sr, _ = oracle.quantize_int4(w, g)
    assert np.array_equal(host(p), pr) and np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))
    assert np.array_equal(host(dq.unpack_int4(p, KK)), oracle.unpack_int4(pr, KK))


def test_quantize_unaligned_input(dq):
    """An input that starts 4 bytes past an allocation runs the general kernels."""
    say("case: quantize unaligned base pointer [64,512] g=128")
    w = np.random.default_rng(8).normal(size=(64, 512)).astype(np.float32)
    buf = torch.zeros(64 * 512 + 1, dtype=torch.float32, device=DEV)
    buf[1:] = dev(w.reshape(-1))
    view = buf[1:].view(64, 512)
    p, s, K = dq.quantize_int4(view, 128)
    pr, sr, _ = oracle.quantize_int4(w, 128)
    assert np.array_equal(host(p), pr) and np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))


def test_unpack_exhaustive_gpu(dq):
    b = np.arange(256, dtype=np.uint8)[None, :]
    for K in (512, 511):
        bb = b if K == 512 else b.copy()
        out = host(dq.unpack_int4(dev(bb), K))
        assert np.array_equal(out, oracle.unpack_int4(bb, K))
    big = np.random.default_rng(6).integers(0, 256, size=(37, 1001), dtype=np.uint8)
    for K in (2002, 2001):
        assert np.array_equal(host(dq.unpack_int4(dev(big), K)), oracle.unpack_int4(big, K))


def test_guard_bytes(dq):
    """Outputs written through the C ABI into the middle of larger buffers leave
    the surrounding canary bytes untouched (odd K pad byte included)."""
    say("case: guard bytes around quantize/unpack/matmul outputs")
    N, K, g, M = 21, 301, 128, 5
    w = np.random.default_rng(2).normal(size=(N, K)).astype(np.float32)
    x = np.random.default_rng(3).normal(size=(M, K)).astype(np.float16)
    G, B, pad = 3, 151, 64
    pbuf = torch.full((N * B + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((N * G + 2 * pad,), 0x5A5A, dtype=torch.int16, device=DEV)
    obuf = torch.full((N * K + 2 * pad,), -91, dtype=torch.int8, device=DEV)
    ybuf = torch.full((M * N + 2 * pad,), 123.0, dtype=torch.float32, device=DEV)
    wd, xd = dev(w), dev(x)
    L = dq.lib
    stream = torch.cuda.current_stream().cuda_stream
    assert L.int4_quantize(wd.data_ptr(), N, K, g, pbuf.data_ptr() + pad, sbuf.data_ptr() + 2 * pad, stream) == 0
    assert L.int4_unpack(pbuf.data_ptr() + pad, N, K, obuf.data_ptr() + pad, stream) == 0
    assert L.int4_matmul(xd.data_ptr(), 1, M, pbuf.data_ptr() + pad, sbuf.data_ptr() + 2 * pad, N, K, g,
                         ybuf.data_ptr() + 4 * pad, stream) == 0
    ph, sh, oh, yh = host(pbuf), host(sbuf), host(obuf), host(ybuf)
    assert np.all(ph[:pad] == 0xA5) and np.all(ph[-pad:] == 0xA5)
    assert np.all(sh[:pad] == 0x5A5A) and np.all(sh[-pad:] == 0x5A5A)
    assert np.all(oh[:pad] == -91) and np.all(oh[-pad:] == -91)
    assert np.all(yh[:pad] == 123.0) and np.all(yh[-pad:] == 123.0)
    pr, sr, _ = oracle.quantize_int4(w, g)
    assert np.array_equal(ph[pad:-pad].reshape(N, B), pr)
    check_matmul(yh[pad:-pad].reshape(M, N), x, pr, sr, K, g, what="guarded")


# --------------------------------------------------------- dequantize parity

@pytest.mark.parametrize("key,case", ALL_CASES, ids=[f"{k}-{c.name}" for k, c in ALL_CASES])
def test_dequantize_bit_exact(dq, key, case):
    """w_hat = q * scale on every config's matrices: float32 exactly, float16
    rounded to nearest even, both bit for bit against the oracle."""
    _, w, p_ref, s_ref = _case_data(key, case.name)
    say(f"case: dequantize {key} {case.name} [{case.N},{case.K}] g={case.group}")
    pd, sd = dev(p_ref), dev(s_ref)
    for dt, npdt in ((torch.float32, np.float32), (torch.float16, np.float16)):
        got = host(dq.dequantize_int4(pd, sd, case.K, case.group, dtype=dt))
        ref = oracle.dequantize_int4(p_ref, s_ref, case.K, case.group, dtype=npdt)
        view = np.uint32 if npdt == np.float32 else np.uint16
        assert np.array_equal(got.view(view), ref.view(view)), f"{key}/{case.name} {npdt.__name__}"


@pytest.mark.parametrize("N,K,g,off", [(7, 301, 1, 0), (9, 33, 3, 0), (6, 200, 96, 0), (5, 64, 32, 1),
                                       (40, 1000, 7, 0), (3, 4096, 128, 2), (130, 96, 48, 0)])
def test_dequantize_ragged_and_unaligned(dq, N, K, g, off):
    """The element-wise kernel: odd K, groups that are not multiples of 32, and
    packed data or output at offsets that are not 16-byte aligned."""
    say(f"case: dequantize ragged N={N} K={K} g={g} offset={off}")
    w = np.random.default_rng(N * K).normal(size=(N, K)).astype(np.float32)
    pr, sr, _ = oracle.quantize_int4(w, g)
    B = (K + 1) // 2
    pbuf = torch.zeros(N * B + off, dtype=torch.uint8, device="cuda")
    pbuf[off:] = dev(pr).reshape(-1)
    sd = dev(sr)
    for dt, npdt in ((torch.float32, np.float32), (torch.float16, np.float16)):
        obuf = torch.full((N * K + off,), 7.0, dtype=dt, device="cuda")
        rc = dq.lib.int4_dequantize(pbuf.data_ptr() + off, sd.data_ptr(), N, K, g,
                                    dq.OUT_F16 if dt == torch.float16 else dq.OUT_F32,
                                    obuf.data_ptr() + off * obuf.element_size(),
                                    torch.cuda.current_stream().cuda_stream)
        assert rc == 0, dq.lib.int4_last_error()
        got = host(obuf)
        assert np.all(got[:off] == 7.0)
        ref = oracle.dequantize_int4(pr, sr, K, g, dtype=npdt)
        view = np.uint32 if npdt == np.float32 else np.uint16
        assert np.array_equal(got[off:].reshape(N, K).view(view), ref.view(view)), npdt.__name__


def test_dequantize_extremes(dq):
    """Subnormal scales (c2's -8 * 2^-24 row) and binary16 overflow of
    -8 * 65504 in the float16 output, through both kernels."""
    say("case: dequantize extremes")
    for K, g in ((64, 32), (6, 6)):
        packed = np.full((2, K // 2), 0x88, np.uint8)                  # every code -8
        scales = np.array([[0x0001] * (K // g), [0x7BFF] * (K // g)], np.uint16).view(np.float16)
        for dt, npdt in ((torch.float32, np.float32), (torch.float16, np.float16)):
            got = host(dq.dequantize_int4(dev(packed), dev(scales), K, g, dtype=dt))
            ref = oracle.dequantize_int4(packed, scales, K, g, dtype=npdt)
            view = np.uint32 if npdt == np.float32 else np.uint16
            assert np.array_equal(got.view(view), ref.view(view)), (K, npdt.__name__)
        assert float(got[0, 0]) == -8 * 2.0 ** -24 and np.isneginf(got[1, 0])


# ------------------------------------------------------------- matmul parity

MM_CASES = [(k, c, M) for (k, c) in ALL_CASES for M in c.Ms]


@pytest.mark.parametrize("key,case,M", MM_CASES, ids=[f"{k}-{c.name}-M{M}" for k, c, M in MM_CASES])
def test_matmul_configs(dq, key, case, M):
    _, w, p_ref, s_ref = _case_data(key, case.name)
    x = workloads.activations(M, case.K, case.x_dtype)
    pd, sd, xd = dev(p_ref), dev(s_ref), dev(x)
    path = dq.matmul_select(xd, pd, sd, case.K, case.group)
    say(f"case: matmul {key} {case.name} [{case.N},{case.K}] g={case.group} M={M} "
        f"x={case.x_dtype} kernel={path}")
    y = host(dq.int4_matmul(xd, pd, sd, case.K, case.group))
    r = check_matmul(y, x, p_ref, s_ref, case.K, case.group, what=f"{key}/{case.name}/M{M}")
    say(f"  max |err|/bound = {r:.2e}")


@pytest.mark.parametrize("N,K,g,M", [(200, 768, 64, 1), (200, 768, 32, 5), (48, 4096, 128, 16),
                                     (136, 1024, 256, 3), (50, 512, 128, 200), (300, 1024, 128, 130),
                                     (129, 256, 32, 257), (64, 2048, 64, 100),
                                     (16400, 2048, 128, 7), (8200, 1024, 64, 9), (9000, 8192, 128, 16),
                                     # 17-64 rows: two or four 16-row tiles in the skinny kernel, one or
                                     # two row groups per block, up to the largest K each form takes
                                     (200, 768, 32, 24), (300, 4096, 128, 64), (8200, 1024, 64, 40),
                                     (16400, 2048, 128, 20), (300, 12288, 128, 48), (64, 16384, 128, 30),
                                     (77, 2048, 128, 33),
                                     # tiled block tiles 64 x 128 and 128 x 128 (four wavefronts along N)
                                     (2048, 1024, 64, 700), (3000, 512, 128, 1100)])
def test_matmul_kernels_agree(dq, N, K, g, M):
    """Every kernel that takes a shape matches the oracle on it (ragged M and N tails)."""
    w = np.random.default_rng(N + K).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = np.random.default_rng(M).normal(size=(M, K)).astype(np.float16)
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd, xd = dev(pr), dev(sr), dev(x)
    for path in ("generic", "skinny", "tiled", "gemv"):
        if (path == "skinny" and (M > 64 or (M > 32 and K // min(g, 128) > 96))) or \
                (path == "gemv" and not gemv_takes(M, K, g)):
            continue
        say(f"case: kernel {path} N={N} K={K} g={g} M={M}")
        y = host(dq.int4_matmul_path(xd, pd, sd, K, g, path))
        check_matmul(y, x, pr, sr, K, g, what=path)


@pytest.mark.parametrize("N,K,g", [(300, 11008, 128), (301, 8192, 64), (4099, 7680, 256), (77, 4096, 96),
                                   (513, 2080, 32), (40, 32768, 128),
                                   (10, 32, 32), (4099, 4096, 128), (8195, 4096, 64), (2051, 2048, 128),
                                   (12300, 8224, 32), (24577, 4096, 96), (6700, 16384, 256)])
def test_matmul_gemv_shapes(dq, N, K, g):
    """The M = 1 kernels: a partial last 1 KB chunk (K = 11008, 2080), a group
    that is not a power of two (96), the largest K (16 chunks), the smallest
    (one lane), N tails for 1, 2 and 4 rows per block; and matrices of 48 MB
    and more, which take the whole-row variant (partial last chunk, group 96,
    its largest K, 16384, ragged rows per wavefront)."""
    say(f"case: gemv N={N} K={K} g={g}")
    w = np.random.default_rng(N + K).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = np.random.default_rng(K).normal(size=(1, K)).astype(np.float16)
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd, xd = dev(pr), dev(sr), dev(x)
    assert dq.matmul_select(xd, pd, sd, K, g) == "gemv"
    y = host(dq.int4_matmul_path(xd, pd, sd, K, g, "gemv"))
    check_matmul(y, x, pr, sr, K, g, what=f"gemv {N}x{K}")


@pytest.mark.parametrize("N,K,g,M", [(300, 11008, 128, 4), (4099, 4096, 128, 2), (513, 2080, 32, 3),
                                     (77, 7680, 256, 4), (10, 32, 32, 3), (8200, 12288, 64, 4),
                                     (2051, 2048, 128, 3), (28672, 8192, 128, 4), (40, 768, 32, 2)])
def test_matmul_gemv_multi_row(dq, N, K, g, M):
    """M = 2 .. 4 through the matrix-core gemv (four x rows in A, rows past M
    zero): column splits for rows of 16 or more column blocks (K = 7680 ..
    12288), a partial last column block (K = 2080), the smallest K (one
    lane), the largest (24 column blocks), N tails, the c5 matrix."""
    say(f"case: gemv M={M} N={N} K={K} g={g}")
    w = np.random.default_rng(N + K + M).normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = np.random.default_rng(K + M).normal(size=(M, K)).astype(np.float16)
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd, xd = dev(pr), dev(sr), dev(x)
    assert dq.matmul_select(xd, pd, sd, K, g) == "gemv"
    y = host(dq.int4_matmul_path(xd, pd, sd, K, g, "gemv"))
    check_matmul(y, x, pr, sr, K, g, what=f"gemv M={M} {N}x{K}")


def test_matmul_gemv_multi_row_one_hot_exact(dq):
    """Four one-hot rows of x through the M = 2 .. 4 gemv: row m of y is
    column k_m of (q * scale)^T bit-exactly (one exact product per output)."""
    for (N, K, g) in [(48, 4096, 128), (300, 11008, 128), (32, 768, 32)]:
        say(f"case: gemv multi-row one-hot N={N} K={K} g={g}")
        w = np.random.default_rng(K + 1).normal(size=(N, K)).astype(np.float32)
        pr, sr, _ = oracle.quantize_int4(w, g)
        what = (oracle.unpack_int4(pr, K).astype(np.float64) *
                np.repeat(sr.astype(np.float64), g, 1)[:, :K]).T
        ks = [0, 33, K // 2 + 7, K - 1]
        for M in (2, 3, 4):
            e = np.zeros((M, K), dtype=np.float16)
            for m in range(M):
                e[m, ks[m]] = 1.0
            y = host(dq.int4_matmul_path(dev(e), dev(pr), dev(sr), K, g, "gemv"))
            for m in range(M):
                assert np.array_equal(y[m].astype(np.float64), what[ks[m]]), f"M={M} m={m}"


def test_matmul_gemv_one_hot_exact(dq):
    """One-hot x through the M = 1 kernel gives column k of (q * scale)^T
    bit-exactly: one exact product per output, zeros elsewhere."""
    for (N, K, g) in [(48, 4096, 128), (300, 11008, 128), (32, 768, 32)]:
        say(f"case: gemv one-hot N={N} K={K} g={g}")
        w = np.random.default_rng(K).normal(size=(N, K)).astype(np.float32)
        pr, sr, _ = oracle.quantize_int4(w, g)
        what = (oracle.unpack_int4(pr, K).astype(np.float64) *
                np.repeat(sr.astype(np.float64), g, 1)[:, :K]).T
        pd, sd = dev(pr), dev(sr)
        for k in sorted({0, 1, 31, 32, K // 2 + 7, K - 33, K - 1}):
            e = np.zeros((1, K), dtype=np.float16)
            e[0, k] = 1.0
            y = host(dq.int4_matmul_path(dev(e), pd, sd, K, g, "gemv"))
            assert np.array_equal(y[0].astype(np.float64), what[k]), f"k={k}"


def test_matmul_gemv_rows_one_hot_exact(dq):
    """One-hot x through the whole-row M = 1 variant (a 50 MB matrix, partial
    last chunk): column k of (q * scale)^T bit-exactly."""
    N, K, g = 12300, 8224, 32
    say(f"case: gemv rows one-hot N={N} K={K} g={g}")
    w = np.random.default_rng(5).normal(size=(N, K)).astype(np.float32)
    pr, sr, _ = oracle.quantize_int4(w, g)
    q = oracle.unpack_int4(pr, K)
    pd, sd = dev(pr), dev(sr)
    for k in (0, 1, 31, 32, 4111, 8191, 8192, K - 1):
        e = np.zeros((1, K), dtype=np.float16)
        e[0, k] = 1.0
        y = host(dq.int4_matmul_path(dev(e), pd, sd, K, g, "gemv"))
        col = q[:, k].astype(np.float64) * sr[:, k // g].astype(np.float64)
        assert np.array_equal(y[0].astype(np.float64), col), f"k={k}"


@pytest.mark.parametrize("N,K,g,M,path", [(300, 1024, 128, 1, "gemv"), (200, 768, 32, 1, "gemv"),
                                          (12300, 8224, 32, 1, "gemv"), (77, 4096, 96, 1, "gemv"),
                                          (301, 11008, 128, 1, "gemv"), (300, 1024, 128, 3, "gemv"),
                                          (301, 11008, 128, 4, "gemv"),
                                          (200, 768, 64, 5, "skinny"), (48, 4096, 128, 16, "skinny"),
                                          (300, 4096, 128, 64, "skinny"), (8200, 1024, 64, 24, "skinny"),
                                          (300, 1024, 128, 130, "tiled"), (129, 256, 32, 600, "tiled"),
                                          (640, 2048, 128, 520, "tiled"), (10880, 256, 64, 300, "tiled"),
                                          (4096, 256, 128, 1600, "tiled"), (4096, 512, 128, 512, "tiled"),
                                          (40, 1000, 7, 6, "generic")])
def test_matmul_epilogue(dq, N, K, g, M, path):
    """The engine page's epilogue act(x @ w_hat.T + bias) through every kernel
    (all three M = 1 variants, the 64/128/256-row tiles, the generic kernel):
    within 2e-3 * bound + 2^-22 * |y| of the oracle, ReLU giving +0 for every
    non-positive value."""
    say(f"case: epilogue {path} N={N} K={K} g={g} M={M}")
    rng = np.random.default_rng(N + M)
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = rng.normal(size=(M, K)).astype(np.float16 if path != "generic" else np.float32)
    b = rng.normal(0, 0.5, size=N).astype(np.float32)
    pr, sr, _ = oracle.quantize_int4(w, g)
    pd, sd, xd, bd = dev(pr), dev(sr), dev(x), dev(b)
    rows = sample_rows_cols(M, N, K)[0] if M > 64 else np.arange(M)
    for relu in (False, True):
        y = host(dq.int4_matmul_path(xd, pd, sd, K, g, path, bias=bd, relu=relu))[rows]
        ref, bound = oracle.int4_matmul_ex(x[rows], pr, sr, K, g, bias=b, relu=relu, with_bound=True)
        err = np.abs(y.astype(np.float64) - ref)
        ok = err <= TOL * bound + 2.0 ** -22 * np.abs(ref) + 1e-30
        assert ok.all(), f"{path} relu={relu}: {int((~ok).sum())} outputs out of tolerance"
        if relu:
            assert np.all(y >= 0) and not np.signbit(y).any()
    y0 = host(dq.int4_matmul_path(xd, pd, sd, K, g, path))
    assert np.array_equal(host(dq.int4_matmul_path(xd, pd, sd, K, g, path, bias=torch.zeros_like(bd))), y0)


@pytest.mark.parametrize("g", [128, 64])
def test_tiled_tile_order_ragged(dq, g):
    """The tiled kernel's per-XCD tile order (taken when the grid is a
    multiple of 8 tiles and of 4 tile rows) on a grid whose last row and
    column of 128 x 256 tiles are partial: M = 1000 (8 tile rows, the last
    one 104 rows), N = 5000 (20 tile columns, the last one 136 columns);
    symmetric and affine codes against the oracle (64 sampled rows, every
    column)."""
    N, K, M = 5000, 512, 1000
    say(f"case: tiled tile order, ragged edges N={N} K={K} g={g} M={M}")
    rng = np.random.default_rng(g)
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    x = rng.normal(size=(M, K)).astype(np.float16)
    pr, sr, _ = oracle.quantize_int4(w, g)
    xd, pd, sd = dev(x), dev(pr), dev(sr)
    assert dq.matmul_select(xd, pd, sd, K, g) == "tiled"
    check_matmul(host(dq.int4_matmul(xd, pd, sd, K, g)), x, pr, sr, K, g, what=f"tile order g={g}")
    pa, sa, za, _ = oracle.quantize_int4_affine(w, g)
    rows = sample_rows_cols(M, N, K)[0]
    ya = host(dq.int4_matmul(xd, dev(pa), dev(sa), K, g, zeros=dev(za)))[rows]
    ref, bound = oracle.int4_matmul_ex(x[rows], pa, sa, K, g, zeros=za, with_bound=True)
    err = np.abs(ya.astype(np.float64) - ref)
    assert np.all(err <= TOL * bound), f"affine tile order g={g}: {int((err > TOL * bound).sum())} outputs"


def test_matmul_fp32_x(dq):
    say("case: binary32 activations, c1/c2 shapes and a [40,1000] g=7 matrix")
    for (N, K, g, M) in [(64, 256, 128, 4), (48, 301, 128, 3), (40, 1000, 7, 6)]:
        w = np.random.default_rng(K).normal(size=(N, K)).astype(np.float32)
        x = np.random.default_rng(M).normal(size=(M, K)).astype(np.float32)
        pr, sr, _ = oracle.quantize_int4(w, g)
        y = host(dq.int4_matmul(dev(x), dev(pr), dev(sr), K, g))
        check_matmul(y, x, pr, sr, K, g, what=f"fp32 {N}x{K}")


def test_matmul_one_hot_exact(dq):
    """x = identity gives y = (q * scale)^T: one product per output. The skinny
    kernel forms each group's integer sum and scales it in binary32, so it is
    exact. The tiled kernel multiplies each code by its scale in binary16
    before the MFMA, so it gives q * scale rounded once to binary16: bit for
    bit the oracle's binary16 dequantization (an index error would be O(1)).
    Tiled kernel at M = K = 256 and 4096; skinny kernel on 16-row slices."""
    for (N, K, g) in [(48, 256, 128), (64, 4096, 128), (32, 768, 64), (32, 768, 32)]:
        say(f"case: one-hot N={N} K={K} g={g}")
        w = np.random.default_rng(K).normal(size=(N, K)).astype(np.float32)
        pr, sr, _ = oracle.quantize_int4(w, g)
        what = (oracle.unpack_int4(pr, K).astype(np.float64) *
                np.repeat(sr.astype(np.float64), g, 1)[:, :K]).T
        what16 = oracle.dequantize_int4(pr, sr, K, g, dtype=np.float16).astype(np.float64).T
        eye = dev(np.eye(K, dtype=np.float16))
        pd, sd = dev(pr), dev(sr)
        y = host(dq.int4_matmul_path(eye, pd, sd, K, g, "tiled"))
        assert np.array_equal(y.astype(np.float64), what16)
        for r0 in (0, K // 2, K - 16):
            ys = host(dq.int4_matmul_path(eye[r0:r0 + 16].contiguous(), pd, sd, K, g, "skinny"))
            assert np.array_equal(ys.astype(np.float64), what[r0:r0 + 16])


def test_matmul_zero_and_empty(dq):
    w = np.random.default_rng(1).normal(size=(64, 512)).astype(np.float32)
    pr, sr, _ = oracle.quantize_int4(w, 128)
    pd, sd = dev(pr), dev(sr)
    for M in (1, 3, 16, 300):
        for path in ("skinny", "tiled", "generic", "gemv"):
            if (path == "skinny" and M > 16) or (path == "gemv" and not gemv_takes(M, 512, 128)):
                continue
            y = host(dq.int4_matmul_path(torch.zeros(M, 512, dtype=torch.float16, device=DEV), pd, sd, 512, 128, path))
            assert np.all(y == 0)
    y = dq.int4_matmul(torch.zeros(0, 512, dtype=torch.float16, device=DEV), pd, sd, 512, 128)
    assert tuple(y.shape) == (0, 64)


def test_matmul_deterministic(dq):
    """No atomics: two calls give the same bits."""
    w = np.random.default_rng(1).normal(0, 0.02, size=(1024, 4096)).astype(np.float32)
    pr, sr, _ = oracle.quantize_int4(w, 128)
    pd, sd = dev(pr), dev(sr)
    for M in (1, 16, 512):
        x = dev(np.random.default_rng(M).normal(size=(M, 4096)).astype(np.float16))
        a = host(dq.int4_matmul(x, pd, sd, 4096, 128))
        b = host(dq.int4_matmul(x, pd, sd, 4096, 128))
        assert np.array_equal(a, b)


def test_rows_independent(dq):
    """Row m of an M-row call equals the 1-row call on x[m] within tolerance."""
    case, w, pr, sr = _case_data("c4", "q_proj_4096x4096")
    x = workloads.activations(512, 4096)
    pd, sd = dev(pr), dev(sr)
    big = host(dq.int4_matmul(dev(x), pd, sd, 4096, 128))
    for m in (0, 255, 511):
        one = host(dq.int4_matmul(dev(x[m:m + 1]), pd, sd, 4096, 128))
        _, bound = oracle.int4_matmul(x[m:m + 1], pr, sr, 4096, 128, with_bound=True)
        assert np.all(np.abs(one[0] - big[m]) <= 2 * TOL * bound[0])


def _near_tie_rows(rng, lo_h, hi_h, scales):
    """Rows of 8 weights whose quotients w / scale sit on and a few ulps
    around half-integers (the cases where a reciprocal multiply could round
    the other way); element 0 fixes the group's scale."""
    rows = []
    for s_target in scales:
        for h in np.arange(lo_h, hi_h + 0.5, 1.0):
            for d in (0.0, 2.0 ** -24, -2.0 ** -24, 2.0 ** -22, -2.0 ** -22, 2.0 ** -19, -2.0 ** -19):
                row = [s_target[0]]
                for j in range(7):
                    t = h + d * (j + 1) * rng.choice([-1, 1])
                    row.append(np.float32(t * s_target[1]))
                rows.append(row)
    return np.array(rows, np.float32)


def test_quantize_near_ties_gpu(dq):
    """Quotients on and within a few ulps of every half-integer code boundary
    (-7.5 .. 6.5) for several non-power-of-two scales: the codes must equal the
    oracle's (IEEE division, ties to even) bit for bit."""
    say("case: quantize near-tie quotients")
    rng = np.random.default_rng(77)
    sc = []
    for target in (0.7, 1.3, 0.0123, 3.7e-3, 5.1):
        sf = float(np.float16(np.float32(np.float32(7 * target) / np.float32(7))))
        sc.append((np.float32(7 * target), sf))
    w = _near_tie_rows(rng, -7.5, 6.5, sc)
    p, s, K = dq.quantize_int4(dev(w), 8)
    pr, sr, _ = oracle.quantize_int4(w, 8)
    assert np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))
    assert np.array_equal(host(p), pr)
