"""The element-wise kernels past one pass of their capped grid, against the oracle.

A dispatch holds fewer than 2^32 work items per grid dimension, so the kernels
that put one thread (or one wavefront) on each element launch at most 2^16
blocks of 256 threads and stride over the rest. Each case here is sized just
past one pass of that grid, so its last elements are produced by the second
trip through the loop: quantize and its affine form on the general path
(group 2), unpack with an odd K (row kernel) and with an even K (flat
kernel, 256 MiB of packed bytes), dequantize with an odd K (element kernel)
and the generic matmul with binary32 and binary16 x. Quantize, unpack and
dequantize must match the oracle byte for byte; the matmul must be within
2e-3 * sum_k |x[m,k] * q[n,k] * scale| of it.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3
PASS_THREADS = (1 << 16) * 256        # threads of one pass of the capped grid
PASS_WAVES = (1 << 16) * 4            # wavefronts of one pass (generic matmul: one per output)


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


def gauss(N, K, seed, shift=0.0):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(N, K)).astype(np.float32) * np.float32(0.05) + np.float32(shift))


def test_quantize_general_path_two_passes(dq):
    N, K, g = 4100, 8193, 2                    # N * ceil(K / 2) and N * G past one pass
    assert N * ((K + 1) // 2) > PASS_THREADS and N * ((K + g - 1) // g) > PASS_THREADS
    say(f"quantize general path N={N} K={K} group={g}")
    w = gauss(N, K, 11)
    p, s, _ = dq.quantize_int4(dev(w), g)
    pr, sr, _ = oracle.quantize_int4(w, g)
    assert np.array_equal(host(p), pr)
    assert np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))
    say(f"quantize_affine general path N={N} K={K} group={g}")
    p, s, z, _ = dq.quantize_int4_affine(dev(gauss(N, K, 12, 0.03)), g)
    pr, sr, zr, _ = oracle.quantize_int4_affine(gauss(N, K, 12, 0.03), g)
    assert np.array_equal(host(p), pr) and np.array_equal(host(z), zr)
    assert np.array_equal(host(s).view(np.uint16), sr.view(np.uint16))


def test_unpack_rows_two_passes(dq):
    N, K = 4100, 8193                          # odd K: one thread per packed byte
    assert N * ((K + 1) // 2) > PASS_THREADS
    say(f"unpack odd K N={N} K={K}")
    rng = np.random.default_rng(13)
    packed = rng.integers(0, 256, size=(N, (K + 1) // 2), dtype=np.uint8)
    packed[:, -1] &= 0x0F                      # the pad nibble of an odd K is zero
    assert np.array_equal(host(dq.unpack_int4(dev(packed), K)), oracle.unpack_int4(packed, K))


def test_unpack_flat_two_passes(dq):
    N, K = 8200, 65536                         # even K: one wavefront per KB of packed bytes
    nbytes = N * K // 2
    assert nbytes > PASS_WAVES * 1024
    say(f"unpack even K N={N} K={K} ({nbytes} packed bytes)")
    gen = torch.Generator(device=DEV).manual_seed(14)
    packed = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=DEV, generator=gen)
    out = dq.unpack_int4(packed, K)
    # rows of the first pass, and those around and past byte 2^28 where the
    # second pass starts (row 8192 with 32768 bytes per row)
    rows = list(range(4)) + list(range(8184, N))
    ph = host(packed[rows])
    assert np.array_equal(host(out[rows]), oracle.unpack_int4(ph, K))
    del out, packed
    torch.cuda.empty_cache()


@pytest.mark.parametrize("affine", [False, True])
def test_dequantize_elem_two_passes(dq, affine):
    N, K, g = 2100, 8193, 128                  # odd K: one thread per output element
    assert N * K > PASS_THREADS
    say(f"dequantize odd K N={N} K={K} group={g} affine={affine}")
    if affine:
        pr, sr, zr, _ = oracle.quantize_int4_affine(gauss(N, K, 15, 0.02), g)
    else:
        pr, sr, _ = oracle.quantize_int4(gauss(N, K, 15), g)
        zr = None
    for dt, ndt in ((torch.float16, np.float16), (torch.float32, np.float32)):
        got = dq.dequantize_int4(dev(pr), dev(sr), K, g, dt, zeros=None if zr is None else dev(zr))
        ref = oracle.dequantize_int4(pr, sr, K, g, ndt, zeros=zr)
        assert np.array_equal(host(got).view(np.uint8), ref.view(np.uint8)), dt


@pytest.mark.parametrize("x_dtype,affine", [(np.float32, False), (np.float16, False), (np.float16, True)])
def test_generic_matmul_two_passes(dq, x_dtype, affine):
    M, N, K, g = 300, 1000, 96, 32             # M * N outputs past one pass of wavefronts
    assert M * N > PASS_WAVES
    say(f"generic matmul M={M} N={N} K={K} group={g} x={np.dtype(x_dtype).name} affine={affine}")
    if affine:
        pr, sr, zr, _ = oracle.quantize_int4_affine(gauss(N, K, 16, 0.02), g)
    else:
        pr, sr, _ = oracle.quantize_int4(gauss(N, K, 16), g)
        zr = None
    x = np.random.default_rng(17).normal(size=(M, K)).astype(x_dtype)
    y = dq.int4_matmul_path(dev(x), dev(pr), dev(sr), K, g, "generic",
                            zeros=None if zr is None else dev(zr))
    y_ref, bound = oracle.int4_matmul_ex(x.astype(np.float32), pr, sr, K, g, with_bound=True, zeros=zr)
    err = np.abs(host(y).astype(np.float64) - y_ref)
    bad = err > TOL * bound
    assert not bad.any(), f"{int(bad.sum())} outputs outside the bound"
