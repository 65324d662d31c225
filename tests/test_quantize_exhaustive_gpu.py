"""Codes at rounding boundaries under every binary16 scale, GPU against the oracle.

The drill page "Implement INT4 group quantization, nibble packing and a
dequantizing matmul" (statement) fixes q = round(w / scale) with the stored
binary16 scale; the reading here is a correctly rounded binary32 division and
ties to even. The kernels form w * rcp(scale) and take the division only
where the product lies close to a half-integer, which must give the codes of
the division exactly. This test leaves that to no argument: for every
positive finite binary16 scale (31743 of them, subnormals included) one group
holds an element of magnitude 7 * scale (so the group's scale is exactly that
one; its sign alternates) and elements on, and 1 to 4 binary32 ulps either
side of, every half-integer multiple of the scale from -6.5 to 6.5. Scales
of 1 to 6 smallest subnormals also get quotients around -9.5 .. 9.5, where
the clamp to [-8, 7] decides. Affine codes get the same sweep with a range of
[-8 s, 7 s] (zero point 8) and [-7 s, 8 s] (zero point 7, odd, where the
order of rounding and adding the zero point matters at ties). Each runs
through the vectorised kernels (group 256) and the general ones (group 160),
and every byte of codes, scales and zero points must equal the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
OFFSETS = (0, 1, -1, 2, -2, 3, -3, 4, -4)      # binary32 ulps from the exact multiple


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dq():
    import dequantizing_gemm_amd as dq
    return dq


def _ulps(v, j):
    """v moved by j binary32 ulps (toward +inf for j > 0)."""
    out = v.copy()
    for _ in range(abs(j)):
        out = np.nextafter(out, np.float32(np.inf) if j > 0 else np.float32(-np.inf)).astype(np.float32)
    return out


def _fill(rows, col, s, halves):
    """Write h * s and its ulp neighbours for each h in halves into rows from column col."""
    centers = (np.asarray(halves, np.float64)[None, :] * s[:, None].astype(np.float64)).astype(np.float32)
    for j in OFFSETS:
        v = _ulps(centers, j)
        rows[:, col:col + v.shape[1]] = v
        col += v.shape[1]
    return col


ALL_SCALES = np.arange(1, 0x7C00, dtype=np.uint16)      # every positive finite binary16


def symmetric_matrix(K):
    s = ALL_SCALES.view(np.float16).astype(np.float32)
    rows = np.zeros((len(s), K), np.float32)
    sign = np.where(np.arange(len(s)) % 2 == 0, 1.0, -1.0).astype(np.float32)
    rows[:, 0] = sign * np.float32(7.0) * s
    col = _fill(rows, 1, s, np.arange(-6.5, 7.0, 1.0))
    assert col <= K
    extra = []
    for k, hs in ((1, (-9.5, -8.5, -7.5, 7.5, 8.5, 9.5)), (2, (-8.5, -7.5, 7.5, 8.5)),
                  (3, (-7.5, 7.5)), (4, (-7.5, 7.5)), (5, (-7.5, 7.5)), (6, (-7.5, 7.5))):
        sk = np.array([k * 2.0 ** -24], np.float32)
        r = np.zeros((1, K), np.float32)
        _fill(r, 0, sk, hs)
        extra.append(r)
    return np.concatenate([rows] + extra), len(s)


def affine_matrix(K, zp):
    s = ALL_SCALES.view(np.float16).astype(np.float32)
    rows = np.zeros((len(s), K), np.float32)
    hi, lo = (7.0, -8.0) if zp == 8 else (8.0, -7.0)
    rows[:, 0] = np.float32(hi) * s
    rows[:, 1] = np.float32(lo) * s
    col = _fill(rows, 2, s, np.arange(lo + 0.5, hi, 1.0))
    assert col <= K
    return rows, len(s)


@pytest.mark.parametrize("g", [256, 160])
def test_quantize_every_scale_at_half_integers(dq, g):
    w, n_main = symmetric_matrix(g)
    say(f"case: quantize every binary16 scale, [{w.shape[0]},{g}] group {g}")
    p, s, K = dq.quantize_int4(dev(w), g)
    pr, sr, _ = oracle.quantize_int4(w, g)
    sh = host(s).view(np.uint16)
    assert np.array_equal(sh[:n_main, 0], ALL_SCALES), "a group's scale is not the intended one"
    assert np.array_equal(sh, sr.view(np.uint16)), "scales differ from the oracle"
    ph = host(p)
    bad = np.argwhere(ph != pr)
    assert len(bad) == 0, f"codes differ from the oracle at {bad[:5].tolist()}"


@pytest.mark.parametrize("zp", [8, 7])
@pytest.mark.parametrize("g", [256, 160])
def test_quantize_affine_every_scale_at_half_integers(dq, g, zp):
    w, n_main = affine_matrix(g, zp)
    say(f"case: quantize_affine every binary16 scale, zero point {zp}, [{w.shape[0]},{g}] group {g}")
    p, s, z, K = dq.quantize_int4_affine(dev(w), g)
    pr, sr, zr, _ = oracle.quantize_int4_affine(w, g)
    sh, zh = host(s).view(np.uint16), host(z)
    assert np.array_equal(sh[:, 0], ALL_SCALES) and np.all(zh == zp), "not the intended scales"
    assert np.array_equal(sh, sr.view(np.uint16)) and np.array_equal(zh, zr)
    ph = host(p)
    bad = np.argwhere(ph != pr)
    assert len(bad) == 0, f"codes differ from the oracle at {bad[:5].tolist()}"
