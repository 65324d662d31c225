"""The C ABI without a GPU: the library loads, exports every declared entry
point, computes sizes, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "int4dq.h")


def _lib():
    import __graft_entry__
    __graft_entry__._ensure_built()
    import dequantizing_gemm_amd as dq
    return dq


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(int4_\w+)\s*\(", src)))


def test_header_declares_the_abi():
    assert _declared() == sorted(["int4_num_groups", "int4_packed_bytes", "int4_quantize", "int4_dequantize",
                                  "int4_unpack", "int4_matmul", "int4_matmul_ex", "int4_matmul_path",
                                  "int4_matmul_select", "int4_last_error", "int4_quantize_affine",
                                  "int4_dequantize_affine", "int4_matmul_affine", "int4_linear",
                                  "int4_linear_ws", "int4_linear_workspace_bytes", "int4_linear_noalloc"])


def test_library_exports_every_declared_symbol():
    dq = _lib()
    raw = ctypes.CDLL(dq.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(_declared()) == set(dq.SIGNATURES)


def test_size_helpers():
    dq = _lib()
    L = dq.lib
    assert L.int4_num_groups(301, 128) == 3 and L.int4_num_groups(256, 128) == 2
    assert L.int4_num_groups(5, 1) == 5 and L.int4_num_groups(3, 1000) == 1
    assert L.int4_num_groups(0, 128) == -1 and L.int4_num_groups(10, 0) == -1
    assert L.int4_packed_bytes(48, 301) == 48 * 151 and L.int4_packed_bytes(1, 1) == 1
    assert L.int4_packed_bytes(28672, 8192) == 117440512
    assert L.int4_packed_bytes(0, 5) == -1 and L.int4_packed_bytes(5, -1) == -1
    assert L.int4_packed_bytes(2 ** 62, 8) == -1                 # overflow
    # storage for the 5 configurations' largest matrix: N*ceil(K/2) + 2*N*G
    N, K, g = 28672, 8192, 128
    assert L.int4_packed_bytes(N, K) + 2 * N * L.int4_num_groups(K, g) == 117440512 + 3670016


FAKE = ctypes.c_void_p(0x1000)    # never dereferenced: validation fails first


@pytest.mark.parametrize("args,needle", [
    ((FAKE, 0, 8, 4, FAKE, FAKE, None), "N and K"),
    ((FAKE, 4, 0, 4, FAKE, FAKE, None), "N and K"),
    ((FAKE, 4, 8, 0, FAKE, FAKE, None), "group"),
    ((None, 4, 8, 4, FAKE, FAKE, None), "non-NULL"),
    ((FAKE, 4, 8, 4, None, FAKE, None), "non-NULL"),
    ((FAKE, 2 ** 62, 8, 4, FAKE, FAKE, None), "overflow"),
])
def test_quantize_rejects(args, needle):
    dq = _lib()
    assert dq.lib.int4_quantize(*args) == dq.EINVAL
    assert needle in dq.lib.int4_last_error().decode()


def test_unpack_rejects():
    dq = _lib()
    assert dq.lib.int4_unpack(FAKE, -1, 8, FAKE, None) == dq.EINVAL
    assert dq.lib.int4_unpack(None, 2, 8, FAKE, None) == dq.EINVAL
    assert dq.lib.int4_unpack(FAKE, 2, 8, None, None) == dq.EINVAL
    assert dq.lib.int4_unpack(FAKE, 2 ** 40, 2 ** 40, FAKE, None) == dq.EINVAL


@pytest.mark.parametrize("args,needle", [
    ((FAKE, FAKE, 0, 8, 4, 1, FAKE, None), "N and K"),
    ((FAKE, FAKE, 4, 0, 4, 1, FAKE, None), "N and K"),
    ((FAKE, FAKE, 4, 8, 0, 1, FAKE, None), "group"),
    ((FAKE, FAKE, 4, 8, 4, 2, FAKE, None), "out_dtype"),
    ((None, FAKE, 4, 8, 4, 1, FAKE, None), "non-NULL"),
    ((FAKE, None, 4, 8, 4, 1, FAKE, None), "non-NULL"),
    ((FAKE, FAKE, 4, 8, 4, 0, None, None), "non-NULL"),
    ((FAKE, FAKE, 2 ** 40, 2 ** 30, 4, 0, FAKE, None), "overflow"),
])
def test_dequantize_rejects(args, needle):
    dq = _lib()
    assert dq.lib.int4_dequantize(*args) == dq.EINVAL
    assert needle in dq.lib.int4_last_error().decode()


@pytest.mark.parametrize("kw,needle", [
    (dict(M=-1), "M must be"),
    (dict(N=0), "N and K"),
    (dict(K=0), "N and K"),
    (dict(group=0), "group"),
    (dict(x_dtype=7), "x_dtype"),
    (dict(x=None), "non-NULL"),
    (dict(y=None), "non-NULL"),
    (dict(packed=None), "non-NULL"),
    (dict(scales=None, M=0), "non-NULL"),
    (dict(M=2 ** 40, K=2 ** 30), "overflow"),
])
def test_matmul_rejects(kw, needle):
    dq = _lib()
    a = dict(x=FAKE, x_dtype=1, M=4, packed=FAKE, scales=FAKE, N=16, K=256, group=128, y=FAKE)
    a.update(kw)
    rc = dq.lib.int4_matmul(a["x"], a["x_dtype"], a["M"], a["packed"], a["scales"], a["N"],
                            a["K"], a["group"], a["y"], None)
    assert rc == dq.EINVAL
    assert needle in dq.lib.int4_last_error().decode()
    assert dq.lib.int4_matmul_select(a["x"], a["x_dtype"], a["M"], a["packed"], a["scales"],
                                     a["N"], a["K"], a["group"], a["y"]) == -1


def test_matmul_m0_is_noop_and_bad_path():
    dq = _lib()
    # M = 0 returns OK without touching the GPU (no pointer is dereferenced)
    assert dq.lib.int4_matmul(None, 1, 0, FAKE, FAKE, 16, 256, 128, None, None) == dq.OK
    assert dq.lib.int4_matmul_path(FAKE, 1, 4, FAKE, FAKE, 16, 256, 128, None, 0, FAKE, 9, None) == dq.EINVAL
    # an unknown activation is rejected before anything is enqueued
    assert dq.lib.int4_matmul_ex(FAKE, 1, 4, FAKE, FAKE, 16, 256, 128, None, 5, FAKE, None) == dq.EINVAL
    assert "activation" in dq.lib.int4_last_error().decode()
    assert dq.lib.int4_matmul_ex(None, 1, 0, FAKE, FAKE, 16, 256, 128, FAKE, 1, None, None) == dq.OK


@pytest.mark.parametrize("args,needle", [
    ((FAKE, 0, 8, 4, FAKE, FAKE, FAKE, None), "N and K"),
    ((FAKE, 4, 8, 0, FAKE, FAKE, FAKE, None), "group"),
    ((FAKE, 4, 8, 4, FAKE, FAKE, None, None), "non-NULL"),
    ((None, 4, 8, 4, FAKE, FAKE, FAKE, None), "non-NULL"),
    ((FAKE, 2 ** 62, 8, 4, FAKE, FAKE, FAKE, None), "overflow"),
])
def test_quantize_affine_rejects(args, needle):
    dq = _lib()
    assert dq.lib.int4_quantize_affine(*args) == dq.EINVAL
    msg = dq.lib.int4_last_error().decode()
    assert needle in msg and "int4_quantize_affine" in msg


def test_affine_entry_points_reject():
    dq = _lib()
    L = dq.lib
    # zeros must be given
    assert L.int4_dequantize_affine(FAKE, FAKE, None, 4, 8, 4, 0, FAKE, None) == dq.EINVAL
    assert "zeros" in L.int4_last_error().decode()
    assert L.int4_matmul_affine(FAKE, 1, 4, FAKE, FAKE, None, 16, 256, 128, None, 0, FAKE, 0, None) == dq.EINVAL
    assert "zeros" in L.int4_last_error().decode()
    # the rest of the validation is the symmetric entry points'
    assert L.int4_dequantize_affine(FAKE, FAKE, FAKE, 4, 8, 4, 2, FAKE, None) == dq.EINVAL
    assert "out_dtype" in L.int4_last_error().decode()
    assert L.int4_matmul_affine(FAKE, 1, 4, FAKE, FAKE, FAKE, 16, 256, 128, None, 5, FAKE, 0, None) == dq.EINVAL
    assert "activation" in L.int4_last_error().decode()
    assert L.int4_matmul_affine(FAKE, 1, 4, FAKE, FAKE, FAKE, 16, 256, 128, None, 0, FAKE, 9, None) == dq.EINVAL
    assert "path" in L.int4_last_error().decode()
    assert L.int4_matmul_affine(FAKE, 7, 4, FAKE, FAKE, FAKE, 16, 256, 128, None, 0, FAKE, 0, None) == dq.EINVAL
    assert L.int4_matmul_affine(None, 1, 0, FAKE, FAKE, FAKE, 16, 256, 128, None, 0, None, 0, None) == dq.OK


def test_linear_rejects():
    dq = _lib()
    L = dq.lib
    args = [FAKE, 1, 4, FAKE, FAKE, None, 16, 256, 128, None, 0, FAKE]
    assert L.int4_linear(*args, 2, None) == dq.EINVAL
    assert "y_dtype" in L.int4_last_error().decode()
    assert L.int4_linear(*args[:10], 3, FAKE, 0, None) == dq.EINVAL
    assert "activation" in L.int4_last_error().decode()
    bad_x = list(args)
    bad_x[1] = 5
    assert L.int4_linear(*bad_x, 0, None) == dq.EINVAL
    assert L.int4_linear(None, 1, 0, FAKE, FAKE, None, 16, 256, 128, None, 0, None, 1, None) == dq.OK


def test_kernel_selection_rules():
    """Which kernel the library picks (host logic only, no launch)."""
    dq = _lib()
    sel = lambda xd, M, K, g, x=0x1000, p=0x2000, N=64: dq.lib.int4_matmul_select(
        ctypes.c_void_p(x), xd, M, ctypes.c_void_p(p), FAKE, N, K, g, FAKE)
    P = dq.PATHS
    assert sel(1, 1, 4096, 128) == P["gemv"] and sel(1, 16, 4096, 128) == P["skinny"]
    assert sel(1, 2, 4096, 128) == P["gemv"] and sel(1, 1, 11008, 128) == P["gemv"]
    # 2-4 rows: the matrix-core gemv while K <= 12288 and group = 32 * 2^p
    assert sel(1, 4, 12288, 128) == P["gemv"] and sel(1, 4, 12416, 128) == P["skinny"]
    assert sel(1, 5, 4096, 128) == P["skinny"] and sel(1, 3, 4096, 96) == P["generic"]
    assert sel(1, 1, 768, 32) == P["gemv"] and sel(1, 1, 768, 64) == P["gemv"]
    assert sel(1, 1, 4096, 16) == P["generic"]                 # group not a multiple of 32
    assert sel(1, 1, 65536, 128) == P["tiled"]                 # K beyond the gemv and skinny kernels
    assert sel(1, 2048, 11008, 128) == P["tiled"] and sel(1, 65, 4096, 128) == P["tiled"]
    # 17-64 rows: skinny while N * ceil(M / 16) <= 12288, else tiled
    assert sel(1, 17, 4096, 128) == P["skinny"] and sel(1, 48, 4096, 128, N=4096) == P["skinny"]
    assert sel(1, 49, 4096, 128, N=4096) == P["tiled"] and sel(1, 32, 4096, 128, N=6144) == P["skinny"]
    assert sel(1, 32, 4096, 128, N=11008) == P["tiled"]
    assert sel(1, 17, 8192, 128, N=28672) == P["tiled"] and sel(1, 16, 8192, 128, N=28672) == P["skinny"]
    # four row tiles do not take more than 96 K-blocks
    assert sel(1, 40, 16384, 128) == P["tiled"] and sel(1, 20, 16384, 128) == P["skinny"]
    assert sel(1, 4, 768, 64) == P["gemv"] and sel(1, 4, 768, 32) == P["gemv"]
    assert sel(0, 4, 256, 128) == P["generic"]                 # binary32 x
    assert sel(1, 3, 301, 128) == P["generic"]                 # odd K
    assert sel(1, 4, 768, 96) == P["generic"]                  # group not 32/64/128k
    assert sel(1, 4, 4096, 128, x=0x1002) == P["generic"]      # unaligned x
    assert sel(1, 512, 4096, 256) == P["tiled"]


def test_kernel_selection_keeps_grids_launchable():
    """A dispatch holds fewer than 2^32 work items per grid dimension. The
    weight-streaming kernels launch up to 128 threads per weight row and the
    tiled kernel 256 per output tile, so the automatic choice passes shapes
    beyond their limits on to a kernel whose grid fits (the generic kernel
    strides over any number of outputs); a forced kernel refuses them."""
    dq = _lib()
    sel = lambda M, N, K=64, g=32: dq.lib.int4_matmul_select(
        ctypes.c_void_p(0x1000), 1, M, ctypes.c_void_p(0x2000), FAKE, N, K, g, FAKE)
    P = dq.PATHS
    assert sel(1, (1 << 25) - 1) == P["gemv"] and sel(4, (1 << 25) - 1) == P["gemv"]
    assert sel(8, (1 << 25) - 1) == P["skinny"]
    # 2^25 weight rows: one 32 x 128 tile per 128 rows, 2^18 tiles
    assert sel(1, 1 << 25) == P["tiled"] and sel(8, 1 << 25) == P["tiled"]
    # 2048 x 2^28 outputs are 2^24 tiles of 128 x 256: one block too many for the tiled grid
    assert sel(2048, (1 << 28) - 256) == P["tiled"] and sel(2048, 1 << 28) == P["generic"]
    assert sel(1, 1 << 31) == P["generic"] and sel(1 << 31, 1) == P["generic"]
    y = ctypes.c_void_p(0x3000)
    for path, M, N in (("gemv", 1, 1 << 25), ("skinny", 8, 1 << 25), ("tiled", 2048, 1 << 28)):
        rc = dq.lib.int4_matmul_path(ctypes.c_void_p(0x1000), 1, M, ctypes.c_void_p(0x2000), FAKE, N, 64, 32,
                                     None, 0, y, P[path], None)
        assert rc == dq.EUNSUPPORTED and b"2^" in dq.lib.int4_last_error(), path


def test_binding_rejects_host_tensors():
    dq = _lib()
    with pytest.raises(ValueError, match="GPU"):
        dq.quantize_int4(torch.zeros(4, 8))
    with pytest.raises(ValueError):
        dq.int4_matmul(torch.zeros(2, 8, dtype=torch.float16), torch.zeros(4, 4, dtype=torch.uint8),
                       torch.zeros(4, 1, dtype=torch.float16), 8, 8)


def _split_bytes(tiles, S, M, N):
    """Workspace of a split of K into S shares: S partial [M, N] binary32
    results (the grid has `tiles` output tiles, S blocks each)."""
    return S * M * N * 4


@pytest.mark.parametrize("M,N,K,g,expect", [
    # 32 x 128 tiles: 4 x 32 = 128 tiles -> 4 shares of 16 sub-steps (8 would be 1024 blocks)
    (128, 4096, 4096, 128, _split_bytes(128, 4, 128, 4096)),
    # K = 11008: 172 sub-steps, shares of 44 (a multiple of the 4-sub-step super-tile)
    (128, 4096, 11008, 128, _split_bytes(128, 4, 128, 4096)),
    # grids of more than 128 tiles are not split (64 x 128 tiles, 8 x 32)
    (512, 4096, 4096, 128, 0), (512, 4096, 11008, 128, 0), (640, 2048, 4096, 128, 0),
    # group 32: 64 x 128 tiles of 32-code sub-steps, 25 tiles -> 8 shares of 32
    (300, 640, 8192, 32, _split_bytes(25, 8, 300, 640)),
    # enough tiles already: 128 x 256 tiles, 16 x 16 and 4 x 43 and 2 x 112
    (2048, 4096, 4096, 128, 0), (512, 11008, 4096, 128, 0), (256, 28672, 8192, 128, 0),
    # the kernels for a few rows of x do not split
    (1, 4096, 4096, 128, 0), (16, 4096, 4096, 128, 0),
    # too short a K for 16 sub-steps per share
    (128, 4096, 1024, 128, 0),
    # 24 tiles of 32 x 128 and K = 8192: 8 shares of 16 sub-steps
    (96, 1024, 8192, 128, _split_bytes(24, 8, 96, 1024)),
    # 64 rows against 1024 weight rows: the skinny kernel, K in 8 shares of 8
    # K-blocks (64 row groups)
    (64, 1024, 8192, 128, 8 * 64 * 1024 * 4),
    # the skinny kernel's split: groups 32 and 64 at M = 32 (24 K-blocks of
    # 128 codes times two row tiles, 4 shares of 6); not taken for less work
    # per row group (groups 32 and 64 at M = 16: 24 K-blocks), where the
    # pipelined form runs (group 128, 5-16 rows) or with 128 row groups or
    # more
    (32, 768, 3072, 32, 4 * 32 * 768 * 4), (16, 768, 3072, 32, 0),
    (32, 768, 3072, 64, 4 * 32 * 768 * 4), (16, 768, 3072, 64, 0),
    (8, 1024, 8192, 128, 0), (32, 2048, 3072, 64, 0),
    # ragged: 65 row groups, 33 K-blocks of 128 codes in 4 shares of 9
    (20, 1030, 4224, 64, 4 * 20 * 1030 * 4),
    # a group of 1024 codes: shares start on a group boundary (16 sub-steps)
    (128, 4096, 4096, 1024, _split_bytes(128, 4, 128, 4096)),
])
def test_workspace_bytes(M, N, K, g, expect):
    dq = _lib()
    assert dq.lib.int4_linear_workspace_bytes(1, M, N, K, g) == expect
    assert dq.linear_workspace_bytes(M, N, K, g) == expect


def test_workspace_bytes_rejects():
    dq = _lib()
    L = dq.lib
    assert L.int4_linear_workspace_bytes(1, -1, 8, 8, 4) == -1
    assert L.int4_linear_workspace_bytes(1, 4, 0, 8, 4) == -1
    assert L.int4_linear_workspace_bytes(7, 4, 8, 8, 4) == -1
    assert L.int4_linear_workspace_bytes(1, 0, 8, 8, 4) == 0
    assert L.int4_linear_workspace_bytes(0, 512, 4096, 4096, 128) == 0    # fp32 x: generic kernel


@pytest.mark.parametrize("ws,nbytes,needle", [
    (None, 1024, "workspace"), (FAKE, -1, "workspace_bytes"),
    (ctypes.c_void_p(0x1010), 1024, "256-byte aligned"),
])
def test_linear_ws_rejects(ws, nbytes, needle):
    dq = _lib()
    rc = dq.lib.int4_linear_ws(FAKE, 1, 4, FAKE, FAKE, None, 8, 64, 32, None, 0, FAKE, 0, ws, nbytes, None)
    assert rc == dq.EINVAL
    assert needle in dq.lib.int4_last_error().decode()


def test_linear_noalloc_rejects_before_any_hip_call():
    dq = _lib()
    L = dq.lib
    assert L.int4_linear_noalloc(FAKE, 1, -1, FAKE, FAKE, None, 8, 64, 32, None, 0, FAKE, 0, None) == dq.EINVAL
    assert L.int4_linear_noalloc(FAKE, 1, 4, None, FAKE, None, 8, 64, 32, None, 0, FAKE, 0, None) == dq.EINVAL
    assert L.int4_linear_noalloc(FAKE, 9, 4, FAKE, FAKE, None, 8, 64, 32, None, 0, FAKE, 0, None) == dq.EINVAL
    assert L.int4_linear_noalloc(FAKE, 1, 4, FAKE, FAKE, None, 8, 64, 32, None, 5, FAKE, 0, None) == dq.EINVAL
