"""INT4 group quantization and fused dequantizing matmul for MI355X (gfx950).

Thin binding over the C ABI in ``include/int4dq.h`` (``libint4dq.so``, built
in-tree by ``dequantizing_gemm_amd/build.py``). The functions keep the names and
signatures of the drill page "Implement INT4 group quantization, nibble
packing and a dequantizing matmul" (statement):

    quantize_int4(w, group=128) -> (packed, scales, K)
    unpack_int4(packed, K) -> int8 [N, K]
    int4_matmul(x, packed, scales, K, group=128) -> float32 [M, N]

plus dequantize_int4(packed, scales, K, group=128, dtype=float16) -> w_hat [N, K],
the reconstruction q * scale that an unfused dequantize-then-GEMM would
materialise, and the affine form of the codes ("Build a Blockwise INT4
Inference Engine", step 2):

    quantize_int4_affine(w, group=128) -> (packed, scales, zeros, K)

whose ``zeros`` are passed to dequantize_int4 / int4_matmul / int4_matmul_path
as ``zeros=``; int4_linear(...) is one layer with fp16 or fp32 output, and
``dequantizing_gemm_amd.linear`` holds the Int4Linear module built on it.

All tensors are torch tensors on the GPU; torch provides the device memory and
the stream (work is enqueued on ``torch.cuda.current_stream()``). Every step of
the computation runs in the library's HIP kernels: this module only checks
shapes and dtypes, allocates outputs and passes pointers. It raises ImportError
when the library has not been built -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["quantize_int4", "quantize_int4_affine", "unpack_int4", "dequantize_int4", "int4_matmul",
           "int4_matmul_path", "int4_linear", "linear_workspace_bytes", "linear_workspace",
           "matmul_select",
           "num_groups", "packed_bytes", "lib", "LIB_PATH", "Int4Error", "PATHS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libint4dq.so")

OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
X_F32, X_F16 = 0, 1
ACT_NONE, ACT_RELU = 0, 1
OUT_F32, OUT_F16 = 0, 1
Y_F32, Y_F16 = 0, 1
PATHS = {"auto": 0, "generic": 1, "skinny": 2, "tiled": 3, "gemv": 4}
PATH_NAMES = {v: k for k, v in PATHS.items()}

# Every function declared in include/int4dq.h, with its ctypes signature.
_i64, _vp, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "int4_num_groups": (_i64, [_i64, _i64]),
    "int4_packed_bytes": (_i64, [_i64, _i64]),
    "int4_quantize": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "int4_unpack": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "int4_dequantize": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _vp, _vp]),
    "int4_matmul": (_int, [_vp, _int, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "int4_matmul_ex": (_int, [_vp, _int, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _vp]),
    "int4_matmul_path": (_int, [_vp, _int, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _int, _vp]),
    "int4_matmul_select": (_int, [_vp, _int, _i64, _vp, _vp, _i64, _i64, _i64, _vp]),
    "int4_quantize_affine": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "int4_dequantize_affine": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _vp]),
    "int4_matmul_affine": (_int, [_vp, _int, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp,
                                  _int, _vp]),
    "int4_linear": (_int, [_vp, _int, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _int, _vp]),
    "int4_linear_ws": (_int, [_vp, _int, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _int,
                              _vp, _i64, _vp]),
    "int4_linear_workspace_bytes": (_i64, [_int, _i64, _i64, _i64, _i64]),
    "int4_linear_noalloc": (_int, [_vp, _int, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _int,
                                   _vp]),
    "int4_last_error": (ctypes.c_char_p, []),
}


class Int4Error(RuntimeError):
    """A HIP launch failure reported by the library."""


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python dequantizing_gemm_amd/build.py` (hipcc, gfx950)")
    cdll = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(cdll, name)
        fn.restype, fn.argtypes = res, args
    return cdll


lib = _load()


def _raise(rc: int, what: str):
    if rc == OK:
        return
    msg = f"{what}: {lib.int4_last_error().decode()}"
    if rc in (EINVAL, EUNSUPPORTED):
        raise ValueError(msg)
    raise Int4Error(msg)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _gpu(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int = 2):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def num_groups(K: int, group: int) -> int:
    return int(lib.int4_num_groups(K, group))


def packed_bytes(N: int, K: int) -> int:
    return int(lib.int4_packed_bytes(N, K))


def quantize_int4(w: torch.Tensor, group: int = 128):
    """w [N, K] float32 -> (packed uint8 [N, ceil(K/2)], scales float16 [N, G], K)."""
    _gpu(w, "w", torch.float32)
    N, K = w.shape
    G = num_groups(K, group)
    if G < 1:
        raise ValueError(f"invalid K={K} / group={group}")
    packed = torch.empty((N, (K + 1) // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=w.device)
    with torch.cuda.device(w.device):
        rc = lib.int4_quantize(w.data_ptr(), N, K, group, packed.data_ptr(), scales.data_ptr(),
                               _stream(w))
    _raise(rc, "int4_quantize")
    return packed, scales, K


def quantize_int4_affine(w: torch.Tensor, group: int = 128):
    """w [N, K] float32 -> (packed uint8 [N, ceil(K/2)] unsigned codes, scales
    float16 [N, G], zero points uint8 [N, G], K)."""
    _gpu(w, "w", torch.float32)
    N, K = w.shape
    G = num_groups(K, group)
    if G < 1:
        raise ValueError(f"invalid K={K} / group={group}")
    packed = torch.empty((N, (K + 1) // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=w.device)
    zeros = torch.empty((N, G), dtype=torch.uint8, device=w.device)
    with torch.cuda.device(w.device):
        rc = lib.int4_quantize_affine(w.data_ptr(), N, K, group, packed.data_ptr(),
                                      scales.data_ptr(), zeros.data_ptr(), _stream(w))
    _raise(rc, "int4_quantize_affine")
    return packed, scales, zeros, K


def _zeros_ptr(zeros, N, K, group, device):
    if zeros is None:
        return None
    _gpu(zeros, "zeros", torch.uint8)
    if tuple(zeros.shape) != (N, num_groups(K, group)) or zeros.device != device:
        raise ValueError(f"zeros must be uint8 [{N}, {num_groups(K, group)}] on {device}")
    return zeros.data_ptr()


def unpack_int4(packed: torch.Tensor, K: int) -> torch.Tensor:
    """packed uint8 [N, ceil(K/2)] -> int8 [N, K], sign-extended."""
    _gpu(packed, "packed", torch.uint8)
    N = packed.shape[0]
    if packed.shape[1] != (K + 1) // 2:
        raise ValueError(f"packed has {packed.shape[1]} bytes per row, K={K} needs {(K + 1) // 2}")
    out = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    with torch.cuda.device(packed.device):
        rc = lib.int4_unpack(packed.data_ptr(), N, K, out.data_ptr(), _stream(packed))
    _raise(rc, "int4_unpack")
    return out


def dequantize_int4(packed: torch.Tensor, scales: torch.Tensor, K: int, group: int = 128,
                    dtype: torch.dtype = torch.float16,
                    zeros: torch.Tensor | None = None) -> torch.Tensor:
    """w_hat [N, K] = q * scale as float32 (exact) or float16 (nearest even);
    with ``zeros`` (affine codes) w_hat = (u - zero point) * scale."""
    _gpu(packed, "packed", torch.uint8)
    _gpu(scales, "scales", torch.float16)
    N = packed.shape[0]
    if packed.shape[1] != (K + 1) // 2:
        raise ValueError(f"packed has {packed.shape[1]} bytes per row, K={K} needs {(K + 1) // 2}")
    if tuple(scales.shape) != (N, num_groups(K, group)):
        raise ValueError(f"scales shape {tuple(scales.shape)} != {(N, num_groups(K, group))}")
    if dtype not in (torch.float32, torch.float16):
        raise ValueError(f"dtype must be float32 or float16 (got {dtype})")
    zp = _zeros_ptr(zeros, N, K, group, packed.device)
    out = torch.empty((N, K), dtype=dtype, device=packed.device)
    od = OUT_F16 if dtype == torch.float16 else OUT_F32
    with torch.cuda.device(packed.device):
        if zp is None:
            rc = lib.int4_dequantize(packed.data_ptr(), scales.data_ptr(), N, K, group, od,
                                     out.data_ptr(), _stream(packed))
        else:
            rc = lib.int4_dequantize_affine(packed.data_ptr(), scales.data_ptr(), zp, N, K, group,
                                            od, out.data_ptr(), _stream(packed))
    _raise(rc, "int4_dequantize")
    return out


def _matmul_args(x, packed, scales, K, group):
    if not isinstance(x, torch.Tensor) or x.dtype not in (torch.float32, torch.float16):
        raise ValueError("x must be a float32 or float16 torch tensor")
    _gpu(x, "x", x.dtype)
    _gpu(packed, "packed", torch.uint8)
    _gpu(scales, "scales", torch.float16)
    M, Kx = x.shape
    N = packed.shape[0]
    if Kx != K:
        raise ValueError(f"x has {Kx} columns, K={K}")
    if packed.shape[1] != (K + 1) // 2:
        raise ValueError(f"packed has {packed.shape[1]} bytes per row, K={K} needs {(K + 1) // 2}")
    if tuple(scales.shape) != (N, num_groups(K, group)):
        raise ValueError(f"scales shape {tuple(scales.shape)} != {(N, num_groups(K, group))}")
    if not (x.device == packed.device == scales.device):
        raise ValueError("x, packed and scales must be on the same device")
    return M, N, (X_F32 if x.dtype == torch.float32 else X_F16)


def int4_matmul_path(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, K: int,
                     group: int = 128, path: str = "auto", out: torch.Tensor | None = None,
                     bias: torch.Tensor | None = None, relu: bool = False,
                     zeros: torch.Tensor | None = None):
    """y [M, N] float32 = act(x @ dequantize(W).T + bias) through a chosen kernel
    (see PATHS); no bias and no ReLU unless given; affine codes with ``zeros``."""
    M, N, xd = _matmul_args(x, packed, scales, K, group)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    else:
        _gpu(out, "out", torch.float32)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out shape {tuple(out.shape)} != {(M, N)}")
    bptr = None
    if bias is not None:
        _gpu(bias, "bias", torch.float32, ndim=1)
        if bias.shape[0] != N or bias.device != x.device:
            raise ValueError(f"bias must be [N] = [{N}] on {x.device}")
        bptr = bias.data_ptr()
    zp = _zeros_ptr(zeros, N, K, group, x.device)
    act = ACT_RELU if relu else ACT_NONE
    with torch.cuda.device(x.device):
        if zp is None:
            rc = lib.int4_matmul_path(x.data_ptr(), xd, M, packed.data_ptr(), scales.data_ptr(), N,
                                      K, group, bptr, act, out.data_ptr(), PATHS[path], _stream(x))
        else:
            rc = lib.int4_matmul_affine(x.data_ptr(), xd, M, packed.data_ptr(), scales.data_ptr(),
                                        zp, N, K, group, bptr, act, out.data_ptr(), PATHS[path],
                                        _stream(x))
    _raise(rc, "int4_matmul")
    return out


def int4_matmul(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, K: int,
                group: int = 128, out: torch.Tensor | None = None, *,
                bias: torch.Tensor | None = None, relu: bool = False,
                zeros: torch.Tensor | None = None) -> torch.Tensor:
    """y [M, N] float32 = x @ dequantize(W).T, one group at a time (integer-first);
    with the engine page's epilogue act(... + bias) when bias or relu is given,
    and affine codes when zeros is given."""
    return int4_matmul_path(x, packed, scales, K, group, "auto", out, bias, relu, zeros)


def linear_workspace_bytes(M: int, N: int, K: int, group: int = 128, x_dtype=torch.float16) -> int:
    """Bytes of workspace int4_linear(..., workspace=) uses for these sizes (0:
    the call does not split K)."""
    xd = X_F16 if x_dtype == torch.float16 else X_F32
    r = lib.int4_linear_workspace_bytes(xd, M, N, K, group)
    if r < 0:
        raise ValueError(f"invalid sizes M={M} N={N} K={K} group={group}")
    return int(r)


def linear_workspace(M: int, N: int, K: int, group: int = 128, device="cuda") -> torch.Tensor:
    """A zero-filled workspace tensor for int4_linear(..., workspace=), or an
    empty one when the shape does not use it."""
    return torch.zeros(max(linear_workspace_bytes(M, N, K, group), 0), dtype=torch.uint8, device=device)


def int4_linear(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, K: int,
                group: int = 128, *, zeros: torch.Tensor | None = None,
                bias: torch.Tensor | None = None, relu: bool = False,
                out_dtype: torch.dtype = torch.float32,
                out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One layer: y [M, N] = act(x @ dequantize(W).T + bias) written as
    ``out_dtype`` (float32, or float16 rounded to nearest even), symmetric or
    (with ``zeros``) affine codes; the kernel is chosen as int4_matmul does.
    ``workspace`` (a uint8 device tensor from linear_workspace) lets the
    many-row kernel split K across blocks when its grid is small."""
    M, N, xd = _matmul_args(x, packed, scales, K, group)
    if out_dtype not in (torch.float32, torch.float16):
        raise ValueError(f"out_dtype must be float32 or float16 (got {out_dtype})")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _gpu(out, "out", out_dtype)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out shape {tuple(out.shape)} != {(M, N)}")
    bptr = None
    if bias is not None:
        _gpu(bias, "bias", torch.float32, ndim=1)
        if bias.shape[0] != N or bias.device != x.device:
            raise ValueError(f"bias must be [N] = [{N}] on {x.device}")
        bptr = bias.data_ptr()
    zp = _zeros_ptr(zeros, N, K, group, x.device)
    act = ACT_RELU if relu else ACT_NONE
    yd = Y_F16 if out_dtype == torch.float16 else Y_F32
    with torch.cuda.device(x.device):
        if workspace is None:
            rc = lib.int4_linear(x.data_ptr(), xd, M, packed.data_ptr(), scales.data_ptr(), zp, N, K,
                                 group, bptr, act, out.data_ptr(), yd, _stream(x))
        else:
            _gpu(workspace, "workspace", torch.uint8, ndim=1)
            if workspace.device != x.device:
                raise ValueError(f"workspace must be on {x.device}")
            wptr = workspace.data_ptr() if workspace.numel() else None
            rc = lib.int4_linear_ws(x.data_ptr(), xd, M, packed.data_ptr(), scales.data_ptr(), zp, N, K,
                                    group, bptr, act, out.data_ptr(), yd, wptr, workspace.numel(),
                                    _stream(x))
    _raise(rc, "int4_linear")
    return out


def matmul_select(x, packed, scales, K, group=128) -> str:
    """Name of the kernel int4_matmul would run for these tensors."""
    M, N, xd = _matmul_args(x, packed, scales, K, group)
    p = lib.int4_matmul_select(x.data_ptr(), xd, M, packed.data_ptr(), scales.data_ptr(), N, K,
                               group, 1)
    return PATH_NAMES.get(p, "invalid")
