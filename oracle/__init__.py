"""CPU oracle for INT4 group quantization and the dequantizing matmul.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. It never touches a GPU and shares
no code with the HIP library: the scalar C in ``int4_oracle.c`` is compiled
with the host ``cc`` into ``liboracle.so`` and called through ctypes on host
NumPy buffers.

The definitions follow the drill page "Implement INT4 group quantization,
nibble packing and a dequantizing matmul", section "statement"; the readings
taken where it is silent are listed in ``int4_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "int4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the scalar C oracle with the host compiler (no GPU involved)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(["cc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first if needed) the oracle library; returns a ctypes CDLL."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        _lib = _declare(ctypes.CDLL(build()))
    return _lib


def _declare(lib):
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.int4_oracle_half_from_float.argtypes = [ctypes.c_float]
    lib.int4_oracle_half_from_float.restype = ctypes.c_uint16
    lib.int4_oracle_half_from_float_array.argtypes = [vp, i64, vp]
    lib.int4_oracle_half_from_float_array.restype = None
    lib.int4_oracle_float_from_half.argtypes = [ctypes.c_uint16]
    lib.int4_oracle_float_from_half.restype = ctypes.c_float
    lib.int4_oracle_num_groups.argtypes = [i64, i64]
    lib.int4_oracle_num_groups.restype = i64
    lib.int4_oracle_packed_row_bytes.argtypes = [i64]
    lib.int4_oracle_packed_row_bytes.restype = i64
    lib.int4_oracle_quantize.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.int4_oracle_quantize.restype = None
    lib.int4_oracle_unpack.argtypes = [vp, i64, i64, vp]
    lib.int4_oracle_unpack.restype = None
    lib.int4_oracle_matmul.argtypes = [vp, i64, vp, vp, i64, i64, i64, vp, vp]
    lib.int4_oracle_matmul.restype = None
    lib.int4_oracle_matmul_ex.argtypes = [vp, i64, vp, vp, vp, i64, i64, i64, vp, ctypes.c_int, vp, vp]
    lib.int4_oracle_matmul_ex.restype = None
    lib.int4_oracle_quantize_affine.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    lib.int4_oracle_quantize_affine.restype = None
    lib.int4_oracle_dequantize.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.int4_oracle_dequantize.restype = None
    lib.int4_oracle_dequantize_half.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.int4_oracle_dequantize_half.restype = None
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def quantize_int4(w: np.ndarray, group: int = 128, lib=None):
    """w [N, K] float32 -> (packed uint8 [N, ceil(K/2)], scales float16 [N, G], K)."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    G = (K + group - 1) // group
    packed = np.empty((N, (K + 1) // 2), dtype=np.uint8)
    scales = np.empty((N, G), dtype=np.uint16)
    lib.int4_oracle_quantize(_ptr(w), N, K, group, _ptr(packed), _ptr(scales))
    return packed, scales.view(np.float16), K


def quantize_int4_affine(w: np.ndarray, group: int = 128, lib=None):
    """w [N, K] float32 -> (packed uint8 [N, ceil(K/2)] unsigned codes,
    scales float16 [N, G], zero points uint8 [N, G], K)."""
    lib = lib or load()
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    G = (K + group - 1) // group
    packed = np.empty((N, (K + 1) // 2), dtype=np.uint8)
    scales = np.empty((N, G), dtype=np.uint16)
    zeros = np.empty((N, G), dtype=np.uint8)
    lib.int4_oracle_quantize_affine(_ptr(w), N, K, group, _ptr(packed), _ptr(scales), _ptr(zeros))
    return packed, scales.view(np.float16), zeros, K


def _zeros_arg(zeros, N, K, group):
    if zeros is None:
        return None, None
    z = np.ascontiguousarray(zeros, dtype=np.uint8)
    assert z.shape == (N, (K + group - 1) // group)
    return z, _ptr(z)


def unpack_int4(packed: np.ndarray, K: int, lib=None) -> np.ndarray:
    """packed uint8 [N, ceil(K/2)] -> int8 [N, K], sign-extended."""
    lib = lib or load()
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    assert packed.shape[1] == (K + 1) // 2
    out = np.empty((N, K), dtype=np.int8)
    lib.int4_oracle_unpack(_ptr(packed), N, K, _ptr(out))
    return out


def int4_matmul(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, K: int,
                group: int = 128, with_bound: bool = False, lib=None):
    """y [M, N] float32 = x @ dequantize(W).T, per group integer-first, in double.

    x may be float32 or float16 (widened exactly). With ``with_bound`` also
    returns sum_k |x[m,k] * q[n,k] * scale| as float64 [M, N].
    """
    lib = lib or load()
    x = np.ascontiguousarray(np.asarray(x).astype(np.float32))
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    s16 = np.ascontiguousarray(np.asarray(scales).view(np.uint16))
    M = x.shape[0]
    N = packed.shape[0]
    assert x.shape[1] == K and packed.shape[1] == (K + 1) // 2
    assert s16.shape == (N, (K + group - 1) // group)
    y = np.empty((M, N), dtype=np.float32)
    bound = np.empty((M, N), dtype=np.float64) if with_bound else None
    lib.int4_oracle_matmul(_ptr(x), M, _ptr(packed), _ptr(s16), N, K, group, _ptr(y),
                           _ptr(bound) if with_bound else None)
    return (y, bound) if with_bound else y


def int4_matmul_ex(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, K: int,
                   group: int = 128, bias: np.ndarray | None = None, relu: bool = False,
                   with_bound: bool = False, zeros: np.ndarray | None = None, lib=None):
    """y [M, N] float32 = act(x @ dequantize(W).T + bias): the matmul sum and the
    bias in double, rounded once, then ReLU (v > 0 ? v : +0) if asked. With
    ``zeros`` the codes are affine (integer weight = code - zero point)."""
    lib = lib or load()
    x = np.ascontiguousarray(np.asarray(x).astype(np.float32))
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    s16 = np.ascontiguousarray(np.asarray(scales).view(np.uint16))
    M = x.shape[0]
    N = packed.shape[0]
    assert x.shape[1] == K and packed.shape[1] == (K + 1) // 2
    assert s16.shape == (N, (K + group - 1) // group)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    assert b is None or b.shape == (N,)
    y = np.empty((M, N), dtype=np.float32)
    bound = np.empty((M, N), dtype=np.float64) if with_bound else None
    z, zp = _zeros_arg(zeros, N, K, group)
    lib.int4_oracle_matmul_ex(_ptr(x), M, _ptr(packed), _ptr(s16), zp, N, K, group,
                              _ptr(b) if b is not None else None, int(bool(relu)), _ptr(y),
                              _ptr(bound) if with_bound else None)
    return (y, bound) if with_bound else y


def dequantize_int4(packed: np.ndarray, scales: np.ndarray, K: int, group: int = 128,
                    dtype=np.float32, zeros: np.ndarray | None = None, lib=None) -> np.ndarray:
    """w_hat [N, K] = q * scale, as float32 (exact) or float16 (the exact
    product rounded to nearest even, by the oracle's own binary16 rounding).
    With ``zeros`` the codes are affine: w_hat = (code - zero point) * scale."""
    lib = lib or load()
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    s16 = np.ascontiguousarray(np.asarray(scales).view(np.uint16))
    N = packed.shape[0]
    assert packed.shape[1] == (K + 1) // 2
    assert s16.shape == (N, (K + group - 1) // group)
    z, zp = _zeros_arg(zeros, N, K, group)
    if np.dtype(dtype) == np.float32:
        out = np.empty((N, K), dtype=np.float32)
        lib.int4_oracle_dequantize(_ptr(packed), _ptr(s16), zp, N, K, group, _ptr(out))
        return out
    if np.dtype(dtype) == np.float16:
        out = np.empty((N, K), dtype=np.uint16)
        lib.int4_oracle_dequantize_half(_ptr(packed), _ptr(s16), zp, N, K, group, _ptr(out))
        return out.view(np.float16)
    raise ValueError(f"dtype {dtype}: float32 or float16")


def half_from_float(f: float, lib=None) -> int:
    return int((lib or load()).int4_oracle_half_from_float(float(f)))


def float_from_half(h: int, lib=None) -> float:
    return float((lib or load()).int4_oracle_float_from_half(int(h)))


def half_bits_from_float_array(f: np.ndarray, lib=None) -> np.ndarray:
    """Element-wise binary32 -> binary16 bit patterns (round to nearest even)."""
    lib = lib or load()
    f = np.ascontiguousarray(f, dtype=np.float32).ravel()
    h = np.empty(f.shape, dtype=np.uint16)
    lib.int4_oracle_half_from_float_array(_ptr(f), f.size, _ptr(h))
    return h
