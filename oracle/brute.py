"""Second, independent CPU oracle in NumPy, for tiny shapes only.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``). It is written separately
from the scalar C oracle so that the two can be checked against each other:
the binary16 rounding here is NumPy's own ``astype(np.float16)`` rather than
the hand-written conversion in C, rounding is ``np.rint``, and the matmul is a
float64 ``@`` of x with the fully dequantized weight matrix.

Definitions: drill page "Implement INT4 group quantization, nibble packing and
a dequantizing matmul", section "statement".
"""
from __future__ import annotations

import numpy as np


def quantize_int4(w: np.ndarray, group: int = 128):
    """w [N, K] float32 -> (packed uint8 [N, ceil(K/2)], scales float16 [N, G], K)."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    G = -(-K // group)
    scales = np.zeros((N, G), dtype=np.float16)
    q = np.zeros((N, K + (K % 2)), dtype=np.int8)       # room for the pad nibble
    for gi in range(G):
        blk = w[:, gi * group:min((gi + 1) * group, K)]
        s16 = (np.abs(blk).max(axis=1) / np.float32(7)).astype(np.float16)
        scales[:, gi] = s16
        sf = s16.astype(np.float32)[:, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            t = blk / sf                                    # float32 / float32
        qb = np.clip(np.rint(t), -8, 7)
        qb[np.broadcast_to(sf == 0, qb.shape)] = 0          # zero scale -> zero codes
        q[:, gi * group:gi * group + blk.shape[1]] = qb.astype(np.int8)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, K


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    """Sign extension via an arithmetic right shift of the nibble placed in the top bits."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p << 4).view(np.int8) >> 4                   # element 2j
    hi = p.view(np.int8) >> 4                          # element 2j+1
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out[:, :K]


def dequantize(packed: np.ndarray, scales: np.ndarray, K: int, group: int = 128) -> np.ndarray:
    """Full float64 reconstruction q * scale, [N, K]."""
    q = unpack_int4(packed, K).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), group, axis=1)[:, :K]
    return q * s


def int4_matmul(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, K: int,
                group: int = 128) -> np.ndarray:
    """y = x @ dequantize(W).T in float64, rounded to float32 at the end."""
    xd = np.asarray(x).astype(np.float64)
    return (xd @ dequantize(packed, scales, K, group).T).astype(np.float32)


# ----------------------------------------------------------- affine variant
# "Build a Blockwise INT4 Inference Engine", step 2 (per-group scale and zero
# point, codes in [0, 15]) with the range widened to include zero
# ("Quantizing a Language Model From Scratch": the zero point makes 0.0 exact).

def quantize_int4_affine(w: np.ndarray, group: int = 128):
    """w [N, K] float32 -> (packed uint8 unsigned codes, scales float16 [N, G],
    zero points uint8 [N, G], K)."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    G = -(-K // group)
    scales = np.zeros((N, G), dtype=np.float16)
    zeros = np.zeros((N, G), dtype=np.uint8)
    q = np.zeros((N, K + (K % 2)), dtype=np.uint8)
    for gi in range(G):
        blk = w[:, gi * group:min((gi + 1) * group, K)]
        lo = np.minimum(blk.min(axis=1), np.float32(0))
        hi = np.maximum(blk.max(axis=1), np.float32(0))
        s16 = ((hi - lo) / np.float32(15)).astype(np.float16)
        sf = s16.astype(np.float32)
        ok = sf != 0
        safe = np.where(ok, sf, np.float32(1))
        zp = np.where(ok, np.clip(np.rint(-lo / safe), 0, 15), 0).astype(np.int64)
        t = (blk / safe[:, None]).astype(np.float64)       # float32 quotient, widened
        qb = np.clip(np.rint(t + zp[:, None]), 0, 15)
        qb[~ok] = 0
        scales[:, gi] = s16
        zeros[:, gi] = zp
        q[:, gi * group:gi * group + blk.shape[1]] = qb.astype(np.uint8)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, zeros, K


def dequantize_affine(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, K: int,
                      group: int = 128) -> np.ndarray:
    """Full float64 reconstruction (code - zero point) * scale, [N, K]."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int64)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    z = np.repeat(np.asarray(zeros, dtype=np.int64), group, axis=1)[:, :K]
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), group, axis=1)[:, :K]
    return (codes[:, :K] - z) * s
