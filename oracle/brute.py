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
