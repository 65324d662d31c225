"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no quantization or matmul arithmetic: it only draws weights
and activations with NumPy's PCG64 ``default_rng`` and builds the special
rows of the edge-case matrix. Both the CPU oracle and the HIP path are fed
from here, and nothing here depends on either.

Recipes (distribution and shapes follow the pages' workloads; see each entry):

* W: ``default_rng(seed).normal(0, sigma, size=(N, K)).astype(float32)`` -- the
  recipe of the drill page's visible round-trip test (normal draws cast to
  float32); sigma 1 for the small cases, 0.02 as a stand-in for trained
  transformer weights.
* 7B-class outliers: ``default_rng(2).choice(N*K, round(1e-3*N*K), replace=False)``
  picks exactly 0.1% of the entries, which are multiplied by 20 (a stand-in for
  the outlier weights discussed on "Quantizing a Language Model From Scratch",
  "The outlier problem").
* x: ``default_rng(1).normal(size=(M, K)).astype(float16 | float32)``, a stand-in
  for normalised hidden states. Rows are a prefix property of the stream: the
  first M1 rows of the M2-row draw equal the M1-row draw.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_W = 0
SEED_X = 1
SEED_OUTLIERS = 2

# Smallest positive binary16 (2^-24). A value of -8 * 2^-24 has absmax/7
# rounding to exactly this scale and then quantizes to -8 (edge-case row 7).
HALF_TINY = 2.0 ** -24


@dataclass(frozen=True)
class Case:
    """One weight matrix of a configuration."""
    name: str
    N: int
    K: int
    group: int
    sigma: float = 1.0
    outliers: bool = False
    edge_rows: bool = False            # zero group in row 5, -8 codes in row 7
    x_dtype: str = "float16"
    Ms: tuple = (1,)


@dataclass(frozen=True)
class Config:
    key: str
    title: str
    cases: tuple = field(default_factory=tuple)


def weights(case: Case) -> np.ndarray:
    rng = np.random.default_rng(SEED_W)
    w = rng.normal(0.0, case.sigma, size=(case.N, case.K)).astype(np.float32)
    if case.outliers:
        count = int(round(1e-3 * case.N * case.K))
        idx = np.random.default_rng(SEED_OUTLIERS).choice(case.N * case.K, count, replace=False)
        w.reshape(-1)[idx] *= np.float32(20.0)
    if case.edge_rows:
        if case.N > 5:
            w[5, :min(case.group, case.K)] = 0.0
        if case.N > 7:
            w[7, :] = np.float32(-8.0 * HALF_TINY)
    return w


def activations(M: int, K: int, dtype: str = "float16", seed: int = SEED_X) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.normal(size=(M, K)).astype(np.dtype(dtype))


def _c3_cases():
    shapes = [("c_attn", 2304, 768), ("attn_c_proj", 768, 768), ("c_fc", 3072, 768),
              ("mlp_c_proj", 768, 3072)]
    return tuple(Case(f"{nm}_g{g}", N, K, g, sigma=0.02, Ms=(1, 4, 16))
                 for g in (64, 32) for (nm, N, K) in shapes)


CONFIGS = {
    "c1": Config("c1", "W [64,256] N(0,1), group 128, x [4,256] fp32",
                 (Case("w64x256", 64, 256, 128, x_dtype="float32", Ms=(4,)),)),
    "c2": Config("c2", "edge sweep W [48,301] (odd K, partial last group), group 128, x [3,301] fp32",
                 (Case("w48x301", 48, 301, 128, edge_rows=True, x_dtype="float32", Ms=(3,)),)),
    "c3": Config("c3", "small-transformer linears N(0,0.02), group 64 and 32, x fp16",
                 _c3_cases()),
    "c4": Config("c4", "7B-class linears N(0,0.02) + 0.1% x20 outliers, group 128, x fp16",
                 (Case("q_proj_4096x4096", 4096, 4096, 128, 0.02, True, Ms=(1, 16, 512, 2048)),
                  Case("up_proj_11008x4096", 11008, 4096, 128, 0.02, True, Ms=(1, 16, 512, 2048)),
                  Case("down_proj_4096x11008", 4096, 11008, 128, 0.02, True, Ms=(1, 16, 512, 2048)))),
    "c5": Config("c5", "large FFN W [28672,8192] N(0,0.02), group 128, x fp16",
                 (Case("ffn_28672x8192", 28672, 8192, 128, 0.02, Ms=(1, 8, 256, 4096)),)),
}
