"""Seeded synthetic inputs for the single-layer LSTM forward + BPTT path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds the workload definitions (shapes and value distributions) and the
random-number recipe, and nothing of the LSTM's arithmetic.

Recipe
------
* one generator per tensor: ``numpy.random.default_rng([seed, tensor_id])``
  with tensor ids W=0, b=1, x=2, h0=3, c0=4, dy=5, dhT=6, dcT=7;
* uniform draws ``rng.uniform(-k, k)``, normal draws ``rng.normal(0, s)``
  where ``s`` is the standard deviation;
* draws are fp64, then rounded to the storage dtype: fp32 by numpy's
  round-to-nearest-even cast, bf16 by rounding that fp32 value to the nearest
  bf16 (ties to even) with integer arithmetic on the bit pattern, f16 by
  numpy's fp32 -> fp16 cast of that fp32 value (nearest, ties to even).  Both sides
  of every comparison consume exactly these stored values (the oracle upcast
  to fp64).

The weight/bias range U(-1/sqrt(H), 1/sqrt(H)) is the usual recurrent-layer
initialisation (k = 1/hidden_size) that the PyTorch recurrent-layer
documentation page states.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TENSOR_IDS = dict(W=0, b=1, x=2, h0=3, c0=4, dy=5, dhT=6, dcT=7)


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32", "bf16" or "f16" (storage); accumulation is always fp32
    T: int
    B: int
    I: int
    H: int
    # distribution per tensor: ("u", k) uniform(-k,k); ("n", s) normal(0,s); ("z",) zero/absent
    dist: dict = field(default_factory=dict)

    @property
    def flops(self) -> float:
        """Algorithmic fwd+bwd FLOPs: the three W-products (W z, W^T dG,
        dG z^T), 2*4H*(H+I) each per (t, b)."""
        return 24.0 * self.T * self.B * self.H * (self.H + self.I)


def _std(H, x="n1", h="n.5", dy="n1", carry="z", wb=None):
    k = 1.0 / np.sqrt(H)
    spec = {"n1": ("n", 1.0), "n.5": ("n", 0.5), "n.1": ("n", 0.1), "z": ("z",)}
    d = dict(W=("u", k), b=("u", k), x=spec[x], h0=spec[h], c0=spec[h], dy=spec[dy],
             dhT=spec[carry], dcT=spec[carry])
    return d


# The five workloads, named by their sizes.
WORKLOADS = {
    "f32_T8_B4_I16_H32": Workload("f32_T8_B4_I16_H32", "f32", 8, 4, 16, 32, _std(32)),
    "f32_T64_B32_I256_H256": Workload("f32_T64_B32_I256_H256", "f32", 64, 32, 256, 256,
                                      _std(256, carry="n1")),
    "bf16_T128_B64_I512_H1024": Workload("bf16_T128_B64_I512_H1024", "bf16", 128, 64, 512, 1024,
                                         _std(1024, h="z")),
    "bf16_T512_B16_I1024_H2048": Workload("bf16_T512_B16_I1024_H2048", "bf16", 512, 16, 1024, 2048,
                                          _std(2048, h="z")),
    "bf16_T256_B256_I1024_H1024": Workload("bf16_T256_B256_I1024_H1024", "bf16", 256, 256, 1024, 1024,
                                           _std(1024, dy="n.1")),
}
# fp16 storage (the FLOAT16 of the operator page's dtype column) on the
# shapes and distributions of the three bf16 workloads
for _n in [n for n in WORKLOADS if n.startswith("bf16_")]:
    _w = WORKLOADS[_n]
    _f = "f16_" + _n[len("bf16_"):]
    WORKLOADS[_f] = Workload(_f, "f16", _w.T, _w.B, _w.I, _w.H, _w.dist)
SMALL = "f32_T8_B4_I16_H32"
# the benchmark's default: the largest workload that fits one GPU
HEADLINE = "bf16_T256_B256_I1024_H1024"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.
    NaN stays NaN (quiet)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 draw -> stored value, returned as fp64 (exactly representable in
    the storage dtype)."""
    a32 = np.asarray(a64, dtype=np.float32)
    if dtype == "f32":
        return a32.astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a32)).astype(np.float64)
    if dtype == "f16":
        return a32.astype(np.float16).astype(np.float64)
    raise ValueError(dtype)


def _draw(seed: int, name: str, shape, dist) -> np.ndarray | None:
    if dist[0] == "z":
        return None
    rng = np.random.default_rng([seed, TENSOR_IDS[name]])
    if dist[0] == "u":
        return rng.uniform(-dist[1], dist[1], size=shape)
    if dist[0] == "n":
        return rng.normal(0.0, dist[1], size=shape)
    raise ValueError(dist)


def make_inputs(T, B, I, H, dtype="f32", seed=0, dist=None, with_bias=True):
    """Draw one set of inputs.  Returns a dict of fp64 arrays holding the
    stored (dtype-rounded) values; absent optional tensors are None."""
    if dist is None:
        dist = _std(H)
    shapes = dict(W=(4 * H, H + I), b=(4 * H,), x=(T, B, I), h0=(B, H), c0=(B, H),
                  dy=(T, B, H), dhT=(B, H), dcT=(B, H))
    out = {}
    for name, shp in shapes.items():
        if name == "b" and not with_bias:
            out[name] = None
            continue
        v = _draw(seed, name, shp, dist[name])
        out[name] = None if v is None else round_to_storage(v, dtype)
    if out["dy"] is None:
        out["dy"] = np.zeros(shapes["dy"])
    out["T"], out["B"], out["I"], out["H"], out["dtype"] = T, B, I, H, dtype
    return out


def workload_inputs(name: str, seed: int = 0):
    w = WORKLOADS[name]
    return make_inputs(w.T, w.B, w.I, w.H, w.dtype, seed, w.dist)
