"""Seeded synthetic inputs for the MoE route-count / dispatch / combine path.

This module only draws inputs.  It holds none of the method's arithmetic (no
counting, slotting, packing or reduction), so both the CPU oracle and the HIP
path can be fed from it without sharing any code with each other.

Workloads (shapes and distributions follow the DeepSeek-like shapes used on the
pages: hidden 7168, top-k 8, 256 experts in "cco + flydsl dispatch/combine"
(ROCm/mori PR 448, PR description) and "Drop cooperative launch from the
CTA-independent local kernels" (MoonEP PR 34, "Measured impact" table)):

  tiny        T=64    H=256   E=8   K=2  uniform routing, bf16 x, identity experts
  decode      T=32    H=6144  E=128 K=8  uniform routing, bf16 x, expert = x * c_e
  prefill     T=4096  H=7168  E=256 K=8  uniform routing, bf16 x, padded layout
  skewed_fp8  T=8192  H=7168  E=256 K=8  Zipf(1.2) routing, bf16 x, fp8 payload
  dedup       T=16384 H=4096  E=64  K=6  R=8 virtual ranks, uniform routing, f32 x
  uniform_bf16 T=8192 H=7168  E=256 K=8  uniform routing, bf16 x and payload (the
              skewed_fp8 shape without the skew and the fp8 pack; seed 4 as well)

Random draws, in this order, from numpy.random.Generator(PCG64(seed)) with
seed = the workload number (1..5; uniform_bf16 shares seed 4):
  1. expert permutation (Zipf only)
  2. routing (distinct top-K experts per token)
  3. gate logits  -> weights = softmax over the K picks, in float64, cast to float32
  4. x ~ N(0,1) float32, rounded to bf16 by torch (round to nearest even) unless f32
  5. expert constants c_e = 0.5 + U[0,1) (decode only)

Uniform distinct routing takes the first K columns of a random permutation of
the E experts per token.  Zipf(s) distinct routing samples without replacement
from p_i ~ i^-s (i = 1..E) by the Gumbel-top-K trick, then maps the ranks
through the seeded expert permutation, so the hot experts are scattered over
the id range.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "uniform_routing", "zipf_routing",
           "softmax_weights", "normal_x", "bf16_bits_from_f32", "f32_from_bf16_bits",
           "inject_outliers"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int
    H: int
    E: int
    K: int
    routing: str            # "uniform" | "zipf"
    x_dtype: str            # "bf16" | "f32"
    packed_dtype: str       # "bf16" | "f32" | "fp8"
    layout: str             # "compact" | "padded"
    expert: str             # "identity" | "scale" | "dequant"
    R: int = 0              # virtual ranks (dedup only)
    zipf_s: float = 1.2


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 256, 8, 2, "uniform", "bf16", "bf16", "compact", "identity"),
    "decode": Workload("decode", 2, 32, 6144, 128, 8, "uniform", "bf16", "bf16", "compact", "scale"),
    "prefill": Workload("prefill", 3, 4096, 7168, 256, 8, "uniform", "bf16", "bf16", "padded", "identity"),
    "skewed_fp8": Workload("skewed_fp8", 4, 8192, 7168, 256, 8, "zipf", "bf16", "fp8", "compact", "dequant"),
    "dedup": Workload("dedup", 5, 16384, 4096, 64, 6, "uniform", "f32", "f32", "compact", "identity", R=8),
    "uniform_bf16": Workload("uniform_bf16", 4, 8192, 7168, 256, 8, "uniform", "bf16", "bf16", "compact",
                             "identity"),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (torch's round-to-nearest-even); return the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniform_routing(rng: np.random.Generator, T: int, E: int, K: int) -> np.ndarray:
    """K distinct experts per token, uniform over the E experts."""
    return np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :K].astype(np.int32)


def zipf_routing(rng: np.random.Generator, T: int, E: int, K: int, s: float,
                 perm: np.ndarray) -> np.ndarray:
    """K distinct experts per token drawn without replacement from p_i ~ i^-s (Gumbel-top-K)."""
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    u = rng.random((T, E))
    keys = logp[None, :] - np.log(-np.log(u))
    ranks = np.argsort(-keys, axis=1, kind="stable")[:, :K]
    return perm[ranks].astype(np.int32)


def softmax_weights(rng: np.random.Generator, T: int, K: int) -> np.ndarray:
    """Softmax of N(0,1) gate logits over the K picks, float64 math, float32 result."""
    z = rng.standard_normal((T, K))
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def normal_x(rng: np.random.Generator, T: int, H: int, dtype: str) -> np.ndarray:
    """x ~ N(0,1): float32 array for "f32", uint16 bf16 bit patterns for "bf16"."""
    x = rng.standard_normal((T, H), dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(dtype)


def inject_outliers(x_bf16: np.ndarray, rows: np.ndarray, factor: float = 1000.0) -> np.ndarray:
    """Scale the given rows of a bf16 bit array by `factor` (re-rounded to bf16).

    Used by tests so that some 128-element blocks exceed the fp8 e4m3 range and
    take the scaled branch of the blockwise pack."""
    out = x_bf16.copy()
    vals = f32_from_bf16_bits(out[rows]) * np.float32(factor)
    out[rows] = bf16_bits_from_f32(vals)
    return out


def make_inputs(name: str, T: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """Draw the inputs of a named workload.

    T overrides the token count (the same distributions, fewer or more rows);
    seed overrides the workload's own seed.  Returns a dict with
      idx  int32 [T,K]     expert ids
      w    float32 [T,K]   gate weights
      x    uint16 [T,H] (bf16 bits) or float32 [T,H]
      c    float32 [E]     expert constants (decode only, else None)
    plus the workload's shape fields.
    """
    wl = WORKLOADS[name]
    T = wl.T if T is None else int(T)
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    perm = rng.permutation(wl.E).astype(np.int64) if wl.routing == "zipf" else None
    if wl.routing == "zipf":
        idx = zipf_routing(rng, T, wl.E, wl.K, wl.zipf_s, perm)
    else:
        idx = uniform_routing(rng, T, wl.E, wl.K)
    w = softmax_weights(rng, T, wl.K)
    x = normal_x(rng, T, wl.H, wl.x_dtype)
    c = (0.5 + rng.random(wl.E)).astype(np.float32) if wl.expert == "scale" else None
    return dict(name=name, T=T, H=wl.H, E=wl.E, K=wl.K, R=wl.R, idx=idx, w=w, x=x, c=c,
                x_dtype=wl.x_dtype, packed_dtype=wl.packed_dtype, layout=wl.layout,
                expert=wl.expert, workload=wl)
