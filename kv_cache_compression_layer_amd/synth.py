"""Seeded synthetic KV-cache generator.

This module only draws inputs. It holds none of the codec's arithmetic, so the
CPU oracle and the HIP path can both be fed from it without sharing code.

The pages this codec follows measure on KV captured from real models
(OPT-125m and Mistral-7B in the CacheGen reproduction thread on zingnex.cn,
section on KV extraction) and on LMCache's synthetic ``_generate_kv`` blobs of
32 layers x 8 heads x 128 in bf16 (LMCache CacheGen page, 0539edu.com, section
on the end-to-end benchmark). No weights or captures are available, so this
generator stands in for them with the same shapes and a value structure that
is typical of KV activations:

* per-channel standard deviation ``sigma ~ LogNormal(0, 0.5)``;
* a fraction of outlier channels per (K|V, layer) whose sigma is multiplied
  by a large factor;
* a stationary AR(1) process along tokens with coefficient ``rho`` and
  Gaussian or unit-variance Laplace innovations.

Recipe (numpy ``default_rng(seed)``, draw order fixed):

1. ``sigma = exp(0.5 * N(0,1))`` of shape ``[2, L, C]``.
2. For each (kv, layer) in that order, ``rng.choice(C, k, replace=False)``
   with ``k = round(frac * C)`` picks outlier channels; their sigma is
   multiplied by ``scale``.
3. Innovations ``e_t`` of shape ``[2, L, C]`` are drawn in token order
   (in blocks of tokens, which yields the same stream as one draw per token):
   ``N(0,1)`` or ``Laplace(0, 1/sqrt(2))``.
4. ``x_0 = sigma * e_0``; ``x_t = rho * x_{t-1} + (sqrt(1-rho^2) * sigma) * e_t``
   in float64.
5. float64 -> float32 (round to nearest even) -> bf16 (round to nearest
   even) and stored as element ``[l, kv, t, c]`` of ``[L, 2, T, H, D]``.

The result is returned as a ``uint16`` array of bf16 bit patterns.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "generate_kv", "generate_workload", "bf16_bits_to_f32", "f32_to_bf16_bits"]


@dataclass(frozen=True)
class Workload:
    """A synthetic KV workload: model-shaped dimensions plus generator knobs."""

    name: str
    nlayers: int
    nheads: int
    head_size: int
    ntokens: int
    rho: float
    innovations: str  # "gauss" or "laplace"
    outlier_frac: float
    outlier_scale: float
    seed: int

    @property
    def nchannels(self) -> int:
        return self.nheads * self.head_size

    @property
    def shape(self) -> tuple:
        return (self.nlayers, 2, self.ntokens, self.nheads, self.head_size)

    @property
    def raw_bytes(self) -> int:
        return 2 * self.nlayers * 2 * self.ntokens * self.nchannels


# Model-shaped workloads. Bins for all of them follow the default per-layer
# rule of the LMCache CacheGen page (section 1, QuantizationSpec).
WORKLOADS = {
    w.name: w
    for w in [
        # OPT-125m: 12 layers, 12 heads x 64, one 64-token chunk, no outliers.
        Workload("opt125m_t64", 12, 12, 64, 64, 0.9, "gauss", 0.0, 1.0, 1001),
        # Mistral-7B: 32 layers, 8 KV heads x 128, one 256-token chunk.
        Workload("mistral7b_t256", 32, 8, 128, 256, 0.9, "gauss", 0.01, 20.0, 1002),
        # Same shape, 768-token call (three 256-token coder chunks).
        Workload("mistral7b_t768", 32, 8, 128, 768, 0.9, "gauss", 0.01, 20.0, 1003),
        # Llama-3.1-8B long context: 32768 tokens, 128 coder chunks.
        Workload("llama31_8b_t32k", 32, 8, 128, 32768, 0.9, "gauss", 0.01, 20.0, 1004),
        # GLM-4-9B: 40 layers, 2 KV heads x 128, heavy tails.
        Workload("glm4_9b_t16k", 40, 2, 128, 16384, 0.8, "laplace", 0.02, 50.0, 1005),
    ]
}


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def generate_kv(
    nlayers: int,
    ntokens: int,
    nheads: int,
    head_size: int,
    *,
    rho: float = 0.9,
    innovations: str = "gauss",
    outlier_frac: float = 0.0,
    outlier_scale: float = 1.0,
    seed: int = 0,
    block_tokens: int = 256,
) -> np.ndarray:
    """Draw a bf16 KV blob ``[L, 2, T, H, D]`` (as uint16 bit patterns)."""
    L, T, C = nlayers, ntokens, nheads * head_size
    if innovations not in ("gauss", "laplace"):
        raise ValueError(f"unknown innovations {innovations!r}")
    rng = np.random.default_rng(seed)
    sigma = np.exp(0.5 * rng.standard_normal((2, L, C)))
    k = int(round(outlier_frac * C))
    if k > 0:
        for kv in range(2):
            for l in range(L):
                idx = rng.choice(C, k, replace=False)
                sigma[kv, l, idx] *= outlier_scale
    a_sigma = math.sqrt(1.0 - rho * rho) * sigma
    out = np.empty((L, 2, T, C), dtype=np.uint16)
    x = None
    for t0 in range(0, T, block_tokens):
        tb = min(block_tokens, T - t0)
        if innovations == "gauss":
            e = rng.standard_normal((tb, 2, L, C))
        else:
            e = rng.laplace(0.0, 1.0 / math.sqrt(2.0), (tb, 2, L, C))
        xs = np.empty((tb, 2, L, C), dtype=np.float64)
        for i in range(tb):
            if x is None:
                x = sigma * e[i]
            else:
                x = rho * x + a_sigma * e[i]
            xs[i] = x
        bits = f32_to_bf16_bits(xs.astype(np.float32))  # [tb, 2, L, C]
        out[:, :, t0 : t0 + tb, :] = bits.transpose(2, 1, 0, 3)
    return out.reshape(L, 2, T, nheads, head_size)


def generate_workload(w: Workload | str) -> np.ndarray:
    """Draw the KV blob of a named workload."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return generate_kv(
        w.nlayers,
        w.ntokens,
        w.nheads,
        w.head_size,
        rho=w.rho,
        innovations=w.innovations,
        outlier_frac=w.outlier_frac,
        outlier_scale=w.outlier_scale,
        seed=w.seed,
    )
