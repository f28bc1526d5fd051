"""Seeded synthetic inputs for the dropless top-k MoE layer.

This module is shared by the CPU oracle (under ``oracle/``) and the HIP path.
It holds only random-number generation and storage-format conversion; none of
the layer's arithmetic lives here.

The benchmark pages (probjax ``kernel_gmm_gpu.json``, ``gpu_nn.json`` and
``gpu_moe_h100.json``) run on seeded Gaussian tokens with uniform routing
(``skew`` 0.0 in every ``config.sources[*].config`` block; the pages also
name a skew of 0.9 without defining it, see ``Problem.skew``) and print
neither seeds nor a generator, so the generator is defined here:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014) used counter-style: draw ``i`` of a stream with
  key ``s`` is ``mix64(s + (i + 1) * GOLDEN)``.
* Each tensor has its own stream, keyed by ``mix64(seed * GOLDEN + tensor_id)``.
* Uniforms in (0, 1) are ``((u >> 11) + 0.5) * 2**-53``.
* Normals come from the Box-Muller transform in double: the pair
  ``(u1, u2) = (draw 2j, draw 2j+1)`` yields element ``2j`` as
  ``r cos(2 pi u2)`` and element ``2j+1`` as ``r sin(2 pi u2)``, with
  ``r = sqrt(-2 ln u1)``.
* A value of standard deviation ``std`` is ``std * z`` in double, rounded to
  nearest-even fp32, then (for bf16 storage) rounded to nearest-even bf16.

Initialisation follows N(0, 1/fan_in) with variance ``1/fan_in`` (untruncated):
fan-in ``d_model`` for the router and for the gate and up projections, the
expert width for an expert's down projection and the shared width for the
shared expert's down projection. Tokens and the upstream gradient ``G`` are
N(0, 1).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Stream id of each tensor (fixed order).
TENSOR_IDS = {
    "x": 0,
    "w_router": 1,
    "w_gate": 2,
    "w_up": 3,
    "w_down": 4,
    "ws_gate": 5,
    "ws_up": 6,
    "ws_down": 7,
    "grad_out": 8,
}

_CHUNK = 1 << 22  # elements generated per numpy pass (bounds temporary memory)


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function (wrapping uint64 arithmetic)."""
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) * GOLDEN + np.uint64(tensor_id)
    return _mix64(np.array([s], dtype=np.uint64))[0]


def uniform_draws(key: np.uint64, start: int, count: int) -> np.ndarray:
    """Draws ``start .. start+count-1`` of stream ``key`` as uniforms in (0,1), float64."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        u = _mix64(key + idx * GOLDEN)
    return ((u >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def standard_normal(seed: int, tensor_id: int, n: int) -> np.ndarray:
    """``n`` N(0,1) values of one tensor's stream, float64."""
    key = stream_key(seed, tensor_id)
    out = np.empty(n, dtype=np.float64)
    npairs = (n + 1) // 2
    for p0 in range(0, npairs, _CHUNK):
        p1 = min(npairs, p0 + _CHUNK)
        u = uniform_draws(key, 2 * p0, 2 * (p1 - p0))
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log(u1))
        th = 2.0 * math.pi * u2
        z = np.empty(2 * (p1 - p0), dtype=np.float64)
        z[0::2] = r * np.cos(th)
        z[1::2] = r * np.sin(th)
        lo, hi = 2 * p0, min(n, 2 * p1)
        out[lo:hi] = z[: hi - lo]
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns (finite inputs)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        return ((b + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp32 widening of uint16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Problem:
    """Problem statement in the pages' record fields: tokens, experts, top_k,
    d_model, d_hidden, shared width (0 = none), dtype, block_m."""

    tokens: int
    experts: int
    top_k: int
    d_model: int
    d_hidden: int
    d_shared: int = 0
    dtype: str = "bf16"  # "fp32" or "bf16": storage dtype of x, expert weights, activations
    block_m: int = 128
    # Routing skew of the generated router (0 = uniform routing). Not a layer
    # argument: it only shapes the synthetic router, see make_inputs.
    skew: float = 0.0
    # Capacity routing (kernel_gmm_gpu.json "routing": "capacity"): at most
    # this many token-slots per expert, the first in flat slot order; 0 =
    # dropless. A layer argument (moe_problem.capacity).
    capacity: int = 0

    @property
    def slots(self) -> int:
        return self.tokens * self.top_k


def capacity_for(p: Problem, factor: float) -> int:
    """Per-expert capacity of a capacity factor: ceil(factor * tokens *
    top_k / experts), the mean load scaled (at least 1)."""
    return max(1, math.ceil(factor * p.tokens * p.top_k / p.experts))


@dataclasses.dataclass
class Tensor:
    """One generated tensor: ``stored`` is what the device receives (fp32 array,
    or uint16 bf16 bit patterns); ``value`` is the exact fp32 widening of it."""

    stored: np.ndarray
    value: np.ndarray


def gen_tensor(seed: int, name: str, shape, std: float, dtype: str) -> Tensor:
    n = int(np.prod(shape))
    z = standard_normal(seed, TENSOR_IDS[name], n)
    f = (z * std).astype(np.float32).reshape(shape)
    if dtype == "fp32":
        return Tensor(stored=f, value=f)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(f).reshape(shape)
        return Tensor(stored=bits, value=bf16_bits_to_f32(bits).reshape(shape))
    raise ValueError(dtype)


def make_inputs(p: Problem, seed: int = 0, with_grad_out: bool = False,
                names: Optional[list] = None) -> Dict[str, Tensor]:
    """All tensors of problem ``p``. The router is always fp32; the rest use ``p.dtype``."""
    T, E, d, h, hs = p.tokens, p.experts, p.d_model, p.d_hidden, p.d_shared
    spec = {
        "x": ((T, d), 1.0, p.dtype),
        "w_router": ((d, E), 1.0 / math.sqrt(d), "fp32"),
        "w_gate": ((E, d, h), 1.0 / math.sqrt(d), p.dtype),
        "w_up": ((E, d, h), 1.0 / math.sqrt(d), p.dtype),
        "w_down": ((E, h, d), 1.0 / math.sqrt(h), p.dtype),
    }
    if hs > 0:
        spec["ws_gate"] = ((d, hs), 1.0 / math.sqrt(d), p.dtype)
        spec["ws_up"] = ((d, hs), 1.0 / math.sqrt(d), p.dtype)
        spec["ws_down"] = ((hs, d), 1.0 / math.sqrt(hs), p.dtype)
    if with_grad_out:
        spec["grad_out"] = ((T, d), 1.0, p.dtype)
    out = {}
    for name, (shape, std, dt) in spec.items():
        if names is not None and name not in names:
            continue
        out[name] = gen_tensor(seed, name, shape, std, dt)
    if p.skew > 0.0 and "w_router" in out:
        # Skewed routing: expert e's router column is scaled by
        # (1 - skew)^(e / (E - 1)), so its logits have standard deviation
        # falling from 1 (expert 0) to 1 - skew (expert E - 1) and top-k picks
        # low-index experts more often (skew 0.9 at E=64, k=8: the busiest
        # expert gets about 2.7 times the mean load). At skew 0 nothing changes.
        e = np.arange(E, dtype=np.float64)
        scale = ((1.0 - p.skew) ** (e / max(E - 1, 1))).astype(np.float32)
        f = (out["w_router"].stored * scale[None, :]).astype(np.float32)
        out["w_router"] = Tensor(stored=f, value=f)
    return out


# The workloads the layer is measured on (the pages' problem fields; shapes
# as stated with each workload). Index 3 is the headline forward workload and
# index 4 the train step. bf16 forward workloads cut expert rows into
# 256-row tiles, the row tile of the 256 x 256 MFMA engine.
WORKLOADS = {
    0: ("fwd fp32, 4096 tok, E8 top-2, d512 h1024", Problem(4096, 8, 2, 512, 1024, 0, "fp32", 128), "fwd"),
    1: ("fwd bf16, 32768 tok, E8 top-2, d512 h1024", Problem(32768, 8, 2, 512, 1024, 0, "bf16", 256), "fwd"),
    2: ("fwd bf16, 32768 tok, E64 top-4, d512 h256", Problem(32768, 64, 4, 512, 256, 0, "bf16", 256), "fwd"),
    3: ("fwd bf16, 131072 tok, E64 top-8, d512 h128, shared 1024",
        Problem(131072, 64, 8, 512, 128, 1024, "bf16", 256), "fwd"),
    4: ("train bf16, 16384 tok, E64 top-8, d512 h128, shared 1024",
        Problem(16384, 64, 8, 512, 128, 1024, "bf16", 128), "train"),
}
