"""Seeded synthetic inputs for the grouped W4A16 MoE FFN.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no dequantisation, GEMV, activation or combine), so both
the HIP path and the CPU oracle can be fed from it.  BF16 rounding of drawn
values uses torch's CPU float32 -> bfloat16 cast.

Shapes follow the LFM2.5-24B-A2B MoE layer: hidden 2048, expert intermediate
1536, 64 experts, top-4, 38 MoE layers ("LFM2.5-24B-A2B on Your Own Hardware:
The RAM, KV Cache and Bandwidth Budget", section "Where do the 2.45B active
parameters actually go?"; "LFM2.5-24B-A2B -- Packed MXFP4 Inference", section
"Model and quantization").

Distributions (stated once, used everywhere):
  * nibbles: uniform random bytes, so every E2M1 code is uniform over 16;
  * E8M0 block scales: exponent byte uniform over 117..123 (2^-10 .. 2^-4);
  * E4M3FN block scales (NVFP4-style variant): uniform over the positive
    normal codes 0x08..0x7E;
  * per-expert FP32 tensor scales {gate/up, down}: uniform in [2^-14, 2^-12];
  * activations x: N(0, 1) rounded to BF16;
  * routing: top-k distinct expert ids, uniform or Zipf(s) over experts
    (rank r has weight r^-s, drawn without replacement and renormalised,
    ranks mapped to ids through a seeded per-layer permutation); routing
    weights are the softmax of k N(0, 1) draws, rounded to BF16.

Every stream has its own numpy PCG64 generator seeded by
SeedSequence([2026, family, stream, layer, index]).
"""
from __future__ import annotations

import dataclasses

import numpy as np

FMT_E8M0_G32 = 0
FMT_E4M3_G16 = 1

_ROOT = 2026
S_NIB, S_SCALE, S_TSCALE, S_X, S_IDS, S_ROUTE_W, S_PERM, S_ROUTER, S_BIAS = range(9)


@dataclasses.dataclass(frozen=True)
class Shape:
    hidden: int = 2048
    inter: int = 1536
    experts: int = 64
    top_k: int = 4
    layers: int = 38

    def group(self, fmt: int) -> int:
        return 16 if fmt == FMT_E4M3_G16 else 32

    def nibble_bytes(self) -> int:
        """Bytes of one expert's packed [gate | up | down] nibbles."""
        return 3 * self.hidden * self.inter // 2

    def scale_bytes(self, fmt: int) -> int:
        """Bytes of one expert's [gate | up | down] block scales."""
        return 3 * self.hidden * self.inter // self.group(fmt)

    def expert_bytes(self, fmt: int) -> int:
        return self.nibble_bytes() + self.scale_bytes(fmt)


LFM24B = Shape()


def _rng(family: int, stream: int, layer: int, index: int) -> np.random.Generator:
    ss = np.random.SeedSequence([_ROOT, int(family), int(stream), int(layer), int(index)])
    return np.random.Generator(np.random.PCG64(ss))


def weight_family(fmt: int) -> int:
    """MXFP4 and NVFP4-style experts use separate weight seeds."""
    return 100 + int(fmt)


def expert_nibbles(shape: Shape, fmt: int, layer: int, expert: int) -> np.ndarray:
    rng = _rng(weight_family(fmt), S_NIB, layer, expert)
    return np.frombuffer(rng.bytes(shape.nibble_bytes()), dtype=np.uint8).copy()


def expert_scales(shape: Shape, fmt: int, layer: int, expert: int) -> np.ndarray:
    rng = _rng(weight_family(fmt), S_SCALE, layer, expert)
    n = shape.scale_bytes(fmt)
    if fmt == FMT_E4M3_G16:
        return rng.integers(0x08, 0x7F, size=n, dtype=np.uint8)
    return rng.integers(117, 124, size=n, dtype=np.uint8)


def expert_triplet(shape: Shape, fmt: int, layer: int, expert: int) -> np.ndarray:
    """One expert as a contiguous byte buffer: nibbles, then scales."""
    return np.concatenate([expert_nibbles(shape, fmt, layer, expert),
                           expert_scales(shape, fmt, layer, expert)])


def router_weights(shape: Shape, family: int, layer: int) -> np.ndarray:
    """BF16 bits [E][H] of one layer's router projection: N(0, 1/H), so that a
    unit-RMS input gives logits of unit variance."""
    rng = _rng(family, S_ROUTER, layer, 0)
    w = rng.standard_normal((shape.experts, shape.hidden), dtype=np.float32)
    return to_bf16_bits(w / np.float32(np.sqrt(shape.hidden)))


def expert_bias(shape: Shape, family: int, layer: int) -> np.ndarray:
    """float32 [E] selection bias of one layer, uniform on [-0.05, 0.05]."""
    rng = _rng(family, S_BIAS, layer, 0)
    return rng.uniform(-0.05, 0.05, shape.experts).astype(np.float32)


def tensor_scales(shape: Shape, fmt: int, layer: int) -> np.ndarray | None:
    """[E][2] float32 {gate/up, down}, or None for the E8M0 format."""
    if fmt != FMT_E4M3_G16:
        return None
    rng = _rng(weight_family(fmt), S_TSCALE, layer, 0)
    return rng.uniform(2.0 ** -14, 2.0 ** -12, size=(shape.experts, 2)).astype(np.float32)


def to_bf16_bits(values) -> np.ndarray:
    """Round to BF16 with torch's CPU cast; returns uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def activations(family: int, layer: int, step: int, tokens: int, hidden: int) -> np.ndarray:
    rng = _rng(family, S_X, layer, step)
    return to_bf16_bits(rng.standard_normal((tokens, hidden), dtype=np.float32))


def _route_weights(family: int, layer: int, step: int, tokens: int, k: int) -> np.ndarray:
    rng = _rng(family, S_ROUTE_W, layer, step)
    z = rng.standard_normal((tokens, k))
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return to_bf16_bits((z / z.sum(axis=1, keepdims=True)).astype(np.float32))


def routing_uniform(family: int, layer: int, step: int, tokens: int, experts: int, k: int):
    """k distinct ids per token, uniform over experts; softmax route weights."""
    rng = _rng(family, S_IDS, layer, step)
    ids = np.stack([rng.choice(experts, size=k, replace=False) for _ in range(tokens)])
    return ids.astype(np.int32), _route_weights(family, layer, step, tokens, k)


def routing_zipf(family: int, layer: int, step: int, tokens: int, experts: int, k: int,
                 s: float = 1.1):
    """k distinct ids per token drawn Zipf(s) over expert ranks without
    replacement; ranks map to ids through a seeded permutation per layer."""
    perm = _rng(family, S_PERM, layer, 0).permutation(experts)
    rng = _rng(family, S_IDS, layer, step)
    base = np.arange(1, experts + 1, dtype=np.float64) ** (-s)
    ids = np.empty((tokens, k), np.int32)
    for t in range(tokens):
        p = base.copy()
        for j in range(k):
            r = rng.choice(experts, p=p / p.sum())
            ids[t, j] = perm[r]
            p[r] = 0.0
    return ids, _route_weights(family, layer, step, tokens, k)


# -- the five workloads ---------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    family: int          # seed family for activations and routing
    fmt: int
    tokens: int          # tokens per call
    layers: int          # distinct layers in play
    steps: int           # calls per layer (decode steps or prefill chunks)
    routing: str         # "uniform" or "zipf"
    chained: bool        # pre-norm + BF16 residual between layers


WORKLOADS = {
    # one MoE layer, one token
    "c0": Workload("c0", 0, FMT_E8M0_G32, 1, 1, 1, "uniform", False),
    # 38 chained MoE layers, batch-1 decode, 64 steps
    "c1": Workload("c1", 1, FMT_E8M0_G32, 1, 38, 64, "uniform", True),
    # concurrency-32 decode, Zipf(1.1) routing, one layer or the 38-layer stack
    "c2": Workload("c2", 2, FMT_E8M0_G32, 32, 38, 64, "zipf", True),
    # prefill: 8192 tokens as 128 chunks of 64 through one layer
    "c3": Workload("c3", 3, FMT_E8M0_G32, 64, 1, 128, "uniform", False),
    # NVFP4-style scales, batch 1 (uniform routing) and batch 32 (Zipf)
    "c4": Workload("c4", 4, FMT_E4M3_G16, 1, 1, 1, "uniform", False),
    "c4b32": Workload("c4b32", 5, FMT_E4M3_G16, 32, 1, 1, "zipf", False),
}


def routing(w: Workload, layer: int, step: int, shape: Shape = LFM24B, tokens: int | None = None):
    T = w.tokens if tokens is None else tokens
    if w.routing == "zipf":
        return routing_zipf(w.family, layer, step, T, shape.experts, shape.top_k)
    return routing_uniform(w.family, layer, step, T, shape.experts, shape.top_k)


def inputs(w: Workload, layer: int, step: int, shape: Shape = LFM24B, tokens: int | None = None):
    """(x, ids, route_w) for one call of workload ``w``."""
    T = w.tokens if tokens is None else tokens
    x = activations(w.family, layer, step, T, shape.hidden)
    ids, rw = routing(w, layer, step, shape, T)
    return x, ids, rw
