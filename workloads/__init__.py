"""Seeded synthetic workloads for the layout-aware reduce-scatter and all-gather placement.

This module holds the *inputs* only: parameter-group shapes, rank and contributor counts, value
scales, and seeded generators of bf16 bit patterns.  It holds none of the method's arithmetic (no
geometry, no sums, no placement), so both the oracle and the GPU path can draw from it without
sharing any of the computation under test.

The shapes are those of public model layer groups (Llama-3.1 8B / 70B decoder layers, a
Qwen3-30B-A3B MoE layer, a Wan2.2 DiT block); the values are normal draws standing in for training
gradients.  No weights or datasets are involved.

bf16 tensors are represented on the host as ``numpy.uint16`` bit patterns (the upper half of an
IEEE binary32), because numpy has no bfloat16 dtype.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

SEED = 20261028


@dataclass(frozen=True)
class GroupConfig:
    """One FSDP parameter group: named shapes, R ranks, C contributors, value scale sigma."""

    name: str
    cfg_id: int
    R: int
    C: int
    sigma: float
    params: tuple = field(default_factory=tuple)  # ((name, shape), ...) in storage order

    @property
    def shapes(self):
        return [tuple(s) for _, s in self.params]

    @property
    def names(self):
        return [n for n, _ in self.params]

    @property
    def P(self):
        return len(self.params)

    def numel(self):
        return sum(int(np.prod(s, dtype=np.int64)) for s in self.shapes)


def _llama(name, cfg_id, hidden, kv, ffn):
    return GroupConfig(
        name=name, cfg_id=cfg_id, R=8, C=8, sigma=1e-3,
        params=(
            ("q", (hidden, hidden)), ("k", (kv, hidden)), ("v", (kv, hidden)),
            ("o", (hidden, hidden)), ("gate", (ffn, hidden)), ("up", (ffn, hidden)),
            ("down", (hidden, ffn)), ("norm1", (hidden,)), ("norm2", (hidden,)),
        ),
    )


def _qwen3_moe():
    ps = [("q", (4096, 2048)), ("k", (512, 2048)), ("v", (512, 2048)), ("o", (2048, 4096)),
          ("router", (128, 2048))]
    for e in range(128):
        ps += [(f"e{e}.gate", (768, 2048)), (f"e{e}.up", (768, 2048)), (f"e{e}.down", (2048, 768))]
    ps += [("norm1", (2048,)), ("norm2", (2048,))]
    return GroupConfig(name="qwen3_30b_a3b", cfg_id=3, R=16, C=8, sigma=1e-3, params=tuple(ps))


def _wan_block():
    ps = []
    for a in ("self", "cross"):
        for n in ("q", "k", "v", "o"):
            ps += [(f"{a}.{n}.w", (5120, 5120)), (f"{a}.{n}.b", (5120,))]
    ps += [("ffn0.w", (13824, 5120)), ("ffn2.w", (5120, 13824))]
    ps += [("norm0", (5120,)), ("norm1", (5120,)), ("norm2", (5120,))]
    return GroupConfig(name="wan2_2_block", cfg_id=4, R=64, C=8, sigma=1e-3, params=tuple(ps))


TINY = GroupConfig(name="tiny", cfg_id=0, R=4, C=4, sigma=1.0,
                   params=(("a", (7, 5)), ("b", (16, 3)), ("c", (1, 9))))
LLAMA8B = _llama("llama3_1_8b_layer", 1, 4096, 1024, 14336)
LLAMA70B = _llama("llama3_1_70b_layer", 2, 8192, 1024, 28672)
QWEN3 = _qwen3_moe()
WAN22 = _wan_block()

CONFIGS = {c.name: c for c in (TINY, LLAMA8B, LLAMA70B, QWEN3, WAN22)}
ORDERED = [TINY, LLAMA8B, LLAMA70B, QWEN3, WAN22]


# ----------------------------------------------------------------------------------------------
# bf16 bit patterns on the host
# ----------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def _stream_key(*parts) -> list:
    return [SEED] + [int(p) for p in parts]


def normal_bf16_bits(shape, sigma: float, *key) -> np.ndarray:
    """Seeded N(0, sigma^2) draws rounded to bf16, as uint16 bits of the given shape.

    The stream is numpy PCG64 keyed by SeedSequence([SEED, *key]); ``key`` is e.g.
    (cfg_id, c, p) for contributor c's gradient of parameter p.
    """
    n = int(np.prod(shape, dtype=np.int64))
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(_stream_key(*key))))
    x = rng.standard_normal(size=n, dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(x).reshape(shape)


def group_grads_np(cfg: GroupConfig, C: int | None = None):
    """grads[c][p] (uint16 bits, shape_p) for every contributor c and parameter p of cfg."""
    C = cfg.C if C is None else C
    return [[normal_bf16_bits(s, cfg.sigma, cfg.cfg_id, c, p) for p, s in enumerate(cfg.shapes)]
            for c in range(C)]


def stage_bits_np(cfg: GroupConfig, numel: int) -> np.ndarray:
    """A seeded bf16 stage buffer of ``numel`` elements (flat uint16 bits)."""
    return normal_bf16_bits((numel,), cfg.sigma, cfg.cfg_id, 1 << 20, 0)


# ----------------------------------------------------------------------------------------------
# Device-side generators (torch), for full-size workloads that are too large to draw on the host.
# ----------------------------------------------------------------------------------------------

def _torch_seed(*key) -> int:
    h = hashlib.sha256(repr(_stream_key(*key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal_bf16_cuda(shape, sigma: float, *key, device="cuda"):
    """Seeded N(0, sigma^2) bf16 tensor drawn on the device with torch's Philox generator.

    Used only where host generation would take minutes; parity checks then read the sampled
    input bytes back from the device, so the generator never affects what is compared.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(*key))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return (x * sigma).to(torch.bfloat16)
