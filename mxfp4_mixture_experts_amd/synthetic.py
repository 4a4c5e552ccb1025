"""Seeded synthetic inputs for the MXFP4 mixture-of-experts expert projection.

This module only draws random numbers and packs them into the storage formats
the projection reads (u8 MXFP4 blocks and E8M0 scale bytes, bf16 bit patterns,
i32 expert ids).  It holds none of the projection's arithmetic: no decoding,
no routing, no products.  Both the GPU path and the CPU oracle are fed from the
arrays it returns.

Tensor shapes follow the gpt-oss-20b files page, README section "MXFP4" (the
checkpoint tensor table): gate_up blocks [32, 5760, 90, 16] u8 with scales
[32, 5760, 90] u8, down blocks [32, 2880, 90, 16] u8 with scales
[32, 2880, 90] u8; biases are bf16 [Experts, Rows] (src/experts.linnet,
block MixtureOfExperts parameters).

Seeding: one independent numpy stream per tensor,
``SeedSequence(seed, spawn_key=(config_index, tensor_id))``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor ids for the per-tensor streams
_T_BLOCKS, _T_SCALES, _T_BIAS, _T_X, _T_LOGITS, _T_IDS, _T_ROUTER_W, _T_ROUTER_B = range(8)


def _rng(seed: int, cfg: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(cfg, tensor)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the u16 bit patterns.

    Inputs must be finite (the generators never draw NaN or inf).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


@dataclass
class MoEProblem:
    """One expert-projection workload, as host arrays.

    blocks  u8  [E, N, K/32, 16]  two E2M1 codes per byte, low nibble = even element
    scales  u8  [E, N, K/32]      E8M0 exponent bytes (bias 127)
    bias    u16 [E, N]            bf16 bit patterns
    x       u16 [T, K] (shared by a token's k slots) or [T, k, K] (one input per slot)
    logits  u16 [T, E] bf16 router logits, or None
    ids_in  i32 [T, k] given expert ids (distinct per token), or None (route from logits)
    """
    name: str
    E: int
    N: int
    K: int
    T: int
    k: int
    blocks: np.ndarray
    scales: np.ndarray
    bias: np.ndarray
    x: np.ndarray
    x_per_slot: bool
    logits: Optional[np.ndarray]
    ids_in: Optional[np.ndarray]
    combine: bool
    meta: dict = field(default_factory=dict)


def _weights(seed, cfg, E, N, K, scale_lo, scale_hi):
    KB = K // 32
    blocks = _rng(seed, cfg, _T_BLOCKS).integers(0, 256, size=(E, N, KB, 16), dtype=np.uint8)
    scales = _rng(seed, cfg, _T_SCALES).integers(scale_lo, scale_hi + 1, size=(E, N, KB), dtype=np.uint8)
    bias = f32_to_bf16_bits(_rng(seed, cfg, _T_BIAS).normal(0.0, 0.02, size=(E, N)).astype(np.float32))
    return blocks, scales, bias


def _normal_bf16(seed, cfg, tensor, shape):
    return f32_to_bf16_bits(_rng(seed, cfg, tensor).standard_normal(size=shape, dtype=np.float32))


def _distinct_uniform_ids(rng, T, E, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def zipf_probabilities(E: int, s: float) -> np.ndarray:
    """p(expert i) proportional to (i + 1) ** -s, i = 0..E-1 (expert 0 is rank 1)."""
    w = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    return w / w.sum()


def _zipf_ids(rng, T, E, k, s):
    p = zipf_probabilities(E, s)
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


CONFIG_NAMES = (
    "tiny",               # E=4 N=256 K=128 T=8 top-2 given ids
    "gate_up_decode_t1",  # gpt-oss-20b gate_up, one token, routed from logits
    "down_decode_t64",    # gpt-oss-20b down, 64 tokens, per-slot inputs, + combine
    "gate_up_prefill_t4096",
    "down_prefill_zipf_t2048",
)


def make_config(index: int, seed: int = 0) -> MoEProblem:
    """The five workloads: 0 tiny, 1 gate_up decode T=1, 2 down decode T=64,
    3 gate_up prefill T=4096, 4 down prefill T=2048 with Zipf(1.2) expert choice."""
    cfg = index
    if index == 0:
        E, N, K, T, k = 4, 256, 128, 8, 2
        blocks, scales, bias = _weights(seed, cfg, E, N, K, 120, 132)
        x = _normal_bf16(seed, cfg, _T_X, (T, K))
        ids = _distinct_uniform_ids(_rng(seed, cfg, _T_IDS), T, E, k)
        return MoEProblem(CONFIG_NAMES[0], E, N, K, T, k, blocks, scales, bias, x, False, None, ids, False)
    if index in (1, 3):
        E, N, K, k = 32, 5760, 2880, 4
        T = 1 if index == 1 else 4096
        blocks, scales, bias = _weights(seed, cfg, E, N, K, 118, 130)
        x = _normal_bf16(seed, cfg, _T_X, (T, K))
        logits = _normal_bf16(seed, cfg, _T_LOGITS, (T, E))
        return MoEProblem(CONFIG_NAMES[index], E, N, K, T, k, blocks, scales, bias, x, False, logits, None, False)
    if index in (2, 4):
        E, N, K, k = 32, 2880, 2880, 4
        T = 64 if index == 2 else 2048
        blocks, scales, bias = _weights(seed, cfg, E, N, K, 118, 130)
        x = _normal_bf16(seed, cfg, _T_X, (T, k, K))
        logits = _normal_bf16(seed, cfg, _T_LOGITS, (T, E))
        ids = None
        meta = {}
        if index == 4:
            ids = _zipf_ids(_rng(seed, cfg, _T_IDS), T, E, k, 1.2)
            meta["zipf_s"] = 1.2
        return MoEProblem(CONFIG_NAMES[index], E, N, K, T, k, blocks, scales, bias, x, True, logits, ids, True, meta)
    raise ValueError(f"config index {index} not in 0..4")


def make_custom(E, N, K, T, k, *, x_per_slot=False, route="logits", seed=0, tag=99,
                scale_lo=118, scale_hi=130, combine=None) -> MoEProblem:
    """A workload of arbitrary shape with the same value distributions.

    route: "logits" (top-k of bf16 N(0,1) logits), "ids" (uniform distinct ids,
    no logits), "ids+logits" (uniform distinct ids and logits for the gates),
    "zipf+logits" (Zipf(1.2) ids and logits for the gates).
    """
    assert K % 32 == 0
    blocks, scales, bias = _weights(seed, tag, E, N, K, scale_lo, scale_hi)
    x = _normal_bf16(seed, tag, _T_X, (T, k, K) if x_per_slot else (T, K))
    logits = _normal_bf16(seed, tag, _T_LOGITS, (T, E)) if "logits" in route else None
    ids = None
    if route.startswith("ids"):
        ids = _distinct_uniform_ids(_rng(seed, tag, _T_IDS), T, E, k) if T > 0 else np.zeros((0, k), np.int32)
    elif route.startswith("zipf"):
        ids = _zipf_ids(_rng(seed, tag, _T_IDS), T, E, k, 1.2) if T > 0 else np.zeros((0, k), np.int32)
    if combine is None:
        combine = logits is not None
    return MoEProblem(f"custom_E{E}_N{N}_K{K}_T{T}_k{k}", E, N, K, T, k, blocks, scales, bias, x,
                      x_per_slot, logits, ids, combine)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns as float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def scale_channels(x_bits: np.ndarray, channels, factor: float) -> np.ndarray:
    """Activations with outlier channels: the given input channels (last axis) of
    every row multiplied by `factor`, rounded back to bf16.  Hidden states of
    trained transformers carry a few such channels, often 100-1000x the rest."""
    f = bf16_bits_to_f32(x_bits).copy()
    f[..., list(channels)] *= np.float32(factor)
    return f32_to_bf16_bits(f)


def lognormal_bf16(shape, sigma: float, *, seed: int = 0, tag: int = 97) -> np.ndarray:
    """Heavy-tailed activations: random sign times exp(sigma * N(0, 1)), as bf16."""
    rng = _rng(seed, tag, _T_X)
    mag = np.exp(sigma * rng.standard_normal(size=shape))
    sign = np.where(rng.integers(0, 2, size=shape) == 0, -1.0, 1.0)
    return f32_to_bf16_bits((sign * mag).astype(np.float32))


@dataclass
class RouterProblem:
    """Router inputs (src/experts.linnet block MixtureOfExperts, sub router: a
    Linear from the hidden width H to the E experts).

    x     u16 [T, H]  bf16 token rows
    w     u16 [E, H]  bf16 weights, row e = expert e
    bias  u16 [E]     bf16
    """
    T: int
    H: int
    E: int
    x: np.ndarray
    w: np.ndarray
    bias: np.ndarray


def make_router(T: int, H: int, E: int, *, seed: int = 0, tag: int = 98) -> RouterProblem:
    """x ~ N(0, 1); w ~ N(0, 1 / H) per entry, so that the logits spread about
    like the N(0, 1) logits of the routing workloads; bias ~ N(0, 0.02)."""
    x = _normal_bf16(seed, tag, _T_X, (T, H))
    w = f32_to_bf16_bits(_rng(seed, tag, _T_ROUTER_W).normal(0.0, 1.0 / np.sqrt(H), size=(E, H)).astype(np.float32))
    b = f32_to_bf16_bits(_rng(seed, tag, _T_ROUTER_B).normal(0.0, 0.02, size=(E,)).astype(np.float32))
    return RouterProblem(T, H, E, x, w, b)
