"""Seeded synthetic workloads for the block-FP8 routed MoE layer.

This module only *produces inputs*: layer shapes, activations, router weights,
router bias and block-FP8 expert banks. It holds none of the layer's own
arithmetic (no E4M3 decoding, no routing, no expert math), so the CPU oracle
and the HIP path can both be fed from it without sharing any computation.

Shapes follow the two model families the colizig page runs ("What this project
is trying to prove", model table): 128 experts with top-8 and no shared expert,
and 512 experts with top-10 plus one always-on shared expert. The pages fix no
hidden/intermediate sizes, block size or value distributions; the recipe here
(activations N(0,1), router N(0, sigma_r), expert weights N(0, 0.02) quantised
per square block to E4M3FN with scale = block amax / 448) is this project's
reading and is the same for every consumer.

Random streams are numpy PCG64 keyed by (ROOT_SEED, config, tensor, index), so
one expert of a bank can be regenerated without generating the others.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
import torch

ROOT_SEED = 20261202

# tensor tags of the seed sequence
_TAG_X = 1
_TAG_ROUTER = 2
_TAG_BIAS = 3
_TAG_GATE_UP = 4
_TAG_DOWN = 5
_TAG_SHARED_GATE_UP = 6
_TAG_SHARED_DOWN = 7

E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Shape and input recipe of one MoE layer workload."""

    name: str
    tokens: int
    hidden: int
    experts: int
    inter: int
    top_k: int
    block: int
    shared: bool
    x_dtype: str  # "f32" or "bf16"
    router_std: float
    bias: Optional[tuple] = None  # ("zipf", s, alpha) | ("plateau_zipf", n_hot, hot_bias, s)
    weight_std: float = 0.02
    seed_id: int = 0  # config index in the seed sequence

    def with_(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.tokens * self.top_k + (self.tokens if self.shared else 0)

    def expert_bytes(self) -> int:
        """Bytes of one expert: E4M3 weights plus fp32 block scales."""
        w = 3 * self.hidden * self.inter
        s = 4 * (2 * self.inter // self.block * (self.hidden // self.block)
                 + self.hidden // self.block * (self.inter // self.block))
        return w + s


# The five workloads. c1 is quoted at batches 1/4/16: the first T rows of one
# 16-token draw (gen_x(shape, tokens=T) returns exactly those rows).
CONFIGS = {
    "c0": LayerShape("tiny", tokens=4, hidden=64, experts=8, inter=32, top_k=2, block=32,
                     shared=False, x_dtype="f32", router_std=0.1, seed_id=0),
    "c1": LayerShape("qwen3moe_decode", tokens=16, hidden=2048, experts=128, inter=768,
                     top_k=8, block=128, shared=False, x_dtype="bf16", router_std=0.02,
                     seed_id=1),
    "c2": LayerShape("qwen3moe_prefill512", tokens=512, hidden=2048, experts=128, inter=768,
                     top_k=8, block=128, shared=False, x_dtype="bf16", router_std=0.02,
                     bias=("zipf", 1.1, 0.25), seed_id=2),
    "c3": LayerShape("e512_decode", tokens=8, hidden=4096, experts=512, inter=1024,
                     top_k=10, block=128, shared=True, x_dtype="bf16", router_std=0.02,
                     seed_id=3),
    "c4": LayerShape("e512_prefill4096", tokens=4096, hidden=4096, experts=512, inter=1024,
                     top_k=10, block=128, shared=True, x_dtype="bf16", router_std=0.02,
                     bias=("plateau_zipf", 16, 1.0, 1.3), seed_id=4),
}


def _rng(shape: LayerShape, tag: int, index: int = 0, salt: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, shape.seed_id, tag, index, salt])
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even), returned as fp32."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def gen_x(shape: LayerShape, tokens: Optional[int] = None, batch: int = 0) -> np.ndarray:
    """Activations x [T][H] ~ N(0, 1) as fp32 values; for bf16 layers the values
    are already rounded to bf16, so the array is exactly what the device gets.
    Different `batch` values give independent draws (rotated inputs)."""
    T = shape.tokens if tokens is None else tokens
    g = _rng(shape, _TAG_X, batch)
    x = g.standard_normal((T, shape.hidden), dtype=np.float32)
    if shape.x_dtype == "bf16":
        x = round_to_bf16(x)
    return x


def gen_router(shape: LayerShape) -> np.ndarray:
    """Router weight Wr [E][H] fp32 ~ N(0, router_std)."""
    g = _rng(shape, _TAG_ROUTER)
    w = g.standard_normal((shape.experts, shape.hidden), dtype=np.float32)
    return (w * np.float32(shape.router_std)).astype(np.float32)


def gen_bias(shape: LayerShape) -> Optional[np.ndarray]:
    """Router bias [E] fp32 giving Zipf-like expert popularity, or None.

    ("zipf", s, alpha):            b_e = -alpha * s * ln(rank_e)
    ("plateau_zipf", n, h, s):     b_e = h for rank_e <= n, else -s * ln(rank_e / n)
    rank_e is a seeded permutation of 1..E (so popularity is not tied to index).
    """
    if shape.bias is None:
        return None
    g = _rng(shape, _TAG_BIAS)
    rank = g.permutation(shape.experts).astype(np.float64) + 1.0
    kind = shape.bias[0]
    if kind == "zipf":
        _, s, alpha = shape.bias
        b = -alpha * s * np.log(rank)
    elif kind == "plateau_zipf":
        _, n_hot, hot_bias, s = shape.bias
        b = np.where(rank <= n_hot, hot_bias, -s * np.log(rank / n_hot))
    else:
        raise ValueError(f"unknown bias recipe {kind!r}")
    return b.astype(np.float32)


def quantise_blocks(w: np.ndarray, block: int):
    """Quantise an fp32 matrix [R][C] to E4M3FN bytes with one fp32 scale per
    block x block tile: scale = amax / 448 (1 for an all-zero tile), code =
    round-to-nearest-even of w / scale after clamping to +-448.
    Returns (codes uint8 [R][C], scales fp32 [R/B][C/B])."""
    R, C = w.shape
    assert R % block == 0 and C % block == 0
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32))
    tiles = t.view(R // block, block, C // block, block)
    amax = tiles.abs().amax(dim=(1, 3))
    scale = amax / E4M3_MAX
    scale = torch.where(amax > 0, scale, torch.ones_like(scale)).to(torch.float32)
    v = (tiles / scale[:, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    q = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return q.numpy(), scale.numpy()


def gen_expert(shape: LayerShape, e: int, shared: bool = False):
    """One expert's block-FP8 weights, regenerated from its own seed stream.
    Returns dict(w_gate_up uint8 [2I][H], s_gate_up f32 [2I/B][H/B],
                 w_down uint8 [H][I], s_down f32 [H/B][I/B])."""
    H, I, B = shape.hidden, shape.inter, shape.block
    tg, td = (_TAG_SHARED_GATE_UP, _TAG_SHARED_DOWN) if shared else (_TAG_GATE_UP, _TAG_DOWN)
    std = np.float32(shape.weight_std)
    wgu = _rng(shape, tg, e).standard_normal((2 * I, H), dtype=np.float32)
    wgu *= std
    wd = _rng(shape, td, e).standard_normal((H, I), dtype=np.float32)
    wd *= std
    qgu, sgu = quantise_blocks(wgu, B)
    qd, sd = quantise_blocks(wd, B)
    return {"w_gate_up": qgu, "s_gate_up": sgu, "w_down": qd, "s_down": sd}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gen_bank(shape: LayerShape, shared: bool = False, threads: Optional[int] = None):
    """A whole bank (E routed experts, or the 1 shared expert) as contiguous
    expert-major arrays, generated expert by expert on a thread pool."""
    n = 1 if shared else shape.experts
    H, I, B = shape.hidden, shape.inter, shape.block
    bank = {
        "w_gate_up": np.empty((n, 2 * I, H), np.uint8),
        "s_gate_up": np.empty((n, 2 * I // B, H // B), np.float32),
        "w_down": np.empty((n, H, I), np.uint8),
        "s_down": np.empty((n, H // B, I // B), np.float32),
    }

    def one(e):
        d = gen_expert(shape, e, shared)
        for k, v in d.items():
            bank[k][e] = v

    nt = threads or _threads()
    if nt == 1 or n == 1:
        for e in range(n):
            one(e)
    else:
        prev = torch.get_num_threads()
        torch.set_num_threads(1)
        try:
            with ThreadPoolExecutor(nt) as ex:
                list(ex.map(one, range(n)))
        finally:
            torch.set_num_threads(prev)
    return bank


def bank_expert(bank: dict, e: int) -> dict:
    """View of expert e of a bank produced by gen_bank."""
    return {k: v[e] for k, v in bank.items()}


def gen_layer(shape: LayerShape, tokens: Optional[int] = None, batch: int = 0,
              with_bank: bool = True):
    """Everything one layer call needs, as host numpy arrays."""
    d = {
        "x": gen_x(shape, tokens, batch),
        "router_w": gen_router(shape),
        "router_bias": gen_bias(shape),
    }
    if with_bank:
        d["bank"] = gen_bank(shape)
        d["shared"] = gen_bank(shape, shared=True) if shape.shared else None
    return d
