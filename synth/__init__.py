"""Seeded synthetic inputs for the W4A16 MoE expert layer.

This module only draws random inputs. It holds none of the layer's arithmetic
(no dequantisation, alignment, GEMM, activation or combine), and both the CPU
oracle and the GPU path read their inputs from here.

Every tensor comes from its own counter-free stream: numpy's SFC64 bit
generator seeded with ``SeedSequence([seed, stream, index])``. A tensor can
therefore be regenerated on its own, e.g. one expert's weights for a sampled
oracle check, without drawing anything else.

Streams:
  0  W13 packed words  (per expert)      1  W13 scales (per expert)
  2  W2 packed words   (per expert)      3  W2 scales  (per expert)
  10 activations x / a3                  11 softmax routing logits
  12 Zipf popularity permutation         13 Zipf Gumbel noise
  14 masked_m counts

Shapes follow the Chord page's problem statement (BF16 activations, uint4
weights packed eight per int32 word, one BF16 scale per group of 32 along K;
Chord page, "TL;DR" and "vLLM integration") at Kimi-K2.x serving sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    name: str
    layout: str            # "indexed" | "contiguous" | "masked"
    E: int                 # experts
    H: int                 # hidden size (W13 K, W2 N)
    I: int                 # moe intermediate size (W13 N = 2I, W2 K)
    T: int                 # tokens (indexed / contiguous)
    topk: int
    routing: str           # "softmax" | "zipf" | "none"
    wseed: int
    iseed: int
    max_m: int = 0         # masked: per-expert row budget
    expected_m: int = 0    # masked: launch hint
    extra: dict = field(default_factory=dict)

    @property
    def flat_rows(self) -> int:
        return self.T * self.topk


WORKLOADS = {
    0: Workload("tiny-indexed-e8-h256-i512-t32-top2", "indexed",
                E=8, H=256, I=512, T=32, topk=2, routing="softmax",
                wseed=100, iseed=200),
    1: Workload("kimi-decode-indexed-e384-h7168-i2048-t448-top8", "indexed",
                E=384, H=7168, I=2048, T=448, topk=8, routing="softmax",
                wseed=101, iseed=201),
    2: Workload("kimi-prefill-contiguous-e384-h7168-i2048-t8192-top8-zipf1.1",
                "contiguous", E=384, H=7168, I=2048, T=8192, topk=8,
                routing="zipf", wseed=101, iseed=202, extra={"zipf_s": 1.1}),
    3: Workload("kimi-masked-e384-h7168-i2048-maxm64-expm16", "masked",
                E=384, H=7168, I=2048, T=0, topk=0, routing="none",
                wseed=101, iseed=203, max_m=64, expected_m=16),
    4: Workload("kimi-tp8-shard-indexed-e384-h7168-i256-t4096-top8", "indexed",
                E=384, H=7168, I=256, T=4096, topk=8, routing="softmax",
                wseed=104, iseed=204),
    # one GPU's EP8 share (experts 0..47 of the 384, the decode workload's
    # weights and routing); the routing draws global ids
    5: Workload("kimi-ep8-share-decode-indexed-e48of384-h7168-i2048-t448-top8", "indexed",
                E=48, H=7168, I=2048, T=448, topk=8, routing="softmax",
                wseed=101, iseed=201, extra={"global_experts": 384}),
    # one GPU's EP8 share at prefill: its 48 experts' rows after the dispatch,
    # grouped and aligned, 512 rows per expert
    6: Workload("kimi-ep8-share-prefill-contiguous-e48-h7168-i2048-512rows-per-expert", "contiguous",
                E=48, H=7168, I=2048, T=0, topk=0, routing="none",
                wseed=101, iseed=206, extra={"rows_per_expert": 512}),
    # batch-1 decode: 8 experts touched, the latency case
    7: Workload("kimi-decode-indexed-e384-h7168-i2048-t1-top8", "indexed",
                E=384, H=7168, I=2048, T=1, topk=8, routing="softmax",
                wseed=101, iseed=207),
}


def scaled(w: Workload, **kw) -> Workload:
    """The same workload recipe at other sizes (for CPU-sized test cases)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


# --------------------------------------------------------------------------
# Random streams
# --------------------------------------------------------------------------


def rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence([seed, stream, index])))


def _to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round float32 draws to BF16 storage (uint16 bit patterns).

    The conversion is torch's own float32 -> bfloat16 cast; it only shapes
    random draws into the input dtype.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _scales(seed: int, stream: int, e: int, rows: int, groups: int) -> np.ndarray:
    z = rng(seed, stream, e).standard_normal((rows, groups), dtype=np.float32)
    return _to_bf16_bits(np.abs(z) * np.float32(0.02) + np.float32(1e-3))


def _words(seed: int, stream: int, e: int, rows: int, words: int) -> np.ndarray:
    # Uniform 32-bit words are exactly eight iid uniform nibbles 0..15.
    return rng(seed, stream, e).integers(0, 2**32, size=(rows, words), dtype=np.uint32).view(np.int32)


def expert_weights(wseed: int, H: int, I: int, e: int):
    """One expert's canonical weights.

    Returns (w13_q int32[2I, H/8], w13_s uint16[2I, H/32],
             w2_q int32[H, I/8],   w2_s uint16[H, I/32]).
    W13 rows [0, I) are the gate projection and rows [I, 2I) the up
    projection.
    """
    return (_words(wseed, 0, e, 2 * I, H // 8), _scales(wseed, 1, e, 2 * I, H // 32),
            _words(wseed, 2, e, H, I // 8), _scales(wseed, 3, e, H, I // 32))


def stacked_weights(w: Workload, out=None, experts=None):
    """All experts' canonical weights stacked along a leading E axis.

    ``out`` may hold four preallocated arrays (e.g. numpy views of pinned host
    tensors) of shapes [E,2I,H/8], [E,2I,H/32], [E,H,I/8], [E,H,I/32].
    """
    E, H, I = w.E, w.H, w.I
    if out is None:
        out = (np.empty((E, 2 * I, H // 8), np.int32), np.empty((E, 2 * I, H // 32), np.uint16),
               np.empty((E, H, I // 8), np.int32), np.empty((E, H, I // 32), np.uint16))
    for e in (range(E) if experts is None else experts):
        for dst, src in zip(out, expert_weights(w.wseed, H, I, e)):
            dst[e] = src
    return out


def activations(seed: int, rows: int, H: int) -> np.ndarray:
    """BF16 N(0,1) activations, uint16 bits [rows, H]."""
    return _to_bf16_bits(rng(seed, 10).standard_normal((rows, H), dtype=np.float32))


def _topk_desc(key: np.ndarray, k: int) -> np.ndarray:
    # Descending key; equal keys go to the lower expert index (stable sort of -key).
    return np.argsort(-key, axis=1, kind="stable")[:, :k].astype(np.int32)


def softmax_routing(seed: int, T: int, E: int, topk: int):
    """Top-k of a softmax over N(0,1) logits.

    Returns ids int32[T, topk] (distinct per token) and weights float32
    [T, topk], the chosen softmax probabilities without renormalisation.
    """
    logits = rng(seed, 11).standard_normal((T, E), dtype=np.float32).astype(np.float64)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ids = _topk_desc(p, topk)
    return ids, np.take_along_axis(p, ids, axis=1).astype(np.float32)


def zipf_routing(seed: int, T: int, E: int, topk: int, s: float = 1.1):
    """Top-k routing with Zipf(s)-skewed expert popularity.

    Expert popularity is proportional to (1+rank)^-s for a random rank
    permutation; per token, k distinct experts are drawn without replacement
    with those probabilities (Gumbel top-k). Weights are the softmax of the
    perturbed keys over all experts at the chosen ids.
    """
    perm = rng(seed, 12).permutation(E)
    logpop = -s * np.log1p(perm.astype(np.float64))
    key = logpop[None, :] + rng(seed, 13).gumbel(size=(T, E))
    ids = _topk_desc(key, topk)
    p = np.exp(key - key.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return ids, np.take_along_axis(p, ids, axis=1).astype(np.float32)


def routing(w: Workload):
    """Token routing of a workload: ids over its experts, or over the global
    pool of an expert-parallel share (extra["global_experts"])."""
    E = w.extra.get("global_experts", w.E)
    if w.routing == "softmax":
        return softmax_routing(w.iseed, w.T, E, w.topk)
    if w.routing == "zipf":
        return zipf_routing(w.iseed, w.T, E, w.topk, w.extra.get("zipf_s", 1.1))
    raise ValueError(f"workload {w.name} has no token routing")


def masked_inputs(w: Workload):
    """Masked-layout inputs: a3 bf16 bits [E, max_m, H] and masked_m int32[E]
    drawn uniformly from 0..max_m inclusive."""
    masked_m = rng(w.iseed, 14).integers(0, w.max_m + 1, size=w.E).astype(np.int32)
    a3 = activations(w.iseed, w.E * w.max_m, w.H).reshape(w.E, w.max_m, w.H)
    return a3, masked_m


def bf16_nan_bits() -> int:
    return 0x7FC0


__all__ = ["Workload", "WORKLOADS", "scaled", "rng", "expert_weights", "stacked_weights",
           "activations", "softmax_routing", "zipf_routing", "routing", "masked_inputs",
           "bf16_nan_bits"]
