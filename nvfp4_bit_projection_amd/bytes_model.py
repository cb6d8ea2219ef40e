"""Algorithmic bytes and multiply-adds of the decode step (the roofline numerator).

Counts only what the method must move from HBM: NVFP4 codes (half a byte per
weight) and E4M3 block scales (one byte per 16 weights) of every matrix a
token touches, plus the unquantised fp32 router.  Per-tensor fp32 scales (a
few bytes per layer) and activations (a few KB per layer) are left out.

Page pins [P3] "Flint: 125 tokens a second is what 2.5B active parameters buy
at 273 GB/s": routed experts read per token 887M parameters and the output
head 307.5M ("The shape, read from the headers", parameter table); at 4.5 bits
per weight they are 499 MB and 173 MB per token, and a 4-bit head row of 2,048
values is 1,024 bytes of codes ("Why active parameters set the speed", byte
table); NVFP4 is 4-bit values plus an 8-bit scale per 16 ("Checking 125 tokens
a second").
"""
from __future__ import annotations

from dataclasses import dataclass


def nvfp4_bytes(rows: int, cols: int) -> int:
    assert cols % 16 == 0
    return rows * cols // 2 + rows * cols // 16


@dataclass(frozen=True)
class LayerShape:
    hidden: int = 2048
    n_experts: int = 256
    expert_width: int = 512
    top_k: int = 6
    shared_width: int = 1024


def expert_bytes(s: LayerShape) -> int:
    """gate [I][H] + up [I][H] + down [H][I]"""
    return 2 * nvfp4_bytes(s.expert_width, s.hidden) + nvfp4_bytes(s.hidden, s.expert_width)


def shared_bytes(s: LayerShape) -> int:
    return 2 * nvfp4_bytes(s.shared_width, s.hidden) + nvfp4_bytes(s.hidden, s.shared_width)


def router_bytes(s: LayerShape) -> int:
    return 4 * s.n_experts * s.hidden


def layer_bytes(s: LayerShape, distinct_experts: float | None = None) -> float:
    """Bytes one MoE layer reads for one decode step: the router, the shared
    expert and `distinct_experts` routed experts (top_k at batch 1)."""
    n = s.top_k if distinct_experts is None else distinct_experts
    return router_bytes(s) + shared_bytes(s) + n * expert_bytes(s)


def head_bytes(vocab: int, hidden: int) -> int:
    return nvfp4_bytes(vocab, hidden)


def token_bytes(s: LayerShape, layers: int, vocab: int) -> int:
    """Batch-1 bytes per token: `layers` MoE layers plus the head."""
    return int(layers * layer_bytes(s)) + head_bytes(vocab, s.hidden)


def layer_macs(s: LayerShape, tokens: int = 1) -> int:
    per = s.n_experts * s.hidden + s.top_k * 3 * s.expert_width * s.hidden + 3 * s.shared_width * s.hidden
    return tokens * per


def head_macs(vocab: int, hidden: int, tokens: int = 1) -> int:
    return tokens * vocab * hidden


def expected_distinct_experts(n_experts: int, top_k: int, batch: int) -> float:
    """E[#distinct experts] when `batch` tokens each pick top_k of n_experts
    uniformly without replacement."""
    return n_experts * (1.0 - (1.0 - top_k / n_experts) ** batch)
