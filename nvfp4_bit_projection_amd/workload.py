"""Device-resident synthetic workloads: seeded fp32 weights drawn on the GPU by
the shared generator (``synth``), packed to NVFP4 by this library's own
quantiser kernel.  Used by the tests and the benchmark; the decode path itself
never generates anything.
"""
from __future__ import annotations

import torch

import synth

from . import flint
from .flint import AttnWeights, LayerWeights, NVFP4Tensor


def _fill(seed: int, kind: int, expert0: int, n_streams: int, n: int, out: torch.Tensor, std: float) -> torch.Tensor:
    synth.normal_device(seed, synth.stream_id(kind, expert0), n, out, std=std, n_streams=n_streams)
    return out


def _pack(w: torch.Tensor, n_mats: int, rows: int, cols: int, ws: torch.Tensor):
    codes = torch.empty((n_mats, rows, cols // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n_mats, rows, cols // 16), dtype=torch.uint8, device=w.device)
    ts = torch.empty(n_mats, dtype=torch.float32, device=w.device)
    flint.quantize_into(w.view(n_mats, rows, cols), codes, scales, ts, ws)
    return codes, scales, ts


def build_layer(dims: synth.MoEDims, seed: int, device="cuda", tmp: torch.Tensor | None = None) -> LayerWeights:
    """One MoE layer drawn with weight seed `seed` (streams as in ``synth``)."""
    H, E, I, Is = dims.hidden, dims.n_experts, dims.expert_width, dims.shared_width
    need = max(E * I * H, Is * H)
    if tmp is None or tmp.numel() < need:
        tmp = torch.empty(need, dtype=torch.float32, device=device)
    ws = flint.workspace(flint.OP_QUANTIZE, None, B=max(E, 1), device=device)
    std = synth.WEIGHT_STD
    router = torch.empty((E, H), dtype=torch.float32, device=device)
    _fill(seed, synth.ROUTER, 0, 1, E * H, router, std)
    mats = {}
    for kind, rows, cols in ((synth.GATE, I, H), (synth.UP, I, H), (synth.DOWN, H, I)):
        t = tmp[:E * rows * cols]
        _fill(seed, kind, 0, E, rows * cols, t, std)
        mats[kind] = _pack(t, E, rows, cols, ws)
    shared = {}
    for kind, rows, cols in ((synth.SHARED_GATE, Is, H), (synth.SHARED_UP, Is, H), (synth.SHARED_DOWN, H, Is)):
        t = tmp[:rows * cols]
        _fill(seed, kind, 0, 1, rows * cols, t, std)
        c, s, ts = _pack(t, 1, rows, cols, ws)
        shared[kind] = NVFP4Tensor(c[0], s[0], ts)
    tscales = torch.stack([mats[synth.GATE][2], mats[synth.UP][2], mats[synth.DOWN][2]], dim=1).contiguous()
    return LayerWeights(router, mats[synth.GATE][0], mats[synth.GATE][1], mats[synth.UP][0], mats[synth.UP][1],
                        mats[synth.DOWN][0], mats[synth.DOWN][1], tscales, shared[synth.SHARED_GATE],
                        shared[synth.SHARED_UP], shared[synth.SHARED_DOWN])


def build_head(vocab: int, hidden: int, seed: int = synth.HEAD_SEED, device="cuda",
               tmp: torch.Tensor | None = None) -> NVFP4Tensor:
    n = vocab * hidden
    if tmp is None or tmp.numel() < n:
        tmp = torch.empty(n, dtype=torch.float32, device=device)
    t = tmp[:n]
    _fill(seed, synth.HEAD, 0, 1, n, t, synth.WEIGHT_STD)
    ws = flint.workspace(flint.OP_QUANTIZE, None, B=1, device=device)
    c, s, ts = _pack(t, 1, vocab, hidden, ws)
    return NVFP4Tensor(c[0], s[0], ts)


def _matrix(seed: int, kind: int, rows: int, cols: int, device, ws: torch.Tensor) -> NVFP4Tensor:
    t = torch.empty(rows * cols, dtype=torch.float32, device=device)
    _fill(seed, kind, 0, 1, rows * cols, t, synth.WEIGHT_STD)
    c, s, ts = _pack(t, 1, rows, cols, ws)
    return NVFP4Tensor(c[0], s[0], ts)


def build_attn(d: synth.AttnDims, seed: int, device="cuda") -> AttnWeights:
    """One attention layer drawn with weight seed `seed` (streams as in ``synth``)."""
    nq, nk, H = d.n_q * d.head_dim, d.n_kv * d.head_dim, d.hidden
    ws = flint.workspace(flint.OP_QUANTIZE, None, B=1, device=device)
    q = _matrix(seed, synth.ATTN_Q, nq, H, device, ws)
    k = _matrix(seed, synth.ATTN_K, nk, H, device, ws)
    v = _matrix(seed, synth.ATTN_V, nk, H, device, ws)
    o = _matrix(seed, synth.ATTN_O, H, nq, device, ws)
    vec = lambda kind, n, mean, std: synth.normal_device(seed, synth.stream_id(kind), n, torch.empty(
        n, dtype=torch.float32, device=device), mean=mean, std=std)
    return AttnWeights(q, k, v, o, vec(synth.Q_NORM, d.head_dim, 1.0, 0.1), vec(synth.K_NORM, d.head_dim, 1.0, 0.1),
                       vec(synth.SINK, d.n_q, 0.0, 1.0))


def kv_cache(d: synth.AttnDims, seed: int, cap: int, kind: int, device="cuda") -> torch.Tensor:
    """A filled BF16 cache [Hkv][cap][D] (int16 bit patterns), as ``synth.kv_cache_bits``."""
    n = d.n_kv * cap * d.head_dim
    t = synth.normal_device(seed, synth.stream_id(kind), n, torch.empty(n, dtype=torch.float32, device=device))
    return t.to(torch.bfloat16).view(torch.int16).view(d.n_kv, cap, d.head_dim)


def build_dense(seed: int, hidden: int, width: int, device="cuda") -> tuple[NVFP4Tensor, NVFP4Tensor, NVFP4Tensor]:
    ws = flint.workspace(flint.OP_QUANTIZE, None, B=1, device=device)
    return (_matrix(seed, synth.DENSE_GATE, width, hidden, device, ws),
            _matrix(seed, synth.DENSE_UP, width, hidden, device, ws),
            _matrix(seed, synth.DENSE_DOWN, hidden, width, device, ws))


def tokens(seeds, hidden: int, device="cuda") -> torch.Tensor:
    """float32 [len(seeds)][hidden], row t = N(0,1) token of seed seeds[t]."""
    seeds = list(seeds)
    x = torch.empty((len(seeds), hidden), dtype=torch.float32, device=device)
    for t, s in enumerate(seeds):
        synth.normal_device(s, synth.stream_id(synth.TOKEN), hidden, x[t], std=1.0)
    return x
