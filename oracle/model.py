"""Oracle composition of the decode step: one MoE layer, the layer stack, the head.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Every step calls the
double-precision routines of ``oracle.c``; the only arithmetic written here is
the weighted sum of expert outputs, the residual add and the norm scaling, in
float64 numpy, in the order the definitions state.

Sources: [P2] "Recursive Releases Flint, a 40B MoE Coding Model That Runs
Locally at 125 Tokens per Second", "How does Flint's architecture work?" (a
router selects 6 experts per token plus one always-active shared expert;
47 MoE layers); [P3] "Flint: 125 tokens a second is what 2.5B active
parameters buy at 273 GB/s", "The shape, read from the headers" (hidden
2,048, 256 experts of width 512, shared expert of width 1,024, vocabulary
150,144, norms in the body) and "Why active parameters set the speed" (4-bit
output head).  Readings: the shared expert is added with weight 1; the stack
is pre-norm residual (RMSNorm with unit gain and eps inside the root before
every MoE layer, and once more before the head).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import synth

from . import NVFP4, argmax, f32_gemv, nvfp4_gemv, quantize, rms_inv, swiglu_expert, topk_softmax


@dataclass
class LayerResult:
    y: np.ndarray          # float64[H]  MoE output (no residual)
    idx: np.ndarray        # int32[k]    ordered by (logit desc, index asc)
    w: np.ndarray          # float64[k]  renormalised routing weights
    logits: np.ndarray     # float64[E]
    gap: float             # k-th minus (k+1)-th logit


class SyntheticWeights:
    """Quantises, on first use, exactly the tensors a computation touches.

    The fp32 tensors come from ``synth`` (the shared input generator); the
    NVFP4 encoding is the oracle's own ``quantize``.
    """

    def __init__(self, dims: synth.MoEDims, vocab: int = 150144, head_seed: int = synth.HEAD_SEED):
        self.dims = dims
        self.vocab = vocab
        self.head_seed = head_seed
        self._router: dict[int, np.ndarray] = {}
        self._experts: dict[tuple[int, int], tuple[NVFP4, NVFP4, NVFP4]] = {}
        self._shared: dict[int, tuple[NVFP4, NVFP4, NVFP4]] = {}
        self._head: NVFP4 | None = None

    def router(self, seed: int) -> np.ndarray:
        if seed not in self._router:
            self._router[seed] = synth.router_f32(seed, self.dims)
        return self._router[seed]

    def expert(self, seed: int, e: int) -> tuple[NVFP4, NVFP4, NVFP4]:
        key = (seed, e)
        if key not in self._experts:
            d = self.dims
            self._experts[key] = tuple(quantize(synth.expert_f32(seed, d, kind, e))
                                       for kind in (synth.GATE, synth.UP, synth.DOWN))
        return self._experts[key]

    def shared(self, seed: int) -> tuple[NVFP4, NVFP4, NVFP4]:
        if seed not in self._shared:
            d = self.dims
            self._shared[seed] = tuple(quantize(synth.shared_f32(seed, d, kind))
                                       for kind in (synth.SHARED_GATE, synth.SHARED_UP, synth.SHARED_DOWN))
        return self._shared[seed]

    def head(self) -> NVFP4:
        if self._head is None:
            self._head = quantize(synth.head_f32(self.head_seed, self.vocab, self.dims.hidden))
        return self._head


def moe_layer(W: SyntheticWeights, seed: int, u: np.ndarray, route_override: np.ndarray | None = None,
              nthreads: int | None = None) -> LayerResult:
    """y = sum_i w_i * expert_{e_i}(u) + shared(u) for the layer drawn with `seed`.

    route_override: use these expert indices instead of the oracle's own top-k
    (for near-tie replay); the weights are then the renormalised softmax over
    that set.
    """
    d = W.dims
    logits = f32_gemv(W.router(seed), u, nthreads)
    idx, w, gap = topk_softmax(logits, d.top_k)
    if route_override is not None:
        idx = np.asarray(route_override, np.int32)
        m = logits.max()
        p = np.exp(logits - m) / np.exp(logits - m).sum()
        w = p[idx] / p[idx].sum()
    y = np.zeros(d.hidden, np.float64)
    for e, we in zip(idx, w):
        g, up, dn = W.expert(seed, int(e))
        y += we * swiglu_expert(g, up, dn, u, nthreads)
    sg, su, sd = W.shared(seed)
    y += swiglu_expert(sg, su, sd, u, nthreads)
    return LayerResult(y, idx, w, logits, gap)


@dataclass
class StackResult:
    logits: np.ndarray                     # float64[V]
    argmax: int
    argmax_gap: float
    routes: list = field(default_factory=list)       # per layer int32[k]
    gaps: list = field(default_factory=list)         # per layer routing gap
    layer_inputs: list = field(default_factory=list) # per layer h_l (float64[H])


def stack_token(W: SyntheticWeights, x: np.ndarray, layers: int, layer_seeds=None, eps: float = 1e-6,
                nthreads: int | None = None, keep_inputs: bool = False, with_head: bool = True) -> StackResult:
    """h_0 = x; h_{l+1} = h_l + MoE_l(h_l * rms_inv(h_l)); logits = head(h_L * rms_inv(h_L))."""
    seeds = list(range(layers)) if layer_seeds is None else list(layer_seeds)
    h = np.asarray(x, np.float64).copy()
    res = StackResult(np.zeros(0), -1, 0.0)
    for l in range(layers):
        if keep_inputs:
            res.layer_inputs.append(h.copy())
        u = h * rms_inv(h, eps)
        lr = moe_layer(W, seeds[l], u, nthreads=nthreads)
        res.routes.append(lr.idx)
        res.gaps.append(lr.gap)
        h = h + lr.y
    if keep_inputs:
        res.layer_inputs.append(h.copy())
    if with_head:
        z = h * rms_inv(h, eps)
        res.logits = nvfp4_gemv(W.head(), z, nthreads)
        res.argmax, res.argmax_gap = argmax(res.logits)
    return res


# ------------------------------------------------------------- whole model --
# Sources: [P2] "How does Flint's architecture work?" (49 layers: 2 dense,
# then 47 MoE; 35 sliding-window and 14 full-attention layers; 32 query and
# 4 key/value heads); [P3] "The shape, read from the headers" (the attention
# and the norms of every layer).  Readings: every layer is pre-norm twice,
# h += Attn(rmsnorm(h)) then h += F(rmsnorm(h)), each RMSNorm with unit gain
# and eps inside the root, and a last one before the head.

@dataclass
class ModelResult:
    logits: np.ndarray
    argmax: int
    argmax_gap: float
    h: np.ndarray                                      # final residual
    gaps: list = field(default_factory=list)           # routing gap of each MoE layer


def model_token(W: SyntheticWeights, attn: list, attn_dims: list, dense: list, moe_seeds: list, head: NVFP4,
                x: np.ndarray, pos: int, k_caches: list, v_caches: list, eps: float = 1e-6,
                nthreads: int | None = None) -> ModelResult:
    """One token through the layers (attention, then dense MLP for the first
    len(dense) layers and MoE for the rest) and the head.  k_caches and
    v_caches (uint16 [n_kv][cap][D] each) are updated in place."""
    from . import attn_decode
    nd = len(dense)
    h = np.asarray(x, np.float64).copy()
    res = ModelResult(np.zeros(0), -1, 0.0, h)
    for l in range(len(attn)):
        d = attn_dims[l]
        u = h * rms_inv(h, eps)
        y, _, _ = attn_decode(attn[l], u, pos, k_caches[l], v_caches[l], n_kv=d.n_kv, window=d.window, rope=d.rope,
                              theta=d.theta, nthreads=nthreads)
        h = h + y
        u = h * rms_inv(h, eps)
        if l < nd:
            h = h + swiglu_expert(*dense[l], u, nthreads)
        else:
            lr = moe_layer(W, moe_seeds[l - nd], u, nthreads=nthreads)
            res.gaps.append(lr.gap)
            h = h + lr.y
    z = h * rms_inv(h, eps)
    res.logits = nvfp4_gemv(head, z, nthreads)
    res.argmax, res.argmax_gap = argmax(res.logits)
    res.h = h
    return res
