"""Pins for the oracle's whole-model composition (attention + dense/MoE
layers + head): with every attention sink far above the scores the attention
adds nothing and the model is the MoE stack; one layer recomposed in plain
numpy from the oracle's own pinned parts."""
import numpy as np

import oracle
import synth
from oracle.model import SyntheticWeights, model_token, stack_token


def small_attn(seed, d):
    mats = [oracle.quantize(synth.attn_f32(seed, d, k)) for k in (synth.ATTN_Q, synth.ATTN_K, synth.ATTN_V,
                                                                   synth.ATTN_O)]
    return oracle.AttnLayer(*mats, synth.attn_gain(seed, d, synth.Q_NORM), synth.attn_gain(seed, d, synth.K_NORM),
                            synth.attn_sinks(seed, d))


def test_silent_attention_reduces_to_the_moe_stack():
    md = synth.MoEDims(n_experts=32)
    W = SyntheticWeights(md, vocab=512)
    d = synth.AttnDims(window=8)
    attn = [small_attn(100 + l, d)._replace(sinks=np.full(d.n_q, 1e4, np.float32)) for l in range(2)]
    caches = [synth.kv_cache_bits(300 + l, d, 8, synth.K_CACHE) for l in range(2)]
    vcaches = [synth.kv_cache_bits(300 + l, d, 8, synth.V_CACHE) for l in range(2)]
    x = synth.token_f32(5, 2048)
    r = model_token(W, attn, [d, d], [], [0, 1], W.head(), x, 11, caches, vcaches)
    s = stack_token(W, x, 2)
    assert np.allclose(r.logits, s.logits, rtol=1e-12, atol=1e-12)
    assert r.argmax == s.argmax


def test_one_dense_layer_recomposed():
    md = synth.MoEDims(n_experts=32)
    W = SyntheticWeights(md, vocab=256)
    d = synth.AttnDims(window=0, rope=False)
    a = small_attn(101, d)
    dense = tuple(oracle.quantize(synth.dense_f32(200, 2048, 2048, k)) for k in (synth.DENSE_GATE, synth.DENSE_UP,
                                                                                 synth.DENSE_DOWN))
    kc = synth.kv_cache_bits(301, d, 16, synth.K_CACHE)
    vc = synth.kv_cache_bits(301, d, 16, synth.V_CACHE)
    x = synth.token_f32(6, 2048).astype(np.float64)
    r = model_token(W, [a], [d], [dense], [], W.head(), x, 9, [kc.copy()], [vc.copy()])
    # by hand: h1 = x + Attn(norm x); h2 = h1 + MLP(norm h1); logits = head(norm h2)
    nrm = lambda v: v / np.sqrt(np.mean(v * v) + 1e-6)
    y, _, _ = oracle.attn_decode(a, nrm(x), 9, kc.copy(), vc.copy(), n_kv=4, window=0, rope=False)
    h1 = x + y
    h2 = h1 + oracle.swiglu_expert(*dense, nrm(h1))
    ref = oracle.dequantize(W.head()).astype(np.float64) @ nrm(h2)
    assert np.allclose(r.logits, ref, rtol=1e-10, atol=1e-12)
