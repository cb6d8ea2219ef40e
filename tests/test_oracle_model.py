"""Pins for the oracle's layer and stack composition, on reduced sizes."""
import numpy as np
import torch

import oracle
import synth
from oracle.model import SyntheticWeights, moe_layer, stack_token

SMALL = synth.MoEDims(hidden=64, n_experts=8, expert_width=32, top_k=2, shared_width=64)


def dense(q):
    return torch.from_numpy(oracle.dequantize(q).astype(np.float64))


def torch_layer(W, seed, u):
    """Independent composition with torch: softmax over all experts, the set of
    the k largest, renormalised weights, SwiGLU experts, shared expert weight 1."""
    d = W.dims
    R = torch.from_numpy(W.router(seed).astype(np.float64))
    U = torch.from_numpy(u)
    logits = R @ U
    p = torch.softmax(logits, dim=0)
    top = torch.topk(logits, d.top_k).indices
    w = p[top] / p[top].sum()
    y = torch.zeros(d.hidden, dtype=torch.float64)
    for e, we in zip(top.tolist(), w):
        g, up, dn = (dense(q) for q in W.expert(seed, e))
        y += we * (dn @ (torch.nn.functional.silu(g @ U) * (up @ U)))
    g, up, dn = (dense(q) for q in W.shared(seed))
    y += dn @ (torch.nn.functional.silu(g @ U) * (up @ U))
    return y.numpy(), sorted(top.tolist())


def test_layer_matches_torch_composition():
    W = SyntheticWeights(SMALL, vocab=96)
    for t in range(5):
        u = synth.token_f32(100 + t, SMALL.hidden).astype(np.float64)
        r = moe_layer(W, 0, u)
        y_ref, set_ref = torch_layer(W, 0, u)
        assert sorted(r.idx.tolist()) == set_ref
        assert np.allclose(r.y, y_ref, rtol=1e-12, atol=1e-14)


def test_expert_relabelling_invariance():
    """Permuting expert ids together with router rows permutes the chosen ids
    and leaves the output unchanged."""
    W = SyntheticWeights(SMALL, vocab=96)
    perm = np.random.default_rng(0).permutation(SMALL.n_experts)
    P = SyntheticWeights(SMALL, vocab=96)
    P._router[0] = W.router(0)[perm]
    for new, old in enumerate(perm):
        P._experts[(0, new)] = W.expert(0, int(old))
    P._shared[0] = W.shared(0)
    u = synth.token_f32(7, SMALL.hidden).astype(np.float64)
    a, b = moe_layer(W, 0, u), moe_layer(P, 0, u)
    assert sorted(perm[b.idx].tolist()) == sorted(a.idx.tolist())
    assert np.allclose(a.y, b.y, rtol=1e-13, atol=1e-15)


def test_stack_is_prenorm_residual_then_head():
    W = SyntheticWeights(SMALL, vocab=96)
    x = synth.token_f32(3, SMALL.hidden)
    res = stack_token(W, x, layers=3, keep_inputs=True)
    h = x.astype(np.float64)
    for l in range(3):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (SMALL.hidden,), eps=1e-6).numpy()
        h = h + moe_layer(W, l, ref).y
        assert np.allclose(res.layer_inputs[l + 1], h, rtol=1e-12, atol=1e-14)
    z = torch.nn.functional.rms_norm(torch.from_numpy(h), (SMALL.hidden,), eps=1e-6)
    logits = (dense(W.head()) @ z).numpy()
    assert np.allclose(res.logits, logits, rtol=1e-11, atol=1e-13)
    assert res.argmax == int(np.argmax(logits))
