"""Pins for the oracle's routing, products, expert, norm and argmax (brute force,
library routines and invariants)."""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
import synth


@pytest.mark.parametrize("E,k", [(4, 1), (4, 4), (8, 3), (16, 6), (32, 6), (256, 6)])
def test_topk_against_full_sort(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for trial in range(30):
        l = rng.normal(size=E)
        if trial % 3 == 0:  # inject ties
            l[rng.integers(0, E, size=E // 2)] = l[0]
        idx, w, gap = oracle.topk_softmax(l, k)
        order = np.lexsort((np.arange(E), -l))  # by -logit, then index
        assert list(idx) == list(order[:k])
        srt = np.sort(l)[::-1]
        assert gap == (srt[k - 1] - srt[k] if E > k else np.inf)
        # renormalised weights: sum 1, equal the softmax over the chosen logits
        assert abs(w.sum() - 1.0) < 1e-12
        assert np.allclose(w, softmax(l[idx]), rtol=1e-12, atol=0)
        # ratios are exp of logit differences
        assert np.allclose(w[0] / w, np.exp(l[idx[0]] - l[idx]), rtol=1e-12)


def test_argmax_first_index_on_ties():
    v = np.array([1.0, 3.0, 2.0, 3.0])
    assert oracle.argmax(v) == (1, 0.0)
    rng = np.random.default_rng(3)
    for _ in range(20):
        x = rng.normal(size=1000)
        i, gap = oracle.argmax(x)
        assert i == int(np.argmax(x))
        assert gap == np.sort(x)[-1] - np.sort(x)[-2]


def test_nvfp4_gemv_matches_dense_matmul():
    W = synth.head_f32(1000, 300, 2048)
    q = oracle.quantize(W)
    x = synth.token_f32(5, 2048).astype(np.float64)
    dense = oracle.dequantize(q).astype(np.float64)
    y = oracle.nvfp4_gemv(q, x, nthreads=3)
    assert np.allclose(y, dense @ x, rtol=1e-12, atol=1e-12)
    assert np.array_equal(y, oracle.nvfp4_gemv(q, x, nthreads=1))  # thread-count independent


def test_one_hot_recovers_dequantised_column():
    W = synth.expert_f32(0, synth.MoEDims(), synth.GATE, 1)
    q = oracle.quantize(W)
    dense = oracle.dequantize(q)
    for k in (0, 1, 15, 16, 777, 2047):
        x = np.zeros(2048)
        x[k] = 1.0
        assert np.array_equal(oracle.nvfp4_gemv(q, x).astype(np.float32), dense[:, k])


def test_f32_gemv_matches_matmul():
    W = synth.router_f32(0, synth.MoEDims(n_experts=32))
    x = synth.token_f32(0, 2048).astype(np.float64)
    assert np.allclose(oracle.f32_gemv(W, x), W.astype(np.float64) @ x, rtol=1e-12, atol=1e-13)


def test_swiglu_expert_matches_torch():
    d = synth.MoEDims()
    g, u, dn = (oracle.quantize(synth.expert_f32(9, d, kind, 4)) for kind in (synth.GATE, synth.UP, synth.DOWN))
    x = synth.token_f32(9, 2048).astype(np.float64)
    y, h = oracle.swiglu_expert(g, u, dn, x, return_hidden=True)
    G = torch.from_numpy(oracle.dequantize(g).astype(np.float64))
    U = torch.from_numpy(oracle.dequantize(u).astype(np.float64))
    D = torch.from_numpy(oracle.dequantize(dn).astype(np.float64))
    X = torch.from_numpy(x)
    H = torch.nn.functional.silu(G @ X) * (U @ X)
    assert np.allclose(h, H.numpy(), rtol=1e-11, atol=1e-14)
    assert np.allclose(y, (D @ H).numpy(), rtol=1e-10, atol=1e-13)


def test_rms_inv_matches_torch_rms_norm():
    h = synth.token_f32(11, 2048).astype(np.float64) * 3.7
    for eps in (1e-6, 1e-2):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (2048,), eps=eps).numpy()
        assert np.allclose(h * oracle.rms_inv(h, eps), ref, rtol=1e-13, atol=0)
