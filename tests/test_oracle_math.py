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


# ---------------------------------------------------- router variants ----
def test_topk_sigmoid_closed_form():
    # sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2, sigmoid(-ln 3) = 1/4
    l = np.array([0.0, np.log(3.0), -np.log(3.0), -5.0])
    idx, w, gap = oracle.topk_sigmoid(l, 3)
    assert list(idx) == [1, 0, 2]
    assert np.allclose(w, [0.5, 1.0 / 3.0, 1.0 / 6.0], rtol=1e-14, atol=0)
    assert gap == pytest.approx(-np.log(3.0) + 5.0, rel=1e-15)
    idx, w, _ = oracle.topk_sigmoid(l, 2)
    assert list(idx) == [1, 0] and np.allclose(w, [0.6, 0.4], rtol=1e-14, atol=0)
    # k = 1 puts all the weight on the best expert; equal logits tie to the lower index
    assert oracle.topk_sigmoid(l, 1)[1][0] == 1.0
    idx, w, gap = oracle.topk_sigmoid(np.zeros(8), 3)
    assert list(idx) == [0, 1, 2] and np.allclose(w, 1.0 / 3.0) and gap == 0.0


@pytest.mark.parametrize("E,k", [(4, 1), (8, 3), (32, 6), (256, 6)])
def test_topk_sigmoid_against_sort_and_expit(E, k):
    from scipy.special import expit
    rng = np.random.default_rng(E * 7 + k)
    for trial in range(30):
        l = rng.normal(size=E) * 3.0
        if trial % 3 == 0:
            l[rng.integers(0, E, size=E // 2)] = l[0]
        idx, w, gap = oracle.topk_sigmoid(l, k)
        order = np.lexsort((np.arange(E), -l))
        assert list(idx) == list(order[:k])
        s = expit(l[idx])
        assert np.allclose(w, s / s.sum(), rtol=1e-13, atol=0)
        assert abs(w.sum() - 1.0) < 1e-12 and (w > 0).all()
        srt = np.sort(l)[::-1]
        assert gap == (srt[k - 1] - srt[k] if E > k else np.inf)


def test_topk_sigmoid_brute_force_subsets():
    """The chosen set is the k-subset with the largest total score."""
    import itertools
    from scipy.special import expit
    rng = np.random.default_rng(11)
    for _ in range(20):
        l = rng.normal(size=9)
        best = max(itertools.combinations(range(9), 3), key=lambda c: expit(l[list(c)]).sum())
        idx, _, _ = oracle.topk_sigmoid(l, 3)
        assert sorted(idx.tolist()) == sorted(best)


def test_topk_sigmoid_tends_to_softmax_for_very_negative_logits():
    # sigmoid(l) = e^l / (1 + e^l): for l << 0 the scores are e^l to relative
    # error e^l, so the renormalised weights approach the softmax ones
    rng = np.random.default_rng(5)
    l = rng.normal(size=64)
    i_s, w_s, _ = oracle.topk_sigmoid(l - 40.0, 6)
    i_m, w_m, _ = oracle.topk_softmax(l, 6)
    assert list(i_s) == list(i_m)
    assert np.allclose(w_s, w_m, rtol=1e-12, atol=0)
    # and differ from them at ordinary logits
    w_o = oracle.topk_sigmoid(l, 6)[1]
    assert np.abs(w_o - w_m).max() > 1e-3


def test_bf16_decode_every_pattern_against_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    got = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.signbit(got[finite]), np.signbit(ref[finite]))
    assert np.isnan(got[~finite]).all()


def test_bf16_decode_known_values():
    b = np.array([0x3F80, 0xC000, 0x3E80, 0x0001, 0x0080, 0x7F7F, 0x8000, 0x4049], np.uint16)
    v = oracle.bf16_decode(b)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.25
    assert v[3] == 2.0 ** -133 and v[4] == 2.0 ** -126
    assert v[5] == (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == 3.140625  # 0x4049: 2 * (1 + 73/128)
