"""Pins for the oracle's prefill GEMM (T tokens through one NVFP4 matrix) and
its A4 variant (activations quantised to NVFP4 first, one tensor scale)."""
import numpy as np

import oracle
import synth


def weights(rows=96, cols=512, seed=1000):
    return oracle.quantize(synth.head_f32(seed, rows, cols))


def test_gemm_matches_numpy_matmul():
    q = weights()
    X = np.stack([synth.token_f32(s, q.cols) for s in range(7)]).astype(np.float64)
    Y = oracle.nvfp4_gemm(q, X)
    assert np.allclose(Y, X @ oracle.dequantize(q).astype(np.float64).T, rtol=1e-12, atol=1e-12)


def test_a4_equals_full_precision_on_representable_activations():
    q = weights()
    X0 = np.stack([synth.token_f32(s, q.cols) for s in range(5)])
    X = oracle.dequantize(oracle.quantize(X0))  # already on the NVFP4 grid of its own tensor scale
    assert np.array_equal(oracle.nvfp4_gemm(q, X, a4=True), oracle.nvfp4_gemm(q, X.astype(np.float64)))


def test_a4_is_the_product_with_the_quantised_activations():
    q = weights()
    X = np.stack([synth.token_f32(10 + s, q.cols) for s in range(6)])
    E = oracle.dequantize(oracle.quantize(X)).astype(np.float64) - X
    W = oracle.dequantize(q).astype(np.float64)
    d = oracle.nvfp4_gemm(q, X, a4=True) - oracle.nvfp4_gemm(q, X.astype(np.float64))
    assert np.allclose(d, E @ W.T, rtol=1e-9, atol=1e-12)
    assert np.abs(d).max() > 0  # quantising N(0, 1) activations does change the result


def test_a4_one_tensor_scale():
    """Scaling all activations by 2^j scales the A4 result by 2^j exactly (the
    tensor scale absorbs it); one large token changes the other tokens'
    result (they share the tensor scale)."""
    q = weights()
    X = np.stack([synth.token_f32(20 + s, q.cols) for s in range(4)])
    Y = oracle.nvfp4_gemm(q, X, a4=True)
    assert np.array_equal(oracle.nvfp4_gemm(q, X * 8.0, a4=True), Y * 8.0)
    X2 = X.copy()
    X2[3] *= 100.0
    Y2 = oracle.nvfp4_gemm(q, X2, a4=True)
    assert not np.array_equal(Y2[:3], Y[:3])
