"""Pins for the oracle's NVFP4 quantiser and dequantiser."""
import numpy as np
import pytest
import torch

import oracle
import synth

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_table(codes):
    codes = np.asarray(codes)
    return E2M1_MAGS[codes & 7] * np.where(codes & 8, -1.0, 1.0)


def e4m3_table(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def pack_nibbles(c):
    """element 2j in the low nibble of byte j"""
    c = np.asarray(c, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("rows,cols,seed", [(8, 64, 0), (33, 2048, 1), (5, 16, 2)])
def test_constructed_round_trip(rows, cols, seed):
    """W built from known codes c, normal E4M3 scales d and a power-of-two S, with a
    +-6 code in every block and one block of scale 448 (so max|W| = 2688 S):
    quantise must return exactly (c, d, S), dequantise exactly W."""
    rng = np.random.default_rng(seed)
    nb = cols // 16
    S = 2.0 ** -12
    c = rng.integers(0, 16, size=(rows, cols))
    blk = c.reshape(rows, nb, 16)
    pos = rng.integers(0, 16, size=(rows, nb))
    sign = rng.integers(0, 2, size=(rows, nb)) * 8
    np.put_along_axis(blk, pos[..., None], (7 + sign)[..., None], axis=2)
    d = rng.integers(0x08, 0x7F, size=(rows, nb))  # normal codes 0x08..0x7E
    d[rows // 2, nb // 2] = 0x7E
    W = (e2m1_table(c).reshape(rows, nb, 16) * e4m3_table(d)[..., None] * S).reshape(rows, cols)
    W32 = W.astype(np.float32)
    assert np.array_equal(W32.astype(np.float64), W)  # exact by construction
    q = oracle.quantize(W32)
    assert q.tscale == S
    assert np.array_equal(q.scales, d.astype(np.uint8))
    assert np.array_equal(q.codes, pack_nibbles(c))
    assert np.array_equal(oracle.dequantize(q).view(np.uint32), W32.view(np.uint32))


def test_idempotent_on_synthetic_weights():
    W = synth.expert_f32(0, synth.MoEDims(), synth.GATE, 5)[:64]
    q1 = oracle.quantize(W)
    q2 = oracle.quantize(oracle.dequantize(q1))
    assert q1.tscale == q2.tscale
    assert np.array_equal(q1.codes, q2.codes) and np.array_equal(q1.scales, q2.scales)


def test_per_element_error_bound():
    """|w - deq(w)| <= 1 * d * S: half the widest E2M1 spacing (2), plus the
    saturation excess (block max at most 6 * 17/16 in code units) stays below it."""
    W = synth.expert_f32(0, synth.MoEDims(), synth.DOWN, 2)
    q = oracle.quantize(W)
    deq = oracle.dequantize(q).astype(np.float64)
    d = e4m3_table(q.scales).repeat(16, axis=1)
    err = np.abs(W.astype(np.float64) - deq)
    assert np.all(err <= 1.0 * d * q.tscale * (1 + 1e-6))
    # and the relative Frobenius error is the few-percent an E2M1 grid gives
    rel = np.linalg.norm(W - deq) / np.linalg.norm(W)
    assert 0.02 < rel < 0.15


def test_zero_tensor_and_zero_block():
    q = oracle.quantize(np.zeros((4, 32), np.float32))
    assert q.tscale == 0.0 and not q.codes.any() and not q.scales.any()
    W = np.ones((2, 32), np.float32)
    W[1, 16:] = 0.0
    W[0, 3] = -0.0
    q = oracle.quantize(W)
    assert q.scales[1, 1] == 0 and not q.codes[1, 8:].any()
    deq = oracle.dequantize(q)
    assert np.array_equal(deq[0, :3], np.ones(3, np.float32))


def test_negative_zero_kept():
    W = np.zeros((1, 16), np.float32)
    W[0, 0] = 1.0
    W[0, 1] = -1e-9      # rounds to zero, keeps its sign
    W[0, 2] = -0.0
    q = oracle.quantize(W)
    codes = np.stack([q.codes[0] & 15, q.codes[0] >> 4], axis=1).reshape(-1)
    assert codes[1] == 8 and codes[2] == 8
    deq = oracle.dequantize(q)
    assert np.signbit(deq[0, 1]) and np.signbit(deq[0, 2])


def test_tensor_scale_definition():
    W = synth.expert_f32(3, synth.MoEDims(), synth.UP, 0)
    q = oracle.quantize(W)
    assert q.tscale == np.float32(np.abs(W).max() / 2688.0)
    # the block holding max|W| gets the largest finite E4M3 scale
    r, k = np.unravel_index(np.abs(W).argmax(), W.shape)
    assert q.scales[r, k // 16] == 0x7E
