"""Pins for the oracle's group-64 affine INT4 codec (BF16 scale and offset
per 64 values): constructed round trips, error bounds, the 4.5 bits per
weight and 1,024 code bytes per 2,048-wide row the pages print, and the GEMV
against numpy."""
import json
import os

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_byte_model.json")


def bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def to_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_constructed_round_trip_is_exact():
    rng = np.random.default_rng(0)
    rows, cols = 8, 256
    q = rng.integers(0, 16, size=(rows, cols))
    q[:, ::64] = 0   # every group holds its minimum code ...
    q[:, 1::64] = 15  # ... and its maximum
    g = cols // 64
    s_bits = to_bf16(rng.uniform(1e-3, 2e-2, size=(rows, g)))
    b_bits = to_bf16(rng.uniform(-0.2, 0.0, size=(rows, g)))
    s, b = bf16_values(s_bits), bf16_values(b_bits)
    w = (np.repeat(s, 64, 1) * q + np.repeat(b, 64, 1)).astype(np.float32)
    out = oracle.int4_quantize(w)
    assert np.array_equal(out.scales, s_bits) and np.array_equal(out.biases, b_bits)
    codes = np.zeros((rows, cols // 2), np.uint8)
    codes[:] = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)  # element 2j in the low nibble
    assert np.array_equal(out.codes, codes)
    assert np.array_equal(oracle.int4_dequantize(out), w)


def test_dequantize_matches_the_affine_formula():
    w = synth.head_f32(1000, 16, 2048)
    q = oracle.int4_quantize(w)
    lo, hi = q.codes & 15, q.codes >> 4
    codes = np.empty((16, 2048), np.int64)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    s = np.repeat(bf16_values(q.scales), 64, 1)
    b = np.repeat(bf16_values(q.biases), 64, 1)
    assert np.array_equal(oracle.int4_dequantize(q), (s * codes + b).astype(np.float32))


def test_error_bound_and_constant_groups():
    for w in (synth.head_f32(1000, 32, 2048), np.random.default_rng(1).normal(size=(8, 512)).astype(np.float32) * 50):
        q = oracle.int4_quantize(w)
        d = oracle.int4_dequantize(q)
        s = np.repeat(bf16_values(q.scales), 64, 1)
        # half a step, plus what BF16 rounding of the scale (x15) and the
        # offset can add, plus fp32 rounding
        bound = 0.5 * s + 16 * s * 2.0 ** -8 + np.abs(np.repeat(bf16_values(q.biases), 64, 1)) * 2.0 ** -8 + \
            np.abs(w) * 2.0 ** -20
        assert (np.abs(d - w) <= bound).all()
    c = np.full((2, 128), 0.3, np.float32)
    q = oracle.int4_quantize(c)
    assert (q.scales == 0).all() and (q.codes == 0).all()
    assert np.array_equal(q.biases, to_bf16(np.full((2, 2), 0.3)))


def test_bits_per_weight_and_row_bytes_match_the_pages():
    pages = json.load(open(GOLDEN))
    q = oracle.int4_quantize(synth.head_f32(1000, 4, 2048))
    bits = 8 * (q.codes.nbytes + q.scales.nbytes + q.biases.nbytes) / (4 * 2048)
    assert bits == pages["bits_per_weight_printed"]
    assert q.codes.shape[1] == pages["head_row_code_bytes_printed"]


def test_int4_gemv_against_numpy_and_one_hot():
    w = synth.head_f32(1000, 64, 4096)
    q = oracle.int4_quantize(w)
    d = oracle.int4_dequantize(q).astype(np.float64)
    x = synth.token_f32(3, 4096).astype(np.float64)
    assert np.allclose(oracle.int4_gemv(q, x), d @ x, rtol=1e-12, atol=1e-12)
    e = np.zeros(4096)
    e[1234] = 1.0
    assert np.array_equal(oracle.int4_gemv(q, e), d[:, 1234])
