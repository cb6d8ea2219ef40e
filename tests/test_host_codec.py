"""The library's host NVFP4 encoder (flint_nvfp4_quantize_host, CPU tier):
bit-exact against the oracle's quantiser on the device quantiser's cases, on
a constructed round trip whose exact answer is known, on every E2M1 and E4M3
rounding midpoint, and independent of the thread split on a large matrix."""
import numpy as np
import pytest

import oracle
import synth
from codec_cases import quant_cases


@pytest.fixture(scope="module")
def F():
    from nvfp4_bit_projection_amd import build
    import os
    if not os.path.exists(build.LIB_PATH):
        build.build_library()
    from nvfp4_bit_projection_amd import flint
    return flint


def assert_same(got, ref):
    codes, scales, ts = got
    assert np.float32(ts).view(np.uint32) == np.float32(ref.tscale).view(np.uint32)
    assert np.array_equal(scales, ref.scales)
    assert np.array_equal(codes, ref.codes)


@pytest.mark.parametrize("name", list(quant_cases().keys()))
def test_host_quantizer_bit_exact(F, name):
    w = quant_cases()[name]
    assert_same(F.quantize_host(w), oracle.quantize(w))


def test_host_quantizer_constructed_round_trip(F):
    """Known codes c, normal E4M3 scales d and a power-of-two S, a +-6 code in
    every block and one block of scale 448: the encoder returns exactly
    (c, d, S)."""
    rng = np.random.default_rng(11)
    rows, cols = 17, 256
    nb, S = cols // 16, 2.0 ** -10
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    c = rng.integers(0, 16, size=(rows, nb, 16))
    pos = rng.integers(0, 16, size=(rows, nb))
    np.put_along_axis(c, pos[..., None], (7 + 8 * rng.integers(0, 2, size=(rows, nb)))[..., None], axis=2)
    d = rng.integers(0x08, 0x7F, size=(rows, nb))
    d[3, 4] = 0x7E
    dv = np.array([oracle.e4m3_value(int(v)) for v in range(256)])[d]
    W = (mags[c & 7] * np.where(c & 8, -1.0, 1.0) * dv[..., None] * S).reshape(rows, cols).astype(np.float32)
    codes, scales, ts = F.quantize_host(W)
    assert ts == np.float32(S)
    assert np.array_equal(scales, d.astype(np.uint8))
    flat = c.reshape(rows, cols)
    assert np.array_equal(codes, (flat[:, 0::2] | (flat[:, 1::2] << 4)).astype(np.uint8))


def test_host_quantizer_midpoints(F):
    """Elements on every E2M1 midpoint (ties to the even code) and block
    maxima on E4M3 midpoints, in one matrix with S = 1 (max|w| = 2688)."""
    w = np.zeros((4, 64), np.float32)
    w[0, 0] = 2688.0                                   # S = 1, that block's scale 448
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 7.0])
    # block scale 1 (blockmax 6 = 6 * 1): elements are the ratios themselves
    w[1, :16] = 0.0
    w[1, 0] = 6.0
    w[1, 1:1 + len(mids)] = mids
    w[1, 10:13] = -mids[:3]
    # block maxima whose ratio r = bm / 6 sits on an E4M3 midpoint
    for j, r in enumerate([1.0625, 1.1875, 2.0 ** -7 * 1.5, 2.0 ** -9 * 0.5, 2.0 ** -9 * 1.5, 464.0]):
        w[2 + j // 4, 16 * (j % 4)] = np.float32(6.0 * r)
    assert_same(F.quantize_host(w), oracle.quantize(w))


def test_host_quantizer_threads_do_not_matter(F):
    """A matrix large enough to be split over host threads gives the oracle's
    bits (the head's first 1,024 rows)."""
    w = synth.head_f32(synth.HEAD_SEED, 150144, 2048, row0=0, rows=1024)
    assert_same(F.quantize_host(w), oracle.quantize(w))


def test_host_quantizer_rejects(F):
    L = F.lib()
    buf = np.zeros(64, np.float32)
    out = np.zeros(64, np.uint8)
    assert L.flint_nvfp4_quantize_host(None, 1, 16, out.ctypes.data, out.ctypes.data, buf.ctypes.data) == -1
    assert L.flint_nvfp4_quantize_host(buf.ctypes.data, 1, 24, out.ctypes.data, out.ctypes.data,
                                       buf.ctypes.data) == -2
    assert L.flint_nvfp4_quantize_host(buf.ctypes.data, 0, 16, out.ctypes.data, out.ctypes.data,
                                       buf.ctypes.data) == -2
