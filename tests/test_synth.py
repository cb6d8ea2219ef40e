"""The shared input generator: known-answer vectors, distribution, reproducibility."""
import numpy as np
import pytest
import torch
from scipy import stats

import synth


# Known-answer vectors of Philox4x32-10 published with the Random123 library
# (Salmon et al., SC'11): counter, key -> output.
PHILOX_KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    assert list(synth.philox4x32_10(ctr, key)) == list(want)


def test_normal_distribution():
    z = synth.normal(7, synth.stream_id(synth.TOKEN), 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3
    assert abs(z.std() - 1.0) < 5e-3
    assert abs(stats.kurtosis(z, fisher=False) - 3.0) < 0.03
    # Kolmogorov-Smirnov against the standard normal CDF
    assert stats.kstest(z[:200000], "norm").pvalue > 1e-4


def test_scaled_weights():
    w = synth.normal(0, synth.stream_id(synth.GATE, 3), 1 << 18, std=synth.WEIGHT_STD)
    assert abs(w.std() - 0.02) < 2e-4


def test_thread_count_and_offset_independence():
    n = 300_001
    a = synth.normal(3, 5, n, nthreads=1)
    b = synth.normal(3, 5, n, nthreads=7)
    assert np.array_equal(a, b)
    for off in (1, 2, 3, 4, 63, 64, 1001):
        c = synth.normal(3, 5, 1000, offset=off)
        assert np.array_equal(c, a[off:off + 1000])


def test_streams_differ():
    a = synth.normal(0, synth.stream_id(synth.GATE, 0), 1024)
    b = synth.normal(0, synth.stream_id(synth.GATE, 1), 1024)
    c = synth.normal(1, synth.stream_id(synth.GATE, 0), 1024)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_workload_shapes():
    d = synth.MoEDims(n_experts=32)
    assert synth.router_f32(0, d).shape == (32, 2048)
    assert synth.expert_f32(0, d, synth.GATE, 1).shape == (512, 2048)
    assert synth.expert_f32(0, d, synth.DOWN, 1).shape == (2048, 512)
    assert synth.shared_f32(0, d, synth.SHARED_DOWN).shape == (2048, 1024)
    full = synth.head_f32(1000, 40, 2048)
    part = synth.head_f32(1000, 40, 2048, row0=17, rows=5)
    assert np.array_equal(full[17:22], part)
    # router rows of the E=32 workload are the first rows of the E=256 one
    assert np.array_equal(synth.router_f32(0, synth.MoEDims()).reshape(256, 2048)[:32], synth.router_f32(0, d))


def test_router_bf16_is_nearest_even():
    d = synth.MoEDims(n_experts=32)
    f = synth.router_f32(3, d).ravel()
    b = synth.router_bf16_bits(3, d).ravel()
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
