"""Pins for the oracle's E2M1 / E4M3 codecs (closed forms and library routines)."""
import math

import numpy as np
import pytest
import torch

import oracle

# E2M1 magnitudes of codes 0..7 (OCP Microscaling formats spec, FP4 E2M1 table)
E2M1_MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_all_codes():
    for c in range(16):
        want = E2M1_MAGS[c & 7] * (-1.0 if c & 8 else 1.0)
        got = oracle.e2m1_value(c)
        assert got == want and math.copysign(1.0, got) == (-1.0 if c & 8 else 1.0)


def test_e4m3_decode_matches_torch_float8():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], c
    assert oracle.e4m3_value(0x7E) == 448.0


def test_e2m1_rne_midpoints_and_saturation():
    # value midpoints between neighbouring magnitudes round to the even code
    mid = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, want in mid.items():
        assert oracle.e2m1_value(oracle.e2m1_encode(v)) == want
        assert oracle.e2m1_value(oracle.e2m1_encode(-v)) == -want
    for v in (6.0, 6.9, 7.0, 100.0, 1e30):
        assert oracle.e2m1_encode(v) == 7 and oracle.e2m1_encode(-v) == 15
    assert oracle.e2m1_encode(-0.0) == 8 and oracle.e2m1_encode(-0.1) == 8
    assert oracle.e2m1_encode(0.0) == 0


def test_e2m1_nearest_against_sorted_grid():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.uniform(0, 7, 4000), np.arange(0, 7.01, 0.125)])
    grid = np.array(E2M1_MAGS)
    for v in vals:
        got = oracle.e2m1_value(oracle.e2m1_encode(v))
        d = np.abs(grid - v)
        best = np.flatnonzero(d == d.min())
        if len(best) == 2:  # tie: even code index
            best = [b for b in best if b % 2 == 0]
        assert got == grid[best[0]], v


def test_e4m3_encode_matches_torch_rne():
    # every representable value, every midpoint between neighbours (exact in
    # float32), and random points, all within [0, 464]
    pos = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(1)
    rnd = np.exp(rng.uniform(np.log(1e-4), np.log(460), 5000))
    vals = np.concatenate([pos, mids, rnd, [464.0, 1e-9, 2.0 ** -10, 3 * 2.0 ** -11]]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, r in zip(vals, ref):
        assert oracle.e4m3_encode(float(v)) == int(r), float(v)


def test_e4m3_saturates():
    for v in (448.0, 470.0, 1e6, float("inf")):
        assert oracle.e4m3_encode(v) == 0x7E


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_encode_decode_identity_on_every_finite_code(fmt):
    if fmt == "e2m1":
        for c in range(16):
            assert oracle.e2m1_encode(oracle.e2m1_value(c)) == c
    else:
        for c in range(0x7F):
            assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c
