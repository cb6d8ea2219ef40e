"""Shared NVFP4 quantiser cases for the host-encoder test (CPU tier) and the
device-quantiser test (GPU tier): expert matrices of the synthetic model, a
slice of the head, a wide dynamic range, zero blocks with -0 and tiny
values, and an all-zero matrix."""
import numpy as np

import synth


def quant_cases():
    d = synth.MoEDims()
    rng = np.random.default_rng(0)
    wide = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 5, (64, 1)))).astype(np.float32)
    special = synth.expert_f32(1, d, synth.UP, 2)[:40].copy()
    special[3, 16:32] = 0.0
    special[5, 7] = -0.0
    special[6, 0:16] = -1e-12
    special[6, 3] = 0.05
    return {
        "gate": synth.expert_f32(0, d, synth.GATE, 0),
        "down": synth.expert_f32(0, d, synth.DOWN, 5),
        "head_slice": synth.head_f32(synth.HEAD_SEED, 150144, 2048, row0=1000, rows=4099),
        "wide_dynamic_range": wide,
        "zero_blocks_neg_zero": special,
        "all_zero": np.zeros((8, 64), np.float32),
    }
