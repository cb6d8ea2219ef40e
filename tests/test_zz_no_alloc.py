"""flint_moe_decode_noalloc (the entry point for callers that cannot
allocate: scratch in a fixed device array inside the library) against
flint_moe_decode with a caller workspace, through the C ABI: identical bits
for the layer output, the chosen experts and their weights, on two calls in
a row with the second one smaller; sizes beyond the fixed array are
rejected before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    from nvfp4_bit_projection_amd import flint, workload
    torch.cuda.set_device(0)
    return flint, workload


def test_no_alloc_matches_decode(F):
    flint, workload = F
    dims = synth.MoEDims()
    d = flint.dims_struct(dims.hidden, dims.n_experts, dims.expert_width, dims.top_k, dims.shared_width)
    layer = workload.build_layer(dims, seed=3)
    for B, seed0 in ((8, 100), (3, 200)):  # the second call smaller than the first
        print(f"no-alloc decode B={B}", flush=True)
        x = workload.tokens(range(seed0, seed0 + B), dims.hidden)
        y_ref, i_ref, w_ref = flint.moe_decode(d, layer, x)
        y = torch.full_like(y_ref, float("nan"))
        idx = torch.full_like(i_ref, -1)
        w = torch.full_like(w_ref, float("nan"))
        flint.moe_decode_noalloc(d, layer, x, y, idx, w)
        torch.cuda.synchronize()
        assert torch.equal(idx, i_ref)
        assert torch.equal(w, w_ref)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32))


def test_no_alloc_reduced_layer_without_route_outputs(F):
    """The 32-expert layer, routes not asked for (kept in the fixed scratch)."""
    flint, workload = F
    dims = synth.MoEDims(n_experts=32)
    d = flint.dims_struct(dims.hidden, dims.n_experts, dims.expert_width, dims.top_k, dims.shared_width)
    layer = workload.build_layer(dims, seed=0)
    x = workload.tokens(range(5, 10), dims.hidden)
    y_ref, _, _ = flint.moe_decode(d, layer, x)
    y = torch.empty_like(y_ref)
    lc = layer.c()
    st = flint.lib().flint_moe_decode_noalloc(ctypes.byref(d), ctypes.byref(lc), x.data_ptr(), 5, y.data_ptr(), None,
                                             None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(y, y_ref)


def test_no_alloc_rejects_beyond_the_array(F):
    flint, workload = F
    dims = synth.MoEDims()
    d = flint.dims_struct(dims.hidden, dims.n_experts, dims.expert_width, dims.top_k, dims.shared_width)
    layer = workload.build_layer(dims, seed=3)
    B = 100
    x = torch.zeros((B, dims.hidden), dtype=torch.float32, device="cuda")
    y = torch.full((B, dims.hidden), 7.0, dtype=torch.float32, device="cuda")
    lc = layer.c()
    st = flint.lib().flint_moe_decode_noalloc(ctypes.byref(d), ctypes.byref(lc), x.data_ptr(), B, y.data_ptr(), None,
                                             None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == -4  # FLINT_E_WORKSPACE, nothing enqueued
    assert bool((y == 7.0).all())
