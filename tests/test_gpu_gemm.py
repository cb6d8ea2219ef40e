"""GPU parity of the prefill GEMM on matrix cores (through the C ABI) against
the CPU oracle: relative L2 <= 1e-4 and max-abs <= 2e-3 * max|ref| for Y;
the A4 variant's quantised activations bit-exact with the oracle's codec."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    from nvfp4_bit_projection_amd import flint
    torch.cuda.set_device(0)
    return flint


def assert_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 1e-4, f"{what}: rel L2 {rel:.3e}"
    assert np.abs(got - ref).max() <= 2e-3 * np.abs(ref).max(), what


@pytest.mark.parametrize("N,K,T", [(200, 2048, 37), (1024, 512, 1), (300, 4096, 100), (2048, 6144, 64),
                                   (129, 256, 33)])
@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_against_oracle(F, N, K, T, mode):
    w = synth.head_f32(1000, N, K)
    ref_q = oracle.quantize(w)
    q = F.quantize(torch.from_numpy(w).cuda())
    X = np.stack([synth.token_f32(500 + t, K) for t in range(T)])
    print(f"gemm N={N} K={K} T={T} mode={mode}", flush=True)
    ws = F.gemm_workspace(T, K, mode)
    Y = F.nvfp4_gemm(q, torch.from_numpy(X).cuda(), mode, ws=ws)
    torch.cuda.synchronize()
    assert_close(Y.cpu().numpy(), oracle.nvfp4_gemm(ref_q, X, a4=bool(mode)), f"N={N} K={K} T={T}")
    if mode == 1:  # the quantised activations the call kept in its workspace
        xr = oracle.quantize(X)
        wsn = ws.cpu().numpy()
        assert np.array_equal(wsn[512:512 + T * K // 2].reshape(T, K // 2), xr.codes)


def test_gemm_repeat_calls_same_workspace(F):
    """A4 twice on one workspace (its counters come back to zero), then a
    larger token count: every call matches the oracle."""
    N, K = 256, 2048
    w = synth.head_f32(1002, N, K)
    ref_q = oracle.quantize(w)
    q = F.quantize(torch.from_numpy(w).cuda())
    ws = F.gemm_workspace(64, K, 1)
    for T in (64, 64, 20):
        X = np.stack([synth.token_f32(900 + T + t, K) for t in range(T)])
        Y = F.nvfp4_gemm(q, torch.from_numpy(X).cuda(), 1, ws=ws)
        torch.cuda.synchronize()
        assert_close(Y.cpu().numpy(), oracle.nvfp4_gemm(ref_q, X, a4=True), f"T={T}")
