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


def wide_tiles(N, T):
    """256 x 256 tiles of a call: at 128 or more the library takes the wide
    kernel (weights decoded once per workgroup into LDS, fp16 activation
    planes), below it the narrow one."""
    return -(-N // 256) * -(-T // 256)


@pytest.mark.parametrize("N,K,T", [(16456, 2048, 1000), (16385, 1024, 1024), (8200, 1024, 2000),
                                   (8448, 256, 1024), (8448, 6144, 1000), (32800, 512, 100)])
@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_wide_against_oracle(F, N, K, T, mode):
    """Shapes on the wide kernel, every output against the oracle: ragged last
    row block (72, 1 and 8 rows; N % 4 = 1 takes the scalar stores), ragged
    last token block, K = 256 (the shortest pipeline: 4 or 8 stages, every
    request past the end clamped), K = 6,144, and one token block of 100
    tokens under 129 row blocks."""
    assert wide_tiles(N, T) >= 128
    w = synth.head_f32(1010, N, K)
    ref_q = oracle.quantize(w)
    q = F.quantize(torch.from_numpy(w).cuda())
    X = synth.normal(1011, synth.stream_id(synth.TOKEN), T * K, std=1.0).reshape(T, K)
    print(f"gemm wide N={N} K={K} T={T} mode={mode}", flush=True)
    Y = F.nvfp4_gemm(q, torch.from_numpy(X).cuda(), mode)
    torch.cuda.synchronize()
    assert_close(Y.cpu().numpy(), oracle.nvfp4_gemm(ref_q, X, a4=bool(mode)), f"N={N} K={K} T={T}")


@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_head_full_size_sampled(F, mode):
    """The 150,144 x 2,048 head and 2,048 tokens, the call the prefill bench
    times: the weights quantised on the device (bit-exact with the oracle's
    quantiser, checked in the codec tests), all 2,048 tokens on 80 sampled
    weight rows (the first and last row blocks among them) against the oracle
    applied to those rows of the oracle's own quantised head."""
    V, H, T = 150144, 2048, 2048
    w = torch.empty(V * H, dtype=torch.float32, device="cuda")
    synth.normal_device(synth.HEAD_SEED, synth.stream_id(synth.HEAD), V * H, w, std=synth.WEIGHT_STD)
    q = F.quantize(w.view(V, H))
    del w
    ref = oracle.quantize(synth.head_f32(synth.HEAD_SEED, V, H))
    X = synth.normal(1020, synth.stream_id(synth.TOKEN), T * H, std=1.0).reshape(T, H)
    print(f"gemm head full size mode={mode}", flush=True)
    Y = F.nvfp4_gemm(q, torch.from_numpy(X).cuda(), mode)
    rng = np.random.default_rng(5)
    sel = np.unique(np.concatenate([[0, 1, 255, 256, V - 256, V - 2, V - 1], rng.integers(0, V, 73)]))
    got = Y[:, torch.from_numpy(sel).cuda()].cpu().numpy()
    torch.cuda.synchronize()
    del Y
    sub = oracle.NVFP4(ref.codes[sel], ref.scales[sel], ref.tscale, len(sel), H)
    assert_close(got, oracle.nvfp4_gemm(sub, X, a4=bool(mode)), f"head sampled mode={mode}")
