"""GPU parity of the group-64 affine INT4 codec (through the C ABI) against
the CPU oracle: quantiser, dequantised weights and argmax bit-exact; GEMV
outputs within relative L2 <= 1e-4 and max-abs <= 2e-3 * max|ref|."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4
MAX_ABS = 2e-3
MARGIN = 1e-5


@pytest.fixture(scope="module")
def F():
    from nvfp4_bit_projection_amd import flint
    torch.cuda.set_device(0)
    return flint


def assert_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e}"
    assert np.abs(got - ref).max() <= MAX_ABS * np.abs(ref).max(), what


def gpu_q(F, q):
    return q.codes.cpu().numpy(), q.scales.cpu().numpy().view(np.uint16), q.biases.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols", [(37, 64), (300, 2048), (129, 4096), (64, 192)])
def test_quantize_and_dequantize_bit_exact(F, rows, cols):
    w = synth.head_f32(1000, rows, cols)
    w[3, :64] = 0.25  # a constant group: scale 0
    print(f"int4 quantize rows={rows} cols={cols}", flush=True)
    q = F.int4_quantize(torch.from_numpy(w).cuda())
    ref = oracle.int4_quantize(w)
    c, s, b = gpu_q(F, q)
    assert np.array_equal(c, ref.codes) and np.array_equal(s, ref.scales) and np.array_equal(b, ref.biases)
    d = F.int4_dequantize(q).cpu().numpy()
    assert np.array_equal(d.view(np.uint32), oracle.int4_dequantize(ref).view(np.uint32))


@pytest.mark.parametrize("rows,cols,B", [(1000, 2048, 1), (1003, 2048, 3), (517, 4096, 2), (260, 6144, 1),
                                         (130, 8192, 2)])
def test_gemv_and_argmax(F, rows, cols, B):
    w = synth.head_f32(1001, rows, cols)
    ref = oracle.int4_quantize(w)
    q = F.int4_quantize(torch.from_numpy(w).cuda())
    xs = np.stack([synth.token_f32(70 + b, cols) for b in range(B)])
    print(f"int4 gemv rows={rows} cols={cols} B={B}", flush=True)
    y, am = F.int4_gemv(q, torch.from_numpy(xs).cuda())
    torch.cuda.synchronize()
    for b in range(B):
        yr = oracle.int4_gemv(ref, xs[b].astype(np.float64))
        assert_close(y[b].cpu().numpy(), yr, f"b={b}")
        i, gap = oracle.argmax(yr)
        if gap >= MARGIN * np.abs(yr).max():
            assert int(am[b]) == i


def test_head_full_size(F):
    """The 150,144 x 2,048 head quantised on the device: every code, scale
    and offset bit-exact against the oracle's quantiser; for two tokens all
    150,144 logits within the bar and the argmax equal to the oracle's (the
    tokens' top-2 margins checked first)."""
    V, H = 150144, 2048
    w = torch.empty(V * H, dtype=torch.float32, device="cuda")
    synth.normal_device(synth.HEAD_SEED, synth.stream_id(synth.HEAD), V * H, w, std=synth.WEIGHT_STD)
    q = F.int4_quantize(w.view(V, H))
    del w
    ref = oracle.int4_quantize(synth.head_f32(synth.HEAD_SEED, V, H))
    c, s, b = gpu_q(F, q)
    assert np.array_equal(c, ref.codes) and np.array_equal(s, ref.scales) and np.array_equal(b, ref.biases)
    seeds = [synth.TOKEN_SEED0, synth.TOKEN_SEED0 + 1]
    x = np.stack([synth.token_f32(sd, H) for sd in seeds])
    print("int4 full head: two tokens", flush=True)
    y, am = F.int4_gemv(q, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    for b_ in range(2):
        yr = oracle.int4_gemv(ref, x[b_].astype(np.float64))
        assert_close(y[b_].cpu().numpy(), yr, f"full head token {b_}")
        i, gap = oracle.argmax(yr)
        assert gap >= MARGIN, "token not screened"
        assert int(am[b_]) == i
