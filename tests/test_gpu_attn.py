"""GPU parity of the attention layer and the dense MLP (through the C ABI)
against the CPU oracle on the same seeded inputs.

Bars: y within relative L2 <= 1e-4 and max-abs <= 2e-3 * max|ref|; every
cache slot other than the new token's untouched (bit for bit); the new
token's key and value rows equal to the oracle's BF16 values except where the
fp32 and fp64 values round to neighbouring BF16 values: at most one BF16 step
apart (sign-aware distance between the bit patterns), or, for values so close
to zero that fp32 rounding alone exceeds a step, within 4e-6 of the largest
magnitude of their head's row; and at most 4 such values per slot.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from bf16_checks import bf16_steps

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4
MAX_ABS = 2e-3


@pytest.fixture(scope="module")
def F():
    from nvfp4_bit_projection_amd import flint, workload
    torch.cuda.set_device(0)
    return flint, workload


def assert_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mabs = np.abs(got - ref).max()
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e}"
    assert mabs <= MAX_ABS * np.abs(ref).max(), f"{what}: max abs {mabs:.3e} vs {np.abs(ref).max():.3e}"


def oracle_layer(d, seed):
    mats = [oracle.quantize(synth.attn_f32(seed, d, k)) for k in (synth.ATTN_Q, synth.ATTN_K, synth.ATTN_V,
                                                                   synth.ATTN_O)]
    return oracle.AttnLayer(*mats, synth.attn_gain(seed, d, synth.Q_NORM), synth.attn_gain(seed, d, synth.K_NORM),
                            synth.attn_sinks(seed, d))


def dims_c(F, d):
    return F[0].attn_dims_struct(d.hidden, d.n_q, d.n_kv, d.head_dim, d.window, d.rope, d.theta)


def check_rows(g, r):
    """g, r: uint16 BF16 rows [n_kv][D] (GPU, oracle) of one written slot."""
    steps = bf16_steps(g, r)
    gv, rv = oracle.bf16_decode(g), oracle.bf16_decode(r)
    near_zero = np.abs(gv - rv) <= 4e-6 * np.abs(rv).max(axis=-1, keepdims=True)
    assert ((steps <= 1) | near_zero).all(), np.argwhere((steps > 1) & ~near_zero)[:4].tolist()
    assert (steps > 0).sum() <= 4, (steps > 0).sum()


def check_caches(gk, gv, rk, rv, slots):
    """gk/gv GPU caches (uint16 numpy [n_kv][cap][D]), rk/rv the oracle's after
    the same steps; slots: the slots written by those steps."""
    slots = np.atleast_1d(slots)
    for g, r in ((gk, rk), (gv, rv)):
        other = np.ones(g.shape[1], bool)
        other[slots] = False
        assert np.array_equal(g[:, other], r[:, other])
        for s in slots:
            check_rows(g[:, s], r[:, s])


def run_case(F, d, seed, pos, cap, tok_seed=0):
    flint, workload = F
    L = oracle_layer(d, seed)
    W = workload.build_attn(d, seed)
    assert np.array_equal(W.q.codes.cpu().numpy(), L.q.codes)
    kc = synth.kv_cache_bits(seed + 1, d, cap, synth.K_CACHE)
    vc = synth.kv_cache_bits(seed + 1, d, cap, synth.V_CACHE)
    x = synth.token_f32(tok_seed, d.hidden)
    gk = torch.from_numpy(kc.view(np.int16).copy()).cuda()
    gv = torch.from_numpy(vc.view(np.int16).copy()).cuda()
    print(f"attn case window={d.window} rope={d.rope} heads={d.n_q}/{d.n_kv} pos={pos} cap={cap}", flush=True)
    y = flint.attn_decode(dims_c(F, d), W, torch.from_numpy(x).cuda(), pos, gk, gv)
    torch.cuda.synchronize()
    y_ref, _, _ = oracle.attn_decode(L, x.astype(np.float64), pos, kc, vc, n_kv=d.n_kv, window=d.window,
                                     rope=d.rope, theta=d.theta)
    assert_close(y.cpu().numpy(), y_ref, f"y pos={pos}")
    check_caches(gk.cpu().numpy().view(np.uint16), gv.cpu().numpy().view(np.uint16), kc, vc, pos % cap)


@pytest.mark.parametrize("pos", [0, 5, 63, 64, 300, 512, 513, 2000, 100000])
def test_sliding_window_rope(F, pos):
    run_case(F, synth.SLIDING, 0, pos, 513)


@pytest.mark.parametrize("pos,cap", [(0, 64), (63, 64), (64, 128), (1000, 4096), (4095, 4096), (40000, 40001)])
def test_full_context_nope(F, pos, cap):
    run_case(F, synth.FULL, 1, pos, cap)


def test_sliding_ring_larger_than_window(F):
    run_case(F, synth.SLIDING, 2, 3000, 1024)


@pytest.mark.parametrize("n_q,n_kv", [(16, 2), (16, 4), (64, 8)])
def test_other_head_counts(F, n_q, n_kv):
    d = synth.AttnDims(n_q=n_q, n_kv=n_kv, window=0, rope=True)
    run_case(F, d, 3, 777, 1024)


def test_consecutive_tokens(F):
    """Five tokens in a row through one cache: each step reads the rows the
    previous steps wrote."""
    flint, workload = F
    d = synth.SLIDING
    L = oracle_layer(d, 4)
    W = workload.build_attn(d, 4)
    cap, p0 = 513, 1020
    kc = synth.kv_cache_bits(5, d, cap, synth.K_CACHE)
    vc = synth.kv_cache_bits(5, d, cap, synth.V_CACHE)
    gk = torch.from_numpy(kc.view(np.int16).copy()).cuda()
    gv = torch.from_numpy(vc.view(np.int16).copy()).cuda()
    ws = flint.attn_workspace(dims_c(F, d))
    for i in range(5):
        x = synth.token_f32(50 + i, d.hidden)
        y = flint.attn_decode(dims_c(F, d), W, torch.from_numpy(x).cuda(), p0 + i, gk, gv, ws=ws)
        y_ref, _, _ = oracle.attn_decode(L, x.astype(np.float64), p0 + i, kc, vc, n_kv=d.n_kv, window=d.window,
                                         rope=True, theta=d.theta)
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy(), y_ref, f"token {i}")
    # both caches: the five written slots within the bar, every other slot
    # untouched
    check_caches(gk.cpu().numpy().view(np.uint16), gv.cpu().numpy().view(np.uint16), kc, vc,
                 [(p0 + i) % cap for i in range(5)])


@pytest.mark.parametrize("width,B", [(6144, 1), (6144, 3), (2048, 2), (8192, 1)])
def test_dense_mlp(F, width, B):
    flint, workload = F
    H = 2048
    print(f"dense case width={width} B={B}", flush=True)
    g, u, dn = workload.build_dense(7, H, width)
    og, ou, od = (oracle.quantize(synth.dense_f32(7, H, width, k)) for k in (synth.DENSE_GATE, synth.DENSE_UP,
                                                                              synth.DENSE_DOWN))
    x = np.stack([synth.token_f32(60 + b, H) for b in range(B)])
    y = flint.dense_mlp(g, u, dn, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    for b in range(B):
        assert_close(y[b].cpu().numpy(), oracle.swiglu_expert(og, ou, od, x[b].astype(np.float64)), f"dense b={b}")
