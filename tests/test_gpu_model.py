"""GPU parity of the whole decode step (flint_model_decode through the C ABI)
against the oracle's composition: a small model (a dense layer, then MoE
layers of 32 experts; sliding and full attention layers alternating) over a
few consecutive tokens sharing the caches, with the MoE layers as the kernel
sequence and as the persistent kernel (one layer per launch).  Logits within
relative L2 <= 1e-4 and max-abs <= 2e-3 * max|ref|, argmax exact, the written
cache rows within that bar plus one BF16 rounding step; token seeds whose
oracle routing or head margin is below 1e-5 are skipped."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.model import SyntheticWeights, model_token

pytestmark = pytest.mark.gpu

MARGIN = 1e-5


@pytest.fixture(scope="module")
def F():
    from nvfp4_bit_projection_amd import flint, workload
    torch.cuda.set_device(0)
    return flint, workload


def attn_oracle(seed, d):
    mats = [oracle.quantize(synth.attn_f32(seed, d, k)) for k in (synth.ATTN_Q, synth.ATTN_K, synth.ATTN_V,
                                                                   synth.ATTN_O)]
    return oracle.AttnLayer(*mats, synth.attn_gain(seed, d, synth.Q_NORM), synth.attn_gain(seed, d, synth.K_NORM),
                            synth.attn_sinks(seed, d))


@pytest.mark.parametrize("persistent_moe,pos0,window,cap_full",
                         [(False, 30, 8, 64), (True, 30, 8, 64), (True, 700, 513, 1024)])
def test_small_model_consecutive_tokens(F, persistent_moe, pos0, window, cap_full):
    """persistent_moe: the MoE layers as one launch each of the persistent
    stack kernel (no head); otherwise as the kernel sequence.  pos0 = 700:
    contexts of several 64-position chunks (513 and 701..703 positions: 9
    and 11 chunks per key/value head, merged with the sinks)."""
    flint, workload = F
    H, V, DW = 2048, 4096, 2048
    md = synth.MoEDims(n_experts=32)
    sliding = synth.AttnDims(window=window, rope=True)
    full = synth.AttnDims(window=0, rope=False)
    is_full = [0, 1, 0, 1]
    dims = [full if f else sliding for f in is_full]
    caps = [cap_full if f else window for f in is_full]
    nl, nd = 4, 1
    moe_seeds = [0, 1, 2]
    # oracle side
    W = SyntheticWeights(md, vocab=V)
    attn_o = [attn_oracle(100 + l, dims[l]) for l in range(nl)]
    dense_o = [tuple(oracle.quantize(synth.dense_f32(200, H, DW, k)) for k in (synth.DENSE_GATE, synth.DENSE_UP,
                                                                               synth.DENSE_DOWN))]
    kc = [synth.kv_cache_bits(300 + l, dims[l], caps[l], synth.K_CACHE) for l in range(nl)]
    vc = [synth.kv_cache_bits(300 + l, dims[l], caps[l], synth.V_CACHE) for l in range(nl)]
    # device side, same seeds
    attn_g = [workload.build_attn(dims[l], 100 + l) for l in range(nl)]
    dense_g = [workload.build_dense(200, H, DW)]
    moe_g = [workload.build_layer(md, seed=s) for s in moe_seeds]
    head = workload.build_head(V, H)
    kg = [torch.from_numpy(c.view(np.int16).copy()).cuda() for c in kc]
    vg = [torch.from_numpy(c.view(np.int16).copy()).cuda() for c in vc]
    ad = lambda d: flint.attn_dims_struct(H, d.n_q, d.n_kv, d.head_dim, d.window, d.rope, d.theta)
    M = flint.Model(flint.dims_struct(md.hidden, md.n_experts, md.expert_width, md.top_k, md.shared_width),
                    ad(sliding), ad(full), attn_g, is_full, kg, vg, dense_g, moe_g, head, V, dense_width=DW,
                    persistent_moe=persistent_moe)
    pos, seed, done = pos0, 40, 0
    while done < 3:
        x = synth.token_f32(seed, H)
        trial_k, trial_v = [c.copy() for c in kc], [c.copy() for c in vc]
        r = model_token(W, attn_o, dims, dense_o, moe_seeds, W.head(), x, pos, trial_k, trial_v)
        seed += 1
        if min(r.gaps) < MARGIN or r.argmax_gap < MARGIN:
            continue  # a near tie: another token
        print(f"model token pos={pos} seed={seed - 1} persistent_moe={persistent_moe}", flush=True)
        lg, am = M.decode(torch.from_numpy(x).cuda(), pos)
        torch.cuda.synchronize()
        got = lg.cpu().numpy().astype(np.float64)
        rel = np.linalg.norm(got - r.logits) / np.linalg.norm(r.logits)
        assert rel <= 1e-4, rel
        assert np.abs(got - r.logits).max() <= 2e-3 * np.abs(r.logits).max()
        assert int(am[0]) == r.argmax
        kc, vc = trial_k, trial_v
        for l in range(nl):  # caches: the written slots within BF16 rounding, the rest untouched
            for g_, o_ in ((kg[l], kc[l]), (vg[l], vc[l])):
                gb = g_.cpu().numpy().view(np.uint16)
                written = np.zeros(o_.shape[1], bool)
                written[[p_ % o_.shape[1] for p_ in range(pos0, pos + 1)]] = True
                assert np.array_equal(gb[:, ~written], o_[:, ~written])
                # the written values: the fp32 bar (max-abs <= 2e-3 * max|ref|
                # per written row) plus one BF16 rounding step
                gv, ov = oracle.bf16_decode(gb[:, written]), oracle.bf16_decode(o_[:, written])
                scale = np.abs(ov).max(axis=2, keepdims=True)
                bad = np.abs(gv - ov) > 2.0 ** -7 * np.abs(ov) + 2e-3 * scale
                assert not bad.any(), (l, pos, np.argwhere(bad)[:4].tolist(), gv[bad][:4], ov[bad][:4])
        pos += 1
        done += 1
    assert M.error() == 0
