"""The C-ABI library on the host: it loads, exports every symbol its header
declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("flint_moe.h", "flint_attn.h", "flint_int4.h", "flint_gemm.h",
                                                       "flint_model.h")]


@pytest.fixture(scope="module")
def F():
    from nvfp4_bit_projection_amd import build
    if not os.path.exists(build.LIB_PATH):
        build.build_library()
    from nvfp4_bit_projection_amd import flint
    return flint


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flint_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(F):
    names = declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(F.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(F.EXPORTED) == names


def test_status_strings(F):
    L = F.lib()
    for code in range(0, -9, -1):
        assert L.flint_status_str(code) and L.flint_status_str(code) != b"unknown status"
    assert L.flint_status_str(5) == b"unknown status"


def test_workspace_sizes(F):
    d = F.dims_struct()
    assert F.workspace_bytes(F.OP_ROUTE, d, 1) > 0
    assert F.workspace_bytes(F.OP_DECODE, d, 4) > F.workspace_bytes(F.OP_DECODE, d, 1)
    assert F.workspace_bytes(F.OP_LMHEAD, None, 1, 150144) > 0
    assert F.workspace_bytes(F.OP_STACK, d, 1, 150144, 47) > 0
    assert F.workspace_bytes(F.OP_QUANTIZE, None, 256) >= 1024
    assert F.workspace_bytes(F.OP_DECODE, d, 0) == 0
    assert F.workspace_bytes(99, d, 1) == 0
    bad = F.dims_struct(top_k=9)
    assert F.workspace_bytes(F.OP_DECODE, bad, 1) == 0


# Host-side validation runs before any HIP call, so these return their codes
# on a machine without a GPU.  Pointers below are fake but never dereferenced.
FAKE = 0x10000


def test_route_rejections(F):
    L = F.lib()
    d = F.dims_struct()
    r = lambda dims, router, x, B, idx, w, ws, wsb: L.flint_moe_route(
        ctypes.byref(dims) if dims is not None else None, router, x, B, idx, w, None, ws, wsb, None)
    need = F.workspace_bytes(F.OP_ROUTE, d, 1)
    assert r(None, FAKE, FAKE, 1, FAKE, FAKE, FAKE, need) == -1
    assert r(d, None, FAKE, 1, FAKE, FAKE, FAKE, need) == -1
    assert r(d, FAKE, FAKE, 0, FAKE, FAKE, FAKE, need) == -2
    assert r(F.dims_struct(top_k=0), FAKE, FAKE, 1, FAKE, FAKE, FAKE, need) == -2
    assert r(F.dims_struct(n_experts=4, top_k=6), FAKE, FAKE, 1, FAKE, FAKE, FAKE, need) == -2
    assert r(F.dims_struct(n_experts=300), FAKE, FAKE, 1, FAKE, FAKE, FAKE, need) == -2
    assert r(F.dims_struct(hidden=1024), FAKE, FAKE, 1, FAKE, FAKE, FAKE, need) == -8
    assert r(F.dims_struct(expert_width=1024, top_k=8), FAKE, FAKE, 1, FAKE, FAKE, FAKE, need) == -8
    assert r(d, FAKE + 4, FAKE, 1, FAKE, FAKE, FAKE, need) == -3
    assert r(d, FAKE, FAKE, 1, FAKE, FAKE, FAKE, need - 1) == -4


def test_route_ex_rejections(F):
    L = F.lib()
    d = F.dims_struct()
    r = lambda dt, sc, router=FAKE, wsb=None: L.flint_moe_route_ex(
        ctypes.byref(d), router, dt, sc, FAKE, 1, FAKE, FAKE, None, FAKE,
        F.workspace_bytes(F.OP_ROUTE, d, 1) if wsb is None else wsb, None)
    assert r(2, 0) == -2
    assert r(-1, 0) == -2
    assert r(0, 2) == -2
    assert r(1, -1) == -2
    assert r(1, 1, router=None) == -1
    assert r(1, 1, router=FAKE + 2) == -3
    assert r(1, 1, wsb=F.workspace_bytes(F.OP_ROUTE, d, 1) - 1) == -4


def test_decode_and_head_rejections(F):
    L = F.lib()
    d = F.dims_struct()
    lay = F.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, F.NVFP4(FAKE, FAKE, FAKE),
                  F.NVFP4(FAKE, FAKE, FAKE), F.NVFP4(FAKE, FAKE, FAKE))
    need = F.workspace_bytes(F.OP_DECODE, d, 1)
    dec = lambda layer, wsb: L.flint_moe_decode(ctypes.byref(d), ctypes.byref(layer), FAKE, 1, FAKE, None, None,
                                                FAKE, wsb, None)
    assert dec(lay, need - 1) == -4
    lay2 = F.Layer(*[getattr(lay, f) for f, _ in F.Layer._fields_])
    lay2.down_codes = None
    assert dec(lay2, need) == -1
    lay3 = F.Layer(*[getattr(lay, f) for f, _ in F.Layer._fields_])
    lay3.shared_up = F.NVFP4(FAKE + 8, FAKE, FAKE)
    assert dec(lay3, need) == -3
    head = F.NVFP4(FAKE, FAKE, FAKE)
    hneed = F.workspace_bytes(F.OP_LMHEAD, None, 1, 100)
    hd = lambda vocab, hidden, wsb: L.flint_lmhead_gemv(ctypes.byref(head), vocab, hidden, FAKE, 1, FAKE, FAKE, FAKE,
                                                        wsb, None)
    assert hd(0, 2048, hneed) == -2
    assert hd(100, 2048, hneed - 1) == -4
    assert hd(100, 1024, hneed) == -8
    assert hd(100, 2000, hneed) == -2


def test_quantize_and_stack_rejections(F):
    L = F.lib()
    q = lambda n, rows, cols, wsb: L.flint_nvfp4_quantize(FAKE, n, rows, cols, FAKE, FAKE, FAKE, FAKE, wsb, None)
    assert q(1, 4, 48, 256) == -2
    assert q(0, 4, 64, 256) == -2
    assert q(300, 4, 64, 256) == -4
    plan = F.StackPlan()
    assert L.flint_stack_decode(ctypes.byref(plan), FAKE, 1, 1e-6, None, FAKE, None, FAKE, 1 << 20, None) in (-1, -2)
    assert L.flint_stack_table_bytes(0) == 0 and L.flint_stack_table_bytes(47) > 47 * ctypes.sizeof(F.Layer)
    # repacked down projections: the routed and shared down matrices of every
    # layer (codes + scales), only for sizes the persistent schedule takes
    full = F.dims_struct()
    per_layer = 256 * 2048 * 512 // 2 + 256 * 2048 * 512 // 16 + 2048 * 1024 // 2 + 2048 * 1024 // 16
    assert L.flint_stack_packed_bytes(ctypes.byref(full), 47) == 47 * per_layer
    assert L.flint_stack_packed_bytes(ctypes.byref(full), 65) == 0      # more layers than the schedule takes
    odd = F.dims_struct(n_experts=256, expert_width=96, top_k=2, shared_width=160)
    assert L.flint_stack_packed_bytes(ctypes.byref(odd), 4) == 0
    assert L.flint_stack_packed_bytes(None, 4) == 0
    # batched step: workspace only for 1 <= B <= 64; argument checks before any work
    assert L.flint_workspace_bytes(F.OP_STACK_BATCH, ctypes.byref(full), 32, 150144, 47) > 0
    assert L.flint_workspace_bytes(F.OP_STACK_BATCH, ctypes.byref(full), 65, 150144, 47) == 0
    assert L.flint_workspace_bytes(F.OP_STACK_BATCH, ctypes.byref(full), 0, 150144, 47) == 0
    # expert and shared widths: 512, 1024 or 2048 only
    for I, Is, ok in ((1024, 2048, True), (512, 512, True), (1536, 512, False), (512, 1536, False),
                      (256, 1024, False)):
        dm = F.dims_struct(expert_width=I, shared_width=Is, top_k=2)
        assert (L.flint_workspace_bytes(F.OP_STACK_BATCH, ctypes.byref(dm), 8, 150144, 47) > 0) == ok, (I, Is)
    assert L.flint_stack_decode_batch(None, FAKE, 8, 1e-6, None, FAKE, None, FAKE, 1 << 20, None) == -1
    assert L.flint_stack_decode_batch(ctypes.byref(plan), FAKE, 8, 1e-6, None, FAKE, None, FAKE, 1 << 20, None) == -1


def test_attn_and_dense_rejections(F):
    L = F.lib()
    d = F.attn_dims_struct()
    assert L.flint_attn_workspace_bytes(ctypes.byref(d)) > 0
    assert L.flint_attn_workspace_bytes(ctypes.byref(F.attn_dims_struct(head_dim=64))) == 0
    assert L.flint_attn_workspace_bytes(ctypes.byref(F.attn_dims_struct(n_q=32, n_kv=2))) == 0  # group 16
    assert L.flint_attn_workspace_bytes(ctypes.byref(F.attn_dims_struct(n_q=24, n_kv=4))) == 0
    m = F.NVFP4(FAKE, FAKE, FAKE)
    lay = F.AttnLayer(m, m, m, m, FAKE, FAKE, FAKE)
    need = L.flint_attn_workspace_bytes(ctypes.byref(d))
    call = lambda dims, layer, pos, cap, wsb=need, x=FAKE: L.flint_attn_decode(
        ctypes.byref(dims), ctypes.byref(layer), x, pos, FAKE, FAKE, cap, FAKE, FAKE, wsb, None)
    assert call(d, lay, 0, 513, x=None) == -1
    assert call(d, lay, -1, 513) == -2
    assert call(d, lay, 0, 512) == -2                      # ring smaller than the window
    full = F.attn_dims_struct(window=0, rope=False)
    assert call(full, lay, 100, 100) == -2                 # full context needs cap > pos
    assert call(d, lay, 0, 513, wsb=need - 1) == -4
    assert call(d, lay, 0, 513, x=FAKE + 4) == -3
    assert call(F.attn_dims_struct(rope=True, theta=0.0), lay, 0, 513) == -2
    assert call(F.attn_dims_struct(head_dim=64), lay, 0, 513) == -8
    bad = F.AttnLayer(m, m, m, F.NVFP4(FAKE, None, FAKE), FAKE, FAKE, FAKE)
    assert call(d, bad, 0, 513) == -1
    # dense MLP
    assert L.flint_dense_workspace_bytes(2048, 6144, 1) > 0
    assert L.flint_dense_workspace_bytes(2048, 5000, 1) == 0
    assert L.flint_dense_workspace_bytes(2048, 6144, 65) == 0
    dn = lambda width, B, wsb: L.flint_dense_mlp(ctypes.byref(m), ctypes.byref(m), ctypes.byref(m), 2048, width,
                                                 FAKE, B, FAKE, FAKE, wsb, None)
    ok = L.flint_dense_workspace_bytes(2048, 6144, 2)
    assert dn(6144, 0, ok) == -2
    assert dn(5000, 1, ok) == -8
    assert dn(6144, 2, ok - 1) == -4


def test_int4_rejections(F):
    L = F.lib()
    assert L.flint_int4_gemv_workspace_bytes(1) > 0 and L.flint_int4_gemv_workspace_bytes(65) == 0
    q = F.INT4(FAKE, FAKE, FAKE)
    need = L.flint_int4_gemv_workspace_bytes(2)
    gv = lambda rows, cols, B, wsb=need, x=FAKE: L.flint_int4_gemv(ctypes.byref(q), rows, cols, x, B, FAKE, None,
                                                                   FAKE, wsb, None)
    assert gv(100, 2048, 2, x=None) == -1
    assert gv(0, 2048, 2) == -2
    assert gv(100, 1024, 2) == -8
    assert gv(100, 2048, 65) == -8
    assert gv(100, 2048, 2, wsb=need - 1) == -4
    assert gv(100, 2048, 2, x=FAKE + 8) == -3
    assert L.flint_int4_quantize(FAKE, 4, 100, FAKE, FAKE, FAKE, None) == -2
    assert L.flint_int4_quantize(FAKE, 4, 128, FAKE, FAKE + 1, FAKE, None) == -3
    assert L.flint_int4_quantize(None, 4, 128, FAKE, FAKE, FAKE, None) == -1


def test_gemm_rejections(F):
    L = F.lib()
    assert L.flint_nvfp4_gemm_workspace_bytes(8, 2048, 0) > 0
    # room for the layout the header gives: A4 codes from byte 512, the block
    # scales, then the fp16 planes ([2][T][K] for A32, [T][K] for A4)
    assert L.flint_nvfp4_gemm_workspace_bytes(8, 2048, 1) >= 512 + 8 * 2048 // 2 + 8 * 2048 // 16 + 8 * 2048 * 2
    assert L.flint_nvfp4_gemm_workspace_bytes(8, 2048, 0) >= 2 * 8 * 2048 * 2
    assert L.flint_nvfp4_gemm_workspace_bytes(8, 100, 0) == 0
    assert L.flint_nvfp4_gemm_workspace_bytes(8, 2048, 2) == 0
    m = F.NVFP4(FAKE, FAKE, FAKE)
    need = L.flint_nvfp4_gemm_workspace_bytes(8, 2048, 1)
    g = lambda N, K, T, mode, wsb=need, x=FAKE: L.flint_nvfp4_gemm(ctypes.byref(m), N, K, x, T, mode, FAKE, FAKE,
                                                                   wsb, None)
    assert g(10, 2048, 8, 1, x=None) == -1
    assert g(0, 2048, 8, 1) == -2
    assert g(10, 2048, 8, 3) == -2
    assert g(10, 2000, 8, 0) == -8
    assert g(10, (1 << 20) + 256, 1, 0) == -8  # K above 2^20
    assert g(10, 2048, 8, 1, wsb=need - 1) == -4
    assert g(10, 2048, 8, 1, x=FAKE + 4) == -3


def test_model_rejections(F):
    L = F.lib()
    m = F.NVFP4(FAKE, FAKE, FAKE)
    n = 3
    attn = (F.AttnLayer * n)(*[F.AttnLayer(m, m, m, m, FAKE, FAKE, FAKE) for _ in range(n)])
    is_full = (ctypes.c_int32 * n)(0, 1, 0)
    kc = (ctypes.c_void_p * n)(FAKE, FAKE, FAKE)
    cap = (ctypes.c_int32 * n)(513, 1024, 513)
    dense = (F.NVFP4 * 3)(m, m, m)
    moe = (F.Layer * 2)(*[F.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, m, m, m) for _ in range(2)])
    mc = F.ModelC(n, 1, 6144, F.dims_struct(), F.attn_dims_struct(), F.attn_dims_struct(window=0, rope=False),
                  ctypes.cast(is_full, ctypes.c_void_p), ctypes.cast(attn, ctypes.c_void_p),
                  ctypes.cast(kc, ctypes.c_void_p), ctypes.cast(kc, ctypes.c_void_p), ctypes.cast(cap, ctypes.c_void_p),
                  ctypes.cast(dense, ctypes.c_void_p), ctypes.cast(moe, ctypes.c_void_p), m, 150144, 1e-6)
    need = L.flint_model_workspace_bytes(ctypes.byref(mc))
    assert need > 0
    dec = lambda pos, wsb=need, x=FAKE: L.flint_model_decode(ctypes.byref(mc), x, pos, None, FAKE, None, FAKE, wsb,
                                                             None)
    assert dec(10, x=None) == -1
    assert dec(-1) == -2
    assert dec(2000) == -2                 # the full layer's cache holds 1024 positions
    assert dec(10, wsb=need - 1) == -4
    assert dec(10, x=FAKE + 4) == -3
    is_full[1] = 2
    assert dec(10) == -2
    is_full[1] = 1
    mc.n_dense = 4
    assert L.flint_model_workspace_bytes(ctypes.byref(mc)) == 0


def test_model_moe_plan_rejections(F):
    """The optional persistent plan of the MoE layers must match the model."""
    L = F.lib()
    m = F.NVFP4(FAKE, FAKE, FAKE)
    n = 3
    attn = (F.AttnLayer * n)(*[F.AttnLayer(m, m, m, m, FAKE, FAKE, FAKE) for _ in range(n)])
    is_full = (ctypes.c_int32 * n)(0, 1, 0)
    kc = (ctypes.c_void_p * n)(FAKE, FAKE, FAKE)
    cap = (ctypes.c_int32 * n)(513, 1024, 513)
    dense = (F.NVFP4 * 3)(m, m, m)
    moe = (F.Layer * 2)(*[F.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, m, m, m) for _ in range(2)])
    mc = F.ModelC(n, 1, 6144, F.dims_struct(), F.attn_dims_struct(), F.attn_dims_struct(window=0, rope=False),
                  ctypes.cast(is_full, ctypes.c_void_p), ctypes.cast(attn, ctypes.c_void_p),
                  ctypes.cast(kc, ctypes.c_void_p), ctypes.cast(kc, ctypes.c_void_p), ctypes.cast(cap, ctypes.c_void_p),
                  ctypes.cast(dense, ctypes.c_void_p), ctypes.cast(moe, ctypes.c_void_p), m, 150144, 1e-6)
    plain = L.flint_model_workspace_bytes(ctypes.byref(mc))
    err = ctypes.c_int32(7)
    assert L.flint_model_error(ctypes.byref(mc), FAKE, plain, ctypes.byref(err)) == 0 and err.value == 0
    plan = F.StackPlan()
    plan.dims = F.dims_struct()
    plan.n_layers = 2
    plan.vocab = 150144
    plan.table = FAKE
    plan.packed = FAKE
    mc.moe_plan = ctypes.cast(ctypes.pointer(plan), ctypes.c_void_p)
    need = L.flint_model_workspace_bytes(ctypes.byref(mc))
    assert need > plain                    # the persistent kernel's exchange area
    dec = lambda wsb=need: L.flint_model_decode(ctypes.byref(mc), FAKE, 10, None, FAKE, None, FAKE, wsb, None)
    assert dec(wsb=need - 1) == -4
    assert L.flint_model_error(ctypes.byref(mc), FAKE, need - 1, ctypes.byref(err)) == -4
    plan.n_layers = 3                      # the model has 2 MoE layers
    assert dec() == -2
    plan.n_layers = 2
    plan.dims = F.dims_struct(n_experts=128)
    assert dec() == -2
    plan.dims = F.dims_struct()
    plan.packed = None                     # no repacked down projections
    assert dec() == -1
