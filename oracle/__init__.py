"""CPU oracle for the NVFP4 sparse-MoE decode step (Python side).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg import this package; the product package
never does, and the oracle imports nothing from it.  The arithmetic lives in
``oracle.c`` (double precision, plain loops); this file only marshals numpy
arrays through ctypes.  ``oracle/model.py`` composes the steps into a layer, a
stack and the head.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import NamedTuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "oracle.c")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB_PATH):
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", SRC_PATH, "-o", LIB_PATH, "-lm", "-lpthread"], check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_int]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e2m1_encode.argtypes = [ctypes.c_double]
        L.oracle_e2m1_encode.restype = ctypes.c_int
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_encode.restype = ctypes.c_int
        L.oracle_nvfp4_quantize.argtypes = [_P, _I64, _I64, _P, _P, _P, ctypes.c_int]
        L.oracle_nvfp4_quantize.restype = None
        L.oracle_nvfp4_dequantize.argtypes = [_P, _P, ctypes.c_float, _I64, _I64, _P]
        L.oracle_nvfp4_dequantize.restype = None
        L.oracle_nvfp4_gemv.argtypes = [_P, _P, ctypes.c_float, _I64, _I64, _P, _P, ctypes.c_int]
        L.oracle_nvfp4_gemv.restype = None
        L.oracle_f32_gemv.argtypes = [_P, _I64, _I64, _P, _P, ctypes.c_int]
        L.oracle_f32_gemv.restype = None
        L.oracle_topk_softmax.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P, _P]
        L.oracle_topk_softmax.restype = None
        L.oracle_topk_sigmoid.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P, _P]
        L.oracle_topk_sigmoid.restype = None
        L.oracle_bf16_decode.argtypes = [_P, _I64, _P]
        L.oracle_bf16_decode.restype = None
        L.oracle_bf16_encode.argtypes = [ctypes.c_double]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [_P, _I64, _P]
        L.oracle_bf16_round.restype = None
        L.oracle_head_rmsnorm.argtypes = [_P, ctypes.c_int, _P, ctypes.c_double]
        L.oracle_head_rmsnorm.restype = None
        L.oracle_rope.argtypes = [_P, ctypes.c_int, _I64, ctypes.c_double]
        L.oracle_rope.restype = None
        L.oracle_attn_decode.argtypes = ([ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_double] + [_P] * 7
                                         + [_I64, _P, _P, _I64, _P, _P, _P, ctypes.c_int])
        L.oracle_attn_decode.restype = ctypes.c_int
        L.oracle_int4_quantize.argtypes = [_P, _I64, _I64, _P, _P, _P]
        L.oracle_int4_quantize.restype = None
        L.oracle_int4_dequantize.argtypes = [_P, _P, _P, _I64, _I64, _P]
        L.oracle_int4_dequantize.restype = None
        L.oracle_int4_gemv.argtypes = [_P, _P, _P, _I64, _I64, _P, _P, ctypes.c_int]
        L.oracle_int4_gemv.restype = None
        L.oracle_nvfp4_gemm.argtypes = [_P, _P, ctypes.c_float, _I64, _I64, _P, _I64, _P, ctypes.c_int]
        L.oracle_nvfp4_gemm.restype = None
        L.oracle_nvfp4_gemm_a4.argtypes = [_P, _P, ctypes.c_float, _I64, _I64, _P, _I64, _P, ctypes.c_int]
        L.oracle_nvfp4_gemm_a4.restype = None
        L.oracle_rms_inv.argtypes = [_P, _I64, ctypes.c_double]
        L.oracle_rms_inv.restype = ctypes.c_double
        L.oracle_swiglu_expert.argtypes = [_P, _P, ctypes.c_float, _P, _P, ctypes.c_float, _P, _P, ctypes.c_float,
                                           _I64, _I64, _P, _P, _P, ctypes.c_int]
        L.oracle_swiglu_expert.restype = None
        L.oracle_argmax.argtypes = [_P, _I64, _P]
        L.oracle_argmax.restype = _I64
        _lib = L
    return _lib


def default_threads() -> int:
    env = os.environ.get("ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


class NVFP4(NamedTuple):
    """An NVFP4 matrix in the interchange layout: codes [rows][cols/2] (element
    2j in the low nibble of byte j), E4M3 scales [rows][cols/16], fp32 S."""
    codes: np.ndarray
    scales: np.ndarray
    tscale: float
    rows: int
    cols: int


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------- codec --
def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def e2m1_encode(v: float) -> int:
    return lib().oracle_e2m1_encode(v)


def e4m3_encode(r: float) -> int:
    return lib().oracle_e4m3_encode(r)


def quantize(w: np.ndarray, nthreads: int | None = None) -> NVFP4:
    w = _c(w, np.float32)
    rows, cols = w.shape
    assert cols % 16 == 0
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    S = np.zeros(1, np.float32)
    lib().oracle_nvfp4_quantize(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data, S.ctypes.data,
                                nthreads or default_threads())
    return NVFP4(codes, scales, float(S[0]), rows, cols)


def dequantize(q: NVFP4) -> np.ndarray:
    out = np.empty((q.rows, q.cols), np.float32)
    codes, scales = _c(q.codes, np.uint8), _c(q.scales, np.uint8)
    lib().oracle_nvfp4_dequantize(codes.ctypes.data, scales.ctypes.data, q.tscale, q.rows, q.cols, out.ctypes.data)
    return out


# ---------------------------------------------------------------- products --
def nvfp4_gemv(q: NVFP4, x: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    x = _c(x, np.float64)
    assert x.shape == (q.cols,)
    y = np.empty(q.rows, np.float64)
    codes, scales = _c(q.codes, np.uint8), _c(q.scales, np.uint8)
    lib().oracle_nvfp4_gemv(codes.ctypes.data, scales.ctypes.data, q.tscale, q.rows, q.cols, x.ctypes.data,
                            y.ctypes.data, nthreads or default_threads())
    return y


def f32_gemv(w: np.ndarray, x: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    w = _c(w, np.float32)
    x = _c(x, np.float64)
    rows, cols = w.shape
    assert x.shape == (cols,)
    y = np.empty(rows, np.float64)
    lib().oracle_f32_gemv(w.ctypes.data, rows, cols, x.ctypes.data, y.ctypes.data, nthreads or default_threads())
    return y


def topk_softmax(logits: np.ndarray, k: int):
    """-> (idx int32[k] ordered by (logit desc, index asc), w float64[k], gap)"""
    logits = _c(logits, np.float64)
    idx = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    gap = np.zeros(1, np.float64)
    lib().oracle_topk_softmax(logits.ctypes.data, logits.size, k, idx.ctypes.data, w.ctypes.data, gap.ctypes.data)
    return idx, w, float(gap[0])


def topk_sigmoid(logits: np.ndarray, k: int):
    """-> (idx int32[k] ordered by (score desc, index asc), w float64[k], gap)"""
    logits = _c(logits, np.float64)
    idx = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    gap = np.zeros(1, np.float64)
    lib().oracle_topk_sigmoid(logits.ctypes.data, logits.size, k, idx.ctypes.data, w.ctypes.data, gap.ctypes.data)
    return idx, w, float(gap[0])


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 BF16 bit patterns -> float64 values (same shape)"""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().oracle_bf16_decode(bits.ctypes.data, bits.size, out.ctypes.data)
    return out


def rms_inv(h: np.ndarray, eps: float) -> float:
    h = _c(h, np.float64)
    return lib().oracle_rms_inv(h.ctypes.data, h.size, eps)


def swiglu_expert(gate: NVFP4, up: NVFP4, down: NVFP4, u: np.ndarray, nthreads: int | None = None,
                  return_hidden: bool = False):
    H, I = gate.cols, gate.rows
    assert up.rows == I and up.cols == H and down.rows == H and down.cols == I
    u = _c(u, np.float64)
    y = np.empty(H, np.float64)
    h = np.empty(I, np.float64)
    args, keep = [], []
    for q in (gate, up, down):
        codes, scales = _c(q.codes, np.uint8), _c(q.scales, np.uint8)
        keep += [codes, scales]
        args += [codes.ctypes.data, scales.ctypes.data, q.tscale]
    lib().oracle_swiglu_expert(*args, H, I, u.ctypes.data, y.ctypes.data, h.ctypes.data, nthreads or default_threads())
    return (y, h) if return_hidden else y


def argmax(v: np.ndarray):
    """-> (first index of the maximum, max minus second largest)"""
    v = _c(v, np.float64)
    gap = np.zeros(1, np.float64)
    i = lib().oracle_argmax(v.ctypes.data, v.size, gap.ctypes.data)
    return int(i), float(gap[0])


# --------------------------------------------------------------- attention --
def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 values -> uint16 BF16 bit patterns (nearest, ties to even)"""
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_round(x.ctypes.data, x.size, out.ctypes.data)
    return out


def head_rmsnorm(v: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    v = np.array(v, np.float64)
    g = _c(gain, np.float32)
    assert g.shape == v.shape
    lib().oracle_head_rmsnorm(v.ctypes.data, v.size, g.ctypes.data, eps)
    return v


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    v = np.array(v, np.float64)
    lib().oracle_rope(v.ctypes.data, v.size, pos, theta)
    return v


class AttnLayer(NamedTuple):
    """One attention layer: NVFP4 q [Hq*D][H], k and v [Hkv*D][H], o [H][Hq*D];
    fp32 gains q_norm, k_norm [D]; fp32 sinks [Hq]."""
    q: NVFP4
    k: NVFP4
    v: NVFP4
    o: NVFP4
    q_norm: np.ndarray
    k_norm: np.ndarray
    sinks: np.ndarray


def attn_decode(L: AttnLayer, x: np.ndarray, pos: int, k_cache: np.ndarray, v_cache: np.ndarray, *, n_kv: int,
                window: int, rope: bool, theta: float = 10000.0, eps: float = 1e-6,
                nthreads: int | None = None):
    """One new token at `pos`.  k_cache / v_cache uint16 [Hkv][cap][D] are
    updated in place.  -> (y float64[H], o float64[Hq*D], qkv float64[...])"""
    D = L.q_norm.size
    Hq, H = L.q.rows // D, L.q.cols
    cap = k_cache.shape[1]
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16 and k_cache.shape == (n_kv, cap, D)
    x = _c(x, np.float64)
    keep = []
    cp, sp = (_P * 4)(), (_P * 4)()
    ts = np.array([m.tscale for m in (L.q, L.k, L.v, L.o)], np.float32)
    for i, m in enumerate((L.q, L.k, L.v, L.o)):
        c, s = _c(m.codes, np.uint8), _c(m.scales, np.uint8)
        keep += [c, s]
        cp[i], sp[i] = c.ctypes.data, s.ctypes.data
    qn, kn, sk = _c(L.q_norm, np.float32), _c(L.k_norm, np.float32), _c(L.sinks, np.float32)
    y = np.empty(H, np.float64)
    o = np.empty(Hq * D, np.float64)
    qkv = np.empty(Hq * D + 2 * n_kv * D, np.float64)
    rc = lib().oracle_attn_decode(H, Hq, n_kv, D, window, int(rope), theta, eps, cp, sp, ts.ctypes.data,
                                  qn.ctypes.data, kn.ctypes.data, sk.ctypes.data, x.ctypes.data, pos,
                                  k_cache.ctypes.data, v_cache.ctypes.data, cap, y.ctypes.data, o.ctypes.data,
                                  qkv.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise ValueError("attn_decode: cache too small for the window or position")
    return y, o, qkv


# ------------------------------------------------------ INT4 affine codec --
class INT4(NamedTuple):
    """Group-64 affine INT4: codes uint8 [rows][cols/2] (element 2j in the low
    nibble of byte j), BF16 scales and offsets uint16 [rows][cols/64]."""
    codes: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    rows: int
    cols: int


def int4_quantize(w: np.ndarray) -> INT4:
    w = _c(w, np.float32)
    rows, cols = w.shape
    assert cols % 64 == 0
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 64), np.uint16)
    biases = np.empty((rows, cols // 64), np.uint16)
    lib().oracle_int4_quantize(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data, biases.ctypes.data)
    return INT4(codes, scales, biases, rows, cols)


def int4_dequantize(q: INT4) -> np.ndarray:
    out = np.empty((q.rows, q.cols), np.float32)
    c, s, b = _c(q.codes, np.uint8), _c(q.scales, np.uint16), _c(q.biases, np.uint16)
    lib().oracle_int4_dequantize(c.ctypes.data, s.ctypes.data, b.ctypes.data, q.rows, q.cols, out.ctypes.data)
    return out


def int4_gemv(q: INT4, x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float64)
    assert x.shape == (q.cols,)
    y = np.empty(q.rows, np.float64)
    c, s, b = _c(q.codes, np.uint8), _c(q.scales, np.uint16), _c(q.biases, np.uint16)
    lib().oracle_int4_gemv(c.ctypes.data, s.ctypes.data, b.ctypes.data, q.rows, q.cols, x.ctypes.data,
                           y.ctypes.data, 1)
    return y


# ------------------------------------------------------------ prefill GEMM --
def nvfp4_gemm(q: NVFP4, X: np.ndarray, a4: bool = False, nthreads: int | None = None) -> np.ndarray:
    """X [T][K] -> Y float64 [T][N] = X deq(W)^T; with a4 the activations are
    first quantised to NVFP4 (one tensor scale over X)."""
    T, K = X.shape
    assert K == q.cols
    Y = np.empty((T, q.rows), np.float64)
    codes, scales = _c(q.codes, np.uint8), _c(q.scales, np.uint8)
    if a4:
        Xf = _c(X, np.float32)
        lib().oracle_nvfp4_gemm_a4(codes.ctypes.data, scales.ctypes.data, q.tscale, q.rows, q.cols, Xf.ctypes.data,
                                   T, Y.ctypes.data, nthreads or default_threads())
    else:
        Xd = _c(X, np.float64)
        lib().oracle_nvfp4_gemm(codes.ctypes.data, scales.ctypes.data, q.tscale, q.rows, q.cols, Xd.ctypes.data, T,
                                Y.ctypes.data, nthreads or default_threads())
    return Y
