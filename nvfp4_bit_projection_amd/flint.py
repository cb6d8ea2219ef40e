"""Thin Python binding of the C ABI in ``include/flint_moe.h``.

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the HIP kernels of
``libflint_moe.so``.  The library must have been built (``__graft_entry__.build()``
or ``nvfp4_bit_projection_amd.build.build_library()``); importing this module
without it raises, and there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from .build import LIB_PATH

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

OP_ROUTE, OP_DECODE, OP_LMHEAD, OP_STACK, OP_QUANTIZE, OP_STACK_BATCH = 1, 2, 3, 4, 5, 6


class FlintError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({_lib.flint_status_str(status).decode()}), "
                         f"hip error {_lib.flint_last_hip_error()}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("hidden", _I32), ("n_experts", _I32), ("expert_width", _I32), ("top_k", _I32),
                ("shared_width", _I32)]


class NVFP4(ctypes.Structure):
    _fields_ = [("codes", _P), ("scales", _P), ("tscale", _P)]


class Layer(ctypes.Structure):
    _fields_ = [("router", _P), ("gate_codes", _P), ("gate_scales", _P), ("up_codes", _P), ("up_scales", _P),
                ("down_codes", _P), ("down_scales", _P), ("expert_tscales", _P), ("shared_gate", NVFP4),
                ("shared_up", NVFP4), ("shared_down", NVFP4)]


class StackPlan(ctypes.Structure):
    _fields_ = [("dims", Dims), ("n_layers", _I32), ("vocab", _I32), ("head", NVFP4), ("layers", _P),
                ("table", _P), ("schedule", _I32), ("packed", _P)]


class AttnDims(ctypes.Structure):
    _fields_ = [("hidden", _I32), ("n_q_heads", _I32), ("n_kv_heads", _I32), ("head_dim", _I32), ("window", _I32),
                ("rope", _I32), ("rope_theta", ctypes.c_float), ("eps", ctypes.c_float)]


class AttnLayer(ctypes.Structure):
    _fields_ = [("q", NVFP4), ("k", NVFP4), ("v", NVFP4), ("o", NVFP4), ("q_norm", _P), ("k_norm", _P),
                ("sinks", _P)]


class ModelC(ctypes.Structure):
    _fields_ = [("n_layers", _I32), ("n_dense", _I32), ("dense_width", _I32), ("moe", Dims), ("sliding", AttnDims),
                ("full", AttnDims), ("is_full", _P), ("attn", _P), ("k_cache", _P), ("v_cache", _P), ("cap", _P),
                ("dense", _P), ("moe_layers", _P), ("head", NVFP4), ("vocab", _I32), ("eps", ctypes.c_float),
                ("moe_plan", _P)]


class INT4(ctypes.Structure):
    _fields_ = [("codes", _P), ("scales", _P), ("biases", _P)]


TRACE_POINTS = 32  # stamps per layer of flint_stack_decode_traced
SCHEDULE_AUTO, SCHEDULE_KERNELS, SCHEDULE_PERSISTENT = 0, 1, 2


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    sigs = {
        "flint_status_str": ([_I32], ctypes.c_char_p),
        "flint_last_hip_error": ([], _I32),
        "flint_workspace_bytes": ([_I32, ctypes.POINTER(Dims), _I32, _I32, _I32], _SZ),
        "flint_moe_route": ([ctypes.POINTER(Dims), _P, _P, _I32, _P, _P, _P, _P, _SZ, _P], _I32),
        "flint_moe_route_ex": ([ctypes.POINTER(Dims), _P, _I32, _I32, _P, _I32, _P, _P, _P, _P, _SZ, _P], _I32),
        "flint_moe_decode": ([ctypes.POINTER(Dims), ctypes.POINTER(Layer), _P, _I32, _P, _P, _P, _P, _SZ, _P], _I32),
        "flint_lmhead_gemv": ([ctypes.POINTER(NVFP4), _I32, _I32, _P, _I32, _P, _P, _P, _SZ, _P], _I32),
        "flint_moe_decode_noalloc": ([ctypes.POINTER(Dims), ctypes.POINTER(Layer), _P, _I32, _P, _P, _P, _P], _I32),
        "flint_stack_table_bytes": ([_I32], _SZ),
        "flint_stack_packed_bytes": ([ctypes.POINTER(Dims), _I32], _SZ),
        "flint_stack_prepare": ([ctypes.POINTER(Dims), ctypes.POINTER(Layer), _I32, ctypes.POINTER(NVFP4), _I32, _P,
                                 _SZ, _P, _SZ, ctypes.POINTER(StackPlan), _P], _I32),
        "flint_stack_decode": ([ctypes.POINTER(StackPlan), _P, _I32, ctypes.c_float, _P, _P, _P, _P, _SZ, _P], _I32),
        "flint_stack_decode_traced": ([ctypes.POINTER(StackPlan), _P, _I32, ctypes.c_float, _P, _P, _P, _P, _SZ, _P,
                                       _P], _I32),
        "flint_stack_decode_batch": ([ctypes.POINTER(StackPlan), _P, _I32, ctypes.c_float, _P, _P, _P, _P, _SZ, _P],
                                     _I32),
        "flint_stack_decode_layers": ([ctypes.POINTER(StackPlan), _I32, _I32, _P, ctypes.c_float, _P, _P, _P, _SZ,
                                       _P], _I32),
        "flint_stack_decode_stress": ([ctypes.POINTER(StackPlan), _P, _I32, ctypes.c_float, _P, _P, _P, _P, _SZ,
                                       ctypes.c_uint32, ctypes.c_uint32, _P], _I32),
        "flint_stack_error": ([_P, _SZ, ctypes.POINTER(_I32)], _I32),
        "flint_stack_batch_tiles_bytes": ([ctypes.POINTER(Dims), _I32], _SZ),
        "flint_stack_batch_tiles": ([ctypes.POINTER(StackPlan), _P, _SZ, _P], _I32),
        "flint_stack_decode_batch_tiled": ([ctypes.POINTER(StackPlan), _P, _P, _I32, ctypes.c_float, _P, _P, _P, _P,
                                            _SZ, _P], _I32),
        "flint_nvfp4_quantize": ([_P, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P], _I32),
        "flint_nvfp4_dequantize": ([ctypes.POINTER(NVFP4), _I64, _I64, _P, _P], _I32),
        "flint_nvfp4_quantize_host": ([_P, _I64, _I64, _P, _P, _P], _I32),
        "flint_stream_read": ([_P, _SZ, _P, _P], _I32),
        "flint_attn_workspace_bytes": ([ctypes.POINTER(AttnDims)], _SZ),
        "flint_attn_decode": ([ctypes.POINTER(AttnDims), ctypes.POINTER(AttnLayer), _P, _I32, _P, _P, _I32, _P, _P,
                               _SZ, _P], _I32),
        "flint_dense_workspace_bytes": ([_I32, _I32, _I32], _SZ),
        "flint_model_workspace_bytes": ([ctypes.POINTER(ModelC)], _SZ),
        "flint_model_decode": ([ctypes.POINTER(ModelC), _P, _I32, _P, _P, _P, _P, _SZ, _P], _I32),
        "flint_model_error": ([ctypes.POINTER(ModelC), _P, _SZ, ctypes.POINTER(_I32)], _I32),
        "flint_nvfp4_gemm_workspace_bytes": ([_I32, _I32, _I32], _SZ),
        "flint_nvfp4_gemm": ([ctypes.POINTER(NVFP4), _I32, _I32, _P, _I32, _I32, _P, _P, _SZ, _P], _I32),
        "flint_int4_quantize": ([_P, _I64, _I64, _P, _P, _P, _P], _I32),
        "flint_int4_dequantize": ([ctypes.POINTER(INT4), _I64, _I64, _P, _P], _I32),
        "flint_int4_gemv_workspace_bytes": ([_I32], _SZ),
        "flint_int4_gemv": ([ctypes.POINTER(INT4), _I32, _I32, _P, _I32, _P, _P, _P, _SZ, _P], _I32),
        "flint_dense_mlp": ([ctypes.POINTER(NVFP4), ctypes.POINTER(NVFP4), ctypes.POINTER(NVFP4), _I32, _I32, _P,
                             _I32, _P, _P, _SZ, _P], _I32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


_lib = _load()

# every symbol include/flint_moe.h declares
EXPORTED = ("flint_status_str", "flint_last_hip_error", "flint_workspace_bytes", "flint_moe_route",
            "flint_moe_route_ex",
            "flint_moe_decode", "flint_moe_decode_noalloc", "flint_lmhead_gemv", "flint_stack_table_bytes", "flint_stack_packed_bytes",
            "flint_stack_prepare",
            "flint_stack_decode", "flint_stack_decode_traced", "flint_stack_decode_batch", "flint_stack_error",
            "flint_stack_decode_layers", "flint_stack_decode_stress",
            "flint_stack_batch_tiles_bytes", "flint_stack_batch_tiles", "flint_stack_decode_batch_tiled",
            "flint_nvfp4_quantize", "flint_nvfp4_dequantize", "flint_nvfp4_quantize_host", "flint_stream_read",
            # include/flint_attn.h
            "flint_attn_workspace_bytes", "flint_attn_decode", "flint_dense_workspace_bytes", "flint_dense_mlp",
            # include/flint_int4.h
            "flint_int4_quantize", "flint_int4_dequantize", "flint_int4_gemv_workspace_bytes", "flint_int4_gemv",
            # include/flint_gemm.h
            "flint_nvfp4_gemm_workspace_bytes", "flint_nvfp4_gemm",
            # include/flint_model.h
            "flint_model_workspace_bytes", "flint_model_decode", "flint_model_error")


def lib():
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise FlintError(status, what)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def dims_struct(hidden=2048, n_experts=256, expert_width=512, top_k=6, shared_width=1024) -> Dims:
    return Dims(hidden, n_experts, expert_width, top_k, shared_width)


def workspace_bytes(op: int, dims: Dims | None, B: int = 1, vocab: int = 0, L: int = 0) -> int:
    return _lib.flint_workspace_bytes(op, ctypes.byref(dims) if dims is not None else None, B, vocab, L)


def workspace(op: int, dims: Dims | None, B: int = 1, vocab: int = 0, L: int = 0, device="cuda") -> torch.Tensor:
    n = workspace_bytes(op, dims, B, vocab, L)
    if n == 0:
        raise ValueError("invalid workspace request")
    return torch.zeros(n, dtype=torch.uint8, device=device)


# ------------------------------------------------------------ weight holders --
@dataclass
class NVFP4Tensor:
    """codes uint8 [..., rows, cols/2], scales uint8 [..., rows, cols/16], tscale float32 [...]."""
    codes: torch.Tensor
    scales: torch.Tensor
    tscale: torch.Tensor

    def c(self, index: int | None = None) -> NVFP4:
        if index is None:
            return NVFP4(self.codes.data_ptr(), self.scales.data_ptr(), self.tscale.data_ptr())
        return NVFP4(self.codes[index].data_ptr(), self.scales[index].data_ptr(), self.tscale[index].data_ptr())


@dataclass
class LayerWeights:
    router: torch.Tensor          # float32 [E][H]
    gate_codes: torch.Tensor      # uint8 [E][I][H/2]
    gate_scales: torch.Tensor     # uint8 [E][I][H/16]
    up_codes: torch.Tensor
    up_scales: torch.Tensor
    down_codes: torch.Tensor      # uint8 [E][H][I/2]
    down_scales: torch.Tensor     # uint8 [E][H][I/16]
    expert_tscales: torch.Tensor  # float32 [E][3]
    shared_gate: NVFP4Tensor
    shared_up: NVFP4Tensor
    shared_down: NVFP4Tensor

    def c(self) -> Layer:
        return Layer(self.router.data_ptr(), self.gate_codes.data_ptr(), self.gate_scales.data_ptr(),
                     self.up_codes.data_ptr(), self.up_scales.data_ptr(), self.down_codes.data_ptr(),
                     self.down_scales.data_ptr(), self.expert_tscales.data_ptr(), self.shared_gate.c(),
                     self.shared_up.c(), self.shared_down.c())


# --------------------------------------------------------------- operations --
def quantize(w: torch.Tensor) -> NVFP4Tensor:
    """w float32 cuda [n_mats, rows, cols] (or [rows, cols]) -> NVFP4 per matrix."""
    squeeze = w.dim() == 2
    if squeeze:
        w = w.unsqueeze(0)
    n, rows, cols = w.shape
    w = w.contiguous()
    codes = torch.empty((n, rows, cols // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, rows, cols // 16), dtype=torch.uint8, device=w.device)
    ts = torch.empty(n, dtype=torch.float32, device=w.device)
    ws = workspace(OP_QUANTIZE, None, B=n, device=w.device)
    _check(_lib.flint_nvfp4_quantize(w.data_ptr(), n, rows, cols, codes.data_ptr(), scales.data_ptr(),
                                     ts.data_ptr(), ws.data_ptr(), ws.numel(), _stream()), "flint_nvfp4_quantize")
    if squeeze:
        return NVFP4Tensor(codes[0], scales[0], ts[:1])
    return NVFP4Tensor(codes, scales, ts)


def stream_read(buf: torch.Tensor, out: torch.Tensor) -> None:
    """One streaming read of buf (a device tensor, byte size a multiple of 16);
    out: a device int32/uint32 tensor of at least one element."""
    _check(_lib.flint_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(), _stream()),
           "flint_stream_read")


def quantize_host(w):
    """w float32 numpy [rows, cols] (host) -> (codes uint8 [rows, cols/2],
    scales uint8 [rows, cols/16], tscale float32) by the library's host
    encoder; no GPU involved."""
    import numpy as np
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 16), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    _check(_lib.flint_nvfp4_quantize_host(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data,
                                          ts.ctypes.data), "flint_nvfp4_quantize_host")
    return codes, scales, ts[0]


def quantize_into(w: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, tscales: torch.Tensor,
                  ws: torch.Tensor) -> None:
    """In-place variant: w [n, rows, cols] into preallocated outputs (views allowed if contiguous)."""
    n, rows, cols = w.shape
    _check(_lib.flint_nvfp4_quantize(w.data_ptr(), n, rows, cols, codes.data_ptr(), scales.data_ptr(),
                                     tscales.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
           "flint_nvfp4_quantize")


def dequantize(q: NVFP4Tensor, rows: int, cols: int, index: int | None = None) -> torch.Tensor:
    out = torch.empty((rows, cols), dtype=torch.float32, device=q.codes.device)
    s = q.c(index)
    _check(_lib.flint_nvfp4_dequantize(ctypes.byref(s), rows, cols, out.data_ptr(), _stream()),
           "flint_nvfp4_dequantize")
    return out


def route(dims: Dims, router: torch.Tensor, x: torch.Tensor, ws: torch.Tensor | None = None):
    """x float32 [B][H] -> (idx int32 [B][k], w float32 [B][k], logits float32 [B][E])"""
    B = x.shape[0]
    idx = torch.empty((B, dims.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((B, dims.top_k), dtype=torch.float32, device=x.device)
    logits = torch.empty((B, dims.n_experts), dtype=torch.float32, device=x.device)
    ws = workspace(OP_ROUTE, dims, B) if ws is None else ws
    _check(_lib.flint_moe_route(ctypes.byref(dims), router.data_ptr(), x.data_ptr(), B, idx.data_ptr(), w.data_ptr(),
                                logits.data_ptr(), ws.data_ptr(), ws.numel(), _stream()), "flint_moe_route")
    return idx, w, logits


ROUTER_F32, ROUTER_BF16 = 0, 1
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1


def route_ex(dims: Dims, router: torch.Tensor, x: torch.Tensor, scoring: int = SCORE_SOFTMAX,
             ws: torch.Tensor | None = None):
    """Router variants.  router float32 [E][H], or int16/uint16 [E][H] BF16 bit
    patterns (or a torch.bfloat16 tensor); x float32 [B][H] ->
    (idx int32 [B][k], w float32 [B][k], logits float32 [B][E])"""
    if router.dtype == torch.float32:
        dtype = ROUTER_F32
    elif router.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        dtype = ROUTER_BF16
    else:
        raise TypeError(f"router dtype {router.dtype} is not float32 or BF16")
    B = x.shape[0]
    idx = torch.empty((B, dims.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((B, dims.top_k), dtype=torch.float32, device=x.device)
    logits = torch.empty((B, dims.n_experts), dtype=torch.float32, device=x.device)
    ws = workspace(OP_ROUTE, dims, B) if ws is None else ws
    _check(_lib.flint_moe_route_ex(ctypes.byref(dims), router.data_ptr(), dtype, scoring, x.data_ptr(), B,
                                   idx.data_ptr(), w.data_ptr(), logits.data_ptr(), ws.data_ptr(), ws.numel(),
                                   _stream()), "flint_moe_route_ex")
    return idx, w, logits


def moe_decode(dims: Dims, layer: LayerWeights, x: torch.Tensor, ws: torch.Tensor | None = None):
    """x float32 [B][H] -> (y float32 [B][H], idx [B][k], w [B][k])"""
    B = x.shape[0]
    y = torch.empty_like(x)
    idx = torch.empty((B, dims.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((B, dims.top_k), dtype=torch.float32, device=x.device)
    ws = workspace(OP_DECODE, dims, B) if ws is None else ws
    lc = layer.c()
    _check(_lib.flint_moe_decode(ctypes.byref(dims), ctypes.byref(lc), x.data_ptr(), B, y.data_ptr(), idx.data_ptr(),
                                 w.data_ptr(), ws.data_ptr(), ws.numel(), _stream()), "flint_moe_decode")
    return y, idx, w


def moe_decode_noalloc(dims: Dims, layer: LayerWeights, x: torch.Tensor, y: torch.Tensor, idx: torch.Tensor,
                       w: torch.Tensor) -> None:
    """flint_moe_decode on the library's own fixed scratch (no workspace):
    x float32 [B][H] -> y [B][H], idx int32 [B][k], w float32 [B][k]
    (preallocated outputs)."""
    lc = layer.c()
    _check(_lib.flint_moe_decode_noalloc(ctypes.byref(dims), ctypes.byref(lc), x.data_ptr(), x.shape[0],
                                         y.data_ptr(), idx.data_ptr(), w.data_ptr(), _stream()),
           "flint_moe_decode_noalloc")


def lmhead(head: NVFP4Tensor, vocab: int, x: torch.Tensor, ws: torch.Tensor | None = None,
           logits: torch.Tensor | None = None, argmax: torch.Tensor | None = None):
    """x float32 [B][H] -> (logits float32 [B][vocab], argmax int32 [B])"""
    B, H = x.shape
    logits = torch.empty((B, vocab), dtype=torch.float32, device=x.device) if logits is None else logits
    argmax = torch.empty(B, dtype=torch.int32, device=x.device) if argmax is None else argmax
    ws = workspace(OP_LMHEAD, None, B, vocab) if ws is None else ws
    hc = head.c()
    _check(_lib.flint_lmhead_gemv(ctypes.byref(hc), vocab, H, x.data_ptr(), B, logits.data_ptr(), argmax.data_ptr(),
                                  ws.data_ptr(), ws.numel(), _stream()), "flint_lmhead_gemv")
    return logits, argmax


class Stack:
    """A prepared layer stack plus head (keeps the C structs and buffers alive)."""

    def __init__(self, dims: Dims, layers: list[LayerWeights], head: NVFP4Tensor, vocab: int, device="cuda",
                 schedule: int = SCHEDULE_AUTO):
        self.dims, self.vocab, self.n_layers = dims, vocab, len(layers)
        self._layers_c = (Layer * len(layers))(*[l.c() for l in layers])
        self._head_c = head.c()
        self._keep = (layers, head)
        tb = _lib.flint_stack_table_bytes(len(layers))
        self.table = torch.zeros(tb, dtype=torch.uint8, device=device)
        # repacked down projections for the persistent schedule (none when the
        # sizes only allow the kernel sequence, or that schedule is asked for)
        pb = _lib.flint_stack_packed_bytes(ctypes.byref(dims), len(layers))
        if schedule == SCHEDULE_KERNELS:
            pb = 0
        self.packed = torch.empty(pb, dtype=torch.uint8, device=device) if pb else None
        self.plan = StackPlan()
        _check(_lib.flint_stack_prepare(ctypes.byref(dims), self._layers_c, len(layers), ctypes.byref(self._head_c),
                                        vocab, self.table.data_ptr(), tb, _ptr(self.packed), pb,
                                        ctypes.byref(self.plan), _stream()),
               "flint_stack_prepare")
        self.plan.schedule = schedule
        self.ws = workspace(OP_STACK, dims, 1, vocab, len(layers), device=device)

    def decode_traced(self, x: torch.Tensor, eps: float = 1e-6):
        """Persistent schedule with phase stamps of the first token:
        -> (argmax, trace int64 [2][L+1][16] ++ [256][16] in 100 MHz ticks, flat)"""
        T = x.shape[0]
        argmax = torch.empty(T, dtype=torch.int32, device=x.device)
        trace = torch.zeros(2 * (self.n_layers + 1) * TRACE_POINTS + 256 * TRACE_POINTS, dtype=torch.int64, device=x.device)
        _check(_lib.flint_stack_decode_traced(ctypes.byref(self.plan), x.data_ptr(), T, eps, None, argmax.data_ptr(),
                                              None, self.ws.data_ptr(), self.ws.numel(), trace.data_ptr(), _stream()),
               "flint_stack_decode_traced")
        return argmax, trace

    def error(self) -> int:
        """The persistent schedule's watchdog flag (0: none); synchronises."""
        e = _I32(0)
        _check(_lib.flint_stack_error(self.ws.data_ptr(), self.ws.numel(), ctypes.byref(e)), "flint_stack_error")
        return e.value

    def make_batch_tiles(self):
        """Allocate and fill the tiled copy of the expert weights used by decode_batch(tiled=True)."""
        n = _lib.flint_stack_batch_tiles_bytes(ctypes.byref(self.dims), self.n_layers)
        if n == 0:
            raise ValueError("the batched step does not take these sizes")
        self.tiles = torch.empty(n, dtype=torch.uint8, device=self.ws.device)
        _check(_lib.flint_stack_batch_tiles(ctypes.byref(self.plan), self.tiles.data_ptr(), n, _stream()),
               "flint_stack_batch_tiles")
        return self.tiles

    def decode_batch(self, x: torch.Tensor, eps: float = 1e-6, logits: torch.Tensor | None = None,
                     argmax: torch.Tensor | None = None, routes: torch.Tensor | None = None,
                     want_logits: bool = True, ws: torch.Tensor | None = None, tiled: bool = False):
        """x float32 [B][H]: one step of B tokens decoded together (each with its
        own routing); -> (logits [B][vocab] or None, argmax [B]).  tiled: read
        the expert weights from make_batch_tiles()'s copy."""
        B = x.shape[0]
        if want_logits and logits is None:
            logits = torch.empty((B, self.vocab), dtype=torch.float32, device=x.device)
        if argmax is None:
            argmax = torch.empty(B, dtype=torch.int32, device=x.device)
        if ws is None:
            ws = workspace(OP_STACK_BATCH, self.dims, B, self.vocab, self.n_layers, device=x.device)
        if tiled:
            _check(_lib.flint_stack_decode_batch_tiled(ctypes.byref(self.plan), self.tiles.data_ptr(), x.data_ptr(), B,
                                                       eps, _ptr(logits), argmax.data_ptr(), _ptr(routes),
                                                       ws.data_ptr(), ws.numel(), _stream()),
                   "flint_stack_decode_batch_tiled")
        else:
            _check(_lib.flint_stack_decode_batch(ctypes.byref(self.plan), x.data_ptr(), B, eps, _ptr(logits),
                                                 argmax.data_ptr(), _ptr(routes), ws.data_ptr(), ws.numel(),
                                                 _stream()), "flint_stack_decode_batch")
        return logits, argmax

    def decode_stress(self, x: torch.Tensor, seed: int, spin_limit: int, eps: float = 1e-6,
                      routes: torch.Tensor | None = None):
        """The persistent decode with injected delays, permuted roles and the
        given wait limit (a test of the exchange protocol) -> (logits, argmax)."""
        T = x.shape[0]
        logits = torch.empty((T, self.vocab), dtype=torch.float32, device=x.device)
        argmax = torch.empty(T, dtype=torch.int32, device=x.device)
        _check(_lib.flint_stack_decode_stress(ctypes.byref(self.plan), x.data_ptr(), T, eps, logits.data_ptr(),
                                              argmax.data_ptr(), _ptr(routes), self.ws.data_ptr(), self.ws.numel(),
                                              seed, spin_limit, _stream()), "flint_stack_decode_stress")
        return logits, argmax

    def decode_layers(self, x: torch.Tensor, l0: int, n: int, eps: float = 1e-6, h_out: torch.Tensor | None = None,
                      routes: torch.Tensor | None = None) -> torch.Tensor:
        """x float32 [H]: one token through layers l0 .. l0+n-1 (persistent
        schedule, no head) -> the final residual float32 [H]."""
        h_out = torch.empty_like(x) if h_out is None else h_out
        _check(_lib.flint_stack_decode_layers(ctypes.byref(self.plan), l0, n, x.data_ptr(), eps, h_out.data_ptr(),
                                              _ptr(routes), self.ws.data_ptr(), self.ws.numel(), _stream()),
               "flint_stack_decode_layers")
        return h_out

    def decode(self, x: torch.Tensor, eps: float = 1e-6, logits: torch.Tensor | None = None,
               argmax: torch.Tensor | None = None, routes: torch.Tensor | None = None, want_logits: bool = True):
        """x float32 [T][H]: T tokens decoded one after the other."""
        T = x.shape[0]
        if want_logits and logits is None:
            logits = torch.empty((T, self.vocab), dtype=torch.float32, device=x.device)
        if argmax is None:
            argmax = torch.empty(T, dtype=torch.int32, device=x.device)
        _check(_lib.flint_stack_decode(ctypes.byref(self.plan), x.data_ptr(), T, eps, _ptr(logits), argmax.data_ptr(),
                                       _ptr(routes), self.ws.data_ptr(), self.ws.numel(), _stream()),
               "flint_stack_decode")
        return logits, argmax


# ------------------------------------------------- attention and dense MLP --
@dataclass
class AttnWeights:
    """One attention layer: NVFP4 q [Hq*D][H], k and v [Hkv*D][H], o [H][Hq*D];
    float32 q_norm, k_norm [D] and sinks [Hq]."""
    q: NVFP4Tensor
    k: NVFP4Tensor
    v: NVFP4Tensor
    o: NVFP4Tensor
    q_norm: torch.Tensor
    k_norm: torch.Tensor
    sinks: torch.Tensor

    def c(self) -> AttnLayer:
        return AttnLayer(self.q.c(), self.k.c(), self.v.c(), self.o.c(), self.q_norm.data_ptr(),
                         self.k_norm.data_ptr(), self.sinks.data_ptr())


def attn_dims_struct(hidden=2048, n_q=32, n_kv=4, head_dim=128, window=513, rope=True, theta=10000.0,
                     eps=1e-6) -> AttnDims:
    return AttnDims(hidden, n_q, n_kv, head_dim, window, int(rope), theta, eps)


def attn_workspace(dims: AttnDims, device="cuda") -> torch.Tensor:
    n = _lib.flint_attn_workspace_bytes(ctypes.byref(dims))
    if n == 0:
        raise ValueError("unsupported attention dims")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def attn_decode(dims: AttnDims, layer: AttnWeights, x: torch.Tensor, pos: int, k_cache: torch.Tensor,
                v_cache: torch.Tensor, ws: torch.Tensor | None = None, y: torch.Tensor | None = None) -> torch.Tensor:
    """x float32 [H]; k_cache, v_cache int16/uint16 [Hkv][cap][D] (BF16 bits),
    updated in place at slot pos % cap -> y float32 [H]"""
    assert k_cache.shape == v_cache.shape and k_cache.element_size() == 2
    cap = k_cache.shape[1]
    ws = attn_workspace(dims, x.device) if ws is None else ws
    y = torch.empty(dims.hidden, dtype=torch.float32, device=x.device) if y is None else y
    lc = layer.c()
    _check(_lib.flint_attn_decode(ctypes.byref(dims), ctypes.byref(lc), x.data_ptr(), pos, k_cache.data_ptr(),
                                  v_cache.data_ptr(), cap, y.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
           "flint_attn_decode")
    return y


def dense_mlp(gate: NVFP4Tensor, up: NVFP4Tensor, down: NVFP4Tensor, x: torch.Tensor,
              ws: torch.Tensor | None = None, y: torch.Tensor | None = None) -> torch.Tensor:
    """x float32 [B][H] -> y float32 [B][H] = down(silu(gate x) * up x)"""
    B, H = x.shape
    width = gate.codes.shape[-2]
    if ws is None:
        n = _lib.flint_dense_workspace_bytes(H, width, B)
        if n == 0:
            raise ValueError("unsupported dense MLP sizes")
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
    y = torch.empty((B, H), dtype=torch.float32, device=x.device) if y is None else y
    g, u, d = gate.c(), up.c(), down.c()
    _check(_lib.flint_dense_mlp(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), H, width, x.data_ptr(), B,
                                y.data_ptr(), ws.data_ptr(), ws.numel(), _stream()), "flint_dense_mlp")
    return y


# ------------------------------------------------------- INT4 affine codec --
@dataclass
class INT4Tensor:
    """codes uint8 [rows][cols/2], BF16 scales and offsets int16 [rows][cols/64]."""
    codes: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor

    def c(self) -> INT4:
        return INT4(self.codes.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr())


def int4_quantize(w: torch.Tensor) -> INT4Tensor:
    """w float32 cuda [rows][cols] (cols a multiple of 64) -> INT4Tensor"""
    rows, cols = w.shape
    w = w.contiguous()
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((rows, cols // 64), dtype=torch.int16, device=w.device)
    biases = torch.empty((rows, cols // 64), dtype=torch.int16, device=w.device)
    _check(_lib.flint_int4_quantize(w.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                    _stream()), "flint_int4_quantize")
    return INT4Tensor(codes, scales, biases)


def int4_dequantize(q: INT4Tensor) -> torch.Tensor:
    rows, half = q.codes.shape
    out = torch.empty((rows, 2 * half), dtype=torch.float32, device=q.codes.device)
    c = q.c()
    _check(_lib.flint_int4_dequantize(ctypes.byref(c), rows, 2 * half, out.data_ptr(), _stream()),
           "flint_int4_dequantize")
    return out


def int4_gemv(q: INT4Tensor, x: torch.Tensor, want_argmax: bool = True, ws: torch.Tensor | None = None,
              y: torch.Tensor | None = None, argmax: torch.Tensor | None = None):
    """x float32 [B][cols] -> (y float32 [B][rows], argmax int32 [B] or None)"""
    B, cols = x.shape
    rows = q.codes.shape[0]
    if ws is None:
        ws = torch.zeros(_lib.flint_int4_gemv_workspace_bytes(B), dtype=torch.uint8, device=x.device)
    y = torch.empty((B, rows), dtype=torch.float32, device=x.device) if y is None else y
    if want_argmax and argmax is None:
        argmax = torch.empty(B, dtype=torch.int32, device=x.device)
    c = q.c()
    _check(_lib.flint_int4_gemv(ctypes.byref(c), rows, cols, x.data_ptr(), B, y.data_ptr(),
                                _ptr(argmax) if want_argmax else None, ws.data_ptr(), ws.numel(), _stream()),
           "flint_int4_gemv")
    return y, (argmax if want_argmax else None)


# ------------------------------------------------------------ prefill GEMM --
GEMM_A32, GEMM_A4 = 0, 1


def gemm_workspace(T: int, K: int, mode: int, device="cuda") -> torch.Tensor:
    n = _lib.flint_nvfp4_gemm_workspace_bytes(T, K, mode)
    if n == 0:
        raise ValueError("unsupported GEMM sizes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def nvfp4_gemm(q: NVFP4Tensor, X: torch.Tensor, mode: int = GEMM_A32, ws: torch.Tensor | None = None,
               Y: torch.Tensor | None = None) -> torch.Tensor:
    """X float32 [T][K] -> Y float32 [T][N] = X deq(W)^T (A4: X quantised to NVFP4 first)"""
    T, K = X.shape
    N = q.codes.shape[-2]
    ws = gemm_workspace(T, K, mode, X.device) if ws is None else ws
    Y = torch.empty((T, N), dtype=torch.float32, device=X.device) if Y is None else Y
    w = q.c()
    _check(_lib.flint_nvfp4_gemm(ctypes.byref(w), N, K, X.data_ptr(), T, mode, Y.data_ptr(), ws.data_ptr(),
                                 ws.numel(), _stream()), "flint_nvfp4_gemm")
    return Y


# ------------------------------------------------------------- whole model --
class Model:
    """A whole decode model: per layer an attention layer (sliding or full),
    then a dense MLP (the first n_dense layers) or a MoE layer, then the head.
    Keeps the C structs, the host arrays and the tensors alive."""

    def __init__(self, moe_dims: Dims, sliding: AttnDims, full: AttnDims, attn: list, is_full: list,
                 k_caches: list, v_caches: list, dense: list, moe_layers: list, head: NVFP4Tensor, vocab: int,
                 dense_width: int = 6144, eps: float = 1e-6, persistent_moe: bool = False):
        """persistent_moe: run every MoE layer as one launch of the persistent
        stack kernel (a plan with repacked down projections is prepared here);
        otherwise as the kernel sequence."""
        n = len(attn)
        assert len(is_full) == n == len(k_caches) == len(v_caches) == len(dense) + len(moe_layers)
        self.keep = (attn, k_caches, v_caches, dense, moe_layers, head)
        self._attn = (AttnLayer * n)(*[a.c() for a in attn])
        self._is_full = (_I32 * n)(*[int(f) for f in is_full])
        self._kc = (_P * n)(*[t.data_ptr() for t in k_caches])
        self._vc = (_P * n)(*[t.data_ptr() for t in v_caches])
        self._cap = (_I32 * n)(*[int(t.shape[1]) for t in k_caches])
        nd = len(dense)
        self._dense = (NVFP4 * max(1, 3 * nd))(*[m.c() for trio in dense for m in trio])
        self._moe = (Layer * max(1, len(moe_layers)))(*[L.c() for L in moe_layers])
        self.vocab = vocab
        self.c = ModelC(n, nd, dense_width, moe_dims, sliding, full, ctypes.cast(self._is_full, _P),
                        ctypes.cast(self._attn, _P), ctypes.cast(self._kc, _P), ctypes.cast(self._vc, _P),
                        ctypes.cast(self._cap, _P), ctypes.cast(self._dense, _P) if nd else None,
                        ctypes.cast(self._moe, _P) if moe_layers else None, head.c(), vocab, eps, None)
        self.moe_stack = None
        if persistent_moe:
            self.moe_stack = Stack(moe_dims, moe_layers, head, vocab, device=head.codes.device)
            if self.moe_stack.packed is None:
                raise ValueError("these MoE sizes do not allow the persistent schedule")
            self.c.moe_plan = ctypes.cast(ctypes.pointer(self.moe_stack.plan), _P)
        nbytes = _lib.flint_model_workspace_bytes(ctypes.byref(self.c))
        if nbytes == 0:
            raise ValueError("invalid model")
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=head.codes.device)

    def decode(self, x: torch.Tensor, pos: int, logits: torch.Tensor | None = None, argmax: torch.Tensor | None = None,
               want_logits: bool = True, h_out: torch.Tensor | None = None):
        """x float32 [H] at position pos -> (logits [vocab] or None, argmax int32 [1])"""
        if want_logits and logits is None:
            logits = torch.empty(self.vocab, dtype=torch.float32, device=x.device)
        if argmax is None:
            argmax = torch.empty(1, dtype=torch.int32, device=x.device)
        _check(_lib.flint_model_decode(ctypes.byref(self.c), x.data_ptr(), pos, _ptr(logits) if want_logits else None,
                                       argmax.data_ptr(), _ptr(h_out), self.ws.data_ptr(), self.ws.numel(),
                                       _stream()), "flint_model_decode")
        return (logits if want_logits else None), argmax

    def error(self) -> int:
        """The persistent MoE layers' watchdog flag (0: none); synchronises."""
        e = _I32(0)
        _check(_lib.flint_model_error(ctypes.byref(self.c), self.ws.data_ptr(), self.ws.numel(), ctypes.byref(e)),
               "flint_model_error")
        return e.value
