"""Seeded synthetic inputs shared by the GPU tests/benchmark and the CPU oracle.

This module only draws Gaussian numbers and names the streams they come
from; it holds none of the NVFP4 method's arithmetic.  The host generator is
``synth.c`` (Philox4x32-10 + Box-Muller, IEEE-only arithmetic, bit-identical on
every host); ``synth_dev.hip`` is the same definition for the GPU, used to fill
device buffers quickly and tested bit-for-bit against the host generator.

Stream naming.  Every tensor of the workloads is the stream
``(seed, kind << 16 | expert)`` of the generator, element ``i`` being the
row-major flat index, so that any single expert matrix can be drawn on its own.
Weights are N(0, 0.02) (0.02 is the standard deviation), tokens N(0, 1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth.so")
SRC_PATH = os.path.join(HERE, "synth.c")
DEV_LIB_PATH = os.path.join(HERE, "libsynth_dev.so")
DEV_SRC_PATH = os.path.join(HERE, "synth_dev.hip")

# stream kinds
ROUTER, GATE, UP, DOWN, SHARED_GATE, SHARED_UP, SHARED_DOWN, HEAD, TOKEN = range(1, 10)
# attention layers and the dense MLP layers (stream expert field = 0)
ATTN_Q, ATTN_K, ATTN_V, ATTN_O, Q_NORM, K_NORM, SINK, K_CACHE, V_CACHE = range(10, 19)
DENSE_GATE, DENSE_UP, DENSE_DOWN = range(19, 22)
WEIGHT_STD = 0.02

# seeds of the stacked workload: layer l uses weight seed l, the head 1000,
# decode token t seed 10000 + t, batched step s slot j seed 20000 + B*s + j
HEAD_SEED = 1000
TOKEN_SEED0 = 10000
BATCH_SEED0 = 20000


def build_host_lib(force: bool = False) -> str:
    if force or not os.path.exists(LIB_PATH):
        cmd = ["gcc", "-O3", "-mavx2", "-ffp-contract=off", "-fno-math-errno", "-fPIC", "-shared",
               SRC_PATH, "-o", LIB_PATH, "-lpthread", "-lm"]
        subprocess.run(cmd, check=True)
    return LIB_PATH


def build_device_lib(force: bool = False) -> str:
    """hipcc build of the device generator (no GPU needed to build)."""
    if force or not os.path.exists(DEV_LIB_PATH):
        tmp = DEV_LIB_PATH + ".tmp"
        cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O3", "-ffp-contract=off",
               "-fPIC", "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", DEV_SRC_PATH,
               "-o", tmp]
        subprocess.run(cmd, check=True, stderr=subprocess.PIPE)
        os.replace(tmp, DEV_LIB_PATH)
    return DEV_LIB_PATH


_dev_lib = None


def dev_lib():
    global _dev_lib
    if _dev_lib is None:
        if not os.path.exists(DEV_LIB_PATH):
            raise ImportError(f"{DEV_LIB_PATH} is not built")
        L = ctypes.CDLL(DEV_LIB_PATH)
        L.synth_dev_normal_f32.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                           ctypes.c_void_p]
        L.synth_dev_normal_f32.restype = ctypes.c_int
        _dev_lib = L
    return _dev_lib


def normal_device(seed: int, stream: int, n: int, out, mean: float = 0.0, std: float = 1.0, offset: int = 0,
                  n_streams: int = 1, hip_stream: int | None = None):
    """Fill the float32 device tensor `out` (n_streams * n elements) with the
    same numbers as ``normal`` for streams stream .. stream+n_streams-1."""
    import torch
    assert out.dtype == torch.float32 and out.is_contiguous() and out.numel() >= n * n_streams
    hs = torch.cuda.current_stream().cuda_stream if hip_stream is None else hip_stream
    rc = dev_lib().synth_dev_normal_f32(seed & 0xFFFFFFFF, stream & 0xFFFFFFFF, offset, n, n_streams, mean, std,
                                        out.data_ptr(), hs)
    if rc:
        raise RuntimeError(f"synth_dev_normal_f32 failed with hip error {rc}")
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        build_host_lib()
        L = ctypes.CDLL(LIB_PATH)
        L.synth_normal_f32.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_int]
        L.synth_normal_f32.restype = None
        L.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.synth_philox4x32_10.restype = None
        _lib = L
    return _lib


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def stream_id(kind: int, expert: int = 0) -> int:
    assert 0 <= expert < 65536
    return (kind << 16) | expert


def normal(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0, offset: int = 0,
           out: np.ndarray | None = None, nthreads: int = 0) -> np.ndarray:
    """n float32 draws of N(mean, std^2): elements offset..offset+n-1 of (seed, stream)."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size >= n
    lib().synth_normal_f32(seed & 0xFFFFFFFF, stream & 0xFFFFFFFF, offset, n, mean, std, out.ctypes.data, nthreads)
    return out


@dataclass(frozen=True)
class MoEDims:
    hidden: int = 2048
    n_experts: int = 256
    expert_width: int = 512
    top_k: int = 6
    shared_width: int = 1024


@dataclass(frozen=True)
class Workload:
    """A named workload: sizes and seeds (no method arithmetic)."""
    name: str
    dims: MoEDims
    vocab: int = 150144
    layers: int = 1
    weight_seed: int = 0
    head_seed: int = HEAD_SEED
    token_seed: int = 0


@dataclass(frozen=True)
class AttnDims:
    """Grouped-query attention of one layer: 32 query heads over 4 key/value
    heads of dimension 128 on a 2,048-wide residual stream; window > 0 is a
    sliding window (513 = the current token and 512 before it), 0 the whole
    context; rope selects rotary position embedding (theta = its base)."""
    hidden: int = 2048
    n_q: int = 32
    n_kv: int = 4
    head_dim: int = 128
    window: int = 513
    rope: bool = True
    theta: float = 10000.0


SLIDING = AttnDims()
FULL = AttnDims(window=0, rope=False)
DENSE_WIDTH = 6144


def bf16_bits(f: np.ndarray) -> np.ndarray:
    """float32 draws stored as BF16 (uint16 bit patterns, nearest even)."""
    u = np.ascontiguousarray(f, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def attn_f32(seed: int, d: AttnDims, kind: int) -> np.ndarray:
    """q [Hq*D][H], k and v [Hkv*D][H], o [H][Hq*D], N(0, 0.02)."""
    nq, nk = d.n_q * d.head_dim, d.n_kv * d.head_dim
    shape = {ATTN_Q: (nq, d.hidden), ATTN_K: (nk, d.hidden), ATTN_V: (nk, d.hidden), ATTN_O: (d.hidden, nq)}[kind]
    return normal(seed, stream_id(kind), shape[0] * shape[1], std=WEIGHT_STD).reshape(shape)


def attn_gain(seed: int, d: AttnDims, kind: int) -> np.ndarray:
    """q or k head-norm gain [D], N(1, 0.1)."""
    return normal(seed, stream_id(kind), d.head_dim, mean=1.0, std=0.1)


def attn_sinks(seed: int, d: AttnDims) -> np.ndarray:
    """per-query-head sink logits [Hq], N(0, 1)."""
    return normal(seed, stream_id(SINK), d.n_q)


def kv_cache_bits(seed: int, d: AttnDims, cap: int, kind: int) -> np.ndarray:
    """A filled cache [Hkv][cap][D] of BF16 N(0, 1) rows (K_CACHE or V_CACHE)."""
    return bf16_bits(normal(seed, stream_id(kind), d.n_kv * cap * d.head_dim)).reshape(d.n_kv, cap, d.head_dim)


def dense_f32(seed: int, hidden: int, width: int, kind: int) -> np.ndarray:
    """Dense MLP matrix: gate/up [width][hidden], down [hidden][width]."""
    shape = (hidden, width) if kind == DENSE_DOWN else (width, hidden)
    return normal(seed, stream_id(kind), hidden * width, std=WEIGHT_STD).reshape(shape)


# the workloads this repository measures and tests
MOE_LAYER_E32 = Workload("moe_layer_e32", MoEDims(n_experts=32))
MOE_LAYER_E256 = Workload("moe_layer_e256", MoEDims())
LMHEAD = Workload("lmhead_v150144", MoEDims(), vocab=150144)
STACK47 = Workload("stack47_lmhead", MoEDims(), vocab=150144, layers=47, token_seed=TOKEN_SEED0)
STACK47_BATCHED = Workload("stack47_lmhead_batched", MoEDims(), vocab=150144, layers=47, token_seed=BATCH_SEED0)


def router_f32(seed: int, dims: MoEDims) -> np.ndarray:
    return normal(seed, stream_id(ROUTER), dims.n_experts * dims.hidden, std=WEIGHT_STD).reshape(
        dims.n_experts, dims.hidden)


def router_bf16_bits(seed: int, dims: MoEDims) -> np.ndarray:
    """The fp32 router draws stored as BF16 (uint16 bit patterns, round to
    nearest even on the top 16 bits), as a checkpoint keeps a BF16 router."""
    return bf16_bits(router_f32(seed, dims))


def expert_f32(seed: int, dims: MoEDims, kind: int, expert: int) -> np.ndarray:
    """One routed expert matrix: gate/up [I][H], down [H][I]."""
    H, I = dims.hidden, dims.expert_width
    shape = (H, I) if kind == DOWN else (I, H)
    return normal(seed, stream_id(kind, expert), H * I, std=WEIGHT_STD).reshape(shape)


def shared_f32(seed: int, dims: MoEDims, kind: int) -> np.ndarray:
    """Shared expert matrix: gate/up [Is][H], down [H][Is]."""
    H, Is = dims.hidden, dims.shared_width
    shape = (H, Is) if kind == SHARED_DOWN else (Is, H)
    return normal(seed, stream_id(kind), H * Is, std=WEIGHT_STD).reshape(shape)


def head_f32(seed: int, vocab: int, hidden: int, row0: int = 0, rows: int | None = None) -> np.ndarray:
    """Rows row0..row0+rows-1 of the output head [vocab][hidden]."""
    rows = vocab - row0 if rows is None else rows
    return normal(seed, stream_id(HEAD), rows * hidden, std=WEIGHT_STD, offset=row0 * hidden).reshape(rows, hidden)


def token_f32(seed: int, hidden: int) -> np.ndarray:
    return normal(seed, stream_id(TOKEN), hidden, std=1.0)
