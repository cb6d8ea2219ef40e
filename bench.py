"""Decode throughput of the 47-layer NVFP4 MoE stack + NVFP4 lm_head at batch 1.

One step = one token through all 47 MoE layers (router top-6 of 256 + shared
expert, NVFP4 experts) and the 150,144-row NVFP4 head with argmax, on seeded
synthetic weights resident in HBM: one call of flint_stack_decode, i.e. one
launch of the persistent stack kernel.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --batch 32        # small-batch decode: B tokens per step
  python bench.py --layer           # one MoE layer (256 experts), 8 layers in turn
  python bench.py --copy-calib      # one 1 GiB device copy (counter calibration)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
RUNS = 5  # timed runs of K steps each in the default bench; the median is reported
KERNEL = "k_stack_decode"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_stack_decode_stack47_b1_traffic.md")
KERNEL_SOURCES = ["nvfp4_bit_projection_amd/csrc/stack.hip", "nvfp4_bit_projection_amd/csrc/flint_device.h",
                  "nvfp4_bit_projection_amd/csrc/flint_internal.h"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_code(text: str) -> str:
    """The code of a C++/HIP source without its comments and with runs of
    whitespace collapsed, so that an edit to comments alone keeps the hash
    (the sources hashed here hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(kernel_code(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic() -> int | None:
    """HBM bytes per launch of the stack kernel from the committed counter
    summary, if it was taken on the current kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    src = re.search(r"source_hash:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return int(val.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s: float = 10.0, max_reps: int = 64) -> dict:
    """The oracle (plain fp64 CPU code) on a bounded sample of the same
    workload: one token through all 47 layers and the full head, with the
    weights it touches prepared beforehand, repeated until about `target_s`
    seconds of oracle compute have been timed (all oracle threads).  Also the
    single layer (256 experts) and the head alone, median of 3 calls each, on
    all oracle threads and on one."""
    import numpy as np

    import oracle
    import synth
    from oracle.model import SyntheticWeights, moe_layer

    dims = synth.MoEDims()
    W = SyntheticWeights(dims, vocab=150144)
    x = synth.token_f32(synth.TOKEN_SEED0, dims.hidden).astype(np.float64)

    def run():
        h = x.copy()
        for l in range(47):
            u = h * oracle.rms_inv(h, 1e-6)
            h = h + moe_layer(W, l, u).y
        z = h * oracle.rms_inv(h, 1e-6)
        return oracle.argmax(oracle.nvfp4_gemv(W.head(), z))

    first = run()              # prepares (quantises) every tensor the token touches
    reps, timed = 0, 0.0
    while timed < target_s and reps < max_reps:
        t0 = time.perf_counter()
        again = run()
        timed += time.perf_counter() - t0
        reps += 1
        if again != first:
            raise RuntimeError("the oracle is not deterministic")

    def median3(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[1]

    u = x * oracle.rms_inv(x, 1e-6)
    nt = oracle.default_threads()
    per_call = {}
    for threads in (nt, 1):
        per_call[f"layer_e256_ms_{threads}t"] = round(1e3 * median3(lambda: moe_layer(W, 0, u, nthreads=threads)), 2)
        per_call[f"head_v150144_ms_{threads}t"] = round(
            1e3 * median3(lambda: oracle.nvfp4_gemv(W.head(), u, nthreads=threads)), 1)
    return {"value": reps / timed, "unit": "tok/s", "cores": nt, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"one token through all 47 layers + full head, weights prepared beforehand, "
                      f"timed {reps} times: {timed:.1f} s on {nt} threads",
            "per_call_median_of_3": per_call}


def achievable_gbs(nbytes: int = 4 << 30, reps: int = 10) -> dict:
    """The library's streaming-read probe (flint_stream_read: 128-bit
    non-temporal loads, nothing else) over a buffer 16x the 256 MB last-level
    cache: the achievable HBM read rate on this machine."""
    import torch

    from nvfp4_bit_projection_amd import flint

    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        flint.stream_read(buf, out)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        flint.stream_read(buf, out)
    ev1.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del buf, out
    torch.cuda.empty_cache()
    return {"kernel": "k_stream_read", "gbs": round(gbs, 1), "bytes": nbytes, "reps": reps,
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def copy_calib() -> int:
    """One device-to-device copy of 1 GiB (reads 1 GiB, writes 1 GiB): the
    reference dispatch for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {4 * n} bytes")
    return 0


def bench_batch(args) -> int:
    """One step = B fresh tokens through the 47 layers (per-token top-6, each
    chosen expert's weights read once per step) and the head: one call of
    flint_stack_decode_batch.  Bytes per step count the distinct experts of
    every layer, taken from the routes of the same inputs."""
    import torch

    import synth
    from nvfp4_bit_projection_amd import bytes_model as bm
    from nvfp4_bit_projection_amd import flint, workload

    torch.cuda.set_device(0)
    dims = synth.MoEDims()
    L, V, B = args.layers, 150144, args.batch
    tmp = torch.empty(dims.n_experts * dims.expert_width * dims.hidden, dtype=torch.float32, device="cuda")
    layers = [workload.build_layer(dims, seed=l, tmp=tmp) for l in range(L)]
    head = workload.build_head(V, dims.hidden, tmp=None)
    del tmp
    d = flint.dims_struct(dims.hidden, dims.n_experts, dims.expert_width, dims.top_k, dims.shared_width)
    stack = flint.Stack(d, layers, head, V, schedule=flint.SCHEDULE_KERNELS)
    T = args.warmup + args.steps
    x = workload.tokens([synth.TOKEN_SEED0 + t for t in range(T * B)], dims.hidden).view(T, B, dims.hidden)
    ws = flint.workspace(flint.OP_STACK_BATCH, stack.dims, B, V, L)
    argmax = torch.empty((T, B), dtype=torch.int32, device="cuda")
    tiled = bool(args.tiled)
    if tiled:
        stack.make_batch_tiles()
    for t in range(args.warmup):
        stack.decode_batch(x[t], argmax=argmax[t], want_logits=False, ws=ws, tiled=tiled)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for t in range(args.warmup, T):
        stack.decode_batch(x[t], argmax=argmax[t], want_logits=False, ws=ws, tiled=tiled)
    ev1.record()
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    # distinct experts per layer of every timed step (same inputs again, routes kept)
    shape = bm.LayerShape()
    routes = torch.empty((L, B, dims.top_k), dtype=torch.int32, device="cuda")
    total = 0
    for t in range(args.warmup, T):
        stack.decode_batch(x[t], routes=routes, want_logits=False, ws=ws, tiled=tiled)
        u = [len(set(routes[l].flatten().tolist())) for l in range(L)]
        total += sum(bm.layer_bytes(shape, n) for n in u) + bm.head_bytes(V, dims.hidden)
    step_bytes = total / args.steps
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    tok_s = B * 1000.0 / ms_per_step
    log(f"batch {B}{' tiled' if tiled else ''}: {args.steps} steps, {ms_per_step * 1e3:.1f} us/step, {tok_s:.1f} tok/s, "
        f"{step_bytes / 1e9:.3f} GB/step, {gbs:.1f} GB/s")
    result = {
        "metric": f"decode tok/s (47-layer NVFP4 MoE+lm_head, batch {B}) and achieved HBM GB/s vs peak",
        "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"stack47_lmhead_b{B}", "layers": L, "hidden": 2048, "experts": 256, "top_k": 6,
                   "expert_width": 512, "shared_width": 1024, "vocab": V, "batch": B,
                   "weights": "nvfp4 e2m1 + e4m3/16 + fp32 tensor scale; fp32 router",
                   "expert_weight_layout": "tiled copy" if tiled else "row-major"},
        "roofline": {"bound": "hbm", "scope": "whole step (all kernels)", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_step": round(step_bytes)},
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_layer(args) -> int:
    """Config 1: one full MoE layer (256 experts, top-6, shared expert) for one
    token.  Eight distinct layers (3.7 GB, 14x the last-level cache) are used
    in turn, so every call streams its weights from HBM.  Timed per call with
    HIP events: the persistent kernel's one-layer launch
    (flint_stack_decode_layers, norm + layer + residual add) and the kernel
    sequence (flint_moe_decode: router/top-k, gate/up, down).  Bytes per call:
    the router, 6 routed experts and the shared expert, 16,252,928 B."""
    import torch

    import synth
    from nvfp4_bit_projection_amd import bytes_model as bm
    from nvfp4_bit_projection_amd import flint, workload

    torch.cuda.set_device(0)
    dims = synth.MoEDims()
    NL = 8
    tmp = torch.empty(dims.n_experts * dims.expert_width * dims.hidden, dtype=torch.float32, device="cuda")
    layers = [workload.build_layer(dims, seed=l, tmp=tmp) for l in range(NL)]
    del tmp
    head = workload.build_head(16, dims.hidden)
    d = flint.dims_struct(dims.hidden, dims.n_experts, dims.expert_width, dims.top_k, dims.shared_width)
    stack = flint.Stack(d, layers, head, 16, schedule=flint.SCHEDULE_PERSISTENT)
    n = args.warmup + args.steps
    x = workload.tokens([synth.TOKEN_SEED0 + t for t in range(n)], dims.hidden)
    h = torch.empty_like(x)
    y = torch.empty((1, dims.hidden), dtype=torch.float32, device="cuda")
    ws = flint.workspace(flint.OP_DECODE, d, 1)
    nbytes = bm.layer_bytes(bm.LayerShape())
    out = []
    calls = (("persistent_one_layer", lambda i: stack.decode_layers(x[i], i % NL, 1, h_out=h[i])),
             ("kernel_sequence", lambda i: flint.moe_decode(d, layers[i % NL], x[i:i + 1], ws=ws)))
    for name, fn in calls:
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for j, i in enumerate(range(args.warmup, n)):
            evs[j][0].record()
            fn(i)
            evs[j][1].record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        med = us[len(us) // 2]
        gbs = nbytes / (med * 1e-6) / 1e9
        log(f"layer {name}: median {med:.2f} us (min {us[0]:.2f}, max {us[-1]:.2f}), {gbs:.0f} GB/s")
        out.append({"schedule": name, "us_median": round(med, 2), "us_min": round(us[0], 2),
                    "us_max": round(us[-1], 2), "bytes": nbytes, "achieved_gbs": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4)})
    assert stack.error() == 0
    print(json.dumps({"metric": "one MoE layer us per token (E=256, batch 1)", "unit": "us",
                      "higher_is_better": False, "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                      "config": {"workload": "moe_layer_e256_b1", "hidden": 2048, "experts": 256, "top_k": 6,
                                 "expert_width": 512, "shared_width": 1024, "distinct_layers_rotated": NL},
                      "peak_gbs": HBM_PEAK_GBS, "schedules": out}), flush=True)
    return 0


ROTATE_BYTES = 384 * 2**20  # 1.5x the 256 MB last-level cache


def rotation(nbytes: int, cap: int = 512) -> int:
    """Distinct copies of a call's working set (nbytes each) used in turn so
    that together they exceed the last-level cache and every call reads its
    bytes from HBM (at least 2)."""
    return max(2, min(cap, -(-ROTATE_BYTES // max(1, nbytes))))


def bench_router(args) -> int:
    """The router call alone (flint_moe_route_ex at E = 256) in its four
    variants: fp32 or BF16 router, softmax or sigmoid weights.  One step = one
    call for `--batch` tokens; bytes = the router matrix read once per token
    (the kernel's rows are streamed once per token)."""
    import torch

    import synth
    from nvfp4_bit_projection_amd import flint, workload

    torch.cuda.set_device(0)
    dims = synth.MoEDims()
    B = args.batch
    d = flint.dims_struct(dims.hidden, dims.n_experts, dims.expert_width, dims.top_k, dims.shared_width)
    r32 = torch.empty((dims.n_experts, dims.hidden), dtype=torch.float32, device="cuda")
    synth.normal_device(0, synth.stream_id(synth.ROUTER), r32.numel(), r32, std=synth.WEIGHT_STD)
    r16 = r32.to(torch.bfloat16)
    # copies of each router used in turn (together 1.5x the last-level cache)
    routers = {"f32": [r32] + [r32.clone() for _ in range(rotation(r32.numel() * 4) - 1)],
               "bf16": [r16] + [r16.clone() for _ in range(rotation(r16.numel() * 2) - 1)]}
    x = workload.tokens([synth.TOKEN_SEED0 + t for t in range(B)], dims.hidden)
    ws = flint.workspace(flint.OP_ROUTE, d, B)
    out = []
    for name, kind, scoring in (("f32_softmax", "f32", flint.SCORE_SOFTMAX), ("f32_sigmoid", "f32", flint.SCORE_SIGMOID),
                                ("bf16_softmax", "bf16", flint.SCORE_SOFTMAX),
                                ("bf16_sigmoid", "bf16", flint.SCORE_SIGMOID)):
        rs = routers[kind]
        for i in range(args.warmup):
            flint.route_ex(d, rs[i % len(rs)], x, scoring=scoring, ws=ws)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(args.steps):
            flint.route_ex(d, rs[i % len(rs)], x, scoring=scoring, ws=ws)
        ev1.record()
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / args.steps
        nbytes = rs[0].numel() * rs[0].element_size() * B
        gbs = nbytes / (us * 1e-6) / 1e9
        log(f"router {name} B={B}: {us:.2f} us/call, {gbs:.1f} GB/s ({len(rs)} copies in turn)")
        out.append({"variant": name, "us_per_call": round(us, 3), "bytes": nbytes, "achieved_gbs": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "copies_rotated": len(rs)})
    print(json.dumps({"metric": "router call us (E=256)", "unit": "us", "batch": B, "steps": args.steps,
                      "warmup": args.warmup, "higher_is_better": False, "data": "synthetic",
                      "config": {"workload": f"router_e256_b{B}"}, "peak_gbs": HBM_PEAK_GBS, "variants": out}),
          flush=True)
    return 0


def bench_attn(args) -> int:
    """One attention layer at decode (flint_attn_decode) for a sliding-window
    layer and for full-context layers at several context lengths, and the
    dense MLP (flint_dense_mlp, width 6144).  Each configuration: eager calls
    timed with HIP events, and the same calls replayed from a HIP graph (no
    host work between launches; every replay's output is checked against the
    eager one).  Bytes per call: the NVFP4 weights read once, plus the BF16
    keys and values of the attended positions."""
    import torch

    import synth
    from nvfp4_bit_projection_amd import flint, workload

    torch.cuda.set_device(0)
    H = 2048
    steps, warm = args.steps, args.warmup
    out = []

    def timed(fns, check):
        """fns: one call per copy of the working set, used in turn; the
        graph holds a whole number of rounds, ending on the last copy."""
        nc = len(fns)
        for i in range(max(warm, nc)):
            fns[i % nc]()
        torch.cuda.synchronize()
        fns[-1]()
        torch.cuda.synchronize()
        ref = check().clone()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(steps):
            fns[i % nc]()
        ev1.record()
        torch.cuda.synchronize()
        eager_us = ev0.elapsed_time(ev1) * 1e3 / steps
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fns[0]()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        per = nc * max(1, 16 // nc)
        with torch.cuda.graph(g):
            for i in range(per):
                fns[i % nc]()
        for _ in range(3):  # replays agree with the eager result
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(check(), ref):
                raise RuntimeError("graph replay differs from the eager call")
        reps = max(1, steps // per)
        ev0.record()
        for _ in range(reps):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        return eager_us, ev0.elapsed_time(ev1) * 1e3 / (reps * per)

    nq, nk = 32 * 128, 4 * 128
    w_bytes = (nq + 2 * nk) * H * 9 // 16 + H * nq * 9 // 16
    for name, d, ctx in (("sliding513", synth.SLIDING, 4096), ("full_1k", synth.FULL, 1024),
                         ("full_8k", synth.FULL, 8192), ("full_32k", synth.FULL, 32768),
                         ("full_128k", synth.FULL, 131072)):
        cap = 513 if d.window else ctx
        nc = rotation(w_bytes + cap * d.n_kv * d.head_dim * 2 * 2, cap=48)  # layers + caches in turn
        Ws = [workload.build_attn(d, c) for c in range(nc)]
        kcs = [workload.kv_cache(d, 1 + c, cap, synth.K_CACHE) for c in range(nc)]
        vcs = [workload.kv_cache(d, 1 + c, cap, synth.V_CACHE) for c in range(nc)]
        x = workload.tokens([synth.TOKEN_SEED0], H)[0]
        dc = flint.attn_dims_struct(H, d.n_q, d.n_kv, d.head_dim, d.window, d.rope, d.theta)
        ws = flint.attn_workspace(dc)
        y = torch.empty(H, dtype=torch.float32, device="cuda")
        pos = ctx - 1
        n = min(pos + 1, d.window) if d.window else pos + 1
        nbytes = w_bytes + n * d.n_kv * d.head_dim * 2 * 2
        fns = [(lambda c=c: flint.attn_decode(dc, Ws[c], x, pos, kcs[c], vcs[c], ws=ws, y=y)) for c in range(nc)]
        eager_us, graph_us = timed(fns, lambda: y)
        gbs = nbytes / (graph_us * 1e-6) / 1e9
        log(f"attention {name}: {n} positions, {eager_us:.2f} us eager, {graph_us:.2f} us graph, {gbs:.0f} GB/s "
            f"({nc} layers in turn)")
        out.append({"layer": name, "positions": n, "bytes": nbytes, "us_eager": round(eager_us, 2),
                    "us_graph": round(graph_us, 2), "achieved_gbs": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "copies_rotated": nc})
        del Ws, kcs, vcs, ws, fns
    nbytes = 3 * synth.DENSE_WIDTH * H * 9 // 16
    nc = rotation(nbytes, cap=48)
    mlps = [workload.build_dense(c, H, synth.DENSE_WIDTH) for c in range(nc)]
    x = workload.tokens([synth.TOKEN_SEED0], H)
    yd = torch.empty((1, H), dtype=torch.float32, device="cuda")
    wsd = torch.empty(4 * synth.DENSE_WIDTH, dtype=torch.uint8, device="cuda")
    fns = [(lambda c=c: flint.dense_mlp(*mlps[c], x, ws=wsd, y=yd)) for c in range(nc)]
    eager_us, graph_us = timed(fns, lambda: yd)
    gbs = nbytes / (graph_us * 1e-6) / 1e9
    log(f"dense MLP 6144: {eager_us:.2f} us eager, {graph_us:.2f} us graph, {gbs:.0f} GB/s ({nc} copies in turn)")
    out.append({"layer": "dense_6144", "bytes": nbytes, "us_eager": round(eager_us, 2),
                "us_graph": round(graph_us, 2), "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                "copies_rotated": nc})
    print(json.dumps({"metric": "attention and dense layer us per token (batch 1)", "unit": "us",
                      "higher_is_better": False, "steps": steps, "warmup": warm, "data": "synthetic",
                      "config": {"workload": "flint_attn_dense_b1", "q_heads": 32, "kv_heads": 4, "head_dim": 128,
                                 "hidden": H, "window": 513, "dense_width": synth.DENSE_WIDTH,
                                 "weights": "nvfp4; bf16 kv cache"},
                      "peak_gbs": HBM_PEAK_GBS, "layers": out}), flush=True)
    return 0


def bench_int4(args) -> int:
    """The 150,144 x 2,048 output head as group-64 affine INT4 (BF16 scale and
    offset) against the same head as NVFP4: one GEMV + argmax per token
    (flint_int4_gemv, flint_lmhead_gemv), timed from HIP-graph replays.  Both
    formats read 1,152 bytes per row (173 MB per call); four copies of each
    head (692 MB, 2.7x the last-level cache) are used in turn, so every call
    streams its head from HBM."""
    import torch

    import synth
    from nvfp4_bit_projection_amd import flint, workload

    torch.cuda.set_device(0)
    V, H, NC = 150144, 2048, 4
    w = torch.empty(V * H, dtype=torch.float32, device="cuda")
    synth.normal_device(synth.HEAD_SEED, synth.stream_id(synth.HEAD), V * H, w, std=synth.WEIGHT_STD)
    q4 = [flint.int4_quantize(w.view(V, H)) for _ in range(NC)]
    del w
    heads = [workload.build_head(V, H) for _ in range(NC)]
    x = workload.tokens([synth.TOKEN_SEED0], H)
    nbytes = V * (H // 2 + H // 16)
    ws4 = torch.zeros(flint.lib().flint_int4_gemv_workspace_bytes(1), dtype=torch.uint8, device="cuda")
    y4 = torch.empty((1, V), dtype=torch.float32, device="cuda")
    a4 = torch.empty(1, dtype=torch.int32, device="cuda")
    wsn = flint.workspace(flint.OP_LMHEAD, None, 1, V)
    yn = torch.empty((1, V), dtype=torch.float32, device="cuda")
    an = torch.empty(1, dtype=torch.int32, device="cuda")
    out = []
    for name, fn, check in (
            ("int4_g64_head", lambda c: flint.int4_gemv(q4[c], x, ws=ws4, y=y4, argmax=a4), lambda: y4),
            ("int4_g64_gemv_no_argmax", lambda c: flint.int4_gemv(q4[c], x, want_argmax=False, ws=ws4, y=y4),
             lambda: y4),
            ("nvfp4_head", lambda c: flint.lmhead(heads[c], V, x, ws=wsn, logits=yn, argmax=an), lambda: yn)):
        for i in range(args.warmup):
            fn(i % NC)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ref = check().clone()
        with torch.cuda.graph(g):
            for i in range(16):
                fn(i % NC)
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(check(), ref):  # every copy holds the same head
            raise RuntimeError("graph replay differs from the eager call")
        reps = max(1, args.steps // 16)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / (reps * 16)
        gbs = nbytes / (us * 1e-6) / 1e9
        log(f"{name}: {us:.2f} us per token, {gbs:.0f} GB/s ({NC} copies in turn)")
        out.append({"kernel": name, "us": round(us, 2), "bytes": nbytes, "achieved_gbs": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4)})
    print(json.dumps({"metric": "output head GEMV + argmax us per token (batch 1)", "unit": "us",
                      "higher_is_better": False, "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                      "config": {"workload": "lmhead_v150144_int4_vs_nvfp4", "vocab": V, "hidden": H,
                                 "head_copies_rotated": NC},
                      "peak_gbs": HBM_PEAK_GBS, "heads": out}), flush=True)
    return 0


def bench_gemm(args) -> int:
    """Prompt processing: T tokens through one NVFP4 matrix (flint_nvfp4_gemm)
    for a few of the model's shapes, A32 and A4, timed from HIP-graph replays.
    Flops = 2 T N K (the algorithmic count; A32 runs two fp16 products per
    multiply-add, so its ceiling is half the fp16 peak)."""
    import torch

    import synth
    from nvfp4_bit_projection_amd import flint

    torch.cuda.set_device(0)
    peak = 2500.0  # dense fp16 MFMA TFLOP/s
    out = []
    shapes = (("shared_gate_1024x2048", 1024, 2048), ("dense_gate_6144x2048", 6144, 2048),
              ("dense_down_2048x6144", 2048, 6144), ("head_150144x2048", 150144, 2048))
    if args.gemm_case:  # one shape, token count and mode, a few plain calls (for counter runs)
        name, T, mode = args.gemm_case.split(":")
        N, K = next((n, k) for nm, n, k in shapes if nm == name)
        w = torch.empty(N * K, dtype=torch.float32, device="cuda")
        synth.normal_device(7, synth.stream_id(synth.HEAD), N * K, w, std=synth.WEIGHT_STD)
        q = flint.quantize(w.view(N, K))
        del w
        X = torch.empty(int(T) * K, dtype=torch.float32, device="cuda")
        synth.normal_device(8, synth.stream_id(synth.TOKEN), int(T) * K, X)
        ws = flint.gemm_workspace(int(T), K, int(mode))
        Y = torch.empty((int(T), N), dtype=torch.float32, device="cuda")
        for _ in range(args.steps):
            flint.nvfp4_gemm(q, X.view(int(T), K), int(mode), ws=ws, Y=Y)
        torch.cuda.synchronize()
        log(f"gemm case {args.gemm_case}: {args.steps} calls done")
        return 0
    for name, N, K in shapes:
        w = torch.empty(N * K, dtype=torch.float32, device="cuda")
        synth.normal_device(7, synth.stream_id(synth.HEAD), N * K, w, std=synth.WEIGHT_STD)
        q = flint.quantize(w.view(N, K))
        del w
        # weight copies used in turn (together 1.5x the last-level cache), so
        # each call starts with its weights in HBM
        nc = rotation(N * K * 9 // 16)
        qs = [q] + [flint.NVFP4Tensor(q.codes.clone(), q.scales.clone(), q.tscale.clone()) for _ in range(nc - 1)]
        for T in (512, 2048):
            X = torch.empty(T * K, dtype=torch.float32, device="cuda")
            synth.normal_device(8, synth.stream_id(synth.TOKEN), T * K, X)
            X = X.view(T, K)
            for mode, mname in ((flint.GEMM_A32, "a32"), (flint.GEMM_A4, "a4")):
                ws = flint.gemm_workspace(T, K, mode)
                Y = torch.empty((T, N), dtype=torch.float32, device="cuda")
                fns = [(lambda c=c: flint.nvfp4_gemm(qs[c], X, mode, ws=ws, Y=Y)) for c in range(nc)]
                for f in fns:
                    f()
                torch.cuda.synchronize()
                ref = Y.clone()  # the last copy's result (all copies hold the same weights)
                g = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    fns[0]()
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                per = nc * max(1, 4 // nc)
                with torch.cuda.graph(g):
                    for i in range(per):
                        fns[i % nc]()
                g.replay()
                torch.cuda.synchronize()
                if not torch.equal(Y, ref):
                    raise RuntimeError("graph replay differs from the eager call")
                reps = max(1, min(args.steps, 64) // per)
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record()
                for _ in range(reps):
                    g.replay()
                ev1.record()
                torch.cuda.synchronize()
                us = ev0.elapsed_time(ev1) * 1e3 / (reps * per)
                tf = 2.0 * T * N * K / (us * 1e-6) / 1e12
                log(f"gemm {name} T={T} {mname}: {us:.1f} us, {tf:.1f} TFLOP/s ({100 * tf / peak:.1f}% of fp16 peak, "
                    f"{nc} weight copies in turn)")
                out.append({"shape": name, "T": T, "mode": mname, "us": round(us, 2), "tflops": round(tf, 1),
                            "frac_fp16_peak": round(tf / peak, 4), "weight_copies_rotated": nc})
                del ws, Y, fns
            del X
        del q, qs
    print(json.dumps({"metric": "prefill GEMM TFLOP/s (NVFP4 weights)", "unit": "TFLOP/s", "higher_is_better": True,
                      "data": "synthetic", "config": {"workload": "nvfp4_prefill_gemm"}, "peak_tflops": peak,
                      "results": out}), flush=True)
    return 0


def full_attention_layer(l: int) -> bool:
    """14 of 49 layers attend to the whole context; the pages do not give
    which, so two of every seven (layers 3, 6, 10, 13, ...)."""
    return l % 7 in (3, 6)


def bench_model(args) -> int:
    """One token through the whole model (flint_model_decode): 49 layers, each
    attention (35 sliding-window with RoPE, 14 full-context) then a dense MLP
    (layers 0-1, width 6,144) or a MoE layer (47 layers, the same weights as
    the MoE stack), then the 150,144-row head with argmax, at a context of
    `--context` positions.  Bytes per token: every weight the token touches
    plus the keys and values it attends to."""
    import torch

    import synth
    from nvfp4_bit_projection_amd import bytes_model as bm
    from nvfp4_bit_projection_amd import flint, workload

    torch.cuda.set_device(0)
    H, V, NL, ND, DW = 2048, 150144, 49, 2, synth.DENSE_WIDTH
    md = synth.MoEDims()
    ctx, T = args.context, args.warmup + args.steps
    is_full = [full_attention_layer(l) for l in range(NL)]
    dims = [synth.FULL if f else synth.SLIDING for f in is_full]
    caps = [ctx + T if f else 513 for f in is_full]
    tmp = torch.empty(md.n_experts * md.expert_width * md.hidden, dtype=torch.float32, device="cuda")
    moe = [workload.build_layer(md, seed=l, tmp=tmp) for l in range(NL - ND)]
    del tmp
    attn = [workload.build_attn(dims[l], 100 + l) for l in range(NL)]
    dense = [workload.build_dense(200 + l, H, DW) for l in range(ND)]
    kc = [workload.kv_cache(dims[l], 300 + l, caps[l], synth.K_CACHE) for l in range(NL)]
    vc = [workload.kv_cache(dims[l], 300 + l, caps[l], synth.V_CACHE) for l in range(NL)]
    head = workload.build_head(V, H)
    ad = lambda d: flint.attn_dims_struct(H, d.n_q, d.n_kv, d.head_dim, d.window, d.rope, d.theta)
    M = flint.Model(flint.dims_struct(md.hidden, md.n_experts, md.expert_width, md.top_k, md.shared_width),
                    ad(synth.SLIDING), ad(synth.FULL), attn, is_full, kc, vc, dense, moe, head, V, dense_width=DW,
                    persistent_moe=not args.moe_kernels)
    x = workload.tokens([synth.TOKEN_SEED0 + t for t in range(T)], H)
    am = torch.empty((T, 1), dtype=torch.int32, device="cuda")
    p0 = ctx - 1
    for t in range(args.warmup):
        M.decode(x[t], p0 + t, argmax=am[t], want_logits=False)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for t in range(args.warmup, T):
        M.decode(x[t], p0 + t, argmax=am[t], want_logits=False)
    ev1.record()
    torch.cuda.synchronize()
    if M.error():
        log("the persistent MoE kernel reported a timed-out wait")
        return 1
    ms = ev0.elapsed_time(ev1) / args.steps
    shape = bm.LayerShape()
    w_attn = NL * ((32 + 2 * 4) * 128 * H * 9 // 16 + H * 32 * 128 * 9 // 16)
    w_dense = ND * 3 * DW * H * 9 // 16
    w_moe = (NL - ND) * bm.layer_bytes(shape)
    pos_mid = p0 + args.warmup + args.steps // 2
    kv = sum((min(pos_mid + 1, 513) if not f else pos_mid + 1) * 2048 for f in is_full)
    nbytes = w_attn + w_dense + w_moe + bm.head_bytes(V, H) + kv
    gbs = nbytes / (ms * 1e-3) / 1e9
    sched = "kernel sequence" if args.moe_kernels else "persistent, one layer per launch"
    log(f"model 49 layers, context {ctx}, MoE {sched}: {ms * 1e3:.1f} us/token, {1000.0 / ms:.1f} tok/s, "
        f"{nbytes / 1e9:.3f} GB/token (KV {kv / 1e6:.1f} MB), {gbs:.0f} GB/s")
    print(json.dumps({"metric": f"whole-model decode tok/s (49 layers + head, context {ctx}, batch 1)",
                      "value": round(1000.0 / ms, 2), "unit": "tok/s", "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(ms, 4), "higher_is_better": True, "data": "synthetic", "dtype": "f32",
                      "config": {"workload": f"flint49_ctx{ctx}_b1", "layers": NL, "dense_layers": ND,
                                 "full_attention_layers": sum(is_full), "context": ctx, "moe_schedule": sched},
                      "roofline": {"bound": "hbm", "scope": "whole step (all kernels)", "achieved": round(gbs, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "bytes_per_token": nbytes}}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=47)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-achievable", action="store_true", help="skip the streaming-read achievable line")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--batch", type=int, default=1,
                    help="tokens per step; above 1 the batched step (experts deduplicated per layer) is timed")
    ap.add_argument("--tiled", action="store_true",
                    help="with --batch: read the expert weights from the tiled copy (flint_stack_batch_tiles)")
    ap.add_argument("--router", action="store_true",
                    help="time the router call alone in its four variants (fp32/BF16 router, softmax/sigmoid)")
    ap.add_argument("--attn", action="store_true",
                    help="time one attention layer (sliding and full context) and the dense MLP")
    ap.add_argument("--layer", action="store_true",
                    help="time one MoE layer of 256 experts (8 distinct layers in turn), both schedules")
    ap.add_argument("--int4", action="store_true",
                    help="time the output head as group-64 affine INT4 against the NVFP4 head")
    ap.add_argument("--gemm", action="store_true", help="time the prefill GEMM (A32 and A4) on model shapes")
    ap.add_argument("--gemm-case", default="", help="with --gemm: only SHAPE:T:MODE, e.g. head_150144x2048:512:0")
    ap.add_argument("--model", action="store_true", help="time the whole 49-layer model (attention + dense/MoE)")
    ap.add_argument("--context", type=int, default=1024, help="context length for --model")
    ap.add_argument("--moe-kernels", action="store_true",
                    help="with --model: run the MoE layers as the kernel sequence instead of the persistent kernel")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (batch-1 decode; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        return 2
    if args.copy_calib:
        return copy_calib()
    if args.router:
        return bench_router(args)
    if args.attn:
        return bench_attn(args)
    if args.int4:
        return bench_int4(args)
    if args.layer:
        return bench_layer(args)
    if args.gemm:
        return bench_gemm(args)
    if args.model:
        return bench_model(args)
    if args.batch > 1:
        return bench_batch(args)

    import torch

    import synth
    from nvfp4_bit_projection_amd import bytes_model as bm
    from nvfp4_bit_projection_amd import flint, workload

    torch.cuda.set_device(0)
    dims = synth.MoEDims()
    L, V = args.layers, 150144
    t0 = time.time()
    tmp = torch.empty(dims.n_experts * dims.expert_width * dims.hidden, dtype=torch.float32, device="cuda")
    layers = [workload.build_layer(dims, seed=l, tmp=tmp) for l in range(L)]
    head = workload.build_head(V, dims.hidden, tmp=None)
    del tmp
    torch.cuda.synchronize()
    log(f"weights ready in {time.time() - t0:.1f}s ({torch.cuda.memory_allocated() / 1e9:.1f} GB)")
    d = flint.dims_struct(dims.hidden, dims.n_experts, dims.expert_width, dims.top_k, dims.shared_width)
    stack = flint.Stack(d, layers, head, V)
    T = args.warmup + args.steps
    x = workload.tokens([synth.TOKEN_SEED0 + t for t in range(T)], dims.hidden)
    argmax = torch.empty(T, dtype=torch.int32, device="cuda")
    logits = torch.empty((1, V), dtype=torch.float32, device="cuda")

    def step(t):
        stack.decode(x[t:t + 1], logits=logits, argmax=argmax[t:t + 1])

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    if stack.error():
        log("the stack kernel raised its error flag")
        return 1
    # RUNS timed runs of exactly K steps each, every run bracketed by
    # synchronisations and one event pair on torch's current stream, the
    # stream every launch goes to: their throughput is the reported value
    # (the median run; min and max are reported with it).  Then RUNS more runs
    # of the same K steps with an event pair around every launch: these give
    # the kernel's launch duration for the roofline.  An event between two
    # launches adds a marker to the queue and widens the gap between them, so
    # the throughput runs carry none; the instrumented runs' own throughput is
    # reported beside it.
    def timed_run(per_launch):
        n = args.steps if per_launch else 0
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        ev0.record()
        if per_launch:
            for i, t in enumerate(range(args.warmup, T)):
                starts[i].record()
                step(t)
                ends[i].record()
        else:
            for t in range(args.warmup, T):
                step(t)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        return ev0.elapsed_time(ev1), [a.elapsed_time(b) for a, b in zip(starts, ends)], wall

    run_ms, launch_ms, walls, inst_ms = [], [], [], []
    for run in range(RUNS):
        ms_run, _, wall = timed_run(False)
        run_ms.append(ms_run)
        walls.append(wall)
    for run in range(RUNS):
        ms_run, per_launch, _ = timed_run(True)
        inst_ms.append(ms_run)
        launch_ms += per_launch
    if stack.error():
        log("the stack kernel raised its error flag")
        return 1
    order = sorted(range(RUNS), key=lambda r: run_ms[r])
    ms = run_ms[order[RUNS // 2]]
    ms_per_step = ms / args.steps
    tok_s = 1000.0 / ms_per_step
    tok_runs = [1000.0 * args.steps / m for m in run_ms]
    launch_ms.sort()
    launch_avg = sum(launch_ms) / len(launch_ms)
    shape = bm.LayerShape()
    token_bytes = bm.token_bytes(shape, L, V)
    gbs = token_bytes / (launch_avg * 1e-3) / 1e9
    log(f"{RUNS} runs of {args.steps} tokens: median {ms:.2f} ms ({tok_s:.1f} tok/s), "
        f"min {min(tok_runs):.1f} max {max(tok_runs):.1f} tok/s; {KERNEL} launch avg {launch_avg * 1e3:.1f} us "
        f"(median {launch_ms[len(launch_ms) // 2] * 1e3:.1f}), {gbs:.1f} GB/s; runs with an event pair around "
        f"every launch: median {1000.0 * args.steps / sorted(inst_ms)[RUNS // 2]:.1f} tok/s")

    traffic = measured_traffic()
    result = {
        "metric": "decode tok/s (47-layer NVFP4 MoE+lm_head, batch 1) and achieved HBM GB/s vs peak",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "stack47_lmhead_b1", "layers": L, "hidden": 2048, "experts": 256, "top_k": 6,
                   "expert_width": 512, "shared_width": 1024, "vocab": V, "batch": 1,
                   "weights": "nvfp4 e2m1 + e4m3/16 + fp32 tensor scale; fp32 router"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": (round(traffic / (launch_avg * 1e-3) / 1e9, 1) if traffic else None),
                     "kernel": KERNEL, "bytes_per_launch": token_bytes,
                     "traffic_bytes_per_launch": traffic, "launch_us": round(launch_avg * 1e3, 2)},
        "runs": {"n": RUNS, "steps_each": args.steps, "tok_s_median": round(tok_s, 2),
                 "tok_s_min": round(min(tok_runs), 2), "tok_s_max": round(max(tok_runs), 2),
                 "tok_s": [round(v, 2) for v in tok_runs], "wall_s": [round(w, 4) for w in walls],
                 "instrumented_tok_s_median": round(1000.0 * args.steps / sorted(inst_ms)[RUNS // 2], 2)},
    }
    # release device memory before the interpreter exits (keeps profilers'
    # teardown away from live allocations)
    del stack, layers, head, x, logits, argmax
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_achievable:
        result["achievable"] = achievable_gbs()
        log(f"achievable (streaming read): {result['achievable']['gbs']} GB/s")
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
