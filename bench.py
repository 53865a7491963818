#!/usr/bin/env python3
"""Throughput of the TACO FP8 compression operator on one MI355X.

One step is one pass of the whole hot path on the GPT-3-6.7B-shaped TP layer
(bf16 [4096, 4096], block 128), i.e. what one GPU does per layer:
  compress(forward activation) -> decompress,
  compress(backward gradient)  -> decompress,
  decompress_sum(4 compressed partial sums of the same shape)
(the 4 partial sums stand for the peers' contributions; they are compressed
once before timing, as the peers would do on their own GPUs).

Inputs are resident in HBM when timing starts.  To keep the timed traffic in
HBM rather than the 256 MB Infinity Cache, the step rotates over R complete
buffer sets (16 by default, 4.3 GB together: even the op with the smallest
inputs, decompress, reads 2 x 16 x 16.8 MB per rotation, twice the cache).  `value` is bf16 bytes moved by the calls
(bf16 in for compress, bf16 out for the decompressions) per second.

Steps are launched as HIP graphs, so the timed region measures the GPU rather
than the host's per-call enqueue cost: one graph holds one step per buffer set
(R steps, replayed K // R times; any remaining steps replay single-step
graphs), because consecutive graph launches leave a gap of several
microseconds on the GPU that one launch per step would add to every step.
Every step still does all of its work.  The per-op durations (and the roofline
of the compress kernels) come from their own timed regions: graphs of
back-to-back calls of one op, OP_PASSES passes over every buffer set.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compress/decompress GB/s (bf16 in) and % of MI355X HBM peak, 1 GPU"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, published
WORKLOAD = "gpt3_6p7b"
TOKENS, HIDDEN, BLOCK, NPARTS = 4096, 4096, 128, 4
COUNTERS_FILE = os.path.join(ROOT, "profiles", "compress_gpt3_6p7b_counters.json")
OP_PASSES = 2                    # passes over the buffer sets per per-op graph


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--rotate", type=int, default=16,
                   help="buffer sets rotated over (16: 4.3 GB, so that every op's inputs over one "
                        "rotation exceed the 256 MB Infinity Cache at least twice)")
    p.add_argument("--cpu-rows", type=int, default=TOKENS,
                   help="rows of the workload the oracle is timed on (cpu_baseline)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="the oracle's step is repeated until at least this much CPU time")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--single-pass", choices=["on", "off"], default="on",
                   help="fused single-pass compress when the tensor fits (default) or the two-kernel path")
    p.add_argument("--all-configs", action="store_true",
                   help="also time cold compress and decompress on the other workload shapes "
                        "(tiny, GPT-2-1.5B, Qwen-7B; reported under 'configs', not the metric)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="before timing, run 8 plain device copies of this many MiB (a known-size "
                        "kernel that calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE in the same process)")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "fp8_compression_tensor_taco_amd", "csrc", "taco.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def measured_counters():
    """The committed rocprofv3 counter run of the compress kernel (HBM bytes
    and MFMA instructions per call), or {} if the kernel source changed since
    the counters were taken."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return {}
    if c.get("kernel_source_sha256") != kernel_source_hash():
        return {}
    return c


def cpu_baseline(rows: int, min_seconds: float):
    """The oracle, as it is, on the first `rows` rows of the same step (1 BLAS
    thread), repeated until at least `min_seconds` of CPU work."""
    from threadpoolctl import threadpool_limits

    import oracle
    from fp8_compression_tensor_taco_amd import workloads as W

    act = W.bf16_bits(W.make("gpt3_6p7b_act", seed=0, tokens=rows))
    grad = W.bf16_bits(W.make("gpt3_6p7b_grad", seed=1, tokens=rows))
    parts = [oracle.compress(W.bf16_bits(W.make("gpt3_6p7b_act", seed=10 + p, tokens=rows)), BLOCK)
             for p in range(NPARTS)]
    runs = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            for x in (act, grad):
                q, a, s = oracle.compress(x, BLOCK)
                oracle.decompress(q, a, s, BLOCK)
            oracle.decompress_sum(parts, BLOCK)
            runs += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    nbytes = 2 * rows * HIDDEN * 5 * runs        # bf16 bytes of the 5 calls per step
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{runs} step(s) on rows 0..{rows - 1} of the [{TOKENS},{HIDDEN}] workload "
                      f"({rows}x{HIDDEN} per tensor; the 4 decompress-sum parts compressed beforehand), "
                      f"numpy fp64, BLAS limited to 1 thread, {dt:.1f} s"}


def time_configs(taco, W, dev, stream, capture, time_us):
    """Cold per-call compress and decompress on the other workload shapes: graphs
    of back-to-back calls over enough buffer sets to exceed 1 GiB (at most 512)."""
    import torch

    res = {}
    for name in ("tiny", "gpt2_1p5b", "qwen_7b"):
        w = W.WORKLOADS[name]
        T, H, B = w.tokens, w.hidden, w.block
        n = T * H
        x0 = W.make(name, seed=0).to(dev)
        set_bytes = 2 * n + n + 4 * n // B + 2 * n
        nsets = min(512, max(4, -(-(1 << 30) // set_bytes)))
        sets = [{"x": x0.clone(), "q": torch.empty((T, H), dtype=torch.uint8, device=dev),
                 "a": torch.empty((T, H // B), dtype=torch.float32, device=dev),
                 "s": torch.empty(1, dtype=torch.float32, device=dev),
                 "y": torch.empty((T, H), dtype=torch.bfloat16, device=dev)} for _ in range(nsets)]
        del x0
        ws = torch.zeros(taco.workspace_bytes(T, H, B), dtype=torch.uint8, device=dev)
        for st in sets:
            taco.compress(st["x"], B, q=st["q"], alpha=st["a"], scale=st["s"], workspace=ws)
        torch.cuda.synchronize()
        gc = capture(lambda: [taco.compress(st["x"], B, q=st["q"], alpha=st["a"], scale=st["s"], workspace=ws)
                              for st in sets])
        gd = capture(lambda: [taco.decompress(st["q"], st["a"], st["s"], B, out=st["y"]) for st in sets])
        gc.replay()
        gd.replay()
        alg = 3 * n + 4 * n // B + 4
        c_us = time_us(gc.replay, nsets, 4)
        d_us = time_us(gd.replay, nsets, 4)
        res[name] = {"shape": [T, H], "block": B, "buffer_sets": nsets,
                     "single_pass": bool(taco.is_single_pass(T, H, B)),
                     "compress_us": round(c_us, 3), "decompress_us": round(d_us, 3),
                     "compress_bf16_GBps": round(2 * n / (c_us * 1e-6) / 1e9, 1),
                     "decompress_bf16_GBps": round(2 * n / (d_us * 1e-6) / 1e9, 1),
                     "compress_hbm_frac": round(alg / (c_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "decompress_hbm_frac": round(alg / (d_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del gc, gd, sets, ws
        torch.cuda.synchronize()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the operator needs no collectives and this build "
              f"has no multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE={world}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_compression_tensor_taco_amd as taco
    from fp8_compression_tensor_taco_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    taco.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- resident inputs, R rotating buffer sets
    act = W.make("gpt3_6p7b_act", seed=0).to(dev)
    grad = W.make("gpt3_6p7b_grad", seed=1).to(dev)
    part_src = [taco.compress(W.make("gpt3_6p7b_act", seed=10 + p).to(dev), BLOCK)
                for p in range(NPARTS)]
    torch.cuda.synchronize()
    nscales = TOKENS * HIDDEN // BLOCK
    sets = []
    for _ in range(args.rotate):
        s = {
            "act": act.clone(), "grad": grad.clone(),
            "parts": [tuple(t.clone() for t in p) for p in part_src],
            "q": [torch.empty((TOKENS, HIDDEN), dtype=torch.uint8, device=dev) for _ in range(2)],
            "a": [torch.empty((TOKENS, HIDDEN // BLOCK), dtype=torch.float32, device=dev) for _ in range(2)],
            "s": [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(2)],
            "xh": [torch.empty((TOKENS, HIDDEN), dtype=torch.bfloat16, device=dev) for _ in range(2)],
            "sum": torch.empty((TOKENS, HIDDEN), dtype=torch.bfloat16, device=dev),
            "rq": torch.empty((TOKENS, HIDDEN), dtype=torch.uint8, device=dev),
            "ra": torch.empty((TOKENS, HIDDEN // BLOCK), dtype=torch.float32, device=dev),
            "rs": torch.empty(1, dtype=torch.float32, device=dev),
            "sblk": torch.empty((TOKENS, HIDDEN // BLOCK), dtype=torch.float32, device=dev),
        }
        sets.append(s)
    del act, grad, part_src
    ws = torch.zeros(taco.workspace_bytes(TOKENS, HIDDEN, BLOCK), dtype=torch.uint8, device=dev)
    ws_rs = torch.zeros(taco.load().taco_decompress_sum_compress_workspace_bytes(TOKENS, HIDDEN, BLOCK),
                        dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    taco.set_single_pass(args.single_pass == "on")
    if args.copy_probe_mib > 0:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    set_bytes = sum(t.numel() * t.element_size() for t in
                    [sets[0]["act"], sets[0]["grad"], *sets[0]["q"], *sets[0]["a"], *sets[0]["xh"],
                     sets[0]["sum"], *[t for p in sets[0]["parts"] for t in p]])

    ops = ["compress", "decompress", "decompress_sum"]

    def op_compress(st, k):
        x = st["act"] if k == 0 else st["grad"]
        taco.compress(x, BLOCK, q=st["q"][k], alpha=st["a"][k], scale=st["s"][k], workspace=ws)

    def op_decompress(st, k):
        taco.decompress(st["q"][k], st["a"][k], st["s"][k], BLOCK, out=st["xh"][k])

    def op_sum(st):
        taco.decompress_sum(st["parts"], BLOCK, out=st["sum"])

    amax = [torch.zeros(taco.TACO_AMAX_FLOATS, dtype=torch.float32, device=dev) for _ in range(2)]

    def op_blockscale(st, k):
        x = st["act"] if k == 0 else st["grad"]
        taco.compress_blockscale(x, BLOCK, q=st["q"][k], alpha=st["a"][k], scale=st["sblk"])

    def op_blockscale_dec(st, k):
        taco.decompress_blockscale(st["q"][k], st["a"][k], st["sblk"], BLOCK, out=st["xh"][k])

    def op_delayed(st, k):
        x = st["act"] if k == 0 else st["grad"]
        taco.compress_delayed(x, BLOCK, amax[0], q=st["q"][k], alpha=st["a"][k], scale=st["s"][k],
                              amax_out=amax[1])

    def op_int8(st, k, block):
        x = st["act"] if k == 0 else st["grad"]
        taco.compress_int8(x, block, q=st["q"][k].view(torch.int8),
                           scale=st["s"][k] if block == 0 else st["sblk"], workspace=ws)

    def op_int8_dec(st, k, block):
        taco.decompress_int8(st["q"][k].view(torch.int8), st["s"][k] if block == 0 else st["sblk"], block,
                             out=st["xh"][k])

    def op_sum_compress(st):
        taco.decompress_sum_compress(st["parts"], BLOCK, q=st["rq"], alpha=st["ra"], scale=st["rs"],
                                     workspace=ws_rs)

    def step(st):
        for k in range(2):
            op_compress(st, k)
            op_decompress(st, k)
        op_sum(st)

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # ---- HIP graphs: one per buffer set for the step, and one per op that runs
    # that op back to back over every set (so its inputs cycle through >1 GiB)
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    step_graphs = [capture(lambda st=st: step(st)) for st in sets]
    cycle_graph = capture(lambda: [step(st) for st in sets])
    P = OP_PASSES
    op_graphs = {
        "compress": (capture(lambda: [op_compress(st, k) for _ in range(P) for st in sets for k in range(2)]),
                     2 * P * len(sets)),
        "decompress": (capture(lambda: [op_decompress(st, k) for _ in range(P) for st in sets for k in range(2)]),
                       2 * P * len(sets)),
        "decompress_sum": (capture(lambda: [op_sum(st) for _ in range(P) for st in sets]), P * len(sets)),
        "decompress_sum_compress": (capture(lambda: [op_sum_compress(st) for _ in range(P) for st in sets]),
                                    P * len(sets)),
        "compress_blockscale": (capture(lambda: [op_blockscale(st, k) for _ in range(P) for st in sets
                                                 for k in range(2)]), 2 * P * len(sets)),
        "decompress_blockscale": (capture(lambda: [op_blockscale_dec(st, k) for _ in range(P) for st in sets
                                                   for k in range(2)]), 2 * P * len(sets)),
        "compress_delayed": (capture(lambda: [op_delayed(st, k) for _ in range(P) for st in sets
                                              for k in range(2)]), 2 * P * len(sets)),
        "compress_int8_tensor": (capture(lambda: [op_int8(st, k, 0) for _ in range(P) for st in sets
                                                  for k in range(2)]), 2 * P * len(sets)),
        "decompress_int8_tensor": (capture(lambda: [op_int8_dec(st, k, 0) for _ in range(P) for st in sets
                                                    for k in range(2)]), 2 * P * len(sets)),
        "compress_int8_block": (capture(lambda: [op_int8(st, k, BLOCK) for _ in range(P) for st in sets
                                                 for k in range(2)]), 2 * P * len(sets)),
        "decompress_int8_block": (capture(lambda: [op_int8_dec(st, k, BLOCK) for _ in range(P) for st in sets
                                                   for k in range(2)]), 2 * P * len(sets)),
    }
    cycle_graph.replay()
    for g in step_graphs:
        g.replay()
    for g, _ in op_graphs.values():
        g.replay()
    torch.cuda.synchronize()

    # ---- timed region: K steps (graph replays) bracketed by events on the launch stream
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    cycles, rest = divmod(args.steps, len(sets))
    for _ in range(cycles):
        cycle_graph.replay()                     # steps on sets 0 .. R-1
    for i in range(rest):
        step_graphs[i].replay()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps

    # ---- per-op timed regions: average duration of one call of each op
    reps = max(1, args.steps // (4 * OP_PASSES))
    avg_us = {}
    extra = ["decompress_sum_compress", "compress_blockscale", "decompress_blockscale", "compress_delayed",
             "compress_int8_tensor", "decompress_int8_tensor", "compress_int8_block", "decompress_int8_block"]
    def time_us(fn, calls, repeat):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(repeat):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / (repeat * calls)

    for op in ops + extra:
        g, calls = op_graphs[op]
        avg_us[op] = time_us(g.replay, calls, reps)

    # ---- warm: the step's ops back to back on one buffer set, whose inputs stay
    # in the 256 MB Infinity Cache (reported apart, labeled; not the metric)
    s0 = sets[0]
    warm = {"compress": (capture(lambda: [op_compress(s0, k) for _ in range(8) for k in range(2)]), 16),
            "decompress": (capture(lambda: [op_decompress(s0, k) for _ in range(8) for k in range(2)]), 16),
            "decompress_sum": (capture(lambda: [op_sum(s0) for _ in range(16)]), 16)}
    warm_us = {}
    for op, (g, calls) in warm.items():
        g.replay()
        warm_us[op] = time_us(g.replay, calls, reps)
    del warm

    # ---- 32 decompress-sum layers back to back (4 parts of [4096, 4096] at block
    # 256, part p drawn with seed p, in 32 distinct layer slots: 2.2 GB of codes):
    # per-layer time of eager launches against the same 32 calls in one graph;
    # the difference is the launch gap.
    B5, L5 = 256, 32
    src5 = [tuple(t.clone() for t in taco.compress(W.make("dsum_part", seed=p).to(dev), B5))
            for p in range(NPARTS)]
    slots5 = [[tuple(t.clone() for t in part) for part in src5] for _ in range(L5)]
    outs5 = [torch.empty((TOKENS, HIDDEN), dtype=torch.bfloat16, device=dev) for _ in range(L5)]
    del src5

    def layers():
        for layer in range(L5):
            taco.decompress_sum(slots5[layer], B5, out=outs5[layer])

    layers()
    eager_us = time_us(layers, L5, 3)
    g5 = capture(layers)
    g5.replay()
    graph_us = time_us(g5.replay, L5, 3)
    del g5, slots5, outs5
    torch.cuda.empty_cache()

    N = TOKENS * HIDDEN
    bf16_bytes_step = 2 * N * 5
    value = bf16_bytes_step / (ms_step / 1e3) / 1e9
    alg = {
        "compress": 2 * N + N + 4 * nscales + 4,
        "decompress": N + 4 * nscales + 4 + 2 * N,
        "decompress_sum": NPARTS * (N + 4 * nscales + 4) + 2 * N,
        "decompress_sum_compress": NPARTS * (N + 4 * nscales + 4) + N + 4 * nscales + 4,
        "compress_blockscale": 3 * N + 8 * nscales,
        "decompress_blockscale": 3 * N + 8 * nscales,
        "compress_delayed": 3 * N + 4 * nscales + 4,
        "compress_int8_tensor": 3 * N + 4,
        "decompress_int8_tensor": 3 * N + 4,
        "compress_int8_block": 3 * N + 4 * nscales,
        "decompress_int8_block": 3 * N + 4 * nscales,
    }
    achieved = alg["compress"] / (avg_us["compress"] * 1e-6) / 1e9
    counters = measured_counters()
    traffic = counters.get("traffic_bytes_per_call")
    mfma_insts = counters.get("mfma_instructions_per_call")
    mfma = None
    if mfma_insts:
        # v_mfma_f32_16x16x32_bf16: 16 x 16 x 32 multiply-adds per instruction
        executed = mfma_insts * 16 * 16 * 32 * 2 / (avg_us["compress"] * 1e-6) / 1e12
        dense = 2 * BLOCK * N / (avg_us["compress"] * 1e-6) / 1e12
        mfma = {"instructions_per_call": mfma_insts,
                "executed_TFLOPs": round(executed, 1),
                "dense_contraction_TFLOPs": round(dense, 1),
                "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                "frac": round(executed / MFMA_BF16_PEAK_TFLOPS, 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "GPT-3-6.7B-shaped TP layer, bf16 [4096, 4096], block 128, target energy 1.0: "
                        "compress+decompress of the forward activation and of the backward gradient, "
                        "plus decompress_sum of 4 compressed partial sums",
            "tokens": TOKENS, "hidden": HIDDEN, "block": BLOCK, "decompress_sum_parts": NPARTS,
            "rotating_buffer_sets": args.rotate,
            "rotating_bytes": set_bytes * args.rotate,
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "kernel": ("compress_fused_lds_kernel (single pass)" if taco.get_single_pass()
                       else "compress_stats_mfma_kernel + compress_quant_mfma_kernel"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": alg["compress"],
            "avg_us": round(avg_us["compress"], 3),
            "mfma": mfma,
        },
        "ops": {
            op: {"avg_us": round(avg_us[op], 3),
                 "bf16_GBps": round(2 * N / (avg_us[op] * 1e-6) / 1e9, 1),
                 "algorithmic_GBps": round(alg[op] / (avg_us[op] * 1e-6) / 1e9, 1),
                 "hbm_frac": round(alg[op] / (avg_us[op] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            for op in ops
        },
        "extra_ops": {
            op: {"avg_us": round(avg_us[op], 3),
                 "algorithmic_GBps": round(alg[op] / (avg_us[op] * 1e-6) / 1e9, 1),
                 "hbm_frac": round(alg[op] / (avg_us[op] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            for op in extra
        },
        "extra_ops_note": "not part of the step: decompress_sum_compress (4 parts -> FP8 of their bf16 "
                          "sum), the per-block-guard and delayed-scale Dual-Scale variants, and the INT8 "
                          "degrade path (absmax per tensor: two kernels, x read twice; per 128-block)",
        "warm_ops": {op: {"avg_us": round(v, 3),
                          "algorithmic_GBps": round(alg[op] / (v * 1e-6) / 1e9, 1)} for op, v in warm_us.items()},
        "warm_ops_note": "Infinity-Cache resident: back-to-back calls on one buffer set; not the metric",
        "decompress_sum_32_layers": {
            "block": B5, "parts": NPARTS, "layers": L5,
            "us_per_layer_eager_launches": round(eager_us, 3),
            "us_per_layer_one_graph": round(graph_us, 3),
            "launch_gap_us_per_layer": round(eager_us - graph_us, 3),
            "algorithmic_GBps_one_graph": round((NPARTS * (N + 4 * (N // B5) + 4) + 2 * N) / (graph_us * 1e-6) / 1e9, 1)},
        "wall_s_timed": round(t_wall, 4),
        "timing": "steps replayed as HIP graphs of one step per buffer set (each step all 5 calls); per-op "
                  f"figures from graphs of back-to-back calls, {OP_PASSES} passes over all buffer sets",
    }
    if args.all_configs:
        out["configs"] = time_configs(taco, W, dev, stream, capture, time_us)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_rows, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
