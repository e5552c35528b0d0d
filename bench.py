"""Benchmark of the fused MoE layer (moe_layer_forward) on one MI355X.

A step is one moe_layer_forward over one batch: router logits, top-k + weights, dispatch,
gate/up + SwiGLU, down projection and combine. Inputs are seeded synthetic tensors resident in
HBM before timing.

The headline (`value`, `ms_per_step`, `roofline`, `cpu_baseline`) is the ZONOS2-shaped skewed
prefill (T=8192 tokens, d=2048, 16 experts, top-1, expert hidden 2816, bf16 weights, fp32
accumulation; expert 0 takes ~40 % of the tokens and two experts none), the largest of the five
workloads and the batched regime where the experts run as a grouped GEMM. The other four
workloads (the fp32 correctness layer, the ZONOS2 and ZONOS3-Mini decode steps, the ZONOS3-Mini
prefill) are timed in the same run and reported under `workloads`, each with its own roofline.

Cold weights: each workload's expert weights are kept in several identical copies and
consecutive steps rotate through them, so that no step finds its weights in the 256 MB Infinity
Cache left over from the step before (the copies together exceed 1.5 GB). The steps are replayed
from HIP graphs (the decode loop of the pages replays a captured graph): one graph holding a whole
cycle of steps over the copies, and one single-step graph per copy for a partial cycle, so that the
timed region runs exactly `--steps` steps after exactly `--warmup` untimed ones, bracketed by
synchronizations. `value` = T / (wall time per step).

Kernel durations come from a second, host-launched pass over the same copies with the layer's
profiling events (moe_layer_args.prof_events): the gate/up kernel, the roofline's dominant kernel,
is launched with its own start/stop events (hipExtLaunchKernelGGL), so its duration is the
kernel's alone.

Prints one JSON line (see `result` in main()).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
HBM_READ_CEILING_GBS = 6436.0  # measured on this MI355X: plain streaming read of 1 GiB, 1024 blocks
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector, published
STAGES = ("route", "dispatch", "gate_up", "down_combine")

METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA TFLOP/s vs MI355X peak"
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "traffic.md")
# sources the expert kernels are built from; the counter-based traffic figure is only reported
# while these are unchanged since the counters were taken
KERNEL_SOURCES = ("expert_routing_grouped_moe_amd/csrc/ffn_bf16.hip",
                  "expert_routing_grouped_moe_amd/csrc/common.hpp",
                  "expert_routing_grouped_moe_amd/csrc/down_epilogue.hpp",
                  "expert_routing_grouped_moe_amd/csrc/kernels.hpp")


def _code_only(text: str) -> str:
    """Source text without // and /* */ comments, whitespace runs collapsed: an edit of comments
    or layout leaves the hash (and the counters it keys) valid."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter table
    (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel calibration), or None when the
    table has no row for it or the kernel sources changed since it was measured."""
    if not os.path.exists(TRAFFIC_TABLE):
        return None
    want = kernel_source_hash()
    with open(TRAFFIC_TABLE) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) < 7 or cells[0] != kernel or cells[1] != workload:
                continue
            if cells[2] != want:
                return None
            fetch_kib, write_kib, sf, sw = (float(c) for c in cells[3:7])
            return (fetch_kib * sf + write_kib * sw) * 1024.0
    return None


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


# fragment-major weight options and the row-major storage they reorder
FRAG_BASE = {"frag": "native", "int8-frag": "int8", "q4-frag": "q4"}


def algorithmic(inp, counts, weights="native"):
    """Bytes and FLOPs the step must move/do (touched experts only; intermediates excluded).
    int8 expert weights: one byte per weight plus the fp32 row scales of the touched experts;
    q4: half a byte per weight plus one 4-byte (scale, bias) pair per group of 64; the
    fragment-major orders move the same bytes as the row-major ones."""
    weights = FRAG_BASE.get(weights, weights)
    T, d, E, k, H = inp.T, inp.d, inp.E, inp.k, inp.H
    ab = 2 if inp.dtype == "bf16" else 4             # activations and router weights
    wb = {"int8": 1, "q4": 0.5}.get(weights, ab)     # expert weights
    sb = 4 if weights == "int8" else 0               # one fp32 scale per expert weight row
    if weights == "q4":
        wb += 4 / 64                                 # (scale, bias) pair per group of 64
    touched = int((counts > 0).sum())
    rows = T * k
    step_bytes = (touched * (3 * d * H * wb + (2 * H + d) * sb) + T * d * ab + E * d * ab +
                  T * d * 4 + rows * 8)
    step_flops = 6 * d * H * rows + 2 * T * d * E
    # the gate/up kernel alone: its weights (and scales), the gathered x rows, the fp16 h it writes
    gu_bytes = touched * (2 * d * H * wb + 2 * H * sb) + rows * d * ab + rows * H * ab
    gu_flops = 4 * d * H * rows
    return dict(touched=touched, step_bytes=step_bytes, step_flops=step_flops, gu_bytes=gu_bytes,
                gu_flops=gu_flops)


def ladder_timing(moe, inp, x, wr, copies, rb, sb, steps, quant=False, w_format="plain"):
    """Serving-side decode with a changing batch width: `steps` steps whose token counts are drawn
    uniformly from 1..T (seeded), run as direct moe_layer_forward calls, as replays of a graph
    ladder with one bucket per batch width, and as replays of a ladder with power-of-two buckets
    (padding rows are extra tokens: more experts touched). One ladder per weight copy, as the
    steps rotate through the copies. Reports microseconds per step and tokens per second."""
    import numpy as np
    import torch
    T, k = inp.T, inp.k
    rng = np.random.default_rng(1234)
    ts = rng.integers(1, T + 1, size=steps)
    pow2 = sorted({min(T, 1 << i) for i in range(T.bit_length() + 1)})
    exact = list(range(1, T + 1))
    stream = torch.cuda.Stream()
    qs = lambda c: ((c["w_gate_scale"], c["w_up_scale"], c["w_down_scale"]) if quant else None)
    mk = lambda buckets: [moe.MoeGraphLadder(x, wr, c["w_gate"], c["w_up"], c["w_down"], k,
                                             inp.scoring, buckets, router_bias=rb, sel_bias=sb,
                                             w_scales=qs(c), stream=stream, w_format=w_format)
                          for c in copies]
    ladders = {"ladder": mk(exact), "ladder_pow2": mk(pow2)}
    ys = [torch.empty((T, inp.d), dtype=torch.float32, device=x.device) for _ in copies]
    wss = [torch.empty(max(1, moe.moe_workspace_size(T, inp.d, inp.E, inp.H, k, moe.MOE_BF16
                                                      if inp.dtype == "bf16" else moe.MOE_F32)),
                       dtype=torch.uint8, device=x.device) for _ in copies]

    def direct(i, t):
        c = copies[i % len(copies)]
        moe.moe_layer_forward(x[:t], wr, c["w_gate"], c["w_up"], c["w_down"], k, inp.scoring,
                              router_bias=rb, sel_bias=sb, y=ys[i % len(copies)][:t],
                              workspace=wss[i % len(copies)], stream=stream, w_scales=qs(c),
                              w_format=w_format)

    def replay(name):
        return lambda i, t: ladders[name][i % len(copies)].run(int(t), stream)

    out = {"steps": steps, "batch_widths": "uniform 1..%d, seed 1234" % T,
           "ladder_buckets": "1..%d" % T, "ladder_pow2_buckets": pow2}
    with torch.cuda.stream(stream):
        for name, fn in (("direct", direct), ("ladder", replay("ladder")),
                         ("ladder_pow2", replay("ladder_pow2"))):
            for i in range(min(steps, 20)):
                fn(i, int(ts[i]))
            stream.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                fn(i, int(ts[i]))
            stream.synchronize()
            el = time.perf_counter() - t0
            out[name + "_us_per_step"] = el / steps * 1e6
            out[name + "_tokens_per_s"] = float(ts.sum()) / el
    for lads in ladders.values():
        for lad in lads:
            lad.close()
    return out


def _spread(ms):
    """Median, p10 and p90 of per-step times given in ms, in us."""
    v = sorted(ms)
    pick = lambda q: v[min(len(v) - 1, int(q * len(v)))] * 1e3
    return {"median": statistics.median(v) * 1e3, "p10": pick(0.1), "p90": pick(0.9), "n": len(v)}


def cpu_baseline(inp, budget_s: float):
    """The fp64 oracle as it stands, timed on this host on the same workload: with the BLAS
    threads numpy starts with (all host cores), then on one thread for a shorter budget."""
    import oracle.moe_oracle as orc
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = os.cpu_count() or 1
    tokens = inp.T
    sample = f"full step ({inp.T} tokens)"
    x = inp.x
    if inp.T > 1024:
        tokens = 512
        x = inp.x[:tokens]
        sample = f"first {tokens} of {inp.T} tokens"

    def timed(budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            orc.layer_ref(x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, inp.k, inp.scoring,
                          router_bias=inp.router_bias, sel_bias=inp.sel_bias)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 50:
                return reps, el

    reps, el = timed(budget_s)
    out = {"value": tokens * reps / el, "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle", "sample": f"{sample} x {reps} runs, {el:.1f} s, numpy fp64"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            reps1, el1 = timed(budget_s / 2)
        out["single_thread"] = {"value": tokens * reps1 / el1, "unit": "tokens/s", "cores": 1,
                                "sample": f"{sample} x {reps1} runs, {el1:.1f} s"}
    return out


HEADLINE = "zonos2-skewed-prefill"
FIVE = ("tiny-fp32", "zonos2-decode", "zonos3mini-decode-cfg", "zonos3mini-prefill",
        "zonos2-skewed-prefill")


def dominant_kernel(inp, weights="native"):
    """The gate/up kernel instantiation the library picks for this shape (the dominant kernel of
    every workload): the weight-streaming kernel for few rows per expert (two-group passes where
    the whole grid stays resident: (H / 16) * E <= 2048 blocks), else the grouped GEMM."""
    T, d, E, k, H = inp.T, inp.d, inp.E, inp.k, inp.H
    if inp.dtype != "bf16":
        return "ffn_f32_kernel<true>"
    if T * k <= 2048 and d % 256 == 0 and H % 256 == 0 and T * k <= 32 * E:
        maxg = 2 if (H // 16) * E <= 2048 else 1
        return "ffn_stream_kernel<true, %d, %d>" % (maxg, {"native": 0, "int8": 1, "q4": 2, "frag": 4,
                                                           "int8-frag": 5, "q4-frag": 6}[weights])
    # fragment-major bf16 stacks run the GEMM's fragment-major variant
    return gemm_kernel_name(T * k, E, True, frag=weights == "frag")


def gemm_kernel_name(rows, E, gateup, frag=False):
    """Name of the grouped-GEMM instantiation for `rows` assignment rows over E experts (the last
    template argument: weight stacks fragment-major)."""
    if rows >= 256 * E:     # experts average a full 256-row tile: the wide tiles
        shape = "true, 256, 256, 2, 64, 64" if gateup else "false, 256, 128, 3, 64, 32"
    else:
        shape = "true, 128, 256, 3, 64, 32" if gateup else "false, 128, 256, 3, 64, 32"
    return "gemm_dma_kernel<%s, %s>" % (shape, "true" if frag else "false")


def ep_shard_timing(gpus=8, calls=48):
    """One GPU's share of expert parallelism at its real shape, on this one GPU: the skewed
    prefill's 16 experts split over `gpus` GPUs, the share that owns experts 0..16/gpus - 1 (expert
    0 takes ~40 % of the tokens: the busiest shard). The routing comes from the library
    (moe_router_logits + moe_route on the whole batch), the shard's token rows are gathered on the
    host side of the boundary, grouped with moe_permute and run through moe_expert_ffn with cold
    weights (rotating copies past the Infinity Cache); back-to-back calls, mean per call. The
    all-to-all exchange around it is not run (one GPU); its bytes are reported."""
    import numpy as np
    import torch
    from expert_routing_grouped_moe_amd import inputs as gen
    from expert_routing_grouped_moe_amd import moe

    dev = "cuda:0"
    inp = gen.make_inputs(HEADLINE)
    T, d, E, k, H = inp.T, inp.d, inp.E, inp.k, inp.H
    if gpus < 2 or E % gpus:
        return {"gpus": gpus, "error": f"{E} experts do not split evenly over {gpus} GPUs"}
    per = E // gpus
    bf = lambda key: torch.from_numpy(inp.bits[key].view(np.int16)).view(torch.bfloat16).to(dev)
    x = bf("x")
    rb = torch.from_numpy(inp.router_bias).to(dev)
    logits = moe.moe_router_logits(x, bf("w_router"), router_bias=rb)
    ids, _, _ = moe.moe_route(logits, k, inp.scoring)
    ids_h = ids.cpu().numpy()
    tokens = np.nonzero((ids_h[:, 0] >= 0) & (ids_h[:, 0] < per))[0]
    x_sh = x[torch.from_numpy(tokens).to(dev)].contiguous()
    local = ids[torch.from_numpy(tokens).to(dev)].contiguous()
    counts = torch.bincount(local.view(-1).long(), minlength=per).to(torch.int32)
    offsets, rows, _ = moe.moe_permute(local, counts, per)
    base = {key: bf(key)[:per].contiguous() for key in ("w_gate", "w_up", "w_down")}
    wbytes = sum(t.numel() * t.element_size() for t in base.values())
    ncopies = max(2, math.ceil(1.6e9 / wbytes))
    copies = [base] + [{key: t.clone() for key, t in base.items()} for _ in range(ncopies - 1)]
    n = len(tokens)
    out = torch.empty((n, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, moe.moe_workspace_size(n, d, per, H, k, moe.MOE_BF16)),
                     dtype=torch.uint8, device=dev)
    call = lambda c: moe.moe_expert_ffn(x_sh, c["w_gate"], c["w_up"], c["w_down"], k, offsets,
                                        rows, expert_out=out, workspace=ws)
    for c in copies:
        call(c)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(calls):
        call(copies[i % ncopies])
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / calls * 1e6
    flops = 6.0 * d * H * n
    return {"gpus": gpus, "experts": list(range(per)), "rows": counts.cpu().tolist(),
            "us_per_call": us, "tflops": flops / us / 1e6,
            "mfma_frac": flops / us / 1e6 / BF16_PEAK_TFLOPS,
            "exchange_bytes": {"x_rows_in_bf16": n * d * 2, "outputs_back_fp32": n * d * 4},
            "note": "moe_expert_ffn on one GPU's expert share, cold weights; the all-to-alls "
                    "around it are not run (one GPU)"}


def run_workload(name, steps, warmup, weights="native", warm=False, eager=False, ladder=0,
                 cpu_budget=0.0, event_steps=200):
    """Times `steps` layer steps of workload `name` (after `warmup` untimed ones) and returns its
    summary: ms/step, tokens/s, the dominant kernel's roofline, the step's HBM and MFMA
    fractions, per-stage medians from the event pass and, when cpu_budget > 0, the oracle's
    timing on this host."""
    import numpy as np
    import torch
    from expert_routing_grouped_moe_amd import inputs as gen
    from expert_routing_grouped_moe_amd import moe

    dev = "cuda:0"
    inp = gen.make_inputs(name)
    T, d, E, k, H = inp.T, inp.d, inp.E, inp.k, inp.H
    dt_code = moe.MOE_BF16 if inp.dtype == "bf16" else moe.MOE_F32

    def up(key):
        if inp.dtype == "bf16":
            return torch.from_numpy(inp.bits[key].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(getattr(inp, key)).to(dev)

    x = up("x")
    wr = up("w_router")
    base = {key: up(key) for key in ("w_gate", "w_up", "w_down")}
    stored = FRAG_BASE.get(weights, weights)
    quant = stored in ("int8", "q4")
    w_format = "frag" if weights in FRAG_BASE else "plain"
    if quant:
        qfn = moe.moe_quantize_rows_i8 if stored == "int8" else moe.moe_quantize_groups_q4
        qs = {key: qfn(t) for key, t in base.items()}
        base = {key: v[0] for key, v in qs.items()}
        base.update({key + "_scale": v[1] for key, v in qs.items()})
        torch.cuda.synchronize()
    if w_format == "frag":
        for key in ("w_gate", "w_up", "w_down"):
            base[key] = moe.moe_pack_weights_frag(base[key])
        torch.cuda.synchronize()
    wbytes = sum(t.numel() * t.element_size() for t in base.values())
    ncopies = 1 if warm else max(2, min(16, math.ceil(1.6e9 / wbytes)))
    copies = [base] + [{key: t.clone() for key, t in base.items()} for _ in range(ncopies - 1)]
    rb = None if inp.router_bias is None else torch.from_numpy(inp.router_bias).to(dev)
    sb = None if inp.sel_bias is None else torch.from_numpy(inp.sel_bias).to(dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    counts = torch.zeros((E,), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, moe.moe_workspace_size(T, d, E, H, k, dt_code)), dtype=torch.uint8,
                     device=dev)

    hip = _hip()
    nev = moe.MOE_PROF_EVENTS
    events, ev_arrays, arg_list = [], [], []
    for c in range(ncopies):
        evs = []
        for _ in range(nev):
            h = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(h)) == 0
            evs.append(h)
        events.append(evs)
        ev_arrays.append((ctypes.c_void_p * nev)(*[e.value for e in evs]))
        scales = ((copies[c]["w_gate_scale"], copies[c]["w_up_scale"], copies[c]["w_down_scale"])
                  if quant else None)
        arg_list.append(moe.make_layer_args(x, wr, copies[c]["w_gate"], copies[c]["w_up"],
                                            copies[c]["w_down"], k, inp.scoring, y, rb, sb,
                                            expert_counts=counts, w_scales=scales,
                                            w_format=w_format))

    stream = torch.cuda.Stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def one_step(c, with_events):
        a = arg_list[c]
        a.prof_events = ctypes.cast(ev_arrays[c], ctypes.c_void_p).value if with_events else None
        st = moe.LIB.moe_layer_forward(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()),
                                       ws.numel(), sptr)
        if st != 0:
            raise moe.MoeError(st, "moe_layer_forward")

    # eager warm-up of every copy (validates the call), then one graph per copy, one step each
    with torch.cuda.stream(stream):
        for c in range(ncopies):
            one_step(c, False)
    torch.cuda.synchronize()
    graphs = []
    for c in range(ncopies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            one_step(c, False)
        graphs.append(g)
    # one more graph holding a whole cycle of steps (copies 0 .. ncopies-1 in order): replayed
    # where a cycle fits, so that fewer graph launches sit between steps; the single-step graphs
    # cover the rest, so exactly the requested number of steps runs
    cycle = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cycle, stream=stream):
        for c in range(ncopies):
            one_step(c, False)
    y.fill_(float("nan"))
    graphs[0].replay()
    torch.cuda.synchronize()
    assert not torch.isnan(y).any().item(), "graph replay did not run the layer"

    def run_steps(n, first):
        if eager:
            with torch.cuda.stream(stream):
                for i in range(first, first + n):
                    one_step(i % ncopies, False)
            return
        i, end = first, first + n
        while i < end:
            if i % ncopies == 0 and end - i >= ncopies:
                cycle.replay()
                i += ncopies
            else:
                graphs[i % ncopies].replay()
                i += 1

    run_steps(warmup, 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(steps, warmup)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / steps * 1e3

    # event pass: host launches with a HIP event at every stage boundary, on the kernels' stream
    stage_ms = {s_: [] for s_ in STAGES}
    n_ev = max(ncopies, min(event_steps, 4 * steps))
    for i0 in range(0, n_ev, ncopies):
        with torch.cuda.stream(stream):
            for c in range(ncopies):
                one_step(c, True)
        torch.cuda.synchronize()
        for c in range(ncopies):
            for i in range(nev - 1):
                f = ctypes.c_float()
                assert hip.hipEventElapsedTime(ctypes.byref(f), events[c][i], events[c][i + 1]) == 0
                stage_ms[STAGES[i]].append(f.value)
    step_ms_ev = [sum(stage_ms[s_][i] for s_ in STAGES) for i in range(len(stage_ms["route"]))]

    cnt = counts.cpu().numpy()
    alg = algorithmic(inp, cnt, weights)
    gu_ms = statistics.mean(stage_ms["gate_up"])
    prefill = gen.WORKLOADS[name].shape == "prefill"
    if prefill:
        ach = alg["gu_flops"] / (gu_ms * 1e-3) / 1e12
        gbs = alg["gu_bytes"] / (gu_ms * 1e-3) / 1e9
        # the HBM side as well: with cold weights and about one row tile per expert the gate/up
        # product has fewer FLOPs per byte than the chip's ridge
        roof = {"bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / BF16_PEAK_TFLOPS, "traffic": None,
                "hbm_achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    else:
        ach = alg["gu_bytes"] / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": None,
                "measured_read_ceiling": HBM_READ_CEILING_GBS,
                "frac_of_measured_ceiling": ach / HBM_READ_CEILING_GBS}
    roof["kernel"] = dominant_kernel(inp, weights)
    traffic = measured_traffic(roof["kernel"], name + ("/" + weights if weights != "native" else ""))
    roof["traffic"] = traffic
    roof["traffic_source"] = ("profiles/traffic.md (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
                              if traffic is not None else "not measured for the current kernel")
    roof["avg_launch_us"] = gu_ms * 1e3
    roof["algorithmic_bytes_per_launch"] = alg["gu_bytes"]
    roof["algorithmic_flops_per_launch"] = alg["gu_flops"]

    step_s = ms_per_step * 1e-3
    out = {
        "tokens_per_s": T / step_s,
        "ms_per_step": ms_per_step,
        "steps": steps,
        "warmup": warmup,
        "dtype": inp.dtype,
        "config": {"workload": name, "T": T, "d": d, "E": E, "k": k, "H": H,
                   "scoring": inp.scoring, "seed": gen.WORKLOADS[name].seed,
                   "weights": "cold (rotating %d copies)" % ncopies if ncopies > 1 else "warm (1 copy)",
                   "expert_weights": {"int8": "int8, fp32 row scales",
                                      "q4": "4-bit affine, groups of 64, bf16 scale and bias",
                                      "frag": "bf16, fragment-major (moe_pack_weights_frag)",
                                      "int8-frag": "int8, fp32 row scales, codes fragment-major",
                                      "q4-frag": "4-bit affine, groups of 64, codes fragment-major"
                                      }.get(weights, inp.dtype),
                   "timing": ("host launches" if eager else
                              "HIP graph replay: cycles of one step per weight copy, single "
                              "steps for a partial cycle")},
        "step_hbm_gbps": alg["step_bytes"] / step_s / 1e9,
        "step_hbm_frac": alg["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBS,
        "step_tflops": alg["step_flops"] / step_s / 1e12,
        "step_mfma_frac": alg["step_flops"] / step_s / 1e12 / (
            BF16_PEAK_TFLOPS if inp.dtype == "bf16" else FP32_PEAK_TFLOPS),
        "touched_experts": alg["touched"],
        # between the [1] and [2] events the weight-streaming path runs no kernel (its expert
        # blocks find their rows themselves): that interval is the launch gap, named as such
        "stage_median_us": {("launch_gap" if s_ == "dispatch" and "ffn_stream" in roof["kernel"]
                             else s_): statistics.median(v) * 1e3 for s_, v in stage_ms.items()},
        "event_step_us": _spread(step_ms_ev),
        "roofline": roof,
    }
    if ladder:
        out["ladder"] = ladder_timing(moe, inp, x, wr, copies, rb, sb, ladder, quant=quant,
                                      w_format=w_format)
    if cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(inp, cpu_budget)
    for evs in events:
        for e in evs:
            hip.hipEventDestroy(e)
    del graphs, cycle, copies, base, x, wr, y, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE,
                    help="the headline workload (default: the skewed prefill)")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload alone (no `workloads` table)")
    ap.add_argument("--other-steps", type=int, default=200,
                    help="timed steps of each of the other workloads (warm-up: a tenth)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="one weight copy (cache-warm, labelled)")
    ap.add_argument("--weights", choices=("native", "int8", "q4", "frag", "int8-frag", "q4-frag"),
                    default="native",
                    help="expert weights as given (bf16/fp32), int8 codes with per-row scales "
                         "(moe_quantize_rows_i8), 4-bit affine codes in groups of 64 "
                         "(moe_quantize_groups_q4), or any of these three reordered fragment-major "
                         "(moe_pack_weights_frag); the codes on decode shapes only; headline "
                         "workload only")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from the host instead of graph replay (counter runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB ten times (counter calibration)")
    ap.add_argument("--ep-shard", type=int, default=8, metavar="GPUS",
                    help="also time moe_expert_ffn on the busiest expert shard of the skewed "
                         "prefill split over GPUS GPUs (one GPU's share; 0 = skip)")
    ap.add_argument("--ladder", type=int, default=0, metavar="STEPS",
                    help="also time STEPS decode steps of seeded random batch widths 1..T, launched "
                         "directly and replayed from a graph ladder (buckets 1, 2, 4, ..., T)")
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 10}))
        return

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print(json.dumps({"error": "--steps must be >= 1 and --warmup >= 0"}))
        sys.exit(2)

    head = run_workload(args.workload, args.steps, args.warmup, weights=args.weights,
                        warm=args.warm, eager=args.eager, ladder=args.ladder,
                        cpu_budget=0.0 if args.no_cpu_baseline else args.cpu_budget)
    print(f"[bench] {args.workload}: {head['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr,
          flush=True)
    others = {}
    if not args.only and args.weights == "native":
        for name in FIVE:
            if name == args.workload:
                continue
            others[name] = run_workload(name, args.other_steps, max(1, args.other_steps // 10),
                                        warm=args.warm, eager=args.eager)
            print(f"[bench] {name}: {others[name]['ms_per_step'] * 1e3:.1f} us/step",
                  file=sys.stderr, flush=True)

    # the decode workloads and the ZONOS3-Mini prefill again on fragment-major bf16 weights (same
    # values, reordered once)
    frag = {}
    if not args.only and args.weights == "native":
        for name in ("zonos2-decode", "zonos3mini-decode-cfg", "zonos3mini-prefill"):
            r = run_workload(name, args.other_steps, max(1, args.other_steps // 10), weights="frag",
                             warm=args.warm, eager=args.eager)
            frag[name] = {key: r[key] for key in ("ms_per_step", "tokens_per_s", "stage_median_us",
                                                   "event_step_us", "roofline")}
            print(f"[bench] {name} (fragment-major weights): {r['ms_per_step'] * 1e3:.1f} us/step",
                  file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "step_hbm_gbps": head["step_hbm_gbps"],
        "step_hbm_frac": head["step_hbm_frac"],
        "step_tflops": head["step_tflops"],
        "step_mfma_frac": head["step_mfma_frac"],
        "touched_experts": head["touched_experts"],
        "stage_median_us": head["stage_median_us"],
        "event_step_us": head["event_step_us"],
        "roofline": head["roofline"],
    }
    if "ladder" in head:
        result["ladder"] = head["ladder"]
    if "cpu_baseline" in head:
        result["cpu_baseline"] = head["cpu_baseline"]
    if not args.only and args.ep_shard > 1 and args.weights == "native":
        result["ep_shard"] = ep_shard_timing(args.ep_shard)
        print(f"[bench] ep shard of {args.ep_shard}: {result['ep_shard']['us_per_call']:.1f} us/call",
              file=sys.stderr, flush=True)
    if others:
        table = {args.workload: {key: v for key, v in head.items() if key != "cpu_baseline"}}
        table.update(others)
        result["workloads"] = {name: table[name] for name in FIVE if name in table}
    if frag:
        result["fragment_major_weights"] = frag
    print(json.dumps(result))


if __name__ == "__main__":
    main()
