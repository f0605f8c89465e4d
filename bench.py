"""Benchmark of the NVFP4 routed-expert layer on one MI355X.

One step = one layer forward through the C ABI (route/permute, quantize x, L1 gate+up + SiLU,
quantize h, L2 down, combine) over one batch of synthetic input already resident in HBM.

Headline (``value``): TFLOP/s of the 8192-token prefill with Zipf-skewed routing over 384
experts (hidden 7168, intermediate 2048, top-6).  Useful FLOPs are 6*H*I per (token, local
expert) assignment.  The same JSON line carries the decode workload (the 48-expert
expert-parallel share of 384 experts at T = 1, 4, 8, with 4 rotated weight copies so weights
come from HBM, not from the 256 MB last-level cache), reported as weight GB/s, where weight
bytes are the NVFP4 bytes of the experts that received at least one token.  The weights carry the
packed copy of their codes (MoEWeights.pack, nvfp4_pack_weight_codes), which the 16-row kernels read
(``--unpacked``: the row-major codes only).

``roofline`` is for the dominant kernel.  Prefill: the L1 large-tile kernel
(gemm_large_kernel<true, false>, experts with more than 16 tokens; 60% of the step), whose launch
duration is timed alone with HIP events on the stream it runs on (the same tiles routed without
the experts of at most 16 tokens, see time_large_tile_kernels); achieved = its useful FLOPs,
4*H*I per assignment of those experts, / that duration, against the 2,516.6 TFLOP/s dense fp16
MFMA peak.  Decode: the 16-row L1 kernel (the only kernel moe_grouped_gemm_l1_silu launches at
decode); achieved = the W13 bytes of the active experts / its launch duration, against 8 TB/s.
``traffic`` is that kernel's HBM bytes per dispatch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
(TRAFFIC_FILE), or null once the GEMM source has changed since the counters were taken.
``cpu_baseline`` times the CPU oracle (float64 NumPy) on a bounded sample of the prefill workload:
the layer restricted to its most-loaded expert.

The routing ids and weights of every workload come from its router logits through the GPU router
(moe_router_topk), whose time is the "router" entry of stage_ms (the timed step starts from the
ids, at route/permute).

Also reported: the other two prefill configurations (512 tokens over all 384 experts with rows
padded to 128, HBM-bound; 16,384 tokens with Zipf routing and +-8 outliers) as sub-objects with
their own step times and fractions; the step time with calibrated global scales (x and h quantized
with the scales of a warm-up forward: no amax pass); per-step p10/p50/p90; GEMM-only time (L1 + L2);
the L2 large-tile kernel alone; the decode aggregate over 64 routing seeds (sum of weight bytes over
sum of step times); and, as context only, a 1 GiB device copy and an 8192^3 fp16 GEMM from the vendor
BLAS measured on the same GPU, with this repository's own measurement kernels (csrc/probe.hip): the
HBM read rate of plain loads at the decode weight size in three access orders, the CU placement of a
two-per-CU launch, and the dense NVFP4 GEMM on random versus zero codes (the clock's dependence on
the operand data).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-seeds N] [--no-cpu-baseline] [--quick]
       [--unpacked]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer TFLOP/s + weight GB/s (% roofline) at decode and 8192-token prefill"
PEAK_FP16_TFLOPS = 2516.6   # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA (context only: this path multiplies in fp16)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
STAGES = ("router", "route", "quant_x", "l1", "quant_h", "l2", "combine")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gpu_routing(wl, T, seed=0, dev="cuda:0"):
    """Router logits of the workload, routed on the GPU (moe_router_topk): device logits, ids and
    weights, and the per-local-expert assignment counts on the host (for bookkeeping)."""
    import torch
    from nvfp4_block_scaled_top_amd import megamoe, synth

    logits = torch.from_numpy(synth.router_logits(wl, T, seed)).to(dev)
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, wl.top_k, dtype=torch.float32, device=dev)
    megamoe.moe_router_topk(logits, wl.top_k, ids, wts)
    h = ids.cpu().numpy()
    loc = h[(h >= wl.expert_begin) & (h < wl.expert_begin + wl.num_experts)] - wl.expert_begin
    return logits, ids, wts, np.bincount(loc, minlength=wl.num_experts)


# The layer's weights carry the packed copy of their codes (MoEWeights.pack), which the 16-row
# kernels read; --unpacked measures them on the row-major codes instead.
PACKED = True


def build_weights(wl, active, copies, dev):
    """NVFP4 weights for the local experts, quantized on the GPU (and packed unless --unpacked);
    experts with no token stay unset."""
    import torch
    from nvfp4_block_scaled_top_amd import layer, synth

    W = layer.MoEWeights.empty(wl.num_experts, wl.hidden, wl.intermediate, device=dev)
    for e in active:
        w13, w2 = synth.expert_weights(wl, wl.expert_begin + e, device=dev)
        layer.quantize_expert_into(W, e, w13, w2)
        del w13, w2
    if PACKED:
        W.pack()
    torch.cuda.synchronize()
    return [W] + [W.clone() for _ in range(copies - 1)]


def time_workload(wl, T, steps, warmup, copies, use_graph, fused=False):
    import torch
    from nvfp4_block_scaled_top_amd import layer, megamoe, synth

    dev = "cuda:0"
    logits, ids_d, wts_d, counts = gpu_routing(wl, T, 0, dev)
    active = [int(e) for e in np.nonzero(counts)[0]]
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(dev)
    Ws = build_weights(wl, active, copies, dev)
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        L.forward(x, ids_d, wts_d, Ws[i % copies])

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    graphs = None
    if use_graph:
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

    # Whole-step timing: exactly `steps` steps between two synchronizations.
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        if graphs is not None:
            graphs[i % copies].replay()
        else:
            step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / steps

    # Per-step spread (a second pass with an event pair around every step).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        if graphs is not None:
            graphs[i % copies].replay()
        else:
            step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    spread = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.percentile(per_step, 50)),
              "p90": float(np.percentile(per_step, 90))}

    # Variants of the step, each captured per weight copy and replayed like the default one:
    # calibrated (the global scales of x and h given, those of the warm-up forward, so neither
    # quantizer derives one from an amax) and, at decode, the fused L1 -> requantize -> L2 launch
    # with and without calibrated scales.
    def variant_ms(**kw):
        vgraphs = []
        for c in range(copies):
            L.forward(x, ids_d, wts_d, Ws[c], **kw)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                L.forward(x, ids_d, wts_d, Ws[c], **kw)
            vgraphs.append(g)
        for g in vgraphs:
            g.replay()
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for i in range(steps):
            vgraphs[i % copies].replay()
        c1.record(stream)
        torch.cuda.synchronize()
        return c0.elapsed_time(c1) / steps

    calibrated_ms = fused_ms = fused_calibrated_ms = None
    if graphs is not None:
        gx, gh = L.x_gs.clone(), L.h_gs.clone()
        calibrated_ms = variant_ms(x_gs=gx, h_gs=gh)
        if fused:
            fused_ms = variant_ms(fused=True)
            fused_calibrated_ms = variant_ms(x_gs=gx, h_gs=gh, fused=True)
            if L.ffn_sync_error():
                raise RuntimeError("a wait inside the fused launch expired")

    # Per-stage durations: a short GPU spin ahead of each stage keeps the launch latency out of
    # the event pair that brackets it.
    stage_fns = {
        "router": lambda i: megamoe.moe_router_topk(logits, wl.top_k, ids_d, wts_d),
        "route": lambda i: L.route(ids_d),
        "quant_x": lambda i: L.quantize_x(x),
        "l1": lambda i: L.l1(Ws[i % copies]),
        "quant_h": lambda i: L.quantize_h(),
        "l2": lambda i: L.l2(Ws[i % copies]),
        "combine": lambda i: L.combine(wts_d),
    }
    reps = max(3, min(steps, 20))
    stage_ms = {}
    for name in STAGES:
        tot = 0.0
        for i in range(reps):
            # restore the inputs each stage expects (they are the outputs of the previous stages)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(200_000)
            a.record(stream)
            stage_fns[name](i)
            b.record(stream)
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        stage_ms[name] = tot / reps
    assign = int(counts.sum())
    flops = 6.0 * wl.hidden * wl.intermediate * assign
    wbytes = len(active) * Ws[0].nbytes_expert()
    w13_bytes = len(active) * (Ws[0].w13_codes[0].numel() + Ws[0].w13_scales[0].numel() + 4)
    del Ws, graphs
    torch.cuda.synchronize()
    return dict(T=T, ms_per_step=ms_per_step, wall_s=wall, stage_ms=stage_ms, spread=spread,
                calibrated_ms=calibrated_ms, fused_ms=fused_ms, fused_calibrated_ms=fused_calibrated_ms,
                assignments=assign,
                active_experts=len(active), flops=flops, weight_bytes=wbytes, w13_bytes=w13_bytes,
                l1_flops=4.0 * wl.hidden * wl.intermediate * assign)


def time_large_tile_kernels(wl, T, reps):
    """Launch duration of the 256-row (large-tile) GEMM kernels of the prefill workload, alone.

    moe_grouped_gemm_l1_silu launches the large-tile kernel for experts with more than 16 tokens and
    then the 16-row kernel for the others.  To time the large-tile kernel by itself with HIP events,
    the same ids are routed with every expert of at most 16 tokens made non-local (id -1) and with
    block_m_override 256: the call then launches gemm_large_kernel<true, false> only, over exactly
    the same tiles as in the full workload (same experts, counts, 256x256 and 128x512 tiles, order),
    only at other row offsets.  The same for the L2 kernel gemm_large_kernel<false, false>.  Each
    launch is timed with an event pair on the stream it runs on, after a short GPU spin."""
    import torch
    from nvfp4_block_scaled_top_amd import layer, synth

    dev = "cuda:0"
    logits, ids_d, wts_d, counts = gpu_routing(wl, T, 0, dev)
    large = np.nonzero(counts > 16)[0]
    ids = ids_d.cpu().numpy()
    loc = ids - wl.expert_begin
    keep = np.isin(loc, large)
    ids_l = np.where(keep, ids, -1).astype(np.int32)
    n_assign = int(keep.sum())
    Ws = build_weights(wl, [int(e) for e in large], 1, dev)
    W = Ws[0]
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin, block_m_override=256, device=dev)
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).to(dev)
    L.forward(x, torch.from_numpy(ids_l).to(dev), wts_d, W)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    out = {}
    for name, fn in (("l1", lambda: L.l1(W)), ("l2", lambda: L.l2(W))):
        fn()
        tot = 0.0
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(200_000)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        out[name] = tot / reps
    del Ws, W, L
    torch.cuda.synchronize()
    H, I = wl.hidden, wl.intermediate
    return {"l1_ms": out["l1"], "l2_ms": out["l2"], "assignments": n_assign, "experts": int(len(large)),
            "l1_flops": 4.0 * H * I * n_assign, "l2_flops": 2.0 * H * I * n_assign}


def prefill_config_entry(wl, steps, warmup, use_graph):
    """The whole-layer numbers of one more prefill configuration (a sub-object of the line)."""
    T = wl.tokens[0]
    log(f"[bench] prefill {wl.name} T={T}")
    r = time_workload(wl, T, steps, warmup, copies=1, use_graph=use_graph)
    sec = r["ms_per_step"] * 1e-3
    tflops, gbs = r["flops"] / sec / 1e12, r["weight_bytes"] / sec / 1e9
    log(f"[bench] prefill {wl.name}: {r['ms_per_step']:.3f} ms/step, {tflops:.1f} TFLOP/s, {gbs:.0f} GB/s")
    return {"tokens": T, "ms_per_step": round(r["ms_per_step"], 4),
            "ms_per_step_p10_p50_p90": [round(r["spread"][q], 4) for q in ("p10", "p50", "p90")],
            "TFLOPs": round(tflops, 2), "mfma_frac": round(tflops / PEAK_FP16_TFLOPS, 4),
            "weight_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "active_experts": r["active_experts"], "assignments": r["assignments"], "weight_bytes": r["weight_bytes"],
            "pad_multiple": wl.pad_multiple,
            "calibrated_gs_ms_per_step": None if r["calibrated_ms"] is None else round(r["calibrated_ms"], 4),
            "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
            "gemm_ms": round(r["stage_ms"]["l1"] + r["stage_ms"]["l2"], 4)}


def decode_seed_aggregate(wl, seeds, reps, copies=4, **fwd_kw):
    """Decode over routing seeds 0..seeds-1 at every T of the workload: sum of algorithmic weight
    bytes over sum of step times (all 48 local experts quantized once, `copies` rotated copies;
    one graph per seed and T holds `copies` layer forwards, one per weight copy).  fwd_kw: options
    of the layer forward (fused=True: the L1 -> requantize -> L2 launch)."""
    import torch
    from nvfp4_block_scaled_top_amd import layer, synth

    dev = "cuda:0"
    Ws = build_weights(wl, list(range(wl.num_experts)), copies, dev)
    per_expert = Ws[0].nbytes_expert()
    stream = torch.cuda.current_stream()
    res = {}
    for T in wl.tokens:
        L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                           expert_begin=wl.expert_begin, device=dev)
        tot_bytes, tot_ms, tot_active, empty = 0, 0.0, 0, 0
        for seed in range(seeds):
            _, idd, wtd, counts = gpu_routing(wl, T, seed, dev)
            nact = int(np.count_nonzero(counts))
            x = torch.from_numpy(synth.activations(wl, T, seed).view(np.int16)).to(dev)
            for c in range(copies):
                L.forward(x, idd, wtd, Ws[c], **fwd_kw)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(copies):
                    L.forward(x, idd, wtd, Ws[c], **fwd_kw)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            tot_ms += a.elapsed_time(b) / (reps * copies)
            tot_bytes += nact * per_expert
            tot_active += nact
            empty += nact == 0
            del g
        gbs = tot_bytes / (tot_ms * 1e-3) / 1e9
        res[f"T{T}"] = {"seeds": seeds, "weight_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                        "mean_us_per_step": round(tot_ms / seeds * 1e3, 2),
                        "mean_active_experts": round(tot_active / seeds, 3), "seeds_without_local_work": empty}
        log(f"[bench] decode T={T} over {seeds} seeds{' ' + str(fwd_kw) if fwd_kw else ''}: {gbs:.0f} GB/s, "
            f"{tot_ms / seeds * 1e3:.1f} us/step")
        del L
    del Ws
    torch.cuda.synchronize()
    return res


def dense_linear_bench(reps=20):
    """nvfp4_linear (the L2 GEMM with one group of every row) at a prefill shape (M=8192, K=7168,
    N=2048: TFLOP/s) and a decode shape (M=8, same K and N: weight GB/s); operands quantized on the
    GPU from random bf16."""
    import torch
    from nvfp4_block_scaled_top_amd import layer, megamoe

    res = {}
    stream = torch.cuda.current_stream()
    K, N = 7168, 2048
    w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
    wc = torch.empty(N, K // 2, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(N, K // 16, dtype=torch.uint8, device="cuda")
    wg = torch.empty(1, dtype=torch.float32, device="cuda")
    layer.quantize_matrix(w, wc, wsc, wg)
    wbytes = wc.numel() + wsc.numel() + 4
    for M in (8192, 8):
        a = (torch.randn(M, K, device="cuda") * 0.09).to(torch.bfloat16)
        ac = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
        asc = torch.empty(M, K // 16, dtype=torch.uint8, device="cuda")
        ag = torch.empty(1, dtype=torch.float32, device="cuda")
        layer.quantize_matrix(a, ac, asc, ag)
        out = torch.empty(M, N, dtype=torch.int16, device="cuda")
        ws = torch.empty(megamoe.megamoe_dense_workspace_bytes(M), dtype=torch.uint8, device="cuda")
        call = lambda: megamoe.nvfp4_linear(ac, asc, ag, wc, wsc, wg, out, ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[f"M{M}_K{K}_N{N}"] = {"ms": round(ms, 5), "TFLOPs": round(2.0 * M * K * N / (ms * 1e-3) / 1e12, 2),
                                  "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1)}
        log(f"[bench] dense linear M={M}: {ms * 1e3:.1f} us, {res[f'M{M}_K{K}_N{N}']['TFLOPs']} TFLOP/s")
    return res


def measured_ceilings():
    """Achievable ceilings on this GPU: a 1 GiB device copy (read + write bytes) and an 8192^3 fp16
    GEMM from the vendor BLAS (torch.matmul)."""
    import torch

    stream = torch.cuda.current_stream()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    n = 8192
    a = torch.randn(n, n, dtype=torch.float16, device="cuda")
    bm = torch.randn(n, n, dtype=torch.float16, device="cuda")
    out = {}
    for name, fn, work in (("hbm_copy_GBps", lambda: dst.copy_(src), 2 * COPY_BYTES / 1e9),
                           ("fp16_gemm_TFLOPs", lambda: torch.matmul(a, bm), 2.0 * n ** 3 / 1e12)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = round(work * 10 / (e0.elapsed_time(e1) * 1e-3), 1)
    del src, dst, a, bm
    torch.cuda.synchronize()
    out["hbm_read"] = hbm_read_ceilings()
    out["decode_gemm_load_stream"] = gemm_stream_ceilings()
    out["workgroup_placement"] = placement_check()
    out["dense_nvfp4_gemm_operand_data"] = dense_data_dependence()
    return out


def probe_lib():
    """bench.py's measurement kernels (csrc/probe.hip, built by __graft_entry__.build())."""
    import ctypes

    from nvfp4_block_scaled_top_amd import build_lib

    if not os.path.exists(build_lib.PROBE_LIB_PATH):
        raise RuntimeError(f"{build_lib.PROBE_LIB_PATH} is missing: run __graft_entry__.build()")
    h = ctypes.CDLL(build_lib.PROBE_LIB_PATH)
    h.megamoe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    h.megamoe_probe_read.restype = ctypes.c_int
    h.megamoe_probe_placement.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    h.megamoe_probe_placement.restype = ctypes.c_int
    h.megamoe_probe_gemm_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p]
    h.megamoe_probe_gemm_stream.restype = ctypes.c_int
    return h


def gemm_stream_ceilings(experts=9, copies=4, reps=100):
    """Read rate (GB/s) of the 16-row L1 GEMM's weight-code stream at decode T=8 (9 active experts'
    W13 codes, 132 MB) with the kernel's launch shape and load structure but no arithmetic
    (csrc/probe.hip, megamoe_probe_gemm_stream): in the kernel's addressing of the row-major codes, in
    a workgroup-contiguous order, and in its addressing of the packed codes with non-temporal loads;
    `copies` rotated buffers keep it out of the last-level cache."""
    import torch

    lib = probe_lib()
    stream = torch.cuda.current_stream()
    nbytes = experts * 4096 * 3584
    bufs = [torch.full((nbytes,), 0x35 + i, dtype=torch.uint8, device="cuda") for i in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    res = {"bytes": nbytes}
    for name, pattern in (("gemm_addressing_GBps", 0), ("workgroup_contiguous_GBps", 1),
                          ("packed_codes_nontemporal_GBps", 2)):
        def run(i):
            rc = lib.megamoe_probe_gemm_stream(bufs[i % copies].data_ptr(), nbytes, experts, pattern,
                                               sink.data_ptr(), ctypes_stream(stream))
            if rc != 0:
                raise RuntimeError(f"megamoe_probe_gemm_stream failed ({rc})")
        for i in range(3):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = round(nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)
    log(f"[bench] decode GEMM load stream without arithmetic: {res}")
    del bufs
    return res


# (name, order, grid, loads in flight per thread): order 0 = all workgroups read neighbouring bytes
# at any moment, 1 = one contiguous slab per workgroup, 2 = one contiguous eighth per XCD.
READ_ORDERS = (("global_order_2048wg", 0, 2048, 1), ("global_order_512wg", 0, 512, 4),
               ("xcd_eighths_512wg", 2, 512, 4), ("workgroup_slabs_512wg", 1, 512, 4))


def hbm_read_ceilings(nbytes=149 * 2 ** 20, copies=4, reps=100):
    """HBM read rate (GB/s) of a plain 16-byte-load kernel over `nbytes` (the decode L1 weight bytes
    at T=8), rotating over `copies` buffers so that the 256 MB last-level cache does not hold them,
    in the access orders of READ_ORDERS."""
    import torch

    lib = probe_lib()
    stream = torch.cuda.current_stream()
    bufs = [torch.full((nbytes,), i + 1, dtype=torch.uint8, device="cuda") for i in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    res = {"bytes": nbytes}
    for name, order, grid, unroll in READ_ORDERS:
        def run(i):
            rc = lib.megamoe_probe_read(bufs[i % copies].data_ptr(), nbytes, order, grid, unroll, sink.data_ptr(),
                                        ctypes_stream(stream))
            if rc != 0:
                raise RuntimeError(f"megamoe_probe_read failed ({rc})")
        for i in range(3):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_GBps"] = round(nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)
    log(f"[bench] HBM read ceilings: {res}")
    del bufs
    return res


def ctypes_stream(stream):
    return stream.cuda_stream


def placement_check():
    """Whether the two workgroups of a 512-workgroup, two-per-CU launch that share a CU are b and
    b + 256 (the 16-row GEMM gives those neighbouring work ranges), read from HW_ID / XCC_ID."""
    import torch

    lib = probe_lib()
    out = torch.zeros(2 * 512, dtype=torch.int32, device="cuda")
    rc = lib.megamoe_probe_placement(out.data_ptr(), 512, ctypes_stream(torch.cuda.current_stream()))
    if rc != 0:
        raise RuntimeError(f"megamoe_probe_placement failed ({rc})")
    torch.cuda.synchronize()
    h = out.cpu().numpy().astype(np.uint32).reshape(512, 2)
    hw, xcc = h[:, 0], h[:, 1]
    # HW_ID: CU in bits 8-11, shader array bit 12, shader engine bits 13-15
    cu_key = [(int(xcc[b]), int((hw[b] >> 13) & 7), int((hw[b] >> 12) & 1), int((hw[b] >> 8) & 15)) for b in range(512)]
    by_cu = {}
    for b, k in enumerate(cu_key):
        by_cu.setdefault(k, []).append(b)
    pairs_ok = all(len(v) == 2 and v[1] - v[0] == 256 for v in by_cu.values())
    # the XCD of workgroup 0 depends on where the previous dispatch left the round-robin; what the
    # tile mappings use is that workgroups with equal b mod 8 share an XCD
    xcd_ok = all(int(xcc[b]) == int(xcc[b % 8]) for b in range(512)) and len({int(x) for x in xcc[:8]}) == 8
    res = {"cus": len(by_cu), "xcd_of_b_depends_on_b_mod_8": xcd_ok, "xcd_of_workgroup_0": int(xcc[0]),
           "cu_pairs_are_b_and_b_plus_256": pairs_ok}
    log(f"[bench] workgroup placement: {res}")
    return res


def dense_data_dependence(reps=200):
    """The same dense NVFP4 GEMM (nvfp4_linear, M=8192, K=7168, N=4096) on random codes and on zero
    codes (same scales): the matrix core does the same work, so the ratio shows how much the clock
    (power) depends on the operand data.  TFLOP/s each, ~0.1 s of work per case."""
    import torch
    from nvfp4_block_scaled_top_amd import megamoe

    M, K, N = 8192, 7168, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    stream = torch.cuda.current_stream()
    a_c = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    w_c = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    a_s = torch.randint(0x28, 0x40, (M, K // 16), dtype=torch.uint8, device="cuda", generator=g)
    w_s = torch.randint(0x28, 0x40, (N, K // 16), dtype=torch.uint8, device="cuda", generator=g)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    out = torch.empty(M, N, dtype=torch.int16, device="cuda")
    ws = torch.empty(megamoe.megamoe_dense_workspace_bytes(M), dtype=torch.uint8, device="cuda")
    res = {"shape": [M, K, N]}
    for name, ac, wc in (("random_codes_TFLOPs", a_c, w_c),
                         ("zero_codes_TFLOPs", torch.zeros_like(a_c), torch.zeros_like(w_c))):
        call = lambda: megamoe.nvfp4_linear(ac, a_s, one, wc, w_s, one, out, ws)
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = round(2.0 * M * K * N / (ms * 1e-3) / 1e12, 1)
    log(f"[bench] dense NVFP4 GEMM, random vs zero codes: {res}")
    return res


def cpu_baseline(wl, T):
    """The CPU oracle on a bounded sample: the prefill layer restricted to its most-loaded expert."""
    import torch
    from nvfp4_block_scaled_top_amd import synth
    from oracle import nvfp4_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    ids, wts = O.router_topk(synth.router_logits(wl, T), wl.top_k)
    counts = O.route(ids, wl.expert_begin, wl.num_experts, wl.pad_multiple)[0]
    e = int(np.argmax(counts))
    x = O.bf16_from_bits(synth.activations(wl, T))
    w13, w2 = synth.expert_weights(wl, wl.expert_begin + e, device="cpu")
    q13 = O.quantize_nvfp4(O.bf16_from_bits(w13.view(torch.int16).numpy().view(np.uint16)))
    q2 = O.quantize_nvfp4(O.bf16_from_bits(w2.view(torch.int16).numpy().view(np.uint16)))
    t0 = time.perf_counter()
    O.moe_layer(x, ids, wts, wl.expert_begin + e, 1, wl.pad_multiple, q13[0][None], q13[1][None],
                np.array([q13[2]], np.float32), q2[0][None], q2[1][None], np.array([q2[2]], np.float32))
    dt = time.perf_counter() - t0
    flops = 6.0 * wl.hidden * wl.intermediate * int(counts[e])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy oracle, whole layer (route, quantize x, L1+SiLU, requantize, L2, combine) "
                      f"for T={T} restricted to its most-loaded expert ({int(counts[e])} tokens), {dt:.1f} s",
            "seconds": dt}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_kernels_prefill_t8192_decode_t4_t8.txt")
GEMM_SRC = os.path.join(ROOT, "nvfp4_block_scaled_top_amd", "csrc", "gemm.hip")
COPY_BYTES = 1 << 30  # the calibration kernel reads and writes this many bytes
TRAFFIC_WORKLOADS = {"prefill": (3, 8192), "decode_t4": (1, 4), "decode_t8": (1, 8)}
L1_LARGE = "gemm_large_kernel<true, false>"
L1_SMALL = "gemm_small_kernel<true, 256, true, false, 2, true>"  # the packed-code instantiation


def gemm_source_hash() -> str:
    import hashlib
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_pass(which: str) -> None:
    """Launch sequence for the HBM-traffic counters (run under rocprofv3 --pmc FETCH_SIZE or
    WRITE_SIZE): a plain elementwise copy of COPY_BYTES (torch.neg on float32, the calibration
    kernel), then two untimed forwards of the workload (TRAFFIC_WORKLOADS) without graphs."""
    import torch
    from nvfp4_block_scaled_top_amd import layer, synth

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    i, T = TRAFFIC_WORKLOADS[which]
    wl = synth.WORKLOADS[i]
    _, idd, wtd, counts = gpu_routing(wl, T, 0, "cuda")
    active = [int(e) for e in np.nonzero(counts)[0]]
    W = build_weights(wl, active, 1, "cuda")[0]
    L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                       expert_begin=wl.expert_begin)
    x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).cuda()
    for _ in range(2):
        L.forward(x, idd, wtd, W)
    torch.cuda.synchronize()
    log(f"[traffic-pass] {which} T={T} done")


def trace_steps(n: int) -> None:
    """Launch sequence for a rocprofv3 kernel trace: for the prefill (T=8192) and decode (T=1, 4, 8)
    workloads in turn, quantize the weights, run n eager layer forwards, quantize expert 0 once
    more (a separator in the trace), then n forwards with calibrated scales (those of the first
    forwards).  No timing."""
    import torch
    from nvfp4_block_scaled_top_amd import layer, synth

    for wl, T, copies in ((synth.WORKLOADS[3], 8192, 1), (synth.WORKLOADS[1], 1, 4), (synth.WORKLOADS[1], 4, 4),
                          (synth.WORKLOADS[1], 8, 4)):
        _, idd, wtd, counts = gpu_routing(wl, T, 0, "cuda")
        # expert 0 is always quantized too, so weight quantization separates every workload in
        # the trace (decode T=1 has no local expert at seed 0)
        Ws = build_weights(wl, sorted({0} | {int(e) for e in np.nonzero(counts)[0]}), copies, "cuda")
        L = layer.MoELayer(T, wl.top_k, wl.num_experts, wl.hidden, wl.intermediate, wl.pad_multiple,
                           expert_begin=wl.expert_begin)
        x = torch.from_numpy(synth.activations(wl, T).view(np.int16)).cuda()
        for i in range(n):
            L.forward(x, idd, wtd, Ws[i % copies])
        torch.cuda.synchronize()
        gx, gh = L.x_gs.clone(), L.h_gs.clone()
        build_weights(wl, [0], 1, "cuda")
        for i in range(n):
            L.forward(x, idd, wtd, Ws[i % copies], x_gs=gx, h_gs=gh)
        torch.cuda.synchronize()
        log(f"[trace-steps] {wl.name} T={T}: {n} forwards, {n} calibrated")
        del Ws, L


def _counter_medians(path: str, counter: str) -> dict:
    """Median per-dispatch value of `counter` for each kernel name in a rocprofv3 counter CSV."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            vals.setdefault(name, []).append(float(r["Counter_Value"]))
    return {k: sorted(v)[len(v) // 2] for k, v in vals.items()}


def summarize_traffic(specs: list) -> None:
    """specs: WORKLOAD=FETCH_CSV,WRITE_CSV for each workload of TRAFFIC_WORKLOADS.  Writes
    TRAFFIC_FILE: HBM bytes per dispatch of each GEMM kernel, counter values scaled by what the same
    counters read for the copy kernel of known size."""
    out = ["# HBM traffic per dispatch of the grouped-GEMM kernels (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE)",
           "# Commands, from /tmp with TMPDIR=/tmp, for W in prefill decode_t4 decode_t8 and C in FETCH_SIZE WRITE_SIZE:",
           "#   rocprofv3 --pmc C -f csv -d <out>/pmc_C_W -o p -- python3 bench.py --traffic-pass W",
           "# then: python3 bench.py --summarize-traffic prefill=<FETCH csv>,<WRITE csv> decode_t4=... decode_t8=...",
           "# Counter KiB per dispatch (median over dispatches) x factor = bytes, where factor = bytes the",
           "# copy kernel (torch.neg on 1 GiB of float32) reads or writes / what the counter reads for it.",
           f"gemm_source_sha256_16: {gemm_source_hash()}"]
    for spec in specs:
        which, files = spec.split("=", 1)
        fpath, wpath = files.split(",")
        fetch = _counter_medians(fpath, "FETCH_SIZE")
        write = _counter_medians(wpath, "WRITE_SIZE")
        ck = [k for k in fetch if "neg" in k.lower() or "unary" in k.lower()][0]
        f_factor = COPY_BYTES / (fetch[ck] * 1024.0)
        w_factor = COPY_BYTES / (write[ck] * 1024.0)
        out.append(f"{which}_copy_kernel: {ck}")
        out.append(f"{which}_copy_fetch_kib: {fetch[ck]:.0f}  (factor {f_factor:.4f})")
        out.append(f"{which}_copy_write_kib: {write[ck]:.0f}  (factor {w_factor:.4f})")
        for k in sorted(fetch):
            if "gemm_" not in k:
                continue
            short = k.replace("megamoe::", "")
            fb, wb = fetch[k] * 1024.0 * f_factor, write.get(k, 0.0) * 1024.0 * w_factor
            out.append(f"{which}|{short}: fetch_kib {fetch[k]:.0f} write_kib {write.get(k, 0.0):.0f} "
                       f"bytes {fb + wb:.0f}")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


TRACE_WORKLOADS = ("prefill T=8192", "prefill T=8192 (calibrated scales)", "decode T=1",
                   "decode T=1 (calibrated scales)", "decode T=4", "decode T=4 (calibrated scales)",
                   "decode T=8", "decode T=8 (calibrated scales)")


def summarize_trace(path: str) -> None:
    """Per-step kernel durations from the kernel-trace CSV of a `--trace-steps N` run.  A layer step
    runs from a routing kernel to the combine; library quantization kernels outside a step (weight
    quantization) separate the workloads, in the order of trace_steps().  Prints, per workload, the
    median over steps of each kernel's duration per step and of their sum."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()

    def short(name):
        n = name.replace("void ", "").split("(")[0]
        return n.replace("megamoe::", "")

    segments, steps, cur, in_step = [], [], None, False
    for t0, t1, name in rows:
        if "megamoe::" not in name:
            continue
        k = short(name)
        if k.startswith("route_") and not in_step:  # route_*, not the router
            in_step, cur = True, {}
        if in_step:
            cur.setdefault(k, []).append((t1 - t0) / 1000.0)
            if k.startswith("combine"):
                steps.append({n: sum(v) for n, v in cur.items()})
                in_step = False
        elif k.startswith("quant") and steps:
            segments.append(steps)
            steps = []
    if steps:
        segments.append(steps)

    def med(v):
        v = sorted(v)
        return v[len(v) // 2]

    out = []
    for label, seg in zip(TRACE_WORKLOADS, segments):
        names = []
        for st in seg:
            names += [n for n in st if n not in names]
        out.append(f"{label}: {len(seg)} layer steps, median kernel duration per step (us)")
        for n in names:
            v = [st.get(n, 0.0) for st in seg]
            out.append(f"  {n:44s} {med(v):8.2f}   (min {min(v):.2f}, max {max(v):.2f})")
        tot = [sum(st.values()) for st in seg]
        out.append(f"  {'(sum of kernels)':44s} {med(tot):8.2f}   (min {min(tot):.2f}, max {max(tot):.2f})")
    print("\n".join(out))


def summarize_counters(path: str) -> None:
    """Median per dispatch of every counter in a rocprofv3 --pmc CSV, for the library's kernels.
    With GRBM_GUI_ACTIVE (summed over the 8 XCDs) also the clock the kernel ran at: GRBM_GUI_ACTIVE
    / 8 / the dispatch's duration (its Start/End timestamps, ns), for dispatches of at least 0.5 ms
    (the counter's window is wider than a short dispatch)."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if "megamoe::" not in name and "megamoe_probe::" not in name:
                continue
            cs = vals.setdefault(name.replace("megamoe::", "").replace("megamoe_probe::", "probe::"), {})
            cs.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and r.get("End_Timestamp"):
                ns = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                if ns >= 5e5:
                    cs.setdefault("clock_GHz", []).append(float(r["Counter_Value"]) / 8.0 / ns)
    for k, cs in vals.items():
        parts = []
        for c, v in sorted(cs.items()):
            v = sorted(v)
            parts.append(f"{c} {v[len(v) // 2]:.4g}")
        print(f"{k:44s} dispatches {max(len(v) for v in cs.values()):3d}  " + "  ".join(parts))


def recorded_traffic(which: str, kernel: str):
    """HBM bytes per dispatch of `kernel` on workload `which` recorded in TRAFFIC_FILE, or None if
    absent or taken on other kernel code."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("gemm_source_sha256_16") != gemm_source_hash():
            return None
        return float(kv[f"{which}|{kernel}"].split("bytes")[1])
    except (OSError, KeyError, ValueError, IndexError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--decode-seeds", type=int, default=64, help="routing seeds of the decode aggregate (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--unpacked", action="store_true",
                    help="weights without the packed copy of their codes (the 16-row kernels read the row-major codes)")
    ap.add_argument("--quick", action="store_true", help="prefill only, no CPU baseline")
    ap.add_argument("--traffic-pass", choices=tuple(TRAFFIC_WORKLOADS),
                    help="launch sequence for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (no timing)")
    ap.add_argument("--trace-steps", type=int, default=0, metavar="N",
                    help="launch sequence for a rocprofv3 kernel trace: N forwards per workload (no timing)")
    ap.add_argument("--summarize-traffic", nargs="+", metavar="W=FETCH_CSV,WRITE_CSV",
                    help="FETCH_SIZE and WRITE_SIZE counter CSVs of each --traffic-pass workload")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="kernel-trace CSV of a --trace-steps run: per-workload medians of kernel time per step")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="rocprofv3 --pmc counter CSV: per-kernel medians of each counter")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="print the measured ceilings (context of the bench line) as JSON and exit")
    args = ap.parse_args()
    global PACKED
    PACKED = not args.unpacked
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from nvfp4_block_scaled_top_amd import megamoe, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    megamoe.lib()
    torch.cuda.set_device(0)
    if args.traffic_pass:
        traffic_pass(args.traffic_pass)
        return
    if args.trace_steps:
        trace_steps(args.trace_steps)
        return
    if args.ceilings_only:
        print(json.dumps(measured_ceilings()))
        return

    pre_wl = synth.WORKLOADS[3]
    T = pre_wl.tokens[0]
    log(f"[bench] prefill {pre_wl.name} T={T}")
    pre = time_workload(pre_wl, T, args.steps, args.warmup, copies=1, use_graph=not args.no_graph)
    tflops = pre["flops"] / (pre["ms_per_step"] * 1e-3) / 1e12
    log(f"[bench] prefill {pre['ms_per_step']:.3f} ms/step, {tflops:.1f} TFLOP/s; stages {pre['stage_ms']}")
    log("[bench] prefill large-tile kernels alone")
    lk = time_large_tile_kernels(pre_wl, T, reps=max(5, min(args.steps, 20)))
    lk_l1_tf = lk["l1_flops"] / (lk["l1_ms"] * 1e-3) / 1e12
    lk_l2_tf = lk["l2_flops"] / (lk["l2_ms"] * 1e-3) / 1e12
    log(f"[bench] {L1_LARGE}: {lk['l1_ms']:.3f} ms = {lk_l1_tf:.0f} TFLOP/s; L2 large {lk['l2_ms']:.3f} ms = "
        f"{lk_l2_tf:.0f} TFLOP/s")

    decode = {}
    if not args.quick:
        dec_wl = synth.WORKLOADS[1]
        for Td in dec_wl.tokens:
            log(f"[bench] decode {dec_wl.name} T={Td}")
            d = time_workload(dec_wl, Td, args.decode_steps, args.warmup, copies=4, use_graph=not args.no_graph,
                              fused=True)
            gbs = d["weight_bytes"] / (d["ms_per_step"] * 1e-3) / 1e9
            # at decode every expert has at most 16 tokens and the layer passes T as the row bound, so
            # moe_grouped_gemm_l1_silu launches exactly one kernel, the 16-row one: the stage time is
            # that kernel's launch duration
            l1_gbs = d["w13_bytes"] / (d["stage_ms"]["l1"] * 1e-3) / 1e9
            decode[f"T{Td}"] = {
                "ms_per_step": round(d["ms_per_step"], 5),
                "ms_per_step_p10_p50_p90": [round(d["spread"][q], 5) for q in ("p10", "p50", "p90")],
                "gemm_ms": round(d["stage_ms"]["l1"] + d["stage_ms"]["l2"], 5), "weight_GBps": round(gbs, 1),
                "calibrated_gs_ms_per_step": None if d["calibrated_ms"] is None else round(d["calibrated_ms"], 5),
                "fused_ffn_ms_per_step": None if d["fused_ms"] is None else round(d["fused_ms"], 5),
                "fused_ffn_calibrated_gs_ms_per_step": (None if d["fused_calibrated_ms"] is None
                                                        else round(d["fused_calibrated_ms"], 5)),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "TFLOPs": round(d["flops"] / (d["ms_per_step"] * 1e-3) / 1e12, 3),
                "active_experts": d["active_experts"], "assignments": d["assignments"],
                "weight_bytes": d["weight_bytes"], "stage_ms": {k: round(v, 5) for k, v in d["stage_ms"].items()},
                "roofline": {"bound": "hbm", "achieved": round(l1_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(l1_gbs / PEAK_HBM_GBS, 4),
                             "traffic": recorded_traffic(f"decode_t{Td}", L1_SMALL) if Td in (4, 8) else None,
                             "kernel": L1_SMALL, "algorithmic_bytes": d["w13_bytes"]},
            }
            log(f"[bench] decode T={Td}: {d['ms_per_step'] * 1e3:.1f} us/step, {gbs:.0f} GB/s; calibrated "
                f"{d['calibrated_ms'] * 1e3:.1f}, fused {d['fused_ms'] * 1e3:.1f}, fused calibrated "
                f"{d['fused_calibrated_ms'] * 1e3:.1f} us/step" if d["fused_ms"] is not None else
                f"[bench] decode T={Td}: {d['ms_per_step'] * 1e3:.1f} us/step, {gbs:.0f} GB/s")

    prefill_configs = None
    if not args.quick:
        prefill_configs = {w.name: prefill_config_entry(w, max(5, args.steps // 2), args.warmup, not args.no_graph)
                           for w in (synth.WORKLOADS[2], synth.WORKLOADS[4])}

    seed_agg = None
    ceilings = None
    dense = None
    if not args.quick:
        if args.decode_seeds > 0:
            log(f"[bench] decode aggregate over {args.decode_seeds} routing seeds")
            seed_agg = decode_seed_aggregate(synth.WORKLOADS[1], args.decode_seeds, reps=10)
        log("[bench] dense NVFP4 linear")
        dense = dense_linear_bench()
        log("[bench] measured ceilings")
        ceilings = measured_ceilings()


    cpu = None
    if not args.no_cpu_baseline and not args.quick:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(pre_wl, T)
        cpu.pop("seconds", None)

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{pre_wl.name}: 384 experts, top-6, hidden 7168, intermediate 2048, T={T}, "
                               "Zipf(1.2) expert bias, NVFP4 weights and activations, seed 0",
                   "global_batch": T, "experts": 384, "top_k": 6, "hidden": 7168, "intermediate": 2048,
                   "active_experts": pre["active_experts"], "assignments": pre["assignments"]},
        "weight_GBps": round(pre["weight_bytes"] / (pre["ms_per_step"] * 1e-3) / 1e9, 1),
        "mfma_frac": round(tflops / PEAK_FP16_TFLOPS, 4),
        "mfma_frac_vs_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
        "ms_per_step_p10_p50_p90": [round(pre["spread"][q], 4) for q in ("p10", "p50", "p90")],
        "stage_ms": {k: round(v, 4) for k, v in pre["stage_ms"].items()},
        "gemm_ms": round(pre["stage_ms"]["l1"] + pre["stage_ms"]["l2"], 4),
        "calibrated_gs_ms_per_step": None if pre["calibrated_ms"] is None else round(pre["calibrated_ms"], 4),
        "roofline": {"bound": "mfma", "achieved": round(lk_l1_tf, 1), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(lk_l1_tf / PEAK_FP16_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill", L1_LARGE), "kernel": L1_LARGE,
                     "algorithmic_flops": lk["l1_flops"], "launch_ms": round(lk["l1_ms"], 4),
                     "assignments": lk["assignments"], "experts": lk["experts"]},
        "large_tile_l2": {"kernel": "gemm_large_kernel<false, false>", "launch_ms": round(lk["l2_ms"], 4),
                          "TFLOPs": round(lk_l2_tf, 1), "frac": round(lk_l2_tf / PEAK_FP16_TFLOPS, 4),
                          "traffic": recorded_traffic("prefill", "gemm_large_kernel<false, false>")},
        "prefill_configs": prefill_configs,
        "decode": decode,
        "decode_seed_aggregate": seed_agg,
        "dense_linear": dense,
        "measured_ceilings_context": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
