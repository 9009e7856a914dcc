"""Benchmark of the FP8 block-scale MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload prefill|decode|skew|tiny|dense|prefill_bias0|skew_zipf]
                    [--tokens T] [--block-m BM] [--dense-m M --dense-n N] [--no-cpu-baseline]
                    [--no-decode] [--sweep block_m|dense]

A step is one pass of the whole layer -- grouped_topk, moe_sort,
fp8_quant_1x128, moe_fp8_blockscale_g1u1, moe_down_combine -- over one batch
of synthetic tokens whose inputs and weights are already resident in HBM.
(`--workload dense` times fp8_quant_1x128 + gemm_fp8_blockscale instead.)
Prints one JSON line.  The default workload is the largest configuration:
the 8192-token prefill layer of DeepSeek-V3 shape (hidden 7168,
intermediate 2048, 256 experts in 8 groups, topk_group 4, top-8), with its
roofline on the FP8 matrix cores; the 64-token decode layer on the same
weights is reported beside it (object "decode", roofline on HBM).

--sweep block_m times the whole layer for every M tile over a range of token
counts (the table behind moe_block_m); --sweep dense times the dense GEMM on
the linear-layer shapes of a DeepSeek-V3 layer; --sweep tiles times the two
grouped GEMMs on hand-built sorted buffers whose 128-row blocks hold r valid
rows each (the cost of a tile against its live rows, with weights shared by
2 or 16 blocks of an expert or read by one block only).  Sweeps print one JSON line
per measurement and no bench line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["decode", "prefill", "skew", "tiny", "dense", "prefill_bias0", "skew_zipf"],
                    help="prefill_bias0 / skew_zipf: labelled routing controls (zero bias; Zipf without the hot bias)")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--tokens", type=int, default=None, help="token count of a MoE workload (default: its own)")
    ap.add_argument("--no-decode", action="store_true", help="prefill: leave out the decode layer beside it")
    ap.add_argument("--sweep", choices=["block_m", "dense", "tiles"], default=None)
    ap.add_argument("--phases", action="store_true",
                    help="per-step phase clocks of the gate/up kernel from the diagnostic library libmoe355_trace.so")
    ap.add_argument("--graph", action="store_true",
                    help="also time the layer captured once as a HIP graph and replayed (graph_ms_per_step)")
    ap.add_argument("--fused", action="store_true",
                    help="the expert computation as one launch (moe_fp8_blockscale_fused) instead of two calls")
    ap.add_argument("--preshuffle", action="store_true",
                    help="weights permuted once into the 128x128-tile layout (the *_wpreshuffle calls)")
    ap.add_argument("--dense-m", type=int, default=64)
    ap.add_argument("--dense-n", type=int, default=18432)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after timing, copy BYTES bytes device-to-device 3 times (plain copy kernel whose "
                         "FETCH_SIZE / WRITE_SIZE calibrate the traffic counters)")
    return ap.parse_args()


def kernel_source_hash():
    from fp8_block_scaled_grouped_amd.tuning.rocprof_summary import source_hash
    return source_hash()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it was taken
    on the current kernel source (else None).  Each counter is scaled by what it read for a
    plain copy of known size in the same runs."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != kernel_source_hash() or kernel not in d.get("kernels", {}):
        return None
    k = d["kernels"][kernel]
    cal = d["copy_calibration"]
    fetch = k["FETCH_SIZE_KiB"] * 1024 * cal["bytes"] / (cal["FETCH_SIZE_KiB"] * 1024)
    write = k["WRITE_SIZE_KiB"] * 1024 * cal["bytes"] / (cal["WRITE_SIZE_KiB"] * 1024)
    return fetch + write


def copy_calibration(nbytes):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def routing_stats(ids, E, block_m, hot=None):
    import numpy as np
    flat = ids.reshape(-1)
    load = np.bincount(flat, minlength=E)
    act = load[load > 0]
    padded = int(sum(-(-int(c) // block_m) * block_m for c in act))
    st = {"active_experts": int(len(act)), "load_min": int(act.min()), "load_mean": float(act.mean()),
          "load_max": int(act.max()), "load_cv": float(act.std() / act.mean()),
          "padded_fraction": float(1 - len(flat) / padded)}
    if hot is not None:
        st["hot_pair_share"] = float(np.isin(flat, np.nonzero(hot)[0]).mean())
    return st


class _ExpertRows:
    """Per-expert host copies of a device weight tensor, fetched on first use."""

    def __init__(self, t):
        self.t, self.d, self.shape = t, {}, tuple(t.shape)

    def __getitem__(self, e):
        e = int(e)
        if e not in self.d:
            self.d[e] = self.t[e].cpu().numpy()
        return self.d[e]


def host_cpu():
    """(cores this process may run on, CPU model name) of the host."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def cpu_baseline_moe(cfg, hidden, logits, bias, w1, s1, w2, s2):
    """The oracle as it stands, timed on the host cores on the whole layer: routing of all
    T tokens, their 1x128 quantisation, and the expert-batched evaluation of every routed
    pair (gate/up, SiLU*up, requantisation, down projection) with the weighted combine.

    The oracle evaluates independent (expert, block of rows) pieces on its thread pool;
    the host copies of the routed experts' weights are made before the clock starts.
    """
    import numpy as np
    import oracle
    from oracle.pool import default_workers
    workers = default_workers()
    ncpu, model = host_cpu()
    hid = oracle.fp8.bf16_bits_to_f32(hidden.cpu().view(torch_int16()).numpy().view(np.uint16))
    logits = logits.cpu().numpy()
    bias = bias.cpu().numpy()
    s1, s2 = s1.cpu().numpy(), s2.cpu().numpy()
    W1, W2 = _ExpertRows(w1), _ExpertRows(w2)
    t0 = time.perf_counter()
    w, ids = oracle.routing.grouped_topk(logits, bias, cfg.n_group, cfg.topk_group, cfg.topk, cfg.renorm,
                                         cfg.routed_scaling_factor)
    t_route = time.perf_counter() - t0
    for e in np.unique(ids):                      # host copies outside the clock
        W1[e], W2[e]
    t0 = time.perf_counter()
    a8, sa = oracle.quant.quant_1x128(hid, workers=workers)
    oracle.moe.layer_tokens(a8, sa, W1, s1, W2, s2, ids, w, workers=workers)
    sec = t_route + time.perf_counter() - t0
    return {"value": cfg.T / sec, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": "all %d of %d tokens through the whole layer (routing, quantisation, every routed pair's "
                      "expert GEMMs and the combine), %.1f s" % (cfg.T, cfg.T, sec),
            "host_cores_available": ncpu, "cpu_model": model, "seconds": sec}


def torch_int16():
    import torch
    return torch.int16


def moe_config(workload, tokens=None):
    from fp8_block_scaled_grouped_amd import inputs
    cfg = {**inputs.MOE_CONFIGS, **inputs.CONTROL_CONFIGS}[workload]
    return inputs.with_tokens(cfg, tokens) if tokens else cfg


def moe_inputs(cfg, seed, weights=None):
    """Device inputs of a MoE workload; the expert weights are generated unless given."""
    import torch
    from fp8_block_scaled_grouped_amd import inputs
    dev = torch.device("cuda:0")
    x = inputs.make_moe_inputs(cfg, "cpu" if cfg.name == "tiny" else dev, seed=seed, weights=weights is None)
    x = {k: v.to(dev) for k, v in x.items()}
    if weights is not None:
        x.update(weights)
    torch.cuda.synchronize()
    return x


def time_layer(cfg, x, bm, steps, warmup, preshuffle=False, graph=False, per_call=True, fused=False):
    """Time K whole layer steps on the current stream; the g1u1 launch of every step (the
    fused launch with fused=True) is bracketed by events on the same stream.  Returns a
    dict of timings and the layer."""
    import torch

    import fp8_block_scaled_grouped_amd as m

    layer = m.MoELayer(cfg, x["bias"], x["w1"], x["w1_scale"], x["w2"], x["w2_scale"], block_m=bm,
                       preshuffle=preshuffle, fused=fused)
    hidden, logits = x["hidden"], x["logits"]
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer.forward(hidden, logits)
    torch.cuda.synchronize()

    c = cfg
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    st = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]  # start of each step
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        st[i].record(stream)
        # routing, sort and (on the layer's side stream) quantisation, as MoELayer.forward runs them
        sid, sw, seid, nv = layer.route_and_quantise(hidden, logits)
        ev[i][0].record(stream)
        if fused:
            m.moe_fp8_blockscale_fused(layer.a8, layer.a_scale, layer.w1, layer.w1_scale, layer.w2, layer.w2_scale,
                                       sid, sw, seid, nv, c.topk, bm, layer.out, layer.fused_ws)
            ev[i][1].record(stream)
        else:
            m.moe_fp8_blockscale_g1u1(layer.a8, layer.a_scale, layer.w1, layer.w1_scale, sid, seid, nv, c.topk, bm,
                                      layer.h8, layer.h_scale, preshuffled=layer.preshuffle)
            ev[i][1].record(stream)
            m.moe_down_combine(layer.h8, layer.h_scale, layer.w2, layer.w2_scale, sid, sw, seid, nv, layer.T,
                               c.topk, bm, layer.out, layer.down_ws, preshuffled=layer.preshuffle)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    g1u1_ms = sum(s.elapsed_time(e) for s, e in ev) / steps
    steps_ms = sorted([st[i].elapsed_time(st[i + 1]) for i in range(steps - 1)] + [st[-1].elapsed_time(end)])
    r = {"ms": ms, "g1u1_ms": g1u1_ms, "layer": layer, "sid": sid, "sw": sw, "seid": seid, "nv": nv,
         "layer_ms": {"median_ms": steps_ms[len(steps_ms) // 2], "min_ms": steps_ms[0]}}

    if graph:
        # the five calls captured once into a HIP graph (the library allocates nothing and
        # never synchronises, so the layer is capturable) and replayed K times
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(hidden, logits)
        for _ in range(warmup):
            g.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        r["graph_ms"] = g0.elapsed_time(g1) / steps
        del g

    if per_call and not fused:
        # per-call breakdown (outside the timed region): events around each of the five calls
        calls = [
            ("grouped_topk", lambda: m.grouped_topk(logits, layer.bias, c.n_group, c.topk_group, c.topk, c.renorm,
                                                    c.routed_scaling_factor, layer.topk_w, layer.topk_ids)),
            ("moe_sort", lambda: m.moe_sort(layer.topk_ids, layer.topk_w, c.E, bm, layer.sort_out, layer.sort_ws)),
            ("fp8_quant_1x128", lambda: m.fp8_quant_1x128(hidden, layer.a8, layer.a_scale)),
            ("moe_fp8_blockscale_g1u1", lambda: m.moe_fp8_blockscale_g1u1(layer.a8, layer.a_scale, layer.w1,
                                                                          layer.w1_scale, sid, seid, nv, c.topk, bm,
                                                                          layer.h8, layer.h_scale,
                                                                          preshuffled=layer.preshuffle)),
            ("moe_down_combine", lambda: m.moe_down_combine(layer.h8, layer.h_scale, layer.w2, layer.w2_scale, sid,
                                                            sw, seid, nv, layer.T, c.topk, bm, layer.out,
                                                            layer.down_ws, preshuffled=layer.preshuffle)),
        ]
        reps = max(10, steps)
        cev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
               for _ in range(reps)]
        for rr in range(reps):
            for (name, fn), (e0, e1) in zip(calls, cev[rr]):
                e0.record(stream)
                fn()
                e1.record(stream)
        torch.cuda.synchronize()
        pc = {}
        for ci, (name, _) in enumerate(calls):
            t = sorted(cev[rr][ci][0].elapsed_time(cev[rr][ci][1]) for rr in range(reps))
            pc[name] = {"median_ms": t[len(t) // 2], "min_ms": t[0]}
        r["per_call_ms"] = pc
    return r


def moe_report(cfg, bm, tm, workload, seed, preshuffle, fused=False):
    """Bench-line fields of one timed MoE workload: tokens/s, layer TFLOP/s and GB/s, the
    routing statistics and the roofline of the dominant kernel (moe_fp8_blockscale_g1u1, or
    the fused launch that holds both expert GEMMs)."""
    import torch
    from fp8_block_scaled_grouped_amd import inputs

    layer = tm["layer"]
    ms, g1u1_ms = tm["ms"], tm["g1u1_ms"]
    ids = layer.topk_ids.cpu().numpy()
    hot = inputs.hot_expert_mask(cfg, torch.device("cuda:0"), seed).cpu().numpy() if cfg.skew else None
    rs = routing_stats(ids, cfg.E, bm, hot)
    n_active = rs["active_experts"]
    flops = inputs.moe_flops(cfg)
    nbytes = inputs.moe_bytes(cfg, n_active)
    H, I, T, k = cfg.H, cfg.I, cfg.T, cfg.topk
    # algorithmic bytes of one g1u1 launch: routed experts' gate/up weights + scales, the
    # quantised activations and their scales, the sort buffers read, and h8 + scales written
    per_expert_w1 = 2 * I * H + 4 * (2 * I // 128) * (H // 128)
    g1u1_bytes = (n_active * per_expert_w1 + T * H + 4 * T * (H // 128) + 4 * layer.max_sorted
                  + T * k * (I + 4 * (I // 128)))
    g1u1_flops = 2.0 * T * k * 2 * I * H
    if fused:
        # the fused launch: both expert GEMMs (w1 and w2 of the routed experts), a8 in, output out
        per_expert_w2 = H * I + 4 * (H // 128) * (I // 128)
        g1u1_bytes = n_active * (per_expert_w1 + per_expert_w2) + T * H + 4 * T * (H // 128) + 8 * layer.max_sorted \
            + 2 * T * H
        g1u1_flops = inputs.moe_flops(cfg)
    if cfg.T <= 512:
        roof = {"bound": "hbm", "achieved": g1u1_bytes / (g1u1_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": g1u1_flops / (g1u1_ms * 1e-3) / 1e12, "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = "moe_fp8_blockscale_fused" if fused else "moe_fp8_blockscale_g1u1"
    roof["kernel_ms"] = g1u1_ms
    roof["algorithmic_per_launch"] = g1u1_bytes if roof["bound"] == "hbm" else g1u1_flops
    roof["traffic"] = None if fused else measured_traffic(workload, "g1u1")
    res = {
        "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
        "config": {"workload": "%s MoE layer: %d tokens, hidden %d, intermediate %d, %d experts / %d groups, "
                               "topk_group %d, top-%d, block_m %d" % (workload, T, H, I, cfg.E, cfg.n_group,
                                                                      cfg.topk_group, k, bm),
                   "tokens": T, "hidden": H, "intermediate": I, "experts": cfg.E, "topk": k, "block_m": bm,
                   "preshuffled_weights": bool(preshuffle), "fused_expert_launch": bool(fused),
                   "quantisation_on_side_stream": tm["layer"].side is not None, "seed": seed},
        "layer_tflops": flops / (ms * 1e-3) / 1e12, "layer_gbs": nbytes / (ms * 1e-3) / 1e9,
        "layer_frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_frac_mfma": flops / (ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "routing": rs, "roofline": roof, "layer_ms": tm["layer_ms"],
    }
    if "per_call_ms" in tm:
        res["per_call_ms"] = tm["per_call_ms"]
    if "graph_ms" in tm:
        res["graph_ms_per_step"] = tm["graph_ms"]
        res["graph_tokens_per_s"] = T / (tm["graph_ms"] * 1e-3)
    return res


def bench_moe(a):
    cfg = moe_config(a.workload, a.tokens)
    bm = a.block_m or cfg.block_m
    t0 = time.time()
    x = moe_inputs(cfg, a.seed)
    gen_s = time.time() - t0
    tm = time_layer(cfg, x, bm, a.steps, a.warmup, a.preshuffle, a.graph, fused=a.fused)
    rep = moe_report(cfg, bm, tm, a.workload, a.seed, a.preshuffle, a.fused)
    res = {"metric": "FP8 blockscale MoE layer tokens/s", "value": rep.pop("tokens_per_s"), "unit": "tokens/s",
           "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": rep.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3 (fp32 accumulate)",
           "data": "synthetic"}
    res.update(rep)
    res["input_gen_s"] = round(gen_s, 2)
    del tm
    if a.workload == "prefill" and not a.no_decode and not a.tokens:
        # the 64-token decode layer on the same expert weights: the HBM-bound configuration
        dcfg = moe_config("decode")
        w = {k: x[k] for k in ("w1", "w1_scale", "w2", "w2_scale")}
        dx = moe_inputs(dcfg, a.seed, weights=w)
        dtm = time_layer(dcfg, dx, dcfg.block_m, max(a.steps, 20), a.warmup, a.preshuffle, per_call=True,
                         fused=a.fused)
        res["decode"] = moe_report(dcfg, dcfg.block_m, dtm, "decode", a.seed, a.preshuffle, a.fused)
        del dtm
    if not a.no_cpu_baseline:
        # the oracle reads the weights as loaded (row-major), not shuffled copies
        layer_scales = (x["w1_scale"], x["w2_scale"])
        res["cpu_baseline"] = cpu_baseline_moe(cfg, x["hidden"], x["logits"], x["bias"], x["w1"], layer_scales[0],
                                               x["w2"], layer_scales[1])
    return res


def sweep_block_m(a):
    """Whole-layer time for every M tile over token counts (prefill routing distribution)."""
    base = moe_config("prefill")
    w = None
    for T in (a.tokens,) if a.tokens else (1, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192):
        cfg = moe_config("prefill", T)
        x = moe_inputs(cfg, a.seed, weights=w)
        w = {k: x[k] for k in ("w1", "w1_scale", "w2", "w2_scale")}
        for bm in (16, 32, 64, 128, 256):
            tm = time_layer(cfg, x, bm, a.steps, a.warmup, a.preshuffle, per_call=False)
            print(json.dumps({"sweep": "block_m", "tokens": T, "block_m": bm, "ms": tm["ms"],
                              "median_ms": tm["layer_ms"]["median_ms"], "g1u1_ms": tm["g1u1_ms"],
                              "hidden": base.H, "intermediate": base.I, "experts": base.E, "topk": base.topk}),
                  flush=True)
            del tm


def sweep_tiles(a):
    """Grouped GEMM time per 128-row tile against its valid rows r: sorted buffers built on the
    host (blocks of 128 rows, the first r of each valid, distinct random pairs of the 8192-token
    prefill layer, the rest the sentinel), with the block's expert chosen so that 2 blocks
    ("pairs") or 16 blocks ("shared16") of one expert share its weights, or every block has an
    expert of its own ("solo")."""
    import torch

    import fp8_block_scaled_grouped_amd as m
    cfg = moe_config("prefill")
    dev = torch.device("cuda:0")
    x = moe_inputs(cfg, a.seed)
    T, k, E, H, I, BM = cfg.T, cfg.topk, cfg.E, cfg.H, cfg.I, 128
    a8, a_s = m.fp8_quant_1x128(x["hidden"])
    ms = m.moe_sort_sizes(T, k, E, BM)[0]
    h8 = torch.zeros((ms, I), dtype=torch.uint8, device=dev)
    hs = torch.ones((ms, I // 128), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(m.moe_down_combine_workspace(T, H, k), dtype=torch.uint8, device=dev)
    gen = torch.Generator().manual_seed(a.seed + 1)
    perm = torch.randperm(T * k, generator=gen).to(torch.int32)

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        return t[n // 2]

    cases = [("pairs", 512, r, lambda b: b // 2) for r in (128, 96, 64, 32, 16, 1)]
    cases += [(lay, 256, r, f) for r in (128, 32, 1) for lay, f in (("solo", lambda b: b), ("shared16", lambda b: b // 16))]
    for lay, nblk, r, expert_of in cases:
        sid = torch.full((ms,), T * k, dtype=torch.int32)
        for b in range(nblk):
            sid[b * BM:b * BM + r] = perm[b * r:(b + 1) * r]
        seid = torch.tensor([expert_of(b) for b in range(nblk)] + [0] * (ms // BM - nblk), dtype=torch.int32)
        sid, seid = sid.to(dev), seid.to(dev)
        sw = torch.full((ms,), 0.5, dtype=torch.float32, device=dev)
        nv = torch.tensor([nblk * BM], dtype=torch.int32, device=dev)
        g = timed(lambda: m.moe_fp8_blockscale_g1u1(a8, a_s, x["w1"], x["w1_scale"], sid, seid, nv, k, BM, h8, hs))
        d = timed(lambda: m.moe_down_combine(h8, hs, x["w2"], x["w2_scale"], sid, sw, seid, nv, T, k, BM, out, ws))
        print(json.dumps({"sweep": "tiles", "layout": lay, "blocks": nblk, "rows_per_block": r, "g1u1_ms": g,
                          "down_combine_ms": d, "g1u1_us_per_tile_per_cu": g * 1e3 * 256 / (nblk * (2 * I // 256)),
                          "down_tiles": nblk * (H // 256)}), flush=True)


# (N, K) of the linear layers of a DeepSeek-V3 layer
V3_LINEAR = [("q_a_proj", 1536, 7168), ("kv_a_proj", 576, 7168), ("q_b_proj", 24576, 1536),
             ("kv_b_proj", 32768, 512), ("o_proj", 7168, 16384), ("dense_mlp_gate_up", 36864, 7168),
             ("dense_mlp_down", 7168, 18432), ("shared_gate_up", 4096, 7168), ("shared_down", 7168, 2048),
             ("config_n2048", 2048, 7168), ("config_n18432", 18432, 7168)]


_SLEEP_PER_MS = None


def hold_stream(stream, ms):
    """Queue a spin kernel of about `ms` milliseconds on `stream`, so that the launches the
    host queues behind it run back to back on the GPU even where one launch takes less
    time on the GPU than its call on the host."""
    import torch

    global _SLEEP_PER_MS
    if _SLEEP_PER_MS is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record(stream)
        torch.cuda._sleep(1 << 20)
        e1.record(stream)
        torch.cuda.synchronize()
        _SLEEP_PER_MS = (1 << 20) / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(_SLEEP_PER_MS * ms))


def time_dense(M, N, K, steps, warmup, seed=0, preshuffle=False):
    """quant + GEMM per step, and the GEMM call alone back to back, over rotated weight copies."""
    import torch

    import fp8_block_scaled_grouped_amd as m
    from fp8_block_scaled_grouped_amd import inputs

    dev = torch.device("cuda:0")
    d = inputs.make_dense_inputs(M, N, K, dev, seed=seed)
    # rotate distinct weight copies so a small B is not served from the 256 MB MALL
    ncopy = max(1, min(48, (8 << 30) // (N * K)))  # >= 40 copies below 200 MB of weights
    bs = [d["b"]] + [d["b"].clone() for _ in range(ncopy - 1)]
    if preshuffle:
        bs = [m.shuffle_weight_128x128(b) for b in bs]
    a8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, -(-K // 128)), dtype=torch.float32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    nws = m.gemm_fp8_blockscale_workspace(M, N, K)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev) if nws else False
    for i in range(warmup):
        m.fp8_quant_1x128(d["a"], a8, sa)
        m.gemm_fp8_blockscale(a8, sa, bs[i % ncopy], d["b_scale"], c, workspace=ws, preshuffled=preshuffle)
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold_stream(stream, 0.1 * steps + 1)  # the steps run back to back on the GPU
    start.record(stream)
    for i in range(steps):
        m.fp8_quant_1x128(d["a"], a8, sa)
        m.gemm_fp8_blockscale(a8, sa, bs[i % ncopy], d["b_scale"], c, workspace=ws, preshuffled=preshuffle)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # the GEMM call alone (with its split-K reduce), K launches back to back on the same stream:
    # events around every microsecond-scale launch would mostly time the events
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_stream(stream, 0.1 * steps + 1)
    g0.record(stream)
    for i in range(steps):
        m.gemm_fp8_blockscale(a8, sa, bs[(i + 1) % ncopy], d["b_scale"], c, workspace=ws, preshuffled=preshuffle)
    g1.record(stream)
    torch.cuda.synchronize()
    gms = g0.elapsed_time(g1) / steps
    flops = 2.0 * M * N * K
    nb, kb = -(-N // 128), -(-K // 128)
    gbytes = N * K + 4 * nb * kb + M * K + 4 * M * kb + 2 * M * N
    del bs, d
    return {"ms": ms, "gemm_ms": gms, "flops": flops, "bytes": gbytes, "copies": ncopy, "workspace": nws}


def dense_roof(M, t):
    if M <= 64:
        roof = {"bound": "hbm", "achieved": t["bytes"] / (t["gemm_ms"] * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": t["flops"] / (t["gemm_ms"] * 1e-3) / 1e12, "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof.update(frac=roof["achieved"] / roof["peak"], kernel="gemm_fp8_blockscale", kernel_ms=t["gemm_ms"])
    return roof


def bench_dense(a):
    from fp8_block_scaled_grouped_amd import inputs
    M, N, K = a.dense_m, a.dense_n, inputs.DENSE_K
    t = time_dense(M, N, K, a.steps, a.warmup, a.seed, a.preshuffle)
    roof = dense_roof(M, t)
    roof["traffic"] = measured_traffic("dense_%d_%d" % (M, N), "dense")
    return {"metric": "FP8 blockscale dense GEMM TFLOP/s", "value": t["flops"] / (t["ms"] * 1e-3) / 1e12,
            "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": t["ms"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3 (fp32 accumulate)",
            "data": "synthetic",
            "config": {"workload": "dense FP8 block-scale GEMM M=%d N=%d K=%d (quant + GEMM)" % (M, N, K),
                       "M": M, "N": N, "K": K, "weight_copies": t["copies"], "split_k_workspace_bytes":
                       t["workspace"], "preshuffled_weights": bool(a.preshuffle), "seed": a.seed},
            "roofline": roof}


SWEEP_M = (1, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096)


def dense_candidates(M, K):
    """(tile_m, tile_n, splits) tilings the dense sweep times for M rows and K."""
    KB = -(-K // 128)
    bms = [16] if M <= 16 else [16, 32] if M <= 32 else [32, 64] if M <= 64 else [64, 128] if M <= 128 else [128]
    least = -(-KB // 128)  # runs of at most 128 K blocks
    splits = sorted({max(least, s) for s in ((1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48) if M <= 256 else (1,))
                     if s == 1 or KB // s >= 2})
    plans = [(bm, bn, s) for bm in bms for bn in (128, 256) for s in splits]
    if M <= 64:  # the small-M kernel: 16-column tiles, K split inside the workgroup
        plans.append((16 if M <= 16 else 32 if M <= 32 else 64, 16, 1))
    return plans


def sweep_dense(a):
    """Every linear-layer shape of a DeepSeek-V3 layer at M in SWEEP_M: the call as it
    stands (default_us), the rule's plan alone (rule) and each candidate tiling
    (gemm_fp8_blockscale_tiled), timed back to back over rotated weight copies; one JSON
    line per (shape, M) with every timing."""
    import torch

    import fp8_block_scaled_grouped_amd as m
    from fp8_block_scaled_grouped_amd import inputs

    dev = torch.device("cuda:0")
    Ms = (a.tokens,) if a.tokens else SWEEP_M
    stream = torch.cuda.current_stream()
    for name, N, K in V3_LINEAR:
        d = inputs.make_dense_inputs(max(Ms), N, K, dev, seed=a.seed)
        ncopy = max(1, min(48, (8 << 30) // (N * K)))
        bs = [d["b"]] + [d["b"].clone() for _ in range(ncopy - 1)]
        a8_all, sa_all = m.fp8_quant_1x128(d["a"])
        for M in Ms:
            a8, sa = a8_all[:M].contiguous(), sa_all[:M].contiguous()
            c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            reps = 10 if M <= 256 else 4

            def timed(fn):
                for i in range(2):
                    fn(bs[i % ncopy])
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                hold_stream(stream, 0.1 * reps + 1)
                e0.record(stream)
                for i in range(reps):
                    fn(bs[(i + 2) % ncopy])
                e1.record(stream)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) / reps * 1e3

            nws = m.gemm_fp8_blockscale_workspace(M, N, K)
            ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
            default_us = timed(lambda b: m.gemm_fp8_blockscale(a8, sa, b, d["b_scale"], c, workspace=ws))
            plans = []
            for bm, bn, sp in dense_candidates(M, K):
                tws = torch.empty(max(m.gemm_fp8_blockscale_tiled_workspace(M, N, K, sp), 16), dtype=torch.uint8,
                                  device=dev)
                plans.append([bm, bn, sp, round(timed(lambda b: m.gemm_fp8_blockscale_tiled(
                    a8, sa, b, d["b_scale"], bm, bn, sp, c, tws)), 3)])
                del tws
            # the rule's plan (what the table's entries must beat), timed as a tiling
            rtm, rtn, rsp = m.gemm_fp8_blockscale_plan(M, N, K, measured=False)
            tws = torch.empty(max(m.gemm_fp8_blockscale_tiled_workspace(M, N, K, rsp), 16), dtype=torch.uint8,
                              device=dev)
            rule = [rtm, rtn, rsp, round(timed(lambda b: m.gemm_fp8_blockscale_tiled(
                a8, sa, b, d["b_scale"], rtm, rtn, rsp, c, tws)), 3)]
            del tws
            best = min(plans, key=lambda p: p[3])
            flops, nbytes = 2.0 * M * N * K, N * K + M * K + 2 * M * N
            print(json.dumps({"sweep": "dense", "layer": name, "M": M, "N": N, "K": K, "default_us": round(default_us, 3),
                              "rule": rule, "best": best, "best_tflops": round(flops / best[3] / 1e6, 2),
                              "best_gbs": round(nbytes / best[3] / 1e3, 1), "plans": plans}),
                  flush=True)
        del bs, d, a8_all, sa_all
        torch.cuda.empty_cache()


def phases(a):
    """Per-step phase clocks of the gate/up kernel (128-row tiles) from the diagnostic
    library libmoe355_trace.so: for K steps 1 .. KB-2 of every traced tile and wave, the
    shader cycles spent waiting for the wave's own stage DMAs, at the barrier that
    publishes the stage, and computing (MFMAs, folds, fragment reads, the next stage's
    DMA issues) until the next step starts."""
    import ctypes

    import numpy as np
    import torch

    from fp8_block_scaled_grouped_amd import moe355
    path = os.path.join(ROOT, "fp8_block_scaled_grouped_amd", "libmoe355_trace.so")
    if not os.path.exists(path):
        sys.exit("bench.py --phases: %s is not built (python -m fp8_block_scaled_grouped_amd.build)" % path)
    moe355.LIB_PATH, moe355._lib = path, None
    import fp8_block_scaled_grouped_amd as m

    wl = a.workload if a.workload in ("prefill", "skew", "prefill_bias0", "skew_zipf") else "prefill"
    cfg = moe_config(wl, a.tokens)
    x = moe_inputs(cfg, a.seed)
    layer = m.MoELayer(cfg, x["bias"], x["w1"], x["w1_scale"], x["w2"], x["w2_scale"], block_m=128)
    for _ in range(max(a.warmup, 1) + 1):  # the trace keeps the last launch's tiles [0, 64)
        layer.forward(x["hidden"], x["logits"])
    torch.cuda.synchronize()
    n = 64 * 8 * 64 * 3
    buf = np.zeros(n, np.uint32)
    fn = m.lib().moe355_phase_trace_read
    fn.argtypes, fn.restype = [ctypes.c_void_p, ctypes.c_size_t], ctypes.c_int
    if fn(buf.ctypes.data, n) != 0:
        sys.exit("bench.py --phases: reading the trace failed")
    t = buf.reshape(64, 8, 64, 3).astype(np.int64)
    KB = min(cfg.H // 128, 64)
    d = lambda x: (x % (1 << 32))  # clocks are the low 32 bits
    wait = d(t[:, :, 1:KB - 1, 1] - t[:, :, 1:KB - 1, 0])
    barrier = d(t[:, :, 1:KB - 1, 2] - t[:, :, 1:KB - 1, 1])
    compute = d(t[:, :, 2:KB, 0] - t[:, :, 1:KB - 1, 2])
    step = d(t[:, :, 2:KB, 0] - t[:, :, 1:KB - 1, 0])
    q = lambda v: {"median": float(np.median(v)), "mean": float(v.mean()), "p10": float(np.percentile(v, 10)),
                   "p90": float(np.percentile(v, 90))}
    per_wave = {ph: [float(np.median(v[:, w_])) for w_ in range(8)]
                for ph, v in (("stage_wait", wait), ("barrier", barrier), ("compute", compute))}
    print(json.dumps({"phases": "moe_fp8_blockscale_g1u1 (128-row tiles, 8 waves, 3 stages)", "workload": wl,
                      "tokens": cfg.T, "k_steps": KB, "tiles_traced": 64, "unit": "shader clock cycles (s_memtime)",
                      "per_step": {"stage_wait": q(wait), "barrier": q(barrier), "compute": q(compute),
                                   "step": q(step)},
                      "per_wave_median": per_wave,
                      "stage_bytes": 48 * 1024, "mfma_cycles_per_step_per_simd": 1024}), flush=True)


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: libmoe355 runs the layer on one GPU (it is not sharded across GPUs); "
              "run without --gpus or with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if a.sweep == "block_m":
        sweep_block_m(a)
        return
    if a.sweep == "dense":
        sweep_dense(a)
        return
    if a.sweep == "tiles":
        sweep_tiles(a)
        return
    if a.phases:
        phases(a)
        return
    res = bench_dense(a) if a.workload == "dense" else bench_moe(a)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
