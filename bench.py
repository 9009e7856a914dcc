"""Benchmark of the FP8 block-scale MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|skew|tiny|dense]
                    [--block-m BM] [--dense-m M --dense-n N] [--no-cpu-baseline]

A step is one pass of the whole layer -- grouped_topk, moe_sort,
fp8_quant_1x128, moe_fp8_blockscale_g1u1, moe_down_combine -- over one batch
of synthetic tokens whose inputs and weights are already resident in HBM.
(`--workload dense` times fp8_quant_1x128 + gemm_fp8_blockscale instead.)
Prints one JSON line.  The default workload is the 64-token decode layer
of DeepSeek-V3 shape (hidden 7168, intermediate 2048, 256 experts in 8
groups, topk_group 4, top-8).
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
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "skew", "tiny", "dense", "prefill_bias0", "skew_zipf"],
                    help="prefill_bias0 / skew_zipf: labelled routing controls (zero bias; Zipf without the hot bias)")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--graph", action="store_true",
                    help="also time the layer captured once as a HIP graph and replayed (graph_ms_per_step)")
    ap.add_argument("--preshuffle", action="store_true",
                    help="weights permuted once into the 128x128-tile layout (the *_wpreshuffle calls)")
    ap.add_argument("--dense-m", type=int, default=64)
    ap.add_argument("--dense-n", type=int, default=18432)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after timing, copy BYTES bytes device-to-device 3 times (plain copy kernel whose "
                         "FETCH_SIZE / WRITE_SIZE calibrate the traffic counters)")
    return ap.parse_args()


KERNEL_SOURCES = ["fp8_block_scaled_grouped_amd/csrc/gemm.hip", "fp8_block_scaled_grouped_amd/csrc/device_common.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


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


def cpu_baseline_moe(cfg, hidden, logits, bias, w1, s1, w2, s2, budget_s):
    """Time the oracle on the host for as many tokens as fit in about budget_s seconds.

    The oracle runs as it stands: routing for all tokens, then token by token the
    1x128 quantisation and the token-major expert evaluation.  Weight copies to the
    host are made before the clock starts.
    """
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = 1
    hid = oracle.fp8.bf16_bits_to_f32(hidden.cpu().view(torch_int16()).numpy().view(np.uint16))
    logits = logits.cpu().numpy()
    bias = bias.cpu().numpy()
    s1, s2 = s1.cpu().numpy(), s2.cpu().numpy()
    W1, W2 = _ExpertRows(w1), _ExpertRows(w2)
    t0 = time.perf_counter()
    w, ids = oracle.routing.grouped_topk(logits, bias, cfg.n_group, cfg.topk_group, cfg.topk, cfg.renorm,
                                         cfg.routed_scaling_factor)
    t_route = time.perf_counter() - t0
    done, el = 0, 0.0
    while done < cfg.T and el < budget_s:
        for e in ids[done]:                       # host copies outside the clock
            W1[e], W2[e]
        t0 = time.perf_counter()
        a8, sa = oracle.quant.quant_1x128(hid[done:done + 1])
        oracle.moe.layer_tokens(a8, sa, W1, s1, W2, s2, ids[done:done + 1], w[done:done + 1])
        el += time.perf_counter() - t0
        done += 1
    sec = el + t_route * done / cfg.T
    return {"value": done / sec, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d of %d tokens through the whole layer (routing of all %d tokens charged pro rata), "
                      "%.1f s" % (done, cfg.T, cfg.T, sec)}


def torch_int16():
    import torch
    return torch.int16


def bench_moe(a):
    import numpy as np
    import torch

    import fp8_block_scaled_grouped_amd as m
    from fp8_block_scaled_grouped_amd import inputs

    cfg = {**inputs.MOE_CONFIGS, **inputs.CONTROL_CONFIGS}[a.workload]
    bm = a.block_m or cfg.block_m
    dev = torch.device("cuda:0")
    t0 = time.time()
    x = inputs.make_moe_inputs(cfg, "cpu" if a.workload == "tiny" else dev, seed=a.seed)
    x = {k: v.to(dev) for k, v in x.items()}
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    layer = m.MoELayer(cfg, x["bias"], x["w1"], x["w1_scale"], x["w2"], x["w2_scale"], block_m=bm,
                       preshuffle=a.preshuffle)
    hidden, logits = x["hidden"], x["logits"]

    stream = torch.cuda.current_stream()
    for _ in range(a.warmup):
        layer.forward(hidden, logits)
    torch.cuda.synchronize()

    # timed region: K whole steps; the dominant kernel (g1u1) bracketed by events inside it
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    st = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]  # start of each step
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c = cfg
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(a.steps):
        st[i].record(stream)
        m.grouped_topk(logits, layer.bias, c.n_group, c.topk_group, c.topk, c.renorm, c.routed_scaling_factor,
                       layer.topk_w, layer.topk_ids)
        sid, sw, seid, nv = m.moe_sort(layer.topk_ids, layer.topk_w, c.E, bm, layer.sort_out, layer.sort_ws)
        m.fp8_quant_1x128(hidden, layer.a8, layer.a_scale)
        ev[i][0].record(stream)
        m.moe_fp8_blockscale_g1u1(layer.a8, layer.a_scale, layer.w1, layer.w1_scale, sid, seid, nv, c.topk, bm,
                                  layer.h8, layer.h_scale, preshuffled=layer.preshuffle)
        ev[i][1].record(stream)
        m.moe_down_combine(layer.h8, layer.h_scale, layer.w2, layer.w2_scale, sid, sw, seid, nv, layer.T, c.topk,
                           bm, layer.out, layer.down_ws, preshuffled=layer.preshuffle)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / a.steps
    g1u1_ms = sum(s.elapsed_time(e) for s, e in ev) / a.steps
    steps_ms = sorted([st[i].elapsed_time(st[i + 1]) for i in range(a.steps - 1)] + [st[-1].elapsed_time(end)])
    layer_stats = {"median_ms": steps_ms[len(steps_ms) // 2], "min_ms": steps_ms[0]}

    graph = None
    if a.graph:
        # the five calls captured once into a HIP graph (the library allocates nothing and
        # never synchronises, so the layer is capturable) and replayed K times
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(hidden, logits)
        for _ in range(a.warmup):
            g.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(a.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph = g0.elapsed_time(g1) / a.steps
        del g

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
        ("moe_down_combine", lambda: m.moe_down_combine(layer.h8, layer.h_scale, layer.w2, layer.w2_scale, sid, sw,
                                                        seid, nv, layer.T, c.topk, bm, layer.out,
                                                        layer.down_ws, preshuffled=layer.preshuffle)),
    ]
    reps = max(10, a.steps)
    cev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
           for _ in range(reps)]
    for r in range(reps):
        for (name, fn), (e0, e1) in zip(calls, cev[r]):
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    per_call = {}
    for ci, (name, _) in enumerate(calls):
        t = sorted(cev[r][ci][0].elapsed_time(cev[r][ci][1]) for r in range(reps))
        per_call[name] = {"median_ms": t[len(t) // 2], "min_ms": t[0]}

    ids = layer.topk_ids.cpu().numpy()
    hot = inputs.hot_expert_mask(cfg, dev, a.seed).cpu().numpy() if cfg.skew else None
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
    hbm_bound = cfg.T <= 512
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": g1u1_bytes / (g1u1_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": g1u1_flops / (g1u1_ms * 1e-3) / 1e12, "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = "moe_fp8_blockscale_g1u1"
    roof["kernel_ms"] = g1u1_ms
    roof["traffic"] = measured_traffic(a.workload, "g1u1")

    res = {
        "metric": "FP8 blockscale MoE layer tokens/s", "value": T / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "%s MoE layer: %d tokens, hidden %d, intermediate %d, %d experts / %d groups, "
                               "topk_group %d, top-%d, block_m %d" % (a.workload, T, H, I, cfg.E, cfg.n_group,
                                                                      cfg.topk_group, k, bm),
                   "tokens": T, "hidden": H, "intermediate": I, "experts": cfg.E, "topk": k, "block_m": bm,
                   "preshuffled_weights": bool(a.preshuffle), "seed": a.seed},
        "layer_tflops": flops / (ms * 1e-3) / 1e12, "layer_gbs": nbytes / (ms * 1e-3) / 1e9,
        "layer_frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_frac_mfma": flops / (ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "routing": rs, "roofline": roof, "layer_ms": layer_stats, "per_call_ms": per_call,
        "input_gen_s": round(gen_s, 2),
    }
    if graph is not None:
        res["graph_ms_per_step"] = graph
        res["graph_tokens_per_s"] = T / (graph * 1e-3)
    if not a.no_cpu_baseline:
        # the oracle reads the weights as loaded (row-major), not the layer's shuffled copies
        res["cpu_baseline"] = cpu_baseline_moe(cfg, hidden, logits, layer.bias, x["w1"], layer.w1_scale, x["w2"],
                                               layer.w2_scale, a.cpu_seconds)
    return res


def bench_dense(a):
    import torch

    import fp8_block_scaled_grouped_amd as m
    from fp8_block_scaled_grouped_amd import inputs

    M, N, K = a.dense_m, a.dense_n, inputs.DENSE_K
    dev = torch.device("cuda:0")
    d = inputs.make_dense_inputs(M, N, K, dev, seed=a.seed)
    # rotate distinct weight copies so a small B is not served from the 256 MB MALL
    ncopy = max(1, min(48, (8 << 30) // (N * K)))  # >= 40 copies below 200 MB of weights
    bs = [d["b"]] + [d["b"].clone() for _ in range(ncopy - 1)]
    if a.preshuffle:
        bs = [m.shuffle_weight_128x128(b) for b in bs]
    a8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    nws = m.gemm_fp8_blockscale_workspace(M, N, K)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else False
    for i in range(a.warmup):
        m.fp8_quant_1x128(d["a"], a8, sa)
        m.gemm_fp8_blockscale(a8, sa, bs[i % ncopy], d["b_scale"], c, workspace=ws, preshuffled=a.preshuffle)
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(a.steps):
        m.fp8_quant_1x128(d["a"], a8, sa)
        m.gemm_fp8_blockscale(a8, sa, bs[i % ncopy], d["b_scale"], c, workspace=ws, preshuffled=a.preshuffle)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / a.steps
    # the GEMM call alone (with its split-K reduce), K launches back to back on the same stream:
    # events around every microsecond-scale launch would mostly time the events
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for i in range(a.steps):
        m.gemm_fp8_blockscale(a8, sa, bs[(i + 1) % ncopy], d["b_scale"], c, workspace=ws, preshuffled=a.preshuffle)
    g1.record(stream)
    torch.cuda.synchronize()
    gms = g0.elapsed_time(g1) / a.steps
    flops = 2.0 * M * N * K
    gbytes = N * K + 4 * (N // 128) * (K // 128) + M * K + 4 * M * (K // 128) + 2 * M * N
    if M <= 64:
        roof = {"bound": "hbm", "achieved": gbytes / (gms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / (gms * 1e-3) / 1e12, "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof.update(frac=roof["achieved"] / roof["peak"], kernel="gemm_fp8_blockscale", kernel_ms=gms,
                traffic=measured_traffic("dense_%d_%d" % (M, N), "dense"))
    return {"metric": "FP8 blockscale dense GEMM TFLOP/s", "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
            "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3 (fp32 accumulate)", "data": "synthetic",
            "config": {"workload": "dense FP8 block-scale GEMM M=%d N=%d K=%d (quant + GEMM)" % (M, N, K),
                       "M": M, "N": N, "K": K, "weight_copies": ncopy, "split_k_workspace_bytes": nws,
                       "preshuffled_weights": bool(a.preshuffle), "seed": a.seed},
            "roofline": roof}


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: libmoe355 runs the layer on one GPU (it is not sharded across GPUs); "
              "run without --gpus or with --gpus 1", file=sys.stderr)
        sys.exit(2)
    res = bench_dense(a) if a.workload == "dense" else bench_moe(a)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
