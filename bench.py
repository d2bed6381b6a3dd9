"""Benchmark of the fp8 block-quantized MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config dsv3_prefill]

One step = one moe_forward over one batch (stage + routing, the w13 GEMM
with SiLU(gate)*up and the fp8 re-quantization fused into its epilogue, the
w2 GEMM, top-k reduce; for the indexed layout the block map, the gather /
scatter GEMMs and the fused mul-sum), inputs resident in HBM.  Prints one JSON line: layer
tokens/s, grouped-GEMM TFLOP/s against the fp8 dense MFMA peak, per-kernel
times, the roofline of the dominant kernel (the fused w13 GEMM) and the CPU
oracle timed on a bounded sample.  Diagnostics go to stderr.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_block_quantized_group_amd as moe  # noqa: E402
import moe_synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3_prefill", choices=list(moe_synth.ALL_CONFIGS))
    ap.add_argument("--kernel-iters", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mfma-workload", default="qwen3",
                    help="workload whose GEMMs are timed for the MFMA-bound figure "
                         "('none' to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--profile-pass", action="store_true",
                    help="for counter runs: a 1 GiB device copy (counter calibration), then "
                         "each kernel of the layer once; prints no JSON")
    return ap.parse_args()


class KernelTimer:
    """HIP events on the stream the library launches on (torch's current
    stream, passed to every C call)."""

    def __init__(self):
        self.stream = torch.cuda.current_stream()

    def time(self, fn, iters, flush=None):
        times = []
        for _ in range(iters):
            if flush is not None:
                flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            fn()
            b.record(self.stream)
            b.synchronize()
            times.append(a.elapsed_time(b))
        return float(np.mean(times)), float(np.min(times))


def algorithmic(cfg, counts, T_valid):
    """Minimum HBM bytes and flops of each step (one launch each)."""
    K, N, k = cfg.K, cfg.N, cfg.top_k
    M = int(counts.sum())
    touched = int((counts > 0).sum())
    group = 32 if cfg.act_quant == "mxfp8" else 128
    sfb = 4 if cfg.act_quant == "fp32" else 1       # bytes per activation scale
    ab = 2 if cfg.act_quant == "bf16" else 1        # bytes per activation value
    if cfg.act_quant == "bf16":
        sfb = 0
    GK, GN = K // group, N // group
    rows_in = int(counts.sum()) if cfg.layout == "batched" else cfg.T
    a = {}
    a["stage"] = rows_in * K * 2 + rows_in * K * ab + rows_in * GK * sfb
    if cfg.weight_quant == "fp8_block128":
        w13_sf, w2_sf = (2 * N // 128) * (K // 128) * 4, (K // 128) * (N // 128) * 4
    else:                                            # E8M0 byte per row and 32 columns
        w13_sf, w2_sf = 2 * N * (K // 32), K * (N // 32)
    w_elem = 0.5 if cfg.weight_quant == "mxfp4" else 1
    w13_in = touched * (2 * N * K * w_elem + w13_sf) + T_valid * (K * ab + GK * sfb)
    a["w13_act_bytes"] = w13_in + M * (N * ab + GN * sfb)   # a2 (+ scales) out
    a["w13_flops"] = 2.0 * M * 2 * N * K
    a["w2_bytes"] = (touched * (K * N * w_elem + w2_sf) + M * (N * ab + GN * sfb) + M * K * 2)
    a["w2_flops"] = 2.0 * M * N * K
    a["reduce"] = M * K * 2 + cfg.T * K * 2 + cfg.T * k * 8
    # indexed layout: slot rows and ids in, one sorted id per routed slot out
    a["align"] = cfg.T * k * (4 + 8) + M * 4
    return a


def per_expert_bound_ms(cfg, counts):
    """Lower bound of each grouped GEMM in ms: every routed expert either
    streams its weights once from HBM or runs its rows on the matrix cores at
    the dense fp8 peak, whichever is slower, summed over experts
    (sum_e max(flops_e / P, weight_bytes_e / B))."""
    K, N = cfg.K, cfg.N
    w_elem = 0.5 if cfg.weight_quant == "mxfp4" else 1
    if cfg.weight_quant == "fp8_block128":
        w13_sf, w2_sf = (2 * N // 128) * (K // 128) * 4, (K // 128) * (N // 128) * 4
    else:
        w13_sf, w2_sf = 2 * N * (K // 32), K * (N // 32)
    P, B = FP8_PEAK_TFLOPS * 1e12, HBM_PEAK_GBS * 1e9
    m = counts[counts > 0].astype(np.float64)
    b13 = np.maximum(2 * m * 2 * N * K / P, (2 * N * K * w_elem + w13_sf) / B).sum()
    b2 = np.maximum(2 * m * N * K / P, (K * N * w_elem + w2_sf) / B).sum()
    return 1e3 * b13, 1e3 * b2


def gemm_figures(cfg, counts, t13_ms, t2_ms):
    """TFLOP/s of both GEMMs, their fraction of the fp8 dense peak and of
    the per-expert bound."""
    M = float(counts.sum())
    flops = 2.0 * M * 2 * cfg.N * cfg.K + 2.0 * M * cfg.N * cfg.K
    tf = flops / ((t13_ms + t2_ms) * 1e-3) / 1e12
    b13, b2 = per_expert_bound_ms(cfg, counts)
    return {"gemm_tflops": round(tf, 2), "gemm_frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
            "w13_bound_ms": round(b13, 4), "w2_bound_ms": round(b2, 4),
            "w13_frac": round(b13 / t13_ms, 4), "w2_frac": round(b2 / t2_ms, 4),
            "frac": round((b13 + b2) / (t13_ms + t2_ms), 4)}


def mfma_bound_workload(name, iters, flush):
    """The GEMMs of the MFMA-bound workload (every expert has hundreds of
    rows), timed like the headline's kernels: MALL flushed before each
    launch, on the stream the library launches on."""
    cfg = moe_synth.ALL_CONFIGS[name]
    log(f"[bench] MFMA-bound workload {name}: generating inputs")
    inp = moe_synth.make_inputs(cfg, "cuda")
    p = moe.Problem.from_config(cfg)
    out = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")
    bufs, calls = layer_kernels(p, cfg, inp, out)
    for _, fn in calls:             # once in order: routing, then each GEMM's input
        fn()
    torch.cuda.synchronize()
    kt = KernelTimer()
    t = {n: kt.time(fn, iters, flush)[0] for n, fn in calls
         if n in ("grouped_gemm_w13_act", "grouped_gemm_w2")}
    counts = bufs["expert_num_tokens"].cpu().numpy()
    fig = gemm_figures(cfg, counts, t["grouped_gemm_w13_act"], t["grouped_gemm_w2"])
    res = {"workload": name, "w13_act_ms": round(t["grouped_gemm_w13_act"], 4),
           "w2_ms": round(t["grouped_gemm_w2"], 4), "gemm_tflops": fig["gemm_tflops"],
           "gemm_frac_fp8_peak": fig["gemm_frac_fp8_peak"],
           "per_expert_roofline_frac": fig["frac"]}
    del inp, bufs, calls, out
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg, inp, st_dev, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of tokens."""
    from oracle import moe_oracle as O
    from threadpoolctl import threadpool_info
    h = {}
    for key, v in inp.items():
        if key in ("w13", "w13_sf", "w2", "w2_sf") or key == "cfg":
            h[key] = v
        elif key == "eplb" and v is not None:
            h[key] = {k2: O._np(v2) for k2, v2 in v.items()}
        else:
            h[key] = O._np(v)
    t0 = time.perf_counter()
    st = O.stage_routing_only(h)
    routed = np.flatnonzero((st["slot_row"] >= 0).any(axis=1))
    rng = np.random.default_rng(1234)
    order = rng.permutation(routed)
    done = 0
    t_route = time.perf_counter() - t0
    t1 = time.perf_counter()
    while done < len(order) and time.perf_counter() - t1 < budget_s:
        O.forward_tokens(h, [int(order[done])], st)
        done += 1
    dt = time.perf_counter() - t1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": done / dt if dt > 0 else 0.0, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"{done} routed tokens of {cfg.name} through the whole layer one by one "
                       f"(numpy fp64), after the full routing layout ({t_route:.2f} s); "
                       f"{dt:.1f} s of CPU work; host has {os.cpu_count()} cpus")}


CALIB_BYTES = 1 << 30


def layer_kernels(p, cfg, inp, out):
    """Buffers and one callable per step of the layer through the separate
    entry points, in moe_forward's launch configuration: (bufs, calls) with
    calls = [(name, fn)] in launch order.  The indexed layout runs the block
    map (moe_align_block_size), the gather / scatter GEMMs and the fused
    mul-sum."""
    s = moe.sizes(p)
    bufs = moe.alloc_stage_outputs(p)
    a2_q, a2_sf = moe.alloc_act_outputs(p)
    down = torch.empty((s["expert_rows"], cfg.K), dtype=torch.bfloat16, device="cuda")
    w2_ws = moe.alloc_w2_workspace(p)

    def do_stage():
        if inp["eplb"] is not None:
            inp["eplb"]["expert_load"].zero_()
        moe.stage(p, inp["hidden"], inp["topk_ids"], inp["topk_weights"], bufs,
                  inp["is_padding"], inp["expert_num_tokens"], inp["eplb"])

    calls = [("stage_and_route", do_stage)]
    if p.layout == moe.LAYOUT_INDEXED:
        ix = moe.alloc_indexed(p, s["tile_m"])
        calls += [
            ("align_block_size",
             lambda: moe.align_block_size(p, bufs["topk_idx"], bufs, ix)),
            ("grouped_gemm_w13_act",
             lambda: moe.grouped_gemm_w13_act_indexed(p, bufs["x_q"], bufs["x_sf"], ix,
                                                      inp["w13"], inp["w13_sf"], a2_q, a2_sf)),
            ("grouped_gemm_w2",
             lambda: moe.grouped_gemm_w2_indexed(p, a2_q, a2_sf, ix, inp["w2"], inp["w2_sf"],
                                                 down, w2_ws)),
            ("topk_reduce",
             lambda: moe.fused_mul_sum(p, down, bufs["topk_idx"], bufs["topk_w"], out)),
        ]
    else:
        calls += [
            ("grouped_gemm_w13_act",
             lambda: moe.grouped_gemm_w13_act(p, bufs["x_q"], bufs["x_sf"], bufs, inp["w13"],
                                              inp["w13_sf"], a2_q, a2_sf)),
            ("grouped_gemm_w2",
             lambda: moe.grouped_gemm_w2(p, a2_q, a2_sf, bufs, inp["w2"], inp["w2_sf"], down,
                                         w2_ws)),
            ("topk_reduce",
             lambda: moe.topk_reduce(p, down, bufs["slot_row"], bufs["topk_w"], out)),
        ]
    return bufs, calls


def profile_pass(p, cfg, inp, out):
    """A plain 1 GiB device-to-device copy (so HBM byte counters can be scaled
    by what they read for a known size), then each kernel of the layer once
    through the separate entry points, in moe_forward's launch configuration."""
    src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    _, calls = layer_kernels(p, cfg, inp, out)
    for _, fn in calls:
        fn()
    cast = stage_ceiling_call(cfg, inp)
    if cast is not None:
        cast()
    torch.cuda.synchronize()
    log(f"[bench] profile pass done ({cfg.name})")


def stage_ceiling_call(cfg, inp):
    """torch's own cast of the hidden states to fp8 e4m3: the same bf16
    bytes read and fp8 bytes written as the staging quantizer (no scales, no
    group maxima), a ceiling for that kernel at this size."""
    if cfg.act_quant == "bf16" or cfg.layout == "batched":
        return None
    dst = torch.empty(inp["hidden"].shape, dtype=torch.float8_e4m3fn, device="cuda")
    return lambda: dst.copy_(inp["hidden"])


# the sources that decide what the fused w13 step moves: the kernel, the tile
# schedules the routing scan builds, and the launch configuration
TRAFFIC_SOURCES = ("grouped_gemm.hip", "route_kernels.hip", "moe_api.hip")


def sources_digest(files=TRAFFIC_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "fp8_block_quantized_group_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per call of the fused w13 step (its launches added), from the
    committed counter summary, only if none of the sources that decide it
    has changed since it was taken."""
    digest = sources_digest()
    path = os.path.join(ROOT, "profiles", f"grouped_gemm_w13_act_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("sources_sha256") != digest:
        return None
    return float(fields["hbm_bytes_per_launch"])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the expert layer "
              "is not sharded across GPUs here.", file=sys.stderr)
        sys.exit(2)
    cfg = moe_synth.ALL_CONFIGS[args.config]
    torch.cuda.set_device(0)
    log(f"[bench] generating {cfg.name} inputs on the GPU")
    inp = moe_synth.make_inputs(cfg, "cuda")
    p = moe.Problem.from_config(cfg)
    layer = moe.MoeLayer(p, inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"])
    out = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")

    def step():
        if inp["eplb"] is not None:
            inp["eplb"]["expert_load"].zero_()
        layer(inp["hidden"], inp["topk_ids"], inp["topk_weights"], out, inp["is_padding"],
              inp["expert_num_tokens"], inp["eplb"])

    if args.profile_pass:
        profile_pass(p, cfg, inp, out)
        return
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / max(args.steps, 1)

    # ---- per-kernel timing through the separate entry points -------------
    s = moe.sizes(p)
    bufs, calls = layer_kernels(p, cfg, inp, out)
    flush_buf = torch.empty(1 << 28, dtype=torch.int32, device="cuda")   # 1 GiB > MALL

    def flush():
        flush_buf.add_(1)

    kt = KernelTimer()
    it = args.kernel_iters
    # each call is timed after the ones before it have run (their outputs are
    # its inputs)
    t = {name: kt.time(fn, it, flush) for name, fn in calls}
    t_stage, t_w13, t_w2, t_red = (t["stage_and_route"], t["grouped_gemm_w13_act"],
                                   t["grouped_gemm_w2"], t["topk_reduce"])
    torch.cuda.synchronize()
    counts = bufs["expert_num_tokens"].cpu().numpy()
    T_valid = cfg.T - (int(inp["is_padding"].sum().item()) if inp["is_padding"] is not None
                       else 0)
    alg = algorithmic(cfg, counts, T_valid)

    def gbs(b, t_ms):
        return b / (t_ms * 1e-3) / 1e9

    kernels = {
        "stage_and_route": {"ms": t_stage[0], "GB/s": gbs(alg["stage"], t_stage[0])},
        "grouped_gemm_w13_act": {"ms": t_w13[0], "GB/s": gbs(alg["w13_act_bytes"], t_w13[0]),
                                 "TFLOP/s": alg["w13_flops"] / (t_w13[0] * 1e-3) / 1e12},
        "grouped_gemm_w2": {"ms": t_w2[0], "GB/s": gbs(alg["w2_bytes"], t_w2[0]),
                            "TFLOP/s": alg["w2_flops"] / (t_w2[0] * 1e-3) / 1e12},
        "topk_reduce": {"ms": t_red[0], "GB/s": gbs(alg["reduce"], t_red[0])},
    }
    cast = stage_ceiling_call(cfg, inp)
    if cast is not None:
        t_cast = kt.time(cast, it, flush)
        cast_bytes = cfg.T * cfg.K * 3
        kernels["stage_ceiling_torch_fp8_cast"] = {"ms": t_cast[0],
                                                  "GB/s": gbs(cast_bytes, t_cast[0])}
    if "align_block_size" in t:
        kernels["align_block_size"] = {"ms": t["align_block_size"][0],
                                       "GB/s": gbs(alg["align"], t["align_block_size"][0])}
    for v in kernels.values():
        v["frac_hbm"] = v["GB/s"] / HBM_PEAK_GBS
    gemm_flops = alg["w13_flops"] + alg["w2_flops"]
    gemm_ms = t_w13[0] + t_w2[0]
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    w13_gbs = kernels["grouped_gemm_w13_act"]["GB/s"]
    traffic = recorded_traffic(cfg.name)
    # with a second (256-row) tile list the fused w13 step is two concurrent
    # launches; the HIP events on the calling stream span both (the second
    # stream joins back to it), and the traffic adds both launches' counters
    roofline = {"bound": "hbm", "achieved": round(w13_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(w13_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "grouped_gemm_w13_act",
                "launches": 2 if s["tall_tile_m"] else 1,
                "algorithmic_bytes_per_launch": alg["w13_act_bytes"]}

    per_expert = gemm_figures(cfg, counts, t_w13[0], t_w2[0])
    mfma_wl = None
    if args.mfma_workload != "none" and args.mfma_workload != cfg.name:
        mfma_wl = mfma_bound_workload(args.mfma_workload, it, flush)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(cfg, inp, bufs, args.cpu_seconds)

    tokens_per_s = cfg.T / (ms * 1e-3)
    line = {
        "metric": "MoE layer tokens/s (+ grouped-GEMM fp8 TFLOP/s as % of MFMA peak), 1 GPU",
        "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "E": cfg.E, "top_k": cfg.top_k,
                   "K": cfg.K, "N": cfg.N, "layout": cfg.layout, "act_quant": cfg.act_quant,
                   "routing": cfg.routing, "pad_frac": cfg.pad_frac, "T_valid": T_valid,
                   "routed_rows": int(counts.sum()), "tile_m": s["tile_m"],
                   "tall_tile_m": s["tall_tile_m"]},
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_frac_fp8_peak": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kernels.items()},
        "roofline": roofline,
        # both GEMMs against the sum over experts of max(MFMA time at the fp8
        # dense peak, weight streaming time at the HBM peak)
        "gemm_per_expert_roofline": {k: per_expert[k] for k in
                                     ("w13_bound_ms", "w2_bound_ms", "w13_frac", "w2_frac",
                                      "frac")},
        "mfma_bound_workload": mfma_wl,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
