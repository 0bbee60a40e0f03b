#!/usr/bin/env python3
"""Throughput of the pre-LN ViT encoder block on one MI355X.

One step = one full block forward (LN1, qkv projection, attention, out
projection + residual, LN2, fc1 + GELU, fc2 + residual) over one batch of
seeded synthetic tokens already resident in HBM, through the C ABI. Prints
one JSON line per workload with tokens/s (K event-free steps), per-stage
device times from a second pass of K steps whose kernels carry HIP start/stop
events on the launch stream, the MFMA-path TFLOP/s and the roofline of the
dominant kernel from those times, and the CPU oracle timed on the host
cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME|all]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encoder-block tokens/sec + attention/GEMM TFLOP/s as % of bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA, 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_F32_TFLOPS = 157.3     # dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
DEFAULT_CONFIG = "c5g_sam3_global"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def describe(spec):
    n = spec["grid_h"] * spec["grid_w"]
    mode = {"mask_unit": "%d mask units" % spec["n_windows"],
            "spatial": "%dx%d windows" % (spec["win_h"], spec["win_w"]),
            "global": "global attention"}[spec["mode"]]
    extra = []
    if spec["q_stride"] == 4:
        extra.append("q/residual 2x2 max-pool, D %d->%d" % (spec["dim_in"], spec["dim_out"]))
    if spec["rope"]:
        extra.append("axial RoPE")
    if spec["qkv"] == "separate":
        extra.append("separate q/k/v")
    if spec.get("weights") == "q8_row":
        extra.append("q8_row int8 weights")
    if spec.get("qk_gain", 1.0) != 1.0:
        extra.append("query/key weights x%g" % spec["qk_gain"])
    return "%s: %d x %dx%d tokens (%d), D %d, %d heads x %d, %s, MLP %d %s-GELU%s" % (
        spec["name"], spec["batch"], spec["grid_h"], spec["grid_w"], n, spec["dim_out"], spec["heads"],
        spec["dim_out"] // spec["heads"], mode, spec["mlp"], spec["gelu"],
        (", " + ", ".join(extra)) if extra else "")


def measured_traffic(config, stage):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current source of the stage's kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    from vision_transformer_encoder_vit_amd.profsum import src_hash
    rec = t.get(config, {}).get(stage)
    if not rec or rec.get("src_sha") != src_hash(stage):
        return None
    return rec["bytes_per_launch"]


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo) and the number
    of cores this process may run on."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return name, len(os.sched_getaffinity(0))


def cpu_baseline(spec, budget_s=20.0, max_runs=3):
    """The float64 CPU oracle on frame 0 of the workload: whole block forwards
    until max_runs are done or budget_s has passed (at least one); the median
    run gives tokens/s. Reports the BLAS threads it used and the CPU model."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import block as ob
    from vision_transformer_encoder_vit_amd import synth
    one = synth.derive(spec, batch=1)
    inp = synth.make_inputs(one, seed=0)
    runs = []
    while len(runs) < max_runs and sum(runs) < budget_s:
        t0 = time.perf_counter()
        ob.block_forward(inp["x"], inp, one)
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    n = one["grid_h"] * one["grid_w"]
    model, ncpu = cpu_model()
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "cpus_available": ncpu,
            "sample": "float64 numpy oracle, one full block forward of frame 0 (%d tokens); median of %d run(s): "
                      "%s s" % (n, len(runs), ", ".join("%.3g" % r for r in runs))}


def oracle_timing(names):
    """The float64 CPU oracle alone: one block forward of frame 0 per workload,
    median of three runs, once on one BLAS thread and once on all of them.
    Prints one JSON line per (workload, threads). No GPU work."""
    from threadpoolctl import threadpool_limits, threadpool_info
    from vision_transformer_encoder_vit_amd import synth
    model, ncpu = cpu_model()
    full = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    for n in names:
        spec = synth.CONFIGS[n]
        for threads in (1, full):
            with threadpool_limits(limits=threads, user_api="blas"):
                line = cpu_baseline(spec, budget_s=60.0, max_runs=3)
            print(json.dumps({"workload": n, "threads": threads, "cpu_model": model, "cpus_available": ncpu,
                              "tokens_per_s": line["value"], "sample": line["sample"]}), flush=True)


def run(spec, steps, warmup, with_cpu):
    import numpy as np
    import torch
    from vision_transformer_encoder_vit_amd import binding as vb
    from vision_transformer_encoder_vit_amd import synth

    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    dt = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32
    q8 = spec.get("weights") == "q8_row"
    gain = spec.get("qk_gain", 1.0)
    inp = synth.make_q8_inputs(spec, seed=0, qk_gain=gain) if q8 else synth.make_inputs(spec, seed=0, qk_gain=gain)
    dev = {}
    for k, a in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        dev[k] = (t.to(dt) if (k == "x" or k.endswith("_w")) and a.dtype != np.int8 else t).cuda()
    plan = vb.Plan(vb.desc_from_spec(spec))
    active = [n for i, n in enumerate(vb.STAGES) if plan.stage_mask() >> i & 1]
    w = vb.weights_struct(dev)
    y = torch.empty((spec["batch"], synth.out_tokens(spec), spec["dim_out"]), dtype=dt, device="cuda")
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    ns = 2 * vb.VIT_NSTAGES
    ev = (ctypes.c_void_p * (ns * steps))()
    slot = lambda i: ctypes.cast(ctypes.addressof(ev) + i * ctypes.sizeof(ctypes.c_void_p),
                                 ctypes.POINTER(ctypes.c_void_p))
    for i in range(ns * steps):
        if hip.hipEventCreate(slot(i)) != 0:
            raise RuntimeError("hipEventCreate failed")
    for _ in range(warmup):
        plan.forward(w, dev["x"], y, ws)
    # timed region: K plain forwards (throughput)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.forward(w, dev["x"], y, ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # kernel-timing pass: the same K forwards with every stage's first/last
    # kernel carrying HIP start/stop events (dispatch-packet timestamps on the
    # launch stream); per-launch durations are averaged over the K steps
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xp, yp, wsp = (ctypes.c_void_p(t.data_ptr()) for t in (dev["x"], y, ws))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        vb.check(vb.lib.vit_block_forward_timed(plan.handle, ctypes.byref(w), xp, yp, wsp, plan.workspace_bytes,
                                                stream, slot(i * ns), ns))
    torch.cuda.synchronize()
    elapsed_timed = time.perf_counter() - t1
    ms = ctypes.c_float()
    stage_us = {}
    for s, name in enumerate(vb.STAGES):
        tot = 0.0
        for i in range(steps):
            a, b = ev[i * ns + 2 * s], ev[i * ns + 2 * s + 1]
            if hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            tot += ms.value
        stage_us[name] = 1e3 * tot / steps
    for i in range(ns * steps):
        hip.hipEventDestroy(ev[i])
    plan.close()

    ms_step = 1e3 * elapsed / steps
    tokens = spec["batch"] * spec["grid_h"] * spec["grid_w"]
    from vision_transformer_encoder_vit_amd.work import stage_work
    wk = stage_work(spec, residual_in_qkv=spec["q_stride"] == 4 and "residual" not in active and "fused" not in active)
    mfma_stages = [st for st in ("qkv", "residual", "attn", "proj", "fc1", "fc2", "fused") if st in active]
    flops = sum(wk[s][0] for s in mfma_stages)
    t_mfma = sum(stage_us[s] for s in mfma_stages) * 1e-6
    peak_c = PEAK_BF16_TFLOPS if spec["dtype"] == "bf16" else PEAK_F32_TFLOPS
    dom = max(active, key=lambda st: stage_us[st])
    f, by = wk[dom]
    t = stage_us[dom] * 1e-6
    ridge = peak_c * 1e12 / (PEAK_HBM_GBS * 1e9)
    if f > 0 and f / by > ridge:
        roof = {"bound": "mfma", "achieved": f / t / 1e12, "peak": peak_c, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": by / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = dom
    roof["traffic"] = measured_traffic(spec["name"], dom)
    line = {
        "metric": METRIC, "value": tokens / (elapsed / steps), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec["dtype"], "data": "synthetic",
        "config": {"workload": describe(spec), "batch": spec["batch"], "tokens_per_frame":
                   spec["grid_h"] * spec["grid_w"], "parallelism": "none (1 GPU)"},
        "attn_gemm_tflops": flops / t_mfma / 1e12,
        "attn_gemm_pct_of_peak": 100.0 * flops / t_mfma / 1e12 / peak_c,
        "stage_us": {k: round(v, 2) for k, v in stage_us.items() if k in active},
        "ms_per_step_with_stage_events": 1e3 * elapsed_timed / steps,
        "roofline": roof,
    }
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(spec)
    return line


COPY_ROWS, COPY_COLS = 65536, 512  # 64 MiB of bf16 read and 64 MiB written per copy


def copy_calibration(steps):
    """K launches of a plain row copy (the unroll kernel with zero levels is
    the identity permutation): each reads and writes exactly
    COPY_ROWS * COPY_COLS * 2 bytes. Prints those bytes per launch."""
    import torch
    from vision_transformer_encoder_vit_amd import binding as vb
    x = torch.randn(1, COPY_ROWS, COPY_COLS, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(x)
    for _ in range(steps):
        vb.vit_unroll(x, y, COPY_ROWS, 1, 0)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    print(json.dumps({"copy_bytes_read_per_launch": COPY_ROWS * COPY_COLS * 2,
                      "copy_bytes_written_per_launch": COPY_ROWS * COPY_COLS * 2, "launches": steps}))


TOWERS = {
    "hiera": "Hiera backbone from pixels: 1 x 512x512x4 -> 7x7/4 patch embed + positions -> 128x128 tokens, "
             "24 blocks (stages of 2/3/16/3, D 112..896), features after blocks 1, 4, 20, 23",
    "sam3": "SAM3 trunk from pixels: 3x1008x1008 -> 14x14 patch embed + tiled positions -> ln_pre -> 32 blocks on "
            "72x72 tokens, D 1024, 24x24 windows, global layers 7/15/23/31",
    "siglip": "SigLIP tower from pixels: 8 frames 3x512x512 -> 16x16 patch embed + bucketized positions -> "
              "12 blocks D 768 on 32x32 tokens -> post_layernorm",
}


def tower_parts(kind):
    """Stem spec, block specs, unroll levels, taps and the LayerNorms before
    (SAM3 ln_pre) and after (SigLIP post_layernorm) the blocks."""
    from vision_transformer_encoder_vit_amd import synth
    pre = post = None
    if kind == "hiera":
        specs, levels, taps = synth.hiera_stack()
    else:
        specs = synth.sam3_trunk() if kind == "sam3" else synth.siglip_tower()
        levels, taps = 0, [len(specs) - 1]
        ln = synth.make_layernorm_params(specs[0]["dim_in"], 0)
        pre, post = (ln, None) if kind == "sam3" else (None, ln)
    return synth.STEMS[kind], specs, levels, taps, pre, post


def run_tower(kind, steps, warmup, with_cpu, q8=False):
    """A whole vision tower from pixels: vit_patch_embed, then (SAM3) ln_pre
    through vit_layernorm, the blocks through vit_stack_forward, then
    (SigLIP) post_layernorm. K event-free forwards timed like the block
    workload; a second pass times the stem alone with events."""
    import numpy as np
    import torch
    from vision_transformer_encoder_vit_amd import binding as vb
    from vision_transformer_encoder_vit_amd import synth, work
    stem, specs, levels, taps, pre, post = tower_parts(kind)
    if q8:
        specs = [dict(s, weights="q8_row") for s in specs]
    sin = synth.make_stem_inputs(stem, seed=0)
    blocks = [(synth.make_q8_inputs if s.get("weights") == "q8_row" else synth.make_inputs)(s, seed=i)
              for i, s in enumerate(specs)]
    for b in blocks:
        del b["x"]
    dt = torch.bfloat16
    dev_w = []
    for w in blocks:
        dev_w.append({k: (torch.from_numpy(np.ascontiguousarray(a)).to(dt) if k.endswith("_w") and a.dtype != np.int8
                          else torch.from_numpy(np.ascontiguousarray(a))).cuda() for k, a in w.items()})
    weights = [vb.weights_struct(w) for w in dev_w]
    px = torch.from_numpy(sin["pixels"]).cuda()
    sw = torch.from_numpy(sin["weight"]).to(dt).cuda()
    sb = torch.from_numpy(sin["bias"]).cuda() if "bias" in sin else None
    spos = torch.from_numpy(sin["pos"]).cuda()
    sdesc = vb.stem_desc_from_spec(stem)
    sws = torch.empty(vb.vit_patch_embed_workspace_size(sdesc), dtype=torch.uint8, device="cuda")
    B, N0, D0 = specs[0]["batch"], specs[0]["grid_h"] * specs[0]["grid_w"], specs[0]["dim_in"]
    tok = torch.empty((B, N0, D0), dtype=dt, device="cuda")
    st = vb.Stack([vb.desc_from_spec(s) for s in specs], levels, taps)
    feats = [torch.empty((specs[t]["batch"], synth.out_tokens(specs[t]), specs[t]["dim_out"]), dtype=dt,
                         device="cuda") for t in taps]
    ws = torch.empty(st.workspace_bytes, dtype=torch.uint8, device="cuda")
    lnd = lambda p: tuple(torch.from_numpy(a).cuda() for a in p) if p is not None else None
    pre_d, post_d = lnd(pre), lnd(post)

    def embed():
        vb.vit_patch_embed(sdesc, px, sw, sb, spos, tok, sws)

    def forward():
        embed()
        if pre_d is not None:
            vb.vit_layernorm(tok, tok, pre_d[0], pre_d[1], specs[0]["eps"])
        st.forward(weights, tok, feats, ws)
        if post_d is not None:
            vb.vit_layernorm(feats[-1], feats[-1], post_d[0], post_d[1], specs[-1]["eps"])

    for _ in range(warmup):
        forward()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        forward()
    torch.cuda.synchronize()
    dt_step = (time.perf_counter() - t0) / steps
    # the stem alone, between whole forwards (so its weights and pixels are
    # as cold as in the timed pass)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        forward()
        e0.record()
        embed()
        e1.record()
    torch.cuda.synchronize()
    stem_us = 1e3 * sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps
    st.close()
    oh, ow = synth.stem_out_grid(stem)
    K = stem["in_ch"] * stem["kernel"] ** 2
    stem_flops = 2.0 * B * oh * ow * stem["dim"] * K
    flops = sum(work.block_flops(s) for s in specs) + stem_flops
    n_q8 = sum(s.get("weights") == "q8_row" for s in specs)
    line = {"metric": "%s tower from pixels, input tokens/sec, 1 GPU" % kind, "value": B * N0 / dt_step,
            "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": 1e3 * dt_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": TOWERS[kind], "batch": B, "tokens_per_frame": N0, "parallelism": "none (1 GPU)",
                       "weights": "q8_row in %d of %d blocks" % (n_q8, len(specs)) if n_q8 else "bf16"},
            "tflops": flops / dt_step / 1e12, "pct_of_bf16_peak": 100.0 * flops / dt_step / 1e12 / PEAK_BF16_TFLOPS,
            "stem_us": round(stem_us, 2), "stem_tflops": round(stem_flops / stem_us / 1e6, 1)}
    if with_cpu and kind in ("hiera", "siglip") and not n_q8:
        # the float64 oracle on one frame (SigLIP: frame 0 of the 8; the
        # SAM3 trunk's 32 full-size layers would take minutes and is skipped)
        from oracle import stack as ost
        from oracle import stem as ostem
        from threadpoolctl import threadpool_info
        one = [synth.derive(s, batch=1) for s in specs]
        stem1 = dict(stem, batch=1)
        sin1 = dict(sin, pixels=sin["pixels"][:1])
        t1 = time.perf_counter()
        x1 = ostem.patch_embed(sin1, stem1)
        if kind == "hiera":
            ost.stack_forward(x1, blocks, one, levels, taps)
        else:
            ost.tower_forward(x1, blocks, one, post_ln=post)
        tc = time.perf_counter() - t1
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        line["cpu_baseline"] = {"value": N0 / tc, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
                                "sample": "float64 numpy oracle, stem and blocks on one frame (%d tokens), %.1f s"
                                          % (N0, tc)}
    return line


def rowops_cold(steps):
    """HBM bandwidth of the memory-bound kernels on working sets larger than
    the 256 MB Infinity Cache: each launch reads and writes a different one of
    several buffer sets (about 0.7-0.8 GB in all), so every launch streams
    from HBM. Prints one JSON line per kernel: algorithmic bytes per launch,
    mean device time per launch (events around K back-to-back launches) and
    GB/s as a fraction of the HBM peak."""
    import torch
    from vision_transformer_encoder_vit_amd import binding as vb
    NB = 3

    def timed(fn):
        for i in range(2 * NB):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    def report(name, shape, nbytes, us):
        gbs = nbytes / us / 1e3
        print(json.dumps({"kernel": name, "shape": shape, "bytes_per_launch": nbytes, "us_per_launch": round(us, 2),
                          "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 3),
                          "working_set_MB": round(NB * nbytes / 1e6)}), flush=True)

    bf = torch.bfloat16
    rows, dim = 65536, 1024
    xs = [torch.randn(rows, dim, device="cuda").to(bf) for _ in range(NB)]
    ys = [torch.empty_like(xs[0]) for _ in range(NB)]
    g, b = torch.ones(dim, device="cuda"), torch.zeros(dim, device="cuda")
    report("layernorm", [rows, dim], 2 * rows * dim * 2,
           timed(lambda i: vb.vit_layernorm(xs[i % NB], ys[i % NB], g, b, 1e-6)))
    del xs, ys
    B, H, W, C = 32, 128, 128, 112
    xs = [torch.randn(B, H * W, C, device="cuda").to(bf) for _ in range(NB)]
    ys = [torch.empty_like(xs[0]) for _ in range(NB)]
    report("unroll (3 levels)", [B, H * W, C], 2 * B * H * W * C * 2,
           timed(lambda i: vb.vit_unroll(xs[i % NB], ys[i % NB], H, W, 3)))
    report("reroll (3 levels)", [B, H * W, C], 2 * B * H * W * C * 2,
           timed(lambda i: vb.vit_reroll(xs[i % NB], ys[i % NB], H, W, 3)))
    del xs, ys
    B, N, C = 16, 16384, 224
    xs = [torch.randn(B, N, C, device="cuda").to(bf) for _ in range(NB)]
    ys = [torch.empty(B, N // 4, C, device="cuda", dtype=bf) for _ in range(NB)]
    report("pool4", [B, N, C], 5 * B * (N // 4) * C * 2, timed(lambda i: vb.vit_pool4(xs[i % NB], ys[i % NB])))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default=DEFAULT_CONFIG, help="workload name, or 'all'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tower", choices=sorted(TOWERS),
                    help="time a whole tower from pixels (patch embed, then hiera: the 24-block stage stack at "
                         "512x512; sam3: ln_pre and the 32-layer trunk; siglip: the 12-layer tower and "
                         "post_layernorm) instead of one block")
    ap.add_argument("--weights", choices=["bf16", "q8_row"], default="bf16",
                    help="weight matrices in bf16, or as q8_row int8 payloads with float16 row scales")
    ap.add_argument("--qk-gain", type=float, default=1.0,
                    help="scale the query and key weights (block workloads): 16 gives the row maxima of "
                         "trained weights (scores of ~100-200), which take the running-maximum softmax")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="only time the float64 CPU oracle on C1-C3 (one thread and all threads)")
    ap.add_argument("--rowops", action="store_true",
                    help="only time LayerNorm, unroll, reroll and pool4 on HBM-resident working sets")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (vit_unroll with 0 levels), to scale "
                         "rocprofv3 FETCH_SIZE/WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only; --gpus %d is not supported (use --gpus 1)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("steps >= 1 and warmup >= 0")
    if args.oracle_timing:
        oracle_timing(["c1_tiny_f32", "c2_hiera_s0", "c3a_hiera_trans", "c3b_hiera_s2"])
        return
    if args.rowops:
        rowops_cold(args.steps)
        return
    if args.tower:
        print(json.dumps(run_tower(args.tower, args.steps, args.warmup, not args.no_cpu_baseline,
                                   q8=args.weights == "q8_row")), flush=True)
        return
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    from vision_transformer_encoder_vit_amd import synth
    names = list(synth.CONFIGS) if args.config == "all" else [args.config]
    for n in names:
        if n not in synth.CONFIGS:
            ap.error("unknown workload %s (choose from %s)" % (n, ", ".join(synth.CONFIGS)))
    for n in names:
        spec = synth.CONFIGS[n]
        if args.weights == "q8_row":
            spec = dict(spec, weights="q8_row")
        if args.qk_gain != 1.0:
            spec = dict(spec, qk_gain=args.qk_gain)
        with_cpu = not args.no_cpu_baseline and n == names[0] and args.weights == "bf16" and args.qk_gain == 1.0
        print(json.dumps(run(spec, args.steps, args.warmup, with_cpu)), flush=True)


if __name__ == "__main__":
    main()
