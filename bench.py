"""Benchmark of prefix-reuse block-causal attention on one MI355X.

One step = one denoising step of the DiT's attention: qi_denoise_attn_step on each of
the 32 layers, every layer with its own prefix cache and its own Q/K/V/O buffers (so
the timed work is not served from a warm cache of one layer's data).  Inputs are resident
in HBM before timing starts; the prefix caches are built (step 0) before the timed region
and the build itself is timed separately.

Prints ONE JSON line.  `value` is useful attention TFLOP/s (4*D*H*allowed pairs; masked
pairs are not counted) on the 1024x1024 text-to-image workload (24 heads x 128, text 256
+ image 4096 tokens); the 2048x2048 edit and the others are reported under "extra".

The default run also times the 2048x2048 edit (the metric's second configuration), the
four-reference edit cached vs full recompute, and the eight-request fp8 wave (its HBM
rate over the compulsory bytes); they are summarised under "north_star".

    python bench.py [--steps K] [--warmup W] [--workload t2i1024] [--kv fp8] [--extra]
                    [--no-extra] [--profile-run] [--no-cpu]
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

METRIC = "block-causal attn TFLOP/s & % MFMA peak per denoise step (1024^2, 2048^2)"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published (no sparsity)
KERNEL_SRC = os.path.join(ROOT, "block_causal_attention_qi_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_denoise_t2i1024_traffic.json")
# (heads, share of the image rows) on which the oracle is timed for the other measured
# configurations: a few seconds of host work each
ORACLE_SAMPLES = {"edit2048": (1, 0.25), "edit4": (2, 1.0), "wave8": (1, 0.25)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


class Layers:
    """Per-layer device buffers of one workload: layer l holds the base inputs rolled by
    97*l tokens (same distribution, different bytes)."""

    def __init__(self, name, layers, dev, need_full=False, kv=None, x=None):
        import dataclasses
        import torch
        from block_causal_attention_qi_amd import qi, synth
        self.w = synth.workload(name)
        if kv is not None:
            self.w = dataclasses.replace(self.w, kv_dtype=kv)
        w = self.w
        if x is None:
            t0 = time.time()
            x = synth.generate(w, steps=1)
            log("[bench] %s: inputs drawn in %.1fs" % (name, time.time() - t0))
        b = lambda a: synth.to_bf16(a, dev)
        base = dict(q_pre=b(x.q_pre), k_pre=b(x.k_pre), v_pre=b(x.v_pre), q_img=b(x.q_img[0]),
                    k_img=b(x.k_img[0]), v_img=b(x.v_img[0]))
        if need_full:
            base.update(zip(("q_all", "k_all", "v_all"), (b(t) for t in x.full(0))))
        del x
        self.plan = qi.Plan(w.requests, w.n_heads, w.head_dim, w.kv_dtype)
        self.ws = torch.empty(max(256, self.plan.workspace_bytes), dtype=torch.uint8, device=dev)
        qi.qi_plan_upload(self.plan, self.ws)
        self.layers = []
        for l in range(layers):
            sh = 97 * l
            t = {k: torch.roll(v, shifts=sh, dims=0).contiguous() for k, v in base.items()}
            t["cache"] = torch.empty(self.plan.cache_bytes, dtype=torch.uint8, device=dev)
            t["o_pre"] = torch.empty_like(t["q_pre"])
            t["o_img"] = torch.empty_like(t["q_img"])
            if need_full:
                t["o_all"] = torch.empty_like(t["q_all"])
            self.layers.append(t)
        del base
        torch.cuda.synchronize()

    def build(self):
        from block_causal_attention_qi_amd import qi
        for t in self.layers:
            qi.qi_prefix_kv_build(self.plan, t["q_pre"], t["k_pre"], t["v_pre"], t["o_pre"],
                                  t["cache"])

    def denoise(self):
        from block_causal_attention_qi_amd import qi
        for t in self.layers:
            qi.qi_denoise_attn_step(self.plan, t["cache"], t["q_img"], t["k_img"], t["v_img"],
                                    t["o_img"])

    def full(self):
        from block_causal_attention_qi_amd import qi
        for t in self.layers:
            qi.qi_attn_full_reference_step(self.plan, t["q_all"], t["k_all"], t["v_all"],
                                           t["o_all"])


def timed(fn, steps, warmup, per_step=None):
    """Warm up, then time exactly `steps` calls of fn with HIP events on the current
    stream (the stream libqi launches on), synchronising on both sides.  Returns the total
    ms; with a list `per_step`, also appends each call's ms (an event after every call)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    if per_step is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[steps])   # ms


def capture(fn):
    """fn captured into a HIP graph on a side stream (torch's capture recipe: one warm-up
    run on the side stream first)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def current_sclk_mhz(text):
    """The current level of a pp_dpm_sclk listing (the line marked '*', e.g. "1: 2152Mhz *"),
    in MHz, or None."""
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            try:
                return int(line.split(":", 1)[1].strip().split("M")[0])
            except (ValueError, IndexError):
                return None
    return None


def sample_clock(fn, seconds=2.0, period=0.02):
    """The shader clock while fn runs back to back for `seconds`: the current level of the
    card's pp_dpm_sclk (sysfs; the line marked '*'), read on a host thread every `period`
    seconds.  None when sysfs does not show exactly one card."""
    import glob
    import statistics
    import threading
    import torch
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if len(paths) != 1:
        return None
    vals, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                with open(paths[0]) as f:
                    v = current_sclk_mhz(f.read())
                if v is not None:
                    vals.append(v)
            except OSError:
                pass
            stop.wait(period)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not vals:
        return None
    return {"sclk_mhz_median": statistics.median(vals), "sclk_mhz_min": min(vals),
            "sclk_mhz_max": max(vals), "samples": len(vals), "source": paths[0],
            "note": "sampled while the timed step ran back to back for %.0f s after the "
                    "timed region" % seconds}


def kernel_label(head_dim, kv):
    """Name of the attention kernel instance a denoising call runs."""
    return "attn_pp_kernel<%d, %s cache>" % (head_dim, kv)


def compulsory_bytes(plan, w):
    """Algorithmic bytes of one denoising launch: image Q, K, V read and O written (bf16),
    plus the prefix cache read once (bf16: 2 bytes per K and V element; fp8: 1; fp8_v: 2
    for K, 1 for V) and the fp8 scales."""
    from block_causal_attention_qi_amd import qi
    pre, img, _ = qi.qi_plan_tokens(plan)
    hd = w.n_heads * w.head_dim
    per_tok = {"bf16": 4, "fp8": 2, "fp8_v": 3}[w.kv_dtype]
    scales = 0 if w.kv_dtype == "bf16" else 8 * w.n_heads * len(w.requests)
    return 4 * img * hd * 2 + per_tok * pre * hd + scales


def measure(name, steps, warmup, layers, dev, with_full=False, with_build=True,
            with_graph=False, kv=None, with_clock=False, oracle_sample=None):
    """Time the denoising step of workload `name` (and optionally its build, graph replay,
    full recompute and clock).  oracle_sample = (heads, row fraction): also time the fp64
    oracle on that sample of the same inputs on the host, before the GPU work."""
    from block_causal_attention_qi_amd import qi, synth
    t0 = time.time()
    x = synth.generate(synth.workload(name), steps=1)
    log("[bench] %s: inputs drawn in %.1fs" % (name, time.time() - t0))
    cpu = oracle_time(name, x, *oracle_sample) if oracle_sample else None
    L = Layers(name, layers, dev, need_full=with_full, kv=kv, x=x)
    del x
    flops = qi.useful_flops(L.plan, qi.QI_CALL_DENOISE)
    items = qi.qi_plan_launch_items(L.plan, qi.QI_CALL_DENOISE)
    live = items[items[:, 0] >= 0]
    res = {"workload": name, "requests": L.w.requests, "heads": L.w.n_heads,
           "head_dim": L.w.head_dim, "kv_cache": L.w.kv_dtype, "layers": layers,
           "kernel": kernel_label(L.w.head_dim, L.w.kv_dtype),
           "denoise_gflop_per_layer": flops / 1e9,
           "denoise_workgroups": int(len(live)),
           "key_chunks": bool((live[:, 4] > 0).any())}
    if cpu:
        res["oracle_cpu"] = dict(cpu, tflops=flops / cpu["seconds_per_layer_step"] / 1e12)
    L.build()   # step 0 of every layer (untimed here: the caches must exist)
    each = []
    ms = timed(L.denoise, steps, warmup, each)
    per_launch = ms / (steps * layers)
    import statistics
    res["step_ms"] = {"median": statistics.median(each), "min": min(each), "max": max(each),
                      "steps": len(each)}
    res.update(ms_per_step=ms / steps, ms_per_layer_step=per_launch,
               tflops=flops / (per_launch * 1e-3) / 1e12)
    res["frac_of_peak"] = res["tflops"] / PEAK_BF16_TFLOPS
    if with_clock:
        res["clock"] = sample_clock(L.denoise)
    if with_graph:
        # the whole step (one launch per layer) replayed from a HIP graph: the share of
        # the eager step that is launch overhead
        g = capture(L.denoise)
        gms = timed(g.replay, steps, warmup)
        res.update(graph_ms_per_step=gms / steps,
                   graph_tflops=flops * layers / (gms / steps * 1e-3) / 1e12,
                   launch_overhead_share=max(0.0, 1.0 - gms / ms))
        del g
    if with_build:
        bflops = qi.useful_flops(L.plan, qi.QI_CALL_PREFIX)
        bms = timed(L.build, max(1, steps // 2), 1) / (max(1, steps // 2) * layers)
        res.update(build_ms_per_layer=bms, build_prefix_tflops=bflops / (bms * 1e-3) / 1e12)
    if with_full:
        fflops = qi.useful_flops(L.plan, qi.QI_CALL_FULL)
        fms = timed(L.full, max(1, steps // 2), 1) / (max(1, steps // 2) * layers)
        res.update(full_ms_per_layer=fms, full_tflops=fflops / (fms * 1e-3) / 1e12,
                   cached_speedup_vs_full=fms / per_launch)
    byts = compulsory_bytes(L.plan, L.w)
    res["compulsory_bytes_per_launch"] = byts
    res["compulsory_gb_per_s"] = byts / (per_launch * 1e-3) / 1e9
    del L
    import torch
    torch.cuda.empty_cache()
    return res


def host_info():
    """The host the oracle runs on: logical CPUs, the BLAS library NumPy calls and its
    thread count, and the thread variables of the environment."""
    info = {"os_cpu_count": os.cpu_count(),
            "env": {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                   "MKL_NUM_THREADS")}}
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = {"library": blas[0].get("internal_api"),
                            "version": blas[0].get("version"),
                            "threads": blas[0].get("num_threads"),
                            "file": os.path.basename(blas[0].get("filepath") or "")}
    except Exception:   # threadpoolctl missing: the BLAS stays unnamed
        pass
    return info


def oracle_time(name, x, heads=None, row_frac=1.0, min_seconds=0.0, max_reps=1):
    import numpy as np
    """Seconds of the fp64 oracle (oracle/attention.py, untuned) for one layer-step of the
    cached denoising call of workload `name` with inputs x: every request, on the first
    `heads` heads (all by default) and the first row_frac of each request's image rows,
    scaled by H / heads / row_frac (the oracle computes every row and head on its own, so
    its time is linear in both).  Repeated until min_seconds have passed or max_reps runs
    were made."""
    from block_causal_attention_qi_amd import synth
    from oracle import attention as A
    w = synth.workload(name)
    nh = w.n_heads if heads is None else min(heads, w.n_heads)
    e = lambda a: synth.bf16_exact(a[:, :nh])
    args, rows = [], 0
    po = io = 0
    for bl in w.requests:
        lp, ni = sum(bl[:-1]), bl[-1]
        nr = max(1, int(round(ni * row_frac)))
        rows += nr
        args.append((bl, e(x.q_img[0][io:io + nr]), e(x.k_pre[po:po + lp]),
                     e(x.v_pre[po:po + lp]), e(x.k_img[0][io:io + ni]),
                     e(x.v_img[0][io:io + ni])))
        po += lp
        io += ni
    reps, t0 = 0, time.perf_counter()
    while reps < 1 or (time.perf_counter() - t0 < min_seconds and reps < max_reps):
        for bl, q, kp, vp, ki, vi in args:
            lp = sum(bl[:-1])
            # the image rows kept: the first q.shape[0] of the block, over every key
            mask = A.allowed_mask(bl, rows=range(lp, lp + q.shape[0]))
            A.masked_attention(q, np.concatenate([kp, ki]), np.concatenate([vp, vi]), mask)
        reps += 1
    elapsed = (time.perf_counter() - t0) / reps
    scale = (w.n_heads / nh) * (sum(w.image_lens) / rows)
    return {"seconds_per_layer_step": elapsed * scale, "measured_seconds": elapsed,
            "repetitions": reps,
            "sample": "heads 0..%d of %d and %d of %d image rows (the first of each request), "
                      "every key, float64 NumPy oracle; time scaled by %.3g to the whole "
                      "layer-step" % (nh - 1, w.n_heads, rows, sum(w.image_lens), scale)}


def cpu_baseline(name, others):
    """The oracle on the host cores: one whole layer-step of the main workload's denoising
    call (all heads, all image rows, repeated for about 10 s), plus the samples timed for
    the other configurations (others: workload -> the oracle_cpu record of its measure)."""
    from block_causal_attention_qi_amd import synth
    from oracle import layout as OL
    w = synth.workload(name)
    x = synth.generate(w, steps=1)
    rec = oracle_time(name, x, min_seconds=10.0, max_reps=8)
    del x
    dt = rec["seconds_per_layer_step"]
    flops = OL.useful_flops(w.requests, OL.CALL_DENOISE, w.n_heads, w.head_dim)
    host = host_info()
    threads = (host.get("blas") or {}).get("threads")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads or os.cpu_count(),
            "kind": "oracle", "seconds_per_layer_step": dt, "repetitions": rec["repetitions"],
            "sample": "one layer-step of the denoising call of %s (all %d heads, all %d image "
                      "rows), float64 NumPy oracle, repeated %d times; cores = threads of the "
                      "BLAS the oracle calls" % (name, w.n_heads, sum(w.image_lens),
                                                 rec["repetitions"]),
            "host": host, "other_configs": others}


def provenance():
    """Device, runtime and source identity of the run."""
    import glob
    import subprocess
    import torch
    rocm = None
    for f in ("/opt/rocm/.info/version",):
        try:
            with open(f) as fh:
                rocm = fh.read().strip()
        except OSError:
            pass
    try:
        git = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        git = None
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "block_causal_attention_qi_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    props = torch.cuda.get_device_properties(0)
    name = torch.cuda.get_device_name(0)
    if not name:   # some boxes report an empty name; the card's sysfs product name instead
        for f in sorted(glob.glob("/sys/class/drm/card*/device/product_name")):
            try:
                with open(f) as fh:
                    name = fh.read().strip()
            except OSError:
                continue
            if name:
                break
    return {"device": name or None,
            "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "rocm": rocm, "torch_hip": torch.version.hip, "torch": torch.__version__,
            "git_commit": git,   # null where the tree has no .git (copies on a GPU machine)
            "csrc_sha256": h.hexdigest()[:16]}


def copy_calibration(nbytes):
    """A plain device copy of a known size, for scaling the HBM byte counters
    (FETCH_SIZE / WRITE_SIZE) of a profiler run: reads nbytes, writes nbytes."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": a.numel() * 4, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--workload", default="t2i1024")
    ap.add_argument("--kv", choices=["bf16", "fp8", "fp8_v"], default=None,
                    help="prefix cache type of the main workload (default: the workload's own)")
    ap.add_argument("--extra", action="store_true",
                    help="also time true CFG (edit1 vs cfg_edit1) and edit10 (ten references: "
                         "cached vs full, and the fp8 / fp8_v caches)")
    ap.add_argument("--no-extra", action="store_true", help="time only the main workload")
    ap.add_argument("--profile-run", action="store_true",
                    help="only the main workload's timed denoising steps (no build timing, "
                         "graph replay or clock sampling), so that a profiler's average for "
                         "the denoising kernel covers exactly the launches the line reports")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (profiler byte-counter scale)")
    a = ap.parse_args()
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (heads or "
              "requests of a wave would shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    from block_causal_attention_qi_amd import qi  # noqa: F401  (fails loudly if not built)

    lean = a.profile_run
    main_res = measure(a.workload, a.steps, a.warmup, a.layers, dev, with_full=False,
                       with_build=not lean, with_graph=not lean, kv=a.kv, with_clock=not lean)
    log("[bench] %s" % json.dumps(main_res))
    extra = {}
    if not (a.no_extra or lean):
        # the second metric configuration, the cached-vs-full ratio on the four-reference
        # edit and the fp8 wave's HBM rate
        for n in ("edit2048", "edit4", "wave8"):
            if n == a.workload:
                continue
            sample = None if a.no_cpu else ORACLE_SAMPLES[n]
            extra[n] = measure(n, max(2, a.steps // 2), 1, a.layers, dev, with_full=(n == "edit4"),
                               oracle_sample=sample)
            log("[bench] %s" % json.dumps(extra[n]))
        # one GPU's head shard (3 of 24 heads) of the edit workloads: the plan splits
        # keys into chunks to fill the chip
        for n in ("edit4@h3", "edit2048@h3"):
            extra[n] = measure(n, max(2, a.steps // 2), 1, a.layers, dev, with_full=(n == "edit4@h3"))
            log("[bench] %s" % json.dumps(extra[n]))
        if a.extra:
            # true CFG: both branches in one wave against the positive branch alone
            for n in ("edit1", "cfg_edit1"):
                extra[n] = measure(n, max(2, a.steps // 2), 1, a.layers, dev, with_build=False)
                log("[bench] %s" % json.dumps(extra[n]))
            extra["cfg_edit1"]["step_time_over_single_branch"] = (
                extra["cfg_edit1"]["ms_per_step"] / extra["edit1"]["ms_per_step"])
            # ten references: ~2.4 GB of buffers per layer, so 8 layers
            for kv in ("bf16", "fp8", "fp8_v"):
                key = "edit10" if kv == "bf16" else "edit10_" + kv
                extra[key] = measure("edit10", 2, 1, min(a.layers, 8), dev,
                                     with_full=(kv == "bf16"), kv=kv)
                log("[bench] %s" % json.dumps(extra[key]))

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        if (rec.get("kernel_source_sha256") == kernel_sha() and rec.get("workload") == a.workload
                and rec.get("kv_cache") == main_res["kv_cache"]
                and rec.get("head_dim") == main_res["head_dim"]):
            traffic = rec["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    flops_launch = main_res["denoise_gflop_per_layer"] * 1e9
    achieved = main_res["tflops"]
    out = {
        "metric": METRIC,
        "value": round(achieved, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "step_ms": {k: (round(v, 4) if isinstance(v, float) else v)
                    for k, v in main_res["step_ms"].items()},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": a.workload, "blocks": main_res["requests"],
                   "heads": main_res["heads"], "head_dim": main_res["head_dim"],
                   "layers": a.layers, "kv_cache": main_res["kv_cache"],
                   "step": "qi_denoise_attn_step on each of %d layers" % a.layers},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": main_res["kernel"],
                     "flop_per_launch": flops_launch,
                     "ms_per_launch": round(main_res["ms_per_layer_step"], 5),
                     "algorithmic_bytes_per_launch": main_res["compulsory_bytes_per_launch"]},
        "extra": extra,
        "provenance": provenance(),
    }
    summary = {}
    if "edit2048" in extra:
        summary["edit2048_tflops"] = round(extra["edit2048"]["tflops"], 1)
        summary["edit2048_frac_of_peak"] = round(extra["edit2048"]["frac_of_peak"], 4)
    if "edit4" in extra:
        summary["edit4_cached_speedup_vs_full"] = round(extra["edit4"]["cached_speedup_vs_full"], 3)
    if "wave8" in extra:
        summary["wave8_fp8_compulsory_gb_per_s"] = round(extra["wave8"]["compulsory_gb_per_s"], 1)
        summary["wave8_fp8_tflops"] = round(extra["wave8"]["tflops"], 1)
    for n in ("edit4", "edit2048"):
        if n + "@h3" in extra and n in extra:
            summary[n + "_h3_tflops"] = round(extra[n + "@h3"]["tflops"], 1)
            summary[n + "_h3_over_h24"] = round(extra[n + "@h3"]["tflops"] / extra[n]["tflops"], 3)
    if summary:
        out["north_star"] = summary
    clk = main_res.get("clock")
    if clk:
        # the published peak scaled to the measured shader clock (it is quoted at 2400 MHz)
        clk["peak_tflops_at_clock"] = round(PEAK_BF16_TFLOPS * clk["sclk_mhz_median"] / 2400.0, 1)
        clk["frac_at_clock"] = round(achieved / clk["peak_tflops_at_clock"], 4)
    out["clock"] = clk
    if "graph_ms_per_step" in main_res:
        out["extra"]["graph_replay"] = {
            "workload": a.workload, "ms_per_step": round(main_res["graph_ms_per_step"], 4),
            "tflops": round(main_res["graph_tflops"], 3),
            "launch_overhead_share": round(main_res["launch_overhead_share"], 4),
            "note": "the same %d-layer step captured once in a HIP graph and replayed" % a.layers}
    if not a.no_cpu:
        others = {n: r["oracle_cpu"] for n, r in extra.items() if "oracle_cpu" in r}
        out["cpu_baseline"] = cpu_baseline(a.workload, others)
        if main_res["kv_cache"] != "bf16":
            out["cpu_baseline"]["sample"] += " (bf16 prefix values, not the %s cache)" % main_res["kv_cache"]
        log("[bench] cpu baseline %s" % json.dumps(out["cpu_baseline"]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
