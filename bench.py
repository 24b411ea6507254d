"""Benchmark of the fused head-dim-64 attention library on one MI355X.

One JSON line on stdout.  A step is one call of the dense flash kernel on the
SDXL level-1 self-attention workload (bf16, B=2, H=10, S=4096, D=64); `value` is
its attention TFLOP/s (4*D flops per query-key pair, inputs already in HBM).  The
other forms of the hot path -- cross-attention against 77 keys, banded and full
differential attention -- are timed the same way and reported under "forms",
each against its own roofline (MFMA for the dense forms, HBM for the banded one).
Kernel time is measured with HIP events recorded on the stream the kernels run
on.  Every form is timed over rotated input copies (together past the 256 MB
last-level cache, so inputs come from HBM: "us", the reported figure) and hot
(one copy again and again: "us_hot").  The fp64 CPU oracle is timed on the same
dense workload for `cpu_baseline`.  `--trace-summary` turns a rocprofv3 kernel
trace of this command into per-kernel median, mean, min and max durations.
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

from head_attention_flash_amd import accounting as acc  # noqa: E402
from head_attention_flash_amd import synth  # noqa: E402

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def up(x, torch):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


PREWARM_S = 0.3  # untimed launches before the warmup steps, so the timed steps run at the sustained clock


def prewarm(fn, nsets, seconds, torch):
    """Launch fn back to back for `seconds` of wall time (untimed).  A fresh process starts the GPU at a
    low clock: without this the first few hundred launches of the dense kernel run ~18% slower."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(32):
            fn(i % nsets)
            i += 1
        torch.cuda.synchronize()


def time_launches(fn, nsets, steps, warmup, torch):
    """Average seconds per launch over `steps` launches, rotating over `nsets` input sets."""
    prewarm(fn, nsets, PREWARM_S, torch)
    for i in range(warmup):
        fn(i % nsets)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(i % nsets)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def time_graph_hot_and_rotated(fn, nsets, steps, warmup, torch):
    """(rotated, hot): seconds per launch over `nsets` rotated input copies (past the last-level cache),
    and over one copy launched again and again (served largely from the caches)."""
    rot = time_graph(fn, nsets, steps, warmup, torch)
    hot = time_graph(fn, 1, steps, warmup, torch) if nsets > 1 else rot
    return rot, hot


def time_graph(fn, nsets, steps, warmup, torch):
    """Like time_launches, with the `steps` launches captured once into a HIP graph and replayed,
    so that host-side call overhead does not hide kernels shorter than it.  The untimed warm-up
    replays the same graph for PREWARM_S of wall time: launches from Python cannot keep a kernel of
    a few tens of microseconds back to back, and at a partial duty cycle the clock stays low."""
    for i in range(warmup):
        fn(i % nsets)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                fn(i % nsets)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= PREWARM_S:
            break
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def copy_calibration(torch):
    """A plain device copy of known size (256 MiB read + 256 MiB written), launched once so a
    counter run of this command also measures what FETCH_SIZE/WRITE_SIZE read for known bytes."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: copy calibration {n} bytes")
    del src, dst


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it still matches the source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(kernel)
    if not ent or ent.get("source_digest") != source_digest(ent.get("sources", [])):
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(wl):
    """The fp64 oracle on the whole dense workload (every query row, all keys), in TFLOP/s."""
    import oracle
    q, k, v = synth.make_dense(wl)
    lib = oracle.load()
    qd, kd, vd = (oracle.widen(x) for x in (q, k, v))  # widening is marshalling, kept outside the timing
    t0 = time.perf_counter()
    oracle.attn(qd, kd, vd, wl.scale, lib=lib)
    dt = time.perf_counter() - t0
    flops = acc.attn_flops(wl.B, wl.H, wl.Sq, wl.Sk)
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole {wl.key} workload ({wl.B * wl.H * wl.Sq} query rows x {wl.Sk} keys), {dt:.2f} s"}


def host_cpu():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gcc_version():
    import subprocess
    try:
        r = subprocess.run(["gcc", "--version"], capture_output=True, text=True, timeout=10)
        return r.stdout.splitlines()[0].strip() if r.stdout else None
    except (OSError, subprocess.SubprocessError):
        return None


def run_env(torch):
    """What the numbers were measured on: device, CU count, ROCm and torch versions, host CPU, gcc
    (which builds the oracle), source revision."""
    env = {"device": torch.cuda.get_device_name(0),
           "cus": torch.cuda.get_device_properties(0).multi_processor_count,
           "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
           "host_cpu": host_cpu(), "host_threads": os.cpu_count(), "gcc": gcc_version()}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    try:
        import subprocess
        here = os.path.dirname(os.path.abspath(__file__))
        r = subprocess.run(["git", "-C", here, "rev-parse", "--short", "HEAD"], capture_output=True, text=True,
                           timeout=10)
        env["git"] = r.stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        env["git"] = None
    return env


# kernels whose HBM traffic profiles/traffic.json records, and the sources each is built from
KERNEL_SOURCES = {
    "attn_bf16_quad": ["head_attention_flash_amd/csrc/attn_dense.hip", "head_attention_flash_amd/csrc/ka_common.hpp"],
    "xattn_bf16": ["head_attention_flash_amd/csrc/attn_dense.hip", "head_attention_flash_amd/csrc/ka_common.hpp"],
    "diff_band": ["head_attention_flash_amd/csrc/diffattn.hip", "head_attention_flash_amd/csrc/ka_common.hpp"],
    "diff_kprep": ["head_attention_flash_amd/csrc/diffattn.hip", "head_attention_flash_amd/csrc/ka_common.hpp"],
    "diff_flash_duo": ["head_attention_flash_amd/csrc/diffattn.hip", "head_attention_flash_amd/csrc/ka_common.hpp"],
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def short_kernel(name):
    for k in list(KERNEL_SOURCES) + [COPY_KERNEL]:
        if k in name:
            return k
    return name


def counter_values(path):
    """{kernel: {counter: {dispatch id: value}}} from a rocprofv3 counter-collection CSV (a counter's
    values over the instances of one dispatch are summed)."""
    import csv
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = acc.setdefault(short_kernel(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return acc


def counter_means(path):
    """{kernel: {counter: mean value per dispatch}}, {kernel: dispatches}."""
    acc = counter_values(path)
    means = {k: {c: sum(v.values()) / len(v) for c, v in d.items()} for k, d in acc.items()}
    return means, {k: max(len(v) for v in d.values()) for k, d in acc.items()}


def traffic_summary(fetch_csv, write_csv):
    """HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, from two runs), each scaled by
    what the same counter reads for the plain 256 MiB device copy that --copy-calibration launches."""
    fetch, nf = counter_means(fetch_csv)
    write, nw = counter_means(write_csv)
    copy_bytes = 256 << 20
    # the calibration copy is the largest copy dispatch (input uploads run the same copy kernel)
    cf = max(counter_values(fetch_csv)[COPY_KERNEL]["FETCH_SIZE"].values())
    cw = max(counter_values(write_csv)[COPY_KERNEL]["WRITE_SIZE"].values())
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    out = {"copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_scale": fs, "write_scale": ws}
    for k, src in KERNEL_SOURCES.items():
        if k in fetch and k in write:
            fk, wk = fetch[k]["FETCH_SIZE"], write[k]["WRITE_SIZE"]
            out[k] = {"sources": src, "source_digest": source_digest(src), "dispatches": [nf[k], nw[k]],
                      "fetch_kib": fk, "write_kib": wk, "hbm_bytes_per_launch": int(round(fk * 1024 * fs + wk * 1024 * ws))}
    return out


def trace_summary(path):
    """Per-kernel count, median, mean, min and max duration (us) of a rocprofv3 kernel-trace CSV."""
    import csv
    import statistics
    by = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = []
    for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        rows.append({"kernel": name, "launches": len(d), "median_us": round(statistics.median(d), 3),
                     "mean_us": round(statistics.fmean(d), 3), "min_us": round(min(d), 3), "max_us": round(max(d), 3)})
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--forms", default="cross,cross_l1,cross_cond257,vae_mid,band,full,band_model,full_model,band_fused",
                    help="extra forms to time (comma list, or 'none')")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print per-kernel launch statistics (median, mean, min, max) of a rocprofv3 kernel "
                         "trace and exit (no GPU needed)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print HBM bytes per launch from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-calibration command, as JSON, and exit (no GPU needed)")
    ap.add_argument("--counter-summary", metavar="COUNTER_CSV",
                    help="print per-kernel mean counter values per dispatch of a rocprofv3 counter run and exit")
    args = ap.parse_args()
    if args.trace_summary:
        for r in trace_summary(args.trace_summary):
            print(json.dumps(r))
        return
    if args.traffic_summary:
        print(json.dumps(traffic_summary(*args.traffic_summary), indent=1))
        return
    if args.counter_summary:
        means, n = counter_means(args.counter_summary)
        for k, d in means.items():
            print(json.dumps({"kernel": k, "dispatches": n[k], **{c: round(v, 1) for c, v in sorted(d.items())}}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_attention_flash_amd as ka
    from head_attention_flash_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    ka.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(torch)

    # ---------------- headline: dense self-attention, SDXL level 1
    wl = synth.WORKLOADS["sdxl_l1_self_b2h10s4096"]
    log(f"bench: {wl.desc}")
    # 8 input copies (336 MB, past the last-level cache): every step reads its inputs from HBM
    dsets = [[up(x, torch) for x in synth.make_dense(wl, seed_base=1000 * wl.index + 10 * s_)] for s_ in range(8)]
    o = torch.empty_like(dsets[0][0])
    flops = acc.attn_flops(wl.B, wl.H, wl.Sq, wl.Sk)

    def step(i):
        ka.ka_attn_fwd(*dsets[i], o=o, scale=wl.scale)

    torch.cuda.synchronize()
    sec = time_launches(step, len(dsets), args.steps, args.warmup, torch)
    sec_hot = time_launches(step, 1, args.steps, args.warmup, torch)
    value = flops / sec / 1e12
    log(f"bench: dense {sec * 1e6:.1f} us/launch ({sec_hot * 1e6:.1f} hot), {value:.1f} TFLOP/s")
    traffic = traffic_for("attn_bf16_quad")
    result = {
        "metric": "attention TFLOP/s (% MFMA peak) dense; GB/s (% HBM peak) banded diff-attn",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1), no dataset)",
        "config": {"workload": wl.key, "form": "dense self-attention", "B": wl.B, "H": wl.H, "Sq": wl.Sq,
                   "Sk": wl.Sk, "D": 64, "scale": wl.scale},
        "roofline": {"bound": "mfma", "achieved": round(flops / sec / 1e12, 3),
                     "peak": acc.MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                     "frac": round(flops / sec / acc.MFMA_BF16_PEAK, 4), "traffic": traffic,
                     "kernel": "attn_bf16_quad", "flops_per_launch": flops, "us": round(sec * 1e6, 3),
                     "us_hot": round(sec_hot * 1e6, 3), "input_copies": len(dsets)},
    }
    del dsets, o

    forms = {}
    wanted = set() if args.forms == "none" else set(args.forms.split(","))

    def form(name, wl, kernel, fn, nsets, flops, nbytes, bound, **extra):
        """Time one form as a HIP-graph replay: over `nsets` rotated input copies (past the 256 MB
        last-level cache) and, when there are several, hot (one copy again and again)."""
        rot, hot = time_graph_hot_and_rotated(fn, nsets, args.steps, args.warmup, torch)
        r = {"workload": wl.key, "kernel": kernel, "us": round(rot * 1e6, 3), "us_hot": round(hot * 1e6, 3),
             "input_copies": nsets, "bound": bound}
        if flops:
            r.update({"TFLOP/s": round(flops / rot / 1e12, 3), "mfma_frac": round(flops / rot / acc.MFMA_BF16_PEAK, 4),
                      "flops": flops})
        if nbytes:
            r.update({"GB/s": round(nbytes / rot / 1e9, 1), "hbm_frac": round(nbytes / rot / acc.HBM_PEAK, 4),
                      "GB/s_hot": round(nbytes / hot / 1e9, 1), "bytes": nbytes})
        r.update(extra)
        forms[name] = r
        log(f"bench: {name} {r}")

    def copies(nbytes, lo=2, hi=64):
        return max(lo, min(hi, -(-600_000_000 // nbytes)))  # input copies: 600 MB, past the last-level cache

    # ---------------- cross-attention: 77 context tokens (SDXL levels 2 and 1), 257 conditioning tokens
    for name, key in (("cross", "sdxl_l2_cross_b2h20q1024k77"), ("cross_l1", "sdxl_l1_cross_b2h10q4096k77"),
                      ("cross_cond257", "sa3_dit_cross_h24q1422k257")):
        if name not in wanted:
            continue
        wl = synth.WORKLOADS[key]
        log(f"bench: {wl.desc}")
        f, b = acc.attn_flops(wl.B, wl.H, wl.Sq, wl.Sk), acc.dense_bytes(wl.B, wl.H, wl.Sq, wl.Sk)
        n = copies(b)
        sets = [[up(x, torch) for x in synth.make_dense(wl, seed_base=1000 * wl.index + 10 * s_)] for s_ in range(n)]
        outs = [torch.empty_like(s_[0]) for s_ in sets]
        kern = "xattn_bf16 (keys in LDS, one pass)" if wl.Sk <= 128 else "xattn_bf16 (keys in LDS, 64-key chunks)"
        form(name, wl, kern, lambda i: ka.ka_xattn_fwd(*sets[i], o=outs[i], scale=wl.scale), n, f, b,
             "hbm" if f / b < acc.MFMA_BF16_PEAK / acc.HBM_PEAK else "mfma",
             **({"traffic": traffic_for("xattn_bf16")} if name == "cross" else {}))
        del sets, outs
    # ---------------- head dim 512: the SDXL VAE's single-head mid-block attention
    if "vae_mid" in wanted:
        wl = synth.WORKLOADS["sdxl_vae_mid_b1h1s16384d512"]
        log(f"bench: {wl.desc}")
        q5, k5, v5 = (up(x, torch) for x in synth.make_dense(wl))
        o5 = torch.empty_like(q5)
        f = acc.attn_flops(wl.B, wl.H, wl.Sq, wl.Sk, D=wl.D)
        sec = time_launches(lambda i: ka.ka_attn_fwd(q5, k5, v5, o=o5, scale=wl.scale), 1, max(5, args.steps // 5),
                            args.warmup, torch)
        forms["vae_mid"] = {"workload": wl.key, "kernel": "attn512_pair", "us": round(sec * 1e6, 3),
                            "TFLOP/s": round(f / sec / 1e12, 3), "mfma_frac": round(f / sec / acc.MFMA_BF16_PEAK, 4),
                            "bound": "mfma", "flops": f}
        log(f"bench: vae_mid {forms['vae_mid']}")
        del q5, k5, v5, o5

    def diff_sets(wl, n):
        out = []
        for s_ in range(n):
            ins, prm = synth.make_diff(wl, seed_base=1000 * wl.index + 10 * s_)
            out.append(([up(x, torch) for x in ins], [up(x, torch) for x in prm]))
        return out

    # ---------------- banded differential attention (HBM-bound: 3 copies = 425 MB > 256 MB cache)
    if "band" in wanted or "band_model" in wanted:
        wl = synth.WORKLOADS["sa3_decoder_banddiff_h8s23086w17"]
        log(f"bench: {wl.desc}")
        sets = diff_sets(wl, 3)
        outs = [torch.empty_like(s_[0][0]) for s_ in sets]
        f, b = acc.diff_flops(wl.B, wl.H, wl.Sq, wl.window), acc.diff_bytes(wl.B, wl.H, wl.Sq)
        if "band" in wanted:
            def band(i):
                ins, (a_, g_, b_, l_) = sets[i]
                ka.ka_diffattn_fwd(*ins, a_, g_, b_, l_, o=outs[i], scale=wl.scale, window=wl.window)
            form("band_diff", wl, "diff_band", band, len(sets), f, b, "hbm", traffic=traffic_for("diff_band"))
        if "band_model" in wanted:
            def band_model(i):
                ins, (a_, g_, b_, l_) = sets[i]
                ka.ka_diffattn_fwd_ex(*ins, l_, o=outs[i], scale=wl.scale, window=wl.window, qk_norm="dyt", alpha=a_,
                                      gamma=g_, beta=b_, rotary_dims=32)
            form("band_diff_model", wl, "diff_band", band_model, len(sets), f, b, "hbm",
                 options="DyT, rotary on 32 of 64 dims")
        del sets, outs
    if "band_fused" in wanted:
        # the decoder form reading q1, k1, v, q2, k2 straight out of one [B, S, 5, H, 64] projection and
        # writing the merged [B, S, H, 64] output (strided views, no transposes)
        wl = synth.WORKLOADS["sa3_decoder_banddiff_h8s23086w17"]
        log(f"bench: {wl.desc}, decoder form on a fused projection")
        sets = []
        for s_ in range(3):
            ins, prm = synth.make_diff(wl, seed_base=1000 * wl.index + 10 * s_)
            t = [up(x, torch) for x in ins]  # q1, k1, q2, k2, v
            X = torch.stack([x.permute(0, 2, 1, 3) for x in (t[0], t[1], t[4], t[2], t[3])], dim=2).contiguous()
            del t
            views = [X[:, :, i].permute(0, 2, 1, 3) for i in (0, 1, 3, 4, 2)]
            out = torch.empty(wl.B, wl.Sq, wl.H, 64, dtype=torch.bfloat16, device="cuda")
            sets.append((X, views, out, [up(x, torch) for x in prm]))
        f, b = acc.diff_flops(wl.B, wl.H, wl.Sq, wl.window), acc.diff_bytes(wl.B, wl.H, wl.Sq)

        def band_fused(i):
            _, views, out, (a_, g_, b_, l_) = sets[i]
            ka.ka_diffattn_fwd_ex(*views, l_, o=out.permute(0, 2, 1, 3), scale=wl.scale, window=wl.window,
                                  qk_norm="dyt", alpha=a_, gamma=g_, beta=b_, rotary_dims=32)

        form("band_diff_fused", wl, "diff_band", band_fused, len(sets), f, b, "hbm",
             options="DyT, rotary on 32 of 64 dims, inputs read from a fused [B,S,5,H,64] projection, output "
                     "written [B,S,H,64]")
        del sets
    # ---------------- full differential attention (DiT-shaped): key prep, then the flash pass
    if "full" in wanted or "full_model" in wanted:
        wl = synth.WORKLOADS["sa3_dit_fulldiff_h16s1422"]
        log(f"bench: {wl.desc}")
        f, b = acc.diff_flops(wl.B, wl.H, wl.Sq, wl.window), acc.diff_bytes(wl.B, wl.H, wl.Sq)
        n = copies(b + ka.ka_diffattn_workspace_bytes(wl.B, wl.H, wl.Sq, 64, wl.window), hi=32)
        sets = diff_sets(wl, n)
        outs = [torch.empty_like(s_[0][0]) for s_ in sets]
        wss = [torch.empty(ka.ka_diffattn_workspace_bytes(wl.B, wl.H, wl.Sq, 64, wl.window), dtype=torch.uint8,
                           device="cuda") for _ in sets]
        if "full" in wanted:
            def full(i):
                ins, (a_, g_, b_, l_) = sets[i]
                ka.ka_diffattn_fwd(*ins, a_, g_, b_, l_, o=outs[i], scale=wl.scale, window=wl.window, workspace=wss[i])
            t1, t2 = traffic_for("diff_kprep"), traffic_for("diff_flash_duo")
            form("full_diff", wl, "diff_kprep + diff_flash_duo", full, len(sets), f, b, "mfma",
                 traffic=(t1 + t2) if t1 is not None and t2 is not None else None)
        if "full_model" in wanted:
            pad = 142
            w_, lm_ = (up(x, torch) for x in synth.make_model_params(wl.H, 1000 * wl.index + 6))
            keep = up(synth.make_v_keep(wl.B, wl.Sq, pad), torch)

            def full_model(i):
                ins = sets[i][0]
                ka.ka_diffattn_fwd_ex(*ins, lm_, o=outs[i], scale=wl.scale, window=wl.window, qk_norm="rms",
                                      rms_weight=w_, rms_eps=1e-6, rotary_dims=32, v_keep=keep, workspace=wss[i])
            form("full_diff_model", wl, "diff_kprep + diff_flash_duo", full_model, len(sets), f, b, "mfma",
                 options=f"RMSNorm, rotary on 32 of 64 dims, {pad} padded")
        del sets, outs, wss
    if forms:
        result["forms"] = forms

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth.WORKLOADS["sdxl_l1_self_b2h10s4096"])
    result["env"] = run_env(torch)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
