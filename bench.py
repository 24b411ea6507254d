"""Benchmark of the fused head-dim-64 attention library on one MI355X.

One JSON line on stdout.  A step is one call of the dense flash kernel on the
SDXL level-1 self-attention workload (bf16, B=2, H=10, S=4096, D=64); `value` is
its attention TFLOP/s (4*D flops per query-key pair, inputs already in HBM).  The
other forms of the hot path -- cross-attention against 77 keys, banded and full
differential attention -- are timed the same way and reported under "forms",
each against its own roofline (MFMA for the dense forms, HBM for the banded one).
Kernel time is measured with HIP events recorded on the stream the kernels run
on.  HBM-bound forms rotate several input copies so that the 256 MB last-level
cache does not serve them.  The fp64 CPU oracle is timed on a bounded sample of
the same workload for `cpu_baseline`.
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


def traffic_for(kernel, launch_units):
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


def run_env(torch):
    """What the numbers were measured on: device, CU count, ROCm and torch versions, source revision."""
    env = {"device": torch.cuda.get_device_name(0),
           "cus": torch.cuda.get_device_properties(0).multi_processor_count,
           "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
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
    args = ap.parse_args()
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
    q, k, v = (up(x, torch) for x in synth.make_dense(wl))
    o = torch.empty_like(q)
    flops = acc.attn_flops(wl.B, wl.H, wl.Sq, wl.Sk)

    def step(_):
        ka.ka_attn_fwd(q, k, v, o=o, scale=wl.scale)

    torch.cuda.synchronize()
    sec = time_launches(step, 1, args.steps, args.warmup, torch)
    value = flops / sec / 1e12
    log(f"bench: dense {sec * 1e6:.1f} us/launch, {value:.1f} TFLOP/s")
    traffic = traffic_for("attn_bf16_quad", 1)
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
                     "kernel": "attn_bf16_quad", "flops_per_launch": flops},
    }
    del q, k, v, o

    forms = {}
    wanted = set() if args.forms == "none" else set(args.forms.split(","))
    # ---------------- cross-attention against 77 keys (HBM-bound: rotate 8 input copies)
    if "cross" in wanted:
        wl = synth.WORKLOADS["sdxl_l2_cross_b2h20q1024k77"]
        log(f"bench: {wl.desc}")
        sets = [[up(x, torch) for x in synth.make_dense(wl, seed_base=1000 * wl.index + 10 * s)] for s in range(8)]
        outs = [torch.empty_like(s[0]) for s in sets]
        f, b = acc.attn_flops(wl.B, wl.H, wl.Sq, wl.Sk), acc.dense_bytes(wl.B, wl.H, wl.Sq, wl.Sk)
        sec = time_graph(lambda i: ka.ka_xattn_fwd(*sets[i], o=outs[i], scale=wl.scale), len(sets), args.steps,
                         args.warmup, torch)
        forms["cross"] = {"workload": wl.key, "kernel": "xattn_bf16", "us": round(sec * 1e6, 3),
                          "TFLOP/s": round(f / sec / 1e12, 3), "mfma_frac": round(f / sec / acc.MFMA_BF16_PEAK, 4),
                          "GB/s": round(b / sec / 1e9, 1), "hbm_frac": round(b / sec / acc.HBM_PEAK, 4),
                          "bound": "hbm", "flops": f, "bytes": b, "input_copies": len(sets)}
        log(f"bench: cross {forms['cross']}")
        del sets, outs
    # ---------------- more conditioning shapes: SDXL level-1 cross (77 keys), the DiT's 257 tokens (streamed)
    for name, key, kern in (("cross_l1", "sdxl_l1_cross_b2h10q4096k77", "xattn_bf16"),
                            ("cross_cond257", "sa3_dit_cross_h24q1422k257", "attn_bf16 (keys streamed)")):
        if name not in wanted:
            continue
        wl = synth.WORKLOADS[key]
        log(f"bench: {wl.desc}")
        f, b = acc.attn_flops(wl.B, wl.H, wl.Sq, wl.Sk), acc.dense_bytes(wl.B, wl.H, wl.Sq, wl.Sk)
        n = max(2, min(64, -(-600_000_000 // b)))  # input copies: 600 MB, past the 256 MB last-level cache
        sets = [[up(x, torch) for x in synth.make_dense(wl, seed_base=1000 * wl.index + 10 * s)] for s in range(n)]
        outs = [torch.empty_like(s[0]) for s in sets]
        sec = time_graph(lambda i: ka.ka_xattn_fwd(*sets[i], o=outs[i], scale=wl.scale), len(sets), args.steps,
                         args.warmup, torch)
        forms[name] = {"workload": wl.key, "kernel": kern, "us": round(sec * 1e6, 3),
                       "TFLOP/s": round(f / sec / 1e12, 3), "mfma_frac": round(f / sec / acc.MFMA_BF16_PEAK, 4),
                       "GB/s": round(b / sec / 1e9, 1), "hbm_frac": round(b / sec / acc.HBM_PEAK, 4),
                       "bound": "hbm" if f / b < acc.MFMA_BF16_PEAK / acc.HBM_PEAK else "mfma", "flops": f, "bytes": b,
                       "input_copies": len(sets)}
        log(f"bench: {name} {forms[name]}")
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
        forms["vae_mid"] = {"workload": wl.key, "kernel": "attn512_bf16", "us": round(sec * 1e6, 3),
                            "TFLOP/s": round(f / sec / 1e12, 3), "mfma_frac": round(f / sec / acc.MFMA_BF16_PEAK, 4),
                            "bound": "mfma", "flops": f}
        log(f"bench: vae_mid {forms['vae_mid']}")
        del q5, k5, v5, o5
    # ---------------- banded differential attention (HBM-bound: 3 copies = 425 MB > 256 MB cache)
    if "band" in wanted:
        wl = synth.WORKLOADS["sa3_decoder_banddiff_h8s23086w17"]
        log(f"bench: {wl.desc}")
        sets = []
        for s in range(3):
            ins, prm = synth.make_diff(wl, seed_base=1000 * wl.index + 10 * s)
            sets.append(([up(x, torch) for x in ins], [up(x, torch) for x in prm]))
        outs = [torch.empty_like(s[0][0]) for s in sets]
        f, b = acc.diff_flops(wl.B, wl.H, wl.Sq, wl.window), acc.diff_bytes(wl.B, wl.H, wl.Sq)

        def band(i):
            ins, (a_, g_, b_, l_) = sets[i]
            ka.ka_diffattn_fwd(*ins, a_, g_, b_, l_, o=outs[i], scale=wl.scale, window=wl.window)

        sec = time_graph(band, len(sets), args.steps, args.warmup, torch)
        forms["band_diff"] = {"workload": wl.key, "kernel": "diff_band", "us": round(sec * 1e6, 3),
                              "GB/s": round(b / sec / 1e9, 1), "hbm_frac": round(b / sec / acc.HBM_PEAK, 4),
                              "TFLOP/s": round(f / sec / 1e12, 3), "bound": "hbm", "flops": f, "bytes": b,
                              "input_copies": len(sets), "traffic": traffic_for("diff_band", 1)}
        log(f"bench: band {forms['band_diff']}")
        del sets, outs
    # ---------------- full differential attention (DiT-shaped)
    if "full" in wanted:
        wl = synth.WORKLOADS["sa3_dit_fulldiff_h16s1422"]
        log(f"bench: {wl.desc}")
        ins, prm = synth.make_diff(wl)
        ins = [up(x, torch) for x in ins]
        a_, g_, b_, l_ = (up(x, torch) for x in prm)
        o = torch.empty_like(ins[0])
        ws = torch.empty(ka.ka_diffattn_workspace_bytes(wl.B, wl.H, wl.Sq, 64, wl.window), dtype=torch.uint8,
                         device="cuda")
        f, b = acc.diff_flops(wl.B, wl.H, wl.Sq, wl.window), acc.diff_bytes(wl.B, wl.H, wl.Sq)
        sec = time_graph(lambda i: ka.ka_diffattn_fwd(*ins, a_, g_, b_, l_, o=o, scale=wl.scale,
                                                      window=wl.window, workspace=ws),
                         1, args.steps, args.warmup, torch)
        forms["full_diff"] = {"workload": wl.key, "kernel": "diff_kprep + diff_flash_split", "us": round(sec * 1e6, 3),
                              "TFLOP/s": round(f / sec / 1e12, 3), "mfma_frac": round(f / sec / acc.MFMA_BF16_PEAK, 4),
                              "GB/s": round(b / sec / 1e9, 1), "bound": "mfma", "flops": f, "bytes": b}
        log(f"bench: full {forms['full_diff']}")
    # ---------------- the model forms: decoder (DyT, 32 rotary dims), DiT (RMSNorm, 32 rotary dims, padded V)
    if "band_model" in wanted:
        wl = synth.WORKLOADS["sa3_decoder_banddiff_h8s23086w17"]
        log(f"bench: {wl.desc}, decoder form (DyT, 32 rotary dims)")
        sets = []
        for s_ in range(3):
            ins, prm = synth.make_diff(wl, seed_base=1000 * wl.index + 10 * s_)
            sets.append(([up(x, torch) for x in ins], [up(x, torch) for x in prm]))
        outs = [torch.empty_like(s_[0][0]) for s_ in sets]
        f, b = acc.diff_flops(wl.B, wl.H, wl.Sq, wl.window), acc.diff_bytes(wl.B, wl.H, wl.Sq)

        def band_model(i):
            ins, (a_, g_, b_, l_) = sets[i]
            ka.ka_diffattn_fwd_ex(*ins, l_, o=outs[i], scale=wl.scale, window=wl.window, qk_norm="dyt", alpha=a_,
                                  gamma=g_, beta=b_, rotary_dims=32)

        sec = time_graph(band_model, len(sets), args.steps, args.warmup, torch)
        forms["band_diff_model"] = {"workload": wl.key, "options": "DyT, rotary on 32 of 64 dims",
                                    "kernel": "diff_band", "us": round(sec * 1e6, 3), "GB/s": round(b / sec / 1e9, 1),
                                    "hbm_frac": round(b / sec / acc.HBM_PEAK, 4), "bound": "hbm", "bytes": b,
                                    "input_copies": len(sets)}
        log(f"bench: band model form {forms['band_diff_model']}")
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

        sec = time_graph(band_fused, len(sets), args.steps, args.warmup, torch)
        forms["band_diff_fused"] = {"workload": wl.key, "options": "DyT, rotary on 32 of 64 dims, inputs read from "
                                    "a fused [B,S,5,H,64] projection, output written [B,S,H,64]",
                                    "kernel": "diff_band", "us": round(sec * 1e6, 3), "GB/s": round(b / sec / 1e9, 1),
                                    "hbm_frac": round(b / sec / acc.HBM_PEAK, 4), "bound": "hbm", "bytes": b,
                                    "input_copies": len(sets)}
        log(f"bench: band fused {forms['band_diff_fused']}")
        del sets
    if "full_model" in wanted:
        wl = synth.WORKLOADS["sa3_dit_fulldiff_h16s1422"]
        pad = 142
        log(f"bench: {wl.desc}, DiT form (RMSNorm, 32 rotary dims, last {pad} tokens padded)")
        ins, _ = synth.make_diff(wl)
        ins = [up(x, torch) for x in ins]
        w_, l_ = (up(x, torch) for x in synth.make_model_params(wl.H, 1000 * wl.index + 6))
        keep = up(synth.make_v_keep(wl.B, wl.Sq, pad), torch)
        o = torch.empty_like(ins[0])
        ws = torch.empty(ka.ka_diffattn_workspace_bytes(wl.B, wl.H, wl.Sq, 64, wl.window), dtype=torch.uint8,
                         device="cuda")
        f, b = acc.diff_flops(wl.B, wl.H, wl.Sq, wl.window), acc.diff_bytes(wl.B, wl.H, wl.Sq)
        sec = time_graph(lambda i: ka.ka_diffattn_fwd_ex(*ins, l_, o=o, scale=wl.scale, window=wl.window,
                                                         qk_norm="rms", rms_weight=w_, rms_eps=1e-6, rotary_dims=32,
                                                         v_keep=keep, workspace=ws),
                         1, args.steps, args.warmup, torch)
        forms["full_diff_model"] = {"workload": wl.key, "options": f"RMSNorm, rotary on 32 of 64 dims, {pad} padded",
                                    "kernel": "diff_kprep + diff_flash_split", "us": round(sec * 1e6, 3),
                                    "TFLOP/s": round(f / sec / 1e12, 3),
                                    "mfma_frac": round(f / sec / acc.MFMA_BF16_PEAK, 4), "bound": "mfma", "flops": f}
        log(f"bench: full model form {forms['full_diff_model']}")
    if forms:
        result["forms"] = forms

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth.WORKLOADS["sdxl_l1_self_b2h10s4096"])
    result["env"] = run_env(torch)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
