"""Benchmark of the vision-to-language bridge on one MI355X.

One step = one vlb_bridge_fused call over one batch: LayerNorm (when the
workload has it), the k x k space-to-depth, Linear + bias + GELU, Linear +
bias, and the scatter of every row into its placeholder slot (plus newline /
separator rows for tiled images).  Inputs, the packed weights and the
workspace are resident in HBM before timing starts.

Every one of the five workloads is timed in the same run (`configs`); the
headline line is the largest one, ragged-3x3 (32 DeepSeek-ViT-style images of
48..96 patches a side, 3x3 pixel-unshuffle, 9216 -> 5120 -> 5120).

Prints one JSON line.  value = visual tokens (projected rows) per second of
the headline workload.  roofline = its first GEMM (the dominant kernel):
algorithmic FLOPs per launch over the mean duration from HIP events recorded
around its launches in every 4th step of the timed region, on the stream it
runs on (an event pair adds a few microseconds to its step, so the other
steps run without; the per-kernel table and Linear2's rate come from a
separate untimed pass in which every launch is bracketed).  cpu_baseline =
the fp64 oracle on the host's cores over a bounded sample of the same
workload's rows.

The defaults (50 warm-up steps, 500 timed steps per workload) measure the
steady state.  The GPU clock ramps up for the first few milliseconds after
idle, so a 20-step run reads slower.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector / MFMA) dense
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "visual tokens/sec through merge+projector+scatter"
PROF_EVERY = 4              # Linear1 is bracketed by HIP events in every 4th timed step
HEADLINE = 4                # ragged-3x3: the largest workload that fits one GPU
EXTRAS = 1                  # training step, depth 3 and embedding call: MoonViT 2x2 + LN


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="all",
                    help="'all' (default: every workload, the headline line on ragged-3x3) or "
                         "one workload index 0..4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the headline CPU-baseline sample")
    ap.add_argument("--cpu-seconds-other", type=float, default=3.0,
                    help="target duration of the other workloads' CPU-baseline samples")
    ap.add_argument("--no-hbm-kernels", action="store_true",
                    help="skip timing the standalone merge and scatter entry points")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip sampling the GFX clock under load (amd-smi, after the timed region)")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip timing the vendor GEMM (torch.matmul) on the headline's two products")
    ap.add_argument("--no-power-probe", action="store_true",
                    help="skip timing Linear1 on the headline workload with all-zero features")
    ap.add_argument("--no-train", action="store_true",
                    help="skip timing the training step (forward + backward)")
    ap.add_argument("--no-depth", action="store_true",
                    help="skip timing the depth-3 projector (one middle Linear hidden -> hidden)")
    ap.add_argument("--no-embed", action="store_true",
                    help="skip timing the call that also writes the text rows from an embedding table")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    return ap.parse_args()


def kernel_sha() -> str:
    """Hash of the GEMM's code (vlb_gemm.hip and vlb_common.h) with comments
    and whitespace removed, so that a comment edit keeps the counters valid
    and any change to the code does not."""
    h = hashlib.sha256()
    for name in ("vlb_gemm.hip", "vlb_common.h"):
        with open(os.path.join(ROOT, "patch_merge_mlp_amd", "csrc", name)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per GEMM1 launch from the committed counter summary, if it was taken
    on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"gemm1_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, _, val = line.partition(":")
            vals[k.strip()] = val.strip()
    if vals.get("kernel_source_sha") != kernel_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_threads():
    """Threads the oracle uses: the CPU share of one GPU on the measurement box
    (16), or fewer when the host has fewer; and what the host reports."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return min(avail, 16), os.cpu_count(), avail


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this bridge is measured on one GPU; images are independent, so a "
              "multi-GPU run would only replicate the weights and split the images", file=sys.stderr)
        sys.exit(2)
    # The clock sampler is started before anything touches the GPU.
    args.sampler = None if (args.no_sclk or args.copy_calibration) else ClockSampler()
    try:
        run(args)
    finally:
        if args.sampler is not None:
            args.sampler.stop()


def run(args):
    import torch

    from patch_merge_mlp_amd import vlbridge as v
    from patch_merge_mlp_amd import workloads as wl

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    which = list(range(wl.N_CONFIGS)) if args.config == "all" else [int(args.config)]
    head = HEADLINE if HEADLINE in which else which[-1]
    configs, head_res = {}, None
    for i in which:
        res = measure_config(args, v, wl, torch, i, headline=(i == head),
                             extras=(i == EXTRAS and len(which) > 1) or len(which) == 1)
        print(f"bench: {res['summary']['workload']} {res['summary']['tokens_per_s']:.4g} tok/s, "
              f"{res['summary']['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
        configs[res["summary"]["workload"]] = res["summary"]
        if i == head:
            head_res = res
        torch.cuda.empty_cache()
    out = head_res["line"]
    out["configs"] = configs
    print(json.dumps(out))


def measure_config(args, v, wl, torch, i, headline, extras):
    """Time workload i; returns {"summary": per-workload figures, "line": the JSON
    line this workload would give as the headline}."""
    w = wl.config(i)
    gen = wl.Generator(w)
    bf16 = w.dtype == "bf16"
    p = v.projector(v.F32 if w.dtype == "f32" else v.BF16, w.C, w.k, w.hidden, w.out_dim,
                    has_ln=w.has_ln, ln_eps=w.ln_eps)
    b = v.Batch(w.grids, w.views_per_image, v.LAYOUT_TILED_2D if w.tiled else v.LAYOUT_PLAIN,
                w.tiles or None, w.global_tail)
    T = v.vlb_num_tokens(p, b)
    P = v.vlb_num_slots(p, b)
    K1 = w.C * w.k * w.k
    npix = sum(gh * gw for gh, gw in w.grids)
    t = gen.tensors(npix, K1, v.vlb_image_slots(p, b))
    d = lambda x: None if x is None else x.to("cuda")
    weights = v.Weights(d(t["w1"]), d(t["b1"]), d(t["w2"]), d(t["b2"]), d(t["ln_gamma"]),
                        d(t["ln_beta"]))
    br = v.Bridge(p, weights)            # packs W1 and W2 once (weight preprocessing, untimed)
    pack_us = None
    if br.p.packed:  # the one-time packing, timed again once the code is loaded
        w1p, w2p = torch.empty_like(br.w.w1), torch.empty_like(br.w.w2)
        v.vlb_prof_enable(1 << v.K_PACK)
        v.vlb_pack_weights(p, weights.w1, weights.w2, w1p, w2p)
        torch.cuda.synchronize()
        v.vlb_prof_enable(False)
        n_pack, ms_pack = v.vlb_prof_read(v.K_PACK)
        pack_us = round(1000.0 * ms_pack, 2) if n_pack else None  # both weights
        del w1p, w2p
    feats, mask = d(t["features"]), d(t["mask"])
    nl, sep = d(t["newline"]), d(t["separator"])
    seq = d(t["seq"])
    ws = br.workspace(b, seq.shape[0])

    def step():
        v.vlb_bridge_fused(br.p, b, feats, br.w, nl, sep, mask, seq, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert v.vlb_check(ws) == v.OK

    # Timed region: HIP events bracket the Linear1 launches of every
    # PROF_EVERY-th step (on the stream they run on); every other launch runs
    # unbracketed.
    v.vlb_prof_enable(1 << v.K_GEMM1)
    v.vlb_prof_resume(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if s % PROF_EVERY == 0:
            v.vlb_prof_resume(1 << v.K_GEMM1)
            step()
            v.vlb_prof_resume(0)
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    v.vlb_prof_enable(False)
    n, ms = v.vlb_prof_read(v.K_GEMM1)
    gemm1_us = 1000.0 * ms / n
    # Per-kernel breakdown from a separate, untimed pass with every launch timed.
    v.vlb_prof_enable(True)
    reps = max(3, args.steps // 4)
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    v.vlb_prof_enable(False)
    kernels = {}
    for kid, name in enumerate(v.KERNEL_NAMES):
        n, ms = v.vlb_prof_read(kid)
        if n:
            kernels[name] = {"launches": n, "mean_us": round(1000.0 * ms / n, 2)}

    sec = (t1 - t0) / args.steps
    flops1 = 2.0 * T * K1 * w.hidden
    flops2 = 2.0 * T * w.hidden * w.out_dim
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    g1 = gemm1_us * 1e-6  # from the timed region
    g2 = kernels["gemm2"]["mean_us"] * kernels["gemm2"]["launches"] / reps * 1e-6
    achieved = flops1 / g1 / 1e12
    traffic = traffic_from_profiles(w.name)
    es = 2 if bf16 else 4
    # The merge kernel on the fused path (with the LayerNorm when the workload
    # has it): read the grid once, write Linear1's merged operand once.
    fused_merge = None
    for name in ("layernorm", "merge"):
        if name in kernels and bf16:
            us = kernels[name]["mean_us"] * kernels[name]["launches"] / reps
            nbytes = (npix * w.C + T * K1) * es
            gbs = nbytes / (us * 1e-6) / 1e9
            fused_merge = {"kernel": name, "us_per_step": round(us, 2), "bytes": nbytes,
                           "GB/s": round(gbs, 1), "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4)}
    config = {
        "workload": w.name, "images": w.n_images, "views": len(w.grids),
        "grid": list(w.grids[0]) if len(set(w.grids)) == 1 else "ragged",
        "C": w.C, "k": w.k, "hidden": w.hidden,
        "out_dim": w.out_dim, "layernorm": w.has_ln, "seq_len": w.seq_len,
        "visual_tokens": T, "placeholder_slots": P, "layout": "tiled_2d" if w.tiled else "plain",
    }
    summary = {
        "workload": w.name,
        "dtype": "bf16" if bf16 else "f32",
        "visual_tokens": T,
        "placeholder_slots": P,
        "tokens_per_s": round(T / sec, 1),
        "ms_per_step": round(sec * 1e3, 4),
        "steps": args.steps,
        "warmup": args.warmup,
        "gemm1": {"mean_us": round(gemm1_us, 2), "TFLOP/s": round(achieved, 1),
                  "frac": round(achieved / peak, 4)},
        "gemm2": {"mean_us": round(g2 * 1e6, 2), "TFLOP/s": round(flops2 / g2 / 1e12, 1),
                  "frac": round(flops2 / g2 / 1e12 / peak, 4)},
        "step_tflops": round((flops1 + flops2) / sec / 1e12, 1),
        "peak_tflops": peak,
        "kernels": kernels,
        "fused_path_merge": fused_merge,
        "weight_pack_us": pack_us,
    }
    line = {
        "metric": METRIC,
        "value": round(T / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) features; random-init weights)",
        "config": config,
        "roofline": {
            "bound": "mfma",
            "kernel": "Linear1 (GEMM + bias + GELU over the merged tokens)",
            "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic,
        },
        "gemm_tflops": {
            "gemm1": round(achieved, 1),
            "gemm2": round(flops2 / g2 / 1e12, 1),
            "both": round((flops1 + flops2) / (g1 + g2) / 1e12, 1),
            "step": round((flops1 + flops2) / sec / 1e12, 1),
        },
        "kernels": kernels,
        "weight_pack_us": pack_us,
    }

    if not args.no_sclk and headline:
        line["sclk"] = sclk_under_load(args.sampler, step, torch, sec)
    if not args.no_power_probe and headline and bf16:
        line["power_probe"] = power_probe(v, torch, args.sampler, step, feats, sec)
    if not args.no_vendor_gemm and headline and bf16:
        line["vendor_gemm"] = vendor_gemm(torch, T, K1, w.hidden, w.out_dim,
                                          gemm1_us, g2 * 1e6)

    if not args.no_hbm_kernels:
        summary["hbm_kernels"] = hbm_kernels(v, torch, w, p, b, t, d, T, K1, args.steps)
        line["hbm_kernels"] = summary["hbm_kernels"]
    if bf16 and not w.has_ln:
        summary["operand_source"] = operand_sources(v, torch, w, p, b, br, feats, nl, sep, mask,
                                                    seq, T, args.steps)
        line["operand_source"] = summary["operand_source"]
    del ws, seq, feats
    if extras and bf16:
        if not args.no_train:
            line["train_step"] = summary["train_step"] = train_step(v, torch, wl, w, p, b, t, d, T,
                                                                    K1, args.steps)
        if not args.no_depth:
            line["depth3_step"] = summary["depth3_step"] = depth3_step(v, torch, wl, w, b, t, d, T,
                                                                       args.steps)
        if not args.no_embed:
            line["embed_step"] = summary["embed_step"] = embed_step(v, torch, wl, w, b, t, d, br,
                                                                    args.steps)
    if not args.no_cpu_baseline:
        target = args.cpu_seconds if headline else args.cpu_seconds_other
        cb = cpu_baseline(w, t, T, target)
        summary["cpu_baseline"] = cb
        if headline:
            line["cpu_baseline"] = cb
    return {"summary": summary, "line": line}


def operand_sources(v, torch, w, p, b, br, feats, nl, sep, mask, seq, T, steps):
    """Both sources of Linear1's operand, timed alike (steps // 2 calls after 10
    warm-ups): the grid merged into a blocked operand first, or gathered by
    Linear1's loads (vlb_projector.gather); which one the automatic choice
    (the timed step above) took, and Linear1's mean time in each."""
    res = {}
    on = v.vlb_projector.from_buffer_copy(br.p)
    on.gather = v.GATHER_ON
    off = v.vlb_projector.from_buffer_copy(br.p)
    off.gather = v.GATHER_OFF
    n_auto = v.vlb_workspace_bytes(br.p, b, w.seq_len)
    res["auto_picks"] = "gather" if n_auto == v.vlb_workspace_bytes(on, b, w.seq_len) else "merge"
    for name, pm in (("merge", off), ("gather", on)):
        ws = torch.empty(v.vlb_workspace_bytes(pm, b, w.seq_len), dtype=torch.uint8, device="cuda")

        def one():
            v.vlb_bridge_fused(pm, b, feats, br.w, nl, sep, mask, seq, ws)

        for _ in range(10):
            one()
        torch.cuda.synchronize()
        assert v.vlb_check(ws) == v.OK
        n = max(10, steps // 2)
        t0 = time.perf_counter()
        for _ in range(n):
            one()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / n
        v.vlb_prof_enable(1 << v.K_GEMM1)
        for _ in range(max(3, n // 4)):
            one()
        torch.cuda.synchronize()
        v.vlb_prof_enable(False)
        k, ms = v.vlb_prof_read(v.K_GEMM1)
        res[name] = {"ms_per_step": round(sec * 1e3, 4), "tokens_per_s": round(T / sec, 1),
                     "gemm1_us": round(1000.0 * ms / k, 2)}
        del ws
    return res


def depth3_step(v, torch, wl, w, b, t, d, T, steps):
    """The same fused call with a depth-3 projector (Linear1 + act, one middle
    Linear(hidden -> hidden) + act, Linear2), seeded middle weights, packed
    once.  Wall time per call over `steps` calls, and the middle GEMM's rate
    (2 * T * hidden * hidden FLOP) from a pass with its launches timed."""
    (wm, bm), = wl.mid_weights(w, 3)
    p3 = v.projector(v.BF16, w.C, w.k, w.hidden, w.out_dim, has_ln=w.has_ln, ln_eps=w.ln_eps,
                     depth=3)
    weights = v.Weights(d(t["w1"]), d(t["b1"]), d(t["w2"]), d(t["b2"]), d(t["ln_gamma"]),
                        d(t["ln_beta"]), w_mid=[d(wm)], b_mid=[d(bm)])
    br3 = v.Bridge(p3, weights)
    feats, mask = d(t["features"]), d(t["mask"])
    nl, sep, seq = d(t["newline"]), d(t["separator"]), d(t["seq"])
    ws = br3.workspace(b, seq.shape[0])

    def one():
        v.vlb_bridge_fused(br3.p, b, feats, br3.w, nl, sep, mask, seq, ws)

    for _ in range(10):
        one()
    torch.cuda.synchronize()
    assert v.vlb_check(ws) == v.OK
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    v.vlb_prof_enable(1 << v.K_GEMM_MID)
    for _ in range(max(3, steps // 4)):
        one()
    torch.cuda.synchronize()
    v.vlb_prof_enable(False)
    n, ms = v.vlb_prof_read(v.K_GEMM_MID)
    us = 1000.0 * ms / n
    return {"ms_per_step": round(sec * 1e3, 4), "tokens_per_s": round(T / sec, 1),
            "gemm_mid": {"mean_us": round(us, 2),
                         "TFLOP/s": round(2.0 * T * w.hidden * w.hidden / (us * 1e-6) / 1e12, 1)}}


def embed_step(v, torch, wl, w, b, t, d, br, steps):
    """vlb_bridge_embed: the same bridge, with every text row of the sequence
    written from a seeded embedding table of 102,400 rows (token-id scan, then
    k_embed_rows).  Wall time per call over `steps` calls, and the embedding
    kernel's rate in algorithmic bytes: each text row read from the table once
    and written once, plus the 4-byte id of every position."""
    ids, table = wl.token_inputs(w, t["mask"])
    n_text = int((ids != wl.IMAGE_TOKEN_ID).sum())
    ids, table = d(ids), d(table)
    seq = torch.empty(w.seq_len, w.out_dim, dtype=w.torch_dtype, device="cuda")
    ws = br.workspace(b, w.seq_len)
    feats, nl, sep = d(t["features"]), d(t["newline"]), d(t["separator"])

    def one():
        v.vlb_bridge_embed(br.p, b, feats, br.w, nl, sep, ids, wl.IMAGE_TOKEN_ID, table, seq, ws)

    for _ in range(10):
        one()
    torch.cuda.synchronize()
    assert v.vlb_check(ws) == v.OK
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    v.vlb_prof_enable(1 << v.K_EMBED)
    reps = max(3, steps // 4)
    for _ in range(reps):
        one()
    torch.cuda.synchronize()
    v.vlb_prof_enable(False)
    n, ms = v.vlb_prof_read(v.K_EMBED)
    us = 1000.0 * ms / n
    nbytes = 2 * n_text * w.out_dim * 2 + 4 * w.seq_len
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"ms_per_step": round(sec * 1e3, 4), "text_rows": n_text,
            "embed_kernel": {"mean_us": round(us, 2), "bytes": nbytes, "GB/s": round(gbs, 1),
                             "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4)}}


def hbm_kernels(v, torch, w, p, b, t, d, T, K1, steps):
    """Standalone merge (materialised space-to-depth) and scatter, in GB/s of
    algorithmic bytes (read + write once)."""
    es = 2 if w.dtype == "bf16" else 4
    pnl = v.projector(p.dtype, w.C, w.k, w.hidden, w.out_dim)  # merge without LayerNorm
    merged = torch.empty(T, K1, dtype=w.torch_dtype, device="cuda")
    ws = v.workspace(pnl, b, w.seq_len)
    feats = d(t["features"])
    rows = torch.randn(T, w.out_dim, device="cuda").to(w.torch_dtype)
    seq = d(t["seq"])
    mask = d(t["mask"])
    nl, sep = d(t["newline"]), d(t["separator"])
    for _ in range(2):
        v.vlb_merge_tokens(pnl, b, feats, None, None, merged, ws)
        v.vlb_scatter_tokens(pnl, b, rows, nl, sep, mask, seq, ws)
    torch.cuda.synchronize()
    v.vlb_prof_enable(True)
    for _ in range(steps):
        v.vlb_merge_tokens(pnl, b, feats, None, None, merged, ws)
        v.vlb_scatter_tokens(pnl, b, rows, nl, sep, mask, seq, ws)
    torch.cuda.synchronize()
    v.vlb_prof_enable(False)
    res = {}
    npix = sum(gh * gw for gh, gw in w.grids)
    nbytes = {
        "merge": (npix * w.C + T * K1) * es,
        "scatter": 2 * T * w.out_dim * es,
    }
    for kid, name in ((v.K_MERGE, "merge"), (v.K_SCATTER, "scatter")):
        n, ms = v.vlb_prof_read(kid)
        sec = ms / n / 1e3
        gbs = nbytes[name] / sec / 1e9
        res[name] = {"mean_us": round(sec * 1e6, 2), "bytes": nbytes[name], "GB/s": round(gbs, 1),
                     "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4)}
    return res


_SAMPLER = r"""
import re, subprocess, sys, time
pat = re.compile(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+) MHz")
while True:
    try:
        r = subprocess.run(["amd-smi", "metric", "-c"], capture_output=True, text=True, timeout=10)
    except Exception:
        sys.exit(0)
    mhz = pat.findall(r.stdout)
    if not mhz:
        sys.exit(0)
    print(time.monotonic(), *mhz, flush=True)
"""


class ClockSampler:
    """GFX clocks of every XCD from amd-smi, sampled back to back by a child
    process that is started before this process touches the GPU (a process that
    has initialised the GPU must not start programs itself).  Each output line is
    a CLOCK_MONOTONIC time stamp and the clocks in MHz."""

    def __init__(self):
        import subprocess
        import threading
        self.lines = []
        try:
            self.proc = subprocess.Popen([sys.executable, "-c", _SAMPLER], stdout=subprocess.PIPE,
                                         stderr=subprocess.DEVNULL, text=True)
        except OSError:
            self.proc = None
            return
        self.reader = threading.Thread(target=self._read, daemon=True)
        self.reader.start()

    def _read(self):
        for line in self.proc.stdout:
            self.lines.append(line.split())

    def window(self, t0, t1):
        """Samples taken in [t0, t1] (time.monotonic()), flattened over XCDs."""
        out = []
        for f in list(self.lines):
            if len(f) > 1 and t0 <= float(f[0]) <= t1:
                out.extend(int(x) for x in f[1:])
        return out

    def stop(self):
        if self.proc is not None and self.proc.poll() is None:
            self.proc.terminate()
            try:
                self.proc.wait(timeout=10)
            except Exception:  # noqa: BLE001
                self.proc.kill()


def sclk_under_load(sampler, step, torch, sec_per_step, seconds=2.5):
    """GFX clock while the step runs back to back for a few seconds after the
    timed region: the samples' median and range in MHz, or None when amd-smi
    gave none."""
    if sampler is None or sampler.proc is None:
        return None
    n = max(1, int(seconds / max(sec_per_step, 1e-6)))
    t0 = time.monotonic()
    for i in range(n):
        step()
        if i % 200 == 199:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t1 = time.monotonic()
    samples = sorted(sampler.window(t0, t1))
    if not samples:
        return None
    q = lambda f: samples[min(len(samples) - 1, int(f * len(samples)))]
    return {"median_mhz": q(0.5), "p10_mhz": q(0.1), "p90_mhz": q(0.9), "samples": len(samples),
            "how": "amd-smi metric -c (per-XCD GFX clocks) in a child process, samples taken "
                   "during an untimed burst of steps"}


def vendor_gemm(torch, T, K1, H, O, gemm1_us, gemm2_us, reps=30):
    """The two products of the step through torch.matmul in bf16 (hipBLASLt on
    ROCm), on seeded operands of the same shapes, for comparison: the plain
    products only -- no bias, activation, tile-blocked output or scatter --
    with the weight passed transposed and contiguous.  Mean over `reps` calls
    between two events, after warm-up; next to it the library's own Linear1
    and Linear2 means from this run."""
    g = torch.Generator(device="cuda").manual_seed(5)
    out = {}
    for name, K, N, ours in (("linear1", K1, H, gemm1_us), ("linear2", H, O, gemm2_us)):
        a = torch.randn(T, K, device="cuda", generator=g).to(torch.bfloat16)
        wt = (torch.randn(N, K, device="cuda", generator=g) * K ** -0.5).to(torch.bfloat16)
        wt = wt.t().contiguous()
        for _ in range(5):
            c = a @ wt
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = a @ wt
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / reps
        flop = 2.0 * T * K * N
        out[name] = {"shape_MxKxN": [T, K, N], "torch_matmul_us": round(us, 1),
                     "torch_matmul_TFLOP/s": round(flop / us / 1e6, 1),
                     "library_us": round(ours, 1), "library_TFLOP/s": round(flop / ours / 1e6, 1)}
        del a, wt, c
    return out


def power_probe(v, torch, sampler, step, feats, sec_per_step, seconds=1.5):
    """Linear1 with the workload's features and with all-zero features (the
    merged operand, and with it half of every MFMA's input, is then zero):
    the same instructions and memory traffic, but the MFMA's power depends on
    the data, so on a power-capped board a loop bound by power runs the zero
    operand faster, at a higher clock, while a loop bound by its instruction
    stream would not change.  For each: Linear1's mean time (HIP events on
    every PROF_EVERY-th step of a burst of steps) and the GFX clock during the
    burst (None without the sampler).  The features are restored afterwards."""
    saved = feats.clone()
    n = max(PROF_EVERY, int(seconds / max(sec_per_step, 1e-6)))
    out = {}
    for name in ("workload_features", "zero_features"):
        if name == "zero_features":
            feats.zero_()
        for _ in range(10):
            step()
        v.vlb_prof_enable(1 << v.K_GEMM1)
        v.vlb_prof_resume(0)
        torch.cuda.synchronize()
        t0 = time.monotonic()
        for i in range(n):
            if i % PROF_EVERY == 0:
                v.vlb_prof_resume(1 << v.K_GEMM1)
                step()
                v.vlb_prof_resume(0)
            else:
                step()
        torch.cuda.synchronize()
        t1 = time.monotonic()
        v.vlb_prof_enable(False)
        k, ms = v.vlb_prof_read(v.K_GEMM1)
        mhz = None
        if sampler is not None and sampler.proc is not None:
            smp = sorted(sampler.window(t0, t1))
            mhz = smp[len(smp) // 2] if smp else None
        out[name] = {"gemm1_us": round(1000.0 * ms / k, 2) if k else None, "sclk_median_mhz": mhz}
    feats.copy_(saved)
    torch.cuda.synchronize()
    return out


def train_step(v, torch, wl, w, p, b, t, d, T, K1, steps):
    """One training step of the projector: the weights packed once (they change
    every step), vlb_bridge_fused_train and vlb_bridge_backward on the packed
    weights, for a seeded sequence gradient.  Wall time over `steps` steps, then a
    separate pass with every launch timed for the per-kernel table and the backward
    GEMMs' rates."""
    w1, w2 = d(t["w1"]), d(t["w2"])
    w1p = torch.empty(v.vlb_packed_bytes(p, 1) // 2, dtype=w1.dtype, device="cuda")
    w2p = torch.empty(v.vlb_packed_bytes(p, 2) // 2, dtype=w2.dtype, device="cuda")
    pp = v.vlb_projector.from_buffer_copy(p)
    pp.packed = 1
    weights = v.Weights(w1p, d(t["b1"]), w2p, d(t["b2"]), d(t["ln_gamma"]), d(t["ln_beta"]))
    feats, mask = d(t["features"]), d(t["mask"])
    nl, sep = d(t["newline"]), d(t["separator"])
    seq = d(t["seq"])
    dseq = d(wl.seq_grad(w))
    S = seq.shape[0]
    fws = torch.empty(v.vlb_workspace_bytes(pp, b, S), dtype=torch.uint8, device="cuda")
    saved = torch.empty(v.vlb_saved_bytes(pp, b), dtype=torch.uint8, device="cuda")
    bws = torch.empty(v.vlb_backward_workspace_bytes(pp, b, S), dtype=torch.uint8, device="cuda")
    g = v.Grads.empty(pp, b)

    def one():
        v.vlb_pack_weights(p, w1, w2, w1p, w2p)
        v.vlb_bridge_fused_train(pp, b, feats, weights, nl, sep, mask, seq, saved, fws)
        v.vlb_bridge_backward(pp, b, feats, weights, mask, dseq, saved, g, bws)

    for _ in range(2):
        one()
    torch.cuda.synchronize()
    assert v.vlb_check(bws) == v.OK
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    v.vlb_prof_enable(True)
    for _ in range(max(3, steps // 4)):
        one()
    torch.cuda.synchronize()
    v.vlb_prof_enable(False)
    kernels = {}
    for kid, name in enumerate(v.KERNEL_NAMES):
        n, ms = v.vlb_prof_read(kid)
        if n:
            kernels[name] = {"launches": n, "mean_us": round(1000.0 * ms / n, 2)}
    reps = max(3, steps // 4)
    H, O = w.hidden, w.out_dim
    f_out = 2.0 * T * H * O   # Linear2-shaped products: dW2, dA1
    f_in = 2.0 * T * H * K1   # Linear1-shaped products: dW1, dXm
    rate = {}
    for name, fl in (("bwd_dw2", f_out), ("bwd_da1", f_out), ("bwd_dw1", f_in), ("bwd_dx", f_in)):
        if name in kernels:
            us = kernels[name]["mean_us"] * kernels[name]["launches"] / reps
            rate[name] = round(fl / (us * 1e-6) / 1e12, 1)
    fwd_fl = f_in + f_out
    step_fl = 3 * fwd_fl  # forward + four backward products
    return {
        "ms_per_step": round(sec * 1e3, 4),
        "tokens_per_s": round(T / sec, 1),
        "flop_per_step": step_fl,
        "tflops_step": round(step_fl / sec / 1e12, 1),
        "gemm_tflops": rate,
        "kernels": kernels,
        "note": "weights packed once per step, forward (training form: merged tokens, Z1 and "
                "act(Z1) kept) + backward; kernel means from a separate pass with every launch "
                "timed",
    }


def cpu_baseline(w, t, T, target_s):
    """The oracle (unchanged) on the host cores, over the first rows of the workload;
    the rate is projected rows per second."""
    from oracle import oracle as o
    spec = o.Spec(grids=w.grids, C=w.C, k=w.k, hidden=w.hidden, out_dim=w.out_dim,
                  views_per_image=w.views_per_image, has_ln=w.has_ln, ln_eps=w.ln_eps,
                  tiled=w.tiled, tiles=w.tiles, global_tail=w.global_tail)
    cores, cpu_count, avail = host_threads()
    args = [t["features"], t["ln_gamma"], t["ln_beta"], t["w1"], t["b1"], t["w2"], t["b2"]]
    wide = [o._f64(a) for a in args]  # widening is input marshalling, outside the timed part
    n = cores
    while True:  # grow the sample until it takes about a second, then scale to the target
        t0 = time.perf_counter()
        o.project_rows(spec, *wide, row_ids=list(range(n)), nthreads=cores)
        dt = time.perf_counter() - t0
        if dt > 1.0 or n >= T:
            break
        n = min(T, n * 4)
    n = int(min(T, max(n, n * target_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    o.project_rows(spec, *wide, row_ids=list(range(n)), nthreads=cores)
    dt = time.perf_counter() - t0
    steps = "LayerNorm, merge" if w.has_ln else "merge"
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host_cpu_count": cpu_count, "host_cpus_available": avail,
            "sample": f"first {n} of {T} token rows of {w.name} through the fp64 oracle "
                      f"({steps}, Linear, GELU, Linear), {dt:.1f} s on {cores} threads"}


if __name__ == "__main__":
    main()
