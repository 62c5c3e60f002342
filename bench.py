"""Benchmark: committed RVQ codes/s of CodePredictor speculative decoding.

One step = cp_spec_decode_frames over the whole workload (every frame of
every stream: prefill, then draft / verify / accept / commit rounds until the
frames are full), inputs resident in HBM.  Default workload: the
Qwen3-TTS-0.6B-shaped CodePredictor (5 layers, H 1024, G 16, V 2048, bf16
weights), 1 stream x 1000 frames, N = 4; the 64-stream tiny workload is
reported alongside.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "committed RVQ codes/sec + accepted codes/verify pass, 1 & 64 streams, N=4"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}  # dense, MI355X
REALTIME_FPS = 12.5
# The next round's drafts formed in this round's verify tail (RVQ section
# 2.2, Figure 3) on every workload where it measured faster on this GPU
# (codes/s against separate draft launches: tiny 1.19x, tiny greedy 1.15x,
# tiny at 64 streams 1.09x, qwen3tts 1.05x, qwen3tts at 64 streams 1.01x);
# the wide decoder at 256 streams keeps separate draft launches (0.91x: its
# R*W extra candidate rows per stream cost more head work than the launches
# saved).  The fused_draft section of the output measures both again.
UNFUSED_WORKLOADS = ("wide-256",)


def fused_for(workload):
    return 0 if workload in UNFUSED_WORKLOADS else 1


def _inputs(c, torch, np):
    import synth
    hf, c0, seeds = synth.make_inputs(c)
    return (torch.from_numpy(hf).cuda(), torch.from_numpy(c0).cuda(),
            torch.from_numpy(seeds.view(np.int64)).cuda(), hf, c0, seeds)


def kernel_table(h, c, B, iters=200):
    """Live per-kernel timing (HIP events on the decode stream) of every
    kernel kind of the round, in its decode launch configuration."""
    from speculative_decoding_rvq_amd import binding
    per_round = {"draft_heads": 1, "target_heads": 1}
    out = {}
    for kind in binding.KERNEL_KINDS:
        if kind == "draft_heads" and c["verify_size"] < 2:
            continue
        t = h.time_kernel(kind, B, iters)
        t["launches_per_round"] = per_round.get(kind, c["layers"])
        t["us_per_round"] = t["avg_us"] * t["launches_per_round"]
        t["achieved_GBps"] = t["bytes_per_launch"] / (t["avg_us"] * 1e3)
        t["achieved_TFLOPs"] = t["flops_per_launch"] / (t["avg_us"] * 1e6)
        out[kind] = t
    return out


# the sources of the kernel a traffic summary was taken on: the GEMV (one
# stream) or the batched matrix-core projections
TRAFFIC_SOURCES = {
    False: ("speculative_decoding_rvq_amd/csrc/gemv_impl.h",
            "speculative_decoding_rvq_amd/csrc/gemv_bf16.hip",
            "speculative_decoding_rvq_amd/csrc/kernels.h"),
    True: ("speculative_decoding_rvq_amd/csrc/bgemm.hip",
           "speculative_decoding_rvq_amd/csrc/dev_common.h",
           "speculative_decoding_rvq_amd/csrc/kernels.h"),
}


def measured_traffic(workload, kind, matrix_cores=False):
    """HBM-side bytes per launch from the committed counter summary
    (profiles/<workload>_<kind>_traffic.md), or None when there is none or
    the kernel's sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_{kind}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", " ", "#")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().split()[0] if v.strip() else ""
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[bool(matrix_cores)]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline(table, weight_dtype, workload=None):
    """Roofline object of the kernel with the largest share of a round:
    HBM-bound for the GEMV path, MFMA-bound (dense peak of the weights'
    dtype; the bf16 path issues two fp16 MFMAs per product, one per
    activation piece, counted once here) when the launch ran on matrix-core
    tiles."""
    kind = max(table, key=lambda k: table[k]["us_per_round"])
    t = table[kind]
    traffic = measured_traffic(workload, kind, t.get("matrix_cores")) if workload else None
    common = {"kernel": kind, "traffic": traffic, "avg_us": t["avg_us"],
              "bytes_per_launch": t["bytes_per_launch"],
              "flops_per_launch": t["flops_per_launch"]}
    if t.get("matrix_cores"):
        peak = MFMA_PEAK_TFLOPS[weight_dtype]
        return {"bound": "mfma", "achieved": t["achieved_TFLOPs"], "peak": peak,
                "unit": "TFLOP/s", "frac": t["achieved_TFLOPs"] / peak, **common}
    return {"bound": "hbm", "achieved": t["achieved_GBps"],
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": t["achieved_GBps"] / HBM_PEAK_GBS, **common}


def run_workload(cid, steps, warmup, verify_size=None, frames=None,
                 kernels=False, offsets=None, **cfg):
    import numpy as np
    import torch

    import synth
    from speculative_decoding_rvq_amd import binding
    over = {}
    if verify_size is not None:
        over["verify_size"] = verify_size
    if frames is not None:
        over["frames"] = frames
    if offsets is not None:  # (K, scale): seeded position-aware draft offsets
        over["draft_offsets"], over["offset_scale"] = offsets
    over.update(cfg)
    c = synth.config(cid, **over)
    w = synth.make_weights(c)
    wdev = binding.weights_to_device(w)
    h = binding.Handle(c, wdev)
    dh, dc, ds, *_ = _inputs(c, torch, np)
    F, B, G = c["frames"], c["streams"], c["groups"]
    out = torch.empty((F, B, G), dtype=torch.int32, device="cuda")
    flags = torch.empty((F, B), dtype=torch.int32, device="cuda")
    st = binding.new_stats_tensor()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        h.decode_frames(dh, dc, ds, out, flags, None)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    t0 = time.perf_counter()
    for i in range(steps):
        h.decode_frames(dh, dc, ds, out, flags, st if i == 0 else None)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    s = binding.get_stats(st)
    codes = F * B * (G - 1)
    res = {
        "workload": cid, "name": c["name"], "streams": B, "frames": F,
        "verify_size": c["verify_size"], "ms_per_step": ms,
        "wall_ms_per_step": 1e3 * wall / steps,
        "codes_per_s": codes / (ms / 1e3),
        "frames_per_s": F * B / (ms / 1e3),
        "frames_per_s_per_stream": F / (ms / 1e3),
        "codes_per_verify_pass": (s["codes"] - s["frames"]) / max(s["rounds"], 1),
        "codes_per_decoder_pass": s["codes"] / max(s["rounds"] + s["prefill_passes"], 1),
        "acceptance_by_offset": [a / p for a, p in zip(s["accepted"], s["proposed"]) if p],
        "stats": s,
    }
    if kernels:
        torch.cuda.synchronize()
        res["kernels"] = kernel_table(h, c, B)
        res["talker_feedback"] = feedback_timing(h, c, out, torch)
    h.close()
    del wdev
    torch.cuda.empty_cache()
    return res, c


def feedback_timing(h, c, out, torch, iters=50):
    """The Talker hand-off (sum of each finished frame's embedding rows) over
    every frame the timed decode produced, HIP events around `iters`
    launches on the current stream."""
    F, B, G = out.shape
    codes = out.reshape(F * B, G).contiguous()
    fb = torch.empty((F * B, c["hidden"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    h.talker_feedback(codes, fb)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        h.talker_feedback(codes, fb)
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / iters
    ws = 2 if c["dtype"] == "bf16" else 4
    nbytes = F * B * (G * c["hidden"] * ws + c["hidden"] * 4 + G * 4)
    return {"rows": F * B, "us_per_launch": us, "us_per_frame": us / (F * B),
            "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / us / 1e3}


def verify_sweep(cid, Ns=(2, 3, 4, 5, 6, 7, 8), frames=None, steps=2):
    """Per-device choice of the verify window N (the package's
    calibrate_window): for each N, codes/s, committed codes per verify pass
    and one pass's time on this GPU (same weights and inputs); the codes per
    round that the widest window's measured acceptance predicts for each N;
    the N chosen from prediction and pass times, and the N with the best
    measured codes/s."""
    import numpy as np
    import torch

    import synth
    from speculative_decoding_rvq_amd import binding
    from speculative_decoding_rvq_amd.calibrate import calibrate_window
    c = synth.config(cid, fused_draft=fused_for(cid), **({"frames": frames} if frames else {}))
    wdev = binding.weights_to_device(synth.make_weights(c))
    dh, dc, ds, *_ = _inputs(c, torch, np)
    cal = calibrate_window(c, wdev, dh, dc, ds, sizes=Ns, repeats=steps)
    del wdev
    torch.cuda.empty_cache()
    return {"workload": cid, "frames": c["frames"], "streams": c["streams"],
            "fused_draft": c["fused_draft"], "best_verify_size": cal["measured_best"],
            "calibrated_verify_size": cal["verify_size"],
            "accepted_share_by_offset": cal["accepted_share_by_offset"],
            "by_verify_size": {str(n): {k: round(v, 4) for k, v in r.items()}
                               for n, r in cal["by_verify_size"].items()}}


def tree_sweep(cid, shapes, frames=300, steps=2, oracle_frames=6):
    """The tree-shaped verify window on this GPU: for each tree (a parent
    list), codes/s, committed codes per verify pass and the per-depth share of
    rounds that accepted a node at that depth, on the same weights and
    inputs; plus the tree oracle's codes/s on the first frames of the first
    tree (host cores, as the CPU baseline)."""
    import numpy as np
    import torch

    import synth
    from speculative_decoding_rvq_amd import binding
    c = synth.config(cid, frames=frames)
    w = synth.make_weights(c)
    wdev = binding.weights_to_device(w)
    dh, dc, ds, hf, c0, seeds = _inputs(c, torch, np)
    F, G = c["frames"], c["groups"]
    out = torch.empty((F, 1, G), dtype=torch.int32, device="cuda")
    rows = []
    for parents in shapes:
        h = binding.Handle(dict(c, tree=list(parents)), wdev, max_streams=1)
        st = binding.new_stats_tensor()
        h.decode_frames(dh, dc, ds, out, None, None)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            h.decode_frames(dh, dc, ds, out, None, st if i == 0 else None)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        s = binding.get_stats(st)
        rows.append({"tree": list(parents), "codes_per_s": F * (G - 1) / (ms / 1e3),
                     "ms_per_step": ms,
                     "codes_per_verify_pass": (s["codes"] - s["frames"]) / max(s["rounds"], 1),
                     "accepted_share_by_depth": [a / p for a, p in zip(s["accepted"], s["proposed"]) if p]})
        h.close()
    del wdev
    torch.cuda.empty_cache()
    from oracle import decoder, spec, tree
    m = decoder.Model(c, w)
    dp = dict(greedy=False, temperature=c["temperature"], top_k=c["top_k"])
    t = tree.Tree(shapes[0])
    t0 = time.perf_counter()
    for f in range(oracle_frames):
        tree.decode_frame_tree(m, dp, t, hf[f, 0], int(c0[f, 0]), int(seeds[f, 0]), spec.new_stats())
    dt = time.perf_counter() - t0
    return {"workload": cid, "frames": F, "by_tree": rows,
            "oracle": {"tree": list(shapes[0]), "codes_per_s": oracle_frames * (G - 1) / dt,
                       "sample": f"first {oracle_frames} frames"}}


def cpu_baseline(cid, n_frames):
    """The oracle, as it stands, on the first n_frames of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle import decoder, spec
    c = synth.config(cid)
    w = synth.make_weights(c)
    hf, c0, seeds = synth.make_inputs(c)
    t_build = time.perf_counter()
    m = decoder.Model(c, w)
    t0 = time.perf_counter()
    st = spec.new_stats()
    dp = dict(verify_size=c["verify_size"], greedy=c["greedy"],
              temperature=c["temperature"], top_k=c["top_k"])
    B = c["streams"]
    done = 0
    for f in range(c["frames"]):
        for b in range(B):
            spec.decode_frame(m, dp, hf[f, b], int(c0[f, b]), int(seeds[f, b]), st)
            done += 1
            if done >= n_frames:
                break
        if done >= n_frames:
            break
    dt = time.perf_counter() - t0
    host = len(os.sched_getaffinity(0))
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": done * (c["groups"] - 1) / dt, "unit": "codes/s",
        "cores": int(min(blas, host)), "kind": "oracle",
        "host_cores": host,
        "threading": "the frame loop is single-threaded Python; its matrix "
                     f"products run on numpy's BLAS pool of {blas} threads",
        "sample": f"first {done} frames of the workload (stream 0), "
                  f"{dt:.1f} s after a {t0 - t_build:.1f} s float64 weight copy",
    }


def oracle_rate(cid, n_frames, **over):
    """Oracle codes/s on the first n_frames (stream 0) of a workload."""
    import synth
    from oracle import decoder, spec
    c = synth.config(cid, **over)
    m = decoder.Model(c, synth.make_weights(c))
    hf, c0, seeds = synth.make_inputs(c, frames=n_frames)
    dp = dict(verify_size=c["verify_size"], greedy=c["greedy"],
              temperature=c["temperature"], top_k=c["top_k"])
    t0 = time.perf_counter()
    for f in range(n_frames):
        spec.decode_frame(m, dp, hf[f, 0], int(c0[f, 0]), int(seeds[f, 0]))
    return n_frames * (c["groups"] - 1) / (time.perf_counter() - t0)


def _leg(r, c, steps, warmup):
    return {"workload": f"{c['name']}: {c['streams']} stream(s) x {c['frames']} frames, "
                        f"G{c['groups']} V{c['vocab']} H{c['hidden']} L{c['layers']}, "
                        f"{c['dtype']} weights, N={c['verify_size']}, "
                        + ("greedy" if c["greedy"] else f"T={c['temperature']}, top-k {c['top_k']}"),
            "steps": steps, "warmup": warmup, "ms_per_step": r["ms_per_step"],
            "codes_per_s": r["codes_per_s"], "frames_per_s": r["frames_per_s"],
            "realtime_factor_vs_12.5fps": r["frames_per_s_per_stream"] / REALTIME_FPS,
            "codes_per_verify_pass": r["codes_per_verify_pass"],
            "codes_per_decoder_pass": r["codes_per_decoder_pass"],
            "acceptance_by_offset": r["acceptance_by_offset"],
            "fused_draft": c.get("fused_draft", 0)}


def baseline_configs(main_line, s64, c64):
    """Every workload the baseline lists, each at its full size: 1 tiny fp32
    (1 x 100, N 3); 2 the headline line itself; 3 the tiny decoder greedy,
    N = 2..8 over 1000 frames; 4 tiny at 64 streams (the streams64 leg);
    5 the wide bf16 decoder at 256 streams x 200 frames with its kernels'
    roofline (its 1.0 GB of decoder and head weights exceed the 256 MB
    Infinity Cache, so its weight traffic comes from HBM)."""
    out = {}
    r1, c1 = run_workload("tiny", 5, 2, fused_draft=fused_for("tiny"))
    out["1"] = _leg(r1, c1, 5, 2)
    out["1"]["cpu_oracle_codes_per_s"] = oracle_rate("tiny", 30)
    out["2"] = {"workload": main_line["config"]["workload"], "see": "value / roofline"}
    sweep = {}
    for N in range(2, 9):
        r3, c3 = run_workload("tiny-greedy", 3, 1, verify_size=N, fused_draft=fused_for("tiny-greedy"))
        leg = _leg(r3, c3, 3, 1)
        sweep[str(N)] = {k: leg[k] for k in ("codes_per_s", "ms_per_step", "codes_per_verify_pass",
                                               "codes_per_decoder_pass", "acceptance_by_offset")}
    out["3"] = {"workload": "tiny-fp32-greedy: 1 stream x 1000 frames, G8 V256 H256 L2, f32 "
                            "weights, greedy, N = 2..8 (N >= 6 commit alike: the window is cut "
                            "to G - 2 - s drafts)",
                "by_verify_size": sweep}
    out["4"] = _leg(s64, c64, 1, 1)
    r5, c5 = run_workload("wide-256", 1, 1, kernels=True, fused_draft=fused_for("wide-256"))
    out["5"] = _leg(r5, c5, 1, 1)
    k5 = r5["kernels"]
    out["5"]["roofline"] = roofline(k5, c5["dtype"], "wide-256")
    # the same launches as weight bytes from HBM per launch time
    dom = out["5"]["roofline"]["kernel"]
    ws = 2 if c5["dtype"] == "bf16" else 4
    out["5"]["roofline"]["hbm_frac_of_weights"] = (
        k5[dom]["bytes_per_launch"] / (k5[dom]["avg_us"] * 1e3)) / HBM_PEAK_GBS
    out["5"]["kernels"] = {k: {kk: round(v, 3) if isinstance(v, float) else v for kk, v in t.items()}
                           for k, t in k5.items()}
    out["5"]["cpu_oracle_codes_per_s"] = oracle_rate("wide-256", 2)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="qwen3tts",
                    help="one of synth.WORKLOADS")
    ap.add_argument("--frames", type=int, default=None)
    ap.add_argument("--cpu-frames", type=int, default=160)
    ap.add_argument("--no-extra", action="store_true",
                    help="only the main workload (no AR / 64-stream / CPU legs)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (reference "
                         "kernel for scaling the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this path runs on one GPU; streams shard across GPUs "
              "with no communication inside a round, so N > 1 is not "
              "measured here", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        x = torch.ones(n, device="cuda")
        y = torch.empty_like(x)
        for _ in range(8):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mb, "launches": 8}), flush=True)
        return

    fd = fused_for(args.workload)
    main_res, c = run_workload(args.workload, args.steps, args.warmup,
                               frames=args.frames, kernels=True, fused_draft=fd)
    line = {
        "metric": METRIC,
        "value": main_res["codes_per_s"],
        "unit": "codes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{c['name']}: {c['streams']} "
                        f"stream(s) x {c['frames']} frames, G{c['groups']} "
                        f"V{c['vocab']} H{c['hidden']} L{c['layers']}, "
                        f"N={c['verify_size']}, T={c['temperature']}, "
                        f"top-k {c['top_k']}",
            "weights": c["dtype"], "streams": c["streams"],
            "frames": c["frames"], "verify_size": c["verify_size"],
            "fused_draft": fd,
        },
        "accepted_codes_per_verify_pass": main_res["codes_per_verify_pass"],
        "codes_per_decoder_pass": main_res["codes_per_decoder_pass"],
        "frames_per_s": main_res["frames_per_s"],
        "realtime_factor_vs_12.5fps": main_res["frames_per_s_per_stream"] / REALTIME_FPS,
        "acceptance_by_offset": main_res["acceptance_by_offset"],
        "roofline": roofline(main_res["kernels"], c["dtype"], args.workload),
        "kernels": {k: {kk: round(v, 3) if isinstance(v, float) else v
                        for kk, v in t.items()}
                    for k, t in main_res["kernels"].items()},
        "talker_feedback": main_res["talker_feedback"],
    }
    if not args.no_extra:
        ar, _ = run_workload(args.workload, 1, 1, verify_size=0, frames=args.frames)
        line["ar_baseline"] = {"codes_per_s": ar["codes_per_s"],
                               "ms_per_step": ar["ms_per_step"],
                               "speedup": main_res["codes_per_s"] / ar["codes_per_s"]}
        s64, c64 = run_workload("tiny-64", 1, 1, kernels=True, fused_draft=fused_for("tiny-64"))
        line["streams64"] = {k: s64[k] for k in (
            "codes_per_s", "frames_per_s", "ms_per_step",
            "codes_per_verify_pass", "codes_per_decoder_pass",
            "acceptance_by_offset")}
        line["streams64"]["roofline"] = roofline(s64["kernels"], c64["dtype"], "tiny-64")
        # the qwen3tts shape at 64 streams: weights large enough for the
        # batched projections' roofline to mean something
        q64, cq64 = run_workload("qwen3tts-64", 1, 1, kernels=True,
                                 fused_draft=fused_for("qwen3tts-64"))
        line["streams64_qwen3tts"] = {k: q64[k] for k in (
            "codes_per_s", "frames_per_s", "ms_per_step",
            "codes_per_verify_pass", "codes_per_decoder_pass")}
        line["streams64_qwen3tts"]["roofline"] = roofline(q64["kernels"], cq64["dtype"],
                                                          "qwen3tts-64")
        line["streams64_qwen3tts"]["kernels"] = {
            k: {kk: round(v, 3) if isinstance(v, float) else v for kk, v in t.items()}
            for k, t in q64["kernels"].items()}
        # position-aware draft offsets (3 seeded vectors): same decode, the
        # draft heads reading h_s + b_t; untrained offsets, so only the cost
        # and the changed acceptance are meaningful
        line["draft_offsets"] = {}
        offs = {}
        for wl, steps in ((args.workload, args.steps), ("qwen3tts-64", 1)):
            ref = main_res if wl == args.workload else q64
            o, co = run_workload(wl, steps, 1, frames=args.frames if wl == args.workload else None,
                                 offsets=(3, 0.1), fused_draft=fused_for(wl))
            offs[wl] = o
            line["draft_offsets"][wl] = {
                "K": co["draft_offsets"], "scale": co["offset_scale"],
                "codes_per_s": o["codes_per_s"], "ms_per_step": o["ms_per_step"],
                "codes_per_verify_pass": o["codes_per_verify_pass"],
                "acceptance_by_offset": o["acceptance_by_offset"],
                "throughput_vs_no_offsets": o["codes_per_s"] / ref["codes_per_s"],
                "round_time_vs_no_offsets": (o["ms_per_step"] / o["stats"]["rounds"]) /
                                                    (ref["ms_per_step"] / ref["stats"]["rounds"]),
            }
        # the next round's drafts formed in this round's verify tail (one
        # heads launch and one softmax launch per round instead of two each),
        # against separate draft launches: each workload's leg above ran in
        # its chosen mode, the other mode runs here
        line["fused_draft"] = {}

        def per_pass_us(r):  # one stream's verify or prefill pass
            return 1e3 * r["ms_per_step"] / ((r["stats"]["rounds"] + r["stats"]["prefill_passes"]) / r["streams"])

        for key, wl, steps, off, have in ((args.workload, args.workload, args.steps, None, main_res),
                                          ("tiny-64", "tiny-64", 1, None, s64),
                                          ("qwen3tts-64", "qwen3tts-64", 1, None, q64),
                                          (args.workload + " K=3", args.workload, args.steps, (3, 0.1),
                                           offs[args.workload])):
            other = run_workload(wl, steps, 1, frames=args.frames if wl == args.workload else None,
                                 offsets=off, fused_draft=1 - fused_for(wl))[0]
            fr, ref = (have, other) if fused_for(wl) else (other, have)
            line["fused_draft"][key] = {
                "codes_per_s": fr["codes_per_s"], "ms_per_step": fr["ms_per_step"],
                "codes_per_verify_pass": fr["codes_per_verify_pass"],
                "unfused_codes_per_s": ref["codes_per_s"],
                "throughput_vs_unfused": fr["codes_per_s"] / ref["codes_per_s"],
                "us_per_pass": per_pass_us(fr),
                "unfused_us_per_pass": per_pass_us(ref),
                "used_by_the_legs_above": bool(fused_for(wl)),
            }
        # the verify window chosen on this device (acceptance saturates while
        # a wider window costs more rows per pass)
        line["verify_sweep"] = [verify_sweep(args.workload, frames=300),
                                verify_sweep("qwen3tts-64", frames=40)]
        # the tree-shaped window at one stream, against the chain above:
        # small trees, 15 nodes (3, 2, 1 children per node over three
        # depths) and 31 (two per node over four depths, a third root child)
        t15 = [0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 5, 6, 7, 8, 9]
        t31 = [0, 0, 0, 1, 1, 2, 2, 4, 4, 5, 5, 6, 6, 7, 7, 8, 8, 9, 9, 10, 10, 11, 11,
               12, 12, 13, 13, 14, 14, 15, 15]
        trees = tree_sweep(args.workload, ([0, 0, 1, 2], [0, 0], [0, 1, 2], t15, t31))
        for row in trees["by_tree"]:
            row["throughput_vs_chain_n4"] = row["codes_per_s"] / main_res["codes_per_s"]
        line["tree_window"] = trees
        line["baseline_configs"] = baseline_configs(line, s64, c64)
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_frames)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
