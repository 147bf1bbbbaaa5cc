"""Benchmark of the Fathom key-scan decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

Workload (default): the Qwen3-8B-shaped cache in HBM -- 36 layers x 8 KV heads = 288
(layer, KV head) pairs, 4 queries per KV head, d = 128, n = 32768 tokens, budget
B = 92 bits per token per KV head, k = 512 winners per query.  One step is one pass of
the whole hot path over all 288 heads in a single fathom_step call: plan, scan, top-k
and sparse attention.  Inputs are seeded synthetic caches (keys s_c N(0,1) with
log-uniform s_c in [0.1, 10], queries N(0,1), V N(0,1) in bf16), resident in HBM before
timing starts.  Before timing, sampled heads are checked against the CPU oracle.

Prints ONE JSON line: value = keys ranked per second over the whole step (Gkeys/s);
roofline = the step's longest kernel (the filtering scan or the attention), its
algorithmic bytes per launch / its mean launch time over a pass of K more steps timed
phase by phase (fathom_step_timed: events on the launch stream between the kernels),
against 8 TB/s; roofline_full_scan = the same for the scan in its full-score form
(fathom_scan, planes read + every fp32 score written), timed alone with cold caches;
cpu_baseline = the oracle on the host cores over a bounded sample of heads.
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

METRIC = "scan Gkeys/s + % of HBM / PCIe roofline; 1M-token decode-step ms"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3_8b_32k_hbm")
    ap.add_argument("--budget", type=int, default=92)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--kernel", default=None,
                    choices=["plan", "scan_prepare", "scan", "topk", "attn", "scan_fixed136",
                             "scan_extract", "scan_topk", "scan_nibble", "scan_b512",
                             "step_1m_host", "step_1m_hbm", "scan_grouped"],
                    help="set up the workload, time only this kernel (for profiler runs)")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--no-host", action="store_true",
                    help="skip the host-resident 1M-token single-layer step")
    ap.add_argument("--host-only", action="store_true",
                    help="run only the host-resident lines (1M-token single-layer step, "
                         "link sweep, full-model host-resident scans)")
    ap.add_argument("--no-host-models", action="store_true",
                    help="skip the full-model host-resident scans (n = 256k and 1M)")
    ap.add_argument("--no-accuracy", action="store_true",
                    help="skip the synthetic accuracy-per-byte sweep")
    ap.add_argument("--no-grouped", action="store_true",
                    help="skip the grouped-store lines (build, append, scan)")
    ap.add_argument("--accuracy-only", action="store_true",
                    help="run only the synthetic accuracy-per-byte sweep")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the per-layer decode passes (36 sequential 8-head steps) "
                         "and print their line (for profiler runs)")
    ap.add_argument("--calibrate", action="store_true",
                    help="with --kernel: also run a 1 GiB streaming read and a 256 MiB "
                         "copy, whose byte counts scale the profiler's HBM counters")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; "
                          f"--gpus {args.gpus} is not supported"}))
        sys.exit(2)

    import torch
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth

    if args.host_only:
        print(json.dumps(host_lines(args)), flush=True)
        return
    if args.accuracy_only:
        print(json.dumps(accuracy_sweep(args)), flush=True)
        return

    if args.kernel in ("step_1m_host", "step_1m_hbm"):
        print(json.dumps(step_1m_kernel(args)), flush=True)
        return
    if args.kernel == "scan_grouped":
        print(json.dumps(grouped_kernel(args)), flush=True)
        return

    cfg = synth.CONFIGS[args.config]
    H, G, n, k, B = cfg.H, cfg.G, cfg.n, cfg.k, args.budget
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sm_scale = float(np.float32(1.0 / np.sqrt(128)))

    # ---------------- inputs, resident in HBM ----------------
    t0 = time.time()
    heads = list(range(H))
    st = F.Store.empty(H, n, dev)
    K = torch.empty((H, n, 128), dtype=torch.bfloat16, device=dev)
    qws = torch.empty(F.workspace_size(F.OP_QUANTIZE, 32, 1, n, 1), dtype=torch.uint8,
                      device=dev)
    sample_heads = sorted({0, H // 2, H - 1})
    sample_keys = {}
    for h0 in range(0, H, 32):
        h1 = min(H, h0 + 32)
        keys = synth.keys_torch(args.seed, cfg.cfg_id, range(h0, h1), n, dev)
        F.fathom_quantize_store(keys, st.view_heads(h0, h1), ws=qws)
        K[h0:h1].copy_(keys)
        for h in sample_heads:
            if h0 <= h < h1:
                sample_keys[h] = keys[h - h0].cpu().numpy()
        del keys
    V = synth.values_torch(args.seed, cfg.cfg_id, heads, n, dev)
    q_np = synth.queries_np(args.seed, cfg.cfg_id, heads, G)
    q = torch.from_numpy(q_np).to(dev)
    ws = F.step_workspace(st, G, k, dev)
    depth = torch.empty((H, 128), dtype=torch.uint8, device=dev)
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    idx = torch.empty((H, G, k), dtype=torch.int32, device=dev)
    out = torch.empty((H, G, 128), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s: H={H} G={G} n={n} B={B} k={k}")

    if args.decode_only:
        per_layer, _, _ = decode_per_layer(F, st, q, K, V, B, k, sm_scale, dev, stream,
                                           passes=max(5, min(args.steps, 20)), layers=H // 8)
        print(json.dumps({"decode_per_layer": per_layer, "config": cfg.name,
                          "budget_bits": B}), flush=True)
        return

    if args.kernel:
        kern = kernel_times(F, st, q, K, V, B, k, sm_scale, depth, scores, idx, out, dev,
                            stream, reps=args.reps, only=args.kernel)
        if args.calibrate:
            flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            sink = torch.zeros(2, dtype=torch.int64, device=dev)
            a = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            for _ in range(3):
                F.fathom_stream_read(flush, flush.numel(), sink)
                b.copy_(a)
            torch.cuda.synchronize()
        print(json.dumps({"kernel": args.kernel, "reps": args.reps,
                          "ms": round(kern[args.kernel + "_ms"], 4),
                          "config": cfg.name, "budget_bits": B}), flush=True)
        return

    # ---------------- bit-exact checks before timing ----------------
    F.fathom_step(st, q, K, V, B, k, sm_scale, out=out, depth_out=depth, scores_out=scores,
                  idx_out=idx, ws=ws)
    torch.cuda.synchronize()
    parity = check_sample(st, q_np, K, V, depth, scores, idx, out, sample_keys, B, k,
                          sm_scale)
    # the timed step runs the fused scan -> select: its winners and output must be those
    # of the full scan + top-k just checked, for every head
    idx_f = torch.empty_like(idx)
    out_f = torch.empty_like(out)
    F.fathom_step(st, q, K, V, B, k, sm_scale, out=out_f, idx_out=idx_f, ws=ws)
    torch.cuda.synchronize()
    parity["fused_equals_full"] = bool(torch.equal(idx_f, idx) and torch.equal(out_f, out))
    parity["ok"] = bool(parity["ok"] and parity["fused_equals_full"])
    kept = ws[:H * 4096].view(torch.int32).view(H, 1024)[:, 28:28 + G].float()
    parity["kept_per_row_mean"] = round(float(kept.mean()), 1)
    parity["kept_per_row_max"] = int(kept.max())
    log(f"[bench] parity on heads {sample_heads}: {parity}")

    # ---------------- timed region: K whole steps ----------------
    for _ in range(args.warmup):
        F.fathom_step(st, q, K, V, B, k, sm_scale, out=out, ws=ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        F.fathom_step(st, q, K, V, B, k, sm_scale, out=out, ws=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = H * n / (ms_per_step * 1e-3) / 1e9
    # per-step GPU times of 30 more steps, each bracketed by its own events
    per_step = []
    for _ in range(30):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        F.fathom_step(st, q, K, V, B, k, sm_scale, out=out, ws=ws)
        b.record(stream)
        b.synchronize()
        per_step.append(a.elapsed_time(b))
    pct = {"median": round(float(np.median(per_step)), 4),
           "p10": round(float(np.percentile(per_step, 10)), 4),
           "p90": round(float(np.percentile(per_step, 90)), 4), "n": len(per_step)}
    log(f"[bench] step {ms_per_step:.3f} ms (GPU time), wall {wall / args.steps * 1e3:.3f} ms"
        f" -> {value:.1f} Gkeys/s")
    # each kernel of the step, live: K more steps through fathom_step_timed, whose events
    # on the launch stream bracket the step's phases
    phases = step_phases(F, st, q, K, V, B, k, sm_scale, out, ws, stream, args.steps)
    kept_total = float(ws[:H * 4096].view(torch.int32).view(H, 1024)[:, 28:28 + G].sum())
    log(f"[bench] phases over {args.steps} steps (ms): {phases}")

    # ---------------- the decode step layer by layer (one sequence, one token) --------
    per_layer = None
    if H % 8 == 0 and H >= 8:
        per_layer, out_layers, idx_layers = decode_per_layer(
            F, st, q, K, V, B, k, sm_scale, dev, stream, passes=max(5, min(args.steps, 20)),
            layers=H // 8)
        # the same winners as the 288-head call; the attention of a layer merges its
        # softmax partials in another order (1024-thread workgroups), so its bf16 outputs
        # may differ from the batched step's by rounding
        F.fathom_step(st, q, K, V, B, k, sm_scale, out=out, idx_out=idx, ws=ws)
        torch.cuda.synchronize()
        per_layer["winners_equal_batched_step"] = bool(torch.equal(idx, idx_layers))
        per_layer["outputs_max_abs_diff_vs_batched_step"] = float(
            (out.float() - out_layers.float()).abs().max())
        log(f"[bench] per-layer decode: {per_layer}")
    by_heads = step_by_heads(F, st, q, K, V, B, k, sm_scale, dev, stream)
    log(f"[bench] step by KV heads: {by_heads}")

    # ---------------- per-kernel times (cold caches between launches) ----------------
    kern = kernel_times(F, st, q, K, V, B, k, sm_scale, depth, scores, idx, out, dev,
                        stream, reps=max(10, min(args.steps, 30)))
    # A scan's algorithmic bytes are the planes it reads, B/8 bytes per key; what it
    # writes (fp32 scores, or candidate records and kept masks) is the implementation's
    # and is reported beside them, with the fraction it would give if counted.
    plane_bytes = B / 8 * n * H
    score_bytes = 4 * G * n * H
    scan_ms = kern["scan_ms"]
    achieved = plane_bytes / (scan_ms * 1e-3) / 1e9
    roofline_full = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("scan_full"), "kernel": "k_scan_main<1,false,false>",
                     "algorithmic_bytes_per_launch": int(plane_bytes),
                     "written_bytes_per_launch": int(score_bytes),
                     "frac_counting_writes": round((plane_bytes + score_bytes) / (scan_ms * 1e-3)
                                                   / 1e9 / HBM_PEAK_GBS, 4),
                     "timing": "fathom_scan alone, cold caches, mean of its own timed launches"}
    # the specified design's scan: bit extraction on the vector ALUs, no matrix cores
    ex_ms = kern.get("scan_extract_ms")
    roofline_extract = None
    if ex_ms:
        gbs = plane_bytes / (ex_ms * 1e-3) / 1e9
        roofline_extract = {"bound": "alu", "achieved_hbm_GBps": round(gbs, 1),
                            "hbm_peak": HBM_PEAK_GBS, "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                            "kernel": "k_scan_extract<4>", "ms_per_launch": round(ex_ms, 4),
                            "algorithmic_bytes_per_launch": int(plane_bytes),
                            "valu": load_counters("scan_extract"),
                            "timing": "fathom_scan_extract alone, cold caches"}
    # the step's own kernels, timed live in the phase pass: the scan (filtering form) and
    # the attention; the roofline is the longer one's
    W = (n + 31) // 32
    live = {
        "scan": ("k_scan_main<1,false,true>", "scan_filter", plane_bytes),
        "attention": ("k_sparse_attn", "attn", H * G * (k * (2 * 128 * 2 + 4) + 128 * 4 + 128 * 2)),
    }
    phase_rooflines = {}
    for name, (kname, tkey, nbytes) in live.items():
        gbs = nbytes / (phases[name] * 1e-3) / 1e9
        phase_rooflines[name] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                 "traffic": load_traffic(tkey), "kernel": kname,
                                 "algorithmic_bytes_per_launch": int(nbytes),
                                 "ms_per_launch": phases[name]}
    # the filtering scan's own writes: 8-byte candidate records and one mask word per
    # 32 tokens of each row
    fw = 8 * kept_total + 4 * W * G * H
    phase_rooflines["scan"]["written_bytes_per_launch"] = int(fw)
    phase_rooflines["scan"]["frac_counting_writes"] = round(
        (plane_bytes + fw) / (phases["scan"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    dominant = max(live, key=lambda nm: phases[nm])
    roofline = dict(phase_rooflines[dominant])
    roofline["timing"] = (f"the step's longest kernel ({dominant}), mean over the "
                          f"{args.steps} steps of the phase pass, events on the launch stream")

    # ---------------- CPU baseline: the oracle on a bounded sample ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args, st, q_np, K, V, B, k, sm_scale, sample_keys)

    host = None
    acc = None
    del K, V, st, ws, scores
    torch.cuda.empty_cache()
    grouped = None if args.no_grouped else grouped_lines(args, kern)
    if not args.no_accuracy:
        acc = accuracy_sweep(args)
    if not args.no_host:
        host = host_lines(args)

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "Gkeys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8+fp32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "kv_heads_x_layers": H, "queries_per_kv_head": G,
                   "tokens": n, "d": 128, "budget_bits": B, "k": k, "residency": "hbm",
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "roofline_full_scan": roofline_full,
        "roofline_scan_extract": roofline_extract,
        "step_is": "one fathom_step over all 36 x 8 (layer, KV head) pairs: the batched "
                   "form (36 sequences x 1 layer), not one sequence's token; per-layer "
                   "sequential decode is under decode_per_layer",
        "decode_per_layer": per_layer,
        "step_by_kv_heads": by_heads,
        "step_phases_ms": phases,
        "step_phase_rooflines": phase_rooflines,
        "cpu_baseline": cpu,
        "kernels_ms": {kk: round(v, 4) for kk, v in kern.items()},
        "scan_gkeys_per_s": round(H * n / (scan_ms * 1e-3) / 1e9, 1),
        "bytes_per_step": {"planes": int(plane_bytes),
                           "candidate_records_written": int(8 * H * G * parity["kept_per_row_mean"]),
                           "kept_masks_written": int(H * G * ((n + 31) // 32) * 4),
                           "scores_written_by_full_scan": int(score_bytes),
                           "winner_rows": int(H * G * k * 512)},
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "step_ms_single_launch": pct,
        "parity_before_timing": parity,
        "decode_1m": one_m_summary(host, per_layer),
        "host_resident": host,
        "accuracy_per_byte": acc,
        "grouped_store": grouped,
    }
    print(json.dumps(result), flush=True)


def one_m_summary(host, per_layer):
    """The metric's "1M-token decode-step ms", lifted out of the host-resident lines: the
    one-layer step at n = 1M (store and K/V rows in pinned host memory, and mirrored in
    HBM), its fraction of the link bound (plane bytes + winner rows over the measured
    link rate L), the full-model scan + top-k at 1M, and the oracle's time."""
    if not host or not isinstance(host.get("layer_1m_step"), dict):
        return None
    ls = host["layer_1m_step"]
    if "step_ms_host" not in ls:
        return None
    m = host.get("qwen3_8b_1m_host") or {}
    f92 = (m.get("budgets") or {}).get("92") or {}
    f136 = (m.get("budgets") or {}).get("fixed136") or {}
    key = "step_ms_plan_fused_scan_topk"
    cpu = ls.get("cpu_baseline") or {}
    return {
        "layer_step_ms_host": ls["step_ms_host"], "layer_step_ms_hbm": ls["step_ms_hbm"],
        "layer_step_frac_of_link_bound": ls.get("step_frac_of_link_bound"),
        "layer_scan_frac_of_link": ls.get("scan_frac_of_link"),
        "L_GBps": ls.get("L_GBps"),
        "model_scan_topk_ms_host_B92": f92.get(key),
        "model_scan_topk_ms_host_fixed136": f136.get(key),
        "model_decode_ms_host_36_layer_steps_extrapolated":
            round(36 * ls["step_ms_host"], 2),
        "model_decode_ms_hbm_36_layer_steps_extrapolated":
            round(36 * ls["step_ms_hbm"], 2),
        "oracle_layer_step_ms_extrapolated": cpu.get("layer_step_ms_extrapolated"),
        "oracle_model_step_ms_extrapolated": cpu.get("model_step_ms_extrapolated"),
        "oracle_cores": cpu.get("cores"),
    }


def check_sample(st, q_np, K, V, depth, scores, idx, out, sample_keys, B, k, sm):
    """Oracle checks on sampled heads of the full-size step (planes, plan exact;
    scores to 1e-5 of the row maximum; top-k exact on the GPU scores; attention)."""
    import torch

    import oracle
    res = {"heads": sorted(sample_keys), "planes": True, "plan": True, "topk": True}
    worst, aerr = 0.0, 0.0
    for h, keys in sample_keys.items():
        s, z, codes = oracle.quantize(keys)
        ref_planes = oracle.pack_planes(codes)
        if not np.array_equal(st.planes[h].cpu().numpy().view(np.uint32)[..., :ref_planes.shape[-1]],
                              ref_planes):
            res["planes"] = False
        var = oracle.channel_var(codes, s)
        ref_depth = oracle.plan(q_np[h], var, B)
        if not np.array_equal(depth[h].cpu().numpy(), ref_depth):
            res["plan"] = False
        ref = oracle.scores(codes, s, z, ref_depth, q_np[h])
        got = scores[h].cpu().numpy()
        worst = max(worst, float((np.abs(got - ref).max(axis=1) /
                                  np.abs(ref).max(axis=1)).max()))
        gi = idx[h].cpu().numpy()
        if not np.array_equal(gi, oracle.topk(got, k)):
            res["topk"] = False
        Kh = K[h].cpu().view(torch.int16).numpy().view(np.uint16)[None]
        Vh = V[h].cpu().view(torch.int16).numpy().view(np.uint16)[None]
        att = oracle.attention(q_np[h][None], Kh, Vh, gi[None], sm)
        aerr = max(aerr, float(np.abs(out[h].float().cpu().numpy() - att[0]).max()))
    res["score_rel_err"] = worst
    res["attn_abs_err"] = aerr
    res["ok"] = bool(res["planes"] and res["plan"] and res["topk"] and worst <= 1e-5
                     and aerr <= 2e-2)
    return res


def kernel_times(F, st, q, K, V, B, k, sm, depth, scores, idx, out, dev, stream, reps,
                 only=None):
    """Mean duration of each kernel of the step, timed with events on the launch stream,
    with a 1 GiB streaming read between launches so that every launch starts with cold
    caches (the 256 MB last-level cache would otherwise hold part of the planes)."""
    import torch
    H, G = q.shape[0], q.shape[1]
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    scan_ws = F.scan_workspace(st, G, dev)
    F.fathom_plan(st, q, B, depth=depth)
    F.fathom_scan_prepare(st, q, depth, scan_ws)
    F.fathom_scan_prepared(st, G, scores, scan_ws)
    F.fathom_topk(scores, k, idx=idx)
    stk_ws = F.scan_topk_workspace(st, G, k, dev)
    idx2 = torch.empty_like(idx)
    nib = F.fathom_pack_nibbles(st)  # the ordinary 4-bit layout, 64 B per token
    calls = {
        "plan_ms": lambda: F.fathom_plan(st, q, B, depth=depth),
        "scan_prepare_ms": lambda: F.fathom_scan_prepare(st, q, depth, scan_ws),
        "scan_ms": lambda: F.fathom_scan_prepared(st, G, scores, scan_ws),
        "topk_ms": lambda: F.fathom_topk(scores, k, idx=idx),
        # the fused form: prepare with thresholds, filtering scan, select of candidates
        "scan_topk_ms": lambda: F.fathom_scan_topk(st, q, depth, k, idx=idx2, ws=stk_ws),
        "attn_ms": lambda: F.fathom_sparse_attn(q, K, V, idx, sm, out=out),
        # comparator: the same scores by per-bit extraction on the integer units
        "scan_extract_ms": lambda: F.fathom_scan_extract(st, q, depth, scores=scores),
        # comparator: the plain 4-bit scan over the ordinary layout (every channel whole)
        "scan_nibble_ms": lambda: F.fathom_scan_nibble(nib, st.scale, st.zero, q,
                                                        scores=scores),
    }
    res = {}

    def timed(fn):
        tot = 0.0
        for _ in range(reps):
            F.fathom_stream_read(flush, flush.numel(), sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            tot += a.elapsed_time(b)
        return tot / reps

    if only == "scan_b512":
        full = torch.full((H, 128), 4, dtype=torch.uint8, device=dev)
        F.fathom_scan_prepare(st, q, full, scan_ws)
        return {"scan_b512_ms": timed(lambda: F.fathom_scan_prepared(st, G, scores, scan_ws))}
    if only == "scan_fixed136":
        fixed = F.fathom_plan_fixed(st, 34)
        F.fathom_scan_prepare(st, q, fixed, scan_ws)
        return {"scan_fixed136_ms": timed(lambda: F.fathom_scan_prepared(st, G, scores,
                                                                          scan_ws))}
    if only is not None:
        fn = calls[only + "_ms"]
        fn()
        return {only + "_ms": timed(fn)}
    for name, fn in calls.items():
        fn()
        res[name] = timed(fn)
    # the 136-bit fixed-depth comparator through the same store and kernel
    fixed = F.fathom_plan_fixed(st, 34)
    F.fathom_scan_prepare(st, q, fixed, scan_ws)
    res["scan_fixed136_ms"] = timed(lambda: F.fathom_scan_prepared(st, G, scores, scan_ws))
    # every plane of every channel: the same numbers the nibble scan computes
    full = torch.full((H, 128), 4, dtype=torch.uint8, device=dev)
    F.fathom_scan_prepare(st, q, full, scan_ws)
    res["scan_b512_ms"] = timed(lambda: F.fathom_scan_prepared(st, G, scores, scan_ws))
    # HBM streaming-read rate of this device (1 GiB, warm launch) for context
    F.fathom_stream_read(flush, flush.numel(), sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        F.fathom_stream_read(flush, flush.numel(), sink)
    b.record(stream)
    b.synchronize()
    res["hbm_stream_read_GBps"] = 5 * flush.numel() / (a.elapsed_time(b) * 1e-3) / 1e9
    del flush
    return res


TRAFFIC_FILES = {  # kernel -> (counter summary under profiles/, the sources it was taken on)
    "scan_full": ("scan_traffic.json", ("scan.hip",)),
    "scan_filter": ("scan_filter_traffic.json", ("scan.hip",)),
    "attn": ("attn_traffic.json", ("attn.hip", "attn_device.h")),
    "scan_extract": ("scan_extract_counters.json", ("scan_extract.hip",)),
}


def sources_sha256(names):
    """sha256 of the named sources under bit_plane_kv_amd/csrc, concatenated in order (one
    file: that file's own sha256)."""
    import hashlib
    h = hashlib.sha256()
    for nm in names:
        h.update(open(os.path.join(ROOT, "bit_plane_kv_amd", "csrc", nm), "rb").read())
    return h.hexdigest()


def load_counters(kernel):
    """The instruction counters of a kernel from its committed rocprofv3 summary (a JSON
    object), if the summary was taken on the current source of that kernel; else None."""
    name, srcs = TRAFFIC_FILES[kernel]
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("source_sha256") != sources_sha256(srcs):
            return None
        return rec.get("counters")
    except Exception:
        return None


def load_traffic(kernel):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter summary, if
    the summary was taken on the current source of that kernel; else None."""
    name, srcs = TRAFFIC_FILES[kernel]
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("source_sha256") != sources_sha256(srcs):
            return None
        return rec.get("traffic_bytes_per_launch")
    except Exception:
        return None


PHASES = ("plan_prepare", "scan", "select", "attention")


def step_phases(F, st, q, K, V, B, k, sm, out, ws, stream, steps):
    """Mean GPU time of each phase of the step over `steps` steps launched back to back
    through fathom_step_timed (events recorded on the launch stream between kernels)."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(F.STEP_PHASES + 1)]
           for _ in range(steps)]
    for e in evs:
        F.fathom_step_timed(st, q, K, V, B, k, sm, e, out=out, ws=ws, stream=stream)
    torch.cuda.synchronize()
    res = {}
    for i, name in enumerate(PHASES):
        res[name] = round(float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])), 4)
    res["step"] = round(float(np.mean([e[0].elapsed_time(e[-1]) for e in evs])), 4)
    return res


def step_by_heads(F, st, q, K, V, B, k, sm, dev, stream, reps=15,
                  sizes=(8, 16, 32, 64, 128, 288)):
    """One fathom_step over the first h KV heads of the cache, for several h: the shape the
    library picks changes with the row count (h x G query rows), and this line shows the
    step's GPU time across those shapes.  Each step runs after a 1 GiB streaming read
    (cold last-level cache), bracketed by events on the launch stream; median of `reps`."""
    import torch
    G = q.shape[1]
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    n = st.n_tokens
    res = []
    for h in [x for x in sizes if x <= st.n_heads]:
        sv = st.view_heads(0, h)
        ws = F.step_workspace(sv, G, k, dev)
        out = torch.empty((h, G, 128), dtype=torch.bfloat16, device=dev)
        times = []
        for r in range(reps + 2):
            F.fathom_stream_read(flush, flush.numel(), sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            F.fathom_step(sv, q[:h], K[:h], V[:h], B, k, sm, out=out, ws=ws)
            b.record(stream)
            b.synchronize()
            if r >= 2:
                times.append(a.elapsed_time(b))
        ms = float(np.median(times))
        res.append({"kv_heads": h, "query_rows": h * G, "ms": round(ms, 4),
                    "gkeys_per_s": round(h * n / (ms * 1e-3) / 1e9, 2)})
        del ws, out
    del flush
    return res


def decode_per_layer(F, st, q, K, V, B, k, sm, dev, stream, passes, layers=36, per_layer=8):
    """A real decode step's shape: the model's layers one after another, each a
    fathom_step over its 8 KV heads (layer l+1's queries would depend on layer l's
    output, so layers cannot be batched), on one stream, with the 256 MB last-level
    cache flushed (a 1 GiB streaming read) before every pass over the layers.

    Timed three ways: (a) eager: the layers' fathom_step calls launched back to back,
    GPU time between events around the pass (host launch cost included if the GPU
    waits for it; host time per layer reported beside it); (b) graph: the same pass
    captured once as a HIP graph and replayed, GPU time per replay, each replay's
    outputs checked against the eager pass; (c) phases: fathom_step_timed per layer
    (events between kernels), mean per phase over all layers and passes."""
    import torch
    G = q.shape[1]
    ws = F.step_workspace(st.view_heads(0, per_layer), G, k, dev)
    views = [(st.view_heads(per_layer * l, per_layer * (l + 1)), q[per_layer * l:per_layer * (l + 1)],
              K[per_layer * l:per_layer * (l + 1)], V[per_layer * l:per_layer * (l + 1)])
             for l in range(layers)]
    out = torch.empty((layers * per_layer, G, 128), dtype=torch.bfloat16, device=dev)
    outs = [out[per_layer * l:per_layer * (l + 1)] for l in range(layers)]
    idx = torch.empty((layers * per_layer, G, k), dtype=torch.int32, device=dev)
    idxs = [idx[per_layer * l:per_layer * (l + 1)] for l in range(layers)]
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)

    def one_pass():
        for (sv, qv, Kv, Vv), ov, iv in zip(views, outs, idxs):
            F.fathom_step(sv, qv, Kv, Vv, B, k, sm, out=ov, idx_out=iv, ws=ws)

    one_pass()
    torch.cuda.synchronize()
    ref = out.clone()
    eager, host = [], []
    for _ in range(passes):
        F.fathom_stream_read(flush, flush.numel(), sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        t0 = time.perf_counter()
        one_pass()
        host.append((time.perf_counter() - t0) * 1e6 / layers)
        b.record(stream)
        b.synchronize()
        eager.append(a.elapsed_time(b))
    same_eager = bool(torch.equal(out, ref))
    # the pass as a graph (no memset nodes: the step's kernels clear what they need)
    replays, same_graph, graph_error = [], True, None
    try:
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            one_pass()  # warm on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=gs):
                one_pass()
        torch.cuda.synchronize()
        for _ in range(passes):
            out.zero_()
            F.fathom_stream_read(flush, flush.numel(), sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graph.replay()
            b.record(stream)
            b.synchronize()
            replays.append(a.elapsed_time(b))
            same_graph = same_graph and bool(torch.equal(out, ref))
        del graph
    except Exception as e:  # report, keep the eager figures
        graph_error = f"{type(e).__name__}: {e}"
        torch.cuda.synchronize()
    # phases, per layer
    ph = {name: [] for name in PHASES}
    for _ in range(passes):
        F.fathom_stream_read(flush, flush.numel(), sink)
        evs = []
        for (sv, qv, Kv, Vv), ov in zip(views, outs):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(F.STEP_PHASES + 1)]
            F.fathom_step_timed(sv, qv, Kv, Vv, B, k, sm, e, out=ov, ws=ws, stream=stream)
            evs.append(e)
        torch.cuda.synchronize()
        for e in evs:
            for i, name in enumerate(PHASES):
                ph[name].append(e[i].elapsed_time(e[i + 1]))
    del flush
    med = lambda v: round(float(np.median(v)), 4)
    res = {"layers": layers, "kv_heads_per_layer": per_layer, "passes": passes,
           "timing": "GPU time of one pass over the layers (one token of one sequence), "
                     "last-level cache flushed before each pass",
           "ms_per_token_graph": med(replays) if replays else None,
           "ms_per_token_eager": med(eager),
           "us_per_layer_graph": (round(float(np.median(replays)) * 1e3 / layers, 2)
                                  if replays else None),
           "graph_error": graph_error,
           "host_us_per_layer_call": round(float(np.median(host)), 1),
           "phase_us_per_layer": {nm: round(float(np.mean(v)) * 1e3, 2) for nm, v in ph.items()},
           "winners_equal_batched_step": None, "eager_repeatable": same_eager,
           "graph_replays_equal_eager": same_graph}
    return res, ref, idx.clone()


def timed_ms(fn, stream, reps, flush=None, sink=None):
    """Mean GPU time of fn over reps launches (events on the launch stream); with flush,
    a 1 GiB streaming read precedes every launch so it starts with cold caches."""
    import torch
    from bit_plane_kv_amd import fathom as F
    fn()
    tot = 0.0
    for _ in range(reps):
        if flush is not None:
            F.fathom_stream_read(flush, flush.numel(), sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        tot += a.elapsed_time(b)
    return tot / reps


def link_rate(dev, stream, nbytes=1 << 30):
    """Host-to-GPU link rate L = max(DMA copy from a pinned buffer, zero-copy streaming
    read of the same pinned buffer by a kernel), GB/s."""
    import torch
    from bit_plane_kv_amd import fathom as F
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    h.fill_(1)
    d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    dma = nbytes / (timed_ms(lambda: d.copy_(h, non_blocking=True), stream, 3) * 1e-3) / 1e9
    zc = nbytes / (timed_ms(lambda: F.fathom_stream_read(h, nbytes, sink), stream, 3) * 1e-3) / 1e9
    del h, d
    return {"dma_h2d_GBps": round(dma, 2), "zero_copy_read_GBps": round(zc, 2),
            "L_GBps": round(max(dma, zc), 2)}


def grouped_lines(args, kern):
    """The grouped store (fp16 scale and zero per 128-token group: 68 B per token per KV
    head, the index size of the blog's "Where this does not work") on the bench workload:
    its build, a decode-time append of one token to every head (the last group
    re-quantized and every variance recomputed), its scan at the bench budget, with
    one sampled head checked against the oracle, and its decode step (plan, scan of every
    score, top-k, attention: fathom_step_grouped) over all heads and over one layer's 8."""
    import torch
    import oracle
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    cfg = synth.CONFIGS[args.config]
    H, G, n, B = cfg.H, cfg.G, cfg.n, args.budget
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    keys = synth.keys_torch(args.seed, cfg.cfg_id, range(H), n, dev)
    q = torch.from_numpy(synth.queries_np(args.seed, cfg.cfg_id, range(H), G)).to(dev)
    ng = (n + 127) // 128
    gs = F.GStore.empty(H, n + 128, dev, n=n - 1)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    build_ms = timed_ms(lambda: F.fathom_quantize_groups(keys[:, :n - 1], gs, 0, ng),
                        stream, 3, flush, sink)
    gs.n_tokens = n   # append token n-1: its group is re-quantized
    g = (n - 1) // 128
    append_ms = timed_ms(lambda: F.fathom_quantize_groups(keys[:, 128 * g:n], gs, g, g + 1),
                         stream, 10, flush, sink)
    depth = F.fathom_plan_grouped(gs, q, B)
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    scan_ms = timed_ms(lambda: F.fathom_scan_grouped(gs, q, depth, scores=scores), stream, 10,
                       flush, sink)
    torch.cuda.synchronize()
    h = H // 2
    kh = keys[h:h + 1].cpu().numpy()
    s16, z16, codes = oracle.quantize_grouped(kh)
    ref_depth = oracle.plan(q[h:h + 1].cpu().numpy(), oracle.var_grouped(codes, s16, z16), B)
    ref = oracle.scores_grouped(codes, s16, z16, ref_depth, q[h:h + 1].cpu().numpy())
    got = scores[h:h + 1].cpu().numpy()
    rel = float((np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max())
    # the decode step over the grouped store: all heads at once, then one layer (8 heads)
    k, sm = cfg.k, float(np.float32(1.0 / np.sqrt(128)))
    Kb = keys.to(torch.bfloat16)
    V = synth.values_torch(args.seed, cfg.cfg_id, list(range(H)), n, dev)
    out = torch.empty((H, G, 128), dtype=torch.bfloat16, device=dev)
    ws = F.step_grouped_workspace(gs, G, k, dev)
    step_ms = timed_ms(lambda: F.fathom_step_grouped(gs, q, Kb, V, B, k, sm, out=out, ws=ws),
                       stream, 10, flush, sink)
    hl = min(H, 8)
    gl = F.GStore(gs.planes[:hl], gs.scale16[:hl], gs.zero16[:hl], gs.sums[:hl], gs.var[:hl],
                  gs.prefix[:hl], gs.prefix_groups[:hl], n)
    wl = F.step_grouped_workspace(gl, G, k, dev)
    layer_ms = timed_ms(lambda: F.fathom_step_grouped(gl, q[:hl], Kb[:hl], V[:hl], B, k, sm,
                                                      out=out[:hl], ws=wl), stream, 10, flush,
                        sink)
    # its winners for the sampled head: the oracle's top-k of the scores it computed
    sh = F.GStore(gs.planes[h:h + 1], gs.scale16[h:h + 1], gs.zero16[h:h + 1],
                  gs.sums[h:h + 1], gs.var[h:h + 1], gs.prefix[h:h + 1],
                  gs.prefix_groups[h:h + 1], n)
    s_h = torch.empty((1, G, n), dtype=torch.float32, device=dev)
    i_h = torch.empty((1, G, k), dtype=torch.int32, device=dev)
    F.fathom_step_grouped(sh, q[h:h + 1], Kb[h:h + 1], V[h:h + 1], B, k, sm, scores_out=s_h,
                          idx_out=i_h)
    torch.cuda.synchronize()
    step_ok = bool(np.array_equal(i_h.cpu().numpy()[0],
                                  oracle.topk(s_h.cpu().numpy()[0], k)) and
                   torch.equal(s_h, scores[h:h + 1]))
    del Kb, V, out, ws, wl
    ok = bool(np.array_equal(gs.scale16[h:h + 1, :ng].cpu().numpy().view(np.uint16)
                             .transpose(0, 2, 1), s16)
              and np.array_equal(depth[h:h + 1].cpu().numpy(), ref_depth) and rel <= 1e-5)
    res = {"bytes_per_token_per_kv_head": 64 + 4, "group_tokens": 128,
           "build_ms": round(build_ms, 3), "append_one_token_ms": round(append_ms, 4),
           "scan_ms": round(scan_ms, 4),
           "scan_ms_per_channel_store_matrix_cores": round(kern["scan_ms"], 4),
           "scan_gkeys_per_s": round(H * n / (scan_ms * 1e-3) / 1e9, 1),
           "oracle_check_head": h, "score_rel_err": rel, "ok": ok,
           "decode_step": {"k": k, "ms_all_heads": round(step_ms, 4),
                           "ms_one_layer": round(layer_ms, 4), "layer_kv_heads": hl,
                           "timing": "fathom_step_grouped (plan, full scan, top-k, attention), "
                                     "cold caches, mean of 10 launches",
                           "winners_check_head": h, "winners_ok": step_ok}}
    log(f"[bench] grouped store: build {build_ms:.2f} ms, append {append_ms * 1e3:.1f} us, "
        f"scan {scan_ms * 1e3:.1f} us (per-channel matrix-core scan "
        f"{kern['scan_ms'] * 1e3:.1f} us), check {ok}; decode step {step_ms * 1e3:.1f} us "
        f"(one layer {layer_ms * 1e3:.1f} us), winners check {step_ok}")
    del keys, gs, scores, flush
    torch.cuda.empty_cache()
    return res


def grouped_store_1m_layer(args, dev):
    """The grouped store of one 1M-token layer (8 KV heads), built on the GPU, and its
    per-query plan at the bench budget."""
    import torch
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    cfg = synth.CONFIGS["qwen3_8b_1m_layer_step"]
    H, G, n = cfg.H, cfg.G, cfg.n
    ng = (n + 127) // 128
    gs = F.GStore.empty(H, n, dev, n=n)
    keys = synth.keys_torch(args.seed, cfg.cfg_id, range(H), n, dev)
    F.fathom_quantize_groups(keys, gs, 0, ng)
    del keys
    q = torch.from_numpy(synth.queries_np(args.seed, cfg.cfg_id, range(H), G)).to(dev)
    depth = F.fathom_plan_grouped(gs, q, args.budget)
    torch.cuda.synchronize()
    return gs, q, depth, cfg


def grouped_host_line(args, L):
    """The grouped store (68 B per token per KV head) of one 1M-token layer with its
    planes, fp16 scales and fp16 zeros in pinned host memory, read by the GPU over the
    host link -- where the blog measures that index ("Where this does not work"): the
    grouped scan's GPU time from host memory and from HBM (cold caches), the bytes it
    reads over the link (the planned planes, and every channel's scale and zero of every
    group) and the fraction of the link bound those bytes give; the scores from host
    memory must equal those from HBM."""
    import torch
    from bit_plane_kv_amd import fathom as F
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    gs_d, q, depth, cfg = grouped_store_1m_layer(args, dev)
    H, G, n, B = cfg.H, cfg.G, cfg.n, args.budget
    ng = (n + 127) // 128
    planes_h = torch.empty(gs_d.planes.shape, dtype=torch.int32, pin_memory=True)
    planes_h.copy_(gs_d.planes)
    s_h = torch.empty(gs_d.scale16.shape, dtype=torch.int16, pin_memory=True)
    s_h.copy_(gs_d.scale16)
    z_h = torch.empty(gs_d.zero16.shape, dtype=torch.int16, pin_memory=True)
    z_h.copy_(gs_d.zero16)
    gs_h = F.GStore(planes_h, s_h, z_h, gs_d.sums, gs_d.var, gs_d.prefix, gs_d.prefix_groups, n)
    sc_d = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    sc_h = torch.empty_like(sc_d)
    F.fathom_scan_grouped(gs_d, q, depth, scores=sc_d)
    F.fathom_scan_grouped(gs_h, q, depth, scores=sc_h)
    torch.cuda.synchronize()
    same = bool(torch.equal(sc_d, sc_h))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    ms_d = timed_ms(lambda: F.fathom_scan_grouped(gs_d, q, depth, scores=sc_d), stream, 5,
                    flush, sink)
    ms_h = timed_ms(lambda: F.fathom_scan_grouped(gs_h, q, depth, scores=sc_h), stream, 5,
                    flush, sink)
    plane_bytes = H * B * n / 8
    sz_bytes = H * 128 * ng * 4
    link_bytes = plane_bytes + sz_bytes
    bound_ms = link_bytes / (L["L_GBps"] * 1e9) * 1e3
    res = {"workload": cfg.name, "kv_heads": H, "tokens": n, "queries_per_kv_head": G,
           "budget_bits": B, "bytes_per_token_per_kv_head": 68,
           "scan_ms_host": round(ms_h, 4), "scan_ms_hbm": round(ms_d, 4),
           "link_bytes": int(link_bytes), "plane_bytes": int(plane_bytes),
           "scale_zero_bytes": int(sz_bytes), "link_GBps": L["L_GBps"],
           "link_bound_ms": round(bound_ms, 4), "frac_of_link_bound": round(bound_ms / ms_h, 3),
           "achieved_link_GBps": round(link_bytes / (ms_h * 1e-3) / 1e9, 2),
           "host_scores_equal_hbm": same,
           "timing": "fathom_scan_grouped alone, 1 GiB streaming read before each of 5 launches"}
    log(f"[bench] grouped 1M layer scan: host {ms_h:.3f} ms, HBM {ms_d:.3f} ms, "
        f"{bound_ms / ms_h:.2f} of the link bound, equal {same}")
    del gs_d, gs_h, planes_h, s_h, z_h, sc_d, sc_h, flush
    return res


def grouped_kernel(args):
    """--kernel scan_grouped: the grouped store on the bench workload, its scan alone
    (for profiler runs)."""
    import torch
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    cfg = synth.CONFIGS[args.config]
    H, G, n, B = cfg.H, cfg.G, cfg.n, args.budget
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    ng = (n + 127) // 128
    gs = F.GStore.empty(H, n, dev, n=n)
    for h0 in range(0, H, 32):
        h1 = min(H, h0 + 32)
        keys = synth.keys_torch(args.seed, cfg.cfg_id, range(h0, h1), n, dev)
        sub = F.GStore(gs.planes[h0:h1], gs.scale16[h0:h1], gs.zero16[h0:h1], gs.sums[h0:h1],
                       gs.var[h0:h1], gs.prefix[h0:h1], gs.prefix_groups[h0:h1], n)
        F.fathom_quantize_groups(keys, sub, 0, ng)
        del keys
    q = torch.from_numpy(synth.queries_np(args.seed, cfg.cfg_id, range(H), G)).to(dev)
    depth = F.fathom_plan_grouped(gs, q, B)
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    ms = timed_ms(lambda: F.fathom_scan_grouped(gs, q, depth, scores=scores), stream,
                  args.reps, flush, sink)
    return {"kernel": "scan_grouped", "reps": args.reps, "ms": round(ms, 4),
            "config": cfg.name, "budget_bits": B}


ACC_BUDGETS = (16, 24, 32, 40, 48, 56, 64, 72, 80, 92, 104, 120, 136, 168, 200, 256, 512)


def attention_references(q, K, V, k, sm):
    """The accuracy sweep's two references, head by head on the GPU in fp64: dense
    softmax attention over all n tokens (logits q . K_i * sm on the bf16 rows, maximum
    subtracted), and the exact top-k -- the k largest fp64 logits, equal logits to the
    lower token index, ascending by index.  tests/test_gpu_accuracy.py checks both
    against the oracle's attention over every row and its fp64 top-k of its logits.
    Returns (dense fp64 [H][G][128], top int32 [H][G][k])."""
    import torch
    H, G = q.shape[0], q.shape[1]
    dense = torch.empty((H, G, 128), dtype=torch.float64, device=q.device)
    top = torch.empty((H, G, k), dtype=torch.int32, device=q.device)
    for h in range(H):
        Kd = K[h].to(torch.float64)                       # exact widening of bf16
        logits = torch.matmul(q[h].to(torch.float64), Kd.t().contiguous()) * sm
        # exp and the normalisation written out: torch's fp64 softmax on this ROCm
        # build agrees with the oracle only to ~2e-8 (an fp32-accurate exponential)
        e = torch.exp(logits - logits.max(dim=-1, keepdim=True).values)
        p = e / e.sum(dim=-1, keepdim=True)
        dense[h] = torch.matmul(p, V[h].to(torch.float64))
        # stable sort: among equal logits the lower index comes first
        order = torch.sort(logits, dim=-1, descending=True, stable=True).indices[:, :k]
        top[h] = order.sort(dim=-1).values.to(torch.int32)
        del Kd, logits, e, p, order
    return dense, top


def accuracy_rows(F, st, q, K, V, k, sm, fixed, budgets, dense, top):
    """Attention error of the per-query plan at each budget (through fathom_step), of
    the fixed-depth comparator plan `fixed` and of the exact top-k, against `dense`."""
    import torch
    H, G = q.shape[0], q.shape[1]
    dn = dense.norm(dim=-1)

    def err(out):
        e = (out.to(torch.float64) - dense).norm(dim=-1) / dn
        return {"mean": round(float(e.mean()), 5), "max": round(float(e.max()), 5)}

    r = {"fathom": {}}
    out = torch.empty((H, G, 128), dtype=torch.bfloat16, device=q.device)
    for B in budgets:
        F.fathom_step(st, q, K, V, B, k, sm, out=out)
        r["fathom"][str(B)] = err(out)
    idx = F.fathom_topk(F.fathom_scan(st, q, fixed), k)
    r["fixed136"] = err(F.fathom_sparse_attn(q, K, V, idx, sm))
    r["exact_topk"] = err(F.fathom_sparse_attn(q, K, V, top, sm))
    match = [B for B in budgets if r["fathom"][str(B)]["mean"] <= r["fixed136"]["mean"]]
    r["bits_to_match_fixed136"] = match[0] if match else None
    r["bytes_ratio_vs_fixed136"] = round(136 / match[0], 2) if match else None
    return r


def accuracy_sweep(args):
    """Attention error against budget on a synthetic cache (blog, "Accuracy per byte": the
    bits per token the per-query plan needs to match the attention error of the 136-bit
    fixed-depth scans).  Four layers of the Qwen3-8B-shaped cache (32 KV heads x 4
    queries, n = 32768, k = 512).  Error of a row = ||o - o_dense|| / ||o_dense||, o_dense =
    softmax attention over all n tokens in fp64 on the bf16 K/V rows (attention_references,
    checked against the oracle).  For every budget B the Fathom plan runs through
    fathom_step; the comparators are the 136-bit fixed-depth scan (34 channels of largest
    variance, all four planes) and the exact top-k (the k largest fp64 logits, ties to the
    lower index).  Synthetic keys and queries stand in for the pages' five models, so this
    is a proxy for their 46-74-bit finding, not a check of it."""
    import torch
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    cfg = synth.CONFIGS["qwen3_8b_32k_hbm"]
    heads = list(range(32))
    H, G, n, k = len(heads), cfg.G, cfg.n, cfg.k
    dev = torch.device("cuda:0")
    t0 = time.time()
    keys = synth.keys_torch(args.seed, cfg.cfg_id, heads, n, dev)
    st = F.Store.empty(H, n, dev)
    F.fathom_quantize_store(keys, st)
    K = keys.to(torch.bfloat16)
    del keys
    V = synth.values_torch(args.seed, cfg.cfg_id, heads, n, dev)
    sm = float(np.float32(1.0 / np.sqrt(128)))
    fixed = F.fathom_plan_fixed(st, 34)
    res = {"workload": "qwen3_8b_32k_hbm, layers 0-3 (32 KV heads x 4 queries)", "k": k,
           "error": "mean over rows of ||o - o_dense|| / ||o_dense||, o_dense in fp64"}
    regimes = {"iid_queries": synth.queries_np(args.seed, cfg.cfg_id, heads, G),
               "heavy_tailed_queries": synth.queries_heavy_np(args.seed, cfg.cfg_id, heads, G)}
    for name, q_np in regimes.items():
        q = torch.from_numpy(q_np).to(dev)
        dense, top = attention_references(q, K, V, k, sm)
        r = accuracy_rows(F, st, q, K, V, k, sm, fixed, ACC_BUDGETS, dense, top)
        res[name] = r
        log(f"[bench] accuracy ({name}): fixed-136 {r['fixed136']}, exact top-k "
            f"{r['exact_topk']}, bits to match {r['bits_to_match_fixed136']}")
        del dense, top
    log(f"[bench] accuracy sweep in {time.time() - t0:.1f}s")
    del K, V, st
    torch.cuda.empty_cache()
    return res


def host_lines(args):
    """All host-resident lines: the link rate and its run-length sweep, the 1M-token
    single-layer step, and (unless --no-host-models) the full-model scans at 256k and
    1M tokens with the store in pinned host memory."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    L = link_rate(dev, stream)
    out = {"link": L}
    try:
        out["link_run_sweep"] = link_sweep(dev, stream)
    except Exception as e:
        out["link_run_sweep"] = {"error": f"{type(e).__name__}: {e}"}
    out["layer_1m_step"] = host_resident_step(args, L)
    try:
        out["grouped_1m_layer_scan"] = grouped_host_line(args, L)
    except Exception as e:  # report, do not lose the other lines
        out["grouped_1m_layer_scan"] = {"error": f"{type(e).__name__}: {e}"}
    torch.cuda.empty_cache()
    if not args.no_host_models:
        for name in ("qwen3_8b_256k_host", "qwen3_8b_1m_host"):
            try:
                out[name] = host_model(args, name, L)
            except Exception as e:  # report, do not lose the other lines
                out[name] = {"error": f"{type(e).__name__}: {e}"}
            torch.cuda.empty_cache()
    return out


def link_sweep(dev, stream, total=1 << 28):
    """Zero-copy reads of pinned host memory in runs of 256 B .. 1 MiB (every other run
    skipped, `total` bytes read per point), and one DMA call per run for a few lengths
    (the blog's "One measurement worth carrying around"), GB/s."""
    import torch
    from bit_plane_kv_amd import fathom as F
    h = torch.empty(2 * total, dtype=torch.uint8, pin_memory=True)
    h.fill_(3)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    rows = []
    for run in [256, 1024, 4096, 16384, 65536, 262144, 1 << 20]:
        n_runs = total // run
        ms = timed_ms(lambda: F.fathom_stream_read_runs(h, run, 2 * run, n_runs, sink),
                      stream, 3)
        rows.append({"run_bytes": run, "zero_copy_GBps": round(total / (ms * 1e-3) / 1e9, 2)})
    d = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    for r in rows:
        run = r["run_bytes"]
        if run < 4096:
            continue
        calls = min(2000, total // run)
        def per_run():
            for i in range(calls):
                d[:run].copy_(h[2 * run * i:2 * run * i + run], non_blocking=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        per_run()
        torch.cuda.synchronize()
        r["dma_call_per_run_GBps_wall"] = round(calls * run / (time.perf_counter() - t0) / 1e9, 3)
    del h, d
    return rows


def host_model(args, name, L):
    """Full-model scan + top-k (36 layers x 8 KV heads x 4 queries, k = 512) with the
    bit-plane store in pinned host memory, read by the GPU over the host link: per budget
    (and for the 136-bit fixed-depth plan) the GPU time of plan + scan + top-k per step,
    the scan's plane bytes and their rate as a fraction of the link rate L, and an oracle
    check of one sampled head (plan exact, scores to 1e-5, top-k exact on the GPU
    scores)."""
    import torch

    import oracle
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    cfg = synth.CONFIGS[name]
    H, G, n, k = cfg.H, cfg.G, cfg.n, cfg.k
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    t0 = time.time()
    Wst = int(F.lib().fathom_word_stride(n))  # the library's row stride for n tokens
    planes_h = torch.empty((H, 128, 4, Wst), dtype=torch.int32, pin_memory=True)
    kw = dict(dtype=torch.float32, device=dev)
    st_h = F.Store(planes_h, torch.empty((H, 128), **kw), torch.empty((H, 128), **kw),
                   torch.empty((H, 128), **kw), n)
    batch = max(1, (8 << 30) // (n * 512))  # about 8 GiB of fp32 keys per batch
    st_b = F.Store.empty(batch, n, dev)
    for h0 in range(0, H, batch):
        h1 = min(H, h0 + batch)
        keys = synth.keys_torch(args.seed, cfg.cfg_id, range(h0, h1), n, dev)
        sv = st_b.view_heads(0, h1 - h0)
        F.fathom_quantize_store(keys, sv)
        planes_h[h0:h1].copy_(sv.planes)
        st_h.scale[h0:h1].copy_(sv.scale)
        st_h.zero[h0:h1].copy_(sv.zero)
        st_h.var[h0:h1].copy_(sv.var)
        del keys
    torch.cuda.synchronize()
    del st_b
    torch.cuda.empty_cache()
    q_np = synth.queries_np(args.seed, cfg.cfg_id, range(H), G)
    q = torch.from_numpy(q_np).to(dev)
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    idx = torch.empty((H, G, k), dtype=torch.int32, device=dev)
    depth = torch.empty((H, 128), dtype=torch.uint8, device=dev)
    sws = F.scan_workspace(st_h, G, dev)
    tneed = F.workspace_size(F.OP_TOPK, H * G, 1, n, k)
    tws = torch.empty(max(tneed, 1), dtype=torch.uint8, device=dev)
    stk_ws = F.scan_topk_workspace(st_h, G, k, dev)
    log(f"[bench] {name}: pinned store of {planes_h.numel() * 4 / 1e9:.2f} GB ready in "
        f"{time.time() - t0:.1f}s")

    def plan_for(b):
        if b == "fixed136":
            return lambda: F.fathom_plan_fixed(st_h, 34, depth=depth)
        return lambda: F.fathom_plan(st_h, q, b, depth=depth)

    res = {"workload": name, "kv_heads_x_layers": H, "queries_per_kv_head": G, "tokens": n,
           "k": k, "residency": "pinned host", "pinned_store_bytes": int(planes_h.numel() * 4),
           "L_GBps": L["L_GBps"], "budgets": {}}
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    reps = 5 if n <= 262144 else 3
    for b in list(cfg.budgets) + (["fixed136"] if name == "qwen3_8b_1m_host" or
                                   name == "qwen3_8b_256k_host" else []):
        plan = plan_for(b)
        planes_read = 136 if b == "fixed136" else b

        def step():
            plan()
            F.fathom_scan(st_h, q, depth, scores=scores, ws=sws)
            F.fathom_topk(scores, k, idx=idx, ws=tws)
        step()
        torch.cuda.synchronize()
        step_ms = timed_ms(step, stream, reps, flush, sink)

        def step_fused():
            plan()
            F.fathom_scan_topk(st_h, q, depth, k, idx=idx, ws=stk_ws)
        step_fused()
        torch.cuda.synchronize()
        fused_ms = timed_ms(step_fused, stream, reps, flush, sink)
        F.fathom_scan_prepare(st_h, q, depth, sws)
        scan_ms = timed_ms(lambda: F.fathom_scan_prepared(st_h, G, scores, sws), stream, reps,
                           flush, sink)
        topk_ms = timed_ms(lambda: F.fathom_topk(scores, k, idx=idx, ws=tws), stream, reps,
                           flush, sink)
        pb = planes_read / 8 * n * H
        gbps = pb / (scan_ms * 1e-3) / 1e9
        res["budgets"][str(b)] = {
            "step_ms_plan_scan_topk": round(step_ms, 3),
            "step_ms_plan_fused_scan_topk": round(fused_ms, 3), "scan_ms": round(scan_ms, 3),
            "topk_ms": round(topk_ms, 3), "scan_plane_bytes": int(pb),
            "scan_plane_GBps": round(gbps, 2), "scan_frac_of_link": round(gbps / L["L_GBps"], 4),
            "scan_gkeys_per_s": round(H * n / (scan_ms * 1e-3) / 1e9, 2),
            "score_bytes_in_hbm": int(4 * G * n * H)}
        log(f"[bench] {name} B={b}: step {step_ms:.2f} ms (fused {fused_ms:.2f} ms), "
            f"scan {scan_ms:.2f} ms = "
            f"{gbps:.1f} GB/s of planes ({gbps / L['L_GBps']:.0%} of L)")
    del flush
    if "fixed136" in res["budgets"] and "92" in res["budgets"]:
        r = res["budgets"]
        res["speedup_b92_vs_fixed136_fused_step"] = round(
            r["fixed136"]["step_ms_plan_fused_scan_topk"] /
            r["92"]["step_ms_plan_fused_scan_topk"], 3)
        res["speedup_b92_vs_fixed136_step"] = round(r["fixed136"]["step_ms_plan_scan_topk"] /
                                                     r["92"]["step_ms_plan_scan_topk"], 3)
    # oracle check of one sampled head at B = 92
    h = H // 2
    F.fathom_plan(st_h, q, 92, depth=depth)
    F.fathom_scan(st_h, q, depth, scores=scores, ws=sws)
    F.fathom_topk(scores, k, idx=idx, ws=tws)
    torch.cuda.synchronize()
    kh = synth.keys_torch(args.seed, cfg.cfg_id, [h], n, dev).cpu().numpy()
    sh, zh, codes = oracle.quantize(kh)
    ref_depth = oracle.plan(q_np[h][None], oracle.channel_var(codes, sh), 92)
    got = scores[h].cpu().numpy()
    ref = oracle.scores(codes, sh, zh, ref_depth, q_np[h][None])[0]
    err = float((np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())
    res["oracle_check"] = {
        "head": h, "budget_bits": 92,
        "plan": bool(np.array_equal(depth[h].cpu().numpy(), ref_depth[0])),
        "score_rel_err": err,
        "topk": bool(np.array_equal(idx[h].cpu().numpy(), oracle.topk(got, k)))}
    del planes_h, st_h, scores
    return res


def host_resident_step(args, L):
    """One layer's decode step at n = 1M (8 KV heads x 4 queries, B = 92, k = 512) with
    the bit-plane store and the bf16 K/V rows in pinned host memory (read by the GPU over
    the host link), against the same store mirrored in HBM; plus the measured link rate
    and the scan's plane-byte rate over the link."""
    import torch
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    cfg = synth.CONFIGS["qwen3_8b_1m_layer_step"]
    H, G, n, k, B = cfg.H, cfg.G, cfg.n, cfg.k, args.budget
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sm = float(np.float32(1.0 / np.sqrt(128)))
    st_d, st_h, q, K_d, V_d, K_h, V_h = layer_1m_stores(args)
    planes_h = st_h.planes
    return host_resident_step_run(args, L, cfg, st_d, st_h, q, K_d, V_d, K_h, V_h, planes_h,
                                  H, G, n, k, B, dev, stream, sm)


def step_1m_kernel(args):
    """--kernel step_1m_host / step_1m_hbm: the 1M-token layer's decode step launched
    `reps` times (cold caches before each), store and K/V rows in pinned host memory or
    in HBM, for profiler runs of its kernels."""
    import torch
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    cfg = synth.CONFIGS["qwen3_8b_1m_layer_step"]
    G, k, B = cfg.G, cfg.k, args.budget
    sm = float(np.float32(1.0 / np.sqrt(128)))
    st_d, st_h, q, K_d, V_d, K_h, V_h = layer_1m_stores(args)
    host = args.kernel == "step_1m_host"
    st, K, V = (st_h, K_h, V_h) if host else (st_d, K_d, V_d)
    ws = F.step_workspace(st_d, G, k, q.device)
    out = torch.empty((cfg.H, G, 128), dtype=torch.bfloat16, device=q.device)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=q.device)
    sink = torch.zeros(2, dtype=torch.int64, device=q.device)
    ms = timed_ms(lambda: F.fathom_step(st, q, K, V, B, k, sm, out=out, ws=ws),
                  torch.cuda.current_stream(), args.reps, flush, sink)
    return {"kernel": args.kernel, "reps": args.reps, "ms": round(ms, 4),
            "config": cfg.name, "budget_bits": B}


def layer_1m_stores(args):
    """The 1M-token layer (8 KV heads): store and bf16 K/V rows in HBM, and the same
    store planes and K/V rows copied to pinned host memory."""
    import torch
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    cfg = synth.CONFIGS["qwen3_8b_1m_layer_step"]
    H, G, n = cfg.H, cfg.G, cfg.n
    dev = torch.device("cuda:0")
    t0 = time.time()
    st_d = F.Store.empty(H, n, dev)
    K_d = torch.empty((H, n, 128), dtype=torch.bfloat16, device=dev)
    for h in range(H):
        keys = synth.keys_torch(args.seed, cfg.cfg_id, [h], n, dev)
        F.fathom_quantize_store(keys, st_d.view_heads(h, h + 1))
        K_d[h].copy_(keys[0])
        del keys
    V_d = synth.values_torch(args.seed, cfg.cfg_id, range(H), n, dev)
    q = torch.from_numpy(synth.queries_np(args.seed, cfg.cfg_id, range(H), G)).to(dev)
    planes_h = torch.empty(st_d.planes.shape, dtype=torch.int32, pin_memory=True)
    planes_h.copy_(st_d.planes)
    K_h = torch.empty(K_d.shape, dtype=torch.bfloat16, pin_memory=True)
    K_h.copy_(K_d)
    V_h = torch.empty(V_d.shape, dtype=torch.bfloat16, pin_memory=True)
    V_h.copy_(V_d)
    st_h = F.Store(planes_h, st_d.scale, st_d.zero, st_d.var, n)
    torch.cuda.synchronize()
    log(f"[bench] host-resident 1M layer ready in {time.time() - t0:.1f}s")
    return st_d, st_h, q, K_d, V_d, K_h, V_h


def host_resident_step_run(args, L, cfg, st_d, st_h, q, K_d, V_d, K_h, V_h, planes_h, H, G,
                           n, k, B, dev, stream, sm):
    import torch
    from bit_plane_kv_amd import fathom as F
    ws = F.step_workspace(st_d, G, k, dev)
    out_d = torch.empty((H, G, 128), dtype=torch.bfloat16, device=dev)
    out_h = torch.empty_like(out_d)
    idx_d = torch.empty((H, G, k), dtype=torch.int32, device=dev)
    idx_h = torch.empty_like(idx_d)
    F.fathom_step(st_d, q, K_d, V_d, B, k, sm, out=out_d, idx_out=idx_d, ws=ws)
    F.fathom_step(st_h, q, K_h, V_h, B, k, sm, out=out_h, idx_out=idx_h, ws=ws)
    torch.cuda.synchronize()
    same = bool(torch.equal(idx_d, idx_h) and torch.equal(out_d, out_h))

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2, dtype=torch.int64, device=dev)
    step_h = timed_ms(lambda: F.fathom_step(st_h, q, K_h, V_h, B, k, sm, out=out_h, ws=ws),
                      stream, 10, flush, sink)
    step_d = timed_ms(lambda: F.fathom_step(st_d, q, K_d, V_d, B, k, sm, out=out_d, ws=ws),
                      stream, 10, flush, sink)
    depth = F.fathom_plan(st_d, q, B)
    sws = F.scan_workspace(st_d, G, dev)
    F.fathom_scan_prepare(st_d, q, depth, sws)
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    scan_h = timed_ms(lambda: F.fathom_scan_prepared(st_h, G, scores, sws), stream, 10,
                      flush, sink)
    scan_d = timed_ms(lambda: F.fathom_scan_prepared(st_d, G, scores, sws), stream, 10,
                      flush, sink)
    fixed = F.fathom_plan_fixed(st_d, 34)
    F.fathom_scan_prepare(st_d, q, fixed, sws)
    scan136_h = timed_ms(lambda: F.fathom_scan_prepared(st_h, G, scores, sws), stream, 10,
                         flush, sink)
    del flush
    plane_bytes = B / 8 * n * H
    plane_gbps = plane_bytes / (scan_h * 1e-3) / 1e9
    oracle_check = layer_oracle_check(args, cfg, q, depth_of(st_d, q, B), idx_d, out_d,
                                      K_d, V_d, B, k, sm)
    oracle_time = None if args.no_cpu_baseline else oracle_layer_time(args, cfg, q, K_d, V_d,
                                                                      B, k, sm)
    step_bytes = plane_bytes + H * G * k * 512
    return {
        "workload": cfg.name, "kv_heads": H, "queries_per_kv_head": G, "tokens": n,
        "budget_bits": B, "k": k, "host_equals_hbm": same, "oracle_check": oracle_check,
        "step_ms_host": round(step_h, 3), "step_ms_hbm": round(step_d, 3),
        "scan_ms_host": round(scan_h, 3), "scan_ms_hbm": round(scan_d, 3),
        "scan_fixed136_ms_host": round(scan136_h, 3),
        "scan_plane_bytes": int(plane_bytes),
        "scan_plane_GBps_host": round(plane_gbps, 2),
        "L_GBps": L["L_GBps"], "scan_frac_of_link": round(plane_gbps / L["L_GBps"], 4),
        "scan_gkeys_per_s_host": round(H * n / (scan_h * 1e-3) / 1e9, 2),
        "pinned_host_bytes": int(planes_h.numel() * 4 + 2 * K_h.numel() * 2),
        "step_link_bytes": int(step_bytes),
        "step_frac_of_link_bound": round(step_bytes / (L["L_GBps"] * 1e9) / (step_h * 1e-3), 4),
        "cpu_baseline": oracle_time,
    }


def depth_of(st, q, B):
    from bit_plane_kv_amd import fathom as F
    return F.fathom_plan(st, q, B)


def layer_oracle_check(args, cfg, q, depth, idx, out, K, V, B, k, sm):
    """Oracle check of head 0 of the 1M-token layer: plan exact, scores to 1e-5 of the
    row maximum, top-k exact on the GPU's scores, attention to 2e-2."""
    import torch

    import oracle
    from bit_plane_kv_amd import fathom as F
    from bit_plane_kv_amd import synth
    h, n, G = 0, cfg.n, cfg.G
    st1 = F.Store.empty(1, n, q.device)
    keys = synth.keys_torch(args.seed, cfg.cfg_id, [h], n, q.device)
    F.fathom_quantize_store(keys, st1)
    sc = F.fathom_scan(st1, q[h:h + 1], depth[h:h + 1])
    torch.cuda.synchronize()
    kh = keys.cpu().numpy()
    del keys
    q_np = q[h:h + 1].cpu().numpy()
    s, z, codes = oracle.quantize(kh)
    ref_depth = oracle.plan(q_np, oracle.channel_var(codes, s), B)
    got = sc[0].cpu().numpy()
    ref = oracle.scores(codes, s, z, ref_depth, q_np)[0]
    err = float((np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())
    gi = idx[h].cpu().numpy()
    Kh = K[h:h + 1].cpu().view(torch.int16).numpy().view(np.uint16)
    Vh = V[h:h + 1].cpu().view(torch.int16).numpy().view(np.uint16)
    att = oracle.attention(q_np, Kh, Vh, gi[None], sm)
    aerr = float(np.abs(out[h].float().cpu().numpy() - att[0]).max())
    return {"head": h, "plan": bool(np.array_equal(depth[h].cpu().numpy(), ref_depth[0])),
            "score_rel_err": err, "topk": bool(np.array_equal(gi, oracle.topk(got, k))),
            "attn_abs_err": aerr}


def oracle_layer_time(args, cfg, q, K, V, B, k, sm, sample_heads=4):
    """The oracle's time for the decode step of the 1M-token layer (plan + fp64 scores +
    top-k + attention), measured on the first `sample_heads` of its 8 KV heads (OpenMP
    over heads) and scaled to the layer and to the 36-layer model: labelled extrapolated."""
    import torch

    import oracle
    from bit_plane_kv_amd import synth
    n, G, H = cfg.n, cfg.G, cfg.H
    hs = list(range(sample_heads))
    keys = synth.keys_torch(args.seed, cfg.cfg_id, hs, n, "cuda").cpu().numpy()
    s, z, codes = oracle.quantize(keys)          # store build: not part of a step
    del keys
    var = oracle.channel_var(codes, s)
    Kh = K[:sample_heads].cpu().view(torch.int16).numpy().view(np.uint16)
    Vh = V[:sample_heads].cpu().view(torch.int16).numpy().view(np.uint16)
    qh = q[:sample_heads].cpu().numpy()
    t0 = time.perf_counter()
    depth = oracle.plan(qh, var, B)
    sc = oracle.scores(codes, s, z, depth, qh)
    idx = oracle.topk(sc.astype(np.float32).reshape(-1, n), k).reshape(sample_heads, G, k)
    oracle.attention(qh, Kh, Vh, idx, sm)
    t = time.perf_counter() - t0
    cores = oracle.threads()
    used = min(cores, sample_heads)
    layer_ms = t * 1e3 * (H / sample_heads)
    return {"kind": "oracle", "cores": used, "cpu_model": cpu_model(),
            "value": round(H * n / (layer_ms * 1e-3) / 1e9, 6), "unit": "Gkeys/s",
            "layer_step_ms_extrapolated": round(layer_ms, 1),
            "model_step_ms_extrapolated": round(layer_ms * 36, 1),
            "sample": f"{sample_heads} of the layer's {H} KV heads (n={n}, G={G}, B={B}, "
                      f"k={k}): plan + fp64 scores + top-k + attention in {t:.2f} s wall on "
                      f"{used} threads (OpenMP over heads); layer = x{H / sample_heads:g}, "
                      f"model = x36 more, both extrapolated"}


def cpu_baseline(cfg, args, st, q_np, K, V, B, k, sm, sample_keys):
    """The oracle (as it stands) on the host cores: plan + scores + top-k + attention
    for a bounded sample of heads of the same workload; keys/s scaled to Gkeys/s."""
    import torch

    import oracle
    from bit_plane_kv_amd import synth
    n, G = cfg.n, cfg.G
    heads, elapsed, done = [], 0.0, 0
    batch = 8
    h = 0
    while elapsed < args.cpu_seconds and h < cfg.H:
        hs = list(range(h, min(cfg.H, h + batch)))
        keys = synth.keys_torch(args.seed, cfg.cfg_id, hs, n, "cuda").cpu().numpy()
        s, z, codes = oracle.quantize(keys)          # store build: not part of a step
        var = oracle.channel_var(codes, s)
        Kh = K[hs[0]:hs[-1] + 1].cpu().view(torch.int16).numpy().view(np.uint16)
        Vh = V[hs[0]:hs[-1] + 1].cpu().view(torch.int16).numpy().view(np.uint16)
        qh = q_np[hs[0]:hs[-1] + 1]
        t0 = time.perf_counter()
        depth = oracle.plan(qh, var, B)
        sc = oracle.scores(codes, s, z, depth, qh)
        idx = oracle.topk(sc.astype(np.float32).reshape(-1, n), k).reshape(len(hs), G, k)
        oracle.attention(qh, Kh, Vh, idx, sm)
        elapsed += time.perf_counter() - t0
        done += len(hs)
        h += len(hs)
    # single-thread figure on the first head of the last batch
    cores = oracle.threads()
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        d1 = oracle.plan(qh[:1], var[:1], B)
        sc1 = oracle.scores(codes[:1], s[:1], z[:1], d1, qh[:1])
        idx1 = oracle.topk(sc1.astype(np.float32).reshape(-1, n), k).reshape(1, G, k)
        oracle.attention(qh[:1], Kh[:1], Vh[:1], idx1, sm)
        t1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(cores)
    return {"value": round(done * n / elapsed / 1e9, 6), "unit": "Gkeys/s",
            "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "value_1_thread": round(n / t1 / 1e9, 6),
            "sample": f"{done} of {cfg.H} heads (n={n}, G={G}, B={B}, k={k}): plan + fp64 "
                      f"scores + top-k + attention, {elapsed:.1f} s wall on {cores} threads; "
                      f"1 head on 1 thread in {t1:.2f} s"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
