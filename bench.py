#!/usr/bin/env python3
"""Benchmark of the gfx950 exact-attention library on one MI355X.

One step is one pass of the hot path over one batch of synthetic inputs that
are already resident in HBM:

* prefill: attn_fwd on the MHA workload B=4, Hq=Hkv=32, Sq=Sk=4096, d=128,
  bf16, BHSD, non-causal (the headline TFLOP/s, FLOP = 4*B*Hq*Sq*Sk*d);
* decode: attn_decode_paged on B=32, Hq=32, Hkv=8, 16-token pages, context
  lengths U{1..4096}, reported as algorithmic HBM GB/s; four independent
  copies of the KV pool (more than 1 GB in all) are rotated so that the
  256 MB last-level cache cannot serve a call from the previous one;
* the other prefill workloads (causal GQA B=8 S=8192, diffusion-style self
  attention S=32760 and its cross attention against 512 keys), timed the
  same way and reported beside the headline (skip with --no-extra);
* the causal GQA shape at head dims 64 and 256 (attn_fwd with d = 64, 256);
* the causal GQA workload with an ALiBi bias (attn_fwd_alibi);
* FP8 (E4M3) inputs on the MHA and causal GQA shapes (attn_fwd_fp8),
  reported beside the headline;
* packed sequences (attn_fwd_varlen): 16 causal GQA sequences of lengths
  U{1..8192}, reported beside the headline;
* the backward (attn_bwd: dQ, dK, dV) of the MHA and causal GQA workloads
  (also with ALiBi and at head dim 64) and of the packed sequences
  (attn_bwd_varlen), reported beside the headline too.

Times come from HIP events on the stream the kernels are launched on.  The
fp64 CPU oracle is timed on the host cores on a bounded sample of the same
workload as a reported baseline.  Prints one JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --counters      # short run for rocprofv3 counter passes
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "attn fwd TFLOP/s & % bf16 MFMA peak (d=128); paged decode HBM GB/s"
ROUNDING_MODES = ("rtne", "rtna", "rtz")   # rules of the bf16 output, timed on the headline


def sha256_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_profiles(kernel_key, source, launches_per_call=1):
    """HBM bytes per launch measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE,
    scaled by a copy kernel of known size), or None if absent or taken on a
    different version of the kernel source."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data[kernel_key]
        if ent.get("source_sha256") != sha256_of(source):
            return None
        return float(ent["hbm_bytes_per_launch"])
    except (KeyError, ValueError, TypeError):
        return None


def time_calls(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def per_call_stats(fn, reps, torch):
    """Median and minimum of `reps` calls timed one by one (an event pair per
    call on the launch stream), in ms."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return {"median_ms": round(t[len(t) // 2], 5), "min_ms": round(t[0], 5), "reps": reps}


def device_clock_info(torch):
    """CU count and peak engine clock of device 0 (hipDeviceGetAttribute,
    hipDeviceAttributeClockRate = 5, in kHz), and the dense bf16 MFMA rate they
    give at 4096 FLOP per CU per clock; None where the runtime does not
    answer."""
    import ctypes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    khz = None
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0 and v.value > 0:
            khz = v.value
    except OSError:
        pass
    peak = cus * khz * 1e3 * 4096 / 1e12 if khz else None
    return {"cus": cus, "clock_mhz": khz / 1e3 if khz else None,
            "bf16_peak_at_clock_TFLOP/s": round(peak, 1) if peak else None}


def snapshot_outputs(p, o, lse, od, torch):
    """Host copies of 64 random rows of the timed prefill's O and LSE and of
    the timed decode's O, for the sampled parity check of the oracle leg."""
    r = np.random.default_rng(0)
    rows = [(int(r.integers(p.B)), int(r.integers(p.Hq)), int(r.integers(p.Sq))) for _ in range(64)]
    og = torch.stack([o[b, h, i] for (b, h, i) in rows]).float().cpu().numpy()
    lg = torch.stack([lse[b, h, i] for (b, h, i) in rows]).cpu().numpy()
    return {"rows": rows, "o": og, "lse": lg, "od": od.float().cpu().numpy()}


def sampled_parity(p, d, snap):
    """The snapshot against the oracle (part of the oracle leg): worst error
    over the tolerance, and the worst LSE error."""
    import oracle.attention as att
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from tolerance import o_tolerance
    rows = snap["rows"]
    o_ref, l_ref = att.attention_sampled(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                         False, p.layout, rows)
    od_ref, _ = att.decode_paged(d.q, d.k_pool, d.v_pool, d.block_table, d.seq_lens, d.Hkv,
                                 d.scale)
    return {"prefill_sampled_rows": len(rows),
            "prefill_max_err_over_tol": round(float(
                (np.abs(snap["o"] - o_ref) / o_tolerance(o_ref)).max()), 4),
            "prefill_max_lse_err": float(np.abs(snap["lse"] - l_ref).max()),
            "decode_max_err_over_tol": round(float(
                (np.abs(snap["od"] - od_ref) / o_tolerance(od_ref)).max()), 4)}


def cpu_baseline(p, budget_s, torch):
    """Time the oracle (as it is) on whole (b, h) heads of the prefill
    workload until about budget_s seconds of host work are done."""
    import oracle.attention as att
    from threadpoolctl import threadpool_info
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    order = [(b, h) for b in range(p.B) for h in range(p.Hq)]
    for (b, h) in order:
        qs = p.q[b:b + 1, h:h + 1]
        ks = p.k[b:b + 1, h:h + 1]
        vs = p.v[b:b + 1, h:h + 1]
        att.attention(qs, ks, vs, 1, 1, 1, p.Sq, p.Sk, p.scale, False, 1, workers=workers)
        flops += 4.0 * p.Sq * p.Sk * 128
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    blas = sorted({i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"})
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{heads} of {p.B * p.Hq} (b,h) heads of the same workload, all "
                      f"{p.Sq} query rows x {p.Sk} keys, fp64 NumPy, {workers} worker threads "
                      f"x 1 BLAS thread (BLAS pool size {blas}); {dt:.1f} s",
            "seconds": dt}


TRAFFIC_FILE = "hbm_traffic__prefill_mha_b4_h32_s4096__decode_b32_hq32_hkv8.json"


def summarize_profiles(ktrace_dir, fetch_dir, write_dir, command):
    """Turn rocprofv3 output (a --kernel-trace --stats run of bench.py and two
    --pmc runs of `bench.py --counters`, FETCH_SIZE then WRITE_SIZE) into the
    short summaries kept under profiles/, one per kernel and workload, and the
    per-launch HBM traffic that bench.py reports."""
    import csv
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    stats = {r["Name"]: r for r in csv.DictReader(open(os.path.join(ktrace_dir,
                                                                    "run_kernel_stats.csv")))}
    # the bench launches each workload's calls back to back in a fixed order,
    # so the n-th dispatch of a kernel belongs to a known workload
    trace = list(csv.DictReader(open(os.path.join(ktrace_dir, "run_kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    by_kernel = {}
    for r in trace:
        by_kernel.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    per_wl = {}   # (workload, kernel part) -> durations
    for kpart, plan in command["plan"].items():
        names = [n for n in by_kernel if kpart in n]
        if len(names) != 1 or len(by_kernel[names[0]]) != sum(c for _, c in plan):
            raise SystemExit(f"summarize: dispatches of {kpart} do not match the bench's plan")
        durs, i = by_kernel[names[0]], 0
        for wl, cnt in plan:
            per_wl[(wl, kpart)] = durs[i:i + cnt]
            i += cnt

    # ---- HBM traffic per launch
    fetch = list(csv.DictReader(open(os.path.join(fetch_dir, "run_counter_collection.csv"))))
    write = list(csv.DictReader(open(os.path.join(write_dir, "run_counter_collection.csv"))))
    wmap = {r["Dispatch_Id"]: r for r in write}
    copy_bytes = float(1 << 30)
    # the reference copy is the largest copyBuffer dispatch (1 GiB read + 1 GiB written)
    copies = [r for r in fetch if "copyBuffer" in r["Kernel_Name"]]
    cref = max(copies, key=lambda r: float(r["Counter_Value"]))
    f_fetch = copy_bytes / (float(cref["Counter_Value"]) * 1024)
    f_write = copy_bytes / (float(wmap[cref["Dispatch_Id"]]["Counter_Value"]) * 1024)
    per = {}
    for r in fetch:
        name = r["Kernel_Name"]
        key = next((kk for kk in ("prefill_kernel", "prefill_fp8_kernel", "decode_partial_kernel",
                                  "decode_merge_kernel",
                                  "bwd_prep_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel")
                    if kk in name), None)
        if key is None:
            continue
        fb = float(r["Counter_Value"]) * 1024 * f_fetch
        wb = float(wmap[r["Dispatch_Id"]]["Counter_Value"]) * 1024 * f_write
        per.setdefault(key, []).append((fb, wb))
    srcs = {"prefill_kernel": "prefill.hip", "prefill_fp8_kernel": "prefill_fp8.hip",
            "decode_partial_kernel": "decode.hip",
            "decode_merge_kernel": "decode.hip", "bwd_prep_kernel": "backward.hip",
            "bwd_dkdv_kernel": "backward.hip", "bwd_dq_kernel": "backward.hip"}
    traffic = {"about": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                        "dispatch), each scaled by the reading of a 1 GiB device copy; prefill "
                        "and backward on mha_prefill_b4_h32_s4096_bhsd (FP8: its E4M3 copy), decode on "
                        "paged_decode_b32_hq32_hkv8_len4096_page16",
               "fetch_scale": f_fetch, "write_scale": f_write,
               "commands": [command["fetch"], command["write"]]}
    trows = {}
    for key, vals in per.items():
        fb = sum(v[0] for v in vals) / len(vals)
        wb = sum(v[1] for v in vals) / len(vals)
        traffic[key] = {"source_sha256": sha256_of(os.path.join(ROOT, "exact_attention_60_amd",
                                                                 "csrc", srcs[key])),
                        "read_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                        "hbm_bytes_per_launch": fb + wb, "launches": len(vals)}
        trows[key] = (f"| {key} | {len(vals)} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                      f"{(fb + wb) / 1e6:.1f} |")
    with open(os.path.join(out_dir, TRAFFIC_FILE), "w") as f:
        json.dump(traffic, f, indent=1)

    def kstats_row(kpart):
        for name, r in stats.items():
            if kpart in name:
                return (f"| `{kpart}` (all workloads of the run) | {r['Calls']} | "
                        f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                        f"{float(r['MaxNs']) / 1e3:.1f} |")
        return f"| `{kpart}` | - | - | - | - |"

    def wl_row(wl, kpart):
        d = per_wl[(wl, kpart)]
        return (f"| `{kpart}` on {wl} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | "
                f"{max(d):.1f} |")

    head = ["Command (from the repository root on the GPU box):", "", "```", command["ktrace"],
            "```", "", "| kernel / workload | dispatches | average us | min us | max us |",
            "|---|---|---|---|---|"]
    thead = ["", "HBM traffic per launch (rocprofv3 --pmc), commands:", "", "```",
             command["fetch"], command["write"], "```", "",
             f"Scale factors from a 1 GiB device copy: FETCH_SIZE x {f_fetch:.4f}, "
             f"WRITE_SIZE x {f_write:.4f}.", "",
             "| kernel | launches | read MB | written MB | total MB |", "|---|---|---|---|---|"]
    files = {
        "prefill_kernel__mha_prefill_b4_h32_s4096_bhsd.md": (
            "# prefill_kernel on mha_prefill_b4_h32_s4096_bhsd (B=4, H=32, S=4096, BHSD)",
            [wl_row("mha_prefill_b4_h32_s4096_bhsd", "prefill_kernel<false, false>")] +
            [wl_row(f"mha_prefill_b4_h32_s4096_bhsd_{m}", "prefill_kernel<false, false>")
             for m in ROUNDING_MODES] +
            [kstats_row("prefill_kernel<false, false>")], ["prefill_kernel"]),
        "decode_partial_and_merge_kernels__paged_decode_b32_hq32_hkv8_len4096.md": (
            "# decode_partial_kernel + decode_merge_kernel on paged_decode_b32_hq32_hkv8_"
            "len4096_page16",
            [wl_row("paged_decode_b32_hq32_hkv8_len4096_page16", "decode_partial_kernel"),
             wl_row("paged_decode_b32_hq32_hkv8_len4096_page16", "decode_merge_kernel"),
             wl_row("paged_decode_b32_hq32_hkv8_len4096_page16_append", "decode_partial_kernel"),
             wl_row("paged_decode_b32_hq32_hkv8_len4096_page16_append", "decode_merge_kernel")],
            ["decode_partial_kernel", "decode_merge_kernel"]),
        "prefill_fp8_kernel__fp8_mha_s4096_and_causal_gqa_s8192.md": (
            "# prefill_fp8_kernel (attn_fwd_fp8, E4M3 inputs) on fp8_mha_prefill_b4_h32_s4096_bhsd "
            "and fp8_gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd",
            [wl_row("fp8_mha_prefill_b4_h32_s4096_bhsd", "prefill_fp8_kernel<false>"),
             wl_row("fp8_gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd", "prefill_fp8_kernel<true>")],
            ["prefill_fp8_kernel"]),
        "prefill_kernel__causal_gqa_s8192_and_diffusion_s32760.md": (
            "# prefill_kernel on the causal GQA and diffusion-style workloads",
            [wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd", "prefill_kernel<true, false>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_alibi",
                    "prefill_kernel<true, true>"),
             wl_row("diffusion_self_b2_h12_s32760_bshd", "prefill_kernel<false, false>"),
             wl_row("diffusion_cross_b2_h12_sq32760_sk512_bshd", "prefill_kernel<false, false>"),
             wl_row("varlen_causal_gqa_b16_hq32_hkv8_len8192", "prefill_kernel<true, false>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_d64_bshd",
                    "prefill_hd_kernel<64, true>"),
             wl_row("gqa_causal_prefill_b4_hq32_hkv8_s4096_d256_bshd",
                    "prefill_hd_kernel<256, true>")],
            []),
        "backward_kernels__mha_b4_h32_s4096_bhsd_and_causal_gqa_s8192.md": (
            "# bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel (attn_bwd) on "
            "mha_prefill_b4_h32_s4096_bhsd and gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd",
            [wl_row("mha_prefill_b4_h32_s4096_bhsd_backward", "bwd_prep_kernel<128>"),
             wl_row("mha_prefill_b4_h32_s4096_bhsd_backward", "bwd_dkdv_kernel<128, false, false, false>"),
             wl_row("mha_prefill_b4_h32_s4096_bhsd_backward", "bwd_dq_kernel<128, false, false, false>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_backward", "bwd_prep_kernel<128>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_backward",
                    "bwd_dkdv_kernel<128, true, false, false>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_backward",
                    "bwd_dq_kernel<128, true, false, false>"),
             wl_row("varlen_causal_gqa_b16_hq32_hkv8_len8192_backward", "bwd_prep_kernel<128>"),
             wl_row("varlen_causal_gqa_b16_hq32_hkv8_len8192_backward",
                    "bwd_dkdv_kernel<128, true, true, false>"),
             wl_row("varlen_causal_gqa_b16_hq32_hkv8_len8192_backward",
                    "bwd_dq_kernel<128, true, true, false>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_alibi_backward", "bwd_prep_kernel<128>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_alibi_backward",
                    "bwd_dkdv_kernel<128, true, false, true>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_alibi_backward",
                    "bwd_dq_kernel<128, true, false, true>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_d64_bshd_backward",
                    "bwd_prep_kernel<64>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_d64_bshd_backward",
                    "bwd_dkdv_kernel<64, true, false, false>"),
             wl_row("gqa_causal_prefill_b8_hq32_hkv8_s8192_d64_bshd_backward",
                    "bwd_dq_kernel<64, true, false, false>")],
            ["bwd_prep_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"]),
    }
    for fname, (title, rows, tkeys) in files.items():
        body = [title, ""] + head + rows
        if tkeys:
            body += thead + [trows[k] for k in tkeys if k in trows]
        with open(os.path.join(out_dir, fname), "w") as f:
            f.write("\n".join(body) + "\n")


def extra_workloads(args, gen, ea, torch, dev, to_dev, log):
    """Time attn_fwd on the other prefill workloads (same method as the
    headline: inputs resident, HIP events on the launch stream)."""
    res = []
    steps = max(3, min(args.steps, 10))
    p4 = None
    for make in (gen.config3, gen.config4_self, lambda: gen.config4_cross(self_problem=p4)):
        p = make()
        if p.Sk == p.Sq == 32760:
            p4 = p
        log(f"timing {p.name}")
        q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
        lay = "bshd" if p.layout == gen.BSHD else "bhsd"
        o = torch.empty_like(q)
        lse = torch.empty((p.B, p.Hq, p.Sq), dtype=torch.float32, device=dev)

        def run(_i):
            ea.attn_fwd(q, k, v, causal=p.causal, scale=p.scale, layout=lay, out=o, lse=lse)

        ms = time_calls(run, steps, 2, torch)
        tf = p.flops / (ms * 1e-3) / 1e12
        res.append({"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Sq": p.Sq,
                    "Sk": p.Sk, "causal": p.causal, "layout": lay, "ms_per_call": round(ms, 4),
                    "flop": p.flops, "TFLOP/s": round(tf, 2),
                    "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        del q, k, v, o, lse
    # FP8 (E4M3) inputs on the MHA and causal GQA shapes (attn_fwd_fp8)
    def u8(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    for make in (gen.fp8_mha_prefill, gen.fp8_causal_gqa):
        p = make()
        log(f"timing {p.name}")
        lay = "bshd" if p.layout == gen.BSHD else "bhsd"
        q, k, v = u8(p.q), u8(p.k), u8(p.v)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty((p.B, p.Hq, p.Sq), dtype=torch.float32, device=dev)

        def run_f(_i):
            ea.attn_fwd_fp8(q, k, v, causal=p.causal, scale=p.scale, layout=lay, out=o, lse=lse)

        ms = time_calls(run_f, steps, 2, torch)
        tf = p.flops / (ms * 1e-3) / 1e12
        ent = {"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Sq": p.Sq, "Sk": p.Sk,
               "inputs": "e4m3", "compute": "fp16 MFMA", "causal": p.causal, "layout": lay,
               "ms_per_call": round(ms, 4), "flop": p.flops, "TFLOP/s": round(tf, 2),
               "frac_of_fp16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        if not p.causal:
            ent["algorithmic_bytes"] = 3 * q.numel() + 2 * o.numel() + 4 * lse.numel()
            ent["traffic"] = traffic_from_profiles(
                "prefill_fp8_kernel",
                os.path.join(ROOT, "exact_attention_60_amd", "csrc", "prefill_fp8.hip"))
        res.append(ent)
        del q, k, v, o, lse
    # head dim 64 on the causal GQA shape
    p = gen.headdim64_causal_gqa()
    log(f"timing {p.name}")
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    o = torch.empty_like(q)
    lse = torch.empty((p.B, p.Hq, p.Sq), dtype=torch.float32, device=dev)

    def run_h(_i):
        ea.attn_fwd(q, k, v, causal=True, scale=p.scale, layout="bshd", out=o, lse=lse)

    ms = time_calls(run_h, steps, 2, torch)
    tf = p.flops / (ms * 1e-3) / 1e12
    res.append({"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Sq": p.Sq, "Sk": p.Sk,
                "d": 64, "causal": True, "layout": "bshd", "ms_per_call": round(ms, 4),
                "flop": p.flops, "TFLOP/s": round(tf, 2),
                "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
    del q, k, v, o, lse
    # head dim 256 on a causal GQA shape (B=4, Hq=32, Hkv=8, S=4096)
    p = gen.prefill_inputs(4, 32, 8, 4096, 4096, layout=gen.BSHD, causal=True, seed=8, d=256,
                           name="gqa_causal_prefill_b4_hq32_hkv8_s4096_d256_bshd")
    log(f"timing {p.name}")
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    o = torch.empty_like(q)
    lse = torch.empty((p.B, p.Hq, p.Sq), dtype=torch.float32, device=dev)

    def run_h2(_i):
        ea.attn_fwd(q, k, v, causal=True, scale=p.scale, layout="bshd", out=o, lse=lse)

    ms = time_calls(run_h2, steps, 2, torch)
    tf = p.flops / (ms * 1e-3) / 1e12
    res.append({"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Sq": p.Sq, "Sk": p.Sk,
                "d": 256, "causal": True, "layout": "bshd", "ms_per_call": round(ms, 4),
                "flop": p.flops, "TFLOP/s": round(tf, 2),
                "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
    del q, k, v, o, lse
    # ALiBi on the causal GQA workload (slopes 2^(-8h/H) of the ALiBi method)
    p = gen.config3()
    log(f"timing {p.name} with ALiBi")
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    sl = torch.from_numpy((2.0 ** (-8.0 * np.arange(1, p.Hq + 1) / p.Hq)).astype(np.float32)).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((p.B, p.Hq, p.Sq), dtype=torch.float32, device=dev)

    def run_a(_i):
        ea.attn_fwd(q, k, v, causal=True, scale=p.scale, layout="bshd", out=o, lse=lse,
                    alibi_slopes=sl)

    ms = time_calls(run_a, steps, 2, torch)
    tf = p.flops / (ms * 1e-3) / 1e12
    res.append({"workload": p.name + "_alibi", "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Sq": p.Sq,
                "Sk": p.Sk, "causal": True, "layout": "bshd", "ms_per_call": round(ms, 4),
                "flop": p.flops, "TFLOP/s": round(tf, 2),
                "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
    del q, k, v, o, lse
    # packed sequences of mixed lengths (attn_fwd_varlen)
    pv = gen.varlen_causal_gqa()
    log(f"timing {pv.name}")
    q, k, v = to_dev(pv.q), to_dev(pv.k), to_dev(pv.v)
    cq = torch.from_numpy(pv.cu_q).to(dev)
    ck = torch.from_numpy(pv.cu_k).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((pv.Hq, q.shape[0]), dtype=torch.float32, device=dev)

    def run_v(_i):
        ea.attn_fwd_varlen(q, k, v, cq, ck, pv.max_q, causal=True, scale=pv.scale, out=o, lse=lse)

    ms = time_calls(run_v, steps, 2, torch)
    tf = pv.flops / (ms * 1e-3) / 1e12
    res.append({"workload": pv.name, "B": pv.B, "Hq": pv.Hq, "Hkv": pv.Hkv,
                "total_tokens": int(pv.cu_q[-1]), "max_seqlen": pv.max_q, "causal": True,
                "layout": "packed [tokens, H, 128]", "ms_per_call": round(ms, 4),
                "flop": pv.flops, "TFLOP/s": round(tf, 2),
                "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return res


def backward_workloads(args, gen, ea, torch, to_dev, log):
    """attn_bwd (dQ, dK, dV from the forward's O and LSE and an upstream dO;
    three launches: row terms, dK/dV, dQ) on the MHA and the causal GQA
    workloads.  FLOP = 10*B*Hq*Sq*Sk*d (the five products S, dP, dV, dQ, dK),
    halved when causal."""
    res = []
    steps = max(3, min(args.steps, 10))
    for make, seed in ((gen.config2, 2), (gen.config3, 3)):
        p = make()
        log(f"timing the backward of {p.name}")
        q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
        do = to_dev(gen.output_grad(p, seed))
        lay = "bshd" if p.layout == gen.BSHD else "bhsd"
        o, lse = ea.attn_fwd(q, k, v, causal=p.causal, scale=p.scale, layout=lay)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(ea.attn_bwd_workspace_bytes(p.B, p.Hq, p.Sq), dtype=torch.uint8,
                         device=q.device)

        def run(_i):
            ea.attn_bwd(q, k, v, o, lse, do, causal=p.causal, scale=p.scale, layout=lay, dq=dq,
                        dk=dk, dv=dv, workspace=ws)

        ms = time_calls(run, steps, 2, torch)
        fl = 10.0 * p.B * p.Hq * p.Sq * p.Sk * 128 / (2 if p.causal else 1)
        tf = fl / (ms * 1e-3) / 1e12
        ent = {"workload": p.name + "_backward", "ms_per_call": round(ms, 4), "flop": fl,
               "TFLOP/s": round(tf, 2), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
               "kernels": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel"}
        if p.name == "mha_prefill_b4_h32_s4096_bhsd":
            # HBM bytes the three kernels moved per call (counter passes), against the
            # algorithmic Q, K, V, O, dO, LSE read once and dQ, dK, dV written once
            src_b = os.path.join(ROOT, "exact_attention_60_amd", "csrc", "backward.hip")
            parts = [traffic_from_profiles(kk, src_b) for kk in
                     ("bwd_prep_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel")]
            ent["algorithmic_bytes"] = 8 * q.numel() * 2 + 4 * p.B * p.Hq * p.Sq
            ent["traffic"] = None if None in parts else sum(parts)
        res.append(ent)
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    # the causal GQA backward with ALiBi (attn_bwd_alibi)
    p = gen.config3()
    log(f"timing the backward of {p.name} with ALiBi")
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    do = to_dev(gen.output_grad(p, 3))
    sl = torch.from_numpy((2.0 ** (-8.0 * np.arange(1, p.Hq + 1) / p.Hq)).astype(np.float32)).to(
        q.device)
    o, lse = ea.attn_fwd(q, k, v, causal=True, scale=p.scale, layout="bshd", alibi_slopes=sl)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(p.B, p.Hq, p.Sq), dtype=torch.uint8,
                     device=q.device)

    def run_a(_i):
        ea.attn_bwd(q, k, v, o, lse, do, causal=True, scale=p.scale, layout="bshd", dq=dq, dk=dk,
                    dv=dv, workspace=ws, alibi_slopes=sl)

    ms = time_calls(run_a, steps, 2, torch)
    fl = 10.0 * p.B * p.Hq * p.Sq * p.Sk * 128 / 2
    res.append({"workload": p.name + "_alibi_backward", "ms_per_call": round(ms, 4), "flop": fl,
                "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
                "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "kernels": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel"})
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    # the causal GQA backward at head dim 64
    p = gen.headdim64_causal_gqa()
    log(f"timing the backward of {p.name}")
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    do = to_dev(gen.output_grad(p, 7))
    o, lse = ea.attn_fwd(q, k, v, causal=True, scale=p.scale, layout="bshd")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(p.B, p.Hq, p.Sq), dtype=torch.uint8,
                     device=q.device)

    def run_d(_i):
        ea.attn_bwd(q, k, v, o, lse, do, causal=True, scale=p.scale, layout="bshd", dq=dq, dk=dk,
                    dv=dv, workspace=ws)

    ms = time_calls(run_d, steps, 2, torch)
    fl = 10.0 * p.B * p.Hq * p.Sq * p.Sk * 64 / 2
    res.append({"workload": p.name + "_backward", "ms_per_call": round(ms, 4), "flop": fl,
                "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
                "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "kernels": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel"})
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    # packed sequences of mixed lengths (attn_bwd_varlen)
    pv = gen.varlen_causal_gqa()
    log(f"timing the backward of {pv.name}")
    q, k, v = to_dev(pv.q), to_dev(pv.k), to_dev(pv.v)
    r = np.random.default_rng(6)
    do = to_dev(gen.f32_to_bf16_bits(r.standard_normal(pv.q.shape).astype(np.float32)))
    cq = torch.from_numpy(pv.cu_q).to(q.device)
    ck = torch.from_numpy(pv.cu_k).to(q.device)
    o, lse = ea.attn_fwd_varlen(q, k, v, cq, ck, pv.max_q, causal=True, scale=pv.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(1, pv.Hq, q.shape[0]), dtype=torch.uint8,
                     device=q.device)

    def run_v(_i):
        ea.attn_bwd_varlen(q, k, v, o, lse, do, cq, ck, pv.max_q, pv.max_q, causal=True,
                           scale=pv.scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    ms = time_calls(run_v, steps, 2, torch)
    fl = 2.5 * pv.flops
    res.append({"workload": pv.name + "_backward", "ms_per_call": round(ms, 4), "flop": fl,
                "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
                "frac_of_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "kernels": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel"})
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def decode_append(args, d, ea, torch, qd, pools, tab, lens, od, lsed, ws, to_dev, log):
    """The decode workload with the current token appended to the cache in the
    same call (attn_decode_paged_append): new K/V rows drawn for every
    sequence; each call writes them into the rotated pools and attends."""
    import attn_inputs as gen
    r = np.random.default_rng(7)
    kn = to_dev(gen.f32_to_bf16_bits(r.standard_normal((d.B, d.Hkv, 128)).astype(np.float32)))
    vn = to_dev(gen.f32_to_bf16_bits(r.standard_normal((d.B, d.Hkv, 128)).astype(np.float32)))
    log(f"timing {d.name} with the cache append")

    def run(i):
        kp, vp = pools[i % len(pools)]
        ea.attn_decode_paged_append(qd, kn, vn, kp, vp, tab, lens, scale=d.scale, out=od,
                                    lse=lsed, workspace=ws)

    ms = time_calls(run, max(args.steps, 20), 3, torch)
    # the plain decode's bytes plus the new rows read and written once
    nbytes = d.bytes + 2 * 2 * d.B * d.Hkv * 128 * 2
    return {"workload": d.name + "_append", "us_per_call": round(ms * 1e3, 2),
            "algorithmic_bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def rounding_modes(args, p, ea, torch, q, k, v, o, lse, log):
    """The headline prefill under each rounding rule of the bf16 output (every
    shape is measured under RTNE, RTNA and RTZ on the pages)."""
    res = {}
    steps = max(3, min(args.steps, 10))
    for mode in ROUNDING_MODES:
        log(f"timing {p.name} with rounding {mode}")

        def run(_i):
            ea.attn_fwd(q, k, v, causal=False, scale=p.scale, layout="bhsd", rounding=mode,
                        out=o, lse=lse)

        ms = time_calls(run, steps, 2, torch)
        res[mode] = {"ms_per_call": round(ms, 4),
                     "TFLOP/s": round(p.flops / (ms * 1e-3) / 1e12, 2)}
    return {"workload": p.name, **res}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="host seconds spent timing the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other prefill workloads (causal GQA, diffusion self/cross)")
    ap.add_argument("--counters", action="store_true",
                    help="no timing: one device copy of 1 GiB, then 3 prefill and 3 decode "
                         "calls, for rocprofv3 counter passes")
    ap.add_argument("--summarize", nargs=3, metavar=("KTRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/kernel_stats.md and profiles/traffic.json from rocprofv3 "
                         "output directories (no GPU needed)")
    args = ap.parse_args()
    if args.summarize:
        st, wu, xs = 30, 5, 12   # bench defaults: steps, warmup; extra workloads 10 + 2
        cmd = {"plan": {"prefill_fp8_kernel<false>": [("fp8_mha_prefill_b4_h32_s4096_bhsd", xs)],
                        "prefill_fp8_kernel<true>": [("fp8_gqa_causal_prefill_b8_hq32_hkv8_s8192"
                                                      "_bshd", xs)],
                        "prefill_hd_kernel<64, true>": [("gqa_causal_prefill_b8_hq32_hkv8_s8192"
                                                         "_d64_bshd", xs),
                                                        ("gqa_causal_prefill_b8_hq32_hkv8_s8192"
                                                         "_d64_bshd_backward_fwd", 1)],
                        "bwd_prep_kernel<64>": [("gqa_causal_prefill_b8_hq32_hkv8_s8192_d64_bshd"
                                                 "_backward", xs)],
                        "bwd_dkdv_kernel<64, true, false, false>": [(
                            "gqa_causal_prefill_b8_hq32_hkv8_s8192_d64_bshd_backward", xs)],
                        "bwd_dq_kernel<64, true, false, false>": [(
                            "gqa_causal_prefill_b8_hq32_hkv8_s8192_d64_bshd_backward", xs)],
                        "prefill_hd_kernel<256, true>": [("gqa_causal_prefill_b4_hq32_hkv8_s4096"
                                                          "_d256_bshd", xs)],
                        "prefill_kernel<true, true>": [("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd"
                                                        "_alibi", xs),
                                                       ("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd"
                                                        "_alibi_backward_fwd", 1)],
                        "prefill_kernel<false, false>": [("mha_prefill_b4_h32_s4096_bhsd",
                                                          st + wu + max(st, 20))] +
                                                 [(f"mha_prefill_b4_h32_s4096_bhsd_{m}", xs)
                                                  for m in ROUNDING_MODES] +
                                                 [("diffusion_self_b2_h12_s32760_bshd", xs),
                                                  ("diffusion_cross_b2_h12_sq32760_sk512_bshd", xs),
                                                  ("mha_prefill_b4_h32_s4096_bhsd_backward_fwd", 1)],
                        "prefill_kernel<true, false>": [("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd",
                                                         xs),
                                                        ("varlen_causal_gqa_b16_hq32_hkv8_len8192",
                                                         xs),
                                                 ("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd"
                                                  "_backward_fwd", 1),
                                                 ("varlen_causal_gqa_b16_hq32_hkv8_len8192"
                                                  "_backward_fwd", 1)],
                        "bwd_prep_kernel<128>": [("mha_prefill_b4_h32_s4096_bhsd_backward", xs),
                                            ("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_backward",
                                             xs),
                                            ("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_alibi"
                                             "_backward", xs),
                                            ("varlen_causal_gqa_b16_hq32_hkv8_len8192_backward",
                                             xs)],
                        "bwd_dkdv_kernel<128, false, false, false>": [("mha_prefill_b4_h32_s4096_bhsd_backward",
                                                           xs)],
                        "bwd_dq_kernel<128, false, false, false>": [("mha_prefill_b4_h32_s4096_bhsd_backward",
                                                         xs)],
                        "bwd_dkdv_kernel<128, true, false, false>": [("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd"
                                                          "_backward", xs)],
                        "bwd_dq_kernel<128, true, false, false>": [("gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd"
                                                        "_backward", xs)],
                        "bwd_dkdv_kernel<128, true, true, false>": [("varlen_causal_gqa_b16_hq32_hkv8_len8192"
                                                         "_backward", xs)],
                        "bwd_dq_kernel<128, true, true, false>": [("varlen_causal_gqa_b16_hq32_hkv8_len8192"
                                                       "_backward", xs)],
                        "bwd_dkdv_kernel<128, true, false, true>": [(
                            "gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_alibi_backward", xs)],
                        "bwd_dq_kernel<128, true, false, true>": [(
                            "gqa_causal_prefill_b8_hq32_hkv8_s8192_bshd_alibi_backward", xs)],
                        "decode_partial_kernel": [("paged_decode_b32_hq32_hkv8_len4096_page16",
                                                   max(st, 20) + wu + max(st, 40)),
                                                  ("paged_decode_b32_hq32_hkv8_len4096_page16_append",
                                                   max(st, 20) + 3)],
                        "decode_merge_kernel": [("paged_decode_b32_hq32_hkv8_len4096_page16",
                                                 max(st, 20) + wu + max(st, 40)),
                                                ("paged_decode_b32_hq32_hkv8_len4096_page16_append",
                                                 max(st, 20) + 3)]},
               "ktrace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/ktrace "
                         "-o run -- python3 -u bench.py --no-cpu-baseline",
               "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch "
                        "-o run -- python3 -u bench.py --counters",
               "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write "
                        "-o run -- python3 -u bench.py --counters"}
        summarize_profiles(*args.summarize, cmd)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus}: this library and benchmark run on one GPU only; "
              "there is no multi-GPU path to measure", file=sys.stderr)
        sys.exit(2)

    import torch
    import attn_inputs as gen
    import exact_attention_60_amd as ea
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    ea.library()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- prefill inputs (resident in HBM before timing)
    p = gen.config2()
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    o = torch.empty_like(q)
    lse = torch.empty((p.B, p.Hq, p.Sq), dtype=torch.float32, device=dev)

    def prefill(_i):
        ea.attn_fwd(q, k, v, causal=False, scale=p.scale, layout="bhsd", out=o, lse=lse)

    # ---- decode inputs: four copies of the pool, rotated
    d = gen.config5()
    qd = to_dev(d.q)
    kp0, vp0 = to_dev(d.k_pool), to_dev(d.v_pool)
    pools = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(3)]
    tab = torch.from_numpy(d.block_table).to(dev)
    lens = torch.from_numpy(d.seq_lens).to(dev)
    od = torch.empty_like(qd)
    lsed = torch.empty((d.B, d.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(ea.attn_decode_workspace_bytes(d.B, d.Hq, d.max_blocks), dtype=torch.uint8,
                     device=dev)

    def decode(i):
        kp, vp = pools[i % len(pools)]
        ea.attn_decode_paged(qd, kp, vp, tab, lens, scale=d.scale, out=od, lse=lsed, workspace=ws)

    if args.counters:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)          # reference: reads and writes exactly 1 GiB
        for i in range(3):
            prefill(i)
        for i in range(3):
            decode(i)
        do = to_dev(gen.output_grad(p, 2))
        for i in range(3):
            ea.attn_bwd(q, k, v, o, lse, do, causal=False, scale=p.scale, layout="bhsd")
        p8 = gen.fp8_mha_prefill()
        q8, k8, v8 = (torch.from_numpy(x).to(dev) for x in (p8.q, p8.k, p8.v))
        for i in range(3):
            ea.attn_fwd_fp8(q8, k8, v8, scale=p8.scale, layout="bhsd", out=o, lse=lse)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": True, "copy_bytes": n}))
        return

    def log(msg):
        print(f"bench: {msg}", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    log("inputs resident; timing prefill")
    ms_p = time_calls(prefill, args.steps, args.warmup, torch)
    log(f"prefill {ms_p:.3f} ms/call; timing decode")
    ms_d = time_calls(decode, max(args.steps, 20), args.warmup, torch)
    log(f"decode {ms_d * 1e3:.1f} us/call")

    tflops = p.flops / (ms_p * 1e-3) / 1e12
    gbs = d.bytes / (ms_d * 1e-3) / 1e9
    # per-call distribution of the same two calls (median and minimum)
    st_p = per_call_stats(prefill, max(args.steps, 20), torch)
    st_d = per_call_stats(decode, max(args.steps, 40), torch)
    dev_info = device_clock_info(torch)
    snap = snapshot_outputs(p, o, lse, od, torch)

    src_p = os.path.join(ROOT, "exact_attention_60_amd", "csrc", "prefill.hip")
    src_d = os.path.join(ROOT, "exact_attention_60_amd", "csrc", "decode.hip")
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_p, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": p.name, "B": p.B, "Hq": p.Hq, "Hkv": p.Hkv, "Sq": p.Sq,
                   "Sk": p.Sk, "d": 128, "layout": "bhsd", "causal": False,
                   "parallelism": "none (one GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profiles("prefill_kernel", src_p),
                     "kernel": "prefill_kernel<false, false>",
                     "per_launch": {"flop": p.flops, "ms": round(ms_p, 4)},
                     "per_call": {**st_p, "TFLOP/s_at_median": round(
                         p.flops / (st_p["median_ms"] * 1e-3) / 1e12, 2)},
                     "device": dev_info,
                     "frac_of_peak_at_device_clock": (
                         round(tflops / dev_info["bf16_peak_at_clock_TFLOP/s"], 4)
                         if dev_info["bf16_peak_at_clock_TFLOP/s"] else None)},
        "decode": {"workload": d.name, "value": round(gbs, 1), "unit": "GB/s",
                   "us_per_call": round(ms_d * 1e3, 2), "tokens": d.tokens,
                   "algorithmic_bytes": d.bytes,
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                "traffic": traffic_from_profiles("decode_partial_kernel", src_d),
                                "kernel": "decode_partial_kernel + decode_merge_kernel"},
                   "per_call": {"median_us": round(st_d["median_ms"] * 1e3, 2),
                                "min_us": round(st_d["min_ms"] * 1e3, 2), "reps": st_d["reps"],
                                "GB/s_at_median": round(d.bytes / (st_d["median_ms"] * 1e-3) / 1e9,
                                                        1)}},
    }
    if not args.no_extra:
        out["decode_append"] = decode_append(args, d, ea, torch, qd, pools, tab, lens, od, lsed,
                                             ws, to_dev, log)
        out["rounding_modes"] = rounding_modes(args, p, ea, torch, q, k, v, o, lse, log)
        out["other_workloads"] = extra_workloads(args, gen, ea, torch, dev, to_dev, log)
        out["backward"] = backward_workloads(args, gen, ea, torch, to_dev, log)
    if not args.no_cpu_baseline:
        # the oracle leg: a sampled parity check of what was timed, then the
        # oracle timed on the host cores
        log("sampled parity against the oracle")
        out["parity"] = sampled_parity(p, d, snap)
        log("timing the CPU oracle baseline")
        cb = cpu_baseline(p, args.cpu_seconds, torch)
        cb["value"] = round(cb["value"], 6)
        cb["seconds"] = round(cb["seconds"], 2)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
