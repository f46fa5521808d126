"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message, and the profile summariser's dispatch plan matches the calls
the benchmark makes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_varlen_workload_is_seeded_and_packed():
    sys.path.insert(0, ROOT)
    import attn_inputs as gen
    a, b = gen.varlen_causal_gqa(), gen.varlen_causal_gqa()
    assert (a.cu_q == b.cu_q).all() and (a.q == b.q).all()
    lens = (a.cu_q[1:] - a.cu_q[:-1])
    assert a.B == 16 and lens.min() >= 1 and lens.max() <= 8192
    assert a.q.shape == (int(a.cu_q[-1]), 32, 128) and a.k.shape == (int(a.cu_k[-1]), 8, 128)


def _fake_profile(tmp, copy_kib, kernels):
    """rocprofv3-shaped CSV output of `bench.py --counters` with known
    counter values: a 1 GiB copy, then for each (workload, kernel names,
    warm-up, calls) the library dispatches in launch order."""
    import csv
    import json
    import bench
    seq, order = [], []
    for wl, kerns, warm, calls in kernels:
        seq.append({"workload": wl, "warmup": warm, "calls": calls, "kernels": kerns,
                    "flop": 1e12, "algorithmic_bytes": 1e9})
        for _ in range(warm + calls):
            order += [f"void attn::(anonymous namespace)::{k}<false>(attn::PrefillArgs)"
                      for k in kerns]
    os.makedirs(tmp / "prof")
    with open(tmp / "prof" / "manifest.json", "w") as f:
        f.write("some log line\n" + json.dumps({"counters_run": True, "copy_bytes": 1 << 30,
                                                "sequence": seq}) + "\n")
    names = ["__amd_rocclr_copyBuffer"] + order
    t = 1000
    spans = []
    for _ in names:
        spans.append((t, t + 400_000))      # 400 us each
        t += 500_000
    cyc = 800_000.0                          # busy cycles of one XCD: 2000 MHz over 400 us
    values = {"FETCH_SIZE": 2.0 * (1 << 20), "WRITE_SIZE": 1.0 * (1 << 20),
              "GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cyc * 1024,
              "SQ_ACTIVE_INST_VALU": 0.25 * cyc * 256, "SQ_LDS_IDX_ACTIVE": 0.1 * cyc * 256,
              "SQ_LDS_BANK_CONFLICT": 0.01 * cyc * 256, "TCC_HIT_sum": 3.0, "TCC_MISS_sum": 1.0,
              "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e12 / 2 / 512, "SQ_INSTS_VALU_MFMA_MOPS_F16":
                  1e12 / 2 / 512}
    for pas, ctrs in [("ktrace", None)] + list(bench.COUNTER_PASSES.items()):
        os.makedirs(tmp / "prof" / pas)
        rows = []
        for i, (n, (a, b)) in enumerate(zip(names, spans)):
            base = {"Dispatch_Id": i + 1, "Kernel_Name": n, "Start_Timestamp": a,
                    "End_Timestamp": b}
            if ctrs is None:
                rows.append(base)
                continue
            for c in ctrs:
                v = values.get(c, 7.0)
                if n.startswith("__amd") and c in ("FETCH_SIZE", "WRITE_SIZE"):
                    v = copy_kib[c]
                rows.append({**base, "Counter_Name": c, "Counter_Value": v})
        f = "run_kernel_trace.csv" if ctrs is None else "run_counter_collection.csv"
        with open(tmp / "prof" / pas / f, "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=list(rows[0]))
            w.writeheader()
            w.writerows(rows)
    with open(tmp / "prof" / "sq" / "run_agent_info.csv", "w") as fh:
        fh.write('"Agent_Type","Cu_Count","Simd_Count","Num_Xcc"\n"CPU",16,0,1\n'
                 '"GPU",256,1024,8\n')


def test_summarize_derives_counters_per_dispatch(tmp_path):
    """The summariser maps dispatches to workloads through the manifest, drops
    warm-up calls, scales FETCH_SIZE / WRITE_SIZE by the copy's readings and
    derives the utilisations from per-XCD busy cycles."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    # the copy reads 2 GiB and writes 1 GiB by the counters: factors 1/2 and 1
    _fake_profile(tmp_path, {"FETCH_SIZE": 2.0 * (1 << 20), "WRITE_SIZE": 1.0 * (1 << 20)},
                  [("wa", ["prefill_pipe_kernel"], 1, 5),
                   ("wd", ["decode_partial_kernel", "decode_merge_kernel"], 1, 5)])
    out = tmp_path / "out"
    os.makedirs(out)
    bench.summarize(str(tmp_path / "prof"), str(out))
    data = json.load(open(out / "profile_data.json"))
    assert abs(data["fetch_scale"] - 0.5) < 1e-12 and abs(data["write_scale"] - 1.0) < 1e-12
    e = data["entries"]["wa::prefill_pipe_kernel"]
    assert e["dispatches"] == 5 and abs(e["avg_us"] - 400.0) < 1e-9
    assert abs(e["read_bytes"] - (1 << 30)) < 1 and abs(e["write_bytes"] - (1 << 30)) < 1
    dv = e["derived"]
    assert abs(dv["mfma_util"] - 0.5) < 1e-4 and abs(dv["valu_busy"] - 0.25) < 1e-4
    assert abs(dv["lds_util"] - 0.1) < 1e-4 and abs(dv["l2_hit_rate"] - 0.75) < 1e-4
    assert abs(dv["mfma_flop_over_algorithmic"] - 1.0) < 1e-4
    assert abs(dv["clock_mhz"] - 2000.0) < 1e-6
    assert {"wd::decode_partial_kernel", "wd::decode_merge_kernel"} <= set(data["entries"])
    assert (out / "prefill_pipe_kernel__wa.md").exists()
    assert (out / "decode_partial_kernel_and_decode_merge_kernel__wd.md").exists()


def test_summarize_rejects_a_sequence_that_does_not_match(tmp_path):
    import pytest
    sys.path.insert(0, ROOT)
    import bench
    _fake_profile(tmp_path, {"FETCH_SIZE": 1.0, "WRITE_SIZE": 1.0},
                  [("wa", ["prefill_kernel"], 1, 5)])
    import json
    p = tmp_path / "prof" / "manifest.json"
    m = json.loads(open(p).read().splitlines()[-1])
    m["sequence"][0]["kernels"] = ["prefill_pipe_kernel"]
    open(p, "w").write(json.dumps(m) + "\n")
    with pytest.raises(SystemExit, match="expected prefill_pipe_kernel"):
        bench.summarize(str(tmp_path / "prof"), str(tmp_path))
