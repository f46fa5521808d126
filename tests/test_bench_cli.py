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
