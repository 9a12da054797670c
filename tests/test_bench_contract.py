"""CPU checks of bench.py's contract: one GPU only, and the committed
counter summaries under profiles/ still describe the kernels' current
sources (a summary whose recorded hash no longer matches would make the
bench line report no traffic)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_counter_summaries_match_the_current_sources():
    b = _bench()
    workloads = {"decode": "decode-64seq-L512..4096-32q8kv-d128-b16-bf16",
                 "decode_q8": "decode-64seq-L512..4096-32q8kv-d128-b16-bf16-kv-int8",
                 "chunk": "mix-48decode-L256..4096+16chunk512-P0..2048-32q8kv-d128-b16-bf16"}
    for kind, workload in workloads.items():
        traffic = b.measured_traffic(workload, kind)
        assert traffic is not None, f"profiles/ counter summary for {kind} is stale or missing"
        assert traffic > 0
