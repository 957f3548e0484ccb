"""bench.py's contract where it needs no GPU: one GPU only (a clear refusal for
--gpus above 1 or a multi-rank launch), and the oracle-only leg that supplies
the cpu_baseline object (one JSON line with the reported fields)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None, timeout=300):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", **(env_extra or {}))
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert not r.stdout.strip()


def test_multi_rank_launch_is_refused():
    r = _run([], env_extra={"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "WORLD_SIZE 2" in r.stderr


def test_oracle_only_line():
    r = _run(["--oracle-only", "--workload", "0", "--cpu-seconds", "0.5", "--oracle-threads", "1"])
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["oracle_only"] is True and d["kind"] == "oracle"
    assert d["unit"] == "GB/s" and d["value"] > 0
    assert d["cores"] == 1 and d["threads_requested"] == 1
    assert (d["T"], d["H"], d["I"], d["E"], d["top_k"]) == (8, 256, 128, 4, 2)
    assert "pass(es) of the layer step" in d["sample"]
