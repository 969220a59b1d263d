"""bench.py's host-side contract (no GPU needed): it measures one GPU, and a
request for more exits with status 2 and a message, before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr
        assert r.stdout == ""


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_cpu_baseline_times_the_oracle_on_rows_first_and_last():
    import photon_inputs as pi
    bench = _bench()
    wl = pi.get(1)
    W = pi.gen_weights(wl.cfg, wl.seed)
    for compute in ("f64", "f32"):
        tok_s, dt, rows, chunks = bench.cpu_baseline_injected(wl, W, 2, target_s=0.2, compute=compute)
        assert rows == [0, wl.batch - 1]
        assert chunks >= 1 and dt >= 0.2 and tok_s > 0
        assert abs(tok_s - len(rows) * wl.cfg.S * chunks / dt) < 1e-6 * tok_s


def test_profile_records_name_only_committed_programs():
    """Every counter summary under profiles/ states the commands that made
    it; they run bench.py or a one-line torch copy, nothing else."""
    import glob
    import json
    recs = glob.glob(os.path.join(ROOT, "profiles", "*.json"))
    assert recs
    for path in recs:
        rec = json.load(open(path))
        assert rec["source_files"] and len(rec["source_sha256"]) == 64
        for f in rec["source_files"]:
            assert os.path.exists(os.path.join(ROOT, f)), f
        for cmd in rec["commands"]:
            prog = cmd.split(" -- ", 1)[1]
            assert prog.startswith("python bench.py ") or prog.startswith("python -c \"import torch;"), prog
            assert "_work" not in cmd


def test_stale_or_unknown_profiles_are_not_reported():
    import dataclasses
    import photon_inputs as pi
    bench = _bench()
    wl = dataclasses.replace(pi.get(5), name="no such workload")
    assert bench.measured_traffic(wl, "attn_top") == (None, None, None)
    assert bench.measured_counters(wl) is None
