"""Host-side logic of bench.py (no GPU): the one-GPU guard, the per-workload step
defaults and the recorded HBM-traffic line the roofline reads."""
import os
import re
import subprocess
import sys

import bench
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_every_workload_has_default_steps():
    assert set(bench.DEFAULT_STEPS) == set(CONFIGS)
    for name, (warmup, steps) in bench.DEFAULT_STEPS.items():
        assert warmup >= 10 and steps >= 2 * warmup, name


def test_recorded_traffic_line_parses():
    """profiles/hbm_traffic.md holds one machine-readable line for the default
    workload's main sweep; the bench reports its bytes only while the digest
    matches the kernel sources."""
    lines = [ln for ln in open(bench.TRAFFIC_FILE) if ln.startswith("traffic ")]
    assert len(lines) == 1
    m = re.match(r"^traffic (\S+) (\S+) (\d+) ([0-9a-f]{16})\s*$", lines[0])
    assert m and m.group(1) == "mamba370m" and m.group(2) == "scan_bwd_main"
    got = bench.recorded_traffic("mamba370m", "scan_bwd_main")
    assert got is None or got == int(m.group(3))
    assert got == (int(m.group(3)) if m.group(4) == bench.source_digest("scan_bwd_main") else None)
