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


def test_recorded_traffic_lines_parse():
    """profiles/hbm_traffic.md holds machine-readable lines for the default workload's main sweep
    and whole call; the bench reports their bytes only while the digest matches the kernel sources."""
    lines = [ln for ln in open(bench.TRAFFIC_FILE) if ln.startswith("traffic ")]
    assert 1 <= len(lines) <= 2
    for ln in lines:
        m = re.match(r"^traffic (\S+) (\S+) (\d+) ([0-9a-f]{16})\s*$", ln)
        assert m and m.group(1) == "mamba370m" and m.group(2) in ("scan_bwd_main", "ssm_scan_bwd")
        got = bench.recorded_traffic("mamba370m", m.group(2))
        assert got == (int(m.group(3)) if m.group(4) == bench.source_digest(m.group(2)) else None)


def test_source_digest_ignores_comments_and_layout():
    """A comment or whitespace edit keeps the digest (the compiled code is the same); a code edit
    changes it.  Comment markers inside string and character literals are code."""
    src = 'int a = 1;  // note\n/* block */ const char* s = "x//y";\nchar q = \'"\';\n'
    assert bench.code_text(src) == 'int a = 1; const char* s = "x//y"; char q = \'"\';'
    assert bench.code_text(src) == bench.code_text(src.replace("// note", "// another note"))
    assert bench.code_text(src) != bench.code_text(src.replace("1;", "2;"))
    assert len(bench.source_digest("scan_bwd_main")) == 16


def test_roofline_fields_follow_the_published_peaks():
    """The scan roofline: HBM bound against 8 TB/s from the algorithmic bytes and the kernel time;
    the arithmetic against 157.3 TFLOP/s (published fp32) and the 78.6 TFLOP/s non-packed ceiling."""
    cfg = CONFIGS["mamba370m"]
    call, main = bench.scan_bytes(cfg, False)
    assert call == 943996928 and main == 941621248
    r = bench.scan_roofline(cfg, 0.5, 0.7, main, call, 1_400_000_000, 2_300_000_000)
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["achieved"] - main / 0.5e-3 / 1e9) < 0.1
    assert abs(r["frac"] - main / 0.5e-3 / 8e12) < 1e-4
    assert r["traffic"] == 1_400_000_000
    alu = r["alu"]
    tf = 21 * cfg.state_elements / 0.5e-3 / 1e12
    assert abs(alu["achieved_TFLOPs"] - tf) < 1e-3
    assert alu["published_fp32_peak_TFLOPs"] == 157.3 and abs(alu["frac_of_published_peak"] - tf / 157.3) < 1e-4
    assert abs(alu["nonpacked_issue_ceiling_TFLOPs"] - 78.6) < 0.05
    assert abs(r["step"]["frac_of_hbm_peak"] - call / 0.7e-3 / 8e12) < 1e-4
    assert r["step"]["counted_over_algorithmic"] == round(2_300_000_000 / call, 3)
