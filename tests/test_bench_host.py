"""Host-side checks of bench.py's arithmetic (no GPU): the algorithmic bytes
and flops its rooflines divide by, the rule that counter traffic is used only
while the kernel sources are unchanged, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench
from gated_delta_rule_prologue_amd.configs import BY_NAME

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def lm():
    w = BY_NAME["lm-130m-layer"]
    return w, 8, 8 * 2048


def test_forward_bytes_match_the_workload_table():
    """The LM layer (B=8, T=2048, H=6, dk=dv=128, L=4, bf16): the prologue moves
    251.9 MB and the scan 129.4 MB per step, over 98,304 head-tokens."""
    w, n, T = lm()
    work = bench.algorithmic_work(w, n, T, 2)
    assert work["head_tokens"] == 98304
    assert abs(work["prologue_bytes"] / 1e6 - 251.9) < 0.05
    assert abs(work["scan_bytes"] / 1e6 - 129.4) < 0.05
    # per head-token: k, u, a, h (two of three slots), b, kw = 2562 B
    assert work["prologue_bytes"] == 2562 * 98304


def test_scan_flops_dense_count():
    """Scan flops per head-token with dense 64 x 64 tiles: 10 C dk + 8 C dv +
    8 dk dv + 2 C^2 / 3 = 281,259 at dk = dv = 128 and 109,227 at 64."""
    w, n, T = lm()
    assert bench.algorithmic_work(w, n, T, 2)["scan_flops"] == 281259 * 98304
    w64 = BY_NAME["recsys-history"]
    assert bench.algorithmic_work(w64, 64, 64 * 1024, 2)["scan_flops"] == 109227 * 64 * 1024 * 4


def test_mfma_counters_only_for_unchanged_sources(monkeypatch):
    m = bench.measured_mfma("scan", "lm-130m-layer")
    if m is None:
        pytest.skip("no MFMA counter summary for the current scan sources")
    assert 0.0 < m[0] < 1.0 and m[1] > 0
    monkeypatch.setattr(bench, "source_sha", lambda paths: "0" * 64)
    assert bench.measured_mfma("scan", "lm-130m-layer") is None


def test_backward_work_models():
    w, n, T = lm()
    assert bench.bwd_flops(w, T) == 37 * 16384 * 6 * 128 * 128
    # inputs read once (q, k, v, u, a, h-slots, g, b, dO: bf16), every gradient
    # written once (fp32), dS_init per chain, conv taps and their gradient
    reads = 2 * (128 + 128 + 128 + 3 * 128 + 3 * 128 + 2 * 128 + 1 + 1 + 128)
    writes = 4 * (128 + 128 + 128 + 3 * 128 * 3 + 1 + 1)
    want = 98304 * (reads + writes) + 4 * 8 * 6 * 128 * 128 + 6 * 128 * 4 * (2 + 4)
    assert bench.bwd_bytes(w, n, T, 2) == want


def test_decode_bytes():
    """One decode step: the fp32 state read and written, plus per chain the
    token's inputs, the history read and written and o."""
    n, H, dk, dv, L = 512, 8, 64, 64, 8
    per_chain = 8 * dk * dv + 2 * (2 * dk + dv + 2 * (L - 1) * dk + (L - 2) * dk + 2 + 6 * dk + dv)
    assert bench.decode_bytes(n, H, dk, dv, L, 2) == n * H * per_chain + H * 4 * dk * 2
    assert bench.decode_bytes(n, H, dk, dv, L, 2) == 149966848


def test_traffic_only_for_unchanged_sources(monkeypatch):
    t = bench.measured_traffic("scan", "lm-130m-layer")
    if t is None:
        pytest.skip("no counter summary for the current scan sources")
    text = open(os.path.join(ROOT, "profiles", "scan_lm-130m-layer_traffic.md")).read()
    line = next(l for l in text.splitlines() if l.startswith("traffic_bytes_per_launch:"))
    assert t == float(line.split(":")[1])
    monkeypatch.setattr(bench, "source_sha", lambda paths: "0" * 64)
    assert bench.measured_traffic("scan", "lm-130m-layer") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout
