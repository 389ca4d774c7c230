"""Host-side pieces of bench.py (CPU only): the one-GPU contract, the
algorithmic flop counts behind the roofline, and the recorded HBM traffic's
guard against stale counters."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_dominant_kernel_flops():
    E, units = 647_168, 4_096
    # one species, folded, large cell: the fused kernel, per edge forward + backward, per receiver M and E_i
    k, phase, flop = bench.dominant_kernel("folded", 1, E, units, 4096)
    assert (k, phase) == ("k_fold_fused", "forward")
    assert flop == (4096 + 8192 + 2048 + 2048 + 2048 + 8192 + 4096) * E + (2 * 16 * 64 * 64 + 2 * 16 * 64) * units
    assert bench.dominant_kernel("folded", 1, E, units, 512)[0] == "k_fold_split"
    assert bench.dominant_kernel("folded", 3, E, units, 5000)[0] == "k_fold_multi"
    assert bench.dominant_kernel("direct", 1, E, units)[0] == "k_backward"
    k, _, flop = bench.dominant_kernel("tabulated", 1, E, units)
    assert k == "k_fold_table"
    assert flop == (2 * 2 * 64 * 10 + 3 * 2048 + 2 * 64) * E + (2 * 16 * 64 * 64 + 2 * 16 * 64) * units


def test_recorded_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    rec = {"k_fold_fused": {"workload": "D4096", "sources_sha256": "0" * 64, "bytes_per_launch": 1.0}}
    p = tmp_path / "hbm_traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.recorded_traffic("k_fold_fused", "D4096") is None
    rec["k_fold_fused"]["sources_sha256"] = bench.sources_digest()
    p.write_text(json.dumps(rec))
    assert bench.recorded_traffic("k_fold_fused", "D4096") == 1.0
    assert bench.recorded_traffic("k_fold_fused", "D512") is None


def test_code_text_drops_comments_and_keeps_code():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* not 3 */\n}\n"
    b = "// a header line\nint f(int x) {\n\n    return 2 * x;\n}   // end\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(a.replace("2 * x", "3 * x"))
    assert bench.code_text('p = "../../include/eec.h";') == 'p = "../../include/eec.h";'
