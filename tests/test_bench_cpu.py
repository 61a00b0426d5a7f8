"""bench.py's measurement arithmetic and its command-line contract, on the
CPU: the algorithmic byte and flop counts behind the GB/s and TFLOP/s figures
(worked by hand for the dense8 workload), the counter-summary lookup that
feeds roofline.traffic, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_dense8_by_hand():
    # 4096 tokens of 4096 bf16 values, K = 2, every pair kept (M = 8192):
    # dispatch reads 4096 rows (33,554,432 B), writes 8192 (67,108,864 B) and
    # moves 12 index bytes per pair (98,304 B); combine is the mirror with
    # 8 index bytes per pair (65,536 B)
    cfg = dict(N=4096, d=4096, K=2)
    disp, comb = bench.algorithmic_bytes(cfg, 8192, 2)
    assert disp == 33554432 + 67108864 + 98304 == 100761600
    assert comb == 67108864 + 33554432 + 65536 == 100728832


def test_algorithmic_bytes_follow_kept_rows():
    # dropped pairs move no row: with half the pairs kept the row bytes halve
    cfg = dict(N=1000, d=64, K=4)
    full, _ = bench.algorithmic_bytes(cfg, 4000, 2)
    half, _ = bench.algorithmic_bytes(cfg, 2000, 2)
    assert full - half == 2000 * 64 * 2


def test_ffn_flops_by_hand():
    # gate and up: 2 x (2 d ffn) per row; down: 2 d ffn per row
    cfg = dict(d=4096, ffn=14336)
    assert bench.ffn_flops(cfg, 8192) == 6 * 8192 * 4096 * 14336 == 2.886218022912e12


def test_traffic_lookup_checks_workload_layout_and_source(tmp_path):
    digest = bench.source_digest(bench.FFN_SOURCES["packed"])
    good = {"workload": "dense8", "weights": "packed", "source_sha256_16": digest,
            "bytes_per_call": 123.0}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(good))
    assert bench.load_traffic(str(p), "dense8", "packed") == 123.0
    assert bench.load_traffic(str(p), "fine128_zipf_c1.25", "packed") is None
    assert bench.load_traffic(str(p), "dense8", "plain") is None
    p.write_text(json.dumps(dict(good, source_sha256_16="0" * 16)))
    assert bench.load_traffic(str(p), "dense8", "packed") is None
    assert bench.load_traffic(str(tmp_path / "missing.json"), "dense8", "packed") is None


def test_source_digest_ignores_comments_and_spacing(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text("int f(int x) { return x + 1; }  // one\n")
    b.write_text("/* two */\nint f(int x)   {\n  return x + 1;\n}\n")
    assert bench.source_digest([str(a)]) == bench.source_digest([str(b)])
    b.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest([str(a)]) != bench.source_digest([str(b)])


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_ffn_and_route_bytes_by_hand():
    # dense8: 8 experts with rows, each 3 x 4096 x 14336 bf16 weights
    # (2,818,572,288 B in all), x_perm read and y_perm written
    # (2 x 8192 x 4096 x 2 B) and h written and read (2 x 8192 x 14336 x 2 B)
    cfg = dict(N=4096, d=4096, ffn=14336, E=8, K=2)
    assert bench.ffn_bytes(cfg, 8192, 8, 2) == 2818572288 + 134217728 + 469762048
    # experts without rows stream no weights
    assert bench.ffn_bytes(cfg, 8192, 8, 2) - bench.ffn_bytes(cfg, 8192, 7, 2) == \
        3 * 4096 * 14336 * 2
    # routing reads N x E fp32 logits and writes K ids and K weights per token
    assert bench.route_bytes(cfg) == 4096 * 8 * 4 + 4096 * 2 * 8
