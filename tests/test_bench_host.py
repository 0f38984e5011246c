"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
consistency of the committed HBM-traffic record with the GEMM source."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "qlora_fine_tuning_amd", "csrc")


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_code_digest_ignores_comments_and_whitespace(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* header */ int f(int x)   { return x + 1; }\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.code_digest(str(a)) == bench.code_digest(str(b))
    assert bench.code_digest(str(a)) != bench.code_digest(str(c))


def test_traffic_record_matches_the_current_gemm_code():
    """profiles/gemm_traffic.json holds the counter figures that bench.py
    reports as roofline.traffic; they are only valid for the gemm.hip code they
    were taken on. A kernel change must come with retaken counters."""
    recs = json.load(open(os.path.join(ROOT, "profiles", "gemm_traffic.json")))
    digest = bench.code_digest(os.path.join(CSRC, "gemm.hip"))
    for rec in recs:
        assert rec["gemm_hip_code_sha256"] == digest, rec["workload_name"]
        got = bench.gemm_traffic(CSRC, rec["workload_name"], rec["dequant_mode"])
        assert got == rec["hbm_bytes_per_launch"] > rec["algorithmic_bytes_per_launch"]
    assert {r["workload_name"] for r in recs} >= {"llama7b_mlp", "mistral7b_qkv"}
    assert bench.gemm_traffic(CSRC, "llama7b_mlp", "fused") is None
