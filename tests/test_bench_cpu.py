"""bench.py's host-side contract, without a GPU: the refusal of more than one
GPU, the committed traffic records (taken on the current kernel sources, so
bench reports them), and the algorithmic byte count of a W4A16 GEMM."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_w4_bytes_counts_codes_scales_zeros_activations_and_output():
    b = _bench()
    # N = 131072, K = 2048, g = 64, M = 1: codes N*K/2, bf16 scales and zeros
    # 2 * 2 * N * K/g, bf16 A 2*K, bf16 C 2*N
    assert b.w4_bytes(1, 131072, 2048, 64) == 134217728 + 16777216 + 4096 + 262144
    assert b.w4_bytes(4, 128, 256, 64, bias=True) == 128 * 128 + 4 * 128 * 4 + 2 * 4 * 256 + \
        2 * 4 * 128 + 2 * 128


@pytest.mark.parametrize("name,sources,shape", [
    ("traffic_decode_w4_m1_n131072.json", "DECODE_SOURCES", (1, 131072, 2048, 64, False)),
    ("traffic_prefill_w4_m512_n131072.json", "PREFILL_SOURCES", (512, 131072, 2048, 64, True)),
])
def test_committed_traffic_records_are_consistent(name, sources, shape):
    # A record's HBM bytes are its counters times the calibration factors,
    # and its algorithmic bytes are the byte formula of the same shape; bench
    # reports the record only while its kernel sources are unchanged (else
    # null).
    b = _bench()
    with open(os.path.join(ROOT, "profiles", name)) as f:
        rec = json.load(f)
    kib = rec["fetch_size_kib_per_dispatch"] * rec["fetch_factor"] + \
        rec["write_size_kib_per_dispatch"] * rec["write_factor"]
    assert abs(kib * 1024 - rec["hbm_bytes_per_launch"]) / rec["hbm_bytes_per_launch"] < 1e-3
    assert rec["algorithmic_bytes_per_launch"] == b.w4_bytes(*shape[:4], bias=shape[4])
    got = b.load_traffic(name, getattr(b, sources))
    current = rec["source_digest"] == b.source_digest(getattr(b, sources))
    assert got == (rec["hbm_bytes_per_launch"] if current else None)


def test_traffic_is_dropped_when_the_sources_differ(tmp_path, monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "src.hip").write_text("kernel v1")
    rec = {"source_digest": b.source_digest(["src.hip"]), "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles" / "t.json").write_text(json.dumps(rec))
    assert b.load_traffic("t.json", ["src.hip"]) == 123
    (tmp_path / "src.hip").write_text("kernel v2")
    assert b.load_traffic("t.json", ["src.hip"]) is None
