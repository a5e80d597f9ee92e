"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts behind the roofline
fractions, the source-hash gating of the recorded rocprofv3 counters, and the one-GPU guard."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_counts():
    # decode: fp32 state read + write (2 x 128 x 128 x 4) + bf16 q, k, v, o + fp32 g + beta
    assert bench.decode_bytes_per_update(128, 128, 2) == 2 * 128 * 128 * 4 + 4 * 128 * 2 + 128 * 4 + 4 == 132612
    # prefill per (token, head): bf16 q, k, v read and o written, fp32 g, beta
    assert bench.prefill_bytes_per_token_head(128, 128, 2) == 1540
    # the chunk form's dense 64-tile flops: 2 C^2 (3 dk + 2 dv) + 3 * 2 C dk dv per chunk, / C
    assert bench.prefill_flops_per_token_head(128, 128) == 180224
    assert bench.prefill_flops_per_token_head(64, 64) == (2 * 64 * 64 * (3 * 64 + 2 * 64) + 6 * 64 * 64 * 64) / 64


def _record(tmp_path, payload):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    rec = dict(payload, sources=[str(src)],
               source_sha256=hashlib.sha256(src.read_bytes()).hexdigest())
    path = tmp_path / "rec.json"
    path.write_text(json.dumps(rec))
    return path, src


def test_counted_traffic_follows_the_source_hash(tmp_path):
    path, src = _record(tmp_path, {"traffic_bytes_per_launch": 123.0})
    assert bench.counted_traffic(str(path)) == 123.0
    src.write_text("// kernel source, changed\n")
    assert bench.counted_traffic(str(path)) is None
    assert bench.counted_traffic(str(tmp_path / "missing.json")) is None


def test_counted_mfma_follows_the_source_hash(tmp_path):
    ks = {"intra": {"us": 100.0, "mfma_busy_pct": 10.0, "mfma_flops_bf16": 2e9, "mfma_flops_f32": 0.0},
          "out": {"us": 300.0, "mfma_busy_pct": 20.0, "mfma_flops_bf16": 1e9, "mfma_flops_f32": 1e9}}
    path, src = _record(tmp_path, {"workloads": {"w": ks}})
    got = bench.counted_mfma(str(path), "w", 400.0)
    assert got["executed_mfma_flops"] == 4e9
    assert got["executed_mfma_frac"] == pytest.approx(4e9 / 400e-6 / (bench.BF16_PEAK_TFLOPS * 1e12))
    assert got["mfma_busy_frac"] == pytest.approx((100 * 10 + 300 * 20) / 400 / 100)
    assert bench.counted_mfma(str(path), "other", 400.0) is None
    src.write_text("// changed\n")
    assert bench.counted_mfma(str(path), "w", 400.0) is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_cpu_model_is_a_name_or_none():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m and "\n" not in m)


def test_mtp_bytes_reduce_to_the_decode_count_at_one_token():
    assert bench.mtp_bytes_per_head(128, 128, 1, 2) == bench.decode_bytes_per_update(128, 128, 2)
    assert bench.mtp_bytes_per_head(128, 128, 4, 2) == 131072 + 4 * 1540


def test_counted_prefill_traffic_follows_the_source_hash(tmp_path):
    wl = {"bytes_per_call": 3e8, "per_kernel": {"intra": {"fetch_bytes": 2e8, "write_bytes": 1e8}}}
    path, src = _record(tmp_path, {"workloads": {"w": wl}})
    got = bench.counted_prefill_traffic(str(path), "w", 100.0, 1e8)
    assert got["bytes_per_call"] == 3e8 and got["ratio_to_algorithmic"] == 3.0
    assert got["GBs_at_call_time"] == pytest.approx(3e8 / 100e-6 / 1e9)
    assert got["per_kernel_bytes"] == {"intra": 3e8}
    assert bench.counted_prefill_traffic(str(path), "other", 100.0, 1e8) is None
    src.write_text("// changed\n")
    assert bench.counted_prefill_traffic(str(path), "w", 100.0, 1e8) is None

