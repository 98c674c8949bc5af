"""Host-side checks of bench.py (no GPU): it refuses more than one GPU before
touching the device, and its roofline arithmetic gives the algorithmic work
per launch that the measurement notes state for each workload."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.fixture(scope="module")
def bench():
    import bench as b
    return b


def _alg(rec, avg_us):
    # achieved GB/s (or TFLOP/s) x the launch time -> work per launch
    scale = 1e9 if rec["unit"] == "GB/s" else 1e12
    return rec["achieved"] * avg_us * 1e-6 * scale


def test_score_stream_bytes_per_launch(bench):
    from gen.workloads import workload
    w = workload(1)
    rec = bench.dominant_roofline(w, {"score_stream": {"avg_us": 625.0}})
    # 32 x 65,536 key rows of 4 heads x 128 fp32 + 32 indexer queries of 2 KB
    assert round(_alg(rec, 625.0)) == 32 * 65536 * 2048 + 32 * 2048 == 4_295_032_832
    assert rec["bound"] == "hbm" and rec["peak"] == 8000.0
    assert rec["frac"] == pytest.approx(rec["achieved"] / 8000.0)
    # the counter record is used only while the stream's sources are unchanged
    assert rec["traffic"] is None or abs(rec["traffic"] / 4_295_032_832 - 1.0) < 0.01
    rec8 = bench.dominant_roofline(w, {"score_stream_e4m3": {"avg_us": 160.0}}, keys="e4m3")
    assert round(_alg(rec8, 160.0)) == 32 * 65536 * 512 + 32 * 2048 == 1_073_807_360


def test_reindex_gather_bytes_per_launch(bench):
    from gen.workloads import workload
    w = workload(4)
    rec = bench.dominant_roofline(w, {"reindex_score": {"avg_us": 340.0}})
    # 64 sequences: min(2,048, ceil(N / 8)) pool blocks of 8 rows, cut at N,
    # plus the 64 Reindex indexer queries of 2 KB
    assert round(_alg(rec, 340.0)) == 1_037_240 * 2048 + 64 * 2048 == 2_124_398_592
    assert rec["kernel"] == "reindex_score" and rec["bound"] == "hbm"


def test_default_line_is_the_mixed_length_workload(bench):
    from gen.workloads import workload
    w = workload(bench.HEADLINE)
    assert w.name == "c4_mixed_reindex" and w.B == 64 and w.kind == "decode_reindex"
    # the largest of the five workloads that fit one GPU: most entries and key bytes
    assert w.rows == max(workload(i).rows for i in range(5))
    assert w.rows * w.row_width * 4 > 28e9


def test_step_statistics_are_the_median_of_the_steps(bench):
    st = bench.summarize([3.0, 1.0, 2.0, 10.0, 2.5])
    assert st["median_ms"] == 2.5 and st["min_ms"] == 1.0 and st["max_ms"] == 10.0
    assert st["n"] == 5


def test_hierarchical_step_counts_the_full_layer_attention(bench):
    from gen.workloads import workload
    w = workload(3)
    a = bench.step_hbm(w, 1.0)["algorithmic_bytes"]
    keys = 8 * (1 << 20) * 2048 + 8 * 2048                 # Full-layer stream
    gather = 8 * 16384 * 2048 + 8 * 2048                   # Reindex over 2,048 x 8 pools
    layer = 2 * 8 * 64 * 512 * 4 + 8 * 512 * 288 + 8 * 128 * 2 * 512 + 8 * 512 * 4
    assert a == keys + gather + 5 * layer                  # Full + Reindex + 3 Reuse attention


def test_prefill_attention_flops_per_launch(bench):
    from gen.workloads import workload
    w = workload(2)
    rec = bench.mfma_utilisation(w, {"attn": {"avg_us": 1000.0}})["attn"]
    # 4,096 queries x 64 heads x (512 + 128) keys x 512 channels x 2 products x 2 flops
    assert round(_alg(rec, 1000.0)) == 4096 * 64 * 640 * 512 * 4 == 343_597_383_680
    assert rec["peak"] == 2500.0
