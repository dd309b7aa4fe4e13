"""bench.py's command-line contract that can be checked without a GPU."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""          # no JSON line for a refused run


def test_profiled_traffic_matches_the_committed_summary():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.profiled_traffic("attn_step_bf16_zigzag_seq8192_cp4.md", "attn_step.hip")
    # null is allowed only when the kernel source changed after the counters were taken
    text = open(os.path.join(ROOT, "profiles", "attn_step_bf16_zigzag_seq8192_cp4.md")).read()
    assert "traffic_bytes_per_launch:" in text
    if t is not None:
        assert 1e8 < t < 2e8


def test_long_sweep_traffic_matches_the_committed_summary():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.profiled_traffic("attn_step_bf16_long_prefill_1M_cp8_sweep.md", "attn_step.hip")
    text = open(os.path.join(ROOT, "profiles", "attn_step_bf16_long_prefill_1M_cp8_sweep.md")).read()
    assert "traffic_bytes_per_launch:" in text and "--long-sweep-only 1" in text
    if t is not None:
        # at least the algorithmic bytes of a sweep launch (7.01 GB), re-reads below L2 included
        assert 7.0e9 < t < 1.0e11


def test_decode_traffic_matches_the_committed_summary():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.profiled_traffic("decode_bf16_gqa_8shards.md", "decode.hip")
    text = open(os.path.join(ROOT, "profiles", "decode_bf16_gqa_8shards.md")).read()
    assert "traffic_bytes_per_launch:" in text
    if t is not None:
        # K + V of 8 shards x 64 requests x 16384 tokens x 8 kv heads x 128 x bf16, read once
        kv = 2 * 8 * 64 * 16384 * 8 * 128 * 2
        assert kv <= t < 1.01 * kv


def test_merge_traffic_matches_the_committed_summary():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.profiled_traffic("lse_merge_2x8M.md", "lse_merge.hip")
    if t is not None:
        rows = 131072 * 64
        algorithmic = 3 * rows * 129 * 4          # two partials read, one result written
        assert algorithmic <= t < 1.01 * algorithmic


def test_summary_for_another_source_is_not_used():
    sys.path.insert(0, ROOT)
    import bench
    # the ring-step summary carries no hash of decode.hip
    assert bench.profiled_traffic("attn_step_bf16_zigzag_seq8192_cp4.md", "decode.hip") is None


def test_roofline_entry_shape():
    sys.path.insert(0, ROOT)
    import bench
    e = bench.roofline_entry("mfma", 500.0, 2500.0, "TFLOP/s", 123)
    assert e == {"bound": "mfma", "achieved": 500.0, "peak": 2500.0, "unit": "TFLOP/s",
                 "frac": 0.2, "traffic": 123}
    json.dumps(e)


def test_host_index_leg_reports_tokens_per_second():
    # the index calls run on the host, so this leg runs without a GPU too
    sys.path.insert(0, ROOT)
    import bench
    r = bench.host_index_bench()
    assert set(r) == {"cp_partition", "cp_slot_mapping", "cp_reorg_index"}
    for v in r.values():
        assert v["unit"] == "M tokens/s" and v["value"] > 0
    json.dumps(r)
