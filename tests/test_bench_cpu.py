"""Host-side contract of bench.py (CPU only; no kernel is launched)."""

import json
import os
import re
import subprocess
import sys

import bench
from paged_kv_cache_362_amd import layouts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def _record():
    text = open(os.path.join(ROOT, bench.TRAFFIC_PROFILE)).read()
    return json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))


def test_traffic_record_is_used_only_for_the_sources_it_was_taken_on(monkeypatch):
    rec = _record()
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["source_hash"])
    for cfg, r in rec["records"].items():
        assert bench.stored_traffic(int(cfg), rec["partition"], rec["fused"]) == \
            r["hbm_bytes_per_launch"]
    # a workload without a record, another form, or changed kernel sources: no figure
    assert bench.stored_traffic(1, rec["partition"], rec["fused"]) is None
    assert bench.stored_traffic(2, 64, rec["fused"]) is None
    assert bench.stored_traffic(2, rec["partition"], not rec["fused"]) is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.stored_traffic(2, rec["partition"], rec["fused"]) is None


def test_traffic_records_are_plausible():
    """HBM bytes per launch within a few % of each workload's algorithmic
    bytes (distinct bytes for the shared prefix, which its cache reuse can
    only lower), and equal to the record's read bytes plus written bytes."""
    from paged_kv_cache_362_amd import sizing
    rec = _record()
    for cfg, r in rec["records"].items():
        b = layouts.make_config(int(cfg))
        cache = sizing.reshape_and_cache_bytes(b.slot_mapping.shape[0], b.num_kv_heads,
                                               b.head_dim, b.elem_bytes)
        alg = sizing.decode_algorithmic_bytes(b.context_lens, b.num_q_heads, b.num_kv_heads,
                                              b.head_dim, b.elem_bytes, b.block_size) + cache
        u = sizing.unique_context_tokens(b.block_tables, b.context_lens, b.block_size)
        distinct = sizing.decode_algorithmic_bytes(
            b.context_lens, b.num_q_heads, b.num_kv_heads, b.head_dim, b.elem_bytes,
            b.block_size, unique_tokens=u) + cache
        assert 0.98 * distinct <= r["hbm_bytes_per_launch"] <= 1.05 * alg
        if distinct == alg:
            assert r["hbm_bytes_per_launch"] <= 1.05 * alg
        assert r["hbm_bytes_per_launch"] == r["read_bytes_from_requests"] + r["write_bytes"]
        # FETCH_SIZE counts 128-byte requests as 64 bytes: the factor is 2
        assert abs(r["fetch_scale"] - 2.0) < 0.01


def test_cpu_baseline_reports_what_it_timed():
    b = layouts.make_config(1)
    cb = bench.cpu_baseline(b, seconds=0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["cores"] == 1
    assert cb["value"] > 0 and cb["seconds"] >= 0.2
    assert "oracle" in cb["sample"]


def test_kernel_trace_record_is_used_only_for_the_sources_it_was_taken_on(monkeypatch, tmp_path):
    """frac_kernel comes from the committed kernel trace only while the kernel
    sources hash to the record's source_hash."""
    rec = {"source_hash": "abcd" * 4, "kernel_avg_us": {"2": 97.0}}
    prof = tmp_path / "trace.md"
    prof.write_text("# trace\n\n```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRACE_PROFILE", "trace.md")
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["source_hash"])
    assert bench.kernel_trace_record()["kernel_avg_us"]["2"] == 97.0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.kernel_trace_record() is None
