"""Host-side pieces of bench.py (no GPU): byte accounting, the counter-summary
read-back and its staleness guard, and the one-GPU contract."""

import os
import subprocess
import sys

import numpy as np

import bench
import oracle
from paged_kv_cache_410_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_tiny_by_hand():
    spec = workloads.CONFIGS["tiny"]
    tb = workloads.make_tables(spec, oracle.BlockManager)
    got = bench.algorithmic_bytes(spec, tb)
    ctx = [1, 17, 100, 250]
    assert tb.context_lens.tolist() == ctx
    e, D, H = 4, 64, 8
    kv = sum(ctx) * H * D * 2 * e
    qo = 2 * 4 * H * D * e
    meta = 4 * (sum((c + 15) // 16 for c in ctx) + 4)
    assert got["decode"] == kv + qo + meta
    assert got["write"] == 4 * 4 * H * D * e          # 4 new tokens, K and V, read + write
    assert got["copy"] == 0
    assert got["flops"] == 4 * sum(ctx) * H * D


def test_unique_bytes_count_shared_rows_once():
    spec = workloads.CONFIGS["tiny"]
    tb = workloads.make_tables(spec, oracle.BlockManager)
    # no sharing in the tiny workload: unique K/V bytes equal the algorithmic K/V bytes
    kv_q = bench.unique_decode_bytes(spec, tb)
    nb = bench.algorithmic_bytes(spec, tb)
    assert kv_q == nb["decode"] - 4 * (sum((c + 15) // 16 for c in tb.context_lens.tolist()) + 4)


def test_traffic_readback_and_staleness(tmp_path, monkeypatch):
    sha = bench.decode_sources_sha()
    (tmp_path / "pa_decode_x_pmc.md").write_text(
        f"traffic_bytes_per_launch: 123456\ndecode_sources_sha: {sha}\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.read_traffic("x") == (123456.0, "ok")
    (tmp_path / "pa_decode_x_pmc.md").write_text(
        "traffic_bytes_per_launch: 123456\ndecode_sources_sha: 0000000000000000\n")
    val, why = bench.read_traffic("x")
    assert val is None and "changed" in why
    assert bench.read_traffic("missing")[0] is None


def test_committed_counter_summary_parses():
    path = os.path.join(ROOT, "profiles", "pa_decode_13b_pmc.md")
    if not os.path.exists(path):
        return
    val, why = bench.read_traffic("13b")
    assert why in ("ok", "decode sources changed since the counters were taken")
    if val is not None:
        assert 1.5e9 < val < 1.8e9


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert np.isscalar(r.returncode)


def _host_inputs(spec, tb):
    vals = workloads.make_values(spec, tb.NB, len(tb.slots))
    conv = (lambda t: t.numpy()) if spec.dtype == "f32" else workloads.to_bits
    return conv(vals.q), conv(vals.k_cache), conv(vals.v_cache)


def test_cpu_baseline_decode_whole_step():
    spec = workloads.CONFIGS["tiny"]
    tb = workloads.make_tables(spec, oracle.BlockManager)
    q, k, v = _host_inputs(spec, tb)
    out, rows, cpu = bench.cpu_baseline((q, k, v), spec, tb, budget_s=0.0)
    assert rows == slice(0, 4) and out.shape == (4, 8, 64)
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert cpu["sample"].startswith("the whole tiny")
    np.testing.assert_array_equal(out, oracle.decode(q, k, v, tb.block_tables, tb.context_lens,
                                                     spec.scale))


def test_cpu_baseline_chunk_sample_is_a_prefix(monkeypatch):
    from paged_kv_cache_410_amd.workloads import Spec
    spec = Spec("mq", "f32", 5, 2, 2, 64, seed=40, lengths=("uniform", 20, 60),
                chunk=("uniform", 2, 6))
    tb = workloads.make_tables(spec, oracle.BlockManager)
    q, k, v = _host_inputs(spec, tb)
    ctx = tb.context_lens.astype(np.int64)
    n = np.diff(tb.query_start).astype(np.int64)
    work = (n * (ctx - n) + n * (n + 1) // 2) * spec.Hq * spec.D * 2
    monkeypatch.setattr(bench, "ORACLE_WORK_CAP", float(work[:2].sum()))
    out, rows, cpu = bench.cpu_baseline((q, k, v), spec, tb, budget_s=0.0)
    assert rows == slice(0, int(tb.query_start[2]))
    assert "first 2 of 5" in cpu["sample"]
    full = oracle.multi_query(q, k, v, tb.block_tables, tb.context_lens, tb.query_start,
                              spec.scale)
    np.testing.assert_array_equal(out, full[rows])


def test_chunk_bytes_and_flops_by_hand():
    from paged_kv_cache_410_amd.workloads import Spec
    spec = Spec("mq", "bf16", 2, 4, 2, 128, seed=41, lengths=("fixed", [40, 7]),
                chunk=("uniform", 3, 3))
    tb = workloads.make_tables(spec, oracle.BlockManager)
    nb = bench.algorithmic_bytes(spec, tb)
    assert tb.query_start.tolist() == [0, 3, 6]
    # rows attend over 38, 39, 40 and 5, 6, 7 tokens
    assert nb["flops"] == 4 * (38 + 39 + 40 + 5 + 6 + 7) * 4 * 128
    kv = (40 + 7) * 2 * 128 * 2 * 2
    assert nb["decode"] == kv + 2 * 6 * 4 * 128 * 2 + 4 * (3 + 1 + 2) + 4 * 3
