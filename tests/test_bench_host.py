"""bench.py's host logic (no GPU): committed counter summaries are attached to
a bench line only for the workload and kernel source they were taken on, and
the closed-form work counts agree with direct sums on small shapes."""
import importlib.util
import json
import os
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write_summary(tmp_path, kernel, workload, digest, hbm):
    rec = {"kernel": kernel, "workload": workload, "source_digest": digest,
           "hbm_bytes_per_launch": hbm}
    (tmp_path / f"{kernel}_counters.json").write_text(json.dumps(rec))


def test_counted_traffic_only_for_its_workload_and_source(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    _write_summary(tmp_path, "block_stats", "gqa_prefill_128k", "abc", 1234.0)
    assert bench.counted_traffic("block_stats", "abc", "gqa_prefill_128k") == 1234.0
    assert bench.counted_traffic("block_stats", "abc", "prefill_32k") is None
    assert bench.counted_traffic("block_stats", "changed", "gqa_prefill_128k") is None
    assert bench.counted_traffic("route_topk", "abc", "gqa_prefill_128k") is None


def test_committed_summaries_name_a_workload(bench):
    for name in os.listdir(bench.PROFILES):
        if name.endswith("_counters.json"):
            rec = json.load(open(os.path.join(bench.PROFILES, name)))
            assert rec.get("workload"), name
            assert rec.get("source_digest"), name


def test_counted_mfma_busy_only_on_its_workload(bench):
    d = bench.kernel_source_digest("route_topk.hip", "ssa_common.hpp")
    assert bench.counted_mfma_busy("route_fast_kernel", d, "prefill_32k") is None


@pytest.mark.parametrize("n,B", [(1024, 64), (1000, 64), (4096, 256), (777, 128)])
def test_route_flops_closed_form_matches_sum(bench, n, B):
    d = 16
    wl = SimpleNamespace(seq_len=n, block=B, head_dim=d, batch=2, n_q_heads=3)
    nb = n // B
    pairs = sum(min(nb, (t + 1) // B) for t in range(n))
    assert bench.route_flops(wl) == pytest.approx(2 * 3 * pairs * (2 * d * d + 4 * d))
