"""Host logic of bench.py (no GPU): the repeat statistics and the rule that a
counter-measured traffic figure is reported only for the kernel sources it was
taken on."""
import os

import numpy as np
import pytest

import bench


@pytest.mark.parametrize("n", [1, 2, 7, 10, 31])
def test_spread_matches_numpy_percentiles(n):
    reps = list(np.random.default_rng(n).uniform(0.5, 2.0, n))
    got = bench.spread(reps, scale=4.0)
    want = np.percentile(np.asarray(reps) / 4.0, [10, 50, 90])   # numpy's default: linear
    assert got["repeats"] == n
    assert got["ms_p10"] == pytest.approx(want[0], abs=1e-6)
    assert got["ms_median"] == pytest.approx(want[1], abs=1e-6)
    assert got["ms_p90"] == pytest.approx(want[2], abs=1e-6)
    assert bench.median_of(reps, 4.0) == pytest.approx(np.median(np.asarray(reps) / 4.0), rel=1e-12)


def test_counter_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.counter_traffic("k", [str(src)]) is None          # no summary yet
    (tmp_path / "k_traffic.md").write_text(
        f"source_sha256: `{bench.source_sha([str(src)])}`\n"
        "traffic_bytes_per_launch: 12345\n")
    assert bench.counter_traffic("k", [str(src)]) == 12345
    src.write_text("// kernel v2\n")                                # the kernel changed
    assert bench.counter_traffic("k", [str(src)]) is None


def test_committed_traffic_summaries_match_the_sources():
    # every summary bench.py reads carries the hash of the sources it was taken on;
    # a kernel edit without a new counter pass turns that workload's traffic to null
    for tag, srcs in (("decode_stack_q8_0", bench.STACK_SRCS),
                      ("prefill_down_q4_operator", bench.DOWN_OP_SRCS),
                      ("prefill_layer_q8_0", bench.PREFILL_SRCS),
                      ("decode_batch_q4_layer", bench.BATCH_SRCS),
                      ("attn_prep_q8_0", bench.ATTN_SRCS)):
        assert os.path.exists(os.path.join(bench.PROFILE_DIR, f"{tag}_traffic.md")), tag
        assert bench.counter_traffic(tag, srcs) is not None, f"{tag}: profile older than the sources"
