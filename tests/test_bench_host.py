"""Host-side logic of bench.py (no GPU): the algorithmic bytes and flops per
call, the roofline entry each call gets, the dominant call, the plain-read
yardstick attached to HBM-bound entries, and the per-call HBM byte records
under profiles/ (present, and matching the sources they name)."""

import importlib.util
import json
import os

import pytest

from speculative_decoding_heads_amd import configs as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_step_bytes_at_the_7b_batch1_shape(bench):
    c = C.BY_NAME["llama7b_bs1"]
    ab = bench.alg_bytes(c)
    # head weights once, the LM projection once per pass, prefix + tree K/V and
    # the tree queries once
    assert ab["draft_hidden"] == 4 * 4096 * 4096 * 2
    assert ab["draft_lm"] == ab["verify_lm"] == 32000 * 4096 * 2
    assert ab["tree_attn"] == 2 * 32 * (2048 + 65) * 128 * 2 + 65 * 32 * 128 * 2
    assert sum(ab.values()) == 693657600
    af = bench.alg_flops(c)
    assert af["verify_lm"] == 2 * 65 * 4096 * 32000


def test_roofline_bound_follows_the_ridge(bench):
    c = C.BY_NAME["llama7b_bs16"]
    hbm = bench.call_roofline(c, "draft_lm", 50.0)
    assert hbm["bound"] == "hbm" and hbm["unit"] == "GB/s" and hbm["peak"] == 8000.0
    assert hbm["achieved"] == pytest.approx(262144000 / 50e-6 / 1e9, rel=1e-3)
    mfma = bench.call_roofline(c, "verify_lm", 280.0)
    assert mfma["bound"] == "mfma" and mfma["unit"] == "TFLOP/s" and mfma["peak"] == 2500.0
    assert mfma["frac"] == pytest.approx(2 * 1040 * 4096 * 32000 / 280e-6 / 1e12 / 2500, rel=1e-3)
    assert bench.call_roofline(c, "topk_tree", 9.0) == {"bound": "latency", "avg_launch_us": 9.0}


def test_dominant_call_and_read_yardstick(bench):
    c = C.BY_NAME["llama7b_bs1"]
    per = {"draft_hidden": 26.0, "draft_lm": 47.0, "topk_tree": 60.0, "tree_attn": 20.0,
           "verify_lm": 42.0, "accept_compact": 11.0}
    blk = bench.summarise(c, 0.144, per)
    # a latency-bound call never becomes the roofline entry, however long it takes
    assert blk["roofline"]["kernel"] == "draft_lm"
    rates = {134217728: 5900.0, 262144000: 6400.0}
    bench.attach_read_yardstick(blk, rates)
    r = blk["roofline"]
    assert r["read_yardstick_GBps"] == 6400.0
    assert r["frac_of_read_yardstick"] == pytest.approx(r["achieved"] / 6400.0, abs=1e-4)
    assert blk["rooflines"]["draft_hidden"]["read_yardstick_GBps"] == 5900.0
    assert "read_yardstick_GBps" not in blk["rooflines"]["tree_attn"]   # no rate for its size
    assert blk["value"] == pytest.approx(1000.0 / 0.144, rel=1e-4)


@pytest.mark.parametrize("workload", ["llama7b_bs1", "llama7b_bs16", "vocab128k_ctx32k_bs32"])
def test_traffic_records_match_their_sources(bench, workload):
    for call in ("draft_hidden", "draft_lm", "tree_attn", "verify_lm"):
        path = os.path.join(ROOT, "profiles", f"traffic_{call}_{workload}.json")
        with open(path) as f:
            rec = json.load(f)
        assert rec["call"] == call and rec["workload"] == workload
        # each figure rounded on its own
        assert abs(rec["traffic_bytes_per_launch"]
                   - rec["fetch_bytes_per_launch"] - rec["write_bytes_per_launch"]) <= 2
        # measured within the step's sources: the bench reports it (not null)
        assert bench.measured_traffic(workload, call) == rec["traffic_bytes_per_launch"], (call, path)
        # at least the algorithmic bytes moved
        assert rec["traffic_bytes_per_launch"] >= 0.99 * bench.alg_bytes(C.BY_NAME[workload])[call]
