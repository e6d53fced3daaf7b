"""Host-side pieces of bench.py: the algorithmic byte and FLOP counts the
roofline divides by, the stage percentiles, and the oracle leg's report."""
import pytest

import bench
import synth


def test_algorithmic_counts_c2():
    a = bench.algorithmic(synth.CONFIGS["c2"])
    # logits read (1,024 rows x 151,936 bf16) and 16 (id, value) pairs written per row
    assert a["topk_bytes"] == 1024 * 151936 * 2 + 1024 * 16 * 8
    # projections: A for every candidate with a successor position (15 of 16 per
    # block), B for all: 2 d r (15,360 + 16,384) rows
    assert a["cand_flop"] == 2 * 2560 * 256 * (64 * 15 * 16 + 64 * 16 * 16)
    # every gathered row once
    assert a["gather_bytes"] == 64 * 16 * 16 * 2560 * 2


class _Ev:
    def __init__(self, t):
        self.t = t

    def elapsed_time(self, other):
        return other.t - self.t


def test_stage_percentiles():
    # 11 steps whose stage k lasts (k + 1) * (1 + i / 10) microseconds
    evs = []
    for i in range(11):
        f = 1 + i / 10
        t = [0.0]
        for k in range(4):
            t.append(t[-1] + (k + 1) * f * 1e-3)
        evs.append([_Ev(x) for x in t])
    p = bench.stage_pcts(evs)
    assert p["gate"] == [pytest.approx(1.1), pytest.approx(1.5), pytest.approx(1.9)]
    assert p["step"][1] == pytest.approx(15.0)
    m = bench.stage_means(evs)
    assert m["pair_walk"] == pytest.approx(6.0)


def test_cpu_baseline_report():
    cfg = synth.CONFIGS["c0"]
    r = bench.cpu_baseline(cfg, synth.make(cfg), run_s=0.2, single_core=True)
    assert r["kind"] == "oracle" and r["unit"] == "blocks/s" and r["value"] > 0 and r["cores"] >= 1
    assert set(r["ms_per_block"]) == {"select_topk", "project", "score_pairs", "walk"}
    assert r["single_core"] is None or r["single_core"]["value"] > 0
    assert "median of 3" in r["sample"] and r["cpu_model"]


def test_headline_is_the_largest_graded_workload():
    assert bench.GRADED == ("c2", "c3", "c4") and bench.HEADLINE == "c4" and bench.LATENCY == "c1"
    assert bench.walk_modes(synth.CONFIGS["c4"]) == [0, 1] and bench.walk_modes(synth.CONFIGS["c3"]) == [1]
    assert bench.dtype_of(synth.CONFIGS["c4"]) == "f32+bf16" and bench.dtype_of(synth.CONFIGS["c2"]) == "bf16"
