"""GPU: every workload of bench.py at small sizes, so that a change of the
library's interface that breaks the benchmark fails here first.  The numbers
are not checked beyond being positive and finite; each run also reads the
device error word and raises if a kernel reported invalid input."""

import math

import pytest

import bench

pytestmark = pytest.mark.gpu


def _positive(x):
    return isinstance(x, (int, float)) and math.isfinite(x) and x > 0


def test_long_context_step():
    r = bench.run_context(4096, steps=3, warmup=1, kernel_reps=1, seed=11)
    assert _positive(r["steps_per_s"]) and _positive(r["graph_only_ms_per_step"])
    assert all(_positive(v) for v in r["us_per_layer"].values())
    assert r["num_splits"] >= 1


def test_speculative_verify():
    r = bench.run_speculative(L0=6000, steps=3, warmup=1, kernel_reps=1, seed=12)
    assert _positive(r["steps_per_s"]) and 0 <= r["accepted_per_step"] <= 4


def test_agentic_turns_with_the_prefix_cache():
    r = bench.run_agentic(first_turn=3000, turns=3, turn_len=5, kernel_reps=1, seed=13)
    assert _positive(r["steps_per_s"]) and r["steps"] == 15
    assert r["prefix_cache"]["turn_boundaries"] == 2 and r["prefix_cache"]["hit_rate"] > 0.9


@pytest.mark.parametrize("cascade", [True, False])
def test_prefix_shared(cascade):
    r = bench.run_prefix_shared(n_seqs=4, prefix=3000, max_suffix=300, steps=3, warmup=1, kernel_reps=1, seed=14,
                                cascade=cascade)
    assert _positive(r["steps_per_s"]) and _positive(r["tokens_per_s"])


def test_gdn_prefill():
    r = bench.run_gdn_prefill(lengths=(100, 200), reps=2, seed=15)
    assert _positive(r["100"]["us_per_layer"]) and _positive(r["200"]["us_per_layer"])
