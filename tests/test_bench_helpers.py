"""Host-side helpers of bench.py (CPU): executed-FLOP count of a mask, the sampled query blocks the oracle checks,
the logit bound and the softmax mode it selects, and the timing summary."""
import importlib.util
import os

import numpy as np
import pytest

from bounds import STATIC_LIMIT, pair_bound, spike_to_bound

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_helpers_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_executed_flops_of_an_all_ones_mask_is_the_dense_count(bench):
    N, heads, d = 4800, 3, 96                       # 38 blocks, the last one 64 tokens
    nb = -(-N // 128)
    ones = np.ones((heads, nb, nb), dtype=np.uint8)
    assert bench.executed_flops(ones, N, d=d) == 4.0 * N * N * d * heads


def test_executed_flops_counts_each_kept_pair_by_its_block_sizes(bench):
    N, d = 300, 96                                  # blocks of 128, 128, 44
    m = np.zeros((1, 3, 3), dtype=np.uint8)
    m[0, 0, 2] = 1                                  # 128 queries x 44 keys
    m[0, 2, 1] = 1                                  # 44 queries x 128 keys
    m[0, 2, 2] = 1                                  # 44 x 44
    assert bench.executed_flops(m, N, d=d) == 4.0 * d * (128 * 44 + 44 * 128 + 44 * 44)


@pytest.mark.parametrize("nb", [1, 2, 3, 5, 8, 977])
def test_sampled_blocks(bench, nb):
    b = bench.sample_blocks(nb)
    assert b == sorted(set(b)) and len(b) <= 8 and all(0 <= i < nb for i in b)
    assert {0, nb - 1, nb // 2} <= set(b)          # first, ragged last, middle
    if nb >= 8:
        assert len(b) == 8
    assert bench.sample_blocks(nb) == b             # seeded


def test_logit_bound_and_mode(bench):
    rng = np.random.default_rng(3)
    d = 96
    wq = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    wk = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    assert bench.logit_bound(wq, wk, d) == pytest.approx(pair_bound(wq, wk, d), rel=1e-12)
    assert bench.softmax_mode(wq, wk, d) == "static"
    at = spike_to_bound(wq, wk, d, 0, target=STATIC_LIMIT - 1.0)
    past = spike_to_bound(wq, wk, d, 0, target=STATIC_LIMIT + 1.0)
    assert bench.softmax_mode(at, wk, d) == "static"
    assert bench.softmax_mode(past, wk, d) == "online"
    bad = wq.copy()
    bad[3] = np.nan
    assert bench.softmax_mode(bad, wk, d) == "online"


def test_timing_summary(bench):
    s = bench.timing_summary([3.0, 1.0, 2.0, 10.0])
    assert s["min"] == 1.0 and s["median"] == 2.5 and s["mean"] == 4.0
