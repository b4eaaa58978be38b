"""The GPU parity comparison against planted errors, on the CPU: the helpers
must reject a 1e-4 relative error in an accept probability (also where p(x)
is about 1e-7, as for the one-hot drafts of the ngram workload), a 2e-5 shift
of a row's log-normaliser and any flagged draw in a small call, and accept
agreement at the rounding level of fp32 arithmetic."""
import copy

import numpy as np
import pytest

from parity import assert_parity, close_lse, close_rel, flag_limit, run_oracle
from workloads import make_workload


def _as_gpu(orc):
    """An oracle result dressed as the GPU's outputs (what a perfect kernel
    would return)."""
    return {
        "out_tokens": orc["out_tokens"].astype(np.int32),
        "out_num_accepted": orc["num_accepted"].astype(np.int32),
        "counters": orc["counters"].copy(),
        "status": int(orc["status"]),
        "row_lse": orc["row_lse"].copy(),
        "accept_prob": orc["accept_prob"].copy(),
        "flags": np.zeros(3, dtype=np.int32),
    }


@pytest.fixture(scope="module")
def ngram_case():
    wl = make_workload("ngram", device="cpu", batch=3)
    orc = run_oracle(wl)
    return orc, _as_gpu(orc)


def test_exact_copy_passes(ngram_case):
    orc, gpu = ngram_case
    assert assert_parity(gpu, orc) == []


def test_rounding_level_error_passes(ngram_case):
    orc, gpu = ngram_case
    g = copy.deepcopy(gpu)
    g["accept_prob"] = g["accept_prob"] * (1 + 3e-6)
    g["row_lse"] = g["row_lse"] + 4e-6
    assert_parity(g, orc)


def test_relative_error_in_tiny_p_fails(ngram_case):
    orc, gpu = ngram_case
    acc = orc["accept_prob"]
    b, i = np.unravel_index(np.argmin(np.where(acc > 0, acc, np.inf)), acc.shape)
    assert 0 < acc[b, i] < 1e-5            # a one-hot draft the target finds unlikely
    g = copy.deepcopy(gpu)
    g["accept_prob"][b, i] *= 1 + 1e-4
    with pytest.raises(AssertionError):
        assert_parity(g, orc)
    # an absolute 1e-5 check would have passed it
    assert abs(g["accept_prob"][b, i] - acc[b, i]) <= 1e-5 * max(1.0, acc[b, i])


def test_relative_error_in_large_p_fails(ngram_case):
    orc, gpu = ngram_case
    acc = orc["accept_prob"]
    b, i = np.unravel_index(np.argmax(acc), acc.shape)
    g = copy.deepcopy(gpu)
    g["accept_prob"][b, i] = acc[b, i] * (1 - 1e-4)
    with pytest.raises(AssertionError):
        assert_parity(g, orc)


def test_normaliser_shift_fails(ngram_case):
    orc, gpu = ngram_case
    g = copy.deepcopy(gpu)
    g["row_lse"][1, 2] += 2e-5
    with pytest.raises(AssertionError):
        assert_parity(g, orc)


def test_zero_must_stay_zero():
    assert close_rel([0.0, 0.5], [0.0, 0.5])
    assert not close_rel([1e-30, 0.5], [0.0, 0.5])
    assert close_rel([np.nan], [np.nan]) and not close_rel([0.0], [np.nan])


def test_flag_limit_is_below_1e4_of_positions(ngram_case):
    assert flag_limit(1024) == 0 and flag_limit(6144) == 0 and flag_limit(9999) == 0
    assert flag_limit(10001) == 1 and flag_limit(20000) == 1 and flag_limit(20001) == 2
    orc, gpu = ngram_case
    o = copy.deepcopy(orc)
    o["flag_gumbel"][0] = 1                # one flagged draw in 12 positions
    with pytest.raises(AssertionError):
        assert_parity(gpu, o)


def test_normaliser_bound():
    assert close_lse([14.0 + 9e-6], [14.0]) and not close_lse([14.0 + 1.5e-5], [14.0])
    assert close_lse([3.2e8 + 2.0], [3.2e8]) and not close_lse([3.2e8 + 200.0], [3.2e8])
    assert close_lse([np.inf], [np.inf]) and close_lse([np.nan], [np.nan])
