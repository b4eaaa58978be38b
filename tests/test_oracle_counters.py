"""The pages' worked counter examples, reproduced through the oracle.

fanout, "Structured output speculative decoding acceptance": R raw drafts,
I grammar-invalidated, D = R - I eligible, A accepted; survival D/R,
acceptance A/D, yield A/R; mean acceptance length 1 + A/steps.  The batches
below are greedy, so every verdict is forced and the counters are exact.
"""
import json
import os

import numpy as np
import pytest

from oracle import sd_rates, sd_verify

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "counter_examples.json")
K, V = 5, 64


def _pack(allowed):
    """[..., V] bool -> [..., ceil(V/32)] int32 words, bit j&31 of word j>>5."""
    V_ = allowed.shape[-1]
    W = -(-V_ // 32)
    words = np.zeros(allowed.shape[:-1] + (W,), dtype=np.int64)
    for j in range(V_):
        words[..., j >> 5] |= allowed[..., j].astype(np.int64) << (j & 31)
    return words.astype(np.uint32).view(np.int32)


def _greedy_batch(kinds, k=K, V=V, seed=0, with_mask=True):
    """kinds: list of 'accept_all' | 'invalid_all' | 'reject_first'."""
    rng = np.random.default_rng(seed)
    B = len(kinds)
    logits = rng.normal(size=(B, k + 1, V))
    g = rng.integers(0, V, size=(B, k + 1))
    for b in range(B):
        for i in range(k + 1):
            logits[b, i, g[b, i]] += 20.0          # unique argmax
    x = np.zeros((B, k), dtype=np.int64)
    allowed = np.ones((B, k + 1, V), dtype=bool)
    for b, kind in enumerate(kinds):
        for i in range(k):
            if kind == "accept_all":
                x[b, i] = g[b, i]
            else:
                x[b, i] = (g[b, i] + 1 + rng.integers(0, V - 1)) % V
                if kind == "invalid_all":
                    allowed[b, i, x[b, i]] = False
    mask = _pack(allowed) if with_mask else None
    return logits, x, mask


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _run(kinds, with_mask=True):
    logits, x, mask = _greedy_batch(kinds, with_mask=with_mask)
    out = sd_verify(logits, x, None, mask, np.zeros(len(kinds)), seed=1)
    R, I, D, A = (int(v) for v in out["counters"])
    return R, I, D, A, out


def test_json_schema_run(golden):
    run = golden["runs"][0]
    kinds = ["accept_all"] * 120 + ["invalid_all"] * 40 + ["reject_first"] * 40
    R, I, D, A, out = _run(kinds)
    assert (R, I, D, A) == (run["R"], run["I"], run["D"], run["A"])
    r = sd_rates(R, I, A, steps=len(kinds))
    assert r["acceptance"] == pytest.approx(run["acceptance"], abs=1e-15)
    assert r["survival"] == pytest.approx(run["survival"], abs=1e-15)
    assert r["yield"] == pytest.approx(run["yield"], abs=1e-15)
    # a grammar-invalid draft is never accepted
    assert np.all(out["num_accepted"][120:160] == 0)


def test_unconstrained_run(golden):
    run = golden["runs"][1]
    kinds = ["accept_all"] * 120 + ["reject_first"] * 80
    R, I, D, A, _ = _run(kinds, with_mask=False)
    assert (R, I, D, A) == (run["R"], run["I"], run["D"], run["A"])
    assert sd_rates(R, I, A, 1)["acceptance"] == pytest.approx(run["acceptance"], abs=1e-15)


def test_third_run(golden):
    run = golden["runs"][2]
    kinds = ["accept_all"] * 150 + ["reject_first"] * 50
    R, I, D, A, _ = _run(kinds)
    assert (R, I, D, A) == (run["R"], run["I"], run["D"], run["A"])
    assert sd_rates(R, I, A, 1)["acceptance"] == pytest.approx(run["acceptance"], abs=1e-15)
    assert A - golden["runs"][0]["A"] == run["accepted_more_than_json_schema"]


def test_mean_acceptance_length(golden):
    m = golden["mean_acceptance_length"]
    # 100 verification steps of k=3 drafts: 60 accept all three, 40 reject first
    logits, x, _ = _greedy_batch(["accept_all"] * 60 + ["reject_first"] * 40, k=3)
    out = sd_verify(logits, x, None, None, np.zeros(100), seed=3)
    A = int(out["counters"][3])
    assert A == m["A"]
    assert sd_rates(int(out["counters"][0]), 0, A, m["steps"])["mean_acceptance_length"] == \
        pytest.approx(m["value"], abs=1e-15)


def test_rates_reject_inconsistent_counters():
    with pytest.raises(ValueError):
        sd_rates(10, 2, 9, 1)
    r = sd_rates(0, 0, 0, 0)
    assert r["survival"] is None and r["acceptance"] is None and r["mean_acceptance_length"] is None
