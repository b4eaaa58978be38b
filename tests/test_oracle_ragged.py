"""Ragged draft lengths through the oracle: the pages' counter examples with
draft lengths that differ per request, agreement with the uniform entry point,
the accepted-length histogram, and malformed offsets.

fanout, "Structured output speculative decoding acceptance": the counters and
their ratios do not depend on how many drafts each request proposed, and the
mean acceptance length holds whatever the configured maximum draft length.
"""
import json
import os

import numpy as np
import pytest

from oracle import sd_rates, sd_verify, sd_verify_ragged
from oracle.verify import ST_BAD_OFFSETS

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "counter_examples.json")
V = 64


def _pack(allowed):
    V_ = allowed.shape[-1]
    W = -(-V_ // 32)
    words = np.zeros(allowed.shape[:-1] + (W,), dtype=np.int64)
    for j in range(V_):
        words[..., j >> 5] |= allowed[..., j].astype(np.int64) << (j & 31)
    return words.astype(np.uint32).view(np.int32)


def _greedy_ragged(kinds, ks, seed=0):
    """Greedy requests, request b with ks[b] drafts; kinds as in the uniform
    counter tests.  Returns flat rows, drafts, offsets and a mask."""
    rng = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    B = len(kinds)
    rows = int(off[-1]) + B
    logits = rng.normal(size=(rows, V))
    g = rng.integers(0, V, size=rows)
    logits[np.arange(rows), g] += 20.0            # unique argmax per row
    x = np.zeros(int(off[-1]), dtype=np.int64)
    allowed = np.ones((rows, V), dtype=bool)
    for b, kind in enumerate(kinds):
        for i in range(ks[b]):
            r = off[b] + b + i
            if kind == "accept_all":
                x[off[b] + i] = g[r]
            else:
                x[off[b] + i] = (g[r] + 1 + rng.integers(0, V - 1)) % V
                if kind == "invalid_all":
                    allowed[r, x[off[b] + i]] = False
    return logits, x, off, _pack(allowed)


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_json_schema_run_with_mixed_draft_lengths(golden):
    run = golden["runs"][0]
    cyc = [3, 4, 5, 6, 7]                      # mean 5: the same totals as k = 5
    kinds = ["accept_all"] * 120 + ["invalid_all"] * 40 + ["reject_first"] * 40
    ks = [cyc[b % 5] for b in range(200)]
    logits, x, off, mask = _greedy_ragged(kinds, ks)
    out = sd_verify_ragged(logits, x, off, None, mask, np.zeros(200), seed=1)
    R, I, D, A = (int(v) for v in out["counters"])
    assert (R, I, D, A) == (run["R"], run["I"], run["D"], run["A"])
    r = sd_rates(R, I, A, steps=200)
    assert (r["acceptance"], r["survival"], r["yield"]) == pytest.approx(
        (run["acceptance"], run["survival"], run["yield"]), abs=1e-15)


def test_mean_acceptance_length_with_mixed_draft_lengths(golden):
    m = golden["mean_acceptance_length"]
    # 60 steps accept all of 2, 3 or 4 drafts (180 in all), 40 reject the
    # first of 3 to 8: the maximum length does not enter
    ks = [2 + (b % 3) for b in range(60)] + [3 + (b % 6) for b in range(40)]
    kinds = ["accept_all"] * 60 + ["reject_first"] * 40
    logits, x, off, _ = _greedy_ragged(kinds, ks, seed=3)
    out = sd_verify_ragged(logits, x, off, None, None, np.zeros(100), seed=3)
    A = int(out["counters"][3])
    assert A == m["A"]
    assert sd_rates(int(out["counters"][0]), 0, A, m["steps"])["mean_acceptance_length"] == \
        pytest.approx(m["value"], abs=1e-15)
    h = out["accept_histogram"]
    assert len(h) == 9 and h[0] == 40 and h[2] == 20 and h[3] == 20 and h[4] == 20


def _random_batch(B, k, V_, rng):
    logits = rng.normal(scale=2.0, size=(B, k + 1, V_)).astype(np.float32)
    q = rng.dirichlet(np.ones(V_), size=(B, k))
    x = np.array([[rng.choice(V_, p=q[b, i]) for i in range(k)] for b in range(B)])
    allowed = rng.random((B, k + 1, V_)) < 0.7
    allowed[..., 0] = True
    T = np.array([1.0, 0.7, 0.0, 1.3, 0.0, 0.9][:B])
    return logits, x, q, _pack(allowed), T


def test_uniform_offsets_reproduce_the_uniform_entry_point():
    rng = np.random.default_rng(7)
    B, k, V_ = 6, 3, 50
    logits, x, q, mask, T = _random_batch(B, k, V_, rng)
    top_k = np.array([0, 5, 0, 2, 0, 0])
    u = sd_verify(logits, x, q, mask, T, seed=11, top_k=top_k)
    off = np.arange(B + 1) * k
    r = sd_verify_ragged(logits.reshape(-1, V_), x.reshape(-1), off, q.reshape(-1, V_),
                         mask.reshape(B * (k + 1), -1), T, seed=11, top_k=top_k)
    assert np.array_equal(r["out_tokens"], u["out_tokens"].reshape(-1))
    assert np.array_equal(r["num_accepted"], u["num_accepted"])
    assert np.array_equal(r["counters"], u["counters"])
    assert np.array_equal(r["row_lse"], u["row_lse"].reshape(-1), equal_nan=True)
    assert np.array_equal(r["accept_prob"], u["accept_prob"].reshape(-1), equal_nan=True)
    assert np.array_equal(r["accept_histogram"], u["accept_histogram"])


def test_each_request_matches_a_uniform_call_of_its_own_length():
    rng = np.random.default_rng(9)
    ks = [0, 3, 1, 5, 2, 4]
    B, V_ = len(ks), 40
    off = np.concatenate([[0], np.cumsum(ks)])
    rows = off[-1] + B
    logits = rng.normal(scale=2.0, size=(rows, V_))
    q = rng.dirichlet(np.ones(V_), size=off[-1])
    x = np.array([rng.choice(V_, p=q[t]) for t in range(off[-1])])
    T = np.array([1.0, 0.0, 0.8, 1.2, 0.0, 0.6])
    r = sd_verify_ragged(logits, x, off, q, None, T, seed=5)
    for b, k in enumerate(ks):
        r0 = off[b] + b
        u = sd_verify(logits[r0:r0 + k + 1][None], x[off[b]:off[b + 1]][None],
                      q[off[b]:off[b + 1]][None], None, T[b:b + 1], seed=5, request_ids=[b])
        assert np.array_equal(r["out_tokens"][r0:r0 + k + 1], u["out_tokens"][0])
        assert r["num_accepted"][b] == u["num_accepted"][0]


def test_histogram_is_the_count_of_accepted_lengths():
    rng = np.random.default_rng(13)
    ks = list(rng.integers(0, 7, size=40))
    B, V_ = len(ks), 30
    off = np.concatenate([[0], np.cumsum(ks)])
    logits = rng.normal(scale=1.0, size=(off[-1] + B, V_))
    x = rng.integers(0, V_, size=off[-1])
    x[::3] = 0
    logits[:, 0] += 3.0                        # drafts of token 0 are often accepted
    T = np.where(rng.random(B) < 0.3, 0.0, 1.0)
    r = sd_verify_ragged(logits, x, off, None, None, T, seed=2, max_draft=6)
    na = r["num_accepted"]
    assert np.array_equal(r["accept_histogram"], np.bincount(na, minlength=7))
    assert int(r["accept_histogram"].sum()) == B
    # accepted drafts per position follow from the histogram
    per_position = [int((na > i).sum()) for i in range(6)]
    assert per_position == [int(r["accept_histogram"][i + 1:].sum()) for i in range(6)]
    assert int(r["counters"][3]) == int(na.sum())
    assert int(r["counters"][0]) == int(sum(ks))


def test_inconsistent_offsets_void_the_call():
    rng = np.random.default_rng(4)
    V_ = 20
    B, total = 5, 11
    logits = rng.normal(size=(total + B, V_))
    x = rng.integers(0, V_, size=total)
    T = np.ones(B)
    good = np.array([0, 2, 4, 6, 9, 11])
    r = sd_verify_ragged(logits, x, good, None, None, T, seed=1, max_draft=4)
    assert r["status"] == 0 and int(r["counters"][0]) == total
    for off, kw in [([0, 2, 1, 6, 9, 11], {}),                    # runs backwards
                    ([0, 2, 4, 6, 9, 11], {"max_draft": 2}),       # a request above max_draft
                    ([1, 2, 4, 6, 9, 11], {}),                    # does not start at 0
                    ([0, 2, 4, 6, 9, 12], {"total_drafts": 11})]:  # does not end at the total
        kw.setdefault("max_draft", 4)
        off = np.array(off)
        lg = logits if int(off[-1]) == total or "total_drafts" in kw else \
            rng.normal(size=(int(off[-1]) + B, V_))
        xx = x if lg is logits else rng.integers(0, V_, size=int(off[-1]))
        r = sd_verify_ragged(lg, xx, off, None, None, T, seed=1, **kw)
        assert list(r["request_status"]) == [ST_BAD_OFFSETS] * B
        assert list(r["num_accepted"]) == [-1] * B
        assert list(r["counters"]) == [0, 0, 0, 0] and int(r["accept_histogram"].sum()) == 0
        assert np.all(r["out_tokens"] == -1)


def test_zero_length_request_is_a_bonus_draw():
    rng = np.random.default_rng(1)
    V_ = 25
    logits = rng.normal(size=(1, V_))
    r = sd_verify_ragged(logits, np.zeros(0, dtype=np.int64), [0, 0], None, None, [1.0], seed=9)
    u = sd_verify(logits[None], np.zeros((1, 0), dtype=np.int64), None, None, [1.0], seed=9)
    assert r["out_tokens"][0] == u["out_tokens"][0, 0] and r["num_accepted"][0] == 0
    assert list(r["counters"]) == [0, 0, 0, 0] and list(r["accept_histogram"]) == [1]
