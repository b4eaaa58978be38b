"""Degenerate and malformed inputs of the oracle: status bits, k = 0, B = 0,
top-k at or beyond the support, rows with one allowed token."""
import numpy as np

from oracle import sd_verify
from oracle import verify as ov


def _base(B=4, k=3, V=50, seed=0):
    rng = np.random.default_rng(seed)
    l = rng.normal(size=(B, k + 1, V))
    x = rng.integers(0, V, size=(B, k))
    return l, x


def test_empty_batch():
    out = sd_verify(np.zeros((0, 4, 10)), np.zeros((0, 3), int), None, None, np.zeros(0))
    assert out["out_tokens"].shape == (0, 4)
    assert list(out["counters"]) == [0, 0, 0, 0] and out["status"] == 0


def test_k_zero_samples_bonus_only():
    rng = np.random.default_rng(1)
    l = rng.normal(size=(300, 1, 6))
    out = sd_verify(l, np.zeros((300, 0), int), None, None, np.ones(300), seed=4)
    assert np.all(out["num_accepted"] == 0)
    assert np.all((out["out_tokens"][:, 0] >= 0) & (out["out_tokens"][:, 0] < 6))
    assert list(out["counters"]) == [0, 0, 0, 0]


def test_status_bits_and_error_outputs():
    l, x = _base()
    T = np.ones(4)
    x_bad = x.copy(); x_bad[0, 1] = 50
    out = sd_verify(l, x_bad, None, None, T)
    assert out["request_status"][0] == ov.ST_DRAFT_ID and out["status"] == ov.ST_DRAFT_ID
    assert np.all(out["out_tokens"][0] == -1) and out["num_accepted"][0] == -1
    assert np.all(out["request_status"][1:] == 0)
    assert int(out["counters"][0]) == 3 * 3          # the bad request is not counted

    for bad_T in (-1.0, np.nan, np.inf):
        T2 = T.copy(); T2[2] = bad_T
        assert sd_verify(l, x, None, None, T2)["request_status"][2] == ov.ST_TEMPERATURE

    l2 = l.copy(); l2[1, 3, 7] = np.nan
    assert sd_verify(l2, x, None, None, T)["request_status"][1] == ov.ST_BAD_LOGIT
    l3 = l.copy(); l3[1, 0, 7] = np.inf
    assert sd_verify(l3, x, None, None, T)["request_status"][1] == ov.ST_BAD_LOGIT
    l4 = l.copy(); l4[3, 2, :] = -np.inf
    assert sd_verify(l4, x, None, None, T)["request_status"][3] == ov.ST_EMPTY_ROW

    q = np.full((4, 3, 50), 1.0 / 50)
    q[2, 0, x[2, 0]] = np.nan
    assert sd_verify(l, x, q, None, T)["request_status"][2] == ov.ST_BAD_DRAFT_PROB


def test_nan_under_a_masked_token_is_ignored():
    l, x = _base(B=1, k=1, V=40)
    l[0, 0, 5] = np.nan
    allowed = np.ones((1, 2, 40), bool)
    allowed[0, 0, 5] = False
    x[0, 0] = 6
    words = np.zeros((1, 2, 2), np.int64)
    for j in range(40):
        words[..., j >> 5] |= allowed[..., j].astype(np.int64) << (j & 31)
    out = sd_verify(l, x, None, words.astype(np.uint32).view(np.int32), np.ones(1))
    assert out["status"] == 0


def test_all_masked_row_is_an_error():
    l, x = _base(B=1, k=1, V=40)
    words = np.full((1, 2, 2), -1, np.int32)
    words[0, 1, :] = 0
    out = sd_verify(l, x, None, words, np.ones(1))
    assert out["request_status"][0] == ov.ST_EMPTY_ROW


def test_top_k_at_or_above_support_changes_nothing():
    l, x = _base(B=20, k=3, V=30, seed=5)
    T = np.full(20, 0.8)
    a = sd_verify(l, x, None, None, T, seed=3)
    for tk in (30, 31, 10**6):
        b = sd_verify(l, x, None, None, T, seed=3, top_k=np.full(20, tk))
        assert np.array_equal(a["out_tokens"], b["out_tokens"])
        assert np.array_equal(a["row_lse"], b["row_lse"])


def test_top_k_one_emits_the_maximum():
    l, x = _base(B=50, k=2, V=30, seed=6)
    out = sd_verify(l, x, None, None, np.ones(50), seed=8, top_k=np.ones(50, int))
    for b in range(50):
        a = out["num_accepted"][b]
        assert out["out_tokens"][b, a] == np.argmax(l[b, a])


def test_single_allowed_token_is_always_accepted():
    rng = np.random.default_rng(7)
    B, k, V = 30, 3, 64
    l = rng.normal(size=(B, k + 1, V))
    x = rng.integers(0, V, size=(B, k))
    words = np.zeros((B, k + 1, 2), np.int64)
    for b in range(B):
        for i in range(k):
            words[b, i, x[b, i] >> 5] |= 1 << (x[b, i] & 31)
        words[b, k, 0] = 1
    out = sd_verify(l, x, None, words.astype(np.uint32).view(np.int32), np.ones(B), seed=2)
    assert np.all(out["num_accepted"] == k)
    assert np.all(out["out_tokens"][:, k] == 0)
    assert np.all(out["accept_prob"] == 1.0)


def test_dense_q_zero_at_draft_accepts_positive_p():
    l, x = _base(B=5, k=2, V=20, seed=9)
    q = np.full((5, 2, 20), 1.0 / 19)
    for b in range(5):
        q[b, 0, x[b, 0]] = 0.0
    out = sd_verify(l, x, q, None, np.ones(5), seed=1)
    assert np.all(out["accept_prob"][:, 0] == 1.0)
    assert np.all(out["num_accepted"] >= 1)


def test_greedy_ignores_temperature_path_and_top_k():
    l, x = _base(B=10, k=3, V=40, seed=10)
    a = sd_verify(l, x, None, None, np.zeros(10), seed=1)
    b = sd_verify(l, x, None, None, np.zeros(10), seed=2, top_k=np.full(10, 2))
    assert np.array_equal(a["out_tokens"], b["out_tokens"])   # no randomness, top-k moot
