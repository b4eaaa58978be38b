"""Pins for the oracle's target law, accept/resample rule and sampler.

* softmax, mask and temperature: SciPy's softmax / logsumexp (library routines)
* greedy: brute-force check of "lowest index of the allowed maximum"
* top-k: brute force "fewer than k allowed tokens are strictly larger"
* accept + residual: exact enumeration at V=8 shows every emitted position
  follows the target law (the losslessness the pyshine page claims in
  "Verification: rejection sampling on the GPU", and infra-guide 5.2 section 4.3
  for one-hot drafts)
* the whole sampler: chi-square tests of emitted tokens against p
* two-level Gumbel-max: chi-square against r / sum(r) for several block sizes
* one-hot drafts: the q = None run equals an explicit one-hot q run bit for bit
"""
import math
import numpy as np
import pytest
from scipy import special, stats

from oracle import sd_verify
from oracle import verify as ov


def _pack(allowed):
    V = allowed.shape[-1]
    W = -(-V // 32)
    words = np.zeros(allowed.shape[:-1] + (W,), dtype=np.int64)
    for j in range(V):
        words[..., j >> 5] |= allowed[..., j].astype(np.int64) << (j & 31)
    return words.astype(np.uint32).view(np.int32)


def _softmax_rows(logits, allowed, T):
    out = np.zeros_like(logits)
    for i in range(logits.shape[0]):
        a = allowed[i]
        out[i, a] = special.softmax(logits[i, a] / T)
    return out


# ---------------------------------------------------------------- target law

def test_target_distribution_matches_scipy():
    rng = np.random.default_rng(0)
    for trial in range(20):
        V = int(rng.integers(5, 400))
        l = rng.normal(scale=3.0, size=V)
        allowed = rng.random(V) < 0.6
        allowed[rng.integers(0, V)] = True
        T = float(rng.uniform(0.2, 2.0))
        p, lse = ov.target_distribution(l, allowed, T, 0)
        want = np.zeros(V)
        want[allowed] = special.softmax(l[allowed] / T)
        assert np.allclose(p, want, rtol=1e-13, atol=1e-300)
        assert lse == pytest.approx(special.logsumexp(l[allowed] / T), rel=1e-14)
        assert p.sum() == pytest.approx(1.0, abs=1e-13)


def test_row_lse_and_accept_prob_through_sd_verify():
    rng = np.random.default_rng(1)
    B, k, V = 6, 3, 100
    l = rng.normal(scale=2.0, size=(B, k + 1, V))
    allowed = rng.random((B, k + 1, V)) < 0.5
    allowed[..., 0] = True
    x = rng.integers(0, V, size=(B, k))
    q = rng.dirichlet(np.ones(V), size=(B, k))
    T = rng.uniform(0.5, 1.5, size=B)
    out = sd_verify(l, x, q, _pack(allowed), T, seed=5)
    for b in range(B):
        p = _softmax_rows(l[b], allowed[b], T[b])
        for i in range(k + 1):
            assert out["row_lse"][b, i] == pytest.approx(
                special.logsumexp(l[b, i][allowed[b, i]] / T[b]), rel=1e-13)
        for i in range(k):
            px, qx = p[i, x[b, i]], q[b, i, x[b, i]]
            want = 0.0 if px == 0 else min(1.0, px / qx)
            assert out["accept_prob"][b, i] == pytest.approx(want, rel=1e-12)


def test_greedy_is_lowest_index_of_allowed_max():
    rng = np.random.default_rng(2)
    for trial in range(200):
        V = int(rng.integers(2, 40))
        l = rng.integers(-3, 4, size=V).astype(float)   # many ties
        allowed = rng.random(V) < 0.7
        allowed[rng.integers(0, V)] = True
        g = ov.greedy_choice(l, allowed)
        assert allowed[g]
        for j in range(V):
            if allowed[j]:
                assert l[j] <= l[g]
                if j < g:
                    assert l[j] < l[g]


def test_greedy_scan_accepts_exactly_while_draft_equals_argmax():
    rng = np.random.default_rng(3)
    B, k, V = 64, 4, 30
    l = rng.integers(-2, 3, size=(B, k + 1, V)).astype(float)
    g = np.array([[ov.greedy_choice(l[b, i], np.ones(V, bool)) for i in range(k + 1)]
                  for b in range(B)])
    n_good = rng.integers(0, k + 1, size=B)
    x = g[:, :k].copy()
    for b in range(B):
        if n_good[b] < k:
            x[b, n_good[b]] = (g[b, n_good[b]] + 1) % V
    out = sd_verify(l, x, None, None, np.zeros(B), seed=11)
    assert np.array_equal(out["num_accepted"], n_good)
    for b in range(B):
        a = n_good[b]
        assert list(out["out_tokens"][b, :a]) == list(x[b, :a])
        assert out["out_tokens"][b, a] == g[b, a]
        assert np.all(out["out_tokens"][b, a + 1:] == -1)


def test_top_k_support_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(300):
        V = int(rng.integers(1, 60))
        l = rng.integers(-4, 5, size=V).astype(float)   # ties at the threshold
        allowed = rng.random(V) < 0.8
        allowed[rng.integers(0, V)] = True
        top_k = int(rng.integers(1, V + 3))
        p, _ = ov.target_distribution(l, allowed, 1.0, top_k)
        brute = np.array([allowed[j] and np.sum(allowed & (l > l[j])) < top_k
                          for j in range(V)])
        assert np.array_equal(p > 0, brute)
        # at least top_k tokens kept unless fewer are allowed
        assert brute.sum() >= min(top_k, allowed.sum())


def _top_p_brute(l, allowed, T, top_p):
    """Keep set of top-p by hand: walk tokens from the largest logit down,
    adding probabilities one token at a time, stop once the running mass
    reaches top_p, then keep every token tied with the last one added."""
    idx = [j for j in range(len(l)) if allowed[j] and np.isfinite(l[j])]
    w = {j: math.exp(l[j] / T) for j in idx}
    Z = sum(w.values())
    order = sorted(idx, key=lambda j: -l[j])
    run, last = 0.0, None
    for j in order:
        run += w[j] / Z
        last = l[j]
        if run >= top_p:
            break
    return np.array([j in w and l[j] >= last for j in range(len(l))])


def test_top_p_support_brute_force():
    rng = np.random.default_rng(41)
    for trial in range(400):
        V = int(rng.integers(1, 40))
        l = rng.normal(scale=2.0, size=V)
        if trial % 3 == 0:
            l = np.round(l)                          # ties at the cut
        allowed = rng.random(V) < 0.8
        allowed[rng.integers(0, V)] = True
        T = float(rng.uniform(0.3, 2.0))
        top_p = float(rng.uniform(0.05, 0.99))
        p, _ = ov.target_distribution(l, allowed, T, 0, top_p)
        brute = _top_p_brute(l, allowed, T, top_p)
        flags = []
        ov.target_distribution(l, allowed, T, 0, top_p, flags)
        if not flags[0]:                             # away from the boundary: exact
            assert np.array_equal(p > 0, brute), (trial, top_p)
        kept = p > 0
        assert kept.any()
        # the kept mass reaches top_p and dropping its smallest value would not
        w = np.where(allowed, np.exp(l / T), 0.0)
        w /= w.sum()
        assert w[kept].sum() >= top_p - 1e-12
        vmin = l[kept].min()
        assert w[kept & (l > vmin)].sum() < top_p + 1e-12


def test_top_p_special_cases():
    l = np.array([3.0, 1.0, 1.0, -2.0, 0.5])
    allowed = np.ones(5, bool)
    # a tiny top_p keeps only the largest logit (and its ties)
    p, _ = ov.target_distribution(l, allowed, 1.0, 0, 1e-9)
    assert list(p > 0) == [True, False, False, False, False]
    # a cut that lands on tied tokens keeps both
    w = np.exp(l) / np.exp(l).sum()
    p, _ = ov.target_distribution(l, allowed, 1.0, 0, w[0] + 0.5 * w[1])
    assert list(p > 0) == [True, True, True, False, False]
    # top_p exactly at a cumulative mass is a boundary row, and flagged
    flags = []
    ov.target_distribution(l, allowed, 1.0, 0, float(w[0]), flags)
    assert flags == [1]
    # outside (0, 1) it is off
    for tp in (0.0, 1.0, -0.5, 2.0):
        p, _ = ov.target_distribution(l, allowed, 1.0, 0, tp)
        assert np.all(p > 0)


def test_top_p_after_top_k():
    """top-k first, then top-p over what top-k kept, renormalised."""
    rng = np.random.default_rng(43)
    for trial in range(200):
        V = int(rng.integers(2, 30))
        l = rng.normal(size=V)
        allowed = np.ones(V, bool)
        top_k = int(rng.integers(1, V + 1))
        top_p = float(rng.uniform(0.1, 0.95))
        p, _ = ov.target_distribution(l, allowed, 1.0, top_k, top_p)
        kept_k = np.array([np.sum(l > l[j]) < top_k for j in range(V)])
        brute = _top_p_brute(np.where(kept_k, l, -np.inf), kept_k, 1.0, top_p)
        flags = []
        ov.target_distribution(l, allowed, 1.0, top_k, top_p, flags)
        if not flags[0]:
            assert np.array_equal(p > 0, brute), trial


# ------------------------------------------------- exact law of one position

def _law_of_emitted(p, q, one_hot_x=None):
    """P(emitted token = v) at one position: accept the draft with
    min(1, p/q), else draw from the residual (oracle building blocks)."""
    V = p.shape[0]
    law = np.zeros(V)
    if one_hot_x is not None:
        x = one_hot_x
        a = ov.accept_probability(p[x], 1.0)
        law[x] += a
        if a < 1.0:
            r = ov.residual_weights(p, None, x, True)
            law += (1.0 - a) * r / r.sum()
        return law
    reject_mass = 0.0
    for x in range(V):
        a = ov.accept_probability(p[x], q[x])
        law[x] += q[x] * a
        reject_mass += q[x] * (1.0 - a)
    r = ov.residual_weights(p, q, None, False)
    if reject_mass > 0:
        law += reject_mass * r / r.sum()
    return law


@pytest.mark.parametrize("mode", ["dense", "dense_masked", "dense_topk", "dense_topp", "one_hot"])
def test_exact_enumeration_v8(mode):
    rng = np.random.default_rng(5)
    V, k = 8, 2
    for trial in range(50):
        l = rng.normal(scale=1.5, size=(k + 1, V))
        allowed = np.ones((k + 1, V), bool)
        top_k = 0
        if mode == "dense_masked":
            allowed = rng.random((k + 1, V)) < 0.6
            allowed[:, 0] = True
        if mode == "dense_topk":
            top_k = 3
        top_p = 0.7 if mode == "dense_topp" else 0.0
        T = float(rng.uniform(0.5, 2.0))
        p = np.array([ov.target_distribution(l[i], allowed[i], T, top_k, top_p)[0]
                      for i in range(k + 1)])
        q = rng.dirichlet(np.ones(V) * 0.7, size=k)
        for i in range(k):      # each drafted position, given the earlier ones accepted
            if mode == "one_hot":
                for x in range(V):
                    assert np.allclose(_law_of_emitted(p[i], None, x), p[i], atol=1e-12)
            else:
                assert np.allclose(_law_of_emitted(p[i], q[i]), p[i], atol=1e-12)


def test_enumeration_detects_unclamped_residual():
    """The pin has teeth: p - q without the clamp is not the target law."""
    rng = np.random.default_rng(6)
    p = rng.dirichlet(np.ones(8))
    q = rng.dirichlet(np.ones(8))
    law = np.zeros(8)
    rej = 0.0
    for x in range(8):
        a = ov.accept_probability(p[x], q[x])
        law[x] += q[x] * a
        rej += q[x] * (1 - a)
    r = p - q
    law += rej * r / r.sum()
    assert not np.allclose(law, p, atol=1e-6)


# -------------------------------------------------- the sampler end to end

def _chi2_ok(counts, probs, alpha=1e-3):
    live = probs > 0                  # zero-probability bins are checked separately
    counts, probs = counts[live], probs[live]
    n = counts.sum()
    exp = probs * n
    big = exp >= 5
    obs = list(counts[big])
    e = list(exp[big])
    if (~big).any():
        obs.append(counts[~big].sum())
        e.append(exp[~big].sum())
    obs, e = np.array(obs, float), np.array(e, float)
    if e.size < 2:
        return True
    e *= obs.sum() / e.sum()
    return stats.chisquare(obs, e).pvalue > alpha


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["dense", "one_hot", "masked", "top_k", "top_p"])
def test_chi_square_emitted_tokens(mode):
    rng = np.random.default_rng(10 + ["dense", "one_hot", "masked", "top_k", "top_p"].index(mode))
    B, k, V = 12000, 2, 8
    l1 = rng.normal(scale=1.0, size=(k + 1, V))
    allowed1 = np.ones((k + 1, V), bool)
    top_k = 0
    if mode == "masked":
        allowed1 = rng.random((k + 1, V)) < 0.7
        allowed1[:, :2] = True
    if mode == "top_k":
        top_k = 4
    top_p = 0.6 if mode == "top_p" else 0.0
    T = 0.9
    p = np.array([ov.target_distribution(l1[i], allowed1[i], T, top_k, top_p)[0]
                  for i in range(k + 1)])
    q1 = rng.dirichlet(np.ones(V), size=k)
    logits = np.broadcast_to(l1, (B, k + 1, V))
    x = np.stack([rng.choice(V, size=B, p=q1[i]) for i in range(k)], axis=1)
    q = None if mode == "one_hot" else np.broadcast_to(q1, (B, k, V))
    mask = None if mode != "masked" else np.broadcast_to(_pack(allowed1), (B, k + 1, 1))
    tk = None if mode != "top_k" else np.full(B, top_k)
    tp = None if mode != "top_p" else np.full(B, top_p)
    out = sd_verify(logits, x, q, mask, np.full(B, T), seed=99, top_k=tk, top_p=tp)
    tok, na = out["out_tokens"], out["num_accepted"]
    for i in range(k + 1):
        sel = na >= i
        counts = np.bincount(tok[sel, i], minlength=V)
        assert counts[p[i] == 0].sum() == 0
        assert _chi2_ok(counts, p[i]), (mode, i)


@pytest.mark.parametrize("block", [1, 3, 4, 8])
def test_two_level_gumbel_chi_square(block):
    rng = np.random.default_rng(20 + block)
    r = rng.dirichlet(np.ones(8))
    r[[2, 5]] = 0.0
    n = 15000
    ys = np.array([ov.gumbel_two_level(r, 1234, b, 1, block)[0] for b in range(n)])
    counts = np.bincount(ys, minlength=8)
    assert counts[r == 0].sum() == 0
    assert _chi2_ok(counts, r / r.sum())


@pytest.mark.parametrize("top_k,top_p", [(20, 0.0), (0, 0.7), (50, 0.9), (1, 0.0)])
def test_dense_residual_lives_on_the_kept_set(top_k, top_p):
    """With a top-k or top-p cut, p is zero outside the kept tokens, so the
    dense residual max(p - q, 0) is too: the residual over the kept tokens
    alone equals the residual over the whole row (what the kernels' listed
    lines rely on), for q spread over every token."""
    rng = np.random.default_rng(71 + top_k)
    V = 5000
    for _ in range(5):
        l = rng.normal(0.0, 2.0, V)
        allowed = rng.random(V) < 0.8
        p, _ = ov.target_distribution(l, allowed, 0.8, top_k, top_p)
        q = special.softmax(rng.normal(0.0, 1.0, V))
        r = ov.residual_weights(p, q, -1, one_hot=False)
        kept = p > 0
        assert kept.sum() < allowed.sum()  # the cut removes tokens
        assert np.all(r[~kept] == 0.0)
        r_kept = np.zeros(V)
        r_kept[kept] = np.maximum(p[kept] - q[kept], 0.0)
        assert np.array_equal(r, r_kept)


def test_one_hot_equals_explicit_one_hot_q():
    rng = np.random.default_rng(30)
    B, k, V = 120, 4, 300
    l = rng.normal(scale=2.0, size=(B, k + 1, V))
    x = rng.integers(0, V, size=(B, k))
    for b in range(0, B, 3):          # some drafts at the argmax to get acceptances
        x[b] = np.argmax(l[b, :k], axis=1)
    q = np.zeros((B, k, V))
    q[np.arange(B)[:, None], np.arange(k)[None, :], x] = 1.0
    T = rng.uniform(0.5, 1.5, size=B)
    a = sd_verify(l, x, None, None, T, seed=77)
    b_ = sd_verify(l, x, q, None, T, seed=77)
    for key in ("out_tokens", "num_accepted", "counters", "accept_prob",
                "flag_accept", "flag_gumbel"):
        assert np.array_equal(a[key], b_[key]), key
    assert a["num_accepted"].max() > 0


def test_near_tie_band_and_its_dense_slack():
    """Reading 13: the near-tie band is GUMBEL_FLAG_EPS, widened for a dense
    residual by DENSE_W_REL_ERR * P_c / W_c for each of the two leading
    blocks; only the top two keys matter."""
    eps = ov.GUMBEL_FLAG_EPS
    keys = np.array([-np.inf, 1.0, 1.0 + 0.9 * eps, 0.5])
    assert ov._near_tie(keys) == 1
    keys[2] = 1.0 + 1.1 * eps
    assert ov._near_tie(keys) == 0
    slack = np.array([0.0, 0.1 * eps, 0.1 * eps, 5.0])  # the third key's slack is irrelevant
    assert ov._near_tie(keys, slack) == 1
    assert ov._near_tie(np.array([2.0, -np.inf])) == 0
    # the slack: block 0 holds p-mass 0.5 on tokens where p > q and residual 0.05
    p = np.array([0.3, 0.2, 0.1, 0.4])
    q = np.array([0.27, 0.18, 0.3, 0.25])
    r = np.maximum(p - q, 0.0)
    s = ov.dense_level1_slack(r, p, block=2)
    assert s[0] == pytest.approx(ov.DENSE_W_REL_ERR * 0.5 / 0.05, rel=1e-12)
    assert s[1] == pytest.approx(ov.DENSE_W_REL_ERR * 0.4 / 0.15, rel=1e-12)
    assert ov.dense_level1_slack(np.zeros(4), p, block=2).tolist() == [0.0, 0.0]
