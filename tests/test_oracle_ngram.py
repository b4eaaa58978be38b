"""The n-gram proposer oracle against what the pages and the mathematics fix.

* the pages' worked lookups (infra-guide 5.2, sections 4.1 and 6), stored in
  tests/golden/ngram_toy.json;
* brute force on small histories: every (window, start) pair that matches is
  listed and the longest window, then the earliest start, is taken;
* a second, independent algorithm: the Z-function of the reversed history
  gives, for each end position, how many tokens before it agree with the tail
  (pyshine "vLLM, part 2", "Choosing a drafter": the search runs over the
  reversed sequence);
* the special cases the rule fixes: no repeated token, a history too short,
  the context-length limit, malformed lengths.
"""
import json
import os

import numpy as np
import pytest

from oracle.ngram import NG_BAD_LENGTH, propose_batch, propose_one

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ngram_toy.json")


def _batch1(h, min_n, max_n, k, max_model_len=0):
    t = np.asarray(h, dtype=np.int64).reshape(1, -1) if len(h) else np.zeros((1, 1), np.int64)
    r = propose_batch(t, [len(h)], min_n, max_n, k, max_model_len)
    n = int(r["match_len"][0])
    return (n if n else None), [int(v) for v in r["drafts"][0, :r["num_drafts"][0]]]


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_pages_worked_lookups(case):
    want = (case["n"], case["proposal"])
    assert propose_one(case["history"], case["min_n"], case["max_n"], case["k"]) == want
    assert _batch1(case["history"], case["min_n"], case["max_n"], case["k"]) == want


def _brute(h, min_n, max_n, k):
    L = len(h)
    hits = [(n, s) for n in range(1, L) for s in range(0, L - n)
            if min_n <= n <= max_n and h[s:s + n] == h[L - n:]]
    if not hits:
        return None, []
    n, s = min(hits, key=lambda ns: (-ns[0], ns[1]))
    return n, h[s + n:s + n + k]


def _zfunc(s):
    n = len(s)
    z = [0] * n
    if n:
        z[0] = n
    lo = hi = 0
    for i in range(1, n):
        if i < hi:
            z[i] = min(hi - i, z[i - lo])
        while i + z[i] < n and s[z[i]] == s[i + z[i]]:
            z[i] += 1
        if i + z[i] > hi:
            lo, hi = i, i + z[i]
    return z


def _by_zfunction(h, min_n, max_n, k):
    # r = reversed history; z[i] = common prefix of r and r[i:], i.e. the
    # number of tokens ending at e = L - i that agree with the tail
    L = len(h)
    z = _zfunc(h[::-1])
    best_n, best_e = 0, None
    for e in range(1, L):              # e = end of the occurrence, before the last token
        n = min(z[L - e], max_n)
        if n >= min_n and n > best_n:  # scanning e upwards keeps the earliest on ties
            best_n, best_e = n, e
    if best_e is None:
        return None, []
    return best_n, h[best_e:best_e + k]


@pytest.mark.parametrize("alphabet", [2, 3, 5])
def test_brute_force_and_z_function(alphabet):
    rng = np.random.default_rng(alphabet)
    for trial in range(400):
        L = int(rng.integers(0, 24))
        h = [int(v) for v in rng.integers(0, alphabet, size=L)]
        min_n = int(rng.integers(1, 5))
        max_n = int(rng.integers(min_n, 8))
        k = int(rng.integers(0, 6))
        want = _brute(h, min_n, max_n, k)
        assert propose_one(h, min_n, max_n, k) == want, (h, min_n, max_n, k)
        assert _by_zfunction(h, min_n, max_n, k) == want, (h, min_n, max_n, k)
        assert _batch1(h, min_n, max_n, k) == want, (h, min_n, max_n, k)


def test_proposal_properties_on_long_histories():
    rng = np.random.default_rng(5)
    for trial in range(30):
        L = int(rng.integers(50, 400))
        h = [int(v) for v in rng.integers(0, 4, size=L)]
        n, p = propose_one(h, 2, 6, 4)
        assert n is not None                       # 4 symbols: some 2-gram repeats
        s = next(s for s in range(L - n) if h[s:s + n] == h[L - n:])
        assert p == h[s + n:s + n + 4] and 1 <= len(p) <= 4
        # no longer window (up to max_n) occurs before the tail
        for m in range(n + 1, 7):
            assert all(h[t:t + m] != h[L - m:] for t in range(L - m))
        assert _by_zfunction(h, 2, 6, 4) == (n, p)


def test_special_cases():
    assert propose_one([1, 2, 3, 4, 5], 2, 4, 3) == (None, [])          # no token repeats
    assert propose_one([1, 2, 3, 4, 5], 1, 4, 3) == (None, [])
    assert propose_one([], 1, 4, 3) == (None, []) and propose_one([7], 1, 4, 3) == (None, [])
    assert propose_one([7, 7], 1, 4, 3) == (1, [7])                     # the tail's own token follows
    assert propose_one([7, 7], 2, 4, 3) == (None, [])                   # a window needs len - 1 >= n
    assert propose_one([5, 5, 5, 5, 5], 2, 3, 4) == (3, [5, 5])         # overlap with the tail is allowed
    assert propose_one([1, 2, 9, 1, 2], 2, 4, 0) == (2, [])             # k = 0: a match, nothing copied
    assert propose_one([1, 2, 3, 1, 2, 3], 3, 3, 5) == (3, [1, 2, 3])   # cut short by the history's end


def test_context_length_limit():
    h = [1, 2, 9, 1, 2]
    assert propose_one(h, 2, 4, 3, max_model_len=8) == (2, [9, 1, 2])   # 5 + 3 fits
    assert propose_one(h, 2, 4, 3, max_model_len=7) == (None, [])       # 5 + 3 would overflow
    assert _batch1(h, 2, 4, 3, max_model_len=7) == (None, [])
    assert _batch1(h, 2, 4, 3, max_model_len=8) == (2, [9, 1, 2])


def test_batch_layout_and_bad_lengths():
    rng = np.random.default_rng(2)
    B, stride = 9, 40
    tokens = rng.integers(0, 3, size=(B, stride))
    lengths = np.array([40, 0, 1, 17, -1, 41, 25, 3, 12])
    r = propose_batch(tokens, lengths, 2, 5, 4)
    for b in range(B):
        L = int(lengths[b])
        if L < 0 or L > stride:
            assert r["request_status"][b] == NG_BAD_LENGTH and r["num_drafts"][b] == 0
            continue
        n, p = propose_one(list(tokens[b, :L]), 2, 5, 4)
        assert r["match_len"][b] == (n or 0) and list(r["drafts"][b, :len(p)]) == p
        assert np.all(r["drafts"][b, len(p):] == -1)
    assert r["status"] == NG_BAD_LENGTH
    off = r["draft_offsets"]
    assert off[0] == 0 and np.array_equal(np.diff(off), r["num_drafts"])
    assert np.array_equal(r["flat"], np.concatenate([r["drafts"][b, :r["num_drafts"][b]] for b in range(B)]))


def test_planted_mistakes_fail_the_pins():
    """Each plausible slip in the search is caught by the pins above: a wrong
    choice among the matching (window, start) pairs, or a copy taken one
    token early."""
    def pick(order, shift=0):
        def wrong(h, min_n, max_n, k):
            L = len(h)
            hits = [(n, s) for n in range(1, L) for s in range(0, L - n)
                    if min_n <= n <= max_n and h[s:s + n] == h[L - n:]]
            if not hits:
                return None, []
            n, s = min(hits, key=order)
            return n, h[s + n + shift:s + n + shift + k]
        return wrong

    latest = pick(lambda ns: (-ns[0], -ns[1]))        # latest occurrence instead of earliest
    short_first = pick(lambda ns: (ns[0], ns[1]))      # short windows before long ones
    off_by_one = pick(lambda ns: (-ns[0], ns[1]), -1)  # copies from the last token of the match

    cases = json.load(open(GOLDEN))["cases"]
    for wrong in (latest, short_first, off_by_one):
        bad = [c["name"] for c in cases
               if wrong(c["history"], c["min_n"], c["max_n"], c["k"]) != (c["n"], c["proposal"])]
        rng = np.random.default_rng(0)
        diverged = False
        for _ in range(200):
            h = [int(v) for v in rng.integers(0, 3, size=int(rng.integers(4, 20)))]
            diverged |= wrong(h, 1, 5, 3) != _brute(h, 1, 5, 3)
        assert bad or diverged, wrong.__name__
