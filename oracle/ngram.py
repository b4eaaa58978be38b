"""The n-gram (prompt lookup) draft proposer, written out plainly.

Test infrastructure only (see the package docstring): never on the product
path.

The rule, in the pages' terms:

* The history is the request's whole token sequence, prompt and generated
  tokens alike; matching compares token ids only (infra-guide 5.2, section 4.1
  "Match the tail, then copy what follows", and section 4.2: the whole history
  is searched).
* The last n tokens (the tail) are looked up earlier in the same history.  The
  window n runs from the longest, max_n (never more than len - 1), down to the
  shortest, min_n; the first n whose tail occurs earlier wins (infra-guide 5.2,
  section 6 "Hands-on: match window and candidate coverage": long windows
  before short ones; section 4.2: the longest match is preferred).
* Among the occurrences of that n-gram the one that starts earliest wins.  An
  occurrence may overlap the tail but may not be the tail itself: its start is
  below len - n (infra-guide 5.2, section 6; pyshine "vLLM, part 2",
  "Choosing a drafter": the earliest position reaching the longest match).
* The proposal is the k tokens that follow the occurrence, fewer when the
  history ends first (infra-guide 5.2, section 6: up to k tokens are copied).
* No occurrence for any n in [min_n, max_n]: no proposal.  A history too short
  for the smallest window, or a request whose k drafts would run past the
  model's context length, gets no proposal either (pyshine, "Choosing a
  drafter": both cases return an empty draft).

Readings where the pages leave a step open (each listed in the design notes):
the context-length case is read as len + k > max_model_len, decided before the
search, and max_model_len = 0 means no limit; a length outside [0, stride] for
a row of the batched table is a data error that leaves the request without a
proposal and sets status bit NG_BAD_LENGTH.
"""

import numpy as np

NG_BAD_LENGTH = 1  # status bit: a history length outside [0, stride]


def _search(h, min_n, max_n):
    """The winning (window, start) for one history h (int64 array), or
    (0, -1) when nothing matches.

    The rule, restated over occurrence ends: the n-gram the tail forms with n
    tokens occurs ending at position e exactly when the n tokens up to e equal
    the last n tokens of the history, i.e. when h[e - t] == h[L - 1 - t] for
    t = 0 .. n - 1.  agree[e] counts how many such t hold in a row from t = 0,
    capped at the longest allowed window.  An occurrence may overlap the tail
    but may not be it, so e stops at L - 2.  The longest window is then the
    largest agree[e] (if it reaches min_n), and its earliest occurrence is the
    one with the smallest end.
    """
    L = h.shape[0]
    cap = min(max_n, L - 1)
    if cap < min_n:
        return 0, -1
    ends = np.arange(L - 1)
    agree = np.zeros(L - 1, dtype=np.int64)
    still = np.ones(L - 1, dtype=bool)     # every step so far agreed
    for t in range(cap):
        pos = ends - t
        ok = still & (pos >= 0)
        ok[ok] = h[pos[ok]] == h[L - 1 - t]
        agree += ok
        still = ok
    n = int(agree.max()) if agree.size else 0
    if n < min_n:
        return 0, -1
    e = int(np.flatnonzero(agree >= n)[0])
    return n, e - n + 1


def propose_batch(tokens, lengths, min_n, max_n, k, max_model_len=0):
    """A batch of histories in a table: row b of ``tokens`` [B, stride] holds
    lengths[b] tokens.  Returns

    * drafts [B, k] int64: the proposal, then -1,
    * num_drafts [B]: its length (0 when nothing is proposed),
    * match_len [B]: the winning window n, 0 when nothing is proposed,
    * draft_offsets [B + 1]: cumulative num_drafts (the ragged layout the
      verifier takes), and flat [draft_offsets[B]] the proposals back to back,
    * request_status [B], status (OR over the batch).
    """
    tokens = np.asarray(tokens)
    lengths = np.asarray(lengths, dtype=np.int64)
    B = lengths.shape[0]
    stride = tokens.shape[1] if tokens.ndim == 2 else 0
    drafts = np.full((B, k), -1, dtype=np.int64)
    num = np.zeros(B, dtype=np.int64)
    match = np.zeros(B, dtype=np.int64)
    rstat = np.zeros(B, dtype=np.int64)
    for b in range(B):
        L = int(lengths[b])
        if L < 0 or L > stride:
            rstat[b] = NG_BAD_LENGTH
            continue
        if max_model_len and L + k > max_model_len:
            continue
        h = tokens[b, :L].astype(np.int64)
        n, start = _search(h, min_n, max_n)
        if n == 0:
            continue
        p = h[start + n:start + n + k]
        match[b] = n
        num[b] = len(p)
        drafts[b, :len(p)] = p
    offsets = np.concatenate([[0], np.cumsum(num)]).astype(np.int64)
    flat = np.concatenate([drafts[b, :num[b]] for b in range(B)] + [np.zeros(0, np.int64)])
    return {"drafts": drafts, "num_drafts": num, "match_len": match, "draft_offsets": offsets,
            "flat": flat, "request_status": rstat,
            "status": int(np.bitwise_or.reduce(rstat)) if B else 0}


def propose_one(history, min_n, max_n, k, max_model_len=0):
    """One history given as a sequence: (n, proposal as a list), or (None, [])
    when nothing is proposed (propose_batch on a one-row table)."""
    h = np.asarray(list(history), dtype=np.int64)
    table = h.reshape(1, -1) if h.size else np.zeros((1, 1), dtype=np.int64)
    r = propose_batch(table, [h.size], min_n, max_n, k, max_model_len)
    n = int(r["match_len"][0])
    return (n if n else None), [int(v) for v in r["drafts"][0, :r["num_drafts"][0]]]
