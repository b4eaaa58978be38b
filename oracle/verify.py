"""Speculative rejection-sampling verification, written out plainly in float64.

Test infrastructure (see the package docstring): never on the product path.

The method (pages cited by title and section):

1. Target logits are taken in full precision (pyshine "vLLM, part 2",
   "Verification: rejection sampling on the GPU": logits are cast to float32
   before anything else; here every bf16/fp32 input value is exact in float64).
2. The grammar bitmask removes the tokens the grammar forbids at each draft
   position and at the bonus position (pyshine, "Grammar gates: structured
   output": one mask row per request and per speculative position; the page's
   "zeroes the logits" is read as "gives those tokens probability zero").
3. Temperature divides the logits and top-k truncates the distribution before
   the softmax (pyshine, "Verification": apply_sampling_constraints applies
   temperature and top-k to the flattened logits, so that accepted sequences keep
   the target's law).  Temperature zero selects the greedy rule.
4. Draft x_i is accepted with probability min(1, p_i(x_i) / q_i(x_i)), using
   one uniform per position and the strict test u < a (vllm-learning code
   walkthrough, RejectionSampler: accept where the random value is below the
   acceptance probability); drafts without probabilities use one-hot q, so the
   acceptance probability is p_i(x_i) (infra-guide 5.2, section 4.3).
5. The scan stops at the first rejection; later drafts are dropped
   (vllm-learning, RejectionSampler, steps 3 and 4).
6. The rejected position is resampled from max(p - q, 0) renormalised
   (pyshine, "Verification": sample_recovered_tokens); for one-hot q that is p
   with the rejected draft removed and renormalised by 1 - p(x) (infra-guide
   5.2, section 4.3).  After full acceptance the bonus position is sampled from
   the target with the request's own settings (pyshine, "Verification" and
   "Choosing a drafter").  Greedy requests accept while the draft equals the
   argmax and emit the argmax (pyshine, "Verification": the greedy variant skips
   randomness).
7. Counters R, I, D = R - I, A (fanout, "Name the three counters").

Readings where the pages are silent (each listed in the design notes): the
RNG streams of ``oracle.philox``; sampling by two-level Gumbel-max over blocks
of ``BLOCK`` tokens; lowest index wins every tie; a token with
p = 0 is rejected, q = 0 with p > 0 accepts; I counts drafts whose own mask bit
is 0; top-k keeps every allowed finite token >= the k-th largest allowed
logit, counted with multiplicity, at every position of a sampling request;
zero residual mass falls back to p; unused output slots hold -1; malformed
requests are reported through status bits and produce -1 outputs.
"""

import math

import numpy as np

from . import philox

BLOCK = 2048            # tokens per level-1 block of the two-level Gumbel-max
ACCEPT_FLAG_EPS = 1e-6  # |u - a| below this marks a boundary accept draw
GUMBEL_FLAG_EPS = 1e-5  # top-2 Gumbel keys closer than this mark a near tie
# Dense residuals: the kernels sum max(p - q, 0) over a block from fp32 p, whose
# relative error (a few units of 2^-24) becomes a relative error of about
# DENSE_W_REL_ERR * P_c / W_c in the block's residual mass W_c, where P_c is the
# p-mass of the block's tokens with p > q.  Level-1 near ties of a dense
# residual widen the band by that much for each of the two blocks.
DENSE_W_REL_ERR = 6e-7
TOP_P_FLAG_EPS = 1e-9   # a cumulative mass within this of top_p marks a boundary row

# status bits (a request with any bit set produces -1 outputs)
ST_DRAFT_ID = 1         # draft id outside [0, V)
ST_TEMPERATURE = 2      # temperature negative, NaN or infinite
ST_EMPTY_ROW = 4        # a row with no allowed token of finite logit
ST_BAD_LOGIT = 8        # NaN or +inf logit at an allowed position
ST_BAD_DRAFT_PROB = 16  # draft probability of a draft token NaN, inf or < 0
ST_BAD_OFFSETS = 32     # ragged drafts: the request's draft offsets are inconsistent


def unpack_bitmask(words, V):
    """Allowed-token booleans from packed int32 words: bit (j & 31) of word j >> 5."""
    w = np.asarray(words).astype(np.int64) & 0xFFFFFFFF
    j = np.arange(V)
    return ((w[..., j >> 5] >> (j & 31)) & 1).astype(bool)


def accept_probability(p, q):
    """min(1, p/q), with p = 0 -> 0 (never accept a token the target forbids)
    and q = 0 < p -> 1."""
    if p == 0.0:
        return 0.0
    if q == 0.0:
        return 1.0
    return min(1.0, p / q)


def top_p_threshold(logits_row, keep, T, top_p):
    """The top-p cut of one row: the largest logit value v such that the
    tokens of `keep` with logit >= v hold at least top_p of the tempered mass
    of `keep` (pyshine, "Verification": top-p is one of the sampling
    constraints applied before the accept test).  Tokens are taken from the
    largest logit down and every token tied with the last one taken stays, so
    the cut does not depend on the order of equal logits.  Returns (v, flag):
    flag is 1 when the mass at v or at the next larger value lies within
    TOP_P_FLAG_EPS of top_p, where another rounding could move the cut."""
    vals = logits_row[keep].astype(np.float64)
    s = vals / T
    w = np.exp(s - s.max())
    w /= w.sum()
    distinct = np.unique(vals)[::-1]                     # largest first
    mass = np.array([w[vals == v].sum() for v in distinct])
    cum = np.cumsum(mass)
    idx = int(np.argmax(cum >= top_p)) if np.any(cum >= top_p) else len(distinct) - 1
    flag = abs(cum[idx] - top_p) < TOP_P_FLAG_EPS or \
        (idx > 0 and abs(top_p - cum[idx - 1]) < TOP_P_FLAG_EPS)
    return float(distinct[idx]), int(flag)


def target_distribution(logits_row, allowed_row, T, top_k, top_p=0.0, flags=None):
    """p over the vocabulary for one row (T > 0), and its log-normaliser.

    Allowed tokens with a finite logit form the support; with top_k > 0 the
    support is cut to the tokens whose logit is >= the top_k-th largest of them,
    and with 0 < top_p < 1 then to the tokens above the top-p cut of what is
    left (top_p_threshold).  Returns (p, lse) with lse = log sum exp(l/T) over
    the support.  `flags` (a list) receives the top-p boundary flag.
    """
    l = logits_row
    keep = allowed_row & np.isfinite(l)
    if top_k > 0:
        vals = np.sort(l[keep])[::-1]
        if vals.size > top_k:
            keep = keep & (l >= vals[top_k - 1])
    if 0.0 < top_p < 1.0 and np.any(keep):
        v, flag = top_p_threshold(l, keep, T, top_p)
        keep = keep & (l >= v)
        if flags is not None:
            flags.append(flag)
    s = l[keep] / T
    m = s.max()
    e = np.zeros(l.shape[0])
    e[keep] = np.exp(s - m)
    S = e.sum()
    return e / S, m + math.log(S)


def greedy_choice(logits_row, allowed_row):
    """Lowest index of the largest allowed logit."""
    return int(np.argmax(np.where(allowed_row, logits_row, -np.inf)))


def residual_weights(p_row, q_row, x, one_hot):
    """Unnormalised law of the token emitted at a rejected position.

    Dense q: max(p - q, 0).  One-hot q: p with the rejected draft removed.
    """
    if one_hot:
        r = p_row.copy()
        r[x] = 0.0
        return r
    return np.maximum(p_row - q_row, 0.0)


def _near_tie(keys, slack=None):
    """1 when the two largest finite keys are closer than the band:
    GUMBEL_FLAG_EPS, plus slack[i] + slack[j] for those two keys' entries
    when a per-entry slack is given."""
    idx = np.nonzero(np.isfinite(keys))[0]
    if idx.size < 2:
        return 0
    order = idx[np.argsort(keys[idx], kind="stable")]
    top1, top2 = order[-1], order[-2]
    band = GUMBEL_FLAG_EPS + (0.0 if slack is None else slack[top1] + slack[top2])
    return int(keys[top1] - keys[top2] < band)


def dense_level1_slack(r, p, block=BLOCK):
    """Per block c of a dense residual r = max(p - q, 0): DENSE_W_REL_ERR *
    P_c / W_c, with W_c the residual mass of the block and P_c the p-mass of
    its tokens with r > 0 (0 for blocks without residual mass)."""
    V = r.shape[0]
    C = -(-V // block)
    W = np.zeros(C * block)
    W[:V] = r
    P = np.zeros(C * block)
    P[:V] = np.where(r > 0, p, 0.0)
    W = W.reshape(C, block).sum(axis=1)
    P = P.reshape(C, block).sum(axis=1)
    out = np.zeros(C)
    live = W > 0
    out[live] = DENSE_W_REL_ERR * P[live] / W[live]
    return out


def gumbel_two_level(r, seed, b, a, block=BLOCK, p=None):
    """Draw a token with probability r_j / sum(r) by two-level Gumbel-max.

    Level 1 picks block c (tokens [c*block, (c+1)*block)) with key
    ln W_c + G(U_blk(b, a, c)), W_c = sum of r over the block; blocks with
    W_c = 0 take no part.  Level 2 picks token j of that block with key
    ln r_j + G(U_tok(b, a, j)) over r_j > 0.  The maximum of Gumbel-perturbed
    log-weights over a block is Gumbel-distributed around ln W_c, so the
    composition is exact; block = len(r) gives the flat Gumbel-max.
    p: the target row when r is a dense residual max(p - q, 0) (the level-1
    near-tie band then widens by DENSE_W_REL_ERR * P_c / W_c per block).
    Returns (token, number of near-tie flags).
    """
    V = r.shape[0]
    C = -(-V // block)
    padded = np.zeros(C * block)
    padded[:V] = r
    W = padded.reshape(C, block).sum(axis=1)
    key1 = np.full(C, -np.inf)
    live = np.nonzero(W > 0)[0]
    key1[live] = np.log(W[live]) + philox.gumbel(philox.u_block(seed, b, a, live))
    slack = None if p is None else dense_level1_slack(r, p, block)
    c_star = int(np.argmax(key1))
    lo, hi = c_star * block, min((c_star + 1) * block, V)
    rr = r[lo:hi]
    key2 = np.full(hi - lo, -np.inf)
    live2 = np.nonzero(rr > 0)[0]
    key2[live2] = np.log(rr[live2]) + philox.gumbel(philox.u_token(seed, b, a, lo + live2))
    y = lo + int(np.argmax(key2))
    return y, _near_tie(key1, slack) + _near_tie(key2)


def _verify_request(l, x, q, allowed, T, top_k, seed, b, block, top_p=0.0):
    """One request.  l: [k+1, V] float64; x: [k]; q: [k, V] or None;
    allowed: [k+1, V] bool.  Returns a dict of per-request results."""
    k, V = x.shape[0], l.shape[1]
    res = {
        "tokens": np.full(k + 1, -1, dtype=np.int64),
        "num_accepted": -1,
        "status": 0,
        "R": 0, "I": 0, "A": 0,
        "row_lse": np.full(k + 1, np.nan),
        "accept_prob": np.full(k, np.nan),
        "flag_accept": 0,
        "flag_gumbel": 0,
        "flag_topp": 0,
    }
    st = 0
    if not (math.isfinite(T) and T >= 0.0):
        st |= ST_TEMPERATURE
    if np.any((x < 0) | (x >= V)):
        st |= ST_DRAFT_ID
    for i in range(k + 1):
        vals = l[i][allowed[i]]
        if np.any(np.isnan(vals) | (vals == np.inf)):
            st |= ST_BAD_LOGIT
        if not np.any(np.isfinite(vals)):
            st |= ST_EMPTY_ROW
    if q is not None and not (st & ST_DRAFT_ID):
        qx = q[np.arange(k), x]
        if np.any(~np.isfinite(qx) | (qx < 0)):
            st |= ST_BAD_DRAFT_PROB
    if st:
        res["status"] = st
        return res

    # grammar-invalid drafts: the draft's own mask bit is 0 (fanout, I)
    invalid = np.array([not allowed[i, x[i]] for i in range(k)], dtype=bool)

    if T == 0.0:
        g = [greedy_choice(l[i], allowed[i]) for i in range(k + 1)]
        n_acc = 0
        while n_acc < k and x[n_acc] == g[n_acc]:
            n_acc += 1
        y = g[n_acc]
        res["row_lse"] = np.array([np.max(l[i][allowed[i]]) for i in range(k + 1)])
        res["accept_prob"] = np.array([1.0 if x[i] == g[i] else 0.0 for i in range(k)])
    else:
        p = np.zeros((k + 1, V))
        lse = np.zeros(k + 1)
        tp_flags = []
        for i in range(k + 1):
            p[i], lse[i] = target_distribution(l[i], allowed[i], T, top_k, top_p, tp_flags)
        res["flag_topp"] = int(sum(tp_flags))
        res["row_lse"] = lse
        acc = np.array([accept_probability(p[i, x[i]], 1.0 if q is None else q[i, x[i]])
                        for i in range(k)])
        res["accept_prob"] = acc
        u = philox.u_accept(seed, b, np.arange(k)) if k else np.zeros(0)
        n_acc = 0
        while n_acc < k:
            if abs(u[n_acc] - acc[n_acc]) < ACCEPT_FLAG_EPS:
                res["flag_accept"] += 1
            if u[n_acc] < acc[n_acc]:
                n_acc += 1
            else:
                break
        dense = n_acc < k and q is not None
        if n_acc == k:
            r = p[k]
        else:
            r = residual_weights(p[n_acc], None if q is None else q[n_acc], x[n_acc], q is None)
        if not r.sum() > 0.0:
            r = p[n_acc]
            dense = False
        y, nflag = gumbel_two_level(r, seed, b, n_acc, block, p[n_acc] if dense else None)
        res["flag_gumbel"] = nflag

    res["tokens"][:n_acc] = x[:n_acc]
    res["tokens"][n_acc] = y
    res["num_accepted"] = n_acc
    res["R"], res["I"], res["A"] = k, int(invalid.sum()), n_acc
    return res


def sd_verify(logits, draft_token_ids, draft_probs=None, bitmask=None, temperature=None,
              seed=0, top_k=None, block=BLOCK, request_ids=None, top_p=None):
    """Verify a batch of drafted requests.

    logits:          [B, k+1, V] float (bf16 values given exactly as float32/64)
    draft_token_ids: [B, k] integer
    draft_probs:     [B, k, V] float or None (drafts without probabilities)
    bitmask:         [B, k+1, ceil(V/32)] int32 or None (all tokens allowed)
    temperature:     [B] float; 0 selects the greedy rule
    seed:            64-bit Philox key
    top_k:           [B] integer or None; values <= 0 switch top-k off
    top_p:           [B] float or None; values outside (0, 1) switch top-p off
    request_ids:     optional [B] global request index of each batch entry, used
                     as b in the Philox counters (for checking a sample of a
                     larger batch one request at a time); default 0 .. B-1

    Returns a dict with out_tokens [B, k+1] (-1 padded), num_accepted [B],
    counters (R, I, D, A), status (OR of request bits), per-request status,
    row_lse [B, k+1], accept_prob [B, k], and per-request flag counts.
    """
    logits = np.asarray(logits)
    B, kp1, V = logits.shape
    k = kp1 - 1
    x_all = np.asarray(draft_token_ids, dtype=np.int64).reshape(B, k)
    T_all = np.asarray(temperature, dtype=np.float64).reshape(B)
    tk_all = np.zeros(B, dtype=np.int64) if top_k is None else \
        np.asarray(top_k, dtype=np.int64).reshape(B)
    tp_all = np.zeros(B) if top_p is None else np.asarray(top_p, dtype=np.float64).reshape(B)
    gid = list(range(B)) if request_ids is None else [int(r) for r in request_ids]

    out = {
        "out_tokens": np.full((B, k + 1), -1, dtype=np.int64),
        "num_accepted": np.full(B, -1, dtype=np.int64),
        "request_status": np.zeros(B, dtype=np.int64),
        "row_lse": np.full((B, k + 1), np.nan),
        "accept_prob": np.full((B, k), np.nan),
        "flag_accept": np.zeros(B, dtype=np.int64),
        "flag_gumbel": np.zeros(B, dtype=np.int64),
        "flag_topp": np.zeros(B, dtype=np.int64),
    }
    R = I = A = 0
    status = 0
    for b in range(B):
        l = logits[b].astype(np.float64)
        if bitmask is None:
            allowed = np.ones((k + 1, V), dtype=bool)
        else:
            allowed = unpack_bitmask(np.asarray(bitmask[b]), V)
        q = None if draft_probs is None else np.asarray(draft_probs[b], dtype=np.float64)
        r = _verify_request(l, x_all[b], q, allowed, float(T_all[b]), int(tk_all[b]),
                            seed, gid[b], block, float(tp_all[b]))
        out["out_tokens"][b] = r["tokens"]
        out["num_accepted"][b] = r["num_accepted"]
        out["request_status"][b] = r["status"]
        out["row_lse"][b] = r["row_lse"]
        out["accept_prob"][b] = r["accept_prob"]
        out["flag_accept"][b] = r["flag_accept"]
        out["flag_gumbel"][b] = r["flag_gumbel"]
        out["flag_topp"][b] = r["flag_topp"]
        status |= r["status"]
        R += r["R"]
        I += r["I"]
        A += r["A"]
    out["counters"] = np.array([R, I, R - I, A], dtype=np.uint64)
    out["status"] = status
    out["accept_histogram"] = accept_histogram(out["num_accepted"], out["request_status"], k)
    return out


def accept_histogram(num_accepted, request_status, kmax):
    """Requests per accepted draft length 0 .. kmax, requests in error left
    out (fanout, "Mean acceptance length uses another denominator": one bucket
    for every possible accepted length, the bonus token not counted)."""
    h = np.zeros(kmax + 1, dtype=np.int64)
    for n, st in zip(num_accepted, request_status):
        if st == 0:
            h[int(n)] += 1
    return h


def sd_verify_ragged(logits, draft_token_ids, draft_offsets, draft_probs=None, bitmask=None,
                     temperature=None, seed=0, top_k=None, max_draft=None, total_drafts=None,
                     block=BLOCK, top_p=None):
    """Requests with their own draft lengths (a drafter that proposes a
    variable number of tokens per request, infra-guide 5.2, dynamic draft
    length).  Request b has k_b = off[b+1] - off[b] drafts; its rows are
    logits[off[b] + b : off[b+1] + b + 1] (k_b draft positions, then the bonus
    position), its drafts draft_token_ids[off[b] : off[b+1]].

    logits:          [rows, V] with rows = off[B] + B
    draft_token_ids: [off[B]] integer
    draft_offsets:   [B + 1] integer
    draft_probs:     [off[B], V] float or None
    bitmask:         [rows, ceil(V/32)] int32 or None
    temperature:     [B]; top_k: [B] or None
    max_draft:       the largest allowed k_b (default: the largest given)
    total_drafts:    the number of drafts the caller declares (default off[B])

    The offsets must start at 0, never decrease, end at total_drafts, and give
    every request at most max_draft drafts.  Otherwise the rows of the call
    cannot be located: every request gets status ST_BAD_OFFSETS and
    num_accepted -1, no output slot is written and the counters stay 0.
    Returns out_tokens [rows] (each request's k_b + 1 slots), num_accepted [B],
    counters, status, request_status, row_lse [rows], accept_prob [off[B]],
    flag counts and the accepted-length histogram [max_draft + 1].
    """
    off = np.asarray(draft_offsets, dtype=np.int64).reshape(-1)
    B = off.shape[0] - 1
    total = int(off[B]) if total_drafts is None else int(total_drafts)
    logits = np.asarray(logits)
    rows, V = logits.shape
    if rows != total + B:
        raise ValueError("logits must hold total_drafts + B rows")
    if total < 0:
        raise ValueError("total_drafts must be >= 0")
    x_all = np.asarray(draft_token_ids, dtype=np.int64).reshape(-1)
    T_all = np.asarray(temperature, dtype=np.float64).reshape(B)
    tk_all = np.zeros(B, dtype=np.int64) if top_k is None else \
        np.asarray(top_k, dtype=np.int64).reshape(B)
    tp_all = np.zeros(B) if top_p is None else np.asarray(top_p, dtype=np.float64).reshape(B)
    kb = off[1:] - off[:-1]
    kmax = int(max(kb.max(), 0)) if max_draft is None and B > 0 else int(max_draft or 0)
    out = {
        "out_tokens": np.full(rows, -1, dtype=np.int64),
        "num_accepted": np.full(B, -1, dtype=np.int64),
        "request_status": np.zeros(B, dtype=np.int64),
        "row_lse": np.full(rows, np.nan),
        "accept_prob": np.full(total, np.nan),
        "flag_accept": np.zeros(B, dtype=np.int64),
        "flag_gumbel": np.zeros(B, dtype=np.int64),
        "flag_topp": np.zeros(B, dtype=np.int64),
    }
    R = I = A = 0
    status = 0
    consistent = B >= 0 and int(off[0]) == 0 and int(off[B]) == total and \
        bool(np.all(kb >= 0)) and bool(np.all(kb <= kmax))
    for b in range(B):
        o0, o1 = int(off[b]), int(off[b + 1])
        if not consistent:
            out["request_status"][b] = ST_BAD_OFFSETS
            status |= ST_BAD_OFFSETS
            continue
        k = o1 - o0
        r0 = o0 + b
        l = logits[r0:r0 + k + 1].astype(np.float64)
        if bitmask is None:
            allowed = np.ones((k + 1, V), dtype=bool)
        else:
            allowed = unpack_bitmask(np.asarray(bitmask[r0:r0 + k + 1]), V)
        q = None if draft_probs is None else np.asarray(draft_probs[o0:o1], dtype=np.float64)
        r = _verify_request(l, x_all[o0:o1], q, allowed, float(T_all[b]), int(tk_all[b]),
                            seed, b, block, float(tp_all[b]))
        out["out_tokens"][r0:r0 + k + 1] = r["tokens"]
        out["num_accepted"][b] = r["num_accepted"]
        out["request_status"][b] = r["status"]
        out["row_lse"][r0:r0 + k + 1] = r["row_lse"]
        out["accept_prob"][o0:o1] = r["accept_prob"]
        out["flag_accept"][b] = r["flag_accept"]
        out["flag_gumbel"][b] = r["flag_gumbel"]
        out["flag_topp"][b] = r["flag_topp"]
        status |= r["status"]
        R += r["R"]
        I += r["I"]
        A += r["A"]
    out["counters"] = np.array([R, I, R - I, A], dtype=np.uint64)
    out["status"] = status
    out["accept_histogram"] = accept_histogram(out["num_accepted"], out["request_status"], kmax)
    return out
