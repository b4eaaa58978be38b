"""Helpers for comparing the HIP verifier with the oracle (not a test module).

Parity rule: every request the oracle does not flag (no accept draw with
|u - a| < 1e-6, no Gumbel level whose top-2 keys are closer than 1e-5) must
match exactly -- accepted count, every output token, error status.
Probabilities must agree to 1e-5 relative: each accept probability
min(1, p/q) within 1e-5 of the oracle's value times that value (an exact zero
stays an exact zero), and each row's log-normaliser within 1e-5 absolute,
which is 1e-5 relative on every probability of the row, plus 2^-22 of its
magnitude: the kernels scale logits by log2(e)/T rounded to fp32 (2^-24
relative), which moves a normaliser of magnitude L by up to about 2^-24 L
(rows of logits near 1e8 differ by units there while every probability
still agrees).  Flagged draws must
stay below 1e-4 of the positions compared (so none at all in a call of fewer
than 10^4 positions).
"""
import concurrent.futures
import os

import numpy as np
import torch

import oracle
from workloads import to_numpy

LSE_ATOL = 1e-5
LSE_FP32_REL = 2.0 ** -22
ACC_RTOL = 1e-5
FLAG_FRACTION = 1e-4


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_gpu(wl, seed=None):
    import rejection_sampling_verification_amd as sdv
    lg = wl["logits"]
    B, kp1, V = lg.shape
    v = sdv.Verifier(B, kp1 - 1, V, lg.dtype, lg.device, debug=True)
    r = v(lg, wl["draft_token_ids"], wl["draft_probs"], wl["bitmask"], wl["temperature"],
          wl["seed"] if seed is None else seed, wl["top_k"], top_p=wl.get("top_p"))
    torch.cuda.synchronize()
    out = {name: getattr(r, name).cpu().numpy().copy() for name in r._fields if getattr(r, name) is not None}
    out["counters"] = out["out_counters"].view(np.uint64)
    out["status"] = int(out["status"].view(np.uint32)[0])
    return out


def run_oracle(wl, requests=None, seed=None):
    n = to_numpy(wl, requests)
    return oracle.sd_verify(n["logits"], n["draft_token_ids"], n["draft_probs"], n["bitmask"],
                            n["temperature"], seed=wl["seed"] if seed is None else seed,
                            top_k=n["top_k"], request_ids=requests, top_p=n.get("top_p"))


_PER_REQUEST = ("out_tokens", "num_accepted", "request_status", "row_lse", "accept_prob",
                "flag_accept", "flag_gumbel", "flag_topp")


def run_oracle_parallel(wl, chunk=8, workers=None, seed=None):
    """The oracle over every request of a (large) workload, chunks of
    requests on a thread pool (the oracle's work is NumPy on large arrays,
    which runs outside the interpreter lock); the same result as run_oracle
    on the whole batch."""
    B = wl["logits"].shape[0]
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = [list(range(s, min(B, s + chunk))) for s in range(0, B, chunk)]
    hosts = [to_numpy(wl, c) for c in chunks]
    sd = wl["seed"] if seed is None else seed

    def work(job):
        req, n = job
        return oracle.sd_verify(n["logits"], n["draft_token_ids"], n["draft_probs"], n["bitmask"],
                                n["temperature"], seed=sd, top_k=n["top_k"], request_ids=req,
                                top_p=n.get("top_p"))

    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(work, zip(chunks, hosts)))
    out = {key: np.concatenate([r[key] for r in parts]) for key in _PER_REQUEST}
    out["counters"] = np.sum([r["counters"] for r in parts], axis=0, dtype=np.uint64)
    out["status"] = int(np.bitwise_or.reduce([int(r["status"]) for r in parts]))
    out["accept_histogram"] = np.sum([r["accept_histogram"] for r in parts], axis=0)
    return out


def close_rel(a, b, rtol=ACC_RTOL):
    """|a - b| <= rtol |b| elementwise (so b = 0 needs a = 0); NaN matches NaN."""
    a = np.asarray(a, float)
    b = np.asarray(b, float)
    both_nan = np.isnan(a) & np.isnan(b)
    with np.errstate(invalid="ignore"):
        ok = np.abs(a - b) <= rtol * np.abs(b)
    return bool(np.all(both_nan | ok))


def close_lse(a, b, atol=LSE_ATOL, rel=LSE_FP32_REL):
    """|a - b| <= atol + rel |b| elementwise; NaN matches NaN and an infinity
    itself."""
    a = np.asarray(a, float)
    b = np.asarray(b, float)
    both_nan = np.isnan(a) & np.isnan(b)
    with np.errstate(invalid="ignore"):
        ok = (a == b) | (np.abs(a - b) <= atol + rel * np.abs(b))
    return bool(np.all(both_nan | ok))


def flag_limit(positions):
    """Flagged draws allowed among `positions` verified positions: strictly
    fewer than FLAG_FRACTION of them."""
    return max(0, int(np.ceil(FLAG_FRACTION * positions)) - 1)


def compare(gpu, orc, requests=None, check_counters=True):
    """Returns (list of mismatching request ids, list of flagged request ids)."""
    B = orc["out_tokens"].shape[0]
    ids = list(range(B)) if requests is None else list(requests)
    mism, flagged = [], []
    for j, b in enumerate(ids):
        err_o = orc["request_status"][j] != 0
        err_g = gpu["out_num_accepted"][b] == -1
        if err_o != err_g:
            mism.append(b)
            continue
        if orc["flag_accept"][j] or orc["flag_gumbel"][j] or orc["flag_topp"][j]:
            flagged.append(b)
            continue
        if (orc["num_accepted"][j] != gpu["out_num_accepted"][b]
                or not np.array_equal(orc["out_tokens"][j], gpu["out_tokens"][b])):
            mism.append(b)
            continue
        if not close_lse(gpu["row_lse"][b], orc["row_lse"][j]):
            mism.append(b)
            continue
        if not close_rel(gpu["accept_prob"][b], orc["accept_prob"][j]):
            mism.append(b)
    if check_counters and requests is None:
        R, I, D, A = (int(v) for v in orc["counters"])
        gR, gI, gD, gA = (int(v) for v in gpu["counters"])
        assert (gR, gI, gD) == (R, I, D), ((gR, gI, gD), (R, I, D))
        k = orc["accept_prob"].shape[1]
        assert abs(gA - A) <= k * len(flagged), (gA, A)
        if not flagged:
            assert gA == A
        assert gpu["status"] == orc["status"], (gpu["status"], orc["status"])
    return mism, flagged


def flagged_draws(orc, idx=None):
    """Near-boundary draws the oracle flagged (accept, Gumbel, top-p)."""
    sel = slice(None) if idx is None else list(idx)
    return int(np.sum(orc["flag_accept"][sel]) + np.sum(orc["flag_gumbel"][sel])
               + np.sum(orc["flag_topp"][sel]))


def assert_parity(gpu, orc, requests=None, allow_flags=None):
    """Exact parity on every unflagged request, the probability tolerances,
    and fewer flagged draws than FLAG_FRACTION of the positions compared
    (allow_flags overrides that limit for inputs built to sit on a
    boundary)."""
    mism, flagged = compare(gpu, orc, requests)
    if mism:
        b = mism[0]
        j = b if requests is None else list(requests).index(b)
        detail = (f"request {b}: gpu tokens {gpu['out_tokens'][b]} nacc {gpu['out_num_accepted'][b]}"
                  f" | oracle {orc['out_tokens'][j]} nacc {orc['num_accepted'][j]}"
                  f" | lse gpu {gpu['row_lse'][b]} oracle {orc['row_lse'][j]}"
                  f" | acc gpu {gpu['accept_prob'][b]} oracle {orc['accept_prob'][j]}")
        raise AssertionError(f"{len(mism)} mismatching requests {mism[:10]}; {detail}")
    positions = int(np.prod(orc["accept_prob"].shape))
    limit = flag_limit(positions) if allow_flags is None else allow_flags
    nflag = flagged_draws(orc)
    assert nflag <= limit, f"{nflag} flagged draws in {positions} positions (limit {limit}): {flagged}"
    if requests is None and "flags" in gpu:
        g = int(gpu["flags"][0]) + int(gpu["flags"][1])
        assert g <= limit + nflag, f"the GPU reports {g} near-boundary draws (limit {limit})"
    return flagged


# ------------------------------------------------------------ ragged calls

def run_gpu_ragged(wl, max_draft, seed=None):
    """wl: logits [rows, V], draft_token_ids [T], draft_offsets [B+1] (device
    int32), draft_probs [T, V] or None, bitmask [rows, W] or None,
    temperature [B], top_k or None, seed."""
    import rejection_sampling_verification_amd as sdv
    lg = wl["logits"]
    B = wl["draft_offsets"].shape[0] - 1
    rows, V = lg.shape
    v = sdv.Verifier(B, max_draft, V, lg.dtype, lg.device, debug=True, histogram=True,
                     total_drafts=rows - B)
    r = v(lg, wl["draft_token_ids"], wl["draft_probs"], wl["bitmask"], wl["temperature"],
          wl["seed"] if seed is None else seed, wl["top_k"], draft_offsets=wl["draft_offsets"],
          top_p=wl.get("top_p"))
    torch.cuda.synchronize()
    out = {name: getattr(r, name).cpu().numpy().copy() for name in r._fields if getattr(r, name) is not None}
    out["counters"] = out["out_counters"].view(np.uint64)
    out["status"] = int(out["status"].view(np.uint32)[0])
    return out


def run_oracle_ragged(wl, max_draft, seed=None):
    def cv(t):
        if t is None:
            return None
        t = t.detach()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.cpu().numpy()
    rows = wl["logits"].shape[0]
    B = wl["draft_offsets"].shape[0] - 1
    return oracle.sd_verify_ragged(cv(wl["logits"]), cv(wl["draft_token_ids"]), cv(wl["draft_offsets"]),
                                   cv(wl["draft_probs"]), cv(wl["bitmask"]), cv(wl["temperature"]),
                                   seed=wl["seed"] if seed is None else seed, top_k=cv(wl["top_k"]),
                                   max_draft=max_draft, total_drafts=rows - B,
                                   top_p=cv(wl.get("top_p")))


def assert_parity_ragged(gpu, orc, off, allow_flags=None):
    """Per request over its own rows and drafts; counters, status and the
    histogram over the call (exact unless a request is flagged)."""
    off = np.asarray(off, dtype=np.int64)
    B = off.shape[0] - 1
    mism, flagged = [], []
    for b in range(B):
        err_o = orc["request_status"][b] != 0
        if err_o != (gpu["out_num_accepted"][b] == -1):
            mism.append(b)
            continue
        if err_o:
            continue
        if orc["flag_accept"][b] or orc["flag_gumbel"][b] or orc["flag_topp"][b]:
            flagged.append(b)
            continue
        k = int(off[b + 1] - off[b])
        r0, d0 = int(off[b]) + b, int(off[b])
        if (orc["num_accepted"][b] != gpu["out_num_accepted"][b]
                or not np.array_equal(orc["out_tokens"][r0:r0 + k + 1], gpu["out_tokens"][r0:r0 + k + 1])
                or not close_lse(gpu["row_lse"][r0:r0 + k + 1], orc["row_lse"][r0:r0 + k + 1])
                or not close_rel(gpu["accept_prob"][d0:d0 + k], orc["accept_prob"][d0:d0 + k])):
            mism.append(b)
    assert not mism, f"{len(mism)} mismatching requests {mism[:10]}"
    positions = int(orc["accept_prob"].shape[0])
    limit = flag_limit(positions) if allow_flags is None else allow_flags
    nflag = flagged_draws(orc)
    assert nflag <= limit, f"{nflag} flagged draws in {positions} positions (limit {limit}): {flagged}"
    R, I, D, A = (int(v) for v in orc["counters"])
    gR, gI, gD, gA = (int(v) for v in gpu["counters"])
    assert (gR, gI, gD) == (R, I, D), ((gR, gI, gD), (R, I, D))
    if not flagged:
        assert gA == A
        assert np.array_equal(gpu["accept_histogram"].astype(np.int64), orc["accept_histogram"])
    assert gpu["status"] == orc["status"], (gpu["status"], orc["status"])
    return flagged
