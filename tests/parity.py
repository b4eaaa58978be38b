"""Helpers for comparing the HIP verifier with the oracle (not a test module).

Parity rule: every request the oracle does not flag (no accept draw with
|u - a| < 1e-6, no Gumbel level whose top-2 keys are closer than 1e-5) must
match exactly -- accepted count, every output token, error status.  Row
log-normalisers and accept probabilities must agree to 1e-5 relative.
"""
import numpy as np
import torch

import oracle
from workloads import to_numpy

LSE_RTOL = 1e-5
ACC_RTOL = 1e-5


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


def _close(a, b, rtol):
    a = np.asarray(a, float)
    b = np.asarray(b, float)
    both_nan = np.isnan(a) & np.isnan(b)
    ok = np.abs(a - b) <= rtol * np.maximum(1.0, np.abs(b))
    return np.all(both_nan | ok)


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
        if not _close(gpu["row_lse"][b], orc["row_lse"][j], LSE_RTOL):
            mism.append(b)
            continue
        if not _close(gpu["accept_prob"][b], orc["accept_prob"][j], ACC_RTOL):
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


def assert_parity(gpu, orc, requests=None, max_flagged=2):
    mism, flagged = compare(gpu, orc, requests)
    if mism:
        b = mism[0]
        j = b if requests is None else list(requests).index(b)
        detail = (f"request {b}: gpu tokens {gpu['out_tokens'][b]} nacc {gpu['out_num_accepted'][b]}"
                  f" | oracle {orc['out_tokens'][j]} nacc {orc['num_accepted'][j]}"
                  f" | lse gpu {gpu['row_lse'][b]} oracle {orc['row_lse'][j]}"
                  f" | acc gpu {gpu['accept_prob'][b]} oracle {orc['accept_prob'][j]}")
        raise AssertionError(f"{len(mism)} mismatching requests {mism[:10]}; {detail}")
    assert len(flagged) <= max_flagged, f"too many flagged requests: {flagged}"
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


def assert_parity_ragged(gpu, orc, off, max_flagged=2):
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
                or not _close(gpu["row_lse"][r0:r0 + k + 1], orc["row_lse"][r0:r0 + k + 1], LSE_RTOL)
                or not _close(gpu["accept_prob"][d0:d0 + k], orc["accept_prob"][d0:d0 + k], ACC_RTOL)):
            mism.append(b)
    assert not mism, f"{len(mism)} mismatching requests {mism[:10]}"
    assert len(flagged) <= max_flagged, f"too many flagged requests: {flagged}"
    R, I, D, A = (int(v) for v in orc["counters"])
    gR, gI, gD, gA = (int(v) for v in gpu["counters"])
    assert (gR, gI, gD) == (R, I, D), ((gR, gI, gD), (R, I, D))
    if not flagged:
        assert gA == A
        assert np.array_equal(gpu["accept_histogram"].astype(np.int64), orc["accept_histogram"])
    assert gpu["status"] == orc["status"], (gpu["status"], orc["status"])
    return flagged
