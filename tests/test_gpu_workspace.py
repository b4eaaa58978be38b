"""The verifier's workspace contract: zero-filled once before its first use,
it is left ready for the next call (its first 16 KB, the row sweep's block
claim counters, are back at zero after every call, on every path), so
verifiers of different shapes can share one workspace."""
import numpy as np
import pytest
import torch

from workloads import make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda"
CLAIM_BYTES = 16384


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outs(r):
    return [t.cpu().numpy().copy() for t in (r.out_tokens, r.out_num_accepted, r.out_counters)]


def _args(wl):
    return (wl["logits"], wl["draft_token_ids"], wl["draft_probs"], wl["bitmask"], wl["temperature"],
            wl["seed"], wl["top_k"])


def _unaligned(wl):
    """The same call with V - 3 tokens per row: rows are no longer 16-byte
    aligned, so the element path runs."""
    V = wl["logits"].shape[-1] - 3
    out = dict(wl)
    out["logits"] = wl["logits"][..., :V].contiguous()
    out["draft_token_ids"] = wl["draft_token_ids"].clamp(max=V - 1).contiguous()
    if wl["draft_probs"] is not None:
        q = wl["draft_probs"][..., :V]
        out["draft_probs"] = (q / q.sum(-1, keepdim=True)).contiguous()
    if wl["bitmask"] is not None:
        out["bitmask"] = wl["bitmask"][..., :(V + 31) // 32].contiguous()
    return out


CASES = [  # (workload, batch, unaligned)
    ("ngram", 16, False),
    ("draft_model", 8, False),
    ("structured", 8, False),   # masks, dense q
    ("long_k", 6, False),       # top-k, masks, greedy rows
    ("tiny", None, False),      # fp32
    ("ngram", 6, True),
]


def test_claim_counters_return_to_zero():
    import rejection_sampling_verification_amd as sdv
    for name, batch, unaligned in CASES:
        print(f"[gpu-case] workspace: counters after {name} B={batch} unaligned={unaligned}", flush=True)
        wl = make_workload(name, device=DEV, batch=batch)
        if unaligned:
            wl = _unaligned(wl)
        B, kp1, V = wl["logits"].shape
        v = sdv.Verifier(B, kp1 - 1, V, wl["logits"].dtype, DEV)
        for _ in range(3):
            v(*_args(wl))
            torch.cuda.synchronize()
            assert int(v.workspace[:CLAIM_BYTES].count_nonzero()) == 0, name


def test_claim_counters_return_to_zero_ragged():
    import rejection_sampling_verification_amd as sdv
    print("[gpu-case] workspace: counters after a ragged call with top-k", flush=True)
    wl = make_workload("long_k", device=DEV, batch=5)
    lg, mask = wl["logits"], wl["bitmask"]
    B, kp1, V = lg.shape
    ks = [3, 0, 12, 7, 1]
    off = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    rows = torch.cat([lg[b, :ks[b] + 1] for b in range(B)]).contiguous()
    drafts = torch.cat([wl["draft_token_ids"][b, :ks[b]] for b in range(B)]).contiguous()
    mr = torch.cat([mask[b, :ks[b] + 1] for b in range(B)]).contiguous()
    offsets = torch.tensor(off, dtype=torch.int32, device=DEV)
    v = sdv.Verifier(B, kp1 - 1, V, lg.dtype, DEV, total_drafts=int(off[-1]))
    for _ in range(2):
        v(rows, drafts, None, mr, wl["temperature"], 3, wl["top_k"], draft_offsets=offsets)
        torch.cuda.synchronize()
        assert int(v.workspace[:CLAIM_BYTES].count_nonzero()) == 0
    # malformed offsets: nothing is swept, the counters stay at zero
    bad = torch.tensor([0, 5, 2, 20, 21, 23], dtype=torch.int32, device=DEV)
    r = v(rows, drafts, None, mr, wl["temperature"], 3, wl["top_k"], draft_offsets=bad)
    torch.cuda.synchronize()
    assert int(r.status.item()) != 0
    assert int(v.workspace[:CLAIM_BYTES].count_nonzero()) == 0


def test_shapes_share_one_workspace():
    import rejection_sampling_verification_amd as sdv
    print("[gpu-case] workspace: three shapes alternate on one workspace", flush=True)
    wls = [make_workload("ngram", device=DEV, batch=24), make_workload("draft_model", device=DEV, batch=8),
           make_workload("structured", device=DEV, batch=4)]
    sizes = [sdv.sd_verify_workspace_size(w["logits"].shape[0], w["logits"].shape[1] - 1, w["logits"].shape[2],
                                          w["logits"].dtype) for w in wls]
    shared = torch.zeros(max(sizes), dtype=torch.uint8, device=DEV)
    own = [sdv.Verifier(w["logits"].shape[0], w["logits"].shape[1] - 1, w["logits"].shape[2],
                        w["logits"].dtype, DEV) for w in wls]
    ref = [_outs(v(*_args(w))) for v, w in zip(own, wls)]
    torch.cuda.synchronize()
    users = [sdv.Verifier(w["logits"].shape[0], w["logits"].shape[1] - 1, w["logits"].shape[2],
                          w["logits"].dtype, DEV, workspace=shared) for w in wls]
    for order in ([0, 1, 2], [2, 0, 1], [1, 1, 0, 2, 0]):
        for i in order:
            got = _outs(users[i](*_args(wls[i])))
            torch.cuda.synchronize()
            for a, b in zip(got, ref[i]):
                assert np.array_equal(a, b), i


def test_workspace_argument_checked():
    import rejection_sampling_verification_amd as sdv
    ws = sdv.sd_verify_workspace_size(4, 3, 1000, torch.float32)
    with pytest.raises(ValueError):
        sdv.Verifier(4, 3, 1000, torch.float32, DEV, workspace=torch.zeros(ws - 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        sdv.Verifier(4, 3, 1000, torch.float32, DEV, workspace=torch.zeros(ws, dtype=torch.int32, device=DEV))
