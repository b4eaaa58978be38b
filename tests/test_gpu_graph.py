"""The verifier and the n-gram proposer captured into a HIP graph (through
torch's graph capture) and replayed: every replay, with eager work and
synchronisations between replays, must reproduce the eager call bit for bit
(the calls launch kernels only: no allocation, copy or memset is recorded)."""
import numpy as np
import pytest
import torch

from workloads import make_histories, make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _snapshot(r):
    out = [t.cpu().numpy().copy() for t in r if t is not None]
    if hasattr(r, "drafts_flat"):  # slots past draft_offsets[B] are documented as untouched
        total = int(r.draft_offsets[-1].item())
        out = [a for a in out]
        i = r._fields.index("drafts_flat")
        out[i] = out[i][:total]
    return out


def _replays_match(fn, eager):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the side stream, as capture requires
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    for rep in range(3):
        scratch = torch.randn(1 << 20, device=DEV)     # eager work between replays
        (scratch * 2.0).sum().item()
        for t in out:
            if t is not None:
                t.fill_(-7)                               # the replay must rewrite every output
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(out)
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), f"replay {rep} differs"


def test_verify_uniform_graph():
    import rejection_sampling_verification_amd as sdv
    print("[gpu-case] graph: uniform ngram B=16", flush=True)
    wl = make_workload("ngram", device=DEV, batch=16)
    lg = wl["logits"]
    B, kp1, V = lg.shape
    v = sdv.Verifier(B, kp1 - 1, V, lg.dtype, DEV, histogram=True)
    args = (wl["draft_token_ids"], wl["draft_probs"], wl["bitmask"], wl["temperature"], wl["seed"], wl["top_k"])
    eager = _snapshot(v(lg, *args))
    torch.cuda.synchronize()
    _replays_match(lambda: v(lg, *args), eager)


def test_verify_ragged_top_k_top_p_dense_graph():
    import rejection_sampling_verification_amd as sdv
    print("[gpu-case] graph: ragged long_k rows with top-k, top-p, dense q, masks", flush=True)
    wl = make_workload("long_k", device=DEV, batch=6)
    lg, q, mask = wl["logits"], wl["draft_probs"], wl["bitmask"]
    B, kp1, V = lg.shape
    k = kp1 - 1
    ks = [3, 0, 12, 7, 1, 5]
    off = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    rows = torch.cat([lg[b, :ks[b] + 1] for b in range(B)]).contiguous()
    drafts = torch.cat([wl["draft_token_ids"][b, :ks[b]] for b in range(B)]).contiguous()
    qr = torch.cat([q[b, :ks[b]] for b in range(B)]).contiguous()
    mr = torch.cat([mask[b, :ks[b] + 1] for b in range(B)]).contiguous()
    top_p = torch.tensor([0.9, 0.5, 0.0, 0.95, 0.7, 0.99], device=DEV)
    offsets = torch.tensor(off, dtype=torch.int32, device=DEV)
    v = sdv.Verifier(B, k, V, lg.dtype, DEV, debug=True, histogram=True, total_drafts=int(off[-1]))
    call = lambda: v(rows, drafts, qr, mr, wl["temperature"], 5, wl["top_k"], draft_offsets=offsets,
                     top_p=top_p)
    eager = _snapshot(call())
    torch.cuda.synchronize()
    _replays_match(call, eager)


def test_proposer_graph():
    import rejection_sampling_verification_amd as sdv
    print("[gpu-case] graph: n-gram proposer B=32", flush=True)
    h = make_histories(device=DEV, batch=32, seed=11, stride=6000, Lmin=500, max_model_len=0)
    p = sdv.NgramProposer(32, 6000, h["min_n"], h["max_n"], h["k"], 0, DEV)
    eager = _snapshot(p(h["tokens"], h["lengths"]))
    torch.cuda.synchronize()
    _replays_match(lambda: p(h["tokens"], h["lengths"]), eager)
