"""Parity of the HIP n-gram proposer with the oracle: every output exact
(integer work), on the full 256-request history table, on small random tables
that span several 2048-position chunks with ragged tails, on long histories,
on the edge cases of the rule, and fed into the ragged verifier."""
import numpy as np
import pytest
import torch

import oracle
from oracle.ngram import NG_BAD_LENGTH, propose_batch
from parity import announce, assert_parity_ragged, run_gpu_ragged, run_oracle_ragged
from workloads import make_histories

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _gpu(tokens, lengths, min_n, max_n, k, max_model_len=0, prop=None):
    import rejection_sampling_verification_amd as sdv
    t = torch.as_tensor(np.asarray(tokens), dtype=torch.int32).to(DEV).contiguous()
    ln = torch.as_tensor(np.asarray(lengths), dtype=torch.int32).to(DEV).contiguous()
    if prop is None:
        prop = sdv.NgramProposer(t.shape[0], t.shape[1], min_n, max_n, k, max_model_len, DEV)
    r = prop(t, ln)
    torch.cuda.synchronize()
    return {name: getattr(r, name).cpu().numpy().copy() for name in r._fields}


def _assert_same(g, o):
    B = o["num_drafts"].shape[0]
    assert np.array_equal(g["num_drafts"], o["num_drafts"]), np.flatnonzero(g["num_drafts"] != o["num_drafts"])[:10]
    assert np.array_equal(g["match_len"], o["match_len"])
    assert np.array_equal(g["drafts"].astype(np.int64), o["drafts"])
    assert np.array_equal(g["draft_offsets"].astype(np.int64), o["draft_offsets"])
    total = int(o["draft_offsets"][B])
    assert np.array_equal(g["drafts_flat"][:total].astype(np.int64), o["flat"])
    assert int(g["status"][0]) == o["status"]


def test_full_history_table():
    announce("ngram_propose full B=256 stride=16384")
    wl = make_histories()
    g = _gpu(wl["tokens"].numpy(), wl["lengths"].numpy(), wl["min_n"], wl["max_n"], wl["k"], wl["max_model_len"])
    o = propose_batch(wl["tokens"].numpy(), wl["lengths"].numpy(), wl["min_n"], wl["max_n"], wl["k"],
                      wl["max_model_len"])
    _assert_same(g, o)
    assert int(o["num_drafts"].sum()) > 600          # the recipe makes most requests hit


@pytest.mark.parametrize("alphabet", [2, 3, 50])
def test_random_tables(alphabet):
    rng = np.random.default_rng(alphabet)
    for trial in range(12):
        B = int(rng.integers(1, 40))
        stride = int(rng.choice([1, 7, 2047, 2048, 2049, 4100, 6145]))
        tokens = rng.integers(0, alphabet, size=(B, stride))
        lengths = rng.integers(0, stride + 1, size=B)
        lengths[rng.random(B) < 0.1] = -1
        lengths[rng.random(B) < 0.1] = stride + 1
        lengths[rng.random(B) < 0.1] = stride
        min_n = int(rng.integers(1, 4))
        max_n = int(rng.choice([min_n, min_n + 2, 8, 256]))
        max_n = max(min_n, min(max_n, 256))
        k = int(rng.choice([0, 1, 4, 7, 64]))
        mml = int(rng.choice([0, stride, stride + 5]))
        announce(f"ngram random alphabet={alphabet} trial={trial} B={B} stride={stride} "
                 f"n={min_n}..{max_n} k={k} max_model_len={mml}")
        g = _gpu(tokens, lengths, min_n, max_n, k, mml)
        o = propose_batch(tokens, lengths, min_n, max_n, k, mml)
        _assert_same(g, o)


def test_long_histories_and_chunk_boundaries():
    """Histories of 2e5 tokens (98 chunks): a constant run (every window hits,
    the earliest end wins), a tail planted once, straddling a chunk boundary,
    and once near the end."""
    rng = np.random.default_rng(11)
    stride = 200_000
    B = 6
    tokens = rng.integers(0, 1 << 20, size=(B, stride))
    lengths = np.array([stride, stride, 150_001, 2048 * 7 + 3, stride - 1, 99_999])
    tokens[0, :] = 5                                          # constant
    tail = tokens[1, stride - 9:stride].copy()
    tokens[1, 4096 - 4:4096 + 5] = tail                       # straddles the boundary at 4096
    tokens[1, 180_000:180_009] = tail                         # a later copy loses
    L2 = 150_001
    tokens[2, L2 - 12:L2 - 6] = tokens[2, L2 - 6:L2]          # the only copy ends right before the tail
    L3 = 2048 * 7 + 3
    tokens[3, 2048 * 3 - 2:2048 * 3 + 3] = tokens[3, L3 - 5:L3]   # ends 3 past a chunk start
    for mn, mx, k in [(1, 5, 4), (2, 9, 7), (3, 256, 64), (9, 9, 3)]:
        announce(f"ngram long histories n={mn}..{mx} k={k}")
        g = _gpu(tokens, lengths, mn, mx, k)
        o = propose_batch(tokens, lengths, mn, mx, k)
        _assert_same(g, o)
    assert o["match_len"][1] == 9 and o["num_drafts"][1] == 3


def test_edge_cases():
    announce("ngram edge cases")
    stride = 12
    rows = [
        ([10, 11, 12, 20, 21, 99, 10, 11, 12], 2, 4, 3),       # the pages' lookups
        ([7, 8, 1, 7, 8, 2, 7, 8], 2, 4, 3),
        ([1, 2, 3, 4, 5], 2, 4, 3),                              # nothing repeats
        ([], 1, 4, 3), ([7], 1, 4, 3), ([7, 7], 1, 4, 3),        # too short, shortest hit
        ([5] * 12, 2, 3, 4),                                     # overlaps the tail
    ]
    for h, mn, mx, k in rows:
        tokens = np.full((1, stride), 1234)
        tokens[0, :len(h)] = h
        g = _gpu(tokens, [len(h)], mn, mx, k)
        o = propose_batch(tokens, [len(h)], mn, mx, k)
        _assert_same(g, o)
        assert (int(g["match_len"][0]) or None, list(g["drafts"][0, :g["num_drafts"][0]])) == \
            oracle.ngram.propose_one(h, mn, mx, k)
    # bad lengths set the status bit and leave the request without drafts
    tokens = np.tile(np.array([1, 2, 1, 2, 1, 2, 1, 2]), (3, 1))
    g = _gpu(tokens, [-3, 8, 9], 1, 3, 2)
    assert list(g["num_drafts"]) == [0, 2, 0] and int(g["status"][0]) == NG_BAD_LENGTH


def test_repeated_calls_share_the_workspace():
    import rejection_sampling_verification_amd as sdv
    announce("ngram repeated calls")
    rng = np.random.default_rng(3)
    B, stride = 64, 5000
    prop = sdv.NgramProposer(B, stride, 2, 6, 5, 0, DEV)
    for trial in range(3):
        tokens = rng.integers(0, 4, size=(B, stride))
        lengths = rng.integers(0, stride + 1, size=B)
        _assert_same(_gpu(tokens, lengths, 2, 6, 5, prop=prop), propose_batch(tokens, lengths, 2, 6, 5))


def test_empty_batch():
    import rejection_sampling_verification_amd as sdv
    announce("ngram empty batch")
    prop = sdv.NgramProposer(0, 100, 2, 4, 3, 0, DEV)
    r = prop(torch.zeros((0, 100), dtype=torch.int32, device=DEV), torch.zeros(0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert r.draft_offsets.cpu().tolist() == [0] and int(r.status.item()) == 0


def test_proposals_feed_the_ragged_verifier():
    """Histories -> GPU drafts -> ragged verify on synthetic target logits,
    against the oracle on the same drafts."""
    announce("ngram drafts into the ragged verifier")
    V = 3000
    wl = make_histories(batch=48, seed=5, V=V, stride=4096, Lmin=256, max_model_len=0)
    g = _gpu(wl["tokens"].numpy(), wl["lengths"].numpy(), wl["min_n"], wl["max_n"], wl["k"])
    off = g["draft_offsets"].astype(np.int64)
    B, total = 48, int(off[-1])
    gen = torch.Generator(device=DEV)
    gen.manual_seed(9)
    rows = total + B
    logits = (torch.randn((rows, V), generator=gen, device=DEV) * 3.0).to(torch.bfloat16)
    x = torch.tensor(g["drafts_flat"][:total], dtype=torch.int32, device=DEV)
    # make the target agree with a share of the drafts, as a target reusing text would
    drow = torch.tensor([int(off[b]) + b + i for b in range(B) for i in range(int(off[b + 1] - off[b]))],
                        dtype=torch.int64, device=DEV)
    if total:
        agree = torch.rand(total, generator=gen, device=DEV) < 0.7
        lf = logits.float()
        lf[drow[agree], x[agree].long()] = lf[drow].max(dim=1).values[agree] + 2.0
        logits = lf.to(torch.bfloat16)
    T = torch.where(torch.rand(B, generator=gen, device=DEV) < 0.3, torch.zeros(B, device=DEV),
                    torch.ones(B, device=DEV))
    vw = {"logits": logits.contiguous(), "draft_token_ids": x.contiguous(),
          "draft_offsets": torch.tensor(off, dtype=torch.int32, device=DEV), "draft_probs": None,
          "bitmask": None, "temperature": T.contiguous(), "top_k": None, "seed": 31}
    gv, ov = run_gpu_ragged(vw, wl["k"]), run_oracle_ragged(vw, wl["k"])
    assert_parity_ragged(gv, ov, off)
    assert int(gv["counters"][0]) == total and total > 0
