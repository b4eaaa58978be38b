"""Parity of the HIP verifier with the oracle for ragged draft lengths (a
cumulative offset table instead of one k), the accepted-length histogram, and
the largest draft count."""
import numpy as np
import pytest
import torch

import oracle
from parity import (announce, assert_parity, assert_parity_ragged, run_gpu, run_gpu_ragged,
                    run_oracle, run_oracle_ragged)
from workloads import make_workload, pack_bitmask

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ragged(ks, V, dtype=torch.bfloat16, dense=True, masked=False, greedy_frac=0.0, seed=0,
            top_k=None, x_argmax_frac=0.3):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    B = len(ks)
    off = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    T_total = int(off[-1])
    rows = T_total + B
    lg = (torch.randn((rows, V), generator=g, device=DEV) * 3.0).to(dtype)
    drow = torch.tensor([int(off[b]) + b + i for b in range(B) for i in range(ks[b])],
                        dtype=torch.int64, device=DEV)
    mask = None
    if masked:
        allowed = torch.rand((rows, V), generator=g, device=DEV) < 0.3
        allowed[:, 0] = True
        mask = pack_bitmask(allowed)
    q = None
    if T_total == 0:
        x = torch.zeros(0, dtype=torch.int64, device=DEV)
    elif dense:
        z = lg[drow].float() + torch.randn((T_total, V), generator=g, device=DEV)
        q = torch.softmax(z, -1).contiguous()
        x = torch.multinomial(q, 1, generator=g)[:, 0]
    else:
        x = torch.randint(0, V, (T_total,), generator=g, device=DEV)
    if T_total:
        amax = torch.argmax(lg[drow].float(), -1)
        pick = torch.rand(T_total, generator=g, device=DEV) < x_argmax_frac
        x = torch.where(pick, amax, x)
    T = 0.5 + torch.rand(B, generator=g, device=DEV)
    T = torch.where(torch.rand(B, generator=g, device=DEV) < greedy_frac, torch.zeros_like(T), T)
    tk = None
    if top_k is not None:
        choice = torch.tensor(list(top_k), dtype=torch.int32, device=DEV)
        tk = choice[torch.randint(0, len(top_k), (B,), generator=g, device=DEV)].contiguous()
    return {"logits": lg.contiguous(), "draft_token_ids": x.to(torch.int32).contiguous(),
            "draft_offsets": torch.tensor(off, dtype=torch.int32, device=DEV),
            "draft_probs": q, "bitmask": mask, "temperature": T.float().contiguous(),
            "top_k": tk, "seed": 4242 + seed}, off


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [1001, 2049, 6150, 40000])
def test_ragged_sizes(V, dtype):
    announce(f"ragged V={V} dtype={dtype}")
    ks = [0, 3, 1, 8, 5, 2, 0, 7, 4, 6, 1, 3]
    for dense, masked, tk in [(True, False, None), (False, True, (0, 3, 50)), (True, True, (0, 20))]:
        wl, off = _ragged(ks, V, dtype, dense=dense, masked=masked, greedy_frac=0.25,
                          seed=V + 3 * dense + masked, top_k=tk)
        gpu, orc = run_gpu_ragged(wl, 8), run_oracle_ragged(wl, 8)
        assert_parity_ragged(gpu, orc, off)


def test_ragged_top_p():
    announce("ragged with top-p")
    ks = [0, 3, 1, 8, 5, 2, 7]
    wl, off = _ragged(ks, 6000, dense=True, masked=True, greedy_frac=0.2, seed=77, top_k=(0, 40))
    wl["top_p"] = torch.tensor([0.9, 0.5, 0.0, 0.95, 0.7, 0.3, 0.99], device=DEV)
    gpu, orc = run_gpu_ragged(wl, 8), run_oracle_ragged(wl, 8)
    assert_parity_ragged(gpu, orc, off)


def test_ragged_largest_draft_count():
    announce("ragged k_b up to 64")
    ks = [64, 0, 17, 64, 3, 40]
    wl, off = _ragged(ks, 3000, dense=True, masked=True, greedy_frac=0.2, seed=64, top_k=(0, 10))
    gpu, orc = run_gpu_ragged(wl, 64), run_oracle_ragged(wl, 64)
    assert_parity_ragged(gpu, orc, off)


def test_uniform_largest_draft_count():
    """k = 64: more rows than waves of the finalize kernel."""
    announce("uniform k=64")
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    B, k, V = 4, 64, 2500
    lg = (torch.randn((B, k + 1, V), generator=g, device=DEV) * 3.0).to(torch.bfloat16).contiguous()
    q = torch.softmax(lg[:, :k].float() + torch.randn((B, k, V), generator=g, device=DEV), -1).contiguous()
    x = torch.multinomial(q.reshape(B * k, V), 1, generator=g)[:, 0].reshape(B, k)
    amax = torch.argmax(lg[:, :k].float(), -1)
    x = torch.where(torch.rand((B, k), generator=g, device=DEV) < 0.9, amax, x)  # long accepted runs
    T = torch.tensor([1.0, 0.0, 0.7, 1.2], device=DEV)
    for probs in (q, None):
        wl = {"logits": lg, "draft_token_ids": x.to(torch.int32).contiguous(), "draft_probs": probs,
              "bitmask": None, "temperature": T, "top_k": None, "seed": 99}
        assert_parity(run_gpu(wl), run_oracle(wl))


def test_ragged_long_dense_rows():
    """Rows of 32 blocks or more: the grid-wide residual kernels, ragged."""
    announce("ragged dense V=65536")
    wl, off = _ragged([2, 0, 5, 1, 3], 65536, dense=True, masked=True, greedy_frac=0.2, seed=5,
                      top_k=(0, 0, 30))
    gpu, orc = run_gpu_ragged(wl, 5), run_oracle_ragged(wl, 5)
    assert_parity_ragged(gpu, orc, off)


def test_ragged_counter_example():
    """fanout, "Work a denominator example", with draft lengths 3..7."""
    announce("ragged counter example")
    cyc = [3, 4, 5, 6, 7]
    kinds = ["accept_all"] * 120 + ["invalid_all"] * 40 + ["reject_first"] * 40
    ks = [cyc[b % 5] for b in range(200)]
    rng = np.random.default_rng(0)
    V = 64
    off = np.concatenate([[0], np.cumsum(ks)]).astype(np.int64)
    rows = int(off[-1]) + 200
    logits = rng.normal(size=(rows, V)).astype(np.float32)
    gmax = rng.integers(0, V, size=rows)
    logits[np.arange(rows), gmax] += 20.0
    x = np.zeros(int(off[-1]), dtype=np.int64)
    allowed = np.ones((rows, V), dtype=bool)
    for b, kind in enumerate(kinds):
        for i in range(ks[b]):
            r = off[b] + b + i
            if kind == "accept_all":
                x[off[b] + i] = gmax[r]
            else:
                x[off[b] + i] = (gmax[r] + 1 + rng.integers(0, V - 1)) % V
                if kind == "invalid_all":
                    allowed[r, x[off[b] + i]] = False
    wl = {"logits": torch.tensor(logits, device=DEV),
          "draft_token_ids": torch.tensor(x, dtype=torch.int32, device=DEV),
          "draft_offsets": torch.tensor(off, dtype=torch.int32, device=DEV),
          "draft_probs": None, "bitmask": pack_bitmask(torch.tensor(allowed, device=DEV)),
          "temperature": torch.zeros(200, device=DEV), "top_k": None, "seed": 1}
    gpu = run_gpu_ragged(wl, 7)
    assert [int(v) for v in gpu["counters"]] == [1000, 200, 800, 600]
    assert_parity_ragged(gpu, run_oracle_ragged(wl, 7), off)


def test_ragged_malformed_offsets():
    announce("ragged malformed offsets")
    ks = [2, 3, 1, 4]
    wl, off = _ragged(ks, 3000, dense=True, seed=8)
    for bad in ([0, 2, 1, 6, 10], [1, 2, 5, 6, 10], [0, 2, 5, 6, 9]):
        # the same row and draft counts, offsets that do not hold
        wl["draft_offsets"] = torch.tensor(bad, dtype=torch.int32, device=DEV)
        gpu = run_gpu_ragged(wl, 4)
        assert list(gpu["out_num_accepted"]) == [-1] * 4
        assert gpu["status"] == oracle.verify.ST_BAD_OFFSETS
        assert [int(v) for v in gpu["counters"]] == [0, 0, 0, 0]
        assert int(gpu["accept_histogram"].sum()) == 0
    # a draft count above the maximum voids the call too
    wl["draft_offsets"] = torch.tensor(off, dtype=torch.int32, device=DEV)
    gpu = run_gpu_ragged(wl, 3)
    assert gpu["status"] == oracle.verify.ST_BAD_OFFSETS


def test_uniform_histogram():
    announce("uniform histogram ngram B=32")
    import rejection_sampling_verification_amd as sdv
    wl = make_workload("ngram", device=DEV, batch=32)
    lg = wl["logits"]
    B, kp1, V = lg.shape
    v = sdv.Verifier(B, kp1 - 1, V, lg.dtype, lg.device, histogram=True)
    r = v(lg, wl["draft_token_ids"], None, None, wl["temperature"], wl["seed"])
    torch.cuda.synchronize()
    orc = run_oracle(wl)
    flagged = [b for b in range(B) if orc["flag_accept"][b] or orc["flag_gumbel"][b]]
    if not flagged:
        assert np.array_equal(r.accept_histogram.cpu().numpy().astype(np.int64), orc["accept_histogram"])
    assert int(r.accept_histogram.sum().item()) == B


def test_ngram_ragged_full():
    """The ragged ngram workload at full size (B=256, k_b 1..7, V=151936),
    every request against the oracle (one-hot drafts keep it quick)."""
    announce("ngram_ragged full")
    wl = make_workload("ngram_ragged", device=DEV)
    off = wl["draft_offsets"].cpu().numpy()
    gpu, orc = run_gpu_ragged(wl, wl["max_draft"]), run_oracle_ragged(wl, wl["max_draft"])
    assert_parity_ragged(gpu, orc, off)
    assert int(gpu["counters"][0]) == int(off[-1]) and gpu["status"] == 0


@pytest.mark.parametrize("case", ["requests", "rows"])
def test_ragged_beyond_the_sweeps_own_mapping(case):
    """Ragged calls with more requests (2100) or more rows (8229) than the
    sweep maps in LDS take the prep kernel's row table; one just inside both
    limits maps itself.  Aligned bf16 rows, no threshold pass."""
    announce(f"ragged beyond the sweep's own mapping: {case}")
    g = np.random.default_rng(7 if case == "requests" else 8)
    if case == "requests":
        ks = list(g.integers(0, 3, size=2100))
    else:
        ks = list(g.integers(1, 9, size=1500))    # 8229 rows with this seed
    wl, off = _ragged(ks, 1024, dense=False, greedy_frac=0.25, seed=11 if case == "requests" else 12)
    kmax = max(int(x) for x in ks)
    gpu, orc = run_gpu_ragged(wl, kmax), run_oracle_ragged(wl, kmax)
    assert_parity_ragged(gpu, orc, off)
    rows = int(off[-1]) + len(ks)
    assert (len(ks) > 2048) if case == "requests" else (rows > 8192)
    # just inside both limits: 2048 requests, at most 8192 rows
    ks2 = [3] * 2048
    wl2, off2 = _ragged(ks2, 1024, dense=False, greedy_frac=0.25, seed=13)
    gpu2, orc2 = run_gpu_ragged(wl2, 3), run_oracle_ragged(wl2, 3)
    assert_parity_ragged(gpu2, orc2, off2)
