"""Parity of the HIP verifier with the oracle on the GPU.

Every workload is compared request by request in full, the full-size ngram,
structured and long_k workloads included (the benchmark's shapes and launch
configuration): tokens, accepted counts, counters and status exactly, accept
probabilities within 1e-5 relative, row log-normalisers within 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import announce, assert_parity, run_gpu, run_oracle, run_oracle_parallel
from workloads import make_workload, pack_bitmask

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _custom(B, k, V, dtype=torch.bfloat16, dense=True, masked=False, greedy_frac=0.0,
            std=3.0, density=0.3, seed=0, x_argmax_frac=0.3, integer_logits=False, top_k=None):
    """Small synthetic case with any shape (inputs only)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    kp1 = k + 1
    if integer_logits:
        lg = torch.randint(-3, 4, (B, kp1, V), generator=g, device=DEV).float()
    else:
        lg = torch.randn((B, kp1, V), generator=g, device=DEV) * std
    lg = lg.to(dtype)
    allowed = None
    mask = None
    if masked:
        allowed = torch.rand((B, kp1, V), generator=g, device=DEV) < density
        allowed[..., 0] = True
        mask = pack_bitmask(allowed)
    q = None
    if dense:
        z = lg[:, :k].float() + torch.randn((B, k, V), generator=g, device=DEV)
        q = torch.softmax(z, -1).contiguous()
        x = torch.multinomial(q.reshape(B * k, V), 1, generator=g)[:, 0].reshape(B, k)
    else:
        x = torch.randint(0, V, (B, k), generator=g, device=DEV)
    amax = torch.argmax(lg[:, :k].float(), -1) if k else x
    pick = torch.rand((B, k), generator=g, device=DEV) < x_argmax_frac
    x = torch.where(pick, amax, x)
    T = 0.5 + torch.rand(B, generator=g, device=DEV)
    T = torch.where(torch.rand(B, generator=g, device=DEV) < greedy_frac, torch.zeros_like(T), T)
    tk = None
    if top_k is not None:  # per request, drawn from the given choices
        choice = torch.tensor(list(top_k), dtype=torch.int32, device=DEV)
        tk = choice[torch.randint(0, len(top_k), (B,), generator=g, device=DEV)].contiguous()
    return {"name": "custom", "logits": lg.contiguous(), "draft_token_ids": x.to(torch.int32).contiguous(),
            "draft_probs": q, "bitmask": mask, "temperature": T.float().contiguous(), "top_k": tk,
            "seed": 12345 + seed}


# ------------------------------------------------------------ whole workloads

def test_tiny_full():
    announce("tiny full")
    wl = make_workload("tiny", device=DEV)
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_draft_model_full():
    announce("draft_model full B=64 k=5 V=32000")
    wl = make_workload("draft_model", device=DEV)
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_draft_model_as_one_hot():
    announce("draft_model drafts without q")
    wl = make_workload("draft_model", device=DEV, batch=32)
    wl["draft_probs"] = None
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_ngram_scaled():
    announce("ngram B=16 k=4 V=151936")
    wl = make_workload("ngram", device=DEV, batch=16)
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_structured_scaled():
    announce("structured B=12 k=5 V=128256")
    wl = make_workload("structured", device=DEV, batch=12)
    gpu, orc = run_gpu(wl), run_oracle(wl)
    assert_parity(gpu, orc)
    R, I, D, A = (int(v) for v in gpu["counters"])
    assert R == 60 and I == 12 and D == 48        # exactly 20% invalid drafts


@pytest.mark.timeout(900)
def test_ngram_full_every_request():
    announce("ngram full B=256 k=4 V=151936, every request against the oracle")
    wl = make_workload("ngram", device=DEV)
    gpu = run_gpu(wl)
    orc = run_oracle_parallel(wl)
    assert_parity(gpu, orc)
    B, k = 256, 4
    R, I, D, A = (int(v) for v in gpu["counters"])
    assert (R, I, D) == (B * k, 0, B * k) and A == int(orc["counters"][3])
    assert gpu["status"] == 0 and int(gpu["flags"][0]) + int(gpu["flags"][1]) == 0


@pytest.mark.timeout(900)
def test_structured_full_every_request():
    announce("structured full B=128 k=5 V=128256, every request against the oracle")
    wl = make_workload("structured", device=DEV)
    gpu = run_gpu(wl)
    orc = run_oracle_parallel(wl)
    assert_parity(gpu, orc)
    R, I, D, A = (int(v) for v in gpu["counters"])
    assert (R, I, D) == (640, 128, 512)           # survival exactly 80%
    assert A == int(orc["counters"][3]) and A <= D


@pytest.mark.timeout(900)
def test_long_k_full_every_request():
    announce("long_k full B=512 k=12 V=151936 top-k 50, every request against the oracle")
    wl = make_workload("long_k", device=DEV)
    gpu = run_gpu(wl)
    orc = run_oracle_parallel(wl)
    assert_parity(gpu, orc)
    B, k = 512, 12
    R, I, D, A = (int(v) for v in gpu["counters"])
    assert R == B * k and D == R - I and A == int(orc["counters"][3]) and gpu["status"] == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [7, 1001, 2049, 6150, 20000])
def test_top_k_sizes(V, dtype):
    announce(f"top-k custom V={V} dtype={dtype}")
    for dense, masked in [(True, False), (False, True), (True, True)]:
        wl = _custom(10, 3, V, dtype=dtype, dense=dense, masked=masked, greedy_frac=0.2,
                     seed=V + 3 * dense + masked, top_k=(0, 1, 2, 5, 50, V + 5))
        assert_parity(run_gpu(wl), run_oracle(wl))


def test_top_k_rows_longer_than_the_single_pass_takes():
    """Aligned bf16 rows of 300000 tokens (147 blocks: more line maxima than
    the single-pass top-k holds), so the two-pass selection runs them."""
    announce("top-k aligned V=300000 (two-pass selection)")
    wl = _custom(3, 2, 300000, dense=False, masked=True, density=0.3, seed=17, top_k=(1, 50, 4000))
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_top_k_ties():
    announce("top-k with integer logits: many ties at the threshold")
    for dtype in (torch.bfloat16, torch.float32):
        wl = _custom(24, 4, 5000, dtype=dtype, dense=True, integer_logits=True, seed=21,
                     top_k=(1, 3, 10, 700))
        assert_parity(run_gpu(wl), run_oracle(wl))


def test_top_k_threshold_far_from_the_first_tokens():
    """The threshold lies far above the first 16 KB of the row (the window
    moves up) or far below it among widely spread magnitudes (it moves down)."""
    announce("top-k window moves")
    B, k, V = 6, 2, 20000
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    for dtype in (torch.float32, torch.bfloat16):
        lg = torch.randn((B, k + 1, V), generator=g, device=DEV)
        lg[:3, :, 4096:] += 60.0                          # far above the first tokens
        mag = torch.exp(torch.rand((3, k + 1, V), generator=g, device=DEV) * 40 - 20)
        lg[3:] = mag * torch.sign(torch.randn((3, k + 1, V), generator=g, device=DEV))
        lg = lg.to(dtype).contiguous()
        x = torch.randint(0, V, (B, k), generator=g, device=DEV).to(torch.int32)
        wl = {"name": "custom", "logits": lg, "draft_token_ids": x, "draft_probs": None,
              "bitmask": None, "temperature": torch.full((B,), 1.5, device=DEV),
              "top_k": torch.tensor([40, 3000, 15000, 40, 3000, 15000], dtype=torch.int32, device=DEV),
              "seed": 77}
        assert_parity(run_gpu(wl), run_oracle(wl))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_top_k_single_pass_edge_rows(dtype):
    """Rows of a top-k call (aligned rows, threshold found after the sweep)
    that leave the usual path: an allowed NaN or +inf (reported), a NaN at a
    masked token (ignored), an empty row, fewer allowed tokens than K (no
    cut), exactly K, K = 1, and K = 2000 (more candidate lines than LDS
    holds)."""
    announce(f"top-k single-pass edge rows dtype={dtype}")
    B, k, V = 10, 3, 8192
    wl = _custom(B, k, V, dtype=dtype, dense=True, masked=False, seed=91, top_k=(50,))
    g = torch.Generator(device=DEV)
    g.manual_seed(92)
    allowed = torch.rand((B, k + 1, V), generator=g, device=DEV) < 0.3
    for b, n in ((4, 20), (5, 50), (8, 1)):          # rows with exactly n allowed tokens
        allowed[b] = False
        for i in range(k + 1):
            allowed[b, i, torch.randperm(V, generator=g, device=DEV)[:n]] = True
    allowed[0, 1, 100] = True
    allowed[1, 2, 5000] = True
    allowed[2, 0, 300] = False
    allowed[3, 1] = False                             # empty row
    wl["bitmask"] = pack_bitmask(allowed)
    wl["logits"][0, 1, 100] = float("nan")
    wl["logits"][1, 2, 5000] = float("inf")
    wl["logits"][2, 0, 300] = float("nan")
    wl["top_k"] = torch.tensor([50, 50, 50, 50, 50, 50, 1, 2000, 50, 7], dtype=torch.int32, device=DEV)
    wl["temperature"][9] = 0.0                        # greedy beside them
    gpu, orc = run_gpu(wl), run_oracle(wl)
    assert list(orc["request_status"]) == [8, 8, 0, 4, 0, 0, 0, 0, 0, 0]
    assert_parity(gpu, orc)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V", [7, 1001, 2049, 6150, 20000])
def test_top_p_sizes(V, dtype):
    announce(f"top-p custom V={V} dtype={dtype}")
    for dense, masked, tk in [(True, False, None), (False, True, (0, 5, 50)), (True, True, (0, 20))]:
        wl = _custom(10, 3, V, dtype=dtype, dense=dense, masked=masked, greedy_frac=0.2,
                     seed=2 * V + 3 * dense + masked, top_k=tk)
        g = torch.Generator(device=DEV)
        g.manual_seed(V)
        choice = torch.tensor([0.0, 0.3, 0.9, 0.99, 1.0], device=DEV)
        wl["top_p"] = choice[torch.randint(0, 5, (10,), generator=g, device=DEV)].contiguous()
        assert_parity(run_gpu(wl), run_oracle(wl))


def test_top_p_ties_and_extremes():
    announce("top-p with integer logits and extreme values")
    for dtype in (torch.bfloat16, torch.float32):
        wl = _custom(24, 4, 5000, dtype=dtype, dense=True, integer_logits=True, seed=31)
        wl["top_p"] = torch.tensor([1e-6, 0.2, 0.5, 0.8, 0.95, 0.999] * 4, device=DEV)
        assert_parity(run_gpu(wl), run_oracle(wl))
        # a wide spread of logits: the cut far below the largest value
        wl = _custom(8, 2, 30000, dtype=dtype, dense=False, std=25.0, seed=32)
        wl["top_p"] = torch.full((8,), 0.97, device=DEV)
        assert_parity(run_gpu(wl), run_oracle(wl))


def test_top_p_after_top_k_paths():
    """bf16 rows whose top-k histogram holds every kept token (the cut comes
    from it), rows whose largest values lie above that histogram's window
    (the cut takes passes over the row), and rows where top-k keeps all."""
    announce("top-p after top-k: histogram and pass paths")
    g = torch.Generator(device=DEV)
    g.manual_seed(8)
    B, k, V = 9, 2, 40000
    lg = torch.randn((B, k + 1, V), generator=g, device=DEV) * 2.0
    lg[3:6, :, 20000:] += 60.0                       # far above the first 16 KB of the row
    x = torch.randint(0, V, (B, k), generator=g, device=DEV).to(torch.int32)
    for dtype in (torch.bfloat16, torch.float32):
        wl = {"name": "custom", "logits": lg.to(dtype).contiguous(), "draft_token_ids": x,
              "draft_probs": None, "bitmask": None, "temperature": torch.full((B,), 0.9, device=DEV),
              "top_k": torch.tensor([50, 700, 5000] * 3, dtype=torch.int32, device=DEV),
              "top_p": torch.tensor([0.5, 0.9, 0.99] * 3, device=DEV), "seed": 78}
        wl["top_k"][6:] = V + 5                      # keeps every token
        assert_parity(run_gpu(wl), run_oracle(wl))


def test_top_p_after_top_k_over_spread_magnitudes():
    """Top-p after top-k where what top-k keeps spans many binades (the cut
    then comes from passes over the row, not the staged candidates' window),
    with more candidate lines than LDS stages, beside top-p alone (top-k 0)."""
    announce("top-p after top-k over widely spread magnitudes")
    B, k, V = 8, 2, 20000
    g = torch.Generator(device=DEV)
    g.manual_seed(15)
    for dtype in (torch.bfloat16, torch.float32):
        mag = torch.exp(torch.rand((B, k + 1, V), generator=g, device=DEV) * 40 - 20)
        lg = (mag * torch.sign(torch.randn((B, k + 1, V), generator=g, device=DEV))).to(dtype).contiguous()
        x = torch.randint(0, V, (B, k), generator=g, device=DEV).to(torch.int32)
        wl = {"name": "custom", "logits": lg, "draft_token_ids": x, "draft_probs": None,
              "bitmask": None, "temperature": torch.full((B,), 20.0, device=DEV),
              "top_k": torch.tensor([40, 3000, 15000, 0, 40, 3000, 15000, 0], dtype=torch.int32, device=DEV),
              "top_p": torch.tensor([0.9, 0.9, 0.99, 0.9, 0.5, 0.3, 0.999, 0.7], device=DEV), "seed": 79}
        assert_parity(run_gpu(wl), run_oracle(wl))


@pytest.mark.parametrize("V", [40000, 70000])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dense_residual_from_listed_lines(V, dtype):
    """Dense q after the single-pass selection: rows whose kept tokens it
    lists by line draw the residual from those lines alone, beside rows it
    does not list (top-k 0, more candidate lines than it stages) in the same
    call; with and without top-p and a mask, rows of 20 blocks (residual
    inside the finalize kernel) and 35 blocks (the grid-wide residual for the
    rows not listed, on a grid of fewer request rows than requests, each
    taking a stripe of them)."""
    B = 48 if V < 65536 else 160
    announce(f"dense residual from listed lines B={B} V={V} dtype={dtype}")
    for masked in (False, True):
        wl = _custom(B, 4, V, dtype=dtype, dense=True, masked=masked, greedy_frac=0.1, density=0.5,
                     seed=41 + masked, x_argmax_frac=0.2, top_k=(0, 1, 5, 50, 400))
        assert_parity(run_gpu(wl), run_oracle(wl))
        g = torch.Generator(device=DEV)
        g.manual_seed(43 + masked)
        wl["top_p"] = torch.where(torch.rand(B, generator=g, device=DEV) < 0.5,
                                  torch.rand(B, generator=g, device=DEV) * 0.9 + 0.05,
                                  torch.zeros(B, device=DEV)).contiguous()
        assert_parity(run_gpu(wl), run_oracle(wl))


@pytest.mark.parametrize("cut", ["top_k", "top_k_top_p"])
def test_chi_square_listed_residual(cut):
    """Emitted tokens follow the cut target law when the residual comes from
    the lines the single-pass selection lists: bf16 rows of two blocks
    (V=4096), the kept tokens spread over several lines of both, dense q
    spread over the whole row, so that most positions reject and resample."""
    from scipy import stats
    from oracle import verify as ov
    announce(f"chi-square of the listed-line residual ({cut})")
    B, k, V = 50000, 2, 4096
    g = torch.Generator(device="cpu")
    g.manual_seed(23)
    l1 = torch.randn((k + 1, V), generator=g).to(torch.bfloat16)
    allowed = torch.ones((k + 1, V), dtype=torch.bool)
    T = 0.9
    top_k = 20 if cut == "top_k" else 30
    top_p = 0.8 if cut == "top_k_top_p" else 0.0
    p = np.array([ov.target_distribution(l1[i].double().numpy(), allowed[i].numpy(), T, top_k, top_p)[0]
                  for i in range(k + 1)])
    q1 = torch.softmax(torch.randn((k, V), generator=g), -1)
    x = torch.stack([torch.multinomial(q1[i], B, replacement=True, generator=g) for i in range(k)], 1)
    wl = {"logits": l1.expand(B, k + 1, V).contiguous().to(DEV),
          "draft_token_ids": x.to(torch.int32).to(DEV),
          "draft_probs": q1.expand(B, k, V).contiguous().to(DEV),
          "bitmask": None,
          "temperature": torch.full((B,), T, device=DEV),
          "top_k": torch.full((B,), top_k, dtype=torch.int32, device=DEV),
          "top_p": torch.full((B,), top_p, device=DEV) if top_p else None,
          "seed": 2025}
    runs = [run_gpu(wl, seed=2025 + r) for r in range(4)]
    tok = np.concatenate([g["out_tokens"] for g in runs])
    na = np.concatenate([g["out_num_accepted"] for g in runs])
    assert (na == 0).mean() > 0.5  # most draws are residual draws
    for i in range(k + 1):
        sel = na >= i
        counts = np.bincount(tok[sel, i], minlength=V)
        assert counts[p[i] == 0].sum() == 0
        if sel.sum() < 2000:  # too few requests reach this position for the test
            continue
        live = p[i] > 0
        assert live.sum() >= 10
        pv = stats.chisquare(counts[live], p[i][live] * counts[live].sum()).pvalue
        assert pv > 1e-3, (cut, i, pv)


def test_top_p_extreme_temperatures_masks_and_errors():
    """Top-p at temperatures that push masses to underflow or make them all
    alike, on masked rows, beside greedy requests and requests in error."""
    announce("top-p extremes")
    for dtype in (torch.bfloat16, torch.float32):
        wl = _custom(12, 3, 3000, dtype=dtype, dense=False, masked=True, density=0.05, seed=41,
                     top_k=(0, 0, 7))
        wl["temperature"] = torch.tensor([1e-3, 0.01, 1.0, 30.0, 1e4, 0.0, 0.7, 1e-3, 5.0, 0.0, 2.0, -1.0],
                                         device=DEV)
        wl["top_p"] = torch.tensor([0.9, 0.5, 0.3, 0.9, 0.99, 0.9, 1e-7, 0.999, 0.6, 0.0, 0.95, 0.9],
                                   device=DEV)
        gpu, orc = run_gpu(wl), run_oracle(wl)
        assert_parity(gpu, orc)
        assert gpu["status"] & oracle.verify.ST_TEMPERATURE


@pytest.mark.parametrize("V", [40960, 270336])
@pytest.mark.parametrize("masked", [False, True])
def test_two_pass_selection_on_raw_codes(masked, V):
    """bf16 rows, 16-byte aligned, of a call with top-k 50 and top-p.  At
    V=40960 the single-pass selection takes both cuts from the line maxima
    and the staged candidates; at V=270336 (more lines than it holds) the
    two-pass selection counts the rows on raw 16-bit codes and takes element
    by element the batches with an allowed NaN or +inf and the windows that
    start at the bottom of the code range.  Rows with -inf among the values,
    an allowed NaN of either sign or +inf (reported), a NaN at a forbidden
    token, the threshold among the most negative finite values, no allowed
    finite value, and exactly K allowed finite values."""
    announce(f"top-k and top-p selection on bf16 rows masked={masked} V={V}")
    B, k = 8, 2
    wl = _custom(B, k, V, dense=False, seed=131 + masked)
    g = torch.Generator(device=DEV)
    g.manual_seed(132 + masked)
    lg = wl["logits"].float()
    if masked:
        allowed = torch.rand((B, k + 1, V), generator=g, device=DEV) < 0.5
    else:
        allowed = torch.ones((B, k + 1, V), dtype=torch.bool, device=DEV)
    lg[0, :, ::97] = float("-inf")
    lg[1, 0, 30001] = float("nan")
    allowed[1, 0, 30001] = True
    lg[1, 1, 777] = float("nan")                      # forbidden when masked, else reported
    allowed[1, 1, 777] = not masked
    lg[2, 2, 12345] = float("inf")
    allowed[2, 2, 12345] = True
    lg[3] = -2.0e38 * (1.0 + 0.5 * torch.rand((k + 1, V), generator=g, device=DEV))
    lg[4] = float("-inf")
    lg[5] = float("-inf")
    for i in range(k + 1):
        idx = torch.randperm(V, generator=g, device=DEV)[:50]
        lg[5, i, idx] = torch.randn(50, generator=g, device=DEV) * 3.0
        allowed[5, i, idx] = True
    lgb = lg.to(torch.bfloat16).contiguous()
    lgb.view(torch.int16)[6, 0, 5000] = -64           # 0xffc0: a NaN with the sign bit set
    allowed[6, 0, 5000] = True
    wl["logits"] = lgb
    wl["bitmask"] = pack_bitmask(allowed) if masked else None
    wl["temperature"][3] = 1e34                       # l / T of row 3 within the fp32 exponent range
    wl["top_k"] = torch.full((B,), 50, dtype=torch.int32, device=DEV)
    wl["top_p"] = torch.tensor([0.9, 0.9, 0.9, 0.9, 0.9, 0.95, 0.5, 0.99], device=DEV)
    gpu, orc = run_gpu(wl), run_oracle(wl)
    assert orc["request_status"][1] and orc["request_status"][2] and orc["request_status"][6]
    assert_parity(gpu, orc)


@pytest.mark.parametrize("V", [8192, 8190])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nan_alone_in_a_block(dtype, V):
    """A NaN that is the only allowed token of its 2048-token block (the
    block's other tokens masked or -inf), on sampling and greedy rows, with
    and without top-k, on aligned rows and on rows of element loads: the
    request is reported."""
    announce(f"NaN alone in a block dtype={dtype} V={V}")
    B, k = 8, 2
    wl = _custom(B, k, V, dtype=dtype, dense=False, seed=141)
    lg = wl["logits"].float()
    allowed = torch.ones((B, k + 1, V), dtype=torch.bool, device=DEV)
    allowed[0:2, 1, 2048:4096] = False                # block 1 of row 1 forbidden but for one token
    allowed[0:2, 1, 3000] = True
    lg[0:2, 1, 3000] = float("nan")
    lg[2:4, 0, 4096:6144] = float("-inf")              # block 2 of row 0 all -inf but one NaN
    lg[2:4, 0, 5000] = float("nan")
    lg[4:6, 2, 2048:4096] = float("-inf")              # the same on the last row
    lg[4:6, 2, 2049] = float("nan")
    wl["logits"] = lg.to(dtype).contiguous()
    wl["bitmask"] = pack_bitmask(allowed)
    wl["temperature"][1::2] = 0.0                     # odd requests greedy
    wl["top_k"] = torch.tensor([0, 0, 0, 0, 50, 50, 0, 50], dtype=torch.int32, device=DEV)
    gpu, orc = run_gpu(wl), run_oracle(wl)
    assert all(int(orc["request_status"][b]) != 0 for b in range(6))
    assert_parity(gpu, orc)


def test_long_k_with_top_p_scaled():
    announce("long_k B=8 with top-k 50 and top-p 0.9")
    wl = make_workload("long_k", device=DEV, batch=8)
    wl["top_p"] = torch.full((8,), 0.9, device=DEV)
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_long_k_top_p_full_every_request():
    """The full long_k call with top-p 0.9 on every request (the cut read off
    the single pass's token window, the residual from the listed lines),
    every request against the oracle."""
    announce("long_k full B=512 k=12 V=151936 top-k 50 top-p 0.9, every request against the oracle")
    wl = make_workload("long_k", device=DEV)
    wl["top_p"] = torch.full((512,), 0.9, device=DEV)
    gpu = run_gpu(wl)
    orc = run_oracle_parallel(wl)
    assert_parity(gpu, orc)
    assert int(gpu["counters"][3]) == int(orc["counters"][3]) and gpu["status"] == 0


# ------------------------------------------------------- shapes and variants

@pytest.mark.parametrize("V", [1, 7, 8, 1001, 2047, 2048, 2049, 6144, 6150])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_vocab_sizes_and_alignment(V, dtype):
    announce(f"custom V={V} dtype={dtype}")
    for dense, masked in [(True, False), (False, True)]:
        wl = _custom(6, 3, V, dtype=dtype, dense=dense, masked=masked, greedy_frac=0.3,
                     seed=V + (7 if dense else 0))
        assert_parity(run_gpu(wl), run_oracle(wl))


@pytest.mark.parametrize("V", [65536, 70001])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dense_long_rows(V, dtype):
    """Rows of 32 blocks or more: the residual masses come from the grid-wide
    kernels (vector path at V = 65536, element path at V = 70001)."""
    announce(f"dense long rows V={V} dtype={dtype}")
    wl = _custom(12, 3, V, dtype=dtype, dense=True, masked=True, greedy_frac=0.2, density=0.5,
                 seed=V % 97, top_k=(0, 0, 20))
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_dense_rows_past_256_blocks():
    """Dense q on rows of 293 blocks (V = 600000): the residual draw's level-1
    race takes its first four rounds of 64 block masses from the loads issued
    with the job and reads the fifth from memory as it goes."""
    announce("dense rows V=600000 (293 blocks)")
    wl = _custom(4, 2, 600000, dense=True, masked=True, density=0.5, seed=11)
    gpu = run_gpu(wl)
    assert_parity(gpu, run_oracle(wl))
    assert (gpu["out_num_accepted"] < 2).any()  # some token comes from the residual


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_masked_dense_one_hot_and_greedy_mix(dtype):
    """Rows of 20 blocks: the dense residual is summed inside the finalize
    kernel, each wave taking two rounds of blocks."""
    announce(f"custom B=24 k=6 V=40000 masked dense greedy mix dtype={dtype}")
    wl = _custom(24, 6, 40000, dtype=dtype, dense=True, masked=True, greedy_frac=0.4, density=0.1, seed=3)
    assert_parity(run_gpu(wl), run_oracle(wl))
    wl["draft_probs"] = None
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_greedy_ties():
    announce("integer logits, greedy, many ties")
    wl = _custom(32, 4, 5000, dense=False, greedy_frac=1.0, integer_logits=True, seed=9,
                 x_argmax_frac=0.8)
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_k_zero_bonus_only():
    announce("k=0")
    wl = _custom(10, 0, 3000, dense=False, greedy_frac=0.3, seed=4)
    wl["draft_token_ids"] = torch.zeros((10, 0), dtype=torch.int32, device=DEV)
    assert_parity(run_gpu(wl), run_oracle(wl))


def test_empty_batch():
    announce("B=0")
    import rejection_sampling_verification_amd as sdv
    v = sdv.Verifier(0, 3, 100, torch.float32, DEV)
    r = v(torch.zeros((0, 4, 100), device=DEV), torch.zeros((0, 3), dtype=torch.int32, device=DEV),
          temperature=torch.zeros(0, device=DEV))
    torch.cuda.synchronize()
    assert r.out_counters.cpu().tolist() == [0, 0, 0, 0] and int(r.status.item()) == 0


def test_malformed_requests():
    announce("status bits")
    wl = _custom(8, 3, 3000, dense=True, masked=True, seed=5)
    wl["draft_token_ids"][1, 2] = 3000                        # draft id out of range
    wl["temperature"][2] = -1.0                               # bad temperature
    wl["logits"][3, 1, 17] = float("nan")                     # NaN at ...
    wl["bitmask"][3, 1, 0] |= (1 << 17)                       # ... an allowed token
    wl["bitmask"][4, 2, :] = 0                                # empty row
    wl["draft_probs"][5, 0, wl["draft_token_ids"][5, 0]] = float("inf")
    gpu, orc = run_gpu(wl), run_oracle(wl)
    assert list(orc["request_status"][:6]) == [0, 1, 2, 8, 4, 16]
    assert_parity(gpu, orc)
    assert gpu["status"] == 1 | 2 | 4 | 8 | 16


@pytest.mark.parametrize("dense", [False, True])
def test_status_bits_past_the_first_rows(dense):
    """k = 64: errors in rows folded after the first wave of rows, in the
    bonus row (row 64, past the 64 lanes of the status scan) and at the last
    draft position, one-hot and dense."""
    announce(f"status bits k=64 dense={dense}")
    wl = _custom(6, 64, 2500, dense=dense, masked=True, seed=21)
    wl["logits"][0, 64, 17] = float("nan")                    # NaN at an allowed token
    wl["bitmask"][0, 64, 0] |= (1 << 17)                      # ... of the bonus row
    wl["bitmask"][1, 40, :] = 0                               # empty row 40
    wl["draft_token_ids"][2, 63] = 2500                       # last draft out of range
    wl["temperature"][3] = 0.0                                # greedy, with a draft
    wl["draft_token_ids"][3, 9] = -1                          # ... out of range at row 9
    if dense:
        wl["draft_probs"][4, 50, wl["draft_token_ids"][4, 50]] = float("inf")
    gpu, orc = run_gpu(wl), run_oracle(wl)
    want = [8, 4, 1, 1, 16 if dense else 0, 0]
    assert list(orc["request_status"]) == want
    assert_parity(gpu, orc)
    assert gpu["status"] == (1 | 4 | 8 | (16 if dense else 0))


def test_largest_batch_counters():
    """SD_MAX_BATCH requests: every workgroup's share reaches the counters,
    with requests in error among them."""
    announce("custom B=65535 k=2 V=2 masked, errors")
    wl = _custom(65535, 2, 2, dense=False, masked=True, greedy_frac=0.5, density=0.5, seed=11)
    wl["draft_token_ids"][100, 0] = 2
    wl["draft_token_ids"][65534, 1] = 7
    wl["temperature"][4000] = float("nan")
    gpu, orc = run_gpu(wl), run_oracle(wl)
    assert int((orc["request_status"] != 0).sum()) == 3
    assert_parity(gpu, orc)


def test_determinism_and_seed():
    announce("determinism")
    wl = make_workload("draft_model", device=DEV, batch=64)
    a, b = run_gpu(wl), run_gpu(wl)
    for key in ("out_tokens", "out_num_accepted", "out_counters", "row_lse", "accept_prob"):
        assert np.array_equal(a[key], b[key]), key
    c = run_gpu(wl, seed=wl["seed"] + 1)
    assert not np.array_equal(a["out_tokens"], c["out_tokens"])


def test_counter_example_on_gpu():
    """fanout, "Work a denominator example": R=1000, I=200, D=800, A=600."""
    announce("counter example")
    B, k, V = 200, 5, 64
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    lg = torch.randn((B, k + 1, V), generator=g)
    gm = torch.randint(0, V, (B, k + 1), generator=g)
    lg.scatter_(2, gm[..., None], 20.0)
    x = gm[:, :k].clone()
    allowed = torch.ones((B, k + 1, V), dtype=torch.bool)
    for b in range(120, 200):
        x[b] = (gm[b, :k] + 1) % V
        if b < 160:
            allowed[b, torch.arange(k), x[b]] = False
    wl = {"logits": lg.to(DEV), "draft_token_ids": x.to(torch.int32).to(DEV), "draft_probs": None,
          "bitmask": pack_bitmask(allowed).to(DEV), "temperature": torch.zeros(B, device=DEV),
          "top_k": None, "seed": 1}
    gpu = run_gpu(wl)
    assert [int(v) for v in gpu["counters"]] == [1000, 200, 800, 600]


@pytest.mark.parametrize("mode", ["dense", "one_hot", "masked", "top_k", "top_p"])
def test_chi_square_on_gpu(mode):
    """Emitted tokens follow the target law (pyshine, "Verification": the output
    is statistically indistinguishable from undrafted decoding)."""
    from scipy import stats
    from oracle import verify as ov
    announce(f"chi-square {mode}")
    B, k, V = 50000, 2, 8    # four calls with different seeds: 200000 samples
    g = torch.Generator(device="cpu")
    g.manual_seed(11)
    l1 = torch.randn((k + 1, V), generator=g)
    allowed = torch.ones((k + 1, V), dtype=torch.bool)
    if mode == "masked":
        allowed = torch.rand((k + 1, V), generator=g) < 0.7
        allowed[:, :2] = True
    T = 0.9
    top_k = 4 if mode == "top_k" else 0
    top_p = 0.6 if mode == "top_p" else 0.0
    p = np.array([ov.target_distribution(l1[i].double().numpy(), allowed[i].numpy(), T, top_k, top_p)[0]
                  for i in range(k + 1)])
    q1 = torch.softmax(torch.randn((k, V), generator=g), -1)
    x = torch.stack([torch.multinomial(q1[i], B, replacement=True, generator=g) for i in range(k)], 1)
    wl = {"logits": l1.expand(B, k + 1, V).contiguous().to(DEV),
          "draft_token_ids": x.to(torch.int32).to(DEV),
          "draft_probs": None if mode == "one_hot" else q1.expand(B, k, V).contiguous().to(DEV),
          "bitmask": None if mode != "masked" else pack_bitmask(allowed).expand(B, k + 1, 1).contiguous().to(DEV),
          "temperature": torch.full((B,), T, device=DEV),
          "top_k": torch.full((B,), top_k, dtype=torch.int32, device=DEV) if top_k else None,
          "top_p": torch.full((B,), top_p, device=DEV) if top_p else None,
          "seed": 2024}
    runs = [run_gpu(wl, seed=2024 + r) for r in range(4)]
    tok = np.concatenate([g["out_tokens"] for g in runs])
    na = np.concatenate([g["out_num_accepted"] for g in runs])
    for i in range(k + 1):
        sel = na >= i
        counts = np.bincount(tok[sel, i], minlength=V)
        assert counts[p[i] == 0].sum() == 0
        live = p[i] > 0
        pv = stats.chisquare(counts[live], p[i][live] * counts[live].sum()).pvalue
        assert pv > 1e-3, (mode, i, pv)
