"""sd_verify_noalloc (the entry point with a static per-device workspace)
against sd_verify on the same inputs: every output equal, over two calls in a
row on one device, the second smaller than the first, then a call of another
mode (masks, dense q, top-k) and the first shape again."""
import numpy as np
import pytest
import torch

from workloads import make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _call(wl, noalloc):
    import rejection_sampling_verification_amd as sdv
    lg = wl["logits"]
    B, kp1, V = lg.shape
    v = sdv.Verifier(B, kp1 - 1, V, lg.dtype, lg.device, debug=True, noalloc=noalloc)
    r = v(lg, wl["draft_token_ids"], wl["draft_probs"], wl["bitmask"], wl["temperature"], wl["seed"],
          wl["top_k"])
    torch.cuda.synchronize()
    return {name: getattr(r, name).cpu().numpy().copy() for name in r._fields if getattr(r, name) is not None}


def _same(a, b, what):
    for key in ("out_tokens", "out_num_accepted", "out_counters", "status", "request_flags", "flags"):
        assert np.array_equal(a[key], b[key]), f"{what}: {key} differs"
    # the same kernels on the same inputs: the probabilities agree exactly
    for key in ("row_lse", "accept_prob"):
        assert np.array_equal(a[key], b[key], equal_nan=True), f"{what}: {key} differs"


def test_noalloc_matches_sd_verify():
    cases = [("ngram", 64), ("ngram", 16), ("structured", 6), ("long_k", 4), ("ngram", 64)]
    for name, batch in cases:
        print(f"[gpu-case] noalloc: {name} B={batch}", flush=True)
        wl = make_workload(name, device=DEV, batch=batch)
        _same(_call(wl, noalloc=True), _call(wl, noalloc=False), f"{name} B={batch}")
