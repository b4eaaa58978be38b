"""The verifier called from C++ through its C ABI alone: tests/c_abi_check
(built with the package) reads a workload from raw files, calls sd_verify on
the GPU and writes the outputs, which must match the oracle like every other
parity case; the host-side refusals are checked too."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, to_numpy

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(BIN):
        pytest.fail("tests/c_abi_check is missing: build the package first")


def _run(tmp_path, logits, drafts, probs, temperature, seed):
    B, kp1, V = logits.shape
    (tmp_path / "meta.txt").write_text(f"{B} {kp1 - 1} {V} {seed} {0 if probs is None else 1}\n")
    np.ascontiguousarray(logits, dtype=np.float32).tofile(tmp_path / "logits.f32")
    np.ascontiguousarray(drafts, dtype=np.int32).tofile(tmp_path / "drafts.i32")
    np.ascontiguousarray(temperature, dtype=np.float32).tofile(tmp_path / "temperature.f32")
    if probs is not None:
        np.ascontiguousarray(probs, dtype=np.float32).tofile(tmp_path / "probs.f32")
    print(f"[gpu-case] c_abi_check B={B} k={kp1 - 1} V={V}", flush=True)
    res = subprocess.run([BIN, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    out = {
        "tokens": np.fromfile(tmp_path / "out_tokens.i32", dtype=np.int32).reshape(B, kp1),
        "nacc": np.fromfile(tmp_path / "num_accepted.i32", dtype=np.int32),
        "counters": np.fromfile(tmp_path / "counters.u64", dtype=np.uint64),
        "status": int(np.fromfile(tmp_path / "status.u32", dtype=np.uint32)[0]),
        "refused": [int(v) for v in (tmp_path / "host_checks.txt").read_text().split()],
    }
    orc = oracle.sd_verify(logits.astype(np.float64), drafts, probs, None, temperature, seed=seed)
    return out, orc


def _check(out, orc):
    assert out["refused"] == [-1, -2, -3, -1]   # bad batch, k too large, small workspace, no logits
    flagged = (orc["flag_accept"] + orc["flag_gumbel"]) > 0
    same = (out["nacc"] == orc["num_accepted"]) & np.all(out["tokens"] == orc["out_tokens"], axis=1)
    assert np.all(same | flagged), np.flatnonzero(~(same | flagged))
    assert flagged.sum() <= 1
    if not flagged.any():
        assert [int(v) for v in out["counters"]] == [int(v) for v in orc["counters"]]
    assert out["status"] == orc["status"]


def test_tiny_workload_through_the_c_abi(tmp_path):
    n = to_numpy(make_workload("tiny", device="cpu"))
    _check(*_run(tmp_path, n["logits"], n["draft_token_ids"], n["draft_probs"], n["temperature"], 0))


def test_mixed_batch_through_the_c_abi(tmp_path):
    rng = np.random.default_rng(21)
    B, k, V = 24, 4, 5000
    logits = (rng.normal(size=(B, k + 1, V)) * 2.5).astype(np.float32)
    z = logits[:, :k] + rng.normal(size=(B, k, V)).astype(np.float32)
    probs = np.exp(z - z.max(-1, keepdims=True))
    probs = (probs / probs.sum(-1, keepdims=True)).astype(np.float32)
    drafts = np.array([[rng.choice(V, p=probs[b, i] / probs[b, i].sum()) for i in range(k)]
                       for b in range(B)], dtype=np.int32)
    drafts[::3, 0] = logits[::3, 0].argmax(-1)
    temperature = np.where(rng.random(B) < 0.3, 0.0, rng.uniform(0.5, 1.5, B)).astype(np.float32)
    _check(*_run(tmp_path, logits, drafts, probs, temperature, 77))
