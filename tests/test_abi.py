"""The C ABI library loads, exports every symbol include/*.h declares, and its
host-only logic behaves (no GPU compute here)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", name) for name in sorted(os.listdir(os.path.join(ROOT, "include")))
           if name.endswith(".h")]


def _declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names |= set(re.findall(r"\b(sd_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_expected_entry_points():
    assert [os.path.basename(h) for h in HEADERS] == ["sd_ngram.h", "sd_verify.h"]
    assert _declared_functions() == sorted(
        ["sd_verify", "sd_verify_workspace_size", "sd_status_string", "sd_rates",
         "sd_verify_noalloc", "sd_ngram_propose", "sd_ngram_workspace_size"])


def test_library_exports_every_declared_symbol():
    import rejection_sampling_verification_amd as sdv
    lib = sdv.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert sorted(sdv.EXPORTED_SYMBOLS) == _declared_functions()


def test_params_struct_layout_matches_header():
    import rejection_sampling_verification_amd as sdv
    # 3 x int32 + enum, then 7 pointers (the last the debug-only timing
    # hooks), offsets, total_drafts, histogram, top_p
    assert ctypes.sizeof(sdv.SdParams) == 16 + 11 * 8
    assert sdv.SdParams.top_p.offset == 16 + 10 * 8
    assert sdv.SdParams.top_k.offset == 16
    assert sdv.SdParams.debug_timing.offset == 16 + 6 * 8
    assert sdv.SdParams.draft_offsets.offset == 16 + 7 * 8
    assert sdv.SdParams.total_drafts.offset == 16 + 8 * 8
    assert sdv.SdParams.accept_histogram.offset == 16 + 9 * 8
    assert ctypes.sizeof(sdv.SdDebugTiming) == 16


def test_status_strings():
    import rejection_sampling_verification_amd as sdv
    assert sdv.sd_status_string(0) == "ok"
    assert "workspace" in sdv.sd_status_string(-3)
    assert sdv.sd_status_string(12345) == "unknown status"


def test_rates_match_the_pages_example():
    """fanout, "Work a denominator example" and "Mean acceptance length"."""
    import rejection_sampling_verification_amd as sdv
    s, a, y, m = sdv.sd_rates([1000, 200, 800, 600], 100)
    assert (s, a, y) == pytest.approx((0.8, 0.75, 0.6), abs=1e-15)
    assert sdv.sd_rates([1000, 0, 1000, 600], 1)[1] == pytest.approx(0.6)
    assert sdv.sd_rates([1000, 0, 1000, 750], 1)[1] == pytest.approx(0.75)
    assert sdv.sd_rates([300, 0, 300, 180], 100)[3] == pytest.approx(2.8)
    r = sdv.sd_rates([0, 0, 0, 0], 0)
    assert all(math.isnan(v) for v in r)
    with pytest.raises(ValueError):
        sdv.sd_rates([10, 2, 9, 1], 1)      # D != R - I
    with pytest.raises(ValueError):
        sdv.sd_rates([10, 2, 8, 9], 1)      # A > D


def test_rates_agree_with_oracle():
    import numpy as np

    import oracle
    import rejection_sampling_verification_amd as sdv
    rng = np.random.default_rng(0)
    for _ in range(100):
        R = int(rng.integers(1, 10**6))
        I = int(rng.integers(0, R + 1))
        A = int(rng.integers(0, R - I + 1))
        steps = int(rng.integers(1, 10**5))
        o = oracle.sd_rates(R, I, A, steps)
        g = sdv.sd_rates([R, I, R - I, A], steps)
        want = [o["survival"], o["acceptance"] if R - I else float("nan"), o["yield"],
                o["mean_acceptance_length"]]
        for gv, wv in zip(g, want):
            assert (math.isnan(gv) and math.isnan(wv)) or gv == pytest.approx(wv, rel=1e-15)


def test_workspace_size():
    import rejection_sampling_verification_amd as sdv
    assert sdv.sd_verify_workspace_size(0, 4, 100) == 0
    assert sdv.sd_verify_workspace_size(4, -1, 100) == 0
    assert sdv.sd_verify_workspace_size(4, 65, 100) == 0
    assert sdv.sd_verify_workspace_size(4, 4, 0) == 0
    # rows * blocks * 8 bytes of block statistics and 4 bytes per row
    ws = sdv.sd_verify_workspace_size(256, 4, 151936)
    rows, C = 256 * 5, -(-151936 // 2048)
    assert ws >= rows * C * 8 + rows * 4 and ws % 256 == 0


def test_workspace_size_with_top_k():
    """A top-k array adds the line maxima (2 bytes per 64 bf16 tokens of every
    row) and each row's list of kept lines (128 two-byte entries and a count);
    the long-draft shape with top-k still fits the allocation-free scratch."""
    import rejection_sampling_verification_amd as sdv
    B, k, V = 512, 12, 151936
    rows, C = B * (k + 1), -(-V // 2048)
    plain = sdv.sd_verify_workspace_size(B, k, V)
    with_k = sdv.sd_verify_workspace_size(B, k, V, top_k=True)
    assert with_k - plain >= rows * C * 32 * 2 + rows * (128 * 2 + 4)
    assert with_k % 256 == 0 and with_k <= 64 << 20


def test_host_argument_checks_return_before_any_launch():
    import rejection_sampling_verification_amd as sdv
    lib = sdv.library()
    p = sdv.SdParams()
    p.batch, p.num_draft, p.vocab, p.logits_dtype = 4, 3, 100, 1
    nul = ctypes.c_void_p(0)
    counters = (ctypes.c_uint64 * 4)()
    # missing params / counters
    assert lib.sd_verify(nul, nul, nul, nul, nul, 0, nul, nul, counters, None, nul, 0, nul) == -1
    assert lib.sd_verify(nul, nul, nul, nul, nul, 0, nul, nul, nul, ctypes.byref(p), nul, 0, nul) == -1
    # bad dtype, bad sizes, unsupported sizes
    p.logits_dtype = 7
    assert lib.sd_verify(nul, nul, nul, nul, nul, 0, nul, nul, counters, ctypes.byref(p), nul, 0, nul) == -1
    p.logits_dtype, p.num_draft = 1, 65
    assert lib.sd_verify(nul, nul, nul, nul, nul, 0, nul, nul, counters, ctypes.byref(p), nul, 0, nul) == -2
    p.num_draft, p.vocab = 3, (1 << 22) + 1
    assert lib.sd_verify(nul, nul, nul, nul, nul, 0, nul, nul, counters, ctypes.byref(p), nul, 0, nul) == -2
    p.vocab, p.batch = 100, 65536
    assert lib.sd_verify(nul, nul, nul, nul, nul, 0, nul, nul, counters, ctypes.byref(p), nul, 0, nul) == -2
    p.batch = 4
    # missing required tensors
    p.vocab = 100
    assert lib.sd_verify(nul, nul, nul, nul, nul, 0, nul, nul, counters, ctypes.byref(p), nul, 0, nul) == -1
    # workspace too small (all tensors given as fake non-null device addresses)
    fake = ctypes.c_void_p(1 << 20)
    assert lib.sd_verify(fake, fake, nul, nul, fake, 0, fake, fake, counters, ctypes.byref(p),
                         fake, 16, nul) == -3


def test_package_refuses_to_import_without_the_library(tmp_path, monkeypatch):
    import importlib.util
    import shutil
    pkg_src = os.path.join(ROOT, "rejection_sampling_verification_amd", "__init__.py")
    dst = tmp_path / "sdv_copy"
    dst.mkdir()
    shutil.copy(pkg_src, dst / "__init__.py")
    spec = importlib.util.spec_from_file_location("sdv_copy", dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="missing"):
        spec.loader.exec_module(mod)


def test_ragged_host_checks_and_workspace():
    import rejection_sampling_verification_amd as sdv
    lib = sdv.library()
    nul = ctypes.c_void_p(0)
    counters = (ctypes.c_uint64 * 4)()
    p = sdv.SdParams()
    p.batch, p.num_draft, p.vocab, p.logits_dtype = 4, 3, 100, 1
    p.draft_offsets = 1 << 20                      # a fake device address; never read here
    for total in (-1, 13):                         # below 0, above B * num_draft
        p.total_drafts = total
        assert lib.sd_verify(nul, nul, nul, nul, nul, 0, nul, nul, counters, ctypes.byref(p), nul, 0, nul) == -1
    assert sdv.sd_verify_workspace_size(4, 3, 100, total_drafts=13) == 0
    ws_r = sdv.sd_verify_workspace_size(4, 3, 100, total_drafts=5)
    ws_u = sdv.sd_verify_workspace_size(4, 3, 100)
    assert ws_r > 0 and ws_u > 0 and ws_r < ws_u + 4096


def test_ngram_params_layout_and_host_checks():
    import rejection_sampling_verification_amd as sdv
    # 4 x int32, stride and max_model_len, then 4 output pointers and the
    # debug-only timing hooks
    assert ctypes.sizeof(sdv.SdNgramParams) == 16 + 2 * 8 + 5 * 8
    assert sdv.SdNgramParams.stride.offset == 16
    assert sdv.SdNgramParams.out_match_len.offset == 32
    assert sdv.SdNgramParams.status.offset == 56
    lib = sdv.library()
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)

    def call(p, ws=nul, nbytes=0):
        return lib.sd_ngram_propose(fake, fake, fake, fake, ctypes.byref(p), ws, nbytes, nul)

    good = dict(batch=4, min_n=2, max_n=5, num_draft=4, stride=5000, max_model_len=0)
    for key, bad, code in [("min_n", 0, -1), ("max_n", 1, -1), ("num_draft", -1, -1), ("stride", 0, -1),
                           ("batch", -1, -1), ("max_model_len", -1, -1), ("max_n", 257, -2),
                           ("num_draft", 65, -2), ("batch", 65536, -2), ("stride", 1 << 31, -2)]:
        kw = dict(good, **{key: bad})
        p = sdv._ngram_params(kw["batch"], kw["min_n"], kw["max_n"], kw["num_draft"], kw["stride"],
                              kw["max_model_len"])
        assert call(p) == code, (key, bad)
        assert sdv.sd_ngram_workspace_size(kw["batch"], kw["stride"], kw["min_n"], kw["max_n"],
                                           kw["num_draft"], kw["max_model_len"]) == 0
    p = sdv._ngram_params(**{"batch": 4, "min_n": 2, "max_n": 5, "num_draft": 4, "stride": 5000,
                             "max_model_len": 0})
    assert lib.sd_ngram_propose(nul, fake, fake, fake, ctypes.byref(p), nul, 0, nul) == -1
    assert lib.sd_ngram_propose(fake, fake, fake, fake, None, nul, 0, nul) == -1
    p.out_drafts_flat = 1 << 20                    # flat drafts need the offsets
    assert call(p) == -1
    p.out_drafts_flat = None
    assert call(p) == -3                           # no workspace
    ws = sdv.sd_ngram_workspace_size(4, 5000, 2, 5, 4)
    assert ws >= 4 * 3 * 8 and ws % 256 == 0       # one 8-byte key per (request, 2048 positions)
    assert call(p, fake, ws - 1) == -3
    assert sdv.sd_ngram_workspace_size(0, 5000, 2, 5, 4) == 0


def test_noalloc_refuses_before_launching():
    """sd_verify_noalloc: a null parameter block, and sizes whose workspace
    exceeds the static scratch, are refused on the host (no HIP call)."""
    import rejection_sampling_verification_amd as sdv
    lib = sdv.library()
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    assert lib.sd_verify_noalloc(fake, fake, nul, nul, fake, 0, fake, fake, fake, None, nul) == -1
    p = sdv.SdParams()
    p.batch, p.num_draft, p.vocab, p.logits_dtype = 8192, 12, 151936, 1   # about 128 MB of workspace
    assert lib.sd_verify_workspace_size(ctypes.byref(p)) > sdv.SD_NOALLOC_SCRATCH_BYTES
    assert lib.sd_verify_noalloc(fake, fake, nul, nul, fake, 0, fake, fake, fake, ctypes.byref(p), nul) == -5
    assert "scratch" in sdv.sd_status_string(-5)
