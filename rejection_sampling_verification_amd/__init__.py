"""Python binding of the MI355X speculative-decoding verifier (libsdverify.so).

Argument marshalling only: every step of verification and of the n-gram draft
proposer runs in the HIP kernels behind the C ABI declared in
include/sd_verify.h and include/sd_ngram.h.  PyTorch supplies device
memory and the current stream.  Importing this package fails loudly when the
library has not been built (python rejection_sampling_verification_amd/build.py).

Entry points mirror the C ABI names: ``sd_verify``, ``sd_verify_workspace_size``,
``sd_status_string``, ``sd_rates``, ``sd_verify_noalloc`` (through
``Verifier(..., noalloc=True)``), ``sd_ngram_propose``,
``sd_ngram_workspace_size``; ``Verifier`` and ``NgramProposer`` keep the
workspace and outputs of repeated same-shape calls.
"""
import ctypes
import math
import os
from typing import NamedTuple, Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG_DIR, "libsdverify.so")

SD_OK = 0
SD_DTYPE_F32 = 0
SD_DTYPE_BF16 = 1
SD_MAX_BATCH = 65535
SD_MAX_DRAFT = 64
SD_MAX_VOCAB = 1 << 22
SD_BLOCK_TOKENS = 2048

SD_STATUS_DRAFT_ID = 1
SD_STATUS_TEMPERATURE = 2
SD_STATUS_EMPTY_ROW = 4
SD_STATUS_BAD_LOGIT = 8
SD_STATUS_BAD_DRAFT_PROB = 16
SD_STATUS_BAD_OFFSETS = 32

SD_NGRAM_MAX_N = 256
SD_NGRAM_MAX_BATCH = 65535
SD_NGRAM_STATUS_BAD_LENGTH = 1

# every symbol include/sd_verify.h and include/sd_ngram.h declare
EXPORTED_SYMBOLS = ("sd_verify", "sd_verify_workspace_size", "sd_status_string", "sd_rates",
                    "sd_verify_noalloc", "sd_ngram_propose", "sd_ngram_workspace_size")
SD_NOALLOC_SCRATCH_BYTES = 64 << 20


class SdDebugTiming(ctypes.Structure):
    """Debug-only timing hooks: hipEvent_t handles recorded around a call's
    main kernel (benchmarks only)."""
    _fields_ = [("kernel_begin", ctypes.c_void_p), ("kernel_end", ctypes.c_void_p)]


class SdParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_draft", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("logits_dtype", ctypes.c_int),
        ("top_k", ctypes.c_void_p),
        ("dbg_row_lse", ctypes.c_void_p),
        ("dbg_accept_prob", ctypes.c_void_p),
        ("dbg_request_flags", ctypes.c_void_p),
        ("dbg_flags", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("debug_timing", ctypes.POINTER(SdDebugTiming)),
        ("draft_offsets", ctypes.c_void_p),
        ("total_drafts", ctypes.c_int64),
        ("accept_histogram", ctypes.c_void_p),
        ("top_p", ctypes.c_void_p),
    ]


class SdNgramParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("min_n", ctypes.c_int32),
        ("max_n", ctypes.c_int32),
        ("num_draft", ctypes.c_int32),
        ("stride", ctypes.c_int64),
        ("max_model_len", ctypes.c_int64),
        ("out_match_len", ctypes.c_void_p),
        ("out_draft_offsets", ctypes.c_void_p),
        ("out_drafts_flat", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("debug_timing", ctypes.POINTER(SdDebugTiming)),
    ]


def _load():
    if not os.path.exists(LIBRARY_PATH):
        raise ImportError(
            f"{LIBRARY_PATH} is missing: build it with "
            "`python rejection_sampling_verification_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIBRARY_PATH)
    lib.sd_verify_workspace_size.argtypes = [ctypes.POINTER(SdParams)]
    lib.sd_verify_workspace_size.restype = ctypes.c_size_t
    lib.sd_verify.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(SdParams), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
    ]
    lib.sd_verify.restype = ctypes.c_int
    lib.sd_verify_noalloc.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(SdParams), ctypes.c_void_p,
    ]
    lib.sd_verify_noalloc.restype = ctypes.c_int
    lib.sd_status_string.argtypes = [ctypes.c_int]
    lib.sd_status_string.restype = ctypes.c_char_p
    lib.sd_rates.argtypes = [ctypes.POINTER(ctypes.c_uint64), ctypes.c_uint64,
                             ctypes.POINTER(ctypes.c_double)]
    lib.sd_rates.restype = ctypes.c_int
    lib.sd_ngram_workspace_size.argtypes = [ctypes.POINTER(SdNgramParams)]
    lib.sd_ngram_workspace_size.restype = ctypes.c_size_t
    lib.sd_ngram_propose.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(SdNgramParams), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
    ]
    lib.sd_ngram_propose.restype = ctypes.c_int
    return lib


_lib = _load()


def library():
    """The loaded ctypes handle of libsdverify.so."""
    return _lib


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return SD_DTYPE_BF16
    if dt == torch.float32:
        return SD_DTYPE_F32
    raise ValueError(f"target_logits must be bfloat16 or float32, got {dt}")


def _params(batch, num_draft, vocab, dtype_code):
    p = SdParams()
    p.batch, p.num_draft, p.vocab, p.logits_dtype = int(batch), int(num_draft), int(vocab), int(dtype_code)
    return p


def sd_verify_workspace_size(batch, num_draft, vocab, logits_dtype=torch.bfloat16,
                             total_drafts=None, top_k=False):
    """Device workspace bytes for these sizes (total_drafts: a ragged call;
    top_k: calls that pass a top-k array, which need a larger workspace)."""
    p = _params(batch, num_draft, vocab, _dtype_code(logits_dtype))
    if total_drafts is not None:
        p.draft_offsets = 1  # any non-null value: the size only depends on the mode
        p.total_drafts = int(total_drafts)
    if top_k:
        p.top_k = 1
    return int(_lib.sd_verify_workspace_size(ctypes.byref(p)))


def sd_status_string(code):
    return _lib.sd_status_string(int(code)).decode()


def sd_rates(counters, steps):
    """(survival D/R, acceptance A/D, yield A/R, mean acceptance length) from
    R, I, D, A counters; NaN where a denominator is zero."""
    c = (ctypes.c_uint64 * 4)(*[int(v) for v in counters])
    out = (ctypes.c_double * 4)()
    rc = _lib.sd_rates(c, ctypes.c_uint64(int(steps)), out)
    if rc != SD_OK:
        raise ValueError(f"sd_rates: {sd_status_string(rc)}")
    return tuple(out)


class VerifyResult(NamedTuple):
    out_tokens: torch.Tensor          # [B, k+1] int32
    out_num_accepted: torch.Tensor    # [B] int32
    out_counters: torch.Tensor        # [4] int64 holding the uint64 R, I, D, A
    status: torch.Tensor              # [1] int32 holding the uint32 status bits
    row_lse: Optional[torch.Tensor] = None         # [B, k+1] float64
    accept_prob: Optional[torch.Tensor] = None     # [B, k] float64
    request_flags: Optional[torch.Tensor] = None   # [B] int32 (uint32 bits)
    flags: Optional[torch.Tensor] = None           # [3] int32 (uint32 counts)
    accept_histogram: Optional[torch.Tensor] = None  # [k+1] int32 (uint32 counts)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Verifier:
    """Outputs and workspace for repeated calls of one shape.

    Each call overwrites the tensors it returns.  `workspace`, if given, is a
    uint8 device tensor of at least sd_verify_workspace_size bytes, zero-filled
    before its first use; verifiers of any shapes may share one, as long as
    their calls do not overlap in time.  With noalloc=True the calls go to
    sd_verify_noalloc instead: no workspace tensor exists, the library's
    static per-device scratch serves every such verifier, and their calls on
    one device must not overlap in time.
    """

    def __init__(self, batch, num_draft, vocab, logits_dtype=torch.bfloat16, device=None,
                 debug=False, histogram=False, total_drafts=None, workspace=None, noalloc=False):
        dev = torch.device(device) if device is not None else torch.device("cuda")
        if dev.type != "cuda":
            raise ValueError("the verifier runs on a HIP device")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.B, self.k, self.V = int(batch), int(num_draft), int(vocab)
        self.dtype = logits_dtype
        self.params = _params(self.B, self.k, self.V, _dtype_code(logits_dtype))
        # ragged calls: draft counts differ per request, total_drafts in all
        self.ragged = total_drafts is not None
        self.T = int(total_drafts) if self.ragged else self.B * self.k
        self.rows = self.T + self.B if self.ragged else self.B * (self.k + 1)
        if self.ragged:
            self.params.draft_offsets = 1  # placeholder until a call supplies the offsets
            self.params.total_drafts = self.T
        # calls with top-k need more (any non-null value: the size only
        # depends on whether a top-k array is given)
        ws = int(_lib.sd_verify_workspace_size(ctypes.byref(self.params)))
        self.params.top_k = 1
        self.workspace_bytes_top_k = int(_lib.sd_verify_workspace_size(ctypes.byref(self.params)))
        self.params.draft_offsets = None
        self.params.top_k = None
        dev = self.device
        self.noalloc = bool(noalloc)
        if self.noalloc:
            if workspace is not None:
                raise ValueError("noalloc verifiers take no workspace")
            if ws > SD_NOALLOC_SCRATCH_BYTES:
                raise ValueError(f"{ws} bytes of workspace exceed the static scratch "
                                 f"({SD_NOALLOC_SCRATCH_BYTES})")
            self.workspace = None
            ws = SD_NOALLOC_SCRATCH_BYTES
        elif workspace is not None:
            if (workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous()
                    or workspace.numel() < ws or workspace.data_ptr() % 256):
                raise ValueError(f"workspace must be a contiguous, 256-byte aligned uint8 tensor of "
                                 f">= {ws} bytes on {dev}")
            self.workspace = workspace
        else:
            # zero-filled once: the library leaves it ready for the next call
            ws = self.workspace_bytes_top_k
            self.workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        self.workspace_bytes = ws if workspace is None else int(workspace.numel())
        tok_shape = (self.rows,) if self.ragged else (self.B, self.k + 1)
        self.out_tokens = torch.empty(tok_shape, dtype=torch.int32, device=dev)
        self.out_num_accepted = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.out_counters = torch.empty(4, dtype=torch.int64, device=dev)
        self.status = torch.empty(1, dtype=torch.int32, device=dev)
        self.params.status = self.status.data_ptr()
        self.debug = debug
        self.accept_histogram = None
        if histogram:
            self.accept_histogram = torch.empty(self.k + 1, dtype=torch.int32, device=dev)
            self.params.accept_histogram = self.accept_histogram.data_ptr()
        if debug:
            lse_shape = (self.rows,) if self.ragged else (self.B, self.k + 1)
            acc_shape = (self.T,) if self.ragged else (self.B, self.k)
            self.row_lse = torch.empty(lse_shape, dtype=torch.float64, device=dev)
            self.accept_prob = torch.empty(acc_shape, dtype=torch.float64, device=dev)
            self.request_flags = torch.empty(self.B, dtype=torch.int32, device=dev)
            self.flags = torch.empty(3, dtype=torch.int32, device=dev)
            self.params.dbg_row_lse = self.row_lse.data_ptr()
            self.params.dbg_accept_prob = self.accept_prob.data_ptr()
            self.params.dbg_request_flags = self.request_flags.data_ptr()
            self.params.dbg_flags = self.flags.data_ptr()

    def __call__(self, target_logits, draft_token_ids, draft_probs=None, bitmask=None,
                 temperature=None, seed=0, top_k=None, stream=None, row_stats_events=None,
                 draft_offsets=None, top_p=None):
        B, k, V, dev = self.B, self.k, self.V, self.device
        W = (V + 31) // 32
        if self.ragged:
            if draft_offsets is None:
                raise ValueError("a ragged verifier needs draft_offsets ([B+1] int32)")
            _check(draft_offsets, "draft_offsets", torch.int32, (B + 1,), dev)
            _check(target_logits, "target_logits", self.dtype, (self.rows, V), dev)
            if self.T > 0 or draft_token_ids is not None:
                _check(draft_token_ids, "draft_token_ids", torch.int32, (self.T,), dev)
            _check(draft_probs, "draft_probs", torch.float32, (self.T, V), dev)
            _check(bitmask, "bitmask", torch.int32, (self.rows, W), dev)
            self.params.draft_offsets = draft_offsets.data_ptr()
        else:
            if draft_offsets is not None:
                raise ValueError("draft_offsets needs a verifier built with total_drafts")
            _check(target_logits, "target_logits", self.dtype, (B, k + 1, V), dev)
            if k > 0 or draft_token_ids is not None:
                _check(draft_token_ids, "draft_token_ids", torch.int32, (B, k), dev)
            _check(draft_probs, "draft_probs", torch.float32, (B, k, V), dev)
            _check(bitmask, "bitmask", torch.int32, (B, k + 1, W), dev)
        if temperature is None:
            raise ValueError("temperature is required ([B] float32, 0 = greedy)")
        _check(temperature, "temperature", torch.float32, (B,), dev)
        _check(top_k, "top_k", torch.int32, (B,), dev)
        if top_k is not None and self.workspace_bytes < self.workspace_bytes_top_k:
            raise ValueError(f"calls with top_k need {self.workspace_bytes_top_k} bytes of workspace, "
                             f"this verifier has {self.workspace_bytes}")
        self.params.top_k = None if top_k is None else top_k.data_ptr()
        _check(top_p, "top_p", torch.float32, (B,), dev)
        self.params.top_p = None if top_p is None else top_p.data_ptr()
        if row_stats_events is not None:
            self._timing = SdDebugTiming(*row_stats_events)
            self.params.debug_timing = ctypes.pointer(self._timing)
        else:
            self.params.debug_timing = None
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        ptrs = (_ptr(target_logits), _ptr(draft_token_ids), _ptr(draft_probs), _ptr(bitmask),
                _ptr(temperature), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                _ptr(self.out_tokens), _ptr(self.out_num_accepted), _ptr(self.out_counters),
                ctypes.byref(self.params))
        if self.noalloc:
            rc = _lib.sd_verify_noalloc(*ptrs, ctypes.c_void_p(int(stream)))
        else:
            rc = _lib.sd_verify(*ptrs, ctypes.c_void_p(self.workspace.data_ptr()),
                                ctypes.c_size_t(self.workspace_bytes), ctypes.c_void_p(int(stream)))
        if rc != SD_OK:
            name = "sd_verify_noalloc" if self.noalloc else "sd_verify"
            raise RuntimeError(f"{name} failed: {sd_status_string(rc)} ({rc})")
        if self.debug:
            return VerifyResult(self.out_tokens, self.out_num_accepted, self.out_counters,
                                self.status, self.row_lse, self.accept_prob,
                                self.request_flags, self.flags, self.accept_histogram)
        return VerifyResult(self.out_tokens, self.out_num_accepted, self.out_counters, self.status,
                            accept_histogram=self.accept_histogram)


def sd_verify(target_logits, draft_token_ids, draft_probs=None, bitmask=None, temperature=None,
              seed=0, top_k=None, debug=False, stream=None, top_p=None):
    """Verify one batch; returns fresh output tensors (see VerifyResult).

    target_logits [B, k+1, V] bf16/fp32, draft_token_ids [B, k] int32,
    draft_probs [B, k, V] fp32 or None (one-hot drafts), bitmask
    [B, k+1, ceil(V/32)] int32 or None, temperature [B] fp32 (0 = greedy),
    seed (64-bit Philox key), top_k [B] int32 or None, top_p [B] fp32 or None.
    """
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, k+1, V]")
    B, kp1, V = target_logits.shape
    v = Verifier(B, kp1 - 1, V, target_logits.dtype, target_logits.device, debug=debug)
    return v(target_logits, draft_token_ids, draft_probs, bitmask, temperature, seed, top_k, stream,
             top_p=top_p)


def sd_verify_ragged(target_logits, draft_token_ids, draft_offsets, draft_probs=None,
                     bitmask=None, temperature=None, seed=0, top_k=None, top_p=None, max_draft=None,
                     debug=False, histogram=False, stream=None):
    """Verify requests with their own draft counts; returns fresh outputs.

    draft_offsets [B+1] int32 on the device (cumulative: request b has
    off[b+1] - off[b] drafts), target_logits [total + B, V], draft_token_ids
    [total], draft_probs [total, V] or None, bitmask [total + B, ceil(V/32)]
    or None, temperature [B]; out_tokens come back as [total + B] (request b's
    k_b + 1 slots from off[b] + b).  max_draft defaults to 64.
    """
    if target_logits.dim() != 2:
        raise ValueError("target_logits must be [total_drafts + B, V]")
    B = draft_offsets.shape[0] - 1
    rows, V = target_logits.shape
    v = Verifier(B, SD_MAX_DRAFT if max_draft is None else max_draft, V, target_logits.dtype,
                 target_logits.device, debug=debug, histogram=histogram, total_drafts=rows - B)
    return v(target_logits, draft_token_ids, draft_probs, bitmask, temperature, seed, top_k, stream,
             draft_offsets=draft_offsets, top_p=top_p)


class NgramResult(NamedTuple):
    drafts: torch.Tensor             # [B, k] int32, -1 after each request's drafts
    num_drafts: torch.Tensor         # [B] int32
    match_len: torch.Tensor          # [B] int32, 0 = nothing proposed
    draft_offsets: torch.Tensor      # [B+1] int32, cumulative num_drafts
    drafts_flat: torch.Tensor        # [B*k] int32: the drafts back to back (first offsets[B])
    status: torch.Tensor             # [1] int32 holding the uint32 status bits


def _ngram_params(batch, min_n, max_n, num_draft, stride, max_model_len):
    p = SdNgramParams()
    p.batch, p.min_n, p.max_n, p.num_draft = int(batch), int(min_n), int(max_n), int(num_draft)
    p.stride, p.max_model_len = int(stride), int(max_model_len)
    return p


def sd_ngram_workspace_size(batch, stride, min_n=1, max_n=1, num_draft=0, max_model_len=0):
    """Device workspace bytes of the n-gram proposer for these sizes."""
    p = _ngram_params(batch, min_n, max_n, num_draft, stride, max_model_len)
    return int(_lib.sd_ngram_workspace_size(ctypes.byref(p)))


class NgramProposer:
    """Outputs and workspace of the n-gram proposer for a history table of
    [batch, stride] int32 tokens; each call overwrites the tensors it returns."""

    def __init__(self, batch, stride, min_n, max_n, num_draft, max_model_len=0, device=None):
        dev = torch.device(device) if device is not None else torch.device("cuda")
        if dev.type != "cuda":
            raise ValueError("the proposer runs on a HIP device")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.B, self.stride, self.k = int(batch), int(stride), int(num_draft)
        self.params = _ngram_params(batch, min_n, max_n, num_draft, stride, max_model_len)
        probe = _ngram_params(max(self.B, 1), min_n, max_n, num_draft, stride, max_model_len)
        if int(_lib.sd_ngram_workspace_size(ctypes.byref(probe))) == 0:
            raise ValueError(f"unsupported n-gram proposer sizes: batch={batch} stride={stride} "
                             f"min_n={min_n} max_n={max_n} k={num_draft}")
        ws = int(_lib.sd_ngram_workspace_size(ctypes.byref(self.params)))
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.workspace_bytes = ws
        self.drafts = torch.empty((self.B, self.k), dtype=torch.int32, device=dev)
        self.num_drafts = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.match_len = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.draft_offsets = torch.empty(self.B + 1, dtype=torch.int32, device=dev)
        self.drafts_flat = torch.empty(max(self.B * self.k, 1), dtype=torch.int32, device=dev)
        self.status = torch.empty(1, dtype=torch.int32, device=dev)
        self.params.out_match_len = self.match_len.data_ptr()
        self.params.out_draft_offsets = self.draft_offsets.data_ptr()
        self.params.out_drafts_flat = self.drafts_flat.data_ptr()
        self.params.status = self.status.data_ptr()

    def __call__(self, tokens, lengths, stream=None, match_events=None):
        dev = self.device
        _check(tokens, "tokens", torch.int32, (self.B, self.stride), dev)
        _check(lengths, "lengths", torch.int32, (self.B,), dev)
        if match_events is not None:
            self._timing = SdDebugTiming(*match_events)
            self.params.debug_timing = ctypes.pointer(self._timing)
        else:
            self.params.debug_timing = None
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        rc = _lib.sd_ngram_propose(
            _ptr(tokens), _ptr(lengths), _ptr(self.drafts), _ptr(self.num_drafts),
            ctypes.byref(self.params), ctypes.c_void_p(self.workspace.data_ptr()),
            ctypes.c_size_t(self.workspace_bytes), ctypes.c_void_p(int(stream)))
        if rc != SD_OK:
            raise RuntimeError(f"sd_ngram_propose failed: {sd_status_string(rc)} ({rc})")
        return NgramResult(self.drafts, self.num_drafts, self.match_len, self.draft_offsets,
                           self.drafts_flat, self.status)


def sd_ngram_propose(tokens, lengths, min_n, max_n, num_draft, max_model_len=0, stream=None):
    """n-gram drafts for a [B, stride] int32 history table whose row b holds
    lengths[b] tokens; returns fresh outputs (see NgramResult)."""
    if tokens.dim() != 2:
        raise ValueError("tokens must be [B, stride]")
    B, stride = tokens.shape
    prop = NgramProposer(B, stride, min_n, max_n, num_draft, max_model_len, tokens.device)
    return prop(tokens, lengths, stream)


def rates_from_counters(counters, steps):
    """Ratios as a dict (convenience over sd_rates)."""
    s, a, y, m = sd_rates(counters, steps)
    nan2none = (lambda v: None if math.isnan(v) else v)
    return {"survival": nan2none(s), "acceptance": nan2none(a), "yield": nan2none(y),
            "mean_acceptance_length": nan2none(m)}
