"""Seeded synthetic verify workloads (inputs only; no verification arithmetic).

Shared by the tests, the smoke check and the benchmark, for both the HIP path
and the CPU oracle.  Every tensor is drawn from a seeded torch.Generator on the
requested device.  The random numbers the verifier itself draws are not made
here: they come from the Philox streams keyed by the call's seed.

Workloads (synthetic stand-ins for drafter/target traffic; the pages name no
dataset).  `batch=` shrinks a workload to fewer requests at the same k and V:

  tiny        B=4,   k=3,  V=1000,   fp32 logits ~ N(0, 2^2); q = softmax(l + N(0,1));
              x ~ q; T = [1, 1, 0, 0]; no bitmask
  draft_model B=64,  k=5,  V=32000,  bf16 ~ N(0, 3^2); q = softmax(0.8 l + N(0,1)); x ~ q;
              T = 0.8
  ngram       B=256, k=4,  V=151936, bf16 ~ N(0, 3^2); x = the row's argmax (lowest
              index) with probability 0.6, else uniform over V; no q; T = 1
  structured  B=128, k=5,  V=128256, bf16 ~ N(0, 3^2); each (request, position) row
              allows exactly round(0.05 V) tokens, uniformly chosen; exactly 20% of the
              draft positions draw x uniformly from their row's disallowed tokens, the
              rest x ~ q with q = softmax(0.8 l + N(0,1)) restricted to the allowed
              tokens; T = 0.7
  ngram_ragged B=256, k_b uniform on 1..7 (max 7, mean 4), V=151936: the ngram recipe
              per request with its own draft count; rows packed without padding
              (draft_offsets [B+1]); "max_draft" = 7
  long_k      B=512, k=12, V=151936, bf16 ~ N(0, 3^2); q = softmax(0.7 l + N(0, 1.5^2));
              x ~ q (unrestricted); a quarter of the requests greedy, the rest
              T ~ U[0.6, 1.2] with top_k = 50; a random half of the requests carry
              bitmasks allowing exactly round(0.1 V) tokens per row, the others
              all-ones rows

History tables for the n-gram proposer (make_histories):

  ngram_propose B=256 token histories in a [256, 16384] int32 table, V=151936,
              windows 2..5, k=4, context length 16384 (so histories longer than
              16380 get no drafts).  Lengths uniform on [2048, 16384].  A history
              is a prompt of uniform random tokens (the first half) followed by
              "generated" text built segment by segment: with probability 0.5 a
              copy of an earlier span (length uniform on 8..64, start uniform over
              the text so far), else a fresh run of 1..16 uniform tokens -- the
              text-reuse pattern prompt lookup serves (summaries quoting their
              source, edited code).  Slots past a row's length hold random tokens
              that the proposer never reads.
"""
import math

import torch

WORKLOADS = {
    "tiny": dict(B=4, k=3, V=1000, dtype=torch.float32),
    "draft_model": dict(B=64, k=5, V=32000, dtype=torch.bfloat16),
    "ngram": dict(B=256, k=4, V=151936, dtype=torch.bfloat16),
    "structured": dict(B=128, k=5, V=128256, dtype=torch.bfloat16),
    "long_k": dict(B=512, k=12, V=151936, dtype=torch.bfloat16),
    "ngram_ragged": dict(B=256, k=7, V=151936, dtype=torch.bfloat16),
}

_SEED_BASE = {"tiny": 1001, "draft_model": 1002, "ngram": 1003, "structured": 1004, "long_k": 1005,
              "ngram_ragged": 1006}


def pack_bitmask(allowed):
    """[..., V] bool -> [..., ceil(V/32)] int32 words; bit j & 31 of word j >> 5."""
    V = allowed.shape[-1]
    W = (V + 31) // 32
    pad = W * 32 - V
    a = allowed
    if pad:
        a = torch.cat([a, torch.zeros(a.shape[:-1] + (pad,), dtype=torch.bool, device=a.device)], -1)
    a = a.reshape(a.shape[:-1] + (W, 32)).to(torch.int64)
    shifts = torch.arange(32, device=a.device, dtype=torch.int64)
    words = (a << shifts).sum(-1)
    words = torch.where(words >= 2**31, words - 2**32, words)
    return words.to(torch.int32)


def _exact_allowed(rows, V, n_allowed, gen, device):
    """[rows, V] bool with exactly n_allowed True per row, uniformly placed."""
    out = torch.zeros(rows, V, dtype=torch.bool, device=device)
    step = max(1, (1 << 27) // V)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        keys = torch.rand(r1 - r0, V, generator=gen, device=device)
        idx = torch.topk(keys, n_allowed, dim=1).indices
        out[r0:r1].scatter_(1, idx, True)
    return out


def _softmax_rows(z):
    return torch.softmax(z, dim=-1)


def _sample_rows(probs2d, gen, chunk=2048):
    """One draw per row of a [n, V] float32 probability matrix."""
    outs = []
    for r0 in range(0, probs2d.shape[0], chunk):
        outs.append(torch.multinomial(probs2d[r0:r0 + chunk], 1, generator=gen)[:, 0])
    return torch.cat(outs) if outs else torch.zeros(0, dtype=torch.int64, device=probs2d.device)


def make_workload(name, device="cpu", batch=None, seed=None):
    """Inputs of one verify call as a dict of tensors on `device`:
    logits, draft_token_ids, draft_probs (or None), bitmask (or None),
    temperature, top_k (or None), and `seed` (the verifier's Philox key)."""
    spec = WORKLOADS[name]
    B = spec["B"] if batch is None else int(batch)
    k, V, dtype = spec["k"], spec["V"], spec["dtype"]
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(_SEED_BASE[name] if seed is None else int(seed))
    kp1 = k + 1

    def normal(shape, std):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std

    q = None
    mask = None
    top_k = None
    if name == "tiny":
        logits = normal((B, kp1, V), 2.0)
        q = _softmax_rows(logits[:, :k] + normal((B, k, V), 1.0)).contiguous()
        x = _sample_rows(q.reshape(B * k, V), gen).reshape(B, k)
        T = torch.tensor([1.0, 1.0, 0.0, 0.0] * ((B + 3) // 4), device=dev)[:B]
    elif name == "draft_model":
        logits = normal((B, kp1, V), 3.0).to(dtype)
        q = _softmax_rows(0.8 * logits[:, :k].float() + normal((B, k, V), 1.0)).contiguous()
        x = _sample_rows(q.reshape(B * k, V), gen).reshape(B, k)
        T = torch.full((B,), 0.8, device=dev)
    elif name == "ngram":
        logits = normal((B, kp1, V), 3.0).to(dtype)
        amax = torch.argmax(logits[:, :k].float(), dim=-1)          # first occurrence
        uni = torch.randint(0, V, (B, k), generator=gen, device=dev)
        pick = torch.rand((B, k), generator=gen, device=dev) < 0.6
        x = torch.where(pick, amax, uni)
        T = torch.ones(B, device=dev)
    elif name == "structured":
        logits = normal((B, kp1, V), 3.0).to(dtype)
        n_allowed = int(round(0.05 * V))
        allowed = _exact_allowed(B * kp1, V, n_allowed, gen, dev).reshape(B, kp1, V)
        z = 0.8 * logits[:, :k].float() + normal((B, k, V), 1.0)
        z = torch.where(allowed[:, :k], z, torch.full_like(z, -math.inf))
        q = _softmax_rows(z).contiguous()
        x = _sample_rows(q.reshape(B * k, V), gen).reshape(B, k)
        n_inv = int(round(0.2 * B * k))
        inv_pos = torch.randperm(B * k, generator=gen, device=dev)[:n_inv]
        dis = (~allowed[:, :k]).reshape(B * k, V)[inv_pos].float()
        x_inv = torch.multinomial(dis, 1, generator=gen)[:, 0]
        x = x.reshape(B * k)
        x[inv_pos] = x_inv
        x = x.reshape(B, k)
        mask = pack_bitmask(allowed)
        T = torch.full((B,), 0.7, device=dev)
    elif name == "long_k":
        logits = torch.empty((B, kp1, V), dtype=dtype, device=dev)
        q = torch.empty((B, k, V), dtype=torch.float32, device=dev)
        x = torch.empty((B, k), dtype=torch.int64, device=dev)
        step = 32
        for b0 in range(0, B, step):
            b1 = min(B, b0 + step)
            lg = normal((b1 - b0, kp1, V), 3.0).to(dtype)
            logits[b0:b1] = lg
            qq = _softmax_rows(0.7 * lg[:, :k].float() + normal((b1 - b0, k, V), 1.5))
            q[b0:b1] = qq
            x[b0:b1] = _sample_rows(qq.reshape(-1, V), gen).reshape(b1 - b0, k)
        perm = torch.randperm(B, generator=gen, device=dev)
        greedy = torch.zeros(B, dtype=torch.bool, device=dev)
        greedy[perm[: B // 4]] = True
        T = 0.6 + 0.6 * torch.rand(B, generator=gen, device=dev)
        T = torch.where(greedy, torch.zeros_like(T), T)
        top_k = torch.where(greedy, torch.zeros(B, dtype=torch.int32, device=dev),
                            torch.full((B,), 50, dtype=torch.int32, device=dev))
        masked = torch.zeros(B, dtype=torch.bool, device=dev)
        masked[torch.randperm(B, generator=gen, device=dev)[: B // 2]] = True
        W = (V + 31) // 32
        mask = torch.full((B, kp1, W), -1, dtype=torch.int32, device=dev)
        if V % 32:
            mask[..., -1] = (1 << (V % 32)) - 1
        mrows = torch.nonzero(masked)[:, 0]
        n_allowed = int(round(0.1 * V))
        for r0 in range(0, mrows.numel(), step):
            sel = mrows[r0:r0 + step]
            al = _exact_allowed(sel.numel() * kp1, V, n_allowed, gen, dev).reshape(-1, kp1, V)
            mask[sel] = pack_bitmask(al)
    elif name == "ngram_ragged":
        ks = torch.randint(1, k + 1, (B,), generator=gen, device=dev)
        off = torch.zeros(B + 1, dtype=torch.int64, device=dev)
        off[1:] = torch.cumsum(ks, 0)
        total = int(off[-1].item())
        rows = total + B
        logits = normal((rows, V), 3.0).to(dtype)
        bidx = torch.repeat_interleave(torch.arange(B, device=dev), ks)
        pos = torch.arange(total, device=dev) - off[bidx]
        drow = off[bidx] + bidx + pos                       # the row of each draft
        amax = torch.argmax(logits[drow].float(), dim=-1)
        uni = torch.randint(0, V, (total,), generator=gen, device=dev)
        pick = torch.rand(total, generator=gen, device=dev) < 0.6
        x = torch.where(pick, amax, uni)
        T = torch.ones(B, device=dev)
        return {
            "name": name, "logits": logits.contiguous(),
            "draft_token_ids": x.to(torch.int32).contiguous(),
            "draft_offsets": off.to(torch.int32).contiguous(), "max_draft": k,
            "draft_probs": None, "bitmask": None, "temperature": T.contiguous(),
            "top_k": None, "seed": 0,
        }
    else:
        raise KeyError(name)

    return {
        "name": name,
        "logits": logits.contiguous(),
        "draft_token_ids": x.to(torch.int32).contiguous(),
        "draft_probs": q,
        "bitmask": mask,
        "temperature": T.to(torch.float32).contiguous(),
        "top_k": top_k,
        "seed": 0,
    }


def to_numpy(wl, requests=None):
    """Host copies for the oracle (bf16 becomes exact float32); optionally only
    the given request indices."""
    def cv(t):
        if t is None:
            return None
        if requests is not None:
            t = t[torch.as_tensor(requests, device=t.device)]
        t = t.detach()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.cpu().numpy()
    return {key: (cv(v) if isinstance(v, torch.Tensor) or v is None else v)
            for key, v in wl.items()}


def algorithmic_bytes(wl, residual_q=0):
    """Bytes the method has to move for one call: every logit once, every mask
    word once, the q values a residual draw depends on (residual_q of them in
    all: the whole q row of a rejected position without a top-k cut, only the
    kept tokens' values with one, since max(p - q, 0) is zero wherever the cut
    sets p to zero), the q gathers at the drafts, the draft ids, temperatures
    and outputs."""
    if "draft_offsets" in wl:
        return _algorithmic_bytes_ragged(wl, residual_q)
    return _algorithmic_bytes_uniform(wl, residual_q)


def residual_q_values(wl, num_accepted):
    """The q values the residual draws of one call depend on: for each sampling
    request (temperature > 0) that rejected a draft, V without a top-k cut,
    else its top-k (the kept tokens).  Zero for one-hot drafts."""
    if wl["draft_probs"] is None:
        return 0
    import numpy as np
    T = wl["temperature"].cpu().numpy()
    nacc = np.asarray(num_accepted.cpu().numpy() if hasattr(num_accepted, "cpu") else num_accepted)
    if "draft_offsets" in wl:
        off = wl["draft_offsets"].cpu().numpy()
        kb = off[1:] - off[:-1]
        V = wl["logits"].shape[1]
    else:
        kb = np.full(T.shape, wl["logits"].shape[1] - 1)
        V = wl["logits"].shape[2]
    rejected = (nacc >= 0) & (nacc < kb) & (T > 0)
    per = np.full(T.shape, V, dtype=np.int64)
    if wl.get("top_k") is not None:
        K = wl["top_k"].cpu().numpy().astype(np.int64)
        per = np.where(K > 0, np.minimum(K, V), V)
    return int(per[rejected].sum())


def _algorithmic_bytes_ragged(wl, residual_q=0):
    logits = wl["logits"]
    rows, V = logits.shape
    B = wl["draft_offsets"].shape[0] - 1
    T = rows - B
    total = logits.numel() * logits.element_size() + (B + 1) * 4
    if wl["bitmask"] is not None:
        total += wl["bitmask"].numel() * 4
    if wl["draft_probs"] is not None:
        total += T * 4 + int(residual_q) * 4
    total += T * 4 + B * 4 + rows * 4 + B * 4
    return total


def _algorithmic_bytes_uniform(wl, residual_q=0):
    logits = wl["logits"]
    B, kp1, V = logits.shape
    k = kp1 - 1
    total = logits.numel() * logits.element_size()
    if wl["bitmask"] is not None:
        total += wl["bitmask"].numel() * 4
    if wl["draft_probs"] is not None:
        total += B * k * 4 + int(residual_q) * 4
    total += B * k * 4 + B * 4 + B * kp1 * 4 + B * 4
    return total


HISTORY_WORKLOADS = {
    "ngram_propose": dict(B=256, stride=16384, Lmin=2048, V=151936, min_n=2, max_n=5, k=4,
                          max_model_len=16384),
}


def _history(rng, L, V, copy_p=0.5, span=(8, 64), fresh=(1, 16)):
    import numpy as np
    h = np.empty(L, dtype=np.int64)
    P = L // 2
    h[:P] = rng.integers(0, V, size=P)
    n = P
    while n < L:
        if n > 0 and rng.random() < copy_p:
            m = int(rng.integers(span[0], span[1] + 1))
            s0 = int(rng.integers(0, n))
            m = min(m, L - n)
            if s0 + m <= n:
                h[n:n + m] = h[s0:s0 + m]
            else:
                for t in range(m):       # overlaps what it copies, like repeated text
                    h[n + t] = h[s0 + t]
        else:
            m = min(int(rng.integers(fresh[0], fresh[1] + 1)), L - n)
            h[n:n + m] = rng.integers(0, V, size=m)
        n += m
    return h


def make_histories(name="ngram_propose", device="cpu", batch=None, seed=None, **overrides):
    """Inputs of one n-gram proposer call: tokens [B, stride] int32 and
    lengths [B] int32 on `device`, plus the call's settings (min_n, max_n, k,
    max_model_len, V).  Built with NumPy's seeded generator on the host."""
    import numpy as np
    cfg = dict(HISTORY_WORKLOADS[name], **overrides)
    B = cfg["B"] if batch is None else int(batch)
    rng = np.random.default_rng(7 if seed is None else seed)
    stride, V = cfg["stride"], cfg["V"]
    lengths = rng.integers(cfg["Lmin"], stride + 1, size=B)
    table = rng.integers(0, V, size=(B, stride))
    for b in range(B):
        table[b, :lengths[b]] = _history(rng, int(lengths[b]), V)
    return {"tokens": torch.tensor(table, dtype=torch.int32, device=device),
            "lengths": torch.tensor(lengths, dtype=torch.int32, device=device),
            "min_n": cfg["min_n"], "max_n": cfg["max_n"], "k": cfg["k"],
            "max_model_len": cfg["max_model_len"], "V": V}
