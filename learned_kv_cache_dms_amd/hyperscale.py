"""Inference-time hyper-scaling harness: spend a KV-cache budget on longer
or more parallel generations, and run the chosen configurations through the
DMS decode path.

Sources: "Inference-Time Hyper-Scaling with KV Cache Compression", the
third-party summary page, sections "TL;DR" and "Key claims", and the arXiv
listing's "Abstract".  Generation cost is set by the size of the KV cache,
not by the number of tokens.  So at a fixed budget of KV-cache memory reads,
or of peak KV tokens, a compressed cache can generate longer chains
(sequential scaling), more chains (parallel scaling) or both.  The best
configurations mix the two.

Budget arithmetic, per (sequence, KV head) and per layer.  The factors
common to every configuration (layers, KV heads, bytes per token) cancel.
* A chain with a P-token prompt that generates L tokens holds |Vis(q)| tokens
  when it attends at position q.  It reads them all at that step.
* Memory reads of W chains = W * sum over q = P .. P+L-1 of |Vis(q)|.
* Peak tokens of W chains = W * |Vis(P+L-1)|.  A step adds one token and
  retires at most one, so the live count never falls.
* Expected |Vis(q)|, for independent decisions marked with probability p_i,
  is sum over i <= q-w-1 of (1 - p_i), plus min(q+1, w+1).  The window's
  tokens are all visible, marked or not.  The vanilla model never marks
  (p = 0), so |Vis(q)| = q + 1.

The runner drives ``dms.Cache``: prompt compression, then L appends and
attentions per chain.  It reports the device's own counters (reads = the sum
of live tokens over the steps) next to the count implied by the actual
decisions.  The two must agree exactly.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# Budget model
# ----------------------------------------------------------------------------

def expected_live_curve(marked_prob: Callable[[np.ndarray], np.ndarray], w: int, q_max: int) -> np.ndarray:
    """E|Vis(q)| for q = 0 .. q_max, for independent decisions that mark
    position i with probability marked_prob(i)."""
    pos = np.arange(q_max + 1)
    keep = 1.0 - np.asarray(marked_prob(pos), dtype=np.float64)
    cum = np.cumsum(keep)                                   # sum over i <= q of (1 - p_i)
    far = np.where(pos - w - 1 >= 0, cum[np.maximum(pos - w - 1, 0)], 0.0)
    return far + np.minimum(pos + 1, w + 1)


@dataclass
class Config:
    width: int        # chains generated in parallel
    length: int       # tokens generated per chain
    reads: float      # expected KV tokens read, all chains, per (KV head, layer)
    peak: float       # expected peak KV tokens, all chains, per (KV head, layer)

    @property
    def tokens(self) -> int:
        return self.width * self.length


class BudgetModel:
    """Expected memory reads and peak tokens of (width, length) configurations
    after a `prompt`-token prompt."""

    def __init__(self, marked_prob: Callable[[np.ndarray], np.ndarray], window: int, prompt: int,
                 max_length: int):
        self.prompt, self.window, self.max_length = prompt, window, max_length
        live = expected_live_curve(marked_prob, window, prompt + max_length - 1)
        # reads_per_chain[L] = sum over q = P .. P+L-1 of E|Vis(q)|
        self.live = live
        self.reads_per_chain = np.concatenate([[0.0], np.cumsum(live[prompt:])])

    def config(self, width: int, length: int) -> Config:
        if not 1 <= length <= self.max_length:
            raise ValueError(f"length {length} outside 1 .. {self.max_length}")
        return Config(width, length, width * float(self.reads_per_chain[length]),
                      width * float(self.live[self.prompt + length - 1]))

    def longest(self, width: int, budget: float, kind: str) -> Optional[Config]:
        """The longest generation of `width` chains within `budget` of
        `kind` ("reads" or "peak"), or None if not even one token fits."""
        per = self.reads_per_chain[1:] if kind == "reads" else self.live[self.prompt:]
        ok = np.nonzero(width * per <= budget * (1 + 1e-12))[0]
        # both curves increase with the length, so the admissible lengths are a prefix
        if len(ok) == 0:
            return None
        return self.config(width, int(ok[-1]) + 1)


def frontier(dms: BudgetModel, budget: float, kind: str, widths: Sequence[int]) -> List[Config]:
    """For each width, the longest DMS generation within the budget."""
    out = []
    for wd in widths:
        c = dms.longest(wd, budget, kind)
        if c is not None:
            out.append(c)
    return out


# ----------------------------------------------------------------------------
# Exact counts from actual decisions (device tensors)
# ----------------------------------------------------------------------------

def exact_reads_and_peak(logits, prompt: int, length: int, window: int):
    """Reads (sum over the L decode positions of |Vis(q)|, all units) and the
    final live count (all units) implied by logits [W, Hkv, P + L] (a torch
    tensor): |Vis(q)| = (unmarked positions <= q - w - 1) + min(q + 1, w + 1)."""
    import torch
    T = prompt + length
    lg = logits[..., :T]
    unmarked = ((lg <= 0) | torch.isnan(lg)).to(torch.int64)
    cu = torch.cumsum(unmarked, dim=-1)
    pos = torch.arange(T, device=lg.device)
    q = pos[prompt:]
    far = torch.where(q - window - 1 >= 0, cu[..., torch.clamp(q - window - 1, min=0)], torch.zeros_like(cu[..., prompt:]))
    live = far + torch.clamp(q + 1, max=window + 1)
    return int(live.sum().item()), int(live[..., -1].sum().item())


# ----------------------------------------------------------------------------
# Runner: a configuration end to end through the C ABI
# ----------------------------------------------------------------------------

@dataclass
class RunResult:
    width: int
    length: int
    seconds: float            # decode steps only (append + attention), device time
    tokens_per_s: float       # generated tokens (width * length) per second
    reads_device: int         # sum over steps of live tokens, from the device counter
    reads_exact: int          # the same implied by the decisions
    peak_device: int          # live tokens after the last step
    peak_exact: int
    kv_bytes_read: float      # reads_device * 2 * d * element size (one layer)


def run_config(wl, width: int, length: int, chunk: int = 512) -> RunResult:
    """Prefills `width` chains of the workload's prompt and generates `length`
    tokens each through dms_append_step + dms_decode_attention.  Inputs are
    generated on the device per chunk of steps, outside the timed part; the
    decode steps of each chunk are timed with HIP events on the stream the
    library launches on."""
    import torch
    from synth import device as dsynth
    from synth import synth
    from . import dms

    w = dataclasses.replace(wl, batch=width, decode_steps=length)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    esize = 2 if w.dtype == "bf16" else 4
    P = int(w.prompt_len)
    lengths = w.prompt_lengths()
    cache = dms.Cache(B, Hq, Hkv, d, w.window, w.max_tokens(), w.pool_blocks(0), dtype=w.dtype)
    mb, ma = w.layer_mu(0)
    K = torch.empty((B, Hkv, P, d), dtype=tdt, device="cuda")
    V = torch.empty_like(K)
    Lall = torch.empty((B, Hkv, P + length), dtype=torch.float32, device="cuda")
    dsynth.fill(K, w.seed, synth.STREAM_K, 0, 0)
    dsynth.fill(V, w.seed, synth.STREAM_V, 0, 0)
    dsynth.logits(Lall, w.seed, 0, 0, mb, ma, w.pos_threshold)
    cache.prefill(K, V, Lall[..., :P].contiguous(), lengths)
    del K, V
    st0 = cache.stats()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    base = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    total_ms = 0.0
    for c0 in range(0, length, chunk):
        n = min(chunk, length - c0)
        qs = torch.empty((n, B, Hq, d), dtype=tdt, device="cuda")
        ks = torch.empty((n, B, Hkv, d), dtype=tdt, device="cuda")
        vs = torch.empty_like(ks)
        for t in range(n):
            pb = base + (c0 + t)
            dsynth.fill(qs[t], w.seed, synth.STREAM_Q, 0, 0, pos_base=pb)
            dsynth.fill(ks[t], w.seed, synth.STREAM_K, 0, 0, pos_base=pb)
            dsynth.fill(vs[t], w.seed, synth.STREAM_V, 0, 0, pos_base=pb)
        lgs = Lall[..., P + c0:P + c0 + n].permute(2, 0, 1).contiguous()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for t in range(n):
            cache.append(ks[t], vs[t], lgs[t])
            cache.attend(qs[t], out)
        b.record()
        torch.cuda.synchronize()
        total_ms += a.elapsed_time(b)
    st1 = cache.stats()
    if st1["sticky_error"] != 0:
        raise RuntimeError(f"device error during the run: {st1}")
    reads_exact, peak_exact = exact_reads_and_peak(Lall, P, length, w.window)
    reads_dev = st1["live_token_steps"] - st0["live_token_steps"]
    secs = total_ms / 1e3
    return RunResult(width, length, secs, width * length / secs, int(reads_dev), reads_exact,
                     int(st1["live_tokens"]), peak_exact, float(reads_dev) * 2 * d * esize)
