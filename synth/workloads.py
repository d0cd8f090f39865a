"""Synthetic workload recipes: shapes, sizes and logit distributions.

Each recipe stands in for a model/dataset pair the DMS pages evaluate on
(Qwen-R1 reasoning traces, Llama 3.2 1B tasks), which are not available
here; only the tensor shapes and the eviction-rate structure are
reproduced.  Values come from ``synth.synth``.

The logit mean for a target marked fraction ``1 - 1/c`` ("CR c" in the
recipes) is ``mu(c) = Phi^-1(1 - 1/c)`` for a unit-variance logit, so that
``P(logit > 0) = 1 - 1/c``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from statistics import NormalDist
from typing import List, Optional

import numpy as np

from . import synth


def mu_for_cr(c: float) -> float:
    """Logit mean that marks a fraction 1 - 1/c of tokens (unit variance)."""
    if c <= 1.0:
        return float("-inf")
    return NormalDist().inv_cdf(1.0 - 1.0 / c)


@dataclass
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    window: int
    decode_steps: int
    seed: int
    prompt_len: int = 0        # uniform prompt length (when lengths_range is None)
    lengths_range: Optional[tuple] = None   # (lo, hi) per-sequence prompt lengths
    num_layers: int = 1
    # logit mean per layer: mu_before for positions < pos_threshold, mu_after beyond
    mu_before: List[float] = field(default_factory=lambda: [0.0])
    mu_after: Optional[List[float]] = None
    pos_threshold: int = synth.MAX_POS
    # per KV head logit mean (the same at every position and layer); when set
    # it replaces mu_before / mu_after: each head reaches its own compression
    head_mu: Optional[List[float]] = None
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def prompt_lengths(self) -> np.ndarray:
        if self.lengths_range is None:
            return np.full(self.batch, self.prompt_len, dtype=np.int64)
        lo, hi = self.lengths_range
        return synth.lengths(self.seed, self.batch, lo, hi)

    def max_tokens(self) -> int:
        return int(self.prompt_lengths().max()) + self.decode_steps

    def layer_mu(self, layer: int):
        """Logit means (below, at or above pos_threshold): scalars, or one
        value per KV head when head_mu is set."""
        if self.head_mu is not None:
            hm = np.asarray(self.head_mu, dtype=np.float64)
            return hm, hm
        before = self.mu_before[layer if len(self.mu_before) > 1 else 0]
        after = before if self.mu_after is None else self.mu_after[layer if len(self.mu_after) > 1 else 0]
        return before, after

    def marked_prob(self, layer: int, pos: np.ndarray, head: int = 0) -> np.ndarray:
        """P(logit > 0) at each position of KV head `head` under the Gaussian
        model of the logit."""
        before, after = self.layer_mu(layer)
        if self.head_mu is not None:
            before = after = float(self.head_mu[head])
        nd = NormalDist()
        pb = 1.0 - nd.cdf(-before) if np.isfinite(before) else 0.0
        pa = 1.0 - nd.cdf(-after) if np.isfinite(after) else 0.0
        return np.where(np.asarray(pos) < self.pos_threshold, pb, pa)

    def pool_blocks(self, layer: int = 0, slack: float = 1.2) -> int:
        """Pool size for one layer: expected live tokens at the last decode
        position of every sequence, times `slack`, in 16-token blocks, plus
        one partly filled block per (sequence, KV head)."""
        total = 0
        heads = range(self.num_kv_heads) if self.head_mu is not None else [0]
        per_head = self.num_kv_heads // len(heads)
        for P in np.unique(self.prompt_lengths()):
            count = int(np.sum(self.prompt_lengths() == P))
            q = int(P) + self.decode_steps - 1
            for h in heads:
                per_unit = int(np.ceil(slack * self.expected_live(layer, q, h) / 16.0)) + 2
                total += per_unit * count * per_head
        return total

    def expected_live(self, layer: int, q: int, head: int = 0) -> float:
        """E|Vis(q)| of KV head `head` under independent marks: unmarked
        tokens plus the window."""
        if q < self.pos_threshold:  # one marking rate over positions 0..q: closed form
            p = float(self.marked_prob(layer, np.array([0]), head)[0])
            return (q + 1) * (1.0 - p) + min(self.window + 1, q + 1) * p
        pos = np.arange(q + 1)
        p = self.marked_prob(layer, pos, head)
        in_window = pos >= q - self.window
        return float(np.sum(1.0 - p) + np.sum(p[in_window]))


def tiny() -> Workload:
    return Workload(
        name="tiny", batch=1, num_q_heads=12, num_kv_heads=2, head_dim=128, dtype="f32",
        window=16, decode_steps=256, seed=1000, prompt_len=256, mu_before=[0.0],
        description="1 sequence, 12 Q / 2 KV heads, head_dim 128, fp32, 256-token prompt + "
                    "256 decode steps, w=16, logits N(0,1) (about half marked)")


def llama_1b() -> Workload:
    return Workload(
        name="llama-3.2-1b-layer", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=64,
        dtype="bf16", window=256, decode_steps=512, seed=1001, prompt_len=4096,
        mu_before=[0.67],
        description="Llama-3.2-1B-shaped layer: 32 Q / 8 KV heads, head_dim 64, bf16, 8 sequences, "
                    "4096-token context, w=256, logits N(0.67,1) (CR 4), 512 decode steps")


def qwen_7b() -> Workload:
    return Workload(
        name="qwen-r1-7b-layer", batch=32, num_q_heads=28, num_kv_heads=4, head_dim=128,
        dtype="bf16", window=256, decode_steps=256, seed=1002, prompt_len=16384,
        mu_before=[1.15],
        description="Qwen-R1-7B-shaped layer: 28 Q / 4 KV heads, head_dim 128, bf16, 32 chains, "
                    "16384-token context, w=256, logits N(1.15,1) (CR 8), 256 decode steps")


def qwen_32b() -> Workload:
    return Workload(
        name="qwen-r1-32b-layer", batch=64, num_q_heads=40, num_kv_heads=8, head_dim=128,
        dtype="bf16", window=256, decode_steps=256, seed=1003, prompt_len=32768,
        mu_before=[mu_for_cr(4.0)], mu_after=[mu_for_cr(12.0)], pos_threshold=10240,
        description="Qwen-R1-32B-shaped layer: 40 Q / 8 KV heads, head_dim 128, bf16, 64 chains at "
                    "32768 tokens, w=256, logit mean for CR 4 below position 10240 and CR 12 "
                    "beyond (overall about 8), 256 decode steps")


def qwen_32b_dense() -> Workload:
    """The Qwen-R1-32B-shaped layer with nothing marked (CR 1): the dense
    baseline through the same kernels.  The logits are N(-8, 1)-like values
    of the Irwin-Hall generator, which never exceed -8 + 6 = -2."""
    w = qwen_32b()
    w.name = "qwen-r1-32b-layer-dense"
    w.seed = 1003
    w.mu_before, w.mu_after, w.pos_threshold = [-8.0], None, synth.MAX_POS
    w.description = ("Qwen-R1-32B-shaped layer as above with every eviction logit below 0: nothing is "
                     "evicted (CR 1), 64 chains x 32768 tokens of dense KV")
    return w


def head_skew_crs(num_kv_heads: int = 8):
    """Per-KV-head compression ratios spread over [2, 16] with arithmetic mean
    8: CR_h = 2 + 14 (h / (H - 1))^1.4 (the exponent puts the mean at 8.0 for
    8 heads).  The CR-2 head keeps about 2.5 times the layer's mean live
    tokens, the CR-16 head about a third of it."""
    H = num_kv_heads
    return [2.0 + 14.0 * (h / (H - 1)) ** 1.4 for h in range(H)]


def qwen_32b_head_skew() -> Workload:
    """The Qwen-R1-32B-shaped layer with per-head compression: KV head h
    marks a fraction 1 - 1/CR_h of its tokens at every position, CR_h from
    head_skew_crs (2 ... 16, mean 8), the same for every sequence (a head's
    rate is a property of the head).  Live counts per (sequence, KV head)
    then differ by up to 7x within the layer."""
    w = qwen_32b()
    w.name = "qwen-r1-32b-layer-head-skew"
    w.seed = 1007
    w.mu_before, w.mu_after, w.pos_threshold = [0.0], None, synth.MAX_POS
    w.head_mu = [mu_for_cr(c) for c in head_skew_crs(w.num_kv_heads)]
    w.description = ("Qwen-R1-32B-shaped layer (64 chains x 32768 tokens, 40 Q / 8 KV heads, d 128, bf16, w 256) "
                     "with per-KV-head CR 2 ... 16 (arithmetic mean 8): live tokens per head differ up to 7x")
    return w


def qwen_32b_hyperscale() -> Workload:
    """Base of the hyper-scaling harness: the Qwen-R1-32B-shaped layer with
    a 1024-token prompt and the vanilla generation that sets the budget
    (8 chains x 16384 tokens); the harness varies the chain count and length."""
    w = qwen_32b()
    w.name = "qwen-r1-32b-hyperscale"
    w.batch, w.prompt_len, w.decode_steps = 8, 1024, 16384
    w.seed = 1005
    w.description = ("Qwen-R1-32B-shaped layer (40 Q / 8 KV heads, d 128, bf16, w 256, CR 4 below position "
                     "10240 and 12 beyond), 1024-token prompt; the vanilla budget is 8 chains x 16384 tokens")
    return w


def full_32b() -> Workload:
    layers = 64
    crs = [4.0 + 8.0 * l / (layers - 1) for l in range(layers)]
    return Workload(
        name="qwen-r1-32b-64-layer-step", batch=256, num_q_heads=40, num_kv_heads=8, head_dim=128,
        dtype="bf16", window=256, decode_steps=128, seed=1004, lengths_range=(1024, 32768),
        num_layers=layers, mu_before=[mu_for_cr(c) for c in crs],
        description="64 layers x (40 Q / 8 KV heads, head_dim 128, bf16), 256 chains with lengths "
                    "uniform in [1024, 32768], w=256, per-layer CR from 4 (layer 0) to 12 "
                    "(layer 63), 128 decode steps")


@dataclass
class TrainWorkload:
    """A layer of the relaxed (training-time) attention: every position of
    `batch` sequences of `seq_len` tokens attends causally, with the soft mask
    of logits ~ mu + N(0, 1) (Irwin-Hall), offset gamma, temperature tau and
    Logistic(0, 1) noise.  dO is a query-shaped draw of seed + 1."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int
    window: int
    gamma: float
    tau: float
    mu: float
    seed: int
    description: str = ""

    def host_slice(self, b_list, kv_heads):
        """Host tensors of sequences b_list and KV heads kv_heads (with their
        query heads): Q, K, V, dO (bf16-exact float32), logits, noise."""
        G = self.num_q_heads // self.num_kv_heads
        qh = [h * G + j for h in kv_heads for j in range(G)]
        pos = np.arange(self.seq_len)
        d = self.head_dim
        Q = synth.tensor(self.seed, synth.STREAM_Q, 0, b_list, qh, pos, d, "bf16")
        K = synth.tensor(self.seed, synth.STREAM_K, 0, b_list, kv_heads, pos, d, "bf16")
        V = synth.tensor(self.seed, synth.STREAM_V, 0, b_list, kv_heads, pos, d, "bf16")
        dO = synth.tensor(self.seed + 1, synth.STREAM_Q, 0, b_list, qh, pos, d, "bf16")
        lg = synth.logits(self.seed, 0, b_list, kv_heads, pos, self.mu)
        g = synth.logistic_noise(self.seed, 0, b_list, kv_heads, pos)
        return Q, K, V, dO, lg, g

    def device_inputs(self):
        """The same values for the whole layer on the current GPU (the device
        twin of the generator; the noise is drawn on the host)."""
        import torch
        from synth import device as dsynth
        B, Hq, Hkv, T, d = self.batch, self.num_q_heads, self.num_kv_heads, self.seq_len, self.head_dim
        q = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device="cuda")
        do = torch.empty_like(q)
        k = torch.empty((B, Hkv, T, d), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        dsynth.fill(q, self.seed, synth.STREAM_Q, 0, 0)
        dsynth.fill(do, self.seed + 1, synth.STREAM_Q, 0, 0)
        dsynth.fill(k, self.seed, synth.STREAM_K, 0, 0)
        dsynth.fill(v, self.seed, synth.STREAM_V, 0, 0)
        lg = torch.empty((B, Hkv, T), dtype=torch.float32, device="cuda")
        dsynth.logits(lg, self.seed, 0, 0, self.mu)
        g = torch.from_numpy(synth.logistic_noise(self.seed, 0, np.arange(B), np.arange(Hkv),
                                                  np.arange(T))).cuda()
        return q, k, v, do, lg, g

    def causal_pairs(self) -> int:
        """(query, key) pairs with key <= query, all heads."""
        T = self.seq_len
        return self.batch * self.num_q_heads * T * (T + 1) // 2


def qwen_32b_train() -> TrainWorkload:
    return TrainWorkload(
        name="qwen-r1-32b-train-layer", batch=4, num_q_heads=40, num_kv_heads=8, head_dim=128, seq_len=4096,
        window=256, gamma=-5.0, tau=0.1, mu=5.0, seed=1006,
        description="Qwen-R1-32B-shaped layer (40 Q / 8 KV heads, d 128, bf16, w 256) at training time: 4 "
                    "sequences x 4096 tokens, relaxed decisions with tau 0.1, gamma -5, logits 5 + N(0, 1), "
                    "Logistic noise")


ALL = {w().name: w for w in (tiny, llama_1b, qwen_7b, qwen_32b, qwen_32b_dense, qwen_32b_head_skew,
                              qwen_32b_hyperscale, full_32b)}
