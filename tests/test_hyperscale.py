"""Host logic of the hyper-scaling harness against the oracle (CPU only)."""
import numpy as np
import torch

from learned_kv_cache_dms_amd import hyperscale as H
from oracle import dms_oracle as O
from synth import workloads as W


def test_expected_live_equals_exact_count_for_certain_decisions():
    """With every p_i in {0, 1} the expectation is the exact visible count."""
    rng = np.random.default_rng(41)
    for w in (0, 3, 17):
        p = (rng.random(200) < 0.7).astype(np.float64)
        curve = H.expected_live_curve(lambda pos: p[pos], w, 199)
        for q in range(200):
            assert curve[q] == len(O.visible(p.astype(bool), q, w)), (w, q)


def test_expected_live_matches_sampled_decisions():
    """Position-dependent marking rates: the mean visible count over 4000
    sampled decision rows is within 5 standard errors of the expectation."""
    rng = np.random.default_rng(42)
    T, w, n = 160, 9, 4000
    probs = np.where(np.arange(T) < 60, 0.75, 0.92)
    curve = H.expected_live_curve(lambda pos: probs[pos], w, T - 1)
    counts = np.empty((n, T))
    for s in range(n):
        a = rng.random(T) < probs
        counts[s] = [len(O.visible(a, q, w)) for q in range(T)]
    mean, se = counts.mean(0), counts.std(0, ddof=1) / np.sqrt(n)
    assert np.all(np.abs(mean - curve) <= 5 * se + 1e-12)


def test_exact_reads_and_peak_against_the_oracle():
    rng = np.random.default_rng(43)
    Wd, Hkv, P, L, w = 3, 2, 40, 70, 6
    lg = rng.standard_normal((Wd, Hkv, P + L)).astype(np.float32) + 0.6
    lg[0, 1, 5] = np.nan
    reads, peak = H.exact_reads_and_peak(torch.from_numpy(lg), P, L, w)
    r_ref = p_ref = 0
    for b in range(Wd):
        for h in range(Hkv):
            a = O.eviction_decision(lg[b, h])
            sizes = [len(O.visible(a, q, w)) for q in range(P, P + L)]
            r_ref += sum(sizes)
            p_ref += sizes[-1]
    assert (reads, peak) == (r_ref, p_ref)


def test_vanilla_budget_and_dms_frontier():
    wl = W.qwen_32b_hyperscale()
    P, L0, W0 = wl.prompt_len, wl.decode_steps, wl.batch
    vanilla = H.BudgetModel(lambda pos: np.zeros(len(pos)), wl.window, P, 4 * L0)
    dms = H.BudgetModel(lambda pos: wl.marked_prob(0, pos), wl.window, P, 4 * L0)
    base = vanilla.config(W0, L0)
    # vanilla: |Vis(q)| = q + 1
    assert base.reads == W0 * sum(q + 1 for q in range(P, P + L0))
    assert base.peak == W0 * (P + L0)
    # the vanilla generation is the longest of its width within its own budget
    assert vanilla.longest(W0, base.reads, "reads").length == L0
    assert vanilla.longest(W0, base.peak, "peak").length == L0
    for kind, budget in (("reads", base.reads), ("peak", base.peak)):
        fr = H.frontier(dms, budget, kind, [W0, 2 * W0, 4 * W0, 8 * W0])
        assert fr[0].width == W0 and fr[0].length > L0          # compression buys longer chains
        for c in fr:
            assert (c.reads if kind == "reads" else c.peak) <= budget * (1 + 1e-9)
            if c.length < dms.max_length:                     # one more token would not fit
                nxt = dms.config(c.width, c.length + 1)
                assert (nxt.reads if kind == "reads" else nxt.peak) > budget * (1 + 1e-9)
        lens = [c.length for c in fr]
        assert lens == sorted(lens, reverse=True)             # more chains, shorter chains
