"""GPU parity of the decode step (dms_decode_step) and of the attention's
work split (whole units, split by live blocks, dms_cache_balance), through
the C ABI against the CPU oracle.

Live-slot sets, pending evictions and live counts bit for bit after every
step; outputs within the tolerances of test_gpu_parity.  The fused step
computes the new token's score on the VALU instead of the matrix cores, so
it agrees with the two-call path to rounding, not bit for bit; its cache
state after every step is bit-identical to theirs.
"""
import dataclasses

import numpy as np
import pytest
import torch

from synth import workloads as W
from test_gpu_parity import SMALL, TOL, _small, _tol

gpu = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util  # noqa: F401  (imports the HIP libraries; fails loudly if unbuilt)


def _all_units(wl):
    return [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]


@gpu
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_fused_step_every_unit(wl):
    """The fused single-launch step (whole units forced: split_wgs 1) on the
    12 small shapes: every unit, every step against the oracle."""
    import gpu_util as U
    st = U.run_decode(wl, wl.decode_steps, _all_units(wl), _tol(wl), mode="step",
                      cache=U.make_cache(wl, split_wgs=1))
    assert st.checks == len(_all_units(wl)) * wl.decode_steps


@gpu
@pytest.mark.parametrize("wl", SMALL[:6], ids=lambda w: w.name)
def test_split_step_every_unit(wl):
    """The step in split mode (fewer units than work-groups: append, the
    attention over equal shares of live blocks, the split merge): every unit,
    every step."""
    import gpu_util as U
    st = U.run_decode(wl, wl.decode_steps, _all_units(wl), _tol(wl), mode="step")
    assert st.checks == len(_all_units(wl)) * wl.decode_steps


@gpu
@pytest.mark.parametrize("split_wgs", [2, 3, 7, 40, 512, 1])
def test_split_shares(split_wgs):
    """One shape, the live blocks split over 2 ... 512 work-groups (pieces cut
    anywhere inside units, several units per work-group, single blocks per
    work-group) and whole units (1): every unit, every step, fp32."""
    import gpu_util as U
    wl = _small(f"f32-split-{split_wgs}", dtype="f32", batch=5, num_q_heads=8, num_kv_heads=2,
                lengths_range=(1, 700), decode_steps=6, mu_before=[0.2], window=16)
    st = U.run_decode(wl, wl.decode_steps, _all_units(wl), TOL["f32"], cache=U.make_cache(wl, split_wgs=split_wgs))
    assert st.checks == len(_all_units(wl)) * wl.decode_steps


@gpu
def test_step_state_equals_calls():
    """dms_decode_step and dms_append_step + dms_decode_attention side by side
    on the same inputs: the exported state is identical after every step and
    the outputs agree to rounding, in whole-unit and in split mode."""
    import gpu_util as U
    wl = _small("bf16-d128-g5-ragged", num_q_heads=10, batch=4, lengths_range=(0, 90), decode_steps=40,
                mu_before=[0.6], window=12)
    lengths = wl.prompt_lengths()
    for split_wgs in (1, 5):
        a = U.make_cache(wl, split_wgs=split_wgs)
        b = U.make_cache(wl, split_wgs=split_wgs)
        K, V, Lg = U.device_prompt(wl, 0, lengths)
        a.prefill(K, V, Lg, lengths)
        b.prefill(K, V, Lg, lengths)
        pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        worst = 0.0
        for t in range(wl.decode_steps):
            q, k, v, lg = U.device_step(wl, 0, pos + t)
            oa = a.step(q, k, v, lg)
            b.append(k, v, lg)
            ob = b.attend(q)
            torch.cuda.synchronize()
            worst = max(worst, float((oa - ob).abs().max()))
            for x, y in zip(a.export(), b.export()):
                assert np.array_equal(x, y), (split_wgs, t)
        assert worst <= 1e-5, (split_wgs, worst)
        assert a.stats() == b.stats()


@gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_from_empty_cache(dtype):
    """Decode steps with no prompt: the first step's output is the new
    token's value row (its only visible token), exactly; then every unit,
    every step against the oracle, in both modes."""
    import gpu_util as U
    wl = _small(f"{dtype}-empty-prompt", dtype=dtype, batch=3, prompt_len=0, decode_steps=30, window=4)
    for split_wgs in (1, 0):
        c = U.make_cache(wl, split_wgs=split_wgs)
        q, k, v, lg = U.device_step(wl, 0, torch.zeros(wl.batch, dtype=torch.int32, device="cuda"))
        out = c.step(q, k, v, lg)
        torch.cuda.synchronize()
        G = wl.group
        want = v.float().repeat_interleave(G, dim=1)
        assert torch.equal(out, want), split_wgs
        st = U.run_decode(wl, wl.decode_steps, _all_units(wl), _tol(wl), mode="step",
                          cache=U.make_cache(wl, split_wgs=split_wgs))
        assert st.checks == len(_all_units(wl)) * wl.decode_steps


@gpu
def test_step_logit_channel():
    """dms_decode_step_channel (logit in a zeroed key channel, and in the
    group's first query head) equals dms_append_step_channel + attention."""
    import gpu_util as U
    wl = _small("bf16-channel-step", batch=4, num_q_heads=8, prompt_len=50, decode_steps=20, mu_before=[0.5])
    lengths = wl.prompt_lengths()
    for source, zero in (("k", True), ("q", False)):
        a = U.make_cache(wl, split_wgs=1)
        b = U.make_cache(wl, split_wgs=1)
        K, V, _ = U.device_prompt(wl, 0, lengths)
        if source == "k":
            a.prefill_channel(K, V, lengths, source="k", channel=3, zero=True)
            b.prefill_channel(K, V, lengths, source="k", channel=3, zero=True)
        else:
            Qp = torch.randn((wl.batch, wl.num_q_heads, K.shape[2], wl.head_dim), device="cuda").to(K.dtype)
            a.prefill_channel(K, V, lengths, source="q", channel=5, q=Qp)
            b.prefill_channel(K, V, lengths, source="q", channel=5, q=Qp)
        pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        ch = 3 if source == "k" else 5
        worst = 0.0
        for t in range(wl.decode_steps):
            q, k, v, _ = U.device_step(wl, 0, pos + t)
            oa = a.step_channel(q, k, v, source=source, channel=ch, zero=zero)
            b.append_channel(k, v, source=source, channel=ch, zero=zero, q=q if source == "q" else None)
            ob = b.attend(q)
            torch.cuda.synchronize()
            worst = max(worst, float((oa - ob).abs().max()))
            for x, y in zip(a.export(), b.export()):
                assert np.array_equal(x, y), (source, t)
        assert worst <= 1e-5, (source, worst)


def _skew_small(batch, steps=6):
    """A layer with per-head compression 2 ... 16 (the head-skew recipe) at a
    small size: per-head live counts differ several-fold."""
    w = W.qwen_32b_head_skew()
    return dataclasses.replace(w, name=f"head-skew-b{batch}", batch=batch, prompt_len=2048, decode_steps=steps,
                               head_mu=list(w.head_mu))


@gpu
@pytest.mark.parametrize("batch,mode", [(8, "calls"), (8, "step"), (160, "step"), (160, "calls")])
def test_balance_head_skew(batch, mode):
    """Per-head CR 2 ... 16: dms_cache_balance picks split mode for 64 units
    (fewer than the work-groups; the CR-2 head's units, one work-group each,
    would take longer than the split) and deals 1280 units whole or split by how
    evenly they pack; every plan gives the oracle's results.  Sampled units
    (every KV head) at every step."""
    import gpu_util as U
    wl = _skew_small(batch)
    rng = np.random.default_rng(batch)
    units = [(int(rng.integers(0, batch)), h) for h in range(wl.num_kv_heads)]
    st = U.run_decode(wl, wl.decode_steps, units, _tol(wl), mode=mode, balance=True)
    assert st.checks == len(units) * wl.decode_steps


@gpu
def test_balance_mode_for_few_units():
    """With fewer (sequence, KV head)s than work-groups, dms_cache_balance
    gives each its own work-group when the units are alike (the
    Llama-3.2-1B-shaped layer: 64 units of about 80 live blocks; the
    Qwen-R1-7B-shaped layer: 128 units of about 143, both at full size, as
    the bench times them) and splits when one head keeps several times the
    others' tokens (per-head CR 2 ... 16, 64 units); every plan gives the
    oracle's results."""
    import gpu_util as U
    for wl, want in ((W.llama_1b(), 0), (W.qwen_7b(), 0), (_skew_small(8), 1)):
        wl = dataclasses.replace(wl, decode_steps=3)
        c = U.make_cache(wl)
        units = [(0, h) for h in range(wl.num_kv_heads)]
        st = U.run_decode(wl, wl.decode_steps, units, _tol(wl), mode="step", balance=True, cache=c)
        assert st.checks == len(units) * wl.decode_steps
        assert c.stats()["split_mode"] == want, wl.name


@gpu
def test_head_skew_full_size():
    """The head-skew workload at full size (64 chains x 32768 tokens, per-head
    CR 2 ... 16) after dms_cache_balance (split mode): sampled units of every
    KV head through 3 fused steps, and every unit's live count against the
    rule."""
    import gpu_util as U
    from oracle import dms_oracle as O
    from synth import synth
    wl = dataclasses.replace(W.qwen_32b_head_skew(), decode_steps=3)
    units = [(0, h) for h in range(8)] + [(63, 0), (31, 7)]
    c = U.make_cache(wl)
    st = U.run_decode(wl, wl.decode_steps, units, _tol(wl), mode="step", balance=True, cache=c)
    assert st.checks == len(units) * wl.decode_steps
    _, _, n = c.export()
    P = wl.prompt_len
    q = P + wl.decode_steps - 1
    for h in range(wl.num_kv_heads):
        lg = synth.logits(wl.seed, 0, np.arange(wl.batch), [h], np.arange(q + 1), *wl.layer_mu(0),
                          wl.pos_threshold)[:, 0]
        want = [len(O.visible(O.eviction_decision(lg[b]), q, wl.window)) for b in range(wl.batch)]
        got = [int(n[b * wl.num_kv_heads + h]) for b in range(wl.batch)]
        assert got == want, h
