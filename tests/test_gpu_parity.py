"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Live-slot sets, pending evictions and live counts must match bit for bit;
outputs within max-abs 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs), plus a
tighter 1e-4 bound for bf16 that follows from the kernel's arithmetic
(exact bf16 products, fp32 accumulation, softmax weights carried to about
16 bits by a hi + lo bf16 split).
"""
import dataclasses

import numpy as np
import pytest
import torch

from synth import workloads as W

gpu = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
TIGHT = {"f32": 1e-5, "bf16": 1e-4}


def _tol(wl):
    return min(TOL[wl.dtype], TIGHT[wl.dtype])


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util  # noqa: F401  (imports the HIP libraries; fails loudly if unbuilt)


@gpu
def test_tiny_every_step_every_unit():
    """1 sequence, 12 Q / 2 KV heads, d=128, fp32, 256-token prompt, 256
    decode steps, w=16, logits N(0,1): every unit, every step."""
    import gpu_util as U
    wl = W.tiny()
    st = U.run_decode(wl, wl.decode_steps, [(0, 0), (0, 1)], TOL["f32"])
    assert st.checks == 2 * wl.decode_steps


def _small(name, **kw):
    base = dict(name=name, batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", window=8,
                decode_steps=48, seed=77, prompt_len=40, mu_before=[0.3])
    base.update(kw)
    return W.Workload(**base)


SMALL = [
    _small("bf16-d128-g4-w8"),
    _small("bf16-d64-g4-w8", head_dim=64),
    _small("f32-d64-g1-w3", dtype="f32", head_dim=64, num_q_heads=2, window=3),
    _small("f32-d128-g6-w0", dtype="f32", num_q_heads=12, window=0, mu_before=[1.0]),
    _small("bf16-d128-g5-w0-allmarked", num_q_heads=10, window=0, mu_before=[8.0]),
    _small("bf16-d128-g7-unmarked", num_q_heads=14, mu_before=[-8.0]),
    _small("bf16-d128-g16-w32", num_q_heads=32, window=32, mu_before=[1.5]),
    _small("bf16-d64-g8-ragged", head_dim=64, num_q_heads=16, lengths_range=(0, 90), batch=5),
    _small("f32-d128-g2-ragged", dtype="f32", num_q_heads=4, lengths_range=(1, 70), batch=4, window=5),
    _small("bf16-d128-g4-window-ge-context", window=500),
    _small("bf16-d128-g4-tiny-prompt", prompt_len=1, decode_steps=70),
    _small("bf16-d128-g6-position-threshold", num_q_heads=12, prompt_len=60, mu_before=[-1.0],
           mu_after=[2.0], pos_threshold=70),
]


@gpu
@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_small_shapes_every_unit(wl):
    import gpu_util as U
    units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    U.run_decode(wl, wl.decode_steps, units, _tol(wl))


@gpu
def test_split_invariance():
    """Whole units versus the default split by live blocks (fp32)."""
    import gpu_util as U
    wl = _small("f32-split", dtype="f32", batch=2, prompt_len=700, decode_steps=4, mu_before=[-0.5],
                window=16)
    outs = []
    for split_wgs in (1, 0):
        c = U.make_cache(wl, split_wgs=split_wgs)
        lengths = wl.prompt_lengths()
        K, V, Lg = U.device_prompt(wl, 0, lengths)
        c.prefill(K, V, Lg, lengths)
        pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        q, k, v, lg = U.device_step(wl, 0, pos)
        c.append(k, v, lg)
        outs.append(c.attend(q).double().cpu())
    assert float((outs[0] - outs[1]).abs().max()) <= 1e-6


@gpu
@pytest.mark.parametrize("blocks", [28, 308], ids=["7-per-wave", "77-per-wave"])
def test_visit_order_strides(blocks):
    """Each of the attention's four waves walks its blocks of an item at a
    stride coprime to their count: 7, else 11, else 13.  Whole units
    (split_wgs 1) and nothing evicted (logits far below 0), so at the first
    step every wave holds exactly blocks / 4 blocks: 7 (stride 11) or 77
    (stride 13).  Every unit, every step, against the oracle."""
    import gpu_util as U
    wl = _small(f"f32-d64-{blocks}-blocks", dtype="f32", head_dim=64, batch=2, num_q_heads=4, num_kv_heads=2,
                window=8, decode_steps=3, prompt_len=blocks * 16 - 1, mu_before=[-8.0])
    units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    st = U.run_decode(wl, wl.decode_steps, units, TOL["f32"], cache=U.make_cache(wl, split_wgs=1))
    assert st.checks == len(units) * wl.decode_steps


@gpu
def test_whole_units_long_runs():
    """512 units (at least one per resident work-group): each unit is one work
    item, never split, and no split merge runs.  Nothing is evicted (logits
    far below 0), so each unit holds 8320 tokens = 520 blocks and every wave
    walks 130 of them (more than 128, with the visit stride of its count).
    Sampled units at every step against the oracle."""
    import gpu_util as U
    wl = _small("bf16-d64-512-units-520-blocks", head_dim=64, batch=64, num_q_heads=8, num_kv_heads=8,
                window=16, decode_steps=2, prompt_len=520 * 16 - 1, mu_before=[-8.0])
    units = [(0, 0), (17, 3), (40, 5), (63, 7)]
    st = U.run_decode(wl, wl.decode_steps, units, _tol(wl))
    assert st.checks == len(units) * wl.decode_steps


@gpu
@pytest.mark.parametrize("batch", [512, 520], ids=["4096-units", "4160-units"])
def test_many_units(batch):
    """As many (sequence, KV head) units as the split mode plans for (4096),
    and more (whole units only).  Ragged prompts of 1-120 tokens, dealt to
    the work-groups by length; sampled units, the first and the last among
    them, checked at every step."""
    import gpu_util as U
    wl = _small(f"bf16-d64-{batch}x8-units", head_dim=64, batch=batch, num_q_heads=16, num_kv_heads=8, window=8,
                decode_steps=6, lengths_range=(1, 120))
    rng = np.random.default_rng(batch)
    units = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, batch, 10), rng.integers(0, 8, 10))}
                   | {(0, 0), (batch - 1, 7)})
    st = U.run_decode(wl, wl.decode_steps, units, _tol(wl))
    assert st.checks == len(units) * wl.decode_steps


@gpu
def test_prefill_equals_appends():
    """A compressed prompt leaves exactly the state of one append per token."""
    import gpu_util as U
    wl = _small("prefill-eq", batch=2, prompt_len=150, decode_steps=1, window=12, mu_before=[0.5])
    lengths = np.array([150, 97])
    a = U.make_cache(wl)
    b = U.make_cache(wl)
    K, V, Lg = U.device_prompt(wl, 0, lengths)
    a.prefill(K, V, Lg, lengths)
    # b: empty prompt, then appends; sequence 1 appends only its first 97 positions
    # (then padding appends at the same positions would diverge), so compare units
    # of sequence 0 fully and sequence 1 by running a separate one-sequence cache.
    b.prefill(K, V, Lg, [0, 0])
    for t in range(150):
        k = K[:, :, t].contiguous()
        v = V[:, :, t].contiguous()
        lg = Lg[:, :, t].contiguous()
        b.append(k, v, lg)
    sa, ra, na = a.export(0, 2)
    sb, rb, nb = b.export(0, 2)
    assert np.array_equal(na, nb)
    for u in range(2):
        # slots are a permutation (appends reuse retired slots); the logical
        # state is the set of live positions and the pending ones by ring entry
        assert np.array_equal(np.sort(sa[u][sa[u] >= 0]), np.sort(sb[u][sb[u] >= 0]))
        pa = np.where(ra[u] >= 0, sa[u][np.maximum(ra[u], 0)], -1)
        pb = np.where(rb[u] >= 0, sb[u][np.maximum(rb[u], 0)], -1)
        assert np.array_equal(pa, pb)
    pos = torch.tensor([150, 150], dtype=torch.int32, device="cuda")
    q, _, _, _ = U.device_step(wl, 0, pos)
    # attention of sequence 0 must agree (same visible set; the slots hold it in
    # another order, so fp32 sums differ by rounding order only)
    oa = a.attend(q)
    ob = b.attend(q)
    assert float((oa[0] - ob[0]).abs().max()) <= 1e-5


@gpu
def test_needles():
    """A key aligned with the query at an evicted position must not move the
    output; at a visible position it must dominate it."""
    import gpu_util as U
    from oracle import dms_oracle as O
    wl = _small("needle", batch=1, num_q_heads=4, num_kv_heads=1, prompt_len=120, decode_steps=1,
                window=4, mu_before=[0.0])
    lengths = wl.prompt_lengths()
    K, V, Lg = U.device_prompt(wl, 0, lengths)
    Lg[0, 0, :] = torch.where(torch.arange(120, device="cuda") % 2 == 0, 1.0, -1.0)
    pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    q, k, v, lg = U.device_step(wl, 0, pos)
    lg.fill_(-1.0)
    qv = q[0, 0].float()
    needle = (40.0 * qv / qv.norm() * (wl.head_dim ** 0.5)).to(K.dtype)

    def run(Kx):
        c = U.make_cache(wl)
        c.prefill(Kx, V, Lg, lengths)
        c.append(k, v, lg)
        return c.attend(q).double().cpu()

    alpha = np.where(np.arange(121) % 2 == 0, True, False)
    alpha[120] = False
    vis = O.visible(alpha, 120, wl.window)
    base = run(K)
    ev = 20
    assert ev not in set(vis)
    K2 = K.clone()
    K2[0, 0, ev] = needle
    assert float((run(K2) - base).abs().max()) == 0.0
    lv = 21
    assert lv in set(vis)
    K3 = K.clone()
    K3[0, 0, lv] = needle
    o3 = run(K3)
    assert float((o3[0, 0] - V[0, 0, lv].double().cpu()).abs().max()) < 1e-3


@gpu
@pytest.mark.parametrize("wl_fn", [W.llama_1b, W.qwen_7b, W.qwen_32b], ids=lambda f: f().name)
def test_full_size_sampled_units(wl_fn):
    """Full-size layer workloads: every decode step, sampled (sequence, KV
    head) units compared with the oracle; all units' live counts checked
    at the last step."""
    import gpu_util as U
    from oracle import dms_oracle as O
    from synth import synth
    wl = wl_fn()
    rng = np.random.default_rng(wl.seed)
    U_ = wl.batch * wl.num_kv_heads
    picks = sorted(set([0, U_ - 1] + list(rng.choice(U_, 2, replace=False))))
    units = [(u // wl.num_kv_heads, u % wl.num_kv_heads) for u in picks]
    cache = U.make_cache(wl)
    st = U.run_decode(wl, wl.decode_steps, units, _tol(wl), cache=cache)
    assert st.checks == len(units) * wl.decode_steps
    # live counts of every unit after the last step
    q = wl.prompt_len + wl.decode_steps - 1
    lg = synth.logits(wl.seed, 0, np.arange(wl.batch), wl.num_kv_heads, np.arange(q + 1),
                      *wl.layer_mu(0), wl.pos_threshold)
    _, _, n = cache.export(0, U_)
    ref = np.array([len(O.visible(O.eviction_decision(lg[b, h]), q, wl.window))
                    for b in range(wl.batch) for h in range(wl.num_kv_heads)])
    assert np.array_equal(n, ref)


@gpu
def test_dense_full_size_sampled_units():
    """The dense baseline shape (Qwen-R1-32B-shaped layer with every logit
    below 0): nothing is evicted, every unit holds all 32768 + t tokens (2064
    blocks, 516 per wave in one work item) and the output is plain causal
    attention.  Sampled units against the oracle at every one of 32 steps,
    and every unit's live count = its position + 1."""
    import dataclasses
    import gpu_util as U
    wl = dataclasses.replace(W.qwen_32b_dense(), decode_steps=32)
    U_ = wl.batch * wl.num_kv_heads
    units = [(0, 0), (21, 5), (63, 7)]
    cache = U.make_cache(wl)
    st = U.run_decode(wl, wl.decode_steps, units, _tol(wl), cache=cache)
    assert st.checks == len(units) * wl.decode_steps
    _, _, n = cache.export(0, U_)
    assert np.all(n == wl.prompt_len + wl.decode_steps)

