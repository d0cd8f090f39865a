"""The 64-layer Qwen-R1-32B-shaped decode step at full size: 64 layers x
(256 chains, 40 Q / 8 KV heads, head_dim 128, bf16), prompt lengths uniform
in [1024, 32768], w = 256, per-layer CR rising from 4 to 12, 128 decode
steps.  One DMS cache per layer, block pools sized from the expected live
counts (about 200 GB of HBM in all).  Each decode step runs append +
attention for every layer in order, as a model would.

Checked against the oracle: sampled (layer, sequence, KV head) units at
sampled steps (visible sets, pending evictions, outputs), and the live
counts of every unit of one layer after the last step.
"""
import time

import numpy as np
import pytest
import torch

from synth import workloads as W

gpu = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@gpu
def test_full_64_layer_step_sampled_parity():
    import gpu_util as U
    from oracle import dms_oracle as O
    from synth import synth

    wl = W.full_32b()
    steps = wl.decode_steps
    lengths = wl.prompt_lengths()
    layers = list(range(wl.num_layers))
    check_layers = [0, 21, 42, 63]
    check_steps = {0, 1, steps // 2, steps - 1}
    rng = np.random.default_rng(7)
    Uc = wl.batch * wl.num_kv_heads
    units = {l: [(int(u) // wl.num_kv_heads, int(u) % wl.num_kv_heads)
                 for u in rng.choice(Uc, 2, replace=False)] for l in check_layers}
    t0 = time.time()
    caches = []
    for l in layers:
        c = U.make_cache(wl, layer=l, pool_blocks=wl.pool_blocks(l, slack=1.1))
        K, V, Lg = U.device_prompt(wl, l, lengths)
        c.prefill(K, V, Lg, lengths)
        del K, V, Lg
        caches.append(c)
        if l % 16 == 0:
            torch.cuda.synchronize()
            U.log(f"layer {l} prefilled ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    host = {(l, bh): U.host_unit(wl, l, bh[0], bh[1], int(lengths[bh[0]]), steps)
            for l in check_layers for bh in units[l]}
    U.log(f"host data ready ({time.time() - t0:.1f} s)")
    pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    st = U.CompareStats()
    for t in range(steps):
        outs = {}
        for l in layers:
            q, k, v, lg = U.device_step(wl, l, pos + t)
            caches[l].append(k, v, lg)
            o = caches[l].attend(q)
            if t in check_steps and l in check_layers:
                outs[l] = o
        if t in check_steps:
            torch.cuda.synchronize()
            for l in check_layers:
                for bh in units[l]:
                    U.check_unit_step(caches[l], wl, host[(l, bh)], t, outs[l], 1e-4, st)
    for l, c in enumerate(caches):
        s = c.stats()
        assert s["sticky_error"] == 0, (l, s)
    U.log(f"decode done ({time.time() - t0:.1f} s), checks={st.checks}, max_err={st.max_err:.2e}")
    # live counts of every unit of layer 63 after the last step
    l = 63
    _, _, n = caches[l].export(0, Uc)
    mb, _ = wl.layer_mu(l)
    for b in range(wl.batch):
        q = int(lengths[b]) + steps - 1
        lg = synth.logits(wl.seed, l, [b], wl.num_kv_heads, np.arange(q + 1), mb)[0]
        for h in range(wl.num_kv_heads):
            assert n[b * wl.num_kv_heads + h] == len(O.visible(O.eviction_decision(lg[h]), q, wl.window))
    assert st.checks == len(check_steps) * sum(len(units[l]) for l in check_layers)
