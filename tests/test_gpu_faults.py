"""Failure handling, forced from the host; every kernel still exits normally.

- an undersized block pool raises the sticky DMS_ERR_OUT_OF_BLOCKS on the
  device (reported by stats, cleared by reset) while all accesses stay in
  bounds;
- argument, state and capacity errors are returned before anything is
  enqueued;
- a NaN logit means "not marked";
- reset returns the cache to a state equal to a fresh one.
"""

import numpy as np
import pytest
import torch

from synth import workloads as W

gpu = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _wl(**kw):
    base = dict(name="fault", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", window=4,
                decode_steps=8, seed=31, prompt_len=64, mu_before=[0.0])
    base.update(kw)
    return W.Workload(**base)


def _prompt(wl, lengths):
    import gpu_util as U
    return U.device_prompt(wl, 0, np.asarray(lengths))


@gpu
def test_pool_exhaustion_in_prefill_is_sticky_and_reset_clears_it():
    import gpu_util as U
    from learned_kv_cache_dms_amd import dms
    wl = _wl(prompt_len=200, mu_before=[-5.0])          # nothing marked: 200 visible tokens per unit
    c = U.make_cache(wl, pool_blocks=20)                 # 4 units x 13 blocks needed
    K, V, Lg = _prompt(wl, [200, 200])
    c.prefill(K, V, Lg, [200, 200])
    st = c.stats()
    assert st["sticky_error"] == dms.DMS_ERR_OUT_OF_BLOCKS
    assert st["allocated_blocks"] <= 20
    # appends and attention still run, in bounds
    pos = torch.tensor([200, 200], dtype=torch.int32, device="cuda")
    q, k, v, lg = U.device_step(wl, 0, pos)
    c.append(k, v, lg)
    c.attend(q)
    torch.cuda.synchronize()
    assert c.stats()["sticky_error"] == dms.DMS_ERR_OUT_OF_BLOCKS
    c.reset()
    st = c.stats()
    assert st["sticky_error"] == 0 and st["live_tokens"] == 0 and st["allocated_blocks"] == 0
    # after reset a prompt that fits works and matches the oracle
    K2, V2, Lg2 = _prompt(wl, [40, 40])
    c.prefill(K2, V2, Lg2, [40, 40])
    _, _, n = c.export()
    assert list(n) == [40, 40, 40, 40]


@gpu
def test_pool_exhaustion_during_decode():
    import gpu_util as U
    from learned_kv_cache_dms_amd import dms
    wl = _wl(prompt_len=32, mu_before=[-5.0], decode_steps=40)
    c = U.make_cache(wl, pool_blocks=8)                  # prompt uses exactly 2 blocks per unit
    K, V, Lg = _prompt(wl, [32, 32])
    c.prefill(K, V, Lg, [32, 32])
    assert c.stats()["sticky_error"] == 0
    pos = torch.tensor([32, 32], dtype=torch.int32, device="cuda")
    for t in range(20):
        q, k, v, lg = U.device_step(wl, 0, pos + t)
        c.append(k, v, lg)
        c.attend(q)
    torch.cuda.synchronize()
    st = c.stats()
    assert st["sticky_error"] == dms.DMS_ERR_OUT_OF_BLOCKS
    assert st["allocated_blocks"] == 8
    _, _, n = c.export()
    assert all(32 <= x <= 48 for x in n)


@gpu
def test_whole_unit_attention_with_units_left_empty():
    """1024 units, more than the resident work-groups (at most 2 per CU on 256
    CUs), so each unit is one work item, found directly by its position in
    the unit order.  An undersized pool leaves the units after the first that
    does not fit empty (n = 0) after the prompt; the unequal prompt lengths
    make the order length-balanced, so empty and full items alternate along
    the work-groups' items.  Full units match the oracle, an empty unit's
    output rows are left as they were."""
    import gpu_util as U
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    wl = _wl(batch=128, num_q_heads=40, num_kv_heads=8, prompt_len=80, mu_before=[-5.0])
    lengths = np.random.default_rng(5).integers(17, 81, size=wl.batch)
    need = int(sum((int(L) + 15) // 16 for L in lengths)) * wl.num_kv_heads
    c = U.make_cache(wl, pool_blocks=need // 2)
    K, V, Lg = _prompt(wl, lengths)
    c.prefill(K, V, Lg, lengths.tolist())
    assert c.stats()["sticky_error"] == dms.DMS_ERR_OUT_OF_BLOCKS
    q, _, _, _ = U.device_step(wl, 0, torch.tensor(lengths, dtype=torch.int32, device="cuda"))
    out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), 7.0, device="cuda")
    c.attend(q, out)
    # the timed call in whole-unit mode (its stop event on the attention launch itself)
    out_t = torch.full_like(out, 7.0)
    timer = dms.KernelTimer()
    c.attend_timed(q, timer, out_t)
    assert timer.elapsed_ms() > 0.0
    timer.close()
    torch.cuda.synchronize()
    assert torch.equal(out, out_t)
    _, _, n = c.export()
    G = wl.group
    full = [u for u in range(len(n)) if n[u] > 0]
    empty = [u for u in range(len(n)) if n[u] == 0]
    assert len(full) > 100 and len(empty) > 100, (len(full), len(empty))
    got = out.double().cpu().numpy()
    for u in empty:
        b, h = divmod(u, wl.num_kv_heads)
        assert np.all(got[b, h * G:(h + 1) * G] == 7.0), (b, h)
    rng = np.random.default_rng(6)
    for u in rng.choice(full, size=48, replace=False):
        b, h = divmod(int(u), wl.num_kv_heads)
        P = int(lengths[b])
        assert n[u] == P  # nothing marked: the whole prompt is live
        ud = U.host_unit(wl, 0, b, h, P, 1)
        ref = O.attend(ud.Q[0], ud.K[:P], ud.V[:P], O.default_scale(wl.head_dim))
        err = float(np.max(np.abs(got[b, h * G:(h + 1) * G] - ref)))
        assert err <= 1e-4, (b, h, err)


@gpu
def test_capacity_state_and_argument_errors():
    import gpu_util as U
    from learned_kv_cache_dms_amd import dms
    wl = _wl(prompt_len=10, decode_steps=2)
    c = U.make_cache(wl, max_tokens=12)
    pos = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    q, k, v, lg = U.device_step(wl, 0, pos)
    with pytest.raises(dms.DmsError) as e:
        c.attend(q)                                      # no token yet
    assert e.value.status == dms.DMS_ERR_STATE
    K, V, Lg = _prompt(wl, [10, 10])
    with pytest.raises(dms.DmsError) as e:
        c.prefill(K, V, Lg, [13, 10])                     # longer than the prompt tensor
    assert e.value.status == dms.DMS_ERR_ARG
    c.prefill(K, V, Lg, [10, 10])
    with pytest.raises(dms.DmsError) as e:
        c.prefill(K, V, Lg, [10, 10])                     # not empty
    assert e.value.status == dms.DMS_ERR_STATE
    c.append(k, v, lg)
    c.append(k, v, lg)
    with pytest.raises(dms.DmsError) as e:
        c.append(k, v, lg)                                # 13 > max_tokens
    assert e.value.status == dms.DMS_ERR_CAPACITY
    assert c.stats()["seen_tokens"] == 4 * 12
    with pytest.raises(ValueError):
        c.append(k.float(), v, lg)                        # dtype checked by the binding
    with pytest.raises(ValueError):
        c.attend(q[:, :4].contiguous())                   # shape checked by the binding
    L = dms.lib
    assert L.dms_append_step(c.handle, None, v.data_ptr(), lg.data_ptr(), None) == dms.DMS_ERR_ARG
    assert L.dms_decode_attention(c.handle, q.data_ptr(), None, None) == dms.DMS_ERR_ARG
    assert L.dms_cache_export(c.handle, 3, 2, None, None, None, None) == dms.DMS_ERR_ARG


@gpu
def test_nan_and_zero_logits_are_not_marked():
    import gpu_util as U
    wl = _wl(prompt_len=30, window=100)
    c = U.make_cache(wl)
    K, V, Lg = _prompt(wl, [30, 30])
    special = torch.tensor([float("nan"), 0.0, -0.0, 1e-30, -1e-30, float("inf"), float("-inf")],
                           device="cuda")
    Lg[:, :, :7] = special
    c.prefill(K, V, Lg, [30, 30])
    slot_pos, ring, n = c.export()
    for u in range(4):
        pend = set(slot_pos[u][ring[u][ring[u] >= 0]].tolist())
        assert 0 not in pend and 1 not in pend and 2 not in pend and 4 not in pend and 6 not in pend
        assert 3 in pend and 5 in pend                   # 1e-30 and +inf are > 0
        assert n[u] == 30


@gpu
def test_reset_equals_fresh_cache():
    import gpu_util as U
    wl = _wl(prompt_len=50, decode_steps=5, mu_before=[0.4])
    a = U.make_cache(wl)
    K, V, Lg = _prompt(wl, [50, 33])
    a.prefill(K, V, Lg, [50, 33])
    pos = torch.tensor([50, 33], dtype=torch.int32, device="cuda")
    for t in range(5):
        q, k, v, lg = U.device_step(wl, 0, pos + t)
        a.append(k, v, lg)
    a.reset()
    b = U.make_cache(wl)
    outs = []
    for c in (a, b):
        c.prefill(K, V, Lg, [50, 33])
        for t in range(5):
            q, k, v, lg = U.device_step(wl, 0, pos + t)
            c.append(k, v, lg)
            o = c.attend(q)
        outs.append((o.clone(), c.export()))
    assert torch.equal(outs[0][0], outs[1][0])
    for x, y in zip(outs[0][1], outs[1][1]):
        assert np.array_equal(x, y)


@gpu
def test_timed_attention_equals_untimed():
    """dms_decode_attention_timed gives the untimed call's results bit for bit
    and has the runtime stamp its events (a positive elapsed time); NULL
    events are argument errors.  4 units on many more work-groups: the units
    are split, so the stop event is bound to the split-merge launch."""
    import gpu_util as U
    from learned_kv_cache_dms_amd import dms
    wl = _wl(prompt_len=100, mu_before=[0.5])
    c = U.make_cache(wl)
    K, V, Lg = _prompt(wl, [100, 77])
    c.prefill(K, V, Lg, [100, 77])
    q, _, _, _ = U.device_step(wl, 0, torch.tensor([100, 77], dtype=torch.int32, device="cuda"))
    a = c.attend(q)
    timer = dms.KernelTimer()
    b = c.attend_timed(q, timer)
    assert timer.elapsed_ms() > 0.0
    assert torch.equal(a, b)
    with pytest.raises(dms.DmsError):
        dms.dms_decode_attention_timed(c.handle, q.data_ptr(), b.data_ptr(), 0, timer.stop.value)
    timer.close()


@gpu
def test_runs_on_a_non_default_stream():
    import gpu_util as U
    wl = _wl(prompt_len=60, decode_steps=3)
    K, V, Lg = _prompt(wl, [60, 60])
    pos = torch.tensor([60, 60], dtype=torch.int32, device="cuda")
    q, k, v, lg = U.device_step(wl, 0, pos)
    ref = U.make_cache(wl)
    ref.prefill(K, V, Lg, [60, 60])
    ref.append(k, v, lg)
    o_ref = ref.attend(q)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = U.make_cache(wl)
        c.prefill(K, V, Lg, [60, 60])
        c.append(k, v, lg)
        o = c.attend(q)
    s.synchronize()
    assert torch.equal(o, o_ref)
