"""GPU parity of the eviction logit read from a repurposed projection channel
(dms_append_step_channel, dms_prefill_compress_channel) against the oracle's
``decode_batch_channel``: visible and pending sets bit-exact at every step,
outputs within the same bounds as the other parity tests."""
import numpy as np
import pytest
import torch

from synth import synth

gpu = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util  # noqa: F401  (imports the HIP libraries; fails loudly if unbuilt)


def _inputs(seed, B, Hq, Hkv, T, d, dtype):
    """Host Q [B,Hq,T,d], K, V [B,Hkv,T,d] from the seeded generator (values
    exact in the element type)."""
    pos = np.arange(T)
    Q = synth.tensor(seed, synth.STREAM_Q, 0, np.arange(B), np.arange(Hq), pos, d, dtype)
    K = synth.tensor(seed, synth.STREAM_K, 0, np.arange(B), np.arange(Hkv), pos, d, dtype)
    V = synth.tensor(seed, synth.STREAM_V, 0, np.arange(B), np.arange(Hkv), pos, d, dtype)
    return Q, K, V


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(
        device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


CASES = [
    # id, dtype, d, source, zero, channel
    ("bf16-d128-k-zero-ch0", "bf16", 128, "k", True, 0),
    ("bf16-d128-k-keep-ch77", "bf16", 128, "k", False, 77),
    ("f32-d64-k-zero-ch63", "f32", 64, "k", True, 63),
    ("bf16-d64-q-ch5", "bf16", 64, "q", False, 5),
    ("f32-d128-q-ch127", "f32", 128, "q", False, 127),
]


@gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_channel_logits_match_oracle(case):
    """Ragged prompts prefilled through the channel variant, then 40 decode
    steps of channel appends; every unit against the oracle at every step."""
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    name, dtype, d, source, zero, ch = case
    B, Hq, Hkv, w, steps = 3, 8, 2, 6, 40
    P = np.array([37, 20, 1])
    T = int(P.max()) + steps
    Q, K, V = _inputs(4000 + d + ch, B, Hq, Hkv, T, d, dtype)
    print(f"[{name}] B={B} Hq={Hq} Hkv={Hkv} d={d} source={source} zero={zero} channel={ch}", flush=True)
    ref = O.decode_batch_channel(Q, K, V, P, steps, w, source, ch, zero)
    cache = dms.Cache(B, Hq, Hkv, d, w, T, 64, dtype=dtype)
    Kd, Vd, Qd = _dev(K, dtype), _dev(V, dtype), _dev(Q, dtype)
    cache.prefill_channel(Kd, Vd, P, source=source, channel=ch, zero=zero,
                          q=Qd if source == "q" else None)
    tol = TOL[dtype]
    bidx = torch.arange(B, device="cuda")
    for t in range(steps):
        at = torch.tensor(P + t, device="cuda")
        k = Kd[bidx, :, at].contiguous()
        v = Vd[bidx, :, at].contiguous()
        q = Qd[bidx, :, at].contiguous()
        cache.append_channel(k, v, source=source, channel=ch, zero=zero, q=q if source == "q" else None)
        out = cache.attend(q)
        torch.cuda.synchronize()
        sp, rg, n = cache.export(0, B * Hkv)
        got = out.double().cpu().numpy()
        for b in range(B):
            for h in range(Hkv):
                rec = ref["records"][(b, h)][t]
                u = b * Hkv + h
                assert n[u] == len(rec.visible), (name, t, b, h)
                assert np.array_equal(np.sort(sp[u][sp[u] >= 0]), rec.visible), (name, t, b, h)
                assert np.array_equal(np.sort(sp[u][rg[u][rg[u] >= 0]]), rec.pending), (name, t, b, h)
        err = float(np.max(np.abs(got - ref["out"][t])))
        assert err <= tol, (name, t, err)
    # the zeroed channel never reached the pool: it cannot change any output,
    # which the oracle (keys with the channel zeroed) already confirmed above


@gpu
def test_channel_path_equals_array_path():
    """Key-channel logits (no zeroing) leave the same state and outputs, bit
    for bit, as the plain path given that channel as its logit array."""
    from learned_kv_cache_dms_amd import dms
    dtype, d, ch = "bf16", 128, 9
    B, Hq, Hkv, w, steps = 4, 10, 2, 5, 24
    P = np.array([50, 31, 8, 64])
    T = int(P.max()) + steps
    Q, K, V = _inputs(4100, B, Hq, Hkv, T, d, dtype)
    Kd, Vd, Qd = _dev(K, dtype), _dev(V, dtype), _dev(Q, dtype)
    a = dms.Cache(B, Hq, Hkv, d, w, T, 64, dtype=dtype)
    b_ = dms.Cache(B, Hq, Hkv, d, w, T, 64, dtype=dtype)
    a.prefill_channel(Kd, Vd, P, source="k", channel=ch)
    b_.prefill(Kd, Vd, Kd[..., ch].float().contiguous(), P)
    bidx = torch.arange(B, device="cuda")
    for t in range(steps):
        at = torch.tensor(P + t, device="cuda")
        k = Kd[bidx, :, at].contiguous()
        v = Vd[bidx, :, at].contiguous()
        q = Qd[bidx, :, at].contiguous()
        a.append_channel(k, v, source="k", channel=ch)
        b_.append(k, v, k[..., ch].float().contiguous())
        oa, ob = a.attend(q), b_.attend(q)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), t
    for x, y in zip(a.export(), b_.export()):
        assert np.array_equal(x, y)


@gpu
def test_channel_argument_errors():
    """Bad sources, channels and combinations are argument errors, reported
    before anything is enqueued (the cache stays usable)."""
    from learned_kv_cache_dms_amd import dms
    B, Hq, Hkv, d = 2, 4, 2, 64
    c = dms.Cache(B, Hq, Hkv, d, 4, 32, 16, dtype="bf16")
    k = torch.zeros((B, Hkv, d), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    h, s = c.handle, c._stream()
    bad = [
        (k.data_ptr(), k.data_ptr(), None, dms.DMS_LOGIT_FROM_K, d, 0),      # channel out of range
        (k.data_ptr(), k.data_ptr(), None, dms.DMS_LOGIT_FROM_K, -1, 0),
        (k.data_ptr(), k.data_ptr(), None, dms.DMS_LOGIT_FROM_Q, 0, 0),      # no queries
        (k.data_ptr(), k.data_ptr(), q.data_ptr(), dms.DMS_LOGIT_FROM_Q, 0, 1),  # zeroing a query channel
        (k.data_ptr(), k.data_ptr(), q.data_ptr(), 7, 0, 0),                 # unknown source
    ]
    for args in bad:
        with pytest.raises(dms.DmsError) as e:
            dms.dms_append_step_channel(h, *args, stream=s)
        assert e.value.status == dms.DMS_ERR_ARG, args
        with pytest.raises(dms.DmsError) as e:
            dms.dms_prefill_compress_channel(h, *args, lengths=[1, 1], max_len=1, stream=s)
        assert e.value.status == dms.DMS_ERR_ARG, args
    c.append_channel(k, k, source="k", channel=3, zero=True)
    st = c.stats()
    assert st["seen_tokens"] == B * Hkv and st["sticky_error"] == 0


@gpu
def test_key_channel_full_size_sampled_units():
    """The Qwen-R1-32B-shaped layer at full size (64 x 32768-token prompts):
    the workload's logits, rounded to bf16, planted in key channel 77 and read
    from there by the prompt compression and 8 appends, with that channel
    stored as 0.  Sampled units at every step against the oracle on the same
    logits and the channel-zeroed keys; every unit's live count at the end."""
    import dataclasses
    import gpu_util as U
    from oracle import dms_oracle as O
    from synth import workloads as W
    ch = 77
    wl = dataclasses.replace(W.qwen_32b(), decode_steps=8)
    B, Hkv = wl.batch, wl.num_kv_heads
    lengths = wl.prompt_lengths()
    cache = U.make_cache(wl)
    K, V, Lg = U.device_prompt(wl, 0, lengths)
    K[..., ch] = Lg.to(torch.bfloat16)
    print(f"[qwen-32b key channel {ch}] prefill", flush=True)
    cache.prefill_channel(K, V, lengths, source="k", channel=ch, zero=True)
    del K, V, Lg
    rng = np.random.default_rng(wl.seed + 2)
    n_units = B * Hkv
    picks = sorted(set([0, n_units - 1] + list(rng.choice(n_units, 2, replace=False))))
    units = [(u // Hkv, u % Hkv) for u in picks]
    host = {}
    for (b, h) in units:
        ud = U.host_unit(wl, 0, b, h, int(lengths[b]), wl.decode_steps)
        lg16 = synth.round_bf16(ud.logit)          # the logit as the channel holds it
        Kz = ud.K.copy()
        Kz[:, ch] = 0.0                            # the channel is stored as 0
        host[(b, h)] = dataclasses.replace(ud, K=Kz, logit=lg16)
    st = U.CompareStats()
    pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    for t in range(wl.decode_steps):
        q, k, v, lg = U.device_step(wl, 0, pos + t)
        k[..., ch] = lg.to(torch.bfloat16)
        cache.append_channel(k, v, source="k", channel=ch, zero=True)
        out = cache.attend(q)
        torch.cuda.synchronize()
        for key in units:
            U.check_unit_step(cache, wl, host[key], t, out, TOL["bf16"], st)
    assert cache.stats()["sticky_error"] == 0
    qlast = wl.prompt_len + wl.decode_steps - 1
    mb, ma = wl.layer_mu(0)
    lgh = synth.round_bf16(synth.logits(wl.seed, 0, np.arange(B), Hkv, np.arange(qlast + 1), mb, ma,
                                        wl.pos_threshold))
    _, _, n = cache.export(0, n_units)
    ref_n = np.array([len(O.visible(O.eviction_decision(lgh[b, h]), qlast, wl.window))
                      for b in range(B) for h in range(Hkv)])
    assert np.array_equal(n, ref_n)
    print(f"  checks={st.checks} max_err={st.max_err:.2e}", flush=True)
