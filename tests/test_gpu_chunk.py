"""GPU parity of dms_decode_chunk (several decode steps per call) against the
oracle's step-by-step decode, and against the GPU's own one-token path:
visible and pending sets bit-exact after every chunk, every output row of
every chunk within the parity bounds."""
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


def _host(seed, B, Hq, Hkv, T, d, dtype, mu):
    pos = np.arange(T)
    Q = synth.tensor(seed, synth.STREAM_Q, 0, np.arange(B), np.arange(Hq), pos, d, dtype)
    K = synth.tensor(seed, synth.STREAM_K, 0, np.arange(B), np.arange(Hkv), pos, d, dtype)
    V = synth.tensor(seed, synth.STREAM_V, 0, np.arange(B), np.arange(Hkv), pos, d, dtype)
    lg = synth.logits(seed, 0, np.arange(B), np.arange(Hkv), pos, mu)
    return Q, K, V, lg


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def _slices(X, P, t0, C):
    """[B, H, C, ...] rows at positions P_b + t0 .. P_b + t0 + C - 1 of each sequence."""
    return np.stack([X[b][:, P[b] + t0:P[b] + t0 + C] for b in range(len(P))])


CASES = [
    # id, B, Hq, Hkv, d, dtype, w, P, mu, chunks
    ("bf16-d128-g4-w8", 3, 8, 2, 128, "bf16", 8, [40, 23, 1], 0.3, [1, 3, 16, 40, 5]),
    ("f32-d64-g1-w3", 2, 2, 2, 64, "f32", 3, [30, 9], 0.0, [4, 1, 17, 2]),
    ("bf16-d64-g8-w0-mostly-marked", 2, 16, 2, 64, "bf16", 0, [50, 33], 1.5, [7, 9, 2]),
    ("bf16-d128-g16-two-column-tiles", 1, 16, 1, 128, "bf16", 12, [70], 0.8, [16, 13, 1]),
    ("f32-d128-g5-w-ge-context", 1, 10, 2, 128, "f32", 400, [60], 0.5, [20, 31]),
    ("bf16-d128-g5-empty-prompt", 2, 10, 2, 128, "bf16", 6, [0, 0], 0.6, [3, 25]),
    # 2, 3 and 4 column tiles per wave (G = 4 at d = 64, G = 5 at d = 128),
    # prompts long enough for many pairs of full blocks, a short window
    ("bf16-d64-g4-two-three-tiles", 2, 8, 2, 64, "bf16", 10, [120, 77], 0.7, [6, 12, 8, 1]),
    ("bf16-d128-g5-three-four-tiles", 2, 10, 2, 128, "bf16", 20, [300, 150], 0.9, [8, 12, 16, 4]),
]


@gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunks_match_oracle(case):
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    name, B, Hq, Hkv, d, dtype, w, P, mu, chunks = case
    P = np.asarray(P)
    steps = int(sum(chunks))
    T = int(P.max()) + steps
    Q, K, V, lg = _host(6000 + d + w, B, Hq, Hkv, T, d, dtype, mu)
    ref = O.decode_batch(Q, K, V, lg, P, steps, w)
    print(f"[{name}] B={B} Hq={Hq} Hkv={Hkv} d={d} w={w} P={list(P)} chunks={chunks}", flush=True)
    cache = dms.Cache(B, Hq, Hkv, d, w, T, B * Hkv * (T // 16 + 2), dtype=dtype)
    pmax = max(int(P.max()), 1)
    Kp = np.zeros((B, Hkv, pmax, d), np.float32)
    Vp = np.zeros_like(Kp)
    Lp = np.zeros((B, Hkv, pmax), np.float32)
    for b in range(B):
        Kp[b, :, :P[b]] = K[b, :, :P[b]]
        Vp[b, :, :P[b]] = V[b, :, :P[b]]
        Lp[b, :, :P[b]] = lg[b, :, :P[b]]
    cache.prefill(_dev(Kp, dtype), _dev(Vp, dtype), torch.from_numpy(Lp).cuda(), P)
    t0 = 0
    for C in chunks:
        q = _dev(_slices(Q, P, t0, C), dtype)
        k = _dev(_slices(K, P, t0, C), dtype)
        v = _dev(_slices(V, P, t0, C), dtype)
        l = torch.from_numpy(np.ascontiguousarray(_slices(lg, P, t0, C))).cuda()
        out = cache.decode_chunk(q, k, v, l)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()                       # [B, Hq, C, d]
        want = ref["out"][t0:t0 + C].transpose(1, 2, 0, 3)     # [B, Hq, C, d]
        err = float(np.max(np.abs(got - want)))
        assert err <= TOL[dtype], (name, t0, C, err)
        sp, rg, n = cache.export()
        for b in range(B):
            for h in range(Hkv):
                rec = ref["records"][(b, h)][t0 + C - 1]
                u = b * Hkv + h
                assert n[u] == len(rec.visible), (name, t0, C, b, h)
                assert np.array_equal(np.sort(sp[u][sp[u] >= 0]), rec.visible), (name, t0, C, b, h)
                assert np.array_equal(np.sort(sp[u][rg[u][rg[u] >= 0]]), rec.pending), (name, t0, C, b, h)
        print(f"  chunk {C} at step {t0}: max_err={err:.2e}", flush=True)
        t0 += C
    assert cache.stats()["sticky_error"] == 0


@gpu
@pytest.mark.parametrize("source,zero,ch", [("k", True, 0), ("k", False, 91), ("q", False, 5)],
                         ids=["key-channel-zeroed", "key-channel", "query-channel"])
def test_chunks_with_channel_logits(source, zero, ch):
    """Prompt and chunks with the eviction logit read from a projection
    channel (dms_prefill_compress_channel, dms_decode_chunk_channel): every
    output row and the state after every chunk against the oracle's
    step-by-step decode with the same logits and, when zeroed, keys."""
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    B, Hq, Hkv, d, w, dtype = 2, 8, 2, 128, 10, "bf16"
    P = np.array([90, 33])
    chunks = [5, 19, 1]
    steps = sum(chunks)
    T = int(P.max()) + steps
    Q, K, V, _ = _host(6200 + ch, B, Hq, Hkv, T, d, dtype, 0.0)
    ref = O.decode_batch_channel(Q, K, V, P, steps, w, source, ch, zero)
    cache = dms.Cache(B, Hq, Hkv, d, w, T, B * Hkv * (T // 16 + 2), dtype=dtype)
    pmax = int(P.max())
    Kp, Vp, Qp = (_dev(np.ascontiguousarray(X[:, :, :pmax]), dtype) for X in (K, V, Q))
    cache.prefill_channel(Kp, Vp, P, source=source, channel=ch, zero=zero, q=Qp if source == "q" else None)
    t0 = 0
    for C in chunks:
        q = _dev(_slices(Q, P, t0, C), dtype)
        k = _dev(_slices(K, P, t0, C), dtype)
        v = _dev(_slices(V, P, t0, C), dtype)
        out = cache.decode_chunk_channel(q, k, v, source=source, channel=ch, zero=zero)
        torch.cuda.synchronize()
        err = float(np.max(np.abs(out.double().cpu().numpy() - ref["out"][t0:t0 + C].transpose(1, 2, 0, 3))))
        assert err <= TOL[dtype], (source, zero, t0, C, err)
        sp, rg, n = cache.export()
        for b in range(B):
            for h in range(Hkv):
                rec = ref["records"][(b, h)][t0 + C - 1]
                u = b * Hkv + h
                assert np.array_equal(np.sort(sp[u][sp[u] >= 0]), rec.visible), (source, t0, b, h)
                assert np.array_equal(np.sort(sp[u][rg[u][rg[u] >= 0]]), rec.pending), (source, t0, b, h)
        t0 += C


@gpu
def test_chunk_equals_token_steps():
    """The same tokens through dms_decode_chunk and through one
    dms_append_step + dms_decode_attention per token: identical logical
    state, outputs equal up to summation order, and the same live-token count."""
    from learned_kv_cache_dms_amd import dms
    B, Hq, Hkv, d, w, dtype = 4, 10, 2, 128, 16, "bf16"
    P = np.array([200, 57, 130, 1])
    C = 24
    T = int(P.max()) + C
    Q, K, V, lg = _host(6100, B, Hq, Hkv, T, d, dtype, 1.15)
    a = dms.Cache(B, Hq, Hkv, d, w, T, 256, dtype=dtype)
    b_ = dms.Cache(B, Hq, Hkv, d, w, T, 256, dtype=dtype)
    pmax = int(P.max())
    Kp = _dev(K[:, :, :pmax], dtype)
    Vp = _dev(V[:, :, :pmax], dtype)
    Lp = torch.from_numpy(np.ascontiguousarray(lg[:, :, :pmax])).cuda()
    a.prefill(Kp, Vp, Lp, P)
    b_.prefill(Kp, Vp, Lp, P)
    q = _dev(_slices(Q, P, 0, C), dtype)
    k = _dev(_slices(K, P, 0, C), dtype)
    v = _dev(_slices(V, P, 0, C), dtype)
    l = torch.from_numpy(np.ascontiguousarray(_slices(lg, P, 0, C))).cuda()
    s0a, s0b = a.stats(), b_.stats()
    oa = a.decode_chunk(q, k, v, l)
    ob = torch.empty_like(oa)
    for j in range(C):
        b_.append(k[:, :, j].contiguous(), v[:, :, j].contiguous(), l[:, :, j].contiguous())
        ob[:, :, j] = b_.attend(q[:, :, j].contiguous())
    torch.cuda.synchronize()
    assert float((oa - ob).abs().max()) <= 1e-5
    sa, ra, na = a.export()
    sb, rb, nb = b_.export()
    assert np.array_equal(na, nb)
    for u in range(B * Hkv):
        assert np.array_equal(np.sort(sa[u][sa[u] >= 0]), np.sort(sb[u][sb[u] >= 0]))
        pa = np.where(ra[u] >= 0, sa[u][np.maximum(ra[u], 0)], -1)
        pb = np.where(rb[u] >= 0, sb[u][np.maximum(rb[u], 0)], -1)
        assert np.array_equal(pa, pb)
    s1a, s1b = a.stats(), b_.stats()
    assert s1a["live_token_steps"] - s0a["live_token_steps"] == s1b["live_token_steps"] - s0b["live_token_steps"]
    assert s1a["seen_tokens"] == s1b["seen_tokens"]


@gpu
def test_chunk_errors():
    from learned_kv_cache_dms_amd import dms
    B, Hq, Hkv, d = 2, 4, 2, 64
    c = dms.Cache(B, Hq, Hkv, d, 4, 20, 16, dtype="bf16")
    mk = lambda H, C: torch.zeros((B, H, C, d), dtype=torch.bfloat16, device="cuda")
    l = torch.zeros((B, Hkv, 21), dtype=torch.float32, device="cuda")
    with pytest.raises(dms.DmsError) as e:
        c.decode_chunk(mk(Hq, 21), mk(Hkv, 21), mk(Hkv, 21), l)
    assert e.value.status == dms.DMS_ERR_CAPACITY
    with pytest.raises(dms.DmsError) as e:
        dms.dms_decode_chunk(c.handle, 1, 1, 1, 1, 0, 1, c._stream())
    assert e.value.status == dms.DMS_ERR_ARG
    big = dms.Cache(1, 1, 1, 64, 4, 8192 * 16 + 1, 4, dtype="bf16")
    x = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dms.DmsError) as e:
        big.decode_chunk(x, x, x, torch.zeros((1, 1, 1), dtype=torch.float32, device="cuda"))
    assert e.value.status == dms.DMS_ERR_ARG
    assert c.stats()["seen_tokens"] == 0


@gpu
def test_chunks_full_size_sampled_units():
    """The Qwen-R1-32B-shaped layer at full size (64 x 32768-token prompts,
    40 Q / 8 KV heads, d = 128, w = 256): chunks of 16, 3 and 16 tokens per
    sequence.  For sampled units, every output row of every chunk against
    the oracle's attention at that row's own position, and the visible and
    pending sets after every chunk (bit-exact); every unit's live count at
    the end."""
    import dataclasses
    import gpu_util as U
    from oracle import dms_oracle as O
    from synth import device as dsynth
    from synth import workloads as W
    chunks = [16, 3, 16]
    wl = dataclasses.replace(W.qwen_32b(), decode_steps=sum(chunks))
    B, Hq, Hkv, d, w, G = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window, wl.group
    lengths = wl.prompt_lengths()
    cache = U.make_cache(wl)
    K, V, Lg = U.device_prompt(wl, 0, lengths)
    cache.prefill(K, V, Lg, lengths)
    del K, V, Lg
    rng = np.random.default_rng(wl.seed + 1)
    n_units = B * Hkv
    picks = sorted(set([0, n_units - 1] + list(rng.choice(n_units, 2, replace=False))))
    units = [(u // Hkv, u % Hkv) for u in picks]
    host = {key: U.host_unit(wl, 0, key[0], key[1], int(lengths[key[0]]), wl.decode_steps) for key in units}
    base = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    mb, ma = wl.layer_mu(0)
    scale = O.default_scale(d)
    st = U.CompareStats()
    worst = 0.0
    t0 = 0
    for C in chunks:
        print(f"[qwen-32b chunk] C={C} at step {t0}", flush=True)
        q = torch.empty((B, Hq, C, d), dtype=torch.bfloat16, device="cuda")
        k = torch.empty((B, Hkv, C, d), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        lg = torch.empty((B, Hkv, C), dtype=torch.float32, device="cuda")
        pb = base + t0  # per-sequence first position of the chunk
        dsynth.fill(q, wl.seed, synth.STREAM_Q, 0, 0, pos_base=pb)
        dsynth.fill(k, wl.seed, synth.STREAM_K, 0, 0, pos_base=pb)
        dsynth.fill(v, wl.seed, synth.STREAM_V, 0, 0, pos_base=pb)
        dsynth.logits(lg, wl.seed, 0, 0, mb, ma, wl.pos_threshold, pos_base=pb)
        out = cache.decode_chunk(q, k, v, lg)
        torch.cuda.synchronize()
        for key in units:
            ud = host[key]
            alpha = O.eviction_decision(ud.logit)
            for j in range(C - 1):
                vis = O.visible(alpha, ud.prompt_len + t0 + j, w)
                ref = O.attend(ud.Q[t0 + j], ud.K[vis], ud.V[vis], scale)
                got = out[ud.b, ud.h * G:(ud.h + 1) * G, j].double().cpu().numpy()
                err = float(np.max(np.abs(got - ref)))
                worst = max(worst, err)
                assert err <= TOL["bf16"], (key, t0 + j, err)
            # the last row, with the cache state after the chunk
            U.check_unit_step(cache, wl, ud, t0 + C - 1, out[:, :, C - 1], TOL["bf16"], st)
        t0 += C
    assert cache.stats()["sticky_error"] == 0
    qlast = wl.prompt_len + wl.decode_steps - 1
    lgh = synth.logits(wl.seed, 0, np.arange(B), Hkv, np.arange(qlast + 1), mb, ma, wl.pos_threshold)
    _, _, n = cache.export(0, n_units)
    ref_n = np.array([len(O.visible(O.eviction_decision(lgh[b, h]), qlast, w)) for b in range(B) for h in range(Hkv)])
    assert np.array_equal(n, ref_n)
    print(f"  max_err={max(worst, st.max_err):.2e} over {len(units)} units", flush=True)
