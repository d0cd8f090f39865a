"""GPU parity of dms_prefill_attention (every prompt query attends its own
visible set) against the oracle's ``prefill_attention``: every output row at
small and medium sizes, sampled rows at the full Qwen-R1-32B-shaped layer.

Tolerances: fp32 rows 1e-5 absolute.  For bf16 rows the kernel feeds the
softmax weights p_i to P.V rounded to bf16 (nearest even, 2^-8 relative) and
keeps their sum in fp32, so an output element is off by at most 2^-8 sum_i
softmax_i |v_i| from the rounding, plus n 2^-24 of the same sum for the fp32
accumulation of n keys, plus 1e-4 for the rest of the fp32 arithmetic (the
decode path's bound).  sum_i softmax_i |v_i| is the oracle's attention with
|V| as the values."""
import numpy as np
import pytest
import torch

from synth import synth

gpu = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-4}
ROUND = 2.0 ** -8   # bf16 rounding of one weight, relative
U32 = 2.0 ** -24    # fp32 unit roundoff


def excess(got, want, mag, n_keys, dtype):
    """max |got - want| / allowed over the elements (at most 1 passes):
    allowed = TOL for fp32 rows; (ROUND + n_keys U32) mag + TOL for bf16
    rows, mag = sum_i softmax_i |v_i| of each element."""
    if not np.all(np.isfinite(got)):
        return float("inf")
    if dtype == "f32":
        return float(np.max(np.abs(got - want))) / TOL["f32"]
    return float(np.max(np.abs(got - want) / ((ROUND + n_keys * U32) * mag + TOL["bf16"])))


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util  # noqa: F401  (imports the HIP libraries; fails loudly if unbuilt)


def _host_prompt(seed, B, Hq, Hkv, T, d, dtype, mu):
    pos = np.arange(T)
    Q = synth.tensor(seed, synth.STREAM_Q, 0, np.arange(B), np.arange(Hq), pos, d, dtype)
    K = synth.tensor(seed, synth.STREAM_K, 0, np.arange(B), np.arange(Hkv), pos, d, dtype)
    V = synth.tensor(seed, synth.STREAM_V, 0, np.arange(B), np.arange(Hkv), pos, d, dtype)
    lg = synth.logits(seed, 0, np.arange(B), np.arange(Hkv), pos, mu)
    return Q, K, V, lg


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(
        device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def _run(B, Hq, Hkv, d, dtype, w, P, mu, seed):
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    P = np.asarray(P)
    T = int(P.max())
    Q, K, V, lg = _host_prompt(seed, B, Hq, Hkv, T, d, dtype, mu)
    ref = O.prefill_attention(Q, K, V, lg, P, w)
    mag = O.prefill_attention(Q, K, np.abs(V), lg, P, w) if dtype == "bf16" else None
    cache = dms.Cache(B, Hq, Hkv, d, w, T + 1, B * Hkv * (T // 16 + 2), dtype=dtype)
    Qd, Kd, Vd = _dev(Q, dtype), _dev(K, dtype), _dev(V, dtype)
    cache.prefill(Kd, Vd, torch.from_numpy(lg).cuda(), P)
    out = torch.full((B, Hq, T, d), 7.0, dtype=torch.float32, device="cuda")
    cache.prefill_attention(Qd, Kd, Vd, out)
    got = out.double().cpu().numpy()
    err = ratio = 0.0
    for b in range(B):
        if P[b] > 0:
            sl = (b, slice(None), slice(0, P[b]))
            err = max(err, float(np.max(np.abs(got[sl] - ref[sl]))), 0.0 if np.all(np.isfinite(got[sl])) else np.inf)
            ratio = max(ratio, excess(got[sl], ref[sl], mag[sl] if mag is not None else None, P[b], dtype))
        assert np.all(got[b, :, P[b]:] == 7.0), "rows past the prompt were written"
    return err, ratio


CASES = [
    # id, B, Hq, Hkv, d, dtype, w, P, mu
    ("bf16-d128-g4-w8-ragged", 3, 8, 2, 128, "bf16", 8, [150, 97, 1], 0.3),
    ("bf16-d64-g8-w0", 2, 16, 2, 64, "bf16", 0, [300, 17], 1.15),
    ("f32-d64-g1-w3", 1, 2, 2, 64, "f32", 3, [200], 0.0),
    ("f32-d128-g6-w-ge-prompt", 2, 12, 2, 128, "f32", 300, [140, 260], 0.5),
    ("bf16-d128-g5-all-marked", 1, 10, 2, 128, "bf16", 16, [333], 8.0),
    ("bf16-d128-g7-none-marked", 1, 7, 1, 128, "bf16", 4, [290], -8.0),
    ("bf16-d128-g16-w32", 1, 16, 1, 128, "bf16", 32, [270], 1.0),
    ("bf16-d128-g5-w64-long", 2, 10, 2, 128, "bf16", 64, [1500, 1100], 1.15),
]


@gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_attention_every_row(case):
    name, B, Hq, Hkv, d, dtype, w, P, mu = case
    print(f"[{name}] B={B} Hq={Hq} Hkv={Hkv} d={d} w={w} P={P} mu={mu}", flush=True)
    err, ratio = _run(B, Hq, Hkv, d, dtype, w, P, mu, seed=5000 + d + w)
    print(f"[{name}] max_err={err:.3e} (fraction of the bound {ratio:.2f})", flush=True)
    assert ratio <= 1.0, (name, err, ratio)


@gpu
@pytest.mark.parametrize("source,zero", [("k", True), ("q", False)], ids=["key-channel-zeroed", "query-channel"])
def test_prefill_attention_after_channel_prefill(source, zero):
    """A prompt compressed with the eviction logit read from a projection
    channel (for keys, stored with that channel at 0): the prompt attention
    reads the window's keys with the same channel at 0, and every row equals
    the oracle on the channel-zeroed keys with the channel's logits."""
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    B, Hq, Hkv, d, w, ch, dtype = 2, 8, 2, 128, 24, 37, "bf16"
    P = np.array([260, 141])
    T = int(P.max())
    Q, K, V, _ = _host_prompt(5300, B, Hq, Hkv, T, d, dtype, 0.0)
    G = Hq // Hkv
    lg = O.logits_from_channel(K if source == "k" else Q, ch, 1 if source == "k" else G)
    Kc = O.without_channel(K, ch) if zero else K
    ref = O.prefill_attention(Q, Kc, V, lg, P, w)
    mag = O.prefill_attention(Q, Kc, np.abs(V), lg, P, w)
    cache = dms.Cache(B, Hq, Hkv, d, w, T + 1, B * Hkv * (T // 16 + 2), dtype=dtype)
    Qd, Kd, Vd = _dev(Q, dtype), _dev(K, dtype), _dev(V, dtype)
    cache.prefill_channel(Kd, Vd, P, source=source, channel=ch, zero=zero, q=Qd if source == "q" else None)
    out = torch.full((B, Hq, T, d), 7.0, dtype=torch.float32, device="cuda")
    cache.prefill_attention(Qd, Kd, Vd, out)
    got = out.double().cpu().numpy()
    for b in range(B):
        sl = (b, slice(None), slice(0, P[b]))
        ratio = excess(got[sl], ref[sl], mag[sl], P[b], dtype)
        assert ratio <= 1.0, (source, b, ratio)


@gpu
def test_prefill_attention_full_size_sampled_rows():
    """The Qwen-R1-32B-shaped layer (64 x 32768 tokens, 40 Q / 8 KV heads,
    d = 128, w = 256, CR 4 below position 10240 and 12 beyond): all rows on
    the GPU, sampled rows (first, window edge, threshold, last) against the
    oracle's definition on the host twin of the inputs."""
    import gpu_util as U
    from oracle import dms_oracle as O
    from synth import workloads as W
    from synth import device as dsynth
    wl = W.qwen_32b()
    B, Hq, Hkv, d, P = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.prompt_len
    lengths = wl.prompt_lengths()
    cache = U.make_cache(wl)
    K, V, Lg = U.device_prompt(wl, 0, lengths)
    cache.prefill(K, V, Lg, lengths)
    del Lg
    Qd = torch.empty((B, Hq, P, d), dtype=torch.bfloat16, device="cuda")
    dsynth.fill(Qd, wl.seed, synth.STREAM_Q, 0, 0, pos0=0)
    out = torch.empty((B, Hq, P, d), dtype=torch.float32, device="cuda")
    print(f"[qwen-32b prefill attention] B={B} Hq={Hq} P={P}", flush=True)
    cache.prefill_attention(Qd, K, V, out)
    torch.cuda.synchronize()
    G = Hq // Hkv
    mb, ma = wl.layer_mu(0)
    samples = [(0, 0, 0), (5, 17, 255), (17, 33, 256), (33, 4, 10239), (63, 39, 10240 + 77), (40, 21, P - 1),
               (12, 9, 20000), (63, 0, P - 257)]
    scale = O.default_scale(d)
    for (b, hq, qpos) in samples:
        h = hq // G
        pos = np.arange(qpos + 1)
        Kh = synth.tensor(wl.seed, synth.STREAM_K, 0, [b], [h], pos, d, wl.dtype)[0, 0]
        Vh = synth.tensor(wl.seed, synth.STREAM_V, 0, [b], [h], pos, d, wl.dtype)[0, 0]
        lg = synth.logits(wl.seed, 0, [b], [h], pos, mb, ma, wl.pos_threshold)[0, 0]
        qv = synth.tensor(wl.seed, synth.STREAM_Q, 0, [b], [hq], [qpos], d, wl.dtype)[0, 0]
        vis = O.visible(O.eviction_decision(lg), qpos, wl.window)
        ref = O.attend(qv, Kh[vis], Vh[vis], scale)[0]
        mag = O.attend(qv, Kh[vis], np.abs(Vh[vis]), scale)[0]
        got = out[b, hq, qpos].double().cpu().numpy()
        err = float(np.max(np.abs(got - ref)))
        ratio = excess(got, ref, mag, len(vis), "bf16")
        print(f"  (b={b}, hq={hq}, q={qpos}) |Vis|={len(vis)} err={err:.2e} ({ratio:.2f} of the bound)", flush=True)
        assert ratio <= 1.0, (b, hq, qpos, err, ratio)


@gpu
def test_prefill_attention_needs_a_fresh_prompt():
    """After an append (slots no longer in position order) or a reset the
    call is a state error and enqueues nothing."""
    from learned_kv_cache_dms_amd import dms
    B, Hq, Hkv, d, T = 2, 4, 2, 64, 40
    Q, K, V, lg = _host_prompt(77, B, Hq, Hkv, T + 1, d, "bf16", 0.5)
    Qd, Kd, Vd = _dev(Q[:, :, :T], "bf16"), _dev(K[:, :, :T], "bf16"), _dev(V[:, :, :T], "bf16")
    c = dms.Cache(B, Hq, Hkv, d, 4, T + 8, 64, dtype="bf16")
    with pytest.raises(dms.DmsError) as e:
        c.prefill_attention(Qd, Kd, Vd)
    assert e.value.status == dms.DMS_ERR_STATE
    c.prefill(Kd, Vd, torch.from_numpy(np.ascontiguousarray(lg[:, :, :T])).cuda(), [T, T - 3])
    c.prefill_attention(Qd, Kd, Vd)
    k1 = _dev(K[:, :, T], "bf16")
    c.append(k1, k1, torch.zeros((B, Hkv), dtype=torch.float32, device="cuda"))
    with pytest.raises(dms.DmsError) as e:
        c.prefill_attention(Qd, Kd, Vd)
    assert e.value.status == dms.DMS_ERR_STATE
    c.reset()
    with pytest.raises(dms.DmsError) as e:
        c.prefill_attention(Qd, Kd, Vd)
    assert e.value.status == dms.DMS_ERR_STATE
