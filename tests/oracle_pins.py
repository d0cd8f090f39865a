"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each pin takes the oracle module ``O`` and raises AssertionError on a
mismatch.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` plants single mistakes in the oracle and checks
that at least one pin fails for each.

References are independent of the oracle's code: hand-worked tables in
``tests/golden/``, a FIFO simulation of delayed eviction, torch's
scaled_dot_product_attention (float64, CPU) for the dense-causal and
sliding-window special cases, scipy's softmax, and closed forms.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch

from synth import synth, workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# visibility and schedule
# --------------------------------------------------------------------------

def pin_golden_visibility(O):
    g = _load("visibility_hand.json")
    alpha = np.array(g["alpha"], dtype=bool)
    for case in g["cases"]:
        w = case["w"]
        for q, (vis, ret) in enumerate(zip(case["visible"], case["retired"])):
            got = O.visible(alpha, q, w)
            assert list(got) == vis, (w, q, list(got), vis)
            assert list(O.retired(alpha, q, w)) == ret, (w, q)


def _fifo_simulation(alpha, w, T):
    """Delayed eviction simulated with explicit expiry times: a marked token
    i is scheduled to leave once the query passes i + w.  Returns, for every
    query q, the live tokens and the scheduled ones among them (marked,
    still live, their removal pending)."""
    live = []
    expiry = {}
    sets, scheduled = [], []
    for q in range(T):
        live.append(q)
        if alpha[q]:
            expiry[q] = q + w
        live = [i for i in live if not (i in expiry and q > expiry[i])]
        sets.append(list(live))
        scheduled.append([i for i in live if i in expiry])
    return sets, scheduled


def _fifo_visible_sets(alpha, w, T):
    return _fifo_simulation(alpha, w, T)[0]


def pin_fifo_simulation(O):
    rng = np.random.default_rng(7)
    for w in (0, 1, 2, 3, 5, 16):
        for p in (0.0, 0.3, 0.7, 1.0):
            T = 70
            alpha = rng.random(T) < p
            ref = _fifo_visible_sets(alpha, w, T)
            for q in range(T):
                assert list(O.visible(alpha, q, w)) == ref[q], (w, p, q)
                prev = set(ref[q - 1]) | {q} if q > 0 else {0}
                assert sorted(prev - set(ref[q])) == list(O.retired(alpha, q, w)), (w, p, q)


def pin_pending_against_fifo(O):
    """The pending set is exactly the simulation's scheduled tokens: every
    marked token still live, oldest included (completeness and soundness),
    and its size is min(q, w) + 1 when every token is marked."""
    rng = np.random.default_rng(19)
    for w in (0, 1, 3, 8, 40):
        for p in (0.0, 0.4, 0.9, 1.0):
            T = 90
            alpha = rng.random(T) < p
            _, sched = _fifo_simulation(alpha, w, T)
            for q in range(T):
                got = [int(i) for i in O.pending(alpha, q, w)]
                assert got == sched[q], (w, p, q, got, sched[q])
    ones = np.ones(50, dtype=bool)
    for w in (0, 5, 60):
        for q in range(50):
            assert len(O.pending(ones, q, w)) == min(q, w) + 1


def pin_special_visibility(O):
    T = 40
    for w in (0, 1, 4, 100):
        zeros = np.zeros(T, dtype=bool)
        ones = np.ones(T, dtype=bool)
        for q in range(T):
            assert list(O.visible(zeros, q, w)) == list(range(q + 1))
            assert list(O.visible(ones, q, w)) == list(range(max(0, q - w), q + 1))
            assert O.retired(zeros, q, w) == []
        if w >= T:
            rng = np.random.default_rng(w)
            a = rng.random(T) < 0.5
            for q in range(T):
                assert list(O.visible(a, q, w)) == list(range(q + 1))


def pin_schedule_invariants(O):
    rng = np.random.default_rng(11)
    for w in (0, 2, 7, 32):
        alpha = rng.random(200) < 0.6
        prev = 0
        for q in range(200):
            vis = O.visible(alpha, q, w)
            ret = O.retired(alpha, q, w)
            assert len(vis) - prev == 1 - len(ret)
            for j in ret:
                assert alpha[j] and j == q - w - 1
            pend = O.pending(alpha, q, w)
            assert len(pend) <= w + 1
            assert all(q - w <= i <= q and alpha[i] for i in pend)
            assert abs(O.compression_ratio(q, len(vis)) - (q + 1) / len(vis)) == 0.0
            prev = len(vis)


def pin_decision_threshold(O):
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    logit = np.array([np.nan, 0.0, -0.0, tiny, -tiny, 1e-30, -1e30, np.inf, -np.inf],
                     dtype=np.float32)
    got = O.eviction_decision(logit)
    assert list(map(bool, got)) == [False, False, False, True, False, True, False, True, False]


def _irwin_hall_cdf(x: float, n: int = 12) -> float:
    """CDF of the sum of n independent U(0,1) variables (closed form)."""
    if x <= 0:
        return 0.0
    if x >= n:
        return 1.0
    return sum((-1) ** k * math.comb(n, k) * (x - k) ** n
               for k in range(int(math.floor(x)) + 1)) / math.factorial(n)


def pin_expected_live_count(O):
    """|Vis(q)| on synthetic logits against its closed-form mean and variance
    under independent marks, within 5 sigma, plus the CR identity.

    The synthetic logit is mu + x with x = IH12 - 6 up to a 2**-16 lattice, so
    P(marked) = 1 - F_IH12(6 - mu)."""
    wl = workloads.llama_1b()
    q = 4095
    lg = synth.logits(wl.seed, 0, np.arange(wl.batch), wl.num_kv_heads, np.arange(q + 1),
                      wl.mu_before[0])
    counts = []
    for b in range(wl.batch):
        for h in range(wl.num_kv_heads):
            a = O.eviction_decision(lg[b, h])
            counts.append(len(O.visible(a, q, wl.window)))
    counts = np.array(counts, dtype=np.float64)
    p = 1.0 - _irwin_hall_cdf(6.0 - wl.mu_before[0])
    n_old = q + 1 - (wl.window + 1)
    mean = n_old * (1 - p) + (wl.window + 1)
    var = n_old * p * (1 - p)
    tol = 5 * math.sqrt(var / len(counts)) + 1e-3 * n_old
    assert abs(counts.mean() - mean) < tol, (counts.mean(), mean, tol)
    total_seen = (q + 1) * len(counts)
    cr = total_seen / counts.sum()
    assert abs(cr - total_seen / np.sum([len(O.visible(O.eviction_decision(lg[b, h]), q, wl.window))
                                          for b in range(wl.batch)
                                          for h in range(wl.num_kv_heads)])) == 0.0
    assert 3.0 < cr < 3.8


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def pin_golden_attention(O):
    g = _load("attention_hand.json")
    d = g["d"]
    qv = np.array([g["q"]])
    K = np.array(g["keys"])
    V = np.array(g["values"])
    scale = O.default_scale(d)
    for case in g["cases"]:
        alpha = np.array(case["alpha"], dtype=bool)
        q = case["query_pos"]
        vis = O.visible(alpha, q, case["w"])
        assert list(vis) == case["visible"]
        wts = O.attention_weights(qv, K[vis], scale)[0]
        np.testing.assert_allclose(wts, case["weights"], rtol=0, atol=1e-14)
        out = O.attend(qv, K[vis], V[vis], scale)[0]
        np.testing.assert_allclose(out, case["out"], rtol=0, atol=1e-13)
        outm = O.attend_masked(qv, K, V, alpha, q, case["w"], scale)[0]
        np.testing.assert_allclose(outm, case["out"], rtol=0, atol=1e-13)


def _sdpa(Q, K, V, allowed, Hq, Hkv):
    """torch reference: Q [Hq, Lq, d], K/V [Hkv, Lk, d], allowed [Lq, Lk] bool."""
    q = torch.from_numpy(Q)[None]
    k = torch.from_numpy(K)[None]
    v = torch.from_numpy(V)[None]
    m = torch.from_numpy(allowed)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m,
                                                         enable_gqa=(Hq != Hkv))
    return o[0].numpy()


def _random_batch(rng, B, Hq, Hkv, T, d):
    Q = rng.standard_normal((B, Hq, T, d))
    K = rng.standard_normal((B, Hkv, T, d))
    V = rng.standard_normal((B, Hkv, T, d))
    return Q, K, V


def _special_case_vs_sdpa(O, marked: bool, w: int):
    rng = np.random.default_rng(3 if marked else 4)
    B, Hq, Hkv, T, d = 2, 6, 2, 48, 16
    P, steps = 20, 28
    Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
    logit = np.full((B, Hkv, T), 1.0 if marked else -1.0, dtype=np.float32)
    res = O.decode_batch(Q, K, V, logit, [P] * B, steps, w)
    qpos = torch.arange(P, P + steps)[:, None]
    kpos = torch.arange(T)[None, :]
    allowed = kpos <= qpos
    if marked:
        allowed = allowed & (kpos >= qpos - w)
    for b in range(B):
        ref = _sdpa(np.ascontiguousarray(Q[b, :, P:P + steps]), K[b], V[b], allowed.numpy(), Hq, Hkv)
        got = res["out"][:, b].transpose(1, 0, 2)       # [Hq, steps, d]
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_unmarked_is_dense_causal(O):
    _special_case_vs_sdpa(O, marked=False, w=5)


def pin_marked_is_sliding_window(O):
    for w in (0, 3, 9):
        _special_case_vs_sdpa(O, marked=True, w=w)


def pin_gather_equals_masked(O):
    rng = np.random.default_rng(5)
    d, T = 8, 64
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    for w in (0, 1, 6):
        alpha = rng.random(T) < 0.6
        for q in (0, 5, 31, 63):
            qv = rng.standard_normal((3, d))
            vis = O.visible(alpha, q, w)
            a = O.attend(qv, K[vis], V[vis], 0.37)
            b = O.attend_masked(qv, K, V, alpha, q, w, 0.37)
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def pin_single_visible_returns_value(O):
    """w = 0 with every token marked leaves only the query's own token, so the
    output is that token's value row exactly."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, T, d = 1, 4, 2, 24, 8
    Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
    logit = np.ones((B, Hkv, T), dtype=np.float32)
    res = O.decode_batch(Q, K, V, logit, [10], 14, 0)
    for t in range(14):
        for hq in range(Hq):
            assert np.array_equal(res["out"][t, 0, hq], V[0, hq // 2, 10 + t])


def pin_constant_values(O):
    rng = np.random.default_rng(8)
    B, Hq, Hkv, T, d = 1, 3, 1, 40, 4
    Q, K, _ = _random_batch(rng, B, Hq, Hkv, T, d)
    V = np.broadcast_to(np.array([1.5, -2.0, 0.25, 7.0]), (B, Hkv, T, d)).copy()
    logit = rng.standard_normal((B, Hkv, T)).astype(np.float32)
    res = O.decode_batch(Q, K, V, logit, [16], 24, 3)
    np.testing.assert_allclose(res["out"][:, 0], np.broadcast_to(V[0, 0, 0], (24, Hq, d)),
                               rtol=0, atol=1e-13)


def pin_one_hot_values(O):
    """V[i] = e_i makes the output equal the softmax weights, checked against
    scipy's softmax of the scores over the hand-built visible set."""
    rng = np.random.default_rng(9)
    d = 40
    T = 40
    K = rng.standard_normal((T, d))
    V = np.eye(T, d)
    qv = rng.standard_normal((2, d))
    alpha = np.array([i % 3 == 0 for i in range(T)])
    w = 4
    q = T - 1
    keep = [i for i in range(q + 1) if (i % 3 != 0) or (q - i <= w)]
    vis = O.visible(alpha, q, w)
    assert list(vis) == keep
    out = O.attend(qv, K[vis], V[vis], 1 / math.sqrt(d))
    ref = np.zeros((2, d))
    ref[:, keep] = scipy.special.softmax(qv @ K[keep].T / math.sqrt(d), axis=1)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-14)


def pin_needles(O):
    """A key aligned with the query and scaled by 40 dominates the softmax
    when visible and must have no effect when evicted."""
    rng = np.random.default_rng(10)
    B, Hq, Hkv, T, d = 1, 2, 1, 64, 16
    Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
    w = 4
    logit = np.where(np.arange(T) % 2 == 0, 1.0, -1.0).astype(np.float32)[None, None]
    P, steps = 40, 1
    q = P
    qv = Q[0, :, q]
    base = O.decode_batch(Q, K, V, logit, [P], steps, w)["out"][0, 0]
    # evicted position: marked (even) and older than the window
    ev = 20
    assert ev not in set(O.visible(O.eviction_decision(logit[0, 0]), q, w))
    K2 = K.copy()
    K2[0, 0, ev] = 40.0 * qv[0] / np.linalg.norm(qv[0]) * math.sqrt(d)
    out_ev = O.decode_batch(Q, K2, V, logit, [P], steps, w)["out"][0, 0]
    np.testing.assert_allclose(out_ev, base, rtol=0, atol=1e-13)
    # live position: unmarked (odd) old token
    lv = 21
    K3 = K.copy()
    K3[0, 0, lv] = 40.0 * qv[0] / np.linalg.norm(qv[0]) * math.sqrt(d)
    out_lv = O.decode_batch(Q, K3, V, logit, [P], steps, w)["out"][0, 0]
    np.testing.assert_allclose(out_lv[0], V[0, 0, lv], rtol=0, atol=1e-6)


def pin_ragged_prompts(O):
    """Per-sequence prompt lengths: each sequence's queries run at its own
    positions; compared with the all-unmarked dense case per sequence."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, T, d = 3, 2, 1, 40, 8
    Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
    logit = np.full((B, Hkv, T), -1.0, dtype=np.float32)
    P = [3, 17, 30]
    res = O.decode_batch(Q, K, V, logit, P, 8, 2)
    for b in range(B):
        qpos = torch.arange(P[b], P[b] + 8)[:, None]
        allowed = (torch.arange(T)[None, :] <= qpos).numpy()
        ref = _sdpa(np.ascontiguousarray(Q[b, :, P[b]:P[b] + 8]), K[b], V[b], allowed, Hq, Hkv)
        np.testing.assert_allclose(res["out"][:, b].transpose(1, 0, 2), ref, rtol=0, atol=1e-12)


def pin_channel_logit_location(O):
    """The logit of KV head h at position i sits at channel c of key head h,
    or of query head h * G: a tensor that is zero except there (plus noise
    in every other channel and in the group's other query heads) gives back
    exactly the values planted."""
    rng = np.random.default_rng(21)
    B, Hkv, G, T, d, c = 2, 3, 4, 7, 6, 2
    for group, H in ((1, Hkv), (G, Hkv * G)):
        X = rng.standard_normal((B, H, T, d)).astype(np.float32) * 50
        planted = np.empty((B, Hkv, T), dtype=np.float32)
        for b in range(B):
            for h in range(Hkv):
                for i in range(T):
                    val = np.float32(100 * b + 10 * h + i + 0.25)
                    X[b, h * group, i, c] = val
                    planted[b, h, i] = val
        got = O.logits_from_channel(X, c, group)
        assert got.dtype == np.float32 and got.shape == (B, Hkv, T)
        assert np.array_equal(got, planted)


def pin_zeroed_channel_is_dropped_feature(O):
    """Keys with channel c zeroed give the attention of queries and keys with
    that channel deleted (d - 1 features), at the same scale 1/sqrt(d)."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, T, d, c = 2, 4, 2, 30, 8, 5
    Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
    logit = rng.standard_normal((B, Hkv, T)).astype(np.float32)
    P, steps, w = [10, 17], 9, 3
    a = O.decode_batch(Q, O.without_channel(K, c), V, logit, P, steps, w, 1 / math.sqrt(d))
    # V loses the same column so that every array has d - 1 channels; the
    # outputs' other columns must agree
    b = O.decode_batch(np.delete(Q, c, axis=-1), np.delete(K, c, axis=-1), np.delete(V, c, axis=-1),
                       logit, P, steps, w, 1 / math.sqrt(d))
    np.testing.assert_allclose(np.delete(a["out"], c, axis=-1), b["out"], rtol=0, atol=1e-12)


def pin_channel_logit_special_cases(O):
    """Key channel c forced below 0 everywhere: nothing is marked, so the
    decode is dense causal attention (torch SDPA with the channel deleted);
    forced above 0: everything is marked, so it is the sliding window."""
    rng = np.random.default_rng(23)
    B, Hq, Hkv, T, d, c, w = 2, 6, 2, 40, 8, 3, 4
    P, steps = 12, 28
    for marked in (False, True):
        Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
        K[..., c] = (np.abs(K[..., c]) + 0.1) * (1.0 if marked else -1.0)
        res = O.decode_batch_channel(Q, K, V, [P] * B, steps, w, "k", c, True)
        qpos = torch.arange(P, P + steps)[:, None]
        kpos = torch.arange(T)[None, :]
        allowed = kpos <= qpos
        if marked:
            allowed = allowed & (kpos >= qpos - w)
        Qd, Kd = np.delete(Q, c, axis=-1), np.delete(K, c, axis=-1)
        for b in range(B):
            # SDPA scales by 1/sqrt(d - 1): rescale the queries to keep 1/sqrt(d)
            qs = np.ascontiguousarray(Qd[b, :, P:P + steps]) * math.sqrt((d - 1) / d)
            ref = _sdpa(qs, np.ascontiguousarray(Kd[b]), V[b], allowed.numpy(), Hq, Hkv)
            got = res["out"][:, b].transpose(1, 0, 2)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _prefill_special_case(O, marked: bool, w: int):
    rng = np.random.default_rng(31 if marked else 32)
    B, Hq, Hkv, T, d = 2, 6, 3, 45, 8
    Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
    logit = np.full((B, Hkv, T), 1.0 if marked else -1.0, dtype=np.float32)
    P = [45, 29]
    out = O.prefill_attention(Q, K, V, logit, P, w)
    for b in range(B):
        pos = torch.arange(P[b])
        allowed = pos[None, :] <= pos[:, None]
        if marked:
            allowed = allowed & (pos[None, :] >= pos[:, None] - w)
        ref = _sdpa(np.ascontiguousarray(Q[b, :, :P[b]]), np.ascontiguousarray(K[b, :, :P[b]]),
                    np.ascontiguousarray(V[b, :, :P[b]]), allowed.numpy(), Hq, Hkv)
        np.testing.assert_allclose(out[b, :, :P[b]], ref, rtol=0, atol=1e-12)
        assert np.all(np.isnan(out[b, :, P[b]:]))


def pin_prefill_unmarked_is_causal_attention(O):
    """No token marked: every prompt query attends all earlier positions
    (torch SDPA, causal mask)."""
    _prefill_special_case(O, marked=False, w=4)


def pin_prefill_marked_is_sliding_window(O):
    """Every token marked: query q attends positions q - w .. q."""
    for w in (0, 5):
        _prefill_special_case(O, marked=True, w=w)


def pin_prefill_equals_masked_form(O):
    """Random decisions: each prompt query's output equals the dense
    additive-mask form over its causal positions."""
    rng = np.random.default_rng(33)
    B, Hq, Hkv, T, d, w = 1, 4, 2, 40, 8, 3
    Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
    logit = rng.standard_normal((B, Hkv, T)).astype(np.float32) + 0.5
    out = O.prefill_attention(Q, K, V, logit, [T], w, 0.3)
    for h in range(Hkv):
        alpha = logit[0, h] > 0
        for hq in (2 * h, 2 * h + 1):
            for q in range(T):
                ref = O.attend_masked(Q[0, hq, q][None], K[0, h], V[0, h], alpha, q, w, 0.3)[0]
                np.testing.assert_allclose(out[0, hq, q], ref, rtol=0, atol=1e-12)


def _soft_inputs(seed, B=2, Hq=4, Hkv=2, T=37, d=8):
    rng = np.random.default_rng(seed)
    Q, K, V = _random_batch(rng, B, Hq, Hkv, T, d)
    logit = rng.standard_normal((B, Hkv, T))
    u = rng.random((B, Hkv, T))
    noise = np.log(u) - np.log1p(-u)          # logistic noise
    dO = rng.standard_normal((B, Hq, T, d))
    return Q, K, V, logit, noise, dO


def _soft_torch(Q, K, V, logit, noise, w, gamma, tau, requires_grad=False):
    """torch SDPA (float64, CPU) with the relaxed mask as a float attn_mask."""
    Hq, Hkv = Q.shape[1], K.shape[1]
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=requires_grad)
    q, k, v, lg = t(Q), t(K), t(V), t(logit)
    T = Q.shape[2]
    pos = torch.arange(T)
    far = (pos[:, None] - pos[None, :]) > w
    causal = pos[None, :] <= pos[:, None]
    x = (lg + gamma + torch.tensor(noise, dtype=torch.float64)) / tau
    bias = torch.log(1.0 - torch.sigmoid(x))                               # [B, Hkv, T]
    bias = bias.repeat_interleave(Hq // Hkv, dim=1)[:, :, None, :]          # [B, Hq, 1, T]
    mask = torch.where(causal, torch.where(far, bias, torch.zeros(())), torch.tensor(-float("inf")))
    o = torch.nn.functional.scaled_dot_product_attention(q, k.repeat_interleave(Hq // Hkv, 1),
                                                         v.repeat_interleave(Hq // Hkv, 1), attn_mask=mask)
    return o, (q, k, v, lg)


def pin_soft_attention_is_sdpa_with_float_mask(O):
    """The relaxed attention equals torch SDPA given the additive mask."""
    Q, K, V, logit, noise, _ = _soft_inputs(51)
    for w, gamma, tau in ((3, 0.0, 1.0), (0, -2.0, 0.3), (10, 1.5, 2.0)):
        got = O.soft_attention(Q, K, V, logit, noise, w, gamma, tau)["out"]
        ref, _ = _soft_torch(Q, K, V, logit, noise, w, gamma, tau)
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def pin_soft_attention_hard_limit(O):
    """Decisions pushed to 0 or 1 (|logit| = 60 at tau = 1) give the hard DMS
    attention of every prompt query (itself pinned above)."""
    Q, K, V, logit, noise, _ = _soft_inputs(52)
    marked = logit > 0
    hard = np.where(marked, 60.0, -60.0)
    zero = np.zeros_like(noise)
    for w in (0, 4):
        got = O.soft_attention(Q, K, V, hard, zero, w, 0.0, 1.0)["out"]
        ref = O.prefill_attention(Q, K, V, marked.astype(np.float32) * 2 - 1, [Q.shape[2]] * Q.shape[0], w)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def pin_soft_attention_lse(O):
    """lse is the log of each row's denominator: exp(s - lse) sums to 1,
    checked through out = sum_i exp(s_i - lse) v_i with V = ones."""
    Q, K, V, logit, noise, _ = _soft_inputs(53)
    res = O.soft_attention(Q, K, np.ones_like(V), logit, noise, 2, 0.5, 0.7)
    np.testing.assert_allclose(res["out"], 1.0, rtol=0, atol=1e-12)
    ref_lse = []
    B, Hq, T, d = Q.shape
    G = Hq // K.shape[1]
    pos = np.arange(T)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            x = (logit[b, h] + 0.5 + noise[b, h]) / 0.7
            bias = np.log1p(-1.0 / (1.0 + np.exp(-x)))
            row = []
            for q in range(T):
                s = [Q[b, hq, q] @ K[b, h, i] / math.sqrt(d) + (bias[i] if q - i > 2 else 0.0) for i in range(q + 1)]
                row.append(scipy.special.logsumexp(s))
            ref_lse.append(row)
    np.testing.assert_allclose(res["lse"].reshape(B * Hq, T), np.array(ref_lse), rtol=0, atol=1e-11)


def pin_soft_attention_grads_are_autograd(O):
    """Gradients equal torch autograd (float64) through SDPA with the float
    mask, for Q, K, V and the logits."""
    Q, K, V, logit, noise, dO = _soft_inputs(54)
    for w, gamma, tau in ((3, 0.0, 1.0), (1, -1.0, 0.4)):
        g = O.soft_attention_grads(Q, K, V, logit, noise, dO, w, gamma, tau)
        o, (q, k, v, lg) = _soft_torch(Q, K, V, logit, noise, w, gamma, tau, requires_grad=True)
        (o * torch.tensor(dO)).sum().backward()
        np.testing.assert_allclose(g["dq"], q.grad.numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(g["dk"], k.grad.numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(g["dv"], v.grad.numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(g["dlogit"], lg.grad.numpy(), rtol=0, atol=1e-11)


def pin_soft_attention_grad_magnitudes(O):
    """The magnitude sums (used to bound a rounded P or dS in the GPU's
    gradient products) against torch: dS is the autograd gradient of the loss
    at the masked scores and P their softmax; dv_mag = P^T |dO|, dk_mag =
    scale |dS|^T |Q|, dq_mag = scale |dS| |K|, summed over each group's heads."""
    Q, K, V, logit, noise, dO = _soft_inputs(55)
    B, Hq, T, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    for w, gamma, tau in ((2, 0.0, 1.0), (0, 1.0, 0.5)):
        g = O.soft_attention_grads(Q, K, V, logit, noise, dO, w, gamma, tau, magnitudes=True)
        pos = torch.arange(T)
        far = (pos[:, None] - pos[None, :]) > w
        causal = pos[None, :] <= pos[:, None]
        x = (torch.tensor(logit, dtype=torch.float64) + gamma + torch.tensor(noise, dtype=torch.float64)) / tau
        bias = torch.log(1.0 - torch.sigmoid(x))
        q, k, v, do = (torch.tensor(a, dtype=torch.float64) for a in (Q, K, V, dO))
        for b in range(B):
            dk_ref = torch.zeros((Hkv, T, d), dtype=torch.float64)
            dv_ref = torch.zeros((Hkv, T, d), dtype=torch.float64)
            for hq in range(Hq):
                h = hq // G
                mask = torch.where(causal, torch.where(far, bias[b, h][None, :], torch.zeros(())),
                                   torch.tensor(-float("inf")))
                s = (scale * (q[b, hq] @ k[b, h].T) + mask).detach().requires_grad_()
                P = torch.softmax(s, dim=1)
                ((P @ v[b, h]) * do[b, hq]).sum().backward()
                dS = s.grad
                np.testing.assert_allclose(g["dq_mag"][b, hq], (scale * dS.abs() @ k[b, h].abs()).numpy(),
                                           rtol=0, atol=1e-12)
                dk_ref[h] += scale * dS.abs().T @ q[b, hq].abs()
                dv_ref[h] += P.detach().T @ do[b, hq].abs()
            np.testing.assert_allclose(g["dk_mag"][b], dk_ref.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(g["dv_mag"][b], dv_ref.numpy(), rtol=0, atol=1e-12)
        for key in ("dq", "dk", "dv"):
            assert np.all(np.abs(g[key]) <= g[key + "_mag"] + 1e-12), key


ALL_PINS = [
    pin_golden_visibility,
    pin_fifo_simulation,
    pin_pending_against_fifo,
    pin_special_visibility,
    pin_schedule_invariants,
    pin_decision_threshold,
    pin_expected_live_count,
    pin_golden_attention,
    pin_unmarked_is_dense_causal,
    pin_marked_is_sliding_window,
    pin_gather_equals_masked,
    pin_single_visible_returns_value,
    pin_constant_values,
    pin_one_hot_values,
    pin_needles,
    pin_ragged_prompts,
    pin_channel_logit_location,
    pin_zeroed_channel_is_dropped_feature,
    pin_channel_logit_special_cases,
    pin_prefill_unmarked_is_causal_attention,
    pin_prefill_marked_is_sliding_window,
    pin_prefill_equals_masked_form,
    pin_soft_attention_is_sdpa_with_float_mask,
    pin_soft_attention_hard_limit,
    pin_soft_attention_lse,
    pin_soft_attention_grads_are_autograd,
    pin_soft_attention_grad_magnitudes,
]
