"""GPU parity of the training-time relaxed attention (dms_soft_attention_forward
and dms_soft_attention_backward) against the oracle's ``soft_attention`` and
``soft_attention_grads``: every output, lse and gradient element at small and
medium sizes (several tiles of every kernel and a ragged tail), sampled KV
heads at the Qwen-R1-32B-shaped training layer, and the hard-decision limit
against the GPU's own prompt attention.

Tolerances: inputs are bf16-exact on both sides, so the differences are the
GPU's arithmetic alone.  The forward's probabilities enter P.V as bf16 hi +
lo pairs (about 2^-17 relative), accumulation is fp32, and exp2 / log2 are
the hardware approximations (about 1 ulp): out and dlogit are compared as
max |got - want| / max(1, max |want|) against 1e-4, lse against 1e-5
absolute.  The backward's gradient products take P and dS rounded to bf16
(nearest even, at most 2^-8 relative per entry), and sum n terms in fp32 (n
keys for dq, G x T queries for dk and dv; at most n 2^-24 of the terms'
magnitudes): each element of dq, dk and dv must lie within (2^-8 + n 2^-24)
times the oracle's magnitude sum of its terms (scale |dS| |k|, scale |dS|^T |q|,
P^T |dO|) plus 1e-4 max(1, max |want|) for the fp32 error of P and dS
themselves."""
import numpy as np
import pytest
import torch

from synth import synth

gpu = pytest.mark.gpu

TOL = 1e-4
TOL_LSE = 1e-5
ROUND = 2.0 ** -8   # bf16 rounding of one P or dS entry, relative
U32 = 2.0 ** -24    # fp32 unit roundoff


def grad_excess(got, want, mag, n_terms):
    """max over elements of |got - want| / allowed (at most 1 passes), the
    allowed error being (ROUND + n_terms U32) mag + TOL max(1, max |want|)."""
    allowed = (ROUND + n_terms * U32) * mag + TOL * max(1.0, float(np.max(np.abs(want))))
    return float(np.max(np.abs(got - want) / allowed))


def grad_errors(grads, refg, T, G, sel_q=None, sel_kv=None):
    """Errors of the four gradients against the oracle's (with magnitudes):
    the bound ratio for dq, dk, dv and the normalized error of dlogit."""
    sq = sel_q if sel_q is not None else (lambda x: x)
    skv = sel_kv if sel_kv is not None else (lambda x: x)
    get = lambda key, sel: sel(grads[key]).double().cpu().numpy()
    return {
        "dq": grad_excess(get("dq", sq), refg["dq"], refg["dq_mag"], T),
        "dk": grad_excess(get("dk", skv), refg["dk"], refg["dk_mag"], G * T),
        "dv": grad_excess(get("dv", skv), refg["dv"], refg["dv_mag"], G * T),
        "dlogit": _nerr(get("dlogit", skv), refg["dlogit"]),
    }


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util  # noqa: F401  (imports the HIP libraries; fails loudly if unbuilt)


def _inputs(seed, B, Hq, Hkv, T, d, mu):
    pos = np.arange(T)
    Q = synth.tensor(seed, synth.STREAM_Q, 0, np.arange(B), np.arange(Hq), pos, d, "bf16")
    K = synth.tensor(seed, synth.STREAM_K, 0, np.arange(B), np.arange(Hkv), pos, d, "bf16")
    V = synth.tensor(seed, synth.STREAM_V, 0, np.arange(B), np.arange(Hkv), pos, d, "bf16")
    # dO drawn as a query-shaped tensor of another seed (bf16-exact)
    dO = synth.tensor(seed + 1, synth.STREAM_Q, 0, np.arange(B), np.arange(Hq), pos, d, "bf16")
    lg = synth.logits(seed, 0, np.arange(B), np.arange(Hkv), pos, mu)
    g = synth.logistic_noise(seed, 0, np.arange(B), np.arange(Hkv), pos)
    return Q, K, V, dO, lg, g


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=torch.bfloat16)


def _f(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _nerr(got, want):
    return float(np.max(np.abs(got - want))) / max(1.0, float(np.max(np.abs(want))))


CASES = [
    # id, B, Hq, Hkv, T, d, w, gamma, tau, mu
    ("d128-g4-w8-ragged", 2, 8, 2, 150, 128, 8, 0.0, 1.0, 0.0),
    ("d64-g8-w0", 1, 16, 2, 97, 64, 0, -2.0, 0.5, 1.0),
    ("d128-g1-w-ge-T-no-far-keys", 1, 2, 2, 70, 128, 100, 0.0, 1.0, 0.0),
    ("d128-g5-low-tau", 1, 10, 2, 333, 128, 16, -5.0, 0.1, 5.0),
    ("d128-g5-one-token", 2, 10, 2, 1, 128, 4, 0.0, 1.0, 0.0),
    ("d64-g4-many-tiles", 1, 4, 1, 1100, 64, 64, 0.0, 1.0, -1.0),
    ("d128-g5-w32", 2, 10, 2, 417, 128, 32, 1.0, 2.0, -0.5),
]


def _run(case):
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    name, B, Hq, Hkv, T, d, w, gamma, tau, mu = case
    Q, K, V, dO, lg, g = _inputs(7000 + T + d, B, Hq, Hkv, T, d, mu)
    print(f"[{name}] B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} w={w} gamma={gamma} tau={tau}", flush=True)
    q, k, v, do = _bf(Q), _bf(K), _bf(V), _bf(dO)
    logit, noise = _f(lg), _f(g)
    out, lse = dms.soft_attention_forward(q, k, v, logit, noise, w, gamma, tau)
    grads = dms.soft_attention_backward(q, k, v, logit, noise, out, lse, do, w, gamma, tau)
    torch.cuda.synchronize()
    ref = O.soft_attention(Q, K, V, lg, g, w, gamma, tau)
    refg = O.soft_attention_grads(Q, K, V, lg, g, dO, w, gamma, tau, magnitudes=True)
    errs = {
        "out": _nerr(out.double().cpu().numpy(), ref["out"]),
        "lse": float(np.max(np.abs(lse.double().cpu().numpy() - ref["lse"]))),
    }
    errs.update(grad_errors(grads, refg, T, Hq // Hkv))
    _report(name, errs, grads, refg)
    return errs, grads, refg


def _report(name, errs, grads=None, refg=None, sel_q=None, sel_kv=None):
    """Prints the errors (dq, dk, dv as fractions of their bound), and the
    gradients' plain normalized errors."""
    line = f"[{name}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items())
    if grads is not None:
        sq = sel_q if sel_q is not None else (lambda x: x)
        skv = sel_kv if sel_kv is not None else (lambda x: x)
        plain = {k: _nerr((sq if k == "dq" else skv)(grads[k]).double().cpu().numpy(), refg[k])
                 for k in ("dq", "dk", "dv")}
        line += " | normalized " + " ".join(f"{k}={v:.2e}" for k, v in plain.items())
    print(line, flush=True)


def _check(errs, ctx):
    assert errs["lse"] <= TOL_LSE, (ctx, errs)
    for key in ("out", "dlogit"):
        assert errs[key] <= TOL, (ctx, key, errs)
    for key in ("dq", "dk", "dv"):
        assert errs[key] <= 1.0, (ctx, key, errs)


@gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_soft_attention_every_element(case):
    errs, grads, refg = _run(case)
    _check(errs, case[0])
    if case[6] >= case[4] - 1:
        # no query is more than w past any key: no key gets a logit gradient
        assert float(grads["dlogit"].abs().max()) == 0.0


@gpu
def test_soft_attention_hard_limit_equals_prompt_attention():
    """With |x| huge (tau tiny) the relaxed mask is the hard rule: the
    forward equals dms_prefill_attention (the inference path) after a
    prefill with the same logits, and no gradient reaches the logits."""
    from learned_kv_cache_dms_amd import dms
    B, Hq, Hkv, T, d, w = 2, 10, 2, 300, 128, 24
    Q, K, V, dO, lg, _ = _inputs(7500, B, Hq, Hkv, T, d, 0.3)
    lg = np.where(lg > 0, 40.0, -40.0).astype(np.float32)
    zero = np.zeros_like(lg)
    q, k, v = _bf(Q), _bf(K), _bf(V)
    out, _ = dms.soft_attention_forward(q, k, v, _f(lg), _f(zero), w, 0.0, 1e-3)
    cache = dms.Cache(B, Hq, Hkv, d, w, T + 1, B * Hkv * (T // 16 + 2), dtype="bf16")
    cache.prefill(k, v, _f(lg), [T] * B)
    hard = torch.empty((B, Hq, T, d), dtype=torch.float32, device="cuda")
    cache.prefill_attention(q, k, v, hard)
    grads = dms.soft_attention_backward(q, k, v, _f(lg), _f(zero), out, _, _bf(dO), w, 0.0, 1e-3)
    torch.cuda.synchronize()
    err = float((out - hard).abs().max())
    print(f"[hard limit] max |soft - prompt attention| = {err:.2e}", flush=True)
    # each is within its own bound of the hard attention: the prompt
    # attention's for bf16-rounded weights, and this forward's TOL
    from oracle import dms_oracle as O
    import test_gpu_prefill_attention as PA
    mag = O.prefill_attention(Q, K, np.abs(V), lg, [T] * B, w)
    allowed = (PA.ROUND + T * PA.U32) * mag + PA.TOL["bf16"] + TOL
    assert np.all(np.abs(hard.double().cpu().numpy() - out.double().cpu().numpy()) <= allowed)
    assert float(grads["dlogit"].abs().max()) == 0.0


@gpu
def test_soft_attention_full_size_sampled_heads():
    """The Qwen-R1-32B-shaped training layer (40 Q / 8 KV heads, d = 128,
    w = 256, T = 4096, tau = 0.1, gamma = -5): all heads on the GPU, two KV
    heads (with their 5 query heads each) of two sequences against the
    oracle."""
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    from synth import workloads as W
    wl = W.qwen_32b_train()
    B, Hq, Hkv, T, d, w = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim, wl.window
    G = Hq // Hkv
    q, k, v, do, logit, noise = wl.device_inputs()
    print(f"[qwen-32b training layer] B={B} Hq={Hq} T={T}", flush=True)
    out, lse = dms.soft_attention_forward(q, k, v, logit, noise, w, wl.gamma, wl.tau)
    grads = dms.soft_attention_backward(q, k, v, logit, noise, out, lse, do, w, wl.gamma, wl.tau)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (B - 1, Hkv - 1)]:
        hs = slice(h * G, (h + 1) * G)
        Q, K, V, dO, lg, g = wl.host_slice([b], [h])
        ref = O.soft_attention(Q, K, V, lg, g, w, wl.gamma, wl.tau)
        refg = O.soft_attention_grads(Q, K, V, lg, g, dO, w, wl.gamma, wl.tau, magnitudes=True)
        sq = lambda x: x[b:b + 1, hs]
        skv = lambda x: x[b:b + 1, h:h + 1]
        errs = {
            "out": _nerr(out[b:b + 1, hs].double().cpu().numpy(), ref["out"]),
            "lse": float(np.max(np.abs(lse[b:b + 1, hs].double().cpu().numpy() - ref["lse"]))),
        }
        errs.update(grad_errors(grads, refg, T, G, sq, skv))
        _report(f"b={b}, h={h}", errs, grads, refg, sq, skv)
        _check(errs, (b, h))


@gpu
def test_soft_attention_errors():
    from learned_kv_cache_dms_amd import dms
    x = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    f = torch.zeros((1, 1, 8), dtype=torch.float32, device="cuda")
    o = torch.zeros((1, 2, 8, 64), dtype=torch.float32, device="cuda")
    l = torch.zeros((1, 2, 8), dtype=torch.float32, device="cuda")
    p = lambda t: t.data_ptr()
    fneed = dms.dms_soft_attention_forward_workspace_bytes(1, 2, 1, 8, 64)
    fws = torch.empty(fneed, dtype=torch.uint8, device="cuda")
    with pytest.raises(dms.DmsError) as e:
        dms.dms_soft_attention_forward(1, 2, 1, 8, 64, 4, 0.0, 0.0, 0.0, p(x), p(x), p(x), p(f), p(f), p(o), p(l),
                                       p(fws), fneed)
    assert e.value.status == dms.DMS_ERR_ARG
    with pytest.raises(dms.DmsError) as e:
        dms.dms_soft_attention_forward(1, 2, 1, 8, 96, 4, 0.0, 1.0, 0.0, p(x), p(x), p(x), p(f), p(f), p(o), p(l),
                                       p(fws), fneed)
    assert e.value.status == dms.DMS_ERR_ARG
    with pytest.raises(dms.DmsError) as e:
        dms.dms_soft_attention_forward(1, 2, 1, 8, 64, 4, 0.0, 1.0, 0.0, p(x), p(x), p(x), p(f), p(f), p(o), p(l),
                                       p(fws), fneed - 1)
    assert e.value.status == dms.DMS_ERR_WORKSPACE
    need = dms.dms_soft_attention_backward_workspace_bytes(1, 2, 1, 8, 64)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(dms.DmsError) as e:
        dms.dms_soft_attention_backward(1, 2, 1, 8, 64, 4, 0.0, 1.0, 0.0, p(x), p(x), p(x), p(f), p(f), p(o), p(l),
                                        p(x), p(o), p(o), p(o), p(f), p(ws), need - 1)
    assert e.value.status == dms.DMS_ERR_WORKSPACE


@gpu
def test_soft_attention_long_ragged_sequence():
    """T = 6000 (not a multiple of any tile: 64 keys per dK/dV work-group,
    64 queries per dQ work-group, 192 per forward work-group, 32-row pairs):
    every output and gradient of one KV head with its query heads against
    the oracle."""
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    B, Hq, Hkv, T, d, w, gamma, tau = 1, 8, 2, 6000, 128, 256, -3.0, 0.25
    Q, K, V, dO, lg, g = _inputs(7700, B, Hq, Hkv, T, d, 3.0)
    print(f"[long ragged] T={T} Hq={Hq} Hkv={Hkv}", flush=True)
    q, k, v, do = _bf(Q), _bf(K), _bf(V), _bf(dO)
    logit, noise = _f(lg), _f(g)
    out, lse = dms.soft_attention_forward(q, k, v, logit, noise, w, gamma, tau)
    grads = dms.soft_attention_backward(q, k, v, logit, noise, out, lse, do, w, gamma, tau)
    torch.cuda.synchronize()
    h = 1
    G = Hq // Hkv
    hs = slice(h * G, (h + 1) * G)
    sl = lambda X: np.ascontiguousarray(X[:, h:h + 1])
    ref = O.soft_attention(Q[:, hs], sl(K), sl(V), sl(lg), sl(g), w, gamma, tau)
    refg = O.soft_attention_grads(Q[:, hs], sl(K), sl(V), sl(lg), sl(g), dO[:, hs], w, gamma, tau,
                                  magnitudes=True)
    sq = lambda x: x[:, hs]
    skv = lambda x: x[:, h:h + 1]
    errs = {
        "out": _nerr(out[:, hs].double().cpu().numpy(), ref["out"]),
        "lse": float(np.max(np.abs(lse[:, hs].double().cpu().numpy() - ref["lse"]))),
    }
    errs.update(grad_errors(grads, refg, T, G, sq, skv))
    _report("long ragged", errs, grads, refg, sq, skv)
    _check(errs, "long ragged")


@gpu
def test_soft_attention_on_a_side_stream():
    """Both calls on a non-default stream, with the inputs written on that
    stream just before: the results equal those of the default stream."""
    from learned_kv_cache_dms_amd import dms
    B, Hq, Hkv, T, d, w = 2, 8, 2, 300, 128, 16
    Q, K, V, dO, lg, g = _inputs(7800, B, Hq, Hkv, T, d, 0.5)
    args = [_bf(Q), _bf(K), _bf(V), _f(lg), _f(g)]
    out0, lse0 = dms.soft_attention_forward(*args, w, 0.0, 0.5)
    g0 = dms.soft_attention_backward(*args, out0, lse0, _bf(dO), w, 0.0, 0.5)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        a = [x.clone() for x in args]          # written on the side stream
        do = _bf(dO).to(torch.bfloat16)
        out1, lse1 = dms.soft_attention_forward(*a, w, 0.0, 0.5)
        g1 = dms.soft_attention_backward(*a, out1, lse1, do, w, 0.0, 0.5)
    side.synchronize()
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
    for key in g0:
        assert torch.equal(g0[key], g1[key]), key


@gpu
def test_soft_attention_autograd_function():
    """dms.soft_attention under torch autograd: out equals the forward call;
    after backward of sum(out * dO) the logits' gradient equals the backward
    call's exactly and the q, k, v gradients are its values rounded to bf16;
    the logit gradient also matches the oracle."""
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    B, Hq, Hkv, T, d, w, gamma, tau = 1, 8, 2, 200, 64, 12, -1.0, 0.5
    Q, K, V, dO, lg, g = _inputs(7900, B, Hq, Hkv, T, d, 1.0)
    q, k, v = (_bf(X).requires_grad_(True) for X in (Q, K, V))
    logit = _f(lg).requires_grad_(True)
    noise = _f(g)
    out = dms.soft_attention(q, k, v, logit, noise, w, gamma, tau)
    (out * _f(dO)).sum().backward()
    torch.cuda.synchronize()
    with torch.no_grad():
        out2, lse2 = dms.soft_attention_forward(q.detach(), k.detach(), v.detach(), logit.detach(), noise, w,
                                                gamma, tau)
        g2 = dms.soft_attention_backward(q.detach(), k.detach(), v.detach(), logit.detach(), noise, out2, lse2,
                                         _bf(dO), w, gamma, tau)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), out2)
    assert torch.equal(logit.grad, g2["dlogit"])
    for t, key in ((q, "dq"), (k, "dk"), (v, "dv")):
        assert t.grad.dtype == torch.bfloat16 and torch.equal(t.grad, g2[key].to(torch.bfloat16)), key
    ref = O.soft_attention_grads(Q, K, V, lg, g, dO, w, gamma, tau)
    assert _nerr(logit.grad.double().cpu().numpy(), ref["dlogit"]) <= TOL
