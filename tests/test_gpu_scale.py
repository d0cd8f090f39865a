"""GPU parity with an attention scale other than the default 1/sqrt(d)
(dms_config.scale for the cache's calls, the scale argument of the relaxed
attention) against the oracle given the same scale: decode steps, the
prompt attention, a chunk and the relaxed attention's forward and backward."""
import numpy as np
import pytest
import torch

from synth import synth

gpu = pytest.mark.gpu

SCALE = 0.29  # far from 1/sqrt(128) = 0.088 and 1/sqrt(64) = 0.125


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util  # noqa: F401  (imports the HIP libraries; fails loudly if unbuilt)


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=torch.bfloat16)


def _f(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


@gpu
def test_cache_paths_with_explicit_scale():
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    B, Hq, Hkv, d, w, P, steps, C = 2, 8, 2, 128, 8, 120, 6, 5
    T = P + steps + C
    pos = np.arange(T)
    Q = synth.tensor(8100, synth.STREAM_Q, 0, np.arange(B), np.arange(Hq), pos, d, "bf16")
    K = synth.tensor(8100, synth.STREAM_K, 0, np.arange(B), np.arange(Hkv), pos, d, "bf16")
    V = synth.tensor(8100, synth.STREAM_V, 0, np.arange(B), np.arange(Hkv), pos, d, "bf16")
    lg = synth.logits(8100, 0, np.arange(B), np.arange(Hkv), pos, 0.4)
    cache = dms.Cache(B, Hq, Hkv, d, w, T, B * Hkv * (T // 16 + 2), dtype="bf16", scale=SCALE)
    cache.prefill(_bf(K[:, :, :P]), _bf(V[:, :, :P]), _f(lg[:, :, :P]), [P] * B)
    # the prompt's own queries
    out_p = torch.empty((B, Hq, P, d), dtype=torch.float32, device="cuda")
    cache.prefill_attention(_bf(Q[:, :, :P]), _bf(K[:, :, :P]), _bf(V[:, :, :P]), out_p)
    ref_p = O.prefill_attention(Q[:, :, :P], K[:, :, :P], V[:, :, :P], lg[:, :, :P], [P] * B, w, scale=SCALE)
    mag_p = O.prefill_attention(Q[:, :, :P], K[:, :, :P], np.abs(V[:, :, :P]), lg[:, :, :P], [P] * B, w,
                                scale=SCALE)
    from test_gpu_prefill_attention import excess
    assert excess(out_p.double().cpu().numpy(), ref_p, mag_p, P, "bf16") <= 1.0
    # decode steps, then one chunk
    ref = O.decode_batch(Q, K, V, lg, [P] * B, steps + C, w, scale=SCALE)
    for t in range(steps):
        q = P + t
        cache.append(_bf(K[:, :, q]), _bf(V[:, :, q]), _f(lg[:, :, q]))
        out = cache.attend(_bf(Q[:, :, q]))
        torch.cuda.synchronize()
        assert float(np.max(np.abs(out.double().cpu().numpy() - ref["out"][t]))) <= 1e-4, t
    s0 = P + steps
    out_c = cache.decode_chunk(_bf(Q[:, :, s0:s0 + C]), _bf(K[:, :, s0:s0 + C]), _bf(V[:, :, s0:s0 + C]),
                               _f(lg[:, :, s0:s0 + C]))
    torch.cuda.synchronize()
    want = ref["out"][steps:steps + C].transpose(1, 2, 0, 3)
    assert float(np.max(np.abs(out_c.double().cpu().numpy() - want))) <= 1e-4


@gpu
def test_relaxed_attention_with_explicit_scale():
    from learned_kv_cache_dms_amd import dms
    from oracle import dms_oracle as O
    B, Hq, Hkv, T, d, w, gamma, tau = 1, 4, 2, 150, 64, 10, 0.0, 1.0
    pos = np.arange(T)
    Q = synth.tensor(8200, synth.STREAM_Q, 0, [0], np.arange(Hq), pos, d, "bf16")
    K = synth.tensor(8200, synth.STREAM_K, 0, [0], np.arange(Hkv), pos, d, "bf16")
    V = synth.tensor(8200, synth.STREAM_V, 0, [0], np.arange(Hkv), pos, d, "bf16")
    dO = synth.tensor(8201, synth.STREAM_Q, 0, [0], np.arange(Hq), pos, d, "bf16")
    lg = synth.logits(8200, 0, [0], np.arange(Hkv), pos, 0.0)
    g = synth.logistic_noise(8200, 0, [0], np.arange(Hkv), pos)
    args = (_bf(Q), _bf(K), _bf(V), _f(lg), _f(g))
    out, lse = dms.soft_attention_forward(*args, w, gamma, tau, scale=SCALE)
    grads = dms.soft_attention_backward(*args, out, lse, _bf(dO), w, gamma, tau, scale=SCALE)
    torch.cuda.synchronize()
    ref = O.soft_attention(Q, K, V, lg, g, w, gamma, tau, scale=SCALE)
    refg = O.soft_attention_grads(Q, K, V, lg, g, dO, w, gamma, tau, scale=SCALE, magnitudes=True)
    from test_gpu_soft_attention import grad_errors
    nerr = lambda a, b: float(np.max(np.abs(a - b))) / max(1.0, float(np.max(np.abs(b))))
    assert nerr(out.double().cpu().numpy(), ref["out"]) <= 1e-4
    assert float(np.max(np.abs(lse.double().cpu().numpy() - ref["lse"]))) <= 1e-5
    errs = grad_errors(grads, refg, T, Hq // Hkv)
    for key in ("dq", "dk", "dv"):
        assert errs[key] <= 1.0, (key, errs)   # fractions of the bf16-rounding bound
    assert errs["dlogit"] <= 1e-4, errs
