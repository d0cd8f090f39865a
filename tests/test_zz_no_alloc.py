"""dms_soft_attention_forward_noalloc, the allocation-free entry point, against
dms_soft_attention_forward (the caller-workspace entry point it shares its
kernels with): two calls in a row on one GPU, the second smaller, each
bit-identical to the workspace call on the same inputs; the smaller also
against the oracle.  The built-in buffer keeps the first call's contents, so
the second call's equality shows that nothing carries over."""
import numpy as np
import pytest
import torch

from oracle import dms_oracle as O
from synth import synth

gpu = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util  # noqa: F401  (imports the HIP libraries; fails loudly if unbuilt)


def _case(seed, B, Hq, Hkv, T, d, mu):
    pos = np.arange(T)
    Q = synth.tensor(seed, synth.STREAM_Q, 0, np.arange(B), np.arange(Hq), pos, d, "bf16")
    K = synth.tensor(seed, synth.STREAM_K, 0, np.arange(B), np.arange(Hkv), pos, d, "bf16")
    V = synth.tensor(seed, synth.STREAM_V, 0, np.arange(B), np.arange(Hkv), pos, d, "bf16")
    lg = synth.logits(seed, 0, np.arange(B), np.arange(Hkv), pos, mu)
    g = synth.logistic_noise(seed, 0, np.arange(B), np.arange(Hkv), pos)
    return Q, K, V, lg, g


def _dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dt)


@gpu
def test_noalloc_forward_two_calls():
    from learned_kv_cache_dms_amd import dms
    shapes = [  # (seed, B, Hq, Hkv, T, d, w, gamma, tau, mu): the second smaller than the first
        (31, 2, 8, 2, 700, 128, 16, -1.0, 0.5, 0.5),
        (32, 1, 4, 1, 90, 64, 5, 0.0, 1.0, 0.0),
    ]
    for (seed, B, Hq, Hkv, T, d, w, gamma, tau, mu) in shapes:
        Q, K, V, lg, g = _case(seed, B, Hq, Hkv, T, d, mu)
        q, k, v = (_dev(x, torch.bfloat16) for x in (Q, K, V))
        lgd, gd = _dev(lg, torch.float32), _dev(g, torch.float32)
        ref_out, ref_lse = dms.soft_attention_forward(q, k, v, lgd, gd, w, gamma, tau)
        out = torch.full((B, Hq, T, d), 7.0, dtype=torch.float32, device="cuda")
        lse = torch.full((B, Hq, T), 7.0, dtype=torch.float32, device="cuda")
        dms.soft_attention_forward_noalloc(q, k, v, lgd, gd, w, out, lse, gamma, tau)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), (T, float((out - ref_out).abs().max()))
        assert torch.equal(lse, ref_lse), T
        if T < 100:
            want = O.soft_attention(Q, K, V, lg, g, w, gamma, tau)
            got = out.double().cpu().numpy()
            err = float(np.max(np.abs(got - want["out"]))) / max(1.0, float(np.max(np.abs(want["out"]))))
            assert err <= 1e-4, err


@gpu
def test_noalloc_forward_rejects_oversized():
    """A shape whose scratch exceeds the built-in buffer is refused before
    any device work."""
    from learned_kv_cache_dms_amd import dms
    cap = dms.dms_soft_attention_forward_noalloc_max_bytes()
    B, Hq, Hkv, T, d = 4, 8, 8, 8192, 128
    assert dms.dms_soft_attention_forward_workspace_bytes(B, Hq, Hkv, T, d) > cap
    with pytest.raises(dms.DmsError) as e:
        dms.dms_soft_attention_forward_noalloc(B, Hq, Hkv, T, d, 8, 0.0, 1.0, 0.0, 1, 1, 1, 1, 1, 1, 1, 0)
    assert e.value.status == dms.DMS_ERR_TOO_LARGE
