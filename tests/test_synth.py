"""Host twin of the synthetic generator (CPU)."""
import math

import numpy as np
import torch

from synth import synth, workloads


def test_splitmix64_published_vectors():
    # Reference outputs of Vigna's splitmix64 generator: seed 0 gives
    # 0xE220A8397B1DCDAF first; seed 1234567 gives the sequence below.
    assert int(synth.splitmix64(np.array([0], dtype=np.uint64))[0]) == 0xE220A8397B1DCDAF
    st = np.array([1234567], dtype=np.uint64)
    got = []
    for _ in range(5):
        got.append(int(synth.splitmix64(st)[0]))
        st = st + np.uint64(0x9E3779B97F4A7C15)
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_irwin_hall_moments_and_range():
    x = synth.normal_from_index(42, synth.STREAM_K, np.arange(2_000_000))
    assert x.dtype == np.float32
    assert abs(float(x.mean())) < 5 * math.sqrt(1 / 2e6)
    assert abs(float(x.var()) - 1.0) < 0.01
    assert float(np.abs(x).max()) <= 6.0
    # exactness: every value is an integer multiple of 2**-17
    assert np.all((x.astype(np.float64) * 2 ** 17) == np.round(x.astype(np.float64) * 2 ** 17))


def test_deterministic_and_shape_independent():
    a = synth.tensor(7, synth.STREAM_V, 3, [0, 1, 2], 4, np.arange(10), 16)
    b = synth.tensor(7, synth.STREAM_V, 3, [2], 4, np.arange(5, 10), 16)
    assert np.array_equal(a[2, :, 5:10], b[0])
    c = synth.tensor(8, synth.STREAM_V, 3, [2], 4, np.arange(5, 10), 16)
    assert not np.array_equal(b, c)


def test_bf16_rounding_matches_torch_nearest_even():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    # include exact ties
    ties = (np.arange(1, 1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ours = synth.round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_logits_one_rounding_and_threshold():
    pos = np.arange(12000)
    lg = synth.logits(5, 0, [0], 2, pos, [0.5, -0.5], [1.5, 2.5], pos_threshold=10240)
    x = synth.normal_from_index(5, synth.STREAM_LOGIT,
                                synth.flat_index(0, 0, np.arange(2)[:, None], pos[None], 0))
    mu = np.where(pos[None] < 10240, np.array([[0.5], [-0.5]]), np.array([[1.5], [2.5]]))
    assert np.array_equal(lg[0], (mu + x.astype(np.float64)).astype(np.float32))


def test_lengths_in_range():
    L = synth.lengths(1004, 256, 1024, 32768)
    assert L.min() >= 1024 and L.max() <= 32768
    assert abs(L.mean() - (1024 + 32768) / 2) < 4 * (32768 - 1024) / math.sqrt(12 * 256)


def test_workload_recipes():
    assert abs(workloads.mu_for_cr(4) - 0.6745) < 1e-4
    assert abs(workloads.mu_for_cr(8) - 1.1503) < 1e-4
    assert abs(workloads.mu_for_cr(12) - 1.3830) < 1e-4
    w = workloads.qwen_32b()
    assert (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim) == (64, 40, 8, 128)
    assert w.max_tokens() == 32768 + 256
    n = w.expected_live(0, 32768 + 127)
    assert 4500 < n < 4900
    f = workloads.full_32b()
    assert len(f.mu_before) == 64


def test_logistic_noise_distribution_and_addressing():
    """Logistic(0, 1): CDF 1 / (1 + e^-g) at a few points and variance pi^2 / 3
    (within 5 standard errors for 400K samples); values addressed by counter,
    not by the shape of the draw."""
    g = synth.logistic_noise(11, 0, np.arange(4), 4, np.arange(25000)).astype(np.float64).ravel()
    n = g.size
    for x in (-np.log(3.0), 0.0, np.log(3.0), 3.0):
        p = 1.0 / (1.0 + np.exp(-x))
        assert abs(np.mean(g <= x) - p) < 5 * np.sqrt(p * (1 - p) / n), x
    assert abs(np.var(g) - np.pi ** 2 / 3) < 0.05
    part = synth.logistic_noise(11, 0, [2], [3], np.arange(100, 200))
    full = synth.logistic_noise(11, 0, np.arange(4), 4, np.arange(25000))
    assert np.array_equal(part[0, 0], full[2, 3, 100:200])
    assert np.all(np.isfinite(g))


def test_device_library_exports():
    """The device twin's library loads and exports its entry points (no GPU
    call is made)."""
    from synth import device
    for name in ("synth_fill", "synth_logits", "synth_read"):
        assert hasattr(device.lib, name), name
