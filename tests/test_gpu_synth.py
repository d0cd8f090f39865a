"""The device twin of the generator equals the host twin bit for bit."""
import numpy as np
import pytest
import torch

from synth import synth

gpu = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fill_matches_host(dtype):
    from synth import device as D
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    out = torch.empty((3, 5, 37, 128), dtype=td, device="cuda")
    D.fill(out, 1234, synth.STREAM_K, 7, 2, pos0=1000)
    host = synth.tensor(1234, synth.STREAM_K, 7, [2, 3, 4], 5, np.arange(1000, 1037), 128, dtype)
    got = out.float().cpu().numpy()
    assert np.array_equal(got.view(np.uint32), host.astype(np.float32).view(np.uint32))


@gpu
def test_fill_per_sequence_positions():
    from synth import device as D
    pos = torch.tensor([5, 900, 32768], dtype=torch.int32, device="cuda")
    out = torch.empty((3, 4, 64), dtype=torch.bfloat16, device="cuda")
    D.fill(out, 99, synth.STREAM_Q, 0, 0, pos_base=pos)
    got = out.float().cpu().numpy()
    for i, p in enumerate([5, 900, 32768]):
        host = synth.tensor(99, synth.STREAM_Q, 0, [i], 4, [p], 64, "bf16")[0, :, 0]
        assert np.array_equal(got[i], host)


@gpu
def test_logits_match_host():
    from synth import device as D
    out = torch.empty((2, 8, 300), dtype=torch.float32, device="cuda")
    mb = np.linspace(-1, 1, 8)
    ma = np.linspace(0.5, 2.5, 8)
    D.logits(out, 1003, 5, 10, mb, ma, pos_threshold=10240, pos0=10100)
    host = synth.logits(1003, 5, [10, 11], 8, np.arange(10100, 10400), mb, ma, pos_threshold=10240)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), host.view(np.uint32))
