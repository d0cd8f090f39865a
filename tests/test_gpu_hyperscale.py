"""The hyper-scaling runner end to end on the GPU: the device's counters of
memory reads and peak live tokens equal the counts implied by the decisions."""
import dataclasses

import pytest
import torch

from synth import workloads as W

gpu = pytest.mark.gpu


@gpu
def test_runner_counts_match_decisions():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util  # noqa: F401
    from learned_kv_cache_dms_amd import hyperscale as H
    wl = dataclasses.replace(W.qwen_32b_hyperscale(), num_q_heads=8, num_kv_heads=4, head_dim=64,
                             prompt_len=300, window=16)
    for width, length in ((3, 257), (9, 40)):
        print(f"[hyperscale runner] chains={width} tokens={length}", flush=True)
        r = H.run_config(wl, width, length, chunk=100)
        assert r.reads_device == r.reads_exact, (width, length, r)
        assert r.peak_device == r.peak_exact, (width, length, r)
        assert r.tokens_per_s > 0
