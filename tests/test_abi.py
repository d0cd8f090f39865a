"""The C-ABI library loads and exports what include/dms.h declares; host-side
validation that returns before any device work (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dms.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dms_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_path_calls():
    names = _declared()
    for required in ("dms_cache_create", "dms_append_step", "dms_decode_attention", "dms_prefill_compress"):
        assert required in names


def test_library_exports_every_declared_symbol():
    from learned_kv_cache_dms_amd import dms
    lib = ctypes.CDLL(dms.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_synth_library_loads():
    from synth import device
    assert hasattr(device.lib, "synth_fill") and hasattr(device.lib, "synth_logits")


def _cfg(**kw):
    from learned_kv_cache_dms_amd import dms
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, window=16, max_tokens=300,
                pool_blocks=64, dtype=dms.DMS_BF16)
    base.update(kw)
    return dms.make_config(**base)


def test_workspace_bytes_valid_and_monotone():
    from learned_kv_cache_dms_amd import dms
    a = dms.dms_workspace_bytes(_cfg())
    b = dms.dms_workspace_bytes(_cfg(pool_blocks=65))
    c = dms.dms_workspace_bytes(_cfg(dtype=dms.DMS_F32))
    assert a > 64 * 8192 and b >= a + 8192 and c > a
    assert a % 256 == 0


@pytest.mark.parametrize("bad", [
    dict(num_q_heads=7), dict(num_q_heads=40, num_kv_heads=2), dict(head_dim=96), dict(window=-1),
    dict(block_tokens=8), dict(max_tokens=0), dict(pool_blocks=0), dict(dtype=5), dict(batch=0),
    dict(scale=float("nan")), dict(split_wgs=-1),
])
def test_workspace_bytes_rejects_invalid(bad):
    from learned_kv_cache_dms_amd import dms
    assert dms.dms_workspace_bytes(_cfg(**bad)) == 0


def test_create_validates_before_touching_the_device():
    from learned_kv_cache_dms_amd import dms
    cfg = _cfg()
    need = dms.dms_workspace_bytes(cfg)
    h = ctypes.c_void_p()
    assert dms.lib.dms_cache_create(ctypes.byref(cfg), None, need, None, ctypes.byref(h)) == dms.DMS_ERR_ARG
    assert dms.lib.dms_cache_create(ctypes.byref(cfg), 0x1001, need, None, ctypes.byref(h)) == dms.DMS_ERR_WORKSPACE
    assert dms.lib.dms_cache_create(ctypes.byref(cfg), 0x1000, need - 1, None, ctypes.byref(h)) == \
        dms.DMS_ERR_WORKSPACE
    bad = _cfg(head_dim=32)
    assert dms.lib.dms_cache_create(ctypes.byref(bad), 0x1000, need, None, ctypes.byref(h)) == dms.DMS_ERR_ARG
    assert dms.lib.dms_cache_create(ctypes.byref(cfg), 0x1000, need, None, None) == dms.DMS_ERR_ARG


def test_null_handle_calls_are_argument_errors():
    from learned_kv_cache_dms_amd import dms
    L = dms.lib
    assert L.dms_cache_reset(None, None) == dms.DMS_ERR_ARG
    assert L.dms_append_step(None, 1, 1, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_decode_attention(None, 1, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_decode_attention_timed(None, 1, 1, 1, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_prefill_attention(None, 1, 1, 1, 1, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_decode_chunk(None, 1, 1, 1, 1, 1, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_decode_chunk_channel(None, 1, 1, 1, 0, 0, 0, 1, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_prefill_compress(None, 1, 1, 1, None, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_append_step_channel(None, 1, 1, None, 0, 0, 0, None) == dms.DMS_ERR_ARG
    assert L.dms_prefill_compress_channel(None, 1, 1, None, 0, 0, 0, None, 1, None) == dms.DMS_ERR_ARG
    assert L.dms_cache_stats(None, None, None) == dms.DMS_ERR_ARG
    assert L.dms_cache_export(None, 0, 0, None, None, None, None) == dms.DMS_ERR_ARG
    assert L.dms_cache_destroy(None) == dms.DMS_OK


def test_status_strings():
    from learned_kv_cache_dms_amd import dms
    for code in range(0, -8, -1):
        assert dms.dms_status_str(code).startswith("DMS_")
    assert "unknown" in dms.dms_status_str(42)


def test_soft_attention_validates_before_touching_the_device():
    from learned_kv_cache_dms_amd import dms
    L = dms.lib
    ok = (1, 4, 2, 100, 128, 8, 0.0, 1.0, 0.0)
    fneed = dms.dms_soft_attention_forward_workspace_bytes(1, 4, 2, 100, 128)
    # v in the transposed operand layout (rows padded to 32) per KV head, then the keys' bias
    assert fneed == 2 * 128 * 128 * 2 + 2 * 128 * 4
    data = [0x1000] * 7

    def fwd(*shape_and_params, ptrs=data, ws=0x1000, nbytes=fneed):
        return L.dms_soft_attention_forward(*shape_and_params, *ptrs, ws, nbytes, None)

    assert fwd(*ok, ptrs=[None] + data[1:]) == dms.DMS_ERR_ARG
    assert fwd(*ok, ws=None) == dms.DMS_ERR_ARG
    assert fwd(*ok, ws=0x1001) == dms.DMS_ERR_WORKSPACE
    assert fwd(*ok, nbytes=fneed - 1) == dms.DMS_ERR_WORKSPACE
    for bad in [(1, 3, 2, 100, 128), (1, 4, 2, 0, 128), (1, 4, 2, 100, 96), (0, 4, 2, 100, 128),
                (1, 4, 2, (1 << 20) + 1, 128)]:
        assert fwd(*bad, 8, 0.0, 1.0, 0.0) == dms.DMS_ERR_ARG, bad
        assert dms.dms_soft_attention_forward_workspace_bytes(*bad) == 0
        assert dms.dms_soft_attention_backward_workspace_bytes(*bad) == 0
    for tau in (0.0, -1.0, float("nan"), float("inf")):
        assert fwd(1, 4, 2, 100, 128, 8, 0.0, tau, 0.0) == dms.DMS_ERR_ARG
    assert fwd(1, 4, 2, 100, 128, -1, 0.0, 1.0, 0.0) == dms.DMS_ERR_ARG
    assert fwd(1, 4, 2, 100, 128, 8, float("nan"), 1.0, 0.0) == dms.DMS_ERR_ARG
    need = dms.dms_soft_attention_backward_workspace_bytes(1, 4, 2, 100, 128)
    # q and dO copies per query head, k per KV head, then delta and the keys' bias
    assert need == (4 * 2 + 2) * 128 * 128 * 2 + 4 * 100 * 4 + 2 * 128 * 4
    bptrs = [0x1000] * 12
    assert L.dms_soft_attention_backward(*ok, *bptrs, 0x1001, need, None) == dms.DMS_ERR_WORKSPACE
    assert L.dms_soft_attention_backward(*ok, *bptrs, 0x1000, need - 1, None) == dms.DMS_ERR_WORKSPACE
    assert L.dms_soft_attention_backward(*ok, *bptrs, None, need, None) == dms.DMS_ERR_ARG
