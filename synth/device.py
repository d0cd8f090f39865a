"""Device twin of the synthetic generator (binding to synth/libdms_synth.so).

Writes the values defined in ``synth.synth`` straight into torch tensors on
the GPU.  Bit-identical to the host twin (checked by the tests).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdms_synth.so")


def _bind_hip_runtime():
    """torch ships its own HIP runtime.  Loading it before the library makes
    the library bind to that same runtime, so device pointers and streams
    from torch are valid here; loaded the other way round a process can end
    up with two HIP runtimes that do not share state."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def _load():
    _bind_hip_runtime()
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} missing; build with `python -m learned_kv_cache_dms_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    lib.synth_fill.restype = ctypes.c_int
    lib.synth_fill.argtypes = [vp, i32, u64, i32, i32, i32, i32, i32, vp, i32, i32, i32, vp]
    lib.synth_logits.restype = ctypes.c_int
    dp = ctypes.POINTER(ctypes.c_double)
    lib.synth_logits.argtypes = [vp, u64, i32, i32, i32, i32, vp, i32, i32, dp, dp, i32, vp]
    lib.synth_read.restype = ctypes.c_int
    lib.synth_read.argtypes = [vp, ctypes.c_int64, i32, vp, vp]
    return lib


lib = _load()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fill(out, seed: int, stream: int, layer: int, b0: int, pos0: int = 0, pos_base=None):
    """out: contiguous cuda tensor [nb, heads, npos, channels] (float32 or
    bfloat16) or [nb, heads, channels] (one position per sequence)."""
    import torch
    shape = tuple(out.shape)
    if len(shape) == 3:
        nb, heads, ch = shape
        npos = 1
    else:
        nb, heads, npos, ch = shape
    assert out.is_contiguous() and out.dtype in (torch.float32, torch.bfloat16)
    pb = 0 if pos_base is None else pos_base.data_ptr()
    rc = lib.synth_fill(out.data_ptr(), 1 if out.dtype == torch.bfloat16 else 0, seed, stream, layer, b0, nb,
                        heads, pb, pos0, npos, ch, _stream())
    if rc != 0:
        raise RuntimeError(f"synth_fill failed ({rc})")
    return out


def logits(out, seed: int, layer: int, b0: int, mu_before, mu_after=None, pos_threshold: int = 1 << 20,
           pos0: int = 0, pos_base=None):
    """out: contiguous float32 cuda tensor [nb, heads, npos] or [nb, heads]."""
    import torch
    shape = tuple(out.shape)
    nb, heads = shape[0], shape[1]
    npos = shape[2] if len(shape) == 3 else 1
    assert out.is_contiguous() and out.dtype == torch.float32
    mb = np.ascontiguousarray(np.broadcast_to(np.asarray(mu_before, dtype=np.float64), (heads,)))
    ma = mb if mu_after is None else np.ascontiguousarray(
        np.broadcast_to(np.asarray(mu_after, dtype=np.float64), (heads,)))
    dp = ctypes.POINTER(ctypes.c_double)
    pb = 0 if pos_base is None else pos_base.data_ptr()
    rc = lib.synth_logits(out.data_ptr(), seed, layer, b0, nb, heads, pb, pos0, npos,
                          mb.ctypes.data_as(dp), ma.ctypes.data_as(dp), pos_threshold, _stream())
    if rc != 0:
        raise RuntimeError(f"synth_logits failed ({rc})")
    return out


def stream_read(src, grid: int, sink):
    """One plain streaming read of the uint8 cuda tensor `src` (length a
    multiple of 16) by `grid` work-groups; sink: uint32 cuda tensor [grid]."""
    rc = lib.synth_read(src.data_ptr(), src.numel(), int(grid), sink.data_ptr(), _stream())
    if rc != 0:
        raise RuntimeError(f"synth_read failed ({rc})")
