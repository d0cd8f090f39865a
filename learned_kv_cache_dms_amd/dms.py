"""Python binding of the DMS C ABI (include/dms.h).

Argument marshalling only: every step of the decode path runs in the HIP
library ``libdms_hip.so``.  Importing this module fails loudly if that
library has not been built; there is no fallback.

The functions keep the C names.  ``Cache`` is a convenience wrapper that
allocates the workspace with torch and passes ``data_ptr()`` values and the
current HIP stream; torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdms_hip.so")

DMS_F32 = 0
DMS_BF16 = 1

DMS_OK = 0
DMS_ERR_ARG = -1
DMS_ERR_WORKSPACE = -2
DMS_ERR_OUT_OF_BLOCKS = -3
DMS_ERR_CAPACITY = -4
DMS_ERR_STATE = -5
DMS_ERR_HIP = -6
DMS_ERR_DEVICE = -7
DMS_ERR_TOO_LARGE = -8

DMS_LOGIT_FROM_K = 0
DMS_LOGIT_FROM_Q = 1


class DmsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dms_status_str(status)} ({status})")


class dms_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("split_wgs", ctypes.c_int32),
        ("pool_blocks", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class dms_stats(ctypes.Structure):
    _fields_ = [
        ("live_tokens", ctypes.c_int64),
        ("seen_tokens", ctypes.c_int64),
        ("allocated_blocks", ctypes.c_int64),
        ("live_token_steps", ctypes.c_int64),
        ("sticky_error", ctypes.c_int32),
        ("split_mode", ctypes.c_int32),
    ]


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
        raise ImportError(
            f"DMS HIP library not found at {LIB_PATH}; build it with "
            "`python -m learned_kv_cache_dms_amd.build` (needs ROCm hipcc).")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "dms_workspace_bytes": (sz, [P(dms_config)]),
        "dms_cache_create": (ctypes.c_int, [P(dms_config), vp, sz, vp, P(vp)]),
        "dms_cache_destroy": (ctypes.c_int, [vp]),
        "dms_cache_reset": (ctypes.c_int, [vp, vp]),
        "dms_prefill_compress": (ctypes.c_int, [vp, vp, vp, vp, P(i32), i32, vp]),
        "dms_append_step": (ctypes.c_int, [vp, vp, vp, vp, vp]),
        "dms_append_step_channel": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp]),
        "dms_prefill_compress_channel": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, P(i32), i32, vp]),
        "dms_decode_attention": (ctypes.c_int, [vp, vp, vp, vp]),
        "dms_decode_attention_timed": (ctypes.c_int, [vp, vp, vp, vp, vp, vp]),
        "dms_decode_step": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp]),
        "dms_decode_step_timed": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "dms_decode_step_channel": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp, vp]),
        "dms_cache_balance": (ctypes.c_int, [vp, vp]),
        "dms_prefill_attention": (ctypes.c_int, [vp, vp, vp, vp, i32, vp, vp]),
        "dms_decode_chunk": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, vp]),
        "dms_decode_chunk_channel": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]),
        "dms_cache_stats": (ctypes.c_int, [vp, P(dms_stats), vp]),
        "dms_cache_export": (ctypes.c_int, [vp, i32, i32, P(i32), P(i32), P(i32), vp]),
        "dms_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "dms_soft_attention_forward": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                                      ctypes.c_float, ctypes.c_float] + [vp] * 8 + [sz, vp]),
        "dms_soft_attention_forward_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "dms_soft_attention_forward_noalloc": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                                              ctypes.c_float, ctypes.c_float] + [vp] * 7 + [vp]),
        "dms_soft_attention_forward_noalloc_max_bytes": (sz, []),
        "dms_soft_attention_backward_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "dms_soft_attention_backward": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                                       ctypes.c_float, ctypes.c_float] + [vp] * 13 + [sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int, where: str):
    if status != DMS_OK:
        raise DmsError(status, where)


def _i32p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def make_config(batch, num_q_heads, num_kv_heads, head_dim, window, max_tokens, pool_blocks,
                dtype=DMS_BF16, split_wgs=0, scale=0.0, block_tokens=16) -> dms_config:
    return dms_config(batch, num_q_heads, num_kv_heads, head_dim, window, block_tokens, max_tokens,
                      split_wgs, pool_blocks, dtype, scale)


def dms_status_str(status: int) -> str:
    return lib.dms_status_str(int(status)).decode()


def dms_workspace_bytes(cfg: dms_config) -> int:
    return int(lib.dms_workspace_bytes(ctypes.byref(cfg)))


def dms_cache_create(cfg: dms_config, d_workspace: int, workspace_bytes: int, stream: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(lib.dms_cache_create(ctypes.byref(cfg), d_workspace, workspace_bytes, stream, ctypes.byref(h)),
           "dms_cache_create")
    return h.value


def dms_cache_destroy(h: int):
    _check(lib.dms_cache_destroy(h), "dms_cache_destroy")


def dms_cache_reset(h: int, stream: int = 0):
    _check(lib.dms_cache_reset(h, stream), "dms_cache_reset")


def dms_prefill_compress(h: int, d_k: int, d_v: int, d_logit: int, lengths: Sequence[int], max_len: int,
                         stream: int = 0):
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    _check(lib.dms_prefill_compress(h, d_k, d_v, d_logit, _i32p(L), int(max_len), stream),
           "dms_prefill_compress")


def dms_append_step(h: int, d_k: int, d_v: int, d_logit: int, stream: int = 0):
    _check(lib.dms_append_step(h, d_k, d_v, d_logit, stream), "dms_append_step")


def dms_append_step_channel(h: int, d_k: int, d_v: int, d_q: Optional[int], source: int, channel: int,
                            zero_channel: bool, stream: int = 0):
    _check(lib.dms_append_step_channel(h, d_k, d_v, d_q, int(source), int(channel), int(bool(zero_channel)),
                                       stream), "dms_append_step_channel")


def dms_prefill_compress_channel(h: int, d_k: int, d_v: int, d_q: Optional[int], source: int, channel: int,
                                 zero_channel: bool, lengths: Sequence[int], max_len: int, stream: int = 0):
    L = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    _check(lib.dms_prefill_compress_channel(h, d_k, d_v, d_q, int(source), int(channel),
                                            int(bool(zero_channel)), _i32p(L), int(max_len), stream),
           "dms_prefill_compress_channel")


def dms_prefill_attention(h: int, d_q: int, d_k: int, d_v: int, max_len: int, d_out: int, stream: int = 0):
    _check(lib.dms_prefill_attention(h, d_q, d_k, d_v, int(max_len), d_out, stream), "dms_prefill_attention")


def dms_decode_chunk(h: int, d_q: int, d_k: int, d_v: int, d_logit: int, chunk: int, d_out: int, stream: int = 0):
    _check(lib.dms_decode_chunk(h, d_q, d_k, d_v, d_logit, int(chunk), d_out, stream), "dms_decode_chunk")


def dms_decode_chunk_channel(h: int, d_q: int, d_k: int, d_v: int, source: int, channel: int, zero_channel: bool,
                             chunk: int, d_out: int, stream: int = 0):
    _check(lib.dms_decode_chunk_channel(h, d_q, d_k, d_v, int(source), int(channel), int(bool(zero_channel)),
                                        int(chunk), d_out, stream), "dms_decode_chunk_channel")


def dms_decode_attention(h: int, d_q: int, d_out: int, stream: int = 0):
    _check(lib.dms_decode_attention(h, d_q, d_out, stream), "dms_decode_attention")


def dms_decode_attention_timed(h: int, d_q: int, d_out: int, start_event: int, stop_event: int, stream: int = 0):
    _check(lib.dms_decode_attention_timed(h, d_q, d_out, start_event, stop_event, stream),
           "dms_decode_attention_timed")


def dms_decode_step(h: int, d_q: int, d_k: int, d_v: int, d_logit: int, d_out: int, stream: int = 0):
    _check(lib.dms_decode_step(h, d_q, d_k, d_v, d_logit, d_out, stream), "dms_decode_step")


def dms_decode_step_timed(h: int, d_q: int, d_k: int, d_v: int, d_logit: int, d_out: int, start_event: int,
                          stop_event: int, stream: int = 0):
    _check(lib.dms_decode_step_timed(h, d_q, d_k, d_v, d_logit, d_out, start_event, stop_event, stream),
           "dms_decode_step_timed")


def dms_decode_step_channel(h: int, d_q: int, d_k: int, d_v: int, source: int, channel: int, zero_channel: bool,
                            d_out: int, stream: int = 0):
    _check(lib.dms_decode_step_channel(h, d_q, d_k, d_v, int(source), int(channel), int(bool(zero_channel)), d_out,
                                       stream), "dms_decode_step_channel")


def dms_cache_balance(h: int, stream: int = 0):
    _check(lib.dms_cache_balance(h, stream), "dms_cache_balance")


_hip = None


def _hip_api():
    """The process's HIP runtime (the one torch loaded; opening its soname
    returns that same library), for the events of dms_decode_attention_timed."""
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so.7")
        vp = ctypes.c_void_p
        h.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
        h.hipEventDestroy.argtypes = [vp]
        h.hipEventSynchronize.argtypes = [vp]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        for f in (h.hipEventCreate, h.hipEventDestroy, h.hipEventSynchronize, h.hipEventElapsedTime):
            f.restype = ctypes.c_int
        _hip = h
    return _hip


class KernelTimer:
    """A start / stop pair of HIP events (timing enabled) for
    dms_decode_attention_timed, which has the runtime stamp them with the
    start and the end of the call's own kernels."""

    def __init__(self):
        h = _hip_api()
        self.start, self.stop = ctypes.c_void_p(), ctypes.c_void_p()
        for e in (self.start, self.stop):
            rc = h.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")

    def elapsed_ms(self) -> float:
        h = _hip_api()
        rc = h.hipEventSynchronize(self.stop)
        t = ctypes.c_float()
        if rc == 0:
            rc = h.hipEventElapsedTime(ctypes.byref(t), self.start, self.stop)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return t.value

    @staticmethod
    def between(a: "KernelTimer", b: "KernelTimer") -> float:
        """ms from the end of a's kernels to the end of b's."""
        h = _hip_api()
        t = ctypes.c_float()
        rc = h.hipEventSynchronize(b.stop)
        if rc == 0:
            rc = h.hipEventElapsedTime(ctypes.byref(t), a.stop, b.stop)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return t.value

    def close(self):
        h = _hip_api()
        for e in (self.start, self.stop):
            if e.value:
                h.hipEventDestroy(e)
                e.value = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dms_cache_stats(h: int, stream: int = 0) -> dict:
    s = dms_stats()
    _check(lib.dms_cache_stats(h, ctypes.byref(s), stream), "dms_cache_stats")
    return {k: getattr(s, k) for k, _ in dms_stats._fields_ if k != "reserved"}


def dms_cache_export(h: int, unit_begin: int, unit_count: int, slot_pos: Optional[np.ndarray],
                     ring: Optional[np.ndarray], n: Optional[np.ndarray], stream: int = 0):
    _check(lib.dms_cache_export(h, unit_begin, unit_count, _i32p(slot_pos), _i32p(ring), _i32p(n), stream),
           "dms_cache_export")


def dms_soft_attention_forward_workspace_bytes(B, Hq, Hkv, T, d) -> int:
    return int(lib.dms_soft_attention_forward_workspace_bytes(int(B), int(Hq), int(Hkv), int(T), int(d)))


def dms_soft_attention_forward(B, Hq, Hkv, T, d, window, gamma, tau, scale, d_q, d_k, d_v, d_logit, d_noise,
                               d_out, d_lse, d_workspace, workspace_bytes, stream: int = 0):
    _check(lib.dms_soft_attention_forward(int(B), int(Hq), int(Hkv), int(T), int(d), int(window), float(gamma),
                                          float(tau), float(scale), d_q, d_k, d_v, d_logit, d_noise, d_out, d_lse,
                                          d_workspace, int(workspace_bytes), stream), "dms_soft_attention_forward")


def dms_soft_attention_forward_noalloc(B, Hq, Hkv, T, d, window, gamma, tau, scale, d_q, d_k, d_v, d_logit,
                                       d_noise, d_out, d_lse, stream: int = 0):
    _check(lib.dms_soft_attention_forward_noalloc(int(B), int(Hq), int(Hkv), int(T), int(d), int(window),
                                                  float(gamma), float(tau), float(scale), d_q, d_k, d_v, d_logit,
                                                  d_noise, d_out, d_lse, stream), "dms_soft_attention_forward_noalloc")


def dms_soft_attention_forward_noalloc_max_bytes() -> int:
    return int(lib.dms_soft_attention_forward_noalloc_max_bytes())


def dms_soft_attention_backward_workspace_bytes(B, Hq, Hkv, T, d) -> int:
    return int(lib.dms_soft_attention_backward_workspace_bytes(int(B), int(Hq), int(Hkv), int(T), int(d)))


def dms_soft_attention_backward(B, Hq, Hkv, T, d, window, gamma, tau, scale, d_q, d_k, d_v, d_logit, d_noise,
                                d_out, d_lse, d_dout, d_dq, d_dk, d_dv, d_dlogit, d_workspace, workspace_bytes,
                                stream: int = 0):
    _check(lib.dms_soft_attention_backward(int(B), int(Hq), int(Hkv), int(T), int(d), int(window), float(gamma),
                                           float(tau), float(scale), d_q, d_k, d_v, d_logit, d_noise, d_out, d_lse,
                                           d_dout, d_dq, d_dk, d_dv, d_dlogit, d_workspace, int(workspace_bytes),
                                           stream), "dms_soft_attention_backward")


def _soft_check(q, k, v, logit, noise):
    import torch
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    for t, shape, dt, name in ((q, (B, Hq, T, d), torch.bfloat16, "q"), (k, (B, Hkv, T, d), torch.bfloat16, "k"),
                               (v, (B, Hkv, T, d), torch.bfloat16, "v"), (logit, (B, Hkv, T), torch.float32, "logit"),
                               (noise, (B, Hkv, T), torch.float32, "noise")):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name}: expected contiguous {dt} {shape} on the GPU, got "
                             f"{t.dtype} {tuple(t.shape)}")
    return B, Hq, Hkv, T, d


def soft_attention_forward(q, k, v, logit, noise, window, gamma=0.0, tau=1.0, scale=0.0, out=None, lse=None,
                           workspace=None):
    """Relaxed DMS attention forward (dms_soft_attention_forward) on torch
    tensors: returns (out, lse), fp32; outputs and workspace are allocated
    here unless given."""
    import torch
    B, Hq, Hkv, T, d = _soft_check(q, k, v, logit, noise)
    if out is None:
        out = torch.empty((B, Hq, T, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(dms_soft_attention_forward_workspace_bytes(B, Hq, Hkv, T, d), dtype=torch.uint8,
                                device=q.device)
    dms_soft_attention_forward(B, Hq, Hkv, T, d, window, gamma, tau, scale, q.data_ptr(), k.data_ptr(),
                               v.data_ptr(), logit.data_ptr(), noise.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               workspace.data_ptr(), workspace.numel(), torch.cuda.current_stream().cuda_stream)
    return out, lse


def soft_attention_forward_noalloc(q, k, v, logit, noise, window, out, lse, gamma=0.0, tau=1.0, scale=0.0):
    """dms_soft_attention_forward_noalloc on torch tensors: the caller passes
    out [B, Hq, T, d] and lse [B, Hq, T] (fp32); the library allocates
    nothing."""
    import torch
    B, Hq, Hkv, T, d = _soft_check(q, k, v, logit, noise)
    for t, shape, name in ((out, (B, Hq, T, d), "out"), (lse, (B, Hq, T), "lse")):
        if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name}: expected contiguous float32 {shape} on the GPU")
    dms_soft_attention_forward_noalloc(B, Hq, Hkv, T, d, window, gamma, tau, scale, q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), logit.data_ptr(), noise.data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return out, lse


def soft_attention_backward(q, k, v, logit, noise, out, lse, dout, window, gamma=0.0, tau=1.0, scale=0.0,
                            workspace=None):
    """Gradients (dms_soft_attention_backward) on torch tensors: returns
    {'dq', 'dk', 'dv', 'dlogit'} in fp32.  dout is bf16 like q."""
    import torch
    B, Hq, Hkv, T, d = _soft_check(q, k, v, logit, noise)
    if tuple(dout.shape) != (B, Hq, T, d) or dout.dtype != torch.bfloat16 or not dout.is_contiguous():
        raise ValueError("dout: expected contiguous bf16 of q's shape")
    nbytes = dms_soft_attention_backward_workspace_bytes(B, Hq, Hkv, T, d)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq = torch.empty((B, Hq, T, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, T, d), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    dlogit = torch.empty((B, Hkv, T), dtype=torch.float32, device=q.device)
    dms_soft_attention_backward(B, Hq, Hkv, T, d, window, gamma, tau, scale, q.data_ptr(), k.data_ptr(),
                                v.data_ptr(), logit.data_ptr(), noise.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dlogit.data_ptr(),
                                workspace.data_ptr(), workspace.numel(), torch.cuda.current_stream().cuda_stream)
    return {"dq": dq, "dk": dk, "dv": dv, "dlogit": dlogit}


def _soft_autograd():
    import torch

    class SoftAttention(torch.autograd.Function):
        """The relaxed attention as an autograd function: the forward keeps
        out and lse for dms_soft_attention_backward.  Gradients come back in
        the inputs' dtypes (bf16 for q, k, v; fp32 for the logits); the
        incoming gradient of out is rounded to bf16, the library's dout
        operand.  The noise is a constant."""

        @staticmethod
        def forward(ctx, q, k, v, logit, noise, window, gamma, tau, scale):
            out, lse = soft_attention_forward(q, k, v, logit, noise, window, gamma, tau, scale)
            ctx.save_for_backward(q, k, v, logit, noise, out, lse)
            ctx.params = (window, gamma, tau, scale)
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, logit, noise, out, lse = ctx.saved_tensors
            window, gamma, tau, scale = ctx.params
            g = soft_attention_backward(q, k, v, logit, noise, out, lse,
                                        dout.to(torch.bfloat16).contiguous(), window, gamma, tau, scale)
            return (g["dq"].to(q.dtype), g["dk"].to(k.dtype), g["dv"].to(v.dtype), g["dlogit"],
                    None, None, None, None, None)

    return SoftAttention


_SOFT_FN = None


def soft_attention(q, k, v, logit, noise, window, gamma=0.0, tau=1.0, scale=0.0):
    """Differentiable relaxed DMS attention (torch autograd over
    dms_soft_attention_forward / dms_soft_attention_backward): returns out
    [B, Hq, T, d] fp32; q, k, v bf16, logit and noise fp32 (see
    soft_attention_forward for the shapes)."""
    global _SOFT_FN
    if _SOFT_FN is None:
        _SOFT_FN = _soft_autograd()
    return _SOFT_FN.apply(q, k, v, logit, noise, window, gamma, tau, scale)


class Cache:
    """A DMS cache whose workspace is a torch uint8 tensor on the current
    device.  Tensors passed in must be contiguous, on that device, with the
    shapes and dtypes of include/dms.h; they are checked here and handed to
    the library by pointer."""

    def __init__(self, batch, num_q_heads, num_kv_heads, head_dim, window, max_tokens, pool_blocks,
                 dtype="bf16", split_wgs=0, scale=0.0):
        import torch
        self._torch = torch
        self.dtype = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.cfg = make_config(batch, num_q_heads, num_kv_heads, head_dim, window, max_tokens, pool_blocks,
                               DMS_BF16 if dtype == "bf16" else DMS_F32, split_wgs, scale)
        self.B, self.Hq, self.Hkv, self.d = batch, num_q_heads, num_kv_heads, head_dim
        self.window, self.max_tokens = window, max_tokens
        self.ring_size = min(window, max_tokens) + 1
        nbytes = dms_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise DmsError(DMS_ERR_ARG, "dms_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.handle = dms_cache_create(self.cfg, self.workspace.data_ptr(), nbytes, self._stream())

    def _stream(self) -> int:
        return self._torch.cuda.current_stream().cuda_stream

    def _chk(self, t, shape, dtype, name):
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on the GPU, got "
                             f"{t.dtype} {tuple(t.shape)} on {t.device}")
        return t.data_ptr()

    def prefill(self, k, v, logit, lengths):
        max_len = k.shape[2]
        pk = self._chk(k, (self.B, self.Hkv, max_len, self.d), self.tdtype, "k")
        pv = self._chk(v, (self.B, self.Hkv, max_len, self.d), self.tdtype, "v")
        pl = self._chk(logit, (self.B, self.Hkv, max_len), self._torch.float32, "logit")
        dms_prefill_compress(self.handle, pk, pv, pl, lengths, max_len, self._stream())

    def append(self, k, v, logit):
        pk = self._chk(k, (self.B, self.Hkv, self.d), self.tdtype, "k")
        pv = self._chk(v, (self.B, self.Hkv, self.d), self.tdtype, "v")
        pl = self._chk(logit, (self.B, self.Hkv), self._torch.float32, "logit")
        dms_append_step(self.handle, pk, pv, pl, self._stream())

    _SOURCES = {"k": DMS_LOGIT_FROM_K, "q": DMS_LOGIT_FROM_Q}

    def prefill_channel(self, k, v, lengths, source="k", channel=0, zero=False, q=None):
        """prefill with the eviction logits read from channel `channel` of the
        keys (source "k") or of each group's first query head (source "q";
        q: [B, Hq, max_len, d])."""
        max_len = k.shape[2]
        pk = self._chk(k, (self.B, self.Hkv, max_len, self.d), self.tdtype, "k")
        pv = self._chk(v, (self.B, self.Hkv, max_len, self.d), self.tdtype, "v")
        pq = None if q is None else self._chk(q, (self.B, self.Hq, max_len, self.d), self.tdtype, "q")
        dms_prefill_compress_channel(self.handle, pk, pv, pq, self._SOURCES[source], channel, zero, lengths,
                                     max_len, self._stream())

    def append_channel(self, k, v, source="k", channel=0, zero=False, q=None):
        """append with the eviction logit read from channel `channel` of the
        key row (source "k") or of the group's first query head (source "q";
        q: [B, Hq, d])."""
        pk = self._chk(k, (self.B, self.Hkv, self.d), self.tdtype, "k")
        pv = self._chk(v, (self.B, self.Hkv, self.d), self.tdtype, "v")
        pq = None if q is None else self._chk(q, (self.B, self.Hq, self.d), self.tdtype, "q")
        dms_append_step_channel(self.handle, pk, pv, pq, self._SOURCES[source], channel, zero, self._stream())

    def prefill_attention(self, q, k, v, out=None):
        """Attention of every prompt query, right after prefill(k, v, ...):
        q [B, Hq, max_len, d]; returns (or fills) out [B, Hq, max_len, d]
        fp32, rows past each prompt's length left untouched."""
        max_len = k.shape[2]
        pq = self._chk(q, (self.B, self.Hq, max_len, self.d), self.tdtype, "q")
        pk = self._chk(k, (self.B, self.Hkv, max_len, self.d), self.tdtype, "k")
        pv = self._chk(v, (self.B, self.Hkv, max_len, self.d), self.tdtype, "v")
        if out is None:
            out = self._torch.zeros((self.B, self.Hq, max_len, self.d), dtype=self._torch.float32, device=q.device)
        po = self._chk(out, (self.B, self.Hq, max_len, self.d), self._torch.float32, "out")
        dms_prefill_attention(self.handle, pq, pk, pv, max_len, po, self._stream())
        return out

    def decode_chunk(self, q, k, v, logit, out=None):
        """`chunk` decode steps at once: q [B, Hq, C, d], k, v [B, Hkv, C, d],
        logit [B, Hkv, C] fp32; returns (or fills) out [B, Hq, C, d] fp32."""
        C = k.shape[2]
        pq = self._chk(q, (self.B, self.Hq, C, self.d), self.tdtype, "q")
        pk = self._chk(k, (self.B, self.Hkv, C, self.d), self.tdtype, "k")
        pv = self._chk(v, (self.B, self.Hkv, C, self.d), self.tdtype, "v")
        pl = self._chk(logit, (self.B, self.Hkv, C), self._torch.float32, "logit")
        if out is None:
            out = self._torch.empty((self.B, self.Hq, C, self.d), dtype=self._torch.float32, device=q.device)
        po = self._chk(out, (self.B, self.Hq, C, self.d), self._torch.float32, "out")
        dms_decode_chunk(self.handle, pq, pk, pv, pl, C, po, self._stream())
        return out

    def decode_chunk_channel(self, q, k, v, source="k", channel=0, zero=False, out=None):
        """decode_chunk with the eviction logits read from channel `channel`
        of the keys (source "k") or of each group's first query head ("q")."""
        C = k.shape[2]
        pq = self._chk(q, (self.B, self.Hq, C, self.d), self.tdtype, "q")
        pk = self._chk(k, (self.B, self.Hkv, C, self.d), self.tdtype, "k")
        pv = self._chk(v, (self.B, self.Hkv, C, self.d), self.tdtype, "v")
        if out is None:
            out = self._torch.empty((self.B, self.Hq, C, self.d), dtype=self._torch.float32, device=q.device)
        po = self._chk(out, (self.B, self.Hq, C, self.d), self._torch.float32, "out")
        dms_decode_chunk_channel(self.handle, pq, pk, pv, self._SOURCES[source], channel, zero, C, po, self._stream())
        return out

    def attend(self, q, out=None):
        pq = self._chk(q, (self.B, self.Hq, self.d), self.tdtype, "q")
        if out is None:
            out = self._torch.empty((self.B, self.Hq, self.d), dtype=self._torch.float32, device=q.device)
        po = self._chk(out, (self.B, self.Hq, self.d), self._torch.float32, "out")
        dms_decode_attention(self.handle, pq, po, self._stream())
        return out

    def attend_timed(self, q, timer: "KernelTimer", out=None):
        """attend, with the call's kernels timed into `timer` (elapsed_ms)."""
        pq = self._chk(q, (self.B, self.Hq, self.d), self.tdtype, "q")
        if out is None:
            out = self._torch.empty((self.B, self.Hq, self.d), dtype=self._torch.float32, device=q.device)
        po = self._chk(out, (self.B, self.Hq, self.d), self._torch.float32, "out")
        dms_decode_attention_timed(self.handle, pq, po, timer.start.value, timer.stop.value, self._stream())
        return out

    def _step_args(self, q, k, v, out):
        pq = self._chk(q, (self.B, self.Hq, self.d), self.tdtype, "q")
        pk = self._chk(k, (self.B, self.Hkv, self.d), self.tdtype, "k")
        pv = self._chk(v, (self.B, self.Hkv, self.d), self.tdtype, "v")
        if out is None:
            out = self._torch.empty((self.B, self.Hq, self.d), dtype=self._torch.float32, device=q.device)
        po = self._chk(out, (self.B, self.Hq, self.d), self._torch.float32, "out")
        return pq, pk, pv, out, po

    def step(self, q, k, v, logit, out=None):
        """One decode step (append + attention, dms_decode_step): q [B, Hq, d],
        k, v [B, Hkv, d], logit [B, Hkv] fp32; returns (or fills) out."""
        pq, pk, pv, out, po = self._step_args(q, k, v, out)
        pl = self._chk(logit, (self.B, self.Hkv), self._torch.float32, "logit")
        dms_decode_step(self.handle, pq, pk, pv, pl, po, self._stream())
        return out

    def step_timed(self, q, k, v, logit, timer: "KernelTimer", out=None):
        """step, with its kernels timed into `timer` (elapsed_ms)."""
        pq, pk, pv, out, po = self._step_args(q, k, v, out)
        pl = self._chk(logit, (self.B, self.Hkv), self._torch.float32, "logit")
        dms_decode_step_timed(self.handle, pq, pk, pv, pl, po, timer.start.value, timer.stop.value, self._stream())
        return out

    def step_channel(self, q, k, v, source="k", channel=0, zero=False, out=None):
        """step with the eviction logit read from channel `channel` of the key
        row (source "k") or of the group's first query head (source "q")."""
        pq, pk, pv, out, po = self._step_args(q, k, v, out)
        dms_decode_step_channel(self.handle, pq, pk, pv, self._SOURCES[source], channel, zero, po, self._stream())
        return out

    def balance(self):
        """Re-plan the attention's work split from the live counts (synchronises)."""
        dms_cache_balance(self.handle, self._stream())

    def split_mode(self) -> bool:
        """True when the attention splits the live blocks in equal shares."""
        return bool(self.stats()["split_mode"])

    def stats(self) -> dict:
        return dms_cache_stats(self.handle, self._stream())

    def export(self, unit_begin=0, unit_count=None):
        if unit_count is None:
            unit_count = self.B * self.Hkv - unit_begin
        slot_pos = np.empty((unit_count, self.max_tokens), dtype=np.int32)
        ring = np.empty((unit_count, self.ring_size), dtype=np.int32)
        n = np.empty(unit_count, dtype=np.int32)
        dms_cache_export(self.handle, unit_begin, unit_count, slot_pos, ring, n, self._stream())
        return slot_pos, ring, n

    def reset(self):
        dms_cache_reset(self.handle, self._stream())

    def close(self):
        if getattr(self, "handle", None):
            dms_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
