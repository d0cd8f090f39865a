"""Helpers for the GPU tests: drive the HIP path through the C ABI on
synthetic inputs and compare it with the CPU oracle.

Device inputs come from the device twin of the generator; the oracle's
inputs for the same (sequence, KV head) units come from the host twin.  The
two twins are checked bit for bit in test_gpu_synth.py.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from oracle import dms_oracle as O
from synth import synth
from synth import device as dsynth
from synth.workloads import Workload


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def tdtype(wl: Workload):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def make_cache(wl: Workload, layer: int = 0, pool_blocks: Optional[int] = None, split_wgs: int = 0,
               max_tokens: Optional[int] = None, window: Optional[int] = None):
    from learned_kv_cache_dms_amd import dms
    return dms.Cache(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                     wl.window if window is None else window,
                     wl.max_tokens() if max_tokens is None else max_tokens,
                     wl.pool_blocks(layer) if pool_blocks is None else pool_blocks,
                     dtype=wl.dtype, split_wgs=split_wgs)


def device_prompt(wl: Workload, layer: int, lengths: np.ndarray):
    """Dense prompt K, V [B, Hkv, max_len, d] and logits [B, Hkv, max_len]."""
    max_len = max(1, int(lengths.max()))
    K = torch.empty((wl.batch, wl.num_kv_heads, max_len, wl.head_dim), dtype=tdtype(wl), device="cuda")
    V = torch.empty_like(K)
    Lg = torch.empty((wl.batch, wl.num_kv_heads, max_len), dtype=torch.float32, device="cuda")
    mb, ma = wl.layer_mu(layer)
    dsynth.fill(K, wl.seed, synth.STREAM_K, layer, 0, pos0=0)
    dsynth.fill(V, wl.seed, synth.STREAM_V, layer, 0, pos0=0)
    dsynth.logits(Lg, wl.seed, layer, 0, mb, ma, wl.pos_threshold, pos0=0)
    return K, V, Lg


def device_step(wl: Workload, layer: int, pos_base: torch.Tensor):
    """Decode inputs at positions pos_base[b]: q [B,Hq,d], k/v [B,Hkv,d], logit [B,Hkv]."""
    B, Hq, Hkv, d = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    q = torch.empty((B, Hq, d), dtype=tdtype(wl), device="cuda")
    k = torch.empty((B, Hkv, d), dtype=tdtype(wl), device="cuda")
    v = torch.empty_like(k)
    lg = torch.empty((B, Hkv), dtype=torch.float32, device="cuda")
    mb, ma = wl.layer_mu(layer)
    dsynth.fill(q, wl.seed, synth.STREAM_Q, layer, 0, pos_base=pos_base)
    dsynth.fill(k, wl.seed, synth.STREAM_K, layer, 0, pos_base=pos_base)
    dsynth.fill(v, wl.seed, synth.STREAM_V, layer, 0, pos_base=pos_base)
    dsynth.logits(lg, wl.seed, layer, 0, mb, ma, wl.pos_threshold, pos_base=pos_base)
    return q, k, v, lg


@dataclass
class UnitData:
    """Host-twin inputs of one (sequence b, KV head h) unit."""
    b: int
    h: int
    K: np.ndarray       # [T, d]
    V: np.ndarray       # [T, d]
    logit: np.ndarray   # [T]
    Q: np.ndarray       # [steps, G, d] queries of the group at prompt_len + t
    prompt_len: int


def host_unit(wl: Workload, layer: int, b: int, h: int, prompt_len: int, steps: int) -> UnitData:
    T = prompt_len + steps
    pos = np.arange(T)
    K = synth.tensor(wl.seed, synth.STREAM_K, layer, [b], [h], pos, wl.head_dim, wl.dtype)[0, 0]
    V = synth.tensor(wl.seed, synth.STREAM_V, layer, [b], [h], pos, wl.head_dim, wl.dtype)[0, 0]
    mb, ma = wl.layer_mu(layer)
    lg = synth.logits(wl.seed, layer, [b], [h], pos, mb, ma, wl.pos_threshold)[0, 0]
    G = wl.group
    heads = list(range(h * G, (h + 1) * G))
    Qg = synth.tensor(wl.seed, synth.STREAM_Q, layer, [b], heads, np.arange(prompt_len, T),
                      wl.head_dim, wl.dtype)[0]
    Q = np.ascontiguousarray(Qg.transpose(1, 0, 2))
    return UnitData(b, h, K, V, lg, Q, prompt_len)


@dataclass
class CompareStats:
    max_err: float = 0.0
    checks: int = 0
    vis_checks: int = 0
    errs: List[float] = field(default_factory=list)


def check_unit_step(cache, wl: Workload, ud: UnitData, t: int, out_gpu: torch.Tensor, tol: float,
                    st: CompareStats, slot_pos=None, ring=None, n=None):
    """Compares one unit after decode step t: visible set, pending ring,
    live count (bit-exact) and the group's outputs (max-abs <= tol)."""
    q = ud.prompt_len + t
    alpha = O.eviction_decision(ud.logit)
    vis = O.visible(alpha, q, wl.window)
    pend = O.pending(alpha, q, wl.window)
    u = ud.b * wl.num_kv_heads + ud.h
    if slot_pos is None:
        sp, rg, nn = cache.export(u, 1)
        slot_pos, ring, n = sp[0], rg[0], int(nn[0])
    live = slot_pos[slot_pos >= 0]
    assert n == len(vis), (ud.b, ud.h, q, n, len(vis))
    assert np.all(slot_pos[:n] >= 0) and np.all(slot_pos[n:] < 0), "live slots are not the prefix [0, n)"
    assert np.array_equal(np.sort(live), vis), (ud.b, ud.h, q)
    gpu_pend = np.sort(slot_pos[ring[ring >= 0]])
    assert np.array_equal(gpu_pend, pend), (ud.b, ud.h, q, gpu_pend[:8], pend[:8])
    for r in np.nonzero(ring >= 0)[0]:
        assert slot_pos[ring[r]] % len(ring) == r
    st.vis_checks += 1
    if out_gpu is not None:
        scale = O.default_scale(wl.head_dim)
        ref = O.attend(ud.Q[t], ud.K[vis], ud.V[vis], scale)
        G = wl.group
        got = out_gpu[ud.b, ud.h * G:(ud.h + 1) * G].double().cpu().numpy()
        err = float(np.max(np.abs(got - ref)))
        st.max_err = max(st.max_err, err)
        st.errs.append(err)
        st.checks += 1
        assert err <= tol, (ud.b, ud.h, q, err, tol)


def run_decode(wl: Workload, steps: int, units: Sequence[Tuple[int, int]], tol: float, layer: int = 0,
               check_every: int = 1, cache=None, host_data: Optional[Dict] = None, mode: str = "calls",
               balance: bool = False) -> CompareStats:
    """Prefill + `steps` decode steps on the GPU, checking `units` against the
    oracle.  mode "calls": dms_append_step then dms_decode_attention; "step":
    dms_decode_step.  balance: dms_cache_balance after the prompt (and every
    64 steps)."""
    lengths = wl.prompt_lengths()
    if cache is None:
        cache = make_cache(wl, layer)
    log(f"[{wl.name}] device prompt {tuple(lengths[:4])}... B={wl.batch} mode={mode} balance={balance}")
    if int(lengths.max()) > 0:
        K, V, Lg = device_prompt(wl, layer, lengths)
        cache.prefill(K, V, Lg, lengths)
        del K, V, Lg
    if host_data is None:
        host_data = {}
        for (b, h) in units:
            host_data[(b, h)] = host_unit(wl, layer, b, h, int(lengths[b]), steps)
    st = CompareStats()
    pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    for t in range(steps):
        if balance and t % 64 == 0:
            cache.balance()
        q, k, v, lg = device_step(wl, layer, pos + t)
        if mode == "step":
            out = cache.step(q, k, v, lg)
        else:
            cache.append(k, v, lg)
            out = cache.attend(q)
        if t % check_every == 0 or t == steps - 1:
            torch.cuda.synchronize()
            for key in units:
                check_unit_step(cache, wl, host_data[key], t, out, tol, st)
    s = cache.stats()
    assert s["sticky_error"] == 0, s
    log(f"[{wl.name}] steps={steps} checks={st.checks} max_err={st.max_err:.3e} stats={s}")
    return st
