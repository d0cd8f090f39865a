"""Plain CPU oracle of the DMS decode path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product (the HIP library and its
Python binding) never calls it and shares no code with it.

What it computes
----------------
Dynamic Memory Sparsification (DMS) gives every KV head a binary eviction
decision per token and delays its effect by a window of w steps.  Sources,
cited by page title and section:

* "Inference-Time Hyper-Scaling with KV Cache Compression", third-party
  paper summary (bud-325.pages.dev), sections "Key claims" and "Method"
  (attributing paper section 3.2, section 5.3 and Fig. 5): a per-head binary
  decision alpha_t in {0, 1}; a token marked at step t remains attendable
  through step t + w inside a sliding window of size w, then it is gone;
  the decisions drive an additive attention mask that is never built.
* The same page, "Method": each head may end at its own compression ratio.
* arXiv listing of 2506.05345 (searcharxiv.org), "Abstract": eviction is
  delayed rather than immediate.

Readings taken where the pages are silent (each listed in the design notes):

* alpha = 1 exactly when the token's own eviction logit is > 0 (fp32
  compare; logit 0, -0 and NaN give alpha = 0).  At inference the
  Gumbel-sigmoid of training is replaced by its noiseless threshold.
* "visible until t + w" is inclusive: a marked token i is visible to the
  queries q in [i, i + w] and to no later query.
* Decisions are per KV head; the G = Hq / Hkv query heads of a group share
  one visible set; query head hq reads KV head floor(hq / G).
* Within a decode step the token at position q is appended first (retiring
  token q - w - 1 if it was marked), then query q attends; it sees itself.
* Attention scale 1 / sqrt(d) unless overridden.
* Position 0 follows the same rule as every other position (no sinks).
* When the logit comes from a repurposed projection channel: for keys, KV
  head h's own channel; for queries, that channel of the group's first query
  head; the channel may be zeroed in the stored keys (``without_channel``).

The result is exact attention restricted to a visibility set, so this
module is that definition written out in float64: a closed form for the
visible set and a max-subtracted softmax over the gathered rows.  A second,
independent form (``attend_masked``) applies the rule as a dense additive
0 / -inf mask over all causal positions.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np


# ----------------------------------------------------------------------------
# Decision and visibility (summary page, "Key claims" / "Method")
# ----------------------------------------------------------------------------

def eviction_decision(logit: np.ndarray) -> np.ndarray:
    """alpha = 1 where the fp32 eviction logit is strictly positive.

    NaN compares false, so a NaN logit gives alpha = 0.
    """
    return np.asarray(logit, dtype=np.float32) > np.float32(0.0)


def visible(alpha_row: np.ndarray, q: int, w: int) -> np.ndarray:
    """Sorted positions i <= q with alpha_i == 0 or q - i <= w.

    ``alpha_row`` holds the decisions of one (sequence, KV head) for
    positions 0..q (longer rows are cut at q).
    """
    i = np.arange(q + 1)
    a = np.asarray(alpha_row[: q + 1], dtype=bool)
    keep = (~a) | (q - i <= w)
    return i[keep]


def retired(alpha_row: np.ndarray, q: int, w: int) -> List[int]:
    """Positions dropped by the step that appends q: q - w - 1 if marked."""
    j = q - w - 1
    if j >= 0 and bool(alpha_row[j]):
        return [j]
    return []


def pending(alpha_row: np.ndarray, q: int, w: int) -> np.ndarray:
    """Marked positions still visible at query q (all lie in [q - w, q])."""
    vis = visible(alpha_row, q, w)
    return vis[np.asarray(alpha_row, dtype=bool)[vis]]


def compression_ratio(q: int, n_visible: int) -> float:
    """Tokens seen over tokens kept, (q + 1) / |Vis(q)|."""
    return (q + 1) / n_visible


def kv_head_of(hq: int, group: int) -> int:
    """Grouped-query mapping: query head hq reads KV head floor(hq / G)."""
    return hq // group


def default_scale(head_dim: int) -> float:
    return 1.0 / np.sqrt(head_dim)


# ----------------------------------------------------------------------------
# Attention restricted to the visible set
# ----------------------------------------------------------------------------

def _softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(qv: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q k^T) v over the gathered rows, float64.

    qv: [G, d]; k_rows, v_rows: [n, d]; returns [G, d].
    """
    qv = np.asarray(qv, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    v = np.asarray(v_rows, dtype=np.float64)
    s = scale * (qv @ k.T)
    return _softmax(s) @ v


def attention_weights(qv: np.ndarray, k_rows: np.ndarray, scale: float) -> np.ndarray:
    qv = np.asarray(qv, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    return _softmax(scale * (qv @ k.T))


def attend_masked(qv: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, alpha_row: np.ndarray,
                  q: int, w: int, scale: float) -> np.ndarray:
    """Second form: dense causal scores over positions 0..q plus an additive
    mask that is 0 where the rule keeps a token and -inf where it drops it."""
    qv = np.asarray(qv, dtype=np.float64)
    k = np.asarray(k_all[: q + 1], dtype=np.float64)
    v = np.asarray(v_all[: q + 1], dtype=np.float64)
    s = scale * (qv @ k.T)
    mask = np.full(q + 1, -np.inf)
    for i in range(q + 1):
        if (not bool(alpha_row[i])) or (q - i <= w):
            mask[i] = 0.0
    s = s + mask[None, :]
    return _softmax(s) @ v


# ----------------------------------------------------------------------------
# Decode of one (sequence, KV head) unit
# ----------------------------------------------------------------------------

@dataclass
class StepRecord:
    q: int                      # position appended and queried
    alpha: bool                 # decision of the appended token
    visible: np.ndarray         # sorted positions in Vis(q)
    retired: List[int]          # positions dropped by this step
    pending: np.ndarray         # marked positions still visible
    out: Optional[np.ndarray]   # [G, d] float64, or None when not requested
    cr: float


def decode_unit(q_rows: Optional[np.ndarray], k: np.ndarray, v: np.ndarray, logit: np.ndarray,
                prompt_len: int, steps: int, w: int, scale: float) -> List[StepRecord]:
    """Decode ``steps`` tokens after a prompt of ``prompt_len`` tokens.

    q_rows: [steps, G, d] queries of the group at positions prompt_len + t
            (None to skip attention); k, v: [T, d] rows by position;
    logit:  [T] eviction logits by position, T >= prompt_len + steps.
    """
    alpha = eviction_decision(logit)
    recs = []
    for t in range(steps):
        q = prompt_len + t
        vis = visible(alpha, q, w)
        out = None
        if q_rows is not None:
            out = attend(q_rows[t], k[vis], v[vis], scale)
        recs.append(StepRecord(q=q, alpha=bool(alpha[q]), visible=vis,
                               retired=retired(alpha, q, w), pending=pending(alpha, q, w),
                               out=out, cr=compression_ratio(q, len(vis))))
    return recs


def decode_batch(Q: np.ndarray, K: np.ndarray, V: np.ndarray, logit: np.ndarray,
                 prompt_lens, steps: int, w: int, scale: Optional[float] = None,
                 units=None) -> Dict:
    """Whole-batch decode.

    Q: [B, Hq, T, d]; K, V: [B, Hkv, T, d]; logit: [B, Hkv, T];
    prompt_lens: [B].  ``units``: optional list of (b, h) to compute (default
    all).  Returns {'out': [steps, B, Hq, d] float64 (NaN where not computed),
    'records': {(b, h): [StepRecord]}}.
    """
    B, Hq, _, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(Hkv)]
    out = np.full((steps, B, Hq, d), np.nan)
    records = {}
    for (b, h) in units:
        P = int(prompt_lens[b])
        heads = [hq for hq in range(Hq) if kv_head_of(hq, G) == h]
        qr = np.stack([Q[b, heads, P + t, :] for t in range(steps)])
        recs = decode_unit(qr, K[b, h], V[b, h], logit[b, h], P, steps, w, scale)
        records[(b, h)] = recs
        for t, r in enumerate(recs):
            out[t, b, heads, :] = r.out
    return {"out": out, "records": records}


# ----------------------------------------------------------------------------
# Attention of the prompt's own queries under the same rule (summary page,
# "Method": the decisions act as an additive attention mask, the same one at
# every position, that never has to be built)
# ----------------------------------------------------------------------------

def prefill_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, logit: np.ndarray, prompt_lens,
                      w: int, scale: Optional[float] = None) -> np.ndarray:
    """Output of every prompt query: query position q of sequence b and
    query head hq attends the visible set Vis(b, h, q) of KV head
    h = floor(hq / G), exactly as a decode query at q would.

    Q: [B, Hq, T, d]; K, V: [B, Hkv, T, d]; logit: [B, Hkv, T];
    prompt_lens: [B] (<= T).  Returns [B, Hq, T, d] float64, NaN at
    positions q >= prompt_lens[b].
    """
    B, Hq, T, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    out = np.full((B, Hq, T, d), np.nan)
    for b in range(B):
        for h in range(Hkv):
            alpha = eviction_decision(logit[b, h])
            heads = [hq for hq in range(Hq) if kv_head_of(hq, G) == h]
            for q in range(int(prompt_lens[b])):
                vis = visible(alpha, q, w)
                out[b, heads, q, :] = attend(Q[b, heads, q, :], K[b, h][vis], V[b, h][vis], scale)
    return out


# ----------------------------------------------------------------------------
# Training-time relaxation (summary page, "Method": the binary decision is
# trained through a Gumbel-sigmoid reparametrisation at low temperature with a
# logit offset gamma; the decisions enter attention as an additive mask).
# Readings: alpha_i = sigmoid((logit_i + gamma + g_i) / tau) with logistic
# noise g_i supplied by the caller; for query q and key i <= q the additive
# bias is 0 while q - i <= w and log(1 - alpha_i) after, which is the hard rule
# exactly when alpha is 0 or 1.
# ----------------------------------------------------------------------------

def soft_decision_arg(logit, noise, gamma: float, tau: float) -> np.ndarray:
    """x_i = (logit_i + gamma + g_i) / tau, so that alpha_i = sigmoid(x_i)."""
    return (np.asarray(logit, np.float64) + gamma + np.asarray(noise, np.float64)) / tau


def soft_bias(x: np.ndarray) -> np.ndarray:
    """log(1 - sigmoid(x)) = -softplus(x), evaluated without overflow."""
    return -np.logaddexp(0.0, x)


def soft_mask(bias: np.ndarray, w: int):
    """The relaxed mask of one (sequence, KV head) over T positions.

    Returns (add, far): add[q, i] is -inf for i > q (causal), 0 for
    q - w <= i <= q (the window) and bias[i] for i < q - w; far[q, i] marks
    the keys that carry their bias (q - i > w, i <= q)."""
    T = len(bias)
    pos = np.arange(T)
    causal = pos[None, :] <= pos[:, None]                # [q, i]
    far = ((pos[:, None] - pos[None, :]) > w) & causal
    add = np.where(causal, np.where(far, np.asarray(bias, np.float64)[None, :], 0.0), -np.inf)
    return add, far


def soft_attention(Q, K, V, logit, noise, w: int, gamma: float, tau: float,
                   scale: Optional[float] = None) -> Dict:
    """Causal attention of every position with the relaxed mask.

    Q: [B, Hq, T, d]; K, V: [B, Hkv, T, d]; logit, noise: [B, Hkv, T].
    Returns {'out': [B, Hq, T, d], 'lse': [B, Hq, T]} in float64 (lse: the
    natural log of each row's softmax denominator, for the backward).
    """
    B, Hq, T, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((B, Hq, T, d))
    lse = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hkv):
            add, _ = soft_mask(soft_bias(soft_decision_arg(logit[b, h], noise[b, h], gamma, tau)), w)
            for hq in range(h * G, (h + 1) * G):
                s = scale * (np.asarray(Q[b, hq], np.float64) @ np.asarray(K[b, h], np.float64).T) + add
                m = np.max(s, axis=1, keepdims=True)
                e = np.exp(s - m)
                z = np.sum(e, axis=1, keepdims=True)
                out[b, hq] = (e / z) @ np.asarray(V[b, h], np.float64)
                lse[b, hq] = (m + np.log(z))[:, 0]
    return {"out": out, "lse": lse}


def soft_attention_grads(Q, K, V, logit, noise, dO, w: int, gamma: float, tau: float,
                         scale: Optional[float] = None, magnitudes: bool = False) -> Dict:
    """Gradients of sum(dO * out) of ``soft_attention`` with respect to Q,
    K, V and the logits (the noise, gamma and tau are constants), written out
    from the chain rule: P = softmax(S), dP = dO V^T, dS = P (dP - rowsum(dO
    out)), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, and for the bias
    -softplus(x) of the far keys, dlogit_i = -sigmoid(x_i) / tau * sum of dS
    over the far (query, head) pairs of key i.  All float64.

    With ``magnitudes``, also the same sums over the terms' absolute values,
    dq_mag = scale |dS| |K|, dk_mag = scale |dS|^T |Q| and dv_mag = P^T |dO|:
    an implementation that rounds each P or dS entry of these products by a
    relative e is off by at most e times them (test tolerances)."""
    B, Hq, T, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    dQ = np.zeros((B, Hq, T, d))
    dK = np.zeros((B, Hkv, T, d))
    dV = np.zeros((B, Hkv, T, d))
    dlogit = np.zeros((B, Hkv, T))
    if magnitudes:
        mag = {"dq_mag": np.zeros_like(dQ), "dk_mag": np.zeros_like(dK), "dv_mag": np.zeros_like(dV)}
    for b in range(B):
        for h in range(Hkv):
            x = soft_decision_arg(logit[b, h], noise[b, h], gamma, tau)
            add, far = soft_mask(soft_bias(x), w)
            Kh = np.asarray(K[b, h], np.float64)
            Vh = np.asarray(V[b, h], np.float64)
            for hq in range(h * G, (h + 1) * G):
                Qh = np.asarray(Q[b, hq], np.float64)
                dOh = np.asarray(dO[b, hq], np.float64)
                s = scale * (Qh @ Kh.T) + add
                P = np.exp(s - np.max(s, axis=1, keepdims=True))
                P /= np.sum(P, axis=1, keepdims=True)
                O = P @ Vh
                dP = dOh @ Vh.T
                dS = P * (dP - np.sum(dOh * O, axis=1, keepdims=True))
                dQ[b, hq] = scale * (dS @ Kh)
                dK[b, h] += scale * (dS.T @ Qh)
                dV[b, h] += P.T @ dOh
                dlogit[b, h] += np.sum(np.where(far, dS, 0.0), axis=0)
                if magnitudes:
                    mag["dq_mag"][b, hq] = scale * (np.abs(dS) @ np.abs(Kh))
                    mag["dk_mag"][b, h] += scale * (np.abs(dS).T @ np.abs(Qh))
                    mag["dv_mag"][b, h] += P.T @ np.abs(dOh)
            sig = 1.0 / (1.0 + np.exp(-x))
            dlogit[b, h] *= -sig / tau
    res = {"dq": dQ, "dk": dK, "dv": dV, "dlogit": dlogit}
    if magnitudes:
        res.update(mag)
    return res


# ----------------------------------------------------------------------------
# Eviction logit read from a repurposed projection channel (summary page,
# "Key claims" and "Method": no parameters are added; one neuron of the K or
# Q projection of each head is repurposed to produce the eviction logit)
# ----------------------------------------------------------------------------

def logits_from_channel(X: np.ndarray, channel: int, group: int = 1) -> np.ndarray:
    """Eviction logits [B, H // group, T] (float32) read from one channel of a
    projection output X [B, H, T, d].

    Keys (group = 1): the logit of KV head h at position i is
    K[b, h, i, channel].  Queries (H = Hq, group = G): it is
    Q[b, h * G, i, channel].  Reading: the pages do not say which query head
    of a group drives the group's shared decision; the group's first query
    head carries the neuron.
    """
    X = np.asarray(X)
    B, H, T, _ = X.shape
    out = np.empty((B, H // group, T), dtype=np.float32)
    for h in range(H // group):
        out[:, h, :] = X[:, h * group, :, channel]
    return out


def without_channel(X: np.ndarray, channel: int) -> np.ndarray:
    """X (float64 copy) with ``channel`` set to 0 in every row.

    Reading: when the caller asks for it, the neuron that now carries the
    eviction logit no longer takes part in q . k (its key entry is stored as
    0); the pages leave open whether the repurposed neuron stays a feature.
    """
    Y = np.array(X, dtype=np.float64, copy=True)
    Y[..., channel] = 0.0
    return Y


def decode_batch_channel(Q: np.ndarray, K: np.ndarray, V: np.ndarray, prompt_lens, steps: int, w: int,
                         source: str, channel: int, zero: bool, scale: Optional[float] = None,
                         units=None) -> Dict:
    """``decode_batch`` with the logits read from channel ``channel`` of the
    keys (source "k") or of the queries (source "q"), and, for source "k"
    with ``zero``, that channel of the keys set to 0 before attention."""
    G = Q.shape[1] // K.shape[1]
    if source == "k":
        logit = logits_from_channel(K, channel, 1)
    elif source == "q":
        logit = logits_from_channel(Q, channel, G)
    else:
        raise ValueError(source)
    Kc = without_channel(K, channel) if zero else K
    if scale is None:
        scale = default_scale(Q.shape[-1])
    return decode_batch(Q, Kc, V, logit, prompt_lens, steps, w, scale, units)
