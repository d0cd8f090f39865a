"""Plausible single mistakes planted in the oracle (on the CPU) must each make
at least one pin fail: evidence that the pins constrain every part of it."""
import numpy as np
import pytest

import oracle_pins
from oracle import dms_oracle as real


def _visible_exclusive(alpha_row, q, w):
    i = np.arange(q + 1)
    a = np.asarray(alpha_row[: q + 1], dtype=bool)
    return i[(~a) | (q - i < w)]


def _visible_drops_self(alpha_row, q, w):
    i = np.arange(q + 1)
    a = np.asarray(alpha_row[: q + 1], dtype=bool)
    return i[((~a) | (q - i <= w)) & (i < q)] if q > 0 else i


def _visible_inverted(alpha_row, q, w):
    i = np.arange(q + 1)
    a = np.asarray(alpha_row[: q + 1], dtype=bool)
    return i[a | (q - i <= w)]


def _visible_window_only(alpha_row, q, w):
    i = np.arange(q + 1)
    return i[q - i <= w]


def _decision_ge(logit):
    return np.asarray(logit, dtype=np.float32) >= 0


def _decision_nan_marks(logit):
    x = np.asarray(logit, dtype=np.float32)
    return (x > 0) | np.isnan(x)


def _retired_off_by_one(alpha_row, q, w):
    j = q - w
    return [j] if j >= 0 and bool(alpha_row[j]) else []


def _pending_empty(alpha_row, q, w):
    return np.zeros(0, dtype=np.int64)


def _pending_window_one_short(alpha_row, q, w):
    i = np.arange(max(0, q - w + 1), q + 1)
    return i[np.asarray(alpha_row, dtype=bool)[i]]


def _kv_head_mod(hq, group):
    return hq % group


def _scale_over_d(d):
    return 1.0 / d


def _attend_kv_swapped(qv, k_rows, v_rows, scale):
    return real._softmax(scale * (np.asarray(qv, float) @ np.asarray(v_rows, float).T)) @ np.asarray(k_rows, float)


def _softmax_wrong_axis(s):
    m = np.max(s, axis=0, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=0, keepdims=True)


def _attend_masked_exclusive(qv, k_all, v_all, alpha_row, q, w, scale):
    k = np.asarray(k_all[: q + 1], float)
    v = np.asarray(v_all[: q + 1], float)
    s = scale * (np.asarray(qv, float) @ k.T)
    mask = np.array([0.0 if (not alpha_row[i]) or (q - i < w) else -np.inf for i in range(q + 1)])
    return real._softmax(s + mask[None]) @ v


def _channel_off_by_one(X, channel, group=1):
    X = np.asarray(X)
    B, H, T, d = X.shape
    return np.stack([X[:, h * group, :, (channel + 1) % d] for h in range(H // group)], axis=1).astype(np.float32)


def _channel_last_query_head(X, channel, group=1):
    X = np.asarray(X)
    B, H, T, d = X.shape
    return np.stack([X[:, h * group + group - 1, :, channel] for h in range(H // group)], axis=1).astype(np.float32)


def _zero_next_channel(X, channel):
    Y = np.array(X, dtype=np.float64, copy=True)
    Y[..., (channel + 1) % Y.shape[-1]] = 0.0
    return Y


def _zero_nothing(X, channel):
    return np.array(X, dtype=np.float64, copy=True)


def _prefill_final_state(Q, K, V, logit, prompt_lens, w, scale=None):
    """Every prompt query attends the visible set of the prompt's last position."""
    B, Hq, T, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = real.default_scale(d) if scale is None else scale
    out = np.full((B, Hq, T, d), np.nan)
    for b in range(B):
        for h in range(Hkv):
            alpha = real.eviction_decision(logit[b, h])
            P = int(prompt_lens[b])
            vis = real.visible(alpha, P - 1, w)
            for hq in range(h * G, (h + 1) * G):
                for q in range(P):
                    vq = vis[vis <= q]
                    out[b, hq, q] = real.attend(Q[b, hq, q][None], K[b, h][vq], V[b, h][vq], scale)[0]
    return out


def _prefill_shifted_query(Q, K, V, logit, prompt_lens, w, scale=None):
    """Query q takes the visible set of q - 1 (the step before its own append)."""
    B, Hq, T, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    scale = real.default_scale(d) if scale is None else scale
    out = np.full((B, Hq, T, d), np.nan)
    for b in range(B):
        for h in range(Hkv):
            alpha = real.eviction_decision(logit[b, h])
            for q in range(int(prompt_lens[b])):
                vis = real.visible(alpha, max(q - 1, 0), w)
                for hq in range(h * G, (h + 1) * G):
                    out[b, hq, q] = real.attend(Q[b, hq, q][None], K[b, h][vis], V[b, h][vis], scale)[0]
    return out


def _soft_bias_positive(x):
    return np.logaddexp(0.0, x)


def _soft_arg_without_noise(logit, noise, gamma, tau):
    return (np.asarray(logit, np.float64) + gamma) / tau


def _soft_grads_dlogit_sign(Q, K, V, logit, noise, dO, w, gamma, tau, scale=None, magnitudes=False):
    g = real.__dict__["_orig_soft_attention_grads"](Q, K, V, logit, noise, dO, w, gamma, tau, scale, magnitudes)
    g["dlogit"] = -g["dlogit"]
    return g


def _soft_mask_window_ge(bias, w):
    """The bias already applies at q - i == w (the window one short)."""
    T = len(bias)
    pos = np.arange(T)
    causal = pos[None, :] <= pos[:, None]
    far = ((pos[:, None] - pos[None, :]) >= w) & causal
    return np.where(causal, np.where(far, np.asarray(bias, float)[None, :], 0.0), -np.inf), far


def _soft_mask_strict_causal(bias, w):
    """A query does not see its own key."""
    T = len(bias)
    pos = np.arange(T)
    causal = pos[None, :] < pos[:, None]
    causal[0, 0] = True  # keep row 0 finite
    far = ((pos[:, None] - pos[None, :]) > w) & causal
    return np.where(causal, np.where(far, np.asarray(bias, float)[None, :], 0.0), -np.inf), far


MUTANTS = {
    "window-exclusive": ("visible", _visible_exclusive),
    "query-misses-itself": ("visible", _visible_drops_self),
    "decision-inverted": ("visible", _visible_inverted),
    "decision-ignored": ("visible", _visible_window_only),
    "threshold-ge-zero": ("eviction_decision", _decision_ge),
    "nan-marks": ("eviction_decision", _decision_nan_marks),
    "retire-off-by-one": ("retired", _retired_off_by_one),
    "pending-empty": ("pending", _pending_empty),
    "pending-window-one-short": ("pending", _pending_window_one_short),
    "gqa-modulo": ("kv_head_of", _kv_head_mod),
    "scale-1-over-d": ("default_scale", _scale_over_d),
    "k-v-swapped": ("attend", _attend_kv_swapped),
    "softmax-axis": ("_softmax", _softmax_wrong_axis),
    "masked-form-exclusive": ("attend_masked", _attend_masked_exclusive),
    "logit-channel-off-by-one": ("logits_from_channel", _channel_off_by_one),
    "logit-last-query-head": ("logits_from_channel", _channel_last_query_head),
    "zero-next-channel": ("without_channel", _zero_next_channel),
    "zero-nothing": ("without_channel", _zero_nothing),
    "prefill-final-state": ("prefill_attention", _prefill_final_state),
    "prefill-query-misses-itself": ("prefill_attention", _prefill_shifted_query),
    "soft-bias-positive": ("soft_bias", _soft_bias_positive),
    "soft-noise-ignored": ("soft_decision_arg", _soft_arg_without_noise),
    "soft-dlogit-sign": ("soft_attention_grads", _soft_grads_dlogit_sign),
    "soft-window-one-short": ("soft_mask", _soft_mask_window_ge),
    "soft-query-misses-itself": ("soft_mask", _soft_mask_strict_causal),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(real, "_orig_" + attr, getattr(real, attr), raising=False)
    monkeypatch.setattr(real, attr, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(real)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
