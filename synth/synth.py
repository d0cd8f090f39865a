"""Seeded, counter-based synthetic inputs (host twin).

This module only makes numbers.  It contains none of the decode path's
arithmetic: no eviction decision, no visibility rule, no attention.  Both the
CPU oracle (through its tests) and the HIP path (through the device twin in
``synth.hip``) draw their inputs from the definition below, and the twins are
checked bit for bit against each other.

Definition
----------
Every value is addressed by ``(seed, stream, idx)``:

* ``idx`` is a flat counter over (layer, sequence b, head, position, channel)
  with fixed strides, so a value never depends on the shape of the batch it
  was drawn in::

      idx = ((((layer * 1024 + b) * 64 + head) * 2**20 + pos) * 128 + ch)

  (layer < 64, b < 1024, head < 64, pos < 2**20, ch < 128).
* Three 64-bit words are drawn with Vigna's public-domain SplitMix64 output
  function applied to the key ``seed ^ (stream << 56) ^ (3*idx + j)``,
  ``j = 0, 1, 2``: add 0x9E3779B97F4A7C15, then xor-shift 30 / multiply by
  0xBF58476D1CE4E5B9, xor-shift 27 / multiply by 0x94D049BB133111EB,
  xor-shift 31.
* The twelve 16-bit lanes ``u_k`` of the three words are summed,
  ``S = sum u_k``, and ``x = float32(2*S - 786420) * 2**-17``.  This is an
  Irwin-Hall(12) variate: mean 0, variance 1 - 1/2**32, |x| <= 6.  The
  conversion is exact because |2S - 786420| < 2**24.
* bf16 inputs are x rounded to nearest-even bf16 by integer arithmetic on the
  fp32 bit pattern.
* Eviction logits are ``float32(float64(mu) + float64(x))``, one rounding.

* Logistic noise (the relaxed decisions' random draw) takes the first word z
  of each counter (channel 0) on stream 5: u = ((z >> 11) + 0.5) * 2**-53,
  in (0, 1), and g = float32(log(u) - log(1 - u)), a Logistic(0, 1) sample
  (the difference of two independent Gumbel(0, 1) samples).

Streams: Q = 0, K = 1, V = 2, logit = 3, lengths = 4, noise = 5.
"""
from __future__ import annotations

import numpy as np

STREAM_Q = 0
STREAM_K = 1
STREAM_V = 2
STREAM_LOGIT = 3
STREAM_LEN = 4
STREAM_NOISE = 5

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK16 = np.uint64(0xFFFF)

MAX_LAYERS = 64
MAX_BATCH = 1024
MAX_HEADS = 64
MAX_POS = 1 << 20
MAX_CH = 128


def splitmix64(key: np.ndarray) -> np.ndarray:
    """SplitMix64 output function of a uint64 key (wrapping arithmetic)."""
    z = np.asarray(key, dtype=np.uint64) + _GOLDEN
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def flat_index(layer, b, head, pos, ch) -> np.ndarray:
    """Fixed-stride counter of one value (all arguments broadcast)."""
    layer = np.asarray(layer, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    head = np.asarray(head, dtype=np.uint64)
    pos = np.asarray(pos, dtype=np.uint64)
    ch = np.asarray(ch, dtype=np.uint64)
    return ((((layer * np.uint64(MAX_BATCH) + b) * np.uint64(MAX_HEADS) + head)
             * np.uint64(MAX_POS) + pos) * np.uint64(MAX_CH) + ch)


def normal_from_index(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """Irwin-Hall(12) variate for each counter value, as float32."""
    idx = np.asarray(idx, dtype=np.uint64)
    base = np.uint64(seed) ^ (np.uint64(stream) << np.uint64(56))
    s = np.zeros(idx.shape, dtype=np.int64)
    for j in range(3):
        z = splitmix64(base ^ (np.uint64(3) * idx + np.uint64(j)))
        for lane in range(4):
            s += ((z >> np.uint64(16 * lane)) & _MASK16).astype(np.int64)
    return (2 * s - 786420).astype(np.float32) * np.float32(2.0 ** -17)


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit pattern (uint16) of finite float32 values."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """x rounded to bf16 and widened back to float32 (exact widening)."""
    return bf16_bits_to_f32(round_bf16_bits(x))


def _heads(heads) -> np.ndarray:
    """An int means heads 0..heads-1; a sequence lists head indices."""
    if np.ndim(heads) == 0:
        return np.arange(int(heads), dtype=np.int64)
    return np.asarray(heads, dtype=np.int64)


def _grid(layer, b_list, heads, positions, channels):
    """Counter values for the tensor [len(b_list), heads, len(positions), channels]
    where ``positions`` may be a 1-D array shared by all b or a 2-D array
    [len(b_list), P] of per-sequence positions."""
    b = np.asarray(b_list, dtype=np.int64).reshape(-1, 1, 1, 1)
    h = _heads(heads).reshape(1, -1, 1, 1)
    pos = np.asarray(positions, dtype=np.int64)
    if pos.ndim == 1:
        pos = pos.reshape(1, 1, -1, 1)
    else:
        pos = pos.reshape(pos.shape[0], 1, pos.shape[1], 1)
    ch = np.arange(channels, dtype=np.int64).reshape(1, 1, 1, -1)
    return flat_index(layer, b, h, pos, ch)


def tensor(seed: int, stream: int, layer: int, b_list, heads: int, positions, channels: int,
           dtype: str = "f32") -> np.ndarray:
    """Values for [B', heads, P, channels] (float32; bf16-rounded if dtype == 'bf16').
    ``heads`` is a count or a list of head indices."""
    x = normal_from_index(seed, stream, _grid(layer, b_list, heads, positions, channels))
    if dtype == "bf16":
        return round_bf16(x)
    if dtype != "f32":
        raise ValueError(dtype)
    return x


def logits(seed: int, layer: int, b_list, heads: int, positions, mu_before, mu_after=None,
           pos_threshold: int = MAX_POS) -> np.ndarray:
    """Eviction logits [B', heads, P] = float32(mu + x).

    ``heads`` is a count or a list of head indices.  ``mu_before`` /
    ``mu_after`` are per-head means (a scalar or one value per head of the
    full head range) used for positions below / at-or-above ``pos_threshold``.
    """
    hl = _heads(heads)
    mu_before = np.asarray(mu_before, dtype=np.float64)
    mu_before = mu_before[hl] if mu_before.ndim == 1 and mu_before.size > 1 else \
        np.broadcast_to(mu_before.reshape(-1)[:1] if mu_before.ndim else mu_before, (len(hl),))
    if mu_after is None:
        mu_after = mu_before
    else:
        mu_after = np.asarray(mu_after, dtype=np.float64)
        mu_after = mu_after[hl] if mu_after.ndim == 1 and mu_after.size > 1 else \
            np.broadcast_to(mu_after.reshape(-1)[:1] if mu_after.ndim else mu_after, (len(hl),))
    idx = _grid(layer, b_list, heads, positions, 1)[..., 0]
    x = normal_from_index(seed, STREAM_LOGIT, idx).astype(np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    pos = pos.reshape(1, 1, -1) if pos.ndim == 1 else pos.reshape(pos.shape[0], 1, pos.shape[1])
    mu = np.where(pos < pos_threshold, mu_before.reshape(1, -1, 1), mu_after.reshape(1, -1, 1))
    return (mu + x).astype(np.float32)


def lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence lengths uniform on [lo, hi] (inclusive), from stream 4.

    Uses the first word of each counter: ``lo + (z mod (hi - lo + 1))``.
    """
    idx = flat_index(0, np.arange(batch), 0, 0, 0)
    base = np.uint64(seed) ^ (np.uint64(STREAM_LEN) << np.uint64(56))
    z = splitmix64(base ^ (np.uint64(3) * idx))
    span = np.uint64(hi - lo + 1)
    return (np.uint64(lo) + z % span).astype(np.int64)


def logistic_noise(seed: int, layer: int, b_list, heads: int, positions) -> np.ndarray:
    """Logistic(0, 1) samples [B', heads, P] (float32), stream 5."""
    idx = _grid(layer, b_list, heads, positions, 1)[..., 0]
    base = np.uint64(seed) ^ (np.uint64(STREAM_NOISE) << np.uint64(56))
    z = splitmix64(base ^ (np.uint64(3) * idx.astype(np.uint64)))
    u = ((z >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
    return (np.log(u) - np.log1p(-u)).astype(np.float32)
