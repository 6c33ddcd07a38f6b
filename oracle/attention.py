"""Causal softmax attention of one isolated prompt, float64.

What the method must reproduce (Korean summary, §어떻게 동작하나; Flide:
Accelerating Decision Inference with Exact State Forking, §研究动机): every
question behaves exactly as the isolated prompt ``s (+) q_i``.  For a
full-attention layer that is ordinary causal attention over the prompt with
rotary positions ``0 .. P+|q_i|-1`` (§무엇과 다른가: question positions continue
from ``P``); a sliding-window layer keeps only keys with ``t_x - t_y < W``
(§方法步骤详情).

Readings where the pages are silent (all listed in the design notes):
* the causal boundary is inclusive — a token attends to itself;
* scores are scaled by ``1/sqrt(d)``;
* grouped-query heads: q head ``h`` uses kv head ``h // (Hq / Hkv)``;
* rotary embedding is the rotate-half form over the full head dimension,
  pair ``(i, i + d/2)`` rotated by ``t * theta**(-2i/d)``;
* checkpointed keys (positions ``0 .. m-1``) are stored already rotated;
  their values are stored as is.

Pinned by tests/test_oracle_attention.py (hand-computed rotations, one visible
key, identical keys, window of one, uniform weights, relative-position
invariance, and the flat-stream masked formulation of the same round).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def rope_rotate(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate the last axis of ``x`` (size d) to position ``pos``.

    ``pos`` broadcasts against ``x.shape[:-1]``.  Pair ``(i, i + d/2)`` is
    rotated by the angle ``pos * theta**(-2i/d)``.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def prompt_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, pos: np.ndarray, theta: float,
                     window: int = 0, cache_k: Optional[np.ndarray] = None,
                     cache_v: Optional[np.ndarray] = None,
                     rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Attention outputs of one prompt.

    q: [L, Hq, d]; k, v: [L, Hkv, d] (not yet rotated); pos: [L] positions of
    the prompt rows (strictly increasing).  cache_k / cache_v: [m, Hkv, d] for
    positions 0..m-1 (cache_k already rotated).  ``rows`` limits the rows
    computed (others are left zero).  Returns o: [L, Hq, d] float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    pos = np.asarray(pos, np.int64)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    qr = rope_rotate(q, pos[:, None], theta)
    kr = rope_rotate(k, pos[:, None], theta)
    if cache_k is not None and len(cache_k) > 0:
        m = cache_k.shape[0]
        keys = np.concatenate([np.asarray(cache_k, np.float64), kr], axis=0)
        vals = np.concatenate([np.asarray(cache_v, np.float64), v], axis=0)
        kpos = np.concatenate([np.arange(m, dtype=np.int64), pos])
    else:
        keys, vals, kpos = kr, v, pos
    scale = 1.0 / np.sqrt(d)
    o = np.zeros((L, Hq, d), np.float64)
    for a in (range(L) if rows is None else rows):
        vis = kpos <= pos[a]
        if window > 0:
            vis &= (pos[a] - kpos) < window
        kk = keys[vis]                                   # [n, Hkv, d]
        vv = vals[vis]
        qa = qr[a].reshape(Hkv, group, d)                # q heads grouped by their kv head
        s = np.einsum("gjd,ngd->gjn", qa, kk) * scale    # [Hkv, group, n]
        s -= s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=-1, keepdims=True)
        o[a] = np.einsum("gjn,ngd->gjd", p, vv).reshape(Hq, d)
    return o
