"""Gated DeltaNet layer of one isolated prompt, float64.

The layer (Flide: Accelerating Decision Inference with Exact State Forking,
§前置知识, gated delta rule): a short causal convolution, then per head the
recurrence

    S_t = alpha_t * S_{t-1} (I - eta_t k_t k_t^T) + eta_t v_t k_t^T,    o_t = S_t q_t

with the state ``S`` of shape [dv, dk].  The two-call fork (§方法步骤详情)
must reproduce exactly this per-token recurrence run over ``s (+) q_i``.

Readings where the pages are silent (all listed in the design notes):
* the input row packs the channels as q (H*dk) | k (H*dk) | v (H*dv), head-major;
* the conv is depthwise over those raw channels, width K, tap ``K-1``
  multiplying the current row; a fresh prompt has zero history, a resumed one
  the K-1 raw rows stored with its checkpoint; no bias, no activation;
* q and k are L2-normalised per head after the conv: ``x / sqrt(sum x^2 + 1e-6)``;
* the output has no extra scale, gate or norm;
* the conv window handed on after a prompt is its last K-1 raw input rows.

Pinned by tests/test_oracle_gdn.py (tap probe, eta = 0 closed form, one-hot
associative memory, d_k = 1 scalar closed form, explicit-matrix form of the
recurrence, and state/window continuation).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

L2_EPS = 1e-6


def causal_conv(x: np.ndarray, w: np.ndarray, history: np.ndarray) -> np.ndarray:
    """Depthwise causal conv: ``y_t[ch] = sum_tau w[ch, tau] * x_{t-(K-1)+tau}[ch]``.

    x: [L, C] raw inputs; w: [C, K]; history: [K-1, C] raw rows preceding x
    (oldest first).  Returns y: [L, C].
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    K = w.shape[1]
    L = x.shape[0]
    ext = np.concatenate([np.asarray(history, np.float64).reshape(K - 1, x.shape[1]), x], axis=0)
    y = np.zeros_like(x)
    for tau in range(K):
        y += w[:, tau] * ext[tau:tau + L]
    return y


def l2_normalise(x: np.ndarray) -> np.ndarray:
    """Normalise the last axis: ``x / sqrt(sum(x^2) + 1e-6)``."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)


def gated_delta_rule(q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray,
                     eta: np.ndarray, S0: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token recurrence over L tokens for all heads at once.

    q, k: [L, H, dk] (normalised); v: [L, H, dv]; alpha, eta: [L, H];
    S0: [H, dv, dk].  Returns (o [L, H, dv], S_L [H, dv, dk]).
    ``S (I - eta k k^T)`` is evaluated as ``S - eta (S k) k^T`` (associativity).
    """
    L, H, dk = q.shape
    dv = v.shape[2]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((L, H, dv), np.float64)
    for t in range(L):
        a = alpha[t][:, None, None]
        e = eta[t][:, None, None]
        kt = k[t]
        Sk = np.einsum("hvk,hk->hv", S, kt)
        S = a * (S - e * Sk[:, :, None] * kt[:, None, :]) + e * v[t][:, :, None] * kt[:, None, :]
        o[t] = np.einsum("hvk,hk->hv", S, q[t])
    return o, S


def split_channels(y: np.ndarray, H: int, dk: int, dv: int):
    """Split packed rows [L, H*(2dk+dv)] into q, k [L, H, dk] and v [L, H, dv]."""
    L = y.shape[0]
    q = y[:, :H * dk].reshape(L, H, dk)
    k = y[:, H * dk:2 * H * dk].reshape(L, H, dk)
    v = y[:, 2 * H * dk:].reshape(L, H, dv)
    return q, k, v


def gdn_prompt(x: np.ndarray, alpha: np.ndarray, eta: np.ndarray, conv_w: np.ndarray,
               H: int, dk: int, dv: int, window0: Optional[np.ndarray] = None,
               S0: Optional[np.ndarray] = None, act: str = "none"):
    """Run the GDN layer over prompt rows ``x`` [L, C] from (window0, S0).

    window0: [K-1, C] raw rows before x (zeros if None); S0: [H, dv, dk] (zeros if None).
    Returns (o [L, H, dv], S_end [H, dv, dk], window_end [K-1, C]).
    """
    x = np.asarray(x, np.float64)
    K = conv_w.shape[1]
    C = x.shape[1]
    hist = np.zeros((K - 1, C)) if window0 is None else np.asarray(window0, np.float64)
    y = causal_conv(x, conv_w, hist)
    if act == "silu":
        y = y / (1.0 + np.exp(-y))
    q, k, v = split_channels(y, H, dk, dv)
    qn, kn = l2_normalise(q), l2_normalise(k)
    S_init = np.zeros((H, dv, dk)) if S0 is None else np.asarray(S0, np.float64)
    o, S = gated_delta_rule(qn, kn, v, np.asarray(alpha, np.float64), np.asarray(eta, np.float64), S_init)
    window_end = np.concatenate([hist, x], axis=0)[-(K - 1):] if K > 1 else np.zeros((0, C))
    return o, S, window_end
