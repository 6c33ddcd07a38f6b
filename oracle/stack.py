"""A multi-layer hybrid stack over isolated prompts, float64 — TEST INFRASTRUCTURE ONLY.

What a stack of token mixers with pointwise layers between them must produce: Proposition 3.1 of the
Korean summary (§무엇과 다른가; "命题 1" of "Flide: Accelerating Decision Inference with Exact State
Forking", §核心方法) is proved by induction over layers, because every layer other than the token mixers
acts row by row (§方法步骤详情, second step).  So every question ``s (+) q_i`` is run as its own prompt
through every layer, and only its last row is read out (§方法步骤详情, fourth step; Eq. (1)).

One layer (pre-norm residual block; the pages fix no block structure, so this is the plainest hybrid
layer, read as listed in the design notes):

    h = rms_norm(x, norm1);  x = x + mixer(h) W_o^T;  h2 = rms_norm(x, norm2)
    x = x + (silu(h2 W_gate^T) * (h2 W_up^T)) W_down^T

with mixer = the Gated DeltaNet layer of oracle.gdn (inputs h W_x^T, alpha = sigmoid(a), eta = sigmoid(e)
for (a, e) = h W_ab^T + b_ab), or the causal attention of oracle.attention over q = h W_q^T, k = h W_k^T,
v = h W_v^T (full, or windowed for a sliding-window layer).  After the last layer the question-final row
is normalised with norm_f and read out: p = softmax(W_opt h_f).

Pinned by tests/test_oracle_stack.py: closed forms of rms_norm and silu; a stack whose output
projections are all zero is the identity on x; a flat-stream multi-layer brute force (masked attention
over the whole stream and the two-call GDN with state indices, layer after layer) equals the isolated
prompts; sibling perturbation; memo order equals isolated order.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from .attention import prompt_attention
from .gdn import gdn_prompt
from .readout import option_probs

NORM_EPS = 1e-6


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float = NORM_EPS) -> np.ndarray:
    """``x / sqrt(mean(x^2) + eps) * g`` over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """``x W^T`` for a weight stored [out, in], one row at a time, so that a row's value does not depend on
    which other rows are evaluated with it (a matrix product's blocking may change its rounding)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    if x.ndim == 1:
        return w @ x
    out = np.empty(x.shape[:-1] + (w.shape[0],))
    for i in range(x.shape[0]):
        out[i] = w @ x[i]
    return out


def mlp(h2: np.ndarray, L: dict) -> np.ndarray:
    gu = linear(h2, L["gate_up"])
    F = gu.shape[-1] // 2
    return linear(silu(gu[..., :F]) * gu[..., F:], L["down"])


class LayerState:
    """What a trunk leaves to its continuations in one layer: the keys and values of its rows (attention)
    or its end state and conv window (GDN)."""

    def __init__(self):
        self.q = self.k = self.v = self.pos = None
        self.S = self.window = None


def mixer(shapes, L: dict, h: np.ndarray, pos: np.ndarray, prev: Optional[LayerState] = None,
          keep: bool = False):
    """Token mixer of one layer over rows h at positions pos, continuing the prefix ``prev`` (None: a fresh
    prompt).  Returns (output [rows, Dm] after W_o, state of the prefix extended by these rows if keep)."""
    s = shapes
    rows = len(h)
    st = LayerState() if keep else None
    if L["kind"] == "gdn":
        xg = linear(h, L["w_x"])
        ab = linear(h, L["w_ab"]) + np.asarray(L["b_ab"], np.float64)
        alpha, eta = sigmoid(ab[:, :s.H]), sigmoid(ab[:, s.H:])
        o, S, win = gdn_prompt(xg, alpha, eta, L["conv_w"], s.H, s.dk, s.dv,
                               None if prev is None else prev.window, None if prev is None else prev.S)
        if keep:
            st.S, st.window = S, win
        return linear(o.reshape(rows, s.H * s.dv), L["w_o"]), st
    q = linear(h, L["w_q"]).reshape(rows, s.Hq, s.d)
    k = linear(h, L["w_k"]).reshape(rows, s.Hkv, s.d)
    v = linear(h, L["w_v"]).reshape(rows, s.Hkv, s.d)
    W = s.window if L["kind"] == "swa" else 0
    if prev is not None:
        q_all = np.concatenate([prev.q, q])
        k_all = np.concatenate([prev.k, k])
        v_all = np.concatenate([prev.v, v])
        p_all = np.concatenate([prev.pos, pos])
        n0 = len(prev.q)
        o = prompt_attention(q_all, k_all, v_all, p_all, s.theta, window=W, rows=range(n0, n0 + rows))[n0:]
    else:
        o = prompt_attention(q, k, v, pos, s.theta, window=W)
    if keep:
        st.q, st.k, st.v = (q, k, v) if prev is None else (q_all, k_all, v_all)
        st.pos = pos if prev is None else p_all
    return linear(o.reshape(rows, s.Hq * s.d), L["w_o"]), st


def run_layers(shapes, weights: dict, x: np.ndarray, pos: np.ndarray, prev: Optional[List[LayerState]] = None,
               keep: bool = False):
    """Every layer over rows x (continuing per-layer prefixes ``prev``).  Returns (per-layer inputs and the
    final x: a list of n_layers + 1 arrays, per-layer states of the extended prefix if keep)."""
    xs = [np.asarray(x, np.float64)]
    states = []
    for li, L in enumerate(weights["layers"]):
        x = xs[-1]
        mix, st = mixer(shapes, L, rms_norm(x, L["norm1"]), pos, None if prev is None else prev[li], keep)
        x = x + mix
        x = x + mlp(rms_norm(x, L["norm2"]), L)
        xs.append(x)
        states.append(st)
    return xs, states


def run_stack_request(stack, j: int, mode: str = "memo") -> Dict[str, object]:
    """Request j of a stack round.  Returns ``xs`` (n_layers + 1 arrays [rows, Dm] in request-local order:
    the input of every layer and the final output), ``hf`` (the normalised final row of every question)
    and ``probs`` (one array per question)."""
    if mode not in ("isolated", "memo"):
        raise ValueError(mode)
    s = stack.shapes
    w = stack.weights()
    req = stack.requests[j]
    pl = stack.payload(j)
    segs = stack.segment_rows(j)
    t0, tn = segs[0]
    n_local = t0 + tn + sum(L for _, L in segs[1:])
    nl = len(s.layers)
    xs = [np.full((n_local, s.Dm), np.nan) for _ in range(nl + 1)]
    trunk = np.arange(t0, t0 + tn)
    tpos = np.arange(0, req.P)
    x0 = np.asarray(pl["x0"], np.float64)
    states = None
    if mode == "memo":
        out_t, states = run_layers(s, w, x0[trunk], tpos, keep=True)
        for li in range(nl + 1):
            xs[li][trunk] = out_t[li]
    hf, probs = [], []
    for i, (qs, L) in enumerate(segs[1:]):
        qrows = np.arange(qs, qs + L)
        qpos = np.arange(req.P, req.P + L)
        if mode == "memo":
            out_q, _ = run_layers(s, w, x0[qrows], qpos, prev=states if tn > 0 else None)
            for li in range(nl + 1):
                xs[li][qrows] = out_q[li]
        else:
            rows_p = np.concatenate([trunk, qrows])
            out_p, _ = run_layers(s, w, x0[rows_p], np.concatenate([tpos, qpos]))
            for li in range(nl + 1):
                if i > 0 and not np.array_equal(out_p[li][:tn], xs[li][trunk]):
                    raise AssertionError("isolated prompts disagree on trunk rows")
                xs[li][rows_p] = out_p[li]
        f = rms_norm(xs[nl][qs + L - 1], w["norm_f"])
        hf.append(f)
        off = int(sum(req.n_opt[:i]))
        probs.append(option_probs(f, pl["w_opt"][off:off + req.n_opt[i]]))
    if mode == "isolated" and not segs[1:]:
        out_t, _ = run_layers(s, w, x0[trunk], tpos)
        for li in range(nl + 1):
            xs[li][trunk] = out_t[li]
    return {"xs": xs, "hf": hf, "probs": probs}
