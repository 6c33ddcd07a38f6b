"""Flat-stream formulation of a multi-layer stack round, float64, for pinning the stack oracle (CPU only).

Every layer runs over the whole flat stream at once, the way Flide lays a round out (Flide: Accelerating
Decision Inference with Exact State Forking, §方法步骤详情): attention through an explicit T x T score
matrix masked by the (j, c, t) visibility rule, the Gated DeltaNet layer as two calls (trunks first, each
emitting its end state and conv window into its slot; then every question from the slot its segment names),
and the row-wise layers applied to every row.  It reuses the independent helpers of tests/brute.py
(complex-number rotation, explicitly padded conv, explicit-matrix recurrence) and shares no arithmetic
with the oracle.
"""
from __future__ import annotations

import numpy as np

from oracle.layout import build_layout, visible
from tests.brute import _conv_padded, _recurrence_explicit, rope_complex


def _norm(x, g, eps=1e-6):
    return x / np.sqrt((x ** 2).sum(-1, keepdims=True) / x.shape[-1] + eps) * np.asarray(g, np.float64)


def _lin(x, w):
    return np.einsum("tk,nk->tn", x, np.asarray(w, np.float64))


def _flat_attn(s, lay, q, k, v, window):
    T = lay["T"]
    tpos = lay["tok_t"][:T]
    qr = rope_complex(q, tpos[:, None], s.theta)
    kr = rope_complex(k, tpos[:, None], s.theta)
    jj, cc, tt = lay["tok_j"], lay["tok_c"], lay["tok_t"]
    mask = np.array([[visible(jj[x], cc[x], tt[x], jj[y], cc[y], tt[y], window) for y in range(T)]
                     for x in range(T)], dtype=bool)
    o = np.zeros((T, s.Hq, s.d))
    group = s.Hq // s.Hkv
    for h in range(s.Hq):
        g = h // group
        S = np.where(mask, (qr[:, h] @ kr[:, g].T) / np.sqrt(s.d), -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        o[:, h] = (P / P.sum(axis=1, keepdims=True)) @ v[:, g]
    return o


def _flat_gdn(s, lay, requests, xg, alpha, eta, conv_w):
    T, H, dk, dv, K = lay["T"], s.H, s.dk, s.dv, s.conv_k
    w = np.asarray(conv_w, np.float64)
    o = np.zeros((T, H, dv))
    states, windows = {}, {}

    def run(seg, S0, hist):
        r0, n = lay["seg_row0"][seg], lay["seg_len"][seg]
        xs = xg[r0:r0 + n]
        y = _conv_padded(xs, w, hist)
        qn = y[:, :H * dk].reshape(n, H, dk)
        kn = y[:, H * dk:2 * H * dk].reshape(n, H, dk)
        vv = y[:, 2 * H * dk:].reshape(n, H, dv)
        qn = qn / np.sqrt((qn ** 2).sum(-1, keepdims=True) + 1e-6)
        kn = kn / np.sqrt((kn ** 2).sum(-1, keepdims=True) + 1e-6)
        oo, S = _recurrence_explicit(qn, kn, vv, alpha[r0:r0 + n], eta[r0:r0 + n], S0.copy())
        o[r0:r0 + n] = oo
        return S, np.vstack([hist, xs])[-(K - 1):]

    R = lay["R"]
    for seg in range(R):  # call 1: trunks
        slot = requests[lay["seg_req"][seg]].out_slot
        states[slot], windows[slot] = run(seg, np.zeros((H, dv, dk)), np.zeros((K - 1, xg.shape[1])))
    for seg in range(R, lay["n_seg"]):  # call 2: questions, by state index
        slot = lay["seg_state"][seg]
        run(seg, states[slot], windows[slot])
    return o


def flat_stack(stack):
    """Per layer the stream rows of x (n_layers + 1 arrays [T, Dm]) and the probabilities of every question
    (stream order)."""
    s = stack.shapes
    w = stack.weights()
    lay = build_layout(stack.requests)
    T = lay["T"]
    x = np.zeros((T, s.Dm))
    for j in range(len(stack.requests)):
        x0 = np.asarray(stack.payload(j)["x0"], np.float64)
        segs = stack.segment_rows(j)
        r0 = lay["req_trunk_row0"][j]
        x[r0:r0 + segs[0][1]] = x0[:segs[0][1]]
        for i, (a, L) in enumerate(segs[1:]):
            rr = lay["seg_row0"][lay["req_q_seg0"][j] + i]
            x[rr:rr + L] = x0[a:a + L]
    xs = [x]
    for L in w["layers"]:
        h = _norm(x, L["norm1"])
        if L["kind"] == "gdn":
            xg = _lin(h, L["w_x"])
            ab = _lin(h, L["w_ab"]) + np.asarray(L["b_ab"], np.float64)
            al, et = 1 / (1 + np.exp(-ab[:, :s.H])), 1 / (1 + np.exp(-ab[:, s.H:]))
            mix = _flat_gdn(s, lay, stack.requests, xg, al, et, L["conv_w"]).reshape(T, -1)
        else:
            q = _lin(h, L["w_q"]).reshape(T, s.Hq, s.d)
            k = _lin(h, L["w_k"]).reshape(T, s.Hkv, s.d)
            v = _lin(h, L["w_v"]).reshape(T, s.Hkv, s.d)
            mix = _flat_attn(s, lay, q, k, v, s.window if L["kind"] == "swa" else 0).reshape(T, -1)
        x = x + _lin(mix, L["w_o"])
        h2 = _norm(x, L["norm2"])
        gu = _lin(h2, L["gate_up"])
        F = gu.shape[1] // 2
        x = x + _lin(gu[:, :F] * np.exp(-np.logaddexp(0.0, -gu[:, :F])) * gu[:, F:], L["down"])
        xs.append(x)
    probs = []
    qi = 0
    for j, r in enumerate(stack.requests):
        W = np.asarray(stack.payload(j)["w_opt"], np.float64)
        off = 0
        for i in range(len(r.q_len)):
            hf = _norm(x[lay["qfin_row"][qi]][None, :], w["norm_f"])[0]
            z = W[off:off + r.n_opt[i]] @ hf
            ez = np.exp(z - z.max())
            probs.append(ez / ez.sum())
            off += r.n_opt[i]
            qi += 1
    return {"layout": lay, "xs": xs, "probs": probs}
