"""Flat-stream formulation of a round, float64, for pinning the oracle (CPU only).

This evaluates a round the way Flide lays it out (Flide: Accelerating Decision
Inference with Exact State Forking, §方法步骤详情): one flat stream, an explicit
T x T score matrix masked by the (j, c, t) visibility rule, and the Gated
DeltaNet layer as two calls — all trunks first (each emitting its end state
and conv window into a slot), then all questions, each starting from the slot
its segment's state index names.

It deliberately shares no arithmetic helper with the oracle: rotary positions
go through complex multiplication, the conv uses an explicitly zero-padded
window, and the recurrence multiplies the explicit matrix (I - eta k k^T).
Only the metadata builder (pinned on its own by a hand-derived example) is
reused to place rows.
"""
from __future__ import annotations

import numpy as np

from oracle.layout import build_layout, visible


def rope_complex(x, pos, theta):
    """Rotary embedding via complex numbers: pair (i, i+d/2) as x_i + i*x_{i+d/2}."""
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    freq = np.exp(-np.log(theta) * 2.0 * np.arange(half) / d)
    z = z * np.exp(1j * np.asarray(pos, np.float64)[..., None] * freq)
    return np.concatenate([z.real, z.imag], axis=-1)


def scatter(rnd, lay, name, width_shape):
    """Place request-local payload rows of ``name`` at their stream rows."""
    T = lay["T"]
    out = np.zeros((T,) + tuple(width_shape))
    R = lay["R"]
    for j in range(R):
        pl = rnd.payload(j)
        arr = np.asarray(pl[name], np.float64)
        segs = rnd.segment_rows(j)
        # trunk
        s0, n0 = segs[0]
        r0 = lay["req_trunk_row0"][j]
        out[r0:r0 + n0] = arr[s0:s0 + n0]
        q0 = lay["req_q_seg0"][j]
        for i, (s, L) in enumerate(segs[1:]):
            rr = lay["seg_row0"][q0 + i]
            out[rr:rr + L] = arr[s:s + L]
    return out


def flat_attention(rnd, lay, prefix="attn", window=0):
    sh = rnd.shapes
    T = lay["T"]
    q = scatter(rnd, lay, prefix + "_q", (sh.Hq, sh.d))
    k = scatter(rnd, lay, prefix + "_k", (sh.Hkv, sh.d))
    v = scatter(rnd, lay, prefix + "_v", (sh.Hkv, sh.d))
    tpos = lay["tok_t"][:T]
    qr = rope_complex(q, tpos[:, None], sh.theta)
    kr = rope_complex(k, tpos[:, None], sh.theta)
    jj, cc, tt = lay["tok_j"], lay["tok_c"], lay["tok_t"]
    mask = np.array([[visible(jj[x], cc[x], tt[x], jj[y], cc[y], tt[y], window) for y in range(T)]
                     for x in range(T)], dtype=bool)
    # cached prefix keys of resumed requests: one column block per request
    cache_prefix = "kv" if prefix == "attn" else "swa_kv"
    o = np.zeros((T, sh.Hq, sh.d))
    group = sh.Hq // sh.Hkv
    for h in range(sh.Hq):
        g = h // group
        S = (qr[:, h, :] @ kr[:, g, :].T) / np.sqrt(sh.d)
        S = np.where(mask, S, -np.inf)
        Vall = v[:, g, :]
        extra_s, extra_v = [], []
        for j, r in enumerate(rnd.requests):
            if r.m > 0:
                pl = rnd.payload(j)
                ck = np.asarray(pl[cache_prefix + "_k"], np.float64)[:, g, :]
                cv = np.asarray(pl[cache_prefix + "_v"], np.float64)[:, g, :]
                sc = (qr[:, h, :] @ ck.T) / np.sqrt(sh.d)
                cpos = np.arange(r.m)
                cm = (jj[:T, None] == j) & (cpos[None, :] <= tt[:T, None])
                if window > 0:
                    cm &= (tt[:T, None] - cpos[None, :]) < window
                extra_s.append(np.where(cm, sc, -np.inf))
                extra_v.append(cv)
        if extra_s:
            S = np.concatenate(extra_s + [S], axis=1)
            Vall = np.concatenate(extra_v + [Vall], axis=0)
        mx = S.max(axis=1, keepdims=True)
        P = np.exp(S - mx)
        P /= P.sum(axis=1, keepdims=True)
        o[:, h, :] = P @ Vall
    return o


def _conv_padded(xseg, w, hist):
    """Explicit padded window: rows [hist; xseg], output row t = sum over the K rows ending at t."""
    K = w.shape[1]
    padded = np.vstack([hist, xseg])
    y = np.zeros_like(xseg)
    for t in range(xseg.shape[0]):
        win = padded[t:t + K]              # K rows, the last one is row t of the segment
        y[t] = np.sum(win.T * w, axis=1)
    return y


def _recurrence_explicit(q, k, v, a, e, S):
    H, dv, dk = S.shape
    o = np.zeros((q.shape[0], H, dv))
    I = np.eye(dk)
    for t in range(q.shape[0]):
        for h in range(H):
            M = I - e[t, h] * np.outer(k[t, h], k[t, h])
            S[h] = a[t, h] * (S[h] @ M) + e[t, h] * np.outer(v[t, h], k[t, h])
            o[t, h] = S[h] @ q[t, h]
    return o, S


def flat_gdn(rnd, lay):
    """Two-call GDN over the flat stream; returns (o [T, H, dv], state slots, window slots)."""
    sh = rnd.shapes
    T = lay["T"]
    x = scatter(rnd, lay, "gdn_x", (sh.channels,))
    al = scatter(rnd, lay, "alpha", (sh.H,))
    et = scatter(rnd, lay, "eta", (sh.H,))
    w = np.asarray(rnd.conv_w(), np.float64)
    K = sh.conv_k
    H, dk, dv = sh.H, sh.dk, sh.dv
    o = np.zeros((T, H, dv))
    state_slots, window_slots = {}, {}

    def run_segment(s, S0, hist):
        r0, n = lay["seg_row0"][s], lay["seg_len"][s]
        xs = x[r0:r0 + n]
        y = _conv_padded(xs, w, hist)
        qn = y[:, :H * dk].reshape(n, H, dk)
        kn = y[:, H * dk:2 * H * dk].reshape(n, H, dk)
        vv = y[:, 2 * H * dk:].reshape(n, H, dv)
        qn = qn / np.sqrt((qn ** 2).sum(-1, keepdims=True) + 1e-6)
        kn = kn / np.sqrt((kn ** 2).sum(-1, keepdims=True) + 1e-6)
        oo, S = _recurrence_explicit(qn, kn, vv, al[r0:r0 + n], et[r0:r0 + n], S0.copy())
        o[r0:r0 + n] = oo
        return S, np.vstack([hist, xs])[-(K - 1):]

    R = lay["R"]
    # call 1: all trunk segments
    for s in range(R):
        j = lay["seg_req"][s]
        r = rnd.requests[j]
        if lay["seg_state"][s] >= 0:
            pl = rnd.payload(j)
            S0 = np.asarray(pl["ckpt_state"], np.float64)
            hist = np.asarray(pl["ckpt_window"], np.float64)
        else:
            S0 = np.zeros((H, dv, dk))
            hist = np.zeros((K - 1, sh.channels))
        S, win = run_segment(s, S0, hist)
        state_slots[r.out_slot] = S
        window_slots[r.out_slot] = win
    # call 2: all question segments, each from the slot its state index names
    for s in range(R, lay["n_seg"]):
        slot = lay["seg_state"][s]
        run_segment(s, state_slots[slot], window_slots[slot])
    return o, state_slots, window_slots


def flat_readout(rnd, lay):
    sh = rnd.shapes
    h = scatter(rnd, lay, "hidden", (sh.hidden,))
    probs = []
    qi = 0
    for j, r in enumerate(rnd.requests):
        W = np.asarray(rnd.payload(j)["w_opt"], np.float64)
        off = 0
        for i in range(len(r.q_len)):
            row = lay["qfin_row"][qi]
            z = W[off:off + r.n_opt[i]] @ h[row]
            ez = np.exp(z - z.max())
            probs.append(ez / ez.sum())
            off += r.n_opt[i]
            qi += 1
    return probs


def flat_round(rnd):
    lay = build_layout(rnd.requests)
    out = {"layout": lay, "attn_o": flat_attention(rnd, lay, "attn", 0)}
    if rnd.shapes.swa_window > 0:
        out["swa_o"] = flat_attention(rnd, lay, "swa", rnd.shapes.swa_window)
    out["gdn_o"], out["state_slots"], out["window_slots"] = flat_gdn(rnd, lay)
    out["probs"] = flat_readout(rnd, lay)
    return out


def to_stream(rnd, lay, per_request, key):
    """Map the oracle's request-local outputs ``key`` onto stream rows."""
    first = per_request[0][key]
    out = np.full((lay["T"],) + first.shape[1:], np.nan)
    for j in range(lay["R"]):
        arr = per_request[j][key]
        segs = rnd.segment_rows(j)
        s0, n0 = segs[0]
        r0 = lay["req_trunk_row0"][j]
        out[r0:r0 + n0] = arr[s0:s0 + n0]
        q0 = lay["req_q_seg0"][j]
        for i, (s, L) in enumerate(segs[1:]):
            rr = lay["seg_row0"][q0 + i]
            out[rr:rr + L] = arr[s:s + L]
    return out
