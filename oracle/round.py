"""A whole round of decision requests, evaluated request by request, float64.

Two evaluation orders of the same definition:

* ``isolated`` — the literal definition (Korean summary, §어떻게 동작하나):
  every question ``i`` of request ``r = (s, q_1..q_n)`` runs the prompt
  ``s (+) q_i`` from scratch (``nP + sum|q_i|`` token steps).  Trunk rows come
  out of every prompt; the oracle checks that all prompts agree on them.
* ``memo`` — the trunk is evaluated once and every question continues from a
  copy of the trunk's end state (``P + sum|q_i|`` token steps).  Causality
  makes this the same arithmetic on the same values, so it must agree with
  ``isolated`` (a CPU test checks this); it is used where ``isolated`` is too slow.

A resumed request (``m > 0``) starts from its checkpoint: the stored GDN state
and conv window at ``m`` and the stored keys/values of positions ``0..m-1``
(Korean summary, §어떻게 쓰나).

Inputs are the per-request payloads of ``workloads`` (request-local row
order: trunk rows for positions ``m..P-1``, then each question's rows).
Outputs use the same request-local row order.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .attention import prompt_attention, rope_rotate
from .gdn import gdn_prompt
from .readout import option_probs


def _attn_layer(pl: dict, prefix: str, cache_prefix: str, sh, window: int, req, rows_of_prompt,
                positions, rows=None):
    q = pl[prefix + "_q"][rows_of_prompt]
    k = pl[prefix + "_k"][rows_of_prompt]
    v = pl[prefix + "_v"][rows_of_prompt]
    ck = pl.get(cache_prefix + "_k") if req.m > 0 else None
    cv = pl.get(cache_prefix + "_v") if req.m > 0 else None
    return prompt_attention(q, k, v, positions, sh.theta, window=window, cache_k=ck, cache_v=cv, rows=rows)


def run_request(rnd, j: int, conv_w: Optional[np.ndarray] = None, mode: str = "memo",
                questions: Optional[Sequence[int]] = None, attn_rows: Optional[Sequence[int]] = None,
                payload: Optional[dict] = None, act: str = "none") -> Dict[str, object]:
    """Evaluate request ``j`` of round ``rnd``.

    questions: question indices (0-based) to evaluate (default: all).
    attn_rows: request-local rows whose attention outputs are needed
    (default: all rows of the evaluated segments).  Rows not computed are NaN.
    Returns a dict with ``attn_o`` [n_local, Hq, d], ``swa_o`` (if the round has
    a sliding-window layer), ``gdn_o`` [n_local, H, dv], ``S_P`` [H, dv, dk],
    ``window_P`` [K-1, C] and ``probs`` (list, one array per question; None
    where not evaluated).
    """
    if mode not in ("isolated", "memo"):
        raise ValueError(mode)
    req = rnd.requests[j]
    sh = rnd.shapes
    pl = rnd.payload(j) if payload is None else payload
    if conv_w is None:
        conv_w = rnd.conv_w()
    segs = rnd.segment_rows(j)
    t0, tn = segs[0]
    n_local = t0 + tn + sum(L for _, L in segs[1:])
    qsel = list(range(len(req.q_len))) if questions is None else list(questions)
    layers = [("attn", "kv", 0)]
    if sh.swa_window > 0:
        layers.append(("swa", "swa_kv", sh.swa_window))
    out: Dict[str, object] = {}
    for name, _, _ in layers:
        out[name + "_o"] = np.full((n_local, sh.Hq, sh.d), np.nan)
    out["gdn_o"] = np.full((n_local, sh.H, sh.dv), np.nan)
    out["probs"] = [None] * len(req.q_len)

    window0 = pl.get("ckpt_window") if req.m > 0 else None
    S0 = pl.get("ckpt_state") if req.m > 0 else None
    trunk_rows = np.arange(t0, t0 + tn)
    trunk_pos = np.arange(req.m, req.P)
    wanted = None if attn_rows is None else set(int(a) for a in attn_rows)

    # ---- trunk: the trunk-only prompt (its end state is S_P) ----
    o_g, S_P, win_P = gdn_prompt(pl["gdn_x"][trunk_rows], pl["alpha"][trunk_rows], pl["eta"][trunk_rows],
                                 conv_w, sh.H, sh.dk, sh.dv, window0, S0, act)
    out["gdn_o"][trunk_rows] = o_g
    out["S_P"] = S_P
    out["window_P"] = win_P
    for name, cpre, W in layers:
        sel = None
        if wanted is not None:
            sel = [a for a in range(tn) if (t0 + a) in wanted]
        o_a = _attn_layer(pl, name, cpre, sh, W, req, trunk_rows, trunk_pos, rows=sel)
        if sel is None:
            out[name + "_o"][trunk_rows] = o_a
        else:
            out[name + "_o"][[t0 + a for a in sel]] = o_a[sel]

    # ---- questions ----
    for i in qsel:
        qs, L = segs[1 + i]
        q_rows = np.arange(qs, qs + L)
        q_pos = np.arange(req.P, req.P + L)
        if mode == "isolated":
            rows_p = np.concatenate([trunk_rows, q_rows])
            pos_p = np.concatenate([trunk_pos, q_pos])
            o_g, _, _ = gdn_prompt(pl["gdn_x"][rows_p], pl["alpha"][rows_p], pl["eta"][rows_p],
                                   conv_w, sh.H, sh.dk, sh.dv, window0, S0, act)
            if not np.array_equal(o_g[:tn], out["gdn_o"][trunk_rows]):
                raise AssertionError("isolated prompts disagree on trunk rows (GDN)")
            out["gdn_o"][q_rows] = o_g[tn:]
            for name, cpre, W in layers:
                if wanted is None:
                    sel = None
                else:
                    sel = [a for a in range(tn + L) if (t0 + a if a < tn else qs + a - tn) in wanted]
                o_a = _attn_layer(pl, name, cpre, sh, W, req, rows_p, pos_p, rows=sel)
                tr_sel = range(tn) if sel is None else [a for a in sel if a < tn]
                for a in tr_sel:
                    if not np.array_equal(o_a[a], out[name + "_o"][t0 + a]):
                        raise AssertionError("isolated prompts disagree on trunk rows (attention)")
                q_sel = range(tn, tn + L) if sel is None else [a for a in sel if a >= tn]
                for a in q_sel:
                    out[name + "_o"][qs + a - tn] = o_a[a]
        else:
            o_g, _, _ = gdn_prompt(pl["gdn_x"][q_rows], pl["alpha"][q_rows], pl["eta"][q_rows],
                                   conv_w, sh.H, sh.dk, sh.dv, win_P, S_P, act)
            out["gdn_o"][q_rows] = o_g
            rows_p = np.concatenate([trunk_rows, q_rows])
            pos_p = np.concatenate([trunk_pos, q_pos])
            for name, cpre, W in layers:
                if wanted is None:
                    sel = list(range(tn, tn + L))
                else:
                    sel = [a for a in range(tn, tn + L) if (qs + a - tn) in wanted]
                o_a = _attn_layer(pl, name, cpre, sh, W, req, rows_p, pos_p, rows=sel)
                for a in sel:
                    out[name + "_o"][qs + a - tn] = o_a[a]
        # readout on the question's final row, Eq. (1)
        off = int(sum(req.n_opt[:i]))
        h = pl["hidden"][qs + L - 1]
        out["probs"][i] = option_probs(h, pl["w_opt"][off:off + req.n_opt[i]])
    return out


def make_checkpoint(rnd, j: int, save_m: int, conv_w: Optional[np.ndarray] = None,
                    payload: Optional[dict] = None, act: str = "none") -> Dict[str, np.ndarray]:
    """The checkpoint of request ``j`` at trunk position ``save_m`` (``m < save_m <= P``): what a later
    round resumes from (Korean summary, §어떻게 쓰나).  It is the trunk-only prompt cut at ``save_m``:
    the GDN state after position ``save_m - 1``, the raw conv window of the ``K - 1`` positions before
    ``save_m``, and per attention layer the rotated keys and the values of positions ``0..save_m-1``
    (positions below the request's own resume point ``m`` are those of its checkpoint).  Keys are named
    like a resumed request's payload: ``ckpt_state``, ``ckpt_window``, ``kv_k``, ``kv_v`` (and
    ``swa_kv_k``, ``swa_kv_v`` with a sliding-window layer)."""
    req = rnd.requests[j]
    if not req.m < save_m <= req.P:
        raise ValueError("need m < save_m <= P")
    sh = rnd.shapes
    pl = rnd.payload(j) if payload is None else payload
    if conv_w is None:
        conv_w = rnd.conv_w()
    t0, _ = rnd.segment_rows(j)[0]
    rows = np.arange(t0, t0 + save_m - req.m)
    pos = np.arange(req.m, save_m)
    window0 = pl.get("ckpt_window") if req.m > 0 else None
    S0 = pl.get("ckpt_state") if req.m > 0 else None
    _, S, win = gdn_prompt(pl["gdn_x"][rows], pl["alpha"][rows], pl["eta"][rows], conv_w, sh.H, sh.dk, sh.dv,
                           window0, S0, act)
    out: Dict[str, np.ndarray] = {"ckpt_state": S, "ckpt_window": win}
    layers = [("attn", "kv")] + ([("swa", "swa_kv")] if sh.swa_window > 0 else [])
    for name, cpre in layers:
        kr = rope_rotate(np.asarray(pl[name + "_k"][rows], np.float64), pos[:, None], sh.theta)
        v = np.asarray(pl[name + "_v"][rows], np.float64)
        if req.m > 0:
            kr = np.concatenate([np.asarray(pl[cpre + "_k"], np.float64), kr], axis=0)
            v = np.concatenate([np.asarray(pl[cpre + "_v"], np.float64), v], axis=0)
        out[cpre + "_k"] = kr
        out[cpre + "_v"] = v
    return out


def run_round(rnd, mode: str = "memo", conv_w: Optional[np.ndarray] = None) -> List[Dict[str, object]]:
    """Evaluate every request of ``rnd`` (see ``run_request``)."""
    if conv_w is None:
        conv_w = rnd.conv_w()
    return [run_request(rnd, j, conv_w, mode) for j in range(len(rnd.requests))]
