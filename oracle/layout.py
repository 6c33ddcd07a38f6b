"""Flat-stream metadata of a round, built independently of the HIP library's planner.

Readings of the pages (Flide: Accelerating Decision Inference with Exact State
Forking, §方法步骤详情 and §核心方法; the Korean summary, §무엇과 다른가):

* Stream order: every request's trunk ("state segment") first, in request
  order, then every question segment, grouped by request and in question
  order inside a request.  No padding between segments; rows past ``T`` up to
  the capacity are tail padding.
* Per row ``(j, c, t)``: request index, branch (``0`` for the trunk, ``i`` for
  question ``i``, 1-based), and position.  Trunk row ``k`` of a request resumed
  at ``m`` has ``t = m + k``; question rows continue from ``P``:
  ``t = P + u``.  Tail rows carry ``(-1, -1, -1)``.
* State index of a segment: a question reads its request's output slot (where
  the trunk call leaves ``S_P`` and the conv window); a trunk reads its
  checkpoint slot when it resumes (``m > 0``) and ``-1`` (zero state) otherwise.
* Splitting (Korean summary, §어떻게 쓰나): a round larger than the largest
  capacity is cut at request boundaries, greedily in request order; a single
  request larger than the capacity becomes its own sub-round that runs without
  a graph ("eager").

Pinned by tests/test_oracle_layout.py (hand-derived worked example of the
one-request, three-question round and brute-force visibility counts).
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np


def request_rows(r) -> int:
    """Stream rows of one request: the new trunk rows plus every question row."""
    return (r.P - r.m) + sum(int(x) for x in r.q_len)


def build_layout(requests: Sequence, t_cap: int | None = None) -> Dict[str, np.ndarray]:
    """Metadata of the flat stream for ``requests`` (objects with P, m, q_len, ckpt_slot, out_slot).

    Returns int32 arrays: ``seg_row0, seg_len, seg_req, seg_branch, seg_pos0,
    seg_state`` (one entry per segment, trunks first), ``req_trunk_row0,
    req_q_seg0`` (per request), ``qfin_row`` (last row of every question, in
    stream order), ``tok_j, tok_c, tok_t`` (per row up to ``t_cap``) and the
    scalars ``T``, ``R``, ``n_seg``, ``n_qst``.
    """
    R = len(requests)
    for r in requests:
        if not (0 <= r.m <= r.P):
            raise ValueError("need 0 <= m <= P")
        if r.m > 0 and r.ckpt_slot < 0:
            raise ValueError("a resumed request needs a checkpoint slot")
        if any(int(L) < 1 for L in r.q_len):
            raise ValueError("every question needs at least one token")
    segs: List[Tuple[int, int, int, int, int, int]] = []
    trunk_row0 = []
    row = 0
    for j, r in enumerate(requests):
        trunk_row0.append(row)
        n_new = r.P - r.m
        segs.append((row, n_new, j, 0, r.m, r.ckpt_slot if r.m > 0 else -1))
        row += n_new
    q_seg0 = []
    qfin = []
    for j, r in enumerate(requests):
        q_seg0.append(len(segs))
        for i, L in enumerate(r.q_len, start=1):
            L = int(L)
            segs.append((row, L, j, i, r.P, r.out_slot))
            qfin.append(row + L - 1)
            row += L
    T = row
    if t_cap is None:
        t_cap = T
    if T > t_cap:
        raise ValueError("round does not fit the capacity")
    seg = np.array(segs, dtype=np.int32).reshape(-1, 6)
    tok_j = np.full(t_cap, -1, np.int32)
    tok_c = np.full(t_cap, -1, np.int32)
    tok_t = np.full(t_cap, -1, np.int32)
    for row0, n, j, c, pos0, _state in segs:
        tok_j[row0:row0 + n] = j
        tok_c[row0:row0 + n] = c
        tok_t[row0:row0 + n] = pos0 + np.arange(n)
    return {
        "T": T, "R": R, "n_seg": len(segs), "n_qst": len(qfin),
        "seg_row0": seg[:, 0].copy(), "seg_len": seg[:, 1].copy(), "seg_req": seg[:, 2].copy(),
        "seg_branch": seg[:, 3].copy(), "seg_pos0": seg[:, 4].copy(), "seg_state": seg[:, 5].copy(),
        "req_trunk_row0": np.array(trunk_row0, np.int32), "req_q_seg0": np.array(q_seg0, np.int32),
        "qfin_row": np.array(qfin, np.int32),
        "tok_j": tok_j, "tok_c": tok_c, "tok_t": tok_t,
    }


def visible(jx: int, cx: int, tx: int, jy: int, cy: int, ty: int, window: int = 0) -> bool:
    """Full-attention visibility of key row y from query row x (tail rows see nothing).

    Same request, key on the trunk or on the query's own branch, key position
    not after the query position; a sliding-window layer additionally needs
    ``tx - ty < window`` (``window == 0`` means no window).
    """
    if jx < 0 or jy < 0:
        return False
    ok = (jy == jx) and (cy == 0 or cy == cx) and (ty <= tx)
    if ok and window > 0:
        ok = (tx - ty) < window
    return ok


def split_round(requests: Sequence, t_max: int) -> Tuple[List[int], List[bool]]:
    """Cut a round at request boundaries into sub-rounds of at most ``t_max`` rows.

    Greedy in request order.  A request with more than ``t_max`` rows forms a
    sub-round of its own, flagged eager (run without a captured graph).
    Returns ``(sub_first, eager)`` with ``sub_first`` of length ``n_sub + 1``.
    """
    if t_max < 1:
        raise ValueError("t_max must be positive")
    first = [0]
    eager: List[bool] = []
    cur_rows = 0
    cur_n = 0
    for j, r in enumerate(requests):
        n = request_rows(r)
        if n > t_max:
            if cur_n:
                first.append(j)
                eager.append(False)
            first.append(j + 1)
            eager.append(True)
            cur_rows, cur_n = 0, 0
            continue
        if cur_n and cur_rows + n > t_max:
            first.append(j)
            eager.append(False)
            cur_rows, cur_n = 0, 0
        cur_rows += n
        cur_n += 1
    if cur_n:
        first.append(len(requests))
        eager.append(False)
    return first, eager
