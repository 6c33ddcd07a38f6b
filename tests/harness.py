"""Helpers for the GPU parity tests: run a round through the C ABI, map outputs, measure errors.

Placement of payload rows uses the oracle's independent layout builder, so a
planner mistake shows up as a parity failure rather than being mapped back
consistently.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from oracle import layout as olayout
from oracle import round as oround

TOL = {"bf16": 2e-2, "f32": 1e-4}
TV_TOL = 1e-3


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over (row, head) of ||y - y^||_inf / max(||y^||_inf, 1e-6); NaN rows of ref are skipped."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ok = ~np.isnan(ref).any(axis=-1)
    if not ok.any():
        return 0.0
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-6)
    return float((num / den)[ok].max())


def tv(p, q) -> float:
    return 0.5 * float(np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)).sum())


def stream_rows(rnd, lay, j: int) -> np.ndarray:
    """Stream row of every request-local row of request j (trunk, then questions)."""
    segs = rnd.segment_rows(j)
    out = []
    s0, n0 = segs[0]
    r0 = int(lay["req_trunk_row0"][j])
    out.extend(range(r0, r0 + n0))
    q0 = int(lay["req_q_seg0"][j])
    for i, (_, L) in enumerate(segs[1:]):
        rr = int(lay["seg_row0"][q0 + i])
        out.extend(range(rr, rr + L))
    return np.asarray(out, np.int64)


def run_gpu(rnd, ctx, mode: str = "direct", spec=None, bufs=None, repeats: int = 1):
    """Run ``rnd`` on the GPU; returns (bufs, layout).  mode: direct | graph | eager."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    from tree_forked_hybrid_amd.runner import RoundBuffers, spec_for_round

    lay = olayout.build_layout(rnd.requests)
    if bufs is None:
        bufs = RoundBuffers(spec or spec_for_round(rnd))
    bufs.fill(rnd, lay)
    img = F.flide_plan_round(rnd.requests, bufs.caps)
    print(f"[gpu] mode={mode} T={lay['T']} R={lay['R']} n_q={lay['n_qst']} caps=({bufs.caps.T_cap},"
          f"{bufs.caps.R_cap},{bufs.caps.Q_cap}) dtype={rnd.dtype}", flush=True)
    bid = None
    if mode == "graph":
        bid = F.flide_graph_capture(ctx, bufs.round_bufs())
    for _ in range(repeats):
        if mode == "direct":
            bufs.upload(ctx, img)
            bufs.run_layers(ctx)
        elif mode == "graph":
            F.flide_graph_replay(ctx, bid, img)
        elif mode == "eager":
            F.flide_round_eager(ctx, bufs.round_bufs(), img)
        else:
            raise ValueError(mode)
    torch.cuda.synchronize()
    if bid is not None:  # the graph holds the buffers' addresses: release it before they can be freed
        F.flide_graph_release(ctx, bid)
    F.flide_check_device(ctx, bufs.caps, bufs.dev_meta)
    return bufs, lay


def run_split(rnd, tables, t_max: Optional[int] = None, co_schedule: bool = False):
    """Run ``rnd`` through bucket tables: split at request boundaries for the tables' largest capacity (or
    ``t_max``), sub-round k filled into table k mod len(tables) (placement by the oracle's layout) and all
    sub-rounds replayed back to back, each in the smallest bucket that holds it (co_schedule: True lets
    runner.FrontScheduler choose its schedule, "overlap" forces the trunk GDN calls beside the attention).  Tables must not be reused
    within one call (len(tables) >= number of sub-rounds).  Returns [(sub-round, table, layout)]."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    t_max = t_max or max(c.T_cap for t in tables for c, _, _ in t.buckets.values())
    first, eager = F.flide_split_round(rnd.requests, t_max)
    assert not any(eager) and len(eager) <= len(tables), (eager, len(tables))
    out = []
    for k in range(len(eager)):
        sub = rnd.subset(list(range(first[k], first[k + 1])))
        lay = olayout.build_layout(sub.requests)
        tables[k].bufs.fill(sub, lay)
        out.append((sub, tables[k], lay))
    if co_schedule:
        from tree_forked_hybrid_amd.runner import FrontScheduler
        sched = FrontScheduler(len(out), overlap_attention=True if co_schedule == "overlap" else None)
        sched.run([tab for _, tab, _ in out], [sub.requests for sub, _, _ in out])
        print(f"[gpu] schedule: {sched.last_mode}", flush=True)
    else:
        for sub, tab, _ in out:
            tab.run(sub.requests)
    for sub, tab, _ in out:
        print(f"[gpu] split sub-round: {len(sub.requests)} requests, T={tab.last[1][tab.bufs.layout.hdr]} "
              f"bucket T_cap={tab.caps_of(tab.last[0]).T_cap}", flush=True)
    torch.cuda.synchronize()
    for _, tab, _ in out:
        tab.check()
    return out


def outputs(bufs) -> Dict[str, np.ndarray]:
    """Host copies (float64) of every output buffer."""
    out = {"attn_o": bufs.o_attn[0].float().cpu().numpy().astype(np.float64),
           "gdn_o": bufs.o_gdn.float().cpu().numpy().astype(np.float64),
           "probs": bufs.probs.cpu().numpy().astype(np.float64),
           "state_pool": bufs.state_pool.cpu().numpy().astype(np.float64),
           "conv_pool": bufs.conv_pool.float().cpu().numpy().astype(np.float64)}
    if bufs.n_attn == 2:
        out["swa_o"] = bufs.o_attn[1].float().cpu().numpy().astype(np.float64)
    return out


def compare_request(rnd, lay, got: Dict[str, np.ndarray], ref: Dict[str, object], j: int, opt_offsets,
                    report: Optional[dict] = None, questions: Optional[Sequence[int]] = None) -> dict:
    """Errors of request j: attention, SWA, GDN (rows the oracle computed), S_P, window, TV."""
    rows = stream_rows(rnd, lay, j)
    rep = {} if report is None else report
    for key in ("attn_o", "swa_o", "gdn_o"):
        if key in ref and key in got:
            e = rel_err(got[key][rows], ref[key])
            rep[key] = max(rep.get(key, 0.0), e)
    r = rnd.requests[j]
    slot = r.out_slot
    H = rnd.shapes.H
    e = rel_err(got["state_pool"][slot].reshape(H, -1), np.asarray(ref["S_P"]).reshape(H, -1))
    rep["S_P"] = max(rep.get("S_P", 0.0), e)
    win_ok = np.array_equal(got["conv_pool"][slot][:rnd.shapes.conv_k - 1], ref["window_P"])
    rep["window_exact"] = rep.get("window_exact", True) and bool(win_ok)
    q_first = sum(len(rr.q_len) for rr in rnd.requests[:j])
    for i, p in enumerate(ref["probs"]):
        if p is None:
            continue
        qi = q_first + i
        a, b = opt_offsets[qi], opt_offsets[qi + 1]
        rep["tv"] = max(rep.get("tv", 0.0), tv(got["probs"][a:b], p))
    return rep


def option_offsets(rnd) -> List[int]:
    off = [0]
    for r in rnd.requests:
        for n in r.n_opt:
            off.append(off[-1] + int(n))
    return off


def check_round(rnd, got, lay, mode="memo", requests=None, questions=None, attn_rows_fn=None, tol=None):
    """Compare GPU outputs with the oracle for the given requests; returns the error report."""
    tol = TOL[rnd.dtype] if tol is None else tol
    off = option_offsets(rnd)
    conv_w = rnd.conv_w()
    rep: dict = {}
    for j in (range(len(rnd.requests)) if requests is None else requests):
        attn_rows = attn_rows_fn(j) if attn_rows_fn else None
        ref = oround.run_request(rnd, j, conv_w, mode, questions=questions, attn_rows=attn_rows,
                                 act=rnd.shapes.gdn_act)
        compare_request(rnd, lay, got, ref, j, off, rep)
    print(f"[parity] {rep} (tol {tol}, tv {TV_TOL})", flush=True)
    for key in ("attn_o", "swa_o", "gdn_o", "S_P"):
        if key in rep:
            assert rep[key] <= tol, (key, rep[key])
    assert rep["window_exact"]
    if "tv" in rep:
        assert rep["tv"] <= TV_TOL, rep["tv"]
    return rep
