"""Whole rounds through captured capacity-bucket tables, and the round-composition invariance suite (needs an
MI355X).

Flat-graph execution with capacity buckets, request-boundary splitting and deterministic bits (Korean
summary §어떻게 쓰나): a round is planned for the smallest captured bucket that holds it
(``flide_select_bucket``), a round over the largest capacity is split at request boundaries and replayed
sub-round by sub-round, and a request's output bits must not depend on the rest of the round, on the
bucket, on the split or on the order of requests and questions.
"""
import dataclasses

import numpy as np
import pytest

from tests import harness
from workloads import LayerShapes, Request, custom_round, make_round

pytestmark = pytest.mark.gpu

ROW_KEYS = ("attn_q", "attn_k", "attn_v", "swa_q", "swa_k", "swa_v", "gdn_x", "alpha", "eta", "hidden")


@pytest.fixture(scope="module")
def ctx():
    import torch
    from tree_forked_hybrid_amd import flide as F
    assert torch.cuda.is_available()
    c = F.Context(0)
    yield c
    c.close()


def _tables(rnd, n, t_max, R_cap, Q_cap, t_min=2048):
    from tree_forked_hybrid_amd.runner import BucketTable, bucket_capacities, spec_for_round
    opt = sum(sum(r.n_opt) for r in rnd.requests)
    spec = spec_for_round(rnd, T_cap=t_max, R_cap=R_cap, Q_cap=Q_cap, opt_cap=opt)
    caps = bucket_capacities(t_max, R_cap, Q_cap, t_min=min(t_min, t_max))
    return [BucketTable(spec, caps) for _ in range(n)]


def _close(tables):
    for t in tables:
        t.close()


def _request_outputs(sub, lay, got, j):
    """Outputs of request j of (sub-)round ``sub`` in request-local order."""
    rows = harness.stream_rows(sub, lay, j)
    out = {k: got[k][rows] for k in ("attn_o", "swa_o", "gdn_o") if k in got}
    r = sub.requests[j]
    out["S_P"] = got["state_pool"][r.out_slot]
    out["window"] = got["conv_pool"][r.out_slot]
    off = harness.option_offsets(sub)
    q0 = sum(len(x.q_len) for x in sub.requests[:j])
    out["probs"] = got["probs"][off[q0]:off[q0 + len(r.q_len)]]
    return out


def _assert_same(a, b, what):
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{what}: {k}")


def _split_request_outputs(res):
    """{request id: outputs} over the sub-rounds of a split run."""
    out = {}
    for sub, tab, lay in res:
        got = harness.outputs(tab.bufs)
        for j, rid in enumerate(sub.req_ids):
            out[rid] = _request_outputs(sub, lay, got, j)
    return out


def _sample_rows(rnd, j, questions, n_trunk=16, seed=0):
    r = rnd.requests[j]
    tn = r.P - r.m
    rng = np.random.default_rng(seed + j)
    rows = sorted(set(rng.choice(tn, min(n_trunk, tn), replace=False).tolist()) | {0, tn - 1}) if tn else []
    segs = rnd.segment_rows(j)
    for i in questions:
        s, L = segs[1 + i]
        rows += sorted({s, s + L // 2, s + L - 1})
    return rows


def test_fan_out_whole_round_three_replays(ctx):
    """The whole 64-question fan-out round (16 requests, 172,207 rows) as one unit: split at request
    boundaries for the 65,536-row capacity into three sub-rounds (6 + 6 + 4 requests), each planned for
    the smallest bucket of its table that holds it (flide_select_bucket), the three replays enqueued back
    to back.  Parity on one request of every replay (the last of the first, the first of the second, the
    last of the third), two questions each, sampled attention rows, every GDN row, the trunk state and
    window, and the readout."""
    full = make_round(3, 0)
    tables = _tables(full, 3, 65536, 8, 384, t_min=16384)
    try:
        res = harness.run_split(full, tables)
        assert [len(s.requests) for s, _, _ in res] == [6, 6, 4]
        assert [t.caps_of(t.last[0]).T_cap for _, t, _ in res] == [65536, 65536, 49152]
        qs = [0, 63]
        for k, (sub, tab, lay) in enumerate(res):
            j = {0: len(sub.requests) - 1, 1: 0, 2: len(sub.requests) - 1}[k]
            print(f"[parity] replay {k}: request {sub.req_ids[j]}", flush=True)
            harness.check_round(sub, harness.outputs(tab.bufs), lay, mode="memo", requests=[j], questions=qs,
                                attn_rows_fn=lambda jj, sub=sub: _sample_rows(sub, jj, qs))
    finally:
        _close(tables)


@pytest.mark.parametrize("config,requests", [(1, range(5)), (2, range(2))])
def test_repeated_runs_are_bitwise_identical(ctx, config, requests):
    """The same round run five times (eager, direct and graph replays interleaved) gives the same bits
    every time: no kernel of the path depends on timing."""
    rnd = make_round(config, 0, requests=requests)
    runs = []
    for mode in ("eager", "direct", "graph", "eager", "direct"):
        bufs, _ = harness.run_gpu(rnd, ctx, mode)
        runs.append(harness.outputs(bufs))
    for i, got in enumerate(runs[1:], 1):
        for k in runs[0]:
            np.testing.assert_array_equal(got[k], runs[0][k], err_msg=f"run {i}: {k}")


def test_chunk_grid_mode_depends_on_stream_position(ctx):
    """GDN with deterministic = 0 cuts chunks on the stream's 64-row grid: outputs still match the oracle,
    but a request's bits change when other requests move it along the stream; with deterministic = 1
    (chunks from each segment's first row) they do not."""
    from tree_forked_hybrid_amd.runner import spec_for_round
    full = make_round(1, 0, requests=range(4))
    one = full.subset([3])
    got = {}
    for det in (False, True):
        b1, l1 = harness.run_gpu(one, ctx, "direct", spec=dataclasses.replace(spec_for_round(one), deterministic=det))
        g1 = harness.outputs(b1)
        b4, l4 = harness.run_gpu(full, ctx, "direct", spec=dataclasses.replace(spec_for_round(full),
                                                                              deterministic=det))
        g4 = harness.outputs(b4)
        if not det:
            harness.check_round(full, g4, l4, mode="memo")
            assert int(l4["req_trunk_row0"][3]) % 64 != 0  # the request lands off the grid in the round
        rows1, rows4 = harness.stream_rows(one, l1, 0), harness.stream_rows(full, l4, 3)
        got[det] = np.array_equal(g1["gdn_o"][rows1], g4["gdn_o"][rows4])
    assert got[True] and not got[False], got


def test_split_equals_unsplit_bitwise(ctx):
    """Twelve short-round requests run once in one 8,192-row bucket and once split at request boundaries
    for a 2,048-row capacity (four or more replays in smaller buckets): every request's attention and GDN
    rows, trunk state, conv window and probabilities are bit-identical."""
    from tree_forked_hybrid_amd import flide as F
    rnd = make_round(1, 0, requests=range(12))
    one = _tables(rnd, 1, 8192, 16, 16)
    try:
        a = _split_request_outputs(harness.run_split(rnd, one))
    finally:
        _close(one)
    n_sub = len(F.flide_split_round(rnd.requests, 2048)[1])
    assert n_sub >= 4
    many = _tables(rnd, n_sub, 2048, 16, 16, t_min=512)
    try:
        res = harness.run_split(rnd, many)
        assert len(res) == n_sub
        b = _split_request_outputs(res)
    finally:
        _close(many)
    for rid in a:
        _assert_same(a[rid], b[rid], f"request {rid}")


def test_coscheduled_fronts_equal_serial_bitwise(ctx):
    """Twelve short-round requests split for a 2,048-row capacity (four or more sub-rounds), replayed once
    one sub-round after another, once with every sub-round's front (metadata expansion, trunk GDN call)
    on a stream of its own and the backs in order (flide_graph_replay_front / _back), and once with the
    trunk calls on side streams beside the attention (flide_graph_replay_parts): every request's outputs
    are bit-identical."""
    from tree_forked_hybrid_amd import flide as F
    rnd = make_round(1, 0, requests=range(12))
    n_sub = len(F.flide_split_round(rnd.requests, 2048)[1])
    assert n_sub >= 4
    outs = []
    for co in (False, True, "overlap"):
        tabs = _tables(rnd, n_sub, 2048, 16, 16, t_min=512)
        try:
            outs.append(_split_request_outputs(harness.run_split(rnd, tabs, co_schedule=co)))
        finally:
            _close(tabs)
    for rid in outs[0]:
        _assert_same(outs[0][rid], outs[1][rid], f"request {rid}")
        _assert_same(outs[0][rid], outs[2][rid], f"request {rid} (trunk calls beside attention)")


def test_graph_replay_parts_rejects_bad_masks(ctx):
    """flide_graph_replay_parts takes masks 1 .. 15, and part 0 (the upload) needs an image: the host checks
    reject the rest before anything is launched."""
    from tree_forked_hybrid_amd import flide as F
    rnd = make_round(1, 0, requests=range(2))
    (tab,) = _tables(rnd, 1, 2048, 8, 8, t_min=2048)
    try:
        bid = next(iter(tab.buckets))
        for parts, image in ((0, None), (16, None), (-1, None), (1, None)):
            with pytest.raises(F.FlideError) as e:
                F.flide_graph_replay_parts(tab.ctx, bid, image, parts)
            assert e.value.status == F.FLIDE_E_INVALID_ARG
    finally:
        _close([tab])


def test_same_round_in_two_buckets_bitwise(ctx):
    """One round replayed in the smallest bucket that holds it and in a bucket twice as large: same bits."""
    rnd = make_round(1, 0, requests=range(12))
    (tab,) = _tables(rnd, 1, 16384, 16, 16, t_min=4096)
    try:
        res = harness.run_split(rnd, [tab])
        sub, _, lay = res[0]
        small = tab.last[0]
        ref = harness.outputs(tab.bufs)
        big = next(b for b, (c, _, _) in tab.buckets.items() if c.T_cap == 2 * tab.caps_of(small).T_cap)
        for t in [tab.bufs.o_gdn, tab.bufs.probs, tab.bufs.state_pool] + list(tab.bufs.o_attn):
            t.zero_()
        tab.run(sub.requests, bid=big)
        import torch
        torch.cuda.synchronize()
        tab.check(big)
        got = harness.outputs(tab.bufs)
        for k in ref:
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    finally:
        tab.close()


def _permute_questions(rnd, j, perm):
    """Round equal to ``rnd`` but with request j's questions in the order ``perm`` (payload rows and option
    rows moved with them)."""
    r = rnd.requests[j]
    pl = rnd.payload(j)
    segs = rnd.segment_rows(j)
    t0, tn = segs[0]
    order = list(range(t0, t0 + tn))
    for i in perm:
        s, L = segs[1 + i]
        order += list(range(s, s + L))
    new = {k: (np.asarray(v)[order] if k in ROW_KEYS else v) for k, v in pl.items()}
    off = np.concatenate([[0], np.cumsum(r.n_opt)])
    new["w_opt"] = np.concatenate([pl["w_opt"][off[i]:off[i + 1]] for i in perm], axis=0)
    r2 = dataclasses.replace(r, q_len=tuple(r.q_len[i] for i in perm), n_opt=tuple(r.n_opt[i] for i in perm))
    reqs = list(rnd.requests)
    reqs[j] = r2
    cache = {jj: rnd.payload(jj) for jj in range(len(reqs)) if jj != j}
    cache[j] = new
    return dataclasses.replace(rnd, requests=reqs, _cache=cache)


def test_permuted_request_and_question_order_bitwise(ctx):
    """Two long-document requests (full and sliding-window attention): reversing the request order, and
    reversing one request's question order, leave every request's (question's) output bits unchanged."""
    from tree_forked_hybrid_amd.runner import spec_for_round
    base = make_round(2, 0, requests=[0, 1])
    for j in range(2):
        base.payload(j, keep=True)
    spec = spec_for_round(base, T_cap=20480)
    b0, l0 = harness.run_gpu(base, ctx, "graph", spec=spec)
    g0 = harness.outputs(b0)
    ref = [_request_outputs(base, l0, g0, j) for j in range(2)]
    # request order reversed (payloads follow their requests)
    rev = base.subset([1, 0])
    rev._cache.update({0: base.payload(1), 1: base.payload(0)})
    b1, l1 = harness.run_gpu(rev, ctx, "graph", bufs=b0)
    g1 = harness.outputs(b1)
    for j, orig in ((0, 1), (1, 0)):
        _assert_same(_request_outputs(rev, l1, g1, j), ref[orig], f"reversed requests, request {orig}")
    # question order of request 0 reversed: each question's rows and probabilities move with it
    n = len(base.requests[0].q_len)
    perm = list(range(n))[::-1]
    pq = _permute_questions(base, 0, perm)
    b2, l2 = harness.run_gpu(pq, ctx, "graph", bufs=b0)
    g2 = harness.outputs(b2)
    got = _request_outputs(pq, l2, g2, 0)
    _assert_same({k: got[k] for k in ("S_P", "window")}, {k: ref[0][k] for k in ("S_P", "window")}, "trunk")
    segs_ref, segs_new = base.segment_rows(0), pq.segment_rows(0)
    off_ref = np.concatenate([[0], np.cumsum(base.requests[0].n_opt)])
    off_new = np.concatenate([[0], np.cumsum(pq.requests[0].n_opt)])
    t0, tn = segs_ref[0]
    for key in ("attn_o", "swa_o", "gdn_o"):
        np.testing.assert_array_equal(got[key][t0:t0 + tn], ref[0][key][t0:t0 + tn], err_msg=f"trunk {key}")
    for new_i, old_i in enumerate(perm):
        (sr, L), (sn, _) = segs_ref[1 + old_i], segs_new[1 + new_i]
        for key in ("attn_o", "swa_o", "gdn_o"):
            np.testing.assert_array_equal(got[key][sn:sn + L], ref[0][key][sr:sr + L],
                                          err_msg=f"question {old_i}: {key}")
        np.testing.assert_array_equal(got["probs"][off_new[new_i]:off_new[new_i + 1]],
                                      ref[0]["probs"][off_ref[old_i]:off_ref[old_i + 1]])
    _assert_same(_request_outputs(pq, l2, g2, 1), ref[1], "request 1 beside the permuted request")


def test_state_index_probe(ctx):
    """With eta = 0 on every question row the question outputs are (prod alpha) S_P[j] q_hat: they reveal
    which trunk state each question read.  Parity with the oracle, and the outputs are far from what the
    neighbouring request's S_P would give (the probe can tell the slots apart)."""
    from oracle import round as oround
    from oracle.gdn import gdn_prompt
    rnd = make_round(1, 0, requests=range(4))
    for j in range(4):
        pl = dict(rnd.payload(j))
        tn = rnd.requests[j].P
        eta = np.array(pl["eta"], copy=True)
        eta[tn:] = 0.0
        pl["eta"] = eta
        rnd._cache[j] = pl
    bufs, lay = harness.run_gpu(rnd, ctx, "graph")
    got = harness.outputs(bufs)
    harness.check_round(rnd, got, lay, mode="memo")
    conv_w = rnd.conv_w()
    sh = rnd.shapes
    for j in range(4):
        other = (j + 1) % 4
        ref_other = oround.run_request(rnd, other, conv_w, "memo")
        pl = rnd.payload(j)
        s, L = rnd.segment_rows(j)[1]
        rows = np.arange(s, s + L)
        wrong, _, _ = gdn_prompt(pl["gdn_x"][rows], pl["alpha"][rows], pl["eta"][rows], conv_w, sh.H, sh.dk, sh.dv,
                                 ref_other["window_P"], ref_other["S_P"], sh.gdn_act)
        mine = got["gdn_o"][harness.stream_rows(rnd, lay, j)[s:s + L]]
        assert harness.rel_err(mine, wrong) > 20 * harness.TOL["bf16"], j


def test_sibling_perturbation_leaves_other_rows_bitwise(ctx):
    """Changing one question's payload (request 0 of a long-document round, question 2 negated) changes
    only that question's rows and probabilities: the trunk, every sibling question and the other request
    keep their bits."""
    base = make_round(2, 0, requests=[0, 1])
    for j in range(2):
        base.payload(j, keep=True)
    from tree_forked_hybrid_amd.runner import spec_for_round
    spec = spec_for_round(base, T_cap=20480)
    b0, l0 = harness.run_gpu(base, ctx, "direct", spec=spec)
    g0 = harness.outputs(b0)
    ref = [_request_outputs(base, l0, g0, j) for j in range(2)]
    s2, L2 = base.segment_rows(0)[3]
    pl = {k: np.array(v, copy=True) for k, v in base.payload(0).items()}
    for k in ROW_KEYS:
        if k in pl and k not in ("alpha", "eta"):
            pl[k][s2:s2 + L2] *= -1.0
    pert = dataclasses.replace(base, _cache={0: pl, 1: base.payload(1)})
    b1, l1 = harness.run_gpu(pert, ctx, "direct", bufs=b0)
    g1 = harness.outputs(b1)
    got = _request_outputs(pert, l1, g1, 0)
    keep = np.ones(len(got["gdn_o"]), bool)
    keep[s2:s2 + L2] = False
    for key in ("attn_o", "swa_o", "gdn_o"):
        np.testing.assert_array_equal(got[key][keep], ref[0][key][keep], err_msg=key)
        assert not np.array_equal(got[key][~keep], ref[0][key][~keep]), key
    np.testing.assert_array_equal(got["S_P"], ref[0]["S_P"])
    off = np.concatenate([[0], np.cumsum(base.requests[0].n_opt)])
    pmask = np.ones(len(got["probs"]), bool)
    pmask[off[2]:off[3]] = False
    np.testing.assert_array_equal(got["probs"][pmask], ref[0]["probs"][pmask])
    _assert_same(_request_outputs(pert, l1, g1, 1), ref[1], "other request")


def test_capacity_above_chunk_offset_range_bitwise(ctx):
    """A short-round request in buffers of 180,224 rows (beyond the ~174.7k rows at which a segment-based
    32-bit buffer offset would overflow) gives the same bits as in buffers of its own size: the GDN layer
    keeps the chunked kernel, whose buffer offsets are relative to each chunk."""
    from tree_forked_hybrid_amd.runner import spec_for_round
    rnd = make_round(1, 0, requests=[0, 1])
    b0, l0 = harness.run_gpu(rnd, ctx, "graph")
    ref = harness.outputs(b0)
    ref_req = [_request_outputs(rnd, l0, ref, j) for j in range(2)]
    del b0, ref
    big, lb = harness.run_gpu(rnd, ctx, "graph", spec=spec_for_round(rnd, T_cap=180224))
    got = harness.outputs(big)
    for j in range(2):
        _assert_same(_request_outputs(rnd, lb, got, j), ref_req[j], f"request {j}")


def test_readout_many_options_and_bad_option_row(ctx):
    """Questions with 9 and 17 options (the readout's multi-batch path) against the oracle; then an option
    row outside w_opt: the device error word reports it and the question's other options stay normalised."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    sh = LayerShapes(H=2, dk=32, dv=32, conv_k=4, Hq=2, Hkv=1, d=32, theta=1e4, hidden=64)
    reqs = [Request(P=20, m=0, q_len=(3, 2, 4), n_opt=(9, 17, 2), out_slot=0),
            Request(P=5, m=0, q_len=(1,), n_opt=(8,), out_slot=1)]
    for dtype in ("f32", "bf16"):
        rnd = custom_round(sh, dtype, reqs, base=53)
        bufs, lay = harness.run_gpu(rnd, ctx, "direct")
        harness.check_round(rnd, harness.outputs(bufs), lay, mode="isolated")
    off = harness.option_offsets(rnd)
    bad = off[1] + 4  # option 4 of the 17-option question
    bufs.opt_id[bad] = bufs.spec.opt_cap  # one past the last row of w_opt
    F.flide_readout(ctx, bufs.caps, bufs.dev_meta, bufs.ro_params, bufs.h, bufs.w_opt, bufs.opt_off, bufs.opt_id,
                    bufs.spec.opt_cap, bufs.probs)
    torch.cuda.synchronize()
    with pytest.raises(F.FlideError) as e:
        F.flide_check_device(ctx, bufs.caps, bufs.dev_meta)
    assert e.value.status == F.FLIDE_E_DEVICE
    p = bufs.probs.cpu().numpy().astype(np.float64)
    assert p[bad] == 0.0
    assert abs(p[off[1]:off[2]].sum() - 1.0) < 1e-5
    F.flide_check_device(ctx, bufs.caps, bufs.dev_meta)  # the word was cleared by the read


def test_graph_round_writes_checkpoint_kv(ctx):
    """A captured round with an interior checkpoint writes the checkpoint's K/V itself (no separate save
    call): the cache slot equals the one the direct path's explicit save writes, bit for bit, and a round
    resumed from it reproduces the uncut round's later rows."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    base = make_round(1, 0, requests=[0])
    r0 = base.requests[0]
    sm, ss = 256, r0.out_slot + 1
    ra = dataclasses.replace(base, requests=[dataclasses.replace(r0, save_m=sm, save_slot=ss)])
    bd, ld = harness.run_gpu(ra, ctx, "direct")
    bd.save_checkpoint_kv(ctx)
    torch.cuda.synchronize()
    F.flide_check_device(ctx, bd.caps, bd.dev_meta)
    kd, vd = bd.k_cache[0][ss].clone(), bd.v_cache[0][ss].clone()
    sd = bd.state_pool[ss].clone()
    bg, lg = harness.run_gpu(ra, ctx, "graph")
    assert torch.equal(bg.k_cache[0][ss], kd) and torch.equal(bg.v_cache[0][ss], vd)
    assert torch.equal(bg.state_pool[ss], sd)
    # resume from the graph-made checkpoint
    ga = harness.outputs(bg)
    row_keys = ("attn_q", "attn_k", "attn_v", "gdn_x", "alpha", "eta", "hidden")
    pb = {k: (np.asarray(v)[sm:] if k in row_keys else v) for k, v in ra.payload(0).items()}
    pb["ckpt_state"] = bg.state_pool[ss].cpu().numpy()
    pb["ckpt_window"] = bg.conv_pool[ss].float().cpu().numpy()
    pb["kv_k"] = bg.k_cache[0][ss, :sm].float().cpu().numpy()
    pb["kv_v"] = np.transpose(bg.v_cache[0][ss, :, :, :sm].float().cpu().numpy(), (2, 0, 1))
    rb = dataclasses.replace(base, requests=[dataclasses.replace(r0, m=sm, ckpt_slot=ss)], _cache={0: pb})
    bb, lb = harness.run_gpu(rb, ctx, "graph")
    gb = harness.outputs(bb)
    rows_a = harness.stream_rows(ra, lg, 0)[sm:]
    rows_b = harness.stream_rows(rb, lb, 0)
    for key in ("gdn_o", "attn_o"):
        np.testing.assert_array_equal(gb[key][rows_b], ga[key][rows_a], err_msg=key)


def test_checkpoint_store_round_trip(ctx):
    """Prefix-match checkpoint store with real rounds: a round writes a checkpoint at position 256 into the
    slot the store reserves (graph mode, which writes the K/V itself) and commits it after the round has
    completed; a later round whose first 256 tokens match (same digests) looks it up among candidates every
    64 positions, resumes there and reproduces the uncut round's later rows bit for bit; a request with a
    different prefix gets no checkpoint."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    store = F.CheckpointStore(8, 2)
    digest = lambda rid, m: (rid * 1000003 + m * 7919) & ((1 << 63) - 1)  # the caller's prefix digest
    base = make_round(1, 0, requests=[0])
    r0 = base.requests[0]
    sm = 256
    slot = store.reserve(sm, digest(0, sm))
    ra = dataclasses.replace(base, requests=[dataclasses.replace(r0, save_m=sm, save_slot=slot)])
    ba, la = harness.run_gpu(ra, ctx, "graph")
    store.commit(slot)
    store.release(slot)
    cands = list(range(64, r0.P, 64))
    m, s = store.lookup(cands, [digest(0, p) for p in cands])
    assert (m, s) == (sm, slot)
    assert store.lookup(cands, [digest(1, p) for p in cands]) == (0, -1)
    ga = harness.outputs(ba)
    row_keys = ("attn_q", "attn_k", "attn_v", "gdn_x", "alpha", "eta", "hidden")
    pb = {k: (np.asarray(v)[m:] if k in row_keys else v) for k, v in ra.payload(0).items()}
    torch.cuda.synchronize()
    pb["ckpt_state"] = ba.state_pool[s].cpu().numpy()
    pb["ckpt_window"] = ba.conv_pool[s].float().cpu().numpy()
    pb["kv_k"] = ba.k_cache[0][s, :m].float().cpu().numpy()
    pb["kv_v"] = np.transpose(ba.v_cache[0][s, :, :, :m].float().cpu().numpy(), (2, 0, 1))
    rb = dataclasses.replace(base, requests=[dataclasses.replace(r0, m=m, ckpt_slot=s)], _cache={0: pb})
    bb, lb = harness.run_gpu(rb, ctx, "graph")
    store.release(s)
    gb = harness.outputs(bb)
    rows_a = harness.stream_rows(ra, la, 0)[m:]
    rows_b = harness.stream_rows(rb, lb, 0)
    for key in ("gdn_o", "attn_o"):
        np.testing.assert_array_equal(gb[key][rows_b], ga[key][rows_a], err_msg=key)
    assert store.stats()["hits"] == 1 and store.stats()["held"] == 0
    store.close()


def test_parameter_checks_match_the_kernels(ctx):
    """A GDN shape the per-token kernel has no instance for is rejected before anything is launched."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    rnd = make_round(0, 0)
    bufs, _ = harness.run_gpu(rnd, ctx, "direct")
    bad = F.flide_gdn_params(2, 16, 32, 4, 0, 64, F.FLIDE_F32, 0)
    with pytest.raises(F.FlideError) as e:
        F.flide_fork_gdn(ctx, bufs.caps, bufs.dev_meta, bad, 0, bufs.x, bufs.conv_w, bufs.alpha, bufs.eta,
                         bufs.state_pool, bufs.conv_pool, bufs.spec.n_slots, bufs.o_gdn)
    assert e.value.status == F.FLIDE_E_UNSUPPORTED
    assert F.flide_last_hip_error(ctx) == 0
    torch.cuda.synchronize()
