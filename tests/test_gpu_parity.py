"""GPU parity of the HIP path against the oracle (needs an MI355X)."""
import numpy as np
import pytest

from tests import harness
from workloads import LayerShapes, Request, custom_round, make_round

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    import torch
    from tree_forked_hybrid_amd import flide as F
    assert torch.cuda.is_available()
    c = F.Context(0)
    yield c
    c.close()


def test_tiny_fork_round_fp32(ctx):
    rnd = make_round(0, 0)
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    # device-expanded (j, c, t) labels equal the oracle's, bit for bit
    from tree_forked_hybrid_amd import flide as F
    L = F.flide_meta_layout_for(bufs.caps)
    meta = bufs.dev_meta.cpu().numpy()
    T = bufs.caps.T_cap
    ref = __import__("oracle").layout.build_layout(rnd.requests, t_cap=T)
    for name in ("tok_j", "tok_c", "tok_t"):
        off = getattr(L, name)
        np.testing.assert_array_equal(meta[off:off + T], ref[name])
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="isolated")


@pytest.mark.parametrize("mode", ["graph", "eager"])
def test_graph_and_eager_equal_direct_bitwise(ctx, mode):
    rnd = make_round(0, 0)
    b0, _ = harness.run_gpu(rnd, ctx, "direct")
    ref = harness.outputs(b0)
    b1, _ = harness.run_gpu(rnd, ctx, mode, repeats=2)
    got = harness.outputs(b1)
    for k in ref:
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


def test_graph_replays_with_eager_work_between(ctx):
    """One captured graph, replayed four times with the program's own eager work (output clears, other
    torch kernels) and synchronizations in between; every replay equals the eager round bit for bit."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    rnd = make_round(1, 0, requests=range(5))
    be, _ = harness.run_gpu(rnd, ctx, "eager")
    ref = harness.outputs(be)
    bg, _ = harness.run_gpu(rnd, ctx, "direct")
    img = F.flide_plan_round(rnd.requests, bg.caps)
    bid = F.flide_graph_capture(ctx, bg.round_bufs())
    scratch = torch.randn(1024, 1024, device="cuda")
    for rep in range(4):
        for t in [bg.o_gdn, bg.probs, bg.state_pool] + list(bg.o_attn):
            t.zero_()
        scratch = torch.tanh(scratch @ scratch.T * 1e-3)  # unrelated eager work on the device
        torch.cuda.synchronize()
        F.flide_graph_replay(ctx, bid, img)
        torch.cuda.synchronize()
        got = harness.outputs(bg)
        for k in ref:
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"replay {rep}: {k}")
    F.flide_check_device(ctx, bg.caps, bg.dev_meta)
    F.flide_graph_release(ctx, bid)
    with pytest.raises(F.FlideError):  # a released bucket is never replayed again
        F.flide_graph_replay(ctx, bid, img)


def test_short_rounds_bf16_subset(ctx):
    rnd = make_round(1, 0, requests=range(6))
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="memo")


@pytest.mark.parametrize("config", [1, 0])
def test_attention_prepare_then_core_equals_fork_attn(ctx, config):
    """flide_attn_prepare + flide_attn_core reproduce flide_fork_attn bit for bit (bf16 MFMA and f32 paths)."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    rnd = make_round(config, 0, requests=range(min(6, len(make_round(config, 0).requests))))
    bufs, _ = harness.run_gpu(rnd, ctx, "direct")
    for l in range(bufs.n_attn):
        ref = bufs.o_attn[l].clone()
        out = torch.zeros_like(ref)
        ws = torch.zeros_like(bufs.ws[l])
        p = bufs.attn_params[l]
        F.flide_attn_prepare(ctx, bufs.caps, bufs.dev_meta, p, bufs.k[l], bufs.v[l], ws)
        F.flide_attn_core(ctx, bufs.caps, bufs.dev_meta, p, bufs.q[l], bufs.v[l], bufs.k_cache[l], bufs.v_cache[l],
                          out, ws)
        torch.cuda.synchronize()
        T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
        assert torch.equal(out[:T], ref[:T])


def test_attention_work_order_does_not_change_bits(ctx):
    """The attention launch gives the same bits in every work order the header can select (tile groups
    of 0 = every head group of a position in turn, 16 and 64 positions per head group): tiles are
    independent.  Agent-resume requests, whose tiles see > 30k keys, so the planner itself picks 64."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    rnd = make_round(4, 0, requests=range(2))
    bufs, _ = harness.run_gpu(rnd, ctx, "direct")
    img = F.flide_plan_round(rnd.requests, bufs.caps)
    L = F.flide_meta_layout_for(bufs.caps)
    assert img[L.hdr + 6] == 64
    T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
    outs = []
    for group in (0, 16, 64):
        img[L.hdr + 6] = group
        bufs.upload(ctx, img)
        p = bufs.attn_params[0]
        out = torch.zeros_like(bufs.o_attn[0])
        F.flide_attn_prepare(ctx, bufs.caps, bufs.dev_meta, p, bufs.k[0], bufs.v[0], bufs.ws[0])
        F.flide_attn_core(ctx, bufs.caps, bufs.dev_meta, p, bufs.q[0], bufs.v[0], bufs.k_cache[0], bufs.v_cache[0],
                          out, bufs.ws[0])
        torch.cuda.synchronize()
        F.flide_check_device(ctx, bufs.caps, bufs.dev_meta)
        outs.append(out[:T].clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert torch.equal(outs[2], bufs.o_attn[0][:T])


EDGE = LayerShapes(H=2, dk=32, dv=32, conv_k=4, Hq=4, Hkv=2, d=64, theta=1e4, hidden=64, swa_window=5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases(ctx, dtype):
    reqs = [Request(P=70, m=0, q_len=(1, 33, 2), n_opt=(1, 3, 2), out_slot=0),   # ragged tiles, |q| = 1
            Request(P=0, m=0, q_len=(3,), n_opt=(2,), out_slot=1),              # empty trunk, P = 0
            Request(P=2, m=0, q_len=(4, 1), n_opt=(2, 5), out_slot=2),          # trunk shorter than the conv
            Request(P=9, m=0, q_len=(), n_opt=(), out_slot=3),                  # no questions
            Request(P=40, m=38, q_len=(5,), n_opt=(3,), ckpt_slot=6, out_slot=4),  # resumed, P - m < K - 1
            Request(P=20, m=20, q_len=(2,), n_opt=(2,), ckpt_slot=7, out_slot=5)]  # resumed, no new trunk rows
    rnd = custom_round(EDGE, dtype, reqs, base=21)
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="isolated")


def _edge_reqs():
    return [Request(P=150, m=0, q_len=(1, 33, 70), n_opt=(1, 3, 2), out_slot=0),  # several key and query tiles
            Request(P=0, m=0, q_len=(3,), n_opt=(2,), out_slot=1),
            Request(P=2, m=0, q_len=(4, 1), n_opt=(2, 5), out_slot=2),
            Request(P=9, m=0, q_len=(), n_opt=(), out_slot=3),
            Request(P=104, m=102, q_len=(5, 17), n_opt=(3, 2), ckpt_slot=6, out_slot=4),
            Request(P=64, m=64, q_len=(2,), n_opt=(2,), ckpt_slot=7, out_slot=5),
            # many short siblings: query tiles that hold units of up to four questions
            Request(P=90, m=0, q_len=(1, 2, 7, 8, 9, 3, 16, 1, 5), n_opt=(2,) * 9, out_slot=9)]


@pytest.mark.parametrize("d,Hq", [(256, 8), (128, 8), (256, 12), (128, 4)])
def test_edge_cases_mfma_path(ctx, d, Hq):
    """Ragged, empty and resumed requests on the matrix-core attention path.  Four q heads per kv head
    (G = 4: each wave holds one 8-row unit of a packed tile), six (head groups of four and two) and two
    (one group of two): the two kernel forms that map query columns to waves."""
    sh = LayerShapes(H=2, dk=32, dv=32, conv_k=4, Hq=Hq, Hkv=2, d=d, theta=1e4, hidden=64, swa_window=40)
    rnd = custom_round(sh, "bf16", _edge_reqs(), base=23)
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="isolated")


def test_long_document_round_with_sliding_window(ctx):
    full = make_round(2, 0)
    j = min(range(len(full.requests)), key=lambda i: full.requests[i].P)
    rnd = full.subset([j])
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    r = rnd.requests[0]
    tn = r.P - r.m
    rng = np.random.default_rng(0)
    rows = sorted(set(rng.choice(tn, 96, replace=False).tolist()) | {0, 1, 63, 64, tn - 1})
    segs = rnd.segment_rows(0)
    for i in range(4):
        s, L = segs[1 + i]
        rows += list(range(s, s + L))
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="memo", questions=[0, 1, 2, 3],
                        attn_rows_fn=lambda _j: rows)


def test_agent_resume_round(ctx):
    rnd = make_round(4, 0, requests=[0])
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    r = rnd.requests[0]
    tn = r.P - r.m
    segs = rnd.segment_rows(0)
    rows = [0, 1, 2, 500, 1023, tn - 1]
    for i in range(2):
        s, L = segs[1 + i]
        rows += [s, s + L // 2, s + L - 1]
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="memo", questions=[0, 1],
                        attn_rows_fn=lambda _j: rows)


def test_deterministic_round_composition_invariance(ctx):
    """Outputs of a request are bit-identical alone and inside a round of eight (agent resume workload)."""
    full = make_round(4, 0)
    one = full.subset([3])
    b1, l1 = harness.run_gpu(one, ctx, "graph")
    g1 = harness.outputs(b1)
    b8, l8 = harness.run_gpu(full, ctx, "graph")
    g8 = harness.outputs(b8)
    rows1 = harness.stream_rows(one, l1, 0)
    rows8 = harness.stream_rows(full, l8, 3)
    for key in ("attn_o", "gdn_o"):
        np.testing.assert_array_equal(g1[key][rows1], g8[key][rows8], err_msg=key)
    slot = full.requests[3].out_slot
    np.testing.assert_array_equal(g1["state_pool"][slot], g8["state_pool"][slot])
    off1, off8 = harness.option_offsets(one), harness.option_offsets(full)
    q0 = sum(len(r.q_len) for r in full.requests[:3])
    n = off1[-1]
    np.testing.assert_array_equal(g1["probs"][:n], g8["probs"][off8[q0]:off8[q0] + n])


def test_short_rounds_full_size_graph_bucket(ctx):
    """The benchmark's launch configuration (whole round, 36864-row bucket, graph replay), sampled parity."""
    from tree_forked_hybrid_amd.runner import spec_for_round
    rnd = make_round(1, 0)
    spec = spec_for_round(rnd, T_cap=36864, R_cap=64, Q_cap=64)
    bufs, lay = harness.run_gpu(rnd, ctx, "graph", spec=spec)
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="memo", requests=[0, 31, 63])


@pytest.mark.parametrize("dtype,act", [("bf16", "none"), ("bf16", "silu")])
def test_edge_cases_chunked_gdn(ctx, dtype, act):
    """dk = dv = 128 routes the GDN layer to the chunked MFMA kernel: partial chunks, a question longer
    than one chunk, empty and short trunks, resumes with fewer new rows than the conv width; with and
    without the SiLU after the conv."""
    sh = LayerShapes(H=2, dk=128, dv=128, conv_k=4, Hq=4, Hkv=1, d=128, theta=1e4, hidden=64, swa_window=40,
                     gdn_act=act)
    reqs = _edge_reqs() + [Request(P=300, m=0, q_len=(64, 65), n_opt=(2, 2), out_slot=8)]
    rnd = custom_round(sh, dtype, reqs, base=29)
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="isolated")


def test_split_round_graph_buckets_and_eager(ctx):
    """A round larger than one capacity: split at request boundaries, sub-rounds replayed in one
    captured bucket of T_max rows, and a request longer than T_max run eagerly in its own buffers."""
    from tree_forked_hybrid_amd import flide as F
    from tree_forked_hybrid_amd.runner import RoundBuffers, spec_for_round
    sh = LayerShapes(H=2, dk=128, dv=128, conv_k=4, Hq=4, Hkv=1, d=128, theta=1e4, hidden=64, swa_window=40)
    reqs = [Request(P=100, m=0, q_len=(20, 9), n_opt=(2, 3), out_slot=0),
            Request(P=260, m=0, q_len=(40,), n_opt=(4,), out_slot=1),
            Request(P=700, m=0, q_len=(30, 12), n_opt=(2, 2), out_slot=2),
            Request(P=150, m=0, q_len=(16,), n_opt=(3,), out_slot=3),
            Request(P=200, m=0, q_len=(8, 8, 8), n_opt=(2, 2, 2), out_slot=4)]
    t_max = 512
    rnd = custom_round(sh, "bf16", reqs, base=41, t_max=t_max)
    first, eager = F.flide_split_round(rnd.requests, t_max)
    assert eager.count(True) == 1 and len(eager) >= 3
    bucket = RoundBuffers(spec_for_round(rnd, T_cap=t_max, R_cap=len(reqs), Q_cap=8))
    for i, is_eager in enumerate(eager):
        sub = rnd.subset(list(range(first[i], first[i + 1])))
        if is_eager:
            bufs, lay = harness.run_gpu(sub, ctx, "eager")
        else:
            bufs, lay = harness.run_gpu(sub, ctx, "graph", bufs=bucket)
        harness.check_round(sub, harness.outputs(bufs), lay, mode="memo")


def _sample_rows(rnd, j, questions, n_trunk=48, seed=0):
    """Request-local rows whose attention the oracle computes: random trunk rows, both trunk ends, and
    the first, middle and last row of each checked question."""
    r = rnd.requests[j]
    tn = r.P - r.m
    rows = []
    if tn > 0:
        rng = np.random.default_rng(seed + j)
        rows = sorted(set(rng.choice(tn, min(n_trunk, tn), replace=False).tolist()) | {0, tn - 1})
    segs = rnd.segment_rows(j)
    for i in questions:
        s, L = segs[1 + i]
        rows += sorted({s, s + L // 2, s + L - 1})
    return rows


def test_long_document_rounds_full_size(ctx):
    """Whole long-document round (4 requests, 48 questions each, full and sliding-window attention) in a
    32768-row bucket graph; requests 0 and 3 checked on sampled attention rows, every GDN row of the
    checked segments, the trunk states and the readout."""
    from tree_forked_hybrid_amd.runner import spec_for_round
    rnd = make_round(2, 0)
    spec = spec_for_round(rnd, T_cap=32768, R_cap=4, Q_cap=192)
    bufs, lay = harness.run_gpu(rnd, ctx, "graph", spec=spec)
    qs = [0, 23, 47]
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="memo", requests=[0, 3], questions=qs,
                        attn_rows_fn=lambda j: _sample_rows(rnd, j, qs, n_trunk=24))


def test_agent_resume_rounds_full_size(ctx):
    """Whole agent-resume round (8 trajectories resumed at m = 30720 from checkpoint slots, 2048 new rows
    and 8 questions each) in deterministic mode; the last trajectory checked on sampled rows (the first is
    checked alone at full size elsewhere, and bitwise composition invariance ties the two together)."""
    from tree_forked_hybrid_amd.runner import spec_for_round
    rnd = make_round(4, 0)
    spec = spec_for_round(rnd, T_cap=20480)
    bufs, lay = harness.run_gpu(rnd, ctx, "graph", spec=spec)
    qs = [0, 7]
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="memo", requests=[7], questions=qs,
                        attn_rows_fn=lambda j: _sample_rows(rnd, j, qs, n_trunk=12))


def _check_created_checkpoint(rnd, bufs, j: int, tol: float):
    """The save slot of request j against the oracle's checkpoint at save_m: GDN state (relative error
    per state row), conv window (exact: raw inputs), and per attention layer the rotated keys (relative
    error per position) and the values (exact: copies)."""
    import torch
    from oracle import round as oround
    r = rnd.requests[j]
    ck = oround.make_checkpoint(rnd, j, r.save_m, act=rnd.shapes.gdn_act)
    torch.cuda.synchronize()
    s = r.save_slot
    st = bufs.state_pool[s].cpu().numpy().astype(np.float64)
    e_state = harness.rel_err(st.reshape(rnd.shapes.H, -1), ck["ckpt_state"].reshape(rnd.shapes.H, -1))
    win = bufs.conv_pool[s].float().cpu().numpy().astype(np.float64)[:rnd.shapes.conv_k - 1]
    print(f"[checkpoint] request {j} save_m={r.save_m} slot={s} state err {e_state:.3e}", flush=True)
    assert e_state <= tol
    np.testing.assert_array_equal(win, ck["ckpt_window"])
    for l, cpre in enumerate(["kv", "swa_kv"][:bufs.n_attn]):
        kc = bufs.k_cache[l][s, :r.save_m].float().cpu().numpy().astype(np.float64)
        vc = bufs.v_cache[l][s, :, :, :r.save_m].float().cpu().numpy().astype(np.float64)
        e_k = harness.rel_err(kc, ck[cpre + "_k"])
        print(f"[checkpoint] layer {l} key err {e_k:.3e}", flush=True)
        assert e_k <= tol
        np.testing.assert_array_equal(vc, np.transpose(ck[cpre + "_v"], (1, 2, 0)))


def test_interior_checkpoint_creation_f32(ctx):
    """Checkpoints made in the same pass (GDN state and window by the trunk call, K/V by the save call):
    a fresh trunk at a chunk boundary, a resumed trunk at its end (the per-token GDN kernel and the fp32
    attention path), against the oracle's cut prompt."""
    shapes = LayerShapes(H=2, dk=32, dv=32, conv_k=4, Hq=2, Hkv=1, d=32, theta=1e4, hidden=32)
    reqs = [Request(P=150, m=0, q_len=(5,), n_opt=(3,), out_slot=0, save_m=128, save_slot=3),
            Request(P=150, m=64, q_len=(4, 6), n_opt=(2, 2), ckpt_slot=1, out_slot=2, save_m=150, save_slot=4)]
    rnd = custom_round(shapes, "f32", reqs, base=21)
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    bufs.save_checkpoint_kv(ctx)
    from tree_forked_hybrid_amd import flide as F
    F.flide_check_device(ctx, bufs.caps, bufs.dev_meta)
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="memo")
    for j in range(len(reqs)):
        _check_created_checkpoint(rnd, bufs, j, harness.TOL["f32"])


def test_interior_checkpoint_creation_bf16(ctx):
    """The same on the chunked GDN kernel and the MFMA attention path: an agent-resume request (resumed
    at 30720) makes a checkpoint 1024 rows further; a short-round request makes one at row 256."""
    import dataclasses
    rnd4 = make_round(4, 0, requests=[0])
    r = rnd4.requests[0]
    rnd4 = dataclasses.replace(rnd4, requests=[dataclasses.replace(r, save_m=r.m + 1024, save_slot=r.out_slot + 8)])
    bufs, lay = harness.run_gpu(rnd4, ctx, "direct")
    bufs.save_checkpoint_kv(ctx)
    from tree_forked_hybrid_amd import flide as F
    F.flide_check_device(ctx, bufs.caps, bufs.dev_meta)
    _check_created_checkpoint(rnd4, bufs, 0, harness.TOL["bf16"])
    rnd1 = make_round(1, 0, requests=[0, 1])
    r0 = rnd1.requests[0]
    new0 = dataclasses.replace(r0, save_m=256, save_slot=max(q.out_slot for q in rnd1.requests) + 1)
    rnd1 = dataclasses.replace(rnd1, requests=[new0, rnd1.requests[1]])
    bufs, lay = harness.run_gpu(rnd1, ctx, "direct")
    bufs.save_checkpoint_kv(ctx)
    F.flide_check_device(ctx, bufs.caps, bufs.dev_meta)
    _check_created_checkpoint(rnd1, bufs, 0, harness.TOL["bf16"])


def test_resume_from_created_checkpoint_matches_uncut_round(ctx):
    """A round resumed from a checkpoint the library made (GDN state and window from the trunk call, K/V
    from the save call) reproduces the uncut round's rows past the checkpoint: the resumed chunks start
    on the same chunk boundary and the key tiles fall on the same 32-key grid, so the arithmetic is the
    same and the outputs must be bit-identical (short-round request, bf16)."""
    import dataclasses
    import torch
    from tree_forked_hybrid_amd import flide as F
    base = make_round(1, 0, requests=[0])
    r0 = base.requests[0]
    sm, ss = 256, r0.out_slot + 1
    ra = dataclasses.replace(base, requests=[dataclasses.replace(r0, save_m=sm, save_slot=ss)])
    ba, la = harness.run_gpu(ra, ctx, "direct")
    ba.save_checkpoint_kv(ctx)
    F.flide_check_device(ctx, ba.caps, ba.dev_meta)
    ga = harness.outputs(ba)
    row_keys = ("attn_q", "attn_k", "attn_v", "gdn_x", "alpha", "eta", "hidden")
    pb = {k: (np.asarray(v)[sm:] if k in row_keys else v) for k, v in ra.payload(0).items()}
    torch.cuda.synchronize()
    pb["ckpt_state"] = ba.state_pool[ss].cpu().numpy()
    pb["ckpt_window"] = ba.conv_pool[ss].float().cpu().numpy()
    pb["kv_k"] = ba.k_cache[0][ss, :sm].float().cpu().numpy()
    pb["kv_v"] = np.transpose(ba.v_cache[0][ss, :, :, :sm].float().cpu().numpy(), (2, 0, 1))
    rb = dataclasses.replace(base, requests=[dataclasses.replace(r0, m=sm, ckpt_slot=ss)], _cache={0: pb})
    bb, lb = harness.run_gpu(rb, ctx, "direct")
    gb = harness.outputs(bb)
    rows_a = harness.stream_rows(ra, la, 0)[sm:]
    rows_b = harness.stream_rows(rb, lb, 0)
    for key in ("gdn_o", "attn_o"):
        np.testing.assert_array_equal(gb[key][rows_b], ga[key][rows_a], err_msg=key)
    np.testing.assert_array_equal(gb["state_pool"][r0.out_slot], ga["state_pool"][r0.out_slot])
    n = harness.option_offsets(ra)[-1]
    np.testing.assert_array_equal(gb["probs"][:n], ga["probs"][:n])
