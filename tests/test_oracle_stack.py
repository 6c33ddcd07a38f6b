"""Pins of the multi-layer stack oracle (oracle/stack.py), CPU only."""
import dataclasses

import numpy as np
import pytest

from oracle import stack as ostack
from oracle.readout import option_probs
from tests.brute_stack import flat_stack
from workloads import Request, StackShapes, make_stack

SHAPES = StackShapes(Dm=32, F=48, layers=("gdn", "attn", "gdn", "swa"), H=2, dk=8, dv=8, conv_k=4, Hq=4, Hkv=2,
                     d=8, theta=1e4, window=6)
REQS = [Request(P=11, m=0, q_len=(3, 5, 1), n_opt=(2, 3, 4), out_slot=0),
        Request(P=0, m=0, q_len=(4,), n_opt=(3,), out_slot=1),
        Request(P=2, m=0, q_len=(2, 6), n_opt=(2, 2), out_slot=2),
        Request(P=7, m=0, q_len=(), n_opt=(), out_slot=3)]


def test_rms_norm_closed_forms():
    # [3, 4]: mean square 12.5
    y = ostack.rms_norm(np.array([3.0, 4.0]), np.ones(2), eps=0.0)
    np.testing.assert_allclose(y, [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], rtol=1e-15)
    # a constant row c: c / sqrt(c^2 + eps) times the gain, element by element
    c, eps = -0.25, 1e-6
    y = ostack.rms_norm(np.full(5, c), np.arange(1.0, 6.0), eps=eps)
    np.testing.assert_allclose(y, np.arange(1.0, 6.0) * c / np.sqrt(c * c + eps), rtol=1e-15)
    # the zero row stays zero; the norm acts on the last axis only
    assert not ostack.rms_norm(np.zeros(4), np.ones(4)).any()
    m = ostack.rms_norm(np.array([[3.0, 4.0], [6.0, 8.0]]), np.ones(2), eps=0.0)
    np.testing.assert_allclose(m[0], m[1], rtol=1e-15)


def test_silu_and_sigmoid_closed_forms():
    assert ostack.silu(np.array(0.0)) == 0.0
    assert ostack.sigmoid(np.array(0.0)) == 0.5
    x = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(ostack.silu(x) - ostack.silu(-x), x, atol=1e-14)   # silu(x) - silu(-x) = x
    np.testing.assert_allclose(ostack.silu(np.array(40.0)), 40.0, rtol=1e-15)
    np.testing.assert_allclose(ostack.silu(np.log(3.0)), np.log(3.0) * 0.75, rtol=1e-15)  # sigmoid(ln 3) = 3/4


def test_linear_orientation():
    # weights are stored [out, in]: a 2x3 weight maps a 3-vector to a 2-vector
    w = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 1.0]])
    np.testing.assert_array_equal(ostack.linear(np.array([[5.0, 7.0, 11.0]]), w), [[5.0, 25.0]])


def test_zero_output_projections_are_the_identity():
    """With every mixer output projection and every MLP down projection zero, each layer leaves x as it is,
    so the readout sees the question's own input row."""
    st = make_stack(SHAPES, "f32", REQS[:1], base=3)
    w = st.weights()
    for L in w["layers"]:
        L["w_o"] = np.zeros_like(L["w_o"])
        L["down"] = np.zeros_like(L["down"])
    out = ostack.run_stack_request(st, 0, "isolated")
    x0 = st.payload(0)["x0"]
    for x in out["xs"]:
        np.testing.assert_array_equal(x, np.asarray(x0, np.float64))
    segs = st.segment_rows(0)
    for i, (a, L) in enumerate(segs[1:]):
        off = sum(REQS[0].n_opt[:i])
        g = np.asarray(w["norm_f"], np.float64)
        row = np.asarray(x0[a + L - 1], np.float64)
        hf = row / np.sqrt(np.mean(row ** 2) + 1e-6) * g
        np.testing.assert_allclose(out["probs"][i], option_probs(hf, st.payload(0)["w_opt"][off:off + REQS[0].n_opt[i]]),
                                   rtol=1e-14)


def test_flat_stream_stack_equals_isolated_prompts():
    """Proposition 3.1 by induction over layers: the whole round run layer by layer over the flat stream
    (masked attention, two-call GDN by state index, row-wise layers on every row) gives every row of every
    layer and every probability of the isolated prompts."""
    st = make_stack(SHAPES, "f32", REQS, base=7)
    flat = flat_stack(st)
    lay = flat["layout"]
    qi = 0
    for j in range(len(REQS)):
        ref = ostack.run_stack_request(st, j, "isolated")
        segs = st.segment_rows(j)
        rows = list(range(lay["req_trunk_row0"][j], lay["req_trunk_row0"][j] + segs[0][1]))
        for i, (_, L) in enumerate(segs[1:]):
            rr = lay["seg_row0"][lay["req_q_seg0"][j] + i]
            rows += list(range(rr, rr + L))
        for li in range(len(SHAPES.layers) + 1):
            np.testing.assert_allclose(flat["xs"][li][rows], ref["xs"][li], rtol=1e-9, atol=1e-11,
                                       err_msg=f"request {j} layer {li}")
        for p in ref["probs"]:
            np.testing.assert_allclose(flat["probs"][qi], p, rtol=1e-9, atol=1e-12)
            qi += 1


def test_memo_order_equals_isolated_bitwise():
    st = make_stack(SHAPES, "f32", REQS, base=11)
    for j in range(len(REQS)):
        a = ostack.run_stack_request(st, j, "isolated")
        b = ostack.run_stack_request(st, j, "memo")
        for xa, xb in zip(a["xs"], b["xs"]):
            np.testing.assert_array_equal(xa, xb)
        for pa, pb in zip(a["probs"], b["probs"]):
            np.testing.assert_array_equal(pa, pb)


def test_sibling_perturbation_leaves_other_rows_bitwise():
    """Negating question 1's input rows changes only that question's rows and probabilities."""
    st = make_stack(SHAPES, "f32", REQS[:1], base=13)
    ref = ostack.run_stack_request(st, 0, "isolated")
    pl = dict(st.payload(0))
    a, L = st.segment_rows(0)[2]
    x0 = np.array(pl["x0"], copy=True)
    x0[a:a + L] *= -1.0
    pl["x0"] = x0
    pert = dataclasses.replace(st, _cache={0: pl})
    pert._w = st.weights()
    got = ostack.run_stack_request(pert, 0, "isolated")
    keep = np.ones(len(x0), bool)
    keep[a:a + L] = False
    for li in range(1, len(SHAPES.layers) + 1):
        np.testing.assert_array_equal(got["xs"][li][keep], ref["xs"][li][keep])
        assert not np.array_equal(got["xs"][li][~keep], ref["xs"][li][~keep])
    for i in (0, 2):
        np.testing.assert_array_equal(got["probs"][i], ref["probs"][i])


def test_stack_rejects_resumed_requests():
    with pytest.raises(ValueError):
        make_stack(SHAPES, "f32", [Request(P=10, m=4, q_len=(2,), n_opt=(2,), ckpt_slot=1, out_slot=0)])
