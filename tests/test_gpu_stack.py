"""Multi-layer hybrid stack on the GPU against the isolated-prompt oracle (needs an MI355X).

Pre-norm residual blocks around Gated DeltaNet, full-attention and sliding-window layers run over the flat
stream through the C ABI; after the last token mixer the row-wise layers and the readout act on
question-final rows only.  Proposition 3.1 by induction over layers: every row must equal its isolated
prompt's."""
import dataclasses

import numpy as np
import pytest

from oracle import layout as olayout
from oracle import stack as ostack
from tests import harness
from workloads import Request, StackShapes, make_stack

pytestmark = pytest.mark.gpu

F32_SHAPES = StackShapes(Dm=64, F=96, layers=("gdn", "attn", "gdn", "swa"), H=2, dk=32, dv=32, conv_k=4, Hq=4,
                         Hkv=2, d=32, theta=1e4, window=12)
# bf16: dk = dv = 128 runs the chunked GDN kernel, d = 128 the MFMA attention
BF16_SHAPES = StackShapes(Dm=256, F=512, layers=("gdn", "gdn", "attn", "swa"), H=2, dk=128, dv=128, conv_k=4,
                          Hq=4, Hkv=2, d=128, theta=1e4, window=64)
REQS = [Request(P=150, m=0, q_len=(10, 33, 1), n_opt=(2, 5, 3), out_slot=0),
        Request(P=0, m=0, q_len=(4,), n_opt=(3,), out_slot=1),
        Request(P=70, m=0, q_len=(20, 12), n_opt=(4, 2), out_slot=2),
        Request(P=9, m=0, q_len=(), n_opt=(), out_slot=3)]
# bf16 activations are rounded at about seven points per layer (unit roundoff 2^-9); over four layers the
# relative error of a row is a few 1e-3 typically, bounded here by 5e-2; probabilities by TV 1e-2
TOL = {"f32": (1e-4, 1e-4), "bf16": (5e-2, 1e-2)}


@pytest.fixture(scope="module")
def ctx():
    import torch
    from tree_forked_hybrid_amd import flide as F
    assert torch.cuda.is_available()
    c = F.Context(0)
    yield c
    c.close()


def _runner(stack):
    from tree_forked_hybrid_amd.runner import StackRunner
    lay = olayout.build_layout(stack.requests)
    n_opt = sum(sum(r.n_opt) for r in stack.requests)
    sr = StackRunner(stack, T_cap=max(lay["T"], 1), R_cap=len(stack.requests), Q_cap=max(lay["n_qst"], 1),
                     opt_cap=max(n_opt, 1))
    sr.fill(lay)
    return sr, lay


def _run(stack, ctx, selective=True):
    import torch
    from tree_forked_hybrid_amd import flide as F
    sr, lay = _runner(stack)
    img = F.flide_plan_round(stack.requests, sr.caps)
    print(f"[stack] dtype={stack.dtype} T={lay['T']} layers={stack.shapes.layers} selective={selective}",
          flush=True)
    sr.upload(ctx, img)
    sr.run(ctx, selective=selective)
    torch.cuda.synchronize()
    F.flide_check_device(ctx, sr.caps, sr.dev_meta)
    return sr, lay, img


def _outputs(sr):
    return {"x": sr.x.float().cpu().numpy().astype(np.float64), "hf": sr.hf.float().cpu().numpy().astype(np.float64),
            "probs": sr.probs.cpu().numpy().astype(np.float64)}


def _check(stack, got, lay, all_rows):
    tol, tv_tol = TOL[stack.dtype]
    rep = {"x": 0.0, "hf": 0.0, "tv": 0.0}
    off = harness.option_offsets(stack)
    qi = 0
    for j in range(len(stack.requests)):
        ref = ostack.run_stack_request(stack, j, "memo")
        rows = harness.stream_rows(stack, lay, j)
        if all_rows:
            rep["x"] = max(rep["x"], harness.rel_err(got["x"][rows], ref["xs"][-1]))
        segs = stack.segment_rows(j)
        for i, p in enumerate(ref["probs"]):
            row = lay["qfin_row"][qi]
            local = segs[1 + i][0] + segs[1 + i][1] - 1
            rep["hf"] = max(rep["hf"], harness.rel_err(got["hf"][row][None], ref["hf"][i][None]))
            rep["x"] = max(rep["x"], harness.rel_err(got["x"][row][None], ref["xs"][-1][local][None]))
            rep["tv"] = max(rep["tv"], harness.tv(got["probs"][off[qi]:off[qi + 1]], p))
            qi += 1
    print(f"[stack parity] {rep} (tol {tol}, tv {tv_tol})", flush=True)
    assert rep["x"] <= tol and rep["hf"] <= tol and rep["tv"] <= tv_tol, rep


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stack_matches_isolated_prompts(ctx, dtype):
    """Every row after the last layer (last MLP on every row), then the selective run's question-final
    rows and probabilities, against the oracle."""
    stack = make_stack(F32_SHAPES if dtype == "f32" else BF16_SHAPES, dtype, REQS, base=31)
    sr, lay, _ = _run(stack, ctx, selective=False)
    _check(stack, _outputs(sr), lay, all_rows=True)
    sr, lay, _ = _run(stack, ctx, selective=True)
    _check(stack, _outputs(sr), lay, all_rows=False)


def test_stack_selective_readout_equals_full(ctx):
    """Running the last layer's MLP on question-final rows only gives those rows' bits and every
    probability exactly as running it on every row (row-wise layers)."""
    stack = make_stack(BF16_SHAPES, "bf16", REQS, base=37)
    full, lay, _ = _run(stack, ctx, selective=False)
    sel, _, _ = _run(stack, ctx, selective=True)
    a, b = _outputs(full), _outputs(sel)
    q = lay["qfin_row"][:lay["n_qst"]]
    np.testing.assert_array_equal(a["x"][q], b["x"][q])
    np.testing.assert_array_equal(a["hf"][q], b["hf"][q])
    np.testing.assert_array_equal(a["probs"], b["probs"])


def test_stack_graph_replays_equal_eager(ctx):
    """The whole stack captured into one HIP graph, replayed three times with other device work and
    synchronisations between the replays; every replay equals the eager run bit for bit."""
    import torch
    from tree_forked_hybrid_amd import flide as F
    stack = make_stack(BF16_SHAPES, "bf16", REQS, base=41)
    sr, lay, img = _run(stack, ctx)
    ref = _outputs(sr)
    sr.capture(ctx)
    scratch = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        sr.fill(lay)                                    # inputs again (the stack updates x in place)
        sr.hf.zero_()
        sr.probs.zero_()
        scratch = torch.tanh(scratch @ scratch.T * 1e-3)
        torch.cuda.synchronize()
        sr.replay(ctx, img)
        torch.cuda.synchronize()
        F.flide_check_device(ctx, sr.caps, sr.dev_meta)
        got = _outputs(sr)
        for k in ref:
            np.testing.assert_array_equal(got[k], ref[k], err_msg=f"replay {rep}: {k}")


def test_stack_bits_do_not_depend_on_the_round(ctx):
    """A request's question-final rows and probabilities are bit-identical alone and inside the round."""
    stack = make_stack(BF16_SHAPES, "bf16", REQS, base=43)
    full, lay, _ = _run(stack, ctx)
    one = dataclasses.replace(stack, requests=[REQS[2]], _cache={0: stack.payload(2)})
    one._w = stack.weights()
    alone, lay1, _ = _run(one, ctx)
    a, b = _outputs(full), _outputs(alone)
    q0 = sum(len(r.q_len) for r in REQS[:2])  # request 2's questions follow those of requests 0 and 1
    q_full = lay["qfin_row"][q0:q0 + 2]
    q_one = lay1["qfin_row"][0:2]
    np.testing.assert_array_equal(a["x"][q_full], b["x"][q_one])
    np.testing.assert_array_equal(a["hf"][q_full], b["hf"][q_one])
    off = harness.option_offsets(stack)
    np.testing.assert_array_equal(a["probs"][off[q0]:off[q0 + 2]], b["probs"][:off[q0 + 2] - off[q0]])
