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


def test_short_rounds_bf16_subset(ctx):
    rnd = make_round(1, 0, requests=range(6))
    bufs, lay = harness.run_gpu(rnd, ctx, "direct")
    harness.check_round(rnd, harness.outputs(bufs), lay, mode="memo")


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
