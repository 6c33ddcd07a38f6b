"""The allocation-free attention entry point (flide_fork_attn_noalloc) against flide_fork_attn, through the
C ABI (needs an MI355X).  Two calls in a row share the library's device scratch; the second has a smaller
input, so stale contents of the first must not leak into it."""
import pytest

from tests import harness
from workloads import make_round

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    import torch
    from tree_forked_hybrid_amd import flide as F
    assert torch.cuda.is_available()
    c = F.Context(0)
    yield c
    c.close()


def _noalloc_equals_fork_attn(ctx, rnd):
    import torch
    from tree_forked_hybrid_amd import flide as F
    bufs, _ = harness.run_gpu(rnd, ctx, "direct")  # flide_fork_attn with the buffers' own workspace
    T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
    # the context's own rotary table (built by flide_fork_attn), then a fresh context, whose call writes
    # the table into the scratch's table region
    with F.Context(0) as fresh:
        for c, name in ((ctx, "context table"), (fresh, "scratch table")):
            for l in range(bufs.n_attn):
                ref = bufs.o_attn[l].clone()
                out = torch.full_like(ref, float("nan"))
                F.flide_fork_attn_noalloc(c, bufs.caps, bufs.dev_meta, bufs.attn_params[l], bufs.q[l], bufs.k[l],
                                          bufs.v[l], bufs.k_cache[l], bufs.v_cache[l], out)
                torch.cuda.synchronize()
                F.flide_check_device(c, bufs.caps, bufs.dev_meta)
                print(f"[noalloc] {name} layer {l}: T={T} caps={bufs.caps.T_cap}", flush=True)
                assert torch.equal(out[:T], ref[:T]), (name, l)
                assert torch.isnan(out[T:]).all()  # tail rows untouched


def test_noalloc_attention_two_calls_second_smaller(ctx):
    # bf16 MFMA path: eight short-round requests, then three
    _noalloc_equals_fork_attn(ctx, make_round(1, 0, requests=range(8)))
    _noalloc_equals_fork_attn(ctx, make_round(1, 0, requests=range(3)))


def test_noalloc_attention_fp32_sliding_window_and_resume(ctx):
    # f32 path (config-0 shapes), then a long-document request's full and sliding-window layers
    _noalloc_equals_fork_attn(ctx, make_round(0, 0))
    full = make_round(2, 0)
    j = min(range(len(full.requests)), key=lambda i: full.requests[i].P)
    _noalloc_equals_fork_attn(ctx, full.subset([j]))


def test_noalloc_attention_rejects_oversized_workspace(ctx):
    from tree_forked_hybrid_amd import flide as F
    from tree_forked_hybrid_amd.runner import spec_for_round
    rnd = make_round(1, 0, requests=range(2))
    bufs, _ = harness.run_gpu(rnd, ctx, "direct", spec=spec_for_round(rnd, T_cap=65536))
    before = bufs.o_attn[0].clone()
    with pytest.raises(F.FlideError) as e:
        F.flide_fork_attn_noalloc(ctx, bufs.caps, bufs.dev_meta, bufs.attn_params[0], bufs.q[0], bufs.k[0],
                                  bufs.v[0], None, None, bufs.o_attn[0])
    assert e.value.status == F.FLIDE_E_CAPACITY
    assert "scratch" in str(e.value)
    import torch
    torch.cuda.synchronize()
    assert torch.equal(bufs.o_attn[0], before)
