"""Pins of the oracle's attention (CPU only).

Each test fixes the oracle against something other than its own formula:
values of cos/sin at known angles, exact softmax outcomes, closed forms, and
the flat-stream masked formulation of Flide (tests/brute.py).
"""
import math

import numpy as np
import pytest

from oracle.attention import prompt_attention, rope_rotate
from tests import brute
from oracle import round as oround
from workloads import LayerShapes, Request, custom_round


def test_rope_pairing_and_frequency_worked_values():
    # pair (0, d/2) turns at 1 rad per position; pair (1, 1+d/2) at theta**(-2/d) rad
    c1, s1 = 0.5403023058681398, 0.8414709848078965          # cos(1), sin(1)
    out = rope_rotate(np.array([1.0, 0.0, 0.0, 0.0]), 1, 10000.0)
    np.testing.assert_allclose(out, [c1, 0.0, s1, 0.0], atol=1e-15)
    # theta = 1e4, d = 4: second pair frequency 1e-2, so position 100 turns it by 1 rad
    out = rope_rotate(np.array([0.0, 1.0, 0.0, 0.0]), 100, 10000.0)
    np.testing.assert_allclose(out, [0.0, c1, 0.0, s1], atol=1e-14)
    # position 0 is the identity
    x = np.random.default_rng(0).standard_normal(32)
    np.testing.assert_array_equal(rope_rotate(x, 0, 1e6), x)


def test_rope_is_a_rotation_group():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    a = rope_rotate(rope_rotate(x, 17, 1e4), 25, 1e4)
    b = rope_rotate(x, 42, 1e4)
    np.testing.assert_allclose(a, b, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(b, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    L, Hq, Hkv, d = 9, 4, 2, 16
    q, k, v = rng.standard_normal((L, Hq, d)), rng.standard_normal((L, Hkv, d)), rng.standard_normal((L, Hkv, d))
    o1 = prompt_attention(q, k, v, np.arange(L), 1e4)
    o2 = prompt_attention(q, k, v, np.arange(L) + 1000, 1e4)
    np.testing.assert_allclose(o1, o2, atol=1e-11)


def test_first_row_sees_only_itself():
    rng = np.random.default_rng(3)
    L, Hq, Hkv, d = 6, 4, 2, 8
    q, k, v = rng.standard_normal((L, Hq, d)), rng.standard_normal((L, Hkv, d)), rng.standard_normal((L, Hkv, d))
    o = prompt_attention(q, k, v, np.arange(L), 1e4)
    np.testing.assert_array_equal(o[0], np.repeat(v[0], 2, axis=0))


def test_window_of_one_returns_own_value():
    rng = np.random.default_rng(4)
    L, Hq, Hkv, d = 7, 2, 1, 8
    q, k, v = rng.standard_normal((L, Hq, d)), rng.standard_normal((L, Hkv, d)), rng.standard_normal((L, Hkv, d))
    o = prompt_attention(q, k, v, np.arange(L), 1e4, window=1)
    np.testing.assert_array_equal(o, np.repeat(v, 2, axis=1))


def test_zero_queries_average_visible_values():
    rng = np.random.default_rng(5)
    L, Hq, Hkv, d, W = 12, 2, 1, 8, 5
    k, v = rng.standard_normal((L, Hkv, d)), rng.standard_normal((L, Hkv, d))
    q = np.zeros((L, Hq, d))
    o = prompt_attention(q, k, v, np.arange(L), 1e4)
    ow = prompt_attention(q, k, v, np.arange(L), 1e4, window=W)
    for a in range(L):
        np.testing.assert_allclose(o[a, 0], v[:a + 1, 0].mean(0), atol=1e-14)
        np.testing.assert_allclose(ow[a, 1], v[max(0, a - W + 1):a + 1, 0].mean(0), atol=1e-14)


def test_score_scale_is_inverse_sqrt_d():
    # d = 2, row 1 sees key 0 (zero vector, score 0) and key 1 (score x/sqrt(2)).
    # With x = sqrt(2)*ln 3 the weights are 1/4 and 3/4.  v0 = 0, v1 = (4, 8) -> o1 = (3, 6).
    x = math.sqrt(2.0) * math.log(3.0)
    q = np.array([[[0.0, 0.0]], [[x, 0.0]]])
    k = np.array([[[0.0, 0.0]], [[1.0, 0.0]]])
    v = np.array([[[0.0, 0.0]], [[4.0, 8.0]]])
    o = prompt_attention(q, k, v, np.array([0, 1]), 1e4)
    np.testing.assert_allclose(o[1, 0], [3.0, 6.0], atol=1e-13)


def test_grouped_query_heads_share_contiguous_kv_heads():
    q = np.ones((1, 4, 4))
    k = np.ones((1, 2, 4))
    v = np.stack([np.full(4, 1.0), np.full(4, 2.0)])[None]
    o = prompt_attention(q, k, v, np.array([0]), 1e4)
    np.testing.assert_array_equal(o[0, :, 0], [1.0, 1.0, 2.0, 2.0])


def test_cached_prefix_equals_full_prompt():
    rng = np.random.default_rng(6)
    L, m, Hq, Hkv, d = 20, 8, 4, 2, 16
    q, k, v = rng.standard_normal((L, Hq, d)), rng.standard_normal((L, Hkv, d)), rng.standard_normal((L, Hkv, d))
    full = prompt_attention(q, k, v, np.arange(L), 1e4, window=6)
    ck = rope_rotate(k[:m], np.arange(m)[:, None], 1e4)
    part = prompt_attention(q[m:], k[m:], v[m:], np.arange(m, L), 1e4, window=6, cache_k=ck, cache_v=v[:m])
    np.testing.assert_allclose(part, full[m:], atol=1e-13)


SMALL = LayerShapes(H=2, dk=8, dv=8, conv_k=4, Hq=4, Hkv=2, d=8, theta=1e4, hidden=8, swa_window=3)


def _small_round():
    reqs = [Request(P=9, m=0, q_len=(3, 2, 4), n_opt=(2, 3, 2), out_slot=0),
            Request(P=5, m=0, q_len=(2,), n_opt=(4,), out_slot=1),
            Request(P=6, m=3, q_len=(1, 2), n_opt=(2, 2), ckpt_slot=2, out_slot=3),
            Request(P=4, m=0, q_len=(), n_opt=(), out_slot=4)]
    return custom_round(SMALL, "f32", reqs, base=11)


def test_flat_stream_mask_equals_isolated_prompts():
    """Proposition 3.1 for attention: the flat masked stream reproduces every isolated prompt."""
    rnd = _small_round()
    flat = brute.flat_round(rnd)
    lay = flat["layout"]
    iso = oround.run_round(rnd, "isolated")
    for key in ("attn_o", "swa_o"):
        ref = brute.to_stream(rnd, lay, iso, key)
        np.testing.assert_allclose(flat[key], ref, atol=1e-12, rtol=0)


def test_sibling_payload_cannot_reach_other_rows():
    rnd = _small_round()
    base = brute.flat_round(rnd)
    # perturb question 2 of request 0 only
    pl = rnd.payload(0, keep=True)
    s, L = rnd.segment_rows(0)[2]
    for name in ("attn_q", "attn_k", "attn_v"):
        pl[name][s:s + L] += 3.0
    pert = brute.flat_round(rnd)
    lay = base["layout"]
    q2 = lay["req_q_seg0"][0] + 1
    r0, n = lay["seg_row0"][q2], lay["seg_len"][q2]
    others = np.ones(lay["T"], bool)
    others[r0:r0 + n] = False
    np.testing.assert_array_equal(base["attn_o"][others], pert["attn_o"][others])
    assert not np.allclose(base["attn_o"][r0:r0 + n], pert["attn_o"][r0:r0 + n])


@pytest.mark.parametrize("mode", ["isolated", "memo"])
def test_modes_agree(mode):
    rnd = _small_round()
    a = oround.run_round(rnd, mode)
    b = oround.run_round(rnd, "isolated")
    for j in range(len(rnd.requests)):
        np.testing.assert_array_equal(a[j]["attn_o"], b[j]["attn_o"])
        np.testing.assert_array_equal(a[j]["gdn_o"], b[j]["gdn_o"])
