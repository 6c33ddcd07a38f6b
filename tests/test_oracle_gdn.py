"""Pins of the oracle's Gated DeltaNet layer (CPU only)."""
import math

import numpy as np
import pytest

from oracle import round as oround
from oracle.gdn import causal_conv, gated_delta_rule, gdn_prompt, l2_normalise
from tests import brute
from workloads import LayerShapes, Request, custom_round


def test_conv_tap_probe_is_a_shift():
    rng = np.random.default_rng(0)
    L, C, K = 10, 6, 4
    x = rng.standard_normal((L, C))
    hist = rng.standard_normal((K - 1, C))
    ext = np.vstack([hist, x])
    for tau in range(K):
        w = np.zeros((C, K))
        w[:, tau] = 1.0
        y = causal_conv(x, w, hist)
        # tap tau reads the row K-1-tau steps back
        np.testing.assert_array_equal(y, ext[tau:tau + L])


def test_l2_normalise_unit_norm_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3, 32))
    n = np.linalg.norm(l2_normalise(x), axis=-1)
    np.testing.assert_allclose(n, 1.0, atol=1e-6)
    np.testing.assert_allclose(l2_normalise(5.0 * x), l2_normalise(x), atol=1e-7)
    assert np.all(l2_normalise(np.zeros((2, 4))) == 0.0)


def _rand_unit(rng, shape):
    z = rng.standard_normal(shape)
    return z / np.linalg.norm(z, axis=-1, keepdims=True)


def test_eta_zero_is_pure_decay():
    rng = np.random.default_rng(2)
    L, H, dk, dv = 9, 2, 5, 3
    q, k = _rand_unit(rng, (L, H, dk)), _rand_unit(rng, (L, H, dk))
    v = rng.standard_normal((L, H, dv))
    alpha = rng.uniform(0.5, 1.0, (L, H))
    S0 = rng.standard_normal((H, dv, dk))
    o, S = gated_delta_rule(q, k, v, alpha, np.zeros((L, H)), S0)
    decay = np.cumprod(alpha, axis=0)
    for t in range(L):
        for h in range(H):
            np.testing.assert_allclose(o[t, h], decay[t, h] * S0[h] @ q[t, h], atol=1e-13)
    np.testing.assert_allclose(S, decay[-1][:, None, None] * S0, atol=1e-13)


def test_one_hot_keys_are_an_associative_memory():
    # alpha = eta = 1 and k = e_i overwrite column i of S with v
    rng = np.random.default_rng(3)
    dk, dv, L = 4, 3, 8
    slots = [2, 0, 2, 3, 1, 0, 2, 1]
    k = np.zeros((L, 1, dk))
    for t, i in enumerate(slots):
        k[t, 0, i] = 1.0
    v = rng.standard_normal((L, 1, dv))
    q = np.zeros((L, 1, dk))
    q[:, 0, 0] = 1.0
    o, S = gated_delta_rule(q, k, v, np.ones((L, 1)), np.ones((L, 1)), np.zeros((1, dv, dk)))
    last = {}
    for t, i in enumerate(slots):
        last[i] = v[t, 0]
        # reading slot 0 returns the latest value written to slot 0 (or zero)
        np.testing.assert_array_equal(o[t, 0], last.get(0, np.zeros(dv)))
    for i in range(dk):
        np.testing.assert_array_equal(S[0][:, i], last[i])


def test_scalar_state_geometric_closed_form():
    # d_k = d_v = 1, k = q = 1, constant alpha, eta, v: S_t = a S_{t-1} + b with a = alpha(1-eta), b = eta v
    L, alpha, eta, vv, s0 = 30, 0.9, 0.3, 2.5, -1.0
    ones = np.ones((L, 1, 1))
    o, S = gated_delta_rule(ones, ones, np.full((L, 1, 1), vv), np.full((L, 1), alpha),
                            np.full((L, 1), eta), np.full((1, 1, 1), s0))
    a, b = alpha * (1 - eta), eta * vv
    for t in range(1, L + 1):
        want = a ** t * s0 + b * (1 - a ** t) / (1 - a)
        assert o[t - 1, 0, 0] == pytest.approx(want, rel=1e-13, abs=1e-13)


def test_channel_order_worked_example():
    # One head, dk = dv = 1, conv width 1 with weight 1 (the identity), input rows [q | k | v]:
    #   row 1: q = +1, k = +2, v = 3   -> k^ = 2/sqrt(4+1e-6), S_1 = eta*v*k^, o_1 = S_1 * q^
    #   row 2: q = -1, k = +1, v = 0   -> S_2 = alpha*S_1*(1 - eta*k^2), o_2 = -S_2
    # With alpha = eta = 1/2: S_1 ~ 1.5, o_1 ~ 1.5, S_2 ~ 0.375, o_2 ~ -0.375 (1e-6 eps effects).
    x = np.array([[1.0, 2.0, 3.0], [-1.0, 1.0, 0.0]])
    w = np.ones((3, 1))
    o, S, _ = gdn_prompt(x, np.full((2, 1), 0.5), np.full((2, 1), 0.5), w, H=1, dk=1, dv=1)
    assert o[0, 0, 0] == pytest.approx(1.5, abs=1e-5)
    assert o[1, 0, 0] == pytest.approx(-0.375, abs=1e-5)
    assert S[0, 0, 0] == pytest.approx(0.375, abs=1e-5)


def test_recurrence_equals_explicit_matrix_form():
    rng = np.random.default_rng(4)
    L, H, dk, dv = 12, 3, 6, 5
    q, k = _rand_unit(rng, (L, H, dk)), _rand_unit(rng, (L, H, dk))
    v = rng.standard_normal((L, H, dv))
    a, e = rng.uniform(0.6, 1.0, (L, H)), rng.uniform(0.0, 1.0, (L, H))
    S0 = rng.standard_normal((H, dv, dk))
    o1, S1 = gated_delta_rule(q, k, v, a, e, S0)
    o2, S2 = brute._recurrence_explicit(q, k, v, a, e, S0.copy())
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(S1, S2, atol=1e-12)


def test_state_and_window_continuation():
    """Splitting a prompt anywhere and continuing from (S, window) equals one pass."""
    rng = np.random.default_rng(5)
    H, dk, dv, K, L = 2, 4, 3, 4, 15
    C = H * (2 * dk + dv)
    x = rng.standard_normal((L, C))
    al, et = rng.uniform(0.5, 1, (L, H)), rng.uniform(0, 1, (L, H))
    w = rng.standard_normal((C, K))
    full, S_full, win_full = gdn_prompt(x, al, et, w, H, dk, dv)
    for cut in (1, 2, 3, 7):
        o1, S1, w1 = gdn_prompt(x[:cut], al[:cut], et[:cut], w, H, dk, dv)
        np.testing.assert_array_equal(w1[-cut:], x[max(0, cut - (K - 1)):cut][-min(cut, K - 1):])
        o2, S2, w2 = gdn_prompt(x[cut:], al[cut:], et[cut:], w, H, dk, dv, window0=w1, S0=S1)
        np.testing.assert_array_equal(np.vstack([o1, o2]), full)
        np.testing.assert_array_equal(S2, S_full)
        np.testing.assert_array_equal(w2, win_full)


SMALL = LayerShapes(H=2, dk=6, dv=5, conv_k=4, Hq=2, Hkv=1, d=4, theta=1e4, hidden=4)


def test_two_call_fork_equals_isolated_prompts():
    """Proposition 3.1 for GDN: trunks first, then questions seeded by state index."""
    reqs = [Request(P=7, m=0, q_len=(3, 1, 4), n_opt=(2, 2, 2), out_slot=3),
            Request(P=2, m=0, q_len=(2, 5), n_opt=(2, 2), out_slot=0),     # trunk shorter than K-1
            Request(P=9, m=6, q_len=(2,), n_opt=(2,), ckpt_slot=1, out_slot=2),
            Request(P=0, m=0, q_len=(3,), n_opt=(2,), out_slot=4)]
    rnd = custom_round(SMALL, "f32", reqs, base=5)
    lay = brute.build_layout(rnd.requests)
    o_flat, states, windows = brute.flat_gdn(rnd, lay)
    iso = oround.run_round(rnd, "isolated")
    np.testing.assert_allclose(o_flat, brute.to_stream(rnd, lay, iso, "gdn_o"), atol=1e-12, rtol=0)
    for j, r in enumerate(reqs):
        np.testing.assert_allclose(states[r.out_slot], iso[j]["S_P"], atol=1e-12, rtol=0)
        np.testing.assert_array_equal(windows[r.out_slot], iso[j]["window_P"])


def test_resume_from_checkpoint_equals_full_run():
    """A checkpoint at m (state, conv window, rotated K and V) resumes to the full run's values."""
    full_req = Request(P=14, m=0, q_len=(3, 2), n_opt=(2, 2), out_slot=0)
    rnd_full = custom_round(SMALL, "f32", [full_req], base=9)
    pl = rnd_full.payload(0)
    cw = rnd_full.conv_w()
    m = 8
    from oracle.attention import rope_rotate
    _, S_m, win_m = gdn_prompt(pl["gdn_x"][:m], pl["alpha"][:m], pl["eta"][:m], cw, SMALL.H, SMALL.dk, SMALL.dv)
    res_req = Request(P=14, m=m, q_len=(3, 2), n_opt=(2, 2), ckpt_slot=1, out_slot=0)
    rnd_res = custom_round(SMALL, "f32", [res_req], base=9)
    res_pl = {k: np.asarray(v)[m:] if k in ("attn_q", "attn_k", "attn_v", "gdn_x", "alpha", "eta", "hidden")
              else v for k, v in pl.items()}
    res_pl["ckpt_state"] = S_m
    res_pl["ckpt_window"] = win_m
    res_pl["kv_k"] = rope_rotate(np.asarray(pl["attn_k"][:m], np.float64), np.arange(m)[:, None], SMALL.theta)
    res_pl["kv_v"] = np.asarray(pl["attn_v"][:m], np.float64)
    a = oround.run_request(rnd_full, 0, cw, "isolated")
    b = oround.run_request(rnd_res, 0, cw, "isolated", payload=res_pl)
    np.testing.assert_array_equal(b["gdn_o"], a["gdn_o"][m:])
    np.testing.assert_array_equal(b["S_P"], a["S_P"])
    np.testing.assert_allclose(b["attn_o"], a["attn_o"][m:], atol=1e-13, rtol=0)
    for pa, pb in zip(a["probs"], b["probs"]):
        np.testing.assert_array_equal(pa, pb)


def test_silu_option_closed_form():
    """act = "silu": with identity conv taps, one-hot keys and queries, alpha = eta = 1 and a zero start
    state, the output equals the activated value input: silu(ln 3) = 0.75 ln 3, silu(-ln 3) = -0.25 ln 3
    (a sigmoid, a missing activation or one applied after the norm fails)."""
    ln3 = np.log(3.0)
    for xv, want in ((ln3, 0.75 * ln3), (-ln3, -0.25 * ln3)):
        x = np.array([[1.0, 0.0, 1.0, 0.0, xv]])  # q (dk = 2) | k (dk = 2) | v (dv = 1)
        o, S, _ = gdn_prompt(x, np.ones((1, 1)), np.ones((1, 1)), np.ones((5, 1)), H=1, dk=2, dv=1, act="silu")
        np.testing.assert_allclose(o[0, 0, 0], want, rtol=1e-5)
        o0, _, _ = gdn_prompt(x, np.ones((1, 1)), np.ones((1, 1)), np.ones((5, 1)), H=1, dk=2, dv=1)
        np.testing.assert_allclose(o0[0, 0, 0], xv, rtol=1e-5)


def _resume_payload(pl: dict, m: int, ckpt: dict) -> dict:
    """Payload of the same request resumed at m from checkpoint ``ckpt`` (stream rows from m on)."""
    out = {k: np.asarray(v)[m:] if k in ("attn_q", "attn_k", "attn_v", "gdn_x", "alpha", "eta", "hidden")
           else v for k, v in pl.items()}
    out.update(ckpt)
    return out


def test_created_checkpoint_resumes_to_full_run():
    """make_checkpoint at an interior position, then a resume from it, reproduces the uncut run: GDN
    outputs, S_P and option probabilities bit for bit, attention to rounding (a checkpoint taken one
    row off, with unrotated keys or without the conv window fails this)."""
    full_req = Request(P=14, m=0, q_len=(3, 2), n_opt=(2, 2), out_slot=0)
    rnd_full = custom_round(SMALL, "f32", [full_req], base=11)
    cw = rnd_full.conv_w()
    a = oround.run_request(rnd_full, 0, cw, "isolated")
    for save_m in (1, 5, 13):
        ck = oround.make_checkpoint(rnd_full, 0, save_m, cw)
        res_req = Request(P=14, m=save_m, q_len=(3, 2), n_opt=(2, 2), ckpt_slot=1, out_slot=0)
        rnd_res = custom_round(SMALL, "f32", [res_req], base=11)
        b = oround.run_request(rnd_res, 0, cw, "isolated", payload=_resume_payload(rnd_full.payload(0), save_m, ck))
        np.testing.assert_array_equal(b["gdn_o"], a["gdn_o"][save_m:])
        np.testing.assert_array_equal(b["S_P"], a["S_P"])
        np.testing.assert_allclose(b["attn_o"], a["attn_o"][save_m:], atol=1e-13, rtol=0)
        for pa, pb in zip(a["probs"], b["probs"]):
            np.testing.assert_array_equal(pa, pb)


def test_checkpoint_of_a_resumed_request_chains():
    """A checkpoint made by a request that itself resumed (positions below its m come from its own
    checkpoint) resumes to the same values as one made by the uncut run; at save_m = P it is the trunk's
    end state and window."""
    full_req = Request(P=14, m=0, q_len=(2,), n_opt=(2,), out_slot=0)
    rnd_full = custom_round(SMALL, "f32", [full_req], base=12)
    cw = rnd_full.conv_w()
    pl = rnd_full.payload(0)
    ck6 = oround.make_checkpoint(rnd_full, 0, 6, cw)
    res_req = Request(P=14, m=6, q_len=(2,), n_opt=(2,), ckpt_slot=1, out_slot=0)
    rnd_res = custom_round(SMALL, "f32", [res_req], base=12)
    pl6 = _resume_payload(pl, 6, ck6)
    direct = oround.make_checkpoint(rnd_full, 0, 11, cw)
    chained = oround.make_checkpoint(rnd_res, 0, 11, cw, payload=pl6)
    for key in direct:
        np.testing.assert_array_equal(chained[key], direct[key], err_msg=key)
    end = oround.make_checkpoint(rnd_full, 0, 14, cw)
    a = oround.run_request(rnd_full, 0, cw, "memo")
    np.testing.assert_array_equal(end["ckpt_state"], a["S_P"])
    np.testing.assert_array_equal(end["ckpt_window"], a["window_P"])
