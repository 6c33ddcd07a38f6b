"""Pins of the oracle's Eq. (1) readout (CPU only)."""
import math

import numpy as np

from oracle.readout import option_probs
from oracle import round as oround
from tests import brute
from workloads import LayerShapes, Request, custom_round


def test_single_option_is_certain():
    p = option_probs(np.array([1.0, -2.0]), np.array([[0.3, 0.7]]))
    np.testing.assert_array_equal(p, [1.0])


def test_equal_logits_are_uniform():
    w = np.tile(np.array([[0.5, -1.5, 2.0]]), (5, 1))
    np.testing.assert_allclose(option_probs(np.array([1.0, 2.0, 3.0]), w), np.full(5, 0.2), atol=1e-15)


def test_two_options_worked_values():
    # logits 0 and ln 3 -> probabilities 1/4 and 3/4
    w = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    np.testing.assert_allclose(option_probs(np.array([1.0, 7.0]), w), [0.25, 0.75], atol=1e-15)


def test_large_logits_stay_finite_and_normalised():
    rng = np.random.default_rng(0)
    w = 100.0 * rng.standard_normal((8, 16))
    p = option_probs(rng.standard_normal(16), w)
    assert np.isfinite(p).all()
    assert abs(p.sum() - 1.0) < 1e-14


def test_readout_uses_question_final_rows():
    sh = LayerShapes(H=1, dk=2, dv=2, conv_k=2, Hq=1, Hkv=1, d=2, theta=1e4, hidden=6)
    reqs = [Request(P=5, m=0, q_len=(2, 3), n_opt=(3, 2), out_slot=0),
            Request(P=3, m=0, q_len=(4,), n_opt=(5,), out_slot=1)]
    rnd = custom_round(sh, "f32", reqs, base=3)
    iso = oround.run_round(rnd, "isolated")
    flat = brute.flat_readout(rnd, brute.build_layout(rnd.requests))
    got = [p for r in iso for p in r["probs"]]
    assert len(got) == len(flat) == 3
    for a, b in zip(got, flat):
        np.testing.assert_allclose(a, b, atol=1e-15)
