"""Pins of the oracle's flat-stream metadata builder and split rule (CPU only)."""
import os

import numpy as np
import pytest

from oracle import layout
from workloads import Request


def _read_golden(path):
    recs = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        recs.setdefault(key, []).append([int(v) for v in vals])
    return recs


def _fig_request():
    return [Request(P=48, m=0, q_len=(5, 7, 9), n_opt=(4, 4, 4), ckpt_slot=-1, out_slot=0)]


def test_worked_example_matches_hand_derivation(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "layout_one_request_three_questions.txt"))
    lay = layout.build_layout(_fig_request())
    assert lay["T"] == g["T"][0][0]
    assert lay["R"] == g["R"][0][0]
    segs = np.stack([lay["seg_row0"], lay["seg_len"], lay["seg_req"], lay["seg_branch"],
                     lay["seg_pos0"], lay["seg_state"]], 1)
    assert segs.tolist() == g["seg"]
    assert lay["qfin_row"].tolist() == g["qfin"][0]
    for row, j, c, t in g["row"]:
        assert (lay["tok_j"][row], lay["tok_c"][row], lay["tok_t"][row]) == (j, c, t)
    T = lay["T"]
    jj, cc, tt = lay["tok_j"], lay["tok_c"], lay["tok_t"]

    def nvis(x):
        return sum(layout.visible(jj[x], cc[x], tt[x], jj[y], cc[y], tt[y]) for y in range(T))

    for row, n in g["vis"]:
        assert nvis(row) == n
    assert sum(nvis(x) for x in range(T)) == g["pairs"][0][0]


def test_tail_rows_are_sentinels():
    lay = layout.build_layout(_fig_request(), t_cap=80)
    assert lay["T"] == 69
    for a in ("tok_j", "tok_c", "tok_t"):
        assert (lay[a][69:] == -1).all() and (lay[a][:69] >= 0).all()


def test_multi_request_order_and_positions():
    reqs = [Request(P=10, m=0, q_len=(2, 3), n_opt=(2, 2), out_slot=5),
            Request(P=7, m=4, q_len=(), n_opt=(), ckpt_slot=1, out_slot=2),
            Request(P=0, m=0, q_len=(1,), n_opt=(3,), out_slot=0)]
    lay = layout.build_layout(reqs)
    # trunks first (10, 3 and 0 rows), then the questions of request 0 and of request 2
    assert lay["seg_row0"].tolist() == [0, 10, 13, 13, 15, 18]
    assert lay["seg_len"].tolist() == [10, 3, 0, 2, 3, 1]
    assert lay["seg_req"].tolist() == [0, 1, 2, 0, 0, 2]
    assert lay["seg_branch"].tolist() == [0, 0, 0, 1, 2, 1]
    assert lay["seg_pos0"].tolist() == [0, 4, 0, 10, 10, 0]
    assert lay["seg_state"].tolist() == [-1, 1, -1, 5, 5, 0]
    assert lay["req_trunk_row0"].tolist() == [0, 10, 13]
    assert lay["req_q_seg0"].tolist() == [3, 5, 5]
    assert lay["qfin_row"].tolist() == [14, 17, 18]
    assert lay["T"] == 19
    assert lay["tok_t"][10:13].tolist() == [4, 5, 6]


@pytest.mark.parametrize("bad", [
    Request(P=4, m=5, q_len=(1,), n_opt=(1,), ckpt_slot=0, out_slot=1),
    Request(P=4, m=2, q_len=(1,), n_opt=(1,), ckpt_slot=-1, out_slot=1),
    Request(P=4, m=0, q_len=(0,), n_opt=(1,), out_slot=1),
])
def test_invalid_requests_rejected(bad):
    with pytest.raises(ValueError):
        layout.build_layout([bad])


def test_window_rule():
    # W keys including the query itself
    assert layout.visible(0, 0, 10, 0, 0, 10, window=1)
    assert not layout.visible(0, 0, 10, 0, 0, 9, window=1)
    assert layout.visible(0, 0, 10, 0, 0, 7, window=4)
    assert not layout.visible(0, 0, 10, 0, 0, 6, window=4)
    # other request / sibling branch / future key
    assert not layout.visible(0, 1, 10, 1, 0, 3)
    assert not layout.visible(0, 1, 10, 0, 2, 9)
    assert not layout.visible(0, 0, 10, 0, 0, 11)
    assert layout.visible(0, 2, 10, 0, 0, 9)


def _R(rows):
    return Request(P=rows, m=0, q_len=(), n_opt=(), out_slot=0)


def test_split_rule():
    reqs = [_R(30), _R(30), _R(50), _R(100), _R(10), _R(95)]
    first, eager = layout.split_round(reqs, 64)
    # [30, 30] | [50] | [100] eager | [10] | [95] eager
    assert first == [0, 2, 3, 4, 5, 6]
    assert eager == [False, False, True, False, True]
    first, eager = layout.split_round(reqs, 1000)
    assert first == [0, 6] and eager == [False]
    assert layout.split_round([], 64) == ([0], [])


def test_split_fan_out_round_three_replays():
    # 16 requests of ~10.7k rows at capacity 65536 split 6 + 6 + 4
    reqs = [Request(P=8192, m=0, q_len=(40,) * 64, n_opt=(2,) * 64, out_slot=j) for j in range(16)]
    first, eager = layout.split_round(reqs, 65536)
    assert first == [0, 6, 12, 16] and eager == [False] * 3
