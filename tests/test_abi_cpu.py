"""C ABI checks that need no GPU: exported symbols, the host planner and the split rule.

The planner's metadata must equal the oracle's independent builder bit for bit
(stream order, (j, c, t) labels, state indices, question-final rows).
"""
import os
import re
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import layout as olayout
from tree_forked_hybrid_amd import flide as F
from workloads import Request, make_round

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flide.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(flide_[a-z_]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = F.load_library()
    declared = _declared_functions()
    assert len(declared) >= 18
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(ln.split()[-1] for ln in out.splitlines() if ln.strip())
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    # the binding wraps exactly the declared entry points
    assert sorted(F.exported_names()) == declared


def test_error_queries_without_a_context():
    """The error queries answer for a NULL context (no GPU needed): no message, no HIP error; entry points
    that need a context refuse NULL before touching anything."""
    lib = F.load_library()
    assert F.flide_last_hip_error(None) == 0
    assert lib.flide_last_error(None) == b""
    assert lib.flide_graph_release(None, 0) == F.FLIDE_E_INVALID_ARG
    assert lib.flide_select_bucket(None, 1, 1, 0, None) == F.FLIDE_E_INVALID_ARG


def test_status_strings_and_version():
    lib = F.load_library()
    for s in range(7):
        assert lib.flide_status_string(s)
    assert lib.flide_status_string(99) == b"unknown status"
    assert "gfx950" in F.flide_version()


def _planner_layout(reqs, caps):
    img = F.flide_plan_round(reqs, caps)
    return F.decode_image(img, caps)


def _assert_same_layout(reqs, caps):
    got = _planner_layout(reqs, caps)
    ref = olayout.build_layout(reqs)
    for key in ("T", "R", "n_seg", "n_qst"):
        assert got[key] == ref[key], key
    for key in ("seg_row0", "seg_len", "seg_req", "seg_branch", "seg_pos0", "seg_state", "req_trunk_row0",
                "req_q_seg0", "qfin_row"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    np.testing.assert_array_equal(got["req_P"], [r.P for r in reqs])
    np.testing.assert_array_equal(got["req_m"], [r.m for r in reqs])
    np.testing.assert_array_equal(got["req_nq"], [len(r.q_len) for r in reqs])
    # the tile list covers every row of every segment exactly once: tiles of four units of up to 8 rows
    # aligned to their segment's start; a trunk tile is 32 consecutive rows of its trunk (aligned to its
    # start), a question tile holds units of questions of one request, packed in question order
    cover = np.zeros(ref["T"], np.int32)
    n_qtiles = {}
    for segs, rows in zip(got["tile_seg"], got["tile_row0"]):
        if segs[0] == -1:  # unused position
            assert (segs == -1).all()
            continue
        used = [(int(s), int(r0)) for s, r0 in zip(segs, rows) if s != -1]
        assert [s for s in segs if s != -1] == [s for s, _ in used] and all(segs[:len(used)] != -1)
        assert len({int(ref["seg_req"][s]) for s, _ in used}) == 1
        trunk = ref["seg_branch"][used[0][0]] == 0
        for u, (s, r0) in enumerate(used):
            a = r0 - ref["seg_row0"][s]
            assert a % 8 == 0 and 0 <= a < ref["seg_len"][s]
            n = min(8, ref["seg_len"][s] - a)
            cover[r0:r0 + n] += 1
            if trunk:
                assert s == used[0][0] and a == (used[0][1] - ref["seg_row0"][s]) + 8 * u
        if trunk:
            assert (used[0][1] - ref["seg_row0"][used[0][0]]) % 32 == 0
        else:
            assert all(ref["seg_branch"][s] > 0 for s, _ in used)
            j = int(ref["seg_req"][used[0][0]])
            n_qtiles[j] = n_qtiles.get(j, 0) + 1
    assert (cover == 1).all()
    for j in range(ref["R"]):  # packing: ceil(question units / 4) tiles per request
        lens = [int(ref["seg_len"][s]) for s in range(ref["n_seg"]) if ref["seg_req"][s] == j and ref["seg_branch"][s] > 0]
        units = sum((n + 7) // 8 for n in lens)
        assert n_qtiles.get(j, 0) == (units + 3) // 4
    # the windowed layer's order: every used position exactly once, nothing else
    used_pos = sorted(int(x) for x in range(len(got["tile_seg"])) if got["tile_seg"][x][0] >= 0)
    swa = [int(x) for x in got["tile_swa"] if x >= 0]
    assert sorted(swa) == used_pos
    # the GDN work list: trunks then questions, each a permutation ordered by length (longest first,
    # ties in stream order)
    R, n_seg = ref["R"], ref["n_seg"]
    order = got["gdn_order"]
    for lo, hi in ((0, R), (R, n_seg)):
        part = order[lo:hi]
        np.testing.assert_array_equal(np.sort(part), np.arange(lo, hi))
        keys = [(-int(ref["seg_len"][s]), int(s)) for s in part]
        assert keys == sorted(keys)
    return got


@pytest.mark.parametrize("config", [0, 1, 2, 4])
def test_planner_matches_oracle_on_workloads(config):
    rnd = make_round(config, 0)
    T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
    caps = F.caps_of(T + 5, len(rnd.requests), sum(len(r.q_len) for r in rnd.requests))
    got = _assert_same_layout(rnd.requests, caps)
    assert got["max_pos"] == max(r.P + max(r.q_len) for r in rnd.requests)


@pytest.mark.parametrize("config,group", [(0, 0), (1, 0), (2, 0), (4, 64)])
def test_planner_attention_work_order(config, group):
    # Rounds whose tiles see >= 4096 keys on average (agent-resume: 30,720 cached keys per request)
    # take the tile-group order; the short and long-document rounds keep the default order.
    rnd = make_round(config, 0)
    T = sum((r.P - r.m) + sum(r.q_len) for r in rnd.requests)
    caps = F.caps_of(T + 5, len(rnd.requests), sum(len(r.q_len) for r in rnd.requests))
    got = _planner_layout(rnd.requests, caps)
    assert got["tile_group"] == group


def test_planner_worked_example_tiles():
    rnd = make_round(0, 0)
    got = _planner_layout(rnd.requests, F.caps_of(69, 1, 3))
    # the three questions (rows 48-52, 53-59, 60-68) packed into one tile of four units (57 keys for its
    # last row), then the trunk tile 32..47 (48 keys), then 0..31
    used = got["tile_seg"][:, 0] >= 0
    rows = [[int(r) for s, r in zip(ss, rr) if s >= 0] for ss, rr in zip(got["tile_seg"][used], got["tile_row0"][used])]
    assert rows == [[48, 53, 60, 68], [32, 40], [0, 8, 16, 24]]


_req = st.builds(
    lambda P, m_frac, qs, slot: (P, min(P, int(P * m_frac)), qs, slot),
    st.integers(0, 70), st.sampled_from([0.0, 0.0, 0.5, 1.0]),
    st.lists(st.integers(1, 40), min_size=0, max_size=5), st.integers(0, 3))


@settings(max_examples=60, deadline=None)
@given(st.lists(_req, min_size=1, max_size=6))
def test_planner_matches_oracle_random(raw):
    reqs = []
    for j, (P, m, qs, _) in enumerate(raw):
        reqs.append(Request(P=P, m=m, q_len=tuple(qs), n_opt=(2,) * len(qs),
                            ckpt_slot=(100 + j if m > 0 else -1), out_slot=j))
    T = sum((r.P - r.m) + sum(r.q_len) for r in reqs)
    caps = F.caps_of(max(T, 1), len(reqs), max(1, sum(len(r.q_len) for r in reqs)))
    _assert_same_layout(reqs, caps)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(0, 120), min_size=0, max_size=12), st.integers(1, 150))
def test_split_matches_oracle(rows, t_max):
    reqs = [Request(P=r, m=0, q_len=(), n_opt=(), out_slot=j) for j, r in enumerate(rows)]
    assert F.flide_split_round(reqs, t_max) == olayout.split_round(reqs, t_max)


@pytest.mark.parametrize("bad", [
    [Request(P=4, m=5, q_len=(1,), n_opt=(1,), ckpt_slot=0, out_slot=1)],
    [Request(P=4, m=2, q_len=(1,), n_opt=(1,), ckpt_slot=-1, out_slot=1)],
    [Request(P=4, m=2, q_len=(1,), n_opt=(1,), ckpt_slot=1, out_slot=1)],
    [Request(P=4, m=0, q_len=(0,), n_opt=(1,), out_slot=1)],
    [Request(P=4, m=0, q_len=(1,), n_opt=(1,), out_slot=-1)],
    [Request(P=4, m=0, q_len=(), n_opt=(), out_slot=1), Request(P=3, m=0, q_len=(), n_opt=(), out_slot=1)],
    [Request(P=4, m=2, q_len=(), n_opt=(), ckpt_slot=5, out_slot=1),
     Request(P=3, m=0, q_len=(), n_opt=(), out_slot=5)],
    # interior checkpoints: position outside (m, P], off a chunk boundary, no slot, slot collisions
    [Request(P=200, m=64, q_len=(), n_opt=(), ckpt_slot=0, out_slot=1, save_m=64, save_slot=2)],
    [Request(P=200, m=0, q_len=(), n_opt=(), out_slot=1, save_m=201, save_slot=2)],
    [Request(P=200, m=0, q_len=(), n_opt=(), out_slot=1, save_m=100, save_slot=2)],
    [Request(P=200, m=0, q_len=(), n_opt=(), out_slot=1, save_m=128, save_slot=-1)],
    [Request(P=200, m=0, q_len=(), n_opt=(), out_slot=1, save_m=128, save_slot=1)],
    [Request(P=200, m=64, q_len=(), n_opt=(), ckpt_slot=2, out_slot=1, save_m=128, save_slot=2)],
    [Request(P=200, m=0, q_len=(), n_opt=(), out_slot=1, save_m=128, save_slot=3),
     Request(P=200, m=0, q_len=(), n_opt=(), out_slot=2, save_m=64, save_slot=3)],
    [Request(P=200, m=0, q_len=(), n_opt=(), out_slot=1, save_m=128, save_slot=3),
     Request(P=200, m=64, q_len=(), n_opt=(), ckpt_slot=3, out_slot=2)],
])
def test_planner_rejects_invalid_rounds(bad):
    caps = F.caps_of(512, 4, 4)
    image = np.full(F.flide_meta_layout_for(caps).host_words, 7, np.int32)
    with pytest.raises(F.FlideError) as e:
        F.flide_plan_round(bad, caps, image)
    assert e.value.status == F.FLIDE_E_INVALID_ARG
    assert (image == 7).all()  # untouched on error


def test_planner_capacity_errors():
    reqs = [Request(P=40, m=0, q_len=(10, 10), n_opt=(2, 2), out_slot=0)]
    for caps in (F.caps_of(59, 1, 2), F.caps_of(60, 1, 1)):
        with pytest.raises(F.FlideError) as e:
            F.flide_plan_round(reqs, caps)
        assert e.value.status == F.FLIDE_E_CAPACITY
    F.flide_plan_round(reqs, F.caps_of(60, 1, 2))


def test_layout_rejects_bad_capacity():
    for caps in (F.caps_of(0, 1, 1), F.caps_of(10, 0, 1), F.caps_of(10, 1, -1)):
        with pytest.raises(F.FlideError):
            F.flide_meta_layout_for(caps)


def test_planner_interior_checkpoints():
    """save_m / save_slot reach the metadata per request (0 / -1 where no checkpoint is made); a
    checkpoint off the chunk grid is accepted only at the trunk's end."""
    reqs = [Request(P=300, m=0, q_len=(3,), n_opt=(2,), out_slot=0, save_m=256, save_slot=4),
            Request(P=90, m=0, q_len=(), n_opt=(), out_slot=1),
            Request(P=200, m=64, q_len=(2,), n_opt=(2,), ckpt_slot=2, out_slot=3, save_m=200, save_slot=5)]
    caps = F.caps_of(1024, 4, 4)
    d = F.decode_image(F.flide_plan_round(reqs, caps), caps)
    assert d["req_save_m"].tolist() == [256, 0, 200]
    assert d["req_save_slot"].tolist() == [4, -1, 5]
    assert d["req_ckpt"].tolist() == [-1, -1, 2]


def test_host_code_under_sanitizers(tmp_path):
    """The planner and the checkpoint store built with AddressSanitizer and UndefinedBehaviorSanitizer
    (plain g++, host code only) run thousands of seeded rounds, valid and broken, into images of exactly
    the size their layout names, and random store operation sequences, without a finding."""
    import shutil
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path / "sanitize_host")
    srcs = [os.path.join(ROOT, "tree_forked_hybrid_amd", "csrc", f) for f in ("plan.cpp", "store.cpp")]
    srcs.append(os.path.join(ROOT, "tests", "sanitize_host.cpp"))
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include")]
    res = subprocess.run([gxx, *flags, *srcs, "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    # verify_asan_link_order=0: the runtime need not come first when the environment preloads a library
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "3000"], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "sanitized host run" in run.stdout
    print(run.stdout.strip())
