"""Prefix-match checkpoint store (host only): a request resumes at m only from a checkpoint whose prefix
matches its own up to m (Korean summary §어떻게 쓰나).  Checked against a plain Python model of the same
rules on random operation sequences, plus worked cases."""
import pytest
from hypothesis import given, settings, strategies as st

from tree_forked_hybrid_amd import flide as F


class Model:
    """The store's rules written out plainly: slots hold (m, digest, refs, committed, last use)."""

    def __init__(self, first, n):
        self.first, self.n = first, n
        self.slots = [None] * n   # None or dict(m, d, refs, vis, t)
        self.t = 0

    def lookup(self, cands):
        best = (0, -1)
        for m, d in cands:
            for k, e in enumerate(self.slots):
                if e and e["vis"] and e["m"] == m and e["d"] == d and m > best[0]:
                    best = (m, self.first + k)
        if best[1] >= 0:
            e = self.slots[best[1] - self.first]
            e["refs"] += 1
            self.t += 1
            e["t"] = self.t
        return best

    def reserve(self, m, d):
        for e in self.slots:
            if e and e["m"] == m and e["d"] == d:
                return "invalid"
        free = [k for k, e in enumerate(self.slots) if e is None]
        if free:
            k = free[0]
        else:
            cand = [k for k, e in enumerate(self.slots) if e["vis"] and e["refs"] == 0]
            if not cand:
                return "capacity"
            k = min(cand, key=lambda k: self.slots[k]["t"])
        self.t += 1
        self.slots[k] = {"m": m, "d": d, "refs": 1, "vis": False, "t": self.t}
        return self.first + k

    def commit(self, slot):
        k = slot - self.first
        if not 0 <= k < self.n or self.slots[k] is None or self.slots[k]["vis"]:
            return "invalid"
        self.slots[k]["vis"] = True
        return None

    def release(self, slot):
        k = slot - self.first
        if not 0 <= k < self.n or self.slots[k] is None or self.slots[k]["refs"] < 1:
            return "invalid"
        e = self.slots[k]
        e["refs"] -= 1
        if not e["vis"] and e["refs"] == 0:
            self.slots[k] = None
        return None


def _status(fn):
    try:
        return fn()
    except F.FlideError as e:
        return {F.FLIDE_E_INVALID_ARG: "invalid", F.FLIDE_E_CAPACITY: "capacity"}[e.status]


ops = st.lists(st.one_of(
    st.tuples(st.just("lookup"), st.lists(st.tuples(st.integers(1, 6), st.integers(0, 2)), max_size=4)),
    st.tuples(st.just("reserve"), st.tuples(st.integers(1, 6), st.integers(0, 2))),
    st.tuples(st.just("commit"), st.integers(0, 6)),
    st.tuples(st.just("release"), st.integers(0, 6)),
), max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops, st.integers(1, 4))
def test_store_matches_model(seq, n):
    first = 2
    store, model = F.CheckpointStore(first, n), Model(first, n)
    for op, arg in seq:
        if op == "lookup":
            pos = [m for m, _ in arg]
            dig = [d for _, d in arg]
            assert store.lookup(pos, dig) == model.lookup(arg)
        elif op == "reserve":
            assert _status(lambda: store.reserve(*arg)) == model.reserve(*arg)
        elif op == "commit":
            assert _status(lambda: store.commit(first + arg - 1)) == model.commit(first + arg - 1)
        else:
            assert _status(lambda: store.release(first + arg - 1)) == model.release(first + arg - 1)
        st_ = store.stats()
        assert st_["used"] == sum(e is not None for e in model.slots)
        assert st_["committed"] == sum(bool(e and e["vis"]) for e in model.slots)
        assert st_["held"] == sum(bool(e and e["refs"] > 0) for e in model.slots)
    store.close()


def test_store_worked_case():
    """Two slots: a checkpoint at 256 and one at 512 of the same document; a request sharing 300 tokens
    resumes at 256, one sharing all 600 at 512; a third prefix evicts the least recently used entry that
    no round holds; a held entry is never evicted."""
    s = F.CheckpointStore(10, 2)
    a = s.reserve(256, 0xAAA)
    assert s.lookup([256], [0xAAA]) == (0, -1)          # invisible until committed
    s.commit(a)
    s.release(a)
    b = s.reserve(512, 0xBBB)
    s.commit(b)
    s.release(b)
    assert {a, b} == {10, 11}
    assert s.lookup([64, 256], [0x1, 0xAAA]) == (256, a)  # longest match among the candidates
    s.release(a)
    assert s.lookup([256, 512], [0xAAA, 0xBBB]) == (512, b)
    s.release(b)
    # both unheld; a was used least recently -> evicted for a new prefix
    c = s.reserve(128, 0xCCC)
    assert c == a
    assert s.lookup([256], [0xAAA]) == (0, -1)
    assert s.stats()["evictions"] == 1
    # c is held (reserved, not committed) and b is held by a lookup: no slot can be reserved
    assert s.lookup([512], [0xBBB]) == (512, b)
    with pytest.raises(F.FlideError) as e:
        s.reserve(64, 0xDDD)
    assert e.value.status == F.FLIDE_E_CAPACITY
    with pytest.raises(F.FlideError):
        s.reserve(512, 0xBBB)                             # already stored
    s.release(c)                                          # abandoned reservation frees its slot
    assert s.stats()["used"] == 1
    with pytest.raises(F.FlideError):
        s.release(c)
    s.close()


def test_store_rejects_bad_arguments():
    with pytest.raises(F.FlideError):
        F.CheckpointStore(-1, 4)
    with pytest.raises(F.FlideError):
        F.CheckpointStore(0, 0)
    s = F.CheckpointStore(0, 2)
    with pytest.raises(F.FlideError):
        s.lookup([0], [1])                                # positions start at 1
    with pytest.raises(F.FlideError):
        s.reserve(0, 1)
    with pytest.raises(F.FlideError):
        s.commit(5)                                       # not a slot of this store
    s.close()
