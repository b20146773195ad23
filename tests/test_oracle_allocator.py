"""Pins of the segment allocator model (CPU): hand-worked sequences whose segments follow from
the policy by hand, and invariants that hold after every operation of long random sequences
(checked with plain slot counting, not with the model's own bookkeeping)."""
import numpy as np
import pytest

from oracle.allocator import AllocatorModel


def test_hand_worked_extend_best_fit_and_failure():
    a = AllocatorModel(10)
    assert a.grow(1, 3) and a.segments(1) == [(0, 3)]
    assert a.grow(2, 2) and a.segments(2) == [(3, 2)]
    # slot 3 (after request 1's end) is taken: the new tokens go to the only free run
    assert a.grow(1, 2) and a.segments(1) == [(0, 3), (5, 2)]
    a.release(2)
    assert a.free_runs() == [(3, 2), (7, 3)]
    # slot 7 follows request 1's last segment: extended in place
    assert a.grow(1, 1) and a.segments(1) == [(0, 3), (5, 3)]
    # two runs of 2 left, (3, 2) and (8, 2): the lower one
    assert a.grow(3, 2) and a.segments(3) == [(3, 2)]
    # 2 free slots, 3 asked: fails and changes nothing
    before = (a.used.copy(), {k: a.segments(k) for k in (1, 3)})
    assert not a.grow(4, 3)
    assert np.array_equal(a.used, before[0]) and {k: a.segments(k) for k in (1, 3)} == before[1]
    assert a.segments(4) == []


def test_hand_worked_largest_first_split():
    a = AllocatorModel(12)
    for r, n in ((1, 2), (2, 1), (3, 3), (4, 1), (5, 5)):
        assert a.grow(r, n)
    assert a.free_tokens() == 0
    for r in (1, 3, 5):
        a.release(r)
    assert a.free_runs() == [(0, 2), (3, 3), (7, 5)]
    # 9 tokens: no run holds them; the largest (7, 5) whole, then (3, 3) whole, then the best
    # fit for the last token, (0, 2), from its start
    assert a.grow(6, 9) and a.segments(6) == [(7, 5), (3, 3), (0, 1)]
    assert a.free_runs() == [(1, 1)]


def test_hand_worked_truncate_and_tables():
    a = AllocatorModel(16)
    assert a.grow(7, 5) and a.grow(8, 2) and a.grow(7, 4)
    assert a.segments(7) == [(0, 5), (7, 4)]
    a.truncate(7, 3)  # drops the 4 keys of (7, 4) and 2 of (0, 5)
    assert a.segments(7) == [(0, 3)]
    assert a.free_runs() == [(3, 2), (7, 9)]
    segs, ind, cu = a.tables([8, 99, 7])
    assert segs.tolist() == [[5, 2], [0, 3]]
    assert ind.tolist() == [0, 1, 1, 2] and cu.tolist() == [0, 2, 2, 5]
    a.truncate(7, 0)
    assert a.segments(7) == [] and a.free_tokens() == 14


def _check_invariants(a: AllocatorModel, lengths):
    owner = np.full(a.pool_tokens, -1)
    for r, segs in a.segs.items():
        total = 0
        for off, ln in segs:
            assert ln > 0 and 0 <= off and off + ln <= a.pool_tokens
            assert (owner[off:off + ln] == -1).all(), "two segments share a slot"
            owner[off:off + ln] = r
            total += ln
        assert total == lengths.get(r, 0)
    assert np.array_equal(owner >= 0, a.used)
    assert a.free_tokens() == a.pool_tokens - sum(lengths.values())
    # free runs are maximal, disjoint and cover exactly the unused slots
    cover = np.zeros(a.pool_tokens, dtype=bool)
    for s, ln in a.free_runs():
        assert ln > 0 and not cover[s:s + ln].any()
        cover[s:s + ln] = True
        assert s == 0 or a.used[s - 1]
        assert s + ln == a.pool_tokens or a.used[s + ln]
    assert np.array_equal(cover, ~a.used)


@pytest.mark.parametrize("seed", range(4))
def test_random_sequences_keep_the_invariants(seed):
    rng = np.random.default_rng(seed)
    a = AllocatorModel(400)
    lengths = {}
    for _ in range(600):
        op = rng.random()
        r = int(rng.integers(0, 12))
        if op < 0.6:
            n = int(rng.integers(0, 60))
            free = a.free_tokens()
            ok = a.grow(r, n)
            assert ok == (n <= free)
            if ok:
                lengths[r] = lengths.get(r, 0) + n
        elif op < 0.8:
            a.release(r)
            lengths.pop(r, None)
        else:
            keep = int(rng.integers(0, lengths.get(r, 0) + 1))
            a.truncate(r, keep)
            if r in lengths:
                lengths[r] = keep
        _check_invariants(a, lengths)
    for r in list(a.segs):
        a.release(r)
    assert a.free_runs() == [(0, 400)]


def test_in_place_extension_is_taken_whenever_possible():
    rng = np.random.default_rng(9)
    a = AllocatorModel(300)
    for step in range(300):
        r = int(rng.integers(0, 6))
        if rng.random() < 0.25:
            a.release(r)
            continue
        segs = a.segments(r)
        n = int(rng.integers(1, 20))
        if not segs or n > a.free_tokens():
            a.grow(r, n)
            continue
        end = segs[-1][0] + segs[-1][1]
        room = 0
        while end + room < a.pool_tokens and not a.used[end + room]:
            room += 1
        assert a.grow(r, n)
        after = a.segments(r)
        # the old last segment grew by min(n, room) and nothing else changed before it
        assert after[:len(segs) - 1] == segs[:-1]
        assert after[len(segs) - 1] == (segs[-1][0], segs[-1][1] + min(n, room))
