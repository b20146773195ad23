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


def test_hand_worked_granule():
    a = AllocatorModel(20, granule=4)
    assert a.grow(1, 1) and a.owned(1) == [(0, 4)] and a.segments(1) == [(0, 1)]
    assert a.grow(2, 1) and a.owned(2) == [(4, 4)]
    # spare capacity first: no new range
    assert a.grow(1, 3) and a.owned(1) == [(0, 4)] and a.segments(1) == [(0, 4)]
    # one more key: slot 4 is request 2's, so a new range of 4 from the best (only) run
    assert a.grow(1, 1) and a.owned(1) == [(0, 4), (8, 4)] and a.segments(1) == [(0, 4), (8, 1)]
    # 8 slots free; a shortfall of 7 rounds up to 8 = all of them; one more fails
    assert a.grow(3, 7) and a.owned(3) == [(12, 8)] and a.segments(3) == [(12, 7)]
    assert a.free_tokens() == 0 and a.grow(3, 1) and not a.grow(3, 1)
    # rounding is dropped when it does not fit: 1 free slot, shortfall 1
    a.release(2)
    assert a.grow(4, 3) and a.owned(4) == [(4, 4)] and a.segments(4) == [(4, 3)]


def test_hand_worked_reserve():
    a = AllocatorModel(20)
    assert a.reserve(5, 10) and a.owned(5) == [(0, 10)] and a.segments(5) == []
    assert a.tables([5])[2].tolist() == [0, 0]
    assert a.grow(5, 3) and a.segments(5) == [(0, 3)] and a.owned(5) == [(0, 10)]
    assert a.grow(6, 4) and a.owned(6) == [(10, 4)]
    # 7 spare slots, 8 asked: one more slot, slot 10 is taken, so from the only free run
    assert a.grow(5, 8) and a.segments(5) == [(0, 10), (14, 1)]
    # reserving less than the capacity changes nothing; more than the free slots fails
    assert a.reserve(5, 4) and a.owned(5) == [(0, 10), (14, 1)]
    assert not a.reserve(5, 11 + 6) and a.owned(5) == [(0, 10), (14, 1)]
    # truncation frees spare capacity too
    a.truncate(5, 2)
    assert a.owned(5) == [(0, 2)] and a.free_runs() == [(2, 8), (14, 6)]
    # truncating to more than the keys keeps everything
    assert a.reserve(5, 6) and a.owned(5) == [(0, 6)]
    a.truncate(5, 5)
    assert a.owned(5) == [(0, 6)] and a.length(5) == 2


def _check_invariants(a: AllocatorModel, lengths):
    owner = np.full(a.pool_tokens, -1)
    for r, segs in a.segs.items():
        total = 0
        for off, ln in segs:
            assert ln > 0 and 0 <= off and off + ln <= a.pool_tokens
            assert (owner[off:off + ln] == -1).all(), "two segments share a slot"
            owner[off:off + ln] = r
            total += ln
        assert total == a.capacity(r) >= lengths.get(r, 0)
        assert sum(ln for _, ln in a.segments(r)) == lengths.get(r, 0)
        if a.granule == 1 and r not in a.reserved:
            assert total == lengths.get(r, 0)
    assert np.array_equal(owner >= 0, a.used)
    assert a.free_tokens() == a.pool_tokens - sum(a.capacity(r) for r in a.segs)
    # free runs are maximal, disjoint and cover exactly the unused slots
    cover = np.zeros(a.pool_tokens, dtype=bool)
    for s, ln in a.free_runs():
        assert ln > 0 and not cover[s:s + ln].any()
        cover[s:s + ln] = True
        assert s == 0 or a.used[s - 1]
        assert s + ln == a.pool_tokens or a.used[s + ln]
    assert np.array_equal(cover, ~a.used)


@pytest.mark.parametrize("seed,granule,reserve", [(0, 1, False), (1, 1, False), (2, 1, True),
                                                  (3, 8, False), (4, 8, True), (5, 64, True)])
def test_random_sequences_keep_the_invariants(seed, granule, reserve):
    rng = np.random.default_rng(seed)
    a = AllocatorModel(400, granule=granule)
    a.reserved = set()
    lengths = {}
    for _ in range(600):
        op = rng.random()
        r = int(rng.integers(0, 12))
        if op < 0.5 or (op < 0.6 and not reserve):
            n = int(rng.integers(0, 60))
            short = lengths.get(r, 0) + n - a.capacity(r)
            free = a.free_tokens()
            ok = a.grow(r, n)
            assert ok == (short <= free)
            if ok:
                lengths[r] = lengths.get(r, 0) + n
        elif op < 0.6:
            c = int(rng.integers(0, 120))
            ok = a.reserve(r, c)
            assert ok == (c - a.capacity(r) <= a.free_tokens()) or not ok
            if ok:
                a.reserved.add(r)
                lengths.setdefault(r, 0)
                assert a.capacity(r) >= c
        elif op < 0.8:
            a.release(r)
            lengths.pop(r, None)
            a.reserved.discard(r)
        else:
            keep = int(rng.integers(0, lengths.get(r, 0) + 1))
            a.truncate(r, keep)
            if r in lengths:
                if keep < lengths[r]:
                    a.reserved.discard(r)
                lengths[r] = keep
        _check_invariants(a, lengths)
    for r in list(a.segs):
        a.release(r)
    assert a.free_runs() == [(0, 400)]


def test_granule_bounds_the_segments_of_interleaved_growth():
    # 32 requests growing one key at a time in turn: with granule G each request gets a new
    # range at most every G keys
    for g in (1, 16, 64):
        a = AllocatorModel(32 * 300, granule=g)
        for _ in range(160):
            for r in range(32):
                assert a.grow(r, 1)
        worst = max(len(a.segments(r)) for r in range(32))
        assert worst <= -(-160 // g)
        if g == 1:
            assert worst == 160  # every neighbour blocks in-place growth


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


# ---------------------------------------------------------------- compaction

from oracle.allocator import apply_moves


def test_compaction_hand_worked():
    # A: [0,3) then [6,8); B: [3,6) then [8,10); free [10,20). Both have two ranges, so A goes
    # first (lower id) into [10,15), B into the rest [15,20); the old ranges free [0,10).
    a = AllocatorModel(20)
    assert a.grow(1, 3) and a.grow(2, 3) and a.grow(1, 2) and a.grow(2, 2)
    assert a.owned(1) == [(0, 3), (6, 2)] and a.owned(2) == [(3, 3), (8, 2)]
    moves = a.compact()
    assert moves == [(0, 10, 3), (6, 13, 2), (3, 15, 3), (8, 18, 2)]
    assert a.owned(1) == [(10, 5)] and a.owned(2) == [(15, 5)]
    assert a.free_runs() == [(0, 10)]
    assert a.compact() == []  # nothing fragmented any more


def test_compaction_leaves_requests_that_fit_nowhere_and_copies_keys_only():
    # free space of 2 slots: neither 5-slot request fits, nothing changes
    a = AllocatorModel(12)
    assert a.grow(1, 3) and a.grow(2, 3) and a.grow(1, 2) and a.grow(2, 2)
    before = (a.owned(1), a.owned(2), a.free_runs())
    assert a.compact() == []
    assert (a.owned(1), a.owned(2), a.free_runs()) == before
    # a request with 3 ranges goes before one with 2; spare capacity is not copied; a request
    # with capacity but no keys moves without any copy
    a = AllocatorModel(40)
    assert a.grow(1, 2) and a.grow(2, 2) and a.grow(1, 2) and a.grow(2, 2) and a.grow(1, 2)
    # 1: [0,2) [4,6) [8,10); 2: [2,4) [6,8); free [10,40)
    assert a.reserve(1, 9)  # 3 more slots for request 1: in place after [8,10) -> [8,13)
    assert a.owned(1) == [(0, 2), (4, 2), (8, 5)] and a.length(1) == 6
    assert a.reserve(3, 2) and a.reserve(2, 4) is True  # 3 takes [13,15)
    assert a.grow(4, 1) and a.reserve(3, 3)  # 4 takes [15,16); 3 gets [16,17) as a 2nd range
    assert a.owned(3) == [(13, 2), (16, 1)] and a.length(3) == 0
    moves = a.compact()
    # 1 (3 ranges, capacity 9) -> [17, 26): copies its 6 keys; then 2 -> [26, 30); then 3 ->
    # [30, 33) with nothing to copy
    assert moves == [(0, 17, 2), (4, 19, 2), (8, 21, 2), (2, 26, 2), (6, 28, 2)]
    assert a.owned(1) == [(17, 9)] and a.owned(2) == [(26, 4)] and a.owned(3) == [(30, 3)]
    assert a.segments(1) == [(17, 6)] and a.length(3) == 0


def test_compaction_keeps_every_key_and_moves_only_between_disjoint_ranges():
    rng = np.random.default_rng(21)
    for trial in range(30):
        pool = int(rng.integers(200, 600))
        a = AllocatorModel(pool, granule=int(rng.choice([1, 4, 16])))
        for _ in range(int(rng.integers(20, 120))):
            r = int(rng.integers(0, 10))
            op = rng.random()
            if op < 0.7:
                a.grow(r, int(rng.integers(0, 25)))
            elif op < 0.8:
                a.reserve(r, int(rng.integers(0, 60)))
            elif op < 0.9:
                a.release(r)
            else:
                a.truncate(r, int(rng.integers(0, a.length(r) + 1)))
        # label every key slot with (request, key index); other slots -1
        label = np.full(pool, -1, dtype=np.int64)
        reqs = sorted(a.segs)
        for r in reqs:
            i = 0
            for off, ln in a.segments(r):
                label[off:off + ln] = r * 10000 + np.arange(i, i + ln)
                i += ln
        used_before = a.used.copy()
        frag_before = {r: len(a.owned(r)) for r in reqs}
        caps = {r: a.capacity(r) for r in reqs}
        moves = a.compact()
        # destinations lie in space that was free; sources in space that was owned; no two
        # ranges of the list (sources and destinations together) share a slot
        cover = np.zeros(pool, dtype=np.int64)
        for src, dst, n in moves:
            assert not used_before[dst:dst + n].any() and used_before[src:src + n].all()
            cover[src:src + n] += 1
            cover[dst:dst + n] += 1
        assert cover.max(initial=0) <= 1
        after = apply_moves(label, moves)
        for r in reqs:
            assert a.capacity(r) == caps[r]
            got = np.concatenate([after[o:o + n] for o, n in a.segments(r)] or [np.zeros(0, np.int64)])
            assert np.array_equal(got, r * 10000 + np.arange(a.length(r)))
            if len(a.owned(r)) > 1:  # not relocated: it fitted nowhere, or had one range
                assert frag_before[r] == len(a.owned(r))
        # the bitmap still equals the union of the owned ranges
        owned = np.zeros(pool, dtype=bool)
        for r in reqs:
            for o, n in a.owned(r):
                assert not owned[o:o + n].any()
                owned[o:o + n] = True
        assert np.array_equal(owned, a.used)
