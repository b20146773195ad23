"""The library's segment allocator (host C++, through the C ABI) against the allocator model:
identical segments for every request and identical free runs after every operation of random
grow / release / truncate sequences, plus its error handling. Host only: no GPU needed."""
import ctypes
import os

import numpy as np
import pytest

from oracle.allocator import AllocatorModel

sa = pytest.importorskip("attention_segmented_kv_amd")


@pytest.fixture(autouse=True)
def _needs_lib():
    if not os.path.exists(sa.library_path()):
        pytest.skip("libsegattn.so not built")


def _same_state(lib_alloc, model, requests):
    segs, ind, cu = lib_alloc.tables(requests)
    ms, mi, mc = model.tables(requests)
    assert np.array_equal(segs.astype(np.int64).reshape(-1, 2), ms)
    assert np.array_equal(ind.astype(np.int64), mi) and np.array_equal(cu.astype(np.int64), mc)
    runs = lib_alloc.free_runs().astype(np.int64).tolist()
    assert [tuple(r) for r in runs] == model.free_runs()
    st = lib_alloc.stats()
    assert st["free_tokens"] == model.free_tokens()
    mr = model.free_runs()
    assert st["free_runs"] == len(mr)
    assert st["largest_free_run"] == max([ln for _, ln in mr], default=0)


@pytest.mark.parametrize("seed,pool,nreq,maxn,granule", [(0, 500, 8, 40, 1), (1, 2000, 30, 200, 1),
                                                         (2, 64, 5, 30, 1), (3, 3000, 100, 12, 1),
                                                         (4, 2000, 20, 30, 16), (5, 4000, 40, 5, 64),
                                                         (6, 300, 6, 50, 7)])
def test_matches_the_model_on_random_sequences(seed, pool, nreq, maxn, granule):
    rng = np.random.default_rng(seed)
    a = sa.SegmentAllocator(pool, granule=granule)
    m = AllocatorModel(pool, granule=granule)
    reqs = list(range(nreq)) + [10 ** 12, -5]  # ids are any int64
    for step in range(800):
        op = rng.random()
        r = reqs[int(rng.integers(0, len(reqs)))]
        if op < 0.55:
            n = int(rng.integers(0, maxn + 1))
            ok = m.grow(r, n)
            if ok:
                a.grow(r, n)
            else:
                with pytest.raises(sa.SegAttnError) as e:
                    a.grow(r, n)
                assert e.value.status == 6
        elif op < 0.6:
            c = int(rng.integers(0, 3 * maxn + 1))
            ok = m.reserve(r, c)
            if ok:
                a.reserve(r, c)
            else:
                with pytest.raises(sa.SegAttnError) as e:
                    a.reserve(r, c)
                assert e.value.status == 6
        elif op < 0.8:
            m.release(r)
            a.release(r)
        elif op < 0.97:
            keep = int(rng.integers(0, m.length(r) + 2))
            m.truncate(r, keep)
            a.truncate(r, keep)
        else:
            # compaction: the same moves (src, dst, length) in the same order, `first` their
            # running sum
            mm = m.compact()
            am = a.compact()
            assert am.shape == (len(mm), 4)
            assert [tuple(x) for x in am[:, :3].tolist()] == mm
            assert am[:, 3].tolist() == np.concatenate([[0], np.cumsum(am[:, 2])])[:-1].tolist()
            _same_state(a, m, reqs)
        assert a.length(r) == m.length(r) and a.capacity(r) == m.capacity(r)
        if step % 10 == 0 or step > 780:
            _same_state(a, m, reqs)
    a.close()


def test_decode_style_growth_segments():
    # 64 requests with 100-key prompts, then 50 one-token steps in turn. Exact growth: each
    # neighbour blocks the next in-place extension, one new segment per token. A granule of 32:
    # the prompt gets 128 slots, so the 50 tokens need one more range. Reserving prompt + 50 up
    # front: one segment each.
    for granule, reserve, worst in ((1, False, 51), (32, False, 2), (1, True, 1)):
        a = sa.SegmentAllocator(64 * 200, granule=granule)
        m = AllocatorModel(64 * 200, granule=granule)
        for r in range(64):
            if reserve:
                a.reserve(r, 150)
                m.reserve(r, 150)
            a.grow(r, 100)
            m.grow(r, 100)
        for _ in range(50):
            for r in range(64):
                a.grow(r, 1)
                m.grow(r, 1)
        _same_state(a, m, list(range(64)))
        segs, ind, cu = a.tables(list(range(64)))
        assert int(np.diff(ind).max()) == worst and int(cu[-1]) == 64 * 150


def test_grow_many_equals_grows_in_order():
    rng = np.random.default_rng(21)
    a = sa.SegmentAllocator(3000, granule=16)
    m = AllocatorModel(3000, granule=16)
    reqs = list(range(25))
    for step in range(60):
        ids = [int(x) for x in rng.choice(reqs, size=int(rng.integers(1, 25)), replace=False)]
        ns = [int(x) for x in rng.integers(0, 30, size=len(ids))]
        done = 0
        for r, n in zip(ids, ns):
            if not m.grow(r, n):
                break
            done += 1
        if done == len(ids):
            a.grow_many(ids, ns)
        else:
            with pytest.raises(sa.SegAttnError) as e:
                a.grow_many(ids, ns)
            assert e.value.status == 6 and e.value.done == done
        if step % 7 == 3:
            for r in ids[: len(ids) // 2]:
                a.release(r)
                m.release(r)
        _same_state(a, m, reqs)


def test_errors_and_edge_cases():
    lib = sa._load()
    P = ctypes.c_void_p
    h = P()
    assert lib.seg_attn_allocator_create(-1, 1, ctypes.byref(h)) == 1
    assert lib.seg_attn_allocator_create(2 ** 31, 1, ctypes.byref(h)) == 1
    assert lib.seg_attn_allocator_create(10, 0, ctypes.byref(h)) == 1
    assert lib.seg_attn_allocator_create(10, 1, None) == 1
    assert lib.seg_attn_allocator_capacity(None, 0) == -1
    assert lib.seg_attn_allocator_grow(None, 0, 1) == 1
    assert lib.seg_attn_allocator_length(None, 0) == -1
    a = sa.SegmentAllocator(0)
    a.grow(1, 0)  # nothing to place, always fits
    with pytest.raises(sa.SegAttnError):
        a.grow(1, 1)
    assert a.tables([1])[0].shape == (0, 2) and a.free_runs().shape == (0, 2)
    a = sa.SegmentAllocator(20)
    with pytest.raises(sa.SegAttnError):
        a.grow(1, -1)
    with pytest.raises(sa.SegAttnError):
        a.truncate(1, -1)
    with pytest.raises(sa.SegAttnError):
        a.reserve(1, -1)
    a.release(42)        # unknown id: no-op
    a.truncate(42, 3)    # unknown id: no-op
    a.grow(7, 20)
    assert a.stats() == {"free_tokens": 0, "largest_free_run": 0, "free_runs": 0, "requests": 1}
    # tables into a too small buffer: status 3, the count is reported, nothing else written
    req = np.array([7], dtype=np.int64)
    ind = np.full(2, -9, dtype=np.int32)
    cu = np.full(2, -9, dtype=np.int32)
    n = ctypes.c_int64(0)
    st = lib.seg_attn_allocator_tables(a._h, req.ctypes.data, 1, None, 0, ind.ctypes.data,
                                       cu.ctypes.data, ctypes.byref(n))
    assert st == 3 and n.value == 1 and (ind == -9).all() and (cu == -9).all()
    a.close()
    a.close()  # twice is harmless


def test_tables_feed_validate_tables():
    rng = np.random.default_rng(11)
    a = sa.SegmentAllocator(5000)
    for _ in range(300):
        r = int(rng.integers(0, 40))
        if rng.random() < 0.75:
            try:
                a.grow(r, int(rng.integers(1, 80)))
            except sa.SegAttnError:
                pass
        else:
            a.release(r)
    reqs = list(range(40))
    segs, ind, cu = a.tables(reqs)
    assert sa.validate_tables(segs, ind, cu, 5000, causal=False) == (0, -1)


def test_compaction_reports_the_moves_it_needs_and_changes_nothing_without_room():
    a = sa.SegmentAllocator(20)
    m = AllocatorModel(20)
    for r, n in ((1, 3), (2, 3), (1, 2), (2, 2)):
        a.grow(r, n)
        m.grow(r, n)
    lib = sa._load()
    cnt = ctypes.c_int64(-1)
    moves = np.zeros((3, 4), dtype=np.int32)  # 4 needed
    st = lib.seg_attn_allocator_compact(a._h, moves.ctypes.data, 3, ctypes.byref(cnt))
    assert st == 3 and cnt.value == 4
    _same_state(a, m, [1, 2])  # unchanged
    got = a.compact()
    assert got.tolist() == [[0, 10, 3, 0], [6, 13, 2, 3], [3, 15, 3, 5], [8, 18, 2, 8]]
    m.compact()
    _same_state(a, m, [1, 2])
    assert lib.seg_attn_allocator_compact(None, None, 0, None) == 1
