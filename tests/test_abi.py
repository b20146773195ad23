"""Host-side checks of the C ABI: the library loads, exports every symbol the header declares,
and rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seg_attn.h")

sa = pytest.importorskip("attention_segmented_kv_amd")


def _lib():
    if not os.path.exists(sa.library_path()):
        pytest.skip("libsegattn.so not built")
    return sa._load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(seg_attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("seg_attn_prefill", "seg_attn_decode", "seg_attn_kv_append", "seg_attn_decode_workspace_bytes",
              "seg_attn_decode_num_splits", "seg_attn_status_string", "seg_attn_validate_tables",
              "seg_attn_version"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    lib = _lib()
    raw = ctypes.CDLL(sa.library_path())
    for s in declared_symbols():
        assert hasattr(raw, s), f"{s} not exported"


@pytest.mark.parametrize("variant,flag", [("release", 0), ("debug", 1)])
def test_both_library_variants_load_and_say_which_they_are(variant, flag):
    """The release and the debug (SEG_ATTN_DEBUG) libraries both export the whole header and
    report their variant; they share every argument check."""
    if not os.path.exists(sa.library_path(variant)):
        pytest.skip(f"{variant} library not built")
    lib = sa.load_library(variant)
    raw = ctypes.CDLL(sa.library_path(variant))
    for s in declared_symbols():
        assert hasattr(raw, s), f"{s} not exported by the {variant} library"
    assert lib.seg_attn_debug_build() == flag
    assert lib.seg_attn_version() == sa.load_library("release").seg_attn_version()
    # an argument error is still caught before anything else (no table read, no launch)
    P = None
    assert lib.seg_attn_prefill(P, P, P, P, P, P, P, 1, 8, 8, 64, 8, 128, 100, 0.1, 1, P, P, P) == 1
    assert lib.seg_attn_version() == 10000


def test_status_strings():
    _lib()
    assert sa.status_string(0) == "ok"
    for st in range(1, 6):
        assert sa.status_string(st) not in ("ok", "unknown status")
    assert sa.status_string(99) == "unknown status"


def _prefill_args(**over):
    # nonzero, suitably aligned stand-ins for device pointers: every case is rejected (or is a
    # no-op) before anything is launched
    a = dict(q=256, k=256, v=256, segs=8, ind=4, cq=4, ck=4, batch=1, mq=4, mk=4, hq=64, hkv=8, d=128,
             pool=16, scale=0.1, causal=1, out=256, lse=None, stream=None)
    a.update(over)
    return [a[k] for k in ("q", "k", "v", "segs", "ind", "cq", "ck", "batch", "mq", "mk", "hq", "hkv",
                           "d", "pool", "scale", "causal", "out", "lse", "stream")]


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(segs=None), 1), (dict(batch=-1), 1),
    (dict(mq=-3), 1), (dict(d=64), 2), (dict(hq=32), 2), (dict(hq=60), 1), (dict(hkv=0), 1),
    (dict(causal=2), 1), (dict(mq=8, mk=4), 1), (dict(scale=float("nan")), 1), (dict(pool=-1), 1),
    (dict(scale=0.0), 1), (dict(scale=-0.1), 1),
])
def test_prefill_rejects_bad_arguments(over, status):
    lib = _lib()
    assert lib.seg_attn_prefill(*_prefill_args(**over)) == status


@pytest.mark.parametrize("over", [
    dict(q=264), dict(k=258), dict(v=260), dict(out=264), dict(segs=12), dict(ind=6), dict(cq=2),
    dict(ck=3), dict(lse=6), dict(q=256 + 8, lse=4),
])
def test_prefill_rejects_misaligned_buffers(over):
    """Q, K/V pool and output rows move as 16-byte pieces, segment records are 8 bytes, table
    entries and LSE values 4 bytes: a pointer that breaks its alignment is rejected."""
    lib = _lib()
    assert lib.seg_attn_prefill(*_prefill_args(**over)) == 1


def test_prefill_empty_batch_is_a_noop():
    lib = _lib()
    assert lib.seg_attn_prefill(*_prefill_args(batch=0, q=None, out=None)) == 0


def _decode_args(**over):
    a = dict(q=256, k=256, v=256, ks=None, vs=None, kvd=0, segs=8, ind=4, ck=4, batch=2, mk=100,
             hq=64, hkv=8, d=128, pool=16, scale=0.1, ns=1, out=256, lse=None, ws=None, wsb=0,
             stream=None)
    a.update(over)
    return [a[k] for k in ("q", "k", "v", "ks", "vs", "kvd", "segs", "ind", "ck", "batch", "mk", "hq",
                           "hkv", "d", "pool", "scale", "ns", "out", "lse", "ws", "wsb", "stream")]


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(kvd=7), 1), (dict(kvd=1), 1), (dict(kvd=1, ks=1), 1), (dict(d=96), 2),
    (dict(ns=-1), 1), (dict(mk=-1), 1), (dict(ns=4), 3), (dict(ns=4, ws=1, wsb=16), 3),
    (dict(ns=0), 3), (dict(ns=1), 3), (dict(kvd=2), 1), (dict(kvd=2, vs=1), 1), (dict(kvd=3), 1),
    (dict(scale=0.0), 1), (dict(scale=-0.1), 1), (dict(scale=float("inf")), 1),
])
def test_decode_rejects_bad_arguments(over, status):
    lib = _lib()
    assert lib.seg_attn_decode(*_decode_args(**over)) == status


@pytest.mark.parametrize("over,status", [
    (dict(q=264), 1), (dict(k=260), 1), (dict(v=257), 1), (dict(out=260), 1), (dict(segs=4), 1),
    (dict(ck=2), 1), (dict(lse=2), 1), (dict(kvd=1, ks=2, vs=4), 1), (dict(kvd=2, ks=4, vs=6), 1),
    (dict(kvd=1, k=256 + 8, ks=4, vs=4), 1), (dict(ws=264, wsb=1 << 40), 3),
])
def test_decode_rejects_misaligned_buffers(over, status):
    """Q and pool rows are copied as 16-byte pieces, scales as 4-byte words, the output is
    written 8 bytes at a time and the workspace holds 16-byte records: a pointer that breaks its
    alignment is rejected (a misaligned workspace as a workspace error)."""
    lib = _lib()
    assert lib.seg_attn_decode(*_decode_args(**over)) == status


def _append_args(**over):
    # nonzero, suitably aligned stand-ins for device pointers: every case is rejected (or is a
    # no-op) before anything is launched
    a = dict(kn=256, vn=256, segs=1, ind=1, cn=1, ck=1, batch=2, tn=5, hkv=8, d=128, pool=16, kvd=0,
             kp=256, vp=256, ks=None, vs=None, stream=None)
    a.update(over)
    return [a[k] for k in ("kn", "vn", "segs", "ind", "cn", "ck", "batch", "tn", "hkv", "d", "pool", "kvd",
                           "kp", "vp", "ks", "vs", "stream")]


@pytest.mark.parametrize("over,status", [
    (dict(kn=None), 1), (dict(vp=None), 1), (dict(cn=None), 1), (dict(batch=-1), 1), (dict(tn=-2), 1),
    (dict(hkv=0), 1), (dict(pool=-1), 1), (dict(kvd=3), 1), (dict(kvd=1), 1), (dict(kvd=1, ks=1), 1),
    (dict(d=64), 2), (dict(pool=2 ** 31), 2), (dict(batch=0), 1),
    (dict(kn=16 + 8), 1), (dict(kp=2), 1), (dict(kvd=1, ks=4, vs=6, kp=8, vp=16), 1),
    (dict(kvd=2), 1), (dict(kvd=2, ks=4, vs=8, kp=4, vp=8), 1),
    (dict(vn=264), 1),
])
def test_kv_append_rejects_bad_arguments(over, status):
    lib = _lib()
    assert lib.seg_attn_kv_append(*_append_args(**over)) == status


def test_kv_append_without_new_tokens_is_a_noop():
    lib = _lib()
    assert lib.seg_attn_kv_append(*_append_args(tn=0, kn=None, vn=None, kp=None, vp=None)) == 0
    assert lib.seg_attn_kv_append(*_append_args(batch=0, tn=0)) == 0


def _linear_args(**over):
    a = dict(q=256, k=256, v=256, g=256, cu=1, slots=1, batch=2, maxl=100, h=16, d=128, scale=0.1,
             init=1, pool=256, npool=4, out=256, ws=None, wsb=0, stream=None)
    a.update(over)
    return [a[k] for k in ("q", "k", "v", "g", "cu", "slots", "batch", "maxl", "h", "d", "scale",
                           "init", "pool", "npool", "out", "ws", "wsb", "stream")]


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(pool=None), 1), (dict(cu=None), 1), (dict(batch=-1), 1), (dict(h=0), 1),
    (dict(d=64), 2), (dict(init=2), 1), (dict(scale=float("inf")), 1), (dict(npool=-1), 1),
    (dict(k=264), 1), (dict(out=260), 1), (dict(batch=0), 0), (dict(maxl=-1), 1),
    # the workspace is checked where it is used: requests longer than the closed form's 4096
    (dict(ws=512, wsb=1024, maxl=5000), 3), (dict(ws=520, wsb=1 << 40, maxl=5000), 1),
])
def test_linear_prefill_rejects_bad_arguments(over, status):
    lib = _lib()
    assert lib.seg_attn_linear_prefill(*_linear_args(**over)) == status


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(slots=None), 1), (dict(d=96), 2), (dict(h=-3), 1), (dict(v=8), 1),
    (dict(batch=0, q=None), 0),
])
def test_linear_decode_rejects_bad_arguments(over, status):
    lib = _lib()
    a = _linear_args(**over)
    del a[15:17]  # no workspace
    del a[11]     # no initial_state
    del a[7]      # no max_seqlen
    del a[4]      # no cu_seqlens
    assert lib.seg_attn_linear_decode(*a) == status


def test_linear_prefill_workspace_size():
    _lib()
    lib = sa._load()
    # dS^T fp32 + S_before^T bf16 per (request, chunk, head), plus one float each
    n = lib.seg_attn_linear_prefill_workspace_bytes(2, 1024, 16, 128)
    assert n >= 2 * 16 * 16 * (128 * 128 * 6 + 4)
    assert lib.seg_attn_linear_prefill_workspace_bytes(2, 1024, 16, 64) == 0


def test_split_plan_and_workspace_size():
    _lib()
    n, ln = sa.decode_num_splits(4, 1000, 8, sa.KV_BF16, 4)
    assert n == 4 and ln == 256 and ln % 64 == 0 and n * ln >= 1000
    n, ln = sa.decode_num_splits(4, 1000, 8, sa.KV_BF16, 1)
    assert n == 1 and ln >= 1000
    n, ln = sa.decode_num_splits(4, 100, 8, sa.KV_BF16, 1000)  # clamped to 64-key splits
    assert n == 2 and ln == 64
    for bsz, mk, kvd in ((128, 8192, 0), (16, 131072, 1), (1, 50, 0), (3, 0, 0)):
        n, ln = sa.decode_num_splits(bsz, mk, 8, kvd, 0)
        assert n >= 1 and ln % 64 == 0 and n * ln >= mk and (n - 1) * ln < max(mk, 1)
        ws = sa.decode_workspace_bytes(bsz, mk, 64, 8, 128, kvd, 0)
        # plan header + chunk offsets + chunk records + one (O, LSE) partial per chunk and head
        assert ws >= 256 + (bsz + 1) * 4 + bsz * n * 64 + bsz * 64 * n * (128 + 1) * 4
    assert sa.decode_workspace_bytes(4, 1000, 64, 8, 64, 0, 4) == 0  # unsupported head dim
    # one-byte formats share the plan: FP8 and INT8 chunks are at least 1024 keys
    assert sa.decode_num_splits(16, 131072, 8, sa.KV_INT8, 0) == sa.decode_num_splits(16, 131072, 8, sa.KV_FP8_E4M3, 0)
    assert sa.decode_num_splits(16, 131072, 8, sa.KV_INT8, 0)[1] == 1024
    assert sa.decode_workspace_bytes(16, 131072, 64, 8, 128, sa.KV_INT8, 0) == \
        sa.decode_workspace_bytes(16, 131072, 64, 8, 128, sa.KV_FP8_E4M3, 0)
    assert sa.decode_workspace_bytes(16, 1000, 64, 8, 128, 3, 0) == 0


def test_validate_tables_accepts_good_and_flags_bad():
    _lib()
    import workloads as wl
    w = wl.make_random(3, batch=3, q_lens=[2, 5, 1], k_lens=[9, 20, 4], max_segs=4, num_heads_q=8,
                       num_heads_kv=1, head_dim=8, zero_length_segments=True)
    segs, ind, cq, ck = wl.host_tables(w)
    st, bad = sa.validate_tables(segs, ind, ck, w.pool_tokens, cu_seqlens_q=cq)
    assert (st, bad) == (0, -1)
    # a request's lengths no longer add up
    ck2 = ck.copy(); ck2[2:] += 1
    assert sa.validate_tables(segs, ind, ck2, w.pool_tokens, cu_seqlens_q=cq)[0] == 5
    # a segment out of the pool
    s2 = segs.copy(); s2[0, 0] = w.pool_tokens
    assert sa.validate_tables(s2, ind, ck, w.pool_tokens, cu_seqlens_q=cq) == (5, 0)
    # two segments overlapping
    nz = [i for i in range(len(segs)) if segs[i, 1] > 0]
    s3 = segs.copy(); s3[nz[1], 0] = s3[nz[0], 0]
    assert sa.validate_tables(s3, ind, ck, w.pool_tokens, cu_seqlens_q=cq)[0] == 5
    # causal with more queries than keys
    cq2 = np.array([0, 2, 7, 12])
    assert sa.validate_tables(segs, ind, ck, w.pool_tokens, cu_seqlens_q=cq2) == (5, 2)
    assert sa.validate_tables(segs, ind, ck, w.pool_tokens, cu_seqlens_q=cq2, causal=False)[0] == 0


def test_decode_noalloc_rejects_bad_arguments_and_calls_beyond_its_scratch():
    """The no-allocation decode takes seg_attn_decode's arguments minus the workspace and checks
    them the same way; a call whose plan needs more than its fixed 64 MiB scratch is refused with
    SEG_ATTN_ERR_SCRATCH before anything is launched."""
    lib = _lib()
    a = _decode_args()
    del a[19:21]  # no workspace, no workspace size
    ok = list(a)
    assert lib.seg_attn_decode_noalloc(*[None if i == 0 else x for i, x in enumerate(ok)]) == 1  # q NULL
    bad = list(ok); bad[13] = 96  # head_dim
    assert lib.seg_attn_decode_noalloc(*bad) == 2
    bad = list(ok); bad[0] = 264  # misaligned q
    assert lib.seg_attn_decode_noalloc(*bad) == 1
    big = list(ok); big[10] = 64 * 100_000; big[16] = 100_000  # max_seqlen_k, num_splits
    assert lib.seg_attn_decode_noalloc(*big) == 7
    assert "scratch" in sa.status_string(7)


def _move_args(**over):
    a = dict(moves=256, n=3, total=10, hkv=8, d=128, pool=100, kvd=0, kp=256, vp=256, ks=None, vs=None,
             stream=None)
    a.update(over)
    return [a[k] for k in ("moves", "n", "total", "hkv", "d", "pool", "kvd", "kp", "vp", "ks", "vs", "stream")]


@pytest.mark.parametrize("over,status", [
    (dict(moves=None), 1), (dict(n=-1), 1), (dict(total=-1), 1), (dict(hkv=0), 1), (dict(d=64), 2),
    (dict(kvd=5), 1), (dict(kvd=1), 1), (dict(kp=None), 1), (dict(total=101), 1), (dict(moves=264), 1),
    (dict(kp=264), 1), (dict(kvd=1, ks=4, vs=6, kp=8, vp=8), 1), (dict(pool=2 ** 31), 1),
    (dict(n=0, moves=None), 0), (dict(total=0), 0),
])
def test_kv_move_rejects_bad_arguments(over, status):
    lib = _lib()
    assert lib.seg_attn_kv_move(*_move_args(**over)) == status
