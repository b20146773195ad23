"""The debug library (SEG_ATTN_DEBUG, libsegattn_debug.so) on the GPU: with good tables its
prefill and decode results are bitwise those of the release library; with tables that would make
a kernel resolve a pool slot outside [0, pool_tokens) it returns SEG_ATTN_ERR_TABLE and launches
nothing (the output buffer keeps its sentinel).

The broken-table cases are only ever given to the debug library, and their pool tensors are views
of larger allocations, so even a read past pool_tokens would stay inside allocated memory."""
import os

import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

sa = pytest.importorskip("attention_segmented_kv_amd")
ERR_TABLE = 5


@pytest.fixture
def use(monkeypatch):
    if not os.path.exists(sa.library_path("debug")):
        pytest.skip("libsegattn_debug.so not built")

    def switch(variant):
        monkeypatch.setattr(sa, "_lib", sa.load_library(variant))
    yield switch


def _padded_pool(t: torch.Tensor, extra: int = 64) -> torch.Tensor:
    """t's rows followed by `extra` spare rows in one allocation; returns the view of t's rows."""
    big = torch.zeros((t.shape[0] + extra, *t.shape[1:]), dtype=t.dtype, device=t.device)
    big[: t.shape[0]] = t
    return big[: t.shape[0]]


def _prefill(w, **kw):
    return sa.prefill(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_q, w.cu_seqlens_k,
                      w.max_seqlen_q, w.max_seqlen_k, causal=True, **kw)


@needs_gpu
def test_debug_prefill_is_bitwise_the_release_prefill(use):
    print("[case] debug library prefill vs release", flush=True)
    w = wl.make_random(41, batch=3, q_lens=[40, 1, 130], k_lens=[100, 64, 130], max_segs=4).to("cuda")
    use("release")
    ref = _prefill(w)
    torch.cuda.synchronize()
    use("debug")
    got = _prefill(w)
    torch.cuda.synchronize()
    assert sa._load().seg_attn_debug_build() == 1
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@needs_gpu
def test_debug_prefill_refuses_a_segment_past_the_pool(use):
    print("[case] debug library prefill, segment past pool_tokens", flush=True)
    w = wl.make_random(42, batch=2, q_lens=[20, 30], k_lens=[70, 50], max_segs=2).to("cuda")
    w.k_pool = _padded_pool(w.k_pool)
    w.v_pool = _padded_pool(w.v_pool)
    pool_tokens = w.k_pool.shape[0]
    segs = w.segs.clone()
    n = int(segs[-1, 1])
    segs[-1, 0] = pool_tokens - n + 3  # the last segment's last 3 slots lie past the pool
    w.segs = segs
    out = torch.full_like(w.q, 7.0)
    use("debug")
    with pytest.raises(sa.SegAttnError) as e:
        _prefill(w, out=out)
    torch.cuda.synchronize()
    assert e.value.status == ERR_TABLE
    assert bool((out == 7.0).all())


@needs_gpu
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_debug_decode_is_bitwise_the_release_decode(use, kv):
    print(f"[case] debug library decode vs release, {kv}", flush=True)
    w = wl.make_random(43, batch=4, q_lens=[1] * 4, k_lens=[900, 33, 2100, 64], max_segs=4,
                       kv_dtype=kv, kind="decode").to("cuda")
    kw = dict(k_scale=w.k_scale, v_scale=w.v_scale) if kv != "bf16" else {}
    res = {}
    for variant in ("release", "debug"):
        use(variant)
        res[variant] = (
            sa.decode(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_k, w.max_seqlen_k, **kw),
            sa.decode_noalloc(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_k, w.max_seqlen_k,
                              **kw))
        torch.cuda.synchronize()
    for a, b in zip(res["release"], res["debug"]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@needs_gpu
def test_debug_decode_refuses_key_counts_that_disagree_with_the_segments(use):
    print("[case] debug library decode, K_b above its segments' total", flush=True)
    w = wl.make_random(44, batch=3, q_lens=[1] * 3, k_lens=[300, 40, 500], max_segs=3, kind="decode").to("cuda")
    w.k_pool = _padded_pool(w.k_pool)
    w.v_pool = _padded_pool(w.v_pool)
    ck = w.cu_seqlens_k.clone()
    ck[2:] += 5  # request 1 claims 5 keys more than its segments hold
    out = torch.full_like(w.q, 7.0)
    use("debug")
    for fn in (sa.decode, sa.decode_noalloc):
        with pytest.raises(sa.SegAttnError) as e:
            fn(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, ck, w.max_seqlen_k + 5, out=out)
        torch.cuda.synchronize()
        assert e.value.status == ERR_TABLE
        assert bool((out == 7.0).all())
