"""GPU parity: the HIP library (through the C ABI) against the CPU float64 oracle.

Every case, the full-size workloads included, is compared element by element over every output
and every LSE; the full-size workloads run in the launch configuration the benchmark times.
Properties that hold at any size (determinism, re-layout invariance, split agreement) are checked
on top.
Bar: max abs error <= 2e-2 and RMS <= 2e-3 on bf16 outputs; LSE within 1e-3.
"""
import time

import numpy as np
import pytest
import torch

import workloads as wl
from tests import _helpers as H

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


@pytest.fixture(params=["auto", "128", "256"])
def prefill_tile(request, monkeypatch):
    """Run a prefill test with the library's automatic tiling and with each tiling forced."""
    if request.param != "auto":
        monkeypatch.setenv("SEG_ATTN_PREFILL_TILE", request.param)
    else:
        monkeypatch.delenv("SEG_ATTN_PREFILL_TILE", raising=False)
    return request.param


def _report(name, mx, rms):
    print(f"[parity] {name}: max_abs={mx:.3e} rms={rms:.3e}", flush=True)


def _full_compare(w, name, num_splits=0):
    out, lse = H.run_gpu(w, num_splits=num_splits)
    torch.cuda.synchronize()
    o_ref, l_ref = H.oracle_full(w)
    got = out.float().cpu().numpy()
    mx, rms = H.assert_close(got, o_ref, name)
    H.assert_lse_close(lse.cpu().numpy(), l_ref, name)
    _report(name, mx, rms)
    return out, lse


# ---------------------------------------------------------------- the named workloads

@needs_gpu
def test_config1_tiny_prefill_full(prefill_tile):
    print("[case] config 1 tiny prefill", flush=True)
    w = wl.make_config(1).to("cuda")
    _full_compare(w, "config1")


@needs_gpu
def test_config2_prefill_1k_full(prefill_tile):
    print("[case] config 2 prefill 1024", flush=True)
    w = wl.make_config(2).to("cuda")
    _full_compare(w, "config2")


# The oracle's result for a named workload, computed once per session: the three prefill
# tilings of config 3 are compared against the same reference.
_REF = {}


def _oracle_cached(w, key):
    if key not in _REF:
        t0 = time.perf_counter()
        _REF[key] = H.oracle_full(w)
        print(f"[oracle] {key}: {time.perf_counter() - t0:.1f} s", flush=True)
    return _REF[key]


def _full_compare_named(w, key, name):
    """Every output element and every LSE of a full-size workload against the oracle, in the
    launch configuration the benchmark times (automatic split count)."""
    out, lse = H.run_gpu(w)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    got_l = lse.cpu().numpy()
    del out, lse
    o_ref, l_ref = _oracle_cached(w, key)
    mx, rms = H.assert_close(got, o_ref, name)
    H.assert_lse_close(got_l, l_ref, name)
    _report(f"{name} (all {got.shape[0] * got.shape[1]} rows)", mx, rms)


@needs_gpu
@pytest.mark.timeout(900)
def test_config3_chunked_prefill_full(prefill_tile):
    print(f"[case] config 3 chunked prefill, every row (tiling {prefill_tile})", flush=True)
    w = wl.make_config(3, device="cuda")
    _full_compare_named(w, "config3", "config3")


@needs_gpu
@pytest.mark.timeout(600)
def test_config4_decode_full():
    print("[case] config 4 decode bf16, every row", flush=True)
    w = wl.make_config(4, device="cuda")
    _full_compare_named(w, "config4", "config4")


@needs_gpu
@pytest.mark.timeout(900)
def test_config5_fp8_decode_full():
    print("[case] config 5 decode fp8, every row", flush=True)
    w = wl.make_config(5, device="cuda")
    _full_compare_named(w, "config5", "config5")
    _REF.pop("config5", None)


@needs_gpu
@pytest.mark.timeout(900)
def test_config6_int8_decode_full():
    print("[case] config 6 decode int8, every row", flush=True)
    w = wl.make_config(6, device="cuda")
    _full_compare_named(w, "config6", "config6")
    _REF.pop("config6", None)


# ---------------------------------------------------------------- ragged and edge cases

RAGGED_PREFILL = [
    # (seed, q_lens, k_lens, causal, max_segs)
    (11, [1], [1], True, 1),
    (12, [17], [17], True, 3),
    (13, [5, 33, 70], [5, 100, 70], True, 4),
    (14, [300, 1, 64], [300, 900, 129], True, 8),
    (15, [16, 15, 47], [16, 200, 333], True, 2),
    (16, [7, 40], [3, 80], False, 4),
    (17, [0, 20, 0, 9], [10, 20, 0, 9], True, 3),
]


@needs_gpu
@pytest.mark.parametrize("case", RAGGED_PREFILL, ids=[f"seed{c[0]}" for c in RAGGED_PREFILL])
def test_prefill_ragged_full(case, prefill_tile):
    seed, ql, kl, causal, ms = case
    print(f"[case] ragged prefill seed={seed} q={ql} k={kl} causal={causal}", flush=True)
    w = wl.make_random(seed, batch=len(ql), q_lens=ql, k_lens=kl, max_segs=ms, causal=causal,
                       zero_length_segments=(seed % 2 == 1)).to("cuda")
    _full_compare(w, f"ragged-prefill-{seed}")


@needs_gpu
def test_prefill_noncausal_empty_keys_gives_zero_and_neg_inf_lse(prefill_tile):
    print("[case] non-causal prefill with K=0", flush=True)
    w = wl.make_random(18, batch=2, q_lens=[3, 4], k_lens=[0, 7], causal=False).to("cuda")
    out, lse = _full_compare(w, "empty-keys")
    assert (out[:3].float() == 0).all() and torch.isneginf(lse[:3]).all()


@needs_gpu
def test_prefill_small_heads_multiple_kv_heads(prefill_tile):
    print("[case] prefill Hq=16 Hkv=2", flush=True)
    w = wl.make_random(19, batch=2, q_lens=[40, 9], k_lens=[50, 130], num_heads_q=16,
                       num_heads_kv=2).to("cuda")
    _full_compare(w, "hq16-hkv2")


RAGGED_DECODE = [
    # (seed, k_lens, max_segs, kv_dtype, num_splits)
    (21, [1, 2, 63, 64, 65], 3, "bf16", 0),
    (22, [700, 1, 4097, 31], 8, "bf16", 0),
    (23, [700, 1, 4097, 31], 8, "bf16", 1),
    (24, [700, 1, 4097, 31], 8, "bf16", 7),
    (25, [0, 5, 0], 2, "bf16", 0),
    (26, [1, 100, 2000, 9000], 6, "fp8_e4m3", 0),
    (27, [1, 100, 2000, 9000], 6, "fp8_e4m3", 1),
    (28, [3000, 129], 8, "fp8_e4m3", 5),
    (29, [1, 100, 2000, 9000], 6, "int8", 0),
    (30, [3000, 129, 64], 8, "int8", 5),
    (31, [0, 7, 1500], 3, "int8", 1),
]


@needs_gpu
@pytest.mark.parametrize("case", RAGGED_DECODE, ids=[f"seed{c[0]}" for c in RAGGED_DECODE])
def test_decode_ragged_full(case):
    seed, kl, ms, kvd, ns = case
    print(f"[case] ragged decode seed={seed} k={kl} {kvd} splits={ns}", flush=True)
    w = wl.make_random(seed, batch=len(kl), q_lens=[1] * len(kl), k_lens=kl, max_segs=ms,
                       kv_dtype=kvd, kind="decode", zero_length_segments=(seed % 2 == 0)).to("cuda")
    _full_compare(w, f"ragged-decode-{seed}", num_splits=ns)


@needs_gpu
@pytest.mark.parametrize("batch,kvd", [(512, "bf16"), (513, "bf16"), (700, "fp8_e4m3"), (600, "int8")])
def test_decode_large_batches(batch, kvd):
    """The decode plan spreads each request's chunks over several threads up to 512 requests and
    walks them one thread per request above that: both sides of the boundary, short requests in
    up to 3 segments, the chunk length forced small so that most requests have several chunks."""
    print(f"[case] large-batch decode B={batch} {kvd}", flush=True)
    kl = [int(x) for x in np.random.default_rng(40 + batch).integers(1, 200, size=batch)]
    w = wl.make_random(40 + batch, batch=batch, q_lens=[1] * batch, k_lens=kl, max_segs=3,
                       kv_dtype=kvd, kind="decode").to("cuda")
    _full_compare(w, f"decode-B{batch}", num_splits=4)


PLAN_PATH_CASES = [
    # (seed, k_lens, max_segs, kv_dtype): more than 8 segments per request (the in-workgroup
    # plan reads a request's segments 8 at a time), empty segments, 1-key requests
    (51, [5000, 1, 3000, 64, 12000, 0, 777], 20, "bf16"),
    (52, [40000, 3, 9000, 513], 30, "fp8_e4m3"),
    (53, [1, 2, 3, 20000, 4096, 4097], 12, "int8"),
]


@needs_gpu
@pytest.mark.parametrize("case", PLAN_PATH_CASES, ids=[f"seed{c[0]}" for c in PLAN_PATH_CASES])
def test_decode_plan_in_workgroup_matches_plan_kernel(case, monkeypatch):
    """With the automatic chunk length, batches of up to 256 requests are planned inside the
    split workgroups; the separate plan launch (SEG_ATTN_DECODE_PLAN=kernel) makes the same
    chunks, so outputs and LSE agree bit for bit, for both decode entry points. The oracle
    checks the in-workgroup result."""
    import attention_segmented_kv_amd as sa
    seed, kl, ms, kvd = case
    print(f"[case] decode plan paths seed={seed} k={kl} {kvd}", flush=True)
    w = wl.make_random(seed, batch=len(kl), q_lens=[1] * len(kl), k_lens=kl, max_segs=ms,
                       kv_dtype=kvd, kind="decode", zero_length_segments=True).to("cuda")
    kw = dict(k_scale=w.k_scale, v_scale=w.v_scale) if kvd != "bf16" else {}
    res = {}
    for path in ("workgroup", "kernel"):
        if path == "kernel":
            monkeypatch.setenv("SEG_ATTN_DECODE_PLAN", "kernel")
        else:
            monkeypatch.delenv("SEG_ATTN_DECODE_PLAN", raising=False)
        res[path] = [f(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_k, w.max_seqlen_k,
                       return_lse=True, **kw)
                     for f in (sa.decode, sa.decode_noalloc)]
        torch.cuda.synchronize()
    monkeypatch.delenv("SEG_ATTN_DECODE_PLAN", raising=False)
    for (oa, la), (ob, lb) in zip(res["workgroup"], res["kernel"]):
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
    _full_compare(w, f"plan-paths-{seed}")


@needs_gpu
@pytest.mark.parametrize("batch", [256, 257])
def test_decode_automatic_plan_at_the_batch_limit(batch):
    """256 requests are planned in the workgroups, 257 by the plan kernel: both against the
    oracle, with the automatic chunk length."""
    print(f"[case] automatic decode plan B={batch}", flush=True)
    kl = [int(x) for x in np.random.default_rng(60 + batch).integers(1, 3000, size=batch)]
    w = wl.make_random(60 + batch, batch=batch, q_lens=[1] * batch, k_lens=kl, max_segs=3,
                       kind="decode").to("cuda")
    _full_compare(w, f"decode-auto-B{batch}")


# ---------------------------------------------------------------- invariants on the device

@needs_gpu
def test_prefill_is_bitwise_deterministic_and_layout_invariant(prefill_tile):
    print("[case] determinism + re-layout", flush=True)
    w = wl.make_random(31, batch=2, q_lens=[100, 37], k_lens=[250, 37], max_segs=1).to("cuda")
    o1 = H.run_gpu(w, return_lse=False)
    o2 = H.run_gpu(w, return_lse=False)
    assert torch.equal(o1, o2)
    # same logical keys re-laid out as many segments elsewhere in a larger pool
    rng = np.random.default_rng(5)
    segs, ind, cq, ck = wl.host_tables(w)
    lens = [wl.cut_lengths(rng, int(ck[b + 1] - ck[b]), 9) for b in range(2)]
    flat = [l for s in lens for l in s]
    pool = 2000
    offs = wl.place_segments(rng, flat, pool)
    kp = torch.full((pool, 8, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = kp.clone()
    si = 0
    for b in range(2):
        src = np.concatenate([np.arange(o, o + n) for o, n in segs[ind[b]:ind[b + 1]].tolist()])
        st = 0
        for n in lens[b]:
            kp[offs[si]:offs[si] + n] = w.k_pool[torch.as_tensor(src[st:st + n], device="cuda")]
            vp[offs[si]:offs[si] + n] = w.v_pool[torch.as_tensor(src[st:st + n], device="cuda")]
            st += n
            si += 1
    import attention_segmented_kv_amd as sa
    new_segs = torch.tensor([[o, n] for o, n in zip(offs, flat)], dtype=torch.int32, device="cuda")
    new_ind = torch.tensor(np.concatenate([[0], np.cumsum([len(s) for s in lens])]), dtype=torch.int32,
                           device="cuda")
    o3 = sa.prefill(w.q, kp, vp, new_segs, new_ind, w.cu_seqlens_q, w.cu_seqlens_k, w.max_seqlen_q,
                    w.max_seqlen_k, causal=True)
    assert torch.equal(o1, o3)


@needs_gpu
def test_causal_first_row_returns_first_value_exactly(prefill_tile):
    print("[case] first causal row = v0", flush=True)
    w = wl.make_random(32, batch=1, q_lens=[40], k_lens=[40], max_segs=3).to("cuda")
    out = H.run_gpu(w, return_lse=False)
    slot0 = int(w.segs[0, 0].item())
    for h in range(64):
        assert torch.equal(out[0, h], w.v_pool[slot0, h // 8])


@needs_gpu
def test_decode_splits_agree_and_match_prefill_last_row():
    print("[case] decode splits vs prefill", flush=True)
    w = wl.make_random(33, batch=3, q_lens=[1, 1, 1], k_lens=[3000, 777, 64], max_segs=5,
                       kind="decode").to("cuda")
    outs = [H.run_gpu(w, num_splits=n, return_lse=False).float() for n in (1, 2, 0, 47)]
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 1e-2
    # the same rows through the prefill kernel (Lq = 1 per request)
    wp = wl.Workload(**{**w.__dict__, "kind": "prefill"})
    op = H.run_gpu(wp, return_lse=False).float()
    assert (op - outs[0]).abs().max().item() <= 1e-2


@needs_gpu
def test_chunked_prefill_equals_suffix_of_full_prefill(prefill_tile):
    print("[case] chunked = suffix", flush=True)
    full = wl.make_random(34, batch=1, q_lens=[512], k_lens=[512], max_segs=4).to("cuda")
    o_full = H.run_gpu(full, return_lse=False).float()
    import attention_segmented_kv_amd as sa
    for lq in (1, 100, 257):
        cq = torch.tensor([0, lq], dtype=torch.int32, device="cuda")
        oc = sa.prefill(full.q[512 - lq:].contiguous(), full.k_pool, full.v_pool, full.segs,
                        full.seg_indptr, cq, full.cu_seqlens_k, lq, 512, causal=True).float()
        assert (oc - o_full[512 - lq:]).abs().max().item() <= 1e-2


# ---------------------------------------------------------------- broken host bounds are loud

@needs_gpu
@pytest.mark.parametrize("num_splits", [0, 3])
def test_decode_key_count_above_max_seqlen_k_gives_nan(num_splits):
    """max_seqlen_k sizes the workspace; a request with more keys than that makes every output
    and LSE of the call NaN instead of a silent result. With a correct bound the same call
    matches the oracle."""
    print(f"[case] decode with K_b > max_seqlen_k, splits={num_splits}", flush=True)
    import attention_segmented_kv_amd as sa
    w = wl.make_random(35, batch=3, q_lens=[1] * 3, k_lens=[100, 2000, 50], max_segs=3,
                       kind="decode").to("cuda")
    out, lse = sa.decode(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_k, 1000,
                         num_splits=num_splits, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()
    _full_compare(w, "decode-bound-ok", num_splits=num_splits)


@needs_gpu
def test_prefill_queries_above_max_seqlen_q_give_nan(prefill_tile):
    """max_seqlen_q sizes the launch grid; query rows past it are marked NaN (output and LSE),
    the rows it covers are still correct."""
    print("[case] prefill with Lq_b > max_seqlen_q", flush=True)
    import attention_segmented_kv_amd as sa
    w = wl.make_random(36, batch=2, q_lens=[40, 100], k_lens=[40, 300], max_segs=3).to("cuda")
    out, lse = sa.prefill(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_q,
                          w.cu_seqlens_k, 64, w.max_seqlen_k, causal=True, return_lse=True)
    torch.cuda.synchronize()
    bad = slice(40 + 64, 140)  # request 1, positions 64..99
    assert torch.isnan(out[bad].float()).all() and torch.isnan(lse[bad]).all()
    good = torch.ones(140, dtype=torch.bool)
    good[bad] = False
    o_ref, l_ref = H.oracle_full(w)
    g = good.numpy()
    H.assert_close(out.float().cpu().numpy()[g], o_ref[g], "prefill-bound")
    H.assert_lse_close(lse.cpu().numpy()[g], l_ref[g], "prefill-bound")
