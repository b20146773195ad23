"""GPU parity of the KV append (seg_attn_kv_append through the binding) against the CPU oracle.

The append is byte work once the FP8 decisions are taken in fp32 on both sides, so the bar is
bit-exact: every byte of both pools and every bit of both scale arrays, written slots and
untouched (NaN-poisoned) ones alike. Small cases compare whole pools; the full-size workloads
compare every written slot and check that the rest of the pool kept its bits.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _sa():
    import attention_segmented_kv_amd as sa
    return sa


def _raw(t: torch.Tensor) -> np.ndarray:
    """Storage bits of a GPU tensor on the host (bf16 -> uint16, fp8 -> uint8, fp32 -> uint32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return wl.bits(t)


def _new_rows(seed: int, total: int, hkv: int = 8, special: bool = True) -> torch.Tensor:
    """[total, hkv, 128] bf16 N(0,1) rows; with ``special`` the first rows are edge cases of the
    FP8 row quantiser: all zero, one nonzero value, bf16 subnormals only, values near the bf16
    maximum, a row whose values are exact multiples of its largest (code ties), a negative row."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(total, hkv, 128, generator=g)
    if special and total > 0:
        r = x.view(-1, 128)
        n = r.shape[0]
        if n > 0: r[0] = 0.0
        if n > 1: r[1] = 0.0; r[1, 77] = -3.5
        if n > 2: r[2] = torch.randn(128, generator=g) * 1e-39          # bf16 subnormals
        if n > 3: r[3] = torch.randn(128, generator=g).sign() * 3.0e38  # near the bf16 maximum
        if n > 4: r[4] = torch.arange(128, dtype=torch.float32) - 64.0  # scale 64/448 ties
        if n > 5: r[5] = -torch.rand(128, generator=g) * 1e4
    return x.to(torch.bfloat16)


def _tables_and_counts(w, n_new):
    segs, ind, _, ck = wl.host_tables(w)
    cu_new = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    return segs, ind, ck, cu_new


def _run_append(w, k_new, v_new, cu_new):
    dev = w.k_pool.device
    cn = torch.as_tensor(cu_new.astype(np.int32)).to(dev)
    _sa().kv_append(k_new.to(dev), v_new.to(dev), w.segs, w.seg_indptr, cn, w.cu_seqlens_k,
                    w.k_pool, w.v_pool, k_scale=w.k_scale, v_scale=w.v_scale)


def _compare_whole(w, k_new, v_new, n_new, name):
    segs, ind, ck, cu_new = _tables_and_counts(w, n_new)
    scaled = w.kv_dtype in ("fp8_e4m3", "int8")
    kp0, vp0 = _raw(w.k_pool), _raw(w.v_pool)
    ks0 = _raw(w.k_scale).view(np.float32) if scaled else None
    vs0 = _raw(w.v_scale).view(np.float32) if scaled else None
    kp, vp, ks, vs = oracle.kv_append(wl.bits(k_new), wl.bits(v_new), segs, ind, cu_new, ck, kp0, vp0,
                                      ks0, vs0, fmt=w.kv_dtype)
    _run_append(w, k_new, v_new, cu_new)
    torch.cuda.synchronize()
    assert np.array_equal(_raw(w.k_pool), kp), f"{name}: k_pool differs"
    assert np.array_equal(_raw(w.v_pool), vp), f"{name}: v_pool differs"
    if scaled:
        assert np.array_equal(_raw(w.k_scale), ks.view(np.uint32)), f"{name}: k_scale differs"
        assert np.array_equal(_raw(w.v_scale), vs.view(np.uint32)), f"{name}: v_scale differs"
    print(f"[parity] append {name}: {int(cu_new[-1])} tokens, pools bit-exact", flush=True)
    return kp, vp, ks, vs


@needs_gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3", "int8"])
def test_append_decode_step_small(fmt):
    """One new token per request (a few requests append none), 1-4 segments with empty ones."""
    print(f"[case] append decode step {fmt}", flush=True)
    rng = np.random.default_rng(11)
    batch = 37
    k_lens = rng.integers(1, 300, size=batch)
    n_new = np.ones(batch, dtype=np.int64)
    n_new[[3, 17, 30]] = 0
    w = wl.make_random(11, batch=batch, q_lens=[1] * batch, k_lens=k_lens.tolist(), max_segs=4,
                       kind="decode", kv_dtype=fmt, zero_length_segments=True, device="cuda")
    k_new = _new_rows(12, int(n_new.sum()))
    v_new = _new_rows(13, int(n_new.sum()), special=False)
    _compare_whole(w, k_new, v_new, n_new, f"decode-step {fmt}")


@needs_gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3", "int8"])
def test_append_prefill_chunks_ragged(fmt):
    """Ragged chunks: none, one token, a chunk spanning segment boundaries, a whole request,
    a chunk not a multiple of 16 rows, and a request with no keys at all."""
    print(f"[case] append prefill chunks {fmt}", flush=True)
    k_lens = [700, 5, 333, 129, 0, 1000]
    n_new = np.array([257, 1, 333, 0, 0, 999], dtype=np.int64)
    w = wl.make_random(21, batch=len(k_lens), q_lens=[1] * len(k_lens), k_lens=k_lens, max_segs=5,
                       kind="decode", kv_dtype=fmt, zero_length_segments=True, device="cuda")
    k_new = _new_rows(22, int(n_new.sum()))
    v_new = _new_rows(23, int(n_new.sum()))
    _compare_whole(w, k_new, v_new, n_new, f"prefill-chunks {fmt}")


@needs_gpu
def test_append_other_kv_head_counts():
    """Hkv = 1 and Hkv = 3: the (token, head) row index and the slot stride follow Hkv."""
    for hkv, seed, fmt in ((1, 31, "fp8_e4m3"), (3, 32, "fp8_e4m3"), (3, 33, "int8")):
        print(f"[case] append hkv={hkv}", flush=True)
        k_lens = [40, 90, 17]
        n_new = np.array([40, 3, 16], dtype=np.int64)
        w = wl.make_random(seed, batch=3, q_lens=[1] * 3, k_lens=k_lens, max_segs=3, kind="decode",
                           kv_dtype=fmt, num_heads_q=8 * hkv, num_heads_kv=hkv, device="cuda")
        k_new = _new_rows(seed + 1, int(n_new.sum()), hkv=hkv)
        v_new = _new_rows(seed + 2, int(n_new.sum()), hkv=hkv)
        _compare_whole(w, k_new, v_new, n_new, f"hkv={hkv} {fmt}")


@needs_gpu
@pytest.mark.parametrize("fmt", ["fp8_e4m3", "int8"])
def test_append_then_decode_reads_what_was_written(fmt):
    """Appending a request's last token, then decoding, gives what the attention oracle gives on
    the pool the append oracle produced: the formats of the two steps agree."""
    print(f"[case] append then decode {fmt}", flush=True)
    from tests import _helpers as H
    k_lens = [300, 1500, 64, 2047]
    w = wl.make_random(41, batch=4, q_lens=[1] * 4, k_lens=k_lens, max_segs=3, kind="decode",
                       kv_dtype=fmt, device="cuda")
    n_new = np.ones(4, dtype=np.int64)
    k_new, v_new = _new_rows(42, 4, special=False), _new_rows(43, 4, special=False)
    h = H.host_inputs(w)
    kp, vp, ks, vs = _compare_whole(w, k_new, v_new, n_new, "before decode")
    out, lse = H.run_gpu(w, num_splits=2)
    torch.cuda.synchronize()
    # the oracle attends over the pools the append oracle produced
    h.update(k_bits=kp, v_bits=vp, k_scale=ks, v_scale=vs)
    o_ref, l_ref = H.oracle_full(w, h)
    H.assert_close(out.float().cpu().numpy(), o_ref, "append+decode")
    H.assert_lse_close(lse.cpu().numpy(), l_ref, "append+decode")


def _full_size_case(c, fmt=None):
    """The append a step of named workload c performs: each request's last Lq_b keys are new
    (one per request for decode, the whole chunk for prefill). With ``fmt`` = "fp8_e4m3" or
    "int8" a bf16 workload's pools are replaced by poisoned pools of that format and the same
    shape (NaN codes, or -128, and NaN scales; the append reads only the tables)."""
    w = wl.make_config(c, device="cuda")
    if fmt in ("fp8_e4m3", "int8") and w.kv_dtype != fmt:
        shape = tuple(w.k_pool.shape)
        if fmt == "fp8_e4m3":
            w.k_pool = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
            w.v_pool = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
        else:
            w.k_pool = torch.full(shape, -128, dtype=torch.int8, device="cuda")
            w.v_pool = torch.full(shape, -128, dtype=torch.int8, device="cuda")
        w.k_scale = torch.full(shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        w.v_scale = torch.full(shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        w.kv_dtype = fmt
    n_new = w.q_lens.astype(np.int64)
    return w, n_new


@needs_gpu
@pytest.mark.parametrize("c,fmt", [(2, None), (3, None), (3, "fp8_e4m3"), (3, "int8"), (4, None), (5, None),
                                   (6, None)])
def test_append_full_size_workloads(c, fmt):
    print(f"[case] append at config {c} size, {fmt or 'its own'} pool", flush=True)
    w, n_new = _full_size_case(c, fmt)
    segs, ind, ck, cu_new = _tables_and_counts(w, n_new)
    hkv = w.num_heads_kv
    total = int(cu_new[-1])
    k_new, v_new = _new_rows(100 + c, total, hkv=hkv), _new_rows(200 + c, total, hkv=hkv)
    slots = np.concatenate([oracle.request_slots(segs, ind, b)[int(ck[b + 1] - ck[b]) - int(n_new[b]):]
                            for b in range(w.batch)]).astype(np.int64)
    assert len(slots) == total
    before = [w.k_pool.clone(), w.v_pool.clone()]
    if w.k_scale is not None:
        before += [w.k_scale.clone(), w.v_scale.clone()]
    _run_append(w, k_new, v_new, cu_new)
    torch.cuda.synchronize()
    idx = torch.as_tensor(slots, device="cuda")
    scaled = w.kv_dtype in ("fp8_e4m3", "int8")
    quant = oracle.quantize_rows if w.kv_dtype == "fp8_e4m3" else oracle.quantize_rows_int8
    for pool, scale, new, nm in ((w.k_pool, w.k_scale, k_new, "k"), (w.v_pool, w.v_scale, v_new, "v")):
        got = _raw(pool[idx])
        if scaled:
            codes, sc = quant(oracle.bf16_bits_to_f32(wl.bits(new)))
            assert np.array_equal(got, codes), f"config {c}: {nm} codes differ"
            assert np.array_equal(_raw(scale[idx]), sc.view(np.uint32)), f"config {c}: {nm} scales differ"
        else:
            assert np.array_equal(got, wl.bits(new)), f"config {c}: {nm} rows differ"
    # every other slot kept its bits (compared on the device: the pools are up to 2 GiB)
    keep = torch.ones(w.pool_tokens, dtype=torch.bool, device="cuda")
    keep[idx] = False
    after = [w.k_pool, w.v_pool] + ([w.k_scale, w.v_scale] if scaled else [])
    for a, b in zip(after, before):
        ai = a.view(torch.uint8) if a.element_size() == 1 else a.view(torch.int16 if a.element_size() == 2 else torch.int32)
        bi = b.view(torch.uint8) if b.element_size() == 1 else b.view(torch.int16 if b.element_size() == 2 else torch.int32)
        assert torch.equal(ai[keep], bi[keep]), f"config {c}: a slot outside the new tokens changed"
    print(f"[parity] append config {c}: {total} tokens bit-exact, rest untouched", flush=True)


@needs_gpu
def test_append_is_deterministic_and_idempotent():
    """The same append twice leaves the same bytes (no read of the destination, no race)."""
    print("[case] append twice", flush=True)
    w = wl.make_random(51, batch=3, q_lens=[1] * 3, k_lens=[100, 200, 300], kind="decode",
                       kv_dtype="fp8_e4m3", device="cuda")
    n_new = np.array([100, 50, 7])
    k_new, v_new = _new_rows(52, int(n_new.sum())), _new_rows(53, int(n_new.sum()))
    _, _, _, cu_new = _tables_and_counts(w, n_new)
    _run_append(w, k_new, v_new, cu_new)
    first = [_raw(t) for t in (w.k_pool, w.v_pool, w.k_scale, w.v_scale)]
    _run_append(w, k_new, v_new, cu_new)
    torch.cuda.synchronize()
    for a, t in zip(first, (w.k_pool, w.v_pool, w.k_scale, w.v_scale)):
        assert np.array_equal(a, _raw(t))


@needs_gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3", "int8"])
def test_append_graph_replays_equal_eager(fmt):
    """A captured append (a decode step's tokens and a prefill chunk's) replayed into a pool
    restored to its NaN-poisoned state each time writes the same bytes as the eager call: the
    benchmark times the appends as such replays."""
    sa = _sa()
    print(f"[case] append graph replay {fmt}", flush=True)
    k_lens = [300, 1, 900, 64]
    n_new = np.array([1, 1, 257, 0], dtype=np.int64)
    w = wl.make_random(61, batch=len(k_lens), q_lens=[1] * len(k_lens), k_lens=k_lens, max_segs=4,
                       kind="decode", kv_dtype=fmt, zero_length_segments=True, device="cuda")
    k_new = _new_rows(62, int(n_new.sum())).cuda()
    v_new = _new_rows(63, int(n_new.sum())).cuda()
    _, _, _, cu_new = _tables_and_counts(w, n_new)
    cn = torch.as_tensor(cu_new.astype(np.int32)).cuda()
    tensors = [t for t in (w.k_pool, w.v_pool, w.k_scale, w.v_scale) if t is not None]
    before = [t.clone() for t in tensors]

    def call():
        sa.kv_append(k_new, v_new, w.segs, w.seg_indptr, cn, w.cu_seqlens_k, w.k_pool, w.v_pool,
                     k_scale=w.k_scale, v_scale=w.v_scale)

    call()
    torch.cuda.synchronize()
    eager = [_raw(t) for t in tensors]
    for t, b in zip(tensors, before):
        t.copy_(b)
    call()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        for t, b in zip(tensors, before):
            t.copy_(b)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, t in zip(eager, tensors):
            assert np.array_equal(e, _raw(t)), f"{fmt}: replay {r} differs"
