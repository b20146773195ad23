"""The whole path as a serving loop drives it: the allocator hands out segments and writes the
tables, seg_attn_kv_append writes each step's new tokens, chunked prefill and decode read them,
finished requests are released and their slots reused by new ones. Every attention call is
compared with the oracle evaluated on pools that the append oracle maintains from the same
inputs, and the pools themselves are compared bit for bit at the end.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests import _helpers as H

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

HQ, HKV, D = 64, 8, 128


def _raw(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return wl.bits(t)


def _dev_tables(segs, ind, cu):
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")
    return f(np.asarray(segs).reshape(-1, 2)), f(ind), f(cu)


@needs_gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3", "int8"])
def test_serving_loop_matches_the_oracle(fmt):
    import attention_segmented_kv_amd as sa
    print(f"[case] serving loop {fmt}", flush=True)
    rng = np.random.default_rng(77)
    gen = torch.Generator().manual_seed(78)
    pool_tokens = 6000
    shape = (pool_tokens, HKV, D)
    if fmt == "bf16":
        kp = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        vp = kp.clone()
        ks = vs = None
    else:
        if fmt == "fp8_e4m3":
            kp = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
        else:
            kp = torch.full(shape, -128, dtype=torch.int8, device="cuda")
        vp = kp.clone()
        ks = torch.full(shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        vs = ks.clone()
    # host pools kept by the append oracle
    hk, hv = _raw(kp), _raw(vp)
    hks = None if ks is None else _raw(ks).view(np.float32).copy()
    hvs = None if vs is None else _raw(vs).view(np.float32).copy()

    alloc = sa.SegmentAllocator(pool_tokens)
    chunk = 96 if fmt == "bf16" else 10 ** 9  # one-byte pools: whole prompts at once, decode only
    live = {}  # id -> [prompt tokens still to prefill, decode steps left]
    next_id = 0
    checked = 0
    for step in range(14):
        # arrivals
        while len(live) < 6:
            live[next_id] = [int(rng.integers(30, 400)), int(rng.integers(2, 6))]
            next_id += 1
        ids = sorted(live)
        n_new = []
        for r in ids:
            pre, _ = live[r]
            n_new.append(min(pre, chunk) if pre > 0 else 1)
        for r, n in zip(ids, n_new):
            alloc.grow(r, n)
        segs, ind, cu = alloc.tables(ids)
        total = int(sum(n_new))
        k_new = torch.randn(total, HKV, D, generator=gen).to(torch.bfloat16)
        v_new = torch.randn(total, HKV, D, generator=gen).to(torch.bfloat16)
        cu_new = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
        # device append, and the oracle's
        ds, di, dc = _dev_tables(segs, ind, cu)
        dn = torch.from_numpy(cu_new.astype(np.int32)).to("cuda")
        sa.kv_append(k_new.to("cuda"), v_new.to("cuda"), ds, di, dn, dc, kp, vp, k_scale=ks, v_scale=vs)
        hk, hv, hks, hvs = oracle.kv_append(wl.bits(k_new), wl.bits(v_new), segs.astype(np.int64), ind,
                                            cu_new, cu, hk, hv, hks, hvs, fmt=fmt)
        # attention: the prefill-phase requests (their chunk as queries), then the decode ones
        pre_ids = [i for i, r in enumerate(ids) if live[r][0] > 0]
        dec_ids = [i for i, r in enumerate(ids) if live[r][0] == 0]
        for group, kind in ((pre_ids, "prefill"), (dec_ids, "decode")):
            if not group or (kind == "prefill" and fmt != "bf16"):
                continue  # one-byte pools are read by decode only; their prompts are appended
            gids = [ids[i] for i in group]
            gs, gi, gc = alloc.tables(gids)
            lq = [n_new[i] for i in group]
            cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
            q = torch.randn(int(cq[-1]), HQ, D, generator=gen).to(torch.bfloat16)
            s_, i_, c_ = _dev_tables(gs, gi, gc)
            if kind == "prefill":
                out, lse = sa.prefill(q.to("cuda"), kp, vp, s_, i_, torch.from_numpy(cq.astype(np.int32)).to("cuda"),
                                      c_, max(lq), int(np.diff(gc).max()), causal=True, return_lse=True)
            else:
                out, lse = sa.decode(q.to("cuda"), kp, vp, s_, i_, c_, int(np.diff(gc).max()),
                                     k_scale=ks, v_scale=vs, return_lse=True)
            torch.cuda.synchronize()
            o_ref, l_ref = oracle.attention(wl.bits(q), hk, hv, gs.astype(np.int64), gi, cq, gc,
                                            num_heads_kv=HKV, softmax_scale=1.0 / np.sqrt(D),
                                            causal=True, kv_format=fmt, k_scale=hks, v_scale=hvs)
            H.assert_close(out.float().cpu().numpy(), o_ref, f"step {step} {kind}")
            H.assert_lse_close(lse.cpu().numpy(), l_ref, f"step {step} {kind}")
            checked += len(group)
        # advance; finished requests leave and free their slots
        for r, n in zip(ids, n_new):
            if live[r][0] > 0:
                live[r][0] -= n
            else:
                live[r][1] -= 1
                if live[r][1] == 0:
                    del live[r]
                    alloc.release(r)
    assert np.array_equal(_raw(kp), hk) and np.array_equal(_raw(vp), hv)
    if ks is not None:
        assert np.array_equal(_raw(ks), hks.view(np.uint32)) and np.array_equal(_raw(vs), hvs.view(np.uint32))
    st = alloc.stats()
    print(f"[parity] serving loop {fmt}: {checked} request-steps checked, {next_id} requests, "
          f"{st['free_runs']} free runs at the end", flush=True)
    assert next_id > 6  # requests finished and slots were reused
