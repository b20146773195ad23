"""Allocator compaction on the device: a pool fragmented by interleaved growth is compacted
(seg_attn_allocator_compact) and its data moved (seg_attn_kv_move). The moved rows and scales must
equal the model's moves applied on the host, bit for bit, every other slot must be unchanged, and
decode and prefill over the new tables must give bit-identical outputs to the calls before."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle.allocator import apply_moves
from tests import _helpers as H

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

POOL = 4096
DT = {"bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn, "int8": torch.int8}


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


@needs_gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3", "int8"])
def test_compaction_moves_data_and_keeps_attention_bitwise(fmt):
    print(f"[case] compaction {fmt}", flush=True)
    import attention_segmented_kv_amd as sa
    rng = np.random.default_rng(51)
    gen = torch.Generator().manual_seed(52)
    alloc = sa.SegmentAllocator(POOL, granule=1)
    ids = list(range(8))
    # interleaved growth fragments every request; releasing two of them leaves holes
    for _ in range(6):
        for r in ids:
            alloc.grow(r, int(rng.integers(5, 60)))
    for r in (2, 5):
        alloc.release(r)
    live = [r for r in ids if r not in (2, 5)]
    segs, ind, cu = alloc.tables(live)
    assert int(np.diff(ind).min()) >= 2  # every live request is fragmented
    # a pool poisoned everywhere, then every key of every live request written by the append
    hkv = 8
    if fmt == "int8":
        kp = torch.full((POOL, hkv, 128), -128, dtype=torch.int8, device="cuda")
    else:
        kp = torch.full((POOL, hkv, 128), float("nan"), device="cuda").to(DT[fmt])
    vp = kp.clone()
    ks = vs = None
    if fmt != "bf16":
        ks = torch.full((POOL, hkv), float("nan"), device="cuda")
        vs = ks.clone()
    total = int(cu[-1])
    kn = torch.randn(total, hkv, 128, generator=gen).to(torch.bfloat16).to("cuda")
    vn = torch.randn(total, hkv, 128, generator=gen).to(torch.bfloat16).to("cuda")
    sa.kv_append(kn, vn, _dev(segs), _dev(ind), _dev(cu), _dev(cu), kp, vp, k_scale=ks, v_scale=vs)
    B = len(live)
    q = torch.randn(B, 64, 128, generator=gen).to(torch.bfloat16).to("cuda")
    maxk = int(np.diff(cu).max())
    out1, lse1 = sa.decode(q, kp, vp, _dev(segs), _dev(ind), _dev(cu), maxk, k_scale=ks, v_scale=vs,
                           return_lse=True)
    if fmt == "bf16":
        lq = np.minimum(np.diff(cu), 37)
        cq = np.concatenate([[0], np.cumsum(lq)])
        qp = torch.randn(int(cq[-1]), 64, 128, generator=gen).to(torch.bfloat16).to("cuda")
        pre1 = sa.prefill(qp, kp, vp, _dev(segs), _dev(ind), _dev(cq), _dev(cu), int(lq.max()), maxk,
                          causal=True)
    torch.cuda.synchronize()
    kp0, vp0 = wl.bits(kp), wl.bits(vp)
    ks0 = None if ks is None else ks.cpu().numpy().copy()
    vs0 = None if vs is None else vs.cpu().numpy().copy()

    moves = alloc.compact()
    assert len(moves) > 0
    sa.kv_move(_dev(moves), kp, vp, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    mv = [tuple(int(x) for x in m[:3]) for m in moves]
    # moved rows and scales bit for bit, every other slot untouched
    assert np.array_equal(wl.bits(kp), apply_moves(kp0, mv))
    assert np.array_equal(wl.bits(vp), apply_moves(vp0, mv))
    if ks is not None:
        assert np.array_equal(ks.cpu().numpy().view(np.uint32), apply_moves(ks0, mv).view(np.uint32))
        assert np.array_equal(vs.cpu().numpy().view(np.uint32), apply_moves(vs0, mv).view(np.uint32))

    segs2, ind2, cu2 = alloc.tables(live)
    assert np.array_equal(cu2, cu) and int(np.diff(ind2).max()) == 1  # one segment each now
    out2, lse2 = sa.decode(q, kp, vp, _dev(segs2), _dev(ind2), _dev(cu2), maxk, k_scale=ks, v_scale=vs,
                           return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    if fmt == "bf16":
        pre2 = sa.prefill(qp, kp, vp, _dev(segs2), _dev(ind2), _dev(cq), _dev(cu2), int(lq.max()), maxk,
                          causal=True)
        torch.cuda.synchronize()
        assert torch.equal(pre1, pre2)
    # and the compacted pool still matches the oracle
    o_ref, l_ref = oracle.attention(wl.bits(q), wl.bits(kp), wl.bits(vp), segs2.astype(np.int64), ind2,
                                    np.arange(B + 1), cu2, num_heads_kv=hkv, softmax_scale=128 ** -0.5,
                                    causal=True, kv_format=fmt,
                                    k_scale=None if ks is None else ks.cpu().numpy(),
                                    v_scale=None if vs is None else vs.cpu().numpy())
    mx, rms = H.assert_close(out2.float().cpu().numpy(), o_ref, f"compaction {fmt}")
    H.assert_lse_close(lse2.cpu().numpy(), l_ref, f"compaction {fmt}")
    print(f"[parity] compaction {fmt}: {len(moves)} moves, max_abs={mx:.3e} rms={rms:.3e}", flush=True)
