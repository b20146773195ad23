"""Prefill and decode over pools larger than 4 GiB per tensor. In prefill, key blocks that
straddle segments are copied row by row; when every row of a kv head lies within 32-bit byte
offsets of its first row the copies go through a buffer with 32-bit offsets, otherwise through
64-bit addresses. Decode bases every tile's buffer at its first row. Here the same keys are
placed once in a small pool and once in a pool past the 4 GiB mark (segments beyond it, across
it and far below it), and each path must give bit-identical outputs and LSEs in the two layouts
(the copy path does not change the arithmetic); the small layout is also checked against the
oracle."""
import pytest
import torch

import attention_segmented_kv_amd as sa
import oracle
import workloads as wl
from tests import _helpers as H

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

BIG_POOL = 17_000_000  # tokens; x 1 kv head x 256 B = 4.35 GB per tensor, past 2^32 bytes
HKV, HQ, D = 1, 8, 128


def _layout():
    """Two requests (300 and 200 keys, causal, queries = keys) in 3 and 2 segments. Returns
    (segment lengths per request, small-pool offsets, big-pool offsets); the big offsets put
    most segments past row 2^32 / 256 = 16,777,216, one across it and one far below it."""
    lens = [[70, 100, 130], [117, 83]]
    small = [[100, 2000, 700], [3000, 1200]]
    big = [[16_900_000, 1000, 16_800_123], [16_950_017, 16_777_180]]
    return lens, small, big


@needs_gpu
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("tile", ["128", "256"])
def test_prefill_pool_beyond_4gib(tile, causal, monkeypatch):
    monkeypatch.setenv("SEG_ATTN_PREFILL_TILE", tile)
    lens, small, big = _layout()
    k_lens = [sum(x) for x in lens]
    print(f"[case] prefill large pool tile={tile} causal={causal} k={k_lens} big offsets={big}", flush=True)
    g = torch.Generator().manual_seed(4242)
    total = sum(k_lens)
    q = torch.randn(total, HQ, D, generator=g).to(torch.bfloat16).cuda()
    rows_k = torch.randn(total, HKV, D, generator=g).to(torch.bfloat16).cuda()
    rows_v = torch.randn(total, HKV, D, generator=g).to(torch.bfloat16).cuda()

    def place(pool_tokens, offsets):
        kp = torch.zeros(pool_tokens, HKV, D, dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        segs = []
        r = 0
        for req_lens, req_offs in zip(lens, offsets):
            for n, off in zip(req_lens, req_offs):
                kp[off:off + n] = rows_k[r:r + n]
                vp[off:off + n] = rows_v[r:r + n]
                segs.append((off, n))
                r += n
        return kp, vp, torch.tensor(segs, dtype=torch.int32, device="cuda")

    indptr = torch.tensor([0, 3, 5], dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, k_lens[0], total], dtype=torch.int32, device="cuda")
    results = []
    for pool_tokens, offsets in ((4096, small), (BIG_POOL, big)):
        kp, vp, segs = place(pool_tokens, offsets)
        out, lse = sa.prefill(q, kp, vp, segs, indptr, cu, cu, max(k_lens), max(k_lens), causal=causal,
                              return_lse=True)
        torch.cuda.synchronize()
        results.append((out.cpu(), lse.cpu()))
        if pool_tokens == 4096:
            small_host = (wl.bits(kp), wl.bits(vp), segs.cpu().numpy())
        del kp, vp
        torch.cuda.empty_cache()
    (o_small, l_small), (o_big, l_big) = results
    assert torch.equal(o_small.view(torch.int16), o_big.view(torch.int16)), "outputs differ between pool layouts"
    assert torch.equal(l_small.view(torch.int32), l_big.view(torch.int32)), "LSEs differ between pool layouts"

    # the small layout against the oracle
    k_bits, v_bits, segs_np = small_host
    cu_np = cu.cpu().numpy()
    o_ref, l_ref = oracle.attention(wl.bits(q), k_bits, v_bits, segs_np, indptr.cpu().numpy(), cu_np, cu_np,
                                    num_heads_kv=HKV, softmax_scale=D ** -0.5, causal=causal)
    name = f"large-pool-{tile}-{'causal' if causal else 'full'}"
    mx, rms = H.assert_close(o_small.float().numpy(), o_ref, name)
    H.assert_lse_close(l_small.numpy(), l_ref, name)
    print(f"[parity] {name}: layouts bit-identical, max_abs={mx:.3e} rms={rms:.3e}", flush=True)


DEC_LENS = [[500, 300], [1], [77, 900, 3]]
DEC_SMALL = [[100, 700], [1050], [1100, 1200, 2200]]


def _dec_big(tok_bytes):
    """Big-pool offsets for the decode layout: past, across and below the 4 GiB mark of a
    tensor whose rows are tok_bytes long."""
    mark = (1 << 32) // tok_bytes
    return [[mark + 123_456, 1000], [mark + 100], [mark - 40, mark + 777_777, 7]], mark + 1_000_000


@needs_gpu
@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("kvd", ["bf16", "fp8_e4m3"])
def test_decode_pool_beyond_4gib(kvd, splits):
    fp8 = kvd == "fp8_e4m3"
    big, big_pool = _dec_big(HKV * D * (1 if fp8 else 2))
    k_lens = [sum(x) for x in DEC_LENS]
    print(f"[case] decode large pool {kvd} splits={splits} k={k_lens} pool={big_pool} big offsets={big}",
          flush=True)
    g = torch.Generator().manual_seed(4343)
    total = sum(k_lens)
    batch = len(k_lens)
    q = torch.randn(batch, HQ, D, generator=g).to(torch.bfloat16).cuda()
    xk = torch.randn(total, HKV, D, generator=g)
    xv = torch.randn(total, HKV, D, generator=g)
    if fp8:
        (rows_k, sk), (rows_v, sv) = wl.encode_fp8_rows(xk), wl.encode_fp8_rows(xv)
        rows_k, rows_v, sk, sv = rows_k.cuda(), rows_v.cuda(), sk.cuda(), sv.cuda()
    else:
        rows_k, rows_v = xk.to(torch.bfloat16).cuda(), xv.to(torch.bfloat16).cuda()

    def place(pool_tokens, offsets):
        kp = torch.zeros(pool_tokens, HKV, D, dtype=rows_k.dtype, device="cuda")
        vp = torch.zeros_like(kp)
        ks = torch.ones(pool_tokens, HKV, dtype=torch.float32, device="cuda") if fp8 else None
        vs = torch.ones_like(ks) if fp8 else None
        segs = []
        r = 0
        for req_lens, req_offs in zip(DEC_LENS, offsets):
            for n, off in zip(req_lens, req_offs):
                kp[off:off + n] = rows_k[r:r + n]
                vp[off:off + n] = rows_v[r:r + n]
                if fp8:
                    ks[off:off + n] = sk[r:r + n]
                    vs[off:off + n] = sv[r:r + n]
                segs.append((off, n))
                r += n
        return kp, vp, ks, vs, torch.tensor(segs, dtype=torch.int32, device="cuda")

    indptr = torch.tensor([0, 2, 3, 6], dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, k_lens[0], k_lens[0] + k_lens[1], total], dtype=torch.int32, device="cuda")
    results = []
    for pool_tokens, offsets in ((4096, DEC_SMALL), (big_pool, big)):
        kp, vp, ks, vs, segs = place(pool_tokens, offsets)
        out, lse = sa.decode(q, kp, vp, segs, indptr, cu, max(k_lens), k_scale=ks, v_scale=vs,
                             num_splits=splits, return_lse=True)
        torch.cuda.synchronize()
        results.append((out.cpu(), lse.cpu()))
        if pool_tokens == 4096:
            small_host = (wl.bits(kp), wl.bits(vp), None if ks is None else ks.cpu().numpy(),
                          None if vs is None else vs.cpu().numpy(), segs.cpu().numpy())
        del kp, vp, ks, vs
        torch.cuda.empty_cache()
    (o_small, l_small), (o_big, l_big) = results
    assert torch.equal(o_small.view(torch.int16), o_big.view(torch.int16)), "outputs differ between pool layouts"
    assert torch.equal(l_small.view(torch.int32), l_big.view(torch.int32)), "LSEs differ between pool layouts"

    k_bits, v_bits, ks_np, vs_np, segs_np = small_host
    cu_np = cu.cpu().numpy()
    cq = list(range(batch + 1))
    o_ref, l_ref = oracle.attention(wl.bits(q), k_bits, v_bits, segs_np, indptr.cpu().numpy(), cq, cu_np,
                                    num_heads_kv=HKV, softmax_scale=D ** -0.5, causal=False,
                                    kv_format=kvd, k_scale=ks_np, v_scale=vs_np)
    mx, rms = H.assert_close(o_small.float().numpy(), o_ref, f"large-pool-decode-{kvd}")
    H.assert_lse_close(l_small.numpy(), l_ref, f"large-pool-decode-{kvd}")
    print(f"[parity] large-pool-decode-{kvd}-{splits}: layouts bit-identical, max_abs={mx:.3e} rms={rms:.3e}",
          flush=True)
