"""Prefill over a pool larger than 4 GiB per tensor. Key blocks that straddle segments are
copied row by row; when every row of a kv head lies within 32-bit byte offsets of its first row
the copies go through a buffer with 32-bit offsets, otherwise through 64-bit addresses. Here the
same keys are placed once in a small pool and once in a 17M-token pool, partly beyond the 4 GiB
mark, and both tilings must give bit-identical outputs and LSEs in the two layouts (the copy path
does not change the arithmetic; the small layout is checked against the oracle by the other
parity tests, and once more here)."""
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
@pytest.mark.parametrize("tile", ["128", "256"])
def test_prefill_pool_beyond_4gib(tile, monkeypatch):
    monkeypatch.setenv("SEG_ATTN_PREFILL_TILE", tile)
    lens, small, big = _layout()
    k_lens = [sum(x) for x in lens]
    print(f"[case] prefill large pool tile={tile} k={k_lens} big offsets={big}", flush=True)
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
        out, lse = sa.prefill(q, kp, vp, segs, indptr, cu, cu, max(k_lens), max(k_lens), causal=True,
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
                                    num_heads_kv=HKV, softmax_scale=D ** -0.5, causal=True)
    mx, rms = H.assert_close(o_small.float().numpy(), o_ref, f"large-pool-{tile}")
    H.assert_lse_close(l_small.numpy(), l_ref, f"large-pool-{tile}")
    print(f"[parity] large-pool-{tile}: layouts bit-identical, max_abs={mx:.3e} rms={rms:.3e}", flush=True)
