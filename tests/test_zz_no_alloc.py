"""seg_attn_decode_noalloc (decode with the library's fixed per-GPU scratch instead of a caller
workspace) against seg_attn_decode on the same inputs, through the C ABI: two calls in a row, the
second smaller than the first, each compared with the workspace entry point and the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from tests import _helpers as H

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _call_noalloc(w, num_splits, out, lse):
    """seg_attn_decode_noalloc called directly through ctypes (no workspace argument exists)."""
    import attention_segmented_kv_amd as sa
    lib = sa._load()
    kvd = {"bf16": sa.KV_BF16, "fp8_e4m3": sa.KV_FP8_E4M3, "int8": sa.KV_INT8}[w.kv_dtype]
    p = lambda t: None if t is None else t.data_ptr()
    st = lib.seg_attn_decode_noalloc(p(w.q), p(w.k_pool), p(w.v_pool), p(w.k_scale), p(w.v_scale), kvd,
                                     p(w.segs), p(w.seg_indptr), p(w.cu_seqlens_k), w.batch, w.max_seqlen_k,
                                     w.num_heads_q, w.num_heads_kv, w.head_dim, w.pool_tokens,
                                     ctypes.c_float(w.softmax_scale), num_splits, p(out), p(lse),
                                     torch.cuda.current_stream().cuda_stream)
    return st


def _check(w, name, num_splits):
    out = torch.empty_like(w.q)
    lse = torch.empty((w.batch, w.num_heads_q), dtype=torch.float32, device=w.q.device)
    assert _call_noalloc(w, num_splits, out, lse) == 0
    ref_out, ref_lse = H.run_gpu(w, num_splits=num_splits)
    torch.cuda.synchronize()
    # the two entry points share every kernel; both must meet the oracle's bar
    o_ref, l_ref = H.oracle_full(w)
    for o, l, tag in ((out, lse, "noalloc"), (ref_out, ref_lse, "workspace")):
        mx, rms = H.assert_close(o.float().cpu().numpy(), o_ref, f"{name} {tag}")
        H.assert_lse_close(l.cpu().numpy(), l_ref, f"{name} {tag}")
        print(f"[parity] {name} {tag}: max_abs={mx:.3e} rms={rms:.3e}", flush=True)
    d = (out.float() - ref_out.float()).abs().max().item()
    print(f"[parity] {name}: noalloc vs workspace max diff {d:.3e}", flush=True)
    assert d <= H.MAX_ABS_TOL


@needs_gpu
@pytest.mark.parametrize("num_splits", [0, 4])
def test_noalloc_decode_matches_workspace_decode_twice(num_splits):
    print(f"[case] noalloc decode, splits={num_splits}: batch 128 lognormal bf16, then batch 3 fp8",
          flush=True)
    w1 = wl.make_config(4, device="cuda")
    _check(w1, "noalloc-b128", num_splits)
    del w1
    torch.cuda.empty_cache()
    w2 = wl.make_random(71, batch=3, q_lens=[1] * 3, k_lens=[900, 33, 2100], max_segs=4,
                        kv_dtype="fp8_e4m3", kind="decode").to("cuda")
    _check(w2, "noalloc-b3-fp8", num_splits)


@needs_gpu
def test_noalloc_decode_rejects_calls_beyond_its_scratch():
    import attention_segmented_kv_amd as sa
    w = wl.make_random(72, batch=4, q_lens=[1] * 4, k_lens=[64, 64, 64, 64], max_segs=1,
                       kind="decode").to("cuda")
    out = torch.empty_like(w.q)
    # 100 000 forced splits per request need far more than 64 MiB of partials
    w.max_seqlen_k = 64 * 100_000
    assert _call_noalloc(w, 100_000, out, None) == 7
    assert "scratch" in sa.status_string(7)
