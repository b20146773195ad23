"""HIP-graph replay of the hot path (the benchmark times replays of a captured step).

A step captured with torch.cuda.graph must give, on every replay, exactly the eager result:
the same kernels run on the same inputs, so outputs agree bit for bit. Each check replays the
graph several times with eager work and synchronisations in between.
"""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _step_fn(w, out, lse, ws, noalloc=False):
    import attention_segmented_kv_amd as sa
    if noalloc:
        def step():
            sa.decode_noalloc(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_k, w.max_seqlen_k,
                              k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale, out=out,
                              lse=lse)
    elif w.kind == "prefill":
        def step():
            sa.prefill(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_q, w.cu_seqlens_k,
                       w.max_seqlen_q, w.max_seqlen_k, causal=w.causal, softmax_scale=w.softmax_scale,
                       out=out, lse=lse)
    else:
        def step():
            sa.decode(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_k, w.max_seqlen_k,
                      k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale, out=out,
                      lse=lse, workspace=ws)
    return step


def _check_replays(w, name, noalloc=False):
    import attention_segmented_kv_amd as sa
    print(f"[case] graph replay {name}", flush=True)
    dev = w.q.device
    ws = None
    if w.kind == "decode":
        kvd = {"fp8_e4m3": sa.KV_FP8_E4M3, "int8": sa.KV_INT8}.get(w.kv_dtype, sa.KV_BF16)
        need = sa.decode_workspace_bytes(w.batch, w.max_seqlen_k, w.num_heads_q, w.num_heads_kv,
                                         w.head_dim, kvd, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    out_e = torch.empty_like(w.q)
    lse_e = torch.empty((w.q.shape[0], w.q.shape[1]), dtype=torch.float32, device=dev)
    _step_fn(w, out_e, lse_e, ws)()
    torch.cuda.synchronize()

    out_g = torch.full_like(w.q, float("nan"))
    lse_g = torch.full((w.q.shape[0], w.q.shape[1]), float("nan"), dtype=torch.float32, device=dev)
    step = _step_fn(w, out_g, lse_g, ws, noalloc)
    step()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    scratch = torch.empty_like(w.q)
    for r in range(4):
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"{name}: replay {r} output differs"
        assert torch.equal(lse_g.view(torch.int32), lse_e.view(torch.int32)), f"{name}: replay {r} lse differs"
        # eager work on the same stream and workspace (or scratch) between replays
        _step_fn(w, scratch, None, ws, noalloc)()
        torch.cuda.synchronize()


@needs_gpu
def test_graph_replay_prefill():
    _check_replays(wl.make_config(2).to("cuda"), "prefill_1k")


@needs_gpu
def test_graph_replay_chunked_prefill_random():
    w = wl.make_random(11, batch=3, q_lens=[300, 64, 129], k_lens=[700, 64, 1000], device="cuda")
    _check_replays(w, "random prefill")


@needs_gpu
def test_graph_replay_decode_bf16():
    w = wl.make_random(12, batch=9, q_lens=[1] * 9, k_lens=[5, 64, 1000, 3000, 1, 77, 4096, 640, 8000],
                       kind="decode", device="cuda")
    _check_replays(w, "decode bf16")


@needs_gpu
def test_graph_replay_decode_fp8():
    w = wl.make_random(13, batch=4, q_lens=[1] * 4, k_lens=[20000, 3, 9000, 512], kind="decode",
                       kv_dtype="fp8_e4m3", device="cuda")
    _check_replays(w, "decode fp8")


@needs_gpu
def test_graph_replay_decode_int8():
    w = wl.make_random(14, batch=6, q_lens=[1] * 6, k_lens=[7000, 1, 300, 12000, 64, 2049], kind="decode",
                       kv_dtype="int8", device="cuda")
    _check_replays(w, "decode int8")


@needs_gpu
@pytest.mark.parametrize("kvd", ["bf16", "fp8_e4m3"])
def test_graph_replay_decode_noalloc(kvd):
    """The allocation-free decode is the entry point for callers that capture graphs: every
    replay, with eager calls sharing its scratch in between, equals the eager result (and the
    workspace decode's, which the eager reference in _check_replays is)."""
    w = wl.make_random(15, batch=5, q_lens=[1] * 5, k_lens=[9000, 2, 640, 4097, 30000], kind="decode",
                       kv_dtype=kvd, device="cuda")
    _check_replays(w, f"decode_noalloc {kvd}", noalloc=True)
