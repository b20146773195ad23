"""GPU parity of segment linear attention (seg_attn_linear_prefill / _decode through the binding)
against the float64 recurrence of the oracle, outputs and final states.

Linear-attention outputs are unnormalised decayed sums (|o| reaches 20 on these inputs), so the
bar is relative to the reference's size: RMS error <= 5e-3 of the reference's RMS and max error
<= 1e-2 of its largest magnitude for outputs, 5e-3 of the largest magnitude for states. A CPU
emulation of the kernel's roundings (bf16 output, bf16 P, K~ and state operand, fp32 state)
gives 2.4e-3, 4e-3 and 2e-3 on the full-size inputs; the bars leave a factor of two.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

REL_RMS, REL_MAX, STATE_REL = 5e-3, 1e-2, 5e-3


def _sa():
    import attention_segmented_kv_amd as sa
    return sa


def _assert_rel(got, ref, name, rms_tol=REL_RMS, max_tol=REL_MAX):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    err = np.abs(got - ref)
    scale_rms = max(np.sqrt((ref ** 2).mean()), 1e-30)
    scale_max = max(np.abs(ref).max(), 1e-30)
    rel_rms = np.sqrt((err ** 2).mean()) / scale_rms
    rel_max = err.max() / scale_max
    print(f"[parity] {name}: rel_rms={rel_rms:.2e} rel_max={rel_max:.2e}", flush=True)
    assert rel_rms <= rms_tol and rel_max <= max_tol, f"{name}: rel_rms {rel_rms:.3e} rel_max {rel_max:.3e}"


def _oracle(w, pool_before):
    s0 = pool_before[w.state_slots.long().cpu()].double().numpy() if w.initial_state else None
    return oracle.linear_attention(wl.bits(w.q), wl.bits(w.k), wl.bits(w.v), w.g.cpu().numpy(),
                                   w.cu_seqlens.cpu().numpy(), s0, w.scale)


# Prefill paths: "fused" (the closed form, one launch; the default up to 4096 tokens),
# "chunked" (chunk-parallel with a workspace; forced here through SEG_ATTN_LINEAR_PREFILL) and
# "sequential" (no workspace).
PATHS = ["fused", "chunked", "sequential"]


@pytest.fixture
def path_env(monkeypatch):
    def use(path):
        if path == "chunked":
            monkeypatch.setenv("SEG_ATTN_LINEAR_PREFILL", "chunked")
        else:
            monkeypatch.delenv("SEG_ATTN_LINEAR_PREFILL", raising=False)
    yield use
    monkeypatch.delenv("SEG_ATTN_LINEAR_PREFILL", raising=False)


def _run(w, path="fused"):
    sa = _sa()
    if w.kind == "decode":
        return sa.linear_decode(w.q, w.k, w.v, w.g, w.state_slots, w.state_pool, scale=w.scale)
    return sa.linear_prefill(w.q, w.k, w.v, w.g, w.cu_seqlens, w.state_slots, w.state_pool,
                             initial_state=w.initial_state, scale=w.scale,
                             parallel=path != "sequential")


def _check(w, name, path="fused"):
    pool_before = w.state_pool.detach().cpu().clone()
    o_ref, st_ref = _oracle(w, pool_before)
    out = _run(w, path)
    torch.cuda.synchronize()
    _assert_rel(out.float().cpu().numpy(), o_ref, name)
    pool_after = w.state_pool.detach().cpu()
    slots = w.state_slots.long().cpu()
    st = pool_after[slots].double().numpy()
    srel = np.abs(st - st_ref).max() / max(np.abs(st_ref).max(), 1e-30)
    print(f"[parity] {name} states: rel_max={srel:.2e}", flush=True)
    assert srel <= STATE_REL, f"{name}: state rel_max {srel:.3e}"
    # slots no request names are untouched (bitwise, NaN poison included)
    keep = torch.ones(pool_after.shape[0], dtype=torch.bool)
    keep[slots] = False
    assert torch.equal(pool_after[keep].view(torch.int32), pool_before[keep].view(torch.int32))


@needs_gpu
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("initial_state", [False, True])
def test_linear_prefill_ragged(initial_state, path, path_env):
    """Lengths around the 32-token tile and the 64-token chunk: 1, 31, 33, 63, 64, 65, 130, an
    empty request."""
    path_env(path)
    print(f"[case] linear prefill ragged initial_state={initial_state} path={path}", flush=True)
    w = wl.make_linear(31, [1, 63, 64, 65, 130, 0, 31, 33], kind="prefill",
                       initial_state=initial_state, num_heads=4).to("cuda")
    _check(w, f"la-ragged-{int(initial_state)}-{path}", path)


@needs_gpu
@pytest.mark.parametrize("name", ["la_prefill_b1_1024", "la_prefill_b2_1024", "la_decode_b64",
                                  "la_decode_b256"])
def test_linear_named_workloads(name):
    print(f"[case] linear {name}", flush=True)
    w = wl.make_linear_config(name, device="cuda")
    _check(w, name)


@needs_gpu
@pytest.mark.parametrize("name", ["la_prefill_b1_1024", "la_prefill_b2_1024"])
def test_linear_named_prefills_chunked(name, path_env):
    path_env("chunked")
    print(f"[case] linear {name} chunked", flush=True)
    w = wl.make_linear_config(name, device="cuda")
    _check(w, name + "-chunked", "chunked")


@needs_gpu
def test_linear_sequential_prefill_full_size():
    print("[case] linear la_prefill_b2_1024 sequential", flush=True)
    w = wl.make_linear_config("la_prefill_b2_1024", device="cuda")
    _check(w, "la_prefill_b2_1024-sequential", "sequential")


@needs_gpu
@pytest.mark.parametrize("path", ["fused", "chunked"])
def test_linear_parallel_prefill_long_request_with_state(path, path_env):
    """A 3000-token request (47 chunks, 94 tiles) next to short ones, from stored states."""
    path_env(path)
    print(f"[case] linear prefill long request path={path}", flush=True)
    w = wl.make_linear(36, [3000, 5, 200], kind="prefill", initial_state=True, num_heads=2).to("cuda")
    _check(w, f"la-long-{path}", path)


@needs_gpu
def test_linear_prefill_past_the_closed_form_length():
    """4200 tokens (above the closed form's 4096) next to a 4096-token request: the call takes the
    chunk-parallel path."""
    print("[case] linear prefill above 4096 tokens", flush=True)
    w = wl.make_linear(38, [4200, 4096], kind="prefill", initial_state=True, num_heads=2).to("cuda")
    _check(w, "la-4200", "chunked")


@needs_gpu
def test_linear_decode_small_heads():
    print("[case] linear decode H=3", flush=True)
    w = wl.make_linear(32, [1] * 9, kind="decode", num_heads=3).to("cuda")
    _check(w, "la-decode-h3")


@needs_gpu
def test_linear_prefill_in_pieces_equals_prefill_at_once():
    """150 tokens at once against 100 then 50 with the state carried through the slot."""
    sa = _sa()
    print("[case] linear prefill in pieces", flush=True)
    w = wl.make_linear(33, [150], kind="prefill", initial_state=True, num_heads=2).to("cuda")
    pool0 = w.state_pool.clone()
    full = sa.linear_prefill(w.q, w.k, w.v, w.g, w.cu_seqlens, w.state_slots, w.state_pool)
    st_full = w.state_pool[w.state_slots.long()].clone()
    w.state_pool.copy_(pool0)
    cu1 = torch.tensor([0, 100], dtype=torch.int32, device="cuda")
    cu2 = torch.tensor([0, 50], dtype=torch.int32, device="cuda")
    a = sa.linear_prefill(w.q[:100].contiguous(), w.k[:100].contiguous(), w.v[:100].contiguous(),
                          w.g[:100].contiguous(), cu1, w.state_slots, w.state_pool)
    b = sa.linear_prefill(w.q[100:].contiguous(), w.k[100:].contiguous(), w.v[100:].contiguous(),
                          w.g[100:].contiguous(), cu2, w.state_slots, w.state_pool)
    torch.cuda.synchronize()
    ref = full.float().cpu().numpy()
    _assert_rel(torch.cat([a, b]).float().cpu().numpy(), ref, "la-pieces")
    st = w.state_pool[w.state_slots.long()].double().cpu().numpy()
    assert np.abs(st - st_full.double().cpu().numpy()).max() <= STATE_REL * np.abs(st).max()


@needs_gpu
def test_linear_decode_equals_one_token_prefill():
    sa = _sa()
    print("[case] linear decode vs one-token prefill", flush=True)
    w = wl.make_linear(34, [1] * 12, kind="decode", num_heads=4).to("cuda")
    pool0 = w.state_pool.clone()
    od = sa.linear_decode(w.q, w.k, w.v, w.g, w.state_slots, w.state_pool)
    sd = w.state_pool.clone()
    w.state_pool.copy_(pool0)
    op = sa.linear_prefill(w.q, w.k, w.v, w.g, w.cu_seqlens, w.state_slots, w.state_pool)
    torch.cuda.synchronize()
    _assert_rel(op.float().cpu().numpy(), od.float().cpu().numpy().astype(np.float64), "la-decode-vs-prefill")
    sl = w.state_slots.long()
    a, b = sd[sl].double().cpu().numpy(), w.state_pool[sl].double().cpu().numpy()
    assert np.abs(a - b).max() <= STATE_REL * np.abs(a).max()


@needs_gpu
@pytest.mark.parametrize("path", PATHS)
def test_linear_prefill_is_deterministic(path, path_env):
    sa = _sa()
    path_env(path)
    parallel = path != "sequential"
    print(f"[case] linear prefill determinism path={path}", flush=True)
    w = wl.make_linear(35, [300, 77], kind="prefill", num_heads=4).to("cuda")
    pool0 = w.state_pool.clone()
    o1 = sa.linear_prefill(w.q, w.k, w.v, w.g, w.cu_seqlens, w.state_slots, w.state_pool, parallel=parallel)
    p1 = w.state_pool.clone()
    w.state_pool.copy_(pool0)
    o2 = sa.linear_prefill(w.q, w.k, w.v, w.g, w.cu_seqlens, w.state_slots, w.state_pool, parallel=parallel)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(p1.view(torch.int32), w.state_pool.view(torch.int32))


@needs_gpu
@pytest.mark.parametrize("path", ["fused", "chunked"])
def test_linear_prefill_tokens_above_max_seqlen_give_nan(path, path_env):
    """max_seqlen bounds the request lengths: tokens of a longer request past it and that
    request's final state are NaN, the tokens before it are still correct."""
    path_env(path)
    print(f"[case] linear prefill with a length above max_seqlen path={path}", flush=True)
    sa = _sa()
    w = wl.make_linear(37, [70, 40, 129], kind="prefill", initial_state=True, num_heads=4).to("cuda")
    pool_before = w.state_pool.detach().cpu().clone()
    o_ref, st_ref = _oracle(w, pool_before)
    out = sa.linear_prefill(w.q, w.k, w.v, w.g, w.cu_seqlens, w.state_slots, w.state_pool,
                            initial_state=True, scale=w.scale, max_seqlen=64)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    bad = np.zeros(239, dtype=bool)
    bad[64:70] = True
    bad[110 + 64:239] = True
    assert np.isnan(got[bad]).all()
    _assert_rel(got[~bad], o_ref[~bad], "linear-bound")
    st = w.state_pool.detach().cpu()[w.state_slots.long().cpu()].double().numpy()
    assert np.isnan(st[0]).all() and np.isnan(st[2]).all()
    assert np.abs(st[1] - st_ref[1]).max() <= STATE_REL * np.abs(st_ref[1]).max()


@needs_gpu
@pytest.mark.parametrize("case", ["fused", "fused-state", "chunked-state", "decode"])
def test_linear_graph_replays_equal_eager(case, path_env):
    """A captured linear-attention call replayed several times (its state slots restored
    before each replay, other eager calls in between) gives the eager outputs and final states
    bit for bit: the timed form of these calls in the benchmark is such a replay."""
    sa = _sa()
    path_env("chunked" if case.startswith("chunked") else "fused")
    print(f"[case] linear graph replay {case}", flush=True)
    if case == "decode":
        w = wl.make_linear(41, [1] * 9, kind="decode", initial_state=True, num_heads=4).to("cuda")
    else:
        w = wl.make_linear(42, [300, 77, 1], kind="prefill", initial_state=case.endswith("state"),
                           num_heads=4).to("cuda")
    out = torch.empty_like(w.q)
    max_len = int(w.lens.max())
    ws = None
    if w.kind == "prefill":
        need = sa._load().seg_attn_linear_prefill_workspace_bytes(w.batch, max_len, w.num_heads, 128)
        ws = torch.empty(max(int(need), 256), dtype=torch.uint8, device="cuda")

    def call(o):
        if w.kind == "decode":
            sa.linear_decode(w.q, w.k, w.v, w.g, w.state_slots, w.state_pool, scale=w.scale, out=o)
        else:
            sa.linear_prefill(w.q, w.k, w.v, w.g, w.cu_seqlens, w.state_slots, w.state_pool,
                              initial_state=w.initial_state, scale=w.scale, out=o, max_seqlen=max_len,
                              workspace=ws)

    pool0 = w.state_pool.clone()
    call(out)
    torch.cuda.synchronize()
    out_e, pool_e = out.clone(), w.state_pool.clone()
    w.state_pool.copy_(pool0)
    out_g = torch.empty_like(w.q)
    call(out_g)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    scratch = torch.empty_like(w.q)
    for r in range(3):
        w.state_pool.copy_(pool0)
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"{case}: replay {r} output"
        assert torch.equal(w.state_pool.view(torch.int32), pool_e.view(torch.int32)), f"{case}: replay {r} states"
        w.state_pool.copy_(pool0)
        call(scratch)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
