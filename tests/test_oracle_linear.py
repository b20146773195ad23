"""Pins of the segment-linear-attention oracle (CPU): the token-by-token recurrence against the
explicit decayed sums (outputs and final states), against causal linear attention written with
torch matmuls when nothing decays, against the single-token limit when everything decays, and
against itself split at any point with the state carried across."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def _tiny(seed, lens, h=2, d=8, with_state=True):
    w = wl.make_linear(seed, lens, num_heads=h, head_dim=d, poison=False)
    s0 = None
    if with_state:
        s0 = w.state_pool[w.state_slots.long()].double().numpy()
    return w, s0


def _run(w, s0, g=None):
    return oracle.linear_attention(wl.bits(w.q), wl.bits(w.k), wl.bits(w.v),
                                   w.g.numpy() if g is None else g, w.cu_seqlens.numpy(), s0, w.scale)


@pytest.mark.parametrize("with_state", [False, True])
def test_recurrence_equals_the_closed_form(with_state):
    w, s0 = _tiny(1, [5, 9, 1], with_state=with_state)
    o, _ = _run(w, s0)
    oc = oracle.linear_attention_closed_form(wl.bits(w.q), wl.bits(w.k), wl.bits(w.v), w.g.numpy(),
                                             w.cu_seqlens.numpy(), s0, w.scale)
    assert np.abs(o - oc).max() < 1e-12 * max(1.0, np.abs(oc).max())


def test_final_state_equals_the_decayed_sum():
    w, s0 = _tiny(2, [6, 4])
    _, st = _run(w, s0)
    k, v = oracle.bf16_to_f64(wl.bits(w.k)), oracle.bf16_to_f64(wl.bits(w.v))
    g = w.g.double().numpy()
    cu = w.cu_seqlens.numpy()
    for b in range(2):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        G = np.cumsum(g[t0:t1], axis=0)
        ref = np.exp(G[-1])[:, None, None] * s0[b]
        for s in range(t0, t1):
            ref += np.exp(G[-1] - G[s - t0])[:, None, None] * (k[s][:, :, None] * v[s][:, None, :])
        assert np.abs(st[b] - ref).max() < 1e-12


def test_no_decay_is_causal_linear_attention():
    w, _ = _tiny(3, [7, 12], h=3, d=16, with_state=False)
    zeros = np.zeros(tuple(w.g.shape))
    o, _ = _run(w, None, g=zeros)
    q, k, v = (t.double() for t in (w.q, w.k, w.v))
    cu = w.cu_seqlens.tolist()
    for b in range(2):
        sl = slice(cu[b], cu[b + 1])
        qb, kb, vb = (t[sl].transpose(0, 1) for t in (q, k, v))  # [H, n, d]
        a = torch.matmul(qb, kb.transpose(1, 2)).tril() * w.scale
        ref = torch.matmul(a, vb).transpose(0, 1).numpy()
        assert np.abs(o[sl] - ref).max() < 1e-12


def test_full_decay_keeps_only_the_current_token():
    w, s0 = _tiny(4, [5, 3])
    g = np.full(tuple(w.g.shape), -1e4)  # exp underflows to exactly 0
    o, st = _run(w, s0, g=g)
    q, k, v = (oracle.bf16_to_f64(wl.bits(t)) for t in (w.q, w.k, w.v))
    ref = w.scale * np.einsum("thd,thd->th", q, k)[:, :, None] * v
    assert np.abs(o - ref).max() < 1e-12
    last = [4, 7]
    for b in range(2):
        assert np.array_equal(st[b], k[last[b]][:, :, None] * v[last[b]][:, None, :])


@pytest.mark.parametrize("cut", [1, 4, 8])
def test_splitting_with_the_state_carried_changes_nothing(cut):
    w, s0 = _tiny(5, [9])
    o, st = _run(w, s0)
    q, k, v, g = wl.bits(w.q), wl.bits(w.k), wl.bits(w.v), w.g.numpy()
    o1, st1 = oracle.linear_attention(q[:cut], k[:cut], v[:cut], g[:cut], [0, cut], s0, w.scale)
    o2, st2 = oracle.linear_attention(q[cut:], k[cut:], v[cut:], g[cut:], [0, 9 - cut], st1, w.scale)
    assert np.array_equal(np.concatenate([o1, o2]), o) and np.array_equal(st2, st)
