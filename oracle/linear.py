"""CPU float64 oracle of segment linear attention — test infrastructure, never on the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module. It shares no code with the HIP library.

The Flood README ("Kernels / Seg-linear-attn") benchmarks its segment linear attention against
flash-linear-attention's simple gated linear attention (chunked for prefill, recurrent for
decode) with 16 query and 16 kv heads of dimension 128. Simple GLA keeps, per request and head,
a d_k x d_v state S and a scalar log-decay g_t <= 0 per token and head:

    S_t = exp(g_t) S_{t-1} + k_t^T v_t,        o_t = scale * q_t S_t

Readings taken (the pages give only the kernel family and shapes):
  * "segment" for linear attention: each request's recurrent state lives in one slot of a shared
    state pool [slots, H, d_k, d_v] fp32 (the counterpart of a request's KV segments; the state
    does not grow with the sequence), named per request by a slot table;
  * a prefill call processes each request's tokens starting from its slot's state (or from zero)
    and writes the final state back to the slot; a decode call is the same for one token;
  * q, k, v are bf16, g is fp32, the state is fp32, the output bf16; scale defaults to d^-1/2.
This module evaluates the recurrence token by token, in float64.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import bf16_to_f64


def linear_attention(q_bits, k_bits, v_bits, g, cu_seqlens, state0: Optional[np.ndarray],
                     scale: float):
    """Outputs [T, H, D] and final states [B, H, D, D] (float64) of a varlen batch.

    q_bits, k_bits, v_bits: [T, H, D] bf16 bit patterns; g: [T, H] log decays; cu_seqlens:
    [B+1]; state0: [B, H, D, D] initial states (None: zero)."""
    q, k, v = bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits)
    g = np.asarray(g, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, D = q.shape
    B = len(cu) - 1
    out = np.zeros((T, H, D))
    states = np.zeros((B, H, D, D)) if state0 is None else np.array(state0, dtype=np.float64)
    for b in range(B):
        S = states[b]  # [H, D, D], updated in place
        for t in range(int(cu[b]), int(cu[b + 1])):
            decay = np.exp(g[t])[:, None, None]
            S *= decay
            S += k[t][:, :, None] * v[t][:, None, :]
            out[t] = scale * np.einsum("hi,hij->hj", q[t], S)
    return out, states


def linear_attention_closed_form(q_bits, k_bits, v_bits, g, cu_seqlens, state0, scale):
    """The same outputs written as explicit sums (a separate derivation, for the pins):
    o_t = scale [ exp(G_t) q_t S0 + sum_{s <= t} exp(G_t - G_s) (q_t . k_s) v_s ],
    with G_t the sum of the request's log decays from its first token up to and including t."""
    q, k, v = bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits)
    g = np.asarray(g, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, D = q.shape
    out = np.zeros((T, H, D))
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        G = np.cumsum(g[t0:t1], axis=0)  # [n, H]
        for t in range(t0, t1):
            i = t - t0
            acc = np.zeros((H, D))
            if state0 is not None:
                acc += np.exp(G[i])[:, None] * np.einsum("hi,hij->hj", q[t], state0[b])
            for s in range(t0, t + 1):
                j = s - t0
                w = np.exp(G[i] - G[j]) * np.einsum("hd,hd->h", q[t], k[s])
                acc += w[:, None] * v[s]
            out[t] = scale * acc
    return out
