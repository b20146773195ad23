"""Shared helpers for the GPU parity tests: run the library through its binding and the CPU
oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import workloads as wl

# Acceptance bar for bf16 outputs against the float64 oracle on bf16-rounded inputs.
MAX_ABS_TOL = 2e-2
RMS_TOL = 2e-3
# LSE is accumulated in fp32 from fp32 probabilities; 1e-3 absolute (natural log units).
LSE_TOL = 1e-3


def run_gpu(w: wl.Workload, *, num_splits: int = 0, return_lse: bool = True):
    import attention_segmented_kv_amd as sa
    if w.kind == "prefill":
        return sa.prefill(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_q,
                          w.cu_seqlens_k, w.max_seqlen_q, w.max_seqlen_k, causal=w.causal,
                          softmax_scale=w.softmax_scale, return_lse=return_lse)
    return sa.decode(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_k, w.max_seqlen_k,
                     k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale,
                     num_splits=num_splits, return_lse=return_lse)


def host_inputs(w: wl.Workload):
    segs, ind, cq, ck = wl.host_tables(w)
    ks = None if w.k_scale is None else w.k_scale.detach().cpu().numpy()
    vs = None if w.v_scale is None else w.v_scale.detach().cpu().numpy()
    return dict(q_bits=wl.bits(w.q), k_bits=wl.bits(w.k_pool), v_bits=wl.bits(w.v_pool), segs=segs,
                seg_indptr=ind, cu_q=cq, cu_k=ck, k_scale=ks, v_scale=vs)


def oracle_full(w: wl.Workload, h=None):
    h = h or host_inputs(w)
    return oracle.attention(h["q_bits"], h["k_bits"], h["v_bits"], h["segs"], h["seg_indptr"],
                            h["cu_q"], h["cu_k"], num_heads_kv=w.num_heads_kv,
                            softmax_scale=w.softmax_scale, causal=w.causal, kv_format=w.kv_dtype,
                            k_scale=h["k_scale"], v_scale=h["v_scale"])


def oracle_rows(w: wl.Workload, rows, h=None):
    h = h or host_inputs(w)
    return oracle.attention_rows(h["q_bits"], h["k_bits"], h["v_bits"], h["segs"], h["seg_indptr"],
                                 h["cu_q"], h["cu_k"], rows, num_heads_kv=w.num_heads_kv,
                                 softmax_scale=w.softmax_scale, causal=w.causal,
                                 kv_format=w.kv_dtype, k_scale=h["k_scale"], v_scale=h["v_scale"])


def errors(got: np.ndarray, ref: np.ndarray):
    d = got.astype(np.float64) - ref
    return float(np.abs(d).max(initial=0.0)), float(math.sqrt(np.mean(d * d))) if d.size else 0.0


def assert_close(got, ref, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, rms = errors(got, ref)
    assert mx <= MAX_ABS_TOL and rms <= RMS_TOL, f"{what}: max abs {mx:.3e}, rms {rms:.3e}"
    return mx, rms


def assert_lse_close(got, ref, what=""):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{what}: -inf pattern of LSE differs"
    if (~inf_ref).any():
        err = np.abs(got[~inf_ref] - ref[~inf_ref]).max()
        assert err <= LSE_TOL, f"{what}: LSE max abs err {err:.3e}"
