"""CPU float64 oracle for attention over a segmentable KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no
code with the HIP library; it reads the raw bits of the inputs and decodes them itself.

What it computes is the plain definition of the attention that Flood's SegmentAttention
kernel evaluates (Flood README, "Introduction": the kernel works on a KV cache made of
segmentable blocks instead of paged blocks; "Kernels / Seg-attn": GQA with 64 query heads,
8 kv heads, head dim 128, compared against flash-attn's varlen forward):

    O[i, h] = sum_j softmax_j(scale * q[i, h] . k[j, g(h)] + mask[i, j]) v[j, g(h)]

for every request, over the keys that the request's segment table names, in table order.
Online softmax and split-K with a log-sum-exp merge are exact reformulations of this sum
(the running max m_i and normaliser l_i of "FlashAttention on Ascend NPU", bottleneck 2; the
blockwise partial results reduced per request of the FlashAccel article, "data layout"), so
the oracle evaluates the definition directly and, separately, the blockwise split-and-merge
form (`split_merge`) whose agreement with the direct form is one of the pins.

Readings of points the pages leave open (each one is listed with its reason in the design
notes):
  * query head h uses kv head h // (Hq / Hkv): consecutive query heads share a kv head, the
    convention of the varlen flash-attn call the Seg-attn table compares against;
  * causal masking is aligned bottom-right: query i of a request with Lq queries and K keys
    sits at absolute position K - Lq + i and sees keys j <= K - Lq + i (chunked prefill, a
    listed Flood feature, needs exactly this; decode then sees every key);
  * a request's logical key order is the order of its segments in the table;
  * pool layout is token-major [pool_tokens, Hkv, D]; FP8 pools are OCP E4M3FN codes times
    one fp32 scale per (token, kv head), INT8 pools two's-complement int8 codes times one fp32
    scale per (token, kv head) (the INT8 KV cache of "FlashAttention on Ascend NPU",
    optimisation 3, with the FP8 cache's per-row scale);
  * a query row with no visible key returns O = 0 and LSE = -inf.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


# ----------------------------------------------------------------------------------------------
# exact decoding of the stored number formats


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper 16 bits of an IEEE-754 binary32 value; widening is exact."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point, E4M3 'FN' variant: 1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; no infinities; the two
    codes with all exponent and mantissa bits set (0x7F, 0xFF) are NaN."""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    out = np.where((b & 0x7F) == 0x7F, np.nan, out)
    return out


def int8_to_f64(bits: np.ndarray) -> np.ndarray:
    """Bytes read as two's-complement 8-bit integers (0x80..0xFF are -128..-1)."""
    return np.asarray(bits).astype(np.uint8).view(np.int8).astype(np.float64)


# The 256 E4M3FN codes decoded once by the definition above; decoding a pool is then a table
# lookup with the same values (the definition's arithmetic per element is slow on long pools).
_E4M3FN_VALUES = e4m3fn_to_f64(np.arange(256))


def decode_kv(bits: np.ndarray, scale: Optional[np.ndarray], fmt: str) -> np.ndarray:
    """Decoded K or V rows [n, Hkv, D] in float64. For FP8 and INT8 the code is multiplied by
    its per-(token, kv head) fp32 scale; the product of two such numbers is exact in float64."""
    if fmt == "bf16":
        return bf16_to_f64(bits)
    if fmt == "fp8_e4m3":
        return _E4M3FN_VALUES[np.asarray(bits).astype(np.uint8)] * np.asarray(scale, dtype=np.float64)[..., None]
    if fmt == "int8":
        return int8_to_f64(bits) * np.asarray(scale, dtype=np.float64)[..., None]
    raise ValueError(f"unknown kv format {fmt}")


# ----------------------------------------------------------------------------------------------
# segment tables


def request_slots(segs: np.ndarray, seg_indptr: np.ndarray, b: int) -> np.ndarray:
    """Pool slot of every key of request b: the segments' ranges [off, off + len) concatenated
    in table order."""
    rows = np.asarray(segs, dtype=np.int64).reshape(-1, 2)[int(seg_indptr[b]):int(seg_indptr[b + 1])]
    parts = [np.arange(off, off + ln, dtype=np.int64) for off, ln in rows.tolist()]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def visible_keys(lq: int, k: int, causal: bool) -> np.ndarray:
    """How many leading keys each of the lq query rows may see (bottom-right causal)."""
    if not causal:
        return np.full(lq, k, dtype=np.int64)
    return np.clip(k - lq + 1 + np.arange(lq, dtype=np.int64), 0, k)


# ----------------------------------------------------------------------------------------------
# the definition


def attend(qh: np.ndarray, kg: np.ndarray, vg: np.ndarray, scale: float,
           visible: np.ndarray, return_weights: bool = False):
    """softmax(scale * qh kg^T + mask) vg for query rows qh [n, D], keys kg/vg [K, D]; row r
    sees keys [0, visible[r]). Returns O [n, D], LSE [n] (natural log) and optionally W."""
    n, K = qh.shape[0], kg.shape[0]
    s = scale * (qh @ kg.T) if K else np.zeros((n, 0))
    masked = np.arange(K)[None, :] >= visible[:, None]
    s = np.where(masked, NEG_INF, s)
    m = s.max(axis=1, initial=NEG_INF)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])
    p = np.where(masked, 0.0, p)
    l = p.sum(axis=1)
    w = p / np.where(empty, 1.0, l)[:, None]
    o = w @ vg if K else np.zeros((n, vg.shape[1]))
    o = np.where(empty[:, None], 0.0, o)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, m_safe + np.log(np.where(empty, 1.0, l)))
    if return_weights:
        return o, lse, w
    return o, lse


def attention(q_bits, k_bits, v_bits, segs, seg_indptr, cu_q, cu_k, *, num_heads_kv: int,
              softmax_scale: float, causal: bool, kv_format: str = "bf16",
              k_scale=None, v_scale=None, requests: Optional[Iterable[int]] = None):
    """Attention for every query row of the selected requests (all by default).

    q_bits [total_q, Hq, D] uint16 (bf16 bits); k_bits/v_bits [pool, Hkv, D] uint16 or uint8
    (E4M3FN codes); k_scale/v_scale [pool, Hkv] fp32 for FP8. Returns O [total_q, Hq, D] and
    LSE [total_q, Hq] in float64; rows of unselected requests are NaN."""
    q_bits = np.asarray(q_bits)
    total_q, hq, d = q_bits.shape
    group = hq // num_heads_kv
    assert group * num_heads_kv == hq
    o = np.full((total_q, hq, d), np.nan)
    lse = np.full((total_q, hq), np.nan)
    batch = len(cu_q) - 1
    for b in (range(batch) if requests is None else requests):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        kb = int(cu_k[b + 1]) - int(cu_k[b])
        slots = request_slots(segs, seg_indptr, b)
        if len(slots) != kb:
            raise ValueError(f"request {b}: segments hold {len(slots)} keys, cu_seqlens_k says {kb}")
        if q1 == q0:
            continue
        kd = decode_kv(np.asarray(k_bits)[slots], None if k_scale is None else np.asarray(k_scale)[slots], kv_format)
        vd = decode_kv(np.asarray(v_bits)[slots], None if v_scale is None else np.asarray(v_scale)[slots], kv_format)
        qd = bf16_to_f64(q_bits[q0:q1])
        vis = visible_keys(q1 - q0, kb, causal)
        for h in range(hq):
            g = h // group
            oh, lh = attend(qd[:, h, :], kd[:, g, :], vd[:, g, :], softmax_scale, vis)
            o[q0:q1, h, :] = oh
            lse[q0:q1, h] = lh
    return o, lse


def attention_rows(q_bits, k_bits, v_bits, segs, seg_indptr, cu_q, cu_k,
                   rows: Sequence[Tuple[int, int, int]], *, num_heads_kv: int,
                   softmax_scale: float, causal: bool, kv_format: str = "bf16",
                   k_scale=None, v_scale=None):
    """Attention for individual (request b, query index i within b, query head h) rows.

    Used on workloads too large to evaluate whole: each row gathers only its request's keys.
    Returns O [len(rows), D] and LSE [len(rows)] in float64."""
    q_bits = np.asarray(q_bits)
    hq, d = q_bits.shape[1], q_bits.shape[2]
    group = hq // num_heads_kv
    out = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    by_req = {}
    for r, (b, i, h) in enumerate(rows):
        by_req.setdefault(int(b), []).append((r, int(i), int(h)))
    for b, items in by_req.items():
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        kb = int(cu_k[b + 1]) - int(cu_k[b])
        slots = request_slots(segs, seg_indptr, b)
        if len(slots) != kb:
            raise ValueError(f"request {b}: segments hold {len(slots)} keys, cu_seqlens_k says {kb}")
        heads = sorted({h // group for _, _, h in items})
        for g in heads:
            kd = decode_kv(np.asarray(k_bits)[slots, g:g + 1],
                           None if k_scale is None else np.asarray(k_scale)[slots, g:g + 1], kv_format)[:, 0]
            vd = decode_kv(np.asarray(v_bits)[slots, g:g + 1],
                           None if v_scale is None else np.asarray(v_scale)[slots, g:g + 1], kv_format)[:, 0]
            vis_all = visible_keys(q1 - q0, kb, causal)
            for r, i, h in items:
                if h // group != g:
                    continue
                qh = bf16_to_f64(q_bits[q0 + i, h])[None, :]
                oh, lh = attend(qh, kd, vd, softmax_scale, vis_all[i:i + 1])
                out[r] = oh[0]
                lse[r] = lh[0]
    return out, lse


# ----------------------------------------------------------------------------------------------
# blockwise form: partial results per key block, reduced per request


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine per-block results (O_s [S, n, D], LSE_s [S, n]) of disjoint key blocks:
    LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s. Blocks with LSE_s = -inf
    contribute nothing; if all are -inf the row is empty (O = 0, LSE = -inf)."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0)
    empty = ~np.isfinite(mx)
    mx_safe = np.where(empty, 0.0, mx)
    wts = np.exp(lse_parts - mx_safe[None, :])
    tot = wts.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, mx_safe + np.log(np.where(empty, 1.0, tot)))
    coef = np.where(empty[None, :], 0.0, np.exp(lse_parts - np.where(empty, 0.0, lse)[None, :]))
    o = np.einsum("sn,snd->nd", coef, o_parts)
    return o, lse


def split_merge(qh: np.ndarray, kg: np.ndarray, vg: np.ndarray, scale: float,
                visible: np.ndarray, boundaries: Sequence[int]):
    """The split-K form: keys cut at ``boundaries`` (0 = b_0 <= b_1 <= ... <= b_S = K) into
    blocks; each block's partial attention (restricted to visible keys inside it) is computed
    on its own and the partials are merged with `merge_partials`."""
    parts_o, parts_l = [], []
    for a, e in zip(boundaries[:-1], boundaries[1:]):
        vis_block = np.clip(visible - a, 0, e - a)
        o_s, l_s = attend(qh, kg[a:e], vg[a:e], scale, vis_block)
        parts_o.append(o_s)
        parts_l.append(l_s)
    return merge_partials(np.stack(parts_o), np.stack(parts_l))
