"""CPU oracle of the KV append step — test infrastructure, never on the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module. It shares no code with the HIP library.

The step writes a batch's new tokens into the segments of their requests, ahead of attention.
The pages imply it without describing it (Flood README, "Introduction": each request's KV
cache is kept as a few contiguous segments of one shared pool instead of paged blocks; the
same README lists an FP8 KV cache among its features). Readings taken here:

- request b appends n_b = cu_new[b+1] - cu_new[b] tokens, and cu_k counts its keys *after*
  the append (the caller has already grown its segments): the new tokens are its last n_b
  keys, logical positions K_b - n_b .. K_b - 1, in the order of the new-token rows;
- a bf16 pool stores the rows as they are;
- an FP8 pool stores, per (token, kv head) row x of D bf16 values, one fp32 scale
  s = fp32(max|x| / 448) (s = 1 for an all-zero row) and the codes e4m3fn(clamp(x / s, ±448)),
  x / s computed as an fp32 division and the conversion rounding to nearest, ties to even
  (OCP E4M3FN: bias 7, largest finite 448);
- an INT8 pool (the INT8 KV cache of "FlashAttention on Ascend NPU", optimisation 3, which the
  page leaves at "quantise to INT8") stores per row the symmetric scale s = fp32(max|x| / 127)
  (1 for an all-zero row) and the codes round(clamp(x / s, ±127)) as two's-complement bytes,
  x / s again an fp32 division and the rounding to nearest, ties to even; -128 is never
  produced.
"""
from typing import Optional

import numpy as np

from .attention import request_slots

FP8_MAX = 448.0
INT8_MAX = 127.0


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (bfloat16 is the upper half of a binary32; exact)."""
    b = np.asarray(bits).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_e4m3fn(x) -> np.ndarray:
    """float32 values with |x| <= 448 -> OCP E4M3FN codes, rounding to nearest, ties to even.

    Normal codes hold (1 + m/8) * 2^(e-7) for exponent field e = 1..15, m = 0..7 (e = 15, m = 7
    is NaN, so 448 = 1.75 * 2^8 is the largest); exponent field 0 holds subnormals m/8 * 2^-6.
    The sign is bit 7 (so -0.0 -> 0x80)."""
    x = np.asarray(x, dtype=np.float32)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > FP8_MAX):
        raise ValueError("f32_to_e4m3fn expects finite values within +-448")
    a = np.abs(x).astype(np.float64)  # exact
    sign = np.signbit(x).astype(np.int64) << 7
    # subnormal range (and zero): multiples of 2^-9; a result of 8 is the smallest normal 2^-6,
    # which code 8 (exponent field 1, mantissa 0) also is
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    # normal range: a = f * 2^e with f in [1, 2) (frexp gives f in [0.5, 1))
    f, e2 = np.frexp(np.where(a > 0, a, 1.0))
    e = e2.astype(np.int64) - 1
    m = np.rint((f * 2.0 - 1.0) * 8.0).astype(np.int64)  # (f*2 - 1)*8 is exact for float32 a
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    normal = ((e + 7) << 3) | m
    code = np.where(a < 2.0 ** -6, sub, normal)
    return (code | sign).astype(np.uint8)


def quantize_rows(x_f32: np.ndarray):
    """Per-row FP8 encoding of float32 rows [..., D]: (codes uint8 [..., D], scales float32 [...])."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)  # float32 division, as the reading fixes
    y = np.clip(y, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return f32_to_e4m3fn(y), scale


def quantize_rows_int8(x_f32: np.ndarray):
    """Per-row INT8 encoding of float32 rows [..., D]: (codes as uint8 bytes [..., D], scales
    float32 [...]). The quotient is rounded to an integer with np.rint (ties to even)."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(INT8_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-INT8_MAX), np.float32(INT8_MAX))
    return np.rint(y).astype(np.int8).view(np.uint8), scale


def kv_append(k_new_bits, v_new_bits, segs, seg_indptr, cu_new, cu_k, k_pool, v_pool,
              k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
              fmt: str = "bf16"):
    """The pools after appending: copies of (k_pool, v_pool, k_scale, v_scale).

    k_new_bits / v_new_bits [T, Hkv, D] bf16 bit patterns (uint16), T = cu_new[B]; pools
    [pool_tokens, Hkv, D] uint16 (bf16) or uint8 (fp8 codes, int8 codes as bytes); scales
    [pool_tokens, Hkv] fp32 for fp8 and int8."""
    kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    ks = None if k_scale is None else np.array(k_scale, dtype=np.float32, copy=True)
    vs = None if v_scale is None else np.array(v_scale, dtype=np.float32, copy=True)
    cu_new = np.asarray(cu_new, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    for b in range(len(cu_new) - 1):
        n = int(cu_new[b + 1] - cu_new[b])
        K = int(cu_k[b + 1] - cu_k[b])
        if n == 0:
            continue
        slots = request_slots(segs, seg_indptr, b)
        if n > K or len(slots) != K:
            raise ValueError(f"request {b}: {n} new tokens, {K} keys, {len(slots)} segment slots")
        dst = slots[K - n:]
        src = slice(int(cu_new[b]), int(cu_new[b + 1]))
        if fmt == "bf16":
            kp[dst] = np.asarray(k_new_bits)[src]
            vp[dst] = np.asarray(v_new_bits)[src]
        elif fmt in ("fp8_e4m3", "int8"):
            quant = quantize_rows if fmt == "fp8_e4m3" else quantize_rows_int8
            kc, kscale = quant(bf16_bits_to_f32(np.asarray(k_new_bits)[src]))
            vc, vscale = quant(bf16_bits_to_f32(np.asarray(v_new_bits)[src]))
            kp[dst], ks[dst] = kc, kscale
            vp[dst], vs[dst] = vc, vscale
        else:
            raise ValueError(f"unknown KV format {fmt}")
    return kp, vp, ks, vs
