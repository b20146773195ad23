"""Pins of the KV-append oracle (CPU): the E4M3FN encoder against torch's float8 conversion,
every code and hand-worked ties; the FP8 and INT8 row quantisers' scales, extremes and ties
(INT8 also against torch's division and rounding); the append against what it must leave in
the pool, read back through the segment tables."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _torch_e4m3fn(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        (rng.standard_normal(100_000) * 100).clip(-448, 448),
        rng.standard_normal(50_000) * 0.01,        # subnormal codes
        rng.uniform(-448, 448, 50_000),
    ]).astype(np.float32)
    assert np.array_equal(oracle.f32_to_e4m3fn(x), _torch_e4m3fn(x))


def test_encoder_round_trips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]  # 0x7F, 0xFF are NaN
    vals = oracle.e4m3fn_to_f64(codes).astype(np.float32)
    vals = np.where(codes == 0x80, np.float32(-0.0), vals)
    assert np.array_equal(oracle.f32_to_e4m3fn(vals), codes)


def test_encoder_ties_go_to_even_codes():
    # hand-worked: 1.0 = 0x38 and 1.125 = 0x39, so 1.0625 -> 0x38; 1.1875 lies between 0x39 and
    # 1.25 = 0x3A -> 0x3A; 2^-10 is half the smallest subnormal 2^-9 -> 0; 3 * 2^-10 lies between
    # 2^-9 (0x01) and 2^-8 (0x02) -> 0x02; 432 lies between 416 (0x7D) and 448 (0x7E) -> 0x7E
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 432.0, -1.0625], dtype=np.float32)
    assert oracle.f32_to_e4m3fn(x).tolist() == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0xB8]
    # every midpoint between adjacent positive codes, and torch agrees
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    v = oracle.e4m3fn_to_f64(pos)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    enc = oracle.f32_to_e4m3fn(mids)
    assert np.all(enc % 2 == 0)
    assert np.array_equal(enc, _torch_e4m3fn(mids))


def test_encoder_error_is_at_most_half_a_step():
    rng = np.random.default_rng(1)
    x = rng.uniform(-448, 448, 20_000).astype(np.float32)
    dec = oracle.e4m3fn_to_f64(oracle.f32_to_e4m3fn(x))
    a = np.abs(x.astype(np.float64))
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(dec - x) <= step / 2)


def test_quantize_rows_scale_extremes_and_zero_rows():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 8, 128)).astype(np.float32)
    x[3, 5] = 0.0
    codes, scale = oracle.quantize_rows(x)
    amax = np.abs(x).max(axis=-1)
    expect = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    assert np.array_equal(scale, expect)
    assert scale[3, 5] == 1.0 and not codes[3, 5].any()
    # the largest-magnitude element of a nonzero row encodes as +-448 (0x7E / 0xFE)
    idx = np.abs(x).argmax(axis=-1)
    top = np.take_along_axis(codes, idx[..., None], axis=-1)[..., 0]
    nz = amax > 0
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # decoded rows are within half a code step of the input: at most 16 code units (the step is
    # 32 in the top binade, 256..448) times the stored scale; exact ties reach the bound
    dec = oracle.e4m3fn_to_f64(codes) * scale[..., None]
    assert np.all(np.abs(dec - x) <= scale[..., None].astype(np.float64) * 16.0 * (1 + 1e-6))


def _torch_fp8_rows(x: np.ndarray):
    """torch's own fp32 division, clamp and float8_e4m3fn cast (round to nearest, ties to even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = t.abs().amax(dim=-1)
    sc = torch.where(amax > 0, amax / torch.tensor(448.0), torch.ones_like(amax))
    q = (t / sc.unsqueeze(-1)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), sc.numpy()


def _positive_bf16_values() -> np.ndarray:
    """Every positive normal bf16 value, as float32."""
    return (np.arange(0x0080, 0x7F80, dtype=np.uint32) << 16).view(np.float32)


def _crafted_fp8_rows():
    """Rows [amax, x, 0, ...] of bf16 values chosen so that the fp32 quotient x / s (s = amax/448)
    decides the code where plausible mistakes decide it differently:
      * 'tie' rows: fl32(x / s) is exactly the midpoint of two adjacent codes while the exact
        quotient is not, so rounding the exact (fp64) quotient straight to a code differs from
        ties-to-even on the fp32 quotient whenever the even code lies on the other side;
      * 'recip' rows: x * fl32(1 / s) rounds to another code than x / s."""
    xs_all = _positive_bf16_values()
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    v = oracle.e4m3fn_to_f64(codes)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    tie, recip = [], []
    for amax in xs_all[(xs_all >= 0.01) & (xs_all <= 1000.0)][::7]:
        s = np.float32(amax / np.float32(448))
        xs = xs_all[xs_all < amax]
        q32 = xs / s
        on_mid = np.isin(q32, mids) & (xs.astype(np.float64) / np.float64(s) != q32)
        tie += [(amax, x) for x in xs[on_mid][:2]]
        qr = xs * np.float32(np.float32(1) / s)
        diff = oracle.f32_to_e4m3fn(np.minimum(qr, 448)) != oracle.f32_to_e4m3fn(np.minimum(q32, 448))
        recip += [(amax, x) for x in xs[diff][:2]]
    rows = np.zeros((len(tie) + len(recip), 128), dtype=np.float32)
    for i, (a, x) in enumerate(tie + recip):
        rows[i, 0], rows[i, 1] = a, x
        rows[i, 2], rows[i, 3] = -a, -x  # the negative twins take the mirrored codes
    return rows, len(tie), len(recip)


def _nearest_code_f64(q: np.ndarray) -> np.ndarray:
    """Mutant encoder for the pin below: the code nearest to an fp64 value (no fp32 step)."""
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    v = oracle.e4m3fn_to_f64(pos)
    a = np.abs(q)
    idx = np.abs(a[..., None] - v).argmin(axis=-1)
    return (pos[idx] | (np.signbit(q).astype(np.uint8) << 7)).astype(np.uint8)


def test_fp8_quantiser_matches_torch_and_catches_plausible_mistakes():
    """The FP8 row quantiser (the reading of the KV append: s = fl32(amax / 448) and codes
    E4M3FN(clamp(x / s, +-448)) from a correctly rounded fp32 quotient, ties to even) against
    torch's own division and float8 cast: random bf16 rows over many magnitudes, plus crafted
    rows on which dividing in fp64 and rounding once, or multiplying by the reciprocal, give
    other codes (checked below, so the pin would see either mistake)."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal((300, 8, 128)),
                        rng.standard_normal((40, 8, 128)) * 1e-30,
                        rng.uniform(-1e4, 1e4, (40, 8, 128))]).astype(np.float32)
    x = oracle.bf16_bits_to_f32((x.view(np.uint32) >> 16).astype(np.uint16))  # bf16 values
    codes, scale = oracle.quantize_rows(x)
    tc, ts = _torch_fp8_rows(x)
    assert np.array_equal(scale, ts) and np.array_equal(codes, tc)

    rows, n_tie, n_recip = _crafted_fp8_rows()
    assert n_tie >= 20 and n_recip >= 20
    codes, scale = oracle.quantize_rows(rows)
    tc, ts = _torch_fp8_rows(rows)
    assert np.array_equal(scale, ts) and np.array_equal(codes, tc)
    s = scale[:, None]
    # mutant 1: the exact quotient rounded straight to a code
    m1 = _nearest_code_f64(np.clip(rows.astype(np.float64) / s.astype(np.float64), -448, 448))
    assert (m1[:n_tie] != tc[:n_tie]).any(axis=1).sum() >= n_tie // 4
    # mutant 2: multiply by the fp32 reciprocal of the scale
    m2 = oracle.f32_to_e4m3fn(np.clip(rows * (np.float32(1) / s).astype(np.float32), -448, 448))
    assert (m2[n_tie:] != tc[n_tie:]).any(axis=1).all()


def _torch_int8_rows(x: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = t.abs().amax(dim=-1)
    sc = torch.where(amax > 0, amax / torch.tensor(127.0), torch.ones_like(amax))
    q = torch.round((t / sc.unsqueeze(-1)).clamp(-127.0, 127.0)).to(torch.int8)
    return q.view(torch.uint8).numpy(), sc.numpy()


def test_int8_quantiser_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal((300, 8, 128)),
                        rng.standard_normal((40, 8, 128)) * 1e-30,
                        rng.uniform(-1e4, 1e4, (40, 8, 128))]).astype(np.float32)
    x = oracle.bf16_bits_to_f32((x.view(np.uint32) >> 16).astype(np.uint16))  # bf16 values
    codes, scale = oracle.quantize_rows_int8(x)
    tc, ts = _torch_int8_rows(x)
    assert np.array_equal(scale, ts) and np.array_equal(codes, tc)


def test_int8_quantiser_ties_extremes_and_zero_rows():
    # a row whose largest magnitude is 127 has scale exactly 1, so x / s = x: the hand-worked
    # ties 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, -0.5 -> 0, 126.5 -> 126
    row = np.zeros(128, dtype=np.float32)
    vals = [0.5, 1.5, 2.5, 3.5, -2.5, -0.5, 126.5, 127.0, -127.0, 5.0]
    row[:len(vals)] = vals
    codes, scale = oracle.quantize_rows_int8(row[None])
    assert scale[0] == 1.0
    got = codes[0, :len(vals)].view(np.int8).tolist()
    assert got == [0, 2, 2, 4, -2, 0, 126, 127, -127, 5]
    # zero row: scale 1, all codes 0; the extreme element of any other row is +-127; the error
    # is at most half a step (exact ties reach it) plus the quotient's fp32 rounding
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 8, 128)).astype(np.float32)
    x[7, 2] = 0.0
    codes, scale = oracle.quantize_rows_int8(x)
    assert scale[7, 2] == 1.0 and not codes[7, 2].any()
    c = codes.view(np.int8).astype(np.int64)
    idx = np.abs(x).argmax(axis=-1)
    top = np.take_along_axis(c, idx[..., None], axis=-1)[..., 0]
    nz = np.abs(x).max(axis=-1) > 0
    assert np.all(np.abs(top[nz]) == 127) and c.min() >= -127
    dec = c * scale[..., None].astype(np.float64)
    # half a step, plus the fp32 rounding of the quotient (at most 127 * 2^-24 steps)
    assert np.all(np.abs(dec - x) <= scale[..., None].astype(np.float64) * (0.5 + 2.0 ** -16))


@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3", "int8"])
def test_kv_append_writes_the_last_keys_and_nothing_else(fmt):
    gen = torch.Generator().manual_seed(3)
    # four requests with segments (one with none), new tokens at the end of each
    w = wl.make_random(3, batch=4, q_lens=[1] * 4, k_lens=[50, 0, 130, 7], max_segs=4, kind="decode",
                       kv_dtype=fmt, zero_length_segments=True)
    segs, ind, _, ck = wl.host_tables(w)
    n_new = [5, 0, 130, 1]
    cu_new = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    T, hkv, d = int(cu_new[-1]), 8, 128
    k_new = wl.bits(torch.randn(T, hkv, d, generator=gen).to(torch.bfloat16))
    v_new = wl.bits(torch.randn(T, hkv, d, generator=gen).to(torch.bfloat16))
    kp0, vp0 = wl.bits(w.k_pool), wl.bits(w.v_pool)
    ks0 = None if w.k_scale is None else w.k_scale.numpy().copy()
    vs0 = None if w.v_scale is None else w.v_scale.numpy().copy()
    kp, vp, ks, vs = oracle.kv_append(k_new, v_new, segs, ind, cu_new, ck, kp0, vp0, ks0, vs0, fmt=fmt)
    touched = np.zeros(kp0.shape[0], dtype=bool)
    for b in range(4):
        K, n = int(ck[b + 1] - ck[b]), n_new[b]
        slots = oracle.request_slots(segs, ind, b)[K - n:]
        touched[slots] = True
        src = slice(int(cu_new[b]), int(cu_new[b + 1]))
        if fmt == "bf16":
            assert np.array_equal(kp[slots], k_new[src]) and np.array_equal(vp[slots], v_new[src])
        elif fmt == "int8":
            for pool, sc, new in ((kp, ks, k_new), (vp, vs, v_new)):
                x = oracle.bf16_to_f64(new[src])
                amax = np.abs(x).max(axis=-1)
                assert np.array_equal(sc[slots], np.where(amax > 0, amax.astype(np.float32) / np.float32(127), 1))
                dec = oracle.int8_to_f64(pool[slots]) * sc[slots][..., None]
                # half a step, plus the fp32 rounding of the quotient (at most 127 * 2^-24 steps)
                assert np.all(np.abs(dec - x) <= sc[slots][..., None].astype(np.float64) * (0.5 + 2.0 ** -16))
        else:
            for pool, sc, new in ((kp, ks, k_new), (vp, vs, v_new)):
                x = oracle.bf16_to_f64(new[src])
                amax = np.abs(x).max(axis=-1)
                assert np.array_equal(sc[slots], np.where(amax > 0, amax.astype(np.float32) / np.float32(448), 1))
                dec = oracle.e4m3fn_to_f64(pool[slots]) * sc[slots][..., None]
                assert np.all(np.abs(dec - x) <= sc[slots][..., None].astype(np.float64) * 16.0 * (1 + 1e-6))
    # every other slot (and scale) is left as it was
    assert np.array_equal(kp[~touched], kp0[~touched]) and np.array_equal(vp[~touched], vp0[~touched])
    if fmt != "bf16":
        assert np.array_equal(ks[~touched], ks0[~touched], equal_nan=True)
        assert np.array_equal(vs[~touched], vs0[~touched], equal_nan=True)


def test_kv_append_rejects_more_new_tokens_than_keys():
    w = wl.make_random(4, batch=1, q_lens=[1], k_lens=[3], max_segs=1, kind="decode")
    segs, ind, _, ck = wl.host_tables(w)
    z = np.zeros((4, 8, 128), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.kv_append(z, z, segs, ind, [0, 4], ck, wl.bits(w.k_pool), wl.bits(w.v_pool))
