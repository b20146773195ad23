"""Pins for the CPU oracle: each test checks it against something other than itself.

* number formats: the oracle's bf16, E4M3FN and INT8 decoders against torch's own conversions
  for every code, plus points fixed by the OCP FP8 definition;
* brute force: an independent pure-Python evaluation (per-key segment lookup, absolute
  positions, math.exp / math.fsum) on tiny inputs;
* a library routine: torch's scaled_dot_product_attention in float64 with an explicit mask;
* closed forms and invariants: weights sum to one, constant V, a single visible key, Q = 0,
  a hand-worked two-key case, re-layout into other segments, split-K merging, chunked prefill
  equal to the suffix of a full prefill, GQA equal to MHA with replicated kv heads, a shift of
  every key, poisoned unreferenced slots.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def _tiny(seed, batch=2, hq=4, hkv=2, d=8, causal=True, kv_dtype="bf16", max_q=5, max_k=9,
          zero_len=False, lq_eq_k=False):
    rng = np.random.default_rng(seed)
    ks = rng.integers(1, max_k + 1, size=batch)
    if lq_eq_k:
        qs = ks.copy()
    else:
        qs = np.array([int(rng.integers(1, min(max_q, int(k)) + 1)) for k in ks])
    return wl.make_random(seed, batch=batch, q_lens=qs.tolist(), k_lens=ks.tolist(), max_segs=4,
                          causal=causal, kv_dtype=kv_dtype, num_heads_q=hq, num_heads_kv=hkv,
                          head_dim=d, zero_length_segments=zero_len)


def _run_oracle(w, **kw):
    segs, ind, cq, ck = wl.host_tables(w)
    return oracle.attention(wl.bits(w.q), wl.bits(w.k_pool), wl.bits(w.v_pool), segs, ind, cq, ck,
                            num_heads_kv=w.num_heads_kv, softmax_scale=w.softmax_scale,
                            causal=w.causal, kv_format=w.kv_dtype,
                            k_scale=None if w.k_scale is None else w.k_scale.numpy(),
                            v_scale=None if w.v_scale is None else w.v_scale.numpy(), **kw)


# ------------------------------------------------------------------------------ number formats

def test_bf16_decoder_matches_torch_for_every_code():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3fn_decoder_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_int8_decoder_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    ours = oracle.int8_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.int8).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    assert ours[0x7F] == 127 and ours[0x80] == -128 and ours[0xFF] == -1


def test_e4m3fn_fixed_points_of_the_format():
    # OCP 8-bit FP, E4M3: bias 7, max normal S.1111.110 = 448, min normal 2^-6,
    # min subnormal 2^-9, 1.0 = 0.0111.000, NaN = S.1111.111, negative zero 0x80.
    pts = {0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0,
           0xB8: -1.0, 0x07: 7 * 2.0 ** -9, 0x77: 240.0}
    got = oracle.e4m3fn_to_f64(np.array(list(pts), dtype=np.uint8))
    assert got.tolist() == list(pts.values())
    assert np.isnan(oracle.e4m3fn_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    z = oracle.e4m3fn_to_f64(np.array([0x80], dtype=np.uint8))[0]
    assert z == 0.0 and math.copysign(1.0, z) < 0


# ------------------------------------------------------------------------------ brute force

def _brute(w):
    """Independent evaluation: each logical key's slot by walking the segment table, absolute
    query positions for the causal test, scalar math.exp and math.fsum."""
    segs, ind, cq, ck = wl.host_tables(w)
    qf = w.q.to(torch.float64).numpy()
    if w.kv_dtype in ("fp8_e4m3", "int8"):
        kf = w.k_pool.to(torch.float64).numpy() * w.k_scale.to(torch.float64).numpy()[..., None]
        vf = w.v_pool.to(torch.float64).numpy() * w.v_scale.to(torch.float64).numpy()[..., None]
    else:
        kf = w.k_pool.to(torch.float64).numpy()
        vf = w.v_pool.to(torch.float64).numpy()
    hq, hkv, d = w.num_heads_q, w.num_heads_kv, w.head_dim
    out = np.full((int(cq[-1]), hq, d), np.nan)
    lse = np.full((int(cq[-1]), hq), np.nan)
    for b in range(len(cq) - 1):
        lq = int(cq[b + 1] - cq[b])
        kk = int(ck[b + 1] - ck[b])

        def slot(j):
            start = 0
            for s in range(int(ind[b]), int(ind[b + 1])):
                off, ln = int(segs[s, 0]), int(segs[s, 1])
                if start <= j < start + ln:
                    return off + (j - start)
                start += ln
            raise AssertionError("key outside segments")

        slots = [slot(j) for j in range(kk)]
        for i in range(lq):
            pos = kk - lq + i
            for h in range(hq):
                g = h * hkv // hq
                logits = []
                for j in range(kk):
                    if w.causal and j > pos:
                        continue
                    dot = math.fsum(qf[cq[b] + i, h, t] * kf[slots[j], g, t] for t in range(d))
                    logits.append((j, w.softmax_scale * dot))
                if not logits:
                    out[cq[b] + i, h] = 0.0
                    lse[cq[b] + i, h] = -math.inf
                    continue
                mx = max(x for _, x in logits)
                e = [(j, math.exp(x - mx)) for j, x in logits]
                z = math.fsum(p for _, p in e)
                for t in range(d):
                    out[cq[b] + i, h, t] = math.fsum(p * vf[slots[j], g, t] for j, p in e) / z
                lse[cq[b] + i, h] = mx + math.log(z)
    return out, lse


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("causal", [True, False])
def test_oracle_equals_brute_force(seed, causal):
    w = _tiny(seed, batch=3 if seed % 2 else 2, hq=[2, 4, 8][seed % 3], hkv=[1, 2, 2][seed % 3],
              d=[4, 8, 16][seed % 3], causal=causal, zero_len=(seed % 2 == 0))
    o, l = _run_oracle(w)
    ob, lb = _brute(w)
    assert np.abs(o - ob).max() < 1e-12
    assert np.abs(l - lb).max() < 1e-12


def test_oracle_equals_brute_force_fp8():
    w = _tiny(11, batch=2, hq=4, hkv=2, d=8, kv_dtype="fp8_e4m3")
    o, l = _run_oracle(w)
    ob, lb = _brute(w)
    assert np.abs(o - ob).max() < 1e-12
    assert np.abs(l - lb).max() < 1e-12


def test_oracle_equals_brute_force_int8():
    w = _tiny(12, batch=3, hq=4, hkv=2, d=8, kv_dtype="int8", zero_len=True)
    o, l = _run_oracle(w)
    ob, lb = _brute(w)
    assert np.abs(o - ob).max() < 1e-12
    assert np.abs(l - lb).max() < 1e-12


def test_oracle_equals_brute_force_full_head_dim():
    w = _tiny(21, batch=1, hq=8, hkv=1, d=128, max_k=6)
    o, l = _run_oracle(w)
    ob, lb = _brute(w)
    assert np.abs(o - ob).max() < 1e-12
    assert np.abs(l - lb).max() < 1e-12


# ------------------------------------------------------------------------------ library routine

def _sdpa(w):
    segs, ind, cq, ck = wl.host_tables(w)
    q = w.q.to(torch.float64)
    if w.kv_dtype in ("fp8_e4m3", "int8"):
        kp = w.k_pool.to(torch.float64) * w.k_scale.to(torch.float64)[..., None]
        vp = w.v_pool.to(torch.float64) * w.v_scale.to(torch.float64)[..., None]
    else:
        kp, vp = w.k_pool.to(torch.float64), w.v_pool.to(torch.float64)
    rep = w.num_heads_q // w.num_heads_kv
    outs = []
    for b in range(len(cq) - 1):
        pieces = [kp[o:o + n] for o, n in segs[ind[b]:ind[b + 1]].tolist()]
        vpieces = [vp[o:o + n] for o, n in segs[ind[b]:ind[b + 1]].tolist()]
        kb = torch.cat(pieces).repeat_interleave(rep, dim=1).transpose(0, 1)  # [Hq, K, d]
        vb = torch.cat(vpieces).repeat_interleave(rep, dim=1).transpose(0, 1)
        qb = q[cq[b]:cq[b + 1]].transpose(0, 1)  # [Hq, Lq, d]
        lq, kk = qb.shape[1], kb.shape[1]
        if w.causal:
            mask = torch.ones(lq, kk, dtype=torch.bool).tril(diagonal=kk - lq)
        else:
            mask = torch.ones(lq, kk, dtype=torch.bool)
        ob = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask,
                                                             scale=w.softmax_scale)
        outs.append(ob.transpose(0, 1))
    return torch.cat(outs).numpy()


@pytest.mark.parametrize("seed", range(4))
def test_oracle_equals_torch_sdpa(seed):
    w = wl.make_random(100 + seed, batch=3, q_lens=[5, 1, 17], k_lens=[9, 30, 40], max_segs=5,
                       num_heads_q=8, num_heads_kv=2, head_dim=32,
                       kv_dtype="fp8_e4m3" if seed == 3 else "bf16")
    o, _ = _run_oracle(w)
    assert np.abs(o - _sdpa(w)).max() < 1e-12


def test_oracle_equals_torch_sdpa_int8():
    w = wl.make_random(104, batch=3, q_lens=[4, 1, 9], k_lens=[12, 33, 20], max_segs=4,
                       num_heads_q=8, num_heads_kv=2, head_dim=32, kv_dtype="int8")
    o, _ = _run_oracle(w)
    assert np.abs(o - _sdpa(w)).max() < 1e-12


def test_oracle_equals_torch_sdpa_noncausal():
    w = wl.make_random(7, batch=2, q_lens=[6, 3], k_lens=[11, 4], max_segs=3, causal=False,
                       num_heads_q=4, num_heads_kv=4, head_dim=16)
    o, _ = _run_oracle(w)
    assert np.abs(o - _sdpa(w)).max() < 1e-12


# ------------------------------------------------------------------------------ closed forms

def test_weights_sum_to_one_and_lse_is_log_partition():
    rng = np.random.default_rng(0)
    qh, kg = rng.standard_normal((7, 16)), rng.standard_normal((12, 16))
    vg = rng.standard_normal((12, 16))
    vis = oracle.visible_keys(7, 12, True)
    o, lse, w = oracle.attend(qh, kg, vg, 0.25, vis, return_weights=True)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-14, rtol=0)
    for r in range(7):
        s = [0.25 * float(qh[r] @ kg[j]) for j in range(vis[r])]
        assert abs(lse[r] - math.log(math.fsum(math.exp(x) for x in s))) < 1e-12
        assert np.all(w[r, vis[r]:] == 0.0)


def test_constant_v_returns_that_row():
    rng = np.random.default_rng(1)
    c = rng.standard_normal(8)
    o, _ = oracle.attend(rng.standard_normal((5, 8)), rng.standard_normal((9, 8)),
                         np.tile(c, (9, 1)), 0.3, oracle.visible_keys(5, 9, True))
    assert np.abs(o - c).max() < 1e-14


def test_single_visible_key_returns_its_value_exactly():
    w = wl.make_random(3, batch=1, q_lens=[6], k_lens=[6], max_segs=3, num_heads_q=4,
                       num_heads_kv=2, head_dim=8)
    o, lse = _run_oracle(w)
    segs, ind, _, _ = wl.host_tables(w)
    slot0 = int(segs[0, 0])
    v0 = w.v_pool[slot0].to(torch.float64).numpy()  # [Hkv, d]
    for h in range(4):
        assert np.array_equal(o[0, h], v0[h // 2])
        q0 = w.q[0, h].to(torch.float64).numpy()
        k0 = w.k_pool[slot0, h // 2].to(torch.float64).numpy()
        assert abs(lse[0, h] - w.softmax_scale * float(q0 @ k0)) < 1e-13


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(2)
    vg = rng.standard_normal((10, 4))
    vis = oracle.visible_keys(3, 10, True)  # 8, 9, 10 visible keys
    o, lse = oracle.attend(np.zeros((3, 4)), rng.standard_normal((10, 4)), vg, 1.0, vis)
    for r in range(3):
        assert np.abs(o[r] - vg[:vis[r]].mean(axis=0)).max() < 1e-14
        assert abs(lse[r] - math.log(vis[r])) < 1e-14


def test_hand_worked_two_key_example():
    # q = (1, 0), k0 = (1, 0), k1 = (0, 0), v0 = (1, 0), v1 = (0, 1), scale 1:
    # logits (1, 0) -> weights (e, 1) / (e + 1) -> O = (e/(e+1), 1/(e+1)), LSE = log(e + 1).
    q = np.array([[1.0, 0.0]])
    k = np.array([[1.0, 0.0], [0.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = oracle.attend(q, k, v, 1.0, np.array([2]))
    e = math.e
    assert abs(o[0, 0] - e / (e + 1)) < 1e-15 and abs(o[0, 1] - 1 / (e + 1)) < 1e-15
    assert abs(lse[0] - math.log(e + 1)) < 1e-15


def test_huge_logits_do_not_overflow():
    q = np.array([[1000.0, 0.0]])
    k = np.array([[1.0, 0.0], [0.999, 0.0]])
    v = np.array([[2.0, 0.0], [0.0, 2.0]])
    o, lse = oracle.attend(q, k, v, 1.0, np.array([2]))
    w0 = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(o[0, 0] - 2 * w0) < 1e-14 and abs(o[0, 1] - 2 * (1 - w0)) < 1e-14
    assert abs(lse[0] - (1000.0 + math.log1p(math.exp(-1.0)))) < 1e-12


def test_empty_rows_and_requests():
    # K = 0 non-causal: O = 0, LSE = -inf; Lq = 0: nothing written (rows stay NaN).
    w = wl.make_random(4, batch=3, q_lens=[2, 0, 3], k_lens=[0, 5, 4], causal=False,
                       num_heads_q=2, num_heads_kv=1, head_dim=4)
    o, lse = _run_oracle(w)
    assert np.all(o[0:2] == 0.0) and np.all(np.isneginf(lse[0:2]))
    assert np.isfinite(o[2:]).all()


# ------------------------------------------------------------------------------ invariants

def test_relayout_into_other_segments_is_bitwise_invariant():
    base = wl.make_random(5, batch=2, q_lens=[7, 3], k_lens=[23, 11], max_segs=1,
                          num_heads_q=4, num_heads_kv=2, head_dim=16)
    o1, l1 = _run_oracle(base)
    # same logical keys, re-laid out as many segments at new offsets of a bigger pool
    segs, ind, cq, ck = wl.host_tables(base)
    rng = np.random.default_rng(9)
    new_lengths = [wl.cut_lengths(rng, int(ck[b + 1] - ck[b]), 6) for b in range(2)]
    flat = [l for s in new_lengths for l in s]
    pool = 200
    offs = wl.place_segments(rng, flat, pool)
    kp = torch.full((pool, 2, 16), float("nan"), dtype=torch.bfloat16)
    vp = kp.clone()
    si = 0
    for b in range(2):
        old = oracle.request_slots(segs, ind, b)
        start = 0
        for ln in new_lengths[b]:
            kp[offs[si]:offs[si] + ln] = base.k_pool[old[start:start + ln]]
            vp[offs[si]:offs[si] + ln] = base.v_pool[old[start:start + ln]]
            start += ln
            si += 1
    new_segs = np.array([[o, l] for o, l in zip(offs, flat)])
    new_ind = np.concatenate([[0], np.cumsum([len(s) for s in new_lengths])])
    o2, l2 = oracle.attention(wl.bits(base.q), wl.bits(kp), wl.bits(vp), new_segs, new_ind, cq, ck,
                              num_heads_kv=2, softmax_scale=base.softmax_scale, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("seed", range(5))
def test_split_merge_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    K, n, d = 37, 9, 16
    qh, kg, vg = (rng.standard_normal((n, d)), rng.standard_normal((K, d)) * 2,
                  rng.standard_normal((K, d)))
    vis = oracle.visible_keys(n, K, causal=bool(seed % 2))
    o, lse = oracle.attend(qh, kg, vg, 0.2, vis)
    # random cut points with repeats (empty blocks) and 1-key blocks
    cuts = sorted(rng.integers(0, K + 1, size=6).tolist() + [1, 2])
    bounds = [0] + cuts + [K]
    o2, l2 = oracle.split_merge(qh, kg, vg, 0.2, vis, bounds)
    assert np.abs(o - o2).max() < 1e-12 and np.abs(lse - l2).max() < 1e-12


def test_merge_of_only_empty_blocks_is_empty():
    o, lse = oracle.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_chunked_prefill_equals_suffix_of_full_prefill():
    full = wl.make_random(6, batch=1, q_lens=[40], k_lens=[40], max_segs=3, num_heads_q=4,
                          num_heads_kv=1, head_dim=16)
    o_full, l_full = _run_oracle(full)
    segs, ind, _, ck = wl.host_tables(full)
    for lq in (1, 7, 40):
        cq = np.array([0, lq])
        o_c, l_c = oracle.attention(wl.bits(full.q[40 - lq:]), wl.bits(full.k_pool), wl.bits(full.v_pool),
                                    segs, ind, cq, ck, num_heads_kv=1,
                                    softmax_scale=full.softmax_scale, causal=True)
        assert np.abs(o_c - o_full[40 - lq:]).max() < 1e-13
        assert np.abs(l_c - l_full[40 - lq:]).max() < 1e-13


def test_gqa_equals_mha_with_replicated_kv_heads():
    w = wl.make_random(8, batch=2, q_lens=[4, 2], k_lens=[10, 6], num_heads_q=8, num_heads_kv=2,
                       head_dim=8)
    o, l = _run_oracle(w)
    segs, ind, cq, ck = wl.host_tables(w)
    kp = w.k_pool.repeat_interleave(4, dim=1)
    vp = w.v_pool.repeat_interleave(4, dim=1)
    o2, l2 = oracle.attention(wl.bits(w.q), wl.bits(kp), wl.bits(vp), segs, ind, cq, ck,
                              num_heads_kv=8, softmax_scale=w.softmax_scale, causal=True)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_decode_row_equals_last_prefill_row():
    w = wl.make_random(10, batch=1, q_lens=[12], k_lens=[12], num_heads_q=4, num_heads_kv=2,
                       head_dim=8)
    o, l = _run_oracle(w)
    segs, ind, _, ck = wl.host_tables(w)
    od, ld = oracle.attention(wl.bits(w.q[11:]), wl.bits(w.k_pool), wl.bits(w.v_pool), segs, ind,
                              np.array([0, 1]), ck, num_heads_kv=2,
                              softmax_scale=w.softmax_scale, causal=True)
    assert np.abs(od - o[11:]).max() < 1e-14
    od2, _ = oracle.attention(wl.bits(w.q[11:]), wl.bits(w.k_pool), wl.bits(w.v_pool), segs, ind,
                              np.array([0, 1]), ck, num_heads_kv=2,
                              softmax_scale=w.softmax_scale, causal=False)
    assert np.abs(od2 - od).max() == 0.0


def test_shift_of_every_key_leaves_output_unchanged():
    rng = np.random.default_rng(12)
    qh, kg, vg = rng.standard_normal((6, 16)), rng.standard_normal((20, 16)), rng.standard_normal((20, 16))
    vis = oracle.visible_keys(6, 20, True)
    o1, _ = oracle.attend(qh, kg, vg, 0.3, vis)
    o2, _ = oracle.attend(qh, kg + rng.standard_normal(16) * 3, vg, 0.3, vis)
    assert np.abs(o1 - o2).max() < 1e-12


def test_causal_alignment_is_bottom_right():
    # Lq < K: the last query sees all K keys (equals non-causal), the first sees K - Lq + 1.
    vis = oracle.visible_keys(4, 10, True)
    assert vis.tolist() == [7, 8, 9, 10]
    w = wl.make_random(13, batch=1, q_lens=[4], k_lens=[10], num_heads_q=2, num_heads_kv=1,
                       head_dim=8)
    oc, _ = _run_oracle(w)
    w.causal = False
    on, _ = _run_oracle(w)
    assert np.array_equal(oc[3], on[3]) and not np.allclose(oc[0], on[0])


def test_unreferenced_poisoned_slots_never_reach_the_output():
    w = wl.make_random(14, batch=3, q_lens=[3, 5, 1], k_lens=[9, 13, 30], max_segs=4,
                       num_heads_q=4, num_heads_kv=1, head_dim=8, poison=True)
    assert torch.isnan(w.k_pool.float()).any()
    o, l = _run_oracle(w)
    assert np.isfinite(o).all() and np.isfinite(l).all()


def test_rows_api_matches_full_api():
    w = wl.make_random(15, batch=3, q_lens=[3, 5, 1], k_lens=[9, 13, 30], num_heads_q=8,
                       num_heads_kv=2, head_dim=16, kv_dtype="fp8_e4m3")
    o, l = _run_oracle(w)
    segs, ind, cq, ck = wl.host_tables(w)
    rows = [(0, 0, 0), (0, 2, 7), (1, 4, 3), (2, 0, 5), (1, 1, 1)]
    orow, lrow = oracle.attention_rows(wl.bits(w.q), wl.bits(w.k_pool), wl.bits(w.v_pool), segs, ind,
                                       cq, ck, rows, num_heads_kv=2,
                                       softmax_scale=w.softmax_scale, causal=True,
                                       kv_format="fp8_e4m3", k_scale=w.k_scale.numpy(),
                                       v_scale=w.v_scale.numpy())
    for r, (b, i, h) in enumerate(rows):
        # one row at a time vs a block of rows: BLAS may order the sums differently
        assert np.abs(orow[r] - o[cq[b] + i, h]).max() < 1e-14
        assert abs(lrow[r] - l[cq[b] + i, h]) < 1e-14
