"""Seeded random sweep of valid prefill and decode calls against the CPU float64 oracle: batch
sizes, query and key lengths, segment counts (empty segments included), kv head counts, pool
formats, split counts, prefill tilings and decode planning paths drawn from one generator per
case, so that combinations no hand-written case names are exercised too. Every output and LSE is
compared under the same bar as the other parity tests; the case's parameters are printed first."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests import _helpers as H

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _compare(w, name, num_splits=0):
    out, lse = H.run_gpu(w, num_splits=num_splits)
    torch.cuda.synchronize()
    o_ref, l_ref = H.oracle_full(w)
    mx, rms = H.assert_close(out.float().cpu().numpy(), o_ref, name)
    H.assert_lse_close(lse.cpu().numpy(), l_ref, name)
    print(f"[parity] {name}: max_abs={mx:.3e} rms={rms:.3e}", flush=True)


@needs_gpu
@pytest.mark.parametrize("seed", range(16))
def test_random_prefill(seed, monkeypatch):
    rng = np.random.default_rng(9000 + seed)
    batch = int(rng.integers(1, 5))
    hkv = int(rng.choice([1, 2, 4, 8]))
    causal = bool(rng.random() < 0.75)
    k_lens = [int(x) for x in rng.integers(1, 700, size=batch)]
    q_lens = [int(rng.integers(0 if not causal else 1, k + 1)) for k in k_lens]
    if not causal and rng.random() < 0.3:
        q_lens[0] = 0
    tile = str(rng.choice(["auto", "128", "256"]))
    max_segs = int(rng.integers(1, 10))
    if tile == "auto":
        monkeypatch.delenv("SEG_ATTN_PREFILL_TILE", raising=False)
    else:
        monkeypatch.setenv("SEG_ATTN_PREFILL_TILE", tile)
    print(f"[case] random prefill seed={seed} B={batch} Hkv={hkv} causal={causal} q={q_lens} "
          f"k={k_lens} segs<={max_segs} tile={tile}", flush=True)
    w = wl.make_random(9000 + seed, batch=batch, q_lens=q_lens, k_lens=k_lens, max_segs=max_segs,
                       causal=causal, num_heads_q=8 * hkv, num_heads_kv=hkv,
                       zero_length_segments=bool(rng.random() < 0.5)).to("cuda")
    _compare(w, f"random-prefill-{seed}")


@needs_gpu
@pytest.mark.parametrize("seed", range(16))
def test_random_decode(seed, monkeypatch):
    rng = np.random.default_rng(9500 + seed)
    batch = int(rng.integers(1, 40))
    hkv = int(rng.choice([1, 2, 4, 8]))
    kvd = str(rng.choice(["bf16", "fp8_e4m3", "int8"]))
    long_tail = rng.random() < 0.3
    k_lens = [int(x) for x in rng.integers(0, 20000 if long_tail else 3000, size=batch)]
    num_splits = int(rng.choice([0, 0, 1, 2, 5]))
    plan = str(rng.choice(["workgroup", "kernel"]))
    max_segs = int(rng.integers(1, 12))
    if plan == "kernel":
        monkeypatch.setenv("SEG_ATTN_DECODE_PLAN", "kernel")
    else:
        monkeypatch.delenv("SEG_ATTN_DECODE_PLAN", raising=False)
    print(f"[case] random decode seed={seed} B={batch} Hkv={hkv} {kvd} k={k_lens} "
          f"segs<={max_segs} splits={num_splits} plan={plan}", flush=True)
    w = wl.make_random(9500 + seed, batch=batch, q_lens=[1] * batch, k_lens=k_lens, max_segs=max_segs,
                       kv_dtype=kvd, num_heads_q=8 * hkv, num_heads_kv=hkv, kind="decode",
                       zero_length_segments=bool(rng.random() < 0.5)).to("cuda")
    _compare(w, f"random-decode-{seed}", num_splits=num_splits)
