"""GPU parity at kv head counts other than 8 (query heads always 8 per kv head, the packed GQA
group): the decode's column mapping (CUs / Hkv columns, heads rotated per round) and the
in-workgroup plan's unit positions depend on Hkv, and so do the prefill grids. Every output and
LSE is compared with the CPU float64 oracle, under the same bar as the other parity tests."""
import pytest
import torch

import workloads as wl
from tests import _helpers as H

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

DECODE_CASES = [
    # (seed, Hkv, kv dtype, key counts, most segments per request)
    (71, 1, "bf16", [1, 700, 5000, 64, 2300], 3),
    (72, 2, "fp8_e4m3", [9000, 1, 129, 3100], 12),
    (73, 4, "int8", [2048, 2049, 7, 6000, 0, 900], 4),
    (74, 16, "bf16", [4000, 333, 1, 8191, 65], 9),
]


def _compare(w, name, num_splits=0):
    out, lse = H.run_gpu(w, num_splits=num_splits)
    torch.cuda.synchronize()
    o_ref, l_ref = H.oracle_full(w)
    mx, rms = H.assert_close(out.float().cpu().numpy(), o_ref, name)
    H.assert_lse_close(lse.cpu().numpy(), l_ref, name)
    print(f"[parity] {name}: max_abs={mx:.3e} rms={rms:.3e}", flush=True)


@needs_gpu
@pytest.mark.parametrize("plan", ["workgroup", "kernel"])
@pytest.mark.parametrize("num_splits", [0, 3])
@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"hkv{c[1]}-{c[2]}" for c in DECODE_CASES])
def test_decode_other_kv_head_counts(case, num_splits, plan, monkeypatch):
    seed, hkv, kvd, kl, ms = case
    if plan == "kernel":
        monkeypatch.setenv("SEG_ATTN_DECODE_PLAN", "kernel")
    else:
        monkeypatch.delenv("SEG_ATTN_DECODE_PLAN", raising=False)
    print(f"[case] decode Hkv={hkv} {kvd} k={kl} splits={num_splits} plan={plan}", flush=True)
    w = wl.make_random(seed, batch=len(kl), q_lens=[1] * len(kl), k_lens=kl, max_segs=ms,
                       kv_dtype=kvd, num_heads_q=8 * hkv, num_heads_kv=hkv, kind="decode",
                       zero_length_segments=True).to("cuda")
    _compare(w, f"decode-hkv{hkv}-{kvd}-s{num_splits}-{plan}", num_splits=num_splits)


PREFILL_CASES = [
    # (seed, Hkv, query counts, key counts)
    (81, 1, [300, 17], [300, 900]),
    (82, 4, [129, 64, 1], [500, 64, 77]),
    (83, 16, [200], [450]),
]


@needs_gpu
@pytest.mark.parametrize("tile", ["auto", "128", "256"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"hkv{c[1]}" for c in PREFILL_CASES])
def test_prefill_other_kv_head_counts(case, tile, monkeypatch):
    seed, hkv, ql, kl = case
    if tile == "auto":
        monkeypatch.delenv("SEG_ATTN_PREFILL_TILE", raising=False)
    else:
        monkeypatch.setenv("SEG_ATTN_PREFILL_TILE", tile)
    print(f"[case] prefill Hkv={hkv} q={ql} k={kl} tile={tile}", flush=True)
    w = wl.make_random(seed, batch=len(ql), q_lens=ql, k_lens=kl, max_segs=4, num_heads_q=8 * hkv,
                       num_heads_kv=hkv).to("cuda")
    _compare(w, f"prefill-hkv{hkv}-{tile}")
