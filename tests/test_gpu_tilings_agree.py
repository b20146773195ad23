"""The two prefill tilings (128-row tiles of 16 positions and 256-row tiles of 32 positions, 8
heads each) compute every row with the same arithmetic in the same order: the same 64-key
blocks in key order, the same MFMA k-order within a block, the same online-softmax updates.
Their outputs and LSEs must therefore agree bit for bit, on causal and full masks, ragged
lengths, empty queries and segment-straddling blocks."""
import numpy as np
import pytest
import torch

import workloads as wl
from tests import _helpers as H

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


@needs_gpu
@pytest.mark.parametrize("seed", range(6))
def test_prefill_tilings_bitwise_equal(seed, monkeypatch):
    rng = np.random.default_rng(9900 + seed)
    batch = int(rng.integers(1, 5))
    hkv = int(rng.choice([1, 2, 8]))
    causal = bool(seed % 2 == 0)
    k_lens = [int(x) for x in rng.integers(1, 900, size=batch)]
    q_lens = [int(rng.integers(1 if causal else 0, k + 1)) for k in k_lens]
    print(f"[case] tilings seed={seed} B={batch} Hkv={hkv} causal={causal} q={q_lens} k={k_lens}", flush=True)
    w = wl.make_random(9900 + seed, batch=batch, q_lens=q_lens, k_lens=k_lens, max_segs=6, causal=causal,
                       num_heads_q=8 * hkv, num_heads_kv=hkv, zero_length_segments=True).to("cuda")
    got = {}
    for tile in ("128", "256"):
        monkeypatch.setenv("SEG_ATTN_PREFILL_TILE", tile)
        out, lse = H.run_gpu(w)
        torch.cuda.synchronize()
        got[tile] = (out.cpu(), lse.cpu())
    (o1, l1), (o2, l2) = got["128"], got["256"]
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "outputs differ between the tilings"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "LSEs differ between the tilings"
