"""Seeded synthetic inputs for segment attention.

Test and benchmark infrastructure shared by the oracle-side and the GPU-side
tests. It draws request lengths, cuts each request's keys into segments,
places the segments at random non-overlapping offsets of a shared token pool,
and fills the referenced pool slots, the queries and (for the FP8 pool) the
per-(token, kv-head) scales with seeded N(0, 1) data. It computes no part of
attention.

Layouts (the same ones the C-ABI takes):
  q            [total_q, Hq, D]        bfloat16
  k_pool/v_pool[pool_tokens, Hkv, D]   bfloat16, float8_e4m3fn or int8
  k_scale/v_scale [pool_tokens, Hkv]   float32 (FP8 and INT8 pools only)
  segs         [nseg, 2] int32 rows of (pool_offset, length), grouped by request
               in logical key order
  seg_indptr   [B + 1] int32, request b owns segs[seg_indptr[b]:seg_indptr[b+1]]
  cu_seqlens_q, cu_seqlens_k  [B + 1] int32 prefix sums of query / key lengths

Pool slots no segment references are filled with NaN when ``poison`` is set
(INT8 pools: code -128 with a NaN scale), so that any read outside the segments
shows up in the output.

The five named configurations follow the workload shapes of the Flood README
("Kernels / Seg-attn" table: 64 query heads, 8 kv heads, head dim 128, batch 1
with Q_len = K_len = 1024, batch 128 with Q_len = 1) plus chunked prefill and a
long FP8 decode; a sixth is the long decode over an INT8 pool. The exact recipe
for each is in ``CONFIGS``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

HQ, HKV, HEAD_DIM = 64, 8, 128
FP8_MAX = 448.0  # largest finite OCP E4M3FN value
INT8_MAX = 127.0  # largest INT8 code the symmetric encoding uses


@dataclass
class Workload:
    name: str
    kind: str                      # "prefill" or "decode"
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    segs: torch.Tensor
    seg_indptr: torch.Tensor
    cu_seqlens_q: torch.Tensor
    cu_seqlens_k: torch.Tensor
    max_seqlen_q: int
    max_seqlen_k: int
    causal: bool
    softmax_scale: float
    kv_dtype: str                  # "bf16" or "fp8_e4m3"
    q_lens: np.ndarray
    k_lens: np.ndarray
    seed: int
    recipe: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(len(self.q_lens))

    @property
    def num_heads_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_heads_kv(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def pool_tokens(self) -> int:
        return int(self.k_pool.shape[0])

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask leaves visible, per query head."""
        total = 0
        for lq, k in zip(self.q_lens.tolist(), self.k_lens.tolist()):
            if self.causal:
                total += lq * (k - lq) + lq * (lq + 1) // 2
            else:
                total += lq * k
        return total

    def to(self, device) -> "Workload":
        def mv(t):
            return None if t is None else t.to(device)
        return Workload(self.name, self.kind, mv(self.q), mv(self.k_pool), mv(self.v_pool),
                        mv(self.k_scale), mv(self.v_scale), mv(self.segs), mv(self.seg_indptr),
                        mv(self.cu_seqlens_q), mv(self.cu_seqlens_k), self.max_seqlen_q,
                        self.max_seqlen_k, self.causal, self.softmax_scale, self.kv_dtype,
                        self.q_lens, self.k_lens, self.seed, self.recipe, dict(self.extra))


# ----------------------------------------------------------------------------------------------
# integer structure: lengths, segment cuts, placement


def cut_lengths(rng: np.random.Generator, k: int, nseg: int) -> List[int]:
    """Split k keys into nseg segments of >= 1 key each (fewer when k < nseg).

    Draws nseg - 1 distinct cut points uniformly from [1, k - 1]."""
    if k == 0:
        return [0] if nseg > 0 else []
    nseg = max(1, min(nseg, k))
    if nseg == 1:
        return [k]
    cuts = np.sort(rng.choice(np.arange(1, k), size=nseg - 1, replace=False))
    edges = np.concatenate([[0], cuts, [k]])
    return [int(x) for x in np.diff(edges)]


def place_segments(rng: np.random.Generator, lengths: Sequence[int], pool_tokens: int) -> List[int]:
    """Offsets for segments of the given lengths, shuffled together, non-overlapping.

    The free space pool_tokens - sum(lengths) is split into len(lengths) + 1 gaps by sorted
    uniform draws; segments are laid out in a seeded random order with those gaps between
    them."""
    n = len(lengths)
    used = int(sum(lengths))
    if used > pool_tokens:
        raise ValueError(f"segments need {used} slots, pool has {pool_tokens}")
    free = pool_tokens - used
    cuts = np.sort(rng.integers(0, free + 1, size=n)) if n else np.zeros(0, np.int64)
    gaps = np.diff(np.concatenate([[0], cuts]))
    order = rng.permutation(n)
    offsets = [0] * n
    pos = 0
    for rank, idx in enumerate(order):
        pos += int(gaps[rank])
        offsets[idx] = pos
        pos += int(lengths[idx])
    return offsets


def _prefix(x: Sequence[int]) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(x, dtype=np.int64))]).astype(np.int64)


# ----------------------------------------------------------------------------------------------
# value generation


def _new_generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _nan_tensor(shape, dtype, device) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=torch.float32 if dtype == torch.float8_e4m3fn else dtype,
                      device=device).to(dtype)


def encode_fp8_rows(x: torch.Tensor):
    """Input encoding of an N(0,1) fp32 block [..., D] as OCP E4M3FN codes plus one fp32 scale
    per row: scale = max|x| / 448, code = round-to-nearest-even(clamp(x / scale)).

    This only prepares the FP8 input pool; the decoded values code * scale are what both the
    oracle and the kernels consume."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    codes = (x / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, scale


def encode_int8_rows(x: torch.Tensor):
    """Input encoding of an N(0,1) fp32 block [..., D] as symmetric INT8 codes plus one fp32
    scale per row: scale = max|x| / 127, code = round-half-even(clamp(x / scale, +-127)), with
    torch's own division and rounding. Like ``encode_fp8_rows`` it only prepares the input
    pool."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / INT8_MAX, torch.ones_like(amax)).to(torch.float32)
    codes = torch.round((x / scale.unsqueeze(-1)).clamp(-INT8_MAX, INT8_MAX)).to(torch.int8)
    return codes, scale


def build(name: str, kind: str, q_lens: Sequence[int], seg_lengths: Sequence[Sequence[int]],
          pool_tokens: int, *, seed: int, rng: np.random.Generator, causal: bool,
          kv_dtype: str = "bf16", num_heads_q: int = HQ, num_heads_kv: int = HKV,
          head_dim: int = HEAD_DIM, softmax_scale: Optional[float] = None,
          device="cpu", poison: bool = True, recipe: str = "",
          offsets: Optional[Sequence[int]] = None) -> Workload:
    """Assemble a workload from per-request query lengths and per-request segment lengths.

    Values are drawn in a fixed order from one torch generator on ``device`` seeded with
    ``seed``: all of Q first, then for each request its K block and then its V block."""
    B = len(q_lens)
    assert len(seg_lengths) == B
    k_lens = np.array([int(sum(s)) for s in seg_lengths], dtype=np.int64)
    q_lens_np = np.array([int(x) for x in q_lens], dtype=np.int64)
    flat = [int(l) for s in seg_lengths for l in s]
    if offsets is None:
        offsets = place_segments(rng, flat, pool_tokens)
    assert len(offsets) == len(flat)
    seg_count = [len(s) for s in seg_lengths]
    seg_indptr = _prefix(seg_count)
    segs = np.array([[o, l] for o, l in zip(offsets, flat)], dtype=np.int64).reshape(-1, 2)
    if segs.size and (segs[:, 0].max(initial=0) + 0 > np.iinfo(np.int32).max):
        raise ValueError("pool offsets exceed int32")
    cu_q = _prefix(q_lens_np)
    cu_k = _prefix(k_lens)
    gen = _new_generator(device, seed)
    total_q = int(cu_q[-1])
    q = torch.randn((total_q, num_heads_q, head_dim), generator=gen, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    if kv_dtype not in ("bf16", "fp8_e4m3", "int8"):
        raise ValueError(f"unknown kv dtype {kv_dtype}")
    fp8 = kv_dtype == "fp8_e4m3"
    int8 = kv_dtype == "int8"
    scaled = fp8 or int8
    pool_dtype = torch.float8_e4m3fn if fp8 else (torch.int8 if int8 else torch.bfloat16)
    shape = (pool_tokens, num_heads_kv, head_dim)
    if poison and int8:
        k_pool = torch.full(shape, -128, dtype=torch.int8, device=device)
        v_pool = torch.full(shape, -128, dtype=torch.int8, device=device)
    elif poison:
        k_pool = _nan_tensor(shape, pool_dtype, device)
        v_pool = _nan_tensor(shape, pool_dtype, device)
    else:
        k_pool = torch.zeros(shape, dtype=pool_dtype, device=device)
        v_pool = torch.zeros(shape, dtype=pool_dtype, device=device)
    k_scale = v_scale = None
    if scaled:
        fill = float("nan") if poison else 1.0
        k_scale = torch.full((pool_tokens, num_heads_kv), fill, dtype=torch.float32, device=device)
        v_scale = torch.full((pool_tokens, num_heads_kv), fill, dtype=torch.float32, device=device)
    si = 0
    for b in range(B):
        kb = int(k_lens[b])
        kx = torch.randn((kb, num_heads_kv, head_dim), generator=gen, device=device, dtype=torch.float32)
        vx = torch.randn((kb, num_heads_kv, head_dim), generator=gen, device=device, dtype=torch.float32)
        if scaled:
            enc = encode_fp8_rows if fp8 else encode_int8_rows
            kc, ks = enc(kx)
            vc, vs = enc(vx)
        else:
            kc, vc = kx.to(torch.bfloat16), vx.to(torch.bfloat16)
        start = 0
        for _ in range(seg_count[b]):
            off, ln = int(segs[si, 0]), int(segs[si, 1])
            if ln:
                k_pool[off:off + ln] = kc[start:start + ln]
                v_pool[off:off + ln] = vc[start:start + ln]
                if scaled:
                    k_scale[off:off + ln] = ks[start:start + ln]
                    v_scale[off:off + ln] = vs[start:start + ln]
            start += ln
            si += 1
        del kx, vx, kc, vc
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(head_dim)
    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32)).to(device)
    return Workload(
        name=name, kind=kind, q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
        segs=i32(segs.reshape(-1, 2)), seg_indptr=i32(seg_indptr), cu_seqlens_q=i32(cu_q),
        cu_seqlens_k=i32(cu_k), max_seqlen_q=int(q_lens_np.max(initial=0)),
        max_seqlen_k=int(k_lens.max(initial=0)), causal=causal, softmax_scale=scale,
        kv_dtype=kv_dtype, q_lens=q_lens_np, k_lens=k_lens, seed=seed, recipe=recipe)


# ----------------------------------------------------------------------------------------------
# the named configurations

CONFIGS = {
    1: "tiny causal prefill: B=1, Lq=K=128, 64/8/128 bf16 N(0,1), KV as 2 segments (80 + 48) at "
       "random offsets of a 4096-slot pool",
    2: "single causal prefill: B=1, Lq=K=1024, 64/8/128 bf16 N(0,1), KV in 1 segment at a random "
       "offset of a 16384-slot pool",
    3: "chunked causal prefill: B=4, Lq=2048, K = prior + 2048 with prior ~ U{0..6144}, 1-4 "
       "segments per request, 65536-slot pool, 64/8/128 bf16",
    4: "decode: B=128, Lq=1, K = clip(round(1024 * exp(z)), 64, 8192), z ~ N(0,1), 1-3 segments "
       "per request, 2^20-slot pool, 64/8/128 bf16",
    5: "FP8 long decode: B=16, Lq=1, K ~ U{32768..131072}, 1-8 segments per request, 2^21-slot "
       "pool, Q bf16, K/V e4m3fn + fp32 scale per (token, kv head), 64/8/128",
    6: "INT8 long decode: the FP8 long decode's shape and recipe with K/V as symmetric int8 codes "
       "+ fp32 scale per (token, kv head)",
}

CONFIG_NAMES = {1: "tiny_prefill_128", 2: "prefill_1k", 3: "chunked_prefill_4x2048",
                4: "decode_bf16_b128_lognormal", 5: "decode_fp8_b16_32k_128k",
                6: "decode_int8_b16_32k_128k"}


def make_config(c: int, *, seed: Optional[int] = None, device="cpu", poison: bool = True) -> Workload:
    """One of the named configurations (1..6), seeded with 1000 + c unless ``seed`` is given."""
    s = 1000 + c if seed is None else seed
    rng = np.random.default_rng(s)
    name, recipe = CONFIG_NAMES[c], CONFIGS[c]
    if c == 1:
        return build(name, "prefill", [128], [[80, 48]], 4096, seed=s, rng=rng, causal=True,
                     device=device, poison=poison, recipe=recipe)
    if c == 2:
        return build(name, "prefill", [1024], [[1024]], 16384, seed=s, rng=rng, causal=True,
                     device=device, poison=poison, recipe=recipe)
    if c == 3:
        B = 4
        prior = rng.integers(0, 6144 + 1, size=B)
        ks = prior + 2048
        nseg = rng.integers(1, 4 + 1, size=B)
        segl = [cut_lengths(rng, int(k), int(n)) for k, n in zip(ks, nseg)]
        return build(name, "prefill", [2048] * B, segl, 65536, seed=s, rng=rng, causal=True,
                     device=device, poison=poison, recipe=recipe)
    if c == 4:
        B = 128
        z = rng.standard_normal(B)
        ks = np.clip(np.rint(1024.0 * np.exp(z)), 64, 8192).astype(np.int64)
        nseg = rng.integers(1, 3 + 1, size=B)
        segl = [cut_lengths(rng, int(k), int(n)) for k, n in zip(ks, nseg)]
        return build(name, "decode", [1] * B, segl, 1 << 20, seed=s, rng=rng, causal=True,
                     device=device, poison=poison, recipe=recipe)
    if c in (5, 6):
        B = 16
        ks = rng.integers(32768, 131072 + 1, size=B)
        nseg = rng.integers(1, 8 + 1, size=B)
        segl = [cut_lengths(rng, int(k), int(n)) for k, n in zip(ks, nseg)]
        return build(name, "decode", [1] * B, segl, 1 << 21, seed=s, rng=rng, causal=True,
                     kv_dtype="fp8_e4m3" if c == 5 else "int8", device=device, poison=poison,
                     recipe=recipe)
    raise ValueError(f"unknown config {c}")


def make_random(seed: int, *, batch: int, q_lens: Sequence[int], k_lens: Sequence[int],
                max_segs: int = 4, pool_slack: float = 2.0, causal: bool = True,
                kv_dtype: str = "bf16", num_heads_q: int = HQ, num_heads_kv: int = HKV,
                head_dim: int = HEAD_DIM, device="cpu", poison: bool = True,
                kind: str = "prefill", zero_length_segments: bool = False) -> Workload:
    """A general seeded case: given lengths, 1..max_segs segments per request, a pool with
    ``pool_slack`` times the needed slots (at least 16), optional empty segments inserted."""
    rng = np.random.default_rng(seed)
    assert len(q_lens) == batch and len(k_lens) == batch
    segl = []
    for k in k_lens:
        n = int(rng.integers(1, max_segs + 1))
        s = cut_lengths(rng, int(k), n)
        if zero_length_segments:
            pos = int(rng.integers(0, len(s) + 1))
            s = s[:pos] + [0] + s[pos:]
        segl.append(s)
    pool = max(16, int(math.ceil(pool_slack * max(1, sum(int(k) for k in k_lens)))))
    return build(f"random_{seed}", kind, list(q_lens), segl, pool, seed=seed, rng=rng,
                 causal=causal, kv_dtype=kv_dtype, num_heads_q=num_heads_q,
                 num_heads_kv=num_heads_kv, head_dim=head_dim, device=device, poison=poison,
                 recipe="random lengths/segments")


# ----------------------------------------------------------------------------------------------
# plain data conversion for the oracle side


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a bf16 (uint16), fp8 or int8 (uint8) tensor as a host numpy array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.int8):
        return t.view(torch.uint8).numpy()
    raise TypeError(f"no bit view for {t.dtype}")


def host_tables(w: Workload):
    """Integer tables as host numpy int64 arrays: segs [nseg, 2], seg_indptr, cu_q, cu_k."""
    f = lambda t: t.detach().cpu().numpy().astype(np.int64)
    return f(w.segs).reshape(-1, 2), f(w.seg_indptr), f(w.cu_seqlens_q), f(w.cu_seqlens_k)


# ----------------------------------------------------------------------------------------------
# segment linear attention (simple gated linear attention over a pool of per-request states)

LA_HEADS, LA_DIM = 16, 128


@dataclass
class LinearWorkload:
    """Inputs of a segment-linear-attention call.

    q, k, v   [T, H, D] bfloat16; g [T, H] float32 log decays (<= 0)
    cu_seqlens [B + 1] int32 (decode: 0, 1, ..., B)
    state_pool [slots, H, D, D] float32, slot state_slots[b] holding request b's state (d_k rows,
               d_v contiguous); slots no request names are NaN when poisoned
    state_slots [B] int32, distinct"""
    name: str
    kind: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    cu_seqlens: torch.Tensor
    state_pool: torch.Tensor
    state_slots: torch.Tensor
    initial_state: bool
    scale: float
    lens: np.ndarray
    seed: int
    recipe: str = ""

    @property
    def batch(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    def to(self, device) -> "LinearWorkload":
        f = lambda t: t.to(device)
        return LinearWorkload(self.name, self.kind, f(self.q), f(self.k), f(self.v), f(self.g),
                              f(self.cu_seqlens), f(self.state_pool), f(self.state_slots),
                              self.initial_state, self.scale, self.lens, self.seed, self.recipe)


def make_linear(seed: int, lens: Sequence[int], *, kind: str = "prefill", initial_state: bool = True,
                num_heads: int = LA_HEADS, head_dim: int = LA_DIM, slack: int = 2,
                device="cpu", poison: bool = True, name: str = "", recipe: str = "") -> LinearWorkload:
    """Seeded inputs: q, k, v ~ N(0, 1) rounded to bf16; g = log(sigmoid(z)) / 16 with
    z ~ N(0, 1) (mean about -0.05: a 64-token chunk keeps a few percent of the state before it);
    initial states 0.1 * N(0, 1) in ``slack`` times as many slots as requests, at random distinct
    slots. Values are drawn in the order q, k, v, z, states from one torch generator."""
    rng = np.random.default_rng(seed)
    lens_np = np.array([int(x) for x in lens], dtype=np.int64)
    B = len(lens_np)
    T = int(lens_np.sum())
    gen = _new_generator(device, seed)
    H, D = num_heads, head_dim
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    q = rnd(T, H, D).to(torch.bfloat16)
    k = rnd(T, H, D).to(torch.bfloat16)
    v = rnd(T, H, D).to(torch.bfloat16)
    g = (torch.nn.functional.logsigmoid(rnd(T, H)) / 16.0).to(torch.float32)
    slots_n = max(1, slack * B)
    pool = torch.full((slots_n, H, D, D), float("nan") if poison else 0.0, dtype=torch.float32,
                      device=device)
    slots = rng.permutation(slots_n)[:B].astype(np.int64)
    for b in range(B):
        pool[int(slots[b])] = 0.1 * rnd(H, D, D)
    cu = _prefix(lens_np)
    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32)).to(device)
    return LinearWorkload(name or f"linear_{seed}", kind, q, k, v, g, i32(cu), pool, i32(slots),
                          bool(initial_state), 1.0 / math.sqrt(D), lens_np, seed, recipe)


LINEAR_CONFIGS = {
    "la_prefill_b1_1024": dict(lens=[1024], kind="prefill", initial_state=False),
    "la_prefill_b2_1024": dict(lens=[1024, 1024], kind="prefill", initial_state=False),
    "la_decode_b64": dict(lens=[1] * 64, kind="decode", initial_state=True),
    "la_decode_b256": dict(lens=[1] * 256, kind="decode", initial_state=True),
}


def make_linear_config(name: str, *, device="cpu", poison: bool = True) -> LinearWorkload:
    """The shapes of the Flood README's Seg-linear-attn table (16 heads, 16 kv heads, head dim
    128; prefill batch 1 and 2 of 1024 tokens from a zero state, decode batch 64 and 256 from
    stored states), seeded with 2000 + the table row."""
    c = LINEAR_CONFIGS[name]
    seed = 2000 + list(LINEAR_CONFIGS).index(name)
    return make_linear(seed, c["lens"], kind=c["kind"], initial_state=c["initial_state"],
                       device=device, poison=poison, name=name,
                       recipe=f"{c['kind']} B={len(c['lens'])} L={max(c['lens'])}, 16/16 heads, d=128")
