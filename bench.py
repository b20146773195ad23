#!/usr/bin/env python3
"""Benchmark of the segment-attention hot path on one MI355X.

Default: the single causal prefill of the Seg-attn kernel table's shape (batch 1,
Q_len = K_len = 1024, 64 q / 8 kv heads, d = 128, bf16, KV in one segment of a 16384-slot
pool). One step = one seg_attn_prefill call over that batch; the headline value is
causal-adjusted TFLOPS (4 * d * Hq * visible (q, k) pairs per second). The other workloads
(chunked prefill, bf16 decode, FP8 long decode) are measured in the same run and reported
under "configs" (prefill: TFLOPS; decode: KV-read GB/s), and the KV appends that precede the
attention calls of those workloads under "append" (GB/s of rows read and written), unless
--quick.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--quick] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_SOURCES = {"prefill": "attention_segmented_kv_amd/csrc/prefill.hip",
                  "decode": "attention_segmented_kv_amd/csrc/decode.hip",
                  "append": "attention_segmented_kv_amd/csrc/append.hip",
                  "linear": "attention_segmented_kv_amd/csrc/linear.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kind: str) -> str:
    with open(os.path.join(ROOT, KERNEL_SOURCES[kind]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def prefill_flops(w) -> float:
    return 4.0 * w.head_dim * w.num_heads_q * w.visible_pairs()


def decode_kv_bytes(w) -> float:
    per_tok = w.num_heads_kv * w.head_dim * (2 if w.kv_dtype == "bf16" else 1) * 2
    if w.kv_dtype != "bf16":
        per_tok += w.num_heads_kv * 4 * 2  # one fp32 scale each for K and V
    return float(w.k_lens.sum()) * per_tok


def append_bytes(n_rows: int, one_byte: bool) -> float:
    """Algorithmic HBM bytes of appending n_rows (token, kv head) rows of K and of V: the bf16
    rows read (2 x 256 B), and either the bf16 rows written (2 x 256 B) or the FP8 / INT8 codes
    and scales written (2 x (128 + 4) B)."""
    return float(n_rows) * (512 + (264 if one_byte else 512))


# The appends measured beside attention: the writes one step of a workload makes before its
# attention call (each request's last Lq_b keys are new), with its tables and pool size.
APPEND_CASES = (("append_chunk_bf16_4x2048", 3, "bf16"), ("append_chunk_fp8_4x2048", 3, "fp8_e4m3"),
                ("append_chunk_int8_4x2048", 3, "int8"), ("append_decode_bf16_b128", 4, "bf16"),
                ("append_decode_fp8_b16", 5, "fp8_e4m3"), ("append_decode_int8_b16", 6, "int8"))


APPEND_REPS = 10


def measure_append(name, c, fmt, steps, warmup, dev):
    import numpy as np
    import torch
    import attention_segmented_kv_amd as sa
    import workloads as wl
    w = wl.make_config(c, device=dev, poison=False)
    n_new = w.q_lens.astype(np.int64)
    cu_new = torch.as_tensor(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).to(dev)
    total = int(n_new.sum())
    g = torch.Generator(device=dev)
    g.manual_seed(7000 + c)
    shape = (total, w.num_heads_kv, w.head_dim)
    k_new = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    v_new = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    one_byte = fmt != "bf16"
    if fmt == w.kv_dtype:
        kp, vp, ks, vs = w.k_pool, w.v_pool, w.k_scale, w.v_scale
    else:  # same tables, another pool format (the append never reads the pool)
        pshape = tuple(w.k_pool.shape)
        pdt = torch.float8_e4m3fn if fmt == "fp8_e4m3" else torch.int8
        kp = torch.zeros(pshape, dtype=torch.uint8, device=dev).view(pdt)
        vp = torch.zeros(pshape, dtype=torch.uint8, device=dev).view(pdt)
        ks = torch.ones(pshape[:2], dtype=torch.float32, device=dev)
        vs = torch.ones(pshape[:2], dtype=torch.float32, device=dev)

    # An append is a few microseconds of GPU work, less than the binding's host time per call,
    # so the timed unit is a HIP graph of APPEND_REPS appends, replayed; per-append figures are
    # per replay / APPEND_REPS.
    def step():
        for _ in range(APPEND_REPS):
            sa.kv_append(k_new, v_new, w.segs, w.seg_indptr, cu_new, w.cu_seqlens_k, kp, vp,
                         k_scale=ks, v_scale=vs)
    t = time_steps(step, steps, warmup, graph=True)
    t["launch_ms_mean"] /= APPEND_REPS
    t["ms_per_step"] /= APPEND_REPS
    work = append_bytes(total * w.num_heads_kv, one_byte)
    achieved = work / (t["launch_ms_mean"] * 1e-3) / 1e9
    rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
          "frac": achieved / PEAK_HBM_GBS, "traffic": load_traffic("append", name)}
    return {"workload": name, "tables_of": w.name, "new_tokens": total, "kv": fmt,
            "value": round(work / (t["ms_per_step"] * 1e-3) / 1e9, 3), "unit": "GB/s",
            "launch_us_mean": round(t["launch_ms_mean"] * 1e3, 2), "roofline": rf,
            "work_per_step": work, "timing": "graph replays of %d appends" % APPEND_REPS}


LINEAR_CASES = ("la_prefill_b1_1024", "la_prefill_b2_1024", "la_decode_b64", "la_decode_b256")


def linear_work(w):
    """Algorithmic work of a segment-linear-attention call. Prefill: the flops of the 64-token
    chunked form, 2 * 64 * 128 * (128 + 64 + 64 + 128) per chunk and head (Q S, Q K^T, P V,
    K~^T V; masked work counted, as the chunk computes it). Decode: HBM bytes, the fp32 state
    read and written (2 * 64 KiB) plus q, k, v, out (4 * 256 B) and g per request and head."""
    H = w.num_heads
    if w.kind == "prefill":
        chunks = int(sum((int(n) + 63) // 64 for n in w.lens))
        return 2.0 * 64 * 128 * (128 + 64 + 64 + 128) * chunks * H
    return float(w.batch * H * (2 * 128 * 128 * 4 + 4 * 256 + 4))


def measure_linear(name, steps, warmup, dev):
    import torch
    import attention_segmented_kv_amd as sa
    import workloads as wl
    w = wl.make_linear_config(name, device=dev, poison=False)
    out = torch.empty_like(w.q)
    max_len = int(w.lens.max())
    need = sa._load().seg_attn_linear_prefill_workspace_bytes(w.batch, max_len, w.num_heads, 128)
    ws = torch.empty(max(int(need), 256), dtype=torch.uint8, device=dev)

    def call():
        if w.kind == "decode":
            sa.linear_decode(w.q, w.k, w.v, w.g, w.state_slots, w.state_pool, scale=w.scale, out=out)
        else:
            sa.linear_prefill(w.q, w.k, w.v, w.g, w.cu_seqlens, w.state_slots, w.state_pool,
                              initial_state=w.initial_state, scale=w.scale, out=out,
                              max_seqlen=max_len, workspace=ws)

    def step():  # graph replays of APPEND_REPS calls, as for the appends
        for _ in range(APPEND_REPS):
            call()
    t = time_steps(step, steps, warmup, graph=True)
    us = t["launch_ms_mean"] * 1e3 / APPEND_REPS
    work = linear_work(w)
    if w.kind == "prefill":
        achieved = work / (us * 1e-6) / 1e12
        rf = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
              "frac": achieved / PEAK_BF16_TFLOPS, "traffic": load_traffic("linear", name),
              "note": "one launch of the closed form (requests up to 4096 tokens); the unit counts "
                      "the chunked form's flops"}
    else:
        achieved = work / (us * 1e-6) / 1e9
        rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
              "frac": achieved / PEAK_HBM_GBS, "traffic": load_traffic("linear", name)}
    return {"workload": name, "recipe": w.recipe, "value": round(us, 2), "unit": "us",
            "higher_is_better": False, "roofline": rf, "work_per_call": work,
            "timing": "graph replays of %d calls" % APPEND_REPS}


def measure_allocator(steps: int = 2000):
    """Host cost of the segment allocator in a decode loop of the bf16 decode workload's shape:
    128 live requests in a 2^20-slot pool, each arriving with a lognormal prompt (median 1024,
    64..8192) and an output length U{64..512}, reserving prompt + output on arrival (granule 64
    for anything beyond). One step grows every live request by one token and writes the batch's
    tables; a request that has produced its output is released and a new one arrives in its place.
    Single-threaded host code through the Python binding: no GPU involved."""
    import numpy as np
    import attention_segmented_kv_amd as sa
    rng = np.random.default_rng(1004)
    a = sa.SegmentAllocator(1 << 20, granule=64)
    left = {}

    def arrive(r):
        prompt = int(np.clip(np.rint(1024.0 * np.exp(rng.standard_normal())), 64, 8192))
        out = int(rng.integers(64, 513))
        a.reserve(r, prompt + out)
        a.grow(r, prompt)
        left[r] = out

    for r in range(128):
        arrive(r)
    nxt, arrivals = 128, 0
    seg_counts = []
    t0 = time.perf_counter()
    for step in range(steps):
        ids = list(left)
        a.grow_many(ids, 1)
        segs, ind, cu = a.tables(ids)
        seg_counts.append(len(segs))
        for r in ids:
            left[r] -= 1
            if left[r] == 0:
                del left[r]
                a.release(r)
                arrive(nxt)
                nxt += 1
                arrivals += 1
    dt = time.perf_counter() - t0
    st = a.stats()
    return {"workload": "allocator_decode_loop_b128", "value": round(steps / dt, 1), "unit": "steps/s",
            "us_per_step": round(dt / steps * 1e6, 2), "bound": "host", "cores": 1,
            "segments_per_request_mean": round(float(np.mean(seg_counts)) / 128, 3),
            "arrivals": arrivals, "free_runs": st["free_runs"],
            "note": "one batched grow of 128 requests by one token + their tables per step, releases "
                    "and arrivals included, via the Python binding"}


def make_step(w):
    import attention_segmented_kv_amd as sa
    import torch
    if w.kind == "prefill":
        out = torch.empty_like(w.q)

        def step():
            sa.prefill(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_q, w.cu_seqlens_k,
                       w.max_seqlen_q, w.max_seqlen_k, causal=w.causal, softmax_scale=w.softmax_scale,
                       out=out)
        return step
    out = torch.empty_like(w.q)
    kvd = {"bf16": sa.KV_BF16, "fp8_e4m3": sa.KV_FP8_E4M3, "int8": sa.KV_INT8}[w.kv_dtype]
    need = sa.decode_workspace_bytes(w.batch, w.max_seqlen_k, w.num_heads_q, w.num_heads_kv, w.head_dim, kvd, 0)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=w.q.device)

    def step():
        sa.decode(w.q, w.k_pool, w.v_pool, w.segs, w.seg_indptr, w.cu_seqlens_k, w.max_seqlen_k,
                  k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale, out=out,
                  workspace=ws)
    return step


def time_steps(step, steps: int, warmup: int, graph: bool = False):
    """W untimed steps, then K timed steps between two device synchronisations.

    The timed loop is bracketed by one pair of events on the stream the kernels run on (torch's
    current stream, which the binding passes to the library); their elapsed time / K is the
    per-launch duration used for the roofline. With graph=True one step is captured into a HIP
    graph after the warmup and the loop replays it instead of calling the binding (on this
    stack a graph launch costs more than the eager call it replaces for these single-kernel
    steps, so eager calls are the default)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        run = g.replay
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = e0.elapsed_time(e1) / steps
    return {"wall_s": wall, "ms_per_step": wall * 1e3 / steps, "launch_ms_mean": mean,
            "graph": 1.0 if graph else 0.0}


def per_call_times(step, calls: int = 100):
    """Per-call GPU durations: `calls` calls issued back to back, each bracketed by its own pair
    of events on the launch stream. Returns the median and mean in microseconds. A call whose
    host-side issue takes longer than the GPU work before it includes that idle gap."""
    import statistics
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    return {"per_call_us_median": round(statistics.median(us), 3),
            "per_call_us_mean": round(statistics.fmean(us), 3), "per_call_n": calls}


def back_to_back(step, calls: int = 1000):
    """`calls` calls between a single pair of events (no synchronisation in between): the
    per-call time with launch gaps amortised."""
    import torch
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(calls):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / calls, 3)


def load_traffic(kind: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they were taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


# The oracle's sample per workload: (requests to evaluate, None = all; passes; how it is named).
# Prefill samples take whole requests (every head and query row); decode samples whole requests
# (every head). Sizes keep each sample at a few seconds to a few tens of seconds of host work.
CPU_SAMPLES = {1: (None, 3), 2: (None, 25), 3: ([0], 1), 4: (None, 1), 5: ([0, 1], 1), 6: ([0, 1], 1)}


def cpu_baseline(w, c: int):
    """The oracle, as it stands, on the host cores, over a bounded sample of the workload (whole
    requests), timed with perf_counter (best of the passes). Prefill: causal-adjusted TFLOP/s of
    the sampled requests; decode: GB/s of the sampled requests' K/V (same algorithmic bytes as the
    GPU figure)."""
    import numpy as np
    import oracle
    import workloads as wl
    reqs, passes = CPU_SAMPLES.get(c, (None, 1))
    segs, ind, cq, ck = wl.host_tables(w)
    qb, kb, vb = wl.bits(w.q), wl.bits(w.k_pool), wl.bits(w.v_pool)
    ks = None if w.k_scale is None else w.k_scale.detach().cpu().numpy()
    vs = None if w.v_scale is None else w.v_scale.detach().cpu().numpy()
    best = float("inf")
    for _ in range(passes):
        t0 = time.perf_counter()
        oracle.attention(qb, kb, vb, segs, ind, cq, ck, num_heads_kv=w.num_heads_kv,
                         softmax_scale=w.softmax_scale, causal=w.causal, kv_format=w.kv_dtype,
                         k_scale=ks, v_scale=vs, requests=reqs)
        best = min(best, time.perf_counter() - t0)
    sel = list(range(w.batch)) if reqs is None else reqs
    ql, kl = w.q_lens[sel], w.k_lens[sel]
    if w.kind == "prefill":
        pairs = sum(int(a) * (int(k) - int(a)) + int(a) * (int(a) + 1) // 2 if w.causal else int(a) * int(k)
                    for a, k in zip(ql, kl))
        value, unit = 4.0 * w.head_dim * w.num_heads_q * pairs / best / 1e12, "TFLOP/s"
    else:
        per_tok = w.num_heads_kv * w.head_dim * (2 if w.kv_dtype == "bf16" else 1) * 2
        if w.kv_dtype != "bf16":
            per_tok += w.num_heads_kv * 8
        value, unit = float(kl.sum()) * per_tok / best / 1e9, "GB/s"
    what = "the whole workload" if reqs is None else f"requests {reqs} of {w.batch} (every head)"
    return {"value": value, "unit": unit, "cores": int(blas_threads()), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{what}, float64 numpy, best of {passes} pass(es): {best:.2f} s"}


def measure(w, steps, warmup, kind, graph=False, loop_1000=False, per_call=True):
    """Time one workload. The per-call loop (each call between its own events) and, for the
    small prefills, the 1000-call loop run first and the W + K step loop last: the GPU's clocks
    ramp up over the first tens of milliseconds of work, and a K-step loop that started right
    after a cold start (with the few warmup steps a short run gives it) would time that ramp
    instead of the kernels."""
    step = make_step(w)
    t = {}
    if per_call:
        t.update(per_call_times(step))
    if loop_1000 and per_call:
        t["back_to_back_1000_us"] = back_to_back(step, 1000)
    t.update(time_steps(step, steps, warmup, graph))
    if kind == "prefill":
        work = prefill_flops(w)
        achieved = work / (t["launch_ms_mean"] * 1e-3) / 1e12
        per_step = work / (t["ms_per_step"] * 1e-3) / 1e12
        rf = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
              "frac": achieved / PEAK_BF16_TFLOPS, "traffic": load_traffic("prefill", w.name)}
        return per_step, "TFLOP/s", rf, t, work
    work = decode_kv_bytes(w)
    achieved = work / (t["launch_ms_mean"] * 1e-3) / 1e9
    per_step = work / (t["ms_per_step"] * 1e-3) / 1e9
    rf = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
          "frac": achieved / PEAK_HBM_GBS, "traffic": load_traffic("decode", w.name),
          "note": "per call: split kernel + merge kernel"}
    return per_step, "GB/s", rf, t, work


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config", type=int, default=2, help="headline workload (1..6)")
    ap.add_argument("--no-per-call", action="store_true",
                    help="only the K-step loop: no per-call events and no 1000-call loop (profiler runs)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph capturing one step instead of eager calls")
    ap.add_argument("--append-only", default=None, metavar="NAME|all",
                    help="only time the KV appends (one named case, or all), one line each on stderr")
    ap.add_argument("--linear-only", default=None, metavar="NAME|all",
                    help="only time segment linear attention (one named case, or all)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 1 GiB, 5 times (reference kernel "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the segment-attention library runs on a single MI355X "
              "and has no multi-GPU mode (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    import attention_segmented_kv_amd as sa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sa._load()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "launches": 5}}))
        return

    if args.append_only:
        res = []
        for name, c, fmt in APPEND_CASES:
            if args.append_only not in ("all", name):
                continue
            log(f"[bench] timing {name}: warmup {args.warmup}, steps {args.steps}")
            r = measure_append(name, c, fmt, args.steps, args.warmup, dev)
            log(f"[bench] {name}: {r['value']:.1f} GB/s per step, launch mean {r['launch_us_mean']:.2f} us, "
                f"roofline frac {r['roofline']['frac']:.3f}")
            res.append(r)
            torch.cuda.empty_cache()
        print(json.dumps({"append": res}), flush=True)
        return

    if args.linear_only:
        res = []
        for name in LINEAR_CASES:
            if args.linear_only not in ("all", name):
                continue
            log(f"[bench] timing {name}: warmup {args.warmup}, steps {args.steps}")
            r = measure_linear(name, args.steps, args.warmup, dev)
            rf = r["roofline"]
            log(f"[bench] {name}: {r['value']:.2f} us per call, {rf['achieved']:.1f} {rf['unit']}, "
                f"roofline frac {rf['frac']:.3f}")
            res.append(r)
            torch.cuda.empty_cache()
        print(json.dumps({"linear": res}), flush=True)
        return

    head_c = args.config
    log(f"[bench] generating headline workload config {head_c}")
    w = wl.make_config(head_c, device="cpu", poison=True).to(dev) if head_c in (1, 2, 3) \
        else wl.make_config(head_c, device=dev)
    kind = w.kind
    log(f"[bench] timing {w.name}: warmup {args.warmup}, steps {args.steps}")
    value, unit, roof, t, work = measure(w, args.steps, args.warmup, kind, args.graph,
                                         loop_1000=head_c in (1, 2), per_call=not args.no_per_call)
    log(f"[bench] {w.name}: {value:.2f} {unit} per step, launch mean {t['launch_ms_mean']*1e3:.1f} us, "
        f"roofline frac {roof['frac']:.3f}")

    result = {
        "metric": "causal-adj attention TFLOPS (prefill) + KV-read GB/s (decode), 64q/8kv/d128",
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else f"{w.kv_dtype} kv / bf16 mfma",
        "data": "synthetic",
        "config": {"workload": w.name, "recipe": w.recipe, "batch": w.batch,
                   "q_len": int(w.q_lens.max()), "k_len": int(w.k_lens.max()), "heads_q": w.num_heads_q,
                   "heads_kv": w.num_heads_kv, "head_dim": w.head_dim, "causal": w.causal,
                   "seed": w.seed, "parallelism": "single GPU"},
        "roofline": roof,
        "timing": {k: round(v, 6) for k, v in t.items()},
        "work_per_step": work,
    }

    def guarded(name, fn):
        # A secondary workload that raises is recorded as failed (and logged) instead of taking
        # the headline's JSON line down with it; the headline above has already been measured.
        try:
            return fn()
        except Exception as e:  # noqa: BLE001 - reported in the line, not swallowed
            log(f"[bench] {name}: FAILED: {type(e).__name__}: {e}")
            torch.cuda.synchronize()
            return {"workload": name, "error": f"{type(e).__name__}: {e}"}

    if not args.quick:
        extra = []
        for c in (1, 2, 3, 4, 5, 6):
            if c == head_c:
                continue

            def one_config(c=c):
                log(f"[bench] config {c}: generating")
                wc = wl.make_config(c, device=dev)
                v, u, rf, tc, wk = measure(wc, max(20, args.steps // 2), args.warmup, wc.kind, args.graph,
                                           loop_1000=c in (1, 2), per_call=not args.no_per_call)
                log(f"[bench] {wc.name}: {v:.2f} {u}, launch mean {tc['launch_ms_mean']*1e3:.1f} us, "
                    f"per-call median {tc.get('per_call_us_median', float('nan')):.1f} us, frac {rf['frac']:.3f}")
                entry = {"workload": wc.name, "value": round(v, 3), "unit": u,
                         "launch_us_mean": round(tc["launch_ms_mean"] * 1e3, 2),
                         "timing": {k: round(x, 6) for k, x in tc.items()},
                         "roofline": rf, "work_per_step": wk}
                if not args.no_cpu_baseline:
                    log(f"[bench] {wc.name}: cpu baseline (oracle)")
                    entry["cpu_baseline"] = cpu_baseline(wc, c)
                    log(f"[bench] {wc.name}: oracle {entry['cpu_baseline']['value']:.4g} "
                        f"{entry['cpu_baseline']['unit']} ({entry['cpu_baseline']['sample']})")
                return entry

            extra.append(guarded(wl.CONFIG_NAMES[c], one_config))
            torch.cuda.empty_cache()
        result["configs"] = extra
        app = []
        for name, c, fmt in APPEND_CASES:
            def one_append(name=name, c=c, fmt=fmt):
                log(f"[bench] {name}: generating")
                r = measure_append(name, c, fmt, max(20, args.steps // 2), args.warmup, dev)
                log(f"[bench] {name}: {r['value']:.1f} GB/s, launch mean {r['launch_us_mean']:.2f} us, "
                    f"frac {r['roofline']['frac']:.3f}")
                return r
            app.append(guarded(name, one_append))
            torch.cuda.empty_cache()
        result["append"] = app
        lin = []
        for name in LINEAR_CASES:
            def one_linear(name=name):
                log(f"[bench] {name}: generating")
                r = measure_linear(name, max(20, args.steps // 2), args.warmup, dev)
                rf = r["roofline"]
                log(f"[bench] {name}: {r['value']:.2f} us, {rf['achieved']:.1f} {rf['unit']}, frac {rf['frac']:.3f}")
                return r
            lin.append(guarded(name, one_linear))
            torch.cuda.empty_cache()
        result["linear"] = lin
        log("[bench] allocator (host)")
        result["allocator"] = guarded("allocator_decode_loop_b128", measure_allocator)
        if "error" not in result["allocator"]:
            log(f"[bench] allocator_decode_loop_b128: {result['allocator']['us_per_step']} us per step, "
                f"{result['allocator']['segments_per_request_mean']} segments per request")

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = guarded(w.name + " cpu baseline", lambda: cpu_baseline(w, head_c))
        if "error" not in result["cpu_baseline"]:
            log(f"[bench] {w.name}: oracle {result['cpu_baseline']['value']:.4g} {result['cpu_baseline']['unit']}")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
