"""Segment attention for MI355X (gfx950): Python binding of libsegattn.so.

Thin ctypes marshalling over the C ABI in include/seg_attn.h: torch tensors supply device
memory and the current stream; every step of the computation runs in the library's HIP
kernels. If the library has not been built, every call raises.

    out = prefill(q, k_pool, v_pool, segs, seg_indptr, cu_seqlens_q, cu_seqlens_k,
                  max_seqlen_q, max_seqlen_k, causal=True)
    out = decode(q, k_pool, v_pool, segs, seg_indptr, cu_seqlens_k, max_seqlen_k,
                 k_scale=None, v_scale=None)
    kv_append(k_new, v_new, segs, seg_indptr, cu_seqlens_new, cu_seqlens_k, k_pool, v_pool,
              k_scale=None, v_scale=None)
    alloc = SegmentAllocator(pool_tokens); alloc.grow(request, n)
    segs, seg_indptr, cu_seqlens_k = alloc.tables(requests)   # host int32 arrays
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["prefill", "decode", "decode_noalloc", "kv_append", "kv_move", "linear_prefill", "linear_decode", "SegmentAllocator",
           "decode_num_splits", "decode_workspace_bytes", "validate_tables",
           "status_string", "version", "library_path", "SegAttnError", "KV_BF16", "KV_FP8_E4M3",
           "KV_INT8"]

KV_BF16 = 0
KV_FP8_E4M3 = 1
KV_INT8 = 2
_KV_OF_DTYPE = {torch.bfloat16: KV_BF16, torch.float8_e4m3fn: KV_FP8_E4M3, torch.int8: KV_INT8}
HEAD_DIM = 128
GROUP = 8

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_FILES = {"release": "libsegattn.so", "debug": "libsegattn_debug.so"}
# SEG_ATTN_LIBRARY=debug makes the binding load the debug build (tables checked on the host
# before every attention launch; see seg_attn_debug_build in include/seg_attn.h)
_VARIANT = os.environ.get("SEG_ATTN_LIBRARY", "release")
if _VARIANT not in _LIB_FILES:
    raise ValueError(f"SEG_ATTN_LIBRARY must be one of {sorted(_LIB_FILES)}, not {_VARIANT!r}")
_LIB_PATH = os.path.join(_PKG_DIR, _LIB_FILES[_VARIANT])
_lib = None
_libs = {}


class SegAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({status_string(status)})")
        self.status = status


def library_path(variant: Optional[str] = None) -> str:
    """Path of the library the binding loads, or of the named variant ("release", "debug")."""
    return _LIB_PATH if variant is None else os.path.join(_PKG_DIR, _LIB_FILES[variant])


def _load():
    global _lib
    if _lib is None:
        _lib = load_library(_VARIANT)
    return _lib


def load_library(variant: str = "release"):
    """The ctypes handle of a library variant, with every entry point's signature set."""
    if variant in _libs:
        return _libs[variant]
    path = library_path(variant)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m attention_segmented_kv_amd.build --all` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.seg_attn_prefill.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I64, F32, I32, P, P, P]
    lib.seg_attn_prefill.restype = I32
    lib.seg_attn_decode.argtypes = [P, P, P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, I64, F32, I32,
                                    P, P, P, SZ, P]
    lib.seg_attn_decode.restype = I32
    lib.seg_attn_decode_noalloc.argtypes = [P, P, P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, I64, F32,
                                            I32, P, P, P]
    lib.seg_attn_decode_noalloc.restype = I32
    lib.seg_attn_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.seg_attn_decode_workspace_bytes.restype = SZ
    lib.seg_attn_decode_num_splits.argtypes = [I32, I32, I32, I32, I32, ctypes.POINTER(I32)]
    lib.seg_attn_decode_num_splits.restype = I32
    lib.seg_attn_kv_append.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I64, I32, P, P, P, P, P]
    lib.seg_attn_kv_append.restype = I32
    lib.seg_attn_status_string.argtypes = [I32]
    lib.seg_attn_status_string.restype = ctypes.c_char_p
    lib.seg_attn_validate_tables.argtypes = [P, I64, P, P, P, I32, I64, I32, ctypes.POINTER(I64)]
    lib.seg_attn_validate_tables.restype = I32
    lib.seg_attn_version.argtypes = []
    lib.seg_attn_version.restype = I32
    lib.seg_attn_linear_prefill.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, F32, I32, P, I64, P, P,
                                            SZ, P]
    lib.seg_attn_linear_prefill_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.seg_attn_linear_prefill_workspace_bytes.restype = SZ
    lib.seg_attn_linear_prefill.restype = I32
    lib.seg_attn_linear_decode.argtypes = [P, P, P, P, P, I32, I32, I32, F32, P, I64, P, P]
    lib.seg_attn_linear_decode.restype = I32
    PI64 = ctypes.POINTER(I64)
    lib.seg_attn_allocator_create.argtypes = [I64, I64, ctypes.POINTER(P)]
    lib.seg_attn_allocator_create.restype = I32
    lib.seg_attn_allocator_destroy.argtypes = [P]
    lib.seg_attn_allocator_destroy.restype = None
    lib.seg_attn_allocator_grow.argtypes = [P, I64, I64]
    lib.seg_attn_allocator_grow.restype = I32
    lib.seg_attn_allocator_grow_batch.argtypes = [P, P, P, I32, ctypes.POINTER(I32)]
    lib.seg_attn_allocator_grow_batch.restype = I32
    lib.seg_attn_allocator_reserve.argtypes = [P, I64, I64]
    lib.seg_attn_allocator_reserve.restype = I32
    lib.seg_attn_allocator_capacity.argtypes = [P, I64]
    lib.seg_attn_allocator_capacity.restype = I64
    lib.seg_attn_allocator_release.argtypes = [P, I64]
    lib.seg_attn_allocator_release.restype = I32
    lib.seg_attn_allocator_truncate.argtypes = [P, I64, I64]
    lib.seg_attn_allocator_truncate.restype = I32
    lib.seg_attn_allocator_length.argtypes = [P, I64]
    lib.seg_attn_allocator_length.restype = I64
    lib.seg_attn_allocator_tables.argtypes = [P, P, I32, P, I64, P, P, PI64]
    lib.seg_attn_allocator_tables.restype = I32
    lib.seg_attn_allocator_stats.argtypes = [P, PI64, PI64, PI64, PI64]
    lib.seg_attn_allocator_stats.restype = I32
    lib.seg_attn_allocator_free_runs.argtypes = [P, P, I64, PI64]
    lib.seg_attn_allocator_free_runs.restype = I32
    lib.seg_attn_allocator_compact.argtypes = [P, P, I64, PI64]
    lib.seg_attn_allocator_compact.restype = I32
    lib.seg_attn_kv_move.argtypes = [P, I32, I64, I32, I32, I64, I32, P, P, P, P, P]
    lib.seg_attn_kv_move.restype = I32
    lib.seg_attn_debug_build.argtypes = []
    lib.seg_attn_debug_build.restype = I32
    _libs[variant] = lib
    return lib


def status_string(status: int) -> str:
    return _load().seg_attn_status_string(int(status)).decode()


def version() -> int:
    return int(_load().seg_attn_version())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, dtypes, device: torch.device, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, has shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_tables(segs, seg_indptr, cu, device, batch_plus_1, names):
    _check(segs, names[0], (torch.int32,), device, 2)
    if segs.shape[1] != 2:
        raise ValueError(f"{names[0]} must have shape [nseg, 2]")
    _check(seg_indptr, names[1], (torch.int32,), device, 1)
    if seg_indptr.shape[0] != batch_plus_1:
        raise ValueError(f"{names[1]} must have batch + 1 entries")
    for t, nm in zip(cu, names[2:]):
        _check(t, nm, (torch.int32,), device, 1)
        if t.shape[0] != batch_plus_1:
            raise ValueError(f"{nm} must have batch + 1 entries")


def _check_workspace(ws: torch.Tensor, device: torch.device):
    """A caller-supplied workspace: a contiguous byte tensor on the device of the other operands
    (its size is checked by the library)."""
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    if ws.dtype != torch.uint8:
        raise TypeError(f"workspace has dtype {ws.dtype}, expected torch.uint8")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def prefill(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, segs: torch.Tensor,
            seg_indptr: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
            max_seqlen_q: int, max_seqlen_k: int, *, causal: bool = True,
            softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Varlen (chunked) prefill over a segmented KV pool; see seg_attn_prefill in seg_attn.h.

    q [total_q, Hq, 128] bf16; k_pool/v_pool [pool_tokens, Hkv, 128] bf16; segs [nseg, 2]
    int32 (pool_offset, length); seg_indptr, cu_seqlens_q, cu_seqlens_k [B+1] int32.
    Returns out [total_q, Hq, 128] bf16 (and lse [total_q, Hq] fp32 if return_lse)."""
    lib = _load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    _check(q, "q", (torch.bfloat16,), dev, 3)
    _check(k_pool, "k_pool", (torch.bfloat16,), dev, 3)
    _check(v_pool, "v_pool", (torch.bfloat16,), dev, 3)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    batch = cu_seqlens_q.shape[0] - 1
    _check_tables(segs, seg_indptr, (cu_seqlens_q, cu_seqlens_k), dev, batch + 1,
                  ("segs", "seg_indptr", "cu_seqlens_q", "cu_seqlens_k"))
    total_q, hq, d = q.shape
    pool_tokens, hkv, dk = k_pool.shape
    if dk != d:
        raise ValueError("q and k_pool head dims differ")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", (torch.bfloat16,), dev, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if return_lse and lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", (torch.float32,), dev, 2)
        if tuple(lse.shape) != (total_q, hq):
            raise ValueError("lse must have shape [total_q, Hq]")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.seg_attn_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(segs), _ptr(seg_indptr),
                                  _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, int(max_seqlen_q),
                                  int(max_seqlen_k), hq, hkv, d, pool_tokens, float(softmax_scale),
                                  1 if causal else 0, _ptr(out), _ptr(lse), stream)
    if st != 0:
        raise SegAttnError("seg_attn_prefill", st)
    return (out, lse) if return_lse else out


def decode_num_splits(batch: int, max_seqlen_k: int, num_heads_kv: int = 8, kv_dtype: int = KV_BF16,
                      num_splits: int = 0):
    """(num_splits, split_len) the decode call will use on the current device."""
    ln = ctypes.c_int32(0)
    n = _load().seg_attn_decode_num_splits(batch, max_seqlen_k, num_heads_kv, kv_dtype, num_splits,
                                           ctypes.byref(ln))
    if n < 0:
        raise ValueError("invalid sizes for decode_num_splits")
    return int(n), int(ln.value)


def decode_workspace_bytes(batch: int, max_seqlen_k: int, num_heads_q: int = 64, num_heads_kv: int = 8,
                           head_dim: int = HEAD_DIM, kv_dtype: int = KV_BF16, num_splits: int = 0) -> int:
    return int(_load().seg_attn_decode_workspace_bytes(batch, max_seqlen_k, num_heads_q, num_heads_kv,
                                                      head_dim, kv_dtype, num_splits))


def _decode_args(q, k_pool, v_pool, segs, seg_indptr, cu_seqlens_k, k_scale, v_scale, softmax_scale,
                 out, lse, return_lse):
    """Argument checks shared by decode and decode_noalloc; allocates out / lse when not given."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    _check(q, "q", (torch.bfloat16,), dev, 3)
    if k_pool.dtype not in _KV_OF_DTYPE:
        raise TypeError(f"k_pool has dtype {k_pool.dtype}: expected bfloat16, float8_e4m3fn or int8")
    kv_dtype = _KV_OF_DTYPE[k_pool.dtype]
    scaled = kv_dtype != KV_BF16
    _check(k_pool, "k_pool", (k_pool.dtype,), dev, 3)
    _check(v_pool, "v_pool", (k_pool.dtype,), dev, 3)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    batch, hq, d = q.shape
    pool_tokens, hkv, _ = k_pool.shape
    _check_tables(segs, seg_indptr, (cu_seqlens_k,), dev, batch + 1,
                  ("segs", "seg_indptr", "cu_seqlens_k"))
    if scaled:
        if k_scale is None or v_scale is None:
            raise ValueError("an fp8 or int8 pool needs k_scale and v_scale")
        for t, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            _check(t, nm, (torch.float32,), dev, 2)
            if tuple(t.shape) != (pool_tokens, hkv):
                raise ValueError(f"{nm} must have shape [pool_tokens, Hkv]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", (torch.bfloat16,), dev, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if return_lse and lse is None:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", (torch.float32,), dev, 2)
        if tuple(lse.shape) != (batch, hq):
            raise ValueError("lse must have shape [B, Hq]")
    return dev, kv_dtype, batch, hq, hkv, d, pool_tokens, float(softmax_scale), out, lse


def decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, segs: torch.Tensor,
           seg_indptr: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_k: int, *,
           k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
           softmax_scale: Optional[float] = None, num_splits: int = 0,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Single-token decode with split-K and a log-sum-exp merge; see seg_attn_decode.

    q [B, Hq, 128] bf16; k_pool/v_pool [pool_tokens, Hkv, 128] bf16, or float8_e4m3fn / int8
    codes with k_scale/v_scale [pool_tokens, Hkv] fp32. A workspace is allocated here unless
    given."""
    lib = _load()
    dev, kv_dtype, batch, hq, hkv, d, pool_tokens, scale, out, lse = _decode_args(
        q, k_pool, v_pool, segs, seg_indptr, cu_seqlens_k, k_scale, v_scale, softmax_scale, out, lse,
        return_lse)
    scaled = kv_dtype != KV_BF16
    if workspace is not None:
        _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        need = int(lib.seg_attn_decode_workspace_bytes(batch, int(max_seqlen_k), hq, hkv, d, kv_dtype,
                                                       int(num_splits)))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.seg_attn_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale if scaled else None),
                                 _ptr(v_scale if scaled else None), kv_dtype, _ptr(segs),
                                 _ptr(seg_indptr), _ptr(cu_seqlens_k), batch, int(max_seqlen_k), hq,
                                 hkv, d, pool_tokens, scale, int(num_splits), _ptr(out), _ptr(lse),
                                 _ptr(workspace), ws_bytes, stream)
    if st != 0:
        raise SegAttnError("seg_attn_decode", st)
    return (out, lse) if return_lse else out


def decode_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, segs: torch.Tensor,
                   seg_indptr: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_k: int, *,
                   k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                   softmax_scale: Optional[float] = None, num_splits: int = 0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   return_lse: bool = False):
    """decode() through seg_attn_decode_noalloc: no workspace; the library's fixed per-GPU
    scratch holds the plan and partials (calls that overlap in time on one GPU race). With out
    (and lse, if wanted) given, nothing is allocated on the device."""
    lib = _load()
    dev, kv_dtype, batch, hq, hkv, d, pool_tokens, scale, out, lse = _decode_args(
        q, k_pool, v_pool, segs, seg_indptr, cu_seqlens_k, k_scale, v_scale, softmax_scale, out, lse,
        return_lse)
    scaled = kv_dtype != KV_BF16
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.seg_attn_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool),
                                         _ptr(k_scale if scaled else None), _ptr(v_scale if scaled else None),
                                         kv_dtype, _ptr(segs), _ptr(seg_indptr), _ptr(cu_seqlens_k), batch,
                                         int(max_seqlen_k), hq, hkv, d, pool_tokens, scale,
                                         int(num_splits), _ptr(out), _ptr(lse), stream)
    if st != 0:
        raise SegAttnError("seg_attn_decode_noalloc", st)
    return (out, lse) if return_lse else out


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, segs: torch.Tensor, seg_indptr: torch.Tensor,
              cu_seqlens_new: torch.Tensor, cu_seqlens_k: torch.Tensor, k_pool: torch.Tensor,
              v_pool: torch.Tensor, *, k_scale: Optional[torch.Tensor] = None,
              v_scale: Optional[torch.Tensor] = None) -> None:
    """Write new tokens into their requests' segments, in place; see seg_attn_kv_append.

    k_new/v_new [total_new, Hkv, 128] bf16; segs/seg_indptr/cu_seqlens_k describe the requests
    after the append (their last n_b keys are the new tokens); cu_seqlens_new [B+1] int32.
    A bf16 pool gets the rows as they are; a float8_e4m3fn or int8 pool gets per-row scaled
    codes and k_scale/v_scale [pool_tokens, Hkv] fp32 the scales."""
    lib = _load()
    dev = k_new.device
    if dev.type != "cuda":
        raise ValueError("k_new must be a GPU tensor")
    _check(k_new, "k_new", (torch.bfloat16,), dev, 3)
    _check(v_new, "v_new", (torch.bfloat16,), dev, 3)
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must have the same shape")
    if k_pool.dtype not in _KV_OF_DTYPE:
        raise TypeError(f"k_pool has dtype {k_pool.dtype}: expected bfloat16, float8_e4m3fn or int8")
    kv_dtype = _KV_OF_DTYPE[k_pool.dtype]
    scaled = kv_dtype != KV_BF16
    _check(k_pool, "k_pool", (k_pool.dtype,), dev, 3)
    _check(v_pool, "v_pool", (k_pool.dtype,), dev, 3)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    total_new, hkv, d = k_new.shape
    pool_tokens = k_pool.shape[0]
    if tuple(k_pool.shape[1:]) != (hkv, d):
        raise ValueError("k_new rows and pool rows differ in shape")
    batch = cu_seqlens_new.shape[0] - 1
    _check_tables(segs, seg_indptr, (cu_seqlens_new, cu_seqlens_k), dev, batch + 1,
                  ("segs", "seg_indptr", "cu_seqlens_new", "cu_seqlens_k"))
    if scaled:
        if k_scale is None or v_scale is None:
            raise ValueError("an fp8 or int8 pool needs k_scale and v_scale")
        for t, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            _check(t, nm, (torch.float32,), dev, 2)
            if tuple(t.shape) != (pool_tokens, hkv):
                raise ValueError(f"{nm} must have shape [pool_tokens, Hkv]")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.seg_attn_kv_append(_ptr(k_new), _ptr(v_new), _ptr(segs), _ptr(seg_indptr),
                                    _ptr(cu_seqlens_new), _ptr(cu_seqlens_k), batch, total_new, hkv, d,
                                    pool_tokens, kv_dtype, _ptr(k_pool), _ptr(v_pool),
                                    _ptr(k_scale if scaled else None),
                                    _ptr(v_scale if scaled else None), stream)
    if st != 0:
        raise SegAttnError("seg_attn_kv_append", st)


def kv_move(moves: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, *,
            k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
            total_tokens: Optional[int] = None) -> None:
    """Apply a compaction's moves to the pools in place (seg_attn_kv_move). moves: int32 [n, 4]
    (src_offset, dst_offset, length, first) on the pools' device; total_tokens (the sum of the
    lengths) is read from the tensor unless given."""
    lib = _load()
    dev = k_pool.device
    if dev.type != "cuda":
        raise ValueError("k_pool must be a GPU tensor")
    if k_pool.dtype not in _KV_OF_DTYPE:
        raise TypeError(f"k_pool has dtype {k_pool.dtype}: expected bfloat16, float8_e4m3fn or int8")
    kv_dtype = _KV_OF_DTYPE[k_pool.dtype]
    scaled = kv_dtype != KV_BF16
    _check(k_pool, "k_pool", (k_pool.dtype,), dev, 3)
    _check(v_pool, "v_pool", (k_pool.dtype,), dev, 3)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    _check(moves, "moves", (torch.int32,), dev, 2)
    if moves.shape[1] != 4:
        raise ValueError("moves must have shape [n, 4]")
    pool_tokens, hkv, d = k_pool.shape
    if scaled:
        if k_scale is None or v_scale is None:
            raise ValueError("an fp8 or int8 pool needs k_scale and v_scale")
        for t, nm in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            _check(t, nm, (torch.float32,), dev, 2)
            if tuple(t.shape) != (pool_tokens, hkv):
                raise ValueError(f"{nm} must have shape [pool_tokens, Hkv]")
    n = moves.shape[0]
    if total_tokens is None:
        total_tokens = int(moves[:, 2].sum().item()) if n else 0
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.seg_attn_kv_move(_ptr(moves), n, int(total_tokens), hkv, d, pool_tokens, kv_dtype,
                                  _ptr(k_pool), _ptr(v_pool), _ptr(k_scale if scaled else None),
                                  _ptr(v_scale if scaled else None), stream)
    if st != 0:
        raise SegAttnError("seg_attn_kv_move", st)


def _check_linear(q, k, v, g, state_slots, state_pool, batch):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, (torch.bfloat16,), dev, 3)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape")
    T, H, D = q.shape
    _check(g, "g", (torch.float32,), dev, 2)
    if tuple(g.shape) != (T, H):
        raise ValueError("g must have shape [T, H]")
    _check(state_slots, "state_slots", (torch.int32,), dev, 1)
    if state_slots.shape[0] != batch:
        raise ValueError("state_slots must have one entry per request")
    _check(state_pool, "state_pool", (torch.float32,), dev, 4)
    if tuple(state_pool.shape[1:]) != (H, D, D):
        raise ValueError("state_pool must have shape [slots, H, D, D]")
    return dev, T, H, D


def linear_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   cu_seqlens: torch.Tensor, state_slots: torch.Tensor, state_pool: torch.Tensor, *,
                   initial_state: bool = True, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                   parallel: bool = True, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Segment linear attention over a varlen batch; see seg_attn_linear_prefill. The final
    states are written to state_pool[state_slots] in place. Returns out [T, H, 128] bf16.

    parallel=True runs all chunks in parallel with a workspace (allocated here unless given;
    max_seqlen is read from cu_seqlens, a device-to-host copy, unless given); parallel=False
    walks each request's chunks in order in one kernel."""
    lib = _load()
    batch = cu_seqlens.shape[0] - 1
    dev, T, H, D = _check_linear(q, k, v, g, state_slots, state_pool, batch)
    _check(cu_seqlens, "cu_seqlens", (torch.int32,), dev, 1)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", (torch.bfloat16,), dev, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    ws_bytes = 0
    if parallel:
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if batch > 0 else 0
        need = int(lib.seg_attn_linear_prefill_workspace_bytes(batch, int(max_seqlen), H, D))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        else:
            _check_workspace(workspace, dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.seg_attn_linear_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(cu_seqlens),
                                         _ptr(state_slots), batch, int(max_seqlen or 0), H, D,
                                         float(scale), 1 if initial_state else 0, _ptr(state_pool),
                                         state_pool.shape[0], _ptr(out), _ptr(workspace), ws_bytes,
                                         stream)
    if st != 0:
        raise SegAttnError("seg_attn_linear_prefill", st)
    return out


def linear_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  state_slots: torch.Tensor, state_pool: torch.Tensor, *, scale: Optional[float] = None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per request (row b of q, k, v, g) against its state slot, updated in place; see
    seg_attn_linear_decode. Returns out [B, H, 128] bf16."""
    lib = _load()
    batch = q.shape[0]
    dev, T, H, D = _check_linear(q, k, v, g, state_slots, state_pool, batch)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", (torch.bfloat16,), dev, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.seg_attn_linear_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state_slots), batch,
                                        H, D, float(scale), _ptr(state_pool), state_pool.shape[0],
                                        _ptr(out), stream)
    if st != 0:
        raise SegAttnError("seg_attn_linear_decode", st)
    return out


class SegmentAllocator:
    """Host-side segment allocator over a pool of ``pool_tokens`` slots (the
    seg_attn_allocator_* functions of seg_attn.h). Not thread-safe.

    grow(request, n) adds n keys and raises SegAttnError (status 6), changing nothing, when the
    request's spare capacity and the free slots hold fewer; shortfalls are rounded up to
    ``granule`` slots. reserve(request, capacity) sets slots aside for a known final length.
    tables(requests) returns host int32 numpy arrays (segs [nseg, 2], seg_indptr [B+1],
    cu_seqlens_k [B+1]) for the entry points; move them to the device with
    torch.from_numpy(...).to(device)."""

    def __init__(self, pool_tokens: int, granule: int = 1):
        self._lib = _load()
        h = ctypes.c_void_p()
        st = self._lib.seg_attn_allocator_create(int(pool_tokens), int(granule), ctypes.byref(h))
        if st != 0:
            raise SegAttnError("seg_attn_allocator_create", st)
        self._h = h
        self.pool_tokens = int(pool_tokens)
        self.granule = int(granule)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value is not None:
            self._lib.seg_attn_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _call(self, name, *args):
        if self._h is None:
            raise RuntimeError("allocator is closed")
        st = getattr(self._lib, name)(self._h, *args)
        if st != 0:
            raise SegAttnError(name, st)

    def grow(self, request: int, n: int) -> None:
        self._call("seg_attn_allocator_grow", int(request), int(n))

    def grow_many(self, requests, n) -> None:
        """grow(requests[i], n[i]) in order in one call; on failure raises SegAttnError with the
        number applied before the failing one in its ``done`` attribute."""
        import numpy as np
        req = np.ascontiguousarray(np.asarray(requests, dtype=np.int64).reshape(-1))
        cnt = np.ascontiguousarray(np.broadcast_to(np.asarray(n, dtype=np.int64), req.shape))
        done = ctypes.c_int32(0)
        if self._h is None:
            raise RuntimeError("allocator is closed")
        st = self._lib.seg_attn_allocator_grow_batch(self._h, req.ctypes.data, cnt.ctypes.data,
                                                     req.shape[0], ctypes.byref(done))
        if st != 0:
            err = SegAttnError("seg_attn_allocator_grow_batch", st)
            err.done = int(done.value)
            raise err

    def reserve(self, request: int, capacity: int) -> None:
        self._call("seg_attn_allocator_reserve", int(request), int(capacity))

    def release(self, request: int) -> None:
        self._call("seg_attn_allocator_release", int(request))

    def truncate(self, request: int, new_length: int) -> None:
        self._call("seg_attn_allocator_truncate", int(request), int(new_length))

    def length(self, request: int) -> int:
        if self._h is None:
            raise RuntimeError("allocator is closed")
        return int(self._lib.seg_attn_allocator_length(self._h, int(request)))

    def capacity(self, request: int) -> int:
        if self._h is None:
            raise RuntimeError("allocator is closed")
        return int(self._lib.seg_attn_allocator_capacity(self._h, int(request)))

    def stats(self) -> dict:
        v = [ctypes.c_int64(0) for _ in range(4)]
        self._call("seg_attn_allocator_stats", *[ctypes.byref(x) for x in v])
        return dict(zip(("free_tokens", "largest_free_run", "free_runs", "requests"),
                        (int(x.value) for x in v)))

    def free_runs(self):
        import numpy as np
        cnt = ctypes.c_int64(0)
        st = self._lib.seg_attn_allocator_free_runs(self._h, None, 0, ctypes.byref(cnt))
        if st not in (0, 3):
            raise SegAttnError("seg_attn_allocator_free_runs", st)
        runs = np.zeros((max(int(cnt.value), 1), 2), dtype=np.int32)
        self._call("seg_attn_allocator_free_runs", runs.ctypes.data, runs.shape[0], ctypes.byref(cnt))
        return runs[:int(cnt.value)]

    def compact(self):
        """Relocate fragmented requests into single ranges (seg_attn_allocator_compact). Returns
        the moves as a host int32 array [n, 4] of (src_offset, dst_offset, length, first); apply
        them to the pools with kv_move before using new tables."""
        import numpy as np
        if self._h is None:
            raise RuntimeError("allocator is closed")
        cnt = ctypes.c_int64(0)
        moves = np.zeros((64, 4), dtype=np.int32)
        while True:
            st = self._lib.seg_attn_allocator_compact(self._h, moves.ctypes.data, moves.shape[0],
                                                      ctypes.byref(cnt))
            if st == 0:
                return moves[:int(cnt.value)]
            if st != 3:
                raise SegAttnError("seg_attn_allocator_compact", st)
            moves = np.zeros((int(cnt.value), 4), dtype=np.int32)

    def tables(self, requests):
        import numpy as np
        req = np.ascontiguousarray(np.asarray(requests, dtype=np.int64).reshape(-1))
        b = req.shape[0]
        ind = np.zeros(b + 1, dtype=np.int32)
        cu = np.zeros(b + 1, dtype=np.int32)
        n = ctypes.c_int64(0)
        st = self._lib.seg_attn_allocator_tables(self._h, req.ctypes.data if b else None, b, None, 0,
                                                 ind.ctypes.data, cu.ctypes.data, ctypes.byref(n))
        if st not in (0, 3):
            raise SegAttnError("seg_attn_allocator_tables", st)
        segs = np.zeros((max(int(n.value), 1), 2), dtype=np.int32)
        self._call("seg_attn_allocator_tables", req.ctypes.data if b else None, b, segs.ctypes.data,
                   segs.shape[0], ind.ctypes.data, cu.ctypes.data, ctypes.byref(n))
        return segs[:int(n.value)], ind, cu


def validate_tables(segs, seg_indptr, cu_seqlens_k, pool_tokens: int, *, cu_seqlens_q=None,
                    causal: bool = True):
    """Host-side table check (seg_attn_validate_tables). Accepts CPU tensors or numpy arrays.
    Returns (status, bad_index)."""
    import numpy as np
    lib = _load()
    as_np = lambda a: np.ascontiguousarray(
        (a.detach().cpu().numpy() if isinstance(a, torch.Tensor) else np.asarray(a)).astype(np.int32))
    s = as_np(segs).reshape(-1, 2)
    ind = as_np(seg_indptr)
    ck = as_np(cu_seqlens_k)
    cq = None if cu_seqlens_q is None else as_np(cu_seqlens_q)
    bad = ctypes.c_int64(0)
    st = lib.seg_attn_validate_tables(s.ctypes.data if s.size else None, s.shape[0], ind.ctypes.data,
                                      None if cq is None else cq.ctypes.data, ck.ctypes.data,
                                      len(ck) - 1, int(pool_tokens), 1 if causal else 0,
                                      ctypes.byref(bad))
    return int(st), int(bad.value)
