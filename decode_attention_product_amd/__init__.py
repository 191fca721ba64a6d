"""Python binding of the PQ-KV decode-attention library (libpqattn.so).

Argument marshalling only: torch tensors supply device memory and the
stream, every step of the computation runs in the library's HIP kernels.
The functions carry the C entry points' names; see include/pqattn.h for
the contract of each.  There is no fallback: if the library is missing or
cannot be loaded, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpqattn.so")

PQ_OK = 0
PQ_ERR_SHAPE_CODE = 2
STATUS_NAMES = {0: "PQ_OK", 1: "PQ_ERR_NULL", 2: "PQ_ERR_SHAPE", 3: "PQ_ERR_UNSUPPORTED",
                4: "PQ_ERR_WORKSPACE", 5: "PQ_ERR_HIP", 6: "PQ_ERR_ALIGN"}

EXPORTED = ("pq_attn_num_chunks", "pq_attn_workspace_bytes", "pq_attn_decode",
            "pq_attn_partials", "pq_attn_partials_timed", "pq_attn_step_workspace_bytes",
            "pq_attn_decode_step", "pq_attn_decode_step_timed", "pq_attn_decode_paged",
            "pq_attn_partials_paged",
            "pq_attn_decode_step_paged", "pq_attn_decode_step_paged_timed", "pq_attn_reduce",
            "pq_encode", "pq_encode_many", "pq_codebook_update", "pq_kmeans",
            "pq_kmeans_many", "pq_attn_decode_fp8cb", "pq_attn_partials_fp8cb",
            "pq_encode_fp8cb", "pq_attn_decode_step_noalloc", "pq_attn_reduce_polyexp",
            "pq_status_string")


class PQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class PQAttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_sub", ctypes.c_int32), ("n_codes", ctypes.c_int32),
                ("max_len", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class PQEncodeDesc(ctypes.Structure):
    _fields_ = [("n_vec", ctypes.c_int64), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_sub", ctypes.c_int32),
                ("n_codes", ctypes.c_int32), ("x_stride_vec", ctypes.c_int64),
                ("x_stride_head", ctypes.c_int64), ("codes_stride_slot", ctypes.c_int64),
                ("codes_stride_head", ctypes.c_int64), ("codes_bytes", ctypes.c_int64)]


class PQPageTable(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("page_tokens", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpqattn.so once; raises if it is missing (build it first with
    ``python -m decode_attention_product_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m decode_attention_product_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.pq_attn_num_chunks.argtypes = [ctypes.POINTER(PQAttnDesc)]
    lib.pq_attn_num_chunks.restype = ctypes.c_int32
    lib.pq_attn_workspace_bytes.argtypes = [ctypes.POINTER(PQAttnDesc)]
    lib.pq_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.pq_attn_decode.argtypes = [ctypes.POINTER(PQAttnDesc), P, P, P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
    lib.pq_attn_decode.restype = ctypes.c_int
    lib.pq_attn_partials.argtypes = [ctypes.POINTER(PQAttnDesc), P, P, P, P, P, P, P, P, P, P]
    lib.pq_attn_partials.restype = ctypes.c_int
    lib.pq_attn_partials_timed.argtypes = [ctypes.POINTER(PQAttnDesc), P, P, P, P, P, P, P, P, P,
                                           P, P, P]
    lib.pq_attn_partials_timed.restype = ctypes.c_int
    lib.pq_attn_step_workspace_bytes.argtypes = [ctypes.POINTER(PQAttnDesc)]
    lib.pq_attn_step_workspace_bytes.restype = ctypes.c_size_t
    lib.pq_attn_decode_step.argtypes = [ctypes.POINTER(PQAttnDesc), P, P, P, P, P, P, P, P, P,
                                        P, ctypes.c_size_t, P]
    lib.pq_attn_decode_step.restype = ctypes.c_int
    lib.pq_attn_decode_step_timed.argtypes = [ctypes.POINTER(PQAttnDesc), P, P, P, P, P, P, P,
                                              P, P, P, ctypes.c_size_t, P, P, P]
    lib.pq_attn_decode_step_timed.restype = ctypes.c_int
    PT = ctypes.POINTER(PQPageTable)
    lib.pq_attn_decode_paged.argtypes = [ctypes.POINTER(PQAttnDesc), PT, P, P, P, P, P, P, P, P,
                                         ctypes.c_size_t, P]
    lib.pq_attn_decode_paged.restype = ctypes.c_int
    lib.pq_attn_partials_paged.argtypes = [ctypes.POINTER(PQAttnDesc), PT, P, P, P, P, P, P, P, P,
                                           P, P]
    lib.pq_attn_partials_paged.restype = ctypes.c_int
    lib.pq_attn_decode_step_paged.argtypes = [ctypes.POINTER(PQAttnDesc), PT, P, P, P, P, P, P,
                                              P, P, P, P, ctypes.c_size_t, P]
    lib.pq_attn_decode_step_paged.restype = ctypes.c_int
    lib.pq_attn_decode_step_paged_timed.argtypes = [ctypes.POINTER(PQAttnDesc), PT, P, P, P, P,
                                                    P, P, P, P, P, P, ctypes.c_size_t, P, P, P]
    lib.pq_attn_decode_step_paged_timed.restype = ctypes.c_int
    lib.pq_attn_reduce.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
    lib.pq_attn_reduce.restype = ctypes.c_int
    lib.pq_attn_reduce_polyexp.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P,
                                           P, P]
    lib.pq_attn_reduce_polyexp.restype = ctypes.c_int
    lib.pq_encode.argtypes = [ctypes.POINTER(PQEncodeDesc), P, P, P, P, P]
    lib.pq_encode.restype = ctypes.c_int
    lib.pq_encode_many.argtypes = [ctypes.POINTER(PQEncodeDesc), ctypes.c_int32,
                                   ctypes.POINTER(P), ctypes.POINTER(P), P, ctypes.POINTER(P), P]
    lib.pq_encode_many.restype = ctypes.c_int
    lib.pq_codebook_update.argtypes = [ctypes.POINTER(PQEncodeDesc), P, P, P, P, P]
    lib.pq_codebook_update.restype = ctypes.c_int
    lib.pq_kmeans.argtypes = [ctypes.POINTER(PQEncodeDesc), P, P, ctypes.c_int32, P, P]
    lib.pq_kmeans.restype = ctypes.c_int
    lib.pq_kmeans_many.argtypes = [ctypes.POINTER(PQEncodeDesc), ctypes.c_int32, ctypes.POINTER(P),
                                   ctypes.POINTER(P), ctypes.c_int32, ctypes.POINTER(P), P]
    lib.pq_kmeans_many.restype = ctypes.c_int
    lib.pq_attn_decode_fp8cb.argtypes = [ctypes.POINTER(PQAttnDesc), P, P, P, P, P, P, P, P,
                                         ctypes.c_size_t, P]
    lib.pq_attn_decode_fp8cb.restype = ctypes.c_int
    lib.pq_attn_partials_fp8cb.argtypes = [ctypes.POINTER(PQAttnDesc), P, P, P, P, P, P, P, P, P, P]
    lib.pq_attn_partials_fp8cb.restype = ctypes.c_int
    lib.pq_encode_fp8cb.argtypes = [ctypes.POINTER(PQEncodeDesc), P, P, P, P, P]
    lib.pq_encode_fp8cb.restype = ctypes.c_int
    lib.pq_attn_decode_step_noalloc.argtypes = [ctypes.POINTER(PQAttnDesc), P, P, P, P, P, P, P, P,
                                                P, P]
    lib.pq_attn_decode_step_noalloc.restype = ctypes.c_int
    lib.pq_status_string.argtypes = [ctypes.c_int]
    lib.pq_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().pq_status_string(int(status)).decode()


pq_status_string = status_string


def _check(status: int, where: str):
    if status != PQ_OK:
        raise PQError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _need(t, name, dtype, shape=None, device=True):
    if t is None:
        return
    # fast path (a call per launch argument): dtypes are singletons, and a
    # torch.Size equals the tuple of its sizes
    if (t.dtype is dtype and (shape is None or t.shape == shape) and t.is_contiguous()
            and (t.is_cuda or not device)):
        return
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    del torch


def attn_desc(q, k_codes, k_cb, *, chunk: int = 0, scale: Optional[float] = None) -> PQAttnDesc:
    """Descriptor from tensor shapes: q [B,Hq,D], k_codes [B,Hkv,Lmax,M],
    k_cb [Hkv,M,K,D/M]."""
    B, Hq, D = q.shape
    _, Hkv, Lmax, M = k_codes.shape
    K = k_cb.shape[2]
    return PQAttnDesc(B, Hq, Hkv, D, M, K, Lmax, int(chunk),
                      float(scale if scale is not None else 1.0 / math.sqrt(D)))


def pq_attn_num_chunks(desc: PQAttnDesc) -> int:
    return int(load_library().pq_attn_num_chunks(ctypes.byref(desc)))


def pq_attn_workspace_bytes(desc: PQAttnDesc) -> int:
    return int(load_library().pq_attn_workspace_bytes(ctypes.byref(desc)))


def _check_attn_inputs(desc, q, k_codes, v_codes, k_cb, v_cb, lens, cb_dtype=None):
    import torch
    B, Hq, Hkv, D = desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.head_dim
    M, K, L = desc.n_sub, desc.n_codes, desc.max_len
    cb_dtype = torch.float16 if cb_dtype is None else cb_dtype
    _need(q, "q", torch.float16, (B, Hq, D))
    _need(k_codes, "k_codes", torch.uint8, (B, Hkv, L, M))
    _need(v_codes, "v_codes", torch.uint8, (B, Hkv, L, M))
    _need(k_cb, "k_cb", cb_dtype, (Hkv, M, K, D // M))
    _need(v_cb, "v_cb", cb_dtype, (Hkv, M, K, D // M))
    _need(lens, "lens", torch.int32, (B,))


def pq_attn_decode(q, k_codes, v_codes, k_cb, v_cb, lens, out=None, *, desc=None, chunk=0,
                   scale=None, workspace=None, stream=None):
    """One decode step (C entry point pq_attn_decode).  Returns ``out``
    (fp32 [B, Hq, D]), allocated if not given.  The workspace is allocated
    through torch when not given."""
    import torch
    if desc is None:
        desc = attn_desc(q, k_codes, k_cb, chunk=chunk, scale=scale)
    _check_attn_inputs(desc, q, k_codes, v_codes, k_cb, v_cb, lens)
    if out is None:
        out = torch.empty((desc.batch, desc.n_q_heads, desc.head_dim), dtype=torch.float32,
                          device=q.device)
    _need(out, "out", torch.float32, (desc.batch, desc.n_q_heads, desc.head_dim))
    ws_bytes = pq_attn_workspace_bytes(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().pq_attn_decode(
        ctypes.byref(desc), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_cb), _ptr(v_cb),
        _ptr(lens), _ptr(out), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "pq_attn_decode")
    return out


def pq_attn_partials(q, k_codes, v_codes, k_cb, v_cb, lens, *, desc=None, chunk=0, scale=None,
                     part_m=None, part_l=None, part_o=None, stream=None, events=None):
    """Chunk statistics (C entry point pq_attn_partials).  Returns
    (part_m [B,Hq,C], part_l [B,Hq,C], part_o [B,Hq,C,D]), fp32.  With
    ``events=(start, stop)`` (raw hipEvent_t handles) the call goes through
    pq_attn_partials_timed and the events bracket the kernel's execution."""
    import torch
    if desc is None:
        desc = attn_desc(q, k_codes, k_cb, chunk=chunk, scale=scale)
    _check_attn_inputs(desc, q, k_codes, v_codes, k_cb, v_cb, lens)
    C = pq_attn_num_chunks(desc)
    if C < 1:
        _check(load_library().pq_attn_partials(ctypes.byref(desc), *([None] * 10)),
               "pq_attn_partials")
    B, Hq, D = desc.batch, desc.n_q_heads, desc.head_dim
    dev = q.device
    part_m = torch.empty((B, Hq, C), dtype=torch.float32, device=dev) if part_m is None else part_m
    part_l = torch.empty((B, Hq, C), dtype=torch.float32, device=dev) if part_l is None else part_l
    part_o = torch.empty((B, Hq, C, D), dtype=torch.float32, device=dev) if part_o is None else part_o
    _need(part_m, "part_m", torch.float32, (B, Hq, C))
    _need(part_l, "part_l", torch.float32, (B, Hq, C))
    _need(part_o, "part_o", torch.float32, (B, Hq, C, D))
    lib = load_library()
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_cb), _ptr(v_cb),
            _ptr(lens), _ptr(part_m), _ptr(part_l), _ptr(part_o), _stream(stream))
    if events is None:
        st = lib.pq_attn_partials(*args)
    else:
        st = lib.pq_attn_partials_timed(*args, events[0], events[1])
    _check(st, "pq_attn_partials")
    return part_m, part_l, part_o


def pq_attn_decode_fp8cb(q, k_codes, v_codes, k_cb, v_cb, lens, out=None, *, desc=None, chunk=0,
                         scale=None, workspace=None, stream=None):
    """pq_attn_decode with FP8 E4M3 codebooks (C entry point
    pq_attn_decode_fp8cb): k_cb and v_cb are uint8 [Hkv, M, K, D/M] tensors
    of E4M3 bytes.  Returns ``out`` (fp32 [B, Hq, D])."""
    import torch
    if desc is None:
        desc = attn_desc(q, k_codes, k_cb, chunk=chunk, scale=scale)
    _check_attn_inputs(desc, q, k_codes, v_codes, k_cb, v_cb, lens, torch.uint8)
    if out is None:
        out = torch.empty((desc.batch, desc.n_q_heads, desc.head_dim), dtype=torch.float32,
                          device=q.device)
    _need(out, "out", torch.float32, (desc.batch, desc.n_q_heads, desc.head_dim))
    ws_bytes = pq_attn_workspace_bytes(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().pq_attn_decode_fp8cb(
        ctypes.byref(desc), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_cb), _ptr(v_cb),
        _ptr(lens), _ptr(out), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "pq_attn_decode_fp8cb")
    return out


def pq_attn_partials_fp8cb(q, k_codes, v_codes, k_cb, v_cb, lens, *, desc=None, chunk=0,
                           scale=None, stream=None):
    """Chunk statistics with FP8 E4M3 codebooks (C entry point
    pq_attn_partials_fp8cb); returns (part_m, part_l, part_o) as
    pq_attn_partials does."""
    import torch
    if desc is None:
        desc = attn_desc(q, k_codes, k_cb, chunk=chunk, scale=scale)
    _check_attn_inputs(desc, q, k_codes, v_codes, k_cb, v_cb, lens, torch.uint8)
    C = pq_attn_num_chunks(desc)
    if C < 1:
        raise PQError(PQ_ERR_SHAPE_CODE, "pq_attn_partials_fp8cb")
    B, Hq, D = desc.batch, desc.n_q_heads, desc.head_dim
    part_m = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    part_l = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    part_o = torch.empty((B, Hq, C, D), dtype=torch.float32, device=q.device)
    st = load_library().pq_attn_partials_fp8cb(
        ctypes.byref(desc), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_cb), _ptr(v_cb),
        _ptr(lens), _ptr(part_m), _ptr(part_l), _ptr(part_o), _stream(stream))
    _check(st, "pq_attn_partials_fp8cb")
    return part_m, part_l, part_o


def pq_attn_step_workspace_bytes(desc: PQAttnDesc) -> int:
    return int(load_library().pq_attn_step_workspace_bytes(ctypes.byref(desc)))


_num_chunks_memo = {}


def _desc_key(desc: PQAttnDesc):
    shape = (desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.head_dim, desc.n_sub, desc.n_codes,
             desc.max_len)
    fields = shape + (desc.chunk,)
    c = _num_chunks_memo.get(fields)
    if c is None:   # the planner is a pure function of these fields
        if len(_num_chunks_memo) >= 4096:
            _num_chunks_memo.clear()
        c = _num_chunks_memo[fields] = pq_attn_num_chunks(desc)
    return shape + (c,)


def step_workspace(desc: PQAttnDesc, device):
    """A zero-filled workspace for pq_attn_decode_step (None when it needs
    none).  Keep it for later steps with the same descriptor: each call
    leaves it ready.  It is tied to that descriptor (the arrival counters'
    offset depends on the shape), and the step functions here refuse it
    for another."""
    import torch
    n = pq_attn_step_workspace_bytes(desc)
    if n == 0:
        return None
    ws = torch.zeros(n, dtype=torch.uint8, device=device)
    ws._pq_step_key = _desc_key(desc)
    return ws


def _check_step_workspace(desc, workspace, where):
    key = getattr(workspace, "_pq_step_key", None)
    if key is not None and key != _desc_key(desc):
        raise ValueError(f"{where}: this step workspace was made for another descriptor "
                         f"{key}; its arrival counters would sit elsewhere -- use "
                         "step_workspace(desc) for this one")


def pq_attn_decode_step(q, k_new, v_new, k_codes, v_codes, k_cb, v_cb, lens, out=None, *,
                        desc=None, chunk=0, scale=None, workspace=None, stream=None,
                        events=None):
    """One decode step with the new token appended (C entry point
    pq_attn_decode_step): encodes k_new/v_new [B, Hkv, D] into slot
    lens[b] - 1 of the code caches (written in place) and returns ``out``
    (fp32 [B, Hq, D]).  ``workspace`` must come from step_workspace() (or be
    zero-filled) when the shape needs one; it is created here if omitted.
    ``events=(start, stop)`` goes through pq_attn_decode_step_timed."""
    import torch
    if desc is None:
        desc = attn_desc(q, k_codes, k_cb, chunk=chunk, scale=scale)
    _check_attn_inputs(desc, q, k_codes, v_codes, k_cb, v_cb, lens)
    shape_new = (desc.batch, desc.n_kv_heads, desc.head_dim)
    _need(k_new, "k_new", torch.float16, shape_new)
    _need(v_new, "v_new", torch.float16, shape_new)
    if out is None:
        out = torch.empty((desc.batch, desc.n_q_heads, desc.head_dim), dtype=torch.float32,
                          device=q.device)
    _need(out, "out", torch.float32, (desc.batch, desc.n_q_heads, desc.head_dim))
    if workspace is None:
        workspace = step_workspace(desc, q.device)
    _check_step_workspace(desc, workspace, "pq_attn_decode_step")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    args = (ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_codes), _ptr(v_codes),
            _ptr(k_cb), _ptr(v_cb), _ptr(lens), _ptr(out), _ptr(workspace), nbytes,
            _stream(stream))
    if events is None:
        st = lib.pq_attn_decode_step(*args)
    else:
        st = lib.pq_attn_decode_step_timed(*args, events[0], events[1])
    _check(st, "pq_attn_decode_step")
    return out


def pq_attn_decode_step_noalloc(q, k_new, v_new, k_codes, v_codes, k_cb, v_cb, lens, out, *,
                                desc=None, chunk=0, scale=None, stream=None):
    """pq_attn_decode_step without a workspace (C entry point
    pq_attn_decode_step_noalloc): the library's own device scratch holds the
    chunk records and counters.  ``out`` (fp32 [B, Hq, D]) is required, so
    nothing is allocated on this path either.  Calls that overlap in time on
    one GPU race (they share the scratch)."""
    import torch
    if desc is None:
        desc = attn_desc(q, k_codes, k_cb, chunk=chunk, scale=scale)
    _check_attn_inputs(desc, q, k_codes, v_codes, k_cb, v_cb, lens)
    shape_new = (desc.batch, desc.n_kv_heads, desc.head_dim)
    _need(k_new, "k_new", torch.float16, shape_new)
    _need(v_new, "v_new", torch.float16, shape_new)
    _need(out, "out", torch.float32, (desc.batch, desc.n_q_heads, desc.head_dim))
    st = load_library().pq_attn_decode_step_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_codes), _ptr(v_codes),
        _ptr(k_cb), _ptr(v_cb), _ptr(lens), _ptr(out), _stream(stream))
    _check(st, "pq_attn_decode_step_noalloc")
    return out


def paged_desc(q, k_pool, k_cb, block_table, page_tokens, *, chunk=0, scale=None):
    """(attention descriptor, page table) from tensor shapes: q [B,Hq,D],
    k_pool [Hkv, n_pages*P, M], block_table int32 [B, max_pages]."""
    B, Hq, D = q.shape
    Hkv, slots, M = k_pool.shape
    P = int(page_tokens)
    max_pages = block_table.shape[1]
    desc = PQAttnDesc(B, Hq, Hkv, D, M, k_cb.shape[2], max_pages * P, int(chunk),
                      float(scale if scale is not None else 1.0 / math.sqrt(D)))
    table = PQPageTable(block_table.data_ptr(), P, max_pages, slots // P if P > 0 else 0)
    return desc, table


def _check_paged_inputs(desc, table, q, k_pool, v_pool, k_cb, v_cb, block_table, lens):
    import torch
    B, Hq, Hkv, D = desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.head_dim
    M, K = desc.n_sub, desc.n_codes
    P, n_pages = table.page_tokens, table.n_pages
    _need(q, "q", torch.float16, (B, Hq, D))
    _need(k_pool, "k_pool", torch.uint8, (Hkv, n_pages * P, M))
    _need(v_pool, "v_pool", torch.uint8, (Hkv, n_pages * P, M))
    _need(k_cb, "k_cb", torch.float16, (Hkv, M, K, D // M))
    _need(v_cb, "v_cb", torch.float16, (Hkv, M, K, D // M))
    _need(block_table, "block_table", torch.int32, (B, table.max_pages))
    _need(lens, "lens", torch.int32, (B,))
    if table.block_table != block_table.data_ptr():
        raise ValueError("the page table does not point at block_table")


def pq_attn_decode_paged(q, k_pool, v_pool, k_cb, v_cb, block_table, lens, out=None, *,
                         page_tokens, chunk=0, scale=None, workspace=None, stream=None):
    """Decode over a paged cache (C entry point pq_attn_decode_paged): pools
    uint8 [Hkv, n_pages * P, M] (page p = slots p*P .. p*P + P - 1),
    block_table int32 [B, max_pages].  Returns ``out`` fp32 [B, Hq, D]."""
    import torch
    desc, table = paged_desc(q, k_pool, k_cb, block_table, page_tokens, chunk=chunk, scale=scale)
    _check_paged_inputs(desc, table, q, k_pool, v_pool, k_cb, v_cb, block_table, lens)
    if out is None:
        out = torch.empty((desc.batch, desc.n_q_heads, desc.head_dim), dtype=torch.float32,
                          device=q.device)
    _need(out, "out", torch.float32, (desc.batch, desc.n_q_heads, desc.head_dim))
    ws_bytes = pq_attn_workspace_bytes(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().pq_attn_decode_paged(
        ctypes.byref(desc), ctypes.byref(table), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_cb),
        _ptr(v_cb), _ptr(lens), _ptr(out), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "pq_attn_decode_paged")
    return out


def pq_attn_partials_paged(q, k_pool, v_pool, k_cb, v_cb, block_table, lens, *, page_tokens,
                           chunk=0, scale=None, stream=None):
    """Chunk records over a paged cache (C entry point pq_attn_partials_paged).
    Returns (part_m [B,Hq,C], part_l [B,Hq,C], part_o [B,Hq,C,D]), fp32."""
    import torch
    desc, table = paged_desc(q, k_pool, k_cb, block_table, page_tokens, chunk=chunk, scale=scale)
    _check_paged_inputs(desc, table, q, k_pool, v_pool, k_cb, v_cb, block_table, lens)
    C = pq_attn_num_chunks(desc)
    if C < 1:
        _check(PQ_ERR_SHAPE_CODE, "pq_attn_partials_paged")
    B, Hq, D = desc.batch, desc.n_q_heads, desc.head_dim
    part_m = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    part_l = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    part_o = torch.empty((B, Hq, C, D), dtype=torch.float32, device=q.device)
    st = load_library().pq_attn_partials_paged(
        ctypes.byref(desc), ctypes.byref(table), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_cb),
        _ptr(v_cb), _ptr(lens), _ptr(part_m), _ptr(part_l), _ptr(part_o), _stream(stream))
    _check(st, "pq_attn_partials_paged")
    return part_m, part_l, part_o


def pq_attn_decode_step_paged(q, k_new, v_new, k_pool, v_pool, k_cb, v_cb, block_table, lens,
                              out=None, *, page_tokens, chunk=0, scale=None, workspace=None,
                              stream=None, events=None):
    """Decode step over a paged cache (C entry point pq_attn_decode_step_paged):
    encodes k_new/v_new [B, Hkv, D] into the slot of token lens[b] - 1 (its page
    must be in block_table) and returns ``out`` (fp32 [B, Hq, D]).  Workspace
    as for pq_attn_decode_step (from step_workspace(desc), zero-filled);
    ``events=(start, stop)`` goes through pq_attn_decode_step_paged_timed."""
    import torch
    desc, table = paged_desc(q, k_pool, k_cb, block_table, page_tokens, chunk=chunk, scale=scale)
    _check_paged_inputs(desc, table, q, k_pool, v_pool, k_cb, v_cb, block_table, lens)
    shape_new = (desc.batch, desc.n_kv_heads, desc.head_dim)
    _need(k_new, "k_new", torch.float16, shape_new)
    _need(v_new, "v_new", torch.float16, shape_new)
    if out is None:
        out = torch.empty((desc.batch, desc.n_q_heads, desc.head_dim), dtype=torch.float32,
                          device=q.device)
    _need(out, "out", torch.float32, (desc.batch, desc.n_q_heads, desc.head_dim))
    if workspace is None:
        workspace = step_workspace(desc, q.device)
    _check_step_workspace(desc, workspace, "pq_attn_decode_step_paged")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    args = (ctypes.byref(desc), ctypes.byref(table), _ptr(q), _ptr(k_new), _ptr(v_new),
            _ptr(k_pool), _ptr(v_pool), _ptr(k_cb), _ptr(v_cb), _ptr(lens), _ptr(out),
            _ptr(workspace), nbytes, _stream(stream))
    if events is None:
        st = lib.pq_attn_decode_step_paged(*args)
    else:
        st = lib.pq_attn_decode_step_paged_timed(*args, events[0], events[1])
    _check(st, "pq_attn_decode_step_paged")
    return out


def pq_attn_reduce(part_m, part_l, part_o, out=None, *, stream=None, polyexp=False):
    """Merge chunk statistics (C entry point pq_attn_reduce, or
    pq_attn_reduce_polyexp with ``polyexp``).  part_m and part_l [..., C],
    part_o [..., C, D]; returns out [..., D] fp32."""
    import torch
    C, D = part_o.shape[-2], part_o.shape[-1]
    lead = tuple(part_o.shape[:-2])
    rows = 1
    for s in lead:
        rows *= s
    _need(part_m, "part_m", torch.float32, (*lead, C))
    _need(part_l, "part_l", torch.float32, (*lead, C))
    _need(part_o, "part_o", torch.float32)
    if out is None:
        out = torch.empty((*lead, D), dtype=torch.float32, device=part_o.device)
    _need(out, "out", torch.float32, (*lead, D))
    fn = load_library().pq_attn_reduce_polyexp if polyexp else load_library().pq_attn_reduce
    st = fn(rows, C, D, _ptr(part_m), _ptr(part_l), _ptr(part_o), _ptr(out), _stream(stream))
    _check(st, "pq_attn_reduce_polyexp" if polyexp else "pq_attn_reduce")
    return out


def pq_encode(x, codebook, codes, *, slots=None, desc=None, stream=None):
    """Nearest-codeword encode (C entry point pq_encode).

    Default layout (desc None): x fp16 [N, H, D] and codes uint8 [N, H, M],
    both contiguous.  Pass ``desc`` (a PQEncodeDesc) for strided layouts, e.g.
    writing straight into a [B, Hkv, Lmax, M] code cache through ``slots``."""
    import torch
    _need(x, "x", torch.float16, None)
    _need(codebook, "codebook", torch.float16, None)
    _need(codes, "codes", torch.uint8, None)
    if slots is not None:
        _need(slots, "slots", torch.int64, None)
    if desc is None:
        N, H, D = x.shape
        _, M, K, _ = codebook.shape
        _need(codes, "codes", torch.uint8, (N, H, M))
        desc = PQEncodeDesc(N, H, D, M, K, H * D, D, H * M, M, codes.numel())
    st = load_library().pq_encode(ctypes.byref(desc), _ptr(x), _ptr(codebook), _ptr(slots),
                                  _ptr(codes), _stream(stream))
    _check(st, "pq_encode")
    return codes


def pq_encode_fp8cb(x, codebook, codes, *, slots=None, desc=None, stream=None):
    """pq_encode against an FP8 E4M3 codebook (C entry point
    pq_encode_fp8cb): codebook is a uint8 [H, M, K, D/M] tensor of E4M3
    bytes; everything else as for pq_encode."""
    import torch
    _need(x, "x", torch.float16, None)
    _need(codebook, "codebook", torch.uint8, None)
    _need(codes, "codes", torch.uint8, None)
    if slots is not None:
        _need(slots, "slots", torch.int64, None)
    if desc is None:
        N, H, D = x.shape
        _, M, K, _ = codebook.shape
        _need(codes, "codes", torch.uint8, (N, H, M))
        desc = PQEncodeDesc(N, H, D, M, K, H * D, D, H * M, M, codes.numel())
    st = load_library().pq_encode_fp8cb(ctypes.byref(desc), _ptr(x), _ptr(codebook), _ptr(slots),
                                        _ptr(codes), _stream(stream))
    _check(st, "pq_encode_fp8cb")
    return codes


def pq_encode_many(xs, codebooks, codes, *, desc, slots=None, stream=None):
    """Encode several tensors of one shape in one launch (C entry point
    pq_encode_many), e.g. a new token's K and V: plane i gets what
    pq_encode(xs[i], codebooks[i], codes[i], ...) gives."""
    import torch
    n = len(xs)
    if not (len(codebooks) == len(codes) == n):
        raise ValueError("xs, codebooks and codes must have the same length")
    for t in xs:
        _need(t, "x", torch.float16, None)
    for t in codebooks:
        _need(t, "codebook", torch.float16, None)
    for t in codes:
        _need(t, "codes", torch.uint8, None)
    if slots is not None:
        _need(slots, "slots", torch.int64, None)
    arr = ctypes.c_void_p * max(n, 1)
    st = load_library().pq_encode_many(
        ctypes.byref(desc), n, arr(*[_ptr(t) for t in xs]), arr(*[_ptr(t) for t in codebooks]),
        _ptr(slots), arr(*[_ptr(t) for t in codes]), _stream(stream))
    _check(st, "pq_encode_many")
    return codes


def _sample_desc(x, codebook, codes):
    N, H, D = x.shape
    _, M, K, _ = codebook.shape
    return PQEncodeDesc(N, H, D, M, K, H * D, D, H * M, M, codes.numel())


def pq_codebook_update(x, codes, codebook, counts=None, *, desc=None, stream=None):
    """Update step of a Lloyd iteration (C entry point pq_codebook_update):
    every codeword named by some code moves to the mean of its segments.
    Default layout (desc None): x fp16 [N, H, D], codes uint8 [N, H, M],
    codebook fp16 [H, M, K, D/M] (updated in place), counts uint32-compatible
    int32 [H, M, K] or None.  Returns the codebook."""
    import torch
    _need(x, "x", torch.float16, None)
    _need(codebook, "codebook", torch.float16, None)
    _need(codes, "codes", torch.uint8, None)
    if counts is not None:
        _need(counts, "counts", torch.int32, tuple(codebook.shape[:3]))
    if desc is None:
        N, H, _ = x.shape
        _need(codes, "codes", torch.uint8, (N, H, codebook.shape[1]))
        desc = _sample_desc(x, codebook, codes)
    st = load_library().pq_codebook_update(ctypes.byref(desc), _ptr(x), _ptr(codes),
                                           _ptr(codebook), _ptr(counts), _stream(stream))
    _check(st, "pq_codebook_update")
    return codebook


def pq_kmeans(x, codebook, n_iter, codes=None, *, desc=None, stream=None):
    """n_iter Lloyd iterations from ``codebook`` (updated in place) on the
    sample x (C entry point pq_kmeans).  Returns (codebook, codes), codes
    being x's codes under the learned codebook."""
    import torch
    _need(x, "x", torch.float16, None)
    _need(codebook, "codebook", torch.float16, None)
    if codes is None:
        codes = torch.empty((x.shape[0], x.shape[1], codebook.shape[1]), dtype=torch.uint8,
                            device=x.device)
    _need(codes, "codes", torch.uint8, None)
    if desc is None:
        N, H, _ = x.shape
        _need(codes, "codes", torch.uint8, (N, H, codebook.shape[1]))
        desc = _sample_desc(x, codebook, codes)
    st = load_library().pq_kmeans(ctypes.byref(desc), _ptr(x), _ptr(codebook), int(n_iter),
                                  _ptr(codes), _stream(stream))
    _check(st, "pq_kmeans")
    return codebook, codes


def pq_kmeans_many(xs, codebooks, n_iter, codes=None, *, desc=None, stream=None):
    """pq_kmeans for 1 or 2 samples of one shape in one call (C entry point
    pq_kmeans_many), e.g. a layer's K and V samples.  Returns (codebooks,
    codes) lists."""
    import torch
    n = len(xs)
    if len(codebooks) != n:
        raise ValueError("xs and codebooks must have the same length")
    for t in xs:
        _need(t, "x", torch.float16, None)
    for t in codebooks:
        _need(t, "codebook", torch.float16, None)
    if codes is None:
        codes = [torch.empty((x.shape[0], x.shape[1], cb.shape[1]), dtype=torch.uint8,
                             device=x.device) for x, cb in zip(xs, codebooks)]
    for t in codes:
        _need(t, "codes", torch.uint8, None)
    if desc is None:
        desc = _sample_desc(xs[0], codebooks[0], codes[0])
    arr = ctypes.c_void_p * max(n, 1)
    st = load_library().pq_kmeans_many(
        ctypes.byref(desc), n, arr(*[_ptr(t) for t in xs]), arr(*[_ptr(t) for t in codebooks]),
        int(n_iter), arr(*[_ptr(t) for t in codes]), _stream(stream))
    _check(st, "pq_kmeans_many")
    return codebooks, codes


def cache_encode_desc(n_vec, batch, n_kv_heads, max_len, head_dim=128, n_sub=4, n_codes=256,
                      x_stride_vec=None):
    """Descriptor that writes the codes of x [N, Hkv, D] (rows x_stride_vec
    apart) into a [B, Hkv, Lmax, M] code cache at token slots
    s = b*Hkv*Lmax + t (pass them as the slots tensor)."""
    if x_stride_vec is None:
        x_stride_vec = n_kv_heads * head_dim
    return PQEncodeDesc(n_vec, n_kv_heads, head_dim, n_sub, n_codes, x_stride_vec, head_dim,
                        n_sub, max_len * n_sub, batch * n_kv_heads * max_len * n_sub)


def paged_encode_desc(n_vec, n_kv_heads, n_pages, page_tokens, head_dim=128, n_sub=4,
                      n_codes=256, x_stride_vec=None):
    """Descriptor that writes the codes of x [N, Hkv, D] into paged pools
    [Hkv, n_pages * P, M] at pool slots s = page * P + offset (pass them as the
    slots tensor; the same slot in every KV head's pool)."""
    if x_stride_vec is None:
        x_stride_vec = n_kv_heads * head_dim
    pool_head = n_pages * page_tokens * n_sub
    return PQEncodeDesc(n_vec, n_kv_heads, head_dim, n_sub, n_codes, x_stride_vec, head_dim,
                        n_sub, pool_head, n_kv_heads * pool_head)
