"""ctypes binding for libkvt.so -- argument marshalling only, same names as include/kvt.h.

Every pointer argument accepts an int address, a torch tensor (its data_ptr()), a numpy array
(its data address) or None (NULL).  Stream arguments accept a torch stream, a raw handle (int)
or None, which means torch's current stream on the current device.  Each call returns nothing
and raises ``KvtError`` (carrying the status code and the library's message) on failure.

There is no fallback: if libkvt.so is missing or does not load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint, c_uint64, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvt.so")

OK, EINVAL, ERANGE, EALIGN, EOVERLAP, ENOMEM, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4, -5, -6, -7
H2D, D2H = 0, 1
COPY_AUTO, COPY_KERNEL, COPY_SDMA, COPY_RUNTIME = 0, 1, 2, 3
F16, BF16, Q8_0 = 1, 2, 3
HOST_COHERENT, HOST_NONCOHERENT, HOST_WRITECOMBINED = 0, 1, 2
PREFILL_IN_PLACE, PREFILL_STAGED, PREFILL_PIPELINED = 0, 1, 2
OP_NONE_NEEDED, OP_INDEX_TOPK, OP_ATTN_DECODE, OP_SPARSE_ROWS, OP_PREFILL_STATE = 0, 1, 2, 3, 4

_P = c_void_p
_SIGNATURES = {
    "kvt_abi_version": (c_int, []),
    "kvt_last_error": (ctypes.c_char_p, []),
    "kvt_host_alloc": (c_int, [c_size_t, c_uint, ctypes.POINTER(c_void_p), ctypes.POINTER(c_void_p)]),
    "kvt_host_free": (c_int, [_P]),
    "kvt_sub_block_ptrs": (c_int, [c_uint64, c_uint64, c_uint64, _P, c_int64, c_int32, c_int32,
                                   _P, c_int64]),
    "kvt_chunks_consumed": (c_int64, [c_int64, c_int32, c_int32]),
    "kvt_swap_blocks": (c_int, [_P, _P, _P, c_int64, c_int32, c_int32, _P]),
    "kvt_set_copy_threshold": (c_uint64, [c_int32, c_uint64]),
    "kvt_index_topk_ws_bytes": (c_size_t, [c_int64, c_int32, c_int32]),
    "kvt_index_topk": (c_int, [_P, c_int64, c_int32, _P, c_int32, c_int32, _P, _P, _P, c_size_t,
                               _P]),
    "kvt_select_positions": (c_int, [_P, c_int32, c_int32, c_int32, c_int64, c_int32, _P, _P]),
    "kvt_gather_blocks": (c_int, [_P, _P, c_int64, c_int32, c_int32, c_int32, c_int64, c_int64,
                                  c_int64, _P, c_int32, _P, c_int32, _P, _P, _P]),
    "kvt_stage_tail": (c_int, [_P, c_int64, c_int64, c_int64, _P, c_int32, _P]),
    "kvt_attn_decode_ws_bytes": (c_size_t, [c_int32, c_int32, c_int64]),
    "kvt_attn_decode": (c_int, [_P, c_int32, c_int32, c_int32, c_int32, _P, _P, c_int64, _P,
                                c_float, _P, _P, c_size_t, _P]),
    "kvt_gather_attn_decode": (c_int, [_P, c_int32, c_int32, c_int32, c_int32, _P, _P, c_int64,
                                       c_int64, c_int64, c_int64, _P, c_int32, _P, c_int32, _P, _P,
                                       c_float, _P, _P, c_size_t, _P]),
    "kvt_gather_attn_decode_noalloc_max_bytes": (c_size_t, []),
    "kvt_gather_attn_decode_noalloc": (c_int, [_P, c_int32, c_int32, c_int32, c_int32, _P, _P,
                                               c_int64, c_int64, c_int64, c_int64, _P, c_int32,
                                               _P, c_int32, _P, _P, c_float, _P, _P]),
    "kvt_pool_rebuild": (c_int, [_P, _P, c_int32, c_int32, c_int32, _P, _P, c_int32, c_int32,
                                 c_int32, c_int64, _P]),
    "kvt_attn_prefill": (c_int, [_P, c_int64, c_int64, c_int32, c_int32, c_int32, _P, _P, c_int64,
                                 _P, _P, c_int64, c_int32, c_int32, c_float, _P, _P]),
    "kvt_attn_prefill_state_bytes": (c_size_t, [c_int64, c_int32, c_int32]),
    "kvt_attn_prefill_range": (c_int, [_P, c_int64, c_int64, c_int32, c_int32, c_int32, _P, _P,
                                       c_int64, _P, _P, c_int64, c_int32, c_int32, c_float,
                                       c_int64, c_int64, _P, c_size_t, _P, _P]),
    "kvt_attn_prefill_pipelined": (c_int, [_P, c_int64, c_int64, c_int32, c_int32, c_int32, _P,
                                           _P, c_int64, _P, _P, c_int64, c_int32, c_int32,
                                           c_float, _P, _P, c_int64, _P, c_size_t, _P, _P, _P]),
    "kvt_attn_prefill_chain": (c_int, [_P, c_int64, c_int64, c_int32, c_int32, c_int32, _P, _P,
                                       c_int64, _P, _P, c_int64, c_int32, c_int32, c_float, _P,
                                       _P, c_int64, c_int64, _P, _P, c_int64, _P, _P, c_int64,
                                       _P, c_size_t, _P, _P, _P]),
    "kvt_worker_create": (c_int, [c_int32, c_int32, ctypes.POINTER(c_void_p)]),
    "kvt_worker_reserve": (c_int, [_P, c_int32, c_int64]),
    "kvt_worker_submit": (c_int, [_P, c_int64, _P, _P, _P, c_int64, _P]),
    "kvt_worker_get_finished": (c_int, [_P, _P, _P, _P, c_int32, ctypes.POINTER(c_int32)]),
    "kvt_worker_wait": (c_int, [_P, _P, c_int32]),
    "kvt_worker_pending": (c_int, [_P]),
    "kvt_worker_destroy": (c_int, [_P]),
    "kvt_sparse_attend_rows_ws_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "kvt_sparse_attend_rows": (c_int, [_P, c_int32, c_int32, c_int32, c_int32, c_int32, _P, _P,
                                       c_int64, c_int64, c_int64, _P, c_int32, c_int64, c_int32,
                                       _P, c_int32, c_float, _P, _P, c_size_t, _P]),
    "kvt_staging_worthwhile": (c_int, [c_int64, c_int64, c_int64, c_int64]),
    "kvt_stage_pages": (c_int, [_P, _P, c_int64, _P, c_int32, c_int64, _P, _P, _P]),
    "kvt_sparse_attend_rows_auto": (c_int, [_P, c_int32, c_int32, c_int32, c_int32, c_int32, _P,
                                            _P, c_int64, c_int64, c_int64, _P, c_int32, c_int32,
                                            _P, c_int32, c_float, _P, _P, c_size_t, _P, _P,
                                            c_size_t, ctypes.POINTER(c_int32), _P]),
    "kvt_workspace_bytes": (c_size_t, [c_int32, _P, c_int32]),
    "kvt_attn_prefill_splitk_ws_bytes": (c_size_t, [c_int64, c_int32, c_int32, c_int64]),
    "kvt_attn_prefill_splitk": (c_int, [_P, c_int64, c_int64, c_int32, c_int32, c_int32, _P, _P,
                                        c_int64, _P, _P, c_int64, c_int32, c_int32, c_float, _P,
                                        c_size_t, _P, _P]),
    "kvt_copy_engines": (c_int, [c_int32]),
    "kvt_attn_prefill_plan": (c_int, [c_int64, c_int64, c_int32, c_int32, c_int64, c_int64,
                                      c_int32, c_int32, c_int64, c_int32]),
    "kvt_attn_prefill_auto_ws_bytes": (c_size_t, [c_int64, c_int32, c_int32, c_int64]),
    "kvt_attn_prefill_conv_bytes": (c_size_t, [c_int64, c_int32, c_int64, c_int32]),
    "kvt_attn_prefill_auto": (c_int, [_P, c_int64, c_int64, c_int32, c_int32, c_int32, _P, _P,
                                      c_int64, _P, _P, c_int64, c_int32, c_int32, c_float, _P,
                                      _P, c_int64, _P, c_size_t, _P, c_size_t, _P,
                                      ctypes.POINTER(c_int32), _P, _P]),
    "kvt_paged_write": (c_int, [_P, _P, _P, c_int32, c_int32, c_int32, _P, _P, c_int32, c_int32,
                                c_int64, _P]),
    "kvt_copy_page": (c_int, [_P, _P, _P, c_int32, c_int64, c_int64, c_int32, c_int32, _P, _P,
                              c_int64, c_int32, _P]),
}
EXPORTED = tuple(_SIGNATURES)

_lib = None


class KvtError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def load():
    """Load libkvt.so (once).  Raises if it is missing: there is no other implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m hbm_kv_cache_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x).__name__}")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn, rc):
    if rc != OK:
        msg = load().kvt_last_error()
        raise KvtError(fn, rc, msg.decode() if msg else "")


def kvt_abi_version() -> int:
    return load().kvt_abi_version()


def kvt_last_error() -> str:
    m = load().kvt_last_error()
    return m.decode() if m else ""


def kvt_host_alloc(nbytes: int, flags: int = HOST_COHERENT):
    """Returns (host_address, device_address) of a zeroed pinned, device-mapped slab."""
    h, d = c_void_p(), c_void_p()
    _check("kvt_host_alloc", load().kvt_host_alloc(int(nbytes), int(flags), ctypes.byref(h),
                                                   ctypes.byref(d)))
    return h.value, d.value


def kvt_host_free(host_ptr: int) -> None:
    _check("kvt_host_free", load().kvt_host_free(host_ptr))


def kvt_sub_block_ptrs(base, row_stride, page_bytes, block_ids, n_ids, bpc, skip, out, n_out):
    _check("kvt_sub_block_ptrs", load().kvt_sub_block_ptrs(
        int(base), int(row_stride), int(page_bytes), _ptr(block_ids), int(n_ids), int(bpc),
        int(skip), _ptr(out), int(n_out)))


def kvt_chunks_consumed(n, skip, bpc) -> int:
    return int(load().kvt_chunks_consumed(int(n), int(skip), int(bpc)))


def kvt_swap_blocks(src, dst, sizes, n, direction, mode=COPY_AUTO, stream=None):
    _check("kvt_swap_blocks", load().kvt_swap_blocks(_ptr(src), _ptr(dst), _ptr(sizes), int(n),
                                                     int(direction), int(mode), _stream(stream)))


def kvt_set_copy_threshold(direction, nbytes) -> int:
    return int(load().kvt_set_copy_threshold(int(direction), int(nbytes)))


def kvt_index_topk_ws_bytes(n_blocks, n_sel, k) -> int:
    return int(load().kvt_index_topk_ws_bytes(int(n_blocks), int(n_sel), int(k)))


def kvt_index_topk(pooled, n_blocks, dim, q_idx, n_sel, k, ids, scores, ws, ws_bytes,
                   stream=None):
    _check("kvt_index_topk", load().kvt_index_topk(
        _ptr(pooled), int(n_blocks), int(dim), _ptr(q_idx), int(n_sel), int(k), _ptr(ids),
        _ptr(scores), _ptr(ws), int(ws_bytes), _stream(stream)))


def kvt_select_positions(ids, n_sel, k, cr, n_tok, k_pad, positions, stream=None):
    _check("kvt_select_positions", load().kvt_select_positions(
        _ptr(ids), int(n_sel), int(k), int(cr), int(n_tok), int(k_pad), _ptr(positions),
        _stream(stream)))


def kvt_gather_blocks(k_plane, v_plane, n_blocks, kvh, hd, elem_bytes, block_stride,
                      head_stride, token_stride, block_table, bt, ids, k, k_out, v_out,
                      stream=None):
    _check("kvt_gather_blocks", load().kvt_gather_blocks(
        _ptr(k_plane), _ptr(v_plane), int(n_blocks), int(kvh), int(hd), int(elem_bytes),
        int(block_stride), int(head_stride), int(token_stride), _ptr(block_table), int(bt),
        _ptr(ids), int(k), _ptr(k_out), _ptr(v_out), _stream(stream)))


def kvt_stage_tail(plane, row_bytes, row_begin, row_end, staging, mode=COPY_AUTO, stream=None):
    _check("kvt_stage_tail", load().kvt_stage_tail(_ptr(plane), int(row_bytes), int(row_begin),
                                                   int(row_end), _ptr(staging), int(mode),
                                                   _stream(stream)))


def kvt_attn_decode_ws_bytes(n_qh, hd, n_kv) -> int:
    return int(load().kvt_attn_decode_ws_bytes(int(n_qh), int(hd), int(n_kv)))


def kvt_attn_decode(q, n_qh, kvh, hd, dtype, k, v, n_kv, n_valid, scale, out, ws, ws_bytes,
                    stream=None):
    _check("kvt_attn_decode", load().kvt_attn_decode(
        _ptr(q), int(n_qh), int(kvh), int(hd), int(dtype), _ptr(k), _ptr(v), int(n_kv),
        _ptr(n_valid), float(scale), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def kvt_gather_attn_decode(q, n_qh, kvh, hd, dtype, k_plane, v_plane, n_blocks, block_stride,
                           head_stride, token_stride, block_table, bt, ids, k, k_out, v_out, scale,
                           out, ws, ws_bytes, stream=None):
    _check("kvt_gather_attn_decode", load().kvt_gather_attn_decode(
        _ptr(q), int(n_qh), int(kvh), int(hd), int(dtype), _ptr(k_plane), _ptr(v_plane),
        int(n_blocks), int(block_stride), int(head_stride), int(token_stride), _ptr(block_table),
        int(bt), _ptr(ids), int(k), _ptr(k_out), _ptr(v_out), float(scale), _ptr(out), _ptr(ws),
        int(ws_bytes), _stream(stream)))


def kvt_gather_attn_decode_noalloc_max_bytes():
    return int(load().kvt_gather_attn_decode_noalloc_max_bytes())


def kvt_gather_attn_decode_noalloc(q, n_qh, kvh, hd, dtype, k_plane, v_plane, n_blocks,
                                   block_stride, head_stride, token_stride, block_table, bt, ids,
                                   k, k_out, v_out, scale, out, stream=None):
    _check("kvt_gather_attn_decode_noalloc", load().kvt_gather_attn_decode_noalloc(
        _ptr(q), int(n_qh), int(kvh), int(hd), int(dtype), _ptr(k_plane), _ptr(v_plane),
        int(n_blocks), int(block_stride), int(head_stride), int(token_stride), _ptr(block_table),
        int(bt), _ptr(ids), int(k), _ptr(k_out), _ptr(v_out), float(scale), _ptr(out),
        _stream(stream)))


def kvt_attn_prefill(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, k_tail, v_tail, n_kv,
                     kv_format, causal, scale, out, stream=None):
    _check("kvt_attn_prefill", load().kvt_attn_prefill(
        _ptr(q), int(n_q), int(q_pos0), int(n_qh), int(kvh), int(hd), _ptr(k_head), _ptr(v_head),
        int(n_head), _ptr(k_tail), _ptr(v_tail), int(n_kv), int(kv_format), int(bool(causal)),
        float(scale), _ptr(out), _stream(stream)))


class HostBuffer:
    """Owner of one pinned, device-mapped host slab from kvt_host_alloc.

    ``.host`` / ``.dev`` are the two addresses; ``.numpy(dtype, shape)`` views the host side;
    ``.free()`` (or garbage collection) releases it -- drop every view first, and make sure no
    queued GPU work still reads it."""

    def __init__(self, nbytes: int, flags: int = HOST_COHERENT):
        self.nbytes = int(nbytes)
        self.host, self.dev = kvt_host_alloc(self.nbytes, flags)

    def numpy(self, dtype="uint8", shape=None):
        import numpy as np
        dt = np.dtype(dtype)
        buf = (ctypes.c_char * self.nbytes).from_address(self.host)
        a = np.frombuffer(buf, dtype=dt, count=self.nbytes // dt.itemsize)
        return a if shape is None else a.reshape(shape)

    def free(self):
        if self.host:
            kvt_host_free(self.host)
            self.host = self.dev = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def kvt_attn_prefill_state_bytes(n_q, n_qh, kvh) -> int:
    return int(load().kvt_attn_prefill_state_bytes(int(n_q), int(n_qh), int(kvh)))


def kvt_attn_prefill_range(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, k_tail, v_tail,
                           n_kv, kv_format, causal, scale, key_begin, key_end, state,
                           state_bytes, out, stream=None):
    _check("kvt_attn_prefill_range", load().kvt_attn_prefill_range(
        _ptr(q), int(n_q), int(q_pos0), int(n_qh), int(kvh), int(hd), _ptr(k_head), _ptr(v_head),
        int(n_head), _ptr(k_tail), _ptr(v_tail), int(n_kv), int(kv_format), int(bool(causal)),
        float(scale), int(key_begin), int(key_end), _ptr(state), int(state_bytes), _ptr(out),
        _stream(stream)))


def kvt_attn_prefill_pipelined(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, k_host,
                               v_host, n_kv, kv_format, causal, scale, arena_k, arena_v,
                               arena_rows, state, state_bytes, out, stream=None,
                               copy_stream=None):
    """copy_stream: a hipStream_t handle or torch Stream; it must differ from `stream`."""
    _check("kvt_attn_prefill_pipelined", load().kvt_attn_prefill_pipelined(
        _ptr(q), int(n_q), int(q_pos0), int(n_qh), int(kvh), int(hd), _ptr(k_head), _ptr(v_head),
        int(n_head), _ptr(k_host), _ptr(v_host), int(n_kv), int(kv_format), int(bool(causal)),
        float(scale), _ptr(arena_k), _ptr(arena_v), int(arena_rows), _ptr(state),
        int(state_bytes), _ptr(out), _stream(stream), _stream(copy_stream)))


def kvt_attn_prefill_chain(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, k_host,
                           v_host, n_kv, kv_format, causal, scale, arena_k, arena_v, arena_rows,
                           staged_rows, next_k_host, next_v_host, next_rows, next_arena_k,
                           next_arena_v, next_arena_rows, state, state_bytes, out, stream=None,
                           copy_stream=None):
    """kvt_attn_prefill_pipelined in a chain of layers (next-layer prefetch)."""
    _check("kvt_attn_prefill_chain", load().kvt_attn_prefill_chain(
        _ptr(q), int(n_q), int(q_pos0), int(n_qh), int(kvh), int(hd), _ptr(k_head), _ptr(v_head),
        int(n_head), _ptr(k_host), _ptr(v_host), int(n_kv), int(kv_format), int(bool(causal)),
        float(scale), _ptr(arena_k), _ptr(arena_v), int(arena_rows), int(staged_rows),
        _ptr(next_k_host), _ptr(next_v_host), int(next_rows), _ptr(next_arena_k),
        _ptr(next_arena_v), int(next_arena_rows), _ptr(state), int(state_bytes), _ptr(out),
        _stream(stream), _stream(copy_stream)))


def kvt_worker_create(direction, mode=COPY_AUTO) -> int:
    """Returns the worker handle (an int address)."""
    h = c_void_p()
    _check("kvt_worker_create", load().kvt_worker_create(int(direction), int(mode),
                                                         ctypes.byref(h)))
    return h.value


def kvt_worker_reserve(w, jobs, entries) -> None:
    _check("kvt_worker_reserve", load().kvt_worker_reserve(w, int(jobs), int(entries)))


def kvt_worker_submit(w, job_id, src, dst, sizes, n, compute_stream=None) -> None:
    """src/dst/sizes: u64 tables in host memory (numpy arrays or addresses); copied at submit."""
    _check("kvt_worker_submit", load().kvt_worker_submit(
        w, int(job_id), _ptr(src), _ptr(dst), _ptr(sizes), int(n), _stream(compute_stream)))


def kvt_worker_get_finished(w, max_jobs=256):
    """Returns [(job_id, bytes, seconds), ...] for finished jobs, oldest first."""
    ids = (c_int64 * max(1, int(max_jobs)))()
    nb = (c_uint64 * max(1, int(max_jobs)))()
    secs = (c_double * max(1, int(max_jobs)))()
    n = c_int32()
    _check("kvt_worker_get_finished", load().kvt_worker_get_finished(
        w, ids, nb, secs, int(max_jobs), ctypes.byref(n)))
    return [(ids[i], nb[i], secs[i]) for i in range(n.value)]


def kvt_worker_wait(w, job_ids) -> None:
    """job_ids: one id or an iterable of ids."""
    ids = [int(j) for j in job_ids] if hasattr(job_ids, "__iter__") else [int(job_ids)]
    arr = (c_int64 * max(1, len(ids)))(*ids)
    _check("kvt_worker_wait", load().kvt_worker_wait(w, arr, len(ids)))


def kvt_worker_pending(w) -> int:
    rc = load().kvt_worker_pending(w)
    if rc < 0:
        _check("kvt_worker_pending", rc)
    return rc


def kvt_worker_destroy(w) -> None:
    _check("kvt_worker_destroy", load().kvt_worker_destroy(w))


def _plane_arrays(srcs, dsts, row_bytes):
    n = len(srcs)
    if len(dsts) != n or len(row_bytes) != n:
        raise ValueError("plane lists differ in length")
    a = (c_void_p * max(1, n))(*[_ptr(x) for x in srcs])
    b = (c_void_p * max(1, n))(*[_ptr(x) for x in dsts])
    c = (c_int64 * max(1, n))(*[int(x) for x in row_bytes])
    return a, b, c, n


def kvt_paged_write(srcs, dsts, row_bytes, bsz, seq, cache_seqlens, block_table, pages_per_seq,
                    page_size, n_pages, stream=None):
    """srcs / dsts / row_bytes: per-plane lists (K, V, raw keys ...)."""
    a, b, c, n = _plane_arrays(srcs, dsts, row_bytes)
    _check("kvt_paged_write", load().kvt_paged_write(
        a, b, c, n, int(bsz), int(seq), _ptr(cache_seqlens), _ptr(block_table),
        int(pages_per_seq), int(page_size), int(n_pages), _stream(stream)))


def kvt_copy_page(src_hosts, dst_hosts, row_bytes, from_page, to_page, page_size, num_tokens,
                  src_pooled=None, dst_pooled=None, pooled_row_bytes=0, cr=1, stream=None):
    a, b, c, n = _plane_arrays(src_hosts, dst_hosts, row_bytes)
    _check("kvt_copy_page", load().kvt_copy_page(
        a, b, c, n, int(from_page), int(to_page), int(page_size), int(num_tokens),
        _ptr(src_pooled), _ptr(dst_pooled), int(pooled_row_bytes), int(cr), _stream(stream)))


def kvt_sparse_attend_rows_ws_bytes(rows, n_qh, kvh, k_pad) -> int:
    return int(load().kvt_sparse_attend_rows_ws_bytes(int(rows), int(n_qh), int(kvh), int(k_pad)))


def kvt_sparse_attend_rows(q, rows, n_qh, kvh, hd, dtype, k_plane, v_plane, n_rows, row_stride,
                           head_stride, block_table, table_cols, table_row_stride, page_size,
                           positions, k_pad, scale, out, ws, ws_bytes, stream=None):
    _check("kvt_sparse_attend_rows", load().kvt_sparse_attend_rows(
        _ptr(q), int(rows), int(n_qh), int(kvh), int(hd), int(dtype), _ptr(k_plane),
        _ptr(v_plane), int(n_rows), int(row_stride), int(head_stride), _ptr(block_table),
        int(table_cols), int(table_row_stride), int(page_size), _ptr(positions), int(k_pad),
        float(scale), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def kvt_staging_worthwhile(rows, k_pad, pages_used, page_size) -> bool:
    return bool(load().kvt_staging_worthwhile(int(rows), int(k_pad), int(pages_used),
                                              int(page_size)))


def kvt_stage_pages(k_plane, v_plane, page_bytes, block_table, n_used, n_pages, k_out, v_out,
                    stream=None):
    _check("kvt_stage_pages", load().kvt_stage_pages(
        _ptr(k_plane), _ptr(v_plane), int(page_bytes), _ptr(block_table), int(n_used),
        int(n_pages), _ptr(k_out), _ptr(v_out), _stream(stream)))


def kvt_sparse_attend_rows_auto(q, rows, n_qh, kvh, hd, dtype, k_plane, v_plane, n_rows,
                                row_stride, head_stride, block_table, pages_used, page_size,
                                positions, k_pad, scale, out, ws, ws_bytes, staging_k=None,
                                staging_v=None, staging_bytes=0, stream=None) -> bool:
    """Returns True when the pages were staged into HBM first."""
    staged = c_int32(-1)
    _check("kvt_sparse_attend_rows_auto", load().kvt_sparse_attend_rows_auto(
        _ptr(q), int(rows), int(n_qh), int(kvh), int(hd), int(dtype), _ptr(k_plane),
        _ptr(v_plane), int(n_rows), int(row_stride), int(head_stride), _ptr(block_table),
        int(pages_used), int(page_size), _ptr(positions), int(k_pad), float(scale), _ptr(out),
        _ptr(ws), int(ws_bytes), _ptr(staging_k), _ptr(staging_v), int(staging_bytes),
        ctypes.byref(staged), _stream(stream)))
    return bool(staged.value)


def kvt_workspace_bytes(op, dims) -> int:
    arr = (c_int64 * max(1, len(dims)))(*[int(d) for d in dims])
    return int(load().kvt_workspace_bytes(int(op), arr, len(dims)))


def kvt_attn_prefill_splitk_ws_bytes(n_q, n_qh, kvh, n_kv) -> int:
    return int(load().kvt_attn_prefill_splitk_ws_bytes(int(n_q), int(n_qh), int(kvh), int(n_kv)))


def kvt_attn_prefill_splitk(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, k_tail,
                            v_tail, n_kv, kv_format, causal, scale, ws, ws_bytes, out,
                            stream=None):
    _check("kvt_attn_prefill_splitk", load().kvt_attn_prefill_splitk(
        _ptr(q), int(n_q), int(q_pos0), int(n_qh), int(kvh), int(hd), _ptr(k_head), _ptr(v_head),
        int(n_head), _ptr(k_tail), _ptr(v_tail), int(n_kv), int(kv_format), int(bool(causal)),
        float(scale), _ptr(ws), int(ws_bytes), _ptr(out), _stream(stream)))


def kvt_copy_engines(direction) -> int:
    """DMA engines KVT_COPY_SDMA spreads its copies over on the current device (0: the runtime
    picks per copy)."""
    rc = load().kvt_copy_engines(int(direction))
    if rc < 0:
        _check("kvt_copy_engines", rc)
    return int(rc)


def kvt_attn_prefill_plan(n_q, q_pos0, n_qh, kvh, n_head, n_kv, kv_format, causal, arena_rows,
                          two_streams) -> int:
    """The plan kvt_attn_prefill_auto takes (PREFILL_*); host only."""
    rc = load().kvt_attn_prefill_plan(int(n_q), int(q_pos0), int(n_qh), int(kvh), int(n_head),
                                      int(n_kv), int(kv_format), int(bool(causal)),
                                      int(arena_rows), int(bool(two_streams)))
    if rc < 0:
        _check("kvt_attn_prefill_plan", rc)
    return int(rc)


def kvt_attn_prefill_auto_ws_bytes(n_q, n_qh, kvh, n_kv) -> int:
    return int(load().kvt_attn_prefill_auto_ws_bytes(int(n_q), int(n_qh), int(kvh), int(n_kv)))


def kvt_attn_prefill_conv_bytes(n_head, kvh, arena_rows, kv_format) -> int:
    return int(load().kvt_attn_prefill_conv_bytes(int(n_head), int(kvh), int(arena_rows),
                                                  int(kv_format)))


def kvt_attn_prefill_auto(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, k_host, v_host,
                          n_kv, kv_format, causal, scale, arena_k, arena_v, arena_rows, ws,
                          ws_bytes, out, stream=None, copy_stream=None, conv=None,
                          conv_bytes=0) -> int:
    """Runs the plan kvt_attn_prefill_plan picks and returns it.  copy_stream None: no second
    stream, so no pipelining.  conv: the optional fp16 conversion buffer."""
    plan = c_int32(-1)
    s = _stream(stream)
    cs = s if copy_stream is None else _stream(copy_stream)
    _check("kvt_attn_prefill_auto", load().kvt_attn_prefill_auto(
        _ptr(q), int(n_q), int(q_pos0), int(n_qh), int(kvh), int(hd), _ptr(k_head), _ptr(v_head),
        int(n_head), _ptr(k_host), _ptr(v_host), int(n_kv), int(kv_format), int(bool(causal)),
        float(scale), _ptr(arena_k), _ptr(arena_v), int(arena_rows), _ptr(ws), int(ws_bytes),
        _ptr(conv), int(conv_bytes), _ptr(out), ctypes.byref(plan), s, cs))
    return int(plan.value)


def kvt_pool_rebuild(raw_k, pooled, dim, bsz, seq, cache_seqlens, block_table, pages_per_seq,
                     page_size, cr, n_pages, stream=None):
    _check("kvt_pool_rebuild", load().kvt_pool_rebuild(
        _ptr(raw_k), _ptr(pooled), int(dim), int(bsz), int(seq), _ptr(cache_seqlens),
        _ptr(block_table), int(pages_per_seq), int(page_size), int(cr), int(n_pages),
        _stream(stream)))
