"""CPU oracle for the tiered KV-cache hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  It wraps ``liboracle.so`` (plain C, fp64, memcpy loops, brute-force top-k, built
from ``kvt_oracle.c`` by ``oracle/build.py``) with numpy-in / numpy-out functions.  It shares no
code with the HIP library in ``hbm_kv_cache_amd``.

Functions and the passages they follow:

* ``sub_block_ptrs``   -- vLLM CPU offloading worker, ``compute_sub_block_ptrs``.
* ``swap``             -- vLLM CPU offloading worker, ``transfer_async`` / ``swap_blocks_batch``.
* ``index_scores``, ``topk`` -- QSA KV offload for ExLlamaV3, ``CacheLayer_qsa_offload``
  docstring (pooled plane scored in full every step, top-k selection).
* ``gather``           -- QSA KV offload, ``sparse_attend`` (selected K/V rows from host planes).
* ``stage_tail``       -- llama.cpp PR #319 commit text (used host rows copied to a VRAM buffer).
* ``attn_decode``      -- QSA KV offload, staged attention (GQA map, softmax normalisation).
* ``attn_prefill``     -- llama.cpp PR #319 (VRAM head + host tail, same output as all-device).
* ``sparse_attend_rows`` -- QSA KV offload, ``qsa_sparse_attend_rows`` (each query row over its
  own selection of cache positions, mapped through the row's page table).
* ``staging_worthwhile`` -- QSA KV offload, ``qsa_staging_worthwhile``.
* ``paged_write``      -- QSA KV offload, ``CacheLayer_qsa_offload`` docstring (new rows reach
  the host pages through the paged cache update; the plain block-table rule).
* ``copy_page``        -- QSA KV offload, ``CacheLayer_qsa_offload.copy_page``.
* ``pool_rebuild``     -- QSA KV offload, ``CacheLayer_qsa_offload`` docstring (the pool kernel
  rebuilds the pooled blocks an append touched, reading the raw key plane at the write head).
  The pooling function is not on the page: the reading taken is the mean of the block's raw
  key rows, rounded once to fp16 (``f64_to_f16``).

Every function here has at least one pin in ``tests/test_oracle.py`` that does not restate its
formula (library routines, closed forms, invariants, worked values).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_int, c_int32, c_int64, c_uint64, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16, Q8_0 = 1, 2, 3
OK, EINVAL, ERANGE, EOVERLAP = 0, -1, -2, -4

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = c_void_p
        sig = {
            "orc_f16_to_f64": (c_double, [ctypes.c_uint16]),
            "orc_bf16_to_f64": (c_double, [ctypes.c_uint16]),
            "orc_sub_block_ptrs": (c_int, [c_uint64, c_uint64, c_uint64, P, c_int64, c_int32,
                                           c_int32, P, c_int64]),
            "orc_chunks_consumed": (c_int64, [c_int64, c_int32, c_int32]),
            "orc_check_disjoint": (c_int, [P, P, P, c_int64]),
            "orc_swap": (c_int, [P, P, P, c_int64, c_int]),
            "orc_index_scores": (c_int, [P, c_int64, c_int32, P, c_int32, P, c_int]),
            "orc_topk": (c_int, [P, c_int32, c_int64, c_int32, P]),
            "orc_gather": (c_int, [P, P, c_int64, c_int32, c_int32, c_int32, c_int64, c_int64,
                                   c_int64, P, c_int32, P, c_int32, P, P]),
            "orc_stage_tail": (c_int, [P, c_int64, c_int64, c_int64, P]),
            "orc_attn_decode": (c_int, [P, c_int32, c_int32, c_int32, c_int32, P, P, c_int64, P,
                                        c_double, P, c_int]),
            "orc_attn_prefill": (c_int, [P, c_int64, c_int64, c_int32, c_int32, c_int32, P, P,
                                         c_int64, P, P, c_int64, c_int32, c_int32, c_double,
                                         c_int64, c_int64, P, c_int]),
            "orc_f64_to_f16": (ctypes.c_uint16, [c_double]),
            "orc_pool_rebuild": (c_int, [P, P, c_int32, c_int32, c_int32, P, P, c_int32, c_int32,
                                         c_int32, c_int64]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _threads(n):
    return int(n) if n else (os.cpu_count() or 1)


class OracleError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {code}")
        self.code = code


def _check(fn, rc):
    if rc != OK:
        raise OracleError(fn, rc)


def f16_to_f64(u16: int) -> float:
    return _load().orc_f16_to_f64(int(u16))


def bf16_to_f64(u16: int) -> float:
    return _load().orc_bf16_to_f64(int(u16))


def sub_block_ptrs(base, row_stride, page_bytes, block_ids, bpc, skip, n_out):
    ids = np.ascontiguousarray(block_ids, dtype=np.int64)
    out = np.zeros(n_out, dtype=np.uint64)
    rc = _load().orc_sub_block_ptrs(int(base), int(row_stride), int(page_bytes), _ptr(ids),
                                    ids.size, int(bpc), int(skip), _ptr(out), int(n_out))
    _check("orc_sub_block_ptrs", rc)
    return out


def chunks_consumed(n, skip, bpc):
    return int(_load().orc_chunks_consumed(int(n), int(skip), int(bpc)))


def check_disjoint(src, dst, sizes):
    src, dst, sizes = (np.ascontiguousarray(x, dtype=np.uint64) for x in (src, dst, sizes))
    return int(_load().orc_check_disjoint(_ptr(src), _ptr(dst), _ptr(sizes), src.size))


def swap(src, dst, sizes, threads=1):
    """memcpy(dst[i], src[i], sizes[i]) on raw host addresses."""
    src, dst, sizes = (np.ascontiguousarray(x, dtype=np.uint64) for x in (src, dst, sizes))
    _check("orc_swap", _load().orc_swap(_ptr(src), _ptr(dst), _ptr(sizes), src.size,
                                        _threads(threads)))


def index_scores(pooled_u16, q_u16, threads=0):
    """pooled: uint16 fp16 bits [n_blocks][d]; q: uint16 fp16 bits [n_sel][d] -> f64 [n_sel][n_blocks]."""
    pooled = np.ascontiguousarray(pooled_u16, dtype=np.uint16)
    q = np.ascontiguousarray(q_u16, dtype=np.uint16)
    n_blocks, d = pooled.shape
    n_sel = q.shape[0]
    assert q.shape[1] == d
    out = np.empty((n_sel, n_blocks), dtype=np.float64)
    _check("orc_index_scores", _load().orc_index_scores(_ptr(pooled), n_blocks, d, _ptr(q), n_sel,
                                                        _ptr(out), _threads(threads)))
    return out


def topk(scores, k):
    s = np.ascontiguousarray(scores, dtype=np.float64)
    n_sel, n_blocks = s.shape
    ids = np.empty((n_sel, k), dtype=np.int32)
    _check("orc_topk", _load().orc_topk(_ptr(s), n_sel, n_blocks, int(k), _ptr(ids)))
    return ids


def token_major_strides(kvh, hd, elem_bytes, block_tokens, row_stride=None):
    """(block, head, token) byte strides of the token-major layout [token][head][dim]."""
    row = kvh * hd * elem_bytes if row_stride is None else row_stride
    return block_tokens * row, hd * elem_bytes, row


def block_head_major_strides(kvh, hd, elem_bytes, block_tokens):
    """(block, head, token) byte strides of the layout [block][head][token][dim]."""
    return kvh * block_tokens * hd * elem_bytes, block_tokens * hd * elem_bytes, hd * elem_bytes


def gather(k_plane, v_plane, n_blocks, kvh, hd, elem_bytes, strides, ids, block_tokens,
           block_table=None, k_out=None, v_out=None):
    """Planes: uint8 arrays addressed through (block, head, token) byte strides."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    kk = ids.shape[1]
    shape = (kvh, kk * block_tokens, hd * elem_bytes)
    if k_out is None:
        k_out = np.zeros(shape, dtype=np.uint8)
    if v_out is None:
        v_out = np.zeros(shape, dtype=np.uint8)
    bt = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    bs, hs, ts = (int(x) for x in strides)
    _check("orc_gather", _load().orc_gather(_ptr(k_plane), _ptr(v_plane), int(n_blocks), kvh, hd,
                                            elem_bytes, bs, hs, ts, _ptr(bt), int(block_tokens),
                                            _ptr(ids), kk, _ptr(k_out), _ptr(v_out)))
    return k_out, v_out


def stage_tail(plane, row_bytes, row_begin, row_end, staging=None):
    if staging is None:
        staging = np.empty((row_end - row_begin) * row_bytes, dtype=np.uint8)
    _check("orc_stage_tail", _load().orc_stage_tail(_ptr(plane), int(row_bytes), int(row_begin),
                                                    int(row_end), _ptr(staging)))
    return staging


def attn_decode(q_u16, k_u16, v_u16, fmt, scale, n_valid=None, threads=0):
    """q: [n_qh][hd] bits; k, v: [kvh][n_kv][hd] bits (fp16 or bf16) -> f64 [n_qh][hd]."""
    q = np.ascontiguousarray(q_u16, dtype=np.uint16)
    k = np.ascontiguousarray(k_u16, dtype=np.uint16)
    v = np.ascontiguousarray(v_u16, dtype=np.uint16)
    n_qh, hd = q.shape
    kvh, n_kv, hd2 = k.shape
    assert hd2 == hd and v.shape == k.shape
    nv = None if n_valid is None else np.ascontiguousarray(n_valid, dtype=np.int32)
    out = np.empty((n_qh, hd), dtype=np.float64)
    _check("orc_attn_decode", _load().orc_attn_decode(_ptr(q), n_qh, kvh, hd, int(fmt), _ptr(k),
                                                      _ptr(v), n_kv, _ptr(nv), float(scale),
                                                      _ptr(out), _threads(threads)))
    return out


def qsa_k_pad(block_topk, cr):
    """Selection width of the QSA indexer: block_topk*cr positions plus up to cr - 1 tail
    positions, rounded up to a multiple of 32."""
    return -(-(block_topk * cr + cr - 1) // 32) * 32


def select_positions(ids, cr, n_tok, k_pad):
    """Token positions of the selected pooled blocks (each covers cr tokens), in id order, then
    the write head's tail (tokens cr*floor(n_tok/cr) .. n_tok-1), then -1 up to k_pad.
    ids: int [n_sel][k], ascending with -1 only at the end."""
    ids = np.asarray(ids)
    out = np.full((ids.shape[0], k_pad), -1, dtype=np.int32)
    tail = list(range(n_tok // cr * cr, n_tok))
    for h in range(ids.shape[0]):
        pos = []
        for b in ids[h]:
            if b < 0:
                break
            pos.extend(int(b) * cr + r for r in range(cr))
        pos.extend(tail)
        assert len(pos) <= k_pad
        out[h, :len(pos)] = pos
    return out


def gather_attn_decode(q_u16, k_plane, v_plane, n_blocks, kvh, hd, fmt, strides, ids,
                       block_tokens, scale, block_table=None, threads=0):
    """Decode attention over the selected blocks' rows (elements of 2 bytes) read through the
    plane strides: per KV head, the keys are the tokens of its selected slots, and a slot
    whose id lies outside [0, n_blocks) -- or whose table entry does -- contributes no key.
    Written as the two definitions above: the valid slots gathered first, then attention with
    n_valid = block_tokens * (valid slots).  Returns (out f64 [n_qh][hd], k_rows, v_rows), the
    rows as uint8 [kvh][k*block_tokens][hd*2] with the valid slots first."""
    ids = np.array(ids, dtype=np.int64)
    valid = (ids >= 0) & (ids < n_blocks)
    if block_table is not None:
        tab = np.asarray(block_table, dtype=np.int64)
        phys = np.where(valid, tab[np.clip(ids, 0, max(n_blocks - 1, 0))], -1)
        valid &= (phys >= 0) & (phys < n_blocks)
    kk = ids.shape[1]
    packed = np.full((kvh, kk), -1, dtype=np.int32)
    n_valid = np.zeros(kvh, dtype=np.int32)
    for h in range(kvh):
        sel = ids[h][valid[h]]
        packed[h, :sel.size] = sel
        n_valid[h] = sel.size * block_tokens
    ko, vo = gather(k_plane, v_plane, n_blocks, kvh, hd, 2, strides, packed, block_tokens,
                    block_table=block_table)
    n_kv = kk * block_tokens
    out = attn_decode(q_u16, ko.view(np.uint16).reshape(kvh, n_kv, hd),
                      vo.view(np.uint16).reshape(kvh, n_kv, hd), fmt, scale, n_valid=n_valid,
                      threads=threads)
    return out, ko, vo


def sparse_attend_rows(q_u16, k_plane, v_plane, n_rows, row_stride, head_stride, kvh, fmt,
                       positions, scale, block_table=None, page_size=1, table_cols=None,
                       threads=0):
    """q: [R][n_qh][hd] bits; planes: uint8 arrays of n_rows rows of row_stride bytes (head h
    of a row at byte h*head_stride); positions: int [R][k_pad] logical positions, -1 = none;
    block_table: None (positions are physical rows) or int [R or 1][cols].  A position takes
    part when it is >= 0, below table_cols*page_size (n_rows without a table), its page's
    table entry is >= 0 and the physical row is below n_rows.  Row r's output is attn_decode
    over the rows of its valid positions in order.  Returns f64 [R][n_qh][hd]."""
    q = np.ascontiguousarray(q_u16, dtype=np.uint16)
    n_r, n_qh, hd = q.shape
    kp = np.ascontiguousarray(k_plane).reshape(-1).view(np.uint8)
    vp = np.ascontiguousarray(v_plane).reshape(-1).view(np.uint8)
    tab = None if block_table is None else np.asarray(block_table, dtype=np.int64)
    if tab is not None and table_cols is None:
        table_cols = tab.shape[1]
    out = np.empty((n_r, n_qh, hd), dtype=np.float64)
    for r in range(n_r):
        phys = []
        for p in np.asarray(positions[r]).tolist():
            if p < 0:
                continue
            if tab is None:
                if p < n_rows:
                    phys.append(p)
                continue
            pg, off = divmod(p, page_size)
            if pg >= table_cols:
                continue
            e = int(tab[r if tab.shape[0] > 1 else 0, pg])
            if e >= 0 and e * page_size + off < n_rows:
                phys.append(e * page_size + off)
        n = len(phys)
        k = np.zeros((kvh, max(n, 1), hd), dtype=np.uint16)
        v = np.zeros((kvh, max(n, 1), hd), dtype=np.uint16)
        for j, x in enumerate(phys):
            for h in range(kvh):
                o = x * row_stride + h * head_stride
                k[h, j] = kp[o:o + 2 * hd].view(np.uint16)
                v[h, j] = vp[o:o + 2 * hd].view(np.uint16)
        out[r] = attn_decode(q[r], k, v, fmt, scale, n_valid=np.full(kvh, n, np.int32),
                             threads=threads)
    return out


def staging_worthwhile(rows, k_pad, pages_used, page_size):
    """Staging the used pages reads pages_used*page_size positions once; the direct path reads
    rows*k_pad.  Stage when the latter exceeds twice the former."""
    return rows * k_pad > 2 * pages_used * page_size


def paged_write(planes, new_rows, cache_seqlens, block_table, page_size):
    """Append token rows to paged planes.  planes: list of uint8 arrays [n_pages][page_size][rb]
    (modified in place); new_rows: matching list of uint8 arrays [bsz][seq][rb];
    cache_seqlens: int [bsz]; block_table: int [bsz][pages_per_seq].  Token t of sequence b sits
    at position cache_seqlens[b] + t of that sequence: logical page p // page_size, row
    p % page_size.  Rows that fall outside the table or on an invalid page are dropped."""
    table = np.asarray(block_table)
    for plane, rows in zip(planes, new_rows):
        n_pages = plane.shape[0]
        bsz, seq = rows.shape[:2]
        for b in range(bsz):
            if cache_seqlens[b] < 0:
                continue
            for t in range(seq):
                p = int(cache_seqlens[b]) + t
                slot = p // page_size
                if slot >= table.shape[1]:
                    continue
                page = int(table[b, slot])
                if 0 <= page < n_pages:
                    plane[page, p % page_size] = rows[b, t]


def copy_page(src_planes, dst_planes, from_page, to_page, num_tokens, src_pooled=None,
              dst_pooled=None, cr=1):
    """The first num_tokens rows of page from_page of each plane -> page to_page; pooled planes
    [n_pages][page_size/cr][..]: the first ceil(num_tokens / cr) rows likewise."""
    for s_, d_ in zip(src_planes, dst_planes):
        d_[to_page, :num_tokens] = s_[from_page, :num_tokens].copy()
    if src_pooled is not None:
        nb = -(-num_tokens // cr)
        dst_pooled[to_page, :nb] = src_pooled[from_page, :nb].copy()


def attn_prefill(q_u16, q_pos0, kvh, k_head, v_head, n_head, k_tail, v_tail, n_kv, fmt, causal,
                 scale, t_begin=0, t_end=None, threads=0):
    """q: [n_q][n_qh][hd] fp16 bits; K/V head and tail: uint8 row arrays -> f64 [rows][n_qh][hd]."""
    q = np.ascontiguousarray(q_u16, dtype=np.uint16)
    n_q, n_qh, hd = q.shape
    if t_end is None:
        t_end = n_q
    out = np.empty((t_end - t_begin, n_qh, hd), dtype=np.float64)
    _check("orc_attn_prefill", _load().orc_attn_prefill(
        _ptr(q), n_q, int(q_pos0), n_qh, kvh, hd, _ptr(k_head), _ptr(v_head), int(n_head),
        _ptr(k_tail), _ptr(v_tail), int(n_kv), int(fmt), int(bool(causal)), float(scale),
        int(t_begin), int(t_end), _ptr(out), _threads(threads)))
    return out


def f64_to_f16(x):
    """fp64 -> fp16 bit pattern, round to nearest even (the oracle's own conversion)."""
    return int(_load().orc_f64_to_f16(float(x)))


def pool_rebuild(raw_u16, pooled_u16, cache_seqlens, seq, block_table, page_size, cr):
    """Rebuild the pooled blocks an append of `seq` tokens at cache_seqlens[b] touched.
    raw: uint16 fp16 bits [n_pages][page_size][dim]; pooled: uint16 [n_pages][page_size/cr][dim],
    modified in place and returned.  block_table: int [bsz][pages_per_seq]."""
    raw = np.ascontiguousarray(raw_u16, dtype=np.uint16)
    assert pooled_u16.dtype == np.uint16 and pooled_u16.flags.c_contiguous
    n_pages, ps, dim = raw.shape
    assert ps == page_size
    lens = np.ascontiguousarray(cache_seqlens, dtype=np.int32)
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    _check("orc_pool_rebuild", _load().orc_pool_rebuild(
        _ptr(raw), _ptr(pooled_u16), int(dim), int(lens.size), int(seq), _ptr(lens), _ptr(table),
        int(table.shape[1]), int(page_size), int(cr), int(n_pages)))
    return pooled_u16
