"""CPU-only checks of the C ABI: the library loads, exports every entry point include/kvt.h
declares, and its host-side logic (pointer tables, argument validation) is right.  No call here
reaches a device: every one either is pure host code or fails its argument check first."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from hbm_kv_cache_amd import kvt, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "kvt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvt_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_all_exported():
    lib = kvt.load()
    names = _declared()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", kvt.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(kvt_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        assert hasattr(lib, n)
    assert set(kvt.EXPORTED) == set(names)


def test_binding_constants_equal_the_header():
    """Every value #define of include/kvt.h (status codes, directions, copy modes, formats, host
    flags, workspace ops) has the same value in the Python binding, and every signature the
    binding declares names a function the header declares."""
    text = open(os.path.join(ROOT, "include", "kvt.h")).read()
    defs = dict(re.findall(r"^#define KVT_(\w+)\s+\(?(-?\d+)u?\)?", text, re.M))
    defs.pop("ABI_VERSION")
    assert {"COPY_RUNTIME", "Q8_0", "OP_PREFILL_STATE", "EHIP"} <= set(defs)
    for name, value in defs.items():
        assert getattr(kvt, name) == int(value), name
    assert set(kvt._SIGNATURES) <= set(_declared())


def test_abi_version():
    assert kvt.kvt_abi_version() == 16


def test_library_has_gfx950_code_object():
    out = subprocess.run(["strings", kvt.LIB_PATH], capture_output=True, text=True).stdout
    assert "gfx950" in out


@pytest.mark.parametrize("bpc,skip", [(1, 0), (4, 0), (4, 3), (2, 1), (8, 7)])
def test_sub_block_ptrs_equal_oracle(bpc, skip):
    g = synth.rng(0, synth.P_MISC, 100 + bpc * 10 + skip)
    ids = g.permutation(1000)[:50].astype(np.int64)
    n_out = 50 * bpc - skip - g.integers(0, bpc)
    base, stride, page = 0x7F00_0000_1000, 135168, 32768
    got = np.zeros(n_out, dtype=np.uint64)
    kvt.kvt_sub_block_ptrs(base, stride, page, ids, ids.size, bpc, skip, got, n_out)
    ref = oracle.sub_block_ptrs(base, stride, page, ids, bpc, skip, n_out)
    assert np.array_equal(got, ref)


def test_sub_block_ptrs_errors_match_oracle_rules():
    out = np.zeros(8, dtype=np.uint64)
    ids = np.array([1, 2], dtype=np.int64)
    for bpc, skip, n, code in [(4, 4, 1, kvt.EINVAL), (4, -1, 1, kvt.EINVAL), (0, 0, 1, kvt.EINVAL),
                               (4, 1, 8, kvt.ERANGE)]:
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_sub_block_ptrs(0, 64, 16, ids, 2, bpc, skip, out, n)
        assert e.value.code == code
    neg = np.array([3, -1], dtype=np.int64)
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_sub_block_ptrs(0, 64, 16, neg, 2, 1, 0, out, 2)
    assert e.value.code == kvt.ERANGE


def test_chunks_consumed_equal_oracle():
    for bpc in (1, 2, 4, 8):
        for skip in range(bpc):
            for n in range(0, 30):
                assert kvt.kvt_chunks_consumed(n, skip, bpc) == oracle.chunks_consumed(n, skip, bpc)


def test_argument_errors_return_before_any_device_work():
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_swap_blocks(None, None, None, 4, kvt.H2D, kvt.COPY_KERNEL, stream=0)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_swap_blocks(None, None, None, 0, 7, kvt.COPY_KERNEL, stream=0)
    assert e.value.code == kvt.EINVAL
    for mode in (-1, 4):   # modes are AUTO, KERNEL, SDMA, RUNTIME
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_swap_blocks(None, None, None, 0, kvt.H2D, mode, stream=0)
        assert e.value.code == kvt.EINVAL
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_stage_tail(16, 16, 0, 1, 16, mode, stream=0)
        assert e.value.code == kvt.EINVAL
    for mode in (kvt.COPY_AUTO, kvt.COPY_KERNEL, kvt.COPY_SDMA, kvt.COPY_RUNTIME):
        kvt.kvt_swap_blocks(None, None, None, 0, kvt.H2D, mode, stream=0)   # n = 0: no-op
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_index_topk(16, 100, 128, 16, 8, 0, 16, None, 16, 1 << 20, stream=0)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:   # workspace too small
        kvt.kvt_index_topk(16, 100, 128, 16, 8, 32, 16, None, 16, 8, stream=0)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_gather_blocks(16, 16, 2, 8, 128, 2, 64 * 100, 256, 100, None, 64, 16, 32, 16, 16,
                              stream=0)
    assert e.value.code == kvt.EALIGN
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_attn_decode(16, 64, 8, 64, kvt.BF16, 16, 16, 10, None, 0.1, 16, 16, 1 << 20,
                            stream=0)
    assert e.value.code == kvt.EUNSUPPORTED
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_attn_decode(16, 63, 8, 128, kvt.BF16, 16, 16, 10, None, 0.1, 16, 16, 1 << 20,
                            stream=0)
    assert e.value.code == kvt.EINVAL
    fused = dict(q=16, n_qh=64, kvh=8, hd=128, dtype=kvt.BF16, k_plane=16, v_plane=16,
                 n_blocks=100, block_stride=16384 * 8, head_stride=16384, token_stride=256,
                 block_table=None, bt=64, ids=16, k=32, k_out=16, v_out=16, scale=0.1, out=16,
                 ws=16, ws_bytes=1 << 20, stream=0)
    for change, code in [(dict(hd=64), kvt.EUNSUPPORTED), (dict(dtype=kvt.Q8_0), kvt.EUNSUPPORTED),
                         (dict(v_out=None), kvt.EINVAL), (dict(n_blocks=0), kvt.EINVAL),
                         (dict(n_qh=63), kvt.EINVAL), (dict(token_stride=264), kvt.EALIGN),
                         (dict(k_plane=24), kvt.EALIGN), (dict(ws_bytes=100), kvt.EINVAL),
                         (dict(k=1 << 26, bt=64), kvt.ERANGE), (dict(ids=None), kvt.EINVAL)]:
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_gather_attn_decode(**{**fused, **change})
        assert e.value.code == code, change
    pre = dict(q=16, n_q=4, q_pos0=0, n_qh=8, kvh=8, hd=128, k_head=16, v_head=16, n_head=100,
               k_tail=16, v_tail=16, n_kv=1000, kv_format=kvt.Q8_0, causal=1, scale=0.1,
               key_begin=0, key_end=128, state=16, state_bytes=1 << 30, out=16, stream=0)
    for change in (dict(key_begin=10), dict(key_end=100), dict(key_end=1001),
                   dict(state_bytes=16), dict(state=None)):
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_attn_prefill_range(**{**pre, **change})
        assert e.value.code == kvt.EINVAL, change
    pipe = {k_: v_ for k_, v_ in pre.items() if k_ not in ("key_begin", "key_end", "k_tail",
                                                           "v_tail")}
    pipe.update(k_host=16, v_host=16, arena_k=16, arena_v=16, arena_rows=4096, copy_stream=8)
    for change in (dict(arena_rows=100), dict(copy_stream=0), dict(state_bytes=16),
                   dict(arena_k=None)):
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_attn_prefill_pipelined(**{**pipe, **change})
        assert e.value.code == kvt.EINVAL, change
    chain = dict(pipe, staged_rows=0, next_k_host=16, next_v_host=16, next_rows=64,
                 next_arena_k=1 << 40, next_arena_v=1 << 41, next_arena_rows=4096)
    for change in (dict(next_rows=2049),                     # more than one next bucket
                   dict(next_arena_rows=100),                # next buckets under 64 keys
                   dict(next_k_host=None), dict(next_arena_v=None),
                   dict(next_arena_k=1 << 40 | 4),           # misaligned
                   dict(next_arena_k=16),                    # overlaps this call's arena
                   dict(next_arena_v=(1 << 40) + 64 * 1088 - 8),   # next K and V overlap
                   dict(next_rows=-1),
                   dict(staged_rows=1),                      # nothing was prefetched
                   dict(copy_stream=0)):
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_attn_prefill_chain(**{**chain, **change})
        assert e.value.code == kvt.EINVAL, change
    assert kvt.kvt_attn_prefill_state_bytes(2048, 32, 8) == 32 * 8 * 8 * 66 * 64 * 4
    assert kvt.kvt_attn_prefill_state_bytes(10, 12, 1) == 0      # group 12: unsupported
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_stage_tail(16, 0, 0, 10, 16, kvt.COPY_AUTO, stream=0)
    assert e.value.code == kvt.EINVAL
    kvt.kvt_stage_tail(16, 34, 10, 10, 16, kvt.COPY_AUTO, stream=0)   # empty range: no-op


def test_workspace_sizes_are_monotone_and_cover_candidates():
    a = kvt.kvt_index_topk_ws_bytes(4096, 8, 32)
    b = kvt.kvt_index_topk_ws_bytes(16384, 8, 32)
    c = kvt.kvt_index_topk_ws_bytes(1 << 20, 8, 32)     # needs intermediate merge levels
    assert 0 < a < b < c
    assert b >= 8 * (16384 // 128) * 32 * 12
    assert kvt.kvt_attn_decode_ws_bytes(64, 128, 2048) == 64 * 32 * 130 * 4


def test_worker_argument_errors_touch_no_device():
    lib = kvt.load()
    h = ctypes.c_void_p()
    assert lib.kvt_worker_create(2, kvt.COPY_AUTO, ctypes.byref(h)) == kvt.EINVAL
    assert lib.kvt_worker_create(kvt.H2D, 7, ctypes.byref(h)) == kvt.EINVAL
    assert lib.kvt_worker_create(kvt.D2H, kvt.COPY_SDMA, None) == kvt.EINVAL
    h2 = ctypes.c_void_p()
    assert lib.kvt_worker_create(kvt.D2H, kvt.COPY_SDMA, ctypes.byref(h2)) == kvt.EUNSUPPORTED
    assert not h2.value
    assert h.value is None
    n = ctypes.c_int32(-1)
    t = np.zeros(4, np.uint64)
    assert lib.kvt_worker_submit(None, 1, t.ctypes.data, t.ctypes.data, t.ctypes.data, 4,
                                 None) == kvt.EINVAL
    assert lib.kvt_worker_get_finished(None, None, None, None, 0, ctypes.byref(n)) == kvt.EINVAL
    assert lib.kvt_worker_wait(None, None, 0) == kvt.EINVAL
    assert lib.kvt_worker_pending(None) == kvt.EINVAL
    assert lib.kvt_worker_reserve(None, 1, 1) == kvt.EINVAL
    assert lib.kvt_worker_destroy(None) == kvt.OK
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_worker_create(5)
    assert e.value.code == kvt.EINVAL and "dir=5" in str(e.value)


def test_paged_write_and_copy_page_argument_errors():
    a = np.zeros(64, np.uint8)
    p = a.ctypes.data
    lens = np.zeros(1, np.int32)
    tab = np.zeros(4, np.int32)
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_paged_write([], [], [], 1, 1, lens, tab, 4, 16, 4, stream=0)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_paged_write([p], [p], [24], 1, 1, lens, tab, 4, 16, 4, stream=0)
    assert e.value.code == kvt.EALIGN
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_paged_write([p], [p], [32], 1, 1, None, tab, 4, 16, 4, stream=0)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_paged_write([p], [p], [32], 1, 1, lens, tab, 0, 16, 4, stream=0)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_paged_write([p] * 5, [p] * 5, [32] * 5, 1, 1, lens, tab, 4, 16, 4, stream=0)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_copy_page([p], [p], [32], 0, 1, 16, 17, stream=0)     # more tokens than a page
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_copy_page([p], [p], [32], 0, 1, 16, 4, p, p, 16, 3, stream=0)   # 3 !| 16
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_copy_page([p], [p], [32], 0, 1, 16, 4, p, None, 16, 4, stream=0)
    assert e.value.code == kvt.EINVAL


def test_staging_rule_equals_oracle_and_rows_argument_errors():
    g = np.random.default_rng(5)
    for _ in range(2000):
        r, k, p, s = (int(x) for x in g.integers(0, 5000, size=4))
        assert kvt.kvt_staging_worthwhile(r, k, p, s) == oracle.staging_worthwhile(r, k, p, s)
    assert kvt.kvt_staging_worthwhile(2048, 2080, 4096, 256)
    assert kvt.kvt_sparse_attend_rows_ws_bytes(1, 64, 8, 2080) == 64 * 33 * 130 * 4
    assert kvt.kvt_sparse_attend_rows_ws_bytes(2048, 32, 8, 2080) == 2048 * 32 * 1 * 130 * 4
    a = np.zeros(1 << 16, np.uint8)
    p = a.ctypes.data
    ws = kvt.kvt_sparse_attend_rows_ws_bytes(2, 16, 4, 100)
    base = dict(q=p, rows=2, n_qh=16, kvh=4, hd=128, dtype=kvt.BF16, k_plane=p, v_plane=p,
                n_rows=64, row_stride=1024, head_stride=256, block_table=None, table_cols=0,
                table_row_stride=0, page_size=16, positions=p, k_pad=100, scale=0.1, out=p,
                ws=p, ws_bytes=ws, stream=0)
    for change, code in [({"hd": 64}, kvt.EUNSUPPORTED), ({"n_qh": 15}, kvt.EINVAL),
                         ({"k_pad": 0}, kvt.EINVAL), ({"row_stride": 1000}, kvt.EALIGN),
                         ({"head_stride": 512}, kvt.EINVAL), ({"ws_bytes": ws - 1}, kvt.EINVAL),
                         ({"rows": 70000}, kvt.EINVAL), ({"positions": None}, kvt.EINVAL),
                         ({"block_table": p, "table_cols": 0}, kvt.EINVAL)]:
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_sparse_attend_rows(**{**base, **change})
        assert e.value.code == code, change
    with pytest.raises(kvt.KvtError) as e:     # the automatic form needs a table
        kvt.kvt_sparse_attend_rows_auto(p, 2, 16, 4, 128, kvt.BF16, p, p, 64, 1024, 256, None, 4,
                                        16, p, 100, 0.1, p, p, ws, stream=0)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_stage_pages(p, None, 4096, p, 4, 8, p, p, stream=0)
    assert e.value.code == kvt.EINVAL


def test_workspace_bytes_dispatches_to_the_per_op_sizes():
    cases = [(kvt.OP_INDEX_TOPK, (4096, 8, 32), kvt.kvt_index_topk_ws_bytes(4096, 8, 32)),
             (kvt.OP_INDEX_TOPK, (65535, 8, 512), kvt.kvt_index_topk_ws_bytes(65535, 8, 512)),
             (kvt.OP_ATTN_DECODE, (64, 128, 2048), kvt.kvt_attn_decode_ws_bytes(64, 128, 2048)),
             (kvt.OP_SPARSE_ROWS, (2048, 64, 8, 2080),
              kvt.kvt_sparse_attend_rows_ws_bytes(2048, 64, 8, 2080)),
             (kvt.OP_PREFILL_STATE, (2048, 32, 8), kvt.kvt_attn_prefill_state_bytes(2048, 32, 8)),
             (kvt.OP_NONE_NEEDED, (), 0)]
    for op, dims, want in cases:
        assert kvt.kvt_workspace_bytes(op, dims) == want > 0 or op == kvt.OP_NONE_NEEDED
    assert kvt.kvt_workspace_bytes(9, (1, 2, 3)) == 0 and "op=9" in kvt.kvt_last_error()
    assert kvt.kvt_workspace_bytes(kvt.OP_ATTN_DECODE, (64, 128)) == 0
    assert "takes 3 dims" in kvt.kvt_last_error()
    assert kvt.kvt_workspace_bytes(kvt.OP_SPARSE_ROWS, (1 << 40, 64, 8, 2080)) == 0
    assert "int32" in kvt.kvt_last_error()


# Chunk length against the stage-or-read-in-place choice over a 180,000-key q8_0 cache with
# 94,208 rows in HBM (8 KV heads, 32 query heads, causal chunk at the end), as measured on
# MI355X in ms (split-K form, staged / in place): 1 token 3.52 / 6.92, 16: 3.54 / 6.91,
# 64: 3.60 / 6.91, 256: 4.31 / 6.93, 512: 5.34 / 7.25, 1024: 7.49 / 7.60, 2048 (one split,
# the single pass): 11.34 / 11.41.  Without a second stream the rule stages up to 512 tokens
# and reads in place from 1024, where the two are within 2%.
@pytest.mark.parametrize("n_q,plan", [(1, kvt.PREFILL_STAGED), (16, kvt.PREFILL_STAGED),
                                      (64, kvt.PREFILL_STAGED), (256, kvt.PREFILL_STAGED),
                                      (512, kvt.PREFILL_STAGED),
                                      (1024, kvt.PREFILL_IN_PLACE),
                                      (2048, kvt.PREFILL_IN_PLACE)])
def test_prefill_plan_follows_the_measured_crossover(n_q, plan):
    n_kv, n_head = 180000, 94208
    got = kvt.kvt_attn_prefill_plan(n_q, n_kv - n_q, 32, 8, n_head, n_kv, kvt.Q8_0, True,
                                    n_kv - n_head, False)
    assert got == plan
    # with a second stream and an arena smaller than the tail every chunk length pipelines;
    # with an arena that holds the tail, chunks whose attention is under a quarter of the copy
    # (up to 64 tokens here: 3.52-3.59 ms staged against 3.60-3.65 pipelined) stage instead
    assert kvt.kvt_attn_prefill_plan(n_q, n_kv - n_q, 32, 8, n_head, n_kv, kvt.Q8_0, True,
                                     2 * 16384, True) == kvt.PREFILL_PIPELINED
    assert kvt.kvt_attn_prefill_plan(n_q, n_kv - n_q, 32, 8, n_head, n_kv, kvt.Q8_0, True,
                                     n_kv - n_head, True) == (
        kvt.PREFILL_STAGED if n_q <= 64 else kvt.PREFILL_PIPELINED)


def test_prefill_plan_rules():
    n_kv, n_head = 8192, 3000
    P = kvt.kvt_attn_prefill_plan
    # nothing in host memory, or no queries: in place (nothing to move)
    assert P(1, n_kv - 1, 32, 8, n_kv, n_kv, kvt.Q8_0, True, 1 << 20, True) == kvt.PREFILL_IN_PLACE
    assert P(0, 0, 32, 8, n_head, n_kv, kvt.Q8_0, True, 1 << 20, True) == kvt.PREFILL_IN_PLACE
    # a second stream and an arena of >= 128 rows (smaller than the tail): pipelined, for
    # short and long chunks
    for n_q in (1, 1024, 2048):
        assert P(n_q, n_kv - n_q, 32, 8, n_head, n_kv, kvt.Q8_0, True, 128,
                 True) == kvt.PREFILL_PIPELINED
        assert P(n_q, n_kv - n_q, 32, 8, n_head, n_kv, kvt.Q8_0, True, 127,
                 True) != kvt.PREFILL_PIPELINED
    # an arena that holds the tail, two streams: one token's attention (~0.2 us) is far under
    # a quarter of the copy (~202 us): staged; 1024 queries (~161 us) pipeline
    assert P(1, n_kv - 1, 32, 8, n_head, n_kv, kvt.Q8_0, True, n_kv - n_head,
             True) == kvt.PREFILL_STAGED
    assert P(1024, n_kv - 1024, 32, 8, n_head, n_kv, kvt.Q8_0, True, n_kv - n_head,
             True) == kvt.PREFILL_PIPELINED
    # one stream: a short chunk stages only into an arena that holds the whole tail
    assert P(1, n_kv - 1, 32, 8, n_head, n_kv, kvt.Q8_0, True, n_kv - n_head,
             False) == kvt.PREFILL_STAGED
    assert P(1, n_kv - 1, 32, 8, n_head, n_kv, kvt.Q8_0, True, n_kv - n_head - 1,
             False) == kvt.PREFILL_IN_PLACE
    # the time model: 1024 causal queries over 8192 keys take ~161 us of attention; staging
    # 5192 or 1192 tail rows takes ~202 or ~46 us
    assert P(1024, n_kv - 1024, 32, 8, 3000, n_kv, kvt.Q8_0, True, 1 << 20,
             False) == kvt.PREFILL_STAGED
    assert P(1024, n_kv - 1024, 32, 8, 7000, n_kv, kvt.Q8_0, True, 1 << 20,
             False) == kvt.PREFILL_IN_PLACE
    # 2048 queries (~301 us) against 5192 rows (~202 us): in place
    assert P(2048, n_kv - 2048, 32, 8, 3000, n_kv, kvt.Q8_0, True, 1 << 20,
             False) == kvt.PREFILL_IN_PLACE
    # bf16: the same 1024 queries at 0.50 PFLOP/s take ~258 us, staging 2 x 5192 rows of 2048
    # bytes ~380 us
    assert P(1024, n_kv - 1024, 32, 8, 3000, n_kv, kvt.BF16, True, 1 << 20,
             False) == kvt.PREFILL_STAGED
    # non-causal chunks visit every key: 1024 x 8192 pairs is ~172 us against ~46 us staging
    assert P(1024, 0, 32, 8, 7000, n_kv, kvt.Q8_0, False, 1 << 20,
             False) == kvt.PREFILL_IN_PLACE
    for bad in [dict(kvh=3), dict(n_head=n_kv + 1), dict(n_q=-1), dict(fmt=9), dict(arena=-1)]:
        a = dict(n_q=1, kvh=8, n_head=n_head, fmt=kvt.Q8_0, arena=0)
        a.update(bad)
        with pytest.raises(kvt.KvtError):
            P(a["n_q"], 0, 32, a["kvh"], a["n_head"], n_kv, a["fmt"], True, a["arena"], True)
