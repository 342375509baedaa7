"""GPU parity of the host tier's write side against the oracle: paged K/V (+ raw key) writes
through a block table into host-mapped pages, and copy_page.  Bit-exact, with canaries:
every byte the oracle does not write must keep its old value."""
import numpy as np
import pytest
import torch

import oracle
from hbm_kv_cache_amd import kvt, synth

pytestmark = pytest.mark.gpu

KV_ROW = 8 * 128 * 2    # 8 KV heads x 128 dims, bf16
RAW_ROW = 128 * 2       # one 128-dim fp16 raw key per token


def _host_planes(n_pages, page_size, row_bytes, seed):
    bufs, views = [], []
    for i, rb in enumerate(row_bytes):
        hb = kvt.HostBuffer(n_pages * page_size * rb)
        v = hb.numpy(np.uint8, (n_pages, page_size, rb))
        synth.fill_random_bytes(synth.rng(12, synth.P_MISC, seed * 8 + i), v)
        bufs.append(hb)
        views.append(v)
    return bufs, views


def _dev(a, gpu):
    return torch.from_numpy(np.ascontiguousarray(a)).to(gpu)


@pytest.mark.parametrize("bsz,seq,lens", [
    (3, 300, [0, 1000, 5000]),     # a prefill chunk per sequence, spanning pages
    (1, 1, [777]),                 # one decode token
    (4, 17, [255, 256, 3, 6140]),  # page boundaries; the last runs past the table
])
def test_paged_write_matches_oracle(gpu, bsz, seq, lens):
    n_pages, ps, pps = 96, 256, 24
    rbs = [KV_ROW, KV_ROW, RAW_ROW]
    bufs, planes = _host_planes(n_pages, ps, rbs, seq)
    g = synth.rng(12, synth.P_PERM_DST, seq)
    table = synth.permutation(g, n_pages)[:bsz * pps].reshape(bsz, pps).astype(np.int32)
    if bsz >= 3:
        table[1, 5] = -1           # a hole: its rows are dropped
        table[2, 20] = 999         # out of range: dropped
    rows = [synth.rng(12, synth.P_K, seq * 4 + i).integers(0, 256, size=(bsz, seq, rb),
                                                             dtype=np.uint8)
            for i, rb in enumerate(rbs)]
    ref = [p.copy() for p in planes]
    oracle.paged_write(ref, rows, np.array(lens), table, ps)
    src = [_dev(r, gpu) for r in rows]
    kvt.kvt_paged_write(src, [b.dev for b in bufs], rbs, bsz, seq,
                        _dev(np.array(lens, np.int32), gpu), _dev(table, gpu), pps, ps, n_pages)
    torch.cuda.synchronize()
    for i in range(3):
        assert np.array_equal(planes[i], ref[i]), f"plane {i}"
    # nothing to write: no change
    kvt.kvt_paged_write(src, [b.dev for b in bufs], rbs, bsz, 0,
                        _dev(np.array(lens, np.int32), gpu), _dev(table, gpu), pps, ps, n_pages)
    torch.cuda.synchronize()
    assert all(np.array_equal(planes[i], ref[i]) for i in range(3))
    del planes
    for b in bufs:
        b.free()


def test_paged_write_into_hbm_planes(gpu):
    """The same rule with the planes in HBM (the all-device cache)."""
    n_pages, ps, pps, bsz, seq = 40, 64, 10, 2, 100
    g = synth.rng(12, synth.P_MISC, 99)
    plane = g.integers(0, 256, size=(n_pages, ps, KV_ROW), dtype=np.uint8)
    table = synth.permutation(g, n_pages)[:bsz * pps].reshape(bsz, pps).astype(np.int32)
    lens = np.array([10, 500], np.int32)
    rows = g.integers(0, 256, size=(bsz, seq, KV_ROW), dtype=np.uint8)
    dplane = _dev(plane, gpu)
    kvt.kvt_paged_write([_dev(rows, gpu)], [dplane], [KV_ROW], bsz, seq, _dev(lens, gpu),
                        _dev(table, gpu), pps, ps, n_pages)
    oracle.paged_write([plane], [rows], lens, table, ps)
    torch.cuda.synchronize()
    assert np.array_equal(dplane.cpu().numpy(), plane)


def test_copy_page_after_queued_write(gpu):
    """A paged write into the source page is queued on the stream, then copy_page runs: the
    copy must see the written rows (it drains the stream first); pooled rows copied on the
    device: ceil(n / cr) of them."""
    n_pages, ps, cr, pps = 48, 256, 4, 4
    rbs = [KV_ROW, KV_ROW, RAW_ROW]
    bufs, planes = _host_planes(n_pages, ps, rbs, 7)
    g = synth.rng(12, synth.P_POOLED, 7)
    pooled_np = g.integers(0, 256, size=(n_pages, ps // cr, 256), dtype=np.uint8)
    pooled = _dev(pooled_np, gpu)
    table = np.array([[7, 8, 9, 10]], np.int32)
    lens = np.array([100], np.int32)
    rows = [g.integers(0, 256, size=(1, 30, rb), dtype=np.uint8) for rb in rbs]
    ref = [p.copy() for p in planes]
    ref_pooled = pooled_np.copy()
    kvt.kvt_paged_write([_dev(r, gpu) for r in rows], [b.dev for b in bufs], rbs, 1, 30,
                        _dev(lens, gpu), _dev(table, gpu), pps, ps, n_pages)
    for nt, (frm, to) in ((130, (7, 30)), (ps, (8, 31)), (1, (9, 32)), (0, (10, 33))):
        kvt.kvt_copy_page([b.host for b in bufs], [b.host for b in bufs], rbs, frm, to, ps, nt,
                          pooled, pooled, 256, cr)
    torch.cuda.synchronize()
    oracle.paged_write(ref, rows, lens, table, ps)
    for nt, (frm, to) in ((130, (7, 30)), (ps, (8, 31)), (1, (9, 32)), (0, (10, 33))):
        oracle.copy_page(ref, ref, frm, to, nt, ref_pooled, ref_pooled, cr)
    for i in range(3):
        assert np.array_equal(planes[i], ref[i]), f"plane {i}"
    assert np.array_equal(pooled.cpu().numpy(), ref_pooled)
    del planes
    for b in bufs:
        b.free()


# ---------------------------------------------------------------------------------------------
# pool rebuild at the write head
# ---------------------------------------------------------------------------------------------

def _pool_golden():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "pool_rebuild_worked.json")) as f:
        return json.load(f)


def test_pool_rebuild_worked_example(gpu):
    """The hand-worked fixture through the GPU: complete and partial blocks, stale rows past
    the write head left out, canaries elsewhere; the three-row partial block."""
    w = _pool_golden()
    ps, cr, dim, n_pages = w["page_size"], w["cr"], w["dim"], w["n_pages"]
    raw = np.zeros((n_pages, ps, dim), dtype=np.float16)
    for r in w["raw_rows"]:
        raw[r["page"], r["row"]] = r["values"]
    raw_d = _dev(raw.view(np.int16), gpu)
    pooled = torch.full((n_pages, ps // cr, dim), w["pooled_canary_bits"], dtype=torch.int16,
                        device=gpu)
    table = _dev(np.array(w["block_table"], np.int32), gpu)
    kvt.kvt_pool_rebuild(raw_d, pooled, dim, 3, w["seq"], _dev(np.array(w["cache_seqlens"],
                         np.int32), gpu), table, 2, ps, cr, n_pages)
    torch.cuda.synchronize()
    want = np.full((n_pages, ps // cr, dim), w["pooled_canary_bits"], dtype=np.uint16)
    for e in w["expected_pooled"]:
        want[e["page"], e["row"]] = e["bits"]
    assert np.array_equal(pooled.cpu().numpy().view(np.uint16), want)
    pooled.fill_(w["pooled_canary_bits"])
    kvt.kvt_pool_rebuild(raw_d, pooled, dim, 3, 3, _dev(np.array([-1, 0, -1], np.int32), gpu),
                         table, 2, ps, cr, n_pages)
    torch.cuda.synchronize()
    assert list(pooled.cpu().numpy().view(np.uint16)[1, 0]) == w["partial_three_rows"]["bits"]


@pytest.mark.parametrize("bsz,seq,lens", [
    (1, 1, [777]),                 # one decode token: one block, partial or complete
    (1, 1, [779]),                 # the token that completes a block
    (3, 300, [0, 1001, 5000]),     # a prefill chunk per sequence, partial first block
    (4, 17, [255, 256, 3, 6140]),  # page boundaries; the last runs past the table
    (2, 2048, [0, 130]),           # a whole prefill chunk
])
def test_pool_rebuild_after_paged_write_matches_oracle(gpu, bsz, seq, lens):
    """The upkeep step at the QSA geometry (cr 4, 128-dim fp16 raw keys, pages of 256
    tokens): new raw key rows reach the host-mapped raw plane through kvt_paged_write, then
    kvt_pool_rebuild recomputes the touched pooled blocks in HBM from them.  Bit-exact against
    oracle.paged_write + oracle.pool_rebuild; untouched pooled rows keep their old values."""
    n_pages, ps, pps, cr, dim = 96, 256, 24, 4, 128
    raw_buf = kvt.HostBuffer(n_pages * ps * dim * 2)
    raw = raw_buf.numpy(np.uint16, (n_pages, ps, dim))
    raw[:] = synth.f16_normal(synth.rng(12, synth.P_K, 900 + seq), (n_pages, ps, dim))
    g = synth.rng(12, synth.P_PERM_DST, 900 + seq)
    table = synth.permutation(g, n_pages)[:bsz * pps].reshape(bsz, pps).astype(np.int32)
    if bsz >= 3:
        table[1, 5] = -1
        table[2, 20] = 999
    new = synth.f16_normal(synth.rng(12, synth.P_V, 900 + seq), (bsz, seq, dim))
    pooled0 = synth.f16_normal(synth.rng(12, synth.P_CANARY, 900 + seq),
                               (n_pages, ps // cr, dim))
    lens_a = np.array(lens, np.int32)
    # oracle: write the rows, then rebuild
    ref_raw = raw.copy()
    oracle.paged_write([ref_raw.view(np.uint8).reshape(n_pages, ps, dim * 2)],
                       [new.view(np.uint8).reshape(bsz, seq, dim * 2)], lens_a, table, ps)
    ref_pooled = oracle.pool_rebuild(ref_raw, pooled0.copy(), lens_a, seq, table, ps, cr)
    # GPU
    pooled = _dev(pooled0.view(np.int16), gpu)
    lens_d, table_d = _dev(lens_a, gpu), _dev(table, gpu)
    kvt.kvt_paged_write([_dev(new.view(np.int16), gpu)], [raw_buf.dev], [dim * 2], bsz, seq,
                        lens_d, table_d, pps, ps, n_pages)
    kvt.kvt_pool_rebuild(raw_buf.dev, pooled, dim, bsz, seq, lens_d, table_d, pps, ps, cr,
                         n_pages)
    torch.cuda.synchronize()
    assert np.array_equal(raw, ref_raw), "raw rows"
    got = pooled.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref_pooled), "pooled rows"
    assert (got != pooled0).any(), "something was rebuilt"
    del raw
    raw_buf.free()


def test_pool_rebuild_rounding_edges(gpu):
    """Blocks whose means fall exactly halfway between fp16 neighbours (ties to even, both
    ways), in the subnormal range, at the top of the range, past it (infinity), and with
    infinite or NaN raw keys: the same bits as the oracle's rounding (NaN as 0x7E00)."""
    cr, ps, n_pages = 2, 2, 1
    pairs = [(1.0, 1.0009765625),            # mean 1 + 2^-11: tie -> 1.0 (even)
             (1.0009765625, 1.001953125),    # mean 1 + 3*2^-11: tie -> 1 + 2^-9 (even)
             (-1.0, -1.0009765625),
             (2.0 ** -24, 0.0),              # mean 2^-25: tie -> 0
             (3 * 2.0 ** -24, 0.0),          # 1.5 units of 2^-24: tie -> 2 units
             (2.0 ** -24, 2.0 ** -23),
             (6.1035e-05, 6.0976e-05),       # around the smallest normal
             (65504.0, 65504.0), (65504.0, 65472.0),
             (65504.0, float("inf")), (float("-inf"), 1.0), (float("inf"), float("-inf")),
             (float("nan"), 1.0), (0.333251953125, 0.333251953125), (-0.0, -0.0)]
    dim = len(pairs)
    raw = np.zeros((n_pages, ps, dim), dtype=np.float16)
    for d, (a, b) in enumerate(pairs):
        raw[0, 0, d], raw[0, 1, d] = a, b
    ref = oracle.pool_rebuild(raw.view(np.uint16), np.zeros((1, 1, dim), np.uint16), [0], 2,
                              [[0]], ps, cr)
    pooled = torch.zeros((1, 1, dim), dtype=torch.int16, device=gpu)
    kvt.kvt_pool_rebuild(_dev(raw.view(np.int16), gpu), pooled, dim, 1, 2,
                         _dev(np.array([0], np.int32), gpu), _dev(np.array([[0]], np.int32), gpu),
                         1, ps, cr, n_pages)
    torch.cuda.synchronize()
    assert np.array_equal(pooled.cpu().numpy().view(np.uint16), ref)
    assert ref[0, 0, 0] == 0x3C00 and ref[0, 0, 1] == 0x3C02 and ref[0, 0, 3] == 0
    assert ref[0, 0, 4] == 2 and ref[0, 0, 12] == 0x7E00


def test_pool_rebuild_argument_errors(gpu):
    raw = torch.zeros((2, 8, 4), dtype=torch.int16, device=gpu)
    pooled = torch.zeros((2, 2, 4), dtype=torch.int16, device=gpu)
    lens = torch.zeros(1, dtype=torch.int32, device=gpu)
    table = torch.zeros((1, 1), dtype=torch.int32, device=gpu)
    for kw, code in [({"cr": 3}, kvt.EINVAL), ({"cr": 0}, kvt.EINVAL), ({"dim": 0}, kvt.EINVAL),
                     ({"page_size": 0}, kvt.EINVAL)]:
        a = dict(dim=4, bsz=1, seq=1, pages_per_seq=1, page_size=8, cr=4, n_pages=2)
        a.update(kw)
        with pytest.raises(kvt.KvtError) as e:
            kvt.kvt_pool_rebuild(raw, pooled, a["dim"], a["bsz"], a["seq"], lens, table,
                                 a["pages_per_seq"], a["page_size"], a["cr"], a["n_pages"])
        assert e.value.code == code
    kvt.kvt_pool_rebuild(raw, pooled, 4, 1, 0, lens, table, 1, 8, 4, 2)    # nothing appended
