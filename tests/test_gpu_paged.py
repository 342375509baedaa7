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
