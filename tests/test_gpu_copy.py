"""GPU parity of the batched swap (kvt_swap_blocks) and tail staging (kvt_stage_tail) against
the oracle's memcpy loops: bit-exact, round trips are the identity, canaries stay untouched."""
import numpy as np
import pytest
import torch

import oracle
from hbm_kv_cache_amd import kvt, synth

pytestmark = pytest.mark.gpu

MODES = [kvt.COPY_KERNEL, kvt.COPY_SDMA, kvt.COPY_RUNTIME, kvt.COPY_AUTO]
MODE_NAMES = {kvt.COPY_KERNEL: "kernel", kvt.COPY_SDMA: "sdma", kvt.COPY_RUNTIME: "runtime",
              kvt.COPY_AUTO: "auto"}


def _tables(n):
    hb = kvt.HostBuffer(max(24 * n, 24))
    assert hb.host == hb.dev, "pinned host memory must share its address with its device alias"
    t = hb.numpy(np.uint64, None)[:3 * n].reshape(3, n)
    return hb, t


def _dev_addr(t: torch.Tensor) -> int:
    return t.data_ptr()


@pytest.mark.parametrize("mode", MODES, ids=lambda m: MODE_NAMES[m])
def test_swap_one_layer_load_store_round_trip(gpu, mode):
    """One layer: K and V planes of 256 blocks x (16 tok x 8 heads x 128 dim fp16) = 32 KiB
    pages in pinned host memory; 64 seeded block ids host -> random HBM slots, then back."""
    nb, page, n = 256, 16 * 8 * 128 * 2, 64
    host = kvt.HostBuffer(2 * nb * page)
    hv = host.numpy(np.uint16, (2, nb, page // 2))
    hv[0] = synth.f16_normal(synth.rng(1, synth.P_K), (nb, page // 2))
    hv[1] = synth.f16_normal(synth.rng(1, synth.P_V), (nb, page // 2))
    dev = torch.full((2, nb, page), 0xA5, dtype=torch.uint8, device=gpu)
    src_ids = synth.permutation(synth.rng(1, synth.P_PERM_SRC), nb)[:n]
    dst_ids = synth.permutation(synth.rng(1, synth.P_PERM_DST), nb)[:n]

    tb, t = _tables(2 * n)
    for p in range(2):
        kvt.kvt_sub_block_ptrs(host.dev + p * nb * page, page, page, src_ids, n, 1, 0,
                               t[0, p * n:], n)
        kvt.kvt_sub_block_ptrs(_dev_addr(dev) + p * nb * page, page, page, dst_ids, n, 1, 0,
                               t[1, p * n:], n)
    t[2] = page
    kvt.kvt_swap_blocks(t[0], t[1], t[2], 2 * n, kvt.H2D, mode)
    torch.cuda.synchronize()

    # oracle: its own tables over the host bytes, into a canary replica of HBM
    hbytes = host.numpy(np.uint8, (2, nb, page))
    ref = np.full((2, nb, page), 0xA5, dtype=np.uint8)
    for p in range(2):
        s = oracle.sub_block_ptrs(hbytes[p].ctypes.data, page, page, src_ids, 1, 0, n)
        d = oracle.sub_block_ptrs(ref[p].ctypes.data, page, page, dst_ids, 1, 0, n)
        oracle.swap(s, d, np.full(n, page, dtype=np.uint64))
    assert np.array_equal(dev.cpu().numpy(), ref)

    # store back into a second, canary-filled host plane at the original ids
    back = kvt.HostBuffer(2 * nb * page)
    bv = back.numpy(np.uint8, (2, nb, page))
    bv[:] = 0x5A
    t2b, t2 = _tables(2 * n)
    t2[0], t2[1], t2[2] = t[1], 0, page
    for p in range(2):
        kvt.kvt_sub_block_ptrs(back.dev + p * nb * page, page, page, src_ids, n, 1, 0,
                               t2[1, p * n:], n)
    kvt.kvt_swap_blocks(t2[0], t2[1], t2[2], 2 * n, kvt.D2H, mode)
    torch.cuda.synchronize()
    assert np.array_equal(bv[:, src_ids], hbytes[:, src_ids])
    rest = np.setdiff1d(np.arange(nb), src_ids)
    assert (bv[:, rest] == 0x5A).all()
    del hv, hbytes, bv
    host.free(); back.free(); tb.free(); t2b.free()


@pytest.mark.parametrize("mode", MODES, ids=lambda m: MODE_NAMES[m])
def test_swap_chunked_strided_layers_with_skip(gpu, mode):
    """The 32-layer geometry, fewer layers and blocks: host rows of 4 x 32 KiB pages + 4 KiB of
    padding (bpc = 4), HBM blocks of one page, a seeded skip on the first host chunk, the same
    id lists for every tensor; uniform random 16-bit payload; padding canaries untouched."""
    tensors, gpu_blocks, bpc, page, pad = 6, 512, 4, 32768, 4096
    host_rows = gpu_blocks // bpc
    stride = bpc * page + pad
    g = synth.rng(2, synth.P_SKIP)
    for trial in range(2):
        skip = int(g.integers(0, bpc))
        n = 300 + trial * 17
        n_chunks = kvt.kvt_chunks_consumed(n, skip, bpc)
        host = kvt.HostBuffer(tensors * host_rows * stride)
        hb = host.numpy(np.uint8, (tensors, host_rows, stride))
        synth.fill_random_bytes(synth.rng(2, synth.P_K, trial), hb)
        canary_pad = hb[:, :, bpc * page:].copy()
        dev = torch.full((tensors, gpu_blocks, page), 0x33, dtype=torch.uint8, device=gpu)
        chunks = synth.permutation(synth.rng(2, synth.P_PERM_SRC, trial), host_rows)[:n_chunks]
        gids = synth.permutation(synth.rng(2, synth.P_PERM_DST, trial), gpu_blocks)[:n]

        # load: host (chunked, skip) -> HBM (bpc 1)
        tb, t = _tables(tensors * n)
        for x in range(tensors):
            kvt.kvt_sub_block_ptrs(host.dev + x * host_rows * stride, stride, page, chunks,
                                   n_chunks, bpc, skip, t[0, x * n:], n)
            kvt.kvt_sub_block_ptrs(_dev_addr(dev) + x * gpu_blocks * page, page, page, gids, n,
                                   1, 0, t[1, x * n:], n)
        t[2] = page
        kvt.kvt_swap_blocks(t[0], t[1], t[2], tensors * n, kvt.H2D, mode)
        torch.cuda.synchronize()
        ref = np.full((tensors, gpu_blocks, page), 0x33, dtype=np.uint8)
        for x in range(tensors):
            s = oracle.sub_block_ptrs(hb[x].ctypes.data, stride, page, chunks, bpc, skip, n)
            d = oracle.sub_block_ptrs(ref[x].ctypes.data, page, page, gids, 1, 0, n)
            oracle.swap(s, d, np.full(n, page, dtype=np.uint64))
        assert np.array_equal(dev.cpu().numpy(), ref), f"load trial {trial} skip {skip}"

        # store: HBM -> the same host chunks after zeroing their pages (round trip identity)
        before = hb.copy()
        for x in range(tensors):
            for o in range(n):
                c, j = divmod(o + skip, bpc)
                hb[x, chunks[c], j * page:(j + 1) * page] = 0
        t[0], t[1] = t[1].copy(), t[0].copy()
        kvt.kvt_swap_blocks(t[0], t[1], t[2], tensors * n, kvt.D2H, mode)
        torch.cuda.synchronize()
        assert np.array_equal(hb, before), f"round trip trial {trial}"
        assert np.array_equal(hb[:, :, bpc * page:], canary_pad)
        del hb, before
        host.free(); tb.free()


@pytest.mark.parametrize("page,offset", [(512, 0), (2048, 0), (2048, 8), (8192, 0), (1000, 8),
                                         (16384, 0), (65536, 0)])
@pytest.mark.parametrize("mode", [kvt.COPY_KERNEL, kvt.COPY_SDMA, kvt.COPY_RUNTIME],
                         ids=lambda m: MODE_NAMES[m])
def test_swap_small_pages_scattered(gpu, page, offset, mode):
    """Many small pages in random scattered order host -> HBM, every page size the small-page
    sweep reports; offset 8 puts the host page bases at 8 mod 16 (the 8-byte path); page 1000
    is 8-byte aligned but not a multiple of 16.  65,536 pages up to 16 KiB (the workload's full
    count), 16,384 of 64 KiB (1 GiB).  The expected HBM image is the oracle's memcpy loop over
    its own pointer tables into a zero-filled host replica of the HBM buffer."""
    n = 65536 if page <= 16384 else 16384
    stride = page + offset
    host = kvt.HostBuffer(n * stride + 64)
    hb = host.numpy(np.uint8, None)[offset:offset + n * stride].reshape(n, stride)
    synth.fill_random_bytes(synth.rng(3, synth.P_K, page), hb)
    dev = torch.zeros((n, page), dtype=torch.uint8, device=gpu)
    src = synth.permutation(synth.rng(3, synth.P_PERM_SRC, page), n)
    dst = synth.permutation(synth.rng(3, synth.P_PERM_DST, page), n)
    tb, t = _tables(n)
    kvt.kvt_sub_block_ptrs(host.dev + offset, stride, page, src, n, 1, 0, t[0], n)
    kvt.kvt_sub_block_ptrs(_dev_addr(dev), page, page, dst, n, 1, 0, t[1], n)
    t[2] = page
    kvt.kvt_swap_blocks(t[0], t[1], t[2], n, kvt.H2D, mode)
    torch.cuda.synchronize()
    ref = np.zeros((n, page), dtype=np.uint8)
    s = oracle.sub_block_ptrs(hb.ctypes.data, stride, page, src, 1, 0, n)
    d = oracle.sub_block_ptrs(ref.ctypes.data, page, page, dst, 1, 0, n)
    oracle.swap(s, d, np.full(n, page, dtype=np.uint64))
    assert np.array_equal(dev.cpu().numpy(), ref)
    del hb, ref
    del dev
    host.free(); tb.free()
    torch.cuda.empty_cache()


def test_swap_zero_sizes_and_empty(gpu):
    host = kvt.HostBuffer(4096)
    dev = torch.full((4096,), 7, dtype=torch.uint8, device=gpu)
    tb, t = _tables(4)
    t[0] = [host.dev, host.dev + 16, host.dev + 32, host.dev + 48]
    t[1] = [dev.data_ptr(), dev.data_ptr() + 100, dev.data_ptr() + 200, dev.data_ptr() + 300]
    t[2] = 0
    for mode in MODES:
        kvt.kvt_swap_blocks(t[0], t[1], t[2], 4, kvt.H2D, mode)
        kvt.kvt_swap_blocks(t[0], t[1], t[2], 0, kvt.H2D, mode)
    torch.cuda.synchronize()
    assert (dev.cpu() == 7).all()
    with pytest.raises(kvt.KvtError) as e:
        t[2] = [8, 8, 12, 8]
        kvt.kvt_swap_blocks(t[0], t[1], t[2], 4, kvt.H2D, kvt.COPY_KERNEL)
    assert e.value.code == kvt.EALIGN
    host.free(); tb.free()


@pytest.mark.parametrize("mode", MODES, ids=lambda m: MODE_NAMES[m])
def test_stage_tail_q8_0_rows(gpu, mode):
    """Tail staging: rows [n_head, n_kv) of a q8_0 plane (1088-byte rows) into HBM."""
    kvh, hd, n_kv, n_head = 8, 128, 20000, 9413
    rows = synth.q8_0_rows(synth.rng(5, synth.P_K), n_kv, kvh, hd)
    row_bytes = rows.shape[1]
    host = kvt.HostBuffer(rows.nbytes)
    hp = host.numpy(np.uint8, rows.shape)
    hp[:] = rows
    staging = torch.full(((n_kv - n_head) * row_bytes + 64,), 0xCC, dtype=torch.uint8, device=gpu)
    kvt.kvt_stage_tail(host.dev, row_bytes, n_head, n_kv, staging, mode)
    torch.cuda.synchronize()
    ref = oracle.stage_tail(rows, row_bytes, n_head, n_kv)
    got = staging.cpu().numpy()
    assert np.array_equal(got[:ref.size], ref)
    assert (got[ref.size:] == 0xCC).all()
    del hp
    host.free()


def test_sdma_runs_of_adjacent_descriptors(gpu):
    """The engine path merges descriptors that continue the previous one on both sides into one
    copy; zero sizes inside a run neither end it nor move it.  Mixed runs, singles and zero
    sizes, in both directions: bit-exact against the oracle's memcpy loop."""
    page, nb = 4096, 96
    host = kvt.HostBuffer(nb * page)
    hb = host.numpy(np.uint8, (nb, page))
    synth.fill_random_bytes(synth.rng(3, synth.P_K, 77), hb)
    dev = torch.full((nb, page), 0x11, dtype=torch.uint8, device=gpu)
    # (src block, dst block, size): a run of 5, a zero inside a run of 3, singles, a run whose
    # source continues but destination does not, and partial sizes ending a run
    plan = [(0, 10, page), (1, 11, page), (2, 12, page), (3, 13, page), (4, 14, page),
            (20, 40, page), (21, 41, 0), (21, 41, page), (22, 42, page),
            (50, 5, page), (60, 7, 1000),
            (30, 70, page), (31, 80, page), (32, 81, 512)]
    n = len(plan)
    tb, t = _tables(n)
    for i, (sb, db, sz) in enumerate(plan):
        t[0, i] = host.dev + sb * page
        t[1, i] = dev.data_ptr() + db * page
        t[2, i] = sz
    kvt.kvt_swap_blocks(t[0], t[1], t[2], n, kvt.H2D, kvt.COPY_SDMA)
    torch.cuda.synchronize()
    ref = np.full((nb, page), 0x11, dtype=np.uint8)
    oracle.swap(np.array([hb.ctypes.data + sb * page for sb, _, _ in plan], np.uint64),
                np.array([ref.ctypes.data + db * page for _, db, _ in plan], np.uint64),
                np.array([sz for _, _, sz in plan], np.uint64))
    assert np.array_equal(dev.cpu().numpy(), ref)
    # the reverse direction into a canary plane
    back = kvt.HostBuffer(nb * page)
    bv = back.numpy(np.uint8, (nb, page))
    bv[:] = 0x22
    for i, (sb, db, sz) in enumerate(plan):
        t[0, i] = dev.data_ptr() + db * page
        t[1, i] = back.dev + sb * page
    kvt.kvt_swap_blocks(t[0], t[1], t[2], n, kvt.D2H, kvt.COPY_SDMA)
    torch.cuda.synchronize()
    want = np.full((nb, page), 0x22, dtype=np.uint8)
    oracle.swap(np.array([ref.ctypes.data + db * page for _, db, _ in plan], np.uint64),
                np.array([want.ctypes.data + sb * page for sb, _, _ in plan], np.uint64),
                np.array([sz for _, _, sz in plan], np.uint64))
    assert np.array_equal(bv, want)
    del hb, bv
    host.free(); back.free(); tb.free()


def test_sdma_is_ordered_on_the_stream(gpu):
    """Engine copies see the stream's earlier kernels and later kernels see the copies: a fill
    kernel writes the source, the SDMA store copies it to the host, an SDMA load brings it
    back, and a copy kernel reads the result, three times over on one stream.  (The mode
    drains the stream before its copies and returns after them.)"""
    n, page = 256, 8192
    src = torch.empty((n, page), dtype=torch.uint8, device=gpu)
    mid = kvt.HostBuffer(n * page)
    mv = mid.numpy(np.uint8, (n, page))
    mv[:] = 0
    dst = torch.zeros((n, page), dtype=torch.uint8, device=gpu)
    tb, t = _tables(n)
    tb2, t2 = _tables(n)
    perm = synth.permutation(synth.rng(3, synth.P_PERM_DST, 5), n)
    t[0] = [src.data_ptr() + i * page for i in range(n)]
    t[1] = [mid.dev + int(perm[i]) * page for i in range(n)]
    t[2] = page
    t2[0], t2[1], t2[2] = t[1], [dst.data_ptr() + i * page for i in range(n)], page
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for rep in range(3):
            src.fill_(rep + 1)
            src[:, :8] = torch.arange(n, dtype=torch.uint8, device=gpu)[:, None]
            kvt.kvt_swap_blocks(t[0], t[1], t[2], n, kvt.D2H, kvt.COPY_SDMA,
                                stream=s.cuda_stream)
            kvt.kvt_swap_blocks(t2[0], t2[1], t2[2], n, kvt.H2D, kvt.COPY_SDMA,
                                stream=s.cuda_stream)
            out = dst.clone()
    s.synchronize()
    want = np.full((n, page), 3, dtype=np.uint8)
    want[:, :8] = np.arange(n, dtype=np.uint8)[:, None]
    assert np.array_equal(out.cpu().numpy(), want)
    del mv
    mid.free(); tb.free(); tb2.free()


def test_sdma_refused_under_graph_capture(gpu):
    """The engine path waits on the host, so it refuses capture; the rest of the capture goes
    on as usual."""
    host = kvt.HostBuffer(1 << 16)
    dev = torch.zeros(1 << 16, dtype=torch.uint8, device=gpu)
    tb, t = _tables(1)
    t[0], t[1], t[2] = host.dev, dev.data_ptr(), 4096
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    code = None
    code_tail = None
    with torch.cuda.graph(g, stream=s):
        try:
            kvt.kvt_swap_blocks(t[0], t[1], t[2], 1, kvt.H2D, kvt.COPY_SDMA,
                                stream=s.cuda_stream)
        except kvt.KvtError as e:
            code = e.code
        try:   # the staging copy's SDMA mode is the same engine path
            kvt.kvt_stage_tail(host.dev, 4096, 0, 1, dev, kvt.COPY_SDMA, stream=s.cuda_stream)
        except kvt.KvtError as e:
            code_tail = e.code
        dev.add_(1)
    assert code == kvt.EUNSUPPORTED and code_tail == kvt.EUNSUPPORTED
    g.replay()
    torch.cuda.synchronize()
    assert (dev.cpu() == 1).all()
    del g
    host.free(); tb.free()


def test_swap_32_layers_full_geometry_sampled(gpu):
    """The 32-layer workload at full size in the launch configuration the bench times (kernel
    mode, 262,144 descriptors per direction): 64 tensors of 8192 HBM blocks; host rows of four
    32 KiB pages + 4 KiB pad (2048 rows per tensor, 16.5 GiB pinned); 4096 random blocks per
    tensor with a random skip on the first host chunk.  Every host page carries its own
    (tensor, row, page) stamp, so a copy from the wrong place cannot match.  The oracle builds
    its own pointer tables over the host planes, and its memcpy loop copies 3000 sampled
    descriptors' pages into a host array; the loaded HBM pages must equal them.  Unselected
    HBM blocks and pads stay untouched, and after the store the oracle's memcpy over the same
    tables reads back the original bytes (round trip)."""
    tensors, gblocks, bpc, page, pad, n = 64, 8192, 4, 32768, 4096, 4096
    hrows = gblocks // bpc
    stride = bpc * page + pad
    host = kvt.HostBuffer(tensors * hrows * stride)
    flat = host.numpy(np.uint8)
    block = np.empty(1 << 28, dtype=np.uint8)
    synth.fill_random_bytes(synth.rng(2, synth.P_K, 99), block)
    for o in range(0, flat.size, block.size):
        m = min(block.size, flat.size - o)
        flat[o:o + m] = block[:m]
    del block
    hb = flat.reshape(tensors, hrows, stride)
    stamps = (np.arange(tensors, dtype=np.uint64)[:, None, None] << np.uint64(40)) | \
             (np.arange(hrows, dtype=np.uint64)[None, :, None] << np.uint64(8)) | \
             np.arange(bpc, dtype=np.uint64)[None, None, :]
    hb.view(np.uint64)[:, :, [j * page // 8 for j in range(bpc)]] = stamps
    hbm = torch.full((tensors, gblocks, page), 0x33, dtype=torch.uint8, device=gpu)
    g = synth.rng(2, synth.P_SKIP, 99)
    skip = int(g.integers(0, bpc))
    nch = kvt.kvt_chunks_consumed(n, skip, bpc)
    chunks = synth.permutation(synth.rng(2, synth.P_PERM_SRC, 99), hrows)[:nch]
    gids = synth.permutation(synth.rng(2, synth.P_PERM_DST, 99), gblocks)[:n]
    tb, t = _tables(tensors * n)
    for x in range(tensors):
        kvt.kvt_sub_block_ptrs(host.dev + x * hrows * stride, stride, page, chunks, nch, bpc, skip,
                               t[0, x * n:], n)
        kvt.kvt_sub_block_ptrs(hbm.data_ptr() + x * gblocks * page, page, page, gids, n, 1, 0,
                               t[1, x * n:], n)
    t[2] = page
    kvt.kvt_swap_blocks(t[0], t[1], t[2], tensors * n, kvt.H2D, kvt.COPY_KERNEL)
    torch.cuda.synchronize()

    pick = synth.rng(2, synth.P_MISC, 99).choice(tensors * n, size=3000, replace=False)
    xs, os_ = pick // n, pick % n
    rows = chunks[(os_ + skip) // bpc]
    # the oracle's tables over the host planes, and its memcpy of the sampled descriptors
    osrc = np.concatenate([oracle.sub_block_ptrs(hb[x].ctypes.data, stride, page, chunks, bpc,
                                                 skip, n) for x in range(tensors)])
    sizes = np.full(pick.size, page, dtype=np.uint64)

    def oracle_read(out):
        oracle.swap(osrc[pick], out.ctypes.data + np.arange(pick.size, dtype=np.uint64) * page,
                    sizes)
        return out

    want = oracle_read(np.empty((pick.size, page), dtype=np.uint8))
    got = hbm[torch.from_numpy(xs).to(gpu), torch.from_numpy(gids[os_]).to(gpu)].cpu().numpy()
    assert np.array_equal(got, want), "loaded pages differ from their host pages"
    rest = np.setdiff1d(np.arange(gblocks), gids)
    xr = synth.rng(2, synth.P_MISC, 98).integers(0, tensors, 500)
    br = rest[synth.rng(2, synth.P_MISC, 97).integers(0, rest.size, 500)]
    assert (hbm[torch.from_numpy(xr).to(gpu), torch.from_numpy(br).to(gpu)] == 0x33).all()

    # store: zero the selected host pages, copy HBM back, compare with the original bytes
    pads = np.stack([hb[x, r, bpc * page:] for x, r in zip(xs, rows)])
    sel_rows = chunks[(np.arange(n) + skip) // bpc]
    sel_js = (np.arange(n) + skip) % bpc
    for x in range(tensors):
        for j in range(bpc):
            hb[x, sel_rows[sel_js == j], j * page:(j + 1) * page] = 0
    t[0], t[1] = t[1].copy(), t[0].copy()
    kvt.kvt_swap_blocks(t[0], t[1], t[2], tensors * n, kvt.D2H, kvt.COPY_KERNEL)
    torch.cuda.synchronize()
    back = oracle_read(np.zeros((pick.size, page), dtype=np.uint8))
    assert np.array_equal(back, want), "round trip changed sampled pages"
    assert np.array_equal(np.stack([hb[x, r, bpc * page:] for x, r in zip(xs, rows)]), pads)
    del hb, flat, got, want, back
    del hbm
    host.free(); tb.free()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", [kvt.COPY_KERNEL, kvt.COPY_AUTO], ids=lambda m: MODE_NAMES[m])
def test_swap_pages_up_to_512_bytes_mixed(gpu, mode):
    """Small pages of mixed sizes (0 to 512 bytes) in one batch, an odd count of descriptors (the
    last group of eight is partial), host pages 16-byte and only 8-byte aligned, in both
    directions; bit-exact against the oracle's memcpy loop, canaries elsewhere untouched."""
    n, slot = 1001, 528
    g = synth.rng(3, synth.P_MISC, 512)
    sizes = g.choice(np.array([0, 8, 64, 200, 504, 512], np.uint64), size=n)
    offs = g.choice(np.array([0, 8], np.int64), size=n)   # 16- or only 8-byte aligned bases
    host = kvt.HostBuffer(n * slot + 64)
    hb = host.numpy(np.uint8)
    synth.fill_random_bytes(synth.rng(3, synth.P_K, 512), hb)
    dev = torch.full((n * slot,), 0x5C, dtype=torch.uint8, device=gpu)
    src_slot = synth.permutation(synth.rng(3, synth.P_PERM_SRC, 512), n)
    dst_slot = synth.permutation(synth.rng(3, synth.P_PERM_DST, 512), n)
    tb, t = _tables(n)
    t[0] = [host.dev + int(src_slot[i]) * slot + int(offs[i]) for i in range(n)]
    t[1] = [dev.data_ptr() + int(dst_slot[i]) * slot for i in range(n)]
    t[2] = sizes
    kvt.kvt_swap_blocks(t[0], t[1], t[2], n, kvt.H2D, mode)
    torch.cuda.synchronize()
    ref = np.full(n * slot, 0x5C, dtype=np.uint8)
    oracle.swap(np.array([hb.ctypes.data + int(src_slot[i]) * slot + int(offs[i])
                          for i in range(n)], np.uint64),
                np.array([ref.ctypes.data + int(dst_slot[i]) * slot for i in range(n)], np.uint64),
                sizes)
    assert np.array_equal(dev.cpu().numpy(), ref)
    # back to a canary-filled host buffer at the source slots, 8 bytes past the slot start
    back = kvt.HostBuffer(n * slot + 64)
    bb = back.numpy(np.uint8)
    bb[:] = 0xA7
    t[0], t[1] = t[1].copy(), [back.dev + int(src_slot[i]) * slot + 8 for i in range(n)]
    kvt.kvt_swap_blocks(t[0], t[1], t[2], n, kvt.D2H, mode)
    torch.cuda.synchronize()
    want = np.full(n * slot + 64, 0xA7, dtype=np.uint8)
    oracle.swap(np.array([ref.ctypes.data + int(dst_slot[i]) * slot for i in range(n)], np.uint64),
                np.array([want.ctypes.data + int(src_slot[i]) * slot + 8 for i in range(n)],
                         np.uint64), sizes)
    assert np.array_equal(bb, want)
    del hb, bb
    host.free(); back.free(); tb.free()


def test_sdma_long_ranges_cut_over_engines(gpu):
    """Ranges longer than 4 MiB go as 4 MiB pieces spread over the engines: one 37 MiB + 13 byte
    range, a 5 MiB run of two adjacent descriptors and a short odd-sized one, loaded and stored
    back, bit-exact against the oracle's memcpy loop."""
    assert kvt.kvt_copy_engines(kvt.H2D) >= 1 and kvt.kvt_copy_engines(kvt.D2H) >= 1
    sizes = [(37 << 20) + 13, 3 << 20, 2 << 20, 777]
    total = 48 << 20
    host = kvt.HostBuffer(total)
    hb = host.numpy(np.uint8, (total,))
    synth.fill_random_bytes(synth.rng(3, synth.P_K, 78), hb)
    dev = torch.full((total,), 0x5A, dtype=torch.uint8, device=gpu)
    base = dev.data_ptr()
    src = np.array([0, 40 << 20, (40 << 20) + (3 << 20), 46 << 20], np.uint64)
    dst = np.array([1 << 20, (39 << 20) + 64, (42 << 20) + 64, 45 << 20], np.uint64)
    for a in (src, dst):   # in bounds, pairwise disjoint
        end = a + np.array(sizes, np.uint64)
        assert (end <= total).all()
        o = np.argsort(a)
        assert (a[o][1:] >= end[o][:-1]).all()
    tabs = kvt.HostBuffer(3 * 4 * 8)
    t = tabs.numpy(np.uint64, (3, 4))
    t[0], t[1], t[2] = src + np.uint64(host.dev), dst + np.uint64(base), sizes
    kvt.kvt_swap_blocks(t[0], t[1], t[2], 4, kvt.H2D, kvt.COPY_SDMA)
    torch.cuda.synchronize()
    ref = np.full(total, 0x5A, np.uint8)
    oracle.swap(src + np.uint64(hb.ctypes.data), dst + np.uint64(ref.ctypes.data),
                np.array(sizes, np.uint64))
    assert np.array_equal(dev.cpu().numpy(), ref)
    # and back: the device bytes into a cleared host buffer
    hb[:] = 0
    t[0], t[1] = dst + np.uint64(base), src + np.uint64(host.dev)
    kvt.kvt_swap_blocks(t[0], t[1], t[2], 4, kvt.D2H, kvt.COPY_SDMA)
    torch.cuda.synchronize()
    back = np.zeros(total, np.uint8)
    oracle.swap(dst + np.uint64(ref.ctypes.data), src + np.uint64(back.ctypes.data),
                np.array(sizes, np.uint64))
    assert np.array_equal(hb, back)
    del hb, t
    tabs.free()
    host.free()


def test_sdma_from_two_threads_at_once(gpu):
    """Two host threads drive the engine mode at the same time, each on its own stream with its
    own tables and buffers (every engine carries copies of both): each result is bit-exact
    against the oracle's memcpy loop."""
    import threading
    page, n = 16384, 2048
    jobs = []
    for j in range(2):
        host = kvt.HostBuffer(n * page)
        hb = host.numpy(np.uint8, (n, page))
        synth.fill_random_bytes(synth.rng(3, synth.P_K, 90 + j), hb)
        dev = torch.zeros((n, page), dtype=torch.uint8, device=gpu)
        src = synth.permutation(synth.rng(3, synth.P_PERM_SRC, 90 + j), n)
        dst = synth.permutation(synth.rng(3, synth.P_PERM_DST, 90 + j), n)
        tb, t = _tables(n)
        kvt.kvt_sub_block_ptrs(host.dev, page, page, src, n, 1, 0, t[0], n)
        kvt.kvt_sub_block_ptrs(_dev_addr(dev), page, page, dst, n, 1, 0, t[1], n)
        t[2] = page
        jobs.append(dict(host=host, hb=hb, dev=dev, src=src, dst=dst, tb=tb, t=t,
                         stream=torch.cuda.Stream(), err=None))

    def run(job):
        try:
            for _ in range(3):
                kvt.kvt_swap_blocks(job["t"][0], job["t"][1], job["t"][2], n, kvt.H2D,
                                    kvt.COPY_SDMA, stream=job["stream"])
        except Exception as e:   # reported by the main thread
            job["err"] = e

    threads = [threading.Thread(target=run, args=(j,)) for j in jobs]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    for job in jobs:
        assert job["err"] is None, job["err"]
        ref = np.zeros((n, page), dtype=np.uint8)
        s = oracle.sub_block_ptrs(job["hb"].ctypes.data, page, page, job["src"], 1, 0, n)
        d = oracle.sub_block_ptrs(ref.ctypes.data, page, page, job["dst"], 1, 0, n)
        oracle.swap(s, d, np.full(n, page, dtype=np.uint64))
        assert np.array_equal(job["dev"].cpu().numpy(), ref)
    for job in jobs:
        del job["hb"], job["t"]
        job["host"].free()
        job["tb"].free()
