"""GPU checks of the transfer worker (kvt_worker_*) and of graph capture of the staging path.

Worker: copies are bit-exact against the oracle's memcpy loop; the caller's tables are free
once submit returns; jobs of one worker run and complete in submission order; a store waits
for the compute stream's writes; reported bytes and event times are consistent; destroy
drains pending jobs.

Graphs: the tail staging copy (copy engine and kernel forms) followed by prefill attention,
and the whole decode step (score + top-k, fused gather + attention), are captured into a HIP
graph and replayed several times, with eager work and new host data between replays; every
replay must equal the eager result bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
from hbm_kv_cache_amd import kvt, synth

pytestmark = pytest.mark.gpu

PAGE = 16 * 8 * 128 * 2     # one block of 16 tokens x 8 heads x 128 dims, fp16


def _plane(nb, seed):
    host = kvt.HostBuffer(nb * PAGE)
    hv = host.numpy(np.uint8, (nb, PAGE))
    synth.fill_random_bytes(synth.rng(9, synth.P_K, seed), hv)
    return host, hv


def _load_tables(host, dev, src_ids, dst_ids):
    n = len(src_ids)
    src = np.empty(n, np.uint64)
    dst = np.empty(n, np.uint64)
    kvt.kvt_sub_block_ptrs(host.dev, PAGE, PAGE, src_ids, n, 1, 0, src, n)
    kvt.kvt_sub_block_ptrs(dev.data_ptr(), PAGE, PAGE, dst_ids, n, 1, 0, dst, n)
    return src, dst, np.full(n, PAGE, np.uint64)


@pytest.mark.parametrize("mode", [kvt.COPY_AUTO, kvt.COPY_RUNTIME], ids=["auto", "runtime"])
def test_worker_jobs_bit_exact_in_order_and_timed(gpu, mode):
    nb, per_job, jobs = 512, 48, 6
    host, hv = _plane(nb, 1)
    dev = torch.full((nb, PAGE), 0x3C, dtype=torch.uint8, device=gpu)
    src_all = synth.permutation(synth.rng(9, synth.P_PERM_SRC), nb)
    dst_all = synth.permutation(synth.rng(9, synth.P_PERM_DST), nb)
    w = kvt.kvt_worker_create(kvt.H2D, mode)
    try:
        for j in range(jobs):
            s_ids = src_all[j * per_job:(j + 1) * per_job]
            d_ids = dst_all[j * per_job:(j + 1) * per_job]
            src, dst, sizes = _load_tables(host, dev, s_ids, d_ids)
            kvt.kvt_worker_submit(w, 100 + j, src, dst, sizes, per_job)
            src[:] = 0       # the worker copied the tables: clobbering them changes nothing
            dst[:] = 0
            sizes[:] = 1
        assert 0 < kvt.kvt_worker_pending(w) <= jobs
        kvt.kvt_worker_wait(w, {100 + j for j in range(jobs)} | {7})   # 7: unknown, skipped
        done = kvt.kvt_worker_get_finished(w)
        assert [d[0] for d in done] == [100 + j for j in range(jobs)]
        assert all(d[1] == per_job * PAGE for d in done)
        assert all(0 < d[2] < 1.0 for d in done)
        assert kvt.kvt_worker_pending(w) == 0
        assert kvt.kvt_worker_get_finished(w) == []
    finally:
        kvt.kvt_worker_destroy(w)
    ref = np.full((nb, PAGE), 0x3C, np.uint8)
    n = jobs * per_job
    s = oracle.sub_block_ptrs(hv.ctypes.data, PAGE, PAGE, src_all[:n], 1, 0, n)
    d = oracle.sub_block_ptrs(ref.ctypes.data, PAGE, PAGE, dst_all[:n], 1, 0, n)
    oracle.swap(s, d, np.full(n, PAGE, dtype=np.uint64))
    assert np.array_equal(dev.cpu().numpy(), ref)
    del hv
    host.free()


def test_worker_later_job_runs_after_earlier_one(gpu):
    """Jobs 2k and 2k+1 write the same HBM slots from different host blocks: the slot must end
    with the later job's bytes, which holds only if the worker keeps submission order."""
    nb, n = 256, 32
    host, hv = _plane(nb, 2)
    dev = torch.zeros((n, PAGE), dtype=torch.uint8, device=gpu)
    w = kvt.kvt_worker_create(kvt.H2D, kvt.COPY_KERNEL)
    try:
        kvt.kvt_worker_reserve(w, 8, n)
        last = None
        for j in range(8):
            s_ids = np.arange(j * n, (j + 1) * n, dtype=np.int64)
            src, dst, sizes = _load_tables(host, dev, s_ids, np.arange(n, dtype=np.int64))
            kvt.kvt_worker_submit(w, j, src, dst, sizes, n)
            last = s_ids
        kvt.kvt_worker_wait(w, 7)
        assert [d[0] for d in kvt.kvt_worker_get_finished(w, 3)] == [0, 1, 2]
        assert [d[0] for d in kvt.kvt_worker_get_finished(w)] == [3, 4, 5, 6, 7]
    finally:
        kvt.kvt_worker_destroy(w)
    assert np.array_equal(dev.cpu().numpy(), hv[last])
    del hv
    host.free()


def test_worker_store_waits_for_compute_stream(gpu):
    """A store submitted right after compute-stream work that writes its source must copy the
    written values (the worker's stream waits for the compute stream at submit)."""
    nb = 128
    dev = torch.zeros((nb, PAGE // 4), dtype=torch.int32, device=gpu)
    back = kvt.HostBuffer(nb * PAGE)
    bv = back.numpy(np.int32, (nb, PAGE // 4))
    bv[:] = -1
    w = kvt.kvt_worker_create(kvt.D2H, kvt.COPY_AUTO)
    try:
        a = torch.randn(4096, 4096, device=gpu)
        for j in range(4):
            a = a @ a * (1 / 64)                    # keeps the compute stream busy a while
            dev.add_(j + 1)
            ids = np.arange(nb, dtype=np.int64)
            src = np.empty(nb, np.uint64)
            dst = np.empty(nb, np.uint64)
            kvt.kvt_sub_block_ptrs(dev.data_ptr(), PAGE, PAGE, ids, nb, 1, 0, src, nb)
            kvt.kvt_sub_block_ptrs(back.dev, PAGE, PAGE, ids, nb, 1, 0, dst, nb)
            kvt.kvt_worker_submit(w, j, src, dst, np.full(nb, PAGE, np.uint64), nb,
                                  torch.cuda.current_stream())
            kvt.kvt_worker_wait(w, j)
            expect = (j + 1) * (j + 2) // 2
            assert (bv == expect).all(), f"store {j}: host holds {np.unique(bv)[:4]}"
        kvt.kvt_worker_get_finished(w)
    finally:
        kvt.kvt_worker_destroy(w)
    del bv
    back.free()


def test_worker_errors_and_destroy_drains(gpu):
    nb, n = 64, 16
    host, hv = _plane(nb, 3)
    dev = torch.zeros((nb, PAGE), dtype=torch.uint8, device=gpu)
    w = kvt.kvt_worker_create(kvt.H2D)
    src, dst, sizes = _load_tables(host, dev, np.arange(n, dtype=np.int64),
                                   np.arange(n, dtype=np.int64))
    kvt.kvt_worker_submit(w, 5, src, dst, sizes, n)
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_worker_submit(w, 5, src, dst, sizes, n)     # job 5 is still pending
    assert e.value.code == kvt.EINVAL
    bad = sizes.copy()
    bad[3] = 12
    w2 = kvt.kvt_worker_create(kvt.H2D, kvt.COPY_KERNEL)
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_worker_submit(w2, 1, src, dst, bad, n)      # kernel path needs sizes % 8 == 0
    assert e.value.code == kvt.EALIGN
    assert kvt.kvt_worker_pending(w2) == 0
    kvt.kvt_worker_submit(w2, 2, src, dst, sizes, 0)        # empty job: ordering only
    kvt.kvt_worker_wait(w2, 2)
    assert kvt.kvt_worker_get_finished(w2) == [(2, 0, pytest.approx(0.0, abs=1e-3))]
    kvt.kvt_worker_wait(w2, 999)                            # unknown job: returns at once
    kvt.kvt_worker_destroy(w2)
    kvt.kvt_worker_submit(w, 6, src[::-1].copy(), dst, sizes, n)
    kvt.kvt_worker_destroy(w)                               # shutdown with jobs pending
    assert np.array_equal(dev[:n].cpu().numpy(), hv[:n][::-1])
    del hv
    host.free()


@pytest.mark.parametrize("mode", [kvt.COPY_RUNTIME, kvt.COPY_KERNEL], ids=["runtime", "kernel"])
def test_graph_staging_then_prefill_replays(gpu, mode):
    """Tail staging (K and V) + prefill attention captured once, replayed three times with the
    host tail rewritten and eager work in between: each replay equals an eager run.  The
    runtime mode is one hipMemcpyAsync, which the runtime runs on a copy engine at this size;
    the library-driven engine mode waits on the host and refuses capture."""
    n_kv, n_head, n_q, n_qh, kvh = 3000, 1100, 64, 16, 4
    k = synth.q8_0_rows(synth.rng(9, synth.P_K, 50), n_kv, kvh, 128)
    v = synth.q8_0_rows(synth.rng(9, synth.P_V, 50), n_kv, kvh, 128)
    rb = k.shape[1]
    q = torch.from_numpy(synth.f16_normal(synth.rng(9, synth.P_Q, 50),
                                          (n_q, n_qh, 128)).view(np.int16)).to(gpu)
    host = kvt.HostBuffer(2 * n_kv * rb)
    hk = host.numpy(np.uint8, (2, n_kv, rb))
    hk[0], hk[1] = k, v
    kd = torch.from_numpy(k[:n_head].copy()).to(gpu)
    vd = torch.from_numpy(v[:n_head].copy()).to(gpu)
    stage = torch.zeros((2, n_kv - n_head, rb), dtype=torch.uint8, device=gpu)
    out = torch.zeros((n_q, n_qh, 128), dtype=torch.float32, device=gpu)
    scale = 1 / math.sqrt(128)

    def step():
        kvt.kvt_stage_tail(host.dev, rb, n_head, n_kv, stage[0], mode)
        kvt.kvt_stage_tail(host.dev + n_kv * rb, rb, n_head, n_kv, stage[1], mode)
        kvt.kvt_attn_prefill(q, n_q, n_kv - n_q, n_qh, kvh, 128, kd, vd, n_head, stage[0],
                             stage[1], n_kv, kvt.Q8_0, 1, scale, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        tail = synth.q8_0_rows(synth.rng(9, synth.P_K, 60 + r), n_kv - n_head, kvh, 128)
        hk[0, n_head:] = tail
        hk[1, n_head:] = tail[::-1]
        noise = torch.randn(1 << 20, device=gpu)
        scratch = noise.sum()                    # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got_out, got_stage = out.clone(), stage.clone()
        out.zero_()
        stage.zero_()
        step()                                   # eager on the same data
        torch.cuda.synchronize()
        assert torch.equal(got_stage[0].cpu(), torch.from_numpy(hk[0, n_head:].copy()))
        assert torch.equal(got_stage, stage), f"replay {r}: staged rows differ"
        assert torch.equal(got_out, out), f"replay {r}: attention differs"
        assert torch.equal(scratch, noise.sum()), f"replay {r}: eager work was disturbed"
    del g, hk
    torch.cuda.synchronize()
    host.free()


def test_graph_decode_step_replays(gpu):
    """The decode step (pooled scoring + top-k, fused gather + attention) captured once and
    replayed with new queries between replays: ids, gathered rows and outputs equal eager."""
    ctx, kvh, hd, bt, k, n_qh = 64 * 1024, 8, 128, 64, 32, 64
    n_blocks = ctx // bt
    row = kvh * hd * 2
    host = kvt.HostBuffer(2 * ctx * row)
    planes = host.numpy(np.uint16, (2, ctx, kvh, hd))
    planes[0] = synth.bf16_normal(synth.rng(9, synth.P_K, 70), (ctx, kvh, hd))
    planes[1] = synth.bf16_normal(synth.rng(9, synth.P_V, 70), (ctx, kvh, hd))
    pooled = torch.from_numpy(synth.f16_normal(synth.rng(9, synth.P_POOLED, 70),
                                               (n_blocks, 128)).view(np.int16)).to(gpu)
    q_idx = torch.zeros((kvh, 128), dtype=torch.int16, device=gpu)
    q = torch.zeros((n_qh, hd), dtype=torch.int16, device=gpu)
    ws_t = kvt.kvt_index_topk_ws_bytes(n_blocks, kvh, k)
    ws_d = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, k * bt)
    wt = torch.empty(ws_t, dtype=torch.uint8, device=gpu)
    wd = torch.empty(ws_d, dtype=torch.uint8, device=gpu)
    ids = torch.zeros((kvh, k), dtype=torch.int32, device=gpu)
    kv = torch.zeros((2, kvh, k * bt, hd), dtype=torch.int16, device=gpu)
    out = torch.zeros((n_qh, hd), dtype=torch.float32, device=gpu)
    strides = (bt * row, hd * 2, row)     # host planes [token][head][dim]

    def step():
        kvt.kvt_index_topk(pooled, n_blocks, 128, q_idx, kvh, k, ids, None, wt, ws_t)
        kvt.kvt_gather_attn_decode(q, n_qh, kvh, hd, kvt.BF16, host.dev, host.dev + ctx * row,
                                   n_blocks, *strides, None, bt, ids, k, kv[0], kv[1],
                                   1 / math.sqrt(hd), out, wd, ws_d)

    def new_queries(r):
        q_idx.copy_(torch.from_numpy(synth.f16_normal(synth.rng(9, synth.P_QIDX, 80 + r),
                                                      (kvh, 128)).view(np.int16)))
        q.copy_(torch.from_numpy(synth.bf16_normal(synth.rng(9, synth.P_Q, 80 + r),
                                                   (n_qh, hd)).view(np.int16)))

    new_queries(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    prev = None
    for r in range(1, 4):
        new_queries(r)
        g.replay()
        torch.cuda.synchronize()
        got = (ids.clone(), kv.clone(), out.clone())
        ids.zero_(); kv.zero_(); out.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], ids), f"replay {r}: ids differ"
        assert torch.equal(got[1], kv), f"replay {r}: gathered rows differ"
        assert torch.equal(got[2], out), f"replay {r}: attention differs"
        if prev is not None:
            assert not torch.equal(prev, got[0]), "new queries should select new blocks"
        prev = got[0]
    del g, planes
    torch.cuda.synchronize()
    host.free()


def test_worker_concurrent_submitters(gpu):
    """Two host threads submit to one worker at once (the calls release the GIL): every job is
    reported exactly once, oldest first in the worker's own order, and every page arrives."""
    import threading
    nb, per_job, jobs_per_thread = 256, 16, 8
    host, hv = _plane(nb, 4)
    dev = torch.zeros((nb, PAGE), dtype=torch.uint8, device=gpu)
    w = kvt.kvt_worker_create(kvt.H2D, kvt.COPY_AUTO)
    errors = []

    def submitter(t):
        try:
            for j in range(jobs_per_thread):
                base = (t * jobs_per_thread + j) * per_job
                ids = np.arange(base, base + per_job, dtype=np.int64)
                src, dst, sizes = _load_tables(host, dev, ids, ids)
                kvt.kvt_worker_submit(w, 1000 * t + j, src, dst, sizes, per_job)
        except Exception as e:   # reported below
            errors.append(e)

    threads = [threading.Thread(target=submitter, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    try:
        assert not errors, errors
        want = {1000 * t + j for t in range(2) for j in range(jobs_per_thread)}
        kvt.kvt_worker_wait(w, want)
        done = kvt.kvt_worker_get_finished(w, 64)
        got = [d[0] for d in done]
        assert sorted(got) == sorted(want) and len(got) == len(want)
        for t in range(2):   # each thread's jobs keep their own submission order
            mine = [x for x in got if x // 1000 == t]
            assert mine == sorted(mine)
        assert kvt.kvt_worker_pending(w) == 0
    finally:
        kvt.kvt_worker_destroy(w)
    assert np.array_equal(dev.cpu().numpy(), hv)
    del hv
    host.free()
