"""GPU parity of the top-k decode path: index scoring + top-k (bit-exact ids and fp64 scores),
the host -> HBM gather (bit-exact), decode attention (<= 2e-3 max-abs vs the fp64 oracle), and
one whole decode step at the 262,144-token geometry."""
import math

import numpy as np
import pytest
import torch

import oracle
from hbm_kv_cache_amd import kvt, synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _u16(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)


def _run_topk(pooled, q_idx, k, dev, want_scores=True):
    n_blocks, dim = pooled.shape
    n_sel = q_idx.shape[0]
    ws_bytes = kvt.kvt_index_topk_ws_bytes(n_blocks, n_sel, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ids = torch.full((n_sel, k), -7, dtype=torch.int32, device=dev)
    scores = torch.empty((n_sel, max(n_blocks, 1)), dtype=torch.float64, device=dev)
    pd = _u16(pooled, dev) if n_blocks else torch.empty(8, dtype=torch.int16, device=dev)
    kvt.kvt_index_topk(pd, n_blocks, dim, _u16(q_idx, dev), n_sel, k, ids,
                       scores if want_scores else None, ws, ws_bytes)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), scores.cpu().numpy()[:, :n_blocks]


@pytest.mark.parametrize("n_blocks,k", [(4096, 32), (16384, 32), (5000, 32), (129, 32), (100, 32),
                                        (1, 32), (32, 32), (70000, 32), (3000, 200), (5, 1),
                                        (65536, 512), (70000, 1000), (5000, 2048), (300, 512),
                                        (65535, 2048), (20000, 1024)])
def test_index_topk_bit_exact(gpu, n_blocks, k):
    g = synth.rng(4, synth.P_POOLED, n_blocks + k)
    pooled = synth.f16_normal(g, (n_blocks, 128))
    q_idx = synth.f16_normal(synth.rng(4, synth.P_QIDX, n_blocks), (8, 128))
    ids, scores = _run_topk(pooled, q_idx, k, gpu)
    ref_scores = oracle.index_scores(pooled, q_idx)
    assert np.array_equal(scores, ref_scores)        # fp64, index order: identical values
    assert np.array_equal(ids, oracle.topk(ref_scores, k))


@pytest.mark.parametrize("dim,n_sel,n_blocks,k", [(8, 5, 300, 32), (64, 32, 1000, 32),
                                                   (136, 7, 257, 32), (256, 3, 2000, 32),
                                                   (256, 5, 3000, 100), (136, 1, 129, 7)])
def test_index_topk_other_dims_and_head_counts(gpu, dim, n_sel, n_blocks, k):
    """Row widths that take one, a partial or two 128-element register batches of the scoring
    chain; head counts that leave a scoring workgroup's second head empty; both selection
    paths."""
    g = synth.rng(4, synth.P_POOLED, 1000 * dim + n_sel)
    pooled = synth.f16_normal(g, (n_blocks, dim))
    q_idx = synth.f16_normal(synth.rng(4, synth.P_QIDX, dim), (n_sel, dim))
    ids, scores = _run_topk(pooled, q_idx, k, gpu)
    ref_scores = oracle.index_scores(pooled, q_idx)
    assert np.array_equal(scores, ref_scores)
    assert np.array_equal(ids, oracle.topk(ref_scores, k))


def test_index_topk_ties_nans_and_duplicates(gpu):
    g = synth.rng(4, synth.P_MISC, 1)
    n_blocks = 3000
    pooled = synth.f16_normal(g, (n_blocks, 128))
    pooled[1000:1100] = pooled[7]                    # 101 identical keys -> exact score ties
    pooled[2000:2010, 3] = 0x7E00                    # NaN in the key -> NaN scores
    q_idx = synth.f16_normal(g, (8, 128))
    q_idx[5] = 0                                     # every score 0 for head 5 (ties everywhere)
    q_idx[6] = 0x8000                                # -0.0: products are signed zeros
    ids, scores = _run_topk(pooled, q_idx, 32, gpu)
    ref = oracle.index_scores(pooled, q_idx)
    same = (scores == ref) | (np.isnan(scores) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(ids, oracle.topk(ref, 32))
    assert ids[5].tolist() == list(range(32))        # all ties: lowest ids
    assert ids[6].tolist() == list(range(32))


@pytest.mark.parametrize("k", [100, 700])
def test_index_topk_selection_path_ties_nans_and_small_inputs(gpu, k):
    """k > 32 (the selection path): exact ties, NaN scores, signed zeros; fewer blocks than k;
    no blocks at all."""
    g = synth.rng(4, synth.P_MISC, 60 + k)
    n_blocks = 9000
    pooled = synth.f16_normal(g, (n_blocks, 128))
    pooled[1000:1900] = pooled[7]                    # 901 identical keys -> exact score ties
    pooled[2000:2010, 3] = 0x7E00                    # NaN scores
    q_idx = synth.f16_normal(g, (8, 128))
    q_idx[5] = 0                                     # every score 0 for head 5
    q_idx[6] = 0x8000                                # -0.0
    ids, scores = _run_topk(pooled, q_idx, k, gpu)
    ref = oracle.index_scores(pooled, q_idx)
    assert np.array_equal(ids, oracle.topk(ref, k))
    assert ids[5].tolist() == list(range(k))
    for nb in (0, 7, k - 1, k):
        pl = pooled[:nb] if nb else np.zeros((0, 128), np.uint16)
        ids, _ = _run_topk(pl, q_idx, k, gpu, want_scores=False)
        assert np.array_equal(ids, oracle.topk(oracle.index_scores(pl, q_idx), k)), nb


def test_index_topk_empty_and_oversized_k(gpu):
    ids, _ = _run_topk(np.zeros((0, 128), np.uint16), np.zeros((8, 128), np.uint16), 16, gpu,
                       want_scores=False)
    assert (ids == -1).all()
    pooled = synth.f16_normal(synth.rng(4, synth.P_MISC, 2), (7, 128))
    q_idx = synth.f16_normal(synth.rng(4, synth.P_MISC, 3), (3, 128))
    ids, _ = _run_topk(pooled, q_idx, 20, gpu)
    ref = oracle.topk(oracle.index_scores(pooled, q_idx), 20)
    assert np.array_equal(ids, ref)
    assert (ids[:, 7:] == -1).all()


def _host_planes(n_tok, kvh, hd, cfg, step=0):
    """Pinned K and V planes [n_tok][kvh][hd] bf16 N(0,1)."""
    row = kvh * hd * 2
    buf = kvt.HostBuffer(2 * n_tok * row)
    planes = buf.numpy(np.uint16, (2, n_tok, kvh, hd))
    step_rows = 1 << 16
    for p, purpose in enumerate((synth.P_K, synth.P_V)):
        g = synth.rng(cfg, purpose, step)
        for t0 in range(0, n_tok, step_rows):
            t1 = min(n_tok, t0 + step_rows)
            planes[p, t0:t1] = synth.bf16_normal(g, (t1 - t0, kvh, hd))
    return buf, planes


LAYOUTS = {"token_major": oracle.token_major_strides,
           "block_head_major": oracle.block_head_major_strides}


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_gather_blocks_bit_exact_with_table_and_negative_ids(gpu, layout):
    n_tok, kvh, hd, bt, k = 64 * 300, 8, 128, 64, 32
    buf, planes = _host_planes(n_tok, kvh, hd, 4, 11)
    n_blocks = n_tok // bt
    strides = LAYOUTS[layout](kvh, hd, 2, bt)
    g = synth.rng(4, synth.P_MISC, 12)
    ids = np.stack([np.sort(g.permutation(n_blocks)[:k]) for _ in range(kvh)]).astype(np.int32)
    ids[3, 20:] = -1
    ids[4, 31] = n_blocks + 5                        # outside the planes: skipped
    table = g.permutation(n_blocks).astype(np.int32)
    for tab in (None, table):
        out = torch.full((2, kvh, k * bt, hd), 0x1234, dtype=torch.int16, device=gpu)
        kvt.kvt_gather_blocks(buf.dev, buf.dev + n_tok * kvh * hd * 2, n_blocks, kvh, hd, 2,
                              *strides, None if tab is None else torch.from_numpy(tab).to(gpu),
                              bt, torch.from_numpy(ids).to(gpu), k, out[0], out[1])
        torch.cuda.synchronize()
        ids_o = ids.copy()
        ids_o[4, 31] = -1
        canary = np.full((kvh, k * bt, hd * 2), 0, dtype=np.uint8)
        canary.view(np.uint16)[:] = 0x1234
        ko, vo = oracle.gather(planes[0].view(np.uint8), planes[1].view(np.uint8), n_blocks, kvh,
                               hd, 2, strides, ids_o, bt, block_table=tab,
                               k_out=canary.copy(), v_out=canary.copy())
        got = out.cpu().numpy().view(np.uint8).reshape(2, kvh, k * bt, hd * 2)
        assert np.array_equal(got[0], ko) and np.array_equal(got[1], vo)
    del planes
    buf.free()


def _decode_inputs(n_qh, kvh, n_kv, fmt, seed):
    g = synth.rng(4, synth.P_Q, seed)
    gen = synth.bf16_normal if fmt == kvt.BF16 else synth.f16_normal
    return gen(g, (n_qh, 128)), gen(g, (kvh, n_kv, 128)), gen(g, (kvh, n_kv, 128))


def _run_decode(q, k, v, fmt, dev, n_valid=None, scale=None):
    n_qh, hd = q.shape
    kvh, n_kv, _ = k.shape
    scale = 1 / math.sqrt(hd) if scale is None else scale
    out = torch.full((n_qh, hd), float("nan"), dtype=torch.float32, device=dev)
    ws_bytes = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, n_kv)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    nv = None if n_valid is None else torch.tensor(n_valid, dtype=torch.int32, device=dev)
    kvt.kvt_attn_decode(_u16(q, dev), n_qh, kvh, hd, fmt, _u16(k, dev), _u16(v, dev), n_kv, nv,
                        scale, out, ws, ws_bytes)
    torch.cuda.synchronize()
    ref = oracle.attn_decode(q, k, v, oracle.BF16 if fmt == kvt.BF16 else oracle.F16, scale,
                             n_valid=n_valid)
    return out.cpu().numpy().astype(np.float64), ref


@pytest.mark.parametrize("n_qh,kvh,n_kv,fmt", [(64, 8, 2048, kvt.BF16), (64, 8, 2000, kvt.BF16),
                                               (64, 8, 2048, kvt.F16), (8, 8, 300, kvt.BF16),
                                               (32, 2, 1000, kvt.F16), (12, 4, 64, kvt.BF16),
                                               (16, 1, 4096, kvt.BF16),
                                               (16, 2, 9000, kvt.F16)])   # 141 chunks to merge
def test_decode_attention_within_tolerance(gpu, n_qh, kvh, n_kv, fmt):
    q, k, v = _decode_inputs(n_qh, kvh, n_kv, fmt, n_qh * 7 + n_kv)
    got, ref = _run_decode(q, k, v, fmt, gpu)
    err = np.max(np.abs(got - ref))
    assert err <= TOL, err


def test_decode_attention_valid_counts_and_degenerate_cases(gpu):
    q, k, v = _decode_inputs(64, 8, 2048, kvt.BF16, 99)
    nv = [2048, 1280, 0, 1, 63, 64, 65, 2047]
    got, ref = _run_decode(q, k, v, kvt.BF16, gpu, n_valid=nv)
    assert np.max(np.abs(got - ref)) <= TOL
    assert (got[16:24] == 0).all()                           # head with no valid key
    assert np.array_equal(got[24:32], np.repeat(ref[24:25], 8, 0))   # one key: that value row
    # all keys equal -> mean of V; a peaked softmax (large scale) still within tolerance
    k_eq = np.repeat(k[:, :1], 2048, axis=1)
    got, ref = _run_decode(q, k_eq, v, kvt.BF16, gpu)
    assert np.max(np.abs(got - ref)) <= TOL
    got, ref = _run_decode(q, k, v, kvt.BF16, gpu, scale=2.0)
    assert np.max(np.abs(got - ref)) <= TOL
    # rows past n_valid hold NaN patterns (as slots a gather skipped may): they take no part
    k_nan, v_nan = k.copy(), v.copy()
    k_nan[:, 1500:] = 0x7FC0
    v_nan[:, 1500:] = 0x7FC0
    got, ref = _run_decode(q, k_nan, v_nan, kvt.BF16, gpu, n_valid=[1500] * 8)
    assert np.isfinite(got).all() and np.max(np.abs(got - ref)) <= TOL
    got, ref = _run_decode(q, k[:, :0], v[:, :0], kvt.BF16, gpu)     # no keys at all
    assert (got == 0).all() and (ref == 0).all()


@pytest.mark.parametrize("ctx,layout", [(262144, "block_head_major"), (262144, "token_major"),
                                        (1048576, "block_head_major")])
def test_decode_step_full_geometry(gpu, ctx, layout):
    """One decode step at full size: pooled plane in HBM, K/V planes in pinned host memory,
    score + top-32 per KV head, gather host -> HBM, GQA attention with 64 query heads.
    Ids and gathered bytes bit-exact; attention within 2e-3 of the fp64 oracle."""
    kvh, hd, bt, k, n_qh = 8, 128, 64, 32, 64
    n_blocks = ctx // bt
    buf, planes = _host_planes(ctx, kvh, hd, 4, ctx)
    pooled = synth.f16_normal(synth.rng(4, synth.P_POOLED, ctx), (n_blocks, 128))
    q_idx = synth.f16_normal(synth.rng(4, synth.P_QIDX, ctx), (kvh, 128))
    q = synth.bf16_normal(synth.rng(4, synth.P_Q, ctx), (n_qh, hd))

    ws_t = kvt.kvt_index_topk_ws_bytes(n_blocks, kvh, k)
    ws_d = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, k * bt)
    ws = torch.empty(ws_t + ws_d, dtype=torch.uint8, device=gpu)
    ids = torch.empty((kvh, k), dtype=torch.int32, device=gpu)
    kg = torch.empty((2, kvh, k * bt, hd), dtype=torch.int16, device=gpu)
    out = torch.empty((n_qh, hd), dtype=torch.float32, device=gpu)
    kvt.kvt_index_topk(_u16(pooled, gpu), n_blocks, 128, _u16(q_idx, gpu), kvh, k, ids, None,
                       ws, ws_t)
    strides = LAYOUTS[layout](kvh, hd, 2, bt)
    kvt.kvt_gather_blocks(buf.dev, buf.dev + ctx * kvh * hd * 2, n_blocks, kvh, hd, 2, *strides,
                          None, bt, ids, k, kg[0], kg[1])
    kvt.kvt_attn_decode(_u16(q, gpu), n_qh, kvh, hd, kvt.BF16, kg[0], kg[1], k * bt, None,
                        1 / math.sqrt(hd), out, ws[ws_t:], ws_d)
    torch.cuda.synchronize()

    ref_ids = oracle.topk(oracle.index_scores(pooled, q_idx), k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ko, vo = oracle.gather(planes[0].view(np.uint8), planes[1].view(np.uint8), n_blocks, kvh,
                           hd, 2, strides, ref_ids, bt)
    got = kg.cpu().numpy().view(np.uint8).reshape(2, kvh, k * bt, hd * 2)
    assert np.array_equal(got[0], ko) and np.array_equal(got[1], vo)
    ref = oracle.attn_decode(q, ko.view(np.uint16).reshape(kvh, k * bt, hd),
                             vo.view(np.uint16).reshape(kvh, k * bt, hd), oracle.BF16,
                             1 / math.sqrt(hd))
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL
    del planes
    buf.free()


def _run_fused(buf, n_tok, kvh, hd, bt, n_blocks, strides, ids, q, fmt, dev, table=None,
               with_out=True, canary=0x1234):
    n_qh = q.shape[0]
    k = ids.shape[1]
    n_kv = k * bt
    out = torch.full((n_qh, hd), float("nan"), dtype=torch.float32, device=dev)
    ws_bytes = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, n_kv)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kv = torch.full((2, kvh, n_kv, hd), canary, dtype=torch.int16, device=dev)
    kvt.kvt_gather_attn_decode(_u16(q, dev), n_qh, kvh, hd, fmt, buf.dev,
                               buf.dev + n_tok * kvh * hd * 2, n_blocks, *strides,
                               None if table is None else torch.from_numpy(table).to(dev), bt,
                               torch.from_numpy(ids).to(dev), k,
                               kv[0] if with_out else None, kv[1] if with_out else None,
                               1 / math.sqrt(hd), out, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), kv.cpu().numpy().view(np.uint8).reshape(
        2, kvh, n_kv, hd * 2)


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("bt,k,n_qh", [(64, 32, 64), (16, 20, 64), (48, 5, 16), (100, 7, 8),
                                       (1, 70, 32), (64, 1, 64)])
def test_gather_attn_decode_matches_oracle(gpu, layout, bt, k, n_qh):
    """Fused gather + attention: out within 2e-3 of the oracle, the HBM copy of the rows
    bit-exact (skipped slots untouched), with a block table and with ids that are -1, repeated,
    or outside the planes, and block sizes that do and do not divide the 64-key chunks."""
    kvh, hd = 8, 128
    n_blocks = 300
    n_tok = n_blocks * bt
    buf, planes = _host_planes(n_tok, kvh, hd, 4, 100 + bt)
    strides = LAYOUTS[layout](kvh, hd, 2, bt)
    g = synth.rng(4, synth.P_MISC, 200 + bt * 3 + k)
    ids = np.stack([np.sort(g.permutation(n_blocks)[:k]) for _ in range(kvh)]).astype(np.int32)
    ids[2, k // 2] = -1                              # a hole in the middle
    ids[5, -1] = n_blocks + 3                        # outside the planes
    ids[6, :] = -1                                   # a head with nothing selected
    if k > 1:
        ids[7, 1] = ids[7, 0]                        # the same block twice
    table = g.permutation(n_blocks).astype(np.int32)
    q = synth.bf16_normal(synth.rng(4, synth.P_Q, bt + k), (n_qh, hd))
    for tab in (None, table):
        got, kv = _run_fused(buf, n_tok, kvh, hd, bt, n_blocks, strides, ids, q, kvt.BF16, gpu,
                             table=tab)
        ref, _, _ = oracle.gather_attn_decode(q, planes[0].view(np.uint8),
                                              planes[1].view(np.uint8), n_blocks, kvh, hd,
                                              oracle.BF16, strides, ids, bt, 1 / math.sqrt(hd),
                                              block_table=tab)
        assert np.isfinite(got).all()
        assert np.max(np.abs(got - ref)) <= TOL
        G = n_qh // kvh
        assert (got[6 * G:7 * G] == 0).all()
        ids_o = np.where((ids >= 0) & (ids < n_blocks), ids, -1).astype(np.int32)
        can = np.zeros((kvh, k * bt, hd * 2), dtype=np.uint8)
        can.view(np.uint16)[:] = 0x1234
        ko, vo = oracle.gather(planes[0].view(np.uint8), planes[1].view(np.uint8), n_blocks, kvh,
                               hd, 2, strides, ids_o, bt, block_table=tab, k_out=can.copy(),
                               v_out=can.copy())
        assert np.array_equal(kv[0], ko) and np.array_equal(kv[1], vo)
    del planes
    buf.free()


@pytest.mark.parametrize("fmt", [kvt.BF16, kvt.F16])
def test_gather_attn_decode_bit_identical_to_gather_then_decode(gpu, fmt):
    """Trailing skipped slots: the fused op equals kvt_gather_blocks + kvt_attn_decode with
    n_valid bit for bit (same chunks, same arithmetic, same merge); without k_out/v_out the
    attention output is the same."""
    kvh, hd, bt, k, n_qh = 8, 128, 64, 32, 64
    n_blocks = 500
    n_tok = n_blocks * bt
    buf, planes = _host_planes(n_tok, kvh, hd, 4, 77)
    if fmt == kvt.F16:                               # reinterpret the plane as N(0,1) fp16
        g = synth.rng(4, synth.P_K, 78)
        for p in range(2):
            for t0 in range(0, n_tok, 1 << 14):
                planes[p, t0:t0 + (1 << 14)] = synth.f16_normal(g, (min(1 << 14, n_tok - t0),
                                                                    kvh, hd))
    strides = oracle.block_head_major_strides(kvh, hd, 2, bt)
    g = synth.rng(4, synth.P_MISC, 79)
    ids = np.stack([np.sort(g.permutation(n_blocks)[:k]) for _ in range(kvh)]).astype(np.int32)
    ids[1, 25:] = -1
    ids[3, 1:] = -1
    gen = synth.bf16_normal if fmt == kvt.BF16 else synth.f16_normal
    q = gen(synth.rng(4, synth.P_Q, 80), (n_qh, hd))
    fused, kv = _run_fused(buf, n_tok, kvh, hd, bt, n_blocks, strides, ids, q, fmt, gpu)
    fused_noout, kv2 = _run_fused(buf, n_tok, kvh, hd, bt, n_blocks, strides, ids, q, fmt, gpu,
                                  with_out=False)
    assert np.array_equal(fused, fused_noout)
    assert (kv2.view(np.uint16) == 0x1234).all()     # nothing written without outputs

    staged = torch.full((2, kvh, k * bt, hd), 0x1234, dtype=torch.int16, device=gpu)
    ids_d = torch.from_numpy(ids).to(gpu)
    kvt.kvt_gather_blocks(buf.dev, buf.dev + n_tok * kvh * hd * 2, n_blocks, kvh, hd, 2, *strides,
                          None, bt, ids_d, k, staged[0], staged[1])
    n_valid = torch.from_numpy(((ids >= 0).sum(1) * bt).astype(np.int32)).to(gpu)
    out = torch.empty((n_qh, hd), dtype=torch.float32, device=gpu)
    ws_bytes = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, k * bt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=gpu)
    kvt.kvt_attn_decode(_u16(q, gpu), n_qh, kvh, hd, fmt, staged[0], staged[1], k * bt, n_valid,
                        1 / math.sqrt(hd), out, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), fused)
    assert np.array_equal(staged.cpu().numpy().view(np.uint8).reshape(kv.shape), kv)
    ofmt = oracle.BF16 if fmt == kvt.BF16 else oracle.F16
    ref, _, _ = oracle.gather_attn_decode(q, planes[0].view(np.uint8), planes[1].view(np.uint8),
                                          n_blocks, kvh, hd, ofmt, strides, ids, bt,
                                          1 / math.sqrt(hd))
    assert np.max(np.abs(fused - ref)) <= TOL
    del planes
    buf.free()


@pytest.mark.parametrize("ctx", [262144, 1048576])
def test_fused_decode_step_full_geometry(gpu, ctx):
    """The decode step with the fused gather + attention at full size (block-local head-major
    host planes): ids bit-exact, the HBM rows bit-exact, attention within 2e-3."""
    kvh, hd, bt, k, n_qh = 8, 128, 64, 32, 64
    n_blocks = ctx // bt
    buf, planes = _host_planes(ctx, kvh, hd, 4, ctx + 1)
    pooled = synth.f16_normal(synth.rng(4, synth.P_POOLED, ctx + 1), (n_blocks, 128))
    q_idx = synth.f16_normal(synth.rng(4, synth.P_QIDX, ctx + 1), (kvh, 128))
    q = synth.bf16_normal(synth.rng(4, synth.P_Q, ctx + 1), (n_qh, hd))
    strides = oracle.block_head_major_strides(kvh, hd, 2, bt)
    ws_t = kvt.kvt_index_topk_ws_bytes(n_blocks, kvh, k)
    ws_d = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, k * bt)
    ws = torch.empty(ws_t + ws_d, dtype=torch.uint8, device=gpu)
    ids = torch.empty((kvh, k), dtype=torch.int32, device=gpu)
    kg = torch.empty((2, kvh, k * bt, hd), dtype=torch.int16, device=gpu)
    out = torch.empty((n_qh, hd), dtype=torch.float32, device=gpu)
    kvt.kvt_index_topk(_u16(pooled, gpu), n_blocks, 128, _u16(q_idx, gpu), kvh, k, ids, None,
                       ws, ws_t)
    kvt.kvt_gather_attn_decode(_u16(q, gpu), n_qh, kvh, hd, kvt.BF16, buf.dev,
                               buf.dev + ctx * kvh * hd * 2, n_blocks, *strides, None, bt, ids, k,
                               kg[0], kg[1], 1 / math.sqrt(hd), out, ws[ws_t:], ws_d)
    torch.cuda.synchronize()
    ref_ids = oracle.topk(oracle.index_scores(pooled, q_idx), k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref, ko, vo = oracle.gather_attn_decode(q, planes[0].view(np.uint8), planes[1].view(np.uint8),
                                            n_blocks, kvh, hd, oracle.BF16, strides, ref_ids, bt,
                                            1 / math.sqrt(hd))
    got = kg.cpu().numpy().view(np.uint8).reshape(2, kvh, k * bt, hd * 2)
    assert np.array_equal(got[0], ko) and np.array_equal(got[1], vo)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL
    del planes
    buf.free()


@pytest.mark.parametrize("cr,n_tok,k", [(4, 1003, 40), (4, 1000, 40), (1, 77, 10), (64, 1285, 7),
                                        (4, 3, 8)])
def test_select_positions_bit_exact(gpu, cr, n_tok, k):
    g = synth.rng(4, synth.P_MISC, cr * 1000 + n_tok)
    n_blocks = n_tok // cr
    rows = [np.sort(g.permutation(n_blocks)[:min(k, n_blocks)]) for _ in range(3)]
    ids = np.full((3, k), -1, dtype=np.int32)
    for h, r in enumerate(rows):
        ids[h, :r.size] = r
    ids[1, k // 2:] = -1
    k_pad = oracle.qsa_k_pad(k, cr)
    pos = torch.full((3, k_pad), 12345, dtype=torch.int32, device=gpu)
    kvt.kvt_select_positions(torch.from_numpy(ids).to(gpu), 3, k, cr, n_tok, k_pad, pos)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), oracle.select_positions(ids, cr, n_tok, k_pad))
    if cr > 1:
        with pytest.raises(kvt.KvtError) as e:              # no room for a full tail
            kvt.kvt_select_positions(torch.from_numpy(ids).to(gpu), 3, k, cr, n_tok,
                                     k * cr + cr - 2, pos)
        assert e.value.code == kvt.EINVAL


def test_qsa_geometry_decode_step(gpu):
    """The page's selection geometry at 262,147 tokens: pooled keys over 4-token blocks
    (65,536 complete blocks), top-512 per KV head, positions + the 3-token write-head tail padded
    to 2080, then the fused gather + attention over those tokens (64 query heads, token-major host
    planes).  Ids, positions and gathered rows bit-exact; attention within 2e-3."""
    kvh, hd, n_qh, cr, k = 8, 128, 64, 4, 512
    n_tok = 262144 + 3
    n_blocks = n_tok // cr
    k_pad = oracle.qsa_k_pad(k, cr)
    buf, planes = _host_planes(n_tok, kvh, hd, 4, 7)
    pooled = synth.f16_normal(synth.rng(4, synth.P_POOLED, 7), (n_blocks, 128))
    q_idx = synth.f16_normal(synth.rng(4, synth.P_QIDX, 7), (kvh, 128))
    q = synth.bf16_normal(synth.rng(4, synth.P_Q, 7), (n_qh, hd))
    ids, _ = _run_topk(pooled, q_idx, k, gpu, want_scores=False)
    ref_ids = oracle.topk(oracle.index_scores(pooled, q_idx), k)
    assert np.array_equal(ids, ref_ids)
    pos = torch.empty((kvh, k_pad), dtype=torch.int32, device=gpu)
    kvt.kvt_select_positions(torch.from_numpy(ids).to(gpu), kvh, k, cr, n_tok, k_pad, pos)
    ref_pos = oracle.select_positions(ref_ids, cr, n_tok, k_pad)
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), ref_pos)
    row = kvh * hd * 2
    strides = (row, hd * 2, row)   # a "block" is one token of the token-major plane
    ws_bytes = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, k_pad)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=gpu)
    kv = torch.full((2, kvh, k_pad, hd), 0x1234, dtype=torch.int16, device=gpu)
    out = torch.empty((n_qh, hd), dtype=torch.float32, device=gpu)
    kvt.kvt_gather_attn_decode(_u16(q, gpu), n_qh, kvh, hd, kvt.BF16, buf.dev,
                               buf.dev + n_tok * row, n_tok, *strides, None, 1, pos, k_pad,
                               kv[0], kv[1], 1 / math.sqrt(hd), out, ws, ws_bytes)
    torch.cuda.synchronize()
    ref, _, _ = oracle.gather_attn_decode(q, planes[0].view(np.uint8), planes[1].view(np.uint8),
                                          n_tok, kvh, hd, oracle.BF16, strides, ref_pos, 1,
                                          1 / math.sqrt(hd))
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= TOL
    can = np.zeros((kvh, k_pad, hd * 2), dtype=np.uint8)
    can.view(np.uint16)[:] = 0x1234
    ko, vo = oracle.gather(planes[0].view(np.uint8), planes[1].view(np.uint8), n_tok, kvh, hd, 2,
                           strides, ref_pos, 1, k_out=can.copy(), v_out=can.copy())
    got = kv.cpu().numpy().view(np.uint8).reshape(2, kvh, k_pad, hd * 2)
    assert np.array_equal(got[0], ko) and np.array_equal(got[1], vo)
    del planes
    buf.free()
