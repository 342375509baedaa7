"""GPU parity of the tiered prefill path: tail staging + flash attention over a q8_0 cache.

* within 2e-3 max-abs of the fp64 oracle (every element at small sizes, sampled query rows at
  the full 180,000-token geometry);
* bit-identical output whether the cache is all in HBM, split into an HBM head plus a staged
  tail, or split with the tail read in place from host memory (staging off)."""
import math

import numpy as np
import pytest
import torch

import oracle
from hbm_kv_cache_amd import kvt, synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


ORACLE_FMT = {kvt.Q8_0: oracle.Q8_0, kvt.F16: oracle.F16, kvt.BF16: oracle.BF16}
FMT_IDS = {kvt.Q8_0: "q8_0", kvt.F16: "f16", kvt.BF16: "bf16"}


def _cache(n_kv, kvh, seed, fmt=kvt.Q8_0):
    """K and V rows as uint8 [n_kv][row bytes]: q8_0 blocks, or N(0,1) fp16 / bf16 values."""
    if fmt == kvt.Q8_0:
        k = synth.q8_0_rows(synth.rng(5, synth.P_K, seed), n_kv, kvh, 128)
        v = synth.q8_0_rows(synth.rng(5, synth.P_V, seed), n_kv, kvh, 128)
        return k, v
    gen = synth.f16_normal if fmt == kvt.F16 else synth.bf16_normal
    k = gen(synth.rng(5, synth.P_K, seed), (n_kv, kvh * 128)).view(np.uint8)
    v = gen(synth.rng(5, synth.P_V, seed), (n_kv, kvh * 128)).view(np.uint8)
    return k, v


def _prefill(q_np, q_pos0, kvh, k_head, v_head, n_head, k_tail, v_tail, n_kv, causal, dev,
             fmt=kvt.Q8_0):
    n_q, n_qh, hd = q_np.shape
    q = torch.from_numpy(q_np.view(np.int16)).to(dev)
    out = torch.full((n_q, n_qh, hd), float("nan"), dtype=torch.float32, device=dev)
    kvt.kvt_attn_prefill(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, k_tail, v_tail,
                         n_kv, fmt, causal, 1 / math.sqrt(hd), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("n_kv,n_q,n_qh,kvh,causal,n_head", [
    (1000, 77, 32, 8, True, 400),       # ragged queries and keys, split mid-tile
    (2048, 64, 16, 4, True, 2048),      # all in HBM
    (1500, 100, 8, 8, True, 0),         # all in the tail
    (700, 33, 8, 4, False, 350),        # non-causal, group 2
    (333, 40, 4, 4, True, 64),          # group 1
    (130, 130, 8, 2, True, 65),         # queries from position 0: first row sees one key
    (600, 50, 16, 2, True, 300),        # group 8
])
def test_prefill_matches_oracle(gpu, n_kv, n_q, n_qh, kvh, causal, n_head):
    k, v = _cache(n_kv, kvh, n_kv + n_q)
    q = synth.f16_normal(synth.rng(5, synth.P_Q, n_kv), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    got = _prefill(q, q_pos0, kvh, kd, vd, n_head, kd[n_head:], vd[n_head:], n_kv, causal, gpu)
    ref = oracle.attn_prefill(q, q_pos0, kvh, k, v, n_head, k[n_head:], v[n_head:], n_kv,
                              oracle.Q8_0, causal, 1 / math.sqrt(128))
    err = np.max(np.abs(got - ref))
    assert np.isfinite(got).all() and err <= TOL, err


def test_prefill_peaked_softmax_within_tolerance(gpu):
    """For every query row, one visible key is the (q8_0-quantised) query itself, so its logit
    (about |q|^2 / sqrt(128), ~11) dominates the others (~N(0,1)): most of the weight sits on
    one key and the rounding of the probabilities and of V matters most.  Still within 2e-3.
    (The bound holds at the usual 1/sqrt(head_dim) scale; the fp16 rounding of dequantised K
    perturbs each logit by up to scale * sum|q k| * 2^-11, which grows with the scale.)"""
    n_kv, n_q, n_qh, kvh = 512, 16, 4, 4
    k, v = _cache(n_kv, kvh, 7)
    q = synth.f16_normal(synth.rng(5, synth.P_Q, 7), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    rows = k.reshape(n_kv, kvh * 4, 34).copy()
    for t in range(n_q):
        j = q_pos0 + t - 3 * (t % 5)                  # a visible key for row t
        x = q[t].view(np.float16).astype(np.float32).reshape(kvh * 4, 32)   # head h -> kv h
        rows[j] = synth.q8_0_encode(x[None])[0]
    k = rows.reshape(n_kv, -1)
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    got = _prefill(q, q_pos0, kvh, kd, vd, n_kv, None, None, n_kv, True, gpu)
    ref = oracle.attn_prefill(q, q_pos0, kvh, k, v, n_kv, None, None, n_kv, oracle.Q8_0, True,
                              1 / math.sqrt(128))
    assert np.max(np.abs(got - ref)) <= TOL


@pytest.mark.parametrize("fmt", [kvt.Q8_0, kvt.F16, kvt.BF16], ids=FMT_IDS.get)
def test_prefill_three_way_bit_identity(gpu, fmt):
    """All-HBM cache == HBM head + staged tail == HBM head + tail read from host memory."""
    n_kv, n_q, n_qh, kvh, n_head = 5000, 300, 32, 8, 2100
    k, v = _cache(n_kv, kvh, 11, fmt)
    row = k.shape[1]
    q = synth.f16_normal(synth.rng(5, synth.P_Q, 11), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    host = kvt.HostBuffer(2 * (n_kv - n_head) * row)
    ht = host.numpy(np.uint8, (2, n_kv - n_head, row))
    ht[0], ht[1] = k[n_head:], v[n_head:]
    all_hbm = _prefill(q, q_pos0, kvh, kd, vd, n_kv, None, None, n_kv, True, gpu, fmt)
    stage = torch.empty((2, n_kv - n_head, row), dtype=torch.uint8, device=gpu)
    for mode in (kvt.COPY_SDMA, kvt.COPY_KERNEL):
        stage.zero_()
        kvt.kvt_stage_tail(host.dev, row, 0, n_kv - n_head, stage[0], mode)
        kvt.kvt_stage_tail(host.dev + (n_kv - n_head) * row, row, 0, n_kv - n_head, stage[1], mode)
        staged = _prefill(q, q_pos0, kvh, kd, vd, n_head, stage[0], stage[1], n_kv, True, gpu,
                          fmt)
        assert np.array_equal(staged.view(np.uint32), all_hbm.view(np.uint32))
    in_place = _prefill(q, q_pos0, kvh, kd, vd, n_head, host.dev,
                        host.dev + (n_kv - n_head) * row, n_kv, True, gpu, fmt)
    assert np.array_equal(in_place.view(np.uint32), all_hbm.view(np.uint32))
    del ht
    host.free()


def _pipelined(q_np, q_pos0, kvh, k_head, v_head, n_head, host, n_kv, arena_rows, dev,
               causal=True, fmt=kvt.Q8_0):
    """kvt_attn_prefill_pipelined with the host tail in `host` (K rows then V rows)."""
    n_q, n_qh, hd = q_np.shape
    row = kvh * (136 if fmt == kvt.Q8_0 else 256)
    n_tail = n_kv - n_head
    q = torch.from_numpy(q_np.view(np.int16)).to(dev)
    out = torch.full((n_q, n_qh, hd), float("nan"), dtype=torch.float32, device=dev)
    arena = torch.full((2, arena_rows, row), 0xA5, dtype=torch.uint8, device=dev)
    sb = kvt.kvt_attn_prefill_state_bytes(n_q, n_qh, kvh)
    state = torch.empty(sb, dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream()
    kvt.kvt_attn_prefill_pipelined(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head,
                                   host.dev, host.dev + n_tail * row, n_kv, fmt, causal,
                                   1 / math.sqrt(hd), arena[0], arena[1], arena_rows, state, sb,
                                   out, copy_stream=copy_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_prefill_range_passes_bit_identical(gpu):
    """The attention as resumable passes over key ranges -- including an empty pass and a pass
    that starts mid-head and ends in the tail -- gives the single pass's bits."""
    n_kv, n_q, n_qh, kvh, n_head = 1000, 77, 32, 8, 400
    k, v = _cache(n_kv, kvh, 21)
    q_np = synth.f16_normal(synth.rng(5, synth.P_Q, 21), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    one = _prefill(q_np, q_pos0, kvh, kd, vd, n_head, kd[n_head:], vd[n_head:], n_kv, True, gpu)
    q = torch.from_numpy(q_np.view(np.int16)).to(gpu)
    sb = kvt.kvt_attn_prefill_state_bytes(n_q, n_qh, kvh)
    state = torch.empty(sb, dtype=torch.uint8, device=gpu)
    for cuts in ([0, 128, 128, 512, 1000], [0, 64, 448, 960, 1000], [0, 1000]):
        out = torch.full((n_q, n_qh, 128), float("nan"), dtype=torch.float32, device=gpu)
        for a, b in zip(cuts[:-1], cuts[1:]):
            kvt.kvt_attn_prefill_range(q, n_q, q_pos0, n_qh, kvh, 128, kd, vd, n_head,
                                       kd[n_head:], vd[n_head:], n_kv, kvt.Q8_0, True,
                                       1 / math.sqrt(128), a, b, state, sb, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), one.view(np.uint32)), cuts
    with pytest.raises(kvt.KvtError) as e:                 # bounds must be whole tiles
        kvt.kvt_attn_prefill_range(q, n_q, q_pos0, n_qh, kvh, 128, kd, vd, n_head, kd[n_head:],
                                   vd[n_head:], n_kv, kvt.Q8_0, True, 0.1, 0, 100, state, sb, out)
    assert e.value.code == kvt.EINVAL
    with pytest.raises(kvt.KvtError) as e:                 # a split pass needs the state
        kvt.kvt_attn_prefill_range(q, n_q, q_pos0, n_qh, kvh, 128, kd, vd, n_head, kd[n_head:],
                                   vd[n_head:], n_kv, kvt.Q8_0, True, 0.1, 0, 128, state, 16, out)
    assert e.value.code == kvt.EINVAL


@pytest.mark.parametrize("n_kv,n_head,arena_rows,n_qh,kvh", [
    (5000, 2100, 128, 32, 8),      # 64-key buckets, head split mid-tile
    (5000, 2048, 1000, 32, 8),     # head on a tile boundary, buckets of 448 keys
    (5000, 0, 3000, 16, 4),        # no head: buckets from key 0
    (5000, 4999, 256, 8, 8),       # one host row
    (3000, 1500, 100000, 32, 8),   # the whole tail in one bucket
    (2000, 2000, 128, 32, 8),      # nothing in host memory
])
def test_prefill_pipelined_bit_identical(gpu, n_kv, n_head, arena_rows, n_qh, kvh):
    """Tail staged in arena buckets on a second stream while the head and earlier buckets are
    attended: the same bits as the single pass over an all-HBM cache, on two calls in a row
    (the second reuses the library's events and the arena)."""
    n_q = 300
    k, v = _cache(n_kv, kvh, n_kv + n_head)
    row = k.shape[1]
    q = synth.f16_normal(synth.rng(5, synth.P_Q, n_head + 7), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    all_hbm = _prefill(q, q_pos0, kvh, kd, vd, n_kv, None, None, n_kv, True, gpu)
    n_tail = n_kv - n_head
    host = kvt.HostBuffer(max(2 * n_tail * row, 16))
    if n_tail:
        ht = host.numpy(np.uint8, (2, n_tail, row))
        ht[0], ht[1] = k[n_head:], v[n_head:]
        del ht
    for _ in range(2):
        got = _pipelined(q, q_pos0, kvh, kd[:max(n_head, 1)], vd[:max(n_head, 1)], n_head, host,
                         n_kv, arena_rows, gpu)
        assert np.array_equal(got.view(np.uint32), all_hbm.view(np.uint32))
    host.free()


def test_prefill_full_geometry_sampled_rows(gpu):
    """180,000-token context, cells [0, 94208) in HBM and the rest in host memory, q8_0 K/V
    (8 KV heads x 128), a 2048-query causal chunk at the tail with 32 query heads: stage the
    host rows into HBM once, run the attention, compare sampled query rows (all heads, all
    dims) with the fp64 oracle; staging on/off and all-HBM agree bit for bit."""
    n_kv, n_head, n_q, n_qh, kvh = 180000, 94208, 2048, 32, 8
    k, v = _cache(n_kv, kvh, 180000)
    row = k.shape[1]
    n_tail = n_kv - n_head
    q = synth.f16_normal(synth.rng(5, synth.P_Q, 180000), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    kd, vd = _dev(k[:n_head], gpu), _dev(v[:n_head], gpu)
    host = kvt.HostBuffer(2 * n_tail * row)
    ht = host.numpy(np.uint8, (2, n_tail, row))
    ht[0], ht[1] = k[n_head:], v[n_head:]
    stage = torch.empty((2, n_tail, row), dtype=torch.uint8, device=gpu)
    kvt.kvt_stage_tail(host.dev, row, 0, n_tail, stage[0], kvt.COPY_AUTO)
    kvt.kvt_stage_tail(host.dev + n_tail * row, row, 0, n_tail, stage[1], kvt.COPY_AUTO)
    staged = _prefill(q, q_pos0, kvh, kd, vd, n_head, stage[0], stage[1], n_kv, True, gpu)
    assert np.array_equal(stage.cpu().numpy().reshape(2, n_tail, row), ht)
    for rows in ((0, 2), (1023, 1025), (2046, 2048)):
        ref = oracle.attn_prefill(q, q_pos0, kvh, k, v, n_kv, None, None, n_kv, oracle.Q8_0, True,
                                  1 / math.sqrt(128), t_begin=rows[0], t_end=rows[1])
        err = np.max(np.abs(staged[rows[0]:rows[1]] - ref))
        assert err <= TOL, (rows, err)
    in_place = _prefill(q, q_pos0, kvh, kd, vd, n_head, host.dev, host.dev + n_tail * row, n_kv,
                        True, gpu)
    assert np.array_equal(in_place.view(np.uint32), staged.view(np.uint32))
    kall, vall = _dev(k, gpu), _dev(v, gpu)
    all_hbm = _prefill(q, q_pos0, kvh, kall, vall, n_kv, None, None, n_kv, True, gpu)
    assert np.array_equal(all_hbm.view(np.uint32), staged.view(np.uint32))
    del kall, vall
    pipelined = _pipelined(q, q_pos0, kvh, kd, vd, n_head, host, n_kv, 32768, gpu)
    assert np.array_equal(pipelined.view(np.uint32), staged.view(np.uint32))
    del ht
    host.free()


def test_prefill_argument_errors(gpu):
    q = torch.zeros((4, 8, 128), dtype=torch.float16, device=gpu)
    out = torch.empty((4, 8, 128), dtype=torch.float32, device=gpu)
    k = torch.zeros((10, 8 * 136), dtype=torch.uint8, device=gpu)
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_attn_prefill(q, 4, 0, 8, 8, 128, k, k, 10, None, None, 10, 7, 1, 0.1, out)
    assert e.value.code == kvt.EUNSUPPORTED            # not a cache format
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_attn_prefill(q, 4, 0, 16, 1, 128, k, k, 10, None, None, 10, kvt.Q8_0, 1, 0.1, out)
    assert e.value.code == kvt.EUNSUPPORTED            # group 16
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_attn_prefill(q, 4, 0, 8, 8, 128, k, k, 10, None, None, 10, kvt.Q8_0, 1, 0.0, out)
    assert e.value.code == kvt.EINVAL                  # scale must be positive
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_attn_prefill(q, 4, 0, 8, 8, 128, k, k, 11, None, None, 10, kvt.Q8_0, 1, 0.1, out)
    assert e.value.code == kvt.EINVAL                  # n_head > n_kv
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_attn_prefill(q, 4, 0, 8, 8, 128, k, k, 5, None, None, 10, kvt.Q8_0, 1, 0.1, out)
    assert e.value.code == kvt.EINVAL                  # tail rows without tail pointers


@pytest.mark.parametrize("fmt", [kvt.F16, kvt.BF16], ids=FMT_IDS.get)
@pytest.mark.parametrize("n_kv,n_q,n_qh,kvh,causal,n_head", [
    (1000, 77, 32, 8, True, 400),       # ragged queries and keys, split mid-tile
    (700, 33, 8, 4, False, 350),        # non-causal, group 2
    (600, 50, 16, 2, True, 0),          # group 8, all in the tail
])
def test_prefill_fp_caches_match_oracle(gpu, fmt, n_kv, n_q, n_qh, kvh, causal, n_head):
    """fp16 and bf16 caches: the values as stored (bf16 converted to fp16, exact at these
    magnitudes) on the same MFMA path; within 2e-3 of the fp64 oracle."""
    k, v = _cache(n_kv, kvh, n_kv + n_q + fmt, fmt)
    q = synth.f16_normal(synth.rng(5, synth.P_Q, n_kv + fmt), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    got = _prefill(q, q_pos0, kvh, kd, vd, n_head, kd[n_head:], vd[n_head:], n_kv, causal, gpu,
                   fmt)
    ref = oracle.attn_prefill(q, q_pos0, kvh, k, v, n_head, k[n_head:], v[n_head:], n_kv,
                              ORACLE_FMT[fmt], causal, 1 / math.sqrt(128))
    err = np.max(np.abs(got - ref))
    assert np.isfinite(got).all() and err <= TOL, err


@pytest.mark.parametrize("fmt", [kvt.F16, kvt.BF16], ids=FMT_IDS.get)
def test_prefill_pipelined_fp_caches_bit_identical(gpu, fmt):
    """The pipelined staging with fp16 / bf16 rows (256-byte head slices) gives the single
    pass's bits over an all-HBM cache."""
    n_kv, n_head, n_q, n_qh, kvh, arena_rows = 4000, 1500, 200, 32, 8, 512
    k, v = _cache(n_kv, kvh, 99 + fmt, fmt)
    row = k.shape[1]
    q = synth.f16_normal(synth.rng(5, synth.P_Q, 99 + fmt), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    all_hbm = _prefill(q, q_pos0, kvh, kd, vd, n_kv, None, None, n_kv, True, gpu, fmt)
    n_tail = n_kv - n_head
    host = kvt.HostBuffer(2 * n_tail * row)
    ht = host.numpy(np.uint8, (2, n_tail, row))
    ht[0], ht[1] = k[n_head:], v[n_head:]
    del ht
    got = _pipelined(q, q_pos0, kvh, kd[:n_head], vd[:n_head], n_head, host, n_kv, arena_rows,
                     gpu, fmt=fmt)
    assert np.array_equal(got.view(np.uint32), all_hbm.view(np.uint32))
    host.free()


def _splitk(q_np, q_pos0, kvh, k_head, v_head, n_head, k_tail, v_tail, n_kv, causal, dev,
            fmt=kvt.Q8_0):
    n_q, n_qh, hd = q_np.shape
    q = torch.from_numpy(q_np.view(np.int16)).to(dev)
    out = torch.full((n_q, n_qh, hd), float("nan"), dtype=torch.float32, device=dev)
    wb = kvt.kvt_attn_prefill_splitk_ws_bytes(n_q, n_qh, kvh, n_kv)
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device=dev)
    kvt.kvt_attn_prefill_splitk(q, n_q, q_pos0, n_qh, kvh, hd, k_head, v_head, n_head, k_tail,
                                v_tail, n_kv, fmt, causal, 1 / math.sqrt(hd), ws, wb, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), wb


@pytest.mark.parametrize("n_kv,n_q,n_qh,kvh,causal,n_head", [
    (5000, 1, 32, 8, True, 2100),      # one decode token: 8 workgroups -> key splits
    (5000, 7, 64, 8, True, 0),         # a few tokens, group 8, all in the tail
    (3000, 64, 16, 4, False, 1500),    # non-causal, group 4
    (2000, 1, 8, 8, True, 350),        # short context: 4 splits of 8 tiles, group 1
])
def test_prefill_splitk_matches_oracle(gpu, n_kv, n_q, n_qh, kvh, causal, n_head):
    k, v = _cache(n_kv, kvh, n_kv + 3 * n_q)
    q = synth.f16_normal(synth.rng(5, synth.P_Q, n_kv + n_q), (n_q, n_qh, 128))
    q_pos0 = n_kv - n_q
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    got, wb = _splitk(q, q_pos0, kvh, kd, vd, n_head, kd[n_head:], vd[n_head:], n_kv, causal, gpu)
    assert wb > 0, "these shapes take the split path"
    ref = oracle.attn_prefill(q, q_pos0, kvh, k, v, n_head, k[n_head:], v[n_head:], n_kv,
                              oracle.Q8_0, causal, 1 / math.sqrt(128))
    err = np.max(np.abs(got - ref))
    assert np.isfinite(got).all() and err <= TOL, err


def test_prefill_splitk_tiers_bit_identical_and_one_split_is_the_single_pass(gpu):
    """Key splits sit at fixed tile boundaries, so HBM head + staged tail, the tail read in
    place and the all-HBM cache give the same bits; a shape that needs no split returns exactly
    kvt_attn_prefill's output."""
    n_kv, n_head, kvh, n_qh = 5000, 2100, 8, 32
    k, v = _cache(n_kv, kvh, 77)
    row = k.shape[1]
    kd, vd = _dev(k, gpu), _dev(v, gpu)
    q1 = synth.f16_normal(synth.rng(5, synth.P_Q, 77), (1, n_qh, 128))
    all_hbm, _ = _splitk(q1, n_kv - 1, kvh, kd, vd, n_kv, None, None, n_kv, True, gpu)
    host = kvt.HostBuffer(2 * (n_kv - n_head) * row)
    ht = host.numpy(np.uint8, (2, n_kv - n_head, row))
    ht[0], ht[1] = k[n_head:], v[n_head:]
    in_place, _ = _splitk(q1, n_kv - 1, kvh, kd, vd, n_head, host.dev,
                          host.dev + (n_kv - n_head) * row, n_kv, True, gpu)
    staged, _ = _splitk(q1, n_kv - 1, kvh, kd, vd, n_head, kd[n_head:], vd[n_head:], n_kv, True,
                        gpu)
    assert np.array_equal(in_place.view(np.uint32), all_hbm.view(np.uint32))
    assert np.array_equal(staged.view(np.uint32), all_hbm.view(np.uint32))
    del ht
    host.free()
    qn = synth.f16_normal(synth.rng(5, synth.P_Q, 78), (2048, n_qh, 128))
    assert kvt.kvt_attn_prefill_splitk_ws_bytes(2048, n_qh, kvh, n_kv) == 0
    single = _prefill(qn, n_kv - 2048, kvh, kd, vd, n_kv, None, None, n_kv, True, gpu)
    one_split, _ = _splitk(qn, n_kv - 2048, kvh, kd, vd, n_kv, None, None, n_kv, True, gpu)
    assert np.array_equal(one_split.view(np.uint32), single.view(np.uint32))
    q = torch.from_numpy(q1.view(np.int16)).to(gpu)
    out = torch.empty((1, n_qh, 128), dtype=torch.float32, device=gpu)
    wb = kvt.kvt_attn_prefill_splitk_ws_bytes(1, n_qh, kvh, n_kv)
    ws = torch.empty(wb, dtype=torch.uint8, device=gpu)
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_attn_prefill_splitk(q, 1, n_kv - 1, n_qh, kvh, 128, kd, vd, n_kv, None, None,
                                    n_kv, kvt.Q8_0, True, 0.1, ws, wb - 4, out)
    assert e.value.code == kvt.EINVAL


def test_prefill_splitk_decode_token_at_full_geometry(gpu):
    """One decode token over the 180,000-row tiered q8_0 cache (tail read in place), against
    the fp64 oracle."""
    n_kv, n_head, n_qh, kvh = 180000, 94208, 32, 8
    k, v = _cache(n_kv, kvh, 180001)
    row = k.shape[1]
    q = synth.f16_normal(synth.rng(5, synth.P_Q, 180001), (1, n_qh, 128))
    kd, vd = _dev(k[:n_head], gpu), _dev(v[:n_head], gpu)
    host = kvt.HostBuffer(2 * (n_kv - n_head) * row)
    ht = host.numpy(np.uint8, (2, n_kv - n_head, row))
    ht[0], ht[1] = k[n_head:], v[n_head:]
    got, wb = _splitk(q, n_kv - 1, kvh, kd, vd, n_head, host.dev, host.dev + (n_kv - n_head) * row,
                      n_kv, True, gpu)
    assert wb > 0
    ref = oracle.attn_prefill(q, n_kv - 1, kvh, k, v, n_head, k[n_head:], v[n_head:], n_kv,
                              oracle.Q8_0, True, 1 / math.sqrt(128))
    assert np.max(np.abs(got - ref)) <= TOL
    del ht
    host.free()
