"""Pins for the CPU oracle.  None of these restates the oracle's formula: each checks it against a
library routine (numpy views and fancy indexing, numpy/torch dtype conversion, np.lexsort,
torch's fp64 scaled-dot-product attention), a closed form, an invariant or a worked value."""
import ctypes
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from hbm_kv_cache_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------------
# scalar decoders (IEEE binary16 / bfloat16)
# ------------------------------------------------------------------------------------------

def test_f16_decoder_matches_numpy_for_every_pattern():
    lib = oracle._load()
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.orc_f16_to_f64(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_decoder_matches_torch_for_every_pattern():
    lib = oracle._load()
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([lib.orc_bf16_to_f64(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ------------------------------------------------------------------------------------------
# O1 sub-block pointers
# ------------------------------------------------------------------------------------------

def test_sub_block_ptrs_worked_value():
    g = json.load(open(os.path.join(GOLDEN, "sub_block_ptrs_worked.json")))
    out = oracle.sub_block_ptrs(g["base"], g["row_stride"], g["page_bytes"], g["block_ids"],
                                g["blocks_per_chunk"], g["skip"], g["n_out"])
    assert [hex(int(x)) for x in out] == g["expected"]


@pytest.mark.parametrize("bpc,skip,pad", [(1, 0, 0), (1, 0, 64), (4, 0, 4096), (4, 3, 4096),
                                          (2, 1, 0), (8, 5, 24)])
def test_sub_block_ptrs_match_numpy_view_addresses(bpc, skip, pad):
    """Addresses come from numpy's own view machinery on a strided (padded) 2-D array."""
    g = synth.rng(0, synth.P_MISC, bpc * 100 + skip)
    page, n_blocks = 256, 12
    buf = np.zeros((n_blocks, bpc * page + pad), dtype=np.uint8)
    t = buf[:, :bpc * page]                      # non-contiguous when pad > 0
    ids = g.permutation(n_blocks)[:5]
    n_out = len(ids) * bpc - skip - (1 if bpc > 1 else 0)
    addr = np.array([[t[b, j * page:(j + 1) * page].__array_interface__["data"][0]
                      for j in range(bpc)] for b in ids], dtype=np.uint64)
    expected = addr.reshape(-1)[skip:skip + n_out]
    got = oracle.sub_block_ptrs(t.__array_interface__["data"][0], t.strides[0], page, ids, bpc,
                                skip, n_out)
    assert np.array_equal(got, expected)


def test_sub_block_ptrs_dereference_labels():
    """Each page holds its (block, sub-block) label; reading through the pointers returns the
    labels in block-major order from the skip on."""
    bpc, page, pad, n_blocks, skip = 4, 64, 40, 9, 2
    buf = np.zeros((n_blocks, bpc * page + pad), dtype=np.uint8)
    for b in range(n_blocks):
        for j in range(bpc):
            buf[b, j * page:(j + 1) * page] = b * 16 + j
    ids = np.array([7, 0, 3])
    n_out = 3 * bpc - skip
    ptrs = oracle.sub_block_ptrs(buf.ctypes.data, buf.strides[0], page, ids, bpc, skip, n_out)
    labels = [ctypes.string_at(int(p), page) for p in ptrs]
    want = [(b * 16 + j) for b in ids for j in range(bpc)][skip:]
    assert [lab[0] for lab in labels] == want
    assert all(len(set(lab)) == 1 for lab in labels)


def test_sub_block_ptrs_argument_errors():
    with pytest.raises(oracle.OracleError) as e:
        oracle.sub_block_ptrs(0, 128, 32, [1, 2], 4, 4, 1)        # skip == bpc
    assert e.value.code == oracle.EINVAL
    with pytest.raises(oracle.OracleError) as e:
        oracle.sub_block_ptrs(0, 128, 32, [1, 2], 4, 1, 8)        # more than 2*4-1 sub-blocks
    assert e.value.code == oracle.ERANGE
    assert len(oracle.sub_block_ptrs(0, 128, 32, [1, 2], 4, 1, 7)) == 7


@pytest.mark.parametrize("bpc", [1, 2, 4, 8])
def test_chunks_consumed_brute_force(bpc):
    for skip in range(bpc):
        for n in range(0, 40):
            touched = {(skip + o) // bpc for o in range(n)}
            assert oracle.chunks_consumed(n, skip, bpc) == (len(touched) if n else
                                                            (1 if skip else 0))


# ------------------------------------------------------------------------------------------
# O2 swap
# ------------------------------------------------------------------------------------------

def _plane_addrs(arr, ids):
    return (arr.ctypes.data + np.asarray(ids, dtype=np.uint64) * np.uint64(arr.strides[0]))


def test_swap_matches_numpy_fancy_index_and_round_trips():
    g = synth.rng(0, synth.P_MISC, 7)
    n_blocks, page = 64, 512
    host = synth.random_bytes(g, n_blocks * page).reshape(n_blocks, page)
    dev = np.full((n_blocks, page), 0xA5, dtype=np.uint8)
    src_ids = g.permutation(n_blocks)[:20]
    dst_ids = g.permutation(n_blocks)[:20]
    sizes = np.full(20, page, dtype=np.uint64)
    oracle.swap(_plane_addrs(host, src_ids), _plane_addrs(dev, dst_ids), sizes, threads=2)
    ref = np.full((n_blocks, page), 0xA5, dtype=np.uint8)
    ref[dst_ids] = host[src_ids]
    assert np.array_equal(dev, ref)
    # store back into a canary plane at the original ids: round trip is the identity there
    back = np.full((n_blocks, page), 0x5A, dtype=np.uint8)
    oracle.swap(_plane_addrs(dev, dst_ids), _plane_addrs(back, src_ids), sizes)
    assert np.array_equal(back[src_ids], host[src_ids])
    untouched = np.setdiff1d(np.arange(n_blocks), src_ids)
    assert (back[untouched] == 0x5A).all()


def test_swap_zero_size_is_noop_and_partial_sizes():
    a = np.arange(100, dtype=np.uint8)
    b = np.zeros(100, dtype=np.uint8)
    oracle.swap([a.ctypes.data, a.ctypes.data + 10], [b.ctypes.data, b.ctypes.data + 50],
                [0, 7])
    ref = np.zeros(100, dtype=np.uint8)
    ref[50:57] = a[10:17]
    assert np.array_equal(b, ref)


def test_disjointness_checker_brute_force():
    g = synth.rng(0, synth.P_MISC, 8)
    for trial in range(300):
        n = 4
        src = g.integers(0, 60, n).astype(np.uint64) + 1000
        dst = g.integers(0, 60, n).astype(np.uint64)
        sizes = g.integers(0, 12, n).astype(np.uint64)
        if trial % 3 == 0:
            dst = dst + 1000                 # can hit sources
        cover = {}
        clash = False
        for i in range(n):
            for x in range(int(dst[i]), int(dst[i] + sizes[i])):
                if x in cover:
                    clash = True
                cover[x] = i
        src_bytes = {x for i in range(n) for x in range(int(src[i]), int(src[i] + sizes[i]))}
        clash = clash or bool(src_bytes & set(cover))
        rc = oracle.check_disjoint(src, dst, sizes)
        assert (rc == oracle.EOVERLAP) == clash


# ------------------------------------------------------------------------------------------
# O3 scoring + top-k
# ------------------------------------------------------------------------------------------

def test_index_scores_one_hot_exact():
    n_blocks, d = 300, 128
    c = np.linspace(-3, 3, n_blocks).astype(np.float16)
    pooled = np.zeros((n_blocks, d), dtype=np.float16)
    pooled[:, 0] = c
    q = np.zeros((2, d), dtype=np.float16)
    q[0, 0] = 1
    q[1, 5] = 1
    s = oracle.index_scores(pooled.view(np.uint16), q.view(np.uint16))
    assert np.array_equal(s[0], c.astype(np.float64))
    assert (s[1] == 0).all()


def test_index_scores_small_integers_equal_numpy_matmul():
    """Small-integer fp16 inputs make every partial sum exact, so any summation order (numpy's
    matmul included) gives the same fp64 value."""
    g = synth.rng(0, synth.P_MISC, 9)
    pooled = g.integers(-8, 9, size=(257, 128)).astype(np.float16)
    q = g.integers(-8, 9, size=(8, 128)).astype(np.float16)
    s = oracle.index_scores(pooled.view(np.uint16), q.view(np.uint16))
    assert np.array_equal(s, q.astype(np.float64) @ pooled.astype(np.float64).T)


def test_index_scores_gaussian_close_to_numpy_matmul():
    g = synth.rng(0, synth.P_MISC, 10)
    pooled = synth.f16_normal(g, (1000, 128))
    q = synth.f16_normal(g, (8, 128))
    s = oracle.index_scores(pooled, q)
    ref = q.view(np.float16).astype(np.float64) @ pooled.view(np.float16).astype(np.float64).T
    assert np.max(np.abs(s - ref)) < 1e-12


def _lexsort_topk(scores, k):
    n_sel, n = scores.shape
    out = np.full((n_sel, k), -1, dtype=np.int32)
    for h in range(n_sel):
        s = scores[h]
        key = np.where(np.isnan(s), np.inf, -s)      # NaN after every number
        order = np.lexsort((np.arange(n), key))       # primary: -score, secondary: id
        take = np.sort(order[:min(k, n)])
        out[h, :len(take)] = take
    return out


@pytest.mark.parametrize("n,k", [(1, 1), (5, 32), (32, 32), (100, 32), (4096, 32), (777, 7)])
def test_topk_matches_lexsort_with_ties_and_nans(n, k):
    g = synth.rng(0, synth.P_MISC, n + k)
    s = g.integers(-5, 6, size=(3, n)).astype(np.float64)   # many exact ties
    s[1] = g.standard_normal(n)
    s[2, g.integers(0, n, size=max(1, n // 10))] = np.nan
    got = oracle.topk(s, k)
    assert np.array_equal(got, _lexsort_topk(s, k))


def test_topk_tie_rule_prefers_lower_id():
    s = np.zeros((1, 10))
    assert oracle.topk(s, 3).tolist() == [[0, 1, 2]]
    s[0, 7] = 1.0
    assert oracle.topk(s, 3).tolist() == [[0, 1, 7]]


# ------------------------------------------------------------------------------------------
# O4 gather / O5 stage tail
# ------------------------------------------------------------------------------------------

def test_gather_all_blocks_is_head_major_transpose():
    """Token-major planes: gathering every block in order is numpy's transpose to head-major."""
    g = synth.rng(0, synth.P_MISC, 11)
    n_tok, kvh, hd, bt = 256, 4, 16, 64
    k = synth.random_u16(g, (n_tok, kvh, hd))
    v = synth.random_u16(g, (n_tok, kvh, hd))
    ids = np.tile(np.arange(n_tok // bt, dtype=np.int32), (kvh, 1))
    ko, vo = oracle.gather(k.view(np.uint8), v.view(np.uint8), n_tok // bt, kvh, hd, 2,
                           oracle.token_major_strides(kvh, hd, 2, bt), ids, bt)
    assert np.array_equal(ko.view(np.uint16).reshape(kvh, n_tok, hd), k.transpose(1, 0, 2))
    assert np.array_equal(vo.view(np.uint16).reshape(kvh, n_tok, hd), v.transpose(1, 0, 2))


def test_gather_block_head_major_layout_is_numpy_transpose():
    """[block][head][token][dim] planes: gathering every block in order is numpy's transpose."""
    g = synth.rng(0, synth.P_MISC, 19)
    nb, kvh, hd, bt = 5, 3, 16, 8
    k = synth.random_u16(g, (nb, kvh, bt, hd))
    ids = np.tile(np.arange(nb, dtype=np.int32), (kvh, 1))
    ko, _ = oracle.gather(k.view(np.uint8), k.view(np.uint8), nb, kvh, hd, 2,
                          oracle.block_head_major_strides(kvh, hd, 2, bt), ids, bt)
    assert np.array_equal(ko.view(np.uint16).reshape(kvh, nb * bt, hd),
                          k.transpose(1, 0, 2, 3).reshape(kvh, nb * bt, hd))
    # the same bytes viewed token-major vs head-major give different gathers unless kvh == 1
    tm, _ = oracle.gather(k.view(np.uint8), k.view(np.uint8), nb, kvh, hd, 2,
                          oracle.token_major_strides(kvh, hd, 2, bt), ids, bt)
    assert not np.array_equal(tm, ko)


def test_gather_random_ids_padded_rows_and_block_table():
    g = synth.rng(0, synth.P_MISC, 12)
    n_blocks, bt, kvh, hd, pad = 20, 8, 3, 32, 48
    n_tok = n_blocks * bt
    row = kvh * hd * 2
    kbuf = synth.random_bytes(g, n_tok * (row + pad)).reshape(n_tok, row + pad)
    vbuf = synth.random_bytes(g, n_tok * (row + pad)).reshape(n_tok, row + pad)
    table = g.permutation(n_blocks).astype(np.int32)
    ids = np.stack([np.sort(g.permutation(n_blocks)[:5]) for _ in range(kvh)]).astype(np.int32)
    ids[1, 3:] = -1
    canary = np.full((kvh, 5 * bt, hd * 2), 0xEE, dtype=np.uint8)
    ko, vo = oracle.gather(kbuf, vbuf, n_blocks, kvh, hd, 2,
                           oracle.token_major_strides(kvh, hd, 2, bt, row + pad), ids, bt,
                           block_table=table, k_out=canary.copy(), v_out=canary.copy())
    k4 = kbuf[:, :row].reshape(n_blocks, bt, kvh, hd * 2)
    v4 = vbuf[:, :row].reshape(n_blocks, bt, kvh, hd * 2)
    for h in range(kvh):
        for i in range(5):
            sl = slice(i * bt, (i + 1) * bt)
            if ids[h, i] < 0:
                assert (ko[h, sl] == 0xEE).all() and (vo[h, sl] == 0xEE).all()
            else:
                assert np.array_equal(ko[h, sl], k4[table[ids[h, i]], :, h])
                assert np.array_equal(vo[h, sl], v4[table[ids[h, i]], :, h])


def test_gather_out_of_range_block_is_an_error():
    k = np.zeros(64 * 16, dtype=np.uint8)
    with pytest.raises(oracle.OracleError) as e:
        oracle.gather(k, k, 1, 1, 8, 2, oracle.token_major_strides(1, 8, 2, 64),
                      np.array([[1]]), 64)
    assert e.value.code == oracle.ERANGE


def test_stage_tail_is_numpy_slice():
    g = synth.rng(0, synth.P_MISC, 13)
    plane = synth.random_bytes(g, 1000 * 34).reshape(1000, 34)
    st = oracle.stage_tail(plane, 34, 613, 1000)
    assert np.array_equal(st.reshape(-1, 34), plane[613:])
    assert oracle.stage_tail(plane, 34, 1000, 1000).size == 0


# ------------------------------------------------------------------------------------------
# O6 decode attention / O7 prefill attention, against torch's fp64 SDPA on the CPU
# ------------------------------------------------------------------------------------------

def _to_f64(bits, fmt):
    if fmt == oracle.F16:
        return torch.from_numpy(bits.view(np.float16).astype(np.float64))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()


def _sdpa(q, k, v, scale, mask=None):
    """q [H][Lq][d], k/v [H][Lk][d] fp64 -> torch's reference attention."""
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)


@pytest.mark.parametrize("fmt", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("n_qh,kvh", [(8, 8), (64, 8), (6, 2)])
def test_decode_matches_torch_sdpa(fmt, n_qh, kvh):
    g = synth.rng(0, synth.P_MISC, 14 + n_qh)
    hd, n_kv = 64, 150
    gen = synth.bf16_normal if fmt == oracle.BF16 else synth.f16_normal
    q, k, v = gen(g, (n_qh, hd)), gen(g, (kvh, n_kv, hd)), gen(g, (kvh, n_kv, hd))
    scale = 1 / math.sqrt(hd)
    out = oracle.attn_decode(q, k, v, fmt, scale)
    G = n_qh // kvh
    kk = _to_f64(k, fmt).repeat_interleave(G, 0)
    vv = _to_f64(v, fmt).repeat_interleave(G, 0)
    ref = _sdpa(_to_f64(q, fmt)[:, None, :], kk, vv, scale)[:, 0, :]
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def test_decode_special_cases():
    g = synth.rng(0, synth.P_MISC, 15)
    hd, n_kv = 32, 40
    q = synth.bf16_normal(g, (4, hd))
    v = synth.bf16_normal(g, (2, n_kv, hd))
    krow = synth.bf16_normal(g, (1, 1, hd))
    k_equal = np.repeat(np.repeat(krow, n_kv, 1), 2, 0)
    out = oracle.attn_decode(q, k_equal, v, oracle.BF16, 0.1)
    mean_v = _to_f64(v, oracle.BF16).numpy().mean(axis=1)
    assert np.allclose(out, np.repeat(mean_v, 2, 0), rtol=0, atol=1e-14)
    # one valid key -> exactly that value row; no valid key -> zeros
    k = synth.bf16_normal(g, (2, n_kv, hd))
    out = oracle.attn_decode(q, k, v, oracle.BF16, 0.1, n_valid=[1, 0])
    assert np.array_equal(out[:2], np.repeat(_to_f64(v[0, :1], oracle.BF16).numpy(), 2, 0))
    assert (out[2:] == 0).all()
    # permuting keys together with their values leaves the output unchanged
    p = g.permutation(n_kv)
    a = oracle.attn_decode(q, k, v, oracle.BF16, 0.1)
    b = oracle.attn_decode(q, k[:, p], v[:, p], oracle.BF16, 0.1)
    assert np.max(np.abs(a - b)) < 1e-13


@pytest.mark.parametrize("with_table", [False, True])
def test_gather_attn_decode_is_sdpa_over_valid_slots(with_table):
    """The selected blocks' tokens read by numpy fancy indexing from a token-major plane, slots
    with ids outside [0, n_blocks) (or table entries outside it) dropped, torch SDPA in fp64."""
    g = synth.rng(0, synth.P_MISC, 40 + with_table)
    kvh, hd, bt, n_blocks, kk, G = 2, 32, 4, 10, 5, 3
    planes = synth.bf16_normal(g, (2, n_blocks * bt, kvh, hd))
    q = synth.bf16_normal(g, (kvh * G, hd))
    ids = np.array([[3, -1, 7, 12, 0], [9, 2, 2, -5, 6]], dtype=np.int32)
    table = None
    if with_table:
        table = g.permutation(n_blocks).astype(np.int32)
        table[6] = n_blocks + 1                      # a table entry outside the planes
    strides = oracle.token_major_strides(kvh, hd, 2, bt)
    out, _, _ = oracle.gather_attn_decode(q, planes[0].view(np.uint8), planes[1].view(np.uint8),
                                          n_blocks, kvh, hd, oracle.BF16, strides, ids, bt, 0.3,
                                          block_table=table)
    for h in range(kvh):
        toks = []
        for b in ids[h]:
            if not 0 <= b < n_blocks:
                continue
            p = b if table is None else table[b]
            if not 0 <= p < n_blocks:
                continue
            toks += list(range(p * bt, p * bt + bt))
        kk_ = _to_f64(planes[0][toks, h], oracle.BF16)[None]
        vv_ = _to_f64(planes[1][toks, h], oracle.BF16)[None]
        qq = _to_f64(q[h * G:(h + 1) * G], oracle.BF16)[None]
        ref = _sdpa(qq, kk_, vv_, 0.3)[0].numpy()
        assert np.max(np.abs(out[h * G:(h + 1) * G] - ref)) < 1e-12


def test_qsa_selection_geometry_worked_values():
    """K_pad and the expanded positions against values worked from the page's definitions."""
    g = json.load(open(os.path.join(GOLDEN, "qsa_positions_worked.json")))
    for c in g["k_pad_cases"]:
        assert oracle.qsa_k_pad(c["block_topk"], c["cr"]) == c["k_pad"]
    c = g["positions_case"]
    got = oracle.select_positions(np.array(c["ids"]), c["cr"], c["n_tok"], c["k_pad"])
    assert got.tolist() == c["expected"]


def test_select_positions_properties():
    """Random selections: valid positions are exactly the union of the blocks' token ranges and
    the tail, strictly ascending, each below n_tok; the rest is -1."""
    g = synth.rng(0, synth.P_MISC, 50)
    for cr, n_tok, k in [(4, 1003, 40), (4, 1000, 40), (1, 77, 10), (64, 64 * 20 + 5, 7)]:
        n_blocks = n_tok // cr
        ids = np.stack([np.sort(g.permutation(n_blocks)[:min(k, n_blocks)]) for _ in range(3)])
        ids = np.concatenate([ids, np.full((3, k - ids.shape[1]), -1)], axis=1)
        ids[1, k // 2:] = -1                                   # fewer valid blocks
        k_pad = oracle.qsa_k_pad(k, cr)
        pos = oracle.select_positions(ids, cr, n_tok, k_pad)
        for h in range(3):
            want = sorted({int(b) * cr + r for b in ids[h] if b >= 0 for r in range(cr)} |
                          set(range(n_tok // cr * cr, n_tok)))
            v = pos[h][pos[h] >= 0]
            assert v.tolist() == want
            assert (pos[h][len(v):] == -1).all() and (v < n_tok).all()


def _dequant_q8_0_numpy(rows, kvh, hd):
    """Independent decode of q8_0 rows with numpy dtypes: [n][kvh][hd] float64."""
    n = rows.shape[0]
    blk = rows.reshape(n, kvh * hd // 32, 34)
    scale = blk[:, :, :2].copy().view(np.float16).astype(np.float64)   # [n][nb][1]
    qv = blk[:, :, 2:].view(np.int8).astype(np.float64)                 # [n][nb][32]
    return (scale * qv).reshape(n, kvh, hd)


def test_q8_0_hand_built_block():
    """One head, 32 dims: scale 0.5 (fp16 0x3800), q = 0, 1, -1, 2, ..., -127 pattern."""
    qs = np.array([0, 1, -1, 2, -2, 3, 127, -127] * 4, dtype=np.int8)
    row = np.concatenate([np.array([0x00, 0x38], dtype=np.uint8), qs.view(np.uint8)])[None, :]
    zero_q = np.zeros((1, 1, 32), dtype=np.uint16)
    # a query that picks dim d: with a single key, attention returns V itself, so use V = row
    for d in (0, 3, 6, 7, 31):
        q = np.zeros((1, 1, 32), dtype=np.float16)
        out = oracle.attn_prefill(q.view(np.uint16), 0, 1, row, row, 1, row, row, 1,
                                  oracle.Q8_0, True, 1.0)
        assert out[0, 0, d] == 0.5 * float(qs[d])
    assert zero_q.sum() == 0


@pytest.mark.parametrize("fmt", [oracle.Q8_0, oracle.F16, oracle.BF16])
def test_prefill_matches_torch_sdpa_with_bottom_right_causal_mask(fmt):
    g = synth.rng(0, synth.P_MISC, 16)
    kvh, n_qh, hd, n_kv, n_q = 2, 8, 64, 300, 37
    q_pos0 = n_kv - n_q
    if fmt == oracle.Q8_0:
        k = synth.q8_0_rows(g, n_kv, kvh, hd)
        v = synth.q8_0_rows(g, n_kv, kvh, hd)
        kd, vd = _dequant_q8_0_numpy(k, kvh, hd), _dequant_q8_0_numpy(v, kvh, hd)
    elif fmt == oracle.F16:
        k = synth.f16_normal(g, (n_kv, kvh * hd)).view(np.uint8).reshape(n_kv, -1)
        v = synth.f16_normal(g, (n_kv, kvh * hd)).view(np.uint8).reshape(n_kv, -1)
        kd = k.view(np.float16).astype(np.float64).reshape(n_kv, kvh, hd)
        vd = v.view(np.float16).astype(np.float64).reshape(n_kv, kvh, hd)
    else:
        k = synth.bf16_normal(g, (n_kv, kvh * hd)).view(np.uint8).reshape(n_kv, -1)
        v = synth.bf16_normal(g, (n_kv, kvh * hd)).view(np.uint8).reshape(n_kv, -1)
        kd = _to_f64(k.view(np.uint16), oracle.BF16).numpy().reshape(n_kv, kvh, hd)
        vd = _to_f64(v.view(np.uint16), oracle.BF16).numpy().reshape(n_kv, kvh, hd)
    q = synth.f16_normal(g, (n_q, n_qh, hd))
    scale = 1 / math.sqrt(hd)
    n_head = 123
    out = oracle.attn_prefill(q, q_pos0, kvh, k, v, n_head, k[n_head:], v[n_head:], n_kv, fmt,
                              True, scale)
    G = n_qh // kvh
    qt = torch.from_numpy(q.view(np.float16).astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(kd).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(vd).permute(1, 0, 2).repeat_interleave(G, 0)
    pos = q_pos0 + torch.arange(n_q)[:, None]
    mask = torch.arange(n_kv)[None, :] <= pos
    ref = _sdpa(qt, kt, vt, scale, mask).permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12


def test_prefill_tier_split_is_invisible_and_rows_subset():
    g = synth.rng(0, synth.P_MISC, 17)
    kvh, n_qh, hd, n_kv, n_q = 2, 4, 32, 200, 16
    k = synth.q8_0_rows(g, n_kv, kvh, hd)
    v = synth.q8_0_rows(g, n_kv, kvh, hd)
    q = synth.f16_normal(g, (n_q, n_qh, hd))
    full = oracle.attn_prefill(q, n_kv - n_q, kvh, k, v, n_kv, k[:0], v[:0], n_kv, oracle.Q8_0,
                               True, 0.2)
    for n_head in (0, 1, 77, 199):
        t = oracle.attn_prefill(q, n_kv - n_q, kvh, k[:n_head], v[:n_head], n_head, k[n_head:],
                                v[n_head:], n_kv, oracle.Q8_0, True, 0.2)
        assert np.array_equal(t, full)
    part = oracle.attn_prefill(q, n_kv - n_q, kvh, k, v, n_kv, k[:0], v[:0], n_kv, oracle.Q8_0,
                               True, 0.2, t_begin=5, t_end=9)
    assert np.array_equal(part, full[5:9])


def test_prefill_single_query_reduces_to_decode():
    """n_q = 1 at position p: prefill over keys [0, p] equals decode over the same keys laid out
    head-major (both fp16)."""
    g = synth.rng(0, synth.P_MISC, 18)
    kvh, n_qh, hd, n_kv = 2, 4, 32, 90
    kb = synth.f16_normal(g, (n_kv, kvh, hd))
    vb = synth.f16_normal(g, (n_kv, kvh, hd))
    q = synth.f16_normal(g, (1, n_qh, hd))
    p = 60
    pre = oracle.attn_prefill(q, p, kvh, kb.view(np.uint8).reshape(n_kv, -1),
                              vb.view(np.uint8).reshape(n_kv, -1), n_kv, None, None, n_kv,
                              oracle.F16, True, 0.3)
    dec = oracle.attn_decode(q[0], kb[:p + 1].transpose(1, 0, 2), vb[:p + 1].transpose(1, 0, 2),
                             oracle.F16, 0.3)
    assert np.max(np.abs(pre[0] - dec)) < 1e-14


def test_paged_write_worked_example():
    """Row placement through the block table against a hand-worked example."""
    g = json.load(open(os.path.join(GOLDEN, "paged_write_worked.json")))
    ps, n_pages, seq = g["page_size"], g["n_pages"], g["seq"]
    lens = g["cache_seqlens"]
    bsz = len(lens)
    plane = np.zeros((n_pages, ps, 1), np.uint8)
    rows = np.array([[[10 * b + t + 1] for t in range(seq)] for b in range(bsz)], np.uint8)
    oracle.paged_write([plane], [rows], lens, np.array(g["block_table"]), ps)
    assert plane[:, :, 0].tolist() == g["expected_pages"]


def test_paged_write_identity_table_is_contiguous_append():
    """With page i of sequence b at table[b][i] = b*pps + i, a sequence's pages are one
    contiguous array, and the write is a plain slice assignment at its length."""
    g = synth.rng(0, synth.P_MISC, 60)
    ps, pps, bsz, rb = 16, 5, 3, 8
    plane = g.integers(0, 256, size=(bsz * pps, ps, rb), dtype=np.uint8)
    lens = np.array([0, 17, 40])
    seq = 23
    rows = g.integers(0, 256, size=(bsz, seq, rb), dtype=np.uint8)
    want = plane.reshape(bsz, pps * ps, rb).copy()
    for b in range(bsz):
        want[b, lens[b]:lens[b] + seq] = rows[b]
    table = np.arange(bsz * pps).reshape(bsz, pps)
    oracle.paged_write([plane], [rows], lens, table, ps)
    assert np.array_equal(plane.reshape(bsz, pps * ps, rb), want)


def test_copy_page_counts_and_untouched_rows():
    """copy_page moves rows [0, n) of each plane and ceil(n / cr) pooled rows; the rest of
    the target page and every other page stay as they were."""
    g = synth.rng(0, synth.P_MISC, 61)
    k = g.integers(0, 256, size=(4, 8, 6), dtype=np.uint8)
    pooled = g.integers(0, 256, size=(4, 4, 3), dtype=np.uint8)      # cr = 2: 4 rows per page
    k0, p0 = k.copy(), pooled.copy()
    oracle.copy_page([k], [k], 1, 3, 5, pooled, pooled, cr=2)
    assert np.array_equal(k[3, :5], k0[1, :5]) and np.array_equal(k[3, 5:], k0[3, 5:])
    assert np.array_equal(pooled[3, :3], p0[1, :3]) and np.array_equal(pooled[3, 3:], p0[3, 3:])
    assert np.array_equal(k[:3], k0[:3]) and np.array_equal(pooled[:3], p0[:3])


@pytest.mark.parametrize("table_kind", ["per_row", "shared", "none"])
def test_sparse_attend_rows_is_sdpa_over_valid_positions(table_kind):
    """Each row's valid positions mapped to physical rows with numpy array arithmetic (a
    vectorised mask, not the oracle's per-position loop), the K/V rows picked by fancy
    indexing from a [row][head][dim] view, torch SDPA in fp64 per row."""
    g = synth.rng(0, synth.P_MISC, 70 + len(table_kind))
    kvh, hd, G, ps, n_pages, R, k_pad = 2, 32, 3, 4, 12, 4, 14
    n_rows = n_pages * ps
    planes = synth.bf16_normal(g, (2, n_rows, kvh, hd))
    q = synth.bf16_normal(g, (R, kvh * G, hd))
    cols = 6
    if table_kind == "none":
        table = None
        pos = g.integers(-3, n_rows + 5, size=(R, k_pad))
    else:
        nt = R if table_kind == "per_row" else 1
        table = np.stack([g.permutation(n_pages)[:cols] for _ in range(nt)]).astype(np.int32)
        table[0, 2] = -1                       # a hole
        table[-1, 4] = n_pages + 3             # outside the pool
        pos = g.integers(-3, cols * ps + 6, size=(R, k_pad))
    pos[1, 5:] = -1
    out = oracle.sparse_attend_rows(q, planes[0].view(np.uint8), planes[1].view(np.uint8),
                                    n_rows, kvh * hd * 2, hd * 2, kvh, oracle.BF16, pos, 0.25,
                                    block_table=table, page_size=ps)
    for r in range(R):
        p = pos[r]
        if table is None:
            ok = (p >= 0) & (p < n_rows)
            phys = p
        else:
            t = table[r if table.shape[0] > 1 else 0]
            pg = np.clip(p // ps, 0, cols - 1)
            e = t[pg].astype(np.int64)
            phys = e * ps + p % ps
            ok = (p >= 0) & (p < cols * ps) & (e >= 0) & (phys < n_rows)
        sel = phys[ok]
        for h in range(kvh):
            kk_ = _to_f64(planes[0][sel, h], oracle.BF16)[None]
            vv_ = _to_f64(planes[1][sel, h], oracle.BF16)[None]
            qq = _to_f64(q[r, h * G:(h + 1) * G], oracle.BF16)[None]
            if sel.size == 0:
                assert (out[r, h * G:(h + 1) * G] == 0).all()
                continue
            ref = _sdpa(qq, kk_, vv_, 0.25)[0].numpy()
            assert np.max(np.abs(out[r, h * G:(h + 1) * G] - ref)) < 1e-12


def test_staging_worthwhile_page_examples():
    """QSA KV offload, qsa_staging_worthwhile's docstring: a 2048-row prefill chunk with 2080
    selections per row against a history of ~4096 pages sits on the staging side; a one-row
    decode does not.  The comparison is strict."""
    assert oracle.staging_worthwhile(2048, 2080, 4096, 256)
    assert not oracle.staging_worthwhile(1, 2080, 4096, 256)
    assert not oracle.staging_worthwhile(1024, 1024, 2048, 256)     # equal: not worthwhile
    assert oracle.staging_worthwhile(1025, 1024, 2048, 256)


# ---------------------------------------------------------------------------------------------
# pool rebuild at the write head (QSA KV offload, CacheLayer_qsa_offload docstring)
# ---------------------------------------------------------------------------------------------

def test_f64_to_f16_matches_numpy_on_every_midpoint_and_random_values():
    """The oracle's rounding against numpy's float64 -> float16 cast: every finite fp16 value,
    every midpoint between neighbours (the ties), values a hair either side of them, and
    random doubles over all binades, signed."""
    pos = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2
    xs = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                         [65504.0, 65519.999, 65520.0, 1e9, 2.0 ** -25, 2.0 ** -26]])
    g = synth.rng(0, synth.P_MISC, 616)
    xs = np.concatenate([xs, g.standard_normal(20000) * np.exp2(g.integers(-30, 17, 20000))])
    xs = np.concatenate([xs, -xs])
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f64_to_f16(x) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert oracle.f64_to_f16(float("inf")) == 0x7C00 and oracle.f64_to_f16(float("-inf")) == 0xFC00
    assert oracle.f64_to_f16(float("nan")) & 0x7C00 == 0x7C00


def _pool_fixture(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_pool_rebuild_worked_example():
    w = _pool_fixture("pool_rebuild_worked.json")
    ps, cr, dim, n_pages = w["page_size"], w["cr"], w["dim"], w["n_pages"]
    raw = np.zeros((n_pages, ps, dim), dtype=np.float16)
    for r in w["raw_rows"]:
        raw[r["page"], r["row"]] = r["values"]
    pooled = np.full((n_pages, ps // cr, dim), w["pooled_canary_bits"], dtype=np.uint16)
    oracle.pool_rebuild(raw.view(np.uint16), pooled, w["cache_seqlens"], w["seq"],
                        w["block_table"], ps, cr)
    want = np.full_like(pooled, w["pooled_canary_bits"])
    for e in w["expected_pooled"]:
        want[e["page"], e["row"]] = e["bits"]
    assert np.array_equal(pooled, want)
    # the partial block of three rows
    pooled[:] = w["pooled_canary_bits"]
    oracle.pool_rebuild(raw.view(np.uint16), pooled, [-1, 0, -1], 3, w["block_table"], ps, cr)
    assert list(pooled[1, 0]) == w["partial_three_rows"]["bits"]


def test_pool_rebuild_closed_form_on_symmetric_blocks():
    """Rows c + delta*(-3, -1, 1, 3) (all exact in fp16) average to c exactly, whatever c and
    delta are; every touched block of every sequence must come out as c."""
    cr, ps, dim, n_pages = 4, 16, 8, 12
    g = synth.rng(0, synth.P_MISC, 617)
    # c: multiples of 2^-4 in [-8, 8]; delta: 2^-4 .. 2^-1.  Every row is then a multiple of
    # 2^-4 below 10 in magnitude (at most 8 significant bits), exact in fp16
    c = g.integers(-128, 129, (n_pages, ps // cr, dim)) / 16.0
    delta = np.exp2(g.integers(-4, 0, (n_pages, ps // cr, dim)))
    raw = np.empty((n_pages, ps, dim), dtype=np.float16)
    for k, f in enumerate((-3, -1, 1, 3)):
        raw[:, k::cr] = (c + f * delta).astype(np.float16)
    exact = np.array([(c + f * delta).astype(np.float16).astype(np.float64) for f in (-3, -1, 1, 3)])
    assert np.array_equal(exact.mean(0), c), "construction: rows representable, mean exact"
    table = synth.permutation(synth.rng(0, synth.P_PERM_DST, 617), n_pages).reshape(4, 3)
    pooled = np.zeros((n_pages, ps // cr, dim), dtype=np.uint16)
    # each sequence appends its whole 48-token range: every block complete
    oracle.pool_rebuild(raw.view(np.uint16), pooled, [0, 0, 0, 0], 48, table, ps, cr)
    assert np.array_equal(pooled.view(np.float16).astype(np.float64), c)


def test_pool_rebuild_equals_numpy_mean_per_touched_block():
    """Random fp16 keys, sequences at varied lengths (complete and partial write-head
    blocks, appends that span pages, a -1 table entry, a negative length): every touched
    block equals numpy's float64 mean of the block's present rows cast to float16; every
    other pooled row keeps its value."""
    cr, ps, dim, n_pages, pps = 4, 32, 64, 40, 6
    g = synth.rng(0, synth.P_MISC, 618)
    raw = synth.f16_normal(g, (n_pages, ps, dim))
    table = synth.permutation(synth.rng(0, synth.P_PERM_DST, 618), n_pages)[:5 * pps].reshape(5, pps)
    table[3, 2] = -1
    lens = np.array([0, 5, 30, 61, -1], dtype=np.int32)
    for seq in (1, 3, 7, 40):
        pooled = synth.f16_normal(synth.rng(0, synth.P_CANARY, seq), (n_pages, ps // cr, dim))
        before = pooled.copy()
        oracle.pool_rebuild(raw, pooled, lens, seq, table, ps, cr)
        want = before.copy()
        for b, ln in enumerate(lens):
            if ln < 0:
                continue
            for j in range(ln // cr, (ln + seq - 1) // cr + 1):
                slot = j * cr // ps
                if slot >= pps or table[b, slot] < 0:
                    continue
                page, row0 = table[b, slot], j * cr % ps
                rows = min(cr, ln + seq - j * cr)
                vals = raw[page, row0:row0 + rows].view(np.float16).astype(np.float64)
                want[page, row0 // cr] = vals.mean(0).astype(np.float16).view(np.uint16)
        assert np.array_equal(pooled, want), seq


def test_pool_rebuild_argument_errors():
    raw = np.zeros((2, 8, 4), dtype=np.uint16)
    pooled = np.zeros((2, 2, 4), dtype=np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.pool_rebuild(raw, pooled, [0], 1, [[0]], 8, 3)     # cr does not divide page_size
