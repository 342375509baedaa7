"""GPU check of kvt_gather_attn_decode_noalloc, the fused gather + decode attention for callers
that cannot allocate: its split partials live in the library's fixed per-GPU scratch array.

Two calls in a row through the C ABI, the second with a smaller input, each compared bit for
bit with kvt_gather_attn_decode given a caller workspace (same kernels, same arithmetic) and
within 2e-3 of the fp64 oracle; then a size past the scratch is refused and enqueues nothing.
"""
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


def _planes(n_tok, kvh, hd):
    row = kvh * hd * 2
    buf = kvt.HostBuffer(2 * n_tok * row)
    planes = buf.numpy(np.uint16, (2, n_tok, kvh, hd))
    planes[0] = synth.bf16_normal(synth.rng(4, synth.P_K, 4242), (n_tok, kvh, hd))
    planes[1] = synth.bf16_normal(synth.rng(4, synth.P_V, 4242), (n_tok, kvh, hd))
    return buf, planes


def _both_forms(buf, planes, n_tok, kvh, hd, n_qh, bt, k, seed, with_out, dev):
    n_blocks = n_tok // bt
    strides = oracle.token_major_strides(kvh, hd, 2, bt)
    g = synth.rng(4, synth.P_MISC, seed)
    ids = np.stack([np.sort(g.permutation(n_blocks)[:k]) for _ in range(kvh)]).astype(np.int32)
    ids[1, k - 1:] = -1                              # a skipped slot at the end of a head
    q = synth.bf16_normal(synth.rng(4, synth.P_Q, seed), (n_qh, hd))
    ids_d, q_d = torch.from_numpy(ids).to(dev), _u16(q, dev)
    n_kv = k * bt
    outs, kvs = [], []
    for form in ("workspace", "noalloc"):
        out = torch.full((n_qh, hd), float("nan"), dtype=torch.float32, device=dev)
        kv = torch.full((2, kvh, n_kv, hd), 0x1234, dtype=torch.int16, device=dev)
        ko, vo = (kv[0], kv[1]) if with_out else (None, None)
        args = (q_d, n_qh, kvh, hd, kvt.BF16, buf.dev, buf.dev + n_tok * kvh * hd * 2, n_blocks,
                *strides, None, bt, ids_d, k, ko, vo, 1 / math.sqrt(hd), out)
        if form == "workspace":
            ws_bytes = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, n_kv)
            ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device=dev)   # NaN patterns
            kvt.kvt_gather_attn_decode(*args, ws, ws_bytes)
        else:
            kvt.kvt_gather_attn_decode_noalloc(*args)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        kvs.append(kv.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "outputs differ"
    assert np.array_equal(kvs[0], kvs[1]), "gathered rows differ"
    ref, _, _ = oracle.gather_attn_decode(q, planes[0].view(np.uint8), planes[1].view(np.uint8),
                                          n_blocks, kvh, hd, oracle.BF16, strides, ids, bt,
                                          1 / math.sqrt(hd))
    assert np.isfinite(outs[1]).all()
    assert np.max(np.abs(outs[1] - ref)) <= TOL
    return outs[1]


def test_noalloc_decode_two_calls_then_smaller(gpu):
    kvh, hd = 8, 128
    n_tok = 64 * 2000
    buf, planes = _planes(n_tok, kvh, hd)
    assert kvt.kvt_gather_attn_decode_noalloc_max_bytes() == 4 << 20
    # the decode step's shape: 64 query heads, top-32 blocks of 64 tokens, gather buffers given
    _both_forms(buf, planes, n_tok, kvh, hd, 64, 64, 32, 1, True, gpu)
    # a smaller call right after: group 2, blocks of 16 tokens, 5 slots, no gather buffers
    _both_forms(buf, planes, n_tok, kvh, hd, 16, 16, 5, 2, False, gpu)
    # the largest call the scratch takes: 126 chunks of 64 keys for 64 query heads
    _both_forms(buf, planes, n_tok, kvh, hd, 64, 64, 126, 3, False, gpu)
    del planes
    buf.free()


def test_noalloc_decode_refuses_more_than_the_scratch(gpu):
    kvh, hd, bt, k, n_qh = 8, 128, 64, 127, 64     # 127 chunks x 64 heads x 130 x 4 B > 4 MiB
    n_tok = 64 * 300
    buf, planes = _planes(n_tok, kvh, hd)
    ids = torch.zeros((kvh, k), dtype=torch.int32, device=gpu)
    q = torch.zeros((n_qh, hd), dtype=torch.int16, device=gpu)
    out = torch.full((n_qh, hd), 7.0, dtype=torch.float32, device=gpu)
    strides = oracle.token_major_strides(kvh, hd, 2, bt)
    with pytest.raises(kvt.KvtError) as e:
        kvt.kvt_gather_attn_decode_noalloc(q, n_qh, kvh, hd, kvt.BF16, buf.dev,
                                           buf.dev + n_tok * kvh * hd * 2, n_tok // bt, *strides,
                                           None, bt, ids, k, None, None, 1 / math.sqrt(hd), out)
    assert e.value.code == kvt.ERANGE
    torch.cuda.synchronize()
    assert (out.cpu() == 7.0).all()
    del planes
    buf.free()
