"""Seeded synthetic inputs shaped like the workloads on the pages.

This module holds input generation only -- no step of the method (no pointer arithmetic, no
scoring, no selection, no copy, no attention).  Both the tests/bench (for the HIP path) and the
oracle take their inputs from here, so the two sides see identical bytes.

Seeds follow one rule: ``np.random.default_rng([cfg, purpose, step])`` with ``cfg`` the workload
number (1 = one-layer swap, 2 = 32-layer swap, 3 = small pages, 4 = top-k decode, 5 = tiered
prefill, 0 = unit tests) and ``purpose`` one of the ids below.
"""
from __future__ import annotations

import numpy as np

# purpose ids
P_K, P_V, P_POOLED, P_QIDX, P_Q, P_PERM_SRC, P_PERM_DST, P_SKIP, P_CANARY, P_MISC = range(10)


def rng(cfg: int, purpose: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(cfg), int(purpose), int(step)])


def f16_normal(g: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) samples rounded to fp16, returned as their uint16 bit patterns."""
    return g.standard_normal(shape, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_normal(g: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) samples rounded (to nearest, ties to even) to bfloat16, as uint16 bit patterns."""
    x = g.standard_normal(shape, dtype=np.float32).view(np.uint32)
    bias = ((x >> 16) & 1) + np.uint32(0x7FFF)
    return ((x + bias) >> 16).astype(np.uint16)


def random_u16(g: np.random.Generator, shape) -> np.ndarray:
    """Uniform random 16-bit patterns (includes NaN/Inf encodings): a pure byte workload."""
    return g.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def random_bytes(g: np.random.Generator, n: int) -> np.ndarray:
    return g.integers(0, 256, size=n, dtype=np.uint8)


def fill_random_bytes(g: np.random.Generator, out: np.ndarray, chunk: int = 1 << 26) -> None:
    """Fill a (possibly huge) uint8 array in place, chunk by chunk, without a full temporary."""
    flat = out.reshape(-1)
    for o in range(0, flat.size, chunk):
        n = min(chunk, flat.size - o)
        flat[o:o + n] = g.integers(0, 256, size=n, dtype=np.uint8)


def q8_0_encode(x: np.ndarray) -> np.ndarray:
    """Encode float data [n][nb][32] as q8_0 blocks: scale = fp16(max|x| / 127) as 2
    little-endian bytes, then q = clamp(rint(x / scale), -127, 127) as 32 int8.  Returns uint8
    [n][nb][34].  (Input generation only: consumers read the stored bytes.)"""
    x = np.asarray(x, dtype=np.float32)
    n, nb, _ = x.shape
    out = np.empty((n, nb, 34), dtype=np.uint8)
    amax = np.abs(x).max(axis=2)
    d16 = (amax / np.float32(127.0)).astype(np.float16)
    d = d16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.where(d[..., None] > 0, x / d[..., None], 0.0)
    q = np.clip(np.rint(qf), -127, 127).astype(np.int8)
    out[:, :, 0:2] = d16.view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:] = q.view(np.uint8)
    return out


def q8_0_rows(g: np.random.Generator, n_rows: int, kvh: int, hd: int) -> np.ndarray:
    """q8_0 cache rows of N(0,1) data (see q8_0_encode).  A row is kvh heads x hd/32 blocks,
    head-major: kvh * hd/32 * 34 bytes.  Returns uint8 [n_rows][row]."""
    assert hd % 32 == 0
    nb = kvh * (hd // 32)
    out = np.empty((n_rows, nb, 34), dtype=np.uint8)
    step = 1 << 16
    for r0 in range(0, n_rows, step):
        r1 = min(n_rows, r0 + step)
        out[r0:r1] = q8_0_encode(g.standard_normal((r1 - r0, nb, 32), dtype=np.float32))
    return out.reshape(n_rows, nb * 34)


def permutation(g: np.random.Generator, n: int) -> np.ndarray:
    return g.permutation(n).astype(np.int64)
