"""CPU-only checks of the engine (SDMA) mode's bookkeeping, with the HSA calls replaced by fakes.

The engine (SDMA) mode of kvt_swap_blocks and kvt_stage_tail submits one DMA-engine copy per
run of adjacent descriptors (a long run cut into pieces of at most max_run bytes), each with a
completion signal of its own (value 1), at most `window` in flight, waited for oldest first;
every signal is destroyed at the end.  tests/engine_runs_check.cpp drives that code
(hbm_kv_cache_amd/csrc/kvt_engine_runs.h, compiled with g++) against fake operations that
report any rule broken: a copy given a signal whose value is not 1, a wait on a signal with
no copy in flight (which would never return on an engine), a reset or destroy while a copy
is in flight, out-of-order waits, signals left alive.  The copies it submits, applied to a
host buffer, must equal the oracle's memcpy loop over the same descriptors.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from hbm_kv_cache_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "engine_runs_check.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("engine") / "engine_runs_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I",
                    os.path.join(ROOT, "hbm_kv_cache_amd", "csrc"), SRC, "-o", exe], check=True)
    return exe


def _run(exe, src, dst, sizes, window, fail_create=-1, fail_copy=-1, max_run=0):
    lines = [f"{len(src)} {window} {fail_create} {fail_copy} {max_run}"]
    lines += [f"{int(a)} {int(b)} {int(c)}" for a, b, c in zip(src, dst, sizes)]
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         check=True).stdout.splitlines()
    t = list(map(int, out[0].split()[1:]))
    tally = dict(zip(["status", "failed_at", "runs", "created", "submitted", "waited",
                      "destroyed"], t))
    copies = [tuple(map(int, l.split()[1:])) for l in out if l.startswith("C ")]
    bad = [l[2:] for l in out if l.startswith("V ")]
    return tally, copies, bad


def _scattered(n, page, seed, zero_every=0, adjacent=0):
    """Descriptors over a source and a destination arena given as offsets: pages in seeded
    order, or with `adjacent` > 0 groups of that many pages adjacent on both sides (the groups
    in seeded order); every `zero_every`-th descriptor or so gets size 0."""
    g = synth.rng(0, synth.P_MISC, seed)
    if adjacent:
        ng = n // adjacent
        gs = synth.permutation(synth.rng(0, synth.P_PERM_SRC, seed), ng)
        gd = synth.permutation(synth.rng(0, synth.P_PERM_DST, seed), ng)
        i = np.arange(ng * adjacent)
        sp = gs[i // adjacent] * adjacent + i % adjacent
        dp = gd[i // adjacent] * adjacent + i % adjacent
    else:
        sp = synth.permutation(synth.rng(0, synth.P_PERM_SRC, seed), n)
        dp = synth.permutation(synth.rng(0, synth.P_PERM_DST, seed), n)
    sizes = np.full(sp.size, page, dtype=np.uint64)
    if zero_every:
        sizes[g.integers(0, sp.size, sp.size // zero_every)] = 0
    return sp.astype(np.uint64) * page, dp.astype(np.uint64) * page, sizes


def _apply(copies, src_mem, n_bytes):
    out = np.zeros(n_bytes, dtype=np.uint8)
    for d, s, ln in copies:
        out[d:d + ln] = src_mem[s:s + ln]
    return out


def _oracle(src, dst, sizes, src_mem, n_bytes):
    ref = np.zeros(n_bytes, dtype=np.uint8)
    oracle.swap(np.asarray(src, np.uint64) + np.uint64(src_mem.ctypes.data),
                np.asarray(dst, np.uint64) + np.uint64(ref.ctypes.data), sizes)
    return ref


@pytest.mark.parametrize("n,window,zero_every,adjacent", [
    (1, 256, 0, 0),          # one copy
    (300, 256, 0, 0),        # more copies than the window: signals reused
    (1000, 7, 5, 0),         # a small window, zero sizes
    (64, 256, 0, 4),         # runs of four adjacent descriptors merge
    (513, 1, 0, 0),          # window of one: strictly one copy at a time
])
def test_engine_bookkeeping_counts_and_bytes(driver, n, window, zero_every, adjacent):
    page = 64
    src, dst, sizes = _scattered(n, page, n + window, zero_every, adjacent)
    tally, copies, bad = _run(driver, src, dst, sizes, window)
    assert bad == []
    assert tally["status"] == 0 and tally["failed_at"] == 0
    assert tally["submitted"] == tally["runs"] == len(copies)
    assert tally["waited"] == tally["submitted"]
    assert tally["created"] == tally["destroyed"] == min(tally["runs"], window)
    mem = synth.random_bytes(synth.rng(0, synth.P_K, n), n * page)
    assert np.array_equal(_apply(copies, mem, n * page), _oracle(src, dst, sizes, mem, n * page))
    if adjacent:
        assert tally["runs"] < n


def test_engine_bookkeeping_all_zero_sizes(driver):
    tally, copies, bad = _run(driver, [0, 64], [0, 64], [0, 0], 256)
    assert bad == [] and copies == []
    assert tally == {"status": 0, "failed_at": 0, "runs": 0, "created": 0, "submitted": 0,
                     "waited": 0, "destroyed": 0}


@pytest.mark.parametrize("fail_copy,window", [(0, 256), (1, 256), (150, 256), (299, 256),
                                              (40, 16)])
def test_engine_bookkeeping_partial_submit(driver, fail_copy, window):
    """A copy that cannot be submitted stops the submission; the copies already submitted are
    waited for (and only they), and every signal is destroyed."""
    src, dst, sizes = _scattered(300, 64, 11)
    tally, copies, bad = _run(driver, src, dst, sizes, window, fail_copy=fail_copy)
    assert bad == []
    assert tally["status"] == 9 and tally["failed_at"] == 2
    assert tally["submitted"] == fail_copy == len(copies)
    assert tally["waited"] == tally["submitted"]
    assert tally["created"] == tally["destroyed"] == min(300, window)


@pytest.mark.parametrize("fail_create", [0, 1, 200])
def test_engine_bookkeeping_signal_creation_fails(driver, fail_create):
    """A signal that cannot be created: the ones created are destroyed, nothing is submitted."""
    src, dst, sizes = _scattered(300, 64, 12)
    tally, copies, bad = _run(driver, src, dst, sizes, 256, fail_create=fail_create)
    assert bad == [] and copies == []
    assert tally["status"] == 7 and tally["failed_at"] == 1
    assert tally["created"] == tally["destroyed"] == fail_create
    assert tally["submitted"] == tally["waited"] == 0


@pytest.mark.parametrize("sizes,max_run,pieces", [
    ([10 << 20], 4 << 20, [4 << 20, 4 << 20, 2 << 20]),     # one range cut in three
    ([4 << 20], 4 << 20, [4 << 20]),                         # exactly one piece
    ([3 << 20, 0, 3 << 20], 4 << 20, [4 << 20, 2 << 20]),    # an adjacent run, then cut
    ([1000, 24], 512, [512, 512]),                           # the cut ignores descriptor ends
    ([10 << 20], 0, [10 << 20]),                             # 0: runs stay whole
])
def test_engine_runs_cut_into_pieces(driver, sizes, max_run, pieces):
    """Runs longer than max_run go as consecutive pieces of max_run bytes and a remainder; the
    pieces cover the run exactly, in order, and equal the oracle's copy."""
    off = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.uint64)
    dst_off = off + np.uint64(64)
    tally, copies, bad = _run(driver, off, dst_off, np.array(sizes, np.uint64), 256,
                              max_run=max_run)
    assert bad == [] and tally["status"] == 0
    assert [c[2] for c in copies] == pieces
    pos = 0
    for d, s_, ln in copies:
        assert s_ == pos and d == pos + 64
        pos += ln
    total = int(sum(sizes)) + 64
    mem = synth.random_bytes(synth.rng(0, synth.P_K, len(sizes)), total)
    assert np.array_equal(_apply(copies, mem, total),
                          _oracle(off, dst_off, np.array(sizes, np.uint64), mem, total))
