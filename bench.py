#!/usr/bin/env python3
"""Benchmark of the tiered KV-cache hot path on one MI355X.

Headline workload: one top-k sparse decode step at 262,144 tokens of context, batch 1 --
score the pooled indexer plane (fp16 [4096][128], HBM) for 8 KV heads, select the top 32
blocks per head, gather their K/V rows (8 KV heads x 128 dim bf16, 64-token blocks) from pinned
host planes into HBM, and run GQA decode attention for 64 query heads.  Every step uses a fresh
query pair, hence a fresh selection (no host data can be served from GPU caches).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--ctx 262144] [--suite]

Prints ONE JSON line.  ``value`` = host->HBM KV gather GB/s over whole steps (8,388,608 bytes
gathered per step / step time).  ``roofline`` is the gather kernel itself (HIP events on the
launch stream) against the PCIe Gen5 x16 per-direction peak; ``cpu_baseline`` is the CPU
oracle running the same step on the host cores.  ``--suite`` adds the other workloads
(one-layer and 32-layer swaps, the small-page sweep of kernel, DMA-engine and runtime copies,
tiered prefill, and prefill over a chain of layers with the next layer's first bucket prefetched).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

GB = 1e9
# PCIe 5.0 x16 per direction: 32 GT/s x 16 lanes x 128/130 (line code) / 8 bits = 63.0 GB/s
PCIE5_X16_PEAK_GBS = 63.0
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--ctx", type=int, default=262144)
    p.add_argument("--layout", default="token_major",
                   choices=["block_head_major", "token_major"],
                   help="host K/V plane layout: token-major [token][head][dim] as on the pages "
                        "(default), or block-local head-major")
    p.add_argument("--suite", nargs="?", const="all", default=None,
                   help="also measure the other workloads: all, or a comma list of "
                        "prefill, chain, swap1, small, swap32, qsa, decode1m, worker, upkeep, "
                        "rows")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="bound on the CPU-oracle baseline's wall time")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the compact per-config figures (one-layer and 32-layer swaps, "
                        "small pages, decode at 1M, tiered prefill)")
    return p.parse_args()


class Timer:
    """HIP events on the stream the work is launched on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record(self.stream)

    def stop_ms(self):
        self.b.record(self.stream)
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def measure_link_peaks(torch, kvt, dev, host_buf, nbytes, reps=5):
    """Best-of-reps runtime copy (hipMemcpyAsync, which runs a copy of this size on a DMA
    engine) of nbytes between pinned host memory and HBM, both directions."""
    stream = torch.cuda.current_stream()
    hbm = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    t = Timer(torch, stream)
    best_h2d = best_d2h = 0.0
    tb = kvt.HostBuffer(24)
    import numpy as np
    tab = tb.numpy(np.uint64, (3, 1))
    for _ in range(reps):
        t.start()
        kvt.kvt_stage_tail(host_buf.dev, nbytes, 0, 1, hbm, kvt.COPY_RUNTIME)
        best_h2d = max(best_h2d, nbytes / (t.stop_ms() * 1e-3) / GB)
    tab[0, 0], tab[1, 0], tab[2, 0] = hbm.data_ptr(), host_buf.dev, nbytes
    for _ in range(reps):
        t.start()
        kvt.kvt_swap_blocks(tab[0], tab[1], tab[2], 1, kvt.D2H, kvt.COPY_RUNTIME)
        best_d2h = max(best_d2h, nbytes / (t.stop_ms() * 1e-3) / GB)
    # the copy kernel over a span of the gather's per-step size (host -> HBM): it is also the
    # plain copy of known size that scales the gather kernel's FETCH_SIZE / WRITE_SIZE counters
    span = 8 << 20
    best_h2d_k = 0.0
    for _ in range(reps):
        t.start()
        kvt.kvt_stage_tail(host_buf.dev, span, 0, 1, hbm, kvt.COPY_KERNEL)
        best_h2d_k = max(best_h2d_k, span / (t.stop_ms() * 1e-3) / GB)
    # HBM: device-to-device copy of the same buffer size (reads + writes count)
    other = torch.empty_like(hbm)
    best_hbm = 0.0
    for _ in range(reps):
        t.start()
        other.copy_(hbm)
        best_hbm = max(best_hbm, 2 * nbytes / (t.stop_ms() * 1e-3) / GB)
    del hbm, other
    tb.free()
    return {"h2d_sdma_gbs": round(best_h2d, 2), "d2h_sdma_gbs": round(best_d2h, 2),
            "h2d_copy_kernel_8mib_gbs": round(best_h2d_k, 2),
            "hbm_copy_gbs": round(best_hbm, 1), "bytes": nbytes}


class DecodeWorkload:
    """Top-k sparse decode at one context length: all inputs resident before timing starts."""

    KVH, HD, BT, K, NQH = 8, 128, 64, 32, 64

    # (block, head, token) byte strides of the host planes, per layout
    LAYOUTS = {
        # [block][head][token][dim]: each (block, head) is one contiguous 16 KiB run
        "block_head_major": lambda kvh, hd, bt: (kvh * bt * hd * 2, bt * hd * 2, hd * 2),
        # [token][head][dim], the pages' layout: 256-byte runs at a 2 KiB stride
        "token_major": lambda kvh, hd, bt: (bt * kvh * hd * 2, hd * 2, kvh * hd * 2),
    }

    def __init__(self, torch, kvt, synth, dev, ctx, n_sets, layout="block_head_major",
                 mode="fused"):
        import numpy as np
        self.torch, self.kvt, self.dev, self.ctx = torch, kvt, dev, ctx
        self.mode = mode   # "fused": gather + attention in one pass; "staged": three kernels
        kvh, hd, bt, k = self.KVH, self.HD, self.BT, self.K
        self.n_blocks = ctx // bt
        self.row = kvh * hd * 2
        self.layout = layout
        self.strides = self.LAYOUTS[layout](kvh, hd, bt)
        t0 = time.time()
        self.host = kvt.HostBuffer(2 * ctx * self.row)
        planes = self.host.numpy(np.uint16, (2, ctx, kvh, hd))
        for p, purpose in enumerate((synth.P_K, synth.P_V)):
            g = synth.rng(4, purpose, ctx)
            for t0_ in range(0, ctx, 1 << 16):
                t1_ = min(ctx, t0_ + (1 << 16))
                planes[p, t0_:t1_] = synth.bf16_normal(g, (t1_ - t0_, kvh, hd))
        self.planes = planes
        log(f"ctx={ctx}: host K/V planes {2 * ctx * self.row / 2**30:.2f} GiB pinned "
            f"in {time.time() - t0:.1f}s")
        self.pooled_np = synth.f16_normal(synth.rng(4, synth.P_POOLED, ctx), (self.n_blocks, 128))
        self.pooled = torch.from_numpy(self.pooled_np.view(np.int16)).to(dev)
        self.n_sets = n_sets
        self.qidx_np = synth.f16_normal(synth.rng(4, synth.P_QIDX, ctx), (n_sets, kvh, 128))
        self.q_np = synth.bf16_normal(synth.rng(4, synth.P_Q, ctx), (n_sets, self.NQH, hd))
        self.qidx = torch.from_numpy(self.qidx_np.view(np.int16)).to(dev)
        self.q = torch.from_numpy(self.q_np.view(np.int16)).to(dev)
        self.ws_t = kvt.kvt_index_topk_ws_bytes(self.n_blocks, kvh, k)
        self.ws_d = kvt.kvt_attn_decode_ws_bytes(self.NQH, hd, k * bt)
        self.ws = torch.empty(self.ws_t + self.ws_d + 256, dtype=torch.uint8, device=dev)
        self.ids = torch.empty((kvh, k), dtype=torch.int32, device=dev)
        self.kv = torch.empty((2, kvh, k * bt, hd), dtype=torch.int16, device=dev)
        self.out = torch.empty((self.NQH, hd), dtype=torch.float32, device=dev)
        self.scale = 1.0 / math.sqrt(hd)
        self.gather_bytes = 2 * kvh * k * bt * hd * 2   # K and V: 8,388,608 at these shapes

    def topk(self, i):
        kvt = self.kvt
        kvt.kvt_index_topk(self.pooled, self.n_blocks, 128, self.qidx[i % self.n_sets], self.KVH,
                           self.K, self.ids, None, self.ws, self.ws_t)

    def gather(self):
        kvt = self.kvt
        kvt.kvt_gather_blocks(self.host.dev, self.host.dev + self.ctx * self.row, self.n_blocks,
                              self.KVH, self.HD, 2, *self.strides, None, self.BT, self.ids, self.K,
                              self.kv[0], self.kv[1])

    def attend(self, i):
        kvt = self.kvt
        kvt.kvt_attn_decode(self.q[i % self.n_sets], self.NQH, self.KVH, self.HD, kvt.BF16,
                            self.kv[0], self.kv[1], self.K * self.BT, None, self.scale, self.out,
                            self.ws[self.ws_t + 128:], self.ws_d)

    def fused(self, i):
        kvt = self.kvt
        kvt.kvt_gather_attn_decode(self.q[i % self.n_sets], self.NQH, self.KVH, self.HD, kvt.BF16,
                                   self.host.dev, self.host.dev + self.ctx * self.row,
                                   self.n_blocks, *self.strides, None, self.BT, self.ids, self.K,
                                   self.kv[0], self.kv[1], self.scale, self.out,
                                   self.ws[self.ws_t + 128:], self.ws_d)

    def step(self, i):
        self.topk(i)
        if self.mode == "fused":
            self.fused(i)
        else:
            self.gather()
            self.attend(i)

    def parts(self, i):
        """The step's launches as (name, callable) pairs, for per-part event timing."""
        if self.mode == "fused":
            return [("topk", lambda: self.topk(i)), ("gather_attn", lambda: self.fused(i))]
        return [("topk", lambda: self.topk(i)), ("gather", self.gather),
                ("attn", lambda: self.attend(i))]

    def run(self, steps, warmup, base=0):
        """warmup + 2*steps steps on query sets base, base+1, ..."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        warmup += base   # query-set indices below run from base on
        for i in range(base, warmup):
            self.step(i)
        torch.cuda.synchronize()
        # whole-step timing: host clock and events around exactly `steps` steps
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            self.step(warmup + i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = ev0.elapsed_time(ev1)
        # per-part timing pass: events bracketing each launch on the same stream
        names = [n for n, _ in self.parts(0)]
        parts = {n: [] for n in names}
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
               for _ in range(steps)]
        for i in range(steps):
            e = evs[i]
            e[0].record(stream)
            for j, (_, fn) in enumerate(self.parts(warmup + steps + i)):
                fn()
                e[j + 1].record(stream)
        torch.cuda.synchronize()
        for e in evs:
            for j, n in enumerate(names):
                parts[n].append(e[j].elapsed_time(e[j + 1]))
        avg = {k: sum(v) / len(v) for k, v in parts.items()}
        return {"wall_s": wall, "event_ms": ev_ms, "ms_per_step": max(wall * 1e3, ev_ms) / steps,
                "part_ms": avg}

    def free(self):
        self.planes = None
        self.host.free()


ROOT = os.path.dirname(os.path.abspath(__file__))
PMC_RECORD = os.path.join(ROOT, "profiles", "decode_step_262k_pmc.json")


def _pmc_record(kernel):
    """The committed counter record of `kernel`, or None when there is none or it was taken on
    another version of the kernel's source file."""
    import hashlib
    try:
        rec = json.load(open(PMC_RECORD))["kernels"][kernel]
        src = hashlib.sha256(open(os.path.join(ROOT, rec["source"]), "rb").read()).hexdigest()
    except (OSError, ValueError, KeyError, TypeError):
        return None
    return rec if rec.get("source_sha256") == src else None


def kernel_traffic(kernel):
    """Bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE record, each
    counter scaled by what it read for a plain copy kernel of known size."""
    rec = _pmc_record(kernel)
    return rec.get("traffic_bytes_per_launch") if rec else None


def kernel_traffic_ea(kernel):
    """Per-launch bytes of `kernel` by destination, from the L2's external-access request
    counters in the same record: host-link (IO) and HBM (DRAM) reads and writes."""
    rec = _pmc_record(kernel)
    return rec.get("ea_counters_per_launch") if rec else None


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        for l in open("/proc/cpuinfo"):
            if l.lower().startswith("model name"):
                return l.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, seconds):
    """The oracle's decode step (fp64 scoring, full-sort top-k, memcpy gather from the same
    pinned host planes, fp64 attention) on the host cores, for a bounded wall time."""
    import numpy as np
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    threads = min(threads, os.cpu_count() or threads)
    kvh, hd, bt, k = wl.KVH, wl.HD, wl.BT, wl.K
    n = 0
    t0 = time.perf_counter()
    while True:
        i = n % wl.n_sets
        s = oracle.index_scores(wl.pooled_np, wl.qidx_np[i], threads=threads)
        ids = oracle.topk(s, k)
        ko, vo = oracle.gather(wl.planes[0].view(np.uint8), wl.planes[1].view(np.uint8),
                               wl.n_blocks, kvh, hd, 2, wl.strides, ids, bt)
        oracle.attn_decode(wl.q_np[i], ko.view(np.uint16).reshape(kvh, k * bt, hd),
                           vo.view(np.uint16).reshape(kvh, k * bt, hd), oracle.BF16, wl.scale,
                           threads=threads)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or (n >= 3 and el * (n + 1) / n > seconds * 1.5):
            break
    steps_s = n / el
    return {"value": round(wl.gather_bytes * steps_s / GB, 4), "unit": "GB/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle", "steps_per_s": round(steps_s, 3),
            "sample": f"{n} oracle decode steps at {wl.ctx} ctx (fp64 scoring of {wl.n_blocks} "
                      f"blocks x 8 heads, full-sort top-32, memcpy gather of 8 MiB, fp64 GQA "
                      f"attention over 2048 keys x 64 heads) in {el:.1f}s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(each GPU would run its own layers or KV heads over its own host link, with no "
              "exchange inside this path)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from hbm_kv_cache_amd import kvt, synth
    kvt.load()    # no fallback: the HIP library must be there
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    dev = torch.device("cuda:0")
    log("device", torch.cuda.get_device_name(0))

    n_run = args.warmup + 2 * args.steps
    n_other = 5 + 2 * max(20, args.steps // 4)
    wl = DecodeWorkload(torch, kvt, synth, dev, args.ctx, 2 * n_run + n_other, args.layout)
    peaks = measure_link_peaks(torch, kvt, dev, wl.host, 1 << 30)
    log("link peaks", peaks)
    # every run draws its own queries (hence its own selections): no host rows are re-read
    r = wl.run(args.steps, args.warmup, base=0)
    log("decode (fused gather + attention)", r)
    wl.mode = "staged"
    r_staged = wl.run(args.steps, args.warmup, base=n_run)
    wl.mode = "fused"
    log("decode (gather, then attention)", r_staged)
    # the same planes read through the other layout's strides: context for the layout choice
    other = "token_major" if args.layout == "block_head_major" else "block_head_major"
    keep = wl.strides
    wl.strides = wl.LAYOUTS[other](wl.KVH, wl.HD, wl.BT)
    r_other = wl.run(max(20, args.steps // 4), 5, base=2 * n_run)
    wl.strides = keep
    log(f"decode with {other} host planes", r_other)

    def gbs(ms_):
        return round(wl.gather_bytes / (ms_ * 1e-3) / GB, 3)

    ms = r["ms_per_step"]
    kern_ms = r["part_ms"]["gather_attn"]
    achieved = wl.gather_bytes / (kern_ms * 1e-3) / GB
    value = wl.gather_bytes / (ms * 1e-3) / GB
    line = {
        "metric": "host->HBM KV gather GB/s (% PCIe peak); tiered decode tok/s at 262k ctx",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V in pinned host memory, fp16 pooled plane)",
        "config": {"workload": f"top-k sparse decode step, batch 1, ctx {args.ctx}: score "
                               f"{wl.n_blocks} pooled blocks x 8 KV heads, top-32 per head, "
                               "gather K/V (8 heads x 128 bf16, 64-token blocks) host->HBM "
                               "and GQA attention (64 q heads) over them in one pass",
                   "ctx": args.ctx, "kv_heads": 8, "head_dim": 128, "q_heads": 64,
                   "block_tokens": 64, "topk": 32, "gather_bytes_per_step": wl.gather_bytes,
                   "host_layout": args.layout},
        "decode_tok_s": round(1e3 / ms, 2),
        "pct_pcie_peak": round(100 * value / PCIE5_X16_PEAK_GBS, 2),
        "pct_measured_h2d_peak": round(100 * value / peaks["h2d_sdma_gbs"], 2),
        "part_ms": {k: round(v, 5) for k, v in r["part_ms"].items()},
        "staged_path": {
            "what": "index_topk, gather_blocks, attn_decode as three launches",
            "value": gbs(r_staged["ms_per_step"]),
            "ms_per_step": round(r_staged["ms_per_step"], 5),
            "decode_tok_s": round(1e3 / r_staged["ms_per_step"], 2),
            "part_ms": {k: round(v, 5) for k, v in r_staged["part_ms"].items()},
            "gather_kernel_gbs": gbs(r_staged["part_ms"]["gather"]),
            "gather_kernel_traffic": kernel_traffic("gather_kernel")},
        f"{other}_host_layout": {
            "value": gbs(r_other["ms_per_step"]),
            "ms_per_step": round(r_other["ms_per_step"], 5),
            "decode_tok_s": round(1e3 / r_other["ms_per_step"], 2),
            "gather_attn_gbs": gbs(r_other["part_ms"]["gather_attn"])},
        "link_peaks": peaks,
        "roofline": {**_pcie_roofline(achieved, peaks,
                                      kernel="gather_decode_partial (timed with its "
                                             "decode_merge: kvt_gather_attn_decode)"),
                     "bytes_per_launch": wl.gather_bytes, "avg_launch_ms": round(kern_ms, 5),
                     "traffic": kernel_traffic("gather_decode_partial"),
                     "traffic_unit": "bytes per launch",
                     "traffic_by_destination": kernel_traffic_ea("gather_decode_partial")},
    }
    if args.suite:
        line["suite"] = run_suite(torch, kvt, synth, dev, wl, args, peaks)
    if not args.no_cpu:
        log("cpu baseline ...")
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    wl.free()
    if not args.no_configs:
        line["configs"] = {"C4_topk_decode_262k": "the headline (value, roofline, cpu_baseline)",
                           **run_configs(torch, kvt, synth, dev, peaks, args)}
    print(json.dumps(line), flush=True)


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


# the three ways a swap can move pages, as named in the suites' output
COPY_MODES_SPEC = (("COPY_KERNEL", "kernel"), ("COPY_SDMA", "sdma"), ("COPY_RUNTIME", "runtime"))


def _swap_rate(torch, kvt, t, tab, n, direction, mode, nbytes):
    t.start()
    kvt.kvt_swap_blocks(tab[0], tab[1], tab[2], n, direction, mode)
    ms = t.stop_ms()
    return nbytes / (ms * 1e-3) / GB, ms


def _cpu_threads():
    n = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    return min(n, os.cpu_count() or n)


def cpu_swap_rates(src, dst_dev, dev_base, sizes, reps=3):
    """The oracle's memcpy loop over the same source descriptors (pinned host pages), into a
    host buffer laid out like the device destination (addresses dst - dev_base + buffer):
    GB/s on one thread and on all host threads.  It is the CPU baseline of a swap."""
    import numpy as np
    import oracle
    src = np.ascontiguousarray(src, dtype=np.uint64)
    dst_dev = np.ascontiguousarray(dst_dev, dtype=np.uint64)
    sizes = np.ascontiguousarray(sizes, dtype=np.uint64)
    span = int((dst_dev - np.uint64(dev_base) + sizes).max())
    buf = np.zeros(span, dtype=np.uint8)
    dst = dst_dev - np.uint64(dev_base) + np.uint64(buf.ctypes.data)
    nbytes = int(sizes.sum())
    out = {"bytes": nbytes, "kind": "oracle"}
    for threads, key in ((1, "one_thread_gbs"), (_cpu_threads(), "all_threads_gbs")):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.swap(src, dst, sizes, threads=threads)
            ts.append(time.perf_counter() - t0)
        out[key] = round(nbytes / _median(ts) / GB, 2)
    out["cores"] = _cpu_threads()
    out["cpu_model"] = cpu_model()
    del buf
    return out


def suite_one_layer(torch, kvt, synth, dev, peaks, reps=20):
    """One layer: K and V planes of 256 x 32 KiB pages in pinned memory; 64 fresh random block
    ids per rep, host -> HBM (load) and HBM -> host (store): the kernel, the copy engines and
    the runtime's copy calls."""
    import numpy as np
    nb, page, n = 256, 16 * 8 * 128 * 2, 64
    host = kvt.HostBuffer(2 * nb * page)
    hv = host.numpy(np.uint16, (2, nb, page // 2))
    hv[0] = synth.f16_normal(synth.rng(1, synth.P_K), (nb, page // 2))
    hv[1] = synth.f16_normal(synth.rng(1, synth.P_V), (nb, page // 2))
    hbm = torch.empty((2, nb, page), dtype=torch.uint8, device=dev)
    tb = kvt.HostBuffer(3 * 8 * 2 * n)
    tab = tb.numpy(np.uint64, (3, 2 * n))
    t = Timer(torch, torch.cuda.current_stream())
    out = {}
    for mode, mname in [(getattr(kvt, c), n) for c, n in COPY_MODES_SPEC]:
        for direction, dname in ((kvt.H2D, "h2d"), (kvt.D2H, "d2h")):
            rates = []
            for r in range(reps):
                hid = synth.permutation(synth.rng(1, synth.P_PERM_SRC, r), nb)[:n]
                gid = synth.permutation(synth.rng(1, synth.P_PERM_DST, r), nb)[:n]
                for p in range(2):
                    hs = tab[0 if direction == kvt.H2D else 1, p * n:]
                    gs = tab[1 if direction == kvt.H2D else 0, p * n:]
                    kvt.kvt_sub_block_ptrs(host.dev + p * nb * page, page, page, hid, n, 1, 0, hs, n)
                    kvt.kvt_sub_block_ptrs(hbm.data_ptr() + p * nb * page, page, page, gid, n, 1, 0,
                                           gs, n)
                tab[2] = page
                rates.append(_swap_rate(torch, kvt, t, tab, 2 * n, direction, mode, 2 * n * page)[0])
            peak = peaks["h2d_sdma_gbs"] if direction == kvt.H2D else peaks["d2h_sdma_gbs"]
            out[f"{dname}_{mname}_gbs"] = round(_median(rates), 2)
            out[f"{dname}_{mname}_pct_measured_peak"] = round(100 * _median(rates) / peak, 1)
    out["bytes_per_direction"] = 2 * n * page
    # CPU baseline: the last load's descriptors (host pages -> a host copy of the HBM planes)
    for p in range(2):
        kvt.kvt_sub_block_ptrs(host.dev + p * nb * page, page, page, hid, n, 1, 0, tab[0, p * n:], n)
        kvt.kvt_sub_block_ptrs(hbm.data_ptr() + p * nb * page, page, page, gid, n, 1, 0,
                               tab[1, p * n:], n)
    tab[2] = page
    out["cpu_baseline"] = cpu_swap_rates(tab[0], tab[1], hbm.data_ptr(), tab[2])
    del hv
    host.free()
    tb.free()
    return out


def suite_32_layers(torch, kvt, synth, dev, peaks, reps=3):
    """32 layers x (K, V) = 64 tensors: HBM [8192][32 KiB] each; host rows of 4 pages + 4 KiB
    pad (2048 rows, 135,168 B stride); 4096 random blocks per tensor with a random skip on the
    first host chunk (blocks_per_chunk 4): 8 GiB per direction."""
    import numpy as np
    tensors, gblocks, bpc, page, pad, n = 64, 8192, 4, 32768, 4096, 4096
    hrows = gblocks // bpc
    stride = bpc * page + pad
    t0 = time.time()
    host = kvt.HostBuffer(tensors * hrows * stride)
    hb = host.numpy(np.uint8, (tensors * hrows * stride,))
    seed_block = np.empty(1 << 28, dtype=np.uint8)
    synth.fill_random_bytes(synth.rng(2, synth.P_K), seed_block)
    for o in range(0, hb.size, seed_block.size):
        m = min(seed_block.size, hb.size - o)
        hb[o:o + m] = seed_block[:m]
    del seed_block
    hbm = torch.empty((tensors, gblocks, page), dtype=torch.uint8, device=dev)
    log(f"32-layer planes: {host.nbytes / 2**30:.1f} GiB pinned + {hbm.numel() / 2**30:.1f} GiB HBM "
        f"in {time.time() - t0:.1f}s")
    tb = kvt.HostBuffer(3 * 8 * tensors * n)
    tab = tb.numpy(np.uint64, (3, tensors * n))
    t = Timer(torch, torch.cuda.current_stream())
    out = {}
    g = synth.rng(2, synth.P_SKIP)
    build_ms = []   # S1 on the host: both sides' tables for all 64 tensors, 128 calls
    for direction, dname in ((kvt.H2D, "h2d"), (kvt.D2H, "d2h")):
        for mode, mname in [(getattr(kvt, c), n) for c, n in COPY_MODES_SPEC]:
            rates = []
            for r in range(reps):
                skip = int(g.integers(0, bpc))
                nch = kvt.kvt_chunks_consumed(n, skip, bpc)
                chunks = synth.permutation(synth.rng(2, synth.P_PERM_SRC, r), hrows)[:nch]
                gids = synth.permutation(synth.rng(2, synth.P_PERM_DST, r), gblocks)[:n]
                hrow = tab[0 if direction == kvt.H2D else 1]
                grow = tab[1 if direction == kvt.H2D else 0]
                t0 = time.perf_counter()
                for x in range(tensors):
                    kvt.kvt_sub_block_ptrs(host.dev + x * hrows * stride, stride, page, chunks, nch,
                                           bpc, skip, hrow[x * n:], n)
                    kvt.kvt_sub_block_ptrs(hbm.data_ptr() + x * gblocks * page, page, page, gids,
                                           n, 1, 0, grow[x * n:], n)
                build_ms.append((time.perf_counter() - t0) * 1e3)
                tab[2] = page
                rate, ms = _swap_rate(torch, kvt, t, tab, tensors * n, direction, mode,
                                      tensors * n * page)
                rates.append(rate)
                log(f"  32-layer {dname} {mname} rep {r}: {rate:.2f} GB/s ({ms:.1f} ms)")
            peak = peaks["h2d_sdma_gbs"] if direction == kvt.H2D else peaks["d2h_sdma_gbs"]
            out[f"{dname}_{mname}_gbs"] = round(_median(rates), 2)
            out[f"{dname}_{mname}_pct_measured_peak"] = round(100 * _median(rates) / peak, 1)
    out["bytes_per_direction"] = tensors * n * page
    out["table_build_ms"] = round(_median(build_ms[1:]), 3)   # the first build pays page faults
    out["table_build_descriptors_per_s"] = round(2 * tensors * n / (_median(build_ms[1:]) * 1e-3))
    # CPU baseline on one tensor's load (4096 pages of 32 KiB = 128 MiB), the last ids drawn
    kvt.kvt_sub_block_ptrs(host.dev, stride, page, chunks, nch, bpc, skip, tab[0], n)
    kvt.kvt_sub_block_ptrs(hbm.data_ptr(), page, page, gids, n, 1, 0, tab[1], n)
    tab[2, :n] = page
    out["cpu_baseline"] = cpu_swap_rates(tab[0, :n], tab[1, :n], hbm.data_ptr(), tab[2, :n])
    out["cpu_baseline"]["sample"] = "one of the 64 tensors' loads: 4096 pages of 32 KiB"
    del hb
    del hbm
    host.free()
    tb.free()
    torch.cuda.empty_cache()
    return out


def suite_small_pages(torch, kvt, synth, dev, peaks, reps=3):
    """65,536 pages in random scattered order host -> HBM, page sizes 512 B .. 64 KiB, kernel
    loads vs the copy engines and vs the runtime's copy calls; then 4 GiB of 128 KiB .. 1 MiB
    pages, where the engines close in on the kernel; plus 2 KiB pages at 8 mod 16
    alignment."""
    import numpy as np
    span = 65536 * 65536
    sizes = [512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072, 262144, 524288, 1048576]
    host = kvt.HostBuffer(span + 64)
    hb = host.numpy(np.uint8)
    synth.fill_random_bytes(synth.rng(3, synth.P_K), hb[:1 << 28])
    for o in range(1 << 28, hb.size, 1 << 28):
        m = min(1 << 28, hb.size - o)
        hb[o:o + m] = hb[:m]
    n = 65536
    hbm = torch.empty(span, dtype=torch.uint8, device=dev)
    tb = kvt.HostBuffer(3 * 8 * n)
    tab = tb.numpy(np.uint64, (3, n))
    t = Timer(torch, torch.cuda.current_stream())
    out = {"pages": n, "sweep": []}
    cross = cross_rt = None
    for size in sizes + [2048]:
        n = min(65536, span // size)
        off = 8 if (size == 2048 and len(out["sweep"]) == len(sizes)) else 0
        row = {"page_bytes": size, "pages": n, "host_offset_mod16": off}
        for mode, mname in [(getattr(kvt, c), nm) for c, nm in COPY_MODES_SPEC]:
            rates = []
            for r in range(reps):
                src = synth.permutation(synth.rng(3, synth.P_PERM_SRC, r), n)
                dst = synth.permutation(synth.rng(3, synth.P_PERM_DST, r), n)
                kvt.kvt_sub_block_ptrs(host.dev + off, size + (8 if off else 0), size, src, n, 1, 0,
                                       tab[0], n)
                kvt.kvt_sub_block_ptrs(hbm.data_ptr(), size, size, dst, n, 1, 0, tab[1], n)
                tab[2] = size
                rates.append(_swap_rate(torch, kvt, t, tab, n, kvt.H2D, mode, n * size)[0])
            row[f"{mname}_gbs"] = round(_median(rates), 2)
        log(f"  small pages {row}")
        out["sweep"].append(row)
        if not off and cross is None and row["sdma_gbs"] >= row["kernel_gbs"]:
            cross = size
        if not off and cross_rt is None and row["runtime_gbs"] >= row["kernel_gbs"]:
            cross_rt = size
    # the smallest page at which the copy engines (runtime copy calls) match the kernel
    out["h2d_crossover_bytes"] = cross
    out["h2d_crossover_bytes_runtime"] = cross_rt
    # CPU baseline: 512-byte pages (all 65,536) and 64 KiB pages (the first 4096 descriptors)
    n = 65536
    cpu = {}
    for size, m in ((512, n), (65536, 4096)):
        src = synth.permutation(synth.rng(3, synth.P_PERM_SRC, 0), n)[:m]
        dst = np.arange(m, dtype=np.int64)
        kvt.kvt_sub_block_ptrs(host.dev, size, size, src, m, 1, 0, tab[0], m)
        kvt.kvt_sub_block_ptrs(hbm.data_ptr(), size, size, dst, m, 1, 0, tab[1], m)
        tab[2, :m] = size
        cpu[f"{size}B"] = cpu_swap_rates(tab[0, :m], tab[1, :m], hbm.data_ptr(), tab[2, :m])
    out["cpu_baseline"] = cpu
    del hb
    del hbm
    host.free()
    tb.free()
    torch.cuda.empty_cache()
    return out


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16


def prefill_flops(n_q, q_pos0, n_qh, hd, n_kv, causal=True):
    """QK^T and PV multiply-adds, 2 flops each: 4*hd*n_qh per (query, visible key) pair."""
    if causal:
        keys = sum(min(q_pos0 + t + 1, n_kv) for t in range(n_q))
    else:
        keys = n_q * n_kv
    return 4 * hd * n_qh * keys


def suite_prefill(torch, kvt, synth, dev, peaks, reps=5, compact=False):
    """Tiered prefill: 180,000-token q8_0 cache (8 KV heads x 128), cells [0, 94208) in HBM and
    the rest in pinned host memory; a 2048-query causal chunk at the tail with 32 query heads.
    Stage the used host rows into HBM once, then flash attention over head + staging.
    compact: only the staging, the staged attention and the pipelined form (16,384-row
    arena), with a shorter CPU baseline."""
    import numpy as np
    n_kv, n_head, n_q, n_qh, kvh, hd = 180000, 94208, 2048, 32, 8, 128
    n_tail = n_kv - n_head
    t0 = time.time()
    k = synth.q8_0_rows(synth.rng(5, synth.P_K, n_kv), n_kv, kvh, hd)
    v = synth.q8_0_rows(synth.rng(5, synth.P_V, n_kv), n_kv, kvh, hd)
    row = k.shape[1]
    q_np = synth.f16_normal(synth.rng(5, synth.P_Q, n_kv), (n_q, n_qh, hd))
    q = torch.from_numpy(q_np.view(np.int16)).to(dev)
    k_all = torch.from_numpy(k).to(dev)
    v_all = torch.from_numpy(v).to(dev)
    host = kvt.HostBuffer(2 * n_tail * row)
    ht = host.numpy(np.uint8, (2, n_tail, row))
    ht[0], ht[1] = k[n_head:], v[n_head:]
    stage = torch.empty((2, n_tail, row), dtype=torch.uint8, device=dev)
    out = torch.empty((n_q, n_qh, hd), dtype=torch.float32, device=dev)
    log(f"prefill inputs ready in {time.time() - t0:.1f}s")
    t = Timer(torch, torch.cuda.current_stream())
    q_pos0 = n_kv - n_q
    scale = 1 / math.sqrt(hd)
    flops = prefill_flops(n_q, q_pos0, n_qh, hd, n_kv)
    stage_bytes = 2 * n_tail * row

    def stage_ms(mode):
        ms = []
        for _ in range(reps):
            t.start()
            kvt.kvt_stage_tail(host.dev, row, 0, n_tail, stage[0], mode)
            kvt.kvt_stage_tail(host.dev + n_tail * row, row, 0, n_tail, stage[1], mode)
            ms.append(t.stop_ms())
        return _median(ms)

    def attn_ms(kh, vh, nh, kt, vt):
        ms = []
        for _ in range(reps):
            t.start()
            kvt.kvt_attn_prefill(q, n_q, q_pos0, n_qh, kvh, hd, kh, vh, nh, kt, vt, n_kv,
                                 kvt.Q8_0, 1, scale, out)
            ms.append(t.stop_ms())
        return _median(ms)

    state_b = kvt.kvt_attn_prefill_state_bytes(n_q, n_qh, kvh)
    state = torch.empty(state_b, dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream()

    def pipe_ms(arena_rows):
        arena = torch.empty((2, arena_rows, row), dtype=torch.uint8, device=dev)
        ms = []
        for _ in range(reps):
            t.start()
            kvt.kvt_attn_prefill_pipelined(q, n_q, q_pos0, n_qh, kvh, hd, k_all, v_all, n_head,
                                           host.dev, host.dev + n_tail * row, n_kv, kvt.Q8_0, 1,
                                           scale, arena[0], arena[1], arena_rows, state, state_b,
                                           out, copy_stream=copy_stream)
            ms.append(t.stop_ms())
        del arena
        return _median(ms)

    def auto_ms(arena_rows):
        """kvt_attn_prefill_auto with two streams, the arena and the fp16 conversion buffer:
        the pipelined plan, its passes on rows converted to fp16 once."""
        arena = torch.empty((2, arena_rows, row), dtype=torch.uint8, device=dev)
        wa = kvt.kvt_attn_prefill_auto_ws_bytes(n_q, n_qh, kvh, n_kv)
        wsa = torch.empty(max(wa, 16), dtype=torch.uint8, device=dev)
        cb = kvt.kvt_attn_prefill_conv_bytes(n_head, kvh, arena_rows, kvt.Q8_0)
        cbuf = torch.empty(cb, dtype=torch.uint8, device=dev)
        ms = []
        for _ in range(reps):
            t.start()
            plan = kvt.kvt_attn_prefill_auto(q, n_q, q_pos0, n_qh, kvh, hd, k_all, v_all, n_head,
                                             host.dev, host.dev + n_tail * row, n_kv, kvt.Q8_0,
                                             1, scale, arena[0], arena[1], arena_rows, wsa, wa,
                                             out, copy_stream=copy_stream, conv=cbuf,
                                             conv_bytes=cb)
            ms.append(t.stop_ms())
        assert plan == kvt.PREFILL_PIPELINED
        del arena, wsa, cbuf
        return _median(ms)

    st_runtime = stage_ms(kvt.COPY_RUNTIME)
    st_sdma = stage_ms(kvt.COPY_SDMA)
    st_kernel = stage_ms(kvt.COPY_KERNEL)
    a_staged = attn_ms(k_all, v_all, n_head, stage[0], stage[1])

    def fp_cache_ms(fmt, dt):
        """The single pass over an fp16 or bf16 cache of the same shape (N(0,1) values, whole
        cache in HBM): for fp16, the kernel the auto plan's passes run once rows are converted."""
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        kf = torch.randn((n_kv, kvh * hd), generator=g, device=dev).to(dt)
        vf = torch.randn((n_kv, kvh * hd), generator=g, device=dev).to(dt)
        ms = []
        for _ in range(reps):
            t.start()
            kvt.kvt_attn_prefill(q, n_q, q_pos0, n_qh, kvh, hd, kf, vf, n_kv, None, None, n_kv,
                                 fmt, 1, scale, out)
            ms.append(t.stop_ms())
        del kf, vf
        return _median(ms)

    if compact:
        p_arena = pipe_ms(2 * 16384)
        p_auto = auto_ms(2 * 16384)
        a_f16 = fp_cache_ms(kvt.F16, torch.float16)
        st = min(st_runtime, st_sdma, st_kernel)
        res = {"n_kv": n_kv, "n_head": n_head, "n_q": n_q, "stage_bytes": stage_bytes,
               "flops": flops, "stage_runtime_ms": round(st_runtime, 4),
               "stage_sdma_ms": round(st_sdma, 4), "stage_kernel_ms": round(st_kernel, 4),
               "stage_gbs": round(stage_bytes / (st * 1e-3) / GB, 2),
               "attn_staged_ms": round(a_staged, 4),
               "attn_tflops": round(flops / (a_staged * 1e-3) / 1e12, 1),
               "prefill_tok_s_staged": round(n_q / ((st + a_staged) * 1e-3), 1),
               "pipelined_arena_16384_ms": round(p_arena, 4),
               "prefill_tok_s_pipelined": round(n_q / (p_arena * 1e-3), 1),
               "auto_arena_16384_ms": round(p_auto, 4),
               "prefill_tok_s_auto": round(n_q / (p_auto * 1e-3), 1),
               "attn_all_hbm_f16_cache_ms": round(a_f16, 4),
               "attn_f16_tflops": round(flops / (a_f16 * 1e-3) / 1e12, 1),
               "cpu_baseline": cpu_prefill(k, v, ht, q_np, n_head, n_kv, kvh, row, scale,
                                           stage_bytes, budget_s=8.0)}
        del ht, k, v
        host.free()
        del k_all, v_all, stage, out, q, state
        torch.cuda.empty_cache()
        return res
    a_inplace = attn_ms(k_all, v_all, n_head, host.dev, host.dev + n_tail * row)
    a_hbm = attn_ms(k_all, v_all, n_kv, None, None)
    p_one = pipe_ms(2 * n_tail)          # the whole tail in one bucket
    p_arena = pipe_ms(2 * 16384)         # bounded arena: buckets of 16,384 rows (17.8 MB/plane)
    p_auto = auto_ms(2 * 16384)          # the same arena through the auto plan (fp16 passes)
    st = min(st_runtime, st_sdma, st_kernel)
    # short chunks (one token = a decode step over the tiered cache): the split-K form, staged
    # (stage + attend) and with the tail read in place, against the single pass -- whether the
    # staging pays below some chunk length, as the page streaming cold weights keeps chunks
    # under 65 tokens zero-copy
    cutoff = {}
    ws_b = max(kvt.kvt_attn_prefill_splitk_ws_bytes(1, n_qh, kvh, n_kv),
               kvt.kvt_attn_prefill_auto_ws_bytes(n_q, n_qh, kvh, n_kv))
    ws_sk = torch.empty(max(ws_b, 16), dtype=torch.uint8, device=dev)
    arena_p = torch.empty((2, 2 * 16384, row), dtype=torch.uint8, device=dev)
    conv_b = kvt.kvt_attn_prefill_conv_bytes(n_head, kvh, n_tail, kvt.Q8_0)
    conv_buf = torch.empty(conv_b, dtype=torch.uint8, device=dev)
    for nq in (1, 16, 64, 256, 512, 1024, 2048):
        qs = q[n_q - nq:]
        outs = out[:nq]
        wb = kvt.kvt_attn_prefill_splitk_ws_bytes(nq, n_qh, kvh, n_kv)
        wa = kvt.kvt_attn_prefill_auto_ws_bytes(nq, n_qh, kvh, n_kv)
        assert wb <= ws_sk.numel() and wa <= ws_sk.numel()
        plan = None

        def run(kind):
            nonlocal plan
            ms = []
            for _ in range(reps):
                t.start()
                if kind in ("auto", "auto_conv"):
                    plan = kvt.kvt_attn_prefill_auto(
                        qs, nq, n_kv - nq, n_qh, kvh, hd, k_all, v_all, n_head, host.dev,
                        host.dev + n_tail * row, n_kv, kvt.Q8_0, 1, scale, stage[0], stage[1],
                        n_tail, ws_sk, wa, outs, copy_stream=copy_stream,
                        conv=conv_buf if kind == "auto_conv" else None,
                        conv_bytes=conv_b if kind == "auto_conv" else 0)
                    ms.append(t.stop_ms())
                    continue
                if kind == "pipelined":
                    kvt.kvt_attn_prefill_pipelined(
                        qs, nq, n_kv - nq, n_qh, kvh, hd, k_all, v_all, n_head, host.dev,
                        host.dev + n_tail * row, n_kv, kvt.Q8_0, 1, scale, arena_p[0],
                        arena_p[1], arena_p.shape[1], ws_sk, wa, outs, copy_stream=copy_stream)
                    ms.append(t.stop_ms())
                    continue
                if kind == "staged":
                    kvt.kvt_stage_tail(host.dev, row, 0, n_tail, stage[0], kvt.COPY_AUTO)
                    kvt.kvt_stage_tail(host.dev + n_tail * row, row, 0, n_tail, stage[1],
                                       kvt.COPY_AUTO)
                    kt_, vt_ = stage[0], stage[1]
                else:
                    kt_, vt_ = host.dev, host.dev + n_tail * row
                if kind == "single_pass_in_place":
                    kvt.kvt_attn_prefill(qs, nq, n_kv - nq, n_qh, kvh, hd, k_all, v_all, n_head,
                                         kt_, vt_, n_kv, kvt.Q8_0, 1, scale, outs)
                else:
                    kvt.kvt_attn_prefill_splitk(qs, nq, n_kv - nq, n_qh, kvh, hd, k_all, v_all,
                                                n_head, kt_, vt_, n_kv, kvt.Q8_0, 1, scale,
                                                ws_sk, wb, outs)
                ms.append(t.stop_ms())
            return _median(ms)
        cutoff[str(nq)] = {k_: round(run(k_), 3) for k_ in
                           ("staged", "in_place", "single_pass_in_place", "pipelined", "auto",
                            "auto_conv")}
        cutoff[str(nq)]["splits"] = (wb // kvt.kvt_attn_prefill_state_bytes(nq, n_qh, kvh)
                                     if wb else 1)
        cutoff[str(nq)]["auto_plan"] = ("in_place", "staged", "pipelined")[plan]
    del ws_sk, arena_p, conv_buf
    log("prefill staging cutoff", cutoff)
    # an fp16 GEMM probe (hipBLASLt through torch, 8192^3) for the measured MFMA rate
    a = torch.randn((8192, 8192), device=dev, dtype=torch.float16)
    b = torch.randn((8192, 8192), device=dev, dtype=torch.float16)
    gms = []
    for _ in range(reps + 2):
        t.start()
        torch.matmul(a, b)
        gms.append(t.stop_ms())
    gemm_tflops = 2 * 8192 ** 3 / (min(gms) * 1e-3) / 1e12
    del a, b
    # the same op over fp16 and bf16 caches (N(0,1) values, 2 bytes each), whole cache in HBM
    fp_ms = {name: fp_cache_ms(fmt, dt) for fmt, name, dt in
             ((kvt.F16, "f16", torch.float16), (kvt.BF16, "bf16", torch.bfloat16))}
    res = {
        "n_kv": n_kv, "n_head": n_head, "n_q": n_q, "q_heads": n_qh, "kv_heads": kvh,
        "stage_bytes": stage_bytes, "flops": flops,
        "stage_runtime_ms": round(st_runtime, 4), "stage_sdma_ms": round(st_sdma, 4),
        "stage_kernel_ms": round(st_kernel, 4),
        "stage_gbs": round(stage_bytes / (st * 1e-3) / GB, 2),
        "stage_pct_measured_h2d_peak": round(100 * stage_bytes / (st * 1e-3) / GB / peaks["h2d_sdma_gbs"], 1),
        "attn_staged_ms": round(a_staged, 4),
        "attn_tflops": round(flops / (a_staged * 1e-3) / 1e12, 1),
        "attn_pct_mfma_fp16_peak": round(100 * flops / (a_staged * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 2),
        "fp16_gemm_probe_tflops": round(gemm_tflops, 1),
        "staging_cutoff_by_chunk": cutoff,
        "attn_pct_of_gemm_probe": round(100 * flops / (a_staged * 1e-3) / 1e12 / gemm_tflops, 1),
        "attn_tail_in_host_ms": round(a_inplace, 4),
        "attn_all_hbm_ms": round(a_hbm, 4),
        "prefill_tok_s_staged": round(n_q / ((st + a_staged) * 1e-3), 1),
        "prefill_tok_s_staging_off": round(n_q / (a_inplace * 1e-3), 1),
        "pipelined_one_bucket_ms": round(p_one, 4),
        "auto_arena_16384_ms": round(p_auto, 4),
        "prefill_tok_s_auto": round(n_q / (p_auto * 1e-3), 1),
        "pipelined_arena_16384_ms": round(p_arena, 4),
        "prefill_tok_s_pipelined": round(n_q / (min(p_one, p_arena) * 1e-3), 1),
        "attn_all_hbm_f16_cache_ms": round(fp_ms["f16"], 4),
        "attn_all_hbm_bf16_cache_ms": round(fp_ms["bf16"], 4),
        "cpu_baseline": cpu_prefill(k, v, ht, q_np, n_head, n_kv, kvh, row, scale, stage_bytes),
    }
    log("prefill", res)
    del ht, k, v
    host.free()
    del k_all, v_all, stage, out, q, state
    torch.cuda.empty_cache()
    return res


def suite_prefill_chain(torch, kvt, synth, dev, peaks, reps=5):
    """Tiered prefill over a chain of 8 layers with the whole 180,000-token q8_0 cache of each
    layer in pinned host memory (n_head 0), a 2048-query causal chunk with 32 query heads, 16,384-
    row buckets: kvt_attn_prefill_pipelined per layer (each waits for its first bucket's copy)
    against kvt_attn_prefill_chain (each call copies the next layer's first bucket behind its
    own copies).  Layers alternate between two sets of host planes (K and V swapped) and two
    arenas."""
    import numpy as np
    n_kv, n_q, n_qh, kvh, hd = 180000, 2048, 32, 8, 128
    n_layers, ch_rows = 8, 2 * 16384
    t0 = time.time()
    k = synth.q8_0_rows(synth.rng(5, synth.P_K, n_kv), n_kv, kvh, hd)
    v = synth.q8_0_rows(synth.rng(5, synth.P_V, n_kv), n_kv, kvh, hd)
    row = k.shape[1]
    q_np = synth.f16_normal(synth.rng(5, synth.P_Q, n_kv), (n_q, n_qh, hd))
    q = torch.from_numpy(q_np.view(np.int16)).to(dev)
    ch_hosts = []
    for kk, vv in ((k, v), (v, k)):
        hbuf = kvt.HostBuffer(2 * n_kv * row)
        hp = hbuf.numpy(np.uint8, (2, n_kv, row))
        hp[0], hp[1] = kk, vv
        del hp
        ch_hosts.append(hbuf)
    del k, v
    ch_arenas = [torch.empty((2, ch_rows, row), dtype=torch.uint8, device=dev) for _ in range(2)]
    out = torch.empty((n_q, n_qh, hd), dtype=torch.float32, device=dev)
    state_b = kvt.kvt_attn_prefill_state_bytes(n_q, n_qh, kvh)
    state = torch.empty(state_b, dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream()
    t = Timer(torch, torch.cuda.current_stream())
    q_pos0 = n_kv - n_q
    scale = 1 / math.sqrt(hd)
    log(f"chain inputs ready in {time.time() - t0:.1f}s")

    def chain_ms(prefetch, reps=reps):
        ms = []
        for _ in range(reps):
            t.start()
            for i in range(n_layers):
                h, hn = ch_hosts[i % 2], ch_hosts[(i + 1) % 2]
                a, an = ch_arenas[i % 2], ch_arenas[(i + 1) % 2]
                kvt.kvt_attn_prefill_chain(
                    q, n_q, q_pos0, n_qh, kvh, hd, None, None, 0, h.dev, h.dev + n_kv * row,
                    n_kv, kvt.Q8_0, 1, scale, a[0], a[1], ch_rows,
                    ch_rows // 2 if prefetch and i > 0 else 0, hn.dev, hn.dev + n_kv * row,
                    ch_rows // 2 if prefetch and i + 1 < n_layers else 0, an[0], an[1], ch_rows,
                    state, state_b, out, copy_stream=copy_stream)
            ms.append(t.stop_ms() / n_layers)
        return _median(ms)

    # untimed: the first passes over freshly pinned planes run up to ten times slower
    chain_ms(False, 1)
    chain_ms(True, 1)
    plain = chain_ms(False)
    chained = chain_ms(True)
    layer_bytes = 2 * n_kv * row
    res = {
        "n_kv": n_kv, "n_head": 0, "n_q": n_q, "q_heads": n_qh, "kv_heads": kvh,
        "layers": n_layers, "bucket_rows": ch_rows // 2, "host_bytes_per_layer": layer_bytes,
        "pipelined_ms_per_layer": round(plain, 4),
        "chain_ms_per_layer": round(chained, 4),
        "chain_link_gbs": round(layer_bytes / (chained * 1e-3) / GB, 2),
        "prefill_tok_s_pipelined": round(n_q / (plain * 1e-3), 1),
        "prefill_tok_s_chain": round(n_q / (chained * 1e-3), 1),
    }
    log("prefill chain", res)
    for hbuf in ch_hosts:
        hbuf.free()
    del ch_arenas, out, q, state
    torch.cuda.empty_cache()
    return res


def cpu_prefill(k, v, ht, q_np, n_head, n_kv, kvh, row, scale, stage_bytes, budget_s=20.0):
    """The oracle's staging (memcpy of the host tail) and fp64 prefill attention over a bounded
    sample of the last query rows (each sees ~180k keys): staging GB/s and attention tok/s."""
    import oracle
    threads = _cpu_threads()
    n_q = q_np.shape[0]
    n_tail = n_kv - n_head
    t0 = time.perf_counter()
    oracle.stage_tail(ht[0], row, 0, n_tail)
    oracle.stage_tail(ht[1], row, 0, n_tail)
    st = time.perf_counter() - t0
    rows, el = 0, 0.0
    while el < budget_s / 2 and rows < n_q:
        r = max(1, rows)                      # 1, 1, 2, 4, ... rows per call
        t0 = time.perf_counter()
        oracle.attn_prefill(q_np, n_kv - n_q, kvh, k, v, n_head, k[n_head:], v[n_head:], n_kv,
                            oracle.Q8_0, True, scale, t_begin=n_q - rows - r, t_end=n_q - rows,
                            threads=threads)
        el += time.perf_counter() - t0
        rows += r
    return {"kind": "oracle", "cores": threads, "cpu_model": cpu_model(),
            "stage_gbs": round(stage_bytes / st / GB, 2),
            "attn_rows_per_s": round(rows / el, 3),
            "sample": f"staging memcpy of the {n_tail}-row tail; fp64 attention of the last {rows} "
                      f"of the {n_q} query rows in {el:.1f}s"}


def suite_qsa(torch, kvt, synth, dev, wl, args, reps=None):
    """The QSA indexer's own selection geometry on the headline's host planes: pooled keys over
    4-token blocks, top-512 per KV head, token positions plus the write head's tail padded to
    K_pad = 2080, then the fused gather + attention over those tokens (token-major addressing).
    262,143 tokens: 65,535 complete pooled blocks and a 3-token tail."""
    import numpy as np
    kvh, hd, n_qh, cr, k = wl.KVH, wl.HD, wl.NQH, 4, 512
    n_tok = wl.ctx - 1
    n_blocks = n_tok // cr
    k_pad = -(-(k * cr + cr - 1) // 32) * 32
    row = kvh * hd * 2
    n_sets = args.warmup + args.steps
    pooled = torch.from_numpy(synth.f16_normal(synth.rng(4, synth.P_POOLED, n_tok),
                                               (n_blocks, 128)).view(np.int16)).to(dev)
    qidx = torch.from_numpy(synth.f16_normal(synth.rng(4, synth.P_QIDX, n_tok),
                                             (n_sets, kvh, 128)).view(np.int16)).to(dev)
    ws_t = kvt.kvt_index_topk_ws_bytes(n_blocks, kvh, k)
    ws_d = kvt.kvt_attn_decode_ws_bytes(n_qh, hd, k_pad)
    ws = torch.empty(ws_t + ws_d + 256, dtype=torch.uint8, device=dev)
    ids = torch.empty((kvh, k), dtype=torch.int32, device=dev)
    pos = torch.empty((kvh, k_pad), dtype=torch.int32, device=dev)
    kv = torch.empty((2, kvh, k_pad, hd), dtype=torch.int16, device=dev)
    out = torch.empty((n_qh, hd), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def parts(i):
        return [("topk", lambda: kvt.kvt_index_topk(pooled, n_blocks, 128, qidx[i % n_sets], kvh,
                                                     k, ids, None, ws, ws_t)),
                ("positions", lambda: kvt.kvt_select_positions(ids, kvh, k, cr, n_tok, k_pad,
                                                                pos)),
                ("gather_attn", lambda: kvt.kvt_gather_attn_decode(
                    wl.q[i % wl.n_sets], n_qh, kvh, hd, kvt.BF16, wl.host.dev,
                    wl.host.dev + wl.ctx * wl.row, n_tok, row, hd * 2, row, None, 1, pos, k_pad,
                    kv[0], kv[1], wl.scale, out, ws[ws_t + 128:], ws_d))]

    for i in range(args.warmup):
        for _, fn in parts(i):
            fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        for _, fn in parts(args.warmup + i):
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    names = [n for n, _ in parts(0)]
    acc = {n: 0.0 for n in names}
    for i in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        evs[0].record(stream)
        for j, (_, fn) in enumerate(parts(args.warmup + i)):
            fn()
            evs[j + 1].record(stream)
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            acc[n] += evs[j].elapsed_time(evs[j + 1]) / args.steps
    host_bytes = kvh * (k * cr + n_tok % cr) * hd * 2 * 2
    res = {"n_tok": n_tok, "cr": cr, "block_topk": k, "k_pad": k_pad, "pooled_blocks": n_blocks,
           "ms_per_step": round(ms, 5), "decode_tok_s": round(1e3 / ms, 2),
           "host_bytes_per_step": host_bytes,
           "gather_gbs_whole_step": round(host_bytes / (ms * 1e-3) / GB, 3),
           "part_ms": {n_: round(v, 5) for n_, v in acc.items()}}
    log("qsa geometry", res)
    return res


def suite_worker(torch, kvt, synth, dev, wl, peaks, jobs=16, pages_per_job=4096):
    """The transfer worker: `jobs` jobs of 4096 random 32 KiB pages (128 MiB, the 32-layer
    geometry's 64 tensors x 64 blocks) loaded host -> HBM through one worker; the same tables
    as one direct kvt_swap_blocks call; a load worker and a store worker running at once (both
    link directions); and the decode step replayed from HIP graphs against eager launches.
    Payload bytes are the zero fill of fresh pinned/HBM memory (a copy's rate does not depend
    on the bytes it moves)."""
    import numpy as np
    page = 32768
    n_pages = jobs * pages_per_job
    hosts = [kvt.HostBuffer(n_pages * page) for _ in range(2)]
    hbm = torch.zeros((2, n_pages, page), dtype=torch.uint8, device=dev)
    tabs = []
    for side in range(2):   # side 0: loads host[0] -> hbm[0]; side 1: stores hbm[1] -> host[1]
        perm_h = synth.permutation(synth.rng(11, synth.P_PERM_SRC, side), n_pages)
        perm_g = synth.permutation(synth.rng(11, synth.P_PERM_DST, side), n_pages)
        hs = np.empty(n_pages, np.uint64)
        gs = np.empty(n_pages, np.uint64)
        kvt.kvt_sub_block_ptrs(hosts[side].dev, page, page, perm_h, n_pages, 1, 0, hs, n_pages)
        kvt.kvt_sub_block_ptrs(hbm[side].data_ptr(), page, page, perm_g, n_pages, 1, 0, gs,
                               n_pages)
        tabs.append((hs, gs) if side == 0 else (gs, hs))
    sizes = np.full(n_pages, page, np.uint64)
    job_bytes = pages_per_job * page
    out = {"job_bytes": job_bytes, "jobs": jobs}

    def run_jobs(workers, reps=3):
        """Submit every job to each worker (one direction each); host-clock GB/s over all."""
        best = None
        for r in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            sub = 0.0
            for j in range(jobs):
                for side, w in workers:
                    a, b = tabs[side]
                    lo, hi = j * pages_per_job, (j + 1) * pages_per_job
                    ts = time.perf_counter()
                    kvt.kvt_worker_submit(w, r * jobs + j, a[lo:hi], b[lo:hi], sizes[lo:hi],
                                          pages_per_job)
                    sub += time.perf_counter() - ts
            for side, w in workers:
                kvt.kvt_worker_wait(w, r * jobs + jobs - 1)
            wall = time.perf_counter() - t0
            per_job = []
            for side, w in workers:
                done = kvt.kvt_worker_get_finished(w, jobs)
                assert [d[0] for d in done] == [r * jobs + j for j in range(jobs)]
                per_job += [d[1] / d[2] / GB for d in done]
            res = {"gbs": len(workers) * jobs * job_bytes / wall / GB,
                   "job_event_gbs_median": _median(per_job),
                   "submit_us_per_job": sub / (jobs * len(workers)) * 1e6}
            if best is None or res["gbs"] > best["gbs"]:
                best = res
        return {k: round(v, 2) for k, v in best.items()}

    for mode, mname in ((kvt.COPY_RUNTIME, "runtime"), (kvt.COPY_KERNEL, "kernel")):
        wl_ = kvt.kvt_worker_create(kvt.H2D, mode)
        ws_ = kvt.kvt_worker_create(kvt.D2H, mode)
        kvt.kvt_worker_reserve(wl_, jobs, pages_per_job)
        kvt.kvt_worker_reserve(ws_, jobs, pages_per_job)
        run_jobs([(0, wl_)], reps=1)   # warm-up
        out[f"load_{mname}"] = run_jobs([(0, wl_)])
        out[f"load_store_{mname}"] = run_jobs([(0, wl_), (1, ws_)])
        kvt.kvt_worker_destroy(wl_)
        kvt.kvt_worker_destroy(ws_)
        # the same tables as one direct call on the current stream
        tb = kvt.HostBuffer(3 * 8 * n_pages)
        tab = tb.numpy(np.uint64, (3, n_pages))
        tab[0], tab[1], tab[2] = tabs[0][0], tabs[0][1], sizes
        t = Timer(torch, torch.cuda.current_stream())
        rates = [_swap_rate(torch, kvt, t, tab, n_pages, kvt.H2D, mode, n_pages * page)[0]
                 for _ in range(3)]
        out[f"direct_load_{mname}_gbs"] = round(max(rates), 2)
        del tab
        tb.free()
    log("worker", out)
    del hbm
    for h in hosts:
        h.free()
    torch.cuda.empty_cache()

    # the decode step from HIP graphs: one graph per query set, replayed in turn
    n_sets, steps = 8, 200
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n_sets):
            wl.step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(n_sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            wl.step(i)
        graphs.append(g)
    torch.cuda.synchronize()

    def timed(fn):
        for i in range(n_sets):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i % n_sets)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    eager = min(timed(wl.step) for _ in range(3))
    graph = min(timed(lambda i: graphs[i].replay()) for _ in range(3))
    out["decode_step_eager_ms"] = round(eager, 5)
    out["decode_step_graph_ms"] = round(graph, 5)
    del graphs
    torch.cuda.synchronize()
    log("decode graph", {"eager_ms": eager, "graph_ms": graph})
    return out


def suite_upkeep(torch, kvt, synth, dev, peaks, reps=20):
    """The write side: a 2048-token prefill chunk appended to host pages (K and V rows of
    8 heads x 128 bf16, raw keys of 128 fp16; 256-token pages at random page ids) and one
    decode token appended, both through kvt_paged_write, each followed by the pool rebuild of
    the blocks it touched (cr 4); then copy_page of a full page (host memcpy of the three
    planes after draining the stream, pooled rows on the device)."""
    import numpy as np
    ps, n_pages, cr = 256, 1024, 4
    rbs = [8 * 128 * 2, 8 * 128 * 2, 128 * 2]
    bufs = [kvt.HostBuffer(n_pages * ps * rb) for rb in rbs]
    pooled = torch.zeros((n_pages, ps // cr, 256), dtype=torch.uint8, device=dev)
    pps = n_pages
    table = torch.from_numpy(synth.permutation(synth.rng(13, synth.P_PERM_DST), n_pages)
                             .astype(np.int32)[None]).to(dev)
    out = {}
    t = Timer(torch, torch.cuda.current_stream())
    for seq, name in ((2048, "prefill_chunk_2048"), (1, "decode_token")):
        src = [torch.randint(0, 256, (1, seq, rb), dtype=torch.uint8, device=dev) for rb in rbs]
        times = []
        for r in range(reps):
            lens = torch.tensor([(r * 4099) % (n_pages * ps - seq)], dtype=torch.int32,
                                device=dev)
            t.start()
            kvt.kvt_paged_write(src, [b.dev for b in bufs], rbs, 1, seq, lens, table, pps, ps,
                                n_pages)
            times.append(t.stop_ms())
        ms = _median(times)
        nbytes = seq * sum(rbs)
        out[name] = {"bytes": nbytes, "us": round(ms * 1e3, 2),
                     "gbs": round(nbytes / (ms * 1e-3) / GB, 2),
                     "pct_measured_d2h": round(100 * nbytes / (ms * 1e-3) / GB /
                                               peaks["d2h_sdma_gbs"], 1)}
        # the pool kernel at the write head: the touched blocks' pooled keys rebuilt from the
        # raw key rows just written (read back over the host link), into the HBM pooled plane
        ptimes = []
        for r in range(reps):
            lens = torch.tensor([(r * 4099) % (n_pages * ps - seq)], dtype=torch.int32,
                                device=dev)
            kvt.kvt_paged_write(src, [b.dev for b in bufs], rbs, 1, seq, lens, table, pps, ps,
                                n_pages)
            t.start()
            kvt.kvt_pool_rebuild(bufs[2].dev, pooled, 128, 1, seq, lens, table, pps, ps, cr,
                                 n_pages)
            ptimes.append(t.stop_ms())
        pms = _median(ptimes)
        blocks = (seq + cr - 1) // cr + 1
        out[name]["pool_rebuild"] = {"blocks_at_most": blocks, "us": round(pms * 1e3, 2),
                                     "raw_bytes_read_at_most": blocks * cr * rbs[2]}
    host_ms = []
    for r in range(reps):
        t0 = time.perf_counter()
        kvt.kvt_copy_page([b.host for b in bufs], [b.host for b in bufs], rbs, 2 * r, 2 * r + 1,
                          ps, ps, pooled, pooled, 256, cr)
        host_ms.append((time.perf_counter() - t0) * 1e3)
    torch.cuda.synchronize()
    page_bytes = ps * sum(rbs)
    ms = _median(host_ms)
    out["copy_page_full"] = {"host_bytes": page_bytes, "us": round(ms * 1e3, 2),
                             "host_memcpy_gbs": round(page_bytes / (ms * 1e-3) / GB, 2)}
    log("upkeep", out)
    for b in bufs:
        b.free()
    return out


def suite_rows(torch, kvt, synth, dev, wl, peaks, row_counts=(1, 16, 64, 128, 256, 512, 2048)):
    """Sparse attention over per-row selections at 262,144 tokens: pages of 256 token rows
    (8 KV heads x 128 bf16) in pinned host memory under a random block table, 64 query heads,
    2080 positions per row (512 pooled blocks of 4 tokens + a 3-token tail, the QSA geometry).
    For each row count: the direct path (every row reads its selection over the link), the
    staged path (the 1024 used pages copied to HBM once, then the rows attend the copy), and
    what the staging rule picks.  The planes are the decode workload's host planes, read as
    [token][head][dim]."""
    import numpy as np
    ps, kvh, hd, n_qh, k_pad = 256, 8, 128, 64, 2080
    ctx = wl.ctx
    n_pages = ctx // ps
    row = kvh * hd * 2
    g = synth.rng(15, synth.P_PERM_DST)
    table = torch.from_numpy(synth.permutation(g, n_pages).astype(np.int32)).to(dev)
    r_max = max(row_counts)
    gp = synth.rng(15, synth.P_MISC)
    pos = np.full((r_max, k_pad), -1, np.int32)
    n_pool = ctx // 4
    for r in range(r_max):
        blocks = np.sort(gp.choice(n_pool - 1, size=512, replace=False))
        pos[r, :2048] = (blocks[:, None] * 4 + np.arange(4)).reshape(-1)
        pos[r, 2048:2051] = ctx - 3 + np.arange(3)
    pos_d = torch.from_numpy(pos).to(dev)
    q = torch.randn((r_max, n_qh, hd), device=dev).to(torch.bfloat16).view(torch.int16)
    out = torch.empty((r_max, n_qh, hd), dtype=torch.float32, device=dev)
    ws_b = kvt.kvt_sparse_attend_rows_ws_bytes(r_max, n_qh, kvh, k_pad)
    ws_b = max(ws_b, kvt.kvt_sparse_attend_rows_ws_bytes(1, n_qh, kvh, k_pad))
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    stage_bytes = n_pages * ps * row
    sk = torch.empty(stage_bytes, dtype=torch.uint8, device=dev)
    sv = torch.empty(stage_bytes, dtype=torch.uint8, device=dev)
    kp, vp = wl.host.dev, wl.host.dev + ctx * row
    t = Timer(torch, torch.cuda.current_stream())
    res = {"k_pad": k_pad, "pages": n_pages, "page_size": ps, "rows": {}}

    def direct(R):
        kvt.kvt_sparse_attend_rows(q, R, n_qh, kvh, hd, kvt.BF16, kp, vp, ctx, row, hd * 2,
                                   table, n_pages, 0, ps, pos_d, k_pad, 1 / math.sqrt(hd), out,
                                   ws, ws_b)

    def staged(R):
        kvt.kvt_sparse_attend_rows_auto(q, R, n_qh, kvh, hd, kvt.BF16, kp, vp, ctx, row, hd * 2,
                                        table, n_pages, ps, pos_d, k_pad, 1 / math.sqrt(hd), out,
                                        ws, ws_b, sk, sv, stage_bytes)

    for R in row_counts:
        reps = 5 if R <= 256 else 2
        d_ms, s_ms = [], []
        for _ in range(reps):
            t.start()
            direct(R)
            d_ms.append(t.stop_ms())
        rule = kvt.kvt_staging_worthwhile(R, k_pad, n_pages, ps)
        if rule:
            for _ in range(reps):
                t.start()
                staged(R)
                s_ms.append(t.stop_ms())
        else:
            # the rule says direct: time the staged form explicitly, stage then attend
            for _ in range(reps):
                t.start()
                kvt.kvt_stage_pages(kp, vp, ps * row, table, n_pages, n_pages, sk, sv)
                kvt.kvt_sparse_attend_rows(q, R, n_qh, kvh, hd, kvt.BF16, sk, sv, ctx, row,
                                           hd * 2, None, 0, 0, 1, pos_d, k_pad,
                                           1 / math.sqrt(hd), out, ws, ws_b)
                s_ms.append(t.stop_ms())
        d, st_ = _median(d_ms), _median(s_ms)
        res["rows"][str(R)] = {"direct_ms": round(d, 4), "staged_ms": round(st_, 4),
                               "rule_stages": bool(rule), "faster": "staged" if st_ < d else "direct",
                               "direct_gbs": round(R * k_pad * row * 2 / (d * 1e-3) / GB, 2)}
        log(f"rows {R}: direct {d:.3f} ms, staged {st_:.3f} ms, rule "
            f"{'stage' if rule else 'direct'}")
    # the staging copy alone
    ms = []
    for _ in range(3):
        t.start()
        kvt.kvt_stage_pages(kp, vp, ps * row, table, n_pages, n_pages, sk, sv)
        ms.append(t.stop_ms())
    res["stage_pages_ms"] = round(_median(ms), 3)
    res["stage_pages_gbs"] = round(2 * stage_bytes / (_median(ms) * 1e-3) / GB, 2)
    log("rows", res)
    del sk, sv, ws, out
    torch.cuda.empty_cache()
    return res


def _pcie_roofline(gbs, peaks, direction="h2d", kernel=None):
    """A host-link kernel against the PCIe Gen5 x16 per-direction peak (63.0 GB/s nominal) and
    against the same run's measured DMA-engine peak."""
    pk = peaks["h2d_sdma_gbs"] if direction == "h2d" else peaks["d2h_sdma_gbs"]
    r = {"bound": "pcie", "achieved": round(gbs, 3), "peak": PCIE5_X16_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / PCIE5_X16_PEAK_GBS, 4), "peak_measured": pk,
         "frac_measured": round(gbs / pk, 4)}
    if kernel:
        r["kernel"] = kernel
    return r


def run_configs(torch, kvt, synth, dev, peaks, args):
    """One compact entry per workload besides the headline: its figure, the roofline of its
    dominant kernel and the CPU oracle's rate on the same data."""
    cfg = {}

    def timed(name, fn):
        t0 = time.time()
        log(f"config: {name}")
        r = fn()
        r["wall_s"] = round(time.time() - t0, 1)
        cfg[name] = r
        log(f"config {name}: {json.dumps(r)[:400]}")

    def c1():
        r = suite_one_layer(torch, kvt, synth, dev, peaks)
        return {"workload": "one layer: K and V planes of 256 x 32 KiB fp16 pages in pinned "
                            "host memory, 64 random block ids host->HBM (4 MiB), then stored back",
                "metric": "load GB/s (kernel)", "value": r["h2d_kernel_gbs"], "unit": "GB/s",
                "store_gbs": r["d2h_kernel_gbs"], "load_sdma_gbs": r["h2d_sdma_gbs"],
                "load_runtime_gbs": r["h2d_runtime_gbs"],
                "roofline": _pcie_roofline(r["h2d_kernel_gbs"], peaks, kernel="copy_desc_kernel"),
                "cpu_baseline": {**r["cpu_baseline"], "value": r["cpu_baseline"]["all_threads_gbs"],
                                 "unit": "GB/s",
                                 "sample": "the last load's 128 descriptors of 32 KiB"}}

    def c2():
        r = suite_32_layers(torch, kvt, synth, dev, peaks, reps=1)
        return {"workload": "32 layers: 64 tensors of 8192 x 32 KiB bf16 blocks, host rows of 4 "
                            "pages + 4 KiB pad, 4096 random blocks per tensor with a random skip "
                            "(262,144 descriptors, 8 GiB a direction)",
                "metric": "load GB/s (kernel)", "value": r["h2d_kernel_gbs"], "unit": "GB/s",
                "store_gbs": r["d2h_kernel_gbs"], "load_sdma_gbs": r["h2d_sdma_gbs"],
                "load_runtime_gbs": r["h2d_runtime_gbs"],
                "table_build_ms": r["table_build_ms"],
                "roofline": _pcie_roofline(r["h2d_kernel_gbs"], peaks, kernel="copy_desc_kernel"),
                "cpu_baseline": {**r["cpu_baseline"],
                                 "value": r["cpu_baseline"]["all_threads_gbs"], "unit": "GB/s"}}

    def c3():
        r = suite_small_pages(torch, kvt, synth, dev, peaks, reps=1)
        row2k = next(x for x in r["sweep"] if x["page_bytes"] == 2048
                     and x["host_offset_mod16"] == 0)
        return {"workload": "65,536 scattered pages host->HBM, 512 B .. 64 KiB, then 4 GiB of "
                            "128 KiB .. 1 MiB pages (kernel, DMA engines, runtime copies); "
                            "2 KiB pages at the workload's size",
                "metric": "2 KiB-page load GB/s (kernel)", "value": row2k["kernel_gbs"],
                "unit": "GB/s", "sdma_gbs_2k": row2k["sdma_gbs"],
                "runtime_gbs_2k": row2k["runtime_gbs"],
                "crossover_bytes_sdma": r["h2d_crossover_bytes"],
                "crossover_bytes_runtime": r["h2d_crossover_bytes_runtime"],
                "sweep_kernel_gbs": {str(x["page_bytes"]) + ("@8mod16" if x["host_offset_mod16"]
                                                              else ""): x["kernel_gbs"]
                                     for x in r["sweep"]},
                "sweep_sdma_gbs": {str(x["page_bytes"]): x["sdma_gbs"] for x in r["sweep"]
                                   if not x["host_offset_mod16"]},
                "sdma_engines": kvt.kvt_copy_engines(kvt.H2D),
                "roofline": _pcie_roofline(row2k["kernel_gbs"], peaks, kernel="copy_small_kernel"),
                "cpu_baseline": {"value": r["cpu_baseline"]["512B"]["all_threads_gbs"],
                                 "unit": "GB/s", "kind": "oracle",
                                 "cores": r["cpu_baseline"]["512B"]["cores"],
                                 "cpu_model": cpu_model(),
                                 "sample": "the memcpy loop over 65,536 pages of 512 B",
                                 "per_size": r["cpu_baseline"]}}

    def c4():
        w1m = DecodeWorkload(torch, kvt, synth, dev, 1 << 20, 2 * (args.warmup + args.steps) + 4,
                             "token_major")
        rr = w1m.run(args.steps, args.warmup)
        kern = w1m.gather_bytes / (rr["part_ms"]["gather_attn"] * 1e-3) / GB
        out = {"workload": "top-k sparse decode step at 1,048,576 tokens (16,384 pooled blocks, "
                           "2 GiB host planes per K/V), token-major host planes",
               "metric": "gather GB/s over whole steps", "unit": "GB/s",
               "value": round(w1m.gather_bytes / (rr["ms_per_step"] * 1e-3) / GB, 3),
               "decode_tok_s": round(1e3 / rr["ms_per_step"], 2),
               "part_ms": {k: round(v, 5) for k, v in rr["part_ms"].items()},
               "roofline": _pcie_roofline(kern, peaks, kernel="gather_decode_partial "
                                          "(with decode_merge)")}
        if not args.no_cpu:
            out["cpu_baseline"] = cpu_baseline(w1m, 5.0)
        w1m.free()
        return out

    def c5():
        r = suite_prefill(torch, kvt, synth, dev, peaks, reps=5, compact=True)
        tf = r["attn_f16_tflops"]
        cb = r["cpu_baseline"]
        return {"workload": "tiered prefill: 180,000-token q8_0 cache, [0, 94208) in HBM and the "
                            "tail in pinned host memory; 2048 causal queries x 32 heads at the "
                            "tail; tail staged host->HBM once, then flash attention",
                "metric": "prefill tok/s (staging overlapped with attention, 16,384-row arena)",
                "value": r["prefill_tok_s_auto"], "unit": "tok/s",
                "plan": "kvt_attn_prefill_auto: pipelined, rows converted to fp16 once",
                "prefill_tok_s_pipelined_q8_0_passes": r["prefill_tok_s_pipelined"],
                "prefill_tok_s_staged": r["prefill_tok_s_staged"],
                "stage_gbs": r["stage_gbs"],
                "attn_q8_0_ms": r["attn_staged_ms"], "attn_q8_0_tflops": r["attn_tflops"],
                "attn_f16_ms": r["attn_all_hbm_f16_cache_ms"], "attn_f16_tflops": tf,
                "roofline": {"bound": "mfma",
                             "kernel": "prefill_attn (fp16): the auto plan's passes run on rows "
                                       "converted from q8_0; timed as one pass over an fp16 "
                                       "cache in HBM (the q8_0 pass is attn_q8_0_tflops)",
                             "achieved": tf, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                             "flops_per_launch": r["flops"]},
                "staging_roofline": _pcie_roofline(r["stage_gbs"], peaks,
                                                   kernel="kvt_stage_tail (DMA engine or "
                                                          "copy_span_kernel, the faster)"),
                "cpu_baseline": {"value": cb["attn_rows_per_s"], "unit": "query rows/s",
                                 "stage_gbs": cb["stage_gbs"], "kind": "oracle",
                                 "cores": cb["cores"], "cpu_model": cb["cpu_model"],
                                 "sample": cb["sample"]}}

    timed("C1_swap_1_layer", c1)
    timed("C3_small_pages", c3)
    timed("C5_tiered_prefill", c5)
    timed("C4_topk_decode_1m", c4)
    timed("C2_swap_32_layers", c2)
    return cfg


def run_suite(torch, kvt, synth, dev, wl, args, peaks):
    want = set(args.suite.split(",")) if args.suite != "all" else {
        "prefill", "chain", "swap1", "small", "swap32", "qsa", "decode1m", "worker", "upkeep",
        "rows"}
    out = {}
    if "prefill" in want:
        log("suite: tiered prefill")
        out["tiered_prefill"] = suite_prefill(torch, kvt, synth, dev, peaks)
    if "chain" in want:
        log("suite: tiered prefill over a chain of layers, cache wholly in host memory")
        out["tiered_prefill_chain"] = suite_prefill_chain(torch, kvt, synth, dev, peaks)
    if "swap1" in want:
        log("suite: one-layer swap")
        out["swap_1_layer"] = suite_one_layer(torch, kvt, synth, dev, peaks)
    if "small" in want:
        log("suite: small pages")
        out["small_pages"] = suite_small_pages(torch, kvt, synth, dev, peaks)
    if "swap32" in want:
        log("suite: 32-layer swap")
        out["swap_32_layers"] = suite_32_layers(torch, kvt, synth, dev, peaks)
    if "qsa" in want:
        log("suite: QSA selection geometry")
        out["qsa_geometry"] = suite_qsa(torch, kvt, synth, dev, wl, args)
    if "worker" in want:
        log("suite: transfer worker and graph replay")
        out["worker"] = suite_worker(torch, kvt, synth, dev, wl, peaks)
    if "upkeep" in want:
        log("suite: paged writes and copy_page")
        out["upkeep"] = suite_upkeep(torch, kvt, synth, dev, peaks)
    if "rows" in want:
        log("suite: sparse attention over per-row selections")
        out["sparse_rows"] = suite_rows(torch, kvt, synth, dev, wl, peaks)
    if "decode1m" in want:
        log("suite: decode at 1,048,576")
        w1m = DecodeWorkload(torch, kvt, synth, dev, 1 << 20, args.warmup + 2 * args.steps)
        r = w1m.run(args.steps, args.warmup)
        out["decode_1m"] = {"ms_per_step": round(r["ms_per_step"], 5),
                            "decode_tok_s": round(1e3 / r["ms_per_step"], 2),
                            "gather_gbs_whole_step":
                                round(w1m.gather_bytes / (r["ms_per_step"] * 1e-3) / GB, 3),
                            "part_ms": {k: round(v, 5) for k, v in r["part_ms"].items()}}
        w1m.free()
    return out


if __name__ == "__main__":
    main()
