#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

A step is one pass of the whole verify hot path over one block of 16 drafted tokens:
40 attention layers (three in four are 512-token sliding-window layers over a 2,048-slot
position ring, every fourth a full-attention layer over a paged pool of 64-token chunks at
context 131,072) and the greedy accept over [17 x 65536] logits.  Inputs are seeded synthetic
data already resident in HBM; the step is captured once in a HIP graph and replayed.

The JSON line also carries the per-layer figure at context 262,144 (one paged verify layer,
both kernels), the roofline of the dominant kernel (the paged split-K attention kernel, timed
live with HIP events on the stream it runs on), the step by layer type, 1,024-token prefill
blocks through the pool and the ring (with their own matrix-core roofline), host paging of
chunks over PCIe and the verify over 8K resident of 256K, the four single-layer
workloads timed one by one (cold and warm, median / p10 / p90), a measured HBM read bandwidth,
and the fp64 oracle timed on the host cores over a bounded sample of the same workload (plus its
wall time per single-layer workload).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload stack_40l_131k|paged_256k]
    python bench.py --mode copy     # plain 1-GiB device copies, for HBM counter calibration
    python bench.py --mode kernel   # the dominant kernel alone (10 launches), for counter runs
    python bench.py --mode prefill-kernel   # the prefill kernel alone at 131,072 (3 launches)
    python bench.py --mode configs  # each single-layer workload and block append (16 and 1,024
                                    # rows) called 200 times (51 at 256K, for the prefill blocks
                                    # and for a page-out and page-in of 128 chunks), a
                                    # cache-evicting read before each, for a kernel trace
    python bench.py --mode traffic --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv
                                    # HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE /
                                    # WRITE_SIZE counter files, scaled by the copy calibration
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV GB/s (% of HBM peak) for 16-token verify attention; µs/layer at 256K"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_chunk_attn_paged_131k.json")
# the paged split kernel's source: its file and the two headers it includes
KERNEL_SRCS = [os.path.join(ROOT, "ring_kv_amd", "csrc", f)
               for f in ("attn_chunked.hip", "rkv_device.hpp", "rkv_launch.hpp")]
# timed calls per single-layer workload: 200 for the short ones, 51 (a multiple of the three
# pool copies) for the 262,144-context layer, the prefill blocks and the paging calls
N_SMALL, N_LARGE = 200, 51
# replays behind the step's per-step distribution (at least this many, or --steps if more)
N_STEP_DIST = 50


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stack_40l_131k",
                    choices=["stack_40l_131k", "paged_256k"])
    ap.add_argument("--mode", default="bench",
                    choices=["bench", "copy", "kernel", "prefill-kernel", "traffic", "configs"])
    for f in ("fetch", "write", "copy_fetch", "copy_write"):
        ap.add_argument("--" + f.replace("_", "-"), default=None)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-256k", action="store_true", help="skip the 262,144-context layer")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the single-layer workloads timed one by one")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 1,024-token prefill blocks")
    ap.add_argument("--no-paging", action="store_true",
                    help="skip host paging and the resident-subset verify")
    return ap.parse_args()


def kernel_hash() -> str:
    """16 hex digits of the sha256 of the paged split kernel's code: its source files with
    comments and blank space taken out, so that an edit to a comment keeps the HBM counter
    record valid and any change to the code drops it."""
    import re
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        src = open(path, encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def graph_ms(fn, inner, reps, torch):
    """ms per call of fn: `inner` calls captured in one HIP graph, replayed `reps` times."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            fn()
    g.replay()
    torch.cuda.synchronize()
    return event_ms(g.replay, reps, torch) / inner


def median_graph_us(fn, reps, torch, rounds=3):
    """µs per call: the median of `rounds` graph measurements of two calls each (the matrix-core
    kernels' clock moves with the card's power draw, by up to ~8% between rounds)."""
    import statistics
    return statistics.median(graph_ms(fn, 2, reps, torch) for _ in range(rounds)) * 1e3


def event_ms(fn, n, torch):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(n):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n


def capture(fn, torch):
    """fn captured in a HIP graph (after one run on a side stream, as torch recommends)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def ring_workspace(torch):
    """A persistent, zeroed workspace for the window layers (16 query / 4 KV heads, head_dim 128,
    2,048-slot ring, window 512): with its counters the layer runs as one launch."""
    import ctypes
    import ring_kv_amd as rk
    from ring_kv_amd._lib import AttnDims
    dims = AttnDims(16, 16, 4, 128, 0.0, 1)
    n = rk.lib().verify_attn_ring_workspace_bytes(ctypes.byref(dims), 2048, 512, 0)
    return torch.zeros(max(1, n), dtype=torch.uint8, device="cuda")


def per_call_ms(fn, n, torch):
    """ms of each of n calls: HIP events recorded around every call."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def pct(xs, q):
    """q-th percentile (0..100) of a list, linear interpolation."""
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=float), q))


def dist(xs, nd=2):
    return {"median": round(pct(xs, 50), nd), "p10": round(pct(xs, 10), nd),
            "p90": round(pct(xs, 90), nd), "n": len(xs)}


def kernel_times(torch, fn, n, pre=None, skip="read_probe"):
    """The device's own kernel durations, from the HIP kernel records the in-process profiler
    (torch.profiler over roctracer) collects: fn is called n times, pre() before each call (its
    kernels, named like `skip`, are not counted).  Returns (per-call sums of the durations of the
    call's kernels in µs, {kernel name: [durations µs]}).  These are the same per-dispatch
    durations a rocprofv3 kernel trace reports; launch gaps are not in them."""
    from torch.autograd import DeviceType
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(n):
            if pre is not None:
                pre()
            fn()
        torch.cuda.synchronize()
    evs = [e for e in prof.events() if e.device_type == DeviceType.CUDA and skip not in e.name]
    evs.sort(key=lambda e: e.time_range.start)
    dur = lambda e: getattr(e, "device_time", None) or e.cuda_time  # noqa: E731
    by_name = {}
    for e in evs:
        by_name.setdefault(e.name, []).append(dur(e))
    if n == 0 or len(evs) % n:
        return [], by_name
    k = len(evs) // n
    return [sum(dur(e) for e in evs[i * k:(i + 1) * k]) for i in range(n)], by_name


def short_name(name):
    """`chunk_attn_kernel<128, 4, 2, true>` from a demangled kernel name."""
    import re
    m = re.search(r"(\w+_kernel(?:<[^>]*>)?)", name)
    return m.group(1) if m else name[:60]


class Stack:
    """Device-resident inputs, outputs and workspaces of the 40-layer verify step."""

    def __init__(self, torch, rk, synth):
        self.torch, self.rk = torch, rk
        t = lambda a: rk.tensor_from_numpy(a, "cuda")  # noqa: E731
        self.layers = []
        self.kv_bytes = 0
        for l in range(synth.STACK_LAYERS):
            c, acc = synth.workload("stack_40l_131k", l, keep_rows=False)
            d = dict(kind=c.kind, q=t(c.q), out=torch.empty((16, 16, 128), dtype=torch.float32, device="cuda"),
                     lse=torch.empty((16, 16), dtype=torch.float32, device="cuda"))
            if c.kind == "ring":
                d.update(k=t(c.k_ring), v=t(c.v_ring), pos0=c.pos0, window=c.window)
            else:
                d.update(k=t(c.k_pool), v=t(c.v_pool), pt=t(c.page_table), ctx=c.ctx_len)
            self.kv_bytes += c.kv_bytes
            self.layers.append(d)
            del c
        self.accept = acc
        self.logits = t(acc.logits)
        self.prop = t(acc.proposals)
        self.acc_len = torch.empty(1, dtype=torch.int32, device="cuda")
        self.committed = torch.empty(17, dtype=torch.int32, device="cuda")
        self.argmax = torch.empty(17, dtype=torch.int32, device="cuda")
        self.accept_bytes = acc.logits.nbytes
        L = rk.lib()
        from ring_kv_amd._lib import AttnDims
        import ctypes
        dims = AttnDims(16, 16, 4, 128, 0.0, 1)
        self.ws_paged = torch.empty(max(1, L.verify_attn_paged_workspace_bytes(ctypes.byref(dims), 131072, 64, 0)),
                                    dtype=torch.uint8, device="cuda")
        self.ws_ring = torch.zeros(max(1, L.verify_attn_ring_workspace_bytes(ctypes.byref(dims), 2048, 512, 0)),
                                   dtype=torch.uint8, device="cuda")
        self.ws_acc = torch.zeros(L.verify_accept_workspace_bytes(16, 65536), dtype=torch.uint8, device="cuda")
        self.splits = rk.verify_attn_paged_auto_splits(16, 4, 128, 16, 131072)
        self.part_o = torch.empty((4, self.splits, 64, 128), dtype=torch.float32, device="cuda")
        self.part_l = torch.empty((4, self.splits, 64), dtype=torch.float32, device="cuda")

    def step(self):
        rk = self.rk
        for d in self.layers:
            if d["kind"] == "ring":
                rk.verify_attn_ring(d["q"], d["k"], d["v"], d["pos0"], d["window"], out=d["out"],
                                    lse=d["lse"], workspace=self.ws_ring)
            else:
                rk.verify_attn_paged(d["q"], d["k"], d["v"], d["pt"], d["ctx"], out=d["out"],
                                     lse=d["lse"], workspace=self.ws_paged)
        rk.verify_accept(self.logits, self.prop, accept_len=self.acc_len, committed=self.committed,
                         row_argmax=self.argmax, workspace=self.ws_acc)

    def ring_round(self):
        for d in self.layers:
            if d["kind"] == "ring":
                self.rk.verify_attn_ring(d["q"], d["k"], d["v"], d["pos0"], d["window"],
                                         out=d["out"], lse=d["lse"], workspace=self.ws_ring)

    def paged_round(self):
        for d in self.layers:
            if d["kind"] == "paged":
                self.rk.verify_attn_paged(d["q"], d["k"], d["v"], d["pt"], d["ctx"], out=d["out"],
                                          lse=d["lse"], workspace=self.ws_paged)

    def accept_once(self):
        self.rk.verify_accept(self.logits, self.prop, accept_len=self.acc_len,
                              committed=self.committed, row_argmax=self.argmax,
                              workspace=self.ws_acc)

    def paged_partial_round(self):
        """The dominant kernel alone: the paged split-K kernel over each paged layer once."""
        for d in self.layers:
            if d["kind"] == "paged":
                self.rk.verify_attn_paged_partial(d["q"], d["k"], d["v"], d["pt"], d["ctx"],
                                                  self.splits, part_out=self.part_o,
                                                  part_lse=self.part_l)

    def decode_setup(self, steps):
        """The decode loop over this step's stores: every layer appends the block's 16 K/V rows
        at the device-resident position, attends, then the accept and the on-device advance by
        a + 1 (the planted agreement of the step's logits).  It starts early enough that `steps`
        replays stay inside the pools (whose tables cover positions up to 131,071) and ends at
        131,056 at the latest.  It writes into the stores: run it after the step's parity."""
        torch = self.torch
        self.adv = self.accept.planted_accept + 1
        self.pos_cap = 131072 - 16
        self.pos_first = self.pos_cap - self.adv * steps
        self.d_pos = torch.tensor([self.pos_first], dtype=torch.int64, device="cuda")
        g = torch.Generator(device="cuda").manual_seed(11)
        for d in self.layers:
            d["k_new"] = torch.randn((16, 4, 128), device="cuda", generator=g).to(torch.bfloat16)
            d["v_new"] = torch.randn((16, 4, 128), device="cuda", generator=g).to(torch.bfloat16)
        L = self.rk.lib()
        from ring_kv_amd._lib import AttnDims
        import ctypes
        dims = AttnDims(16, 16, 4, 128, 0.0, 1)
        self.ws_paged_dev = torch.empty(max(1, L.verify_attn_paged_workspace_bytes(
            ctypes.byref(dims), self.pos_cap + 16, 64, 0)), dtype=torch.uint8, device="cuda")

    def decode_step_fused(self):
        """decode_step with each layer's append inside its attention launch."""
        rk, cap, dp = self.rk, self.pos_cap, self.d_pos
        for d in self.layers:
            if d["kind"] == "ring":
                rk.verify_attn_ring_append_dev(d["q"], d["k_new"], d["v_new"], d["k"], d["v"], dp,
                                               cap, d["window"], out=d["out"], lse=d["lse"],
                                               workspace=self.ws_ring)
            else:
                rk.verify_attn_paged_append_dev(d["q"], d["k_new"], d["v_new"], d["k"], d["v"],
                                                d["pt"], dp, cap, out=d["out"], lse=d["lse"],
                                                workspace=self.ws_paged_dev)
        rk.verify_accept(self.logits, self.prop, accept_len=self.acc_len, committed=self.committed,
                         row_argmax=self.argmax, workspace=self.ws_acc)
        rk.verify_pos_advance(dp, self.acc_len)

    def decode_step(self):
        rk, cap, dp = self.rk, self.pos_cap, self.d_pos
        for d in self.layers:
            if d["kind"] == "ring":
                rk.verify_kv_append_ring_dev(d["k_new"], d["v_new"], dp, cap, d["k"], d["v"])
                rk.verify_attn_ring_dev(d["q"], d["k"], d["v"], dp, cap, d["window"], out=d["out"],
                                        lse=d["lse"], workspace=self.ws_ring)
            else:
                rk.verify_kv_append_paged_dev(d["k_new"], d["v_new"], dp, cap, d["k"], d["v"],
                                              d["pt"])
                rk.verify_attn_paged_dev(d["q"], d["k"], d["v"], d["pt"], dp, cap, out=d["out"],
                                         lse=d["lse"], workspace=self.ws_paged_dev)
        rk.verify_accept(self.logits, self.prop, accept_len=self.acc_len, committed=self.committed,
                         row_argmax=self.argmax, workspace=self.ws_acc)
        rk.verify_pos_advance(dp, self.acc_len)

    def decode_kv_bytes(self, pos):
        """KV bytes the decode step at block position `pos` attends: 30 window spans of 527
        positions and 10 pools of pos + 16 positions, 2,048 B per position (K and V, 4 KV heads,
        D 128, bf16)."""
        return 30 * 527 * 2048 + 10 * (pos + 16) * 2048


def attn_flops(c):
    """QK^T + PV flops of an attention case, counting exactly the keys each query sees."""
    vis = 0
    for i in range(c.q_len):
        p = c.pos0 + i if c.kind == "ring" else c.ctx_len - c.q_len + i
        vis += min(p + 1, c.window) if c.window else p + 1
    return 4 * c.head_dim * c.n_q_heads * vis


class ReadProbe:
    """The streaming read probe (ring_kv_amd/libring_kv_probe.so): plain 16-byte loads over a
    buffer, nothing else.  Used to flush the caches without leaving dirty lines behind, and to
    measure the HBM read bandwidth this GPU delivers."""

    def __init__(self, torch):
        import ctypes
        self.torch = torch
        self.L = ctypes.CDLL(os.path.join(ROOT, "ring_kv_amd", "libring_kv_probe.so"))
        self.L.rkv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p]
        self.sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")

    def read(self, buf, workgroups=1024):
        rc = self.L.rkv_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), workgroups,
                                   self.sink.data_ptr(),
                                   self.torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"rkv_probe_read: hip error {rc}")


def config_timings(torch, rk, synth, probe, n_small, n_large):
    """The single-layer workloads (plus the small accept and the block appends), each captured n
    times in one HIP graph: warm = back-to-back calls; cold (calls of 20 µs and more) = every call
    preceded by a 512 MiB streaming read that evicts L2 and the last-level cache without dirtying
    them, minus a graph of the reads alone; the 256K pool also rotates over three copies.  Mean
    µs per call, launch gaps included.  Beside them, the device's own kernel time per call (the
    call's kernel durations summed, from the in-process kernel records), warm and cold: median,
    p10, p90 over the same n calls (200 for the small workloads, 51 at 256K)."""
    t = lambda a: rk.tensor_from_numpy(a, "cuda")  # noqa: E731
    scratch = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    flush = lambda: probe.read(scratch)  # noqa: E731
    flush_us = graph_ms(flush, n_small, 3, torch) * 1e3
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")  # noqa: E731
    out = {"flush_us": round(flush_us, 1)}

    def entry(name, fns, n, nbytes, flops, peak_tflops, flops_unit, note):
        turn = [0]

        def op():
            turn[0] += 1
            fns[turn[0] % len(fns)]()

        def cold_op():
            flush()
            op()

        n = n // len(fns) * len(fns)
        warm = graph_ms(op, n, 3, torch) * 1e3
        e = {"us_warm": round(warm, 2), "calls_per_graph": n, "note": note}
        # the device's own kernel time per call (the sum of the call's kernel durations, as a
        # kernel trace gives them): back to back (warm) and after a cache-evicting read (cold)
        kw, _ = kernel_times(torch, op, n)
        kc, _ = kernel_times(torch, op, n, pre=flush)
        if kw and kc:
            e["kernel_us_warm"] = dist(kw)
            e["kernel_us_cold"] = dist(kc)
            if nbytes and e["kernel_us_cold"]["median"] > 0:
                kmed = e["kernel_us_cold"]["median"]
                e["gbps_kernel_cold"] = round(nbytes / (kmed * 1e-6) / 1e9, 1)
                e["hbm_frac_kernel_cold"] = round(e["gbps_kernel_cold"] / HBM_PEAK_GBPS, 4)
        t, which = warm, "warm"
        if warm >= 20.0:
            # the difference of two graphs resolves only calls well above the launch overlap;
            # shorter calls get their cold per-dispatch durations from the kernel trace of
            # `bench.py --mode configs`
            cold = graph_ms(cold_op, n, 3, torch) * 1e3 - flush_us
            e["us_cold"] = round(cold, 2)
            t, which = cold, "cold"
        if nbytes:
            e["gbps_" + which] = round(nbytes / (t * 1e-6) / 1e9, 1)
            e["hbm_frac_" + which] = round(e["gbps_" + which] / HBM_PEAK_GBPS, 4)
        if flops:
            tf = flops / (t * 1e-6) / 1e12
            e.update({"flops": flops, "tflops_" + which: round(tf, 2), "peak_tflops": peak_tflops,
                      "util_" + flops_unit: round(tf / peak_tflops, 4)})
        out[name] = e

    # C1: contiguous 1,024-key verify, f32 (VALU arithmetic), and the accept over [17 x 4096]
    c, acc = synth.workload("contig_1k_f32")
    q, k, v = t(c.q), t(c.k_rows), t(c.v_rows)
    o1, l1 = f32(16, 8, 64), f32(16, 8)
    entry("contig_1k_f32", [lambda: rk.decode_attn_ref_layout(q, k, v, 1024, out=o1, lse=l1)],
          n_small, c.kv_bytes, attn_flops(c), 157.3, "mfma_fp32",
          "decode_attn_ref_layout, auto splits; bound: launch latency")
    lg, pr = t(acc.logits), t(acc.proposals)
    al, cm, am = (torch.empty(n, dtype=torch.int32, device="cuda") for n in (1, 17, 17))
    entry("accept_17x4096", [lambda: rk.verify_accept(lg, pr, accept_len=al, committed=cm,
                                                      row_argmax=am)],
          n_small, acc.logits.nbytes, 0, 0, "", "verify_accept; bound: launch latency")
    # C2: window 512 over the 2,048-slot ring (a persistent workspace, counters zeroed once: the
    # layer in one launch)
    c, _ = synth.workload("ring_w512_r2048", keep_rows=False)
    q2, kr, vr = t(c.q), t(c.k_ring), t(c.v_ring)
    o, l = f32(16, 16, 128), f32(16, 16)
    wsr = ring_workspace(torch)
    entry("ring_w512_r2048", [lambda: rk.verify_attn_ring(q2, kr, vr, c.pos0, c.window, out=o,
                                                          lse=l, workspace=wsr)],
          n_small, c.kv_bytes, attn_flops(c), 2500.0, "mfma_bf16",
          "verify_attn_ring, one chunk per split, merged in the same launch; bound: launch latency")
    # C3: paged 8K
    c3, _ = synth.workload("paged_8k", keep_rows=False)
    q3, kp3, vp3, pt3 = t(c3.q), t(c3.k_pool), t(c3.v_pool), t(c3.page_table)
    entry("paged_8k", [lambda: rk.verify_attn_paged(q3, kp3, vp3, pt3, 8192, out=o, lse=l)],
          n_small, c3.kv_bytes, attn_flops(c3), 2500.0, "mfma_bf16",
          "verify_attn_paged, auto splits + merge")
    # C4: paged 256K, three pool copies in turn
    c4, _ = synth.workload("paged_256k", keep_rows=False)
    q4, pt4 = t(c4.q), t(c4.page_table)
    pools = [(t(c4.k_pool), t(c4.v_pool))]
    pools += [(pools[0][0].clone(), pools[0][1].clone()) for _ in range(2)]
    fns = [lambda kp=kp, vp=vp: rk.verify_attn_paged(q4, kp, vp, pt4, 262144, out=o, lse=l)
           for kp, vp in pools]
    entry("paged_256k", fns, n_large, c4.kv_bytes, attn_flops(c4), 2500.0, "mfma_bf16",
          "verify_attn_paged, 64 splits + merge; warm = back-to-back over the three pool copies")
    del pools, fns
    # the block's own K/V rows appended before its attention (16 rows, 4 KV heads, D 128): the
    # ring and the pool (the pool append also writes the page-table entries of chunks it starts)
    g = torch.Generator(device="cuda").manual_seed(0)
    kb = torch.randn((16, 4, 128), device="cuda", generator=g).to(torch.bfloat16)
    vb = torch.randn((16, 4, 128), device="cuda", generator=g).to(torch.bfloat16)
    kr = torch.zeros((32, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros((32, 4, 128, 64), dtype=torch.bfloat16, device="cuda")
    entry("append_ring_16", [lambda: rk.verify_kv_append_ring(kb, vb, 131056, kr, vr)], n_small,
          2 * kb.numel() * 2, 0, 0, "", "verify_kv_append_ring, 16 rows; bound: launch latency")
    kp = torch.zeros((2048, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((2048, 4, 128, 64), dtype=torch.bfloat16, device="cuda")
    table = torch.arange(2050, dtype=torch.int32, device="cuda") % 2048
    entry("append_paged_16", [lambda: rk.verify_kv_append_paged(kb, vb, 131064, kp, vp, table,
                                                                2048, [2047])], n_small,
          2 * kb.numel() * 2, 0, 0, "", "verify_kv_append_paged, 16 rows starting one chunk")
    # a 1,024-token prefill block's rows appended (4 KV heads, D 128: 2 MiB of K and V)
    kb1 = torch.randn((1024, 4, 128), device="cuda", generator=g).to(torch.bfloat16)
    vb1 = torch.randn((1024, 4, 128), device="cuda", generator=g).to(torch.bfloat16)
    entry("append_ring_1024", [lambda: rk.verify_kv_append_ring(kb1, vb1, 130048, kr, vr)], n_small,
          2 * kb1.numel() * 2, 0, 0, "", "verify_kv_append_ring, 1,024 rows")
    new16 = list(range(2032, 2048))
    entry("append_paged_1024", [lambda: rk.verify_kv_append_paged(kb1, vb1, 130048, kp, vp, table,
                                                                  2032, new16)], n_small,
          2 * kb1.numel() * 2, 0, 0, "", "verify_kv_append_paged, 1,024 rows starting 16 chunks")
    copy_src = torch.empty(2 << 20, dtype=torch.uint8, device="cuda")
    copy_dst = torch.empty_like(copy_src)
    entry("copy_2mib", [lambda: copy_dst.copy_(copy_src)], n_small, 2 * (2 << 20), 0, 0, "",
          "a plain 2 MiB device copy (torch), for comparison with the 1,024-row appends")
    pager = rk.Pager(4096, 4096)
    t0 = time.perf_counter()
    for i in range(2000):
        pager.reserve(16)
        pager.commit(1 + i % 16)
    out["pager_reserve_commit_host_us"] = round((time.perf_counter() - t0) / 2000 * 1e6, 2)
    pager.close()
    del scratch, kp, vp
    torch.cuda.empty_cache()
    return out


def config_calls(torch, rk, synth, probe, n_small, n_large):
    """Eager calls of the single-layer workloads, each preceded by a 512 MiB streaming read, for
    a rocprofv3 kernel trace (per-dispatch durations: median, p10, p90)."""
    t = lambda a: rk.tensor_from_numpy(a, "cuda")  # noqa: E731
    scratch = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")  # noqa: E731

    def run(fn, n):
        for _ in range(n):
            probe.read(scratch)
            fn()
        torch.cuda.synchronize()

    c, acc = synth.workload("contig_1k_f32")
    q, k, v = t(c.q), t(c.k_rows), t(c.v_rows)
    o1, l1 = f32(16, 8, 64), f32(16, 8)
    run(lambda: rk.decode_attn_ref_layout(q, k, v, 1024, out=o1, lse=l1), n_small)
    lg, pr = t(acc.logits), t(acc.proposals)
    run(lambda: rk.verify_accept(lg, pr), n_small)
    o, l = f32(16, 16, 128), f32(16, 16)
    for name, n in (("ring_w512_r2048", n_small), ("paged_8k", n_small), ("paged_256k", n_large)):
        c, _ = synth.workload(name, keep_rows=False)
        q = t(c.q)
        if c.kind == "ring":
            kr, vr = t(c.k_ring), t(c.v_ring)
            wsr = ring_workspace(torch)
            run(lambda: rk.verify_attn_ring(q, kr, vr, c.pos0, c.window, out=o, lse=l,
                                            workspace=wsr), n)
        else:
            kp, vp, pt = t(c.k_pool), t(c.v_pool), t(c.page_table)
            run(lambda: rk.verify_attn_paged(q, kp, vp, pt, c.ctx_len, out=o, lse=l), n)
            del kp, vp
        torch.cuda.empty_cache()
    kb = torch.ones((16, 4, 128), dtype=torch.bfloat16, device="cuda")
    kr = torch.zeros((32, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros((32, 4, 128, 64), dtype=torch.bfloat16, device="cuda")
    run(lambda: rk.verify_kv_append_ring(kb, kb, 131056, kr, vr), n_small)
    kp = torch.zeros((2048, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((2048, 4, 128, 64), dtype=torch.bfloat16, device="cuda")
    table = torch.arange(2050, dtype=torch.int32, device="cuda") % 2048
    run(lambda: rk.verify_kv_append_paged(kb, kb, 131064, kp, vp, table, 2048, [2047]), n_small)
    kb1 = torch.ones((1024, 4, 128), dtype=torch.bfloat16, device="cuda")
    run(lambda: rk.verify_kv_append_ring(kb1, kb1, 130048, kr, vr), n_small)
    new16 = list(range(2032, 2048))
    run(lambda: rk.verify_kv_append_paged(kb1, kb1, 130048, kp, vp, table, 2032, new16), n_small)
    del kp, vp
    torch.cuda.empty_cache()
    # 1,024-token prefill blocks through the pool and the ring
    for name in ("prefill_pool_8k", "prefill_ring_w512", "prefill_pool_131k"):
        c, _ = synth.workload(name, keep_rows=False)
        q = t(c.q)
        o, l = f32(c.q_len, 16, 128), f32(c.q_len, 16)
        if c.kind == "ring":
            kr, vr = t(c.k_ring), t(c.v_ring)
            run(lambda: rk.verify_attn_ring(q, kr, vr, c.pos0, c.window, out=o, lse=l), n_large)
        else:
            kp, vp, pt = t(c.k_pool), t(c.v_pool), t(c.page_table)
            run(lambda: rk.verify_attn_paged(q, kp, vp, pt, c.ctx_len, out=o, lse=l), n_large)
            del kp, vp
        torch.cuda.empty_cache()
    # host paging: 128 chunks out to pinned host memory and back, one run of chunk ids
    kp = torch.zeros((1024, 4, 64, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((1024, 4, 128, 64), dtype=torch.bfloat16, device="cuda")
    kh = torch.empty((1024, 4, 64, 128), dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty((1024, 4, 128, 64), dtype=torch.bfloat16, pin_memory=True)
    slots, ids = list(range(512, 640)), list(range(200, 328))
    ws = torch.empty(rk.lib().kv_page_workspace_bytes(4, 128, 128), dtype=torch.uint8,
                     device="cuda")
    run(lambda: rk.kv_page_out(kp, vp, slots, ids, kh, vh, workspace=ws), n_large)
    run(lambda: rk.kv_page_in(kh, vh, ids, slots, kp, vp, workspace=ws), n_large)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure


def prefill_timings(torch, rk, synth, reps):
    """Batched prefill: 1,024-token blocks through the pool (after 8,192 and 130,048 prior
    tokens) and the ring (window 512), each call captured in a HIP graph and replayed (mean µs
    per call; the calls are bound by the matrix cores, so warm and cold agree).  Also the paged
    split kernel alone at 131,072 (the prefill roofline: flops of the keys each query sees over
    its launch time) and the attention of one prefill block through the 40-layer stack."""
    import ctypes
    from ring_kv_amd._lib import AttnDims
    t = lambda a: rk.tensor_from_numpy(a, "cuda")  # noqa: E731
    out = {}
    for name in ("prefill_pool_8k", "prefill_ring_w512", "prefill_pool_131k"):
        c, _ = synth.workload(name, keep_rows=False)
        q = t(c.q)
        o = torch.empty((c.q_len, c.n_q_heads, c.head_dim), dtype=torch.float32, device="cuda")
        l = torch.empty((c.q_len, c.n_q_heads), dtype=torch.float32, device="cuda")
        flops = attn_flops(c)
        e = {"q_len": c.q_len, "flops": flops}
        if c.kind == "ring":
            kr, vr = t(c.k_ring), t(c.v_ring)
            fn = lambda: rk.verify_attn_ring(q, kr, vr, c.pos0, c.window, out=o, lse=l)  # noqa: E731
            e["splits"] = 1
        else:
            kp, vp, pt = t(c.k_pool), t(c.v_pool), t(c.page_table)
            S = rk.verify_attn_paged_auto_splits(16, 4, 128, c.q_len, c.ctx_len)
            ws = torch.empty(rk.lib().verify_attn_paged_workspace_bytes(
                ctypes.byref(AttnDims(c.q_len, 16, 4, 128, 0.0, 1)), c.ctx_len, 64, 0),
                dtype=torch.uint8, device="cuda")
            fn = lambda: rk.verify_attn_paged(q, kp, vp, pt, c.ctx_len, out=o, lse=l,  # noqa: E731
                                              workspace=ws)
            e["splits"] = S
            if name == "prefill_pool_131k":
                rows = c.q_len * 4
                po = torch.empty((4, S, rows, 128), dtype=torch.float32, device="cuda")
                pl = torch.empty((4, S, rows), dtype=torch.float32, device="cuda")
                part = lambda: rk.verify_attn_paged_partial(q, kp, vp, pt, c.ctx_len, S,  # noqa: E731
                                                            part_out=po, part_lse=pl)
                k_us = median_graph_us(part, reps, torch)
                tf = flops / (k_us * 1e-6) / 1e12
                out["roofline_mfma"] = {
                    "bound": "mfma",
                    "kernel": "prefill_attn_kernel (paged, 256-row tiles, 4 splits) at 131,072",
                    "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "us_per_launch": round(k_us, 1),
                    "algorithmic_flops_per_launch": flops, "traffic": None}
        us = median_graph_us(fn, reps, torch)
        tf = flops / (us * 1e-6) / 1e12
        e.update({"us": round(us, 1), "tflops": round(tf, 1),
                  "util_mfma_bf16": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                  "tokens_per_s_one_layer": round(c.q_len / (us * 1e-6))})
        out[name] = e
        del c
        torch.cuda.empty_cache()
    ring_us, pool_us = out["prefill_ring_w512"]["us"], out["prefill_pool_131k"]["us"]
    stack_us = 30 * ring_us + 10 * pool_us
    out["stack_40l_131k_block_attention"] = {
        "us": round(stack_us, 1), "tokens_per_s": round(1024 / (stack_us * 1e-6)),
        "note": "attention only (30 ring layers + 10 paged layers at 131,072) of one 1,024-token "
                "prefill block; the pages' ~3,500 tok/s is whole-engine prefill on an RTX 3090"}
    return out


PCIE_PEAK_GBPS = 64.0   # PCIe 5.0 x16, one direction, vendor figure


def paging_timings(torch, rk, reps):
    """Host paging: 128 chunks (8,192 positions, 4 KV heads, D 128: 16 MiB of K and V) paged out
    to pinned host memory and back in, as one run of consecutive chunk ids and as 128 scattered
    ones (µs per call, events around `reps` eager calls); and the pages' own configuration, a
    verify block at context 262,144 with 8,192 positions resident (128 drawn chunks + the block's
    own), attention over the resident subset in graph replay."""
    g = torch.Generator(device="cuda").manual_seed(7)
    n, n_slots, n_host, hkv, d = 128, 1024, 1024, 4, 128
    kp = torch.randn((n_slots, hkv, 64, d), device="cuda", generator=g).to(torch.bfloat16)
    vp = torch.randn((n_slots, hkv, d, 64), device="cuda", generator=g).to(torch.bfloat16)
    kh = torch.empty((n_host, hkv, 64, d), dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty((n_host, hkv, d, 64), dtype=torch.bfloat16, pin_memory=True)
    perm = torch.randperm(n_slots, generator=torch.Generator().manual_seed(8)).tolist()
    slots = perm[:n]
    runs = {"one_run": list(range(200, 200 + n)),
            "scattered": sorted(torch.randperm(n_host, generator=torch.Generator().manual_seed(9))
                                [:n].tolist())}
    nbytes = n * 2 * hkv * 64 * d * 2
    ws = rk.kv_page_out(kp, vp, slots, runs["one_run"], kh, vh)
    out = {"chunks": n, "bytes": nbytes, "pcie_peak_gbps": PCIE_PEAK_GBPS}
    for name, ids in runs.items():
        for way in ("out", "in"):
            if way == "out":
                fn = lambda ids=ids: rk.kv_page_out(kp, vp, slots, ids, kh, vh, workspace=ws)  # noqa: E731
            else:
                fn = lambda ids=ids: rk.kv_page_in(kh, vh, ids, slots, kp, vp, workspace=ws)  # noqa: E731
            for _ in range(3):
                fn()
            # median of three rounds (the first copies to a fresh pinned buffer in a process
            # can take several times longer)
            us = sorted(event_ms(fn, reps, torch) for _ in range(3))[1] * 1e3
            gbps = nbytes / (us * 1e-6) / 1e9
            out[f"page_{way}_{name}"] = {"us": round(us, 1), "gbps": round(gbps, 2),
                                          "pcie_frac": round(gbps / PCIE_PEAK_GBPS, 4)}
    del kp, vp, kh, vh, ws
    torch.cuda.empty_cache()
    # verify at 262,144 with 8K resident: 128 drawn chunks below the block's + chunk 4,095
    gen = torch.Generator().manual_seed(10)
    ids = sorted(torch.randperm(4095, generator=gen)[:128].tolist()) + [4095]
    n_res = len(ids)
    kp = torch.randn((n_res, hkv, 64, d), device="cuda", generator=g).to(torch.bfloat16)
    vp = torch.randn((n_res, hkv, d, 64), device="cuda", generator=g).to(torch.bfloat16)
    q = torch.randn((16, 16, d), device="cuda", generator=g).to(torch.bfloat16)
    d_slots = torch.arange(n_res, dtype=torch.int32, device="cuda")
    o = torch.empty((16, 16, d), dtype=torch.float32, device="cuda")
    l = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    fn = lambda: rk.verify_attn_paged_resident(q, kp, vp, d_slots, ids, 262144, out=o, lse=l)  # noqa: E731
    us = graph_ms(fn, 20, reps, torch) * 1e3
    kv = n_res * 2 * hkv * 64 * d * 2
    out["verify_256k_8k_resident"] = {"us": round(us, 2), "resident_chunks": n_res,
                                      "kv_bytes": kv, "gbps": round(kv / (us * 1e-6) / 1e9, 1),
                                      "note": "the pages' configuration: 8K of the 256K context "
                                              "resident; graph replay, back to back"}
    return out


def read_bw_probe(torch, probe):
    """Measured HBM read bandwidth of this GPU: the streaming read probe over four 1 GiB buffers
    in turn (so no pass is served from the last-level cache), best of several grid sizes."""
    bufs = [torch.zeros(1 << 30, dtype=torch.uint8, device="cuda") for _ in range(4)]
    res = {}
    for wgs in (256, 512, 1024, 2048):
        turn = [0]

        def f():
            turn[0] += 1
            probe.read(bufs[turn[0] % 4], wgs)

        us = graph_ms(f, 8, 3, torch) * 1e3
        res[str(wgs)] = round((1 << 30) / (us * 1e-6) / 1e9, 1)
    del bufs
    torch.cuda.empty_cache()
    return {"gbps": max(res.values()), "by_workgroups": res,
            "method": "16-byte non-temporal loads over four 1 GiB buffers in turn, graph replay "
                      "(ring_kv_amd/csrc/probe.hip)"}


def cpu_info():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = ""
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                         if i.get("user_api") == "blas")
    except Exception:  # noqa: BLE001
        pass
    return model, blas


def oracle_per_config(synth, oracle):
    """The oracle's wall time per single-layer workload (µs): the median of three timed calls
    for the short workloads, one call at 262,144."""
    import statistics

    def timed(f, calls):
        ts = []
        for _ in range(calls):
            t0 = time.perf_counter()
            f()
            ts.append((time.perf_counter() - t0) * 1e6)
        return round(statistics.median(ts), 1)

    res = {}
    c, acc = synth.workload("contig_1k_f32")
    res["contig_1k_f32"] = timed(lambda: oracle.attention_contiguous(
        c.q, c.k_rows, c.v_rows, c.ctx_len, window=c.window, dtype=c.dtype), 3)
    res["accept_17x4096"] = timed(lambda: oracle.greedy_accept(acc.logits, acc.proposals), 3)
    for name, calls in (("ring_w512_r2048", 3), ("paged_8k", 3), ("paged_256k", 1)):
        c, _ = synth.workload(name, keep_rows=False)
        if c.kind == "ring":
            res[name] = timed(lambda: oracle.attention_ring(
                c.q, c.k_ring, c.v_ring, c.pos0, c.ring_head, c.ring_size, c.window), calls)
        else:
            res[name] = timed(lambda: oracle.attention_paged(
                c.q, c.k_pool, c.v_pool, c.page_table, c.ctx_len), calls)
        del c
    return res


CPU_SAMPLE_MIN_SECONDS = 10.0


def cpu_baseline(synth, oracle):
    """The fp64 oracle on a bounded sample of the step, timed on the host cores: one paged layer
    at 131,072, three ring layers and the accept (the step's 1:3 mix of layer types; ten samples
    are one step's work), repeated until at least CPU_SAMPLE_MIN_SECONDS of work.  Returns the
    oracle's results of the sample (by layer, and "accept") and the baseline entry."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    layer_ids = (3, 0, 1, 2)
    cases = [synth.workload("stack_40l_131k", l, keep_rows=False)[0] for l in layer_ids]
    acc = synth.workload("stack_40l_131k", 0, keep_rows=False)[1]
    kv = sum(c.kv_bytes for c in cases)
    reps, dt = 0, 0.0
    results = {}
    while dt < CPU_SAMPLE_MIN_SECONDS:
        t0 = time.perf_counter()
        for l, c in zip(layer_ids, cases):
            if c.kind == "paged":
                r = oracle.attention_paged(c.q, c.k_pool, c.v_pool, c.page_table, c.ctx_len)
            else:
                r = oracle.attention_ring(c.q, c.k_ring, c.v_ring, c.pos0, c.ring_head,
                                          c.ring_size, c.window)
            results.setdefault(l, r)
        results.setdefault("accept", oracle.greedy_accept(acc.logits, acc.proposals))
        dt += time.perf_counter() - t0
        reps += 1
    model, blas = cpu_info()
    return results, {"value": round(kv * reps / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3), "samples": reps,
            "sample": f"1 paged layer (ctx 131,072) + 3 ring layers + accept [17x65536] of the "
                      f"40-layer step (its 1:3 mix of layer types), {reps} times in a row (10 "
                      f"times = one step's work); KV bytes of the samples / wall time",
            "cpu": model, "blas": blas,
            "us_per_call": oracle_per_config(synth, oracle)}


def step_parity(step_out, ref):
    """The timed step's own outputs of layers 0-3 (three window layers, one paged layer at
    131,072) and of the accept, against the fp64 oracle's results of the baseline sample."""
    import numpy as np
    layers = sorted(k for k in ref if k != "accept")
    err_o = max(float(np.abs(step_out[l][0] - ref[l][0]).max()) for l in layers)
    err_l = max(float(np.abs(step_out[l][1] - ref[l][1]).max()) for l in layers)
    a, committed = step_out["accept"]
    ra, rcommitted, _ = ref["accept"]
    exact = a == ra and np.array_equal(committed[:a + 1], rcommitted) and \
        bool(np.all(committed[a + 1:] == -1))
    return {"layers": layers, "max_abs_out": err_o, "max_abs_lse": err_l, "tolerance": 1e-2,
            "within_tolerance": err_o <= 1e-2 and err_l <= 1e-2, "accept_exact": exact,
            "note": "the timed step's outputs of these layers and of the accept [17 x 65,536] "
                    "against the fp64 oracle (the cpu_baseline sample)"}


def counter_kib(path, kernel_substr):
    """Mean Counter_Value (KiB per dispatch) over the dispatches of one kernel in a rocprofv3
    counter_collection.csv."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"{path}: no dispatch of a kernel named like {kernel_substr!r}")
    return sum(vals) / len(vals), len(vals)


def traffic_summary(args):
    """HBM bytes per launch of the paged split kernel at 131,072: FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch), each scaled by the bytes a plain 1-GiB device copy moves over what the same
    counter reads for it."""
    copy_bytes = 1 << 30
    cf, _ = counter_kib(args.copy_fetch, "copy")
    cw, _ = counter_kib(args.copy_write, "copy")
    kf, n = counter_kib(args.fetch, "chunk_attn_kernel")
    kw, _ = counter_kib(args.write, "chunk_attn_kernel")
    f_scale, w_scale = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    fetch, write = kf * 1024 * f_scale, kw * 1024 * w_scale
    algo = 2 * 131072 * 4 * 128 * 2
    out = {"kernel": "chunk_attn_kernel (paged, split-K, 64 splits) at 131,072",
           "kernel_sha": kernel_hash(), "dispatches": n,
           "fetch_kib_raw": kf, "write_kib_raw": kw,
           "copy_fetch_kib_raw": cf, "copy_write_kib_raw": cw,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_fetch_bytes_per_launch": round(fetch), "hbm_write_bytes_per_launch": round(write),
           "hbm_bytes_per_launch": round(fetch + write),
           "algorithmic_bytes_per_launch": algo,
           "traffic_over_algorithmic": round((fetch + write) / algo, 4),
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_k_FETCH_SIZE -o p "
               "-- python3 bench.py --mode kernel",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_k_WRITE_SIZE -o p "
               "-- python3 bench.py --mode kernel",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_c_FETCH_SIZE -o p "
               "-- python3 bench.py --mode copy",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_c_WRITE_SIZE -o p "
               "-- python3 bench.py --mode copy",
               "python3 bench.py --mode traffic --fetch gpurun_out/pmc_k_FETCH_SIZE/p_counter_collection.csv "
               "--write gpurun_out/pmc_k_WRITE_SIZE/p_counter_collection.csv "
               "--copy-fetch gpurun_out/pmc_c_FETCH_SIZE/p_counter_collection.csv "
               "--copy-write gpurun_out/pmc_c_WRITE_SIZE/p_counter_collection.csv"]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def traffic_entry(per_launch_bytes):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
    except Exception:  # noqa: BLE001
        return None
    if t.get("kernel_sha") != kernel_hash():
        return None          # the kernel changed since the counters were taken
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.mode == "traffic":
        traffic_summary(args)
        return
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import ring_kv_amd as rk

    rk.lib()   # fails loudly if the HIP library is not built

    if args.mode == "copy":
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        ms = event_ms(lambda: b.copy_(a), 5, torch)
        print(json.dumps({"mode": "copy", "bytes_per_copy": n, "ms_per_copy": ms,
                          "gbps": 2 * n / ms / 1e6}), flush=True)
        return

    import ctypes

    import synth
    from ring_kv_amd._lib import AttnDims

    if args.mode == "kernel":
        # the dominant kernel alone: 10 launches of the paged split kernel over one layer
        c, _ = synth.workload("stack_40l_131k", 3, keep_rows=False)
        t = lambda a: rk.tensor_from_numpy(a, "cuda")  # noqa: E731
        q, kp, vp, pt = t(c.q), t(c.k_pool), t(c.v_pool), t(c.page_table)
        splits = rk.verify_attn_paged_auto_splits(16, 4, 128, 16, 131072)
        po = torch.empty((4, splits, 64, 128), dtype=torch.float32, device="cuda")
        pl = torch.empty((4, splits, 64), dtype=torch.float32, device="cuda")
        for _ in range(10):
            rk.verify_attn_paged_partial(q, kp, vp, pt, 131072, splits, part_out=po, part_lse=pl)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "kernel", "launches": 10, "splits": splits}), flush=True)
        return

    if args.mode == "prefill-kernel":
        # the prefill kernel alone: 3 launches over the 1,024-token block ending at 131,072,
        # 4 splits (partials, no merge)
        c, _ = synth.workload("prefill_pool_131k", keep_rows=False)
        t = lambda a: rk.tensor_from_numpy(a, "cuda")  # noqa: E731
        q, kp, vp, pt = t(c.q), t(c.k_pool), t(c.v_pool), t(c.page_table)
        po = torch.empty((4, 4, 4096, 128), dtype=torch.float32, device="cuda")
        pl = torch.empty((4, 4, 4096), dtype=torch.float32, device="cuda")
        for _ in range(3):
            rk.verify_attn_paged_partial(q, kp, vp, pt, c.ctx_len, 4, part_out=po, part_lse=pl)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "prefill-kernel", "launches": 3, "splits": 4}), flush=True)
        return

    if args.mode == "configs":
        config_calls(torch, rk, synth, ReadProbe(torch), N_SMALL, N_LARGE)
        print(json.dumps({"mode": "configs"}), flush=True)
        return

    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) bf16 K/V, planted-argmax logits)"}

    if args.workload == "stack_40l_131k":
        log("building the 40-layer step inputs")
        st = Stack(torch, rk, synth)
        for _ in range(args.warmup):
            st.step()
        torch.cuda.synchronize()
        eager_ms = event_ms(st.step, max(1, args.steps // 2), torch)
        log(f"eager step {eager_ms:.3f} ms")
        ms = eager_ms
        graph = False
        if not args.no_graph:
            g = capture(st.step, torch)
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            # the timed region: exactly `steps` replays between two synchronisations
            ms = event_ms(g.replay, args.steps, torch)
            graph = True
            log(f"graph step {ms:.3f} ms")
            step_fn = g.replay
        else:
            step_fn = st.step
        # the step's distribution: events around each replay; the device's kernel time per step
        # (the sum of its 82 kernels' durations) from the in-process kernel records
        per_step = per_call_ms(step_fn, max(N_STEP_DIST, args.steps), torch)
        k_step, k_by = kernel_times(torch, step_fn, min(5, args.steps))
        # dominant kernel: the paged split-K kernel at 131,072 over the 10 paged layers, three
        # rounds of 10 launches in one HIP graph; HIP events on the replay stream (launch gaps
        # included), and the kernels' own durations from the kernel records of the same replays
        st.paged_partial_round()
        gk = capture(lambda: [st.paged_partial_round() for _ in range(3)], torch)
        k_ms = event_ms(gk.replay, max(3, args.steps // 4), torch) / 30
        _, k_dom = kernel_times(torch, gk.replay, 2)
        dom = [v for n, v in k_dom.items() if "chunk_attn_kernel" in n]
        k_us = dom[0] if len(dom) == 1 else []
        per_launch = 2 * 131072 * 4 * 128 * 2
        achieved = per_launch / (k_ms * 1e-3) / 1e9
        kern_mean = sum(k_us) / len(k_us) if k_us else None
        log(f"paged split kernel {k_ms * 1e3:.1f} us/launch (events), "
            f"{kern_mean if kern_mean is None else round(kern_mean, 2)} us (kernel records)")
        # the step by layer type, each type captured alone (30 ring layers, 10 paged, accept)
        ring_us = graph_ms(st.ring_round, 1, max(3, args.steps // 2), torch) * 1e3 / 30
        paged_us = graph_ms(st.paged_round, 1, max(3, args.steps // 2), torch) * 1e3 / 10
        acc_us = graph_ms(st.accept_once, 5, max(3, args.steps // 2), torch) * 1e3
        log(f"per layer: ring {ring_us:.2f} us, paged {paged_us:.2f} us, accept {acc_us:.2f} us")
        res["per_layer_type_us"] = {"ring_w512": round(ring_us, 2), "paged_131k": round(paged_us, 2),
                                    "accept_17x65536": round(acc_us, 2),
                                    "sum_40_layers_and_accept": round(30 * ring_us + 10 * paged_us
                                                                      + acc_us, 1)}
        kv_gbps = st.kv_bytes / (ms * 1e-3) / 1e9
        res.update({
            "value": round(kv_gbps, 2), "unit": "GB/s",
            "ms_per_step": round(ms, 4), "eager_ms_per_step": round(eager_ms, 4),
            "hbm_frac": round(kv_gbps / HBM_PEAK_GBPS, 4),
            "step_ms": dist(per_step, 4),
            "step_kernel_ms": dist([x / 1e3 for x in k_step], 4) if k_step else None,
            "step_kernels_us": {short_name(n): dist(v) for n, v in k_by.items()},
            "with_logits_gbps": round((st.kv_bytes + st.accept_bytes) / (ms * 1e-3) / 1e9, 2),
            "config": {"workload": "stack_40l_131k", "layers": 40, "ring_layers": 30,
                       "paged_layers": 10, "q_len": 16, "n_q_heads": 16, "n_kv_heads": 4,
                       "head_dim": 128, "ring_size": 2048, "window": 512, "paged_ctx": 131072,
                       "chunk": 64, "vocab": 65536, "hip_graph": graph,
                       "kv_bytes_per_step": st.kv_bytes, "logit_bytes_per_step": st.accept_bytes},
            "roofline": {"bound": "hbm", "kernel": "chunk_attn_kernel (paged, split-K) at 131,072",
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "us_per_launch": round(k_ms * 1e3, 2),
                         "kernel_us": round(kern_mean, 2) if kern_mean else None,
                         "kernel_us_dist": dist(k_us) if k_us else None,
                         "frac_kernel": round(per_launch / (kern_mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                         if kern_mean else None,
                         "algorithmic_bytes_per_launch": per_launch,
                         "traffic": traffic_entry(per_launch)},
        })
        step_out = {l: (st.layers[l]["out"].cpu().numpy(), st.layers[l]["lse"].cpu().numpy())
                    for l in (0, 1, 2, 3)}
        step_out["accept"] = (int(st.acc_len.cpu()[0]), st.committed.cpu().numpy())
        if not args.no_graph:
            # the decode loop: one captured step (appends + attention + accept + advance, the
            # block position on the device) replayed as the context grows
            n_dec = args.warmup + args.steps + 1
            def decode_loop(step_fn):
                st.decode_setup(n_dec)
                gd = capture(step_fn, torch)         # the capture's warm-up run advances once
                for _ in range(args.warmup):
                    gd.replay()
                torch.cuda.synchronize()
                p_start = int(st.d_pos.cpu()[0])
                dec = per_call_ms(gd.replay, args.steps, torch)
                p_end = int(st.d_pos.cpu()[0])
                assert p_end - p_start == args.steps * st.adv and p_end <= st.pos_cap + st.adv
                dec_bytes = sum(st.decode_kv_bytes(p_start + i * st.adv)
                                for i in range(args.steps))
                dec_ms = sum(dec) / len(dec)
                del gd
                return {"ms_per_step": round(dec_ms, 4), "step_ms": dist(dec, 4),
                        "kv_gbps": round(dec_bytes / args.steps / (dec_ms * 1e-3) / 1e9, 1),
                        "positions": [p_start, p_end - st.adv], "advance_per_step": st.adv}
            two = decode_loop(st.decode_step)
            fused = decode_loop(st.decode_step_fused)
            log(f"decode step with appends {fused['ms_per_step']:.3f} ms "
                f"({two['ms_per_step']:.3f} ms with separate append launches)")
            res["step_with_appends"] = dict(fused, two_calls=two, note=(
                "one captured graph replayed as the decode loop: per layer the block's 16 K/V "
                "rows appended at the device-resident position inside the attention launch "
                "(two_calls: a separate append launch per layer), then the accept and the "
                "on-device advance by a + 1"))
        del st
        torch.cuda.empty_cache()

    if args.workload == "paged_256k" or not args.no_256k:
        log("building the 262,144-context layer")
        c, _ = synth.workload("paged_256k", keep_rows=False)
        t = lambda a: rk.tensor_from_numpy(a, "cuda")  # noqa: E731
        q, pt = t(c.q), t(c.page_table)
        # three copies of the pool in distinct memory, used in turn: each launch reads KV the
        # previous two did not touch, as consecutive layers of a model would (512 MiB per pool,
        # twice the last-level cache), so no launch is served from what the last one cached
        pools = [(t(c.k_pool), t(c.v_pool))]
        pools += [(pools[0][0].clone(), pools[0][1].clone()) for _ in range(2)]
        kv = c.kv_bytes
        del c
        out = torch.empty((16, 16, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((16, 16), dtype=torch.float32, device="cuda")
        splits = rk.verify_attn_paged_auto_splits(16, 4, 128, 16, 262144)
        po = torch.empty((4, splits, 64, 128), dtype=torch.float32, device="cuda")
        pl = torch.empty((4, splits, 64), dtype=torch.float32, device="cuda")
        ws = torch.empty(rk.lib().verify_attn_paged_workspace_bytes(
            ctypes.byref(AttnDims(16, 16, 4, 128, 0.0, 1)), 262144, 64, 0), dtype=torch.uint8,
            device="cuda")
        turn = [0]

        def next_pool():
            turn[0] += 1
            return pools[turn[0] % len(pools)]

        def fn():
            kp, vp = next_pool()
            rk.verify_attn_paged(q, kp, vp, pt, 262144, out=out, lse=lse, workspace=ws)

        def part():
            kp, vp = next_pool()
            rk.verify_attn_paged_partial(q, kp, vp, pt, 262144, splits, part_out=po, part_lse=pl)

        for _ in range(max(2, args.warmup)):
            fn()
        n = max(6, args.steps // 3 * 3)      # a multiple of the pool count
        # graph replay, as in the step: n layers per graph, HIP events around the replays
        us = graph_ms(fn, n, 3, torch) * 1e3
        us_split = graph_ms(part, n, 3, torch) * 1e3
        log(f"256K layer {us:.1f} us (split kernel {us_split:.1f} us)")
        res.update({"us_per_layer_256k": round(us, 2),
                    "kv_gbps_256k": round(kv / (us * 1e-6) / 1e9, 1),
                    "hbm_frac_256k": round(kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "split_kernel_us_256k": round(us_split, 2)})
        if args.workload == "paged_256k":
            res.update({"value": res["kv_gbps_256k"], "unit": "GB/s", "ms_per_step": round(us / 1e3, 5),
                        "config": {"workload": "paged_256k", "ctx": 262144, "q_len": 16,
                                   "n_q_heads": 16, "n_kv_heads": 4, "head_dim": 128,
                                   "chunk": 64, "splits": splits},
                        "roofline": {"bound": "hbm", "kernel": "chunk_attn_kernel (paged, split-K) at 262,144",
                                     "achieved": round(kv / (us_split * 1e-6) / 1e9, 1),
                                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                     "frac": round(kv / (us_split * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                                     "us_per_launch": round(us_split, 2),
                                     "algorithmic_bytes_per_launch": kv, "traffic": None}})
        del q, pt, pools
        torch.cuda.empty_cache()

    if not args.no_prefill:
        log("batched prefill blocks")
        res["prefill_gpu"] = prefill_timings(torch, rk, synth, max(3, args.steps // 4))

    if not args.no_paging:
        log("host paging")
        res["paging_gpu"] = paging_timings(torch, rk, max(5, args.steps // 2))

    if not args.no_configs:
        log("single-layer workloads, cold and warm")
        probe = ReadProbe(torch)
        res["configs_gpu"] = config_timings(torch, rk, synth, probe, N_SMALL, N_LARGE)
        res["read_bw_probe"] = read_bw_probe(torch, probe)
        if "us_per_layer_256k" in res:
            # The headline 256K figure: the layer's two kernels (split + merge), their own
            # durations summed per call, caches evicted before each call (median of 51 calls
            # over three pool copies).  Alongside: the cold graph figure (calls in a graph minus a
            # graph of the evicting reads: launch gaps included) and the back-to-back graph
            # figure (long series of this kernel reach the card's power limit).
            c256 = res["configs_gpu"]["paged_256k"]
            kv256 = 2 * 262144 * 4 * 128 * 2
            res["us_per_layer_256k_back_to_back"] = res["us_per_layer_256k"]
            res["us_per_layer_256k_graph_cold"] = c256["us_cold"]
            cold = c256["kernel_us_cold"]["median"] if "kernel_us_cold" in c256 else c256["us_cold"]
            res.update({"us_per_layer_256k": cold,
                        "us_per_layer_256k_dist": c256.get("kernel_us_cold"),
                        "kv_gbps_256k": round(kv256 / (cold * 1e-6) / 1e9, 1),
                        "hbm_frac_256k": round(kv256 / (cold * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                        "hbm_frac_256k_of_read_probe": round(
                            kv256 / (cold * 1e-6) / 1e9 / res["read_bw_probe"]["gbps"], 4)})
        if "roofline" in res:
            res["roofline"]["frac_of_read_probe"] = round(
                res["roofline"]["achieved"] / res["read_bw_probe"]["gbps"], 4)

    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline (oracle)")
        ref, res["cpu_baseline"] = cpu_baseline(synth, oracle)
        if args.workload == "stack_40l_131k":
            res["parity"] = step_parity(step_out, ref)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
