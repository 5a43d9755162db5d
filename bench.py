#!/usr/bin/env python3
"""Benchmark of small-q GQA decode attention on one MI355X.

One step is one call of the hot path (QK^T, masked softmax, PV, and the
split combine) over one batch of the workload: for the default pi0.5 action
step, 18 independent layer instances of n_head=8, n_tok=10, hd=256 and a KV
head of 1024 keys (968 valid) per call.

Inputs are resident in HBM before timing starts and cold in the caches: every
call reads a different copy of the batch from a rotating pool of at least
1 GiB, so neither the 4 MB per-XCD L2 nor the 256 MB MALL can serve it.  The
K timed calls are queued behind a bounded GPU sleep, so they run back to back
at device speed rather than at the host's launch rate; HIP events bracket the
timed region, and the library's event hook brackets each call's main kernel
on the stream it is launched on.  The reported call time comes from a region
of plain calls; the kernel durations from a second region of the same calls
with the event hook installed.

Prints ONE JSON line (rank 0, one GPU):
  value      = microseconds per call (lower is better)
  roofline   = algorithmic bytes of one call / average main-kernel duration,
               against the 8 TB/s HBM peak
  cpu_baseline = the fp64 oracle on the host cores, on the same inputs
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of peak) for small-q GQA decode attention"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_F16_MFMA_TFLOPS = 2500.0  # MI355X dense f16 matrix cores
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["gqa_decode_attention_fr_amd/csrc/fr_fused.hip",
                  "gqa_decode_attention_fr_amd/csrc/fr_device.h",
                  "gqa_decode_attention_fr_amd/csrc/fr_plan.hip",
                  "gqa_decode_attention_fr_amd/csrc/fr_decomposed.hip",
                  "gqa_decode_attention_fr_amd/csrc/fr_copy.hip",
                  "gqa_decode_attention_fr_amd/csrc/fr_qkv.hip"]


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks or empty lines: what the
    compiler sees (a comment edit leaves the kernels, and their counters, as
    they were)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines())
    return "\n".join(l for l in lines if l)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pi05_action_step_h8_hd256_t10_kv1024_x18",
                    help="workload name, or 'all' for one line per workload")
    ap.add_argument("--variant", choices=["auto", "fused", "decomposed"], default="auto")
    ap.add_argument("--round-f16", action="store_true", help="f32 Q rounded to f16 once")
    ap.add_argument("--pool-gib", type=float, default=1.0)
    ap.add_argument("--warm", action="store_true",
                    help="also time the same buffers every call (cache-resident, auxiliary)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-calls", action="store_true",
                    help="also time a batch as back-to-back single-instance calls (a second "
                         "grid of the same kernels, so kept out of default runs)")
    ap.add_argument("--cpu-repeats", type=int, default=3)
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the machine probes (launch floor, read rates, merge A/B)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run --steps plain 256 MiB device copies (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE to bytes)")
    return ap.parse_args(argv)


class Pool:
    """R copies of one batch at distinct HBM addresses (one slab per tensor)."""

    def __init__(self, torch, w, g, pool_bytes):
        n = w.n_inst
        per = (g["q"].nbytes + g["k"].nbytes + g["v"].nbytes + g["mask"].nbytes
               + n * w.M * w.hd * 4)
        self.R = max(2, int(math.ceil(pool_bytes / per)))
        dev = "cuda"

        def slab(a):
            t = torch.from_numpy(a.view(np.float16) if a.dtype == np.uint16 else a).to(dev)
            s = torch.empty((self.R,) + tuple(t.shape), dtype=t.dtype, device=dev)
            s.copy_(t.unsqueeze(0).expand_as(s))
            return s

        self.q, self.k, self.v, self.mask = (slab(g[x]) for x in ("q", "k", "v", "mask"))
        self.out = torch.zeros((self.R, n, w.n_tok, w.n_head, w.hd), dtype=torch.float32,
                               device=dev)
        self.bytes = per * self.R


def make_call(F, w, pool, flags):
    """One call over the whole batch: fr_decode_attn_ex, or fr_decode_attn_gqa
    for workloads with several KV heads."""
    fmt = F.FR_Q_F16 if w.q_dtype == "f16" else F.FR_Q_F32
    M = w.M
    lib = F.binding.load()
    kvh_stride = w.n_kv * w.hd
    qs, ks, ms, os_ = M * w.hd, w.n_kv_head * kvh_stride, w.n_tok * w.n_kv, M * w.hd
    ptrs = [(pool.q[r].data_ptr(), pool.k[r].data_ptr(), pool.v[r].data_ptr(),
             pool.mask[r].data_ptr(), pool.out[r].data_ptr()) for r in range(pool.R)]

    kv_len = None
    n_kv = w.n_kv
    if w.dynamic_len:   # valid keys as device counts, one per instance
        import torch
        kv_len = torch.full((w.n_inst,), w.n_valid, dtype=torch.int32, device="cuda")
    kv_len_ptr = None if kv_len is None else kv_len.data_ptr()

    def call(slot, stream):
        q, k, v, m, o = ptrs[slot]
        if w.mask_kind == "none":
            m = None
        if w.n_kv_head == 1 and kv_len is None:
            st = lib.fr_decode_attn_ex(q, fmt, k, v, m, o, w.n_inst, qs, ks, ms, os_, w.n_head,
                                       w.n_tok, n_kv, w.hd, w.scale, flags, None, 0, stream)
        else:
            st = lib.fr_decode_attn_gqa(q, fmt, k, v, m, kv_len_ptr, o, w.n_inst, qs, ks, ms, os_,
                                        w.n_head, w.n_kv_head, kvh_stride, w.n_tok, n_kv,
                                        w.hd, w.scale, flags, None, 0, stream)
        if st != 0:
            raise F.FrError(st, "decode attention call")

    call.keep = kv_len   # the device counts live as long as the call
    return call


def make_single_calls(F, w, pool, flags):
    """The same batch as n_inst back-to-back single-instance calls."""
    fmt = F.FR_Q_F16 if w.q_dtype == "f16" else F.FR_Q_F32
    M = w.M
    lib = F.binding.load()
    qe = 2 if w.q_dtype == "f16" else 4
    kvh_stride = w.n_kv * w.hd
    steps = (M * w.hd * qe, w.n_kv_head * kvh_stride * 2, w.n_kv_head * kvh_stride * 2,
             w.n_tok * w.n_kv * 2, M * w.hd * 4)
    ptrs = [(pool.q[r].data_ptr(), pool.k[r].data_ptr(), pool.v[r].data_ptr(),
             pool.mask[r].data_ptr(), pool.out[r].data_ptr()) for r in range(pool.R)]
    kv_len = None
    if w.dynamic_len:
        import torch
        kv_len = torch.full((1,), w.n_valid, dtype=torch.int32, device="cuda")
    kv_len_ptr = None if kv_len is None else kv_len.data_ptr()

    def call(slot, stream):
        base = ptrs[slot]
        for i in range(w.n_inst):
            q, k, v, m, o = (b + i * d for b, d in zip(base, steps))
            if w.mask_kind == "none":
                m = None
            st = lib.fr_decode_attn_gqa(q, fmt, k, v, m, kv_len_ptr, o, 1, 0, 0, 0, 0, w.n_head,
                                        w.n_kv_head, kvh_stride, w.n_tok, w.n_kv, w.hd,
                                        w.scale, flags, None, 0, stream)
            if st != 0:
                raise F.FrError(st, "fr_decode_attn_gqa")

    call.keep = kv_len
    return call


def sleep_cycles_for(torch, ms: float) -> int:
    """Calibrate torch.cuda._sleep (a bounded spin kernel) to about `ms`."""
    cycles = 1_000_000
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(cycles)
    e1.record()
    torch.cuda.synchronize()
    per_ms = cycles / max(e0.elapsed_time(e1), 1e-3)
    return int(per_ms * ms)


def timed_region(torch, F, call, R, steps, stream_handle, same_slot=False, hook=True):
    """K calls queued behind a GPU sleep, bracketed by two stream events.

    Returns (ms per call, list of main-kernel ms).  With `hook`, the library's
    profiling events ride on each split-kernel launch (hipExtLaunchKernel), so
    they read that kernel's own start/end timestamps on the stream it runs on.
    """
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if hook else []
    stops = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if hook else []
    for e in starts + stops:   # instantiate the underlying hipEvents
        e.record()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # host enqueue rate, to size the sleep that keeps the queue ahead of the GPU
    h0 = time.perf_counter()
    for i in range(min(steps, 20)):
        call(0 if same_slot else i % R, stream_handle)
    torch.cuda.synchronize()
    host_per_call = (time.perf_counter() - h0) / min(steps, 20)
    cycles = sleep_cycles_for(torch, max(20.0, 3.0 * host_per_call * 1e3 * steps))

    torch.cuda.synchronize()
    torch.cuda._sleep(cycles)
    t0.record()
    for i in range(steps):
        if hook:
            F.fr_decode_attn_profile_events(starts[i].cuda_event, stops[i].cuda_event)
        call(0 if same_slot else i % R, stream_handle)
    if hook:
        F.fr_decode_attn_profile_events(None, None)
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    kern = [a.elapsed_time(b) for a, b in zip(starts, stops)]
    return ms_total / steps, kern


def graph_region(torch, call, R, steps):
    """The same K calls captured once into a HIP graph (the way a serving loop
    replays a decode step) and replayed behind a GPU sleep; ms per call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            h = int(s.cuda_stream)
            for i in range(steps):
                call(i % R, h)
    torch.cuda.current_stream().wait_stream(s)
    graph.replay()                      # the first replay uploads the graph
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(sleep_cycles_for(torch, 20.0))
    t0.record()
    graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del graph
    return ms


def achievable_copy_gbps(torch, reps=20):
    """Read+write bytes per second of a plain 256 MiB device copy (larger than
    the MALL), the practical ceiling next to the 8 TB/s data-sheet peak."""
    n = 64 << 20
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    gbps = 2 * n * 4 * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del src, dst
    return gbps


def achievable_read_gbps(torch, reps=20):
    """Bytes per second of a plain streaming read: torch's row sums of 1 GiB of
    float32 (four times the MALL) as 8192 rows, which read every byte once and
    write 8192 floats.  (A sum to one scalar reaches only about two thirds of
    this rate; the row form is the fastest simple read torch offers here.)"""
    n = 256 << 20
    x = torch.ones(n, dtype=torch.float32, device="cuda").view(8192, -1)
    s = x.sum(1)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        s = x.sum(1)
    t1.record()
    torch.cuda.synchronize()
    gbps = n * 4 * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del x, s
    return gbps


def traffic_record(w_name: str, variant=None):
    """The committed rocprofv3 counter record of a workload, or None if missing,
    taken on different kernel sources or (for attention workloads) with another
    variant."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    rec = t.get("workloads", {}).get(w_name)
    if not rec or rec.get("variant") != variant:
        return None
    return rec


def traffic_for(w_name: str, variant=None):
    """HBM bytes per main-kernel launch from the committed counters (or None)."""
    rec = traffic_record(w_name, variant)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def call_traffic_for(w_name: str, variant=None):
    """HBM bytes per call: the main kernel's plus, where the call has one, the
    combine kernel's (or None)."""
    rec = traffic_record(w_name, variant)
    if rec is None or rec.get("hbm_bytes_per_launch") is None:
        return None
    comb = rec.get("combine_kernel")
    return rec["hbm_bytes_per_launch"] + (comb["hbm_bytes_per_launch"] if comb else 0)


def cpu_baseline(w, g, gpu_out, repeats):
    import oracle
    q_kind = oracle.Q_F16 if w.q_dtype == "f16" else oracle.Q_F32
    times, threads = [], 0
    out = None
    for _ in range(max(1, repeats)):
        t = time.perf_counter()
        res = []
        for i in range(w.n_inst):
            if w.mask_kind == "none":   # no mask; the valid keys only
                k, v = g["k"][i][..., :w.n_valid, :], g["v"][i][..., :w.n_valid, :]
                o, threads = oracle.decode_attn(g["q"][i], k, v, None, w.n_head, w.n_tok,
                                                w.n_valid, w.hd, w.scale, q_kind=q_kind,
                                                return_threads=True, n_kv_head=w.n_kv_head)
            else:
                o, threads = oracle.decode_attn(g["q"][i], g["k"][i], g["v"][i], g["mask"][i],
                                                w.n_head, w.n_tok, w.n_kv, w.hd, w.scale,
                                                q_kind=q_kind, return_threads=True,
                                                n_kv_head=w.n_kv_head)
            res.append(o)
        times.append(time.perf_counter() - t)
        out = np.stack(res)
    med = statistics.median(times)
    err = float(np.max(np.abs(out - gpu_out.astype(np.float64))))
    return {"value": round(med * 1e6, 1), "unit": "us/call", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the full {w.n_inst}-instance batch of the timed workload, "
                      f"median of {len(times)} fp64 runs",
            "max_abs_vs_gpu": err}


PROBE_LIB = os.path.join(ROOT, "gqa_decode_attention_fr_amd", "libfrprobe.so")


def machine_probes(torch):
    """Machine figures behind the design's limits, measured in this run with
    the committed probe kernels (libfrprobe.so, csrc/fr_probe.hip):

    - the launch floor: microseconds per launch of back-to-back empty kernels
      queued behind a GPU sleep, eager and replayed from a captured graph;
    - HBM read rates: one workgroup (one compute unit) streaming 1 MiB it has
      not touched before (caches scrubbed by a 512 MiB read elsewhere) with
      32 KiB or 128 KiB of loads in flight, and 256 workgroups streaming 1 MiB
      each (the whole chip); and the chip's rate for reads served by L2 (the
      workgroups of one XCD reading the same 512 KiB) against distinct data;
    - the LDS read rate of one workgroup with one or two waves per SIMD, for
      the 16-byte reads of K and the transposing reads of V;
    - merging key-split partials: 256 workgroups in groups of 2, 4 or 8, each
      reading 64 KiB and writing a 48 KiB partial; the merge as a second
      launch against one launch whose last-arriving workgroup merges its group
      (agent-scope acquire/release fences, or device-coherent sc1 accesses),
      one launch where the last publisher of each column slice merges that
      slice, and one launch with combine workgroups that wait for their group.
    """
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.frp_empty.argtypes = [i32, i32, vp]
    lib.frp_read.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.frp_merge.argtypes = [i32, vp, vp, vp, vp, i32, i32, vp]
    lib.frp_lds.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.frp_read_shared.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.frp_issue.argtypes = [i32, i32, i32, vp, vp, vp]
    for f in (lib.frp_empty, lib.frp_read, lib.frp_merge, lib.frp_lds, lib.frp_read_shared,
              lib.frp_issue):
        f.restype = i32
    grid, pf, wb = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib.frp_merge_sizes(ctypes.byref(grid), ctypes.byref(pf), ctypes.byref(wb))
    grid, pf, wb = grid.value, pf.value, wb.value

    def ok(st, what):
        if st != 0:
            raise RuntimeError(f"probe {what} failed ({st})")

    stream = int(torch.cuda.current_stream().cuda_stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    # launch floor
    K = 200
    ok(lib.frp_empty(1, 20, stream), "empty")
    torch.cuda._sleep(sleep_cycles_for(torch, 5.0))
    ev0.record()
    ok(lib.frp_empty(1, K, stream), "empty")
    ev1.record()
    torch.cuda.synchronize()
    res["empty_kernel_us_per_launch_eager"] = round(ev0.elapsed_time(ev1) * 1e3 / K, 3)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            ok(lib.frp_empty(1, K, int(s.cuda_stream)), "empty")
    torch.cuda.current_stream().wait_stream(s)
    graph.replay()
    torch.cuda.synchronize()
    torch.cuda._sleep(sleep_cycles_for(torch, 5.0))
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    res["empty_kernel_us_per_launch_graph"] = round(ev0.elapsed_time(ev1) * 1e3 / K, 3)
    del graph

    # HBM read rates: [0, 512 MiB) is the scrub area, reads come from above it
    mib = 1 << 20
    buf = torch.zeros(1024 * mib // 4, dtype=torch.float32, device="cuda")
    times = torch.zeros(2 * 256, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1024, dtype=torch.float32, device="cuda")
    base = buf.data_ptr()

    def scrub():
        ok(lib.frp_read(base, 2 * mib, 256, 8, times.data_ptr(), sink.data_ptr(), stream), "read")

    def read(off, per_wg, n_wg, unroll):
        scrub()
        ok(lib.frp_read(base + off, per_wg, n_wg, unroll, times.data_ptr(), sink.data_ptr(),
                        stream), "read")
        torch.cuda.synchronize()
        t = times[: 2 * n_wg].cpu().numpy().reshape(n_wg, 2)
        return per_wg, t   # ticks of 10 ns

    off = 512 * mib
    for unroll, kib in ((8, 32), (32, 128)):
        per, t = read(off, mib, 1, unroll)
        off += mib
        res[f"read_one_cu_GBps_{kib}KiB_in_flight"] = round(per / ((t[0, 1] - t[0, 0]) * 10.0), 1)
    per, t = read(off, mib, 256, 8)
    res["read_chip_256_workgroups_GBps"] = round(256 * per / ((t[:, 1].max() - t[:, 0].min())
                                                              * 10.0), 1)
    res["read_chip_per_workgroup_GBps"] = round(float(np.median(per / ((t[:, 1] - t[:, 0])
                                                                       * 10.0))), 1)
    # the same reads served by L2: 256 workgroups of 512 lanes reading 512 KiB twice,
    # either 8 regions (each shared by the 32 workgroups of one XCD) or all distinct
    t3 = torch.zeros(3 * 256, dtype=torch.int64, device="cuda")
    for n_region, label in ((8, "shared_by_xcd"), (256, "distinct")):
        scrub()
        ok(lib.frp_read_shared(base + 512 * mib, 512 << 10, 256, n_region, t3.data_ptr(),
                               sink.data_ptr(), stream), "read_shared")
        torch.cuda.synchronize()
        t = t3.cpu().numpy().reshape(256, 3)
        res[f"read_chip_second_pass_{label}_GBps"] = round(
            256 * (512 << 10) / ((t[:, 2].max() - t[:, 1].min()) * 10.0), 1)
    del times, sink, t3

    # LDS read rate of one workgroup (bytes per ns; at 2.4 GHz, / 2.4 = bytes per clock)
    t2 = torch.zeros(2, dtype=torch.int64, device="cuda")
    s2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    for kind, kname, per_lane in ((0, "b128", 16), (1, "tr_b16_b64", 8)):
        for lanes in (256, 512):
            iters = 2000
            ok(lib.frp_lds(kind, lanes, iters, t2.data_ptr(), s2.data_ptr(), stream), "lds")
            torch.cuda.synchronize()
            tt = t2.cpu().numpy()
            res[f"lds_{kname}_bytes_per_ns_{lanes // 256}_waves_per_simd"] = round(
                iters * 16 * per_lane * lanes / ((tt[1] - tt[0]) * 10.0), 1)
    # how matrix-core and vector-ALU work share a SIMD: ns per trip of 8 MFMAs
    # (16x16x32 f16) and/or 32 fp32 fma, alone, interleaved in one wave, or in
    # two waves of one SIMD (one MFMA wave, one VALU wave)
    sf = torch.zeros(1, dtype=torch.float32, device="cuda")
    for mode, lanes, label in ((0, 256, "mfma8_1_wave_per_simd"), (1, 256, "fma32_1_wave_per_simd"),
                               (2, 256, "mfma8_and_fma32_same_wave"),
                               (0, 512, "mfma8_2_waves_per_simd"), (1, 512, "fma32_2_waves_per_simd"),
                               (3, 512, "mfma8_wave_and_fma32_wave_per_simd")):
        iters = 20000
        ok(lib.frp_issue(mode, lanes, iters, t2.data_ptr(), sf.data_ptr(), stream), "issue")
        torch.cuda.synchronize()
        tt = t2.cpu().numpy()
        res[f"issue_ns_per_trip_{label}"] = round(float(tt[1] - tt[0]) * 10.0 / iters, 2)
    del t2, s2, sf

    # merging key-split partials: two launches against one
    part = torch.zeros(grid * pf, dtype=torch.float32, device="cuda")
    out = torch.zeros(grid * pf, dtype=torch.float32, device="cuda")
    cnt = torch.zeros(2 * grid, dtype=torch.int32, device="cuda")
    slot = grid * wb                       # 16 MiB of cold work input per call
    n_slots = (512 * mib) // slot
    merge = {}
    names = {0: "two_launches", 1: "one_launch_fenced", 2: "one_launch_sc1",
             3: "one_launch_sliced", 4: "one_launch_waiting_combine"}
    for n_split in (2, 4, 8):
        for mode in (0, 1, 2, 3, 4):
            calls = 40
            for it in range(4):            # warm-up
                ok(lib.frp_merge(mode, base + 512 * mib + (it % n_slots) * slot, part.data_ptr(),
                                 cnt.data_ptr(), out.data_ptr(), n_split, it, stream), "merge")
            torch.cuda.synchronize()
            torch.cuda._sleep(sleep_cycles_for(torch, 5.0))
            ev0.record()
            for it in range(calls):
                ok(lib.frp_merge(mode, base + 512 * mib + (it % n_slots) * slot, part.data_ptr(),
                                 cnt.data_ptr(), out.data_ptr(), n_split, it, stream), "merge")
            ev1.record()
            torch.cuda.synchronize()
            got = out[: (grid // n_split) * pf].cpu().numpy().reshape(grid // n_split, pf)
            it = calls - 1
            c = np.arange(pf)
            want = sum(((it * 131 + s_ * 7 + c) % 1021).astype(np.float64) for s_ in range(n_split))
            correct = bool(np.array_equal(got, np.broadcast_to(want, got.shape)))
            merge[f"{names[mode]}_groups_of_{n_split}_us"] = round(ev0.elapsed_time(ev1) * 1e3
                                                                  / calls, 3)
            if not correct:
                merge[f"{names[mode]}_groups_of_{n_split}_wrong"] = True
    res["merge_partials"] = merge
    del buf, part, out, cnt
    torch.cuda.empty_cache()
    return res


RIDGE_FLOP_PER_BYTE = PEAK_F16_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # ~312


def roofline(w, kern_ms, achieved_gbs, traffic, ms_call=None, call_traffic=None):
    """The bound of the split kernel (the dominant kernel) from the workload's
    algorithmic intensity: below the ridge it is HBM bytes per second against
    8 TB/s; above it (long context, prefill) the two contractions' flops against
    the dense f16 matrix-core peak.  (An f32 query runs its score contraction
    twice, hi and lo; those extra flops are not counted: the figure is
    algorithmic.)  Beside it, the same figure for the whole call (every launch
    of it, from the plain-call rate) and the call's counter traffic (split plus
    combine kernel)."""
    hbm = w.flops() / w.algorithmic_bytes() <= RIDGE_FLOP_PER_BYTE
    if hbm:
        rec = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS,
               "unit": "GB/s", "frac": round(achieved_gbs / PEAK_HBM_GBS, 4),
               "traffic": traffic}
    else:
        tflops = w.flops() / (kern_ms * 1e-3) / 1e12
        rec = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_MFMA_TFLOPS,
               "unit": "TFLOP/s", "frac": round(tflops / PEAK_F16_MFMA_TFLOPS, 4),
               "traffic": traffic}
    if ms_call is not None:
        if hbm:
            call = w.algorithmic_bytes() / (ms_call * 1e-3) / 1e9
            rec["call_achieved"] = round(call, 1)
            rec["call_frac"] = round(call / PEAK_HBM_GBS, 4)
        else:
            call = w.flops() / (ms_call * 1e-3) / 1e12
            rec["call_achieved"] = round(call, 2)
            rec["call_frac"] = round(call / PEAK_F16_MFMA_TFLOPS, 4)
        rec["call_traffic"] = call_traffic
    return rec


def run_workload(args, torch, F, W, w, probes=None):
    flags = {"auto": 0, "fused": F.FR_VARIANT_FUSED,
             "decomposed": F.FR_VARIANT_DECOMPOSED}[args.variant]
    if args.round_f16:
        flags |= F.FR_Q_ROUND_F16
    # several KV heads run as n_inst*n_kv_head units of n_head/n_kv_head heads
    units, grp = w.n_inst * w.n_kv_head, w.n_head // w.n_kv_head
    plan_flags = flags | (F.FR_PLAN_UNMASKED if w.mask_kind == "none" else 0)
    plan = F.fr_decode_attn_plan(units, grp, w.n_tok, w.n_kv, w.hd, plan_flags)
    g = W.generate(w)
    pool = Pool(torch, w, g, args.pool_gib * (1 << 30))
    F.fr_decode_attn_reserve(units, grp, w.n_tok, w.n_kv, w.hd, flags)
    call = make_call(F, w, pool, flags)
    stream = int(torch.cuda.current_stream().cuda_stream)

    for i in range(args.warmup):
        call(i % pool.R, stream)
    torch.cuda.synchronize()
    # every slot holds the same inputs, so every slot's output must be identical
    outs = pool.out[: min(pool.R, max(args.warmup, 1))]
    if not bool(torch.isfinite(outs).all()) or not bool((outs == outs[0]).all()):
        raise RuntimeError("warm-up outputs differ across pool slots or are not finite")
    gpu_out = pool.out[0].cpu().numpy()

    # the reported time: K plain calls; then the same K calls again with the
    # library's profiling events riding on each split-kernel launch, for the
    # kernel's own duration (those events add time between calls, so that
    # region's call rate is not reported)
    ms_call, _ = timed_region(torch, F, call, pool.R, args.steps, stream, hook=False)
    ms_hooked, kern = timed_region(torch, F, call, pool.R, args.steps, stream, hook=True)
    kern_ms = statistics.mean(kern)
    alg = w.algorithmic_bytes()
    achieved = alg / (kern_ms * 1e-3) / 1e9
    call_gbs = alg / (ms_call * 1e-3) / 1e9
    aux = {
        "us_per_instance": round(ms_call * 1e3 / w.n_inst, 3),
        "call_GBps": round(call_gbs, 1),
        "call_frac_of_hbm_peak": round(call_gbs / PEAK_HBM_GBS, 4),
        "main_kernel_us_mean": round(kern_ms * 1e3, 3),
        "main_kernel_us_median": round(statistics.median(kern) * 1e3, 3),
        "us_per_call_with_event_hook": round(ms_hooked * 1e3, 3),
        "mfma_frac_of_f16_peak": round(w.flops() / (kern_ms * 1e-3) / 1e12 / PEAK_F16_MFMA_TFLOPS,
                                       4),
        "plan": plan,
        "pool_copies": pool.R,
        "pool_GiB": round(pool.bytes / (1 << 30), 3),
        "algorithmic_bytes": alg,
        "flops": w.flops(),
    }
    ms_graph = graph_region(torch, call, pool.R, args.steps)
    aux["graph_replayed_us_per_call"] = round(ms_graph * 1e3, 3)
    if w.n_inst > 1 and args.single_calls:
        singles = make_single_calls(F, w, pool, flags)
        n_b = max(1, args.steps // 10)
        ms_single, _ = timed_region(torch, F, singles, pool.R, n_b, stream, hook=False)
        aux["single_instance_calls_us_per_batch"] = round(ms_single * 1e3, 3)
    copy_gbps = achievable_copy_gbps(torch)
    aux["achievable_copy_GBps"] = round(copy_gbps, 1)
    aux["kernel_frac_of_achievable_copy"] = round(achieved / copy_gbps, 4)
    read_gbps = achievable_read_gbps(torch)
    aux["achievable_read_GBps"] = round(read_gbps, 1)
    aux["kernel_frac_of_achievable_read"] = round(achieved / read_gbps, 4)
    if args.warm:
        # as for the cold figures: the call rate from plain calls, the kernel's
        # duration from a second region with the profiling events
        ms_warm, _ = timed_region(torch, F, call, pool.R, args.steps, stream, same_slot=True,
                                  hook=False)
        _, kern_warm = timed_region(torch, F, call, pool.R, args.steps, stream,
                                    same_slot=True)
        aux["warm_cache_resident_us_per_call"] = round(ms_warm * 1e3, 3)
        aux["warm_cache_resident_kernel_us"] = round(statistics.mean(kern_warm) * 1e3, 3)

    if probes:
        aux["machine"] = probes
    traffic = traffic_for(w.name, plan["variant"])
    rec = {
        "metric": METRIC,
        "value": round(ms_call * 1e3, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_call, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 mfma, fp32 accumulate/softmax" + (
            " (f32 Q as hi+lo f16)" if w.q_dtype == "f32" and not args.round_f16 else ""),
        "data": "synthetic (seeded normal Q/K/V, f16 0/-inf masks; no checkpoint)",
        "config": {"workload": w.name, "n_inst": w.n_inst, "n_head": w.n_head,
                   "n_kv_head": w.n_kv_head, "n_tok": w.n_tok, "n_kv": w.n_kv, "n_valid": w.n_valid, "hd": w.hd,
                   "q_dtype": w.q_dtype, "variant": args.variant,
                   "round_f16": bool(args.round_f16)},
        "roofline": roofline(w, kern_ms, achieved, traffic, ms_call,
                             call_traffic_for(w.name, plan["variant"])),
        "aux": aux,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, g, gpu_out, args.cpu_repeats)
    del pool
    torch.cuda.empty_cache()
    return rec


def calibrate_copy(torch, steps):
    """A plain device-to-device copy of known size, for counter calibration."""
    n = 64 << 20                      # 64 Mi float32 = 256 MiB each way
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(max(1, steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n * 4,
                      "bytes_written_per_copy": n * 4, "copies": max(1, steps)}), flush=True)


COPY_WORKLOAD = "kv_tail_copy_pi05_l18_rows968_hd256"


def run_copy_workload(args, torch, F):
    """The batched persistent-KV tail copies after a pi0.5 prefill: per layer
    (18) and KV tensor (K, V), the 968 prefix rows of 256 f32 -> f16, as one
    call.  Cold inputs from a >= 1 GiB rotating pool, K plain calls behind a
    GPU sleep; bytes = 4 read + 2 written per element."""
    n_copy, rows, hd = 36, 968, 256
    n = rows * hd
    per = n_copy * n * 6
    R = max(2, int(math.ceil(args.pool_gib * (1 << 30) / per)))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    src = torch.randn((R, n_copy, n), dtype=torch.float32, device="cuda", generator=gen) * 0.5
    dst = torch.empty((R, n_copy, n), dtype=torch.float16, device="cuda")
    lib = F.binding.load()
    arrs = []
    for r in range(R):
        arr = (F.binding.F16Copy * n_copy)()
        for c in range(n_copy):
            arr[c] = F.binding.F16Copy(src[r, c].data_ptr(), dst[r, c].data_ptr(), n)
        arrs.append(arr)

    def call(slot, stream):
        st = lib.fr_f16_copy_batch(arrs[slot], n_copy, stream)
        if st != 0:
            raise F.FrError(st, "fr_f16_copy_batch")

    stream = int(torch.cuda.current_stream().cuda_stream)
    for i in range(args.warmup):
        call(i % R, stream)
    torch.cuda.synchronize()
    ms_call, _ = timed_region(torch, F, call, R, args.steps, stream, hook=False)
    ms_graph = graph_region(torch, call, R, args.steps)
    gbs = per / (ms_call * 1e-3) / 1e9
    rec = {
        "metric": "µs/call and achieved HBM GB/s for the batched f32->f16 KV tail copies",
        "value": round(ms_call * 1e3, 3), "unit": "us/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_call, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32->f16",
        "data": "synthetic (normal f32 rows)",
        "config": {"workload": COPY_WORKLOAD, "copies": n_copy, "rows": rows, "hd": hd},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(COPY_WORKLOAD)},
        "aux": {"bytes_per_call": per, "graph_replayed_us_per_call": round(ms_graph * 1e3, 3),
                "pool_copies": R,
                "note": "achieved is per whole call (one launch), launch gap included"},
    }
    del src, dst
    torch.cuda.empty_cache()
    return rec


QKV_WORKLOAD = "qkv_post_pi05_l18_h8_hd256_t10"


def run_qkv_workload(args, torch, F):
    """The producer ahead of the window for one pi0.5 action step: 18 layers
    (instances) of 10 tokens, 8 query heads and 1 KV head of 256, RoPE base
    10000, K/V rows stored into 1024-row caches.  Cold inputs from a rotating
    pool; bytes = qkv read + positions + f16 query, key and value rows."""
    n_inst, n_tok, n_head, n_kvh, hd, cap = 18, 10, 8, 1, 256, 1024
    width = (n_head + 2 * n_kvh) * hd
    per_in = n_inst * n_tok * (width * 4 + 4)
    per_out = n_inst * n_tok * (n_head + 2 * n_kvh) * hd * 2
    per = per_in + per_out
    R = max(2, int(math.ceil(args.pool_gib * (1 << 30) / (per_in + n_inst * 2 * cap * hd * 2))))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    qkv = torch.randn((R, n_inst, n_tok, width), dtype=torch.float32, device="cuda",
                      generator=gen)
    pos = (torch.arange(n_tok, dtype=torch.int32, device="cuda") + 958).repeat(R, n_inst, 1)
    q16 = torch.empty((R, n_inst, n_tok, n_head, hd), dtype=torch.float16, device="cuda")
    kc = torch.zeros((R, n_inst, n_kvh, cap, hd), dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    lib = F.binding.load()

    def call(slot, stream):
        st = lib.fr_qkv_post(qkv[slot].data_ptr(), pos[slot].data_ptr(), q16[slot].data_ptr(),
                             kc[slot].data_ptr(), vc[slot].data_ptr(), n_inst, n_tok * width,
                             n_tok, n_tok * n_head * hd, n_kvh * cap * hd, cap * hd, n_head,
                             n_kvh, n_tok, hd, cap, 10000.0, 1.0, stream)
        if st != 0:
            raise F.FrError(st, "fr_qkv_post")

    stream = int(torch.cuda.current_stream().cuda_stream)
    for i in range(args.warmup):
        call(i % R, stream)
    torch.cuda.synchronize()
    ms_call, _ = timed_region(torch, F, call, R, args.steps, stream, hook=False)
    ms_graph = graph_region(torch, call, R, args.steps)
    gbs = per / (ms_call * 1e-3) / 1e9
    rec = {
        "metric": "µs/call and achieved HBM GB/s for the query/KV producer (RoPE, f16 rows)",
        "value": round(ms_call * 1e3, 3), "unit": "us/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_call, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 -> f16 (angles f64)", "data": "synthetic (normal f32 projections)",
        "config": {"workload": QKV_WORKLOAD, "n_inst": n_inst, "n_tok": n_tok,
                   "n_head": n_head, "n_kv_head": n_kvh, "hd": hd},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for(QKV_WORKLOAD)},
        "aux": {"bytes_per_call": per, "graph_replayed_us_per_call": round(ms_graph * 1e3, 3),
                "pool_copies": R,
                "note": "one launch of 180 workgroups; the call is launch-latency bound"},
    }
    del qkv, pos, q16, kc, vc
    torch.cuda.empty_cache()
    return rec


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: the library and this benchmark run on one GPU; --gpus {args.gpus} "
              "is not supported (independent instances or KV shards would each run this "
              "kernel on their own GPU).", file=sys.stderr)
        return 2
    import torch

    import gqa_decode_attention_fr_amd as F
    from gqa_decode_attention_fr_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy(torch, args.steps)
        return 0
    F.binding.load()
    names = ([w.name for w in W.WORKLOADS + W.EXTRA_WORKLOADS] + [COPY_WORKLOAD, QKV_WORKLOAD]
             if args.workload == "all" else [args.workload])
    probes = None if args.no_probes else machine_probes(torch)
    for name in names:
        if name == COPY_WORKLOAD:
            print(json.dumps(run_copy_workload(args, torch, F)), flush=True)
            continue
        if name == QKV_WORKLOAD:
            print(json.dumps(run_qkv_workload(args, torch, F)), flush=True)
            continue
        if name not in W.BY_NAME:
            print(f"unknown workload {name}; choose from {list(W.BY_NAME)}", file=sys.stderr)
            return 1
        rec = run_workload(args, torch, F, W, W.BY_NAME[name], probes)
        print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
