#!/usr/bin/env python3
"""Benchmark of the MoE dispatch / combine hot path on one MI355X.

One step = one pass of the whole path over one batch: ep_layout_dispatch
(routing layout and scatter in one call) and ep_combine (gather-reduce) --
or, with --path separate, ep_layout, ep_dispatch and ep_combine -- by
default on the 4096-token prefill workload: T=4096, H=7168, E=256 experts, top-8
group-limited routing (8 groups of 32, top-4 groups), bf16 payload,
contiguous layout, seed 0.  Inputs are synthetic, seeded, and already
resident in HBM when the timed region starts.

Prints one JSON line.  `value` is effective GB/s of the whole step:
algorithmic bytes of dispatch (layout included) plus combine, divided by the
mean step time over K steps, each run after a cache flush (a 512 MiB fill
and a 1 GiB read, outside the timing) and timed by one HIP event pair on the
kernels' stream.  Beside it in `detail`:
  sustained_cold      K steps back to back over rotating copies of the
                      inputs and outputs (no step finds its inputs in a
                      cache), one event pair around all K -- no flush or
                      per-step marker inside the timed region;
  event_pair_overhead_us  an empty event pair after a flush: what the two
                      markers add to each flushed single step;
  warm_back_to_back   K steps back to back on one set of buffers;
  graph_back_to_back  20 steps captured in a HIP graph, replayed back to
                      back (what a serving loop that cannot afford the
                      host's per-call launch work sees).
`roofline` reports the dominant call against the 8 TB/s HBM peak, its
duration measured by HIP events around each call over K more flushed
steps (a call of ep_layout_dispatch is one to three kernels: it is reported
as a unit).  detail.configs times workloads 1-5 the same way,
each in a child process of its own (see config_table).
`cpu_baseline` times the CPU oracle on the same inputs on 1 and on N host
threads.  --sweep skew instead prints one line per routing-skew variant.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config 3]
                  [--path separate|fused] [--scales fp32|ue8m0] [--sweep skew]
                  [--flush both|write|read|none] [--no-config-table]
                  [--config-steps 20] [--no-cpu-baseline] [--cpu-seconds 12]
                  [--copy-calibration]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "dispatch+combine effective GB/s and µs/call, % of HBM peak, 1×MI355X"


def algorithmic_bytes(wl, count=None, scale_bytes=4):
    """Bytes the method must move (each input read once, each output written
    once), per call.  V = routing entries that get a receive row; scale_bytes
    = 4 for fp32 block scales, 1 for UE8M0."""
    T, H, k, E = wl.T, wl.H, wl.k, wl.E
    V = T * k if count is None else int(sum(min(c, wl.cap) if wl.cap else c for c in count))
    p = 1 if wl.fp8 else 2
    scales = scale_bytes * V * (H // 128) if wl.fp8 else 0
    R = T * k if wl.cap == 0 else E * wl.cap
    layout_k = 4 * T * k + 4 * T * k + 4 * R + 4 * (2 * E + 1) + 8
    dispatch_k = 2 * T * H + 4 * T * k + V * H * p + scales
    combine_k = 2 * V * H + 4 * T * k + 4 * T * k + 2 * T * H
    # whole-path totals: intermediate re-reads of slot_of are not counted
    b_disp = 2 * T * H + 4 * T * k + V * H * p + scales + 4 * T * k + 4 * V + 4 * (2 * E + 1)
    b_comb = 2 * V * H + 4 * T * k + 4 * T * k + 2 * T * H
    return dict(V=V, layout_kernels=layout_k, dispatch_kernel=dispatch_k,
                combine_kernel=combine_k, dispatch_total=b_disp, combine_total=b_comb)


def _code_only(text):
    """Source text without comments and with whitespace runs collapsed: what
    the compiler sees (no string literal in these sources holds a comment
    marker)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(*names):
    """Digest of the code (comments and layout aside) of kernel source files
    and of every csrc header they include, directly or not (quoted
    includes)."""
    csrc = os.path.join(ROOT, "combine_ep_layout_09_amd", "csrc")
    seen, todo = [], list(names)
    while todo:
        f = todo.pop(0)
        if f in seen or not os.path.exists(os.path.join(csrc, f)):
            continue
        seen.append(f)
        for line in open(os.path.join(csrc, f)):
            if line.startswith('#include "'):
                todo.append(line.split('"')[1])
    h = hashlib.sha256()
    for f in sorted(seen):
        with open(os.path.join(csrc, f)) as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode() + b"\0")
    return h.hexdigest()[:16]


def read_traffic(kernel, sources, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    # several kernels of one ep_layout_dispatch call: one summary for the call
    key = "ep_layout_dispatch" if "+" in kernel else kernel
    path = os.path.join(ROOT, "profiles", f"pmc_{key}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            key, _, v = line.partition(":")
            vals[key.strip()] = v.strip()
    if vals.get("source_digest") != kernel_source_digest(*sources):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HipEvents:
    """Timing events recorded on the stream the kernels run on, created with
    hipEventDisableSystemFence: recording one does not write back and
    invalidate the caches, so the kernels between two events run as they
    would without the events."""

    _FLAGS = 0x20000000  # hipEventDisableSystemFence (timing stays enabled)

    def __init__(self, n):
        import ctypes
        self._ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self._FLAGS)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(h)

    def record(self, i, stream_handle):
        if self.lib.hipEventRecord(self.ev[i], self._ct.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self._ct.c_float()
        if self.lib.hipEventElapsedTime(self._ct.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.ev:
            self.lib.hipEventDestroy(h)
        self.ev = []


def measure_copy_gbps(torch, nbytes=1 << 30, reps=10):
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
        b.copy_(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3 / reps
    del a, b
    return 2 * nbytes / t / 1e9


def host_cores():
    """Host threads for the oracle: the cores this process may run on, at
    most 16 (one GPU's share of a GPU host's CPUs)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, eo_host, bytes_total, target_s, fp8_mode):
    """The CPU oracle as it stands on the same host arrays: one full pass =
    layout (serial) + dispatch + combine, with dispatch and combine run on
    1 thread and on N threads (N = host_cores(); token ranges, same
    results), each repeated until about target_s / 2 seconds."""
    import oracle
    n = host_cores()

    def timed(threads):
        reps, elapsed = 0, 0.0
        while reps < 1 or (elapsed < target_s / 2 and reps < 50):
            t0 = time.perf_counter()
            lay = oracle.layout(wl.topk_idx, wl.E, wl.cap)
            oracle.dispatch(wl.x, lay["slot_of"], wl.R, fp8_mode, threads=threads)
            oracle.combine(eo_host, lay["slot_of"], wl.topk_weights, want_acc=False,
                           threads=threads)
            elapsed += time.perf_counter() - t0
            reps += 1
        return elapsed / reps, reps

    per1, reps1 = timed(1)
    perN, repsN = timed(n)
    return {"value": round(bytes_total / perN / 1e9, 3), "unit": "GB/s", "cores": n,
            "kind": "oracle",
            "sample": f"full passes (layout + dispatch + combine) of the benchmarked workload "
                      f"on the same host arrays: {repsN} passes on {n} threads at "
                      f"{perN * 1e3:.1f} ms each (layout serial, dispatch and combine split by "
                      f"token range), {reps1} serial passes at {per1 * 1e3:.1f} ms each",
            "value_1_thread": round(bytes_total / per1 / 1e9, 3),
            "ms_per_pass": {"1_thread": round(per1 * 1e3, 2), f"{n}_threads": round(perN * 1e3, 2)},
            "cpu_model": cpu_model()}


def one_launch(wl):
    """Whether ep_layout_dispatch takes this problem in its one-kernel form
    (the library's own rule: at most 8192 routing entries and 2^23 id visits
    over all workgroups)."""
    n = wl.T * wl.k
    nvec = wl.H // 8
    vpl = 1 if wl.T < 1024 else (8 if nvec >= 1024 else (nvec + 127) // 128)
    tiles = (nvec + 128 * vpl - 1) // (128 * vpl)
    nwg = max(1, (wl.T * tiles + 1) // 2)
    return n <= 8192 and n * nwg <= (1 << 23)


def persistent_launch(wl, ncu):
    """Whether ep_layout_dispatch takes its one-launch form of one 1024-lane
    workgroup per CU (the library's rule: 8192 < T*k <= 32768, T*k a
    multiple of 4, between 1 and 14 (bf16) or 16 (FP8) chunks of 64 pieces
    per wave, the workgroup's own entries within 1024 and its LDS within
    64 KiB)."""
    n = wl.T * wl.k
    if n <= 8192 or n > 32768 or n % 4 or (wl.fp8 and wl.H % 128):
        return False
    C = -(-(wl.H // 8) // 64)
    nw = ncu * 16
    chunks = wl.T * C
    if chunks < nw or chunks > nw * (16 if wl.fp8 else 14):
        return False
    Q = -(-chunks // nw)
    maxtok = (16 * Q - 1) // C + 2
    own = maxtok * wl.k
    if own > 1024:
        return False
    rw = -(-own // 64)
    copies = 8 if wl.E < 128 else 1  # histogram copies below 128 experts
    head = ((2 * copies + 1 + rw) * (wl.E + 1) + 3) & ~3
    return (head + maxtok * ((wl.k + 3) & ~3)) * 4 <= 65536


# sources of the kernels each form of an ep_layout_dispatch call launches (a
# counter summary's digest covers these and the headers they include)
FUSED_SOURCES = {
    "layout_dispatch_small_kernel": ("ep_fused.hip",),
    "layout_dispatch_persistent_kernel": ("ep_fused_persist.hip",),
    "layout_dispatch_persistent_fp8_kernel": ("ep_fused_persist.hip",),
    "layout_hist_kernel+layout_dispatch_ranked_kernel": ("ep_fused.hip", "ep_layout.hip"),
    "layout_hist_kernel+layout_rank_kernel+dispatch_fp8_kernel": ("ep_layout.hip", "ep_dispatch.hip"),
    "layout_whole_kernel+dispatch_fp8_kernel": ("ep_layout.hip", "ep_dispatch.hip"),
    "layout_small_kernel+dispatch_fp8_kernel": ("ep_layout.hip", "ep_dispatch.hip"),
}


def fused_call_name(wl, ncu):
    """The kernels of one ep_layout_dispatch call on this workload (the
    library's rule: one kernel for small tables; one persistent kernel for
    prefill-sized tables that fit it; the histogram kernel and the
    ranking dispatch kernel for other bf16 rows or k >= 8; otherwise the
    layout kernel(s) and the dispatch kernel)."""
    if one_launch(wl):
        return "layout_dispatch_small_kernel"
    if persistent_launch(wl, ncu):
        return "layout_dispatch_persistent_fp8_kernel" if wl.fp8 else "layout_dispatch_persistent_kernel"
    if not wl.fp8 or wl.k >= 8:
        return "layout_hist_kernel+layout_dispatch_ranked_kernel"
    if wl.T * wl.k <= 8192:  # a small table over too many workgroups for one kernel
        return "layout_small_kernel+dispatch_fp8_kernel"
    if whole_table_layout(wl):
        return "layout_whole_kernel+dispatch_fp8_kernel"
    return "layout_hist_kernel+layout_rank_kernel+dispatch_fp8_kernel"


def whole_table_layout(wl):
    """Whether ep_layout takes its one-kernel form for mid-size tables (the
    library's rule: 8192 < T*k <= 65536, at least 32 experts, and its LDS --
    (2 c + 17) (E + 1) int32 with c = 8 histogram copies below 128 experts,
    else 1 -- within 64 KiB)."""
    n = wl.T * wl.k
    c = 8 if wl.E < 128 else 1
    return 8192 < n <= 65536 and wl.E >= 32 and (2 * c + 17) * (wl.E + 1) * 4 <= 65536


def combine_kernel_name(wl, ncu):
    """The kernel ep_combine runs on this workload (the library's rule: the
    persistent form when every wave of one 1024-lane workgroup per CU gets at
    least one 64-piece chunk and at most 16 launches of at most 16 chunks per
    wave cover the batch)."""
    nvec = wl.H // 8
    C = -(-nvec // 64)
    nw = ncu * 16
    chunks = wl.T * C
    launches = max(1, -(-chunks // (nw * 16)))
    while -(-(-(-wl.T // launches) * C) // nw) > 16:
        launches += 1
    if chunks >= nw and launches <= 16:
        return "combine_persistent_kernel"
    return "combine_kernel"


class Flush:
    """Evicts the caches between timed steps, outside the events: a fill of a
    512 MiB scratch buffer (2x the 256 MB MALL), then a read of a second
    1 GiB buffer.  The read leaves L2 and MALL holding clean lines of data no
    step touches, so a timed step finds neither its inputs in cache nor
    another kernel's dirty lines to write back.  mode: "both" (default),
    "write" (the fill only), "read" (the read only) or "none"."""

    def __init__(self, torch, mode="both"):
        self.mode = mode
        self.w = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") \
            if mode in ("both", "write") else None
        self.r = torch.ones(1 << 28, dtype=torch.int32, device="cuda") \
            if mode in ("both", "read") else None
        self.i = 0

    def __call__(self):
        self.i += 1
        if self.w is not None:
            self.w.fill_(self.i & 0xFF)
        if self.r is not None:
            self.sink = self.r.max()


def device_inputs(ep, torch, wl, prob, eo_host=None):
    """Device copies of one workload's inputs and outputs.  Expert outputs
    come from eo_host when given, else from a seeded N(0,1) bf16 draw on the
    GPU (timing does not depend on their values)."""
    import numpy as np
    dev = "cuda"
    d = dict(idx=torch.from_numpy(wl.topk_idx).to(dev),
             w=torch.from_numpy(wl.topk_weights).to(dev),
             x=torch.from_numpy(wl.x.view(np.int16)).to(dev).view(torch.bfloat16))
    if eo_host is not None:
        d["eo"] = torch.from_numpy(eo_host.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        g = torch.Generator(device=dev)
        g.manual_seed(1000 * wl.seed + wl.cid)
        d["eo"] = torch.randn((wl.R, wl.H), generator=g, device=dev, dtype=torch.bfloat16)
    d["lay"] = ep.Layout.empty(prob, dev)
    d["ws"] = ep.alloc_workspace(prob, dev)
    d["recv_x"], d["recv_s"] = ep.alloc_recv(prob, dev)
    d["y"] = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
    return d


def stats_ms(v):
    import statistics
    return dict(mean=sum(v) / len(v), median=statistics.median(v), min=min(v), max=max(v))


def run_steps(ep, torch, wl, prob, fused, K, W, flush, eo_host=None, per_call=True,
              rotating=True):
    """W warm-up steps, then:
      flushed: K steps, each after a cache flush, timed by one HIP event pair
               around the step on the kernels' stream (the headline);
      calls:   K more flushed steps with an event before, between and after
               the calls (per-call durations; the middle event adds a small
               bubble, so the step time comes from `flushed`);
      warm:    K steps back to back, nothing between them, one HIP event pair
               around all K;
    then graph replays, the empty event pair and, if `rotating`, the
    sustained cold-input steps (rotating_steps)."""
    d = device_inputs(ep, torch, wl, prob, eo_host)
    lay = d["lay"]
    if fused:
        do_layout = lambda s: None  # noqa: E731  (one call does both)
        do_dispatch = ep.prepare_layout_dispatch(prob, d["idx"], lay, d["ws"], d["x"],
                                                 d["recv_x"], d["recv_s"])
    else:
        do_layout = ep.prepare_layout(prob, d["idx"], lay, d["ws"])
        do_dispatch = ep.prepare_dispatch(prob, d["x"], lay, d["recv_x"], d["recv_s"])
    do_combine = ep.prepare_combine(prob, d["eo"], lay, d["w"], d["y"])
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step():
        do_layout(stream)
        do_dispatch(stream)
        do_combine(stream)

    print(f"[bench] {wl.name}: warmup {W} steps", file=sys.stderr, flush=True)
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    count = lay.count.cpu().numpy()

    ev = HipEvents(2 * K)
    for i in range(K):
        flush()
        ev.record(2 * i, sh)
        step()
        ev.record(2 * i + 1, sh)
    torch.cuda.synchronize()
    flushed = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)]
    ev.close()
    print(f"[bench] {wl.name}: {K} flushed steps, mean {sum(flushed) / K * 1e3:.2f} us",
          file=sys.stderr, flush=True)

    out = dict(count=count, flushed=stats_ms(flushed))
    if per_call:
        # events before, between and after the calls (ep_layout has its own
        # pair only on the separate path: an empty pair costs a few us)
        n = 3 if fused else 4
        ev = HipEvents(n * K)
        for i in range(K):
            flush()
            e = n * i
            ev.record(e, sh)
            if not fused:
                do_layout(stream)
                e += 1
                ev.record(e, sh)
            do_dispatch(stream)
            ev.record(e + 1, sh)
            do_combine(stream)
            ev.record(e + 2, sh)
        torch.cuda.synchronize()

        def mean_ms(a, b):
            return sum(ev.elapsed_ms(n * i + a, n * i + b) for i in range(K)) / K

        if fused:
            out.update(layout_ms=0.0, dispatch_ms=mean_ms(0, 1), combine_ms=mean_ms(1, 2))
        else:
            out.update(layout_ms=mean_ms(0, 1), dispatch_ms=mean_ms(1, 2),
                       combine_ms=mean_ms(2, 3))
        ev.close()

    torch.cuda.synchronize()
    ev = HipEvents(2)
    ev.record(0, sh)
    for _ in range(K):
        step()
    ev.record(1, sh)
    torch.cuda.synchronize()
    out["warm_ms"] = ev.elapsed_ms(0, 1) / K
    ev.close()

    def step_on(s):
        do_layout(s)
        do_dispatch(s)
        do_combine(s)

    out["graph_ms"] = graph_step_ms(torch, step_on)

    # an event pair with nothing between it, after a flush: what the two
    # markers add to each flushed step's measured time
    ev = HipEvents(2 * K)
    for i in range(K):
        flush()
        ev.record(2 * i, sh)
        ev.record(2 * i + 1, sh)
    torch.cuda.synchronize()
    out["empty_pair_ms"] = sum(ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)) / K
    ev.close()

    nb = algorithmic_bytes(wl)
    step_bytes = nb["dispatch_total"] + nb["combine_total"]
    if rotating and step_bytes >= (64 << 20):
        out.update(rotating_steps(ep, torch, wl, prob, fused, d, K, step_bytes))
    else:
        # a step this small would need dozens of buffer sets (up to 17 GB)
        out.update(rotating_ms=None, rotating_sets=None)
    del d
    return out


def rotating_steps(ep, torch, wl, prob, fused, d, K, step_bytes):
    """Sustained steps with cold inputs: K steps back to back, timed by one
    HIP event pair around all K, no flush or per-step marker inside.  Step i
    reads input set i mod S_in (x, topk_idx, topk_weights) and uses buffer
    set i mod S_out (expert outputs, layout, receive rows, y, workspace).
    Most of a step's traffic is non-temporal and need not displace a plainly
    loaded input from the 256 MB MALL, so the input sets alone must cycle
    through at least 1 GiB between two uses of one (measured: with three
    whole-step sets the skewed step's x stayed in the MALL, 131 against 141 us
    with six or more); S_in = ceil(1 GiB / input bytes) + 1 (3 to 64), and
    S_out = 3 (larger than the MALL together at these sizes)."""
    import math
    in_bytes = sum(t.numel() * t.element_size() for t in (d["idx"], d["w"], d["x"]))
    s_in = int(max(3, min(64, math.ceil((1 << 30) / max(in_bytes, 1)) + 1)))
    s_out = 3
    ins = [d] + [dict(idx=d["idx"].clone(), w=d["w"].clone(), x=d["x"].clone())
                 for _ in range(s_in - 1)]
    outs = [d]
    for _ in range(s_out - 1):
        c = dict(eo=d["eo"].clone(), lay=ep.Layout.empty(prob, "cuda"),
                 ws=ep.alloc_workspace(prob, "cuda"), y=torch.empty_like(d["y"]))
        c["recv_x"], c["recv_s"] = ep.alloc_recv(prob, "cuda")
        outs.append(c)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(i):
        a, o = ins[i % s_in], outs[i % s_out]
        if fused:
            ep.ep_layout_dispatch(prob, a["idx"], o["lay"], o["ws"], a["x"], o["recv_x"],
                                  o["recv_s"], stream=stream)
        else:
            ep.ep_layout(prob, a["idx"], o["lay"], o["ws"], stream=stream)
            ep.ep_dispatch(prob, a["x"], o["lay"], o["recv_x"], o["recv_s"], stream=stream)
        ep.ep_combine(prob, o["eo"], o["lay"], a["w"], o["y"], stream=stream)

    for i in range(max(s_in, s_out)):
        step(i)
    torch.cuda.synchronize()
    ev = HipEvents(2)
    ev.record(0, sh)
    for i in range(K):
        step(i)
    ev.record(1, sh)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / K
    ev.close()
    # the copies go back to torch's cache, not to the driver: for a few
    # seconds after gigabytes are freed with hipFree, steps run about 2%
    # slower (measured), which would fall on whatever is timed next
    del ins, outs
    return dict(rotating_ms=ms, rotating_sets=s_in)


def graph_step_ms(torch, step_on, G=20, R=10):
    """Back-to-back steps replayed from a HIP graph: G steps captured once
    (on a side stream, after one eager warm-up step there), the graph
    replayed R times in a row on the current stream and timed by one HIP
    event pair; returns ms per step.  The calls allocate nothing and issue
    no memset, so the graph holds only the library's kernel launches; what
    it removes is the host's per-call launch work, which the eager
    back-to-back loop pays for small batches."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_on(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(G):
            step_on(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    sh = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    ev.record(0, sh)
    for _ in range(R):
        g.replay()
    ev.record(1, sh)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / (R * G)
    ev.close()
    del g
    return ms


def skew_sweep(ep, torch, workloads, args, flush):
    """Sensitivity of the step to routing skew: the 4096-token prefill shape
    with 16 hot experts at 1.0-3.0x the mean load, and the skewed shape with
    Zipf exponents 0.8, 1.2, 1.6.  One JSON line per variant."""
    import numpy as np
    variants = [(3, dict(), "hot 1.0x")] + \
        [(3, dict(hot_experts=16, hot_ratio=r), f"hot {r}x") for r in (1.5, 2.0, 3.0)] + \
        [(4, dict(zipf_s=s), f"zipf {s}") for s in (0.8, 1.2, 1.6)]
    for cid, over, label in variants:
        wl = workloads.make(cid, **over)
        prob = ep.Problem(wl.T, wl.H, wl.k, wl.E, wl.cap, int(wl.fp8))
        # no sustained cold-input steps: their buffer sets would slow the
        # variants timed after them in this process
        r = run_steps(ep, torch, wl, prob, args.path == "fused", args.steps, args.warmup, flush,
                      rotating=False)
        nb = algorithmic_bytes(wl, r["count"])
        ms = r["flushed"]["mean"]
        total = nb["dispatch_total"] + nb["combine_total"]
        counts = np.asarray(r["count"])
        print(json.dumps({
            "metric": METRIC, "sweep": "skew", "variant": label, "path": args.path,
            "value": round(total / (ms / 1e3) / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(ms, 5),
            "pct_of_hbm_peak": round(100 * total / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 2),
            "warm_ms_per_step": round(r["warm_ms"], 5),
            "config": {"workload": wl.name, "tokens": wl.T, "hidden": wl.H, "experts": wl.E,
                       "topk": wl.k, "payload": "e4m3" if wl.fp8 else "bf16", **over,
                       "hot_load_ratio": wl.meta.get("hot_load_ratio")},
            "max_over_mean_expert_load": round(float(counts.max() / counts.mean()), 3),
            "us_per_call": {"layout": round(r["layout_ms"] * 1e3, 3) if args.path != "fused" else None,
                            "dispatch": round(r["dispatch_ms"] * 1e3, 3),
                            "combine": round(r["combine_ms"] * 1e3, 3)},
        }), flush=True)
    return 0


def config_table(args):
    """Every workload (1-5) timed the same ways as the headline (flushed,
    sustained cold, back to back, graph replay, per-call events), each in a
    child process of its own running this script, so that each is measured
    as when it runs alone: in one process, what one workload leaves behind
    reaches the next (for a few seconds after gigabytes are returned to the
    driver, steps run about 2% slower: skewed workload, flushed, 142.4-143.4
    against 139.3-140.0 us, on the very same buffers).  The parent does no
    GPU work meanwhile.
    A child that fails leaves an "error" entry; the rest are still timed."""
    import subprocess
    out = {}
    for cid in (1, 2, 3, 4, 5):
        print(f"[bench] config table: workload {cid} (child process)", file=sys.stderr, flush=True)
        cmd = [sys.executable, "-u", os.path.abspath(__file__), "--config", str(cid),
               "--steps", str(args.config_steps), "--warmup", str(min(args.warmup, 5)),
               "--flush", args.flush, "--path", args.path, "--scales", args.scales,
               "--no-config-table", "--no-cpu-baseline", "--eo-on-device"]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        lines = r.stdout.strip().splitlines()
        if r.returncode != 0 or not lines:
            out[f"workload_{cid}"] = {"error": f"exit {r.returncode}: {r.stderr[-500:]}"}
            continue
        c = json.loads(lines[-1])
        det, cfg = c["detail"], c["config"]
        f = det["flushed_step_us"]
        pc = det["us_per_call_flushed"]
        sc = det["sustained_cold"]
        out[cfg["workload"]] = {
            "shape": f"T={cfg['tokens']} H={cfg['hidden']} E={cfg['experts']} k={cfg['topk']} "
                     f"cap={cfg['capacity']} {cfg['payload']}",
            "bytes_per_step": det["algorithmic_bytes"]["dispatch_total"] +
                              det["algorithmic_bytes"]["combine_total"],
            "flushed": {"us_per_step": round(f["mean"], 2), "GBps": c["value"],
                        "pct_of_hbm_peak": det["pct_of_hbm_peak"],
                        "us_median": round(f["median"], 2), "us_min": round(f["min"], 2),
                        "us_max": round(f["max"], 2)},
            "warm": {k: det["warm_back_to_back"][k] for k in ("us_per_step", "GBps",
                                                               "pct_of_hbm_peak")},
            "sustained_cold": None if sc is None else
            {k: sc[k] for k in ("us_per_step", "GBps", "pct_of_hbm_peak", "buffer_sets")},
            "event_pair_overhead_us": det["event_pair_overhead_us"],
            "graph": det["graph_back_to_back"],
            "us_per_call_flushed": {"layout": pc["layout"], "dispatch": pc["dispatch"],
                                    "combine": pc["combine"]},
        }
    return out


def target_text(wl, pct_flushed, pct_sustained):
    """The 70% bar of the 4096-token prefill step, stated for both cold-cache
    measurements."""
    if wl.cid != 3:
        return "n/a (the bar is stated for the 4096-token prefill)"

    def verdict(p):
        if p is None:
            return "not measured"
        return f"{'met' if p >= 70 else 'not met'} ({p:.2f}%)"

    return ("(B_dispatch + B_combine) / step >= 70% of 8 TB/s at the 4096-token prefill: "
            f"flushed single steps {verdict(pct_flushed)}; sustained steps with cold inputs "
            f"{verdict(pct_sustained)}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--flush", choices=["both", "write", "read", "none"], default="both",
                    help="cache eviction before each timed step (outside the events): a "
                         "512 MiB fill and a 1 GiB read (both), one of them, or none")
    ap.add_argument("--eo-on-device", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-config-table", action="store_true",
                    help="skip timing workloads 1-5 (detail.configs)")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="flushed and back-to-back steps per workload of detail.configs")
    ap.add_argument("--sweep", choices=["skew"], default=None,
                    help="skew: routing-skew sensitivity (one JSON line per variant) instead "
                         "of the single benchmark line")
    ap.add_argument("--scales", choices=["fp32", "ue8m0"], default="fp32",
                    help="block-scale format of the FP8 workloads (2, 4, 5)")
    ap.add_argument("--path", choices=["separate", "fused"], default="fused",
                    help="fused: ep_layout_dispatch; separate: ep_layout then ep_dispatch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run one device-to-device copy of 256 MiB (for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not "
              "supported (the multi-GPU exchange is not part of it)", file=sys.stderr)
        return 2

    import torch

    import combine_ep_layout_09_amd as ep
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.copy_calibration:
        a = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": a.numel()}))
        return 0
    flush = Flush(torch, args.flush)
    if args.sweep == "skew":
        return skew_sweep(ep, torch, workloads, args, flush)

    print(f"[bench] generating workload {args.config}", file=sys.stderr, flush=True)
    wl = workloads.make(args.config)
    # expert outputs drawn on the GPU (the config table's child runs): timing
    # does not depend on their values, and the CPU baseline is not run there
    eo_host = None if args.eo_on_device and args.no_cpu_baseline else wl.expert_out()
    ue8m0 = bool(wl.fp8) and args.scales == "ue8m0"
    prob = ep.Problem(wl.T, wl.H, wl.k, wl.E, wl.cap, 2 if ue8m0 else int(wl.fp8))
    fused = args.path == "fused"
    K = args.steps
    r = run_steps(ep, torch, wl, prob, fused, K, args.warmup, flush, eo_host=eo_host)
    nb = algorithmic_bytes(wl, r["count"], scale_bytes=1 if ue8m0 else 4)
    layout_ms, dispatch_ms, combine_ms = r["layout_ms"], r["dispatch_ms"], r["combine_ms"]
    ms_per_step = r["flushed"]["mean"]
    total_bytes = nb["dispatch_total"] + nb["combine_total"]
    value = total_bytes / (ms_per_step / 1e3) / 1e9
    warm_gbps = total_bytes / (r["warm_ms"] / 1e3) / 1e9

    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    if fused:
        # the whole ep_layout_dispatch call: the layout's and the dispatch's
        # algorithmic bytes, over the call's duration
        disp_entry = (fused_call_name(wl, ncu),
                      (dispatch_ms, nb["dispatch_total"], FUSED_SOURCES[fused_call_name(wl, ncu)]))
    else:
        disp_entry = ("dispatch_bf16_kernel" if not wl.fp8 else "dispatch_fp8_kernel",
                      (dispatch_ms, nb["dispatch_kernel"], ("ep_dispatch.hip",)))
    comb = combine_kernel_name(wl, ncu)
    kernels = {disp_entry[0]: disp_entry[1],
               comb: (combine_ms, nb["combine_kernel"], ("ep_combine.hip",))}
    dom = max(kernels, key=lambda n: kernels[n][0])
    dom_ms, dom_bytes, dom_src = kernels[dom]
    achieved = dom_bytes / (dom_ms / 1e3) / 1e9
    traffic = read_traffic(dom, dom_src, wl.name + ("_ue8m0" if ue8m0 else ""))

    copy_gbps = measure_copy_gbps(torch)
    configs = None if args.no_config_table else config_table(args)
    pct = 100 * value / HBM_PEAK_GBPS

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3+ue8m0" if ue8m0 else "fp8e4m3") if wl.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.T, "hidden": wl.H, "experts": wl.E,
                   "topk": wl.k, "capacity": wl.cap,
                   "payload": "e4m3" if wl.fp8 else "bf16",
                   "scales": ("ue8m0" if ue8m0 else "fp32") if wl.fp8 else None, "seed": wl.seed,
                   "routing": {1: "uniform distinct", 2: "uniform distinct",
                               3: "group-limited 8x32 top-4 groups",
                               4: "Zipf 1.2 without replacement",
                               5: "group-limited + 16 hot experts at 1.5x"}[wl.cid],
                   "parallelism": "single GPU, all experts local",
                   "path": "ep_layout_dispatch + ep_combine" if fused
                           else "ep_layout + ep_dispatch + ep_combine",
                   "timing": f"each step after a cache flush ({args.flush}), one HIP event "
                             "pair around the step"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": dom_bytes,
                     "avg_launch_us": round(dom_ms * 1e3, 3)},
        "detail": {
            "pct_of_hbm_peak": round(pct, 2),
            "target": target_text(wl, pct, None if r["rotating_ms"] is None else
                                  100 * total_bytes / r["rotating_ms"] * 1e3 / 1e9 / HBM_PEAK_GBPS),
            "flushed_step_us": {k: round(v * 1e3, 3) for k, v in r["flushed"].items()},
            "warm_back_to_back": {"us_per_step": round(r["warm_ms"] * 1e3, 3),
                                  "GBps": round(warm_gbps, 2),
                                  "pct_of_hbm_peak": round(100 * warm_gbps / HBM_PEAK_GBPS, 2)},
            "us_per_call_flushed": {"layout": round(layout_ms * 1e3, 3) if not fused else None,
                                    "dispatch": round(dispatch_ms * 1e3, 3),
                                    "dispatch_incl_layout": round((layout_ms + dispatch_ms) * 1e3, 3),
                                    "combine": round(combine_ms * 1e3, 3)},
            "sustained_cold": None if r["rotating_ms"] is None else {
                "us_per_step": round(r["rotating_ms"] * 1e3, 3),
                "GBps": round(total_bytes / r["rotating_ms"] * 1e3 / 1e9, 2),
                "pct_of_hbm_peak": round(100 * total_bytes / r["rotating_ms"] * 1e3 / 1e9 / HBM_PEAK_GBPS, 2),
                "buffer_sets": r["rotating_sets"],
                "how": "K steps back to back, step i reading input set i mod S (x, topk_idx, "
                       "topk_weights; S copies cycling through >= 1 GiB) and using output set i mod 3 "
                       "(expert outputs, layout, receive rows, y), one HIP event pair around all K steps"},
            "event_pair_overhead_us": round(r["empty_pair_ms"] * 1e3, 3),
            "graph_back_to_back": {"us_per_step": round(r["graph_ms"] * 1e3, 3),
                                   "GBps": round(total_bytes / r["graph_ms"] * 1e3 / 1e9, 2),
                                   "pct_of_hbm_peak": round(
                                       100 * total_bytes / r["graph_ms"] * 1e3 / 1e9 / HBM_PEAK_GBPS, 2)},
            "GBps_per_call": {
                "dispatch_incl_layout": round(nb["dispatch_total"] / ((layout_ms + dispatch_ms) / 1e3) / 1e9, 2),
                "combine_kernel": round(nb["combine_kernel"] / (combine_ms / 1e3) / 1e9, 2)},
            "algorithmic_bytes": nb,
            "device_copy_GBps_1GiB": round(copy_gbps, 1),
            "device": torch.cuda.get_device_name(0),
            "configs": configs,
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, eo_host, total_bytes, args.cpu_seconds,
                                           prob.use_fp8)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
