"""ep_layout_dispatch_noalloc (the library's fixed device array as the layout
workspace) against ep_layout_dispatch with a caller-allocated workspace:
every layout array, every receive row and every scale bit for bit, on calls
in a row, each smaller than the one before.  The first two take forms of the
call that use the workspace -- FP8 rows with k = 6 over 16 experts (the
histogram and ranking kernels of the layout, then the dispatch kernel) and
FP8 rows with k = 8 (the histogram kernel, then the ranking dispatch
kernel) -- which the test checks against bench.py's mirror of the library's
launch rules; the decode workload (one kernel) does not touch it."""
import importlib.util
import os

import numpy as np
import pytest
import torch

import combine_ep_layout_09_amd as ep
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _launch_rules():
    spec = importlib.util.spec_from_file_location("bench_rules", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(prob, idx, x, noalloc):
    lay = ep.Layout.empty(prob, DEV)
    for t in (lay.count, lay.offset, lay.slot_of, lay.src_of_slot, lay.status):
        t.fill_(-7)
    recv_x, recv_s = ep.alloc_recv(prob, DEV)
    recv_x.view(torch.uint8).fill_(0xFF)
    recv_s.view(torch.uint8).fill_(0xFF)
    if noalloc:
        ep.ep_layout_dispatch_noalloc(prob, idx, lay, x, recv_x, recv_s)
    else:
        ws = ep.alloc_workspace(prob, DEV)
        ws.fill_(0xAB)
        ep.ep_layout_dispatch(prob, idx, lay, ws, x, recv_x, recv_s)
    torch.cuda.synchronize()
    out = {n: getattr(lay, n).cpu().numpy() for n in ("count", "offset", "slot_of",
                                                        "src_of_slot", "status")}
    out["recv_x"] = recv_x.view(torch.uint8).cpu().numpy()
    out["recv_s"] = recv_s.view(torch.uint8).cpu().numpy()
    return out


def test_noalloc_matches_layout_dispatch():
    cases = [
        # skewed shape over 16 experts: T=8192, H=4096, k=6, FP8, Zipf routing
        (workloads.make(4, E=16), 1),
        # a smaller problem with more experts and k = 8, UE8M0 scales
        (workloads.make(5, T=2000, H=1024, E=128), 2),
        # the decode workload (one kernel; the workspace is not touched)
        (workloads.make(2), 1),
    ]
    rules = _launch_rules()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    assert rules.fused_call_name(cases[0][0], ncu) == \
        "layout_hist_kernel+layout_rank_kernel+dispatch_fp8_kernel"
    assert rules.fused_call_name(cases[1][0], ncu) == \
        "layout_hist_kernel+layout_dispatch_ranked_kernel"
    inputs, want = [], []
    for wl, mode in cases:
        prob = ep.Problem(wl.T, wl.H, wl.k, wl.E, wl.cap, mode)
        idx = torch.from_numpy(wl.topk_idx).to(DEV)
        x = torch.from_numpy(wl.x.view(np.int16)).to(DEV).view(torch.bfloat16)
        inputs.append((wl, prob, idx, x))
        want.append(_run(prob, idx, x, noalloc=False))
    # the allocation-free calls back to back, larger problem first
    got = []
    for wl, prob, idx, x in inputs:
        print(f"[gpu] noalloc: {prob!r}", flush=True)
        got.append(_run(prob, idx, x, noalloc=True))
    for (wl, prob, _, _), g, w in zip(inputs, got, want):
        for n in w:
            assert np.array_equal(g[n].view(np.uint8), w[n].view(np.uint8)), (prob, n)
        ref = oracle.layout(wl.topk_idx, wl.E, wl.cap)
        for n in ("count", "offset", "slot_of", "src_of_slot", "status"):
            np.testing.assert_array_equal(g[n], ref[n], err_msg=f"{prob!r}: {n}")
