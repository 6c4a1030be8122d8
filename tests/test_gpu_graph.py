"""The path under HIP graph capture: ep_layout_dispatch_noalloc and ep_combine
captured once into a torch CUDA graph (a HIP graph on ROCm), then replayed
over new inputs copied into the captured buffers.  Every replay is checked
bit for bit against the same calls made eagerly (layout arrays, receive rows,
scales, combine output); the outputs are refilled with a sentinel before each
replay, and eager work and synchronisations run between the replays.

The captured calls allocate nothing (the layout workspace is the library's
device array) and issue no memset, so the graph holds only the library's
kernel launches.  Shapes: the decode workload (one layout+dispatch kernel,
the per-token combine), the skewed workload (the one-kernel layout, FP8
dispatch, persistent combine), a 2048-token prefill (the one-launch layout +
dispatch of one workgroup per CU), and two forms whose kernels pass tables
through the workspace array between launches: a 2047-token bf16 batch with
k = 7 (the histogram kernel, then the ranking dispatch kernel) and the skewed
shape over 16 experts (the histogram and ranking kernels of the layout, then
the FP8 dispatch kernel)."""
import numpy as np
import pytest
import torch

import combine_ep_layout_09_amd as ep
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    ("decode", dict(cid=2), 1),
    ("skewed", dict(cid=4), 1),
    ("prefill_2048", dict(cid=3, T=2048), 0),
    ("decode_ue8m0", dict(cid=2), 2),
    ("ranked_workspace", dict(cid=3, T=2047, k=7, H=2048), 0),
    ("hist_rank_workspace", dict(cid=4, E=16), 1),
]


def _inputs(spec, mode, seed):
    """Host arrays of one input set (seeded), in the shapes of `spec`."""
    over = dict(spec)
    cid = over.pop("cid")
    wl = workloads.make(cid, seed=seed, **over)
    prob = ep.Problem(wl.T, wl.H, wl.k, wl.E, wl.cap, mode)
    return prob, dict(idx=wl.topk_idx, x=wl.x, w=wl.topk_weights, eo=wl.expert_out())


class Buffers:
    """Device inputs and outputs of one problem (allocated once, outside any
    capture)."""

    def __init__(self, prob, host):
        self.prob = prob
        self.idx = torch.empty(host["idx"].shape, dtype=torch.int32, device=DEV)
        self.x = torch.empty(host["x"].shape, dtype=torch.bfloat16, device=DEV)
        self.w = torch.empty(host["w"].shape, dtype=torch.float32, device=DEV)
        self.eo = torch.empty(host["eo"].shape, dtype=torch.bfloat16, device=DEV)
        self.lay = ep.Layout.empty(prob, DEV)
        self.recv_x, self.recv_s = ep.alloc_recv(prob, DEV)
        self.y = torch.empty(host["x"].shape, dtype=torch.bfloat16, device=DEV)

    def load(self, host):
        self.idx.copy_(torch.from_numpy(np.ascontiguousarray(host["idx"], np.int32)))
        self.x.view(torch.int16).copy_(torch.from_numpy(host["x"].view(np.int16)))
        self.w.copy_(torch.from_numpy(np.ascontiguousarray(host["w"], np.float32)))
        self.eo.view(torch.int16).copy_(torch.from_numpy(host["eo"].view(np.int16)))

    def clear(self):
        for t in (self.lay.count, self.lay.offset, self.lay.slot_of, self.lay.src_of_slot,
                  self.lay.status):
            t.fill_(-7)
        self.recv_x.view(torch.uint8).fill_(0xFF)
        if self.recv_s is not None:
            self.recv_s.view(torch.uint8).fill_(0xFF)
        self.y.view(torch.int16).fill_(0x5555)

    def step_noalloc(self):
        ep.ep_layout_dispatch_noalloc(self.prob, self.idx, self.lay, self.x, self.recv_x,
                                      self.recv_s)
        ep.ep_combine(self.prob, self.eo, self.lay, self.w, self.y)

    def outputs(self):
        out = {n: getattr(self.lay, n).cpu().numpy().copy()
               for n in ("count", "offset", "slot_of", "src_of_slot", "status")}
        out["recv_x"] = self.recv_x.view(torch.uint8).cpu().numpy().copy()
        if self.recv_s is not None:
            out["recv_s"] = self.recv_s.view(torch.uint8).cpu().numpy().copy()
        out["y"] = self.y.view(torch.int16).cpu().numpy().copy()
        return out


def _eager(prob, host):
    """The eager calls with a caller-allocated workspace."""
    b = Buffers(prob, host)
    b.load(host)
    b.clear()
    ws = ep.alloc_workspace(prob, DEV)
    ws.fill_(0xAB)
    ep.ep_layout_dispatch(prob, b.idx, b.lay, ws, b.x, b.recv_x, b.recv_s)
    ep.ep_combine(prob, b.eo, b.lay, b.w, b.y)
    torch.cuda.synchronize()
    return b.outputs()


@pytest.mark.parametrize("name,spec,mode", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, spec, mode):
    seeds = (0, 1, 2)
    sets = [_inputs(spec, mode, s) for s in seeds]
    prob = sets[0][0]
    want = [_eager(prob, host) for _, host in sets]

    b = Buffers(prob, sets[0][1])
    b.load(sets[0][1])
    b.clear()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.step_noalloc()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    print(f"[gpu] graph capture: {name} {prob!r}", flush=True)
    with torch.cuda.graph(g, stream=side):
        b.step_noalloc()
    torch.cuda.synchronize()

    # replays over the three input sets, then the first again
    for r, i in enumerate((0, 1, 2, 0)):
        b.load(sets[i][1])
        b.clear()
        torch.cuda.synchronize()
        print(f"[gpu] graph replay {r}: {name} inputs of seed {seeds[i]}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = b.outputs()
        for n, v in want[i].items():
            assert np.array_equal(got[n], v), f"{name}: replay {r} (seed {seeds[i]}): {n}"
