"""Two problems in flight at once on two streams (two micro-batches of a
pipeline, say): the decode batch and a 2048-token prefill batch, each
ep_layout_dispatch + ep_combine on its own stream with its own workspace,
launched interleaved so that the kernels of both can run together.  Every
output of both must equal the same calls made one after the other on one
stream, bit for bit: the library keeps no state between calls that two
streams could share (the allocation-free entry point's device array aside,
which these calls do not use)."""
import numpy as np
import pytest
import torch

import combine_ep_layout_09_amd as ep
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


class Batch:
    def __init__(self, wl, mode):
        self.prob = ep.Problem(wl.T, wl.H, wl.k, wl.E, wl.cap, mode)
        self.idx = torch.from_numpy(wl.topk_idx).to(DEV)
        self.x = torch.from_numpy(wl.x.view(np.int16)).to(DEV).view(torch.bfloat16)
        self.w = torch.from_numpy(wl.topk_weights).to(DEV)
        self.eo = torch.from_numpy(wl.expert_out().view(np.int16)).to(DEV).view(torch.bfloat16)
        self.lay = ep.Layout.empty(self.prob, DEV)
        self.ws = ep.alloc_workspace(self.prob, DEV)
        self.recv_x, self.recv_s = ep.alloc_recv(self.prob, DEV)
        self.y = torch.empty_like(self.x)

    def clear(self):
        for t in (self.lay.count, self.lay.offset, self.lay.slot_of, self.lay.src_of_slot,
                  self.lay.status):
            t.fill_(-7)
        self.recv_x.view(torch.uint8).fill_(0xFF)
        if self.recv_s is not None:
            self.recv_s.view(torch.uint8).fill_(0xFF)
        self.y.view(torch.int16).fill_(0x5555)

    def dispatch(self, stream):
        ep.ep_layout_dispatch(self.prob, self.idx, self.lay, self.ws, self.x, self.recv_x,
                              self.recv_s, stream=stream)

    def combine(self, stream):
        ep.ep_combine(self.prob, self.eo, self.lay, self.w, self.y, stream=stream)

    def outputs(self):
        out = {n: getattr(self.lay, n).cpu().numpy().copy()
               for n in ("count", "offset", "slot_of", "src_of_slot", "status")}
        out["recv_x"] = self.recv_x.view(torch.uint8).cpu().numpy().copy()
        if self.recv_s is not None:
            out["recv_s"] = self.recv_s.view(torch.uint8).cpu().numpy().copy()
        out["y"] = self.y.view(torch.int16).cpu().numpy().copy()
        return out


def test_two_batches_on_two_streams():
    a = Batch(workloads.make(2), 1)           # decode: one-kernel layout + dispatch
    b = Batch(workloads.make(3, T=2048), 0)   # prefill: one launch of one workgroup per CU
    main = torch.cuda.current_stream()

    # reference: one batch after the other on one stream
    want = []
    for bt in (a, b):
        bt.clear()
        bt.dispatch(main)
        bt.combine(main)
        torch.cuda.synchronize()
        want.append(bt.outputs())

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        a.clear()
        b.clear()
        torch.cuda.synchronize()
        print(f"[gpu] two streams, round {rep}: {a.prob!r} and {b.prob!r}", flush=True)
        b.dispatch(s2)
        a.dispatch(s1)
        a.combine(s1)
        b.combine(s2)
        torch.cuda.synchronize()
        for bt, w in zip((a, b), want):
            got = bt.outputs()
            for n, v in w.items():
                assert np.array_equal(got[n], v), f"{bt.prob!r}: round {rep}: {n}"
