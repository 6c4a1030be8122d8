"""Many problems back to back on one stream, with no synchronisation between
the calls: decode-sized and prefill-sized routing tables across the launch
forms of ep_layout_dispatch (the allocation-free call for every other
problem, so that consecutive calls share the library's device array), each
followed by ep_combine, each problem with buffers of its own.  The host waits
once, after the last call.  Every problem's layout arrays, receive rows,
scales and combine output are then checked against the CPU oracle (bit for
bit; combine within one bf16 ulp), and the sentinel left in receive rows no
entry fills shows that no call wrote where it must not: nothing a call leaves
behind in the device array, the caches or the stream reaches the next."""
import numpy as np
import pytest
import torch

import combine_ep_layout_09_amd as ep

from tests.test_gpu_parity import DEV, _random_case, check_case, dev_bf16, host_u16

pytestmark = pytest.mark.gpu

# (T, H, k, E, cap, payload mode): 0 bf16, 1 E4M3FN + fp32 scales, 2 + UE8M0
SHAPES = [
    (128, 1024, 8, 256, 128, 1),    # decode: one layout + dispatch kernel
    (2048, 2048, 8, 64, 0, 0),      # one launch of one workgroup per CU, bf16
    (3000, 1024, 8, 128, 0, 1),     # the same form, FP8
    (3000, 256, 5, 50, 0, 0),       # histogram kernel + ranking dispatch, bf16 (bad ids)
    (6000, 1024, 6, 64, 0, 1),      # one-kernel whole-table layout + FP8 dispatch
    (6000, 512, 6, 16, 0, 2),       # histogram + ranking kernels + FP8 dispatch, UE8M0
    (600, 1024, 16, 64, 0, 1),      # histogram kernel + ranking dispatch, FP8 k = 16
    (15001, 1800, 2, 16, 0, 0),     # ranking dispatch; persistent combine in two launches
    (1000, 264, 7, 33, 0, 0),       # one kernel, ragged rows
    (2500, 256, 6, 7, 3, 1),        # capacity overflow through the layout kernels
    (50, 2304, 4, 16, 64, 0),       # small table with capacity
    (3, 8, 5, 1000, 2, 0),          # few tokens, many experts
]


def _cases():
    out = []
    for i, (T, H, k, E, cap, mode) in enumerate(SHAPES):
        ids = None
        if i == 3:  # ids outside [0, E) and duplicates inside tokens
            rng = np.random.default_rng(77)
            ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
            ids[::9, 1] = ids[::9, 0]
            ids[::13, 2] = -1
            ids[::17, 3] = E
        out.append(_random_case(T, H, k, E, cap, mode, seed=500 + i, ids=ids,
                                name=f"seq{i}_T{T}_H{H}_k{k}_E{E}_c{cap}_m{mode}"))
    return out


class Buffers:
    def __init__(self, c):
        self.prob = ep.Problem(c.T, c.H, c.k, c.E, c.cap, c.fp8)
        self.lay = ep.Layout.empty(self.prob, DEV)
        for t in (self.lay.count, self.lay.offset, self.lay.slot_of, self.lay.src_of_slot,
                  self.lay.status):
            t.fill_(-7)
        self.ws = ep.alloc_workspace(self.prob, DEV)
        self.ws.fill_(0xAB)
        self.recv_x, self.recv_s = ep.alloc_recv(self.prob, DEV)
        self.recv_x.view(torch.uint8).fill_(0xFF)
        if self.recv_s is not None:
            self.recv_s.view(torch.uint8).fill_(0xFF)
        self.y = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)
        self.y.view(torch.int16).fill_(0x5555)
        self.idx = torch.from_numpy(np.ascontiguousarray(c.idx, np.int32)).to(DEV)
        self.w = torch.from_numpy(np.ascontiguousarray(c.w, np.float32)).to(DEV)
        self.x = dev_bf16(c.x)
        self.eo = dev_bf16(c.eo)

    def outputs(self, c):
        out = {n: getattr(self.lay, n).cpu().numpy()
               for n in ("count", "offset", "slot_of", "src_of_slot", "status")}
        out["recv_x"] = self.recv_x.view(torch.uint8).cpu().numpy().reshape(
            c.R, c.H * (1 if c.fp8 else 2))
        out["recv_s"] = None if self.recv_s is None else self.recv_s.cpu().numpy()
        out["y"] = host_u16(self.y)
        return out


def test_back_to_back_problems_on_one_stream():
    cases = _cases()
    bufs = [Buffers(c) for c in cases]
    torch.cuda.synchronize()
    for i, (c, b) in enumerate(zip(cases, bufs)):
        noalloc = i % 2 == 1
        print(f"[gpu] sequence {i}: {b.prob!r} {'noalloc' if noalloc else 'workspace'}",
              flush=True)
        if noalloc:
            ep.ep_layout_dispatch_noalloc(b.prob, b.idx, b.lay, b.x, b.recv_x, b.recv_s)
        else:
            ep.ep_layout_dispatch(b.prob, b.idx, b.lay, b.ws, b.x, b.recv_x, b.recv_s)
        ep.ep_combine(b.prob, b.eo, b.lay, b.w, b.y)
    torch.cuda.synchronize()
    for c, b in zip(cases, bufs):
        check_case(c, b.outputs(c))
