"""GPU parity of the FP8 dispatch quantiser over every (x, block maximum) pair.

The dispatch kernels reach the code of the IEEE quotient fl(x / scale) with
a reciprocal multiply and fall back to the division next to E4M3 rounding
midpoints.  This test runs the dispatch kernels themselves (not the
elementwise encoder) over every pair of bf16 values (x, amax) with
|x| <= amax, amax a positive finite bf16 value, both signs of x, and compares
payload bytes and scale bits with the CPU oracle: fp32 scales
(scale = amax / 448) and UE8M0 scales.

Layout of the inputs: one 128-channel block per block maximum a (or several,
when the 2(a + 1) values |x| <= a of both signs do not fit in 127 channels):
channel 0 holds +a or -a (alternating from block to block), channels 1..127
run through +0, +1 ulp, ..., +a, -0, ..., -a, wrapping round to fill the last
block of each a.  Blocks are packed 16 to a token row (H = 2048, two 16-byte
pieces per lane: the launch shape of prefill-sized FP8 dispatch), with zero
blocks padding the last row.  The bf16 values are taken in ranges of block
maxima so that each GPU call moves about 64 M channels.
"""
import os

import numpy as np
import pytest
import torch

import combine_ep_layout_09_amd as ep
import oracle

DEV = "cuda:0"
H = 2048
BLOCKS_PER_ROW = H // 128
MAX_BF16 = 0x7F7F          # largest finite bf16 magnitude pattern
CHUNK_VALUES = 64 << 20    # channels per GPU call (about)


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except (AttributeError, OSError):
        return 4


def _amax_ranges():
    """Consecutive ranges [a0, a1) of block-maximum patterns, each holding
    about CHUNK_VALUES (x, amax) pairs."""
    out, a0, acc = [], 1, 0
    for a in range(1, MAX_BF16 + 1):
        acc += 2 * (a + 1)
        if acc >= CHUNK_VALUES or a == MAX_BF16:
            out.append((a0, a + 1))
            a0, acc = a + 1, 0
    return out


AMAX_RANGES = _amax_ranges()


_PATTERNS = np.arange(MAX_BF16 + 1, dtype=np.uint16)


def exhaustive_rows(a0, a1):
    """uint16 [rows, H] bf16 patterns covering every pair (x, a) with a in
    [a0, a1) and |x| <= a, both signs of x (see the module docstring)."""
    a_all = np.arange(a0, a1, dtype=np.int64)
    nb = (2 * (a_all + 1) + 126) // 127            # blocks per block maximum
    B = int(nb.sum())
    rows = -(-B // BLOCKS_PER_ROW)
    blocks = np.zeros((rows * BLOCKS_PER_ROW, 128), np.uint16)
    b = 0
    for a, nblk in zip(a_all.tolist(), nb.tolist()):
        n = 2 * (a + 1)
        vals = np.empty(nblk * 127, np.uint16)
        vals[:a + 1] = _PATTERNS[:a + 1]
        vals[a + 1:n] = _PATTERNS[:a + 1] | np.uint16(0x8000)
        for w in range(n, nblk * 127, n):          # wrap round to fill the last block
            m = min(n, nblk * 127 - w)
            vals[w:w + m] = vals[:m]
        blk = blocks[b:b + nblk]
        blk[:, 1:] = vals.reshape(nblk, 127)
        blk[:, 0] = a
        b += nblk
    blocks[1:B:2, 0] |= np.uint16(0x8000)      # -a in every other block
    return blocks.reshape(rows, H)


def test_exhaustive_rows_cover_every_pair():
    """The generator itself (host only, on a small range): every pair (x, a)
    with |x| <= a appears, channel 0 holds the block maximum, and no value
    exceeds it."""
    a0, a1 = 1, 300
    rows = exhaustive_rows(a0, a1)
    blocks = rows.reshape(-1, 128)
    mag = blocks & 0x7FFF
    seen = set()
    for blk in blocks:
        amax = int(blk[0] & 0x7FFF)
        if amax == 0:
            assert (blk & 0x7FFF == 0).all()
            continue
        assert (blk[1:] & 0x7FFF <= amax).all()
        seen.update((amax, int(v)) for v in blk[1:])
    want = {(a, v) for a in range(a0, a1) for m in range(a + 1) for v in (m, m | 0x8000)}
    assert want <= seen
    assert mag.max() == a1 - 1


def _run(mode, x_host, fused, k=1):
    """Dispatch of rows x_host (T tokens, one expert, k copies each);
    returns (recv_x [T*k, H] uint8, recv_scales) on the host."""
    T = x_host.shape[0]
    prob = ep.Problem(T, H, k, 1, 0, mode)
    x = torch.from_numpy(x_host.view(np.int16)).to(DEV).view(torch.bfloat16)
    recv_x, recv_s = ep.alloc_recv(prob, DEV)
    recv_x.fill_(0xFF)
    recv_s.view(torch.uint8).fill_(0xFF)
    if fused:
        lay = ep.Layout.empty(prob, DEV)
        ws = ep.alloc_workspace(prob, DEV)
        idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
        ep.ep_layout_dispatch(prob, idx, lay, ws, x, recv_x, recv_s)
    else:
        slot = torch.arange(T * k, dtype=torch.int32, device=DEV).view(T, k)
        lay = ep.Layout(None, None, slot, None, None)
        ep.ep_dispatch(prob, x, lay, recv_x, recv_s)
    torch.cuda.synchronize()
    return recv_x.cpu().numpy(), recv_s.cpu().numpy()


def _check(mode, x_host, got_x, got_s, k=1):
    T = x_host.shape[0]
    slot = np.arange(T * k, dtype=np.int32).reshape(T, k)
    rx, rs = oracle.dispatch(x_host, slot, T * k, mode, threads=_threads())
    bad = np.flatnonzero((got_x != rx).any(axis=1))
    assert bad.size == 0, (f"payload differs in {bad.size} rows, first row {bad[0]} "
                           f"(token {bad[0] // k})")
    np.testing.assert_array_equal(got_s.view(np.uint8), rs.view(np.uint8), err_msg="scales")


@pytest.mark.gpu
def test_dispatch_quantiser_every_pair():
    """ep_dispatch over all 1.07e9 pairs (x, amax), fp32 and UE8M0 scales, in
    calls of about 64 M channels each."""
    total = 0
    for a0, a1 in AMAX_RANGES:
        x_host = exhaustive_rows(a0, a1)
        for mode in (1, 2):
            print(f"[gpu] exhaustive quantiser mode {mode}: block maxima "
                  f"{a0:#06x}..{a1 - 1:#06x}, {x_host.shape[0]} rows", flush=True)
            got_x, got_s = _run(mode, x_host, fused=False)
            _check(mode, x_host, got_x, got_s)
        total += x_host.size
    print(f"[gpu] exhaustive quantiser: {total} channels bit-exact in both scale modes",
          flush=True)


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [1, 2], ids=["fp32_scales", "ue8m0"])
def test_layout_dispatch_quantiser_sampled_ranges(mode):
    """The same inputs through ep_layout_dispatch, whose other forms carry
    their own copy of the tile code: the one-kernel form for small tables
    (512 tokens, k = 8: 4096 routing entries), the one-launch form of one
    workgroup per CU (4096 tokens: 32768 entries) and the ranking dispatch
    kernel (8192 tokens: 65536 entries), on the first, a middle and the last
    range of block maxima."""
    picks = [AMAX_RANGES[0], AMAX_RANGES[len(AMAX_RANGES) // 2], AMAX_RANGES[-1]]
    for a0, a1 in picks:
        rows = exhaustive_rows(a0, a1)
        for T in (512, 4096, 8192):
            for start in range(0, rows.shape[0], max(T, rows.shape[0] // 3)):
                x_host = np.ascontiguousarray(rows[start:start + T])
                print(f"[gpu] layout_dispatch quantiser mode {mode}: maxima "
                      f"{a0:#06x}..{a1 - 1:#06x}, rows {start}..{start + x_host.shape[0]}, k 8",
                      flush=True)
                got_x, got_s = _run(mode, x_host, fused=True, k=8)
                _check(mode, x_host, got_x, got_s, k=8)
