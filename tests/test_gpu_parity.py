"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Bar: layout arrays, dispatch payload bytes and scale bits are bit-exact;
combine output equals the oracle's bf16 bit for bit or lies within 2^-8
relative of the oracle's fp32 sum (one bf16 ulp); the bit-exact fraction is
reported.  Receive buffers are pre-filled with 0xFF bytes (NaN in bf16 and in
E4M3FN) so that rows the method must not write are checked untouched, and
expert-output rows no entry uses are NaN so that reading them would show.
"""
import functools
import os
import zlib

import numpy as np
import pytest
import torch

import combine_ep_layout_09_amd as ep
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAN_BF16 = 0x7FC0


def _threads():
    """Host threads for the oracle (token ranges; same result as serial)."""
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except (AttributeError, OSError):
        return 4


def dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Case:
    def __init__(self, T, H, k, E, cap, fp8, x, idx, w, eo, name="case"):
        # fp8: 0 bf16 payload, 1 E4M3FN + fp32 scales, 2 E4M3FN + UE8M0 scales
        self.T, self.H, self.k, self.E, self.cap, self.fp8 = T, H, k, E, cap, int(fp8)
        self.x, self.idx, self.w, self.eo, self.name = x, idx, w, eo, name

    @property
    def R(self):
        return self.T * self.k if self.cap == 0 else self.E * self.cap

    @classmethod
    def from_workload(cls, wl, nan_unused=True):
        eo = wl.expert_out()
        c = cls(wl.T, wl.H, wl.k, wl.E, wl.cap, wl.fp8, wl.x, wl.topk_idx, wl.topk_weights, eo,
                name=wl.name)
        if nan_unused:
            c.nan_unused_rows()
        return c

    def with_mode(self, fp8, name):
        """The same inputs with another payload mode (0, 1 or 2)."""
        return Case(self.T, self.H, self.k, self.E, self.cap, fp8, self.x, self.idx, self.w,
                    self.eo, name=name)

    def nan_unused_rows(self):
        ref = oracle.layout(self.idx, self.E, self.cap)
        self.eo = self.eo.copy()
        self.eo[ref["src_of_slot"] < 0] = NAN_BF16


def run_gpu(c, stream=None, fused=False):
    prob = ep.Problem(c.T, c.H, c.k, c.E, c.cap, c.fp8)
    print(f"[gpu] {c.name}: {prob!r} {'fused layout+dispatch' if fused else 'separate calls'}",
          flush=True)
    lay = ep.Layout.empty(prob, DEV)
    for t in (lay.count, lay.offset, lay.slot_of, lay.src_of_slot, lay.status):
        t.fill_(-7)
    ws = ep.alloc_workspace(prob, DEV)
    ws.fill_(0xAB)
    recv_x, recv_s = ep.alloc_recv(prob, DEV)
    recv_x.view(torch.uint8).fill_(0xFF)
    if recv_s is not None:
        recv_s.view(torch.uint8).fill_(0xFF)
    y = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)
    y.view(torch.int16).fill_(0x5555)
    idx = torch.from_numpy(np.ascontiguousarray(c.idx, np.int32)).to(DEV)
    w = torch.from_numpy(np.ascontiguousarray(c.w, np.float32)).to(DEV)
    x = dev_bf16(c.x)
    eo = dev_bf16(c.eo)
    torch.cuda.synchronize()
    ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream())
    with ctx:
        if fused:
            ep.ep_layout_dispatch(prob, idx, lay, ws, x, recv_x, recv_s)
        else:
            ep.ep_layout(prob, idx, lay, ws)
            ep.ep_dispatch(prob, x, lay, recv_x, recv_s)
        ep.ep_combine(prob, eo, lay, w, y)
    torch.cuda.synchronize()
    out = {n: getattr(lay, n).cpu().numpy() for n in ("count", "offset", "slot_of", "src_of_slot", "status")}
    out["recv_x"] = recv_x.view(torch.uint8).cpu().numpy().reshape(c.R, c.H * (1 if c.fp8 else 2))
    out["recv_s"] = None if recv_s is None else recv_s.cpu().numpy()
    out["y"] = host_u16(y)
    return out


def check_case(c, got, tokens=None):
    """Compare one run with the oracle.  tokens: None = every token, else the
    token ids whose receive rows and combine outputs are checked."""
    ref = oracle.layout(c.idx, c.E, c.cap)
    for n in ("count", "offset", "slot_of", "src_of_slot", "status"):
        np.testing.assert_array_equal(got[n], ref[n], err_msg=f"{c.name}: layout {n}")
    H = c.H
    pb = 1 if c.fp8 else 2
    placed = ref["src_of_slot"] >= 0
    # rows no entry fills keep the 0xFF sentinel (payload and scales)
    assert (got["recv_x"][~placed] == 0xFF).all(), f"{c.name}: unused receive rows written"
    if c.fp8:
        assert (got["recv_s"][~placed].view(np.uint8) == 0xFF).all(), f"{c.name}: unused scale rows written"
    if c.T == 0:
        return 1.0
    tok = np.arange(c.T) if tokens is None else np.asarray(tokens)
    s_sel = ref["slot_of"][tok]                       # [n, k] global receive rows
    rows = s_sel[s_sel >= 0]                          # in (t, j) order
    compact = np.full_like(s_sel, -1)
    compact[s_sel >= 0] = np.arange(len(rows), dtype=np.int32)
    x_sel = np.ascontiguousarray(c.x[tok])
    nt = _threads()
    if c.fp8:
        rx, rs = oracle.dispatch(x_sel, compact, len(rows), c.fp8, threads=nt)
    else:
        rx, _ = oracle.dispatch(x_sel, compact, len(rows), False, threads=nt)
        rx = rx.view(np.uint8)
    np.testing.assert_array_equal(got["recv_x"][rows], rx, err_msg=f"{c.name}: payload")
    if c.fp8:
        np.testing.assert_array_equal(got["recv_s"][rows].view(np.uint8), rs.view(np.uint8),
                                      err_msg=f"{c.name}: scales")
    ry, racc = oracle.combine(c.eo, s_sel, np.ascontiguousarray(c.w[tok]), threads=nt)
    gy = got["y"][tok]
    gyf = oracle.bf16_to_float(gy).astype(np.float64)
    racc = racc.astype(np.float64)
    exact = gy == ry
    ok = exact | (np.abs(gyf - racc) <= 2.0 ** -8 * np.abs(racc))
    assert ok.all(), f"{c.name}: combine outside tolerance at {np.argwhere(~ok)[:5]}"
    frac = float(exact.mean())
    print(f"[gpu] {c.name}: layout+dispatch bit-exact, combine bit-exact fraction {frac:.6f} "
          f"({int(exact.sum())}/{exact.size})", flush=True)
    return frac


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_workload_full(cid, fused):
    c = Case.from_workload(workloads.make(cid))
    check_case(c, run_gpu(c, fused=fused))


@functools.lru_cache(maxsize=1)
def _large_prefill():
    """T=16384, H=7168, E=256, k=8 (every routing entry valid, so every one of
    the 131072 receive rows is used); built once for the tests below."""
    return Case.from_workload(workloads.make(5), nan_unused=False)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("mode", [1, 2], ids=["fp32_scales", "ue8m0"])
def test_workload_large_prefill_full(mode, fused):
    """T=16384, H=7168, E=256, k=8, FP8: every layout array, every receive
    row (0.94 GB of payload, past the 2 GiB offsets of the bf16 expert
    outputs), every scale row and every combine output (the combine's
    several launches) against the oracle, with fp32 and UE8M0 scales."""
    base = _large_prefill()
    c = base.with_mode(mode, name=f"large_prefill_m{mode}")
    check_case(c, run_gpu(c, fused=fused))


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _random_case(T, H, k, E, cap, fp8, seed, ids=None, name="edge", scale=1.0):
    rng = np.random.default_rng(seed)
    x = workloads.to_bf16_bits((rng.standard_normal((T, H)) * scale).astype(np.float32))
    if ids is None:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    R = T * k if cap == 0 else E * cap
    eo = workloads.to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    c = Case(T, H, k, E, cap, fp8, x, np.asarray(ids, np.int32).reshape(T, k), w, eo, name=name)
    c.nan_unused_rows()
    return c


EDGE = [
    dict(T=0, H=256, k=2, E=8, cap=0, fp8=False, name="empty_T0"),
    dict(T=0, H=256, k=2, E=8, cap=4, fp8=True, name="empty_T0_capacity"),
    dict(T=1, H=128, k=1, E=1, cap=0, fp8=True, name="single_token_single_expert_H128"),
    dict(T=1, H=8, k=3, E=5, cap=0, fp8=False, name="smallest_hidden_H8"),
    dict(T=37, H=136, k=3, E=5, cap=0, fp8=False, name="ragged_hidden_H136"),
    dict(T=1000, H=264, k=7, E=33, cap=0, fp8=False, name="multi_block_ragged_tail"),
    dict(T=3001, H=128, k=5, E=1024, cap=0, fp8=True, name="max_experts"),
    dict(T=129, H=256, k=32, E=64, cap=0, fp8=False, name="max_topk"),
    dict(T=300, H=384, k=4, E=1, cap=0, fp8=True, name="one_expert"),
    dict(T=2500, H=256, k=6, E=7, cap=3, fp8=True, name="capacity_overflow"),
    dict(T=50, H=2304, k=4, E=16, cap=64, fp8=False, name="capacity_bf16_no_overflow"),
    # the largest hidden size (65536 channels, 512 blocks per row): bf16, FP8
    # with capacity overflow, UE8M0 through the one-kernel form, and a batch
    # that takes the persistent combine (128 chunks per row)
    dict(T=20, H=65536, k=2, E=8, cap=0, fp8=False, name="max_hidden_bf16"),
    dict(T=20, H=65536, k=2, E=8, cap=4, fp8=1, name="max_hidden_fp8_capacity"),
    dict(T=300, H=65536, k=4, E=64, cap=0, fp8=2, name="max_hidden_ue8m0"),
    dict(T=64, H=65536, k=2, E=8, cap=0, fp8=False, name="max_hidden_persistent_combine"),
    # routing tables around the size where the layout leaves the small-table
    # kernel (8192 entries): just above it the one-kernel whole-table layout
    # (64 experts), or the histogram and ranking kernels where its LDS tables
    # do not fit (1000 experts); and a large two-pass table
    dict(T=1024, H=128, k=8, E=64, cap=0, fp8=True, name="layout_single_pass_largest"),
    dict(T=1025, H=136, k=8, E=64, cap=0, fp8=False, name="layout_whole_table_smallest"),
    dict(T=1171, H=128, k=7, E=1000, cap=0, fp8=False, name="layout_two_pass_many_experts"),
    dict(T=40000, H=128, k=8, E=256, cap=1500, fp8=True, name="layout_two_pass_capacity"),
    # the largest table the one-kernel layout + dispatch takes (8192 entries),
    # and few experts (many equal ids, many queries per workgroup)
    dict(T=1024, H=256, k=8, E=16, cap=0, fp8=False, name="fused_largest_table"),
    dict(T=2730, H=128, k=3, E=2, cap=3000, fp8=True, name="fused_two_experts_capacity"),
    dict(T=3, H=8, k=5, E=1000, cap=2, fp8=False, name="fused_few_tokens_many_experts"),
    # ep_layout_dispatch above 8192 entries with bf16 rows or FP8 and k >= 8:
    # histogram tables, then a dispatch kernel that ranks each token's
    # entries itself.  Tokens straddling layout blocks (k does not divide the
    # block size), more entries than 16-lane rows in a workgroup, blocks wider
    # than one pass over the ids, rows of two column tiles, few tokens with a
    # wide k, one expert, capacity with overflow (shapes outside the
    # one-launch form below: fewer than one chunk per wave, or T*k > 32768).
    dict(T=3000, H=256, k=5, E=50, cap=0, fp8=False, name="ranked_odd_k_straddle"),
    dict(T=1024, H=1024, k=16, E=128, cap=0, fp8=False, name="ranked_k16_two_rounds"),
    dict(T=4500, H=3584, k=8, E=96, cap=0, fp8=False, name="ranked_wide_blocks_bf16"),
    dict(T=4100, H=9216, k=8, E=64, cap=0, fp8=False, name="ranked_two_tiles_bf16"),
    dict(T=600, H=1024, k=16, E=64, cap=0, fp8=True, name="ranked_few_tokens_k16"),
    dict(T=40000, H=128, k=1, E=1, cap=0, fp8=False, name="ranked_one_expert"),
    dict(T=1800, H=512, k=8, E=20, cap=700, fp8=True, name="ranked_capacity_overflow"),
    dict(T=2300, H=256, k=6, E=20, cap=700, fp8=False, name="ranked_capacity_overflow_bf16_k6"),
    # FP8 with k < 8 above 8192 entries: the layout kernels, then dispatch
    dict(T=2300, H=512, k=6, E=20, cap=700, fp8=True, name="fp8_k6_capacity_overflow"),
    # ep_layout_dispatch in one launch of one workgroup per CU (bf16 rows,
    # 8192 < T*k <= 32768, at least one 64-piece chunk per wave): tokens
    # straddling two workgroups and a partly filled last workgroup (5 chunks
    # per row, 32 per workgroup), capacity with overflow, an odd k (slot rows
    # padded to 4), k above 8 (the generic store loop), the most experts,
    # the largest table with k = 32, one expert, ragged rows
    dict(T=1500, H=2560, k=8, E=64, cap=0, fp8=False, name="persistent_dispatch_straddle"),
    dict(T=2048, H=2048, k=8, E=64, cap=200, fp8=False, name="persistent_dispatch_capacity_overflow"),
    dict(T=2400, H=1800, k=5, E=37, cap=0, fp8=False, name="persistent_dispatch_odd_k_ragged_row"),
    dict(T=1300, H=3072, k=12, E=256, cap=0, fp8=False, name="persistent_dispatch_k12"),
    dict(T=1700, H=2048, k=8, E=1024, cap=0, fp8=False, name="persistent_dispatch_max_experts"),
    dict(T=1024, H=4096, k=32, E=128, cap=0, fp8=False, name="persistent_dispatch_k32_largest_table"),
    dict(T=12000, H=512, k=2, E=1, cap=0, fp8=False, name="persistent_dispatch_one_expert"),
    # FP8 rows at prefill sizes (8192 < T*k <= 32768 with at least one
    # 64-piece chunk per wave: the one-launch form; else the multi-kernel
    # forms): rows of 15 blocks (a last chunk of 3 blocks), UE8M0 scales with
    # capacity overflow, 49152 entries over 48 experts (the one-kernel
    # layout, then the dispatch kernel)
    dict(T=2000, H=1920, k=8, E=64, cap=0, fp8=1, name="prefill_fp8_ragged_blocks"),
    dict(T=3000, H=1024, k=6, E=32, cap=400, fp8=2, name="prefill_ue8m0_capacity_overflow"),
    dict(T=8192, H=4096, k=6, E=48, cap=0, fp8=1, name="prefill_fp8_k6_48_experts"),
    # the one-launch FP8 form: tokens straddling two workgroups, an odd k with
    # a last chunk of 2 blocks, k above 8 (the generic store loop) with UE8M0
    # scales, k = 32, the most experts with capacity overflow, a table that
    # fills the second half of the table registers only in part, a row of
    # one block
    dict(T=1500, H=2560, k=8, E=64, cap=0, fp8=1, name="persistent_fp8_straddle"),
    dict(T=2400, H=1792, k=5, E=37, cap=0, fp8=1, name="persistent_fp8_odd_k_ragged_chunk"),
    dict(T=1300, H=3072, k=12, E=256, cap=0, fp8=2, name="persistent_ue8m0_k12"),
    dict(T=1024, H=4096, k=32, E=128, cap=0, fp8=1, name="persistent_fp8_k32"),
    dict(T=1700, H=2048, k=8, E=1024, cap=12, fp8=2, name="persistent_ue8m0_max_experts_capacity"),
    dict(T=5000, H=1024, k=8, E=160, cap=0, fp8=1, name="persistent_fp8_table_second_half_partial"),
    dict(T=12000, H=2816, k=1, E=3, cap=0, fp8=1, name="persistent_fp8_k1_22_blocks"),
    # the persistent combine at 14 chunks per wave: a partly filled last
    # workgroup with ragged rows (875 pieces per row: 13 full chunks and one
    # of 43), and k = 1 with capacity drops (entries without a slot)
    dict(T=4000, H=7000, k=5, E=64, cap=0, fp8=False, name="persistent_combine_ragged_partial"),
    dict(T=4096, H=7168, k=1, E=16, cap=300, fp8=False, name="persistent_combine_k1_capacity"),
    # the persistent combine (at least one 64-piece chunk per wave of one
    # workgroup per CU) with k > 8: entries in batches of 8
    dict(T=2200, H=1536, k=16, E=64, cap=0, fp8=False, name="persistent_combine_k16"),
    # two launches of unequal token ranges (7501 + 7500 tokens), ragged
    # chunks (225 pieces per row: 3 full chunks and one of 33)
    dict(T=15001, H=1800, k=2, E=16, cap=0, fp8=False, name="persistent_combine_two_launches"),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("spec", EDGE, ids=[e["name"] for e in EDGE])
def test_edge_shapes(spec, fused):
    spec = dict(spec)
    name = spec.pop("name")
    c = _random_case(**spec, seed=zlib.crc32(name.encode()) % 1000, name=name)
    check_case(c, run_gpu(c, fused=fused))


def _random_shapes(n, seed=2026):
    """Seeded random problem shapes across every launch rule of the library:
    one-launch and two-launch layout+dispatch, FP8 with small and large k,
    capacity with and without overflow, decode-sized and prefill-sized
    combines (persistent and per-token, ragged rows), all three payload
    modes.  Even entries are decode-sized, odd ones prefill-sized (more than
    8192 routing entries); receive buffers stay under about 150 MB."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        large = len(out) % 2 == 1
        fp8 = int(rng.integers(0, 3))
        if large:
            T = int(rng.integers(1100, 20000))
            k = int(rng.choice([5, 6, 8, 8, 9, 16]))
        else:
            T = int(np.exp(rng.uniform(0, np.log(1000))))
            k = int(rng.choice([1, 2, 3, 5, 6, 8, 8, 16]))
        E = int(rng.choice([1, 3, 16, 64, 100, 256, 1000]))
        cap = 0 if rng.random() < 0.6 else int(rng.integers(1, max(2, 2 * T * k // E + 2)))
        R = T * k if cap == 0 else E * cap
        unit = 128 if fp8 else 8
        hmax = int(min(6144, 150e6 / (2 * R))) // unit * unit
        if hmax < unit or (large and T * k <= 8192):
            continue
        H = int(rng.integers(1, hmax // unit + 1)) * unit
        out.append(dict(T=T, H=H, k=k, E=E, cap=cap, fp8=fp8,
                        name=f"r{len(out)}_T{T}_H{H}_k{k}_E{E}_c{cap}_m{fp8}"))
    return out


RANDOM_SHAPES = _random_shapes(24)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("spec", RANDOM_SHAPES, ids=[e["name"] for e in RANDOM_SHAPES])
def test_random_shapes(spec, fused):
    spec = dict(spec)
    name = spec.pop("name")
    c = _random_case(**spec, seed=zlib.crc32(name.encode()) % 1000, name=name)
    check_case(c, run_gpu(c, fused=fused))


def _bench_rules():
    """bench.py's mirror of the library's launch rules."""
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py")
    spec = importlib.util.spec_from_file_location("bench_rules", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _random_one_launch_shapes(n, seed=2027, ncu=256):
    """Seeded random shapes that ep_layout_dispatch takes in one launch of one
    workgroup per CU (8192 < T*k <= 32768, T*k a multiple of 4, between 1
    and 14 (bf16) or 16 (FP8) chunks per wave): bf16 and both FP8 scale
    formats, k from 1 to 32, 1 to 1024 experts, with and without capacity,
    rows of any length the rule allows (ragged last chunks included).  The
    launch form of each is checked against bench.py's mirror of the rules,
    which the kernel traces confirm on the five workloads."""
    from types import SimpleNamespace
    rules = _bench_rules()
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        fp8 = int(rng.integers(0, 3))
        k = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 8, 8, 12, 16, 32]))
        n_ent = int(rng.integers(8193, 32769)) // 4 * 4
        if n_ent % k:
            continue
        T = n_ent // k
        E = int(rng.choice([1, 7, 32, 64, 100, 256, 1024]))
        cap = 0 if rng.random() < 0.7 else int(rng.integers(1, max(2, 2 * T * k // E + 2)))
        unit = 128 if fp8 else 8
        H = int(rng.integers(1, 7168 // unit + 1)) * unit
        R = T * k if cap == 0 else E * cap
        wl = SimpleNamespace(T=T, H=H, k=k, E=E, cap=cap, fp8=bool(fp8), cid=0)
        if R * H * 2 > 150e6 or not rules.persistent_launch(wl, ncu):
            continue
        out.append(dict(T=T, H=H, k=k, E=E, cap=cap, fp8=fp8,
                        name=f"o{len(out)}_T{T}_H{H}_k{k}_E{E}_c{cap}_m{fp8}"))
    return out


ONE_LAUNCH_SHAPES = _random_one_launch_shapes(12)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("spec", ONE_LAUNCH_SHAPES, ids=[e["name"] for e in ONE_LAUNCH_SHAPES])
def test_random_one_launch_shapes(spec, fused):
    spec = dict(spec)
    name = spec.pop("name")
    c = _random_case(**spec, seed=zlib.crc32(name.encode()) % 1000, name=name)
    check_case(c, run_gpu(c, fused=fused))


def test_duplicate_and_invalid_ids():
    rng = np.random.default_rng(9)
    T, k, E = 700, 4, 12
    ids = rng.integers(0, E, size=(T, k))
    ids[::7, 1] = ids[::7, 0]                     # duplicates inside a row
    ids[::11, 2] = -1                              # below range
    ids[::13, 3] = E                               # one past the end
    ids[::17, 0] = 1 << 30                         # far out of range
    ids[5] = 3                                     # all k entries to one expert
    for cap, fp8, fused in ((0, False, False), (0, True, False), (40, True, False),
                            (0, False, True), (40, True, True)):
        c = _random_case(T, 256, k, E, cap, fp8, seed=cap, ids=ids, name=f"dup_invalid_cap{cap}")
        got = run_gpu(c, fused=fused)
        check_case(c, got)
        assert got["status"][0] == int(((ids < 0) | (ids >= E)).sum())


def test_duplicate_and_invalid_ids_large_table():
    """The same id mix above 8192 entries (ep_layout: the one-kernel
    whole-table layout; ep_layout_dispatch: ranking inside the dispatch
    kernel at H = 256, one launch of one workgroup per CU at H = 640, bf16 or
    FP8 rows), with and without capacity,
    at a size the persistent combine takes (tokens with no valid entry
    included)."""
    rng = np.random.default_rng(10)
    T, k, E = 2100, 8, 40
    ids = rng.integers(0, E, size=(T, k))
    ids[::7, 1] = ids[::7, 0]
    ids[::11, 2] = -1
    ids[::13, 3] = E
    ids[::17, 0] = 1 << 30
    ids[100:140] = 5                               # a run of one expert across tokens
    ids[200:203] = -1                              # tokens without any valid entry
    for H, cap, fp8, fused in ((640, 0, False, False), (640, 0, False, True),
                               (640, 300, False, True), (256, 0, False, True),
                               (640, 300, True, False), (640, 300, True, True),
                               (640, 0, 2, True)):
        c = _random_case(T, H, k, E, cap, fp8, seed=cap + 1, ids=ids,
                         name=f"dup_invalid_large_H{H}_cap{cap}_fp8{int(fp8)}")
        got = run_gpu(c, fused=fused)
        check_case(c, got)
        assert got["status"][0] == int(((ids < 0) | (ids >= E)).sum())


CAP_SMALL = [
    # (T, H, k, E, cap, fp8, hot, name): fixed capacity with at most 1024
    # routing entries (decode batches): the one-kernel layout + dispatch
    (128, 7168, 8, 256, 128, 1, False, "decode_shape"),
    (100, 1024, 8, 12, 40, 1, True, "overflow_dup_invalid"),
    (100, 1024, 8, 12, 40, 2, True, "overflow_dup_invalid_ue8m0"),
    (100, 1024, 8, 12, 40, 0, True, "overflow_dup_invalid_bf16"),
    (32, 4096, 32, 64, 12, 1, True, "k32_two_tokens_per_workgroup"),
    (37, 2304, 7, 9, 20, 1, False, "table_259_entries_odd_k"),
    (1, 128, 1, 1, 1, 1, False, "single_entry"),
    (3, 8, 5, 1000, 2, 0, False, "few_tokens_many_experts"),
    (170, 1920, 6, 33, 17, 2, True, "ragged_blocks_1020_entries"),
    (128, 7168, 8, 256, 3, 1, True, "decode_shape_tiny_capacity"),
]


@pytest.mark.parametrize("spec", CAP_SMALL, ids=[c[-1] for c in CAP_SMALL])
def test_capacity_small_tables(spec):
    """Small routing tables with a fixed capacity through ep_layout_dispatch
    (one kernel: workgroups that are not workgroup 0 count only the experts
    whose empty rows they mark) and through ep_layout + ep_dispatch: every
    layout array, receive row, scale and combine output against the oracle.  "hot": duplicate ids inside rows, ids outside
    [0, E) (-1, E, 2^30), a run of one expert across tokens and one token
    whose k entries are all one expert -- with capacities that drop entries."""
    T, H, k, E, cap, fp8, hot, name = spec
    rng = np.random.default_rng(zlib.crc32(name.encode()) % 1000)
    ids = rng.integers(0, E, size=(T, k))
    if hot:
        ids[::7, min(1, k - 1)] = ids[::7, 0]
        ids[::11, min(2, k - 1)] = -1
        ids[::13, min(3, k - 1)] = E
        ids[::17, 0] = 1 << 30
        ids[T // 3:T // 3 + max(1, T // 10)] = E // 2
        ids[T - 1] = 0
    for fused in (True, False):
        c = _random_case(T, H, k, E, cap, fp8, seed=cap + T, ids=ids, name=f"cap_small_{name}")
        got = run_gpu(c, fused=fused)
        check_case(c, got)
        assert got["status"][0] == int(((ids < 0) | (ids >= E)).sum())


def test_whole_table_layout_ids_and_tails():
    """The one-kernel layout of mid-size tables (8192 < T*k <= 65536, at
    least 32 experts: every workgroup reads the whole table) through
    ep_layout: duplicate ids in a row, ids outside [0, E), a run of one
    expert across tokens, tokens without a valid entry, with and without
    capacity (overflow included), tables whose length is not a multiple of 4
    (the last ids are read one by one), fewer than 128 experts (the
    histograms counted in 8 copies; a third of the ids on one hot expert in
    the skewed cases), and the same id mix on a larger table that takes the
    two-kernel layout."""
    rng = np.random.default_rng(12)
    for T, k, E, cap, hot in ((3000, 8, 160, 0, False), (3000, 8, 160, 100, False),
                              (3001, 7, 130, 0, False), (4681, 14, 256, 0, False),
                              (3001, 7, 64, 0, True), (3000, 8, 32, 300, True),
                              (6000, 6, 127, 0, False), (8000, 8, 40, 0, True),
                              (16384, 8, 256, 600, False)):
        ids = rng.integers(0, E, size=(T, k))
        if hot:
            ids[rng.random((T, k)) < 0.33] = E // 3
        ids[::7, 1] = ids[::7, 0]
        ids[::11, 2] = -1
        ids[::13, 3] = E
        ids[::17, 0] = 1 << 30
        ids[100:140] = 5
        ids[200:203] = -1
        H = 128 if T * k > 65536 else 256
        c = _random_case(T, H, k, E, cap, False, seed=T + cap + E, ids=ids,
                         name=f"whole_layout_T{T}_k{k}_E{E}_cap{cap}")
        got = run_gpu(c)
        check_case(c, got)
        assert got["status"][0] == int(((ids < 0) | (ids >= E)).sum())


def _fp8_special_xf(rng, T, H):
    """fp32 rows (T >= 6) whose first six rows hold the special FP8 cases."""
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf[0] = 0.0                                            # whole row zero
    xf[1, 128:256] = 0.0                                   # one zero block
    xf[1, 256:384] = -0.0                                  # negative-zero block
    sub = (np.arange(1, 129, dtype=np.uint32) << 16).view(np.float32)
    xf[2, :128] = sub * np.where(np.arange(128) % 2, -1, 1)  # bf16 subnormals only
    xf[3, :128] = -(2.0 ** -40) * rng.random(128)            # tiny negatives
    xf[3, 0] = -3.0e38                                       # dominated block: quotients underflow
    xf[4] *= 100.0                                           # outlier row
    tab = oracle.e4m3_decode_table()
    pos = tab[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    for b in range(H // 128):                                # block max 448 * 2^m, midpoints inside
        m = int(rng.integers(-8, 8))
        xf[5, 128 * b: 128 * b + 126] = rng.choice(mids, 126) * 2.0 ** m * rng.choice([-1, 1], 126)
        xf[5, 128 * b + 126] = 448.0 * 2.0 ** m
        xf[5, 128 * b + 127] = -(2.0 ** (m - 10))            # exact tie with zero
    return xf


def test_fp8_special_rows():
    """All-zero rows and blocks (scale 0), blocks of bf16 subnormals only,
    negative zeros and tiny negatives, huge/tiny mixes whose quotients
    underflow, x100 outliers, and quotients next to E4M3 rounding midpoints."""
    rng = np.random.default_rng(31)
    T, H, E, k = 12, 1024, 4, 2
    x = workloads.to_bf16_bits(_fp8_special_xf(rng, T, H))
    ids = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E], axis=1).astype(np.int32)
    w = np.full((T, k), 0.5, np.float32)
    eo = workloads.to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    for cap in (0, 8):
        c = Case(T, H, k, E, cap, True, x, ids, w, eo if cap == 0 else
                 workloads.to_bf16_bits(rng.standard_normal((E * cap, H)).astype(np.float32)),
                 name=f"fp8_special_cap{cap}")
        c.nan_unused_rows()
        check_case(c, run_gpu(c))
        check_case(c, run_gpu(c, fused=True))


def test_fp8_special_rows_prefill():
    """The same special rows at a prefill size (2100 tokens, k = 8: the
    one-launch layout + dispatch of FP8 rows), with fp32 and UE8M0 scales,
    with and without capacity."""
    rng = np.random.default_rng(32)
    T, H, E, k = 2100, 1024, 40, 8
    x = workloads.to_bf16_bits(_fp8_special_xf(rng, T, H))
    for mode, cap in ((1, 0), (2, 0), (1, 500), (2, 500)):
        c = _random_case(T, H, k, E, cap, mode, seed=mode + cap, name=f"fp8_special_prefill_m{mode}_cap{cap}")
        c.x = x
        check_case(c, run_gpu(c, fused=True))


def _near_midpoint_rows(T, H, seed, tries=150):
    """bf16 rows whose 128-channel blocks have a non-power-of-two scale and
    many channels whose quotient by it lies within 8 fp32 ulps of a midpoint
    between two E4M3 values: the channels the dispatch kernel must divide
    instead of multiplying by the reciprocal.  (With bf16 inputs a quotient
    is either that close to a midpoint, through the rounding of the scale, or
    about 2^11 ulps or more away, so these are the cases that matter.)  For
    each block the block maximum is picked, among `tries` random bf16
    values, as the one giving the most such quotients."""
    rng = np.random.default_rng(seed)
    pos = (np.arange(0x0080, 0x7F80, dtype=np.uint32) << 16).view(np.float32)  # normal bf16 > 0
    pos = pos[pos < 512.0]
    xf = np.empty((T, H), np.float32)
    for t in range(T):
        for b in range(H // 128):
            best = None
            for amax in rng.choice(pos[pos > 0.25], tries):
                amax = np.float32(amax)
                scale = np.float32(amax / np.float32(448.0))
                if scale.view(np.uint32) & 0x7FFFFF == 0:
                    continue  # power-of-two scale: exact quotients
                cand = pos[pos < amax]
                q = (cand / scale).astype(np.float32)
                d = np.abs((q.view(np.uint32) & 0xFFFFF).astype(np.int64) - 0x80000)
                near = cand[(d <= 8) & (q >= 2.0 ** -6)]
                if best is None or near.size > best[1].size:
                    best = (amax, near, cand)
            amax, near, cand = best
            blk = np.concatenate([near, rng.choice(cand, 128)])[:128]
            blk = blk * rng.choice(np.float32([-1, 1]), 128)
            blk[int(rng.integers(128))] = amax
            xf[t, 128 * b:128 * (b + 1)] = blk
    return workloads.to_bf16_bits(xf)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_fp8_near_midpoint_quotients(fused):
    T, H, E, k = 8, 1024, 8, 2
    x = _near_midpoint_rows(T, H, seed=77)
    rng = np.random.default_rng(78)
    ids = np.stack([np.arange(T) % E, (np.arange(T) + 3) % E], axis=1).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    eo = workloads.to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    c = Case(T, H, k, E, 0, True, x, ids, w, eo, name="fp8_near_midpoint")
    check_case(c, run_gpu(c, fused=fused))


@pytest.mark.parametrize("mode", [1, 2], ids=["fp32_scales", "ue8m0"])
def test_fp8_special_rows_prefill_batch(mode):
    """The special FP8 rows and near-midpoint rows inside a prefill-sized
    batch (2048 tokens of 1024 channels, k = 5: above the small-table
    forms)."""
    rng = np.random.default_rng(41)
    T, H, E, k = 2048, 1024, 16, 5
    xf = _fp8_special_xf(rng, T, H)
    x = workloads.to_bf16_bits(xf)
    x[6:14] = _near_midpoint_rows(8, H, seed=79)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    eo = workloads.to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    c = Case(T, H, k, E, 0, mode, x, ids, w, eo, name=f"fp8_special_prefill_m{mode}")
    check_case(c, run_gpu(c, fused=True))


@pytest.mark.parametrize("over", [dict(cid=3, T=1024, hot_experts=16, hot_ratio=3.0),
                                  dict(cid=3, T=2048, hot_experts=16, hot_ratio=3.0),
                                  dict(cid=4, T=2048, zipf_s=1.6),
                                  dict(cid=4, T=2048, zipf_s=0.8)],
                         ids=["hot3x", "hot3x_one_launch", "zipf1.6", "zipf0.8"])
def test_skew_sweep_variants(over):
    """The routing-skew sweep's extreme variants, at reduced token counts,
    through the separate calls and ep_layout_dispatch (at 2048 prefill tokens
    its one-launch form: hot experts put many LDS histogram atomics of a wave
    on one address)."""
    over = dict(over)
    c = Case.from_workload(workloads.make(over.pop("cid"), **over))
    check_case(c, run_gpu(c))
    check_case(c, run_gpu(c, fused=True))


# ---------------------------------------------------------------------------
# UE8M0 scales (use_fp8 = 2)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("cid", [2, 4])
def test_ue8m0_workloads(cid, fused):
    """The decode and skewed workloads with UE8M0 block scales."""
    wl = workloads.make(cid)
    c = Case.from_workload(wl)
    c.fp8 = 2
    c.name = wl.name + "_ue8m0"
    check_case(c, run_gpu(c, fused=fused))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_ue8m0_special_blocks(fused):
    """Block maxima at exactly 448*2^j and one bf16 step either side of it,
    bf16-subnormal blocks (exponent clamped at -127), zero and -0 blocks,
    x100 outliers, with ragged tails and capacity overflow."""
    rng = np.random.default_rng(41)
    T, H, E, k = 40, 896, 6, 3
    xf = (rng.standard_normal((T, H)) * 2.0 ** rng.integers(-40, 40, size=(T, 1))).astype(np.float32)
    for t in range(T):
        for b in range(H // 128):
            sl = slice(128 * b, 128 * b + 128)
            kind = (t * 7 + b) % 7
            j = int(rng.integers(-110, 110))
            if kind in (0, 1, 2):
                base = np.float32(448.0 * 2.0 ** j).view(np.uint32)
                amax = (base + np.uint32((kind == 1) << 16) - np.uint32((kind == 2) << 16)).view(np.float32)
                xf[t, sl] = np.clip(xf[t, sl], -amax * 0.99, amax * 0.99)
                xf[t, 128 * b + int(rng.integers(128))] = amax * rng.choice([-1, 1])
            elif kind == 3:
                xf[t, sl] = ((rng.integers(1, 128, 128).astype(np.uint32) << 16).view(np.float32)
                             * rng.choice(np.float32([-1, 1]), 128))
            elif kind == 4:
                xf[t, sl] = -0.0 if t % 2 else 0.0
            elif kind == 5:
                xf[t, sl] *= 100.0
    x = workloads.to_bf16_bits(xf)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    for cap in (0, 9):
        R = T * k if cap == 0 else E * cap
        eo = workloads.to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
        c = Case(T, H, k, E, cap, 2, x, ids, w, eo, name=f"ue8m0_special_cap{cap}")
        c.nan_unused_rows()
        check_case(c, run_gpu(c, fused=fused))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_non_default_stream(fused):
    s = torch.cuda.Stream()
    c = _random_case(333, 512, 4, 16, 0, True, seed=5, name="side_stream")
    check_case(c, run_gpu(c, stream=s, fused=fused))
    # a prefill-sized bf16 batch (fused: the one-launch form; the persistent
    # combine either way)
    c = _random_case(2048, 2048, 8, 64, 0, False, seed=6, name="side_stream_prefill")
    check_case(c, run_gpu(c, stream=s, fused=fused))


def test_fused_equals_separate_bitwise():
    """ep_layout_dispatch writes exactly what ep_layout + ep_dispatch write,
    receive rows and scales included, on the tiny and the decode workloads
    (small-table kernel), the prefill workload (one launch of one workgroup
    per CU) and the skewed workload (FP8 with k = 6: the one-kernel layout,
    then the dispatch kernel)."""
    for cid in (1, 2, 3, 4):
        c = Case.from_workload(workloads.make(cid))
        a = run_gpu(c)
        b = run_gpu(c, fused=True)
        for n in a:
            if a[n] is not None:  # bit patterns: untouched rows hold NaN fill
                assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), (cid, n)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_deterministic_reruns(cid, fused):
    """Two runs of each workload give identical bits, every output included.
    The one-launch prefill kernel hands chunks to whichever wave asks first,
    so which wave stores a row differs from run to run; the bytes must not."""
    c = _large_prefill() if cid == 5 else Case.from_workload(workloads.make(cid))
    a = run_gpu(c, fused=fused)
    b = run_gpu(c, fused=fused)
    for n in a:
        if a[n] is not None:
            assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), (cid, n)


def test_identity_round_trip():
    """dispatch (bf16) -> identity experts -> combine with weights summing to 1
    returns x bit for bit, on the GPU alone."""
    wl = workloads.make(3, T=512)
    prob = ep.Problem(wl.T, wl.H, wl.k, wl.E, 0, 0)
    lay = ep.Layout.empty(prob, DEV)
    ws = ep.alloc_workspace(prob, DEV)
    recv_x, _ = ep.alloc_recv(prob, DEV)
    y = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    idx = torch.from_numpy(wl.topk_idx).to(DEV)
    w = torch.from_numpy(wl.topk_weights).to(DEV)
    x = dev_bf16(wl.x)
    ep.ep_layout(prob, idx, lay, ws)
    ep.ep_dispatch(prob, x, lay, recv_x)
    ep.ep_combine(prob, recv_x, lay, w, y)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(y), wl.x)


# ---------------------------------------------------------------------------
# the E4M3FN encoder, every binary32 input
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("sign", [0, 0x80000000], ids=["positive", "negative"])
def test_e4m3_encoder_exhaustive(sign):
    """Every finite binary32: the device encoder equals torch's CPU
    float8_e4m3fn conversion where that conversion is defined to round
    (|v| <= 464; torch == oracle there, pinned on the CPU), and 0x7E / 0xFE
    (saturation) above; plus the oracle itself on a strided subset."""
    chunk = 1 << 27
    lim464 = int(np.array(464.0, np.float32).view(np.uint32))
    inf = 0x7F800000
    out = torch.empty(chunk, dtype=torch.uint8, device=DEV)
    for lo in range(0, inf, chunk):
        hi = min(inf, lo + chunk)
        bits = (np.arange(lo, hi, dtype=np.uint64).astype(np.uint32) | np.uint32(sign))
        v = bits.view(np.float32)
        vin = torch.from_numpy(v).to(DEV)
        ep.ep_e4m3_encode(vin, out[: hi - lo])
        got = out[: hi - lo].cpu().numpy()
        mag = bits & 0x7FFFFFFF
        inr = mag <= lim464
        want = torch.from_numpy(v[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got[inr], want), hex(lo | sign)
        assert (got[~inr] == (0xFE if sign else 0x7E)).all(), hex(lo | sign)
        sub = slice(0, hi - lo, 4099)
        assert np.array_equal(got[sub], oracle.e4m3_encode(v[sub])), hex(lo | sign)
