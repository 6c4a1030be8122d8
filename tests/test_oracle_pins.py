"""Pins for the CPU oracle: each check compares the oracle with something other
than itself -- brute force on tiny inputs, library routines (numpy's stable
sort and cumulative sum, torch's bf16 and float8_e4m3fn conversions), closed
forms of the OCP E4M3FN format, exact arithmetic, and invariants of the method.

A planted mistake anywhere in the oracle (a dropped term, a wrong sign or
index, an off-by-one in the scan, ties rounded the wrong way, an exchanged
operand) fails at least one of these; see test_planted_mistakes_are_caught.
"""
import itertools
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads

NTHREADS = max(1, min(8, len(os.sched_getaffinity(0))))


# ---------------------------------------------------------------------------
# layout
# ---------------------------------------------------------------------------

def brute_layout(idx, E, cap):
    """Closed-form definition of every layout output, computed entry by entry.

    For entry i with valid expert e:
      rank(i)  = #{i' < i : idx[i'] == e}
      contiguous slot = #{i' : 0 <= idx[i'] < e} + rank(i)
      capacity slot   = e*cap + rank(i) if rank(i) < cap else -1
    """
    flat = [int(v) for v in np.asarray(idx).ravel()]
    n = len(flat)
    T, k = np.asarray(idx).shape
    valid = [0 <= e < E for e in flat]
    count = [sum(1 for e in flat if e == x) for x in range(E)]
    offset = [sum(1 for e in flat if 0 <= e < x) for x in range(E + 1)]
    R = n if cap == 0 else E * cap
    slot_of = []
    dropped = 0
    for i, e in enumerate(flat):
        if not valid[i]:
            slot_of.append(-1)
            continue
        rank = sum(1 for ip in range(i) if flat[ip] == e)
        if cap == 0:
            slot_of.append(offset[e] + rank)
        elif rank < cap:
            slot_of.append(e * cap + rank)
        else:
            slot_of.append(-1)
            dropped += 1
    src = [-1] * R
    for i, s in enumerate(slot_of):
        if s >= 0:
            src[s] = i
    return dict(count=count, offset=offset, slot_of=np.array(slot_of).reshape(T, k).tolist(),
                src_of_slot=src, status=[n - sum(valid), dropped])


def _as_lists(lay):
    return {k: np.asarray(v).tolist() for k, v in lay.items()}


@pytest.mark.parametrize("T,k,E", [(0, 1, 1), (1, 1, 1), (1, 2, 2), (2, 1, 3), (2, 2, 2),
                                   (3, 1, 2), (3, 2, 3), (2, 3, 2)])
def test_layout_exhaustive_tiny(T, k, E):
    """Every routing table with ids in {-1, .., E} (both invalid sides), every capacity."""
    ids = list(range(-1, E + 1))
    for cap in (0, 1, 2):
        for combo in itertools.product(ids, repeat=T * k):
            idx = np.array(combo, np.int32).reshape(T, k)
            got = _as_lists(oracle.layout(idx, E, cap))
            want = brute_layout(idx, E, cap)
            assert got == want, (idx.tolist(), cap)


def test_layout_fuzz_vs_stable_sort():
    """Contiguous layout == numpy stable argsort by expert id; count == bincount;
    offset == cumulative sum (library routines)."""
    rng = np.random.default_rng(123)
    for _ in range(2000):
        T = int(rng.integers(0, 65))
        k = int(rng.integers(1, 5))
        E = int(rng.integers(1, 17))
        idx = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)
        lay = oracle.layout(idx, E, 0)
        flat = idx.ravel()
        valid = (flat >= 0) & (flat < E)
        np.testing.assert_array_equal(lay["count"], np.bincount(flat[valid], minlength=E))
        np.testing.assert_array_equal(lay["offset"], np.concatenate([[0], np.cumsum(lay["count"])]))
        order = np.argsort(np.where(valid, flat, E), kind="stable")[: valid.sum()]
        np.testing.assert_array_equal(lay["src_of_slot"][: valid.sum()], order)
        assert lay["status"].tolist() == [int((~valid).sum()), 0]


def test_layout_capacity_fuzz_vs_brute():
    rng = np.random.default_rng(7)
    for _ in range(300):
        T = int(rng.integers(0, 24))
        k = int(rng.integers(1, 4))
        E = int(rng.integers(1, 6))
        cap = int(rng.integers(1, 6))
        idx = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)
        assert _as_lists(oracle.layout(idx, E, cap)) == brute_layout(idx, E, cap)


def check_layout_invariants(idx, E, cap, lay):
    T, k = idx.shape
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < E)
    count, offset = lay["count"], lay["offset"]
    slot_of, src = lay["slot_of"].ravel(), lay["src_of_slot"]
    assert count.sum() == valid.sum()
    assert offset[E] == valid.sum()
    placed = slot_of >= 0
    # each placed entry owns exactly one row and that row points back at it
    assert len(np.unique(slot_of[placed])) == placed.sum()
    np.testing.assert_array_equal(src[slot_of[placed]], np.nonzero(placed)[0])
    # every row that is claimed is claimed by exactly the entry it names
    claimed = src >= 0
    assert claimed.sum() == placed.sum()
    np.testing.assert_array_equal(slot_of[src[claimed]], np.nonzero(claimed)[0])
    # inside each expert's segment the source entry strictly increases
    for e in range(E):
        if cap == 0:
            seg = src[offset[e]:offset[e + 1]]
        else:
            seg = src[e * cap: e * cap + min(count[e], cap)]
            assert (src[e * cap + min(count[e], cap): (e + 1) * cap] == -1).all()
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_layout_invariants_on_workloads(cid):
    wl = workloads.make(cid)
    lay = oracle.layout(wl.topk_idx, wl.E, wl.cap)
    assert lay["count"].sum() == wl.T * wl.k          # all ids valid, nothing dropped
    assert lay["status"].tolist() == [0, 0]
    check_layout_invariants(wl.topk_idx, wl.E, wl.cap, lay)


def test_layout_capacity_overflow_drops_later_tokens():
    idx = np.array([[0, 1], [0, 1], [0, 2], [1, 0]], np.int32)
    lay = oracle.layout(idx, 3, 2)
    # expert 0 appears at entries 0, 2, 4, 7 -> the 3rd and 4th are dropped
    assert lay["slot_of"].tolist() == [[0, 2], [1, 3], [-1, 4], [-1, -1]]
    assert lay["count"].tolist() == [4, 3, 1]         # never clamped
    assert lay["status"].tolist() == [0, 3]
    assert lay["src_of_slot"].tolist() == [0, 2, 1, 3, 5, -1]


# ---------------------------------------------------------------------------
# E4M3FN codec
# ---------------------------------------------------------------------------

# Named values of the OCP 8-bit floating point specification (OFP8 v1.0),
# E4M3 format: exponent bias 7, largest finite 448 = S.1111.110, smallest
# normal 2^-6 = S.0001.000, smallest subnormal 2^-9 = S.0000.001,
# NaN = S.1111.111, no infinities.
NAMED_DECODE = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
                0x38: 1.0, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0,
                0x80: -0.0}


def test_e4m3_decode_named_and_structure():
    tab = oracle.e4m3_decode_table()
    for c, v in NAMED_DECODE.items():
        assert tab[c] == v and math.copysign(1, tab[c]) == math.copysign(1, v), hex(c)
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    pos = tab[:0x7F]
    assert (np.diff(pos) > 0).all()                   # strictly increasing codes
    np.testing.assert_array_equal(tab[0x80:0xFF], -pos)  # sign symmetric
    # subnormals and the first binade are evenly spaced by 2^-9; every later
    # binade of 8 codes doubles the spacing
    assert np.all(np.diff(pos[:16]) == 2.0 ** -9)
    for b in range(1, 15):
        step = np.diff(pos[8 * b: 8 * b + 8])
        if len(step):
            assert np.all(step == 2.0 ** (b - 10)), b


# (input, expected code): ties go to the code whose last mantissa bit is 0.
NAMED_ENCODE = [
    (0.0, 0x00), (-0.0, 0x80), (2.0 ** -10, 0x00), (-(2.0 ** -10), 0x80),
    (3 * 2.0 ** -10, 0x02), (5 * 2.0 ** -10, 0x02), (7 * 2.0 ** -10, 0x04),
    (1.0625, 0x38), (1.1875, 0x3A), (-1.0625, 0xB8), (2.0 ** -6, 0x08),
    (15 * 2.0 ** -10, 0x08),           # midpoint of 7*2^-9 and 2^-6 -> even 0x08
    (448.0, 0x7E), (456.0, 0x7E), (464.0, 0x7E), (465.0, 0x7E), (1e6, 0x7E),
    (-464.0, 0xFE), (-3e38, 0xFE), (1e-30, 0x00), (-1e-30, 0x80),
    (240.0, 0x77), (248.0, 0x78), (232.0, 0x76),  # 232 is the 224/240 midpoint -> 0x76
]


def test_e4m3_named_ties_and_saturation():
    v = np.array([a for a, _ in NAMED_ENCODE], np.float32)
    got = oracle.e4m3_encode(v)
    assert [int(g) for g in got] == [c for _, c in NAMED_ENCODE]


def _torch_e4m3(v):
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _fp32_from_bits(lo, hi):
    return np.arange(lo, hi, dtype=np.uint64).astype(np.uint32).view(np.float32)


def _parallel_ranges(lo, hi, fn, chunk=1 << 23):
    starts = list(range(lo, hi, chunk))
    with ThreadPoolExecutor(NTHREADS) as ex:
        return list(ex.map(lambda s: fn(s, min(hi, s + chunk)), starts))


def test_e4m3_encode_exhaustive_in_range_vs_torch():
    """Every binary32 with |v| <= 464 (both signs): oracle == torch's
    float8_e4m3fn conversion (round to nearest even).  Beyond 464 torch gives
    NaN while the definition saturates; that region is pinned by the named
    cases above and by test_e4m3_saturation_region."""
    lim = int(np.array(464.0, np.float32).view(np.uint32)) + 1

    def run(lo, hi):
        bad = 0
        for sign in (0, 0x80000000):
            v = (np.arange(lo, hi, dtype=np.uint64).astype(np.uint32) | np.uint32(sign)).view(np.float32)
            bad += int((oracle.e4m3_encode(v) != _torch_e4m3(v)).sum())
        return bad

    assert sum(_parallel_ranges(0, lim, run)) == 0


def test_e4m3_saturation_region():
    lo = int(np.array(464.0, np.float32).view(np.uint32)) + 1
    hi = int(np.array(np.inf, np.float32).view(np.uint32))
    rng = np.random.default_rng(5)
    bits = np.concatenate([np.arange(lo, lo + 100000), rng.integers(lo, hi, 1000000),
                           np.arange(hi - 1000, hi)]).astype(np.uint32)
    v = bits.view(np.float32)
    assert (oracle.e4m3_encode(v) == 0x7E).all()
    assert (oracle.e4m3_encode(-v) == 0xFE).all()


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def _torch_bf16(v):
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_exhaustive_vs_torch():
    """Every finite binary32 (both signs): oracle == torch's bf16 conversion."""
    inf = int(np.array(np.inf, np.float32).view(np.uint32))

    def run(lo, hi):
        bad = 0
        for sign in (0, 0x80000000):
            v = (np.arange(lo, hi, dtype=np.uint64).astype(np.uint32) | np.uint32(sign)).view(np.float32)
            bad += int((oracle.bf16_round(v) != _torch_bf16(v)).sum())
        return bad

    assert sum(_parallel_ranges(0, inf, run, chunk=1 << 24)) == 0


def test_bf16_named():
    cases = [(1.0, 0x3F80), (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82),
             (-0.0, 0x8000), (3.4e38, 0x7F80), (float(np.finfo(np.float32).tiny) / 2, 0x0040)]
    v = np.array([a for a, _ in cases], np.float32)
    assert oracle.bf16_round(v).tolist() == [c for _, c in cases]


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------

def test_dispatch_bf16_is_row_copy_and_leaves_unused_rows():
    wl = workloads.make(1)
    lay = oracle.layout(wl.topk_idx, wl.E, 0)
    recv, _ = oracle.dispatch(wl.x, lay["slot_of"], wl.R, False)
    for r in range(wl.R):
        np.testing.assert_array_equal(recv[r], wl.x[lay["src_of_slot"][r] // wl.k])
    # capacity layout: rows nobody maps to stay at their sentinel
    idx = np.array([[0, 1], [1, 1]], np.int32)
    lay = oracle.layout(idx, 3, 2)
    x = workloads.to_bf16_bits(np.arange(2 * 8, dtype=np.float32).reshape(2, 8))
    recv, _ = oracle.dispatch(x, lay["slot_of"], 6, False)
    assert recv[[1, 4, 5]].tolist() == [[0xFFFF] * 8] * 3
    np.testing.assert_array_equal(recv[[0, 2, 3]], x[[0, 0, 1]])


def test_dispatch_fp8_exact_when_scale_is_power_of_two():
    """Rows built from E4M3-representable values times 2^m with a block
    maximum of exactly 448*2^m: the scale is exactly 2^m, every quotient is
    exact, so decode(q) * scale must reproduce x exactly -- this pins the
    448 constant, the block boundaries, the division direction, the sign and
    the code assignment at once."""
    rng = np.random.default_rng(11)
    tab = oracle.e4m3_decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(tab[c])])
    H, T = 512, 6
    nblk = H // 128
    xf = np.empty((T, H), np.float32)
    exps = rng.integers(-20, 20, size=(T, nblk))
    codes = rng.choice(finite, size=(T, H))
    for t in range(T):
        for b in range(nblk):
            sl = slice(128 * b, 128 * b + 128)
            codes[t, sl][rng.integers(0, 128)] = 0x7E if rng.random() < 0.5 else 0xFE
            xf[t, sl] = tab[codes[t, sl]] * 2.0 ** exps[t, b]
    x = workloads.to_bf16_bits(xf)
    assert (oracle.bf16_to_float(x) == xf).all()      # bf16 holds these exactly
    idx = np.stack([np.arange(T) % 3, 3 + np.arange(T) % 2], axis=1).astype(np.int32)
    lay = oracle.layout(idx, 5, 0)
    q, s = oracle.dispatch(x, lay["slot_of"], T * 2, True)
    for t in range(T):
        for j in range(2):
            r = lay["slot_of"][t, j]
            np.testing.assert_array_equal(s[r], (2.0 ** exps[t]).astype(np.float32))
            dec = tab[q[r]].reshape(nblk, 128) * s[r][:, None]
            np.testing.assert_array_equal(dec.ravel(), xf[t])
            # zero keeps its sign: +0 -> 0x00, -0 -> 0x80
            zero = xf[t] == 0
            np.testing.assert_array_equal(q[r][zero], np.where(np.signbit(xf[t][zero]), 0x80, 0x00))


def _ue8m0_blocks(rng, T, H):
    """bf16 rows whose blocks have maxima at exactly 448*2^j, one bf16 step
    either side of it, random normals, bf16 subnormals (below 448*2^-127,
    where the exponent is clamped), and all-zero blocks."""
    nblk = H // 128
    xf = (rng.standard_normal((T, H)) * 2.0 ** rng.integers(-30, 30, size=(T, 1))).astype(np.float32)
    for t in range(T):
        for b in range(nblk):
            sl = slice(128 * b, 128 * b + 128)
            kind = (t * nblk + b) % 6
            j = int(rng.integers(-100, 100))
            if kind == 0:
                amax = np.float32(448.0 * 2.0 ** j)
            elif kind in (1, 2):
                base = np.float32(448.0 * 2.0 ** j).view(np.uint32)
                amax = (base + (1 << 16) if kind == 1 else base - (1 << 16)).view(np.float32)
            elif kind == 3:
                xf[t, sl] = ((rng.integers(1, 128, 128).astype(np.uint32) << 16).view(np.float32)
                             * rng.choice(np.float32([-1, 1]), 128))
                continue
            elif kind == 4:
                xf[t, sl] = 0.0
                continue
            else:
                continue
            xf[t, sl] = np.clip(xf[t, sl], -amax * 0.99, amax * 0.99)
            xf[t, 128 * b + int(rng.integers(128))] = amax * rng.choice([-1, 1])
    return workloads.to_bf16_bits(xf)


def test_dispatch_ue8m0_vs_exact_exponent_and_torch():
    """UE8M0 scales: the exponent byte is the smallest s >= -127 with
    448 * 2^s >= amax, checked with exact rationals; every code is torch's
    float8_e4m3fn conversion of x * 2^-s (a power-of-two scaling, exact in
    float64); all-zero blocks give byte 0 and codes 0x00."""
    from fractions import Fraction
    rng = np.random.default_rng(31)
    T, H = 24, 768
    nblk = H // 128
    x = _ue8m0_blocks(rng, T, H)
    xf = oracle.bf16_to_float(x)
    idx = np.stack([np.arange(T) % 4, 4 + np.arange(T) % 3], axis=1).astype(np.int32)
    lay = oracle.layout(idx, 7, 0)
    q, e = oracle.dispatch(x, lay["slot_of"], T * 2, 2)
    assert e.dtype == np.uint8
    for t in range(T):
        want_e = np.empty(nblk, np.uint8)
        want_q = np.empty(H, np.uint8)
        for b in range(nblk):
            blk = xf[t, 128 * b:128 * (b + 1)].astype(np.float64)
            amax = Fraction(float(np.abs(blk).max()))
            if amax == 0:
                want_e[b], want_q[128 * b:128 * (b + 1)] = 0, 0
                continue
            s = -127
            while Fraction(448) * Fraction(2) ** s < amax:
                s += 1
            want_e[b] = s + 127
            scaled = torch.from_numpy(blk * 2.0 ** -s).to(torch.float32)
            want_q[128 * b:128 * (b + 1)] = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        for j in range(2):
            r = lay["slot_of"][t, j]
            np.testing.assert_array_equal(e[r], want_e)
            np.testing.assert_array_equal(q[r], want_q)


def test_dispatch_fp8_near_ties_vs_exact_rational():
    """Blocks whose quotients x/scale fall next to E4M3 rounding midpoints --
    the inputs where the order of rounding matters most.  Expected values are
    computed exactly: scale = amax/448 as an exact rational rounded once to
    fp32, the quotient x/scale as an exact rational rounded once to fp32, then
    torch's float8_e4m3fn conversion (round to nearest even)."""
    from fractions import Fraction
    rng = np.random.default_rng(21)
    tab = oracle.e4m3_decode_table()
    pos = tab[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    xs_all = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    nblk = 48
    xf = np.zeros(nblk * 128, np.float32)
    n_near = 0
    for b, amax_bits in enumerate(rng.integers(0x3000, 0x4800, nblk)):
        amax = float(np.array([amax_bits << 16], np.uint32).view(np.float32)[0])
        s = float(round_to_f32(Fraction(amax) / 448))
        xs = xs_all[xs_all < amax]
        qd = xs / s
        j = np.clip(np.searchsorted(mids, qd), 1, len(mids) - 1)
        dist = np.minimum(np.abs(qd - mids[j - 1]), np.abs(qd - mids[j]))
        near = xs[dist <= 2.0 ** -18 * qd][:127]
        n_near += len(near)
        fill = rng.choice(xs, 127 - len(near))
        vals = np.concatenate([near, fill]) * rng.choice([-1.0, 1.0], 127)
        xf[128 * b] = amax if b % 2 else -amax
        xf[128 * b + 1: 128 * (b + 1)] = vals
    assert n_near > 200
    x = workloads.to_bf16_bits(xf[None, :])
    q, sc = oracle.dispatch(x, np.zeros((1, 1), np.int32), 1, True)
    want_q = np.empty(nblk * 128, np.float32)
    for b in range(nblk):
        blk = xf[128 * b: 128 * (b + 1)]
        scale = round_to_f32(Fraction(float(np.abs(blk).max())) / 448)
        assert sc[0, b].view(np.uint32) == scale.view(np.uint32)
        for c in range(128):
            want_q[128 * b + c] = round_to_f32(Fraction(float(blk[c])) / Fraction(float(scale)))
    np.testing.assert_array_equal(q[0], _torch_e4m3(want_q))


@pytest.mark.parametrize("cid", [2, 4])
def test_dispatch_fp8_invariants(cid):
    """Per 128-channel block: scale == 0 iff the block is all zero (then every
    code is 0x00); otherwise the channel(s) at the block maximum encode +-448
    and every channel satisfies the closed-form error bound of RNE to E4M3
    (relative 2^-4 in the normal range, absolute 2^-10 * scale below it),
    widened by the fp32 quotient's own rounding (2^-23 relative)."""
    wl = workloads.make(cid, T=64) if cid == 4 else workloads.make(cid)
    if cid == 4:
        wl.x[3] = 0                                   # an all-zero row
        wl.x[5, :128] = 0                             # one all-zero block
    lay = oracle.layout(wl.topk_idx, wl.E, wl.cap)
    q, s = oracle.dispatch(wl.x, lay["slot_of"], wl.R, True)
    tab = oracle.e4m3_decode_table()
    xf = oracle.bf16_to_float(wl.x).astype(np.float64)
    nblk = wl.H // 128
    for t in range(wl.T):
        rows = lay["slot_of"][t]
        r0 = rows[0]
        for r in rows[1:]:
            assert (q[r] == q[r0]).all() and (s[r].view(np.uint32) == s[r0].view(np.uint32)).all()
        xb = xf[t].reshape(nblk, 128)
        qb = q[r0].reshape(nblk, 128)
        amax = np.abs(xb).max(axis=1)
        assert ((s[r0] == 0) == (amax == 0)).all()
        assert (qb[amax == 0] == 0).all()
        nz = amax > 0
        at_max = np.abs(xb) == amax[:, None]
        assert (np.isin(qb[nz][at_max[nz]], (0x7E, 0xFE))).all()
        dec = tab[qb] * s[r0][:, None].astype(np.float64)
        err = np.abs(dec - xb)
        bound = np.maximum(2.0 ** -4 * np.abs(xb), 2.0 ** -10 * s[r0][:, None]) * (1 + 2.0 ** -19)
        assert (err[nz] <= bound[nz]).all()
        nzd = dec != 0
        assert (np.signbit(dec[nzd]) == np.signbit(xb[nzd])).all()


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------

def test_combine_single_term_is_gather():
    rng = np.random.default_rng(3)
    R, H, T = 40, 64, 40
    eo = workloads.to_bf16_bits(rng.standard_normal((R, H), dtype=np.float32))
    slot = rng.permutation(R)[:T].astype(np.int32).reshape(T, 1)
    y, _ = oracle.combine(eo, slot, np.ones((T, 1), np.float32))
    np.testing.assert_array_equal(y, eo[slot[:, 0]])


def test_combine_vs_exact_sum():
    """acc within Higham's bound gamma_k * sum|w v| of the exact sum (the
    products are exact in float64 and the k-term float64 sum is exact to far
    below the bound); y == the bf16 rounding of acc (torch)."""
    wl = workloads.make(3, T=64, H=256)
    lay = oracle.layout(wl.topk_idx, wl.E, 0)
    eo = wl.expert_out()
    y, acc = oracle.combine(eo, lay["slot_of"], wl.topk_weights)
    v = oracle.bf16_to_float(eo).astype(np.float64)[lay["slot_of"]]   # [T, k, H]
    prod = wl.topk_weights.astype(np.float64)[:, :, None] * v
    exact = prod.sum(axis=1)
    k = wl.k
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    assert (np.abs(acc - exact) <= gamma * np.abs(prod).sum(axis=1)).all()
    np.testing.assert_array_equal(y, _torch_bf16(acc))


def round_to_f32(fr):
    """Exact rational -> nearest binary32, ties to even (subnormals kept)."""
    from fractions import Fraction
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, -126) - 23                     # quantum of the binade (or of subnormals)
    m = a / Fraction(2) ** q
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** q))


def test_combine_fma_chain_vs_exact_rational():
    """acc is the fixed-order chain of fused multiply-adds from +0: each step
    rounds w_j*v_j + acc exactly once (checked with exact rationals).  An
    unfused chain, another term order or another start value fails."""
    from fractions import Fraction
    rng = np.random.default_rng(17)
    T, k, H = 64, 8, 8
    w = (rng.standard_normal((T, k)) * 0.3).astype(np.float32)
    eo = workloads.to_bf16_bits((rng.standard_normal((T * k, H)) * np.exp(rng.standard_normal((T * k, 1)) * 3)).astype(np.float32))
    slot = np.arange(T * k, dtype=np.int32).reshape(T, k)
    _, acc = oracle.combine(eo, slot, w)
    vf = oracle.bf16_to_float(eo)
    for t in range(T):
        for c in range(H):
            a = np.float32(0.0)
            for j in range(k):
                a = round_to_f32(Fraction(float(w[t, j])) * Fraction(float(vf[slot[t, j], c])) + Fraction(float(a)))
            assert a.view(np.uint32) == acc[t, c].view(np.uint32), (t, c)


def test_combine_skips_unplaced_entries():
    rng = np.random.default_rng(4)
    eo = workloads.to_bf16_bits(rng.standard_normal((4, 16), dtype=np.float32))
    w = np.array([[0.5, 0.25, 0.25]], np.float32)
    y_full, a_full = oracle.combine(eo, np.array([[0, -1, 2]], np.int32), w)
    y_two, a_two = oracle.combine(eo[[0, 2]], np.array([[0, 1]], np.int32), w[:, [0, 2]])
    np.testing.assert_array_equal(a_full, a_two)


@pytest.mark.parametrize("cid", [1, 3])
def test_identity_round_trip_returns_x(cid):
    """dispatch, identity experts (expert_out = recv_x), combine with weights
    summing to 1 returns x bit for bit."""
    wl = workloads.make(cid) if cid == 1 else workloads.make(cid, T=128)
    lay = oracle.layout(wl.topk_idx, wl.E, wl.cap)
    recv, _ = oracle.dispatch(wl.x, lay["slot_of"], wl.R, False)
    y, _ = oracle.combine(recv, lay["slot_of"], wl.topk_weights)
    np.testing.assert_array_equal(y, wl.x)


def test_fp8_identity_round_trip_within_bound():
    wl = workloads.make(4, T=64)
    lay = oracle.layout(wl.topk_idx, wl.E, 0)
    q, s = oracle.dispatch(wl.x, lay["slot_of"], wl.R, True)
    tab = oracle.e4m3_decode_table()
    deq = (tab[q] * np.repeat(s.astype(np.float64), 128, axis=1)).astype(np.float32)
    y, _ = oracle.combine(workloads.to_bf16_bits(deq), lay["slot_of"], wl.topk_weights)
    xf = oracle.bf16_to_float(wl.x).astype(np.float64)
    yf = oracle.bf16_to_float(y).astype(np.float64)
    amax = np.abs(xf.reshape(wl.T, -1, 128)).max(axis=2).repeat(128, axis=1)
    # E4M3 rounding (2^-4 relative, or 2^-10 * scale near zero) plus the
    # roundings to fp32 and bf16 on the way out (2^-8 relative in total)
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * amax / 448) + 2.0 ** -7 * np.abs(xf)
    assert (np.abs(yf - xf) <= bound * 1.01).all()


# ---------------------------------------------------------------------------
# generator
# ---------------------------------------------------------------------------

def test_generator_is_deterministic_and_seeded():
    import hashlib

    def h(wl):
        m = hashlib.sha256()
        for a in (wl.x, wl.topk_idx, wl.topk_weights):
            m.update(np.ascontiguousarray(a).tobytes())
        return m.hexdigest()

    for cid in (1, 2, 4):
        assert h(workloads.make(cid)) == h(workloads.make(cid))
        assert h(workloads.make(cid)) != h(workloads.make(cid, seed=1))


def test_generator_shapes_and_routing_models():
    wl = workloads.make(3)
    assert wl.topk_idx.shape == (4096, 8)
    # distinct experts per token, and all 8 inside at most 4 of the 8 groups
    assert all(len(set(r)) == 8 for r in wl.topk_idx.tolist())
    assert max(len(set((np.asarray(r) // 32).tolist())) for r in wl.topk_idx) <= 4
    np.testing.assert_allclose(wl.topk_weights.sum(axis=1), 1.0, rtol=1e-6)
    w5 = workloads.make(5)
    assert abs(w5.meta["hot_load_ratio"] - 1.5) <= 0.015
    w4 = workloads.make(4)
    assert len(w4.meta["outlier_rows"]) == 82
