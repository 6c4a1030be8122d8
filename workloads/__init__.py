"""Seeded synthetic inputs for MoE dispatch / combine.

This module only draws inputs: hidden states, routing tables, routing weights
and expert outputs.  It holds none of the dispatch / combine arithmetic, so
the CPU oracle and the GPU library can both consume it without sharing any
of the method's code.

The pages measure on no public dataset; every workload here is synthetic.
Five workloads are defined (ids 1..5), each with a fixed shape and routing
model:

  1 tiny     T=64,    H=256,  E=8,   k=2, uniform distinct routing, bf16, contiguous
  2 decode   T=128,   H=7168, E=256, k=8, uniform distinct routing, FP8, capacity 128
  3 prefill  T=4096,  H=7168, E=256, k=8, group-limited routing,    bf16, contiguous
  4 skewed   T=8192,  H=4096, E=64,  k=6, Zipf(1.2) routing,        FP8, contiguous,
             1% of rows scaled x100
  5 large    T=16384, H=7168, E=256, k=8, group-limited + 16 hot experts at 1.5x
             mean load, FP8, contiguous

Random numbers come from numpy's PCG64, one independent substream per
(seed, workload id, purpose); the two large normal arrays (hidden states and
expert outputs) take one substream per block of 2048 rows as well, so that
their blocks can be drawn by several host threads with the same result.
Normal draws are fp32 and are rounded to bf16 with torch's CPU conversion
(round to nearest even).

bf16 arrays are returned as uint16 bit patterns; ids as int32; weights fp32.
"""
from dataclasses import dataclass, field
import math

import numpy as np

# substream tags
_X, _ROUTE, _WLOGIT, _EOUT, _HOT, _OUTLIER = 1, 2, 3, 4, 5, 6

CONFIGS = {
    1: dict(name="tiny", T=64, H=256, E=8, k=2, cap=0, fp8=False, routing="uniform"),
    2: dict(name="ll_decode", T=128, H=7168, E=256, k=8, cap=128, fp8=True, routing="uniform"),
    3: dict(name="prefill", T=4096, H=7168, E=256, k=8, cap=0, fp8=False, routing="group"),
    4: dict(name="skewed", T=8192, H=4096, E=64, k=6, cap=0, fp8=True, routing="zipf",
            zipf_s=1.2, outlier_frac=0.01, outlier_scale=100.0),
    5: dict(name="large_prefill", T=16384, H=7168, E=256, k=8, cap=0, fp8=True,
            routing="group", hot_experts=16, hot_ratio=1.5),
}


def _rng(seed, cid, tag):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, tag])))


def to_bf16_bits(f32):
    """fp32 numpy array -> bf16 bit patterns (uint16) via torch's CPU rounding."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


BLOCK_ROWS = 2048


def _threads():
    try:
        import os
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except (AttributeError, OSError):
        return 4


def normal_f32_blocks(seed, cid, tag, shape):
    """N(0,1) fp32 array of the given 2-D shape; rows [b*2048, (b+1)*2048)
    come from substream (seed, cid, tag, b).  Blocks are drawn in host
    threads (numpy releases the GIL while it fills an array); the result does
    not depend on the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    rows, cols = shape
    out = np.empty((rows, cols), np.float32)

    def fill(b):
        r0, r1 = b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, tag, b])))
        out[r0:r1] = g.standard_normal((r1 - r0, cols), dtype=np.float32)

    nblk = -(-rows // BLOCK_ROWS)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def normal_bf16_blocks(seed, cid, tag, shape):
    """bf16 bit patterns (uint16) of normal_f32_blocks, rounded block by block."""
    from concurrent.futures import ThreadPoolExecutor
    rows, cols = shape
    out = np.empty((rows, cols), np.uint16)

    def fill(b):
        r0, r1 = b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, tag, b])))
        out[r0:r1] = to_bf16_bits(g.standard_normal((r1 - r0, cols), dtype=np.float32))

    nblk = -(-rows // BLOCK_ROWS)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def _softmax_f32(logits):
    l = logits.astype(np.float64)
    l = l - l.max(axis=1, keepdims=True)
    e = np.exp(l)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def _topk_desc(keys, k):
    """Indices of the k largest keys per row, largest first; ties -> lower index."""
    return np.argsort(-keys, axis=1, kind="stable")[:, :k]


def _uniform_distinct(rng, T, E, k):
    # k distinct experts per token, every ordered k-subset equally likely
    # (ranking i.i.d. uniform keys is a uniformly random permutation).
    return _topk_desc(rng.random((T, E)), k)


def _zipf_distinct(rng, T, E, k, s, perm):
    # p(perm[r]) proportional to (r+1)^-s; k draws without replacement, each
    # draw renormalised over the experts not yet drawn.  Ranking
    # log p + Gumbel noise is the same distribution (Gumbel-top-k), and its
    # descending order is the draw order.
    p = np.empty(E)
    p[perm] = (np.arange(E) + 1.0) ** (-s)
    p /= p.sum()
    g = -np.log(-np.log(rng.random((T, E))))
    return _topk_desc(np.log(p)[None, :] + g, k)


def group_limited_topk(logits, k, n_groups=8, topk_groups=4):
    """Group-limited expert choice on gate logits [T, E].

    Groups are runs of E/n_groups consecutive experts.  A group's score is the
    sum of its two largest logits; the topk_groups best groups are kept and
    the k largest logits among their experts are chosen, largest first.
    """
    T, E = logits.shape
    gsz = E // n_groups
    l64 = logits.astype(np.float64)
    g = np.sort(l64.reshape(T, n_groups, gsz), axis=2)
    gscore = g[:, :, -1] + g[:, :, -2]
    gsel = _topk_desc(gscore, topk_groups)
    keep = np.zeros((T, n_groups), bool)
    keep[np.arange(T)[:, None], gsel] = True
    masked = np.where(np.repeat(keep, gsz, axis=1), l64, -np.inf)
    return _topk_desc(masked, k)


_beta_cache = {}


def _hot_bias(logits, hot, k, ratio, key):
    """Bisection for the logit bias on `hot` experts that makes their mean load
    `ratio` x the mean load of all experts (within 1%)."""
    if key in _beta_cache:
        return _beta_cache[key]
    T, E = logits.shape
    mean_load = T * k / E

    def load_ratio(beta):
        l = logits.copy()
        l[:, hot] += np.float32(beta)
        idx = group_limited_topk(l, k)
        load = np.bincount(idx.ravel(), minlength=E)
        return load[hot].mean() / mean_load

    lo, hi = 0.0, 4.0
    beta = 0.5 * (lo + hi)
    for _ in range(40):
        beta = 0.5 * (lo + hi)
        r = load_ratio(beta)
        if abs(r - ratio) <= 0.01 * ratio:
            break
        if r < ratio:
            lo = beta
        else:
            hi = beta
    _beta_cache[key] = (beta, r)
    return beta, r


@dataclass
class Workload:
    cid: int
    name: str
    seed: int
    T: int
    H: int
    E: int
    k: int
    cap: int
    fp8: bool
    x: np.ndarray            # uint16 [T, H] bf16 bits
    topk_idx: np.ndarray     # int32 [T, k]
    topk_weights: np.ndarray  # float32 [T, k]
    meta: dict = field(default_factory=dict)

    @property
    def R(self):
        return self.T * self.k if self.cap == 0 else self.E * self.cap

    def expert_out(self):
        """bf16 N(0,1) expert outputs [R, H] in the receive-row layout."""
        return normal_bf16_blocks(self.seed, self.cid, _EOUT, (self.R, self.H))

    def describe(self):
        return dict(workload=self.name, config_id=self.cid, seed=self.seed, T=self.T,
                    H=self.H, E=self.E, topk=self.k, capacity=self.cap,
                    payload="e4m3" if self.fp8 else "bf16")


def make(cid, seed=0, **overrides):
    """Build workload `cid` (1..5).  Keyword overrides (T, H, E, k, cap, fp8)
    change the shape while keeping that workload's routing model."""
    cfg = dict(CONFIGS[cid])
    cfg.update(overrides)
    T, H, E, k, cap, fp8 = (cfg[n] for n in ("T", "H", "E", "k", "cap", "fp8"))
    meta = {}

    xf = normal_f32_blocks(seed, cid, _X, (T, H))
    if cfg.get("outlier_frac"):
        n_out = math.ceil(cfg["outlier_frac"] * T)
        rows = _rng(seed, cid, _OUTLIER).choice(T, size=n_out, replace=False) if T else []
        xf[rows] *= np.float32(cfg["outlier_scale"])
        meta["outlier_rows"] = np.sort(np.asarray(rows, np.int64))
    x = to_bf16_bits(xf)

    rr = _rng(seed, cid, _ROUTE)
    routing = cfg["routing"]
    if routing == "uniform":
        idx = _uniform_distinct(rr, T, E, k)
        weights = _softmax_f32(_rng(seed, cid, _WLOGIT).standard_normal((T, k)))
    elif routing == "zipf":
        perm = rr.permutation(E)
        idx = _zipf_distinct(rr, T, E, k, cfg["zipf_s"], perm)
        weights = _softmax_f32(_rng(seed, cid, _WLOGIT).standard_normal((T, k)))
        meta["zipf_perm"] = perm
    elif routing == "group":
        logits = rr.standard_normal((T, E), dtype=np.float32)
        if cfg.get("hot_experts"):
            hot = _rng(seed, cid, _HOT).permutation(E)[: cfg["hot_experts"]]
            beta, r = _hot_bias(logits, hot, k, cfg["hot_ratio"],
                                (seed, cid, T, E, k, len(hot), cfg["hot_ratio"]))
            logits[:, hot] += np.float32(beta)
            meta.update(hot_experts=np.sort(hot), hot_bias=beta, hot_load_ratio=r)
        idx = group_limited_topk(logits, k)
        sel = np.take_along_axis(logits, idx, axis=1)
        weights = _softmax_f32(sel)
    else:
        raise ValueError(routing)

    return Workload(cid=cid, name=cfg["name"], seed=seed, T=T, H=H, E=E, k=k, cap=cap,
                    fp8=bool(fp8), x=x, topk_idx=np.ascontiguousarray(idx, np.int32),
                    topk_weights=np.ascontiguousarray(weights, np.float32), meta=meta)
