// ep_layout_dev.h -- device code of the routing layout, shared by the layout
// kernels and the fused layout + dispatch kernel.  The algorithm is described
// at the top of ep_layout.hip.
#pragma once

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace layout {


constexpr int kHistThreads = 256;             // layout_hist workgroup
constexpr int kRankThreads = 1024;            // layout_rank / layout_single workgroup
constexpr int kRankRunWords = 4112;           // LDS words for the per-wave running ranks
constexpr int kTwoPassMaxBlocks = 64;
constexpr int kTableStride = kTwoPassMaxBlocks;  // rows per table column
constexpr int kKeySteps = 4;                  // 64-entry steps of a run held in registers

__device__ __forceinline__ int key_bits(int E) {
    // number of bits needed for ids 0..E-1
    return (E <= 1) ? 0 : 32 - __clz(E - 1);
}

__device__ __forceinline__ bool valid_id(int32_t key, int E) {
    return static_cast<uint32_t>(key) < static_cast<uint32_t>(E);
}

// Inclusive integer scans on DPP lane moves (no LDS traffic).  row_shr by
// 1, 2, 4, 8 scans each row of 16 lanes (lanes shifted in from outside the
// row read 0); row_bcast 15 and 31 then carry row totals into later rows.
constexpr int kDppRowShr = 0x110;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

__device__ __forceinline__ int32_t row16_inclusive_scan(int32_t v) {
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr | 1, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr | 2, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr | 4, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr | 8, 0xf, 0xf, false);
    return v;
}

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
    v = row16_inclusive_scan(v);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xa, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xc, 0xf, false);
    return v;
}

// Waves that rank a block's entries: as many as the workgroup has (16), as
// long as their running-rank rows fit in kRankRunWords.  Rows are E+1 words
// apart so the 16 lanes reading one expert across 16 waves hit 16 different
// LDS banks.
__host__ __device__ constexpr int rank_waves(int E) {
    return (kRankRunWords / (E + 1) >= kRankThreads / kWave) ? kRankThreads / kWave
           : (kRankRunWords / (E + 1) >= 4 ? kRankRunWords / (E + 1) : 4);
}

__host__ __device__ constexpr size_t rank_lds_bytes(int E) {
    return static_cast<size_t>(((3 * E + 1 + rank_waves(E) * (E + 1)) + 3) & ~3) * 4;
}

// LDS layout shared by both ranking kernels (int32 words).
struct RankLds {
    int32_t* total;  // [E]   valid entries per expert in the whole table
    int32_t* prior;  // [E]   valid entries per expert in blocks before this one
    int32_t* off;    // [E+1] exclusive scan of total
    int32_t* run;    // [rank waves][E+1] running first rank per ranking wave
};

__device__ __forceinline__ RankLds carve(int32_t* sm, int E) {
    RankLds l;
    l.total = sm;
    l.prior = sm + E;
    l.off = sm + 2 * E;
    l.run = sm + 3 * E + 1;
    return l;
}

// The contiguous run of entries one ranking wave owns:
// [wbegin, wbegin + S) clipped to the block's end.  S is a multiple of 64 and
// rw * S covers the block; waves at or past rw (or past the block) own nothing.
struct Run {
    int64_t wbegin;
    int64_t wend;
    int S;
    int passes;  // passes of kKeySteps * 64 entries
};

__device__ __forceinline__ Run wave_run(int64_t begin, int64_t end, int chunk, int rw, int wave) {
    Run r;
    r.S = ((chunk / rw + kWave - 1) / kWave) * kWave;
    r.wbegin = begin + static_cast<int64_t>(wave) * r.S;
    const int64_t e = r.wbegin + r.S;
    r.wend = (wave < rw) ? (e < end ? e : end) : r.wbegin;
    r.passes = (r.S + kKeySteps * kWave - 1) / (kKeySteps * kWave);
    return r;
}

// Ids of one pass of a run (entry p0 + 64*s + lane); entries outside the run
// are not loaded.
__device__ __forceinline__ void load_pass(const int32_t* __restrict__ idx, int64_t p0,
                                          int64_t wend, uint32_t lane, int32_t (&key)[kKeySteps]) {
#pragma unroll
    for (int s = 0; s < kKeySteps; ++s) {
        const int64_t i = p0 + s * kWave + lane;
        key[s] = (i < wend) ? idx[i] : -1;
    }
}

// Adds one pass of this wave's ids to its running-count row.
__device__ __forceinline__ void count_pass(const int32_t (&key)[kKeySteps], int64_t p0,
                                           int64_t wend, uint32_t lane, int E, int nbits,
                                           int32_t* wrun) {
#pragma unroll
    for (int s = 0; s < kKeySteps; ++s) {
        if (p0 + s * kWave >= wend) break;  // uniform: past the end of the run
        const int64_t i = p0 + s * kWave + lane;
        const bool valid = i < wend && valid_id(key[s], E);
        const uint64_t peers = match_peers(valid ? key[s] : 0, nbits, __ballot(valid));
        if (valid && (peers & lanemask_lt()) == 0) wrun[key[s]] += __popcll(peers);
    }
}

// Ranks one pass of this wave's entries, writing slot_of and src_of_slot.
__device__ __forceinline__ void rank_pass(const int32_t (&key)[kKeySteps], int64_t p0,
                                          int64_t wend, uint32_t lane, int E, int cap,
                                          int nbits, int64_t R, int32_t* wrun,
                                          int32_t* __restrict__ slot_of,
                                          int32_t* __restrict__ src_of_slot) {
#pragma unroll
    for (int s = 0; s < kKeySteps; ++s) {
        if (p0 + s * kWave >= wend) break;  // uniform: past the end of the run
        const int64_t i = p0 + s * kWave + lane;
        const bool in = i < wend;
        const bool valid = in && valid_id(key[s], E);
        const uint64_t peers = match_peers(valid ? key[s] : 0, nbits, __ballot(valid));
        int32_t first = 0;
        if (valid) first = wrun[key[s]];
        if (valid && (peers & lanemask_lt()) == 0) wrun[key[s]] = first + __popcll(peers);
        if (in) {
            int32_t slot = -1;
            if (valid) {
                const int32_t r = first + __popcll(peers & lanemask_lt());
                if (cap == 0) {
                    slot = r;
                } else if (r < cap) {
                    slot = key[s] * cap + r;
                }
            }
            slot_of[i] = slot;
            if (slot >= 0 && slot < R) src_of_slot[slot] = static_cast<int32_t>(i);
        }
    }
}

// Per-wave counts of the wave's whole run.  The first pass's ids are already
// in `key` (loaded early); later passes (blocks above 16K entries) reload.
__device__ __forceinline__ void count_run(const int32_t* __restrict__ idx, const Run& r,
                                          const int32_t (&key)[kKeySteps], uint32_t lane, int E,
                                          int nbits, int32_t* wrun) {
    count_pass(key, r.wbegin, r.wend, lane, E, nbits, wrun);
    for (int p = 1; p < r.passes; ++p) {
        int32_t k2[kKeySteps];
        const int64_t p0 = r.wbegin + static_cast<int64_t>(p) * kKeySteps * kWave;
        load_pass(idx, p0, r.wend, lane, k2);
        count_pass(k2, p0, r.wend, lane, E, nbits, wrun);
    }
}

// Everything after total, prior and num_invalid are in LDS and every ranking
// wave has counted its run (all threads call it, after a barrier).
__device__ void finish_layout(int b, const int32_t* __restrict__ idx, int E, int cap,
                              int nblocks, int64_t R, const RankLds& l, const Run& r,
                              const int32_t (&key)[kKeySteps], int32_t num_invalid,
                              int32_t* s_dropped, int32_t* __restrict__ count,
                              int32_t* __restrict__ offset, int32_t* __restrict__ slot_of,
                              int32_t* __restrict__ src_of_slot, int32_t* __restrict__ status) {
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const uint32_t lane = lane_id();
    const int rw = rank_waves(E);
    const int rs = E + 1;  // row stride of l.run

    // Exclusive scan of total into off (wave 0; each lane owns a run of
    // consecutive experts), and the number of entries dropped by the capacity.
    if (wave == 0) {
        const int per = (E + kWave - 1) / kWave;
        const int e0 = min(E, static_cast<int>(lane) * per);
        const int e1 = min(E, e0 + per);
        int32_t local = 0, drop = 0;
        for (int e = e0; e < e1; ++e) {
            local += l.total[e];
            if (cap > 0 && l.total[e] > cap) drop += l.total[e] - cap;
        }
        const int32_t incl = wave_inclusive_scan(local);
        int32_t run_sum = incl - local;
        for (int e = e0; e < e1; ++e) {
            l.off[e] = run_sum;
            run_sum += l.total[e];
        }
        if (lane == kWave - 1) l.off[E] = incl;
        if (cap > 0) {
            const int32_t drop_all = wave_inclusive_scan(drop);
            if (lane == kWave - 1) *s_dropped = drop_all;
        } else if (lane == 0) {
            *s_dropped = 0;
        }
    }
    __syncthreads();

    if (b == 0) {
        for (int e = tid; e < E; e += kRankThreads) {
            count[e] = l.total[e];
            offset[e] = l.off[e];
        }
        if (tid == 0) {
            offset[E] = l.off[E];
            status[0] = num_invalid;
            status[1] = *s_dropped;
        }
    }

    // First rank of each (wave, expert): entries in earlier blocks, then in
    // earlier waves of this block.  For the contiguous layout the expert's
    // offset is folded in, so the value is directly a receive row; for the
    // fixed-capacity layout it stays the rank inside the expert.  Each
    // 16-lane row takes one expert, lane w holding wave w's count, and an
    // exclusive row scan gives every wave its start (rw <= 16).
    for (int e0 = 0; e0 < E; e0 += kRankThreads / 16) {
        const int e = e0 + tid / 16;
        const int w = tid & 15;
        const bool mine = e < E && w < rw;
        const int32_t c = mine ? l.run[w * rs + e] : 0;
        const int32_t before = row16_inclusive_scan(c) - c;
        if (mine) l.run[w * rs + e] = l.prior[e] + (cap == 0 ? l.off[e] : 0) + before;
    }
    __syncthreads();

    // Rank pass in (t, j) order: lane rank among same-expert lanes below it.
    if (wave < rw) {
        const int nbits = key_bits(E);
        int32_t* wrun = l.run + wave * rs;
        rank_pass(key, r.wbegin, r.wend, lane, E, cap, nbits, R, wrun, slot_of, src_of_slot);
        for (int p = 1; p < r.passes; ++p) {
            int32_t k2[kKeySteps];
            const int64_t p0 = r.wbegin + static_cast<int64_t>(p) * kKeySteps * kWave;
            load_pass(idx, p0, r.wend, lane, k2);
            rank_pass(k2, p0, r.wend, lane, E, cap, nbits, R, wrun, slot_of, src_of_slot);
        }
    }

    // Receive rows that no entry fills get src_of_slot = -1.
    if (cap == 0) {
        const int64_t gtid = static_cast<int64_t>(b) * kRankThreads + tid;
        const int64_t gstride = static_cast<int64_t>(nblocks) * kRankThreads;
        for (int64_t row = l.off[E] + gtid; row < R; row += gstride) src_of_slot[row] = -1;
    } else {
        for (int e = b; e < E; e += nblocks) {
            int32_t* rows = src_of_slot + static_cast<int64_t>(e) * cap;
            for (int rr = min(l.total[e], cap) + tid; rr < cap; rr += kRankThreads) rows[rr] = -1;
        }
    }
}

// ---- two-pass path -----------------------------------------------------------

// Reads 16-byte groups of routing entries [i0, i0+4) (entries at or past
// `end` read as -1).  idx is 16-byte aligned.
__device__ __forceinline__ int4 load_group(const int32_t* __restrict__ idx, int64_t i0, int64_t end) {
    int4 q;
    if (i0 + 3 < end) {
        q = *reinterpret_cast<const int4*>(idx + i0);
    } else {
        q.x = (i0 + 0 < end) ? idx[i0 + 0] : -1;
        q.y = (i0 + 1 < end) ? idx[i0 + 1] : -1;
        q.z = (i0 + 2 < end) ? idx[i0 + 2] : -1;
        q.w = -1;
    }
    return q;
}

// Histogram of block b's entries, stored as column entries b of the
// block-histogram table (the whole workgroup, kHistThreads wide, calls it;
// hist is LDS of E+1 words; the last block zeroes the table's padding).
// PREFIX: also the exclusive scan of the block's valid counts over experts,
// as column entries b of a second table of the same shape right after the
// first (its column E holds the block's number of valid entries), and block
// 0 zeroes status[1] for the dispatch kernel that ranks from these tables.
template <bool PREFIX = false>
__device__ void hist_block(int b, int32_t* hist, const int32_t* __restrict__ idx, int64_t n,
                           int E, int chunk, int nblocks, int32_t* __restrict__ block_hist,
                           int32_t* __restrict__ status = nullptr) {
    for (int e = threadIdx.x; e <= E; e += kHistThreads) hist[e] = 0;
    __syncthreads();

    const int64_t begin = static_cast<int64_t>(b) * chunk;
    const int64_t end = (begin + chunk < n) ? begin + chunk : n;
    const int ng = chunk / 4;
    int32_t invalid = 0;
    for (int g0 = 0; g0 < ng; g0 += 4 * kHistThreads) {
        int4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int g = g0 + u * kHistThreads + threadIdx.x;
            q[u] = (g < ng) ? load_group(idx, begin + 4 * g, end) : make_int4(-1, -1, -1, -1);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i0 = begin + 4 * (g0 + u * kHistThreads + threadIdx.x);
            const int32_t key[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (valid_id(key[c], E)) atomicAdd(&hist[key[c]], 1);
                else if (i0 + c < end) ++invalid;
            }
        }
    }
    if (invalid) atomicAdd(&hist[E], invalid);
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += kHistThreads) {
        block_hist[static_cast<int64_t>(e) * kTableStride + b] = hist[e];
        // zero the padding so column sums can read whole columns
        if (b == nblocks - 1)
            for (int p = nblocks; p < kTableStride; ++p)
                block_hist[static_cast<int64_t>(e) * kTableStride + p] = 0;
    }
    if (PREFIX) {
        int32_t* prefix = block_hist + static_cast<int64_t>(E + 1) * kTableStride;
        if (b == 0 && threadIdx.x == 0) status[1] = 0;
        if (threadIdx.x < kWave) {  // wave 0: each lane scans a run of experts
            const uint32_t lane = lane_id();
            const int per = (E + kWave - 1) / kWave;
            const int e0 = min(E, static_cast<int>(lane) * per);
            const int e1 = min(E, e0 + per);
            int32_t local = 0;
            for (int e = e0; e < e1; ++e) local += hist[e];
            const int32_t incl = wave_inclusive_scan(local);
            int32_t run = incl - local;
            for (int e = e0; e < e1; ++e) {
                prefix[static_cast<int64_t>(e) * kTableStride + b] = run;
                run += hist[e];
            }
            if (lane == kWave - 1) prefix[static_cast<int64_t>(E) * kTableStride + b] = incl;
        }
        if (b == nblocks - 1)
            for (int e = threadIdx.x; e <= E; e += kHistThreads)
                for (int p = nblocks; p < kTableStride; ++p)
                    prefix[static_cast<int64_t>(e) * kTableStride + p] = 0;
    }
}


// Ranks block b of the two-pass path (the whole workgroup calls it; sm is
// the workgroup's dynamic LDS of rank_lds_bytes(E)).
// kMaxLoads bounds the table loads per wave (E + 1 columns over 16 waves, 4
// columns per load): (E + 64) / 64 loads suffice.
template <int kMaxLoads = (kMaxExperts + 64) / 64>
__device__ void rank_block(int b, int32_t* sm, const int32_t* __restrict__ idx, int64_t n, int E,
                           int cap, int chunk, int nblocks, int64_t R,
                           const int32_t* __restrict__ block_hist, int32_t* __restrict__ count,
                           int32_t* __restrict__ offset, int32_t* __restrict__ slot_of,
                           int32_t* __restrict__ src_of_slot, int32_t* __restrict__ status) {
    __shared__ int32_t s_invalid, s_dropped;
    const RankLds l = carve(sm, E);
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const uint32_t lane = lane_id();
    const int rw = rank_waves(E);
    const int64_t begin = static_cast<int64_t>(b) * chunk;
    const int64_t end = (begin + chunk < n) ? begin + chunk : n;
    const Run r = wave_run(begin, end, chunk, rw, wave);

    // Every global load of the prologue is issued before any is used: first
    // this wave's run of ids, then the whole table, read as 1 KiB per wave
    // instruction with 16 lanes (a DPP row) per column and 4 columns per
    // instruction.
    int32_t key[kKeySteps];
    load_pass(idx, r.wbegin, r.wend, lane, key);
    constexpr int kColsPerLoad = kWave / 16;
    constexpr int kColsPerRound = kColsPerLoad * (kRankThreads / kWave);
    const int ncols = E + 1;
    const int loads_per_wave = (ncols + kColsPerRound - 1) / kColsPerRound;
    const int grp = lane & 15;  // 16-byte group inside the column
    int4 q[kMaxLoads];
#pragma unroll
    for (int m = 0; m < kMaxLoads; ++m) {
        const int col = (m * (kRankThreads / kWave) + wave) * kColsPerLoad + lane / 16;
        if (m < loads_per_wave && col < ncols)
            q[m] = reinterpret_cast<const int4*>(block_hist + static_cast<int64_t>(col) * kTableStride)[grp];
        else
            q[m] = make_int4(0, 0, 0, 0);
    }

    // This wave's counts, built while the table loads are in flight.
    int32_t* wrun = l.run + wave * (E + 1);
    if (wave < rw) {
        for (int e = lane; e <= E; e += kWave) wrun[e] = 0;
        count_run(idx, r, key, lane, E, key_bits(E), wrun);
    }

    // Column totals and the part of each column before this block.
#pragma unroll
    for (int m = 0; m < kMaxLoads; ++m) {
        if (m < loads_per_wave) {  // uniform across the wave
            const int col = (m * (kRankThreads / kWave) + wave) * kColsPerLoad + lane / 16;
            const int32_t v[4] = {q[m].x, q[m].y, q[m].z, q[m].w};
            int32_t tot = 0, pre = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                tot += v[c];
                pre += (4 * grp + c < b) ? v[c] : 0;
            }
            tot = row16_inclusive_scan(tot);
            pre = row16_inclusive_scan(pre);
            if (grp == 15 && col < ncols) {
                if (col < E) {
                    l.total[col] = tot;
                    l.prior[col] = pre;
                } else {
                    s_invalid = tot;
                }
            }
        }
    }
    __syncthreads();

    finish_layout(b, idx, E, cap, nblocks, R, l, r, key, s_invalid, &s_dropped, count, offset,
                  slot_of, src_of_slot, status);
}


}  // namespace layout
}  // namespace ep
