// ep_small_dev.h -- device code for small routing tables (at most
// kFusedMaxEntries ids), shared by the one-kernel layout of ep_layout and the
// one-kernel layout + dispatch of ep_layout_dispatch.
//
// Every workgroup works from the whole table, staged in its LDS, and needs
// no other workgroup:
//   * an LDS histogram of the ids, scanned into the expert offsets, gives
//     count, offset and the number of entries dropped by the capacity;
//   * the rank of each of the workgroup's (at most 64) entries is the number
//     of equal ids ahead of it.  Each entry sets its bit in a 64-bit mask
//     kept per expert; one pass over the ids ahead of the entries looks each
//     id up in that table and adds one to every entry whose bit is set and
//     which lies after the id (a hit is rare: about entries/E per id).
#pragma once

#include "ep_device.h"
#include "ep_internal.h"
#include "ep_layout_dev.h"

namespace ep {
namespace small {

using layout::valid_id;
using layout::wave_inclusive_scan;

constexpr int kThreads = 256;      // workgroup size of both small-table kernels
constexpr int kMaxEntries = 64;    // routing entries ranked per workgroup
static_assert(kFusedMaxEntries % (4 * kThreads) == 0, "whole staging steps");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Dynamic LDS (int32 words first):
//   ids  [4 * ceil(n / 4)]  the routing table, padded with -1 to whole quads
//   hist [E + 1]            ids per expert; hist[E] counts ids outside [0, E)
//   off  [E + 1]            exclusive scan of hist[0..E); off[E] = valid ids
//   map  [E]                uint64: bit q set if the workgroup's entry q has id e
struct Tables {
    int32_t* ids;
    int32_t* hist;
    int32_t* off;
    uint64_t* map;
};

__host__ __device__ inline size_t words_before_map(int n, int E) {
    return static_cast<size_t>((n + 3) / 4) * 4 + 2 * static_cast<size_t>(E + 1);
}

__host__ __device__ inline size_t lds_bytes(int n, int E) {
    return ((words_before_map(n, E) * 4 + 7) / 8) * 8 + static_cast<size_t>(E) * 8;
}

__device__ inline Tables carve(int32_t* dyn, int n, int E) {
    Tables t;
    t.ids = dyn;
    t.hist = dyn + static_cast<size_t>((n + 3) / 4) * 4;
    t.off = t.hist + (E + 1);
    t.map = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(dyn) +
                                        ((words_before_map(n, E) * 4 + 7) / 8) * 8);
    return t;
}

// The routing table on its way into LDS: load() issues the global loads
// (16 bytes per lane per step; idx is 16-byte aligned), store() writes LDS,
// so that other loads can be issued in between.
struct IdStage {
    static constexpr int kSteps = kFusedMaxEntries / (4 * kThreads);
    u32x4 q[kSteps];
    int32_t tail;

    __device__ __forceinline__ void load(const int32_t* __restrict__ idx, int n) {
        const int n4 = n / 4;
#pragma unroll
        for (int m = 0; m < kSteps; ++m) {
            const int i = m * kThreads + static_cast<int>(threadIdx.x);
            if (i < n4) q[m] = reinterpret_cast<const u32x4*>(idx)[i];
        }
        const int r = 4 * n4 + static_cast<int>(threadIdx.x);
        tail = (static_cast<int>(threadIdx.x) < 4 && r < n) ? idx[r] : -1;
    }

    __device__ __forceinline__ void store(int n, int32_t* ids) const {
        const int n4 = n / 4;
#pragma unroll
        for (int m = 0; m < kSteps; ++m) {
            const int i = m * kThreads + static_cast<int>(threadIdx.x);
            if (i < n4) reinterpret_cast<u32x4*>(ids)[i] = q[m];
        }
        if (threadIdx.x < 4 && n % 4 != 0) ids[4 * n4 + threadIdx.x] = tail;
    }
};

// Zeroes hist and map (the caller puts a barrier before their use).
__device__ inline void zero_tables(const Tables& t, int E) {
    for (int e = threadIdx.x; e <= E; e += kThreads) t.hist[e] = 0;
    for (int e = threadIdx.x; e < E; e += kThreads) t.map[e] = 0;
}

// Entry q (< 64) with id `key` sets bit q of map[key]; invalid ids set
// nothing.
__device__ inline void mark_entry(const Tables& t, int E, int q, int32_t key) {
    if (valid_id(key, E))
        atomicOr(reinterpret_cast<unsigned long long*>(&t.map[key]), 1ull << q);
}

__device__ inline void histogram(const Tables& t, int n, int E) {
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int32_t id = t.ids[i];
        atomicAdd(&t.hist[valid_id(id, E) ? id : E], 1);
    }
}

// Whether workgroup b builds the whole histogram (and the offsets): always
// with the contiguous layout and in workgroup 0 (which writes count, offset
// and status); otherwise only when it marks the empty rows of more than two
// experts, since count_experts takes one pass over the table per expert and
// the histogram one LDS add per id (decode: 448 workgroups over 256 experts
// count; a 16-workgroup layout over 256 experts builds the histogram).
__device__ inline bool whole_histogram(int cap, int b, int E, int nwg) {
    return cap == 0 || b == 0 || E > 2 * nwg;
}

// With fixed capacity a workgroup other than workgroup 0 needs no offsets
// (its slots are e*cap + rank) and, of the histogram, only the counts of the
// experts whose empty rows it marks (b, b + nwg, ...): those are counted
// here, one wave sum and one LDS add per wave and expert, into hist (zeroed
// by the caller before a barrier).
__device__ inline void count_experts(const Tables& t, int n, int E, int b, int nwg) {
    for (int e = b; e < E; e += nwg) {
        int32_t c = 0;
        for (int i = threadIdx.x; i < n; i += kThreads) c += (t.ids[i] == e) ? 1 : 0;
        c = wave_inclusive_scan(c);
        if (lane_id() == kWave - 1 && c != 0) atomicAdd(&t.hist[e], c);
    }
}

// Adds, for every id at position i < end, one to eq[q] for each entry q in
// map[id] & ahead(i), where ahead(i) is the mask of entries after position
// i.  eq is LDS, zeroed by the caller before a barrier.
template <typename AheadF>
__device__ void count_ahead(const Tables& t, int end, int E, AheadF ahead, int32_t* eq) {
    for (int i = threadIdx.x; i < end; i += kThreads) {
        const int32_t id = t.ids[i];
        if (!valid_id(id, E)) continue;
        uint64_t m = t.map[id];
        if (m == 0) continue;
        m &= ahead(i);
        while (m) {
            atomicAdd(&eq[__builtin_ctzll(m)], 1);
            m &= m - 1;
        }
    }
}

// Wave 0: off = exclusive scan of hist (off[E] = valid ids) and the number
// of entries the capacity drops.  Call after the histogram is complete.
__device__ inline void scan_offsets(const Tables& t, int E, int cap, int32_t* s_drop) {
    if (threadIdx.x >= kWave) return;
    const uint32_t lane = lane_id();
    const int per = (E + kWave - 1) / kWave;
    const int lo = min(E, static_cast<int>(lane) * per);
    const int hi = min(E, lo + per);
    int32_t local = 0, drop = 0;
    for (int e = lo; e < hi; ++e) {
        local += t.hist[e];
        if (cap > 0 && t.hist[e] > cap) drop += t.hist[e] - cap;
    }
    const int32_t incl = wave_inclusive_scan(local);
    const int32_t drop_all = wave_inclusive_scan(drop);
    int32_t run = incl - local;
    for (int e = lo; e < hi; ++e) {
        t.off[e] = run;
        run += t.hist[e];
    }
    if (lane == kWave - 1) {
        t.off[E] = incl;
        *s_drop = (cap > 0) ? drop_all : 0;
    }
}

// The slot of a valid entry with id e and rank r (contiguous or fixed
// capacity); -1 for an invalid id or a rank past the capacity.
__device__ inline int32_t slot_for(const Tables& t, int E, int cap, int32_t e, int32_t r) {
    if (!valid_id(e, E)) return -1;
    if (cap == 0) return t.off[e] + r;
    return (r < cap) ? e * cap + r : -1;
}

// count, offset and status (one workgroup).
__device__ inline void write_totals(const Tables& t, int E, int32_t drop, int32_t* count,
                                    int32_t* offset, int32_t* status) {
    for (int e = threadIdx.x; e < E; e += kThreads) {
        count[e] = t.hist[e];
        offset[e] = t.off[e];
    }
    if (threadIdx.x == 0) {
        offset[E] = t.off[E];
        status[0] = t.hist[E];
        status[1] = drop;
    }
}

// Receive rows no entry fills get src_of_slot = -1: the rows past the count
// of experts b, b + nwg, ... (fixed capacity), or the rows past the valid
// entries, strided over the nwg workgroups (contiguous).
__device__ inline void fill_empty_rows(const Tables& t, int E, int cap, int64_t R, int b, int nwg,
                                       int32_t* src_of_slot) {
    if (cap > 0) {
        for (int e = b; e < E; e += nwg) {
            int32_t* rows = src_of_slot + static_cast<int64_t>(e) * cap;
            for (int r = min(t.hist[e], cap) + static_cast<int>(threadIdx.x); r < cap; r += kThreads)
                rows[r] = -1;
        }
    } else {
        for (int64_t r = t.off[E] + static_cast<int64_t>(b) * kThreads + threadIdx.x; r < R;
             r += static_cast<int64_t>(nwg) * kThreads)
            src_of_slot[r] = -1;
    }
}

}  // namespace small
}  // namespace ep
