// ep_layout.hip -- routing layout: per-expert histogram, exclusive scan into
// expert-major offsets, and a stable slot for every routing entry.
//
// The count per expert and the expert-major receive rows follow the
// low-latency dispatch of "[GH-ISSUE #282] Redundant atomics in internode_ll"
// (per-expert token counts, receive counts indexed by local expert); the
// stable order inside an expert follows the order-consistency requirement in
// "[GH-ISSUE #18] Reasons for not calling NVSHMEM public APIs?".
//
// Two kernels, both over the same partition of the T*k entries into blocks of
// `chunk` consecutive entries (row-major (t, j) order):
//
//   layout_hist  each block builds its expert histogram in LDS (one LDS add
//                per distinct expert per wave, found with key-bit ballots)
//                and stores it, plus its count of invalid ids, as one row of
//                the block-histogram table in the workspace.
//   layout_rank  each block sums the table's columns (all blocks: totals;
//                earlier blocks: its own prefix), scans the totals into
//                offsets, then ranks its entries: per-wave histograms of its
//                chunk give each wave a starting rank per expert, and inside
//                a wave each 64-entry step ranks lanes against lower lanes with
//                the same expert by ballot matching.  Block 0 writes count,
//                offset and status; all blocks together mark empty receive
//                rows with -1.
//
// The result is deterministic and does not depend on the order in which
// blocks run: no block waits on another and no global atomics are used.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = kLayoutThreads;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ int key_bits(int E) {
    // number of bits needed for ids 0..E-1
    return (E <= 1) ? 0 : 32 - __clz(E - 1);
}

__global__ __launch_bounds__(kThreads) void layout_hist_kernel(
        const int32_t* __restrict__ idx, int64_t n, int E, int chunk,
        int32_t* __restrict__ block_hist) {
    extern __shared__ int32_t hist[];  // [E + 1]; hist[E] counts invalid ids
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e <= E; e += kThreads) hist[e] = 0;
    __syncthreads();

    const int nbits = key_bits(E);
    const int64_t begin = static_cast<int64_t>(b) * chunk;
    const int64_t end = (begin + chunk < n) ? begin + chunk : n;
    for (int64_t base = begin; base < begin + chunk; base += kThreads) {
        const int64_t i = base + threadIdx.x;
        const bool in = i < end;
        const int32_t key = in ? idx[i] : -1;
        const bool valid = in && static_cast<uint32_t>(key) < static_cast<uint32_t>(E);
        const uint64_t active = __ballot(valid);
        const uint64_t peers = match_peers(valid ? key : 0, nbits, active);
        if (valid && (peers & lanemask_lt()) == 0) atomicAdd(&hist[key], __popcll(peers));
        const uint64_t invalid = __ballot(in && !valid);
        if (lane_id() == 0 && invalid) atomicAdd(&hist[E], __popcll(invalid));
    }
    __syncthreads();
    int32_t* row = block_hist + static_cast<int64_t>(b) * (E + 1);
    for (int e = threadIdx.x; e <= E; e += kThreads) row[e] = hist[e];
}

// Inclusive scan across the 64 lanes of a wave.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t t = __shfl_up(v, d);
        if (lane >= static_cast<uint32_t>(d)) v += t;
    }
    return v;
}

__global__ __launch_bounds__(kThreads) void layout_rank_kernel(
        const int32_t* __restrict__ idx, int64_t n, int E, int cap, int chunk, int nblocks,
        int64_t R, const int32_t* __restrict__ block_hist, int32_t* __restrict__ count,
        int32_t* __restrict__ offset, int32_t* __restrict__ slot_of,
        int32_t* __restrict__ src_of_slot, int32_t* __restrict__ status) {
    extern __shared__ int32_t sm[];
    int32_t* total = sm;               // [E]    entries per expert, all blocks
    int32_t* prior = total + E;        // [E]    entries per expert in blocks before this one
    int32_t* off = prior + E;          // [E+1]  exclusive scan of total
    int32_t* run = off + E + 1;        // [kWaves][E] running first rank per wave
    __shared__ int32_t s_invalid, s_dropped;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const uint32_t lane = lane_id();

    // 1. Column sums of the block-histogram table, eight rows in flight.
    for (int e = tid; e <= E; e += kThreads) {
        int32_t tot = 0, pre = 0;
        int bb = 0;
        for (; bb + 8 <= nblocks; bb += 8) {
            int32_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = block_hist[static_cast<int64_t>(bb + q) * (E + 1) + e];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                tot += v[q];
                pre += (bb + q < b) ? v[q] : 0;
            }
        }
        for (; bb < nblocks; ++bb) {
            const int32_t v = block_hist[static_cast<int64_t>(bb) * (E + 1) + e];
            tot += v;
            pre += (bb < b) ? v : 0;
        }
        if (e < E) {
            total[e] = tot;
            prior[e] = pre;
        } else {
            s_invalid = tot;
        }
    }
    __syncthreads();

    // 2. Exclusive scan of total into off (wave 0; each lane owns a run of
    //    consecutive experts), and the number dropped by the capacity.
    if (wave == 0) {
        const int per = (E + kWave - 1) / kWave;
        const int e0 = min(E, static_cast<int>(lane) * per);
        const int e1 = min(E, e0 + per);
        int32_t local = 0, drop = 0;
        for (int e = e0; e < e1; ++e) {
            local += total[e];
            if (cap > 0 && total[e] > cap) drop += total[e] - cap;
        }
        const int32_t incl = wave_inclusive_scan(local);
        int32_t run_sum = incl - local;
        for (int e = e0; e < e1; ++e) {
            off[e] = run_sum;
            run_sum += total[e];
        }
        if (lane == kWave - 1) off[E] = incl;
        const int32_t drop_all = wave_inclusive_scan(drop);
        if (lane == kWave - 1) s_dropped = drop_all;
    }
    __syncthreads();

    if (b == 0) {
        for (int e = tid; e < E; e += kThreads) {
            count[e] = total[e];
            offset[e] = off[e];
        }
        if (tid == 0) {
            offset[E] = off[E];
            status[0] = s_invalid;
            status[1] = s_dropped;
        }
    }

    // 3. Per-wave histograms of this block's chunk.  Wave w owns the
    //    contiguous sub-chunk [begin + w*S, begin + (w+1)*S).
    const int nbits = key_bits(E);
    const int64_t begin = static_cast<int64_t>(b) * chunk;
    const int64_t end = (begin + chunk < n) ? begin + chunk : n;
    const int S = chunk / kWaves;
    const int64_t wbegin = begin + static_cast<int64_t>(wave) * S;
    int32_t* wrun = run + wave * E;
    for (int e = tid; e < kWaves * E; e += kThreads) run[e] = 0;
    __syncthreads();
    for (int step = 0; step < S; step += kWave) {
        const int64_t i = wbegin + step + lane;
        const bool in = i < end;
        const int32_t key = in ? idx[i] : -1;
        const bool valid = in && static_cast<uint32_t>(key) < static_cast<uint32_t>(E);
        const uint64_t peers = match_peers(valid ? key : 0, nbits, __ballot(valid));
        if (valid && (peers & lanemask_lt()) == 0) wrun[key] += __popcll(peers);
    }
    __syncthreads();

    // 4. First rank of each (wave, expert): entries in earlier blocks, then in
    //    earlier waves of this block.  For the contiguous layout the expert's
    //    offset is folded in, so the value is directly a receive row; for the
    //    fixed-capacity layout it stays the rank inside the expert.
    for (int e = tid; e < E; e += kThreads) {
        int32_t acc = prior[e] + (cap == 0 ? off[e] : 0);
        for (int w = 0; w < kWaves; ++w) {
            const int32_t c = run[w * E + e];
            run[w * E + e] = acc;
            acc += c;
        }
    }
    __syncthreads();

    // 5. Rank pass in (t, j) order: lane rank among same-expert lanes below it.
    for (int step = 0; step < S; step += kWave) {
        const int64_t i = wbegin + step + lane;
        const bool in = i < end;
        const int32_t key = in ? idx[i] : -1;
        const bool valid = in && static_cast<uint32_t>(key) < static_cast<uint32_t>(E);
        const uint64_t peers = match_peers(valid ? key : 0, nbits, __ballot(valid));
        int32_t first = 0;
        if (valid) first = wrun[key];
        if (valid && (peers & lanemask_lt()) == 0) wrun[key] = first + __popcll(peers);
        if (in) {
            int32_t slot = -1;
            if (valid) {
                const int32_t r = first + __popcll(peers & lanemask_lt());
                if (cap == 0) {
                    slot = r;
                } else if (r < cap) {
                    slot = key * cap + r;
                }
            }
            slot_of[i] = slot;
            if (slot >= 0 && slot < R) src_of_slot[slot] = static_cast<int32_t>(i);
        }
    }

    // 6. Receive rows that no entry fills get src_of_slot = -1.
    const int64_t gtid = static_cast<int64_t>(b) * kThreads + tid;
    const int64_t gstride = static_cast<int64_t>(nblocks) * kThreads;
    if (cap == 0) {
        for (int64_t r = off[E] + gtid; r < R; r += gstride) src_of_slot[r] = -1;
    } else {
        for (int64_t r = gtid; r < R; r += gstride) {
            const int e = static_cast<int>(r / cap);
            const int rr = static_cast<int>(r - static_cast<int64_t>(e) * cap);
            if (rr >= min(total[e], cap)) src_of_slot[r] = -1;
        }
    }
}

}  // namespace

LayoutGeometry layout_geometry(const ep_problem& p) {
    LayoutGeometry g;
    g.entries = static_cast<int64_t>(p.num_tokens) * p.num_topk;
    // Aim for at most ~32 blocks so that each block's column sums stay short,
    // with 1..64 entries per thread.
    constexpr int64_t kTargetBlocks = 32;
    int64_t per_thread = (g.entries + static_cast<int64_t>(kThreads) * kTargetBlocks - 1) /
                         (static_cast<int64_t>(kThreads) * kTargetBlocks);
    if (per_thread < 1) per_thread = 1;
    if (per_thread > 64) per_thread = 64;
    g.chunk = static_cast<int32_t>(per_thread * kThreads);
    int64_t blocks = (g.entries + g.chunk - 1) / g.chunk;
    g.blocks = static_cast<int32_t>(blocks < 1 ? 1 : blocks);
    return g;
}

int64_t layout_workspace_bytes(const ep_problem& p) {
    const LayoutGeometry g = layout_geometry(p);
    const int64_t bytes = static_cast<int64_t>(g.blocks) * (p.num_experts + 1) * 4;
    return ((bytes + 255) / 256) * 256;
}

hipError_t launch_layout(const ep_problem& p, const int32_t* topk_idx, const ep_layout_t& out,
                         int32_t* block_hist, hipStream_t stream) {
    const LayoutGeometry g = layout_geometry(p);
    const int E = p.num_experts;
    const int64_t R = (p.capacity == 0) ? g.entries
                                        : static_cast<int64_t>(E) * p.capacity;
    const size_t lds_hist = static_cast<size_t>(E + 1) * 4;
    hipLaunchKernelGGL(layout_hist_kernel, dim3(g.blocks), dim3(kThreads), lds_hist, stream,
                       topk_idx, g.entries, E, g.chunk, block_hist);
    const size_t lds_rank = static_cast<size_t>(3 * E + 1 + kWaves * E) * 4;
    hipLaunchKernelGGL(layout_rank_kernel, dim3(g.blocks), dim3(kThreads), lds_rank, stream,
                       topk_idx, g.entries, E, p.capacity, g.chunk, g.blocks, R, block_hist,
                       out.count, out.offset, out.slot_of, out.src_of_slot, out.status);
    return hipGetLastError();
}

}  // namespace ep
