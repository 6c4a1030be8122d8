// ep_layout.hip -- routing layout: per-expert histogram, exclusive scan into
// expert-major offsets, and a stable slot for every routing entry.
//
// The count per expert and the expert-major receive rows follow the
// low-latency dispatch of "[GH-ISSUE #282] Redundant atomics in internode_ll"
// (per-expert token counts, receive counts indexed by local expert); the
// stable order inside an expert follows the order-consistency requirement in
// "[GH-ISSUE #18] Reasons for not calling NVSHMEM public APIs?".
//
// The T*k entries (row-major (t, j) order) are split into blocks of `chunk`
// consecutive entries; each workgroup ranks one block.  Before it can rank, a
// workgroup needs, per expert, the number of valid entries in the whole table
// (for the offsets) and in the blocks before its own (for the ranks).
//
// Single-pass path (tables up to kSinglePassMaxEntries entries: decode-sized
// batches): one kernel.  Every workgroup reads the whole routing table and
// builds both histograms itself with LDS atomics; no workgroup waits on
// another.  LDS atomics cost about one wave instruction per 64 entries per
// workgroup, which is why this path stops at small tables.
//
// Two-pass path (larger tables): layout_hist writes each block's histogram to
// a column-major table in the workspace (64 rows per column, zero padded);
// layout_rank reads the whole table as 1 KiB per wave instruction, 16 lanes
// (one DPP row) per column, and row-reduces each column into its total and
// its part before this block.  The kernel boundary is the only
// synchronisation between blocks.
//
// Ranking, in both paths: the block's entries are split into one contiguous
// run per ranking wave.  A wave loads its run's ids into registers before
// anything else, so its own histogram (per-wave counts in LDS) is built while
// the table loads are still in flight.  After one barrier, wave 0 scans the
// totals into offsets, and each expert's per-wave counts are scanned across
// waves (one 16-lane DPP row per expert) into every wave's first rank.
// Inside a wave, each 64-entry step ranks a lane against the lower lanes with
// the same expert, found with one ballot per key bit.  All workgroups
// together mark empty receive rows with -1.  The result is deterministic and
// independent of workgroup scheduling.

#include "ep_layout_dev.h"

namespace ep {
namespace {

using namespace layout;

// ---- single-pass path --------------------------------------------------------

__global__ __launch_bounds__(kRankThreads) void layout_single_kernel(
        const int32_t* __restrict__ idx, int64_t n, int E, int cap, int chunk, int nblocks,
        int64_t R, int32_t* __restrict__ count, int32_t* __restrict__ offset,
        int32_t* __restrict__ slot_of, int32_t* __restrict__ src_of_slot,
        int32_t* __restrict__ status) {
    extern __shared__ __align__(16) int32_t sm[];
    __shared__ int32_t s_invalid, s_dropped;
    const RankLds l = carve(sm, E);
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const uint32_t lane = lane_id();
    const int rw = rank_waves(E);
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t end = (begin + chunk < n) ? begin + chunk : n;
    const Run r = wave_run(begin, end, chunk, rw, wave);
    int32_t key[kKeySteps];
    load_pass(idx, r.wbegin, r.wend, lane, key);

    for (int e = tid; e < E; e += kRankThreads) {
        l.total[e] = 0;
        l.prior[e] = 0;
    }
    int32_t* wrun = l.run + wave * (E + 1);
    if (wave < rw)
        for (int e = lane; e <= E; e += kWave) wrun[e] = 0;
    if (tid == 0) s_invalid = 0;
    __syncthreads();

    // Whole-table histogram, and the histogram of the entries before this
    // block.  Each lane reads 16-byte groups of 4 entries, kGroups groups in
    // flight per pass (idx is 16-byte aligned; the last, partial group is read
    // entry by entry).
    constexpr int kGroups = 8;
    const int64_t ngroups = (n + 3) / 4;
    const int4* idx4 = reinterpret_cast<const int4*>(idx);
    int32_t invalid = 0;
    for (int64_t g0 = 0; g0 < ngroups; g0 += kGroups * kRankThreads) {
        int4 q[kGroups];
#pragma unroll
        for (int u = 0; u < kGroups; ++u) {
            const int64_t g = g0 + u * kRankThreads + tid;
            if (4 * g + 3 < n) {
                q[u] = idx4[g];
            } else {
                q[u].x = (4 * g + 0 < n) ? idx[4 * g + 0] : E;
                q[u].y = (4 * g + 1 < n) ? idx[4 * g + 1] : E;
                q[u].z = (4 * g + 2 < n) ? idx[4 * g + 2] : E;
                q[u].w = E;
            }
        }
#pragma unroll
        for (int u = 0; u < kGroups; ++u) {
            const int64_t i0 = 4 * (g0 + u * kRankThreads + tid);
            const int32_t k4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (valid_id(k4[c], E)) {
                    atomicAdd(&l.total[k4[c]], 1);
                    if (i0 + c < begin) atomicAdd(&l.prior[k4[c]], 1);
                } else if (i0 + c < n) {
                    ++invalid;
                }
            }
        }
    }
    if (invalid) atomicAdd(&s_invalid, invalid);
    if (wave < rw) count_run(idx, r, key, lane, E, key_bits(E), wrun);
    __syncthreads();

    finish_layout(blockIdx.x, idx, n, E, cap, nblocks, R, l, r, key, s_invalid, &s_dropped, count,
                  offset, slot_of, src_of_slot, status);
}

// ---- two-pass path -----------------------------------------------------------

__global__ __launch_bounds__(kHistThreads) void layout_hist_kernel(
        const int32_t* __restrict__ idx, int64_t n, int E, int chunk, int nblocks,
        int32_t* __restrict__ block_hist) {
    extern __shared__ int32_t hist[];  // [E + 1]; hist[E] counts invalid ids
    hist_block(blockIdx.x, hist, idx, n, E, chunk, nblocks, block_hist);
}

__global__ __launch_bounds__(kRankThreads) void layout_rank_kernel(
        const int32_t* __restrict__ idx, int64_t n, int E, int cap, int chunk, int nblocks,
        int64_t R, const int32_t* __restrict__ block_hist, int32_t* __restrict__ count,
        int32_t* __restrict__ offset, int32_t* __restrict__ slot_of,
        int32_t* __restrict__ src_of_slot, int32_t* __restrict__ status) {
    extern __shared__ __align__(16) int32_t sm[];
    rank_block<>(blockIdx.x, sm, idx, n, E, cap, chunk, nblocks, R, block_hist, count, offset,
                 slot_of, src_of_slot, status);
}

}  // namespace

LayoutGeometry layout_geometry(const ep_problem& p) {
    LayoutGeometry g;
    g.entries = static_cast<int64_t>(p.num_tokens) * p.num_topk;
    g.single_pass = g.entries <= kSinglePassMaxEntries;
    // Up to 64 workgroups (single pass: each pays for the whole-table
    // histogram; two passes: the table has 64 rows per column).  Chunks are
    // multiples of 256 entries (16-byte groups of the histogram kernel, whole
    // 64-entry ranking steps).
    int64_t chunk = (g.entries + kTwoPassMaxBlocks - 1) / kTwoPassMaxBlocks;
    chunk = ((chunk + 255) / 256) * 256;
    if (chunk < 256) chunk = 256;
    g.chunk = static_cast<int32_t>(chunk);
    const int64_t blocks = (g.entries + chunk - 1) / chunk;
    g.blocks = static_cast<int32_t>(blocks < 1 ? 1 : blocks);
    return g;
}

LayoutGeometry layout_geometry_two_pass(const ep_problem& p) {
    LayoutGeometry g = layout_geometry(p);
    g.single_pass = false;
    return g;
}

int64_t layout_workspace_bytes(const ep_problem& p) {
    // the block-histogram table of the two-pass path
    const int64_t bytes = static_cast<int64_t>(kTableStride) * (p.num_experts + 1) * 4;
    return ((bytes + 255) / 256) * 256;
}

hipError_t launch_layout(const ep_problem& p, const int32_t* topk_idx, const ep_layout_t& out,
                         int32_t* workspace, hipStream_t stream) {
    const LayoutGeometry g = layout_geometry(p);
    int32_t* block_hist = workspace;
    const int E = p.num_experts;
    const int64_t R = (p.capacity == 0) ? g.entries : static_cast<int64_t>(E) * p.capacity;
    if (g.single_pass) {
        hipLaunchKernelGGL(layout_single_kernel, dim3(g.blocks), dim3(kRankThreads),
                           rank_lds_bytes(E), stream, topk_idx, g.entries, E, p.capacity,
                           g.chunk, g.blocks, R, out.count, out.offset, out.slot_of,
                           out.src_of_slot, out.status);
        return hipGetLastError();
    }
    const size_t lds_hist = static_cast<size_t>(E + 1) * 4;
    hipLaunchKernelGGL(layout_hist_kernel, dim3(g.blocks), dim3(kHistThreads), lds_hist, stream,
                       topk_idx, g.entries, E, g.chunk, g.blocks, block_hist);
    hipLaunchKernelGGL(layout_rank_kernel, dim3(g.blocks), dim3(kRankThreads), rank_lds_bytes(E),
                       stream, topk_idx, g.entries, E, p.capacity, g.chunk, g.blocks, R,
                       block_hist, out.count, out.offset, out.slot_of, out.src_of_slot,
                       out.status);
    return hipGetLastError();
}

}  // namespace ep
