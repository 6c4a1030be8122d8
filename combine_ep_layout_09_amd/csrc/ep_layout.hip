// ep_layout.hip -- routing layout: per-expert histogram, exclusive scan into
// expert-major offsets, and a stable slot for every routing entry.
//
// The count per expert and the expert-major receive rows follow the
// low-latency dispatch of "[GH-ISSUE #282] Redundant atomics in internode_ll"
// (per-expert token counts, receive counts indexed by local expert); the
// stable order inside an expert follows the order-consistency requirement in
// "[GH-ISSUE #18] Reasons for not calling NVSHMEM public APIs?".
//
// Small tables (up to kFusedMaxEntries entries: decode-sized batches): one
// kernel, in which every workgroup stages the whole routing table in LDS,
// builds its histogram there, and ranks 64 entries by looking the ids ahead
// of them up in a per-expert mask of those entries (ep_small_dev.h).  No
// workgroup waits for another.
//
// Larger tables: the T*k entries (row-major (t, j) order) are split into
// blocks of `chunk` consecutive entries; each workgroup ranks one block.
// Before it can rank, a workgroup needs, per expert, the number of valid
// entries in the whole table (for the offsets) and in the blocks before its
// own (for the ranks).  layout_hist writes each block's histogram to
// a column-major table in the workspace (64 rows per column, zero padded);
// layout_rank reads the whole table as 1 KiB per wave instruction, 16 lanes
// (one DPP row) per column, and row-reduces each column into its total and
// its part before this block.  The kernel boundary is the only
// synchronisation between blocks.
//
// Ranking a block: its entries are split into one contiguous
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
#include "ep_small_dev.h"

namespace ep {
namespace {

using namespace layout;

// ---- small tables: one kernel --------------------------------------------------

// Workgroup b ranks entries [64b, 64b + 64); the whole table is staged in its
// LDS (ep_small_dev.h).
__global__ __launch_bounds__(small::kThreads) void layout_small_kernel(
        const int32_t* __restrict__ idx, int n, int E, int cap, int64_t R, int nwg,
        int32_t* __restrict__ count, int32_t* __restrict__ offset, int32_t* __restrict__ slot_of,
        int32_t* __restrict__ src_of_slot, int32_t* __restrict__ status) {
    __shared__ int32_t s_eq[small::kMaxEntries];
    __shared__ int32_t s_drop;
    extern __shared__ __align__(16) int32_t s_dyn[];
    const small::Tables tab = small::carve(s_dyn, n, E);
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int a = b * small::kMaxEntries;  // this workgroup's first entry
    const int cnt = max(0, min(small::kMaxEntries, n - a));

    small::IdStage stage;
    stage.load(idx, n);
    stage.store(n, tab.ids);
    small::zero_tables(tab, E);
    if (tid < small::kMaxEntries) s_eq[tid] = 0;
    __syncthreads();

    if (tid < cnt) small::mark_entry(tab, E, tid, tab.ids[a + tid]);
    small::histogram(tab, n, E);
    __syncthreads();

    // Entry q sits at position a + q: an id at position i is ahead of the
    // entries q > i - a.
    const uint64_t all = (cnt == 64) ? ~0ull : ((1ull << cnt) - 1);
    auto ahead = [&](int i) -> uint64_t {
        return (i < a) ? all : (all & (~0ull << (i - a + 1)));
    };
    small::count_ahead(tab, cnt > 0 ? a + cnt - 1 : 0, E, ahead, s_eq);
    small::scan_offsets(tab, E, cap, &s_drop);
    __syncthreads();

    if (tid < cnt) {
        const int32_t slot = small::slot_for(tab, E, cap, tab.ids[a + tid], s_eq[tid]);
        slot_of[a + tid] = slot;
        if (slot >= 0 && slot < R) src_of_slot[slot] = a + tid;
    }
    if (b == 0) small::write_totals(tab, E, s_drop, count, offset, status);
    small::fill_empty_rows(tab, E, cap, R, b, nwg, src_of_slot);
}

// ---- two-pass path -----------------------------------------------------------

template <bool PREFIX>
__global__ __launch_bounds__(kHistThreads) void layout_hist_kernel(
        const int32_t* __restrict__ idx, int64_t n, int E, int chunk, int nblocks,
        int32_t* __restrict__ block_hist, int32_t* __restrict__ status) {
    extern __shared__ int32_t hist[];  // [E + 1]; hist[E] counts invalid ids
    hist_block<PREFIX>(blockIdx.x, hist, idx, n, E, chunk, nblocks, block_hist, status);
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
    g.single_pass = g.entries <= kFusedMaxEntries;
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
    // the block-histogram table of the two-pass path, and the table of
    // per-block expert prefixes that the ranking dispatch kernel reads
    const int64_t bytes = 2 * static_cast<int64_t>(kTableStride) * (p.num_experts + 1) * 4;
    return ((bytes + 255) / 256) * 256;
}
static_assert(kTableStride == 64, "kMaxLayoutWorkspaceBytes assumes 64-row table columns");

hipError_t launch_layout_tables(const ep_problem& p, const int32_t* topk_idx,
                                const LayoutGeometry& g, int32_t* workspace, int32_t* status,
                                hipStream_t stream) {
    const size_t lds_hist = static_cast<size_t>(p.num_experts + 1) * 4;
    hipLaunchKernelGGL(layout_hist_kernel<true>, dim3(g.blocks), dim3(kHistThreads), lds_hist,
                       stream, topk_idx, g.entries, p.num_experts, g.chunk, g.blocks, workspace,
                       status);
    return hipGetLastError();
}

hipError_t launch_layout(const ep_problem& p, const int32_t* topk_idx, const ep_layout_t& out,
                         int32_t* workspace, hipStream_t stream) {
    const LayoutGeometry g = layout_geometry(p);
    int32_t* block_hist = workspace;
    const int E = p.num_experts;
    const int64_t R = (p.capacity == 0) ? g.entries : static_cast<int64_t>(E) * p.capacity;
    if (g.single_pass) {
        const int n = static_cast<int>(g.entries);
        const int nwg = n > 0 ? (n + small::kMaxEntries - 1) / small::kMaxEntries : 1;
        hipLaunchKernelGGL(layout_small_kernel, dim3(nwg), dim3(small::kThreads),
                           small::lds_bytes(n, E), stream, topk_idx, n, E, p.capacity, R, nwg,
                           out.count, out.offset, out.slot_of, out.src_of_slot, out.status);
        return hipGetLastError();
    }
    const size_t lds_hist = static_cast<size_t>(E + 1) * 4;
    hipLaunchKernelGGL(layout_hist_kernel<false>, dim3(g.blocks), dim3(kHistThreads), lds_hist,
                       stream, topk_idx, g.entries, E, g.chunk, g.blocks, block_hist, nullptr);
    hipLaunchKernelGGL(layout_rank_kernel, dim3(g.blocks), dim3(kRankThreads), rank_lds_bytes(E),
                       stream, topk_idx, g.entries, E, p.capacity, g.chunk, g.blocks, R,
                       block_hist, out.count, out.offset, out.slot_of, out.src_of_slot,
                       out.status);
    return hipGetLastError();
}

}  // namespace ep
