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
    // count, offset and status come from workgroup 0; with fixed capacity the
    // others need neither offsets nor the whole histogram (they build it only
    // where that is cheaper than counting their own experts)
    const bool totals = small::whole_histogram(cap, b, E, nwg);
    if (totals) small::histogram(tab, n, E);
    else small::count_experts(tab, n, E, b, nwg);
    __syncthreads();

    // Entry q sits at position a + q: an id at position i is ahead of the
    // entries q > i - a.
    const uint64_t all = (cnt == 64) ? ~0ull : ((1ull << cnt) - 1);
    auto ahead = [&](int i) -> uint64_t {
        return (i < a) ? all : (all & (~0ull << (i - a + 1)));
    };
    small::count_ahead(tab, cnt > 0 ? a + cnt - 1 : 0, E, ahead, s_eq);
    if (totals) small::scan_offsets(tab, E, cap, &s_drop);
    __syncthreads();

    if (tid < cnt) {
        const int32_t slot = small::slot_for(tab, E, cap, tab.ids[a + tid], s_eq[tid]);
        slot_of[a + tid] = slot;
        if (slot >= 0 && slot < R) src_of_slot[slot] = a + tid;
    }
    if (b == 0) small::write_totals(tab, E, s_drop, count, offset, status);
    small::fill_empty_rows(tab, E, cap, R, b, nwg, src_of_slot);
}

// ---- mid-size tables: one kernel, every workgroup reads the whole table ------
//
// Workgroup b ranks entries [1024 b, 1024 b + 1024), one per lane.  It needs,
// per expert, the valid entries of the whole table (for the offsets) and
// those before its first entry P0 (for the ranks): it reads the whole table
// itself (served by L2 after the first workgroups of an XCD) and builds two
// LDS histograms split at P0.  An own entry's rank is then the ids ahead of
// P0 with its expert, plus the own entries of earlier waves with that expert
// (per-wave counts), plus the lower lanes of its wave with that expert (one
// ballot per key bit).  No workgroup waits for another; the one launch
// replaces the histogram and ranking kernels of the two-pass path.

constexpr int kWholeThreads = 1024;
constexpr int kWholeWaves = kWholeThreads / kWave;
constexpr int kWholeQuadSteps = 8;  // table quads a lane has in flight

// Copies of the two histograms: with few experts many lanes of one LDS
// atomic instruction hit the same bin (skewed routing more so), and the
// atomics to one address are applied one lane at a time; lane l counts into
// copy l mod nc, and the copies are summed once the table is counted.
__host__ __device__ inline int whole_copies(int E) { return E < 128 ? 8 : 1; }

__host__ __device__ inline size_t whole_lds_words(int E) {
    return static_cast<size_t>(2 * whole_copies(E) + 1 + kWholeWaves) * (E + 1);
}

__global__ __launch_bounds__(kWholeThreads) void layout_whole_kernel(
        const int32_t* __restrict__ idx, int n, int E, int cap, int64_t R, int nwg,
        int32_t* __restrict__ count, int32_t* __restrict__ offset, int32_t* __restrict__ slot_of,
        int32_t* __restrict__ src_of_slot, int32_t* __restrict__ status) {
    extern __shared__ __align__(16) int32_t sm[];
    __shared__ int32_t s_wsum[kWholeWaves];
    __shared__ int32_t s_wover[kWholeWaves];
    const int W = E + 1;
    const int nc = whole_copies(E);
    int32_t* part = sm;            // [nc][2][E+1]: ids before P0, the rest (bin E: invalid)
    int32_t* off = sm + nc * 2 * W;  // [E+1]
    int32_t* wcnt = off + W;       // [waves][E+1]: own entries per expert of each wave

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = static_cast<int>(lane_id());
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int b = static_cast<int>(blockIdx.x);
    const int P0 = b * kWholeThreads;
    const int i_own = P0 + tid;
    const bool has_own = i_own < n;
    // the own entry first: a wave's loads return in issue order
    const int32_t own_id = idx[has_own ? i_own : n - 1];
    for (int e = tid; e < (2 * nc + kWholeWaves) * W; e += kWholeThreads)
        (e < 2 * nc * W ? part[e] : wcnt[e - 2 * nc * W]) = 0;
    __syncthreads();

    // Own entries: rank among the lower lanes of the wave, and per-wave
    // counts (the lowest lane of each expert's peers records them).
    const bool mine = has_own && valid_id(own_id, E);
    const uint64_t peers = match_peers(static_cast<uint32_t>(mine ? own_id : 0), key_bits(E),
                                       __ballot(mine));
    const uint64_t lower = peers & lanemask_lt();
    if (mine && lower == 0) wcnt[wave * W + own_id] = __popcll(peers);

    // Histograms of the whole table, split at P0: kWholeQuadSteps 16-byte
    // loads per lane in flight, then their counts.
    const int nq = n / 4;
    const int4* quads = reinterpret_cast<const int4*>(idx);
    int32_t* mypart = part + (lane & (nc - 1)) * 2 * W;
    for (int q0 = 0; q0 < nq; q0 += kWholeQuadSteps * kWholeThreads) {
        int4 g[kWholeQuadSteps];
#pragma unroll
        for (int u = 0; u < kWholeQuadSteps; ++u)
            g[u] = quads[min(q0 + u * kWholeThreads + tid, nq - 1)];
#pragma unroll
        for (int u = 0; u < kWholeQuadSteps; ++u) {
            const int qi = q0 + u * kWholeThreads + tid;
            if (qi < nq) {
                const int32_t id4[4] = {g[u].x, g[u].y, g[u].z, g[u].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int32_t id = id4[c];
                    atomicAdd(&mypart[(valid_id(id, E) ? id : E) + (4 * qi + c < P0 ? 0 : W)], 1);
                }
            }
        }
    }
    if (tid < n - 4 * nq) {  // the last n % 4 ids
        const int i = 4 * nq + tid;
        const int32_t id = idx[i];
        atomicAdd(&mypart[(valid_id(id, E) ? id : E) + (i < P0 ? 0 : W)], 1);
    }
    __syncthreads();
    if (nc > 1) {  // uniform
        for (int e = tid; e < 2 * W; e += kWholeThreads) {
            int32_t sum = part[e];
            for (int c = 1; c < nc; ++c) sum += part[c * 2 * W + e];
            part[e] = sum;
        }
        __syncthreads();
    }

    // Offsets: exclusive scan of the totals over experts (E <= 1024: one lane
    // per expert), and the entries the capacity drops.
    int32_t tot = 0, over = 0;
    if (tid < E) {
        tot = part[tid] + part[W + tid];
        over = (cap > 0 && tot > cap) ? tot - cap : 0;
    }
    const int32_t incl = wave_inclusive_scan(tot);
    const int32_t oincl = wave_inclusive_scan(over);
    if (lane == kWave - 1) {
        s_wsum[wave] = incl;
        s_wover[wave] = oincl;
    }
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += s_wsum[w];
    if (tid < E) {
        off[tid] = before + incl - tot;
        if (b == 0) {
            count[tid] = tot;
            offset[tid] = before + incl - tot;
        }
    }
    if (tid == 0) {
        int32_t valid = 0, drop = 0;
        for (int w = 0; w < kWholeWaves; ++w) {
            valid += s_wsum[w];
            drop += s_wover[w];
        }
        off[E] = valid;
        if (b == 0) {
            offset[E] = valid;
            status[0] = part[E] + part[W + E];
            status[1] = drop;
        }
    }
    __syncthreads();

    if (has_own) {
        int32_t slot = -1;
        if (mine) {
            int32_t r = part[own_id] + __popcll(lower);
            for (int w = 0; w < wave; ++w) r += wcnt[w * W + own_id];
            if (cap == 0) slot = off[own_id] + r;
            else if (r < cap) slot = own_id * cap + r;
        }
        slot_of[i_own] = slot;
        if (slot >= 0 && slot < R) src_of_slot[slot] = i_own;
    }
    // Receive rows no entry fills: past each expert's count (fixed capacity,
    // experts b, b + nwg, ...), or past the valid entries (contiguous).
    if (cap > 0) {
        for (int e = b; e < E; e += nwg) {
            int32_t* rows = src_of_slot + static_cast<int64_t>(e) * cap;
            const int32_t filled = min(part[e] + part[W + e], cap);
            for (int r = filled + tid; r < cap; r += kWholeThreads) rows[r] = -1;
        }
    } else {
        for (int64_t r = off[E] + static_cast<int64_t>(b) * kWholeThreads + tid; r < R;
             r += static_cast<int64_t>(nwg) * kWholeThreads)
            src_of_slot[r] = -1;
    }
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

bool layout_whole_fits(const ep_problem& p) {
    const int64_t n = static_cast<int64_t>(p.num_tokens) * p.num_topk;
    // Every workgroup counts the whole table, so past 65536 entries the
    // histogram and ranking kernels are faster (16384 x 8 over 256 experts:
    // about 16 against 15 us; 4096 x 8: about 8 against 12 us, event-timed).
    // Below 128 experts the histograms need their copies (one copy: the
    // skewed 8192 x 6 table over 64 experts took 12.5 us against 4.6 + 5.6 us
    // for the two kernels); with 8 copies the FP8 layout + dispatch call of
    // that table is 61.6-62.6 against 63.0-63.7 us, also about 1 us faster at
    // 32 and 96 experts, and 0.4 us slower at 16 (event-timed, the benchmark's
    // order of calls).
    return n > kFusedMaxEntries && n <= kWholeMaxEntries && p.num_experts >= kWholeMinExperts &&
           whole_lds_words(p.num_experts) * 4 <= 65536;
}

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
    if (layout_whole_fits(p)) {
        const int n = static_cast<int>(g.entries);
        const int nwg = (n + kWholeThreads - 1) / kWholeThreads;
        hipLaunchKernelGGL(layout_whole_kernel, dim3(nwg), dim3(kWholeThreads),
                           whole_lds_words(E) * 4, stream, topk_idx, n, E, p.capacity, R, nwg,
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
