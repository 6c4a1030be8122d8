// ep_fused.hip -- ep_layout_dispatch: the routing layout and the dispatch of
// token rows with fewer launches than ep_layout followed by ep_dispatch.
//
// For routing entry i = t*k + j with valid expert e:
//   rank(i)   = #{entries before i with id e}           (stable counting sort)
//   offset[e] = #{valid ids below e}                    (exclusive scan of count)
//   slot      = offset[e] + rank   (contiguous)
//             = e*cap + rank if rank < cap, else -1     (fixed capacity)
// which is what ep_layout computes; the results of both forms below are
// identical to ep_layout followed by ep_dispatch.
//
// Small routing tables (decode batches): one kernel.  Decode-sized batches
// move little data, so separate layout and dispatch kernels are bound by
// launches and by the layout's chain of dependent memory round trips.  Here
// no workgroup waits for another: every workgroup derives, from the whole
// table staged in its LDS, exactly the slots it needs (ep_small_dev.h), while
// its token rows load.  Two maintainer answers on the pages bear on this:
// in "[GH-ISSUE #18] Reasons for not calling NVSHMEM public APIs?" the sync
// and atomic operations a general API performs are named as too costly for
// microsecond-level latency (here: no workgroup waits for another), and in
// "[GH-ISSUE #166] Why does DeepEP LL kernel use double send/recv/signal
// buffers?" the clearing of the next buffer runs in parallel with the use of
// the current one to save latency (here: the only clearing the layout needs,
// marking unused receive rows, runs inside the same kernel, beside the row
// stores, rather than as a pass of its own).  Workgroup b scatters
// items 2b and 2b+1 (token, column tile), one per 128-lane group, as the
// dispatch kernel does; its entries are the 2k entries of those two tokens.
// Tile 0 of a token writes its slot_of and src_of_slot entries.  Workgroup b
// also marks the empty receive rows of experts b, b + D, b + 2D, ... (D
// workgroups; contiguous layout: the rows past the valid entries, strided
// over the workgroups), and workgroup 0 writes count, offset and status.
//
// Larger tables (prefill batches): two kernels instead of three.  The
// histogram kernel of the layout also writes, per block of entries, the
// exclusive scan of the block's counts over experts; the dispatch kernel
// then finds each token's slots itself from two table columns per entry and
// the block's ids ahead of the token, before it loads the row (see
// layout_dispatch_ranked_kernel).

#include "ep_dispatch_dev.h"
#include "ep_internal.h"
#include "ep_small_dev.h"

namespace ep {
namespace {

using dispatch::Bf16Tile;
using dispatch::Fp8Tile;
using dispatch::u32x2;
using dispatch::u32x4;
using small::kThreads;

constexpr int kGroupThreads = 128;  // one scatter item per group
constexpr int kGroups = kThreads / kGroupThreads;

static_assert(kGroupThreads % kWave == 0, "groups are whole waves");
static_assert(kGroupThreads >= kMaxTopk, "one lane per routing entry of a token");
static_assert(kGroups * kMaxTopk <= small::kMaxEntries, "a workgroup's entries fit a mask");
static_assert(kGroups == 2, "two tokens per workgroup");

struct SmallParams {
    const int32_t* idx;
    int n;  // T * k <= kFusedMaxEntries
    int E, cap;
    int64_t R;
    int32_t* count;
    int32_t* offset;
    int32_t* slot_of;
    int32_t* src_of_slot;
    int32_t* status;
    const u32x4* x;
    void* recv_x;
    void* recv_scales;  // fp32 scales or UE8M0 bytes
    int T, k, nvec, tiles, nwg;
};

// Mask of the entries of a k-entry token starting at position `start` (bits
// [base, base + k)) that lie after position i.
__device__ inline uint64_t token_ahead(int i, int start, int k, int base) {
    const uint64_t all = ((k == 64) ? ~0ull : ((1ull << k) - 1)) << base;
    if (i < start) return all;
    const int d = i - start + 1;  // the token's entries at or before i
    return (d >= k) ? 0ull : (all & (~0ull << (base + d)));
}

// MODE: 0 bf16 payload, 1 E4M3FN + fp32 scales, 2 E4M3FN + UE8M0 scales.
template <int VPL, int MODE>
__global__ __launch_bounds__(kThreads) void layout_dispatch_small_kernel(SmallParams p) {
    constexpr bool FP8 = MODE != 0;
    __shared__ int32_t s_eq[small::kMaxEntries];
    __shared__ int32_t s_slot[kGroups][kMaxTopk];
    __shared__ int32_t s_drop;
    __shared__ float s_scale[kGroups][kGroupThreads * VPL / 16 > 0 ? kGroupThreads * VPL / 16 : 1];
    extern __shared__ __align__(16) int32_t s_dyn[];

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int g = tid / kGroupThreads;
    const int gtid = tid % kGroupThreads;
    const int k = p.k;
    const int E = p.E;
    const small::Tables tab = small::carve(s_dyn, p.n, E);
    const int items = p.T * p.tiles;
    // the same for every lane of a wave (a group is whole waves)
    const int item = __builtin_amdgcn_readfirstlane(b * kGroups + g);
    const bool active = item < items;
    const int t = active ? item / p.tiles : 0;
    const int tile = active ? item % p.tiles : 0;
    const int e0 = t * k;  // the token's first entry

    // Global loads first: the routing table, then the row.
    small::IdStage stage;
    stage.load(p.idx, p.n);
    Bf16Tile<VPL> bt;
    Fp8Tile<VPL, MODE == 2> ft;
    if (active) {
        if (FP8) ft.load(p.x, p.nvec, t, tile, kGroupThreads, gtid);
        else bt.load(p.x, p.nvec, t, tile, kGroupThreads, gtid);
    }
    stage.store(p.n, tab.ids);
    small::zero_tables(tab, E);
    if (tid < small::kMaxEntries) s_eq[tid] = 0;
    __syncthreads();

    // Entry j of group gq is mask bit gq*k + j.  The token starts of the two
    // groups (an inactive group has no entries).
    int start[kGroups];
    bool live[kGroups];
#pragma unroll
    for (int gq = 0; gq < kGroups; ++gq) {
        const int it = b * kGroups + gq;
        live[gq] = it < items;
        start[gq] = live[gq] ? (it / p.tiles) * k : 0;
    }
    if (tid < kGroups * k) {
        const int gq = tid / k;
        if (live[gq]) small::mark_entry(tab, E, tid, tab.ids[start[gq] + (tid - gq * k)]);
    }
    // count, offset and status come from workgroup 0; with fixed capacity the
    // others need neither offsets nor the whole histogram (they build it only
    // where that is cheaper than counting their own experts)
    const bool totals = small::whole_histogram(p.cap, b, E, p.nwg);
    if (totals) small::histogram(tab, p.n, E);
    else small::count_experts(tab, p.n, E, b, p.nwg);
    __syncthreads();

    // Equal ids ahead of each entry, up to the last entry of the later token.
    int end = 0;
#pragma unroll
    for (int gq = 0; gq < kGroups; ++gq)
        if (live[gq]) end = max(end, start[gq] + k - 1);
    auto ahead = [&](int i) -> uint64_t {
        uint64_t m = 0;
#pragma unroll
        for (int gq = 0; gq < kGroups; ++gq)
            if (live[gq]) m |= token_ahead(i, start[gq], k, gq * k);
        return m;
    };
    small::count_ahead(tab, end, E, ahead, s_eq);
    if (totals) small::scan_offsets(tab, E, p.cap, &s_drop);
    if (FP8 && active) ft.quantise(p.nvec, tile, kGroupThreads, gtid, s_scale[g]);
    __syncthreads();

    if (active && gtid < k) {
        const int j = gtid;
        const int32_t slot = small::slot_for(tab, E, p.cap, tab.ids[e0 + j], s_eq[g * k + j]);
        s_slot[g][j] = slot;
        if (tile == 0) {
            p.slot_of[e0 + j] = slot;
            if (slot >= 0 && slot < p.R) p.src_of_slot[slot] = e0 + j;
        }
    }
    if (b == 0) small::write_totals(tab, E, s_drop, p.count, p.offset, p.status);
    __syncthreads();

    if (active) {
        const int32_t* slots = s_slot[g];
        const int32_t slot_vec = (lane_id() < static_cast<uint32_t>(k)) ? slots[lane_id()] : -1;
        if (FP8) {
            ft.store_lanes(slot_vec, k, p.R, static_cast<u32x2*>(p.recv_x), p.nvec);
            if (MODE == 2)
                dispatch::fp8_store_scales(s_scale[g], slots, k, p.R,
                                           static_cast<uint8_t*>(p.recv_scales), p.nvec / 16,
                                           tile, kGroupThreads, VPL, gtid);
            else
                dispatch::fp8_store_scales(s_scale[g], slots, k, p.R,
                                           static_cast<float*>(p.recv_scales), p.nvec / 16, tile,
                                           kGroupThreads, VPL, gtid);
        } else {
            bt.store_lanes(slot_vec, k, p.R, static_cast<u32x4*>(p.recv_x), p.nvec);
        }
    }
    small::fill_empty_rows(tab, E, p.cap, p.R, b, p.nwg, p.src_of_slot);
}

// ---- larger tables: histogram kernel, then a dispatch kernel that ranks ----

struct RankedParams {
    const int32_t* idx;
    int E, cap, k, chunk;
    int64_t R;
    const int32_t* hist;    // [E + 1][kTableStride] block counts (column E: invalid ids)
    const int32_t* prefix;  // [E + 1][kTableStride] block scans over experts (column E: valid)
    int32_t* count;
    int32_t* offset;
    int32_t* slot_of;
    int32_t* src_of_slot;
    int32_t* status;
    const u32x4* x;
    void* recv_x;
    void* recv_scales;  // fp32 scales or UE8M0 bytes
    int T, nvec;
};

using layout::kTableStride;
using layout::row16_inclusive_scan;
using layout::valid_id;

// Loads the 16-byte groups of table column `col` that lane grp (0..15) of a
// DPP row owns: rows 4 grp .. 4 grp + 3.
__device__ __forceinline__ int4 column_group(const int32_t* __restrict__ table, int col, int grp) {
    return reinterpret_cast<const int4*>(table + static_cast<int64_t>(col) * kTableStride)[grp];
}

// One workgroup per (token t, column tile), shaped like the dispatch kernels.
// The slot of the token's entry i = t*k + j with valid expert e, in block
// B = i / chunk, is
//   offset[e]        = sum over blocks of the block's count of valid ids below e
//   + before_B[e]    = sum over blocks before B of the block's count of e
//   + equal ids ahead of i in block B,
// the first two from the histogram kernel's tables (one column of each per
// entry, summed by a 16-lane DPP row), the last from the block's ids, looked
// up in a per-expert mask of the token's entries, as the small-table kernels
// do.  With fixed capacity the rank (the last two terms) gives the row
// e*cap + rank when below cap.  Tile 0 of token t writes its slot_of and
// src_of_slot entries, and also the totals of columns t, t + T, ...:
// count[e], offset[e], with column E offset[E] and status[0]; receive rows no
// entry fills get src_of_slot = -1 and, with fixed capacity, the rows an
// expert loses to the capacity are added to status[1] (zeroed by the
// histogram kernel).
template <int VPL, int MODE>
__global__ __launch_bounds__(1024) void layout_dispatch_ranked_kernel(RankedParams p) {
    constexpr bool FP8 = MODE != 0;
    constexpr int IDS = 8;  // block ids per lane and pass
    __shared__ uint32_t s_map[kMaxExperts];  // bit j: entry j of this token has id e
    __shared__ int32_t s_ahead[kMaxTopk];    // equal ids ahead of entry j in its block
    __shared__ int32_t s_sum[2][kMaxTopk];   // entry j: offset[e], count of e in earlier blocks
    __shared__ int32_t s_slot[kMaxTopk];
    __shared__ int32_t s_col[2];
    extern __shared__ float s_scale[];  // FP8: block scales of this tile

    const int t = blockIdx.x;
    const int tile = blockIdx.y;
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const uint32_t lane = lane_id();
    const int k = p.k;
    const int E = p.E;
    const int e0 = t * k;                      // T * k < 2^31
    const int lo = (e0 / p.chunk) * p.chunk;   // start of the block of entry e0
    // Positions below are relative to lo: the token's entries are at
    // [first, first + k), and the ids ahead of any of them lie in [0, end).
    const int first = e0 - lo;
    const int end = first + k - 1;
    const int span = IDS * nth;  // ids per pass of the workgroup

    // The slots come first, the row last.  A wave's vector memory results
    // return in the order its loads were issued, behind whatever the CU has
    // queued before them; table loads issued after the row would wait for
    // the rows of every workgroup on the CU, and no store could start until
    // then.  So: the token's ids (each wave its own copy; a clamped address,
    // so that the load is unconditional) and the block's ids up to the token
    // (one load per lane and step; a lane past the token loads nothing) ...
    const int32_t tok = p.idx[e0 + min(static_cast<int>(lane), k - 1)];
    const int32_t my_id = (lane < static_cast<uint32_t>(k)) ? tok : -1;
    int32_t ids[IDS];
#pragma unroll
    for (int u = 0; u < IDS; ++u) {
        ids[u] = -1;
        if (u * nth + tid < end) ids[u] = p.idx[lo + u * nth + tid];
    }
    for (int e = tid; e < E; e += nth) s_map[e] = 0;
    if (tid < k) s_ahead[tid] = 0;

    // ... then, once the token's ids are in, the table columns of entry
    // j = tid / 16 (first round) by its DPP row; rows past the last entry,
    // and entries with an invalid id, load nothing ...
    const int rows = nth / 16;
    const int grp = tid & 15;
    const int jr = tid / 16;
    const int32_t ej = __shfl(my_id, jr & (kWave - 1));
    const bool use = jr < k && valid_id(ej, E);
    int4 ch = make_int4(0, 0, 0, 0), cp = make_int4(0, 0, 0, 0);
    if (use) {
        ch = column_group(p.hist, ej, grp);
        cp = column_group(p.prefix, ej, grp);
    }

    __syncthreads();
    if (tid < k && valid_id(my_id, E)) atomicOr(&s_map[my_id], 1u << tid);
    __syncthreads();

    // ... and while they load, the equal ids ahead: an id at position
    // pos < end is ahead of the entries j with first + j > pos in pos's block
    // (entries from jb on lie in the next block, which starts at position
    // chunk).
    const uint32_t all = (k == 32) ? ~0u : ((1u << k) - 1u);
    const int jb = min(k, p.chunk - first);
    const uint32_t first_block = (jb >= 32) ? ~0u : ((1u << jb) - 1u);
    auto visit = [&](const int32_t (&q)[IDS], int base) {
#pragma unroll
        for (int u = 0; u < IDS; ++u) {
            const int pos = base + u * nth + tid;
            const int32_t id = q[u];
            if (pos < end && valid_id(id, E)) {
                uint32_t m = s_map[id];
                if (m != 0) {
                    const int d = pos - first;  // <= k - 2
                    m &= (d < 0) ? all : (all & ~((2u << d) - 1u));
                    if (pos < p.chunk) m &= first_block;
                    while (m) {
                        atomicAdd(&s_ahead[__builtin_ctz(m)], 1);
                        m &= m - 1;
                    }
                }
            }
        }
    };
    visit(ids, 0);
    for (int base = span; base < end; base += span) {  // blocks wider than a pass
        int32_t more[IDS];
#pragma unroll
        for (int u = 0; u < IDS; ++u) {
            const int pos = base + u * nth + tid;
            more[u] = (pos < end) ? p.idx[lo + pos] : -1;
        }
        visit(more, base);
    }

    // Column sums: all of the prefix column, the count column above block B.
    auto column_sums = [&](int j, const int4& h, const int4& q) {
        const int B = lo / p.chunk + (first + j >= p.chunk ? 1 : 0);
        int32_t sp = q.x + q.y + q.z + q.w;
        int32_t sh = (4 * grp < B ? h.x : 0) + (4 * grp + 1 < B ? h.y : 0) +
                     (4 * grp + 2 < B ? h.z : 0) + (4 * grp + 3 < B ? h.w : 0);
        sp = row16_inclusive_scan(sp);
        sh = row16_inclusive_scan(sh);
        if (grp == 15 && j < k) {
            s_sum[0][j] = sp;
            s_sum[1][j] = sh;
        }
    };
    column_sums(jr, ch, cp);
    // More entries than DPP rows (k > nth / 16).
    for (int j0 = rows; j0 < k; j0 += rows) {
        const int j = j0 + jr;
        const int32_t e = __shfl(my_id, j & (kWave - 1));
        int4 h = make_int4(0, 0, 0, 0), q = make_int4(0, 0, 0, 0);
        if (j < k && valid_id(e, E)) {
            h = column_group(p.hist, e, grp);
            q = column_group(p.prefix, e, grp);
        }
        column_sums(j, h, q);
    }
    __syncthreads();

    if (tid < k) {  // wave 0: lane j holds entry j's id
        int32_t slot = -1;
        if (valid_id(my_id, E)) {
            const int32_t r = s_sum[1][tid] + s_ahead[tid];
            if (p.cap == 0) slot = s_sum[0][tid] + r;
            else if (r < p.cap) slot = my_id * p.cap + r;
        }
        s_slot[tid] = slot;
        if (tile == 0) {
            p.slot_of[e0 + tid] = slot;
            if (slot >= 0 && slot < p.R) p.src_of_slot[slot] = static_cast<int32_t>(e0 + tid);
        }
    }

    // The row (its loads are in flight while the slots settle).
    Bf16Tile<VPL> bt;
    Fp8Tile<VPL, MODE == 2> ft;
    if (FP8) ft.load_quantise(p.x, p.nvec, t, tile, nth, tid, s_scale);
    else bt.load(p.x, p.nvec, t, tile, nth, tid);
    __syncthreads();

    const int32_t slot_vec = (lane < static_cast<uint32_t>(k)) ? s_slot[lane] : -1;
    if (FP8) {
        ft.store_lanes(slot_vec, k, p.R, static_cast<u32x2*>(p.recv_x), p.nvec);
        if (MODE == 2)
            dispatch::fp8_store_scales(s_scale, s_slot, k, p.R,
                                       static_cast<uint8_t*>(p.recv_scales), p.nvec / 16, tile,
                                       nth, VPL, tid);
        else
            dispatch::fp8_store_scales(s_scale, s_slot, k, p.R, static_cast<float*>(p.recv_scales),
                                       p.nvec / 16, tile, nth, VPL, tid);
    } else {
        bt.store_lanes(slot_vec, k, p.R, static_cast<u32x4*>(p.recv_x), p.nvec);
    }

    // Column totals, the layout's per-expert outputs and the empty rows.
    if (tile != 0) return;
    for (int col = t; col <= E; col += p.T) {
        if (tid < kWave) {
            int4 h = make_int4(0, 0, 0, 0), q = make_int4(0, 0, 0, 0);
            if (tid < 16) {
                h = column_group(p.hist, col, tid);
                q = column_group(p.prefix, col, tid);
            }
            const int32_t sh = row16_inclusive_scan(h.x + h.y + h.z + h.w);
            const int32_t sp = row16_inclusive_scan(q.x + q.y + q.z + q.w);
            if (tid == 15) {
                s_col[0] = sh;
                s_col[1] = sp;
            }
        }
        __syncthreads();
        const int32_t total = s_col[0];
        const int32_t before = s_col[1];
        if (col < E) {
            if (tid == 0) {
                p.count[col] = total;
                p.offset[col] = before;
                if (p.cap > 0 && total > p.cap) atomicAdd(&p.status[1], total - p.cap);
            }
            if (p.cap > 0) {
                int32_t* rows_e = p.src_of_slot + static_cast<int64_t>(col) * p.cap;
                for (int r = min(total, p.cap) + tid; r < p.cap; r += nth) rows_e[r] = -1;
            }
        } else {
            if (tid == 0) {
                p.offset[E] = before;  // valid entries
                p.status[0] = total;   // invalid ids
            }
            if (p.cap == 0)
                for (int64_t r = before + tid; r < p.R; r += nth) p.src_of_slot[r] = -1;
        }
        __syncthreads();  // s_col is rewritten by the next column
    }
}

template <int VPL>
void launch_ranked(const RankedParams& r, dim3 grid, int threads, int mode, hipStream_t stream) {
    const size_t lds = mode ? static_cast<size_t>(threads) * VPL / 16 * 4 : 0;
    if (mode == 2)
        hipLaunchKernelGGL((layout_dispatch_ranked_kernel<VPL, 2>), grid, dim3(threads), lds,
                           stream, r);
    else if (mode == 1)
        hipLaunchKernelGGL((layout_dispatch_ranked_kernel<VPL, 1>), grid, dim3(threads), lds,
                           stream, r);
    else
        hipLaunchKernelGGL((layout_dispatch_ranked_kernel<VPL, 0>), grid, dim3(threads), lds,
                           stream, r);
}

template <int VPL>
void launch_small(const SmallParams& p, int mode, hipStream_t stream) {
    const size_t lds = small::lds_bytes(p.n, p.E);
    if (mode == 2)
        hipLaunchKernelGGL((layout_dispatch_small_kernel<VPL, 2>), dim3(p.nwg), dim3(kThreads),
                           lds, stream, p);
    else if (mode == 1)
        hipLaunchKernelGGL((layout_dispatch_small_kernel<VPL, 1>), dim3(p.nwg), dim3(kThreads),
                           lds, stream, p);
    else
        hipLaunchKernelGGL((layout_dispatch_small_kernel<VPL, 0>), dim3(p.nwg), dim3(kThreads),
                           lds, stream, p);
}

// Larger tables: the histogram kernel writes both tables, then one
// (token, tile) workgroup per dispatch item ranks and stores.
hipError_t launch_tables_ranked(const ep_problem& p, const int32_t* topk_idx,
                                const ep_layout_t& out, int32_t* workspace, const void* x,
                                void* recv_x, void* recv_scales, hipStream_t stream) {
    const LayoutGeometry g = layout_geometry_two_pass(p);
    hipError_t err = launch_layout_tables(p, topk_idx, g, workspace, out.status, stream);
    if (err != hipSuccess) return err;
    const int E = p.num_experts;
    RankedParams r;
    r.idx = topk_idx;
    r.E = E;
    r.cap = p.capacity;
    r.k = p.num_topk;
    r.chunk = g.chunk;
    r.R = p.capacity == 0 ? g.entries : static_cast<int64_t>(E) * p.capacity;
    r.hist = workspace;
    r.prefix = workspace + static_cast<int64_t>(E + 1) * kTableStride;
    r.count = out.count;
    r.offset = out.offset;
    r.slot_of = out.slot_of;
    r.src_of_slot = out.src_of_slot;
    r.status = out.status;
    r.x = static_cast<const u32x4*>(x);
    r.recv_x = recv_x;
    r.recv_scales = recv_scales;
    r.T = p.num_tokens;
    r.nvec = p.hidden / 8;
    const DispatchShape ds = dispatch_shape(r.nvec, p.num_tokens, p.use_fp8 != 0);
    const dim3 grid(p.num_tokens, ds.tile.tiles);
    const int th = ds.tile.threads;
    switch (ds.vpl) {
        case 1: launch_ranked<1>(r, grid, th, p.use_fp8, stream); break;
        case 2: launch_ranked<2>(r, grid, th, p.use_fp8, stream); break;
        case 3: launch_ranked<3>(r, grid, th, p.use_fp8, stream); break;
        case 4: launch_ranked<4>(r, grid, th, p.use_fp8, stream); break;
        case 5: launch_ranked<5>(r, grid, th, p.use_fp8, stream); break;
        case 6: launch_ranked<6>(r, grid, th, p.use_fp8, stream); break;
        case 7: launch_ranked<7>(r, grid, th, p.use_fp8, stream); break;
        default: launch_ranked<8>(r, grid, th, p.use_fp8, stream); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layout_dispatch(const ep_problem& p, const int32_t* topk_idx,
                                  const ep_layout_t& out, void* workspace, const void* x,
                                  void* recv_x, void* recv_scales, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(p.num_tokens) * p.num_topk;
    const int nvec = p.hidden / 8;
    // Few tokens: one piece per lane and more tiles, so that more groups run.
    const int vpl = (p.num_tokens < 1024) ? 1 : dispatch::two_wave_vpl(nvec);
    const int tiles = (nvec + kGroupThreads * vpl - 1) / (kGroupThreads * vpl);
    const int64_t items = static_cast<int64_t>(p.num_tokens) * tiles;
    // at least one workgroup: it also writes count, offset and status
    const int64_t nwg = items > 0 ? (items + kGroups - 1) / kGroups : 1;
    // Every workgroup reads the whole table: past a few million id visits in
    // all, the layout kernels followed by the dispatch kernel are faster.
    if (n > kFusedMaxEntries || n * nwg > kFusedMaxVisits) {
        int dev = 0, ncu = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err == hipSuccess)
            err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return err;
        if (layout_dispatch_persistent_fits(p, ncu))
            return launch_layout_dispatch_persistent(p, topk_idx, out, x, recv_x, recv_scales,
                                                     ncu, stream);
        // Ranking inside the dispatch kernel puts two dependent round trips
        // (the token's ids, then its table columns) ahead of each
        // workgroup's row; that pays for bf16 rows and for FP8 with k >= 8,
        // while FP8 with fewer receive rows per token is faster with the
        // layout kernels followed by the dispatch kernel (measured on MI355X).
        if (p.use_fp8 == 0 || p.num_topk >= 8)
            return launch_tables_ranked(p, topk_idx, out, static_cast<int32_t*>(workspace), x,
                                        recv_x, recv_scales, stream);
        err = launch_layout(p, topk_idx, out, static_cast<int32_t*>(workspace), stream);
        if (err != hipSuccess) return err;
        return launch_dispatch(p, x, out.slot_of, recv_x, recv_scales, stream);
    }
    SmallParams a;
    a.idx = topk_idx;
    a.n = static_cast<int>(n);
    a.E = p.num_experts;
    a.cap = p.capacity;
    a.R = p.capacity == 0 ? n : static_cast<int64_t>(p.num_experts) * p.capacity;
    a.count = out.count;
    a.offset = out.offset;
    a.slot_of = out.slot_of;
    a.src_of_slot = out.src_of_slot;
    a.status = out.status;
    a.x = static_cast<const u32x4*>(x);
    a.recv_x = recv_x;
    a.recv_scales = recv_scales;
    a.T = p.num_tokens;
    a.k = p.num_topk;
    a.nvec = nvec;
    a.tiles = tiles;
    a.nwg = static_cast<int>(nwg);
    switch (vpl) {
        case 1: launch_small<1>(a, p.use_fp8, stream); break;
        case 2: launch_small<2>(a, p.use_fp8, stream); break;
        case 3: launch_small<3>(a, p.use_fp8, stream); break;
        case 4: launch_small<4>(a, p.use_fp8, stream); break;
        case 5: launch_small<5>(a, p.use_fp8, stream); break;
        case 6: launch_small<6>(a, p.use_fp8, stream); break;
        case 7: launch_small<7>(a, p.use_fp8, stream); break;
        default: launch_small<8>(a, p.use_fp8, stream); break;
    }
    return hipGetLastError();
}

}  // namespace ep
