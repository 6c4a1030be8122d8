// ep_fused.hip -- layout and dispatch of a small routing table in one kernel.
//
// Decode-sized batches move little data, so separate layout and dispatch
// kernels are bound by launches and by the layout's chain of dependent
// memory round trips.  For small routing tables this kernel does both, and
// no workgroup waits for another: every workgroup derives, from the whole
// table staged in its LDS, exactly the slots it needs (ep_small_dev.h), while
// its token rows load.  This follows the pages' low-latency design advice:
// "[GH-ISSUE #18] Reasons for not calling NVSHMEM public APIs?" on keeping
// synchronisation and atomics off the microsecond path, and "[GH-ISSUE #166]
// Why does DeepEP LL kernel use double send/recv/signal buffers?" on folding
// clean-up work into the communication kernel itself.
//
// For routing entry i = t*k + j with valid expert e:
//   rank(i)   = #{entries before i with id e}           (stable counting sort)
//   offset[e] = #{valid ids below e}                    (exclusive scan of count)
//   slot      = offset[e] + rank   (contiguous)
//             = e*cap + rank if rank < cap, else -1     (fixed capacity)
// which is what ep_layout computes.
//
// Work split.  Workgroup b scatters items 2b and 2b+1 (token, column tile),
// one per 128-lane group, as the dispatch kernel does; its entries are the
// 2k entries of those two tokens.  Tile 0 of a token writes its slot_of and
// src_of_slot entries.  Workgroup b also marks the empty receive rows of
// experts b, b + D, b + 2D, ... (D workgroups; contiguous layout: the rows
// past the valid entries, strided over the workgroups), and workgroup 0
// writes count, offset and status.  The results are identical to ep_layout
// followed by ep_dispatch.

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
    small::histogram(tab, p.n, E);
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
    small::scan_offsets(tab, E, p.cap, &s_drop);
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
        if (FP8) {
            ft.store(slots, k, p.R, static_cast<u32x2*>(p.recv_x), p.nvec);
            if (MODE == 2)
                dispatch::fp8_store_scales(s_scale[g], slots, k, p.R,
                                           static_cast<uint8_t*>(p.recv_scales), p.nvec / 16,
                                           tile, kGroupThreads, VPL, gtid);
            else
                dispatch::fp8_store_scales(s_scale[g], slots, k, p.R,
                                           static_cast<float*>(p.recv_scales), p.nvec / 16, tile,
                                           kGroupThreads, VPL, gtid);
        } else {
            bt.store(slots, k, p.R, static_cast<u32x4*>(p.recv_x), p.nvec);
        }
    }
    small::fill_empty_rows(tab, E, p.cap, p.R, b, p.nwg, p.src_of_slot);
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
        hipError_t err = launch_layout(p, topk_idx, out, static_cast<int32_t*>(workspace), stream);
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
