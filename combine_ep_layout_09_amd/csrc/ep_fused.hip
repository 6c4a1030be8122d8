// ep_fused.hip -- layout and dispatch of a small routing table in one kernel.
//
// Decode-sized batches move little data, so separate layout and dispatch
// kernels are bound by launches and by the layout's chain of dependent
// memory round trips.  For routing tables of up to kFusedMaxEntries ids this
// kernel does both, and no workgroup waits for another: every workgroup
// derives, from the whole table (a few KiB, served by the L2 after the first
// reads), exactly the slots it needs.  This follows the pages' low-latency
// design advice: "[GH-ISSUE #18] Reasons for not calling NVSHMEM public
// APIs?" on keeping synchronisation and atomics off the microsecond path, and
// "[GH-ISSUE #166] Why does DeepEP LL kernel use double send/recv/signal
// buffers?" on folding clean-up work into the communication kernel itself.
//
// For routing entry i = t*k + j with valid expert e:
//   rank(i)   = #{entries before i with id e}           (stable counting sort)
//   offset[e] = #{valid ids below e}                    (exclusive scan of count)
//   slot      = offset[e] + rank   (contiguous)
//             = e*cap + rank if rank < cap, else -1     (fixed capacity)
// which is what ep_layout computes.  A workgroup copies the routing table
// into LDS (one round trip, while its rows load) and builds an LDS histogram
// of it, whose scan gives the offsets.  For the rank, each of its entries
// sets its bit in a per-expert 64-bit mask; one pass over the ids ahead of
// its tokens then looks each id up in the mask table, and the rare hits add
// one to the entries concerned.  The entries of the token itself are
// compared directly.
//
// Work split.  Workgroup b scatters items 2b and 2b+1 (token, column tile),
// one per 128-lane group, as the dispatch kernel does.  Tile 0 of a token
// writes its slot_of and src_of_slot entries.  Workgroup b also marks the
// empty receive rows of experts b, b + D, b + 2D, ... (D workgroups;
// contiguous layout: the rows past the valid entries, strided over the
// workgroups), and workgroup 0 writes count, offset and status.  The results
// are identical to ep_layout followed by ep_dispatch.

#include "ep_dispatch_dev.h"
#include "ep_internal.h"
#include "ep_layout_dev.h"

namespace ep {
namespace {

using dispatch::Bf16Tile;
using dispatch::Fp8Tile;
using dispatch::u32x2;
using dispatch::u32x4;
using layout::valid_id;
using layout::wave_inclusive_scan;

constexpr int kThreads = 256;
constexpr int kGroupThreads = 128;  // one scatter item per group
constexpr int kGroups = kThreads / kGroupThreads;
constexpr int kMaxEntries = kGroups * kMaxTopk;  // routing entries of a workgroup

static_assert(kGroupThreads % kWave == 0, "groups are whole waves");
static_assert(kGroupThreads >= kMaxTopk, "one lane per routing entry of a token");
static_assert(kMaxEntries <= 64, "a workgroup's entries fit a 64-bit mask");
static_assert(kGroups == 2, "two token starts per workgroup");

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
    float* recv_scales;
    int T, k, nvec, tiles, nwg;
};

// Dynamic LDS of the kernel, in 16-byte units first (int32 words):
//   ids  [4 * n4]  the routing table, padded with -1 to whole quads
//   hist [E + 1]   ids per expert; hist[E] counts ids outside [0, E)
//   off  [E + 1]   exclusive scan of hist[0..E)
//   map  [E]       uint64: bit q set if the workgroup's entry q has id e
__host__ __device__ inline size_t small_lds_bytes(int n, int E) {
    const size_t words = static_cast<size_t>((n + 3) / 4) * 4 + 2 * static_cast<size_t>(E + 1);
    return ((words * 4 + 7) / 8) * 8 + static_cast<size_t>(E) * 8;
}

// The routing table on its way into LDS: load() issues the global loads
// (16 bytes per lane per step; idx is 16-byte aligned), store() writes LDS
// (padded with -1 to whole quads), so that other loads can be issued in
// between.
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
static_assert(kFusedMaxEntries % (4 * kThreads) == 0, "whole staging steps");

template <int VPL, bool FP8>
__global__ __launch_bounds__(kThreads) void layout_dispatch_small_kernel(SmallParams p) {
    __shared__ int32_t s_key[kGroups][kMaxTopk];
    __shared__ int32_t s_eq[kMaxEntries];
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
    const int n4 = (p.n + 3) / 4;
    int32_t* s_ids = s_dyn;
    int32_t* s_hist = s_ids + 4 * n4;
    int32_t* s_off = s_hist + (E + 1);
    uint64_t* s_map = reinterpret_cast<uint64_t*>(
        reinterpret_cast<char*>(s_dyn) + ((static_cast<size_t>(4 * n4 + 2 * (E + 1)) * 4 + 7) / 8) * 8);
    const int items = p.T * p.tiles;
    // the same for every lane of a wave (a group is whole waves)
    const int item = __builtin_amdgcn_readfirstlane(b * kGroups + g);
    const bool active = item < items;
    const int t = active ? item / p.tiles : 0;
    const int tile = active ? item % p.tiles : 0;
    const int e0 = t * k;  // the token's first entry

    // Global loads first: the token's ids, the routing table, then the row.
    int32_t my_key = -1;
    if (active && gtid < k) my_key = p.idx[e0 + gtid];
    IdStage stage;
    stage.load(p.idx, p.n);
    Bf16Tile<VPL> bt;
    Fp8Tile<VPL> ft;
    if (active) {
        if (FP8) ft.load(p.x, p.nvec, t, tile, kGroupThreads, gtid);
        else bt.load(p.x, p.nvec, t, tile, kGroupThreads, gtid);
    }
    stage.store(p.n, s_ids);
    if (gtid < kMaxTopk) s_key[g][gtid] = my_key;
    for (int e = tid; e <= E; e += kThreads) s_hist[e] = 0;
    for (int e = tid; e < E; e += kThreads) s_map[e] = 0;
    if (tid < kMaxEntries) s_eq[tid] = 0;
    __syncthreads();

    // Entry q = gq*k + j (group gq, entry j of its token) sets bit q of its
    // expert's mask; every id goes into the histogram.
    const int nent = kGroups * k;
    if (tid < nent) {
        const int gq = tid / k;
        const int32_t key = s_key[gq][tid - gq * k];
        if (valid_id(key, E)) atomicOr(reinterpret_cast<unsigned long long*>(&s_map[key]), 1ull << tid);
    }
    for (int i = tid; i < p.n; i += kThreads) {
        const int32_t id = s_ids[i];
        atomicAdd(&s_hist[valid_id(id, E) ? id : E], 1);
    }
    __syncthreads();

    // Equal ids ahead of each entry's token: the ids before the later token
    // start, each looked up in the mask table (a hit is rare: ~2k/E).
    int lim[kGroups];
#pragma unroll
    for (int gq = 0; gq < kGroups; ++gq) {
        const int it = b * kGroups + gq;
        lim[gq] = (it < items) ? (it / p.tiles) * k : 0;
    }
    const uint64_t low = (k == 64) ? ~0ull : ((1ull << k) - 1);
    const int lim_max = max(lim[0], lim[1]);
    for (int i = tid; i < lim_max; i += kThreads) {
        const int32_t id = s_ids[i];
        if (!valid_id(id, E)) continue;
        uint64_t m = s_map[id];
        if (m == 0) continue;
        m &= ((i < lim[0]) ? low : 0ull) | ((i < lim[1]) ? (low << k) : 0ull);
        while (m) {
            atomicAdd(&s_eq[__builtin_ctzll(m)], 1);
            m &= m - 1;
        }
    }
    // Wave 0 scans the histogram into the expert offsets (and the entries
    // dropped by the capacity).
    if (tid < kWave) {
        const uint32_t lane = lane_id();
        const int per = (E + kWave - 1) / kWave;
        const int lo = min(E, static_cast<int>(lane) * per);
        const int hi = min(E, lo + per);
        int32_t local = 0, drop = 0;
        for (int e = lo; e < hi; ++e) {
            local += s_hist[e];
            if (p.cap > 0 && s_hist[e] > p.cap) drop += s_hist[e] - p.cap;
        }
        const int32_t incl = wave_inclusive_scan(local);
        const int32_t drop_all = wave_inclusive_scan(drop);
        int32_t run = incl - local;
        for (int e = lo; e < hi; ++e) {
            s_off[e] = run;
            run += s_hist[e];
        }
        if (lane == kWave - 1) {
            s_off[E] = incl;
            s_drop = (p.cap > 0) ? drop_all : 0;
        }
    }
    if (FP8 && active) ft.quantise(p.nvec, tile, kGroupThreads, gtid, s_scale[g]);
    __syncthreads();

    const bool contiguous = p.cap == 0;
    if (active && gtid < k) {
        const int j = gtid;
        int32_t slot = -1;
        if (valid_id(my_key, E)) {
            int32_t rank = s_eq[g * k + j];
            for (int jj = 0; jj < j; ++jj) rank += (s_key[g][jj] == my_key) ? 1 : 0;
            if (contiguous) slot = s_off[my_key] + rank;
            else if (rank < p.cap) slot = my_key * p.cap + rank;
        }
        s_slot[g][j] = slot;
        if (tile == 0) {
            p.slot_of[e0 + j] = slot;
            if (slot >= 0 && slot < p.R) p.src_of_slot[slot] = e0 + j;
        }
    }
    if (b == 0) {
        // count, offset and status
        for (int e = tid; e < E; e += kThreads) {
            p.count[e] = s_hist[e];
            p.offset[e] = s_off[e];
        }
        if (tid == 0) {
            p.offset[E] = s_off[E];
            p.status[0] = s_hist[E];
            p.status[1] = s_drop;
        }
    }
    __syncthreads();

    if (active) {
        const int32_t* slots = s_slot[g];
        if (FP8) {
            ft.store(slots, k, p.R, static_cast<u32x2*>(p.recv_x), p.nvec);
            dispatch::fp8_store_scales(s_scale[g], slots, k, p.R, p.recv_scales, p.nvec / 16, tile,
                                       kGroupThreads, VPL, gtid);
        } else {
            bt.store(slots, k, p.R, static_cast<u32x4*>(p.recv_x), p.nvec);
        }
    }

    // Receive rows that no entry fills get src_of_slot = -1: rows past the
    // count of experts b, b + D, ... (fixed capacity), or the rows past the
    // valid entries, strided over the workgroups (contiguous).
    if (!contiguous) {
        for (int e = b; e < E; e += p.nwg) {
            int32_t* rows = p.src_of_slot + static_cast<int64_t>(e) * p.cap;
            for (int r = min(s_hist[e], p.cap) + tid; r < p.cap; r += kThreads) rows[r] = -1;
        }
    } else {
        for (int64_t r = s_off[E] + static_cast<int64_t>(b) * kThreads + tid; r < p.R;
             r += static_cast<int64_t>(p.nwg) * kThreads)
            p.src_of_slot[r] = -1;
    }
}

template <int VPL>
void launch_small(const SmallParams& p, bool fp8, hipStream_t stream) {
    const size_t lds = small_lds_bytes(p.n, p.E);
    if (fp8)
        hipLaunchKernelGGL((layout_dispatch_small_kernel<VPL, true>), dim3(p.nwg), dim3(kThreads),
                           lds, stream, p);
    else
        hipLaunchKernelGGL((layout_dispatch_small_kernel<VPL, false>), dim3(p.nwg), dim3(kThreads),
                           lds, stream, p);
}

}  // namespace

hipError_t launch_layout_dispatch(const ep_problem& p, const int32_t* topk_idx,
                                  const ep_layout_t& out, void* workspace, const void* x,
                                  void* recv_x, float* recv_scales, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(p.num_tokens) * p.num_topk;
    if (n > kFusedMaxEntries) {
        // Larger batches: the layout is a small part of the call there.
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
    a.nvec = p.hidden / 8;
    // Few tokens: one piece per lane and more tiles, so that more groups run.
    const int vpl = (p.num_tokens < 1024) ? 1 : dispatch::two_wave_vpl(a.nvec);
    a.tiles = (a.nvec + kGroupThreads * vpl - 1) / (kGroupThreads * vpl);
    const int items = a.T * a.tiles;
    // at least one workgroup: it also writes count, offset and status
    a.nwg = items > 0 ? (items + kGroups - 1) / kGroups : 1;
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
