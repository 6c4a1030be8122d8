// ep_fused_persist.hip -- ep_layout_dispatch for prefill-sized routing tables
// and bf16 payloads in one launch of one 1024-lane workgroup per CU.
//
// The problem is the one of ep_layout followed by ep_dispatch.  For routing
// entry i = t*k + j with valid expert e:
//   rank(i)   = #{entries before i with id e}           (stable counting sort)
//   offset[e] = #{valid ids below e}                    (exclusive scan of count)
//   slot      = offset[e] + rank   (contiguous)
//             = e*cap + rank if rank < cap, else -1     (fixed capacity)
// and every entry with a slot receives a bit copy of token t's row.  As in
// ep_layout.hip, the per-expert counts and expert-major receive rows follow
// the dispatch code quoted in "[GH-ISSUE #282] Redundant atomics in
// internode_ll", the order inside an expert the order consistency of
// "[GH-ISSUE #18] Reasons for not calling NVSHMEM public APIs?", and a
// token's payload the hidden data of "[PR #693] Pipeline direct NVLink
// dispatch with triple-buffered prefetch" (Summary).
//
// Workgroup b owns a contiguous run of (token, 64-piece chunk) units -- 16 Q
// of them, Q <= kHold -- and so a contiguous run of tokens [tA, tB); wave w
// holds chunks w, w + 16, ... of the run.  Nothing waits for another
// workgroup:
//   1. every lane issues all of its loads at once: the workgroup's own
//      routing entries (one per lane), the whole routing table (kIdQuads
//      quads per lane), then all Q row chunks of its wave (kept in
//      registers until they are stored);
//   2. while the rows are in flight, the table builds two LDS histograms:
//      the ids ahead of the workgroup's first entry, and the rest (the
//      counting sort's "entries before i" split at the workgroup's start);
//      each wave holding own entries ranks them among themselves with one
//      ballot per key bit and records its per-expert counts;
//   3. the sum of the two histograms, scanned over experts, gives offset;
//      an own entry's rank is the ids ahead of the workgroup with its
//      expert, plus the own entries of earlier waves, plus the peers of
//      lower lanes in its wave;
//   4. every wave waits once for its rows, then issues the stores of all of
//      its chunks to the k receive rows of their tokens with no wait in
//      between.  A wave's loads and stores share one counter and stores
//      complete in any order, so a wait for a row load issued after a store
//      also waits for that store; loading every row before the first store
//      keeps the stores back to back, and with the caches flushed between
//      calls the reads of x (at the start) and the writes (after it) no
//      longer alternate on the HBM bus.  Measured at the 4096-token prefill
//      with cold caches: 105-107 us against 110-111 us for a ring of four
//      chunks loaded ahead of each store step.
// Every workgroup builds the same whole-table histogram (a read of the table
// from L2 per CU): the price of needing no other workgroup, paid while the
// workgroup's rows arrive from HBM.  Workgroup 0 writes count, offset and
// status; the workgroup holding chunk 0 of a token writes its slot_of and
// src_of_slot entries; receive rows that no entry fills are marked -1 by
// workgroups in turn.
//
// Why one launch: at the 4096-token prefill shape the two-launch form (a
// histogram kernel, then a dispatch kernel that ranks each token) pays a
// kernel boundary of about 4 us between the two; here the layout runs under
// the row loads of the same launch.

#include "ep_dispatch_dev.h"
#include "ep_internal.h"
#include "ep_layout_dev.h"

namespace ep {
namespace {

using dispatch::u32x4;
using layout::key_bits;
using layout::valid_id;
using layout::wave_inclusive_scan;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kHold = 14;        // row chunks per wave of one launch, at most (Q)
constexpr int kIdQuads = 8;      // routing-table quads per lane (32 ids)
constexpr int kMaxIds = 4 * kIdQuads * kThreads;  // routing entries (T*k) of this form
constexpr size_t kMaxLds = 65536;

struct PersistParams {
    const int32_t* idx;
    int n;  // T * k
    int E, cap, k;
    int64_t R;
    int32_t* count;
    int32_t* offset;
    int32_t* slot_of;
    int32_t* src_of_slot;
    int32_t* status;
    const u32x4* x;
    u32x4* recv_x;
    int T, nvec;
    int C;     // 64-piece chunks per row
    int Q;     // chunks per wave (<= kHold)
    int rw;    // waves that hold own entries: ceil(own entries / 64), <= kWaves
    int maxtok;  // tokens a workgroup touches, at most
    int nwg;
};

// Dynamic LDS (int32 words):
//   part [2][E+1]   part[0]: ids ahead of the workgroup's first entry,
//                   part[1]: the others; bin E counts ids outside [0, E)
//   off  [E+1]      exclusive scan over experts of part[0] + part[1]
//   wcnt [rw][E+1]  own entries per expert of each ranking wave
//   slot [maxtok][kp] receive rows of each own token, rows padded to kp =
//                   k rounded up to 4 words (16-byte aligned rows)
__host__ __device__ inline int slot_stride(int k) { return (k + 3) & ~3; }

__host__ __device__ inline size_t persist_lds_words(int E, int rw, int maxtok, int k) {
    const size_t head = static_cast<size_t>(3 + rw) * (E + 1);
    return ((head + 3) & ~static_cast<size_t>(3)) + static_cast<size_t>(maxtok) * slot_stride(k);
}

// K: the top-k count when it is 1..8 (the store loop is unrolled over the
// token's receive rows, read from LDS together), 0 for any k.
template <int K>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void layout_dispatch_persistent_kernel(PersistParams p) {
    extern __shared__ __align__(16) int32_t s_dyn[];
    __shared__ int32_t s_wsum[kWaves];
    __shared__ int32_t s_wover[kWaves];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = static_cast<int>(lane_id());
    // the same for every lane of a wave: scalar from here on
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int b = static_cast<int>(blockIdx.x);
    const int E = p.E;
    const int k = K > 0 ? K : p.k;
    const int kp = slot_stride(k);
    const int W = E + 1;
    int32_t* part = s_dyn;
    int32_t* off = part + 2 * W;
    int32_t* wcnt = off + W;
    int32_t* s_slot = s_dyn + ((static_cast<size_t>(3 + p.rw) * W + 3) & ~static_cast<size_t>(3));

    const int all_chunks = p.T * p.C;  // < 2^31: at most (CUs * 16 * kHold) here
    const int c_begin = b * kWaves * p.Q;
    const int c_end = min(c_begin + kWaves * p.Q, all_chunks);
    const bool has = c_begin < c_end;
    const int tA = has ? c_begin / p.C : 0;
    const int tB = has ? (c_end - 1) / p.C + 1 : 0;
    const int P0 = tA * k;         // the workgroup's first routing entry
    const int n_own = (tB - tA) * k;  // <= rw * 64 (host-checked)

    // 1. Loads, in the order their results are needed: a wave's loads return
    // in issue order.  The own entry (clamped address: unconditional) ...
    const int32_t own_raw = p.idx[P0 + min(tid, max(n_own, 1) - 1)];
    const int32_t own_id = (tid < n_own) ? own_raw : -1;
    // ... the routing table (n is a multiple of 4; quads past the end load
    // the last quad again and are not counted) ...
    const int4* quads = reinterpret_cast<const int4*>(p.idx);
    const int nq = p.n / 4;
    int4 q[kIdQuads];
#pragma unroll
    for (int u = 0; u < kIdQuads; ++u) q[u] = quads[min(u * kThreads + tid, nq - 1)];
    // ... and the wave's Q row chunks (chunks w, w + 16, ... of the
    // workgroup's run, non-temporal: each is read once); cid[j] is the chunk
    // buf[j] holds, -1 for none.  Every load is issued -- a slot with no
    // chunk reads the run's last chunk again (a cache hit, never stored) --
    // because with loads under branches the compiler could no longer count
    // which of them are still in flight, and the histogram below would wait
    // for the rows instead of only for the table.
    const int c_last = max(c_end - 1, 0);
    u32x4 buf[kHold];
    int cid[kHold];
#pragma unroll
    for (int j = 0; j < kHold; ++j) {
        const int c = c_begin + wave + j * kWaves;
        const bool mine = j < p.Q && c < c_end;
        const int cc = mine ? c : c_last;
        const int t = cc / p.C;
        const int v = min((cc - t * p.C) * kWave + lane, p.nvec - 1);
        buf[j] = __builtin_nontemporal_load(p.x + static_cast<int64_t>(t) * p.nvec + v);
        cid[j] = mine ? c : -1;
    }

    for (int e = tid; e < (2 + p.rw) * W; e += kThreads)
        (e < 2 * W ? part[e] : wcnt[e - 2 * W]) = 0;
    __syncthreads();

    // 2. Histograms of the table, split at the workgroup's first entry.
    auto count_quad = [&](const int4& g, int qi) {
        if (qi < nq) {
            const int32_t id4[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int32_t id = id4[c];
                const int bin = (valid_id(id, E) ? id : E) + (4 * qi + c < P0 ? 0 : W);
                atomicAdd(&part[bin], 1);
            }
        }
    };
#pragma unroll
    for (int u = 0; u < kIdQuads; ++u) count_quad(q[u], u * kThreads + tid);

    // Own entries: rank among the same wave's lower lanes, and per-wave
    // counts (the lowest lane of each expert's peers records them).
    int32_t below = 0;
    if (wave < p.rw) {
        const bool mine = valid_id(own_id, E);
        const uint64_t peers = match_peers(static_cast<uint32_t>(own_id), key_bits(E), __ballot(mine));
        const uint64_t lower = peers & lanemask_lt();
        below = __popcll(lower);
        if (mine && lower == 0) wcnt[wave * W + own_id] = __popcll(peers);
    }
    __syncthreads();

    // 3. Offsets (exclusive scan of the totals over experts), the entries the
    // capacity drops, then the own entries' slots.
    int32_t tot = 0, over = 0;
    if (tid < E) {
        tot = part[tid] + part[W + tid];
        over = (p.cap > 0 && tot > p.cap) ? tot - p.cap : 0;
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
            p.count[tid] = tot;
            p.offset[tid] = before + incl - tot;
        }
    }
    if (tid == 0) {
        int32_t valid = 0, drop = 0;
        for (int w = 0; w < kWaves; ++w) {
            valid += s_wsum[w];
            drop += s_wover[w];
        }
        off[E] = valid;
        if (b == 0) {
            p.offset[E] = valid;
            p.status[0] = part[E] + part[W + E];
            p.status[1] = drop;
        }
    }
    __syncthreads();

    if (tid < n_own) {
        int32_t slot = -1;
        if (valid_id(own_id, E)) {
            int32_t r = part[own_id] + below;
            for (int w = 0; w < wave; ++w) r += wcnt[w * W + own_id];
            if (p.cap == 0) slot = off[own_id] + r;
            else if (r < p.cap) slot = own_id * p.cap + r;
        }
        s_slot[(tid / k) * kp + tid % k] = slot;
        // the workgroup holding the token's chunk 0 writes its layout entries
        const int t = tA + tid / k;
        if (t * p.C >= c_begin) {
            p.slot_of[P0 + tid] = slot;
            if (slot >= 0 && slot < p.R) p.src_of_slot[slot] = P0 + tid;
        }
    }
    // Receive rows no entry fills: past each expert's count (fixed capacity,
    // experts b, b + nwg, ...), or past the valid entries (contiguous).
    if (p.cap > 0) {
        for (int e = b; e < E; e += p.nwg) {
            int32_t* rows = p.src_of_slot + static_cast<int64_t>(e) * p.cap;
            const int32_t filled = min(part[e] + part[W + e], p.cap);
            for (int r = filled + tid; r < p.cap; r += kThreads) rows[r] = -1;
        }
    } else {
        for (int64_t r = off[E] + static_cast<int64_t>(b) * kThreads + tid; r < p.R;
             r += static_cast<int64_t>(p.nwg) * kThreads)
            p.src_of_slot[r] = -1;
    }
    __syncthreads();

    // 4. Stores: one wait for the rows, then every store of the wave with no
    // wait in between.
    auto store_chunk = [&](int c, const u32x4& data) {
        const int t = c / p.C;
        const int v = min((c - t * p.C) * kWave + lane, p.nvec - 1);
        const int32_t* sl = s_slot + (t - tA) * kp;
        u32x4* dst = p.recv_x + v;
        if (K > 0) {
            int32_t slot[K > 0 ? K : 1];
#pragma unroll
            for (int j = 0; j < K; ++j) slot[j] = __builtin_amdgcn_readfirstlane(sl[j]);
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (slot[j] >= 0 && slot[j] < p.R)
                    __builtin_nontemporal_store(data, dst + static_cast<int64_t>(slot[j]) * p.nvec);
        } else {
            for (int j = 0; j < k; ++j) {
                const int32_t slot = __builtin_amdgcn_readfirstlane(sl[j]);
                if (slot >= 0 && slot < p.R)
                    __builtin_nontemporal_store(data, dst + static_cast<int64_t>(slot) * p.nvec);
            }
        }
    };
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    // Issue priority falls from 3 to 0 over the quarters of a wave's chunks:
    // a SIMD issues for its oldest wave first, and a wave ahead of the others
    // yields the SIMD to them, as in the persistent combine.
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int j = 0; j < kHold; ++j) {
        if (cid[j] >= 0) {  // uniform
            store_chunk(cid[j], buf[j]);
            const int level = (4 * (j + 1)) / p.Q;
            if (level == 1) __builtin_amdgcn_s_setprio(2);
            else if (level == 2) __builtin_amdgcn_s_setprio(1);
            else if (level >= 3) __builtin_amdgcn_s_setprio(0);
        }
    }
}

}  // namespace

bool layout_dispatch_persistent_fits(const ep_problem& p, int ncu) {
    if (p.use_fp8 != 0 || p.num_tokens <= 0) return false;
    const int64_t n = static_cast<int64_t>(p.num_tokens) * p.num_topk;
    // whole quads of routing entries (the table is loaded 16 bytes a lane)
    if (n <= kFusedMaxEntries || n > kMaxIds || n % 4 != 0) return false;
    const int nvec = p.hidden / 8;
    const int64_t C = (nvec + kWave - 1) / kWave;
    const int64_t nw = static_cast<int64_t>(ncu) * kWaves;
    const int64_t all_chunks = static_cast<int64_t>(p.num_tokens) * C;
    // every wave gets a chunk, and one launch holds all of them
    if (all_chunks < nw || all_chunks > nw * kHold) return false;
    const int64_t Q = (all_chunks + nw - 1) / nw;
    const int64_t maxtok = (kWaves * Q - 1) / C + 2;
    const int64_t own = maxtok * p.num_topk;
    if (own > kThreads) return false;
    const int rw = static_cast<int>((own + kWave - 1) / kWave);
    return persist_lds_words(p.num_experts, rw, static_cast<int>(maxtok), p.num_topk) * 4 <= kMaxLds;
}

hipError_t launch_layout_dispatch_persistent(const ep_problem& p, const int32_t* topk_idx,
                                             const ep_layout_t& out, const void* x, void* recv_x,
                                             int ncu, hipStream_t stream) {
    PersistParams a;
    a.idx = topk_idx;
    a.n = p.num_tokens * p.num_topk;
    a.E = p.num_experts;
    a.cap = p.capacity;
    a.k = p.num_topk;
    a.R = p.capacity == 0 ? static_cast<int64_t>(a.n) : static_cast<int64_t>(a.E) * p.capacity;
    a.count = out.count;
    a.offset = out.offset;
    a.slot_of = out.slot_of;
    a.src_of_slot = out.src_of_slot;
    a.status = out.status;
    a.x = static_cast<const u32x4*>(x);
    a.recv_x = static_cast<u32x4*>(recv_x);
    a.T = p.num_tokens;
    a.nvec = p.hidden / 8;
    a.C = (a.nvec + kWave - 1) / kWave;
    const int64_t nw = static_cast<int64_t>(ncu) * kWaves;
    a.Q = static_cast<int>((static_cast<int64_t>(a.T) * a.C + nw - 1) / nw);
    a.maxtok = (kWaves * a.Q - 1) / a.C + 2;
    a.rw = (a.maxtok * a.k + kWave - 1) / kWave;
    a.nwg = ncu;
    const size_t lds = persist_lds_words(a.E, a.rw, a.maxtok, a.k) * 4;
    const dim3 grid(ncu), block(kThreads);
    switch (a.k) {
        case 1: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<1>, grid, block, lds, stream, a); break;
        case 2: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<2>, grid, block, lds, stream, a); break;
        case 3: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<3>, grid, block, lds, stream, a); break;
        case 4: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<4>, grid, block, lds, stream, a); break;
        case 5: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<5>, grid, block, lds, stream, a); break;
        case 6: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<6>, grid, block, lds, stream, a); break;
        case 7: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<7>, grid, block, lds, stream, a); break;
        case 8: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<8>, grid, block, lds, stream, a); break;
        default: hipLaunchKernelGGL(layout_dispatch_persistent_kernel<0>, grid, block, lds, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace ep
