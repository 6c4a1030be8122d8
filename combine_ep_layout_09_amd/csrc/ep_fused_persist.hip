// ep_fused_persist.hip -- ep_layout_dispatch for prefill-sized routing tables
// (8192 < T*k <= 32768) in one launch of one 1024-lane workgroup per CU, for
// bf16 and FP8 payloads.
//
// The problem is the one of ep_layout followed by ep_dispatch.  For routing
// entry i = t*k + j with valid expert e:
//   rank(i)   = #{entries before i with id e}           (stable counting sort)
//   offset[e] = #{valid ids below e}                    (exclusive scan of count)
//   slot      = offset[e] + rank   (contiguous)
//             = e*cap + rank if rank < cap, else -1     (fixed capacity)
// and every entry with a slot receives token t's row (a bit copy, or its
// E4M3 codes and block scales as in ep_dispatch.hip).  As in
// ep_layout.hip, the per-expert counts and expert-major receive rows follow
// the dispatch code quoted in "[GH-ISSUE #282] Redundant atomics in
// internode_ll", the order inside an expert the order consistency of
// "[GH-ISSUE #18] Reasons for not calling NVSHMEM public APIs?", and a
// token's payload the hidden data of "[PR #693] Pipeline direct NVLink
// dispatch with triple-buffered prefetch" (Summary).
//
// Workgroup b owns a contiguous run of (token, 64-piece chunk) units -- 16 Q
// of them, Q <= kHold (bf16) or kHoldFp8 -- and so a contiguous run of tokens
// [tA, tB); wave w
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
//      chunks loaded ahead of each store step.  FP8 rows are quantised
//      chunk by chunk as they arrive, and each chunk is stored once it is
//      quantised (see the FP8 kernel).
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

using dispatch::u32x2;
using dispatch::u32x4;
using layout::key_bits;
using layout::valid_id;
using layout::wave_inclusive_scan;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kHold = 14;        // bf16: row chunks per wave of one launch, at most (Q)
constexpr int kHoldFp8 = 16;     // FP8: the same (quantised chunks take fewer registers)
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
    void* recv_x;       // bf16 rows (u32x4 pieces) or E4M3 rows (u32x2 pieces)
    void* recv_scales;  // FP8: fp32 or UE8M0 block scales [R, nblk]
    int T, nvec;
    int nblk;  // FP8: 128-channel blocks per row
    int C;     // 64-piece chunks per row
    int Q;     // chunks per wave (<= kHold, kHoldFp8)
    int rw;    // waves that hold own entries: ceil(own entries / 64), <= kWaves
    int maxtok;  // tokens a workgroup touches, at most
    int nwg;
};

// Dynamic LDS (int32 words):
//   part [nc][2][E+1]  part[0]: ids ahead of the workgroup's first entry,
//                   part[1]: the others; bin E counts ids outside [0, E);
//                   nc copies, lane l counting into copy l mod nc, summed
//                   into copy 0 once the table is counted
//   off  [E+1]      exclusive scan over experts of part[0] + part[1]
//   wcnt [rw][E+1]  own entries per expert of each ranking wave
//   slot [maxtok][kp] receive rows of each own token, rows padded to kp =
//                   k rounded up to 4 words (16-byte aligned rows)
__host__ __device__ inline int slot_stride(int k) { return (k + 3) & ~3; }

// Copies of the histograms: with few experts many lanes of one LDS atomic
// instruction hit the same bin (skewed routing more so), and the atomics to
// one address are applied one lane at a time.
__host__ __device__ inline int persist_copies(int E) { return E < 128 ? 8 : 1; }

__host__ __device__ inline size_t persist_head_words(int E, int rw) {
    const size_t head = static_cast<size_t>(2 * persist_copies(E) + 1 + rw) * (E + 1);
    return (head + 3) & ~static_cast<size_t>(3);
}

__host__ __device__ inline size_t persist_lds_words(int E, int rw, int maxtok, int k) {
    const size_t head = persist_head_words(E, rw);
    return head + static_cast<size_t>(maxtok) * slot_stride(k);
}

// The workgroup's view of the problem: its run of chunks and tokens and its
// LDS tables.
struct Part {
    int tid, lane, wave, b, E, k, kp, W, nc;
    int c_begin, c_end, tA, P0, n_own;
    int32_t* part;
    int32_t* mypart;  // this lane's copy of part
    int32_t* off;
    int32_t* wcnt;
    int32_t* s_slot;
};

template <int K>
__device__ __forceinline__ Part make_part(const PersistParams& p, int32_t* s_dyn) {
    Part w;
    w.tid = static_cast<int>(threadIdx.x);
    w.lane = static_cast<int>(lane_id());
    // the same for every lane of a wave: scalar from here on
    w.wave = __builtin_amdgcn_readfirstlane(w.tid / kWave);
    w.b = static_cast<int>(blockIdx.x);
    w.E = p.E;
    w.k = K > 0 ? K : p.k;
    w.kp = slot_stride(w.k);
    w.W = w.E + 1;
    w.nc = persist_copies(w.E);
    w.part = s_dyn;
    w.mypart = w.part + (w.lane & (w.nc - 1)) * 2 * w.W;
    w.off = w.part + 2 * w.nc * w.W;
    w.wcnt = w.off + w.W;
    w.s_slot = s_dyn + persist_head_words(w.E, p.rw);
    const int all_chunks = p.T * p.C;  // < 2^31: at most CUs * 16 * kHoldFp8 here
    w.c_begin = w.b * kWaves * p.Q;
    w.c_end = min(w.c_begin + kWaves * p.Q, all_chunks);
    const bool has = w.c_begin < w.c_end;
    w.tA = has ? w.c_begin / p.C : 0;
    const int tB = has ? (w.c_end - 1) / p.C + 1 : 0;
    w.P0 = w.tA * w.k;             // the workgroup's first routing entry
    w.n_own = (tB - w.tA) * w.k;   // <= rw * 64 (host-checked)
    return w;
}

// Adds the 4 ids of table quad qi (quads past the end are not counted) to
// the histogram of the ids ahead of the workgroup's first entry or to that
// of the others.
__device__ __forceinline__ void count_quad(const Part& w, int nq, const int4& g, int qi) {
    if (qi < nq) {
        const int32_t id4[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int32_t id = id4[c];
            const int bin = (valid_id(id, w.E) ? id : w.E) + (4 * qi + c < w.P0 ? 0 : w.W);
            atomicAdd(&w.mypart[bin], 1);
        }
    }
}

// Zeroes the histogram copies and the per-wave counts (a barrier follows).
__device__ __forceinline__ void zero_tables(const Part& w, int rw) {
    const int parts = 2 * w.nc * w.W;
    for (int e = w.tid; e < parts + rw * w.W; e += kThreads)
        (e < parts ? w.part[e] : w.wcnt[e - parts]) = 0;
}

// After the table is counted (barrier before): the copies summed into copy 0.
// Ends with a barrier when there is more than one copy.
__device__ __forceinline__ void merge_copies(const Part& w) {
    if (w.nc == 1) return;  // uniform
    for (int e = w.tid; e < 2 * w.W; e += kThreads) {
        int32_t sum = w.part[e];
        for (int c = 1; c < w.nc; ++c) sum += w.part[c * 2 * w.W + e];
        w.part[e] = sum;
    }
    __syncthreads();
}

// Own entries: rank among the same wave's lower lanes, and per-wave counts
// (the lowest lane of each expert's peers records them).  Returns the rank
// among lower lanes.
__device__ __forceinline__ int32_t rank_own(const Part& w, int rw, int32_t own_id) {
    int32_t below = 0;
    if (w.wave < rw) {
        const bool mine = valid_id(own_id, w.E);
        const uint64_t peers = match_peers(static_cast<uint32_t>(own_id), key_bits(w.E), __ballot(mine));
        const uint64_t lower = peers & lanemask_lt();
        below = __popcll(lower);
        if (mine && lower == 0) w.wcnt[w.wave * w.W + own_id] = __popcll(peers);
    }
    return below;
}

// After the histograms and the own ranks are complete (barrier before):
// offsets (exclusive scan of the totals over experts), the entries the
// capacity drops, the own entries' slots (to LDS, and to slot_of /
// src_of_slot from the workgroup holding the token's chunk 0), count,
// offset and status (workgroup 0), and the receive rows no entry fills.
// Ends with a barrier.
__device__ __forceinline__ void finish_layout(const PersistParams& p, const Part& w,
                                              int32_t own_id, int32_t below, int32_t* s_wsum,
                                              int32_t* s_wover) {
    const int tid = w.tid, E = w.E, W = w.W;
    int32_t tot = 0, over = 0;
    if (tid < E) {
        tot = w.part[tid] + w.part[W + tid];
        over = (p.cap > 0 && tot > p.cap) ? tot - p.cap : 0;
    }
    const int32_t incl = wave_inclusive_scan(tot);
    const int32_t oincl = wave_inclusive_scan(over);
    if (w.lane == kWave - 1) {
        s_wsum[w.wave] = incl;
        s_wover[w.wave] = oincl;
    }
    __syncthreads();
    int32_t before = 0;
    for (int v = 0; v < w.wave; ++v) before += s_wsum[v];
    if (tid < E) {
        w.off[tid] = before + incl - tot;
        if (w.b == 0) {
            p.count[tid] = tot;
            p.offset[tid] = before + incl - tot;
        }
    }
    if (tid == 0) {
        int32_t valid = 0, drop = 0;
        for (int v = 0; v < kWaves; ++v) {
            valid += s_wsum[v];
            drop += s_wover[v];
        }
        w.off[E] = valid;
        if (w.b == 0) {
            p.offset[E] = valid;
            p.status[0] = w.part[E] + w.part[W + E];
            p.status[1] = drop;
        }
    }
    __syncthreads();

    if (tid < w.n_own) {
        int32_t slot = -1;
        if (valid_id(own_id, E)) {
            int32_t r = w.part[own_id] + below;
            for (int v = 0; v < w.wave; ++v) r += w.wcnt[v * W + own_id];
            if (p.cap == 0) slot = w.off[own_id] + r;
            else if (r < p.cap) slot = own_id * p.cap + r;
        }
        w.s_slot[(tid / w.k) * w.kp + tid % w.k] = slot;
        // the workgroup holding the token's chunk 0 writes its layout entries
        const int t = w.tA + tid / w.k;
        if (t * p.C >= w.c_begin) {
            p.slot_of[w.P0 + tid] = slot;
            if (slot >= 0 && slot < p.R) p.src_of_slot[slot] = w.P0 + tid;
        }
    }
    // Receive rows no entry fills: past each expert's count (fixed capacity,
    // experts b, b + nwg, ...), or past the valid entries (contiguous).
    if (p.cap > 0) {
        for (int e = w.b; e < E; e += p.nwg) {
            int32_t* rows = p.src_of_slot + static_cast<int64_t>(e) * p.cap;
            const int32_t filled = min(w.part[e] + w.part[W + e], p.cap);
            for (int r = filled + tid; r < p.cap; r += kThreads) rows[r] = -1;
        }
    } else {
        for (int64_t r = w.off[E] + static_cast<int64_t>(w.b) * kThreads + tid; r < p.R;
             r += static_cast<int64_t>(p.nwg) * kThreads)
            p.src_of_slot[r] = -1;
    }
    __syncthreads();
}

// Issue priority for chunk j of Q: it falls from 3 to 0 over the quarters of
// a wave's chunks, so that a SIMD issues for its oldest wave first and a wave
// ahead of the others yields the SIMD to them, as in the persistent combine.
__device__ __forceinline__ void lower_priority(int j, int Q) {
    const int level = (4 * (j + 1)) / Q;
    if (level == 1) __builtin_amdgcn_s_setprio(2);
    else if (level == 2) __builtin_amdgcn_s_setprio(1);
    else if (level >= 3) __builtin_amdgcn_s_setprio(0);
}

// The k slots of the token a chunk belongs to, the same in every lane.
template <int K>
struct TokenSlots {
    int32_t s[K > 0 ? K : 1];
    __device__ __forceinline__ void read(const int32_t* sl) {
#pragma unroll
        for (int j = 0; j < K; ++j) s[j] = __builtin_amdgcn_readfirstlane(sl[j]);
    }
};

// K: the top-k count when it is 1..8 (the store loop is unrolled over the
// token's receive rows, read from LDS together), 0 for any k.
template <int K>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void layout_dispatch_persistent_kernel(PersistParams p) {
    extern __shared__ __align__(16) int32_t s_dyn[];
    __shared__ int32_t s_wsum[kWaves];
    __shared__ int32_t s_wover[kWaves];

    const Part w = make_part<K>(p, s_dyn);
    const int tid = w.tid, lane = w.lane, wave = w.wave;
    const int k = w.k;

    // 1. Loads, in the order their results are needed: a wave's loads return
    // in issue order.  The own entry (clamped address: unconditional) ...
    const int32_t own_raw = p.idx[w.P0 + min(tid, max(w.n_own, 1) - 1)];
    const int32_t own_id = (tid < w.n_own) ? own_raw : -1;
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
    const int c_last = max(w.c_end - 1, 0);
    u32x4 buf[kHold];
    int cid[kHold];
#pragma unroll
    for (int j = 0; j < kHold; ++j) {
        const int c = w.c_begin + wave + j * kWaves;
        const bool mine = j < p.Q && c < w.c_end;
        const int cc = mine ? c : c_last;
        const int t = cc / p.C;
        const int v = min((cc - t * p.C) * kWave + lane, p.nvec - 1);
        buf[j] = __builtin_nontemporal_load(p.x + static_cast<int64_t>(t) * p.nvec + v);
        cid[j] = mine ? c : -1;
    }

    zero_tables(w, p.rw);
    __syncthreads();

    // 2. Histograms of the table, split at the workgroup's first entry, and
    // the own entries' ranks.
#pragma unroll
    for (int u = 0; u < kIdQuads; ++u) count_quad(w, nq, q[u], u * kThreads + tid);
    const int32_t below = rank_own(w, p.rw, own_id);
    __syncthreads();
    merge_copies(w);

    // 3. Offsets, slots and the layout outputs.
    finish_layout(p, w, own_id, below, s_wsum, s_wover);

    // 4. Stores: one wait for the rows, then every store of the wave with no
    // wait in between.
    u32x4* recv = static_cast<u32x4*>(p.recv_x);
    auto store_chunk = [&](int c, const u32x4& data) {
        const int t = c / p.C;
        const int v = min((c - t * p.C) * kWave + lane, p.nvec - 1);
        const int32_t* sl = w.s_slot + (t - w.tA) * w.kp;
        u32x4* dst = recv + v;
        if (K > 0) {
            TokenSlots<K> ts;
            ts.read(sl);
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (ts.s[j] >= 0 && ts.s[j] < p.R)
                    __builtin_nontemporal_store(data, dst + static_cast<int64_t>(ts.s[j]) * p.nvec);
        } else {
            for (int j = 0; j < k; ++j) {
                const int32_t slot = __builtin_amdgcn_readfirstlane(sl[j]);
                if (slot >= 0 && slot < p.R)
                    __builtin_nontemporal_store(data, dst + static_cast<int64_t>(slot) * p.nvec);
            }
        }
    };
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int j = 0; j < kHold; ++j) {
        if (cid[j] >= 0) {  // uniform
            store_chunk(cid[j], buf[j]);
            lower_priority(j, p.Q);
        }
    }
}

// FP8 rows.  The same layout; each chunk is quantised (one 128-channel block
// per 16 lanes, as in the other dispatch kernels) and stored once it has
// arrived and the layout is known.  A wave's loads are all issued before its
// first store.  Its stores sit under branches (an entry without a slot, the
// lanes that write a scale), so where the paths meet the compiler counts
// none of them, and quantising chunk j waits until at most 15 - j of the
// wave's memory operations are in flight: for chunk j, and for most stores
// of the chunks two and more before it.  That holds each wave to about two
// chunks of stores in flight; branch-free stores with exact waits (a buffer
// resource of size 0 where there is nothing to store) ran slower.
//
// UE8M0: power-of-two scales held as exponent bytes.
template <int K, bool UE8M0>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void layout_dispatch_persistent_fp8_kernel(PersistParams p) {
    extern __shared__ __align__(16) int32_t s_dyn[];
    __shared__ int32_t s_wsum[kWaves];
    __shared__ int32_t s_wover[kWaves];

    const Part w = make_part<K>(p, s_dyn);
    const int tid = w.tid, lane = w.lane, wave = w.wave;
    const int k = w.k;

    // Loads as in the bf16 kernel: the own entry, the table, the rows.
    const int32_t own_raw = p.idx[w.P0 + min(tid, max(w.n_own, 1) - 1)];
    const int32_t own_id = (tid < w.n_own) ? own_raw : -1;
    const int4* quads = reinterpret_cast<const int4*>(p.idx);
    const int nq = p.n / 4;
    int4 q[kIdQuads];
#pragma unroll
    for (int u = 0; u < kIdQuads; ++u) q[u] = quads[min(u * kThreads + tid, nq - 1)];
    // Chunk j of the wave: pieces past the end of the row map, 16 lanes at a
    // time, onto the row's last 128-channel block (they redo its codes and
    // store the same bytes to the same place).
    const int c_last = max(w.c_end - 1, 0);
    u32x4 buf[kHoldFp8];
    int cid[kHoldFp8];
#pragma unroll
    for (int j = 0; j < kHoldFp8; ++j) {
        const int c = w.c_begin + wave + j * kWaves;
        const bool mine = j < p.Q && c < w.c_end;
        const int cc = mine ? c : c_last;
        const int t = cc / p.C;
        const int vv = (cc - t * p.C) * kWave + lane;
        const int v = vv < p.nvec ? vv : p.nvec - 16 + (vv & 15);
        buf[j] = __builtin_nontemporal_load(p.x + static_cast<int64_t>(t) * p.nvec + v);
        cid[j] = mine ? c : -1;
    }

    zero_tables(w, p.rw);
    __syncthreads();

#pragma unroll
    for (int u = 0; u < kIdQuads; ++u) count_quad(w, nq, q[u], u * kThreads + tid);
    const int32_t below = rank_own(w, p.rw, own_id);
    __syncthreads();
    merge_copies(w);

    finish_layout(p, w, own_id, below, s_wsum, s_wover);

    u32x2* recv = static_cast<u32x2*>(p.recv_x);
    auto quant_store = [&](int c, const u32x4& data) {
        const int t = c / p.C;
        const int vv = (c - t * p.C) * kWave + lane;
        const int v = vv < p.nvec ? vv : p.nvec - 16 + (vv & 15);
        const float amax = dispatch::row16_max(dispatch::absmax8(data));
        u32x2 code;
        float sval;  // fp32 scale, or the UE8M0 exponent byte
        if (UE8M0) {
            const int s = dispatch::ue8m0_exponent(amax);
            const float factor = __uint_as_float(static_cast<uint32_t>(127 - s) << 23);
            code = dispatch::quant8_pow2(data, factor, amax == 0.0f);
            sval = static_cast<float>(s + 127);
        } else {
            const float scale = amax / 448.0f;
            code = dispatch::quant8(data, scale);
            sval = scale;
        }
        const int32_t* sl = w.s_slot + (t - w.tA) * w.kp;
        u32x2* dst = recv + v;
        // one lane per block writes its scale (plain stores: the 16-byte
        // pieces of a scale row from the row's chunks meet in L2)
        const bool scale_lane = (lane & 15) == 0 && vv < p.nvec;
        const int64_t sidx = vv >> 4;
        if (K > 0) {
            TokenSlots<K> ts;
            ts.read(sl);
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (ts.s[j] >= 0 && ts.s[j] < p.R)
                    __builtin_nontemporal_store(code, dst + static_cast<int64_t>(ts.s[j]) * p.nvec);
            if (scale_lane) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    if (ts.s[j] < 0 || ts.s[j] >= p.R) continue;
                    const int64_t at = static_cast<int64_t>(ts.s[j]) * p.nblk + sidx;
                    if (UE8M0) static_cast<uint8_t*>(p.recv_scales)[at] = static_cast<uint8_t>(sval);
                    else static_cast<float*>(p.recv_scales)[at] = sval;
                }
            }
        } else {
            for (int j = 0; j < k; ++j) {
                const int32_t slot = __builtin_amdgcn_readfirstlane(sl[j]);
                if (slot < 0 || slot >= p.R) continue;
                __builtin_nontemporal_store(code, dst + static_cast<int64_t>(slot) * p.nvec);
                if (scale_lane) {
                    const int64_t at = static_cast<int64_t>(slot) * p.nblk + sidx;
                    if (UE8M0) static_cast<uint8_t*>(p.recv_scales)[at] = static_cast<uint8_t>(sval);
                    else static_cast<float*>(p.recv_scales)[at] = sval;
                }
            }
        }
    };
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int j = 0; j < kHoldFp8; ++j) {
        if (cid[j] >= 0) {  // uniform
            quant_store(cid[j], buf[j]);
            lower_priority(j, p.Q);
        }
    }
}

struct PersistShape {
    int C, Q, maxtok, rw;
};

PersistShape persist_shape(const ep_problem& p, int ncu) {
    PersistShape s;
    const int nvec = p.hidden / 8;
    s.C = (nvec + kWave - 1) / kWave;
    const int64_t nw = static_cast<int64_t>(ncu) * kWaves;
    s.Q = static_cast<int>((static_cast<int64_t>(p.num_tokens) * s.C + nw - 1) / nw);
    s.maxtok = (kWaves * s.Q - 1) / s.C + 2;
    s.rw = (s.maxtok * p.num_topk + kWave - 1) / kWave;
    return s;
}

template <template <int> class Launch, typename... A>
void launch_by_k(int k, A... a) {
    switch (k) {
        case 1: Launch<1>::run(a...); break;
        case 2: Launch<2>::run(a...); break;
        case 3: Launch<3>::run(a...); break;
        case 4: Launch<4>::run(a...); break;
        case 5: Launch<5>::run(a...); break;
        case 6: Launch<6>::run(a...); break;
        case 7: Launch<7>::run(a...); break;
        case 8: Launch<8>::run(a...); break;
        default: Launch<0>::run(a...); break;
    }
}

template <int K>
struct LaunchBf16 {
    static void run(const PersistParams& a, dim3 grid, size_t lds, hipStream_t stream) {
        hipLaunchKernelGGL(layout_dispatch_persistent_kernel<K>, grid, dim3(kThreads), lds, stream, a);
    }
};
template <int K>
struct LaunchFp8 {
    static void run(const PersistParams& a, dim3 grid, size_t lds, hipStream_t stream) {
        hipLaunchKernelGGL((layout_dispatch_persistent_fp8_kernel<K, false>), grid, dim3(kThreads), lds, stream, a);
    }
};
template <int K>
struct LaunchUe8m0 {
    static void run(const PersistParams& a, dim3 grid, size_t lds, hipStream_t stream) {
        hipLaunchKernelGGL((layout_dispatch_persistent_fp8_kernel<K, true>), grid, dim3(kThreads), lds, stream, a);
    }
};

}  // namespace

bool layout_dispatch_persistent_fits(const ep_problem& p, int ncu) {
    if (p.num_tokens <= 0) return false;
    const bool fp8 = p.use_fp8 != 0;
    const int64_t n = static_cast<int64_t>(p.num_tokens) * p.num_topk;
    // whole quads of routing entries (the table is loaded 16 bytes a lane)
    if (n <= kFusedMaxEntries || n > kMaxIds || n % 4 != 0) return false;
    if (fp8 && p.hidden % 128 != 0) return false;
    const int nvec = p.hidden / 8;
    const int64_t C = (nvec + kWave - 1) / kWave;
    const int64_t nw = static_cast<int64_t>(ncu) * kWaves;
    const int64_t all_chunks = static_cast<int64_t>(p.num_tokens) * C;
    // every wave gets a chunk, and one launch holds all of them
    if (all_chunks < nw || all_chunks > nw * (fp8 ? kHoldFp8 : kHold)) return false;
    const int64_t Q = (all_chunks + nw - 1) / nw;
    const int64_t maxtok = (kWaves * Q - 1) / C + 2;
    const int64_t own = maxtok * p.num_topk;
    if (own > kThreads) return false;
    const int rw = static_cast<int>((own + kWave - 1) / kWave);
    return persist_lds_words(p.num_experts, rw, static_cast<int>(maxtok), p.num_topk) * 4 <= kMaxLds;
}

hipError_t launch_layout_dispatch_persistent(const ep_problem& p, const int32_t* topk_idx,
                                             const ep_layout_t& out, const void* x, void* recv_x,
                                             void* recv_scales, int ncu, hipStream_t stream) {
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
    a.recv_x = recv_x;
    a.recv_scales = recv_scales;
    a.T = p.num_tokens;
    a.nvec = p.hidden / 8;
    a.nblk = p.hidden / 128;
    const PersistShape s = persist_shape(p, ncu);
    a.C = s.C;
    a.Q = s.Q;
    a.maxtok = s.maxtok;
    a.rw = s.rw;
    a.nwg = ncu;
    const size_t lds = persist_lds_words(a.E, a.rw, a.maxtok, a.k) * 4;
    const dim3 grid(ncu);
    if (p.use_fp8 == 0) launch_by_k<LaunchBf16>(a.k, a, grid, lds, stream);
    else if (p.use_fp8 == 1) launch_by_k<LaunchFp8>(a.k, a, grid, lds, stream);
    else launch_by_k<LaunchUe8m0>(a.k, a, grid, lds, stream);
    return hipGetLastError();
}

}  // namespace ep
