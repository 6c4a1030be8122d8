// ep_combine.hip -- gather each token's k expert-output rows and form the
// routing-weighted sum in fp32, rounded once to bf16.
//
// The pages measure combine only as a transfer rate ("[PR #693] Pipeline
// direct NVLink dispatch with triple-buffered prefetch", Validation tables);
// on one GPU it is a gather-reduce over the receive rows the layout assigned.
//
// Summation order is fixed: acc starts at +0.0f and takes one fused
// multiply-add per routing entry, j = 0 .. k-1, skipping entries without a
// slot (slot -1, or outside [0, R), which a layout of this problem never
// holds).  Every lane follows exactly that chain for each of its channels, so
// the result does not depend on the launch shape.
//
// Two launch forms compute exactly this chain.  Prefill-sized batches use
// the persistent form further down (every wave reads all its rows before it
// writes).  Otherwise: one
// workgroup per (token, column tile), VPL 16-byte pieces per lane spaced one
// workgroup-width apart (the same tiling as dispatch; small batches take one
// piece per lane and narrower tiles, so that every CU gets work).
// Entries are taken in batches of KB: the lane first issues the loads of all
// KB expert rows for all its pieces -- with no branches, so they are all in
// flight together -- and then runs the FMA chain.  An entry without a slot
// loads a row the token does use (a cache hit) and its FMA result is
// discarded by a select, which keeps the chain exactly "skip this term".
// Expert rows are read with non-temporal loads: each is read once.  The
// output rows are written with non-temporal stores too: written with plain
// stores they stay dirty in the caches and their write-back lands on the
// kernels that run next (measured: 235 MB of plain-stored output slows the
// following FP8 dispatch of the 16384-token workload by about a third).

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxThreads = 1024;

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int KB, int VPL>
__global__ __launch_bounds__(kMaxThreads) void combine_kernel(
        const u32x4* __restrict__ eo, int nvec, int k, const int32_t* __restrict__ slot_of,
        int64_t R, const float* __restrict__ weights, u32x4* __restrict__ y) {
    const int t = blockIdx.x;
    const int32_t* slots = slot_of + static_cast<int64_t>(t) * k;
    const float* w = weights + static_cast<int64_t>(t) * k;
    const int base = blockIdx.y * blockDim.x * VPL + threadIdx.x;
    int v[VPL];
#pragma unroll
    for (int u = 0; u < VPL; ++u) v[u] = min(base + u * static_cast<int>(blockDim.x), nvec - 1);

    // A receive row this token uses, for the loads of entries it does not use.
    int32_t safe = -1;
    for (int j = 0; j < k; ++j) {
        const int32_t s = slots[j];
        if (s >= 0 && s < R) {
            safe = s;
            break;
        }
    }

    float acc[VPL][8];
#pragma unroll
    for (int u = 0; u < VPL; ++u)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[u][c] = 0.0f;

    if (safe >= 0) {
        for (int j0 = 0; j0 < k; j0 += KB) {
            bool ok[KB];
            float wj[KB];
            const u32x4* src[KB];
#pragma unroll
            for (int jj = 0; jj < KB; ++jj) {
                const int j = j0 + jj;
                const int32_t s = (j < k) ? slots[j] : -1;
                ok[jj] = s >= 0 && s < R;
                wj[jj] = ok[jj] ? w[j] : 0.0f;
                src[jj] = eo + static_cast<int64_t>(ok[jj] ? s : safe) * nvec;
            }
            u32x4 buf[VPL][KB];
#pragma unroll
            for (int jj = 0; jj < KB; ++jj)
#pragma unroll
                for (int u = 0; u < VPL; ++u) buf[u][jj] = __builtin_nontemporal_load(src[jj] + v[u]);
#pragma unroll
            for (int jj = 0; jj < KB; ++jj) {
#pragma unroll
                for (int u = 0; u < VPL; ++u) {
                    const u32x4 p = buf[u][jj];
                    const float f[8] = {lo16(p.x), hi16(p.x), lo16(p.y), hi16(p.y),
                                        lo16(p.z), hi16(p.z), lo16(p.w), hi16(p.w)};
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float a = __builtin_fmaf(wj[jj], f[c], acc[u][c]);
                        acc[u][c] = ok[jj] ? a : acc[u][c];
                    }
                }
            }
        }
    }

    u32x4* out = y + static_cast<int64_t>(t) * nvec;
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
        u32x4 r;
        r.x = f32_to_bf16_rne(acc[u][0]) | (f32_to_bf16_rne(acc[u][1]) << 16);
        r.y = f32_to_bf16_rne(acc[u][2]) | (f32_to_bf16_rne(acc[u][3]) << 16);
        r.z = f32_to_bf16_rne(acc[u][4]) | (f32_to_bf16_rne(acc[u][5]) << 16);
        r.w = f32_to_bf16_rne(acc[u][6]) | (f32_to_bf16_rne(acc[u][7]) << 16);
        __builtin_nontemporal_store(r, out + v[u]);
    }
}

// ---- persistent form: every wave reads all its rows, then writes ----------
//
// HBM pays for switching between reads and writes; a combine whose 2TH bytes
// of output stores are spread evenly through its 2VH bytes of row loads
// runs well below the rate of the loads alone (measured: the prefill
// combine's loads alone take about 70 us, its stores alone about 13 us,
// interleaved about 93 us).  Here one 1024-lane workgroup per CU owns a
// contiguous run of (token, 64-piece chunk) units, each of its waves up to
// kHold of them, which it computes into registers -- one chunk at a time per
// wave, since its loads must not be hoisted into the held registers -- and
// only then stores.  Every wave does the same amount of work from the same start, so
// the waves of the whole chip reach their store bursts at about the same
// time, without any barrier.  Larger problems take one launch per kHold
// chunks per wave, over consecutive token ranges: a kernel boundary keeps
// each launch's read and write phases aligned across the chip, which waves
// looping over rounds inside one launch do not stay (measured: 4 rounds in
// one launch at the 16384-token prefill were 7% slower than the per-token
// kernel).

constexpr int kPersistThreads = 1024;
constexpr int kPersistWaves = kPersistThreads / kWave;
// chunks held per lane (64 registers); with 16 rather than 14, the skewed
// 8192-token shape (16 chunks per wave) takes one launch instead of two
// (76.6 us against 2 x 40.3 us)
constexpr int kHold = 16;
constexpr int kMaxPersistLaunches = 16;

struct PersistShape {
    int C;        // 64-piece chunks per token row
    int t0;       // first token of this launch
    int chunks;   // chunks of this launch: (its tokens) * C, <= waves * kHold
    int Q;        // chunks per wave, <= kHold
};

// One 16-byte output piece v of token t: the fixed-order FMA chain over the
// token's entries, rounded to bf16.  An entry without a slot loads receive
// row 0 (which always exists) and its FMA result is discarded by a select,
// so that the slot loads do not depend on each other.  EXACT: k == KB, a
// compile-time count, so that the token's slots and weights are unconditional
// (merged) scalar loads.
template <int KB, bool EXACT>
__device__ __forceinline__ u32x4 combine_piece(const u32x4* __restrict__ eo, int nvec, int k_arg,
                                               const int32_t* __restrict__ slots,
                                               const float* __restrict__ w, int64_t R, int v) {
    const int k = EXACT ? KB : k_arg;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += KB) {
        bool ok[KB];
        float wj[KB];
        u32x4 buf[KB];
#pragma unroll
        for (int jj = 0; jj < KB; ++jj) {
            const int j = j0 + jj;
            const int32_t s = (j < k) ? slots[j] : -1;
            ok[jj] = s >= 0 && s < R;
            wj[jj] = (j < k) ? w[j] : 0.0f;
            buf[jj] = __builtin_nontemporal_load(eo + static_cast<int64_t>(ok[jj] ? s : 0) * nvec + v);
        }
        // all of the batch's loads are issued before the first is used
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < KB; ++jj) {
            const u32x4 p = buf[jj];
            const float f[8] = {lo16(p.x), hi16(p.x), lo16(p.y), hi16(p.y),
                                lo16(p.z), hi16(p.z), lo16(p.w), hi16(p.w)};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float a = __builtin_fmaf(wj[jj], f[c], acc[c]);
                acc[c] = ok[jj] ? a : acc[c];
            }
        }
    }
    u32x4 r;
    r.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    r.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    r.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
    r.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
    return r;
}

// The KB slots and weights of a token (scalar loads).  PIN: the values are
// tied to this point by an empty asm, so that the loads are issued here --
// under the row loads of the chunk before -- and not sunk by the compiler
// to their first use, in front of the next chunk's row loads.
template <int KB, bool PIN = false>
__device__ __forceinline__ void load_entries(const int32_t* __restrict__ slots,
                                             const float* __restrict__ w, int32_t (&s)[KB],
                                             float (&wt)[KB]) {
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        s[jj] = slots[jj];
        wt[jj] = w[jj];
    }
    if (PIN) {
#pragma unroll
        for (int jj = 0; jj < KB; ++jj) asm volatile("" : "+s"(s[jj]), "+s"(wt[jj]));
    }
}

// combine_piece for k == KB with the token's slots and weights already in
// hand (s, w): issues the KB row loads, runs `between` (which fetches the
// next chunk's entries into s and w's successors), then the FMA chain.  On
// return s and w hold what `between` fetched.
template <int KB, typename Between>
__device__ __forceinline__ u32x4 reduce_rows(const u32x4* __restrict__ eo, int nvec, int64_t R,
                                             int v, int32_t (&s)[KB], float (&w)[KB],
                                             Between between) {
    bool ok[KB];
    u32x4 buf[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        ok[jj] = s[jj] >= 0 && s[jj] < R;
        buf[jj] = __builtin_nontemporal_load(eo + static_cast<int64_t>(ok[jj] ? s[jj] : 0) * nvec + v);
    }
    float wj[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) wj[jj] = w[jj];
    between(s, w);
    // all of the rows' loads (and the next entries' fetch) are issued before
    // the first row is used
    __builtin_amdgcn_sched_barrier(0);
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        const u32x4 p = buf[jj];
        const float f[8] = {lo16(p.x), hi16(p.x), lo16(p.y), hi16(p.y),
                            lo16(p.z), hi16(p.z), lo16(p.w), hi16(p.w)};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float a = __builtin_fmaf(wj[jj], f[c], acc[c]);
            acc[c] = ok[jj] ? a : acc[c];
        }
    }
    u32x4 r;
    r.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    r.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    r.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
    r.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
    return r;
}

// One workgroup per CU is four waves per SIMD; telling the compiler so lets
// it keep all of a chunk's row loads in flight instead of trading them for
// registers.
template <int KB, bool EXACT>
__global__ __launch_bounds__(kPersistThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void combine_persistent_kernel(
        const u32x4* __restrict__ eo, int nvec, int k, const int32_t* __restrict__ slot_of,
        int64_t R, const float* __restrict__ weights, u32x4* __restrict__ y, PersistShape ps) {
    const int lane = static_cast<int>(lane_id());
    // the same for every lane of a wave: scalar from here on
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    // Workgroup b owns the contiguous chunks [b * 16 Q, (b + 1) * 16 Q) of the
    // launch; wave w takes chunks w, w + 16, w + 32, ... of them, so that the
    // waves of a CU work on neighbouring chunks -- different column chunks of
    // a few rows -- at any time.  With a contiguous run per wave, all waves
    // of the chip read the same column chunk of their rows at once, which for
    // rows of a multiple of 4 KiB lands on the same HBM channels (measured
    // at H = 4096: 57.8 us against 52.9 us for the per-token kernel; strided,
    // 52.4 us).
    const int base = static_cast<int>(blockIdx.x) * kPersistWaves * ps.Q + wave;
    auto chunk_of = [&](int i, int& t, int& v) {
        const int c = base + i * kPersistWaves;  // chunks of one launch < 2^31
        const int tt = c / ps.C;
        t = ps.t0 + tt;
        v = min((c - tt * ps.C) * kWave + lane, nvec - 1);
    };
    u32x4 out[kHold];
    uint32_t dep = 0;
    // k == KB: the slots and weights of the chunk about to be reduced,
    // fetched one chunk ahead (a scalar load of them in front of every
    // chunk's row loads was a dependent round trip per chunk)
    int32_t sc[KB];
    float wc[KB];
    if (EXACT) {
        const int64_t t0 = ps.t0 + min(base, ps.chunks - 1) / ps.C;
        load_entries<KB>(slot_of + t0 * KB, weights + t0 * KB, sc, wc);
    }
#pragma unroll
    for (int i = 0; i < kHold; ++i) {
        // A SIMD issues for its oldest wave first, so with equal shares the
        // older waves of a CU finish their reads well before the younger
        // ones and start their stores while the others still read.  Each
        // wave lowers its issue priority as it gets through its share (3 for
        // its first quarter of chunks, 0 for its last), which keeps the waves
        // of a CU in step (measured at the 4096-token prefill: 87.2-87.9 us
        // against 89.8-90.2 us).
        const int level = (4 * i) / ps.Q;  // uniform
        if (level == 0) __builtin_amdgcn_s_setprio(3);
        else if (level == 1) __builtin_amdgcn_s_setprio(2);
        else if (level == 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        if (i < ps.Q && base + i * kPersistWaves < ps.chunks) {  // uniform
            int t, v;
            chunk_of(i, t, v);
            // this chunk's loads may not move above the previous result
            asm volatile("" : "+v"(v) : "v"(dep));
            if (EXACT) {
                out[i] = reduce_rows<KB>(eo, nvec, R, v, sc, wc, [&](int32_t (&sn)[KB], float (&wn)[KB]) {
                    // the next chunk's slots and weights, while this chunk's
                    // rows load (the last chunk of a launch refetches its own)
                    const int cn = min(base + (i + 1) * kPersistWaves, ps.chunks - 1);
                    const int64_t tn = ps.t0 + cn / ps.C;
                    load_entries<KB, true>(slot_of + tn * KB, weights + tn * KB, sn, wn);
                });
            } else {
                out[i] = combine_piece<KB, EXACT>(eo, nvec, k, slot_of + static_cast<int64_t>(t) * k,
                                                  weights + static_cast<int64_t>(t) * k, R, v);
            }
            dep = out[i].x;
        }
    }
#pragma unroll
    for (int i = 0; i < kHold; ++i) {
        if (i < ps.Q && base + i * kPersistWaves < ps.chunks) {
            int t, v;
            chunk_of(i, t, v);
            __builtin_nontemporal_store(out[i], y + static_cast<int64_t>(t) * nvec + v);
        }
    }
}

template <int KB>
void launch_kb(int vpl, dim3 grid, int threads, hipStream_t stream, const u32x4* eo, int nvec,
               int k, const int32_t* slot_of, int64_t R, const float* w, u32x4* y) {
    if (vpl == 1)
        hipLaunchKernelGGL((combine_kernel<KB, 1>), grid, dim3(threads), 0, stream, eo, nvec, k,
                           slot_of, R, w, y);
    else
        hipLaunchKernelGGL((combine_kernel<KB, 2>), grid, dim3(threads), 0, stream, eo, nvec, k,
                           slot_of, R, w, y);
}

// k <= 8: KB = k exactly; larger k: batches of 8.
template <int KB>
void launch_persistent(int nwg, hipStream_t stream, const u32x4* eo, int nvec, int k,
                       const int32_t* slot_of, int64_t R, const float* w, u32x4* y,
                       const PersistShape& ps) {
    if (k == KB)
        hipLaunchKernelGGL((combine_persistent_kernel<KB, true>), dim3(nwg),
                           dim3(kPersistThreads), 0, stream, eo, nvec, k, slot_of, R, w, y, ps);
    else
        hipLaunchKernelGGL((combine_persistent_kernel<KB, false>), dim3(nwg),
                           dim3(kPersistThreads), 0, stream, eo, nvec, k, slot_of, R, w, y, ps);
}

}  // namespace

hipError_t launch_combine(const ep_problem& p, const void* expert_out, const int32_t* slot_of,
                          const float* topk_weights, void* y, hipStream_t stream) {
    const int T = p.num_tokens;
    if (T == 0) return hipSuccess;
    const int64_t R = p.capacity == 0 ? static_cast<int64_t>(T) * p.num_topk
                                      : static_cast<int64_t>(p.num_experts) * p.capacity;
    const int nvec = p.hidden / 8;
    const auto* eo = static_cast<const u32x4*>(expert_out);
    auto* yo = static_cast<u32x4*>(y);
    const int k = p.num_topk;

    // Persistent form when every wave of one workgroup per CU gets at least
    // one chunk: launches over consecutive token ranges of at most kHold
    // chunks per wave each, up to kMaxPersistLaunches of them (more would
    // pay more in launch gaps than the aligned phases save).
    int dev = 0, ncu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const int C = (nvec + kWave - 1) / kWave;
    const int64_t nw = static_cast<int64_t>(ncu) * kPersistWaves;
    const int64_t all_chunks = static_cast<int64_t>(T) * C;
    int64_t launches = (all_chunks + nw * kHold - 1) / (nw * kHold);
    int64_t per = 0;  // tokens per launch, so that no wave gets more than kHold chunks
    for (;; ++launches) {
        per = (T + launches - 1) / launches;
        if ((per * C + nw - 1) / nw <= kHold) break;
    }
    if (all_chunks >= nw && launches <= kMaxPersistLaunches) {
        for (int64_t t0 = 0; t0 < T; t0 += per) {
            PersistShape ps;
            ps.C = C;
            ps.t0 = static_cast<int>(t0);
            ps.chunks = static_cast<int>(min(per, static_cast<int64_t>(T) - t0) * C);
            ps.Q = static_cast<int>((ps.chunks + nw - 1) / nw);
            switch (k) {
                case 1: launch_persistent<1>(ncu, stream, eo, nvec, k, slot_of, R, topk_weights, yo, ps); break;
                case 2: launch_persistent<2>(ncu, stream, eo, nvec, k, slot_of, R, topk_weights, yo, ps); break;
                case 3: launch_persistent<3>(ncu, stream, eo, nvec, k, slot_of, R, topk_weights, yo, ps); break;
                case 4: launch_persistent<4>(ncu, stream, eo, nvec, k, slot_of, R, topk_weights, yo, ps); break;
                case 5: launch_persistent<5>(ncu, stream, eo, nvec, k, slot_of, R, topk_weights, yo, ps); break;
                case 6: launch_persistent<6>(ncu, stream, eo, nvec, k, slot_of, R, topk_weights, yo, ps); break;
                case 7: launch_persistent<7>(ncu, stream, eo, nvec, k, slot_of, R, topk_weights, yo, ps); break;
                default: launch_persistent<8>(ncu, stream, eo, nvec, k, slot_of, R, topk_weights, yo, ps); break;
            }
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    }

    TileShape s = row_tile_shape(nvec, 2);
    int vpl = 2;
    if (static_cast<int64_t>(T) * s.tiles < 2 * static_cast<int64_t>(ncu)) {
        // Small batches (decode): one piece per lane and narrower column
        // tiles, so that every CU gets about two workgroups.
        const int want = static_cast<int>(min(static_cast<int64_t>((nvec + 63) / 64),
                                              (2 * static_cast<int64_t>(ncu) + T - 1) / T));
        const int per = (nvec + want - 1) / want;
        s.threads = min(1024, ((per + 63) / 64) * 64);
        s.tiles = (nvec + s.threads - 1) / s.threads;
        vpl = 1;
    }
    const dim3 grid(T, s.tiles);
    switch (k) {
        case 1: launch_kb<1>(vpl, grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 2: launch_kb<2>(vpl, grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 3: launch_kb<3>(vpl, grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 4: launch_kb<4>(vpl, grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 5: launch_kb<5>(vpl, grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 6: launch_kb<6>(vpl, grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 7: launch_kb<7>(vpl, grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        default: launch_kb<8>(vpl, grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
    }
    return hipGetLastError();
}

}  // namespace ep
