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
// Launch shape: one workgroup per (token, column tile), VPL 16-byte pieces
// per lane spaced one workgroup-width apart (the same tiling as dispatch).
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

template <int KB>
void launch_kb(dim3 grid, int threads, hipStream_t stream, const u32x4* eo, int nvec, int k,
               const int32_t* slot_of, int64_t R, const float* w, u32x4* y) {
    hipLaunchKernelGGL((combine_kernel<KB, 2>), grid, dim3(threads), 0, stream, eo, nvec, k,
                       slot_of, R, w, y);
}

}  // namespace

hipError_t launch_combine(const ep_problem& p, const void* expert_out, const int32_t* slot_of,
                          const float* topk_weights, void* y, hipStream_t stream) {
    const int T = p.num_tokens;
    if (T == 0) return hipSuccess;
    const int64_t R = p.capacity == 0 ? static_cast<int64_t>(T) * p.num_topk
                                      : static_cast<int64_t>(p.num_experts) * p.capacity;
    const int nvec = p.hidden / 8;
    const TileShape s = row_tile_shape(nvec, 2);
    const dim3 grid(T, s.tiles);
    const auto* eo = static_cast<const u32x4*>(expert_out);
    auto* yo = static_cast<u32x4*>(y);
    const int k = p.num_topk;
    switch (k) {
        case 1: launch_kb<1>(grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 2: launch_kb<2>(grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 3: launch_kb<3>(grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 4: launch_kb<4>(grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 5: launch_kb<5>(grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 6: launch_kb<6>(grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        case 7: launch_kb<7>(grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
        default: launch_kb<8>(grid, s.threads, stream, eo, nvec, k, slot_of, R, topk_weights, yo); break;
    }
    return hipGetLastError();
}

}  // namespace ep
