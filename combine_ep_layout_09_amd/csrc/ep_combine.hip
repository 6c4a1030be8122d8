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
// One workgroup per token.  The slots and weights of the token are uniform
// (scalar loads).  For each 16-byte piece of the output row a lane first
// issues the loads of up to 8 expert rows, then runs the FMA chain, so up to
// 8 independent 16-byte loads per lane are in flight.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;   // expert rows loaded before their FMAs

__device__ __forceinline__ void fma8(float (&acc)[8], float w, const uint4& p) {
    acc[0] = __builtin_fmaf(w, bf16_lo(p.x), acc[0]);
    acc[1] = __builtin_fmaf(w, bf16_hi(p.x), acc[1]);
    acc[2] = __builtin_fmaf(w, bf16_lo(p.y), acc[2]);
    acc[3] = __builtin_fmaf(w, bf16_hi(p.y), acc[3]);
    acc[4] = __builtin_fmaf(w, bf16_lo(p.z), acc[4]);
    acc[5] = __builtin_fmaf(w, bf16_hi(p.z), acc[5]);
    acc[6] = __builtin_fmaf(w, bf16_lo(p.w), acc[6]);
    acc[7] = __builtin_fmaf(w, bf16_hi(p.w), acc[7]);
}

__global__ __launch_bounds__(kThreads) void combine_kernel(
        const uint4* __restrict__ eo, int nvec, int k, const int32_t* __restrict__ slot_of,
        int64_t R, const float* __restrict__ weights, uint4* __restrict__ y) {
    const int t = blockIdx.x;
    const int32_t* slots = slot_of + static_cast<int64_t>(t) * k;
    const float* w = weights + static_cast<int64_t>(t) * k;
    uint4* out = y + static_cast<int64_t>(t) * nvec;
    for (int v = threadIdx.x; v < nvec; v += kThreads) {
        float acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += kBatch) {
            uint4 buf[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int j = j0 + u;
                if (j < k) {
                    const int32_t slot = slots[j];
                    if (slot >= 0 && slot < R) buf[u] = eo[static_cast<int64_t>(slot) * nvec + v];
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int j = j0 + u;
                if (j < k && slots[j] >= 0 && slots[j] < R) fma8(acc, w[j], buf[u]);
            }
        }
        uint4 r;
        r.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
        r.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
        r.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
        r.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
        out[v] = r;
    }
}

}  // namespace

hipError_t launch_combine(const ep_problem& p, const void* expert_out, const int32_t* slot_of,
                          const float* topk_weights, void* y, hipStream_t stream) {
    const int T = p.num_tokens;
    if (T == 0) return hipSuccess;
    const int64_t R = p.capacity == 0 ? static_cast<int64_t>(T) * p.num_topk
                                      : static_cast<int64_t>(p.num_experts) * p.capacity;
    hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(expert_out), p.hidden / 8, p.num_topk, slot_of,
                       R, topk_weights, static_cast<uint4*>(y));
    return hipGetLastError();
}

}  // namespace ep
