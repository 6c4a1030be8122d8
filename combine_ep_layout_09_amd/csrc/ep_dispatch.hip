// ep_dispatch.hip -- scatter each token's row into its k receive rows, either
// as a bf16 copy or quantised once to OCP E4M3FN with one fp32 scale per 128
// channels.
//
// The payload of a dispatched token (hidden data plus scale factors) is the
// per-token message of "[PR #693] Pipeline direct NVLink dispatch with
// triple-buffered prefetch", Summary; on one GPU the message is written
// straight into the expert-major receive rows chosen by the layout.
//
// One workgroup per token.  The token's k slots are uniform across the
// workgroup (scalar loads).  A slot of -1 (or one outside [0, R), which a
// layout of this problem never holds) writes nothing.  Each lane loads 16-byte pieces of the token row
// once, holds them in registers, and stores them to every slot, so x is read
// from HBM exactly once however large k is.
//
// FP8: a lane holds 8 channels, so a 128-channel block is 16 adjacent lanes
// (one DPP row).  The block maximum of |x| is reduced across the row, the
// scale is amax / 448 (IEEE fp32 division), each channel is divided by it
// (IEEE fp32 division) and encoded with round-to-nearest-even.  The block
// scales of the token are collected in LDS and written as one contiguous run
// per slot.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte pieces in flight per lane

__global__ __launch_bounds__(kThreads) void dispatch_bf16_kernel(
        const uint4* __restrict__ x, int nvec, int k, const int32_t* __restrict__ slot_of,
        int64_t R, uint4* __restrict__ recv) {
    const int t = blockIdx.x;
    const int32_t* slots = slot_of + static_cast<int64_t>(t) * k;
    const uint4* row = x + static_cast<int64_t>(t) * nvec;
    for (int v0 = threadIdx.x; v0 < nvec; v0 += kThreads * kUnroll) {
        uint4 buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int v = v0 + u * kThreads;
            if (v < nvec) buf[u] = row[v];
        }
        for (int j = 0; j < k; ++j) {
            const int32_t slot = slots[j];
            if (slot < 0 || slot >= R) continue;  // -1: no row; >= R: not this problem's
            uint4* dst = recv + static_cast<int64_t>(slot) * nvec;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int v = v0 + u * kThreads;
                if (v < nvec) dst[v] = buf[u];
            }
        }
    }
}

// Maximum across the 16 lanes of a DPP row (all lanes get the result).
__device__ __forceinline__ float row16_max(float m) {
    m = fmaxf(m, __shfl_xor(m, 1, 16));
    m = fmaxf(m, __shfl_xor(m, 2, 16));
    m = fmaxf(m, __shfl_xor(m, 4, 16));
    m = fmaxf(m, __shfl_xor(m, 8, 16));
    return m;
}

__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, float scale) {
    const float f[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t c = (scale == 0.0f) ? 0u : f32_to_e4m3_rne(f[i] / scale);
        packed |= c << (8 * i);
    }
    return packed;
}

__device__ __forceinline__ float absmax8(const uint4& p) {
    float m = fabsf(bf16_lo(p.x));
    m = fmaxf(m, fabsf(bf16_hi(p.x)));
    m = fmaxf(m, fabsf(bf16_lo(p.y)));
    m = fmaxf(m, fabsf(bf16_hi(p.y)));
    m = fmaxf(m, fabsf(bf16_lo(p.z)));
    m = fmaxf(m, fabsf(bf16_hi(p.z)));
    m = fmaxf(m, fabsf(bf16_lo(p.w)));
    m = fmaxf(m, fabsf(bf16_hi(p.w)));
    return m;
}

// nvec = H / 8 (multiple of 16); nblk = H / 128.
__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
        const uint4* __restrict__ x, int nvec, int nblk, int k,
        const int32_t* __restrict__ slot_of, int64_t R, uint2* __restrict__ recv_q,
        float* __restrict__ recv_scales) {
    extern __shared__ float s_scale[];  // [nblk]
    const int t = blockIdx.x;
    const int32_t* slots = slot_of + static_cast<int64_t>(t) * k;
    const uint4* row = x + static_cast<int64_t>(t) * nvec;
    // Lanes of one 16-lane row are all in range or all out of range because
    // nvec is a multiple of 16 and the loop start is a multiple of 64.
    for (int v0 = 0; v0 < nvec; v0 += kThreads * kUnroll) {
        uint4 buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int v = v0 + u * kThreads + threadIdx.x;
            if (v < nvec) buf[u] = row[v];
        }
        uint2 q[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int v = v0 + u * kThreads + threadIdx.x;
            if (v0 + u * kThreads < nvec) {  // uniform across the workgroup
                const float amax = row16_max(v < nvec ? absmax8(buf[u]) : 0.0f);
                const float scale = amax / 448.0f;
                if (v < nvec) {
                    q[u].x = quant4(buf[u].x, buf[u].y, scale);
                    q[u].y = quant4(buf[u].z, buf[u].w, scale);
                    if ((threadIdx.x & 15) == 0) s_scale[v >> 4] = scale;
                }
            }
        }
        for (int j = 0; j < k; ++j) {
            const int32_t slot = slots[j];
            if (slot < 0 || slot >= R) continue;  // -1: no row; >= R: not this problem's
            uint2* dst = recv_q + static_cast<int64_t>(slot) * nvec;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int v = v0 + u * kThreads + threadIdx.x;
                if (v < nvec) dst[v] = q[u];
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < k * nblk; i += kThreads) {
        const int j = i / nblk;
        const int blk = i - j * nblk;
        const int32_t slot = slots[j];
        if (slot >= 0 && slot < R) recv_scales[static_cast<int64_t>(slot) * nblk + blk] = s_scale[blk];
    }
}

// Elementwise use of the same encoder, for callers that quantise other data.
__global__ __launch_bounds__(kThreads) void e4m3_encode_kernel(
        const float* __restrict__ in, uint8_t* __restrict__ out, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += stride) {
        out[i] = static_cast<uint8_t>(f32_to_e4m3_rne(in[i]));
    }
}

}  // namespace

hipError_t launch_dispatch(const ep_problem& p, const void* x, const int32_t* slot_of,
                           void* recv_x, float* recv_scales, hipStream_t stream) {
    const int T = p.num_tokens;
    if (T == 0) return hipSuccess;
    const int nvec = p.hidden / 8;
    const int64_t R = p.capacity == 0 ? static_cast<int64_t>(T) * p.num_topk
                                      : static_cast<int64_t>(p.num_experts) * p.capacity;
    if (p.use_fp8) {
        const int nblk = p.hidden / 128;
        hipLaunchKernelGGL(dispatch_fp8_kernel, dim3(T), dim3(kThreads),
                           static_cast<size_t>(nblk) * 4, stream,
                           static_cast<const uint4*>(x), nvec, nblk, p.num_topk, slot_of, R,
                           static_cast<uint2*>(recv_x), recv_scales);
    } else {
        hipLaunchKernelGGL(dispatch_bf16_kernel, dim3(T), dim3(kThreads), 0, stream,
                           static_cast<const uint4*>(x), nvec, p.num_topk, slot_of, R,
                           static_cast<uint4*>(recv_x));
    }
    return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(e4m3_encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace ep
