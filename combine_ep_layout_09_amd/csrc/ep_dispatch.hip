// ep_dispatch.hip -- scatter each token's row into its k receive rows, either
// as a bf16 copy or quantised once to OCP E4M3FN with one fp32 scale per 128
// channels.
//
// The payload of a dispatched token (hidden data plus scale factors) is the
// per-token message of "[PR #693] Pipeline direct NVLink dispatch with
// triple-buffered prefetch", Summary; on one GPU the message is written
// straight into the expert-major receive rows chosen by the layout.
//
// Launch shape: one workgroup per (token, column tile).  A lane owns VPL
// 16-byte pieces of the row, spaced one workgroup-width apart so that every
// load and store instruction of a wave covers contiguous memory (see
// dispatch_shape for the tile sizes); lanes past the end of the row redo the
// last piece (last 16-lane group for FP8) and store the same bytes to the
// same place, which keeps the loads free of branches.  All VPL loads are issued before
// any store, the row is read from HBM once however large k is, and the
// token's k slots are uniform across the workgroup (scalar loads).  Receive
// rows and scales are written with non-temporal stores: they are not read
// again by this kernel, and plain stores would leave them dirty in the caches
// for the next kernels to write back.
//
// A slot of -1 (or one outside [0, R), which a layout of this problem never
// holds) writes nothing.
//
// FP8: a lane holds 8 channels, so a 128-channel block is 16 adjacent lanes
// (one DPP row).  The block maximum of |x| is reduced across the row, the
// scale is amax / 448 (IEEE fp32 division), and each channel gets the
// round-to-nearest-even E4M3 code of its IEEE quotient by the scale, reached
// with one reciprocal per 8 channels and a division only next to E4M3
// rounding midpoints (quant8 in ep_dispatch_dev.h).  The block scales of the
// tile are collected in LDS and written as one contiguous run per slot.

#include "ep_dispatch_dev.h"
#include "ep_internal.h"

namespace ep {
namespace {

using namespace dispatch;

constexpr int kMaxThreads = 1024;

template <int VPL>
__global__ __launch_bounds__(kMaxThreads) void dispatch_bf16_kernel(
        const u32x4* __restrict__ x, int nvec, int k, const int32_t* __restrict__ slot_of,
        int64_t R, u32x4* __restrict__ recv) {
    Bf16Tile<VPL> tile;
    tile.load(x, nvec, blockIdx.x, blockIdx.y, blockDim.x, threadIdx.x);
    tile.store(slot_of + static_cast<int64_t>(blockIdx.x) * k, k, R, recv, nvec);
}

template <int VPL, bool UE8M0>
__global__ __launch_bounds__(kMaxThreads) void dispatch_fp8_kernel(
        const u32x4* __restrict__ x, int nvec, int nblk, int k,
        const int32_t* __restrict__ slot_of, int64_t R, u32x2* __restrict__ recv_q,
        void* __restrict__ recv_scales) {
    extern __shared__ float s_scale[];  // [blockDim * VPL / 16] scales of this tile
    const int32_t* slots = slot_of + static_cast<int64_t>(blockIdx.x) * k;
    Fp8Tile<VPL, UE8M0> tile;
    tile.load_quantise(x, nvec, blockIdx.x, blockIdx.y, blockDim.x, threadIdx.x, s_scale);
    tile.store(slots, k, R, recv_q, nvec);
    __syncthreads();
    if (UE8M0)
        fp8_store_scales(s_scale, slots, k, R, static_cast<uint8_t*>(recv_scales), nblk,
                         blockIdx.y, blockDim.x, VPL, threadIdx.x);
    else
        fp8_store_scales(s_scale, slots, k, R, static_cast<float*>(recv_scales), nblk,
                         blockIdx.y, blockDim.x, VPL, threadIdx.x);
}

// Elementwise use of the same encoder, for callers that quantise other data.
__global__ __launch_bounds__(256) void e4m3_encode_kernel(
        const float* __restrict__ in, uint8_t* __restrict__ out, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += stride) {
        out[i] = static_cast<uint8_t>(f32_to_e4m3_rne(in[i]));
    }
}

}  // namespace

TileShape row_tile_shape(int nvec, int vpl) {
    const int lanes = (nvec + vpl - 1) / vpl;
    const int tiles = (lanes + kMaxThreads - 1) / kMaxThreads;
    const int per_tile = (lanes + tiles - 1) / tiles;
    return {((per_tile + 63) / 64) * 64, tiles};
}

// For batches of 1024 tokens or more, bf16 dispatch tiles are two waves wide
// with up to eight 16-byte pieces per lane, so one workgroup covers a whole
// row of up to 1024 pieces (H = 8192); FP8 tiles have two pieces per lane and
// as many lanes as the row needs (up to 1024).  The pieces of a lane are all
// loaded before the first store.
DispatchShape dispatch_shape(int nvec, int T, bool fp8) {
    // Few tokens (decode batches): one piece per lane, and the row split into
    // as many column tiles as it takes to have about 512 workgroups (two per
    // CU), each at least one wave wide, so that enough waves exist to keep
    // HBM busy.
    if (T < 1024) {
        const int want = min((nvec + 63) / 64, (512 + T - 1) / T);
        const int per = (nvec + want - 1) / want;
        const int threads = min(1024, ((per + 63) / 64) * 64);
        return {1, {threads, (nvec + threads - 1) / threads}};
    }
    if (nvec <= 128) return {1, {((nvec + 63) / 64) * 64, 1}};
    // FP8: quantising holds each piece's raw and encoded forms at once, so two
    // pieces per lane keep the kernel at full occupancy (eight waves per SIMD).
    if (fp8) return {2, row_tile_shape(nvec, 2)};
    const int vpl = two_wave_vpl(nvec);
    return {vpl, {128, (nvec + 128 * vpl - 1) / (128 * vpl)}};
}

namespace {

template <int VPL>
void launch_vpl(const ep_problem& p, dim3 grid, int threads, const void* x, int nvec,
                const int32_t* slot_of, int64_t R, void* recv_x, void* recv_scales,
                hipStream_t stream) {
    if (p.use_fp8) {
        const size_t lds = static_cast<size_t>(threads) * VPL / 16 * 4;
        if (p.use_fp8 == 2)
            hipLaunchKernelGGL((dispatch_fp8_kernel<VPL, true>), grid, dim3(threads), lds, stream,
                               static_cast<const u32x4*>(x), nvec, p.hidden / 128, p.num_topk,
                               slot_of, R, static_cast<u32x2*>(recv_x), recv_scales);
        else
            hipLaunchKernelGGL((dispatch_fp8_kernel<VPL, false>), grid, dim3(threads), lds, stream,
                               static_cast<const u32x4*>(x), nvec, p.hidden / 128, p.num_topk,
                               slot_of, R, static_cast<u32x2*>(recv_x), recv_scales);
    } else {
        hipLaunchKernelGGL(dispatch_bf16_kernel<VPL>, grid, dim3(threads), 0, stream,
                           static_cast<const u32x4*>(x), nvec, p.num_topk, slot_of, R,
                           static_cast<u32x4*>(recv_x));
    }
}

}  // namespace

hipError_t launch_dispatch(const ep_problem& p, const void* x, const int32_t* slot_of,
                           void* recv_x, void* recv_scales, hipStream_t stream) {
    const int T = p.num_tokens;
    if (T == 0) return hipSuccess;
    const int nvec = p.hidden / 8;
    const int64_t R = p.capacity == 0 ? static_cast<int64_t>(T) * p.num_topk
                                      : static_cast<int64_t>(p.num_experts) * p.capacity;
    const DispatchShape ds = dispatch_shape(nvec, T, p.use_fp8 != 0);
    const dim3 grid(T, ds.tile.tiles);
    const int th = ds.tile.threads;
    switch (ds.vpl) {
        case 1: launch_vpl<1>(p, grid, th, x, nvec, slot_of, R, recv_x, recv_scales, stream); break;
        case 2: launch_vpl<2>(p, grid, th, x, nvec, slot_of, R, recv_x, recv_scales, stream); break;
        case 3: launch_vpl<3>(p, grid, th, x, nvec, slot_of, R, recv_x, recv_scales, stream); break;
        case 4: launch_vpl<4>(p, grid, th, x, nvec, slot_of, R, recv_x, recv_scales, stream); break;
        case 5: launch_vpl<5>(p, grid, th, x, nvec, slot_of, R, recv_x, recv_scales, stream); break;
        case 6: launch_vpl<6>(p, grid, th, x, nvec, slot_of, R, recv_x, recv_scales, stream); break;
        case 7: launch_vpl<7>(p, grid, th, x, nvec, slot_of, R, recv_x, recv_scales, stream); break;
        default: launch_vpl<8>(p, grid, th, x, nvec, slot_of, R, recv_x, recv_scales, stream); break;
    }
    return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(e4m3_encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, in, out, n);
    return hipGetLastError();
}

}  // namespace ep
