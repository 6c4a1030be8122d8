// ep_dispatch_dev.h -- device code of dispatch, shared by the dispatch kernels
// and the fused layout + dispatch kernel.
//
// A "tile" is the part of one token row that one group of lanes (gsize lanes,
// a multiple of 64) moves: lane gtid owns VPL 16-byte pieces spaced gsize
// pieces apart, so every wave instruction covers 1 KiB of contiguous memory.
// Loading (and, for FP8, quantising) is separate from storing, so a caller can
// issue its row loads before it knows the receive rows.  Lanes past the end of
// the row redo the last piece (the last 16-lane group for FP8) and store the
// same bytes to the same place, which keeps the loads free of branches.
//
// FP8: a lane holds 8 channels, so a 128-channel block is 16 adjacent lanes
// (one DPP row).  The block maximum of |x| is reduced across the row, the
// scale is amax / 448 (IEEE fp32 division), and each channel gets the
// round-to-nearest-even E4M3 code of its IEEE fp32 quotient by the scale
// (see quant8 for how that is reached with one division per 8 channels).
#pragma once

#include "ep_device.h"

namespace ep {
namespace dispatch {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int VPL>
struct Bf16Tile {
    int v[VPL];
    u32x4 buf[VPL];

    __device__ __forceinline__ void load(const u32x4* __restrict__ x, int nvec, int t, int tile,
                                         int gsize, int gtid) {
        const u32x4* row = x + static_cast<int64_t>(t) * nvec;
        const int base = tile * gsize * VPL + gtid;
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            v[u] = min(base + u * gsize, nvec - 1);
            buf[u] = row[v[u]];
        }
    }

    // Non-temporal stores to every slot in [0, R); slots[j] is the same for
    // every lane of the wave.
    __device__ __forceinline__ void store(const int32_t* slots, int k, int64_t R,
                                          u32x4* __restrict__ recv, int nvec) const {
        for (int j = 0; j < k; ++j) {
            const int32_t slot = __builtin_amdgcn_readfirstlane(slots[j]);
            if (slot < 0 || slot >= R) continue;
            u32x4* dst = recv + static_cast<int64_t>(slot) * nvec;
#pragma unroll
            for (int u = 0; u < VPL; ++u) __builtin_nontemporal_store(buf[u], dst + v[u]);
        }
    }

    // The same with the k <= 32 slots held one per lane (lane j: slot j), so
    // that they come from one LDS read instead of k dependent ones.
    __device__ __forceinline__ void store_lanes(int32_t slot_vec, int k, int64_t R,
                                                u32x4* __restrict__ recv, int nvec) const {
        for (int j = 0; j < k; ++j) {
            const int32_t slot = __builtin_amdgcn_readlane(slot_vec, j);
            if (slot < 0 || slot >= R) continue;
            u32x4* dst = recv + static_cast<int64_t>(slot) * nvec;
#pragma unroll
            for (int u = 0; u < VPL; ++u) __builtin_nontemporal_store(buf[u], dst + v[u]);
        }
    }
};

// Maximum across the 16 lanes of a DPP row (all lanes get the result), for
// values >= 0: rotating the row right by 8, 4, 2 and 1 lanes and keeping the
// larger value leaves every lane with the maximum of all 16.  Non-negative
// floats order like their bit patterns, so the comparison is on integers,
// and the lane moves are DPP operands rather than LDS round trips.
constexpr int kDppRowRor = 0x120;  // row_ror:n is kDppRowRor + n

__device__ __forceinline__ float row16_max(float m) {
    uint32_t b = __float_as_uint(m);
    b = max(b, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), kDppRowRor + 8, 0xf, 0xf, false)));
    b = max(b, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), kDppRowRor + 4, 0xf, 0xf, false)));
    b = max(b, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), kDppRowRor + 2, 0xf, 0xf, false)));
    b = max(b, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), kDppRowRor + 1, 0xf, 0xf, false)));
    return __uint_as_float(b);
}

// E4M3 codes of the 8 channels of one 16-byte piece, each the code of the
// IEEE quotient fl(f / scale) (scale == 0: all codes 0).
//
// Dividing every channel is the ALU cost of FP8 dispatch, so the quotients
// come from one IEEE reciprocal per piece instead: r = fl(1 / scale) and
// p = fl(f * r) carry two roundings of relative error <= 2^-24 each, so p
// lies within 3 * 2^-24 |f / scale| of q = fl(f / scale), inside the interval
// between p (1 - 2^-21) and p (1 + 2^-21) even after the rounding of its two
// ends.  Round-to-nearest-even onto E4M3 is monotone in the value, so where
// both ends of that interval have the same code, q has it too (this holds at
// zero, where the interval is a point, and for fp32-subnormal quotients,
// whose codes are all a signed zero).  A channel whose two end codes differ
// -- a quotient next to a rounding midpoint -- and every channel when r is
// not finite (scale tiny) take the division instead, in a branch a wave
// enters only when one of its lanes needs it.
// Every value encoded here is below 464 in magnitude (|f| <= 448 * scale, and
// the ends exceed p by less than 2^-20 relative), so no clamp is needed.
__device__ __forceinline__ u32x2 quant8(const u32x4& w, float scale) {
    const float f[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                        bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
    u32x2 q;
    if (scale == 0.0f) {
        q.x = 0;
        q.y = 0;
        return q;
    }
    const float r = 1.0f / scale;
    const bool r_ok = __float_as_uint(r) < 0x7f800000u;  // finite (r > 0)
    constexpr float kDown = 1.0f - 0x1p-21f;
    constexpr float kUp = 1.0f + 0x1p-21f;
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = f[i] * r;
    q.x = f32x4_to_e4m3_rne_le464(p[0], p[1], p[2], p[3]);
    q.y = f32x4_to_e4m3_rne_le464(p[4], p[5], p[6], p[7]);
    const uint32_t lo0 = f32x4_to_e4m3_rne_le464(p[0] * kDown, p[1] * kDown, p[2] * kDown, p[3] * kDown);
    const uint32_t hi0 = f32x4_to_e4m3_rne_le464(p[0] * kUp, p[1] * kUp, p[2] * kUp, p[3] * kUp);
    const uint32_t lo1 = f32x4_to_e4m3_rne_le464(p[4] * kDown, p[5] * kDown, p[6] * kDown, p[7] * kDown);
    const uint32_t hi1 = f32x4_to_e4m3_rne_le464(p[4] * kUp, p[5] * kUp, p[6] * kUp, p[7] * kUp);
    const uint32_t d0 = r_ok ? lo0 ^ hi0 : ~0u;  // nonzero byte: that channel divides
    const uint32_t d1 = r_ok ? lo1 ^ hi1 : ~0u;
    if (__ballot((d0 | d1) != 0)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if ((d0 >> (8 * i)) & 0xffu) p[i] = f[i] / scale;
            if ((d1 >> (8 * i)) & 0xffu) p[4 + i] = f[4 + i] / scale;
        }
        q.x = f32x4_to_e4m3_rne_le464(p[0], p[1], p[2], p[3]);
        q.y = f32x4_to_e4m3_rne_le464(p[4], p[5], p[6], p[7]);
    }
    return q;
}

// UE8M0 block scale: the exponent s of the smallest power of two 2^s,
// s >= -127, with 448 * 2^s >= amax (>= 0).  For amax = (1 + M/2^23) 2^e,
// amax / 448 = ((1 + M/2^23) / 1.75) 2^(e-8), and the first factor lies in
// (0.57, 1] when M <= 0x600000 (1.75 = 1 + 0x600000/2^23) and in (1, 1.15)
// otherwise; subnormal and zero amax fall to the clamp.
__device__ __forceinline__ int ue8m0_exponent(float amax) {
    const uint32_t b = __float_as_uint(amax);
    const int s = static_cast<int>(b >> 23) - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
    return s < -127 ? -127 : s;
}

// E4M3 codes of the 8 channels of one piece scaled by a power of two
// (factor = 2^-s: the product is exact, so this is the code of x / 2^s); an
// all-zero block gives all codes 0.
__device__ __forceinline__ u32x2 quant8_pow2(const u32x4& w, float factor, bool zero_block) {
    const float f[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                        bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
    u32x2 q;  // |f * factor| <= 448: no clamp needed
    q.x = zero_block ? 0u : f32x4_to_e4m3_rne_le464(f[0] * factor, f[1] * factor, f[2] * factor, f[3] * factor);
    q.y = zero_block ? 0u : f32x4_to_e4m3_rne_le464(f[4] * factor, f[5] * factor, f[6] * factor, f[7] * factor);
    return q;
}

__device__ __forceinline__ float absmax8(const u32x4& p) {
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

// nvec = H / 8 (a multiple of 16).  gsize is a multiple of 64, so 16-lane
// groups never straddle the end of the row: a group past the end maps as a
// whole onto the row's last group.
// UE8M0 = false: fp32 scale amax / 448 per block; true: power-of-two scale
// held as its exponent byte (kept as a small float in s_scale).
template <int VPL, bool UE8M0 = false>
struct Fp8Tile {
    int v[VPL];
    u32x2 q[VPL];
    u32x4 buf[VPL];  // raw bf16 pieces between load() and quantise()

    __device__ __forceinline__ void load(const u32x4* __restrict__ x, int nvec, int t, int tile,
                                         int gsize, int gtid) {
        const u32x4* row = x + static_cast<int64_t>(t) * nvec;
        const int tile0 = tile * gsize * VPL;
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const int vv = tile0 + u * gsize + gtid;
            v[u] = (vv < nvec) ? vv : nvec - 16 + (vv & 15);
            buf[u] = row[v[u]];
        }
    }

    // s_scale: this tile's gsize * VPL / 16 block scales (LDS).
    __device__ __forceinline__ void quantise(int nvec, int tile, int gsize, int gtid,
                                             float* s_scale) {
        const int tile0 = tile * gsize * VPL;
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const float amax = row16_max(absmax8(buf[u]));
            float stored;
            if (UE8M0) {
                const int s = ue8m0_exponent(amax);
                const float factor = __uint_as_float(static_cast<uint32_t>(127 - s) << 23);
                q[u] = quant8_pow2(buf[u], factor, amax == 0.0f);
                stored = static_cast<float>(s + 127);
            } else {
                const float scale = amax / 448.0f;
                q[u] = quant8(buf[u], scale);
                stored = scale;
            }
            const int vv = tile0 + u * gsize + gtid;
            if ((gtid & 15) == 0 && vv < nvec) s_scale[(vv - tile0) >> 4] = stored;
        }
    }

    __device__ __forceinline__ void load_quantise(const u32x4* __restrict__ x, int nvec, int t,
                                                  int tile, int gsize, int gtid, float* s_scale) {
        load(x, nvec, t, tile, gsize, gtid);
        quantise(nvec, tile, gsize, gtid, s_scale);
    }

    __device__ __forceinline__ void store(const int32_t* slots, int k, int64_t R,
                                          u32x2* __restrict__ recv_q, int nvec) const {
        for (int j = 0; j < k; ++j) {
            const int32_t slot = __builtin_amdgcn_readfirstlane(slots[j]);
            if (slot < 0 || slot >= R) continue;
            u32x2* dst = recv_q + static_cast<int64_t>(slot) * nvec;
#pragma unroll
            for (int u = 0; u < VPL; ++u) __builtin_nontemporal_store(q[u], dst + v[u]);
        }
    }

    // With the k <= 32 slots held one per lane (lane j: slot j).
    __device__ __forceinline__ void store_lanes(int32_t slot_vec, int k, int64_t R,
                                                u32x2* __restrict__ recv_q, int nvec) const {
        for (int j = 0; j < k; ++j) {
            const int32_t slot = __builtin_amdgcn_readlane(slot_vec, j);
            if (slot < 0 || slot >= R) continue;
            u32x2* dst = recv_q + static_cast<int64_t>(slot) * nvec;
#pragma unroll
            for (int u = 0; u < VPL; ++u) __builtin_nontemporal_store(q[u], dst + v[u]);
        }
    }
};

// Writes the tile's block scales (staged in s_scale by quantise, after a
// barrier) as one contiguous run per slot: fp32 scales (S = float) or UE8M0
// exponent bytes (S = uint8_t).
template <typename S>
__device__ __forceinline__ void fp8_store_scales(const float* s_scale, const int32_t* slots, int k,
                                                 int64_t R, S* __restrict__ recv_scales,
                                                 int nblk, int tile, int gsize, int vpl, int gtid) {
    const int b0 = (tile * gsize * vpl) >> 4;
    const int nb = min(gsize * vpl / 16, nblk - b0);
    for (int i = gtid; i < k * nb; i += gsize) {
        const int j = i / nb;
        const int b = i - j * nb;
        const int32_t slot = slots[j];
        if (slot >= 0 && slot < R)
            __builtin_nontemporal_store(static_cast<S>(s_scale[b]),
                                        recv_scales + static_cast<int64_t>(slot) * nblk + b0 + b);
    }
}

// Pieces per lane for two-wave tiles covering whole rows of up to 1024 pieces.
__host__ __device__ constexpr int two_wave_vpl(int nvec) {
    return nvec >= 1024 ? 8 : (nvec + 127) / 128;
}

}  // namespace dispatch
}  // namespace ep
