// ep_device.h -- device-side helpers shared by the libep kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

// Immediate of s_waitcnt on gfx9-family ISAs, gfx950 included: vmcnt is split
// over bits [3:0] (low four bits) and [15:14] (high two bits), expcnt is bits
// [6:4] and lgkmcnt bits [11:8].  A field at its maximum (vmcnt 63, expcnt 7,
// lgkmcnt 15) does not wait on that counter.
constexpr unsigned waitcnt_imm(unsigned vmcnt, unsigned expcnt, unsigned lgkmcnt) {
    return (vmcnt & 0xfu) | ((vmcnt >> 4) << 14) | ((expcnt & 0x7u) << 4) |
           ((lgkmcnt & 0xfu) << 8);
}
// Wait until every vector memory operation of the wave has completed (loads
// and stores share the counter); LDS, scalar and export counters untouched.
constexpr unsigned kWaitVmcnt0 = waitcnt_imm(0, 7, 15);
static_assert(kWaitVmcnt0 == 0x0f70u, "gfx9 s_waitcnt encoding of vmcnt(0)");

// Lanes below this one in the wave.
__device__ __forceinline__ uint64_t lanemask_lt() {
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Lanes of `active` whose `key` equals this lane's key, found with one ballot
// per key bit (keys < 2^nbits).  Every lane of the wave must execute it.
__device__ __forceinline__ uint64_t match_peers(uint32_t key, int nbits, uint64_t active) {
    uint64_t m = active;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// bf16 bit patterns (two per 32-bit word, low half first) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN with its sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> OCP E4M3FN code, round to nearest even, saturating to +-448, sign
// kept on zero.  Input must not be NaN.
//   |v| >= 448            -> 0x7E (everything from 448 up rounds to 448 once
//                            the format's top code is NaN and values saturate)
//   2^-6 <= |v| < 448     -> normal codes (3 fraction bits, bias 7)
//   |v| < 2^-6            -> subnormal codes m * 2^-9, m = |v| * 2^9 rounded
//                            to the nearest even integer
// gfx950's v_cvt_pk_fp8_f32 converts two fp32 values to OCP E4M3FN with
// round-to-nearest-even, subnormals included, but gives NaN (0x7F) from 464
// (exclusive) up; clamping the input to [-448, 448] first (v_med3_f32)
// leaves every code below 448 as it is and gives 448 above.  Both are checked
// exhaustively through ep_e4m3_encode: every finite binary32 against a
// library encoder and the saturation rule.
__device__ __forceinline__ float e4m3_clamp(float v) {
    return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// Codes of a, b, c, d in bytes 0..3 of one word.
__device__ __forceinline__ uint32_t f32x4_to_e4m3_rne(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
    return static_cast<uint32_t>(w);
}

// The same for values known to lie in [-464, 464], with no clamp: the
// conversion itself rounds 448 < |v| <= 464 to 448.
__device__ __forceinline__ uint32_t f32x4_to_e4m3_rne_le464(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return static_cast<uint32_t>(w);
}

__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float v) {
    const float c = e4m3_clamp(v);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xffu;
}

}  // namespace ep
