// ep_oracle.cpp -- plain, serial CPU oracle for MoE token dispatch / combine.
//
// TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
// GPU library is checked against.  Only the tests, the smoke check and the
// CPU-baseline leg of the benchmark load it.  It shares no source, header,
// table or helper with the GPU library and must never be linked into it.
//
// Built with g++ -O2 -ffp-contract=off -fno-fast-math: every float operation
// below is one IEEE-754 binary32 operation rounded to nearest-even, with
// subnormals, exactly as written (no contraction, no reassociation).
//
// What the pages fix and what they leave open
// -------------------------------------------
// * Per-expert token counts and the expert-major receive layout: the low-latency
//   dispatch code quoted in "[GH-ISSUE #282] Redundant atomics in
//   internode_ll" keeps a count of tokens sent per expert and a receive count
//   array indexed [local expert][source rank]; with one GPU holding every
//   expert that is count[E].
// * Order inside one expert's segment: "[GH-ISSUE #18] Reasons for not calling
//   NVSHMEM public APIs?" (maintainer answer on low-latency mode) requires data
//   of one expert to stay in order; read here as ascending (t, j) row-major
//   order of the routing table, i.e. a stable counting sort.
// * Per-token dispatch message = hidden data + scale factors + metadata +
//   routing information: "[PR #693] Pipeline direct NVLink dispatch with
//   triple-buffered prefetch", Summary.
// * The arithmetic itself (one fp32 scale per 128 channels, scale = amax/448,
//   OCP E4M3FN round-to-nearest-even, fp32 weighted sum rounded to bf16 with a
//   fixed top-k order) is not on the pages; it is the definition this library
//   implements and is written out below exactly as defined.  The UE8M0 scale
//   variant is named on the pages ("[PR #206] [MERGED] Support UE8M0 data
//   format") and read as a power-of-two scale held as its exponent byte.
//
// Parity pins (what checks this file against something other than itself)
// live in tests/test_oracle_pins.py.

#include <cassert>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------

// A bf16 value is the top 16 bits of a binary32; widening is exact.
float bf16_bits_to_float(uint16_t b) {
    uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return f;
}

uint32_t float_bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, sizeof u);
    return u;
}

// Value of a bf16 magnitude pattern (sign cleared), treating the all-ones
// exponent with zero mantissa as 2^128 so that "round up past the largest
// finite value" is an ordinary candidate (IEEE rounds with unbounded exponent
// and then overflows to infinity).
double bf16_magnitude_value(uint32_t mag) {
    uint32_t exp = mag >> 7, man = mag & 0x7f;
    if (exp == 0) return std::ldexp(static_cast<double>(man), -133);       // subnormal: m * 2^-133
    return std::ldexp(1.0 + man / 128.0, static_cast<int>(exp) - 127);    // normal
}

// Round a finite binary32 to the nearest bf16, ties to the even pattern.
// Definition written out: take the two bf16 magnitudes that bracket |f|,
// pick the nearer in exact (double) arithmetic, break a tie toward the
// pattern whose last mantissa bit is 0.  Overflow past the largest finite
// bf16 gives infinity.  NaN gives the quiet NaN with the same sign.
uint16_t bf16_round(float f) {
    uint32_t u = float_bits(f);
    uint32_t sign = u >> 31;
    if (std::isnan(f)) return static_cast<uint16_t>((sign << 15) | 0x7fc0);
    if (std::isinf(f)) return static_cast<uint16_t>((sign << 15) | 0x7f80);
    double a = std::fabs(static_cast<double>(f));
    uint32_t lo = (u & 0x7fffffffu) >> 16;   // largest bf16 magnitude <= |f|
    uint32_t hi = lo + 1;                      // next one up
    double dlo = a - bf16_magnitude_value(lo);
    double dhi = bf16_magnitude_value(hi) - a;
    uint32_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = (lo % 2 == 0) ? lo : hi;
    if (pick >= 0x7f80) pick = 0x7f80;        // overflow -> infinity
    return static_cast<uint16_t>((sign << 15) | pick);
}

// ---------------------------------------------------------------------------
// OCP 8-bit floating point, E4M3FN variant (OFP8 v1.0): 1 sign, 4 exponent
// bits with bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111,
// largest finite 448 (0x7E), smallest normal 2^-6, smallest subnormal 2^-9.
// ---------------------------------------------------------------------------

// Closed-form decode of a code (NaN codes return NaN).
double e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xf, m = c & 0x7;
    if (e == 0xf && m == 0x7) return std::nan("");
    double mag = (e == 0) ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

// The 127 non-negative finite values in code order 0x00..0x7E; increasing.
struct E4m3Table {
    double v[127];
    E4m3Table() {
        for (int c = 0; c < 127; ++c) v[c] = e4m3_decode(static_cast<uint8_t>(c));
    }
};
const E4m3Table kE4m3;

// Round a finite binary32 to E4M3FN: nearest representable value, ties to the
// code whose last mantissa bit is 0 (the even code), saturating to +-448 for
// magnitudes beyond the largest finite value.  The sign bit is kept on zero
// results (-0.0 and small negatives give 0x80).
uint8_t e4m3_encode(float f) {
    assert(std::isfinite(f));
    uint8_t sign = std::signbit(f) ? 0x80 : 0x00;
    double a = std::fabs(static_cast<double>(f));
    if (a >= kE4m3.v[126]) return sign | 0x7e;          // at or above 448: saturate
    // Largest code c with value <= a (binary search over the increasing table).
    int lo = 0, hi = 126;                                // invariant: v[lo] <= a < v[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (kE4m3.v[mid] <= a) lo = mid; else hi = mid;
    }
    double dlo = a - kE4m3.v[lo];
    double dhi = kE4m3.v[hi] - a;
    int c;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo % 2 == 0) ? lo : hi;                    // tie: even code
    return sign | static_cast<uint8_t>(c);
}

}  // namespace

extern "C" {

// ---- codec entry points (used by the pins) --------------------------------

uint16_t orc_bf16_round(float f) { return bf16_round(f); }
float orc_bf16_to_float(uint16_t b) { return bf16_bits_to_float(b); }
uint8_t orc_e4m3_encode(float f) { return e4m3_encode(f); }
double orc_e4m3_decode(uint8_t c) { return e4m3_decode(c); }

void orc_bf16_round_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(in[i]);
}
void orc_e4m3_encode_array(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(in[i]);
}

// ---- layout ---------------------------------------------------------------
//
// Inputs: topk_idx int32 [T, k] row-major; E experts; cap = 0 for the
// contiguous layout, cap > 0 for the fixed-capacity layout [E, cap, H].
// Outputs:
//   count[E]       number of valid routing entries per expert (never clamped)
//   offset[E+1]    exclusive prefix sum of count; offset[E] = valid entries
//   slot_of[T*k]   receive row of entry (t, j), or -1 (invalid id / dropped)
//   src_of_slot[R] entry index t*k+j held by each receive row, or -1
//   status[2]      {entries with id outside [0, E), entries dropped by cap}
// R = T*k (contiguous) or E*cap (fixed capacity).
// Returns 0, or -1 for bad sizes.
int orc_layout(int32_t T, int32_t k, int32_t E, int32_t cap, const int32_t* topk_idx,
               int32_t* count, int32_t* offset, int32_t* slot_of, int32_t* src_of_slot,
               int32_t* status) {
    if (T < 0 || k < 1 || E < 1 || cap < 0) return -1;
    const int64_t n = static_cast<int64_t>(T) * k;
    const int64_t R = cap == 0 ? n : static_cast<int64_t>(E) * cap;

    // Histogram of valid ids.
    int32_t num_invalid = 0;
    for (int32_t e = 0; e < E; ++e) count[e] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = topk_idx[i];
        if (e >= 0 && e < E) ++count[e]; else ++num_invalid;
    }
    // Exclusive prefix sum.
    offset[0] = 0;
    for (int32_t e = 0; e < E; ++e) offset[e + 1] = offset[e] + count[e];

    // Stable slot assignment: walk entries in row-major (t, j) order and give
    // each the next free row of its expert.
    for (int64_t r = 0; r < R; ++r) src_of_slot[r] = -1;
    std::vector<int32_t> cursor(static_cast<size_t>(E), 0);
    int32_t num_dropped = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = topk_idx[i];
        int64_t slot = -1;
        if (e >= 0 && e < E) {
            int32_t r = cursor[e]++;
            if (cap == 0) {
                slot = static_cast<int64_t>(offset[e]) + r;
            } else if (r < cap) {
                slot = static_cast<int64_t>(e) * cap + r;
            } else {
                ++num_dropped;
            }
        }
        slot_of[i] = static_cast<int32_t>(slot);
        if (slot >= 0) src_of_slot[slot] = static_cast<int32_t>(i);
    }
    status[0] = num_invalid;
    status[1] = num_dropped;
    return 0;
}

// ---- dispatch ---------------------------------------------------------------
//
// For tokens t in [t0, t1): for each j with slot = slot_of[t*k+j] >= 0, write
// the token's payload into receive row `slot`.
//   use_fp8 = 0: recv_x is bf16 [R, H]; the row is a bit copy of x[t].
//   use_fp8 = 1: recv_x is E4M3FN bytes [R, H], recv_scales fp32 [R, H/128].
//     For each block b of 128 channels starting at channel 0:
//       amax  = max over the block of |x|            (exact in fp32)
//       scale = amax / 448                           (one IEEE fp32 division)
//       q[c]  = E4M3FN_RNE_saturating(x[c] / scale)  (fp32 division, then encode)
//     amax == 0 gives scale = 0 and every code 0x00 (the quotient is 0/0).
//   use_fp8 = 2: as 1, but each block's scale is a power of two held as one
//     UE8M0 byte (an unsigned 8-bit exponent, value 2^(byte - 127)); the format
//     is named, not defined, in "[PR #206] [MERGED] Support UE8M0 data format".
//     Reading: the scale is the smallest power of two 2^s, s >= -127, with
//     448 * 2^s >= amax, so no quotient exceeds 448 (as with the fp32 scale);
//     recv_scales holds the bytes s + 127, [R, H/128].  The quotient x / 2^s is
//     exact.  amax == 0 gives byte 0 and every code 0x00.
// x is bf16 [T, H].  Receive rows that no entry maps to are not touched.
// Returns 0, or -1 for bad sizes.
int orc_dispatch(int32_t T, int32_t H, int32_t k, int64_t R, int32_t use_fp8, int32_t t0,
                 int32_t t1, const uint16_t* x, const int32_t* slot_of, void* recv_x,
                 void* recv_scales) {
    if (T < 0 || H < 1 || k < 1 || t0 < 0 || t1 > T || t0 > t1) return -1;
    if (use_fp8 < 0 || use_fp8 > 2) return -1;
    if (use_fp8 && H % 128 != 0) return -1;
    const int32_t nblk = H / 128;
    std::vector<uint8_t> q(static_cast<size_t>(H));
    std::vector<float> scales(static_cast<size_t>(use_fp8 ? nblk : 0));
    std::vector<uint8_t> exps(static_cast<size_t>(use_fp8 ? nblk : 0));
    for (int32_t t = t0; t < t1; ++t) {
        const uint16_t* xt = x + static_cast<int64_t>(t) * H;
        if (use_fp8) {
            for (int32_t b = 0; b < nblk; ++b) {
                float amax = 0.0f;
                for (int32_t c = 0; c < 128; ++c) {
                    float v = bf16_bits_to_float(xt[b * 128 + c]);
                    assert(std::isfinite(v));
                    float av = std::fabs(v);
                    if (av > amax) amax = av;
                }
                float scale;
                if (use_fp8 == 1) {
                    scale = amax / 448.0f;
                } else if (amax == 0.0f) {
                    scale = 0.0f;
                    exps[b] = 0;
                } else {
                    int s = -127;  // step up to the first power of two that is large enough
                    while (448.0 * std::ldexp(1.0, s) < static_cast<double>(amax)) ++s;
                    scale = std::ldexp(1.0f, s);
                    exps[b] = static_cast<uint8_t>(s + 127);
                }
                scales[b] = scale;
                for (int32_t c = 0; c < 128; ++c) {
                    float v = bf16_bits_to_float(xt[b * 128 + c]);
                    q[b * 128 + c] = (scale == 0.0f) ? 0x00 : e4m3_encode(v / scale);
                }
            }
        }
        for (int32_t j = 0; j < k; ++j) {
            int32_t slot = slot_of[static_cast<int64_t>(t) * k + j];
            if (slot < 0) continue;
            if (slot >= R) return -1;
            if (use_fp8) {
                uint8_t* dst = static_cast<uint8_t*>(recv_x) + static_cast<int64_t>(slot) * H;
                std::memcpy(dst, q.data(), static_cast<size_t>(H));
                if (use_fp8 == 1)
                    std::memcpy(static_cast<float*>(recv_scales) + static_cast<int64_t>(slot) * nblk,
                                scales.data(), sizeof(float) * static_cast<size_t>(nblk));
                else
                    std::memcpy(static_cast<uint8_t*>(recv_scales) + static_cast<int64_t>(slot) * nblk,
                                exps.data(), static_cast<size_t>(nblk));
            } else {
                uint16_t* dst = static_cast<uint16_t*>(recv_x) + static_cast<int64_t>(slot) * H;
                std::memcpy(dst, xt, sizeof(uint16_t) * static_cast<size_t>(H));
            }
        }
    }
    return 0;
}

// ---- combine ----------------------------------------------------------------
//
// For tokens t in [t0, t1) and every channel c:
//   acc = +0.0f
//   for j = 0 .. k-1 with slot = slot_of[t*k+j] >= 0:
//       acc = fmaf(topk_weights[t*k+j], expert_out[slot][c], acc)
//   y[t][c] = bf16_RNE(acc)
// expert_out is bf16 [R, H]; the fused multiply-add rounds once.  `acc`
// (optional, may be NULL) receives the fp32 sums, [T, H].
// Returns 0, or -1 for bad sizes.
int orc_combine(int32_t T, int32_t H, int32_t k, int64_t R, int32_t t0, int32_t t1,
                const uint16_t* expert_out, const int32_t* slot_of, const float* topk_weights,
                uint16_t* y, float* acc_out) {
    if (T < 0 || H < 1 || k < 1 || t0 < 0 || t1 > T || t0 > t1) return -1;
    for (int32_t t = t0; t < t1; ++t) {
        for (int32_t c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                int64_t e = static_cast<int64_t>(t) * k + j;
                int32_t slot = slot_of[e];
                if (slot < 0) continue;
                if (slot >= R) return -1;
                float v = bf16_bits_to_float(expert_out[static_cast<int64_t>(slot) * H + c]);
                acc = std::fmaf(topk_weights[e], v, acc);
            }
            y[static_cast<int64_t>(t) * H + c] = bf16_round(acc);
            if (acc_out) acc_out[static_cast<int64_t>(t) * H + c] = acc;
        }
    }
    return 0;
}

}  // extern "C"
