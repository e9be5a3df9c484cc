// Device helpers for the gfx950 decode kernels: number-format decoding and
// encoding, wavefront reductions, dependency counters and the wait watchdog.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbg {

constexpr int kWave = 64;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: data read once per step).
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ BF16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// binary32 -> BF16, nearest with ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------- FP8 E4M3FN

// Two E4M3FN codes (bytes 0,1 or 2,3 of w) to binary32 with the gfx950
// conversion unit (OCP format on this target).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
    auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    o[0] = a[0];
    o[1] = a[1];
    o[2] = b[0];
    o[3] = b[1];
}

// binary32 -> E4M3FN, nearest with ties to even, saturating at +-448;
// NaN -> 0x7F with the sign.  Integer rounding of the binary32 fields:
// below 2^-6 the value is a multiple of 2^-9 (subnormal grid), above it the
// 23-bit mantissa is rounded to 3 bits with carry into the exponent.
__device__ __forceinline__ uint8_t f32_to_fp8e4m3(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return (uint8_t)(sign | 0x7Fu);
    if (a >= 0x43E00000u) return (uint8_t)(sign | 0x7Eu);         // >= 448 (and inf)
    if (a < 0x3C800000u) {                                          // < 2^-6
        const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling
        return (uint8_t)(sign | (uint32_t)q);                       // 0..8 (8 = 2^-6)
    }
    int e = (int)(a >> 23) - 127;                                   // -6 .. 8
    uint32_t m = (a >> 20) & 7u;
    const uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) { m = 0u; ++e; }
    if (e > 8 || (e == 8 && m > 6u)) { e = 8; m = 6u; }
    return (uint8_t)(sign | ((uint32_t)(e + 7) << 3) | m);
}

// ------------------------------------------------------------------ MXFP4

// E8M0 byte -> binary32 2^(e-127) (e = 0 gives the subnormal 2^-127,
// e = 255 NaN).  Branch-free: the two special codes are the ones for which
// (e + 1) mod 256 <= 1, and both only add bit 22 to e << 23 (0 -> 2^-127,
// 0x7F800000 -> quiet NaN).  A per-lane branch here would put divergent
// control flow into every streaming loop, where it costs the load waits
// their precision.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    const uint32_t special = ((e + 1u) & 0xFFu) <= 1u ? 0x00400000u : 0u;
    return __uint_as_float((e << 23) | special);
}

// Eight E2M1 codes of one 32-bit word (element 2i in the low nibble of byte
// i) times `scale`, with the gfx950 scaled FP4 conversion.
__device__ __forceinline__ void fp4x8_to_f32(uint32_t w, float scale, float* o) {
    auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0);
    auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1);
    auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2);
    auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3);
    o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
    o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
}

// ------------------------------------------------------------ reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum within aligned groups of 4, 8 or 16 lanes; every lane of a group gets
// the same, order-fixed result (each step adds a lane and its partner, and
// a + b == b + a exactly).
__device__ __forceinline__ float group4_sum(float v) {
    v += dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]
    return v;
}
__device__ __forceinline__ float group8_sum(float v) {
    v = group4_sum(v);
    v += dpp_f<0x141>(v);  // row_half_mirror: lane i <-> 7-i
    return v;
}
__device__ __forceinline__ float group16_sum(float v) {
    v = group8_sum(v);
    v += dpp_f<0x140>(v);  // row_mirror: lane i <-> 15-i
    return v;
}
// Values of the two 16-lane rows of each row pair (rows 0/1 and 2/3) and of
// the two 32-lane halves, exchanged by the gfx950 permlane swaps (plain VALU,
// no LDS round trip).  Swapping a register with itself leaves in every lane
// the even row's (lower half's) value in the first result and the odd row's
// (upper half's) in the second.
__device__ __forceinline__ void row_pair(float v, float& even, float& odd) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    even = __uint_as_float(r[0]);
    odd = __uint_as_float(r[1]);
}
__device__ __forceinline__ void wave_halves(float v, float& lo, float& hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}

// Whole-wavefront sum, identical in every lane: rows, then row pairs, then
// halves, in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
    v = group16_sum(v);
    float a, b;
    row_pair(v, a, b);
    v = a + b;
    wave_halves(v, a, b);
    return a + b;
}

// Sum within aligned groups of N lanes (4 .. 64), the same tree as above.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
    if constexpr (N == 4) return group4_sum(v);
    else if constexpr (N == 8) return group8_sum(v);
    else if constexpr (N == 16) return group16_sum(v);
    else if constexpr (N == 32) {
        float a, b;
        row_pair(group16_sum(v), a, b);
        return a + b;
    } else return wave_sum(v);
}

// Whole-wavefront maximum, identical in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    float a, b;
    row_pair(v, a, b);
    v = fmaxf(a, b);
    wave_halves(v, a, b);
    return fmaxf(a, b);
}

// Whole-wavefront maximum of 64-bit unsigned keys, identical in every lane:
// the same DPP and permlane pattern as wave_max on both 32-bit halves (VALU
// lane moves, no LDS round trip per step).
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
    v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
    v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
    {
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        v = max_u64(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
    }
    {
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        v = max_u64(((unsigned long long)hi[0] << 32) | lo[0], ((unsigned long long)hi[1] << 32) | lo[1]);
    }
    return v;
}

// Whole-wavefront maximum of 32-bit unsigned values, identical in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
    v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
    v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
    v = max(v, dpp_u32<0x140>(v));   // row_mirror
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(r[0], r[1]);
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(r[0], r[1]);
}

// The same over 64-bit keys (both halves move through the same lane
// permutation, then one 64-bit compare per step).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) {
    return a > b ? a : b;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<0xB1>(v));
    v = max_u64(v, dpp_u64<0x4E>(v));
    v = max_u64(v, dpp_u64<0x141>(v));
    v = max_u64(v, dpp_u64<0x140>(v));
    uint32_t h = (uint32_t)(v >> 32), l = (uint32_t)v;
    auto rh = __builtin_amdgcn_permlane16_swap(h, h, false, false);
    auto rl = __builtin_amdgcn_permlane16_swap(l, l, false, false);
    v = max_u64(((uint64_t)rh[0] << 32) | rl[0], ((uint64_t)rh[1] << 32) | rl[1]);
    h = (uint32_t)(v >> 32);
    l = (uint32_t)v;
    rh = __builtin_amdgcn_permlane32_swap(h, h, false, false);
    rl = __builtin_amdgcn_permlane32_swap(l, l, false, false);
    return max_u64(((uint64_t)rh[0] << 32) | rl[0], ((uint64_t)rh[1] << 32) | rl[1]);
}

// Inclusive prefix sum within each 16-lane row (Hillis-Steele over row
// shifts; lanes shifted in from outside the row contribute 0).
__device__ __forceinline__ uint32_t row_prefix_sum(uint32_t v) {
    v += dpp_u32<0x111>(v);   // row_shr:1
    v += dpp_u32<0x112>(v);   // row_shr:2
    v += dpp_u32<0x114>(v);   // row_shr:4
    v += dpp_u32<0x118>(v);   // row_shr:8
    return v;
}

// The value of lane (this lane ^ MSK): 8 within a row is a half-row
// rotation (DPP), 16 and 32 are the permlane swaps above.
template <int MSK>
__device__ __forceinline__ float xor_lanes(float v) {
    if constexpr (MSK == 8) {
        return dpp_f<0x128>(v);   // row_ror:8
    } else if constexpr (MSK == 16 || MSK == 32) {
        float a, b;
        if constexpr (MSK == 16) row_pair(v, a, b);
        else wave_halves(v, a, b);
        return (__lane_id() & MSK) ? a : b;
    } else {
        return __shfl_xor(v, MSK, kWave);
    }
}


// s_waitcnt immediates (gfx9 encoding: vmcnt in bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]); unnamed counters are left at their maximum.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int waitcnt_lgkm0() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// ------------------------------------------------- counters and watchdog

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_release(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add_acq_rel(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ void fence_release() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

// Record the first error of a launch (later ones keep the first).
__device__ __forceinline__ void latch_error(uint32_t* status, uint32_t code) {
    uint32_t zero = 0;
    __hip_atomic_compare_exchange_strong(status, &zero, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mbg
