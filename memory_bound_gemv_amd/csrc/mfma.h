// Skinny matrix-core tile for the verify window (k = 2 .. 4 activation
// columns): the 163.com Ling-3.0-flash article's optimisation 3 checks a
// 4-token window in one pass, and at batch 1 the routed experts are what
// that pass pays for.  With k columns the plain FMA GEMV (gemv.h) does k
// multiply-adds per weight on the vector ALU, which for MXFP4 rows makes the
// window compute-bound; here a wavefront instead feeds 16 weight rows at a
// time to v_mfma_f32_16x16x32_bf16.
//
//   * A (16 rows x 32 k): weights.  MXFP4 vectors (32 elements, one E8M0
//     scale) are decoded to BF16 with the scaled FP4 conversion, which is
//     exact (an E2M1 value times a power of two has at most 2 significant
//     bits); BF16 rows are used as loaded.
//   * B (32 k x 16 columns): activation column c in B column c as BF16 (hi =
//     nearest BF16 of the binary32 value) and in B column NC + c as the BF16
//     of the remainder (lo = value - hi), so hi + lo carries the binary32
//     activation to ~2^-16 relative; columns 2 NC .. 15 are zero.  The
//     product accumulates in binary32; row r of column c is D[r][c] +
//     D[r][NC + c].
//   * Lane layouts (checked on gfx950): lane l holds A[l % 16][8 (l / 16) +
//     i] and B[8 (l / 16) + i][l % 16], i < 8, and D[4 (l / 16) + i][l % 16],
//     i < 4.
//   * A lane loads one 16-byte vector of its row per unit: vector
//     4 u + l / 16 of row l % 16.  For BF16 that vector is the A operand of
//     one instruction (the k of unit u, in the order above).  For MXFP4 it
//     holds 32 elements, and its dword m is the A operand of instruction
//     (u, m), so the k of one instruction are 128 u + 32 (l / 16) + 8 m + i:
//     a fixed permutation of k, matched by the B layout.
//   * B is prepared once per task in LDS, one 16-byte entry per (instruction,
//     lane), so each instruction reads its B operand with one conflict-free
//     LDS read.
#pragma once

#include <type_traits>

#include "gemv.h"

namespace mbg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4m __attribute__((ext_vector_type(4)));

template <int F>
struct MfmaFmt;
template <>
struct MfmaFmt<F_BF16> { static constexpr int kElemsPerUnit = 32, kInstPerUnit = 1; };
template <>
struct MfmaFmt<F_MXFP4> { static constexpr int kElemsPerUnit = 128, kInstPerUnit = 4; };

// Bytes of LDS the prepared B operands of a row length K take.
template <int K>
constexpr int mfma_b_bytes() { return (K / 32) * kWave * 16; }

// Pack 8 binary32 into BF16 (nearest-even).
__device__ __forceinline__ u32x4 pack_bf16x8(const float (&v)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    return w;
}

// Prepare the B operands of NC activation columns (xs[c * ldx + k], binary32
// in LDS) for rows of length K into bprep (LDS, mfma_b_bytes<K>() bytes).
// All waves of the workgroup share the work; ends with a barrier.
template <int F, int NC, int K>
__device__ __forceinline__ void mfma_prep_b(const lds_f32* xs, int ldx, MBG_LDS u32x4* bprep, int wave, int nwaves,
                                            int lane) {
    static_assert(2 * NC <= 16, "hi and lo columns fit the 16 B columns");
    constexpr int NI = K / 32;   // instructions per 16-row block
    const int n = lane & 15, kq = lane >> 4;
    for (int t = wave; t < NI; t += nwaves) {
        int k0;
        if constexpr (F == F_MXFP4) k0 = 128 * (t >> 2) + 32 * kq + 8 * (t & 3);
        else k0 = 32 * t + 8 * kq;
        float v[8];
        if (n < 2 * NC) {
            const int c = n < NC ? n : n - NC;
            const lds_f32* src = xs + c * ldx + k0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = src[i];
                const float hi = bf16_to_f32(f32_to_bf16(x));
                v[i] = n < NC ? x : x - hi;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        bprep[t * kWave + lane] = pack_bf16x8(v);
    }
    __syncthreads();
}

// One wavefront streams its rows rr = 0 .. nrows-1 (row(rr) gives a GRow; it
// is called with a per-lane rr) in blocks of 16 against the prepared B.  For
// each finished block b, out(b, d) is called by every lane with d = this
// lane's hi + lo sums: lanes with l % 16 < NC hold column l % 16 of rows
// 16 b + 4 (l / 16) + i in d[i] (rows past nrows are to be ignored).
//
// One block of loads (U per lane) is in flight: while unit u of block b is
// consumed, unit u of block b + 1 is requested into the same registers.
// The last block is a separate instance that requests nothing, so in the
// main one every unit has the same number of loads behind it on every path
// and the compiler waits for that unit alone.
template <int F, int NC, int K>
struct MfmaStream {
    static constexpr int EPU = MfmaFmt<F>::kElemsPerUnit;
    static constexpr int IPU = MfmaFmt<F>::kInstPerUnit;
    static constexpr int U = K / EPU;    // 16-byte loads per lane per block
    static_assert(K % EPU == 0, "row length");
    static_assert(U <= 24, "a block's loads stay within the registers and the load counter");

    int nrows, lane;
    __device__ __forceinline__ MfmaStream(int nrows_, int lane_) : nrows(nrows_), lane(lane_) {}

    template <class RowFn, class OutFn>
    __device__ __forceinline__ void run(RowFn& row, const MBG_LDS u32x4* bprep, OutFn& out) const {
        const int nblocks = (nrows + 15) / 16;
        if (nblocks == 0) return;
        const int r16 = lane & 15, kq = lane >> 4;
        uint4 wv[U];
        uint32_t sv[U];
        auto issue = [&](const GRow& g, int u) {
            const int vec = 4 * u + kq;
            wv[u] = ld_stream_g(g.data + vec);
            if constexpr (F == F_MXFP4) sv[u] = g.scale[vec];
        };
        auto block_row = [&](int b) { return row(min(16 * b + r16, nrows - 1)); };
        {
            const GRow g0 = block_row(0);
#pragma unroll
            for (int u = 0; u < U; ++u) issue(g0, u);
        }
        // consume block b; with Refill, request block b + 1 unit by unit
        auto block = [&](int b, auto refill) {
            constexpr bool kRefill = decltype(refill)::value;
            GRow gn{nullptr, nullptr};
            if constexpr (kRefill) gn = block_row(b + 1);
            f32x4m acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (F == F_MXFP4) {
                    const float sc = e8m0_to_f32(sv[u]);
                    const uint32_t ws[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[m], sc, 0);
                        const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[m], sc, 1);
                        const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[m], sc, 2);
                        const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ws[m], sc, 3);
                        bf16x8 av;
                        av[0] = p0[0]; av[1] = p0[1]; av[2] = p1[0]; av[3] = p1[1];
                        av[4] = p2[0]; av[5] = p2[1]; av[6] = p3[0]; av[7] = p3[1];
                        const u32x4 bq = bprep[(IPU * u + m) * kWave + lane];
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bq), acc, 0, 0, 0);
                    }
                } else {
                    const u32x4 bq = bprep[u * kWave + lane];
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[u]),
                                                                    __builtin_bit_cast(bf16x8, bq), acc, 0, 0, 0);
                }
                if constexpr (kRefill) issue(gn, u);
            }
            // hi + lo, read in the basic block of the matrix instructions
            // that wrote the accumulator (a read behind a branch can follow
            // the last one with fewer wait states than it needs: measured
            // as wrong rows 2 and 3 of each group of 4)
            float d[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float part = __int_as_float(
                    __builtin_amdgcn_update_dpp(0, __float_as_int(acc[i]), 0x100 + NC, 0xF, 0xF, false));
                d[i] = acc[i] + part;   // row_shl:NC: the lo column of this lane's column
            }
            out(b, d);
        };
        for (int b = 0;; ++b) {
            if (b + 1 >= nblocks) {
                block(b, std::false_type{});
                break;
            }
            block(b, std::true_type{});
        }
    }
};

}  // namespace mbg
