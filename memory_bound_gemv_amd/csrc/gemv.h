// Batch-1 (and k <= 4 column) GEMV core for gfx950.
//
// At batch 1 a decode step is a chain of matrix-vector products whose cost is
// the bytes of weight they stream (Kog article "Real-time LLM inference on
// standard GPUs: 3k tokens/s per request", section on memory bandwidth as the
// bottleneck: about 1 FLOP per byte for FP16, 2 for FP8, 4 for FP4).  So the
// core is built around the load stream, not around matrix units:
//   * a wavefront owns whole rows; a row is NV 16-byte vectors and lane l
//     reads vectors l, l + 64, ... (1 KiB per wave instruction, coalesced);
//     NV is a compile-time constant, so the loads of a row are one scalar
//     base plus immediate offsets;
//   * rows are streamed in chunks of RPC rows; two chunk buffers live in
//     registers and chunk c + 1 is issued before chunk c is multiplied; the
//     first chunk is issued before the workgroup waits for its input vector
//     (weights do not depend on it);
//   * the activation columns sit in LDS as binary32; a lane reads its slice
//     once per chunk and uses it for all RPC rows and, in a verify window,
//     each weight vector for all k columns (each weight byte read once);
//   * products accumulate in binary32 in a fixed order and a row's lane
//     sums are combined by an order-fixed DPP/swizzle tree, so results are
//     bitwise reproducible and independent of scheduling.
#pragma once

#include "device.h"

#define MBG_GLOBAL __attribute__((address_space(1)))
#define MBG_LDS __attribute__((address_space(3)))
#define MBG_CONST __attribute__((address_space(4)))

namespace mbg {

enum : int { F_BF16 = 1, F_FP8 = 2, F_MXFP4 = 3 };

template <int F>
struct FmtInfo;
template <>
struct FmtInfo<F_BF16> { static constexpr int kEPV = 8; };
template <>
struct FmtInfo<F_FP8> { static constexpr int kEPV = 16; };
template <>
struct FmtInfo<F_MXFP4> { static constexpr int kEPV = 32; };


template <class T>
__device__ __forceinline__ MBG_GLOBAL T* gp(T* p) {
    return (MBG_GLOBAL T*)p;
}
template <class T>
__device__ __forceinline__ const MBG_GLOBAL T* gp(const T* p) {
    return (const MBG_GLOBAL T*)p;
}

typedef MBG_LDS float lds_f32;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream_g(const MBG_GLOBAL uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const MBG_GLOBAL u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte load through the cache hierarchy (data written earlier in the step).
__device__ __forceinline__ uint4 ld_g(const MBG_GLOBAL uint4* p) {
    const u32x4 v = *reinterpret_cast<const MBG_GLOBAL u32x4*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes per lane from global memory straight into LDS: lane l's data
// lands at dst + 16 * l (dst is the same for the whole wave).  Written as
// inline assembly so that the compiler does not order it against other LDS
// traffic with whole-counter waits; callers wait for these loads
// explicitly (vmcnt), which stays correct for the compiler's own waits
// because vector memory operations complete in issue order.
__device__ __forceinline__ void lds_dma16(const MBG_GLOBAL void* src, MBG_LDS void* dst) {
    const uint32_t lds = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
                 : "memory");
}

// The same with the device-scope (sc1) cache policy: for data other
// workgroups wrote earlier in the same launch.
__device__ __forceinline__ void lds_dma16_coh(const MBG_GLOBAL void* src, MBG_LDS void* dst) {
    const uint32_t lds = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off sc1"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
                 : "memory");
}

// Address of one weight row (scalar): 16-byte vectors plus, for MXFP4, one
// E8M0 byte per vector.
struct GRow {
    const MBG_GLOBAL uint4* data;
    const MBG_GLOBAL uint8_t* scale;
};

template <int F>
__device__ __forceinline__ void decode16(const uint4 w, uint32_t sbyte, float* wf) {
    if constexpr (F == F_BF16) {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wf[2 * q] = bf16_lo(ws[q]);
            wf[2 * q + 1] = bf16_hi(ws[q]);
        }
    } else if constexpr (F == F_FP8) {
        fp8x4_to_f32(w.x, wf + 0);
        fp8x4_to_f32(w.y, wf + 4);
        fp8x4_to_f32(w.z, wf + 8);
        fp8x4_to_f32(w.w, wf + 12);
    } else {
        const float sc = e8m0_to_f32(sbyte);
        fp4x8_to_f32(w.x, sc, wf + 0);
        fp4x8_to_f32(w.y, sc, wf + 8);
        fp4x8_to_f32(w.z, sc, wf + 16);
        fp4x8_to_f32(w.w, sc, wf + 24);
    }
}

// Rows per chunk: keep the two chunk buffers near 128 VGPRs.
template <int F, int NC, int NV>
struct ChunkRows {
    static constexpr int NJ = (NV + kWave - 1) / kWave;
    static constexpr int budget = (F == F_MXFP4) ? (NC <= 2 ? 8 : 4) : (NC <= 2 ? 16 : 8);
    static constexpr int value = budget / NJ > 0 ? budget / NJ : 1;
};

// Per-row binary32 scales of a wavefront's rows (its row rr is global row
// idx(rr)) held in registers: lane l keeps rows l + 64 i, i < 4, so a row's
// scale is one lane read instead of a memory load in the row epilogue
// (which would wait for every load issued before it); rows from 256 on are
// read from memory.
struct RowScales {
    float v[4];
    const MBG_GLOBAL float* p;

    template <class Idx>
    __device__ __forceinline__ void load(const MBG_GLOBAL float* p_, int nrows, int lane, Idx idx) {
        p = p_;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = lane + kWave * i;
            v[i] = rr < nrows ? p[idx(rr)] : 1.0f;
        }
    }
    // rr is wave-uniform; r is its global row index
    __device__ __forceinline__ float get(int rr, uint32_t r) const {
        if (rr >= 4 * kWave) return p[r];
        const float t = rr < kWave ? v[0] : rr < 2 * kWave ? v[1] : rr < 3 * kWave ? v[2] : v[3];
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), rr & (kWave - 1)));
    }
};

// One wavefront streams `nrows` rows (its own numbering; `row(rr)` gives the
// address) of NV vectors each against NC activation columns in LDS
// (xs[c * ldx + k]).  out(rr, sums) is called by every lane with the
// wave-uniform row results.
template <int F, int NC, int NV, int RPC = ChunkRows<F, NC, NV>::value>
struct RowStream {
    static constexpr int NJ = (NV + kWave - 1) / kWave;
    static constexpr int LASTN = NV - kWave * (NJ - 1);  // lanes active in the last vector column
    static constexpr bool PART = LASTN != kWave;
    static constexpr int E = FmtInfo<F>::kEPV;
    static constexpr int kRowBytes = NV * 16;   // weight bytes per row (scales aside)
    static constexpr int kRpc = RPC;

    struct Buf {
        uint4 w[RPC][NJ];
        uint32_t s[RPC][NJ];
    };

    int nrows, lane;

    __device__ __forceinline__ RowStream(int nrows_, int lane_) : nrows(nrows_), lane(lane_) {}

    __device__ __forceinline__ static bool active(int j, int lane) { return !PART || j < NJ - 1 || lane < LASTN; }

    // Issue rows [r0, r1) of chunk c into b.  Rows past the end are skipped
    // and so are the idle lanes of a partial last column, unless kClamp:
    // then every load is issued, rows past the end repeating the last row
    // and idle lanes the row's last vector (lines the same instruction or
    // chunk already requests), so that the number of loads behind a chunk
    // is the same on every path (what the split loop of run() needs).
    template <bool kClamp, class RowFn>
    __device__ __forceinline__ void issue_rows(Buf& b, int c, RowFn& row, int r0, int r1) const {
#pragma unroll
        for (int r = 0; r < RPC; ++r) {
            const int rr = c * RPC + r;
            if constexpr (kClamp) {
                if (r >= r0 && r < r1) {
                    const GRow g = row(rr < nrows ? rr : nrows - 1);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int v = active(j, lane) ? lane + kWave * j : NV - 1;
                        b.w[r][j] = ld_stream_g(g.data + v);
                        if constexpr (F == F_MXFP4) b.s[r][j] = g.scale[v];
                    }
                }
            } else if (r >= r0 && r < r1 && rr < nrows) {
                const GRow g = row(rr);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (active(j, lane)) {
                        b.w[r][j] = ld_stream_g(g.data + lane + kWave * j);
                        if constexpr (F == F_MXFP4) b.s[r][j] = g.scale[lane + kWave * j];
                    }
                }
            }
        }
    }
    template <class RowFn>
    __device__ __forceinline__ void issue(Buf& b, int c, RowFn& row) const {
        issue_rows<false>(b, c, row, 0, RPC);
    }

    // With kFence the activations, read from LDS in every chunk, are kept
    // from being hoisted out of the chunk loop by a compiler barrier (held
    // in registers across all compute sites of the split loop they can
    // spill).
    template <bool kFence = false, class OutFn>
    __device__ __forceinline__ void compute(const Buf& b, int c, const lds_f32* xs, int ldx, OutFn& out) const {
        if constexpr (kFence) asm volatile("" ::: "memory");
        float acc[RPC][NC][2];
#pragma unroll
        for (int r = 0; r < RPC; ++r)
#pragma unroll
            for (int q = 0; q < NC; ++q) acc[r][q][0] = acc[r][q][1] = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (!active(j, lane)) continue;
            const int k = (lane + kWave * j) * E;
            float xv[NC][E];
#pragma unroll
            for (int q = 0; q < NC; ++q) {
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    const f32x4 t = *reinterpret_cast<const MBG_LDS f32x4*>(xs + q * ldx + k + e);
                    xv[q][e] = t[0];
                    xv[q][e + 1] = t[1];
                    xv[q][e + 2] = t[2];
                    xv[q][e + 3] = t[3];
                }
            }
#pragma unroll
            for (int r = 0; r < RPC; ++r) {
                if (c * RPC + r >= nrows) continue;
                float wf[E];
                decode16<F>(b.w[r][j], b.s[r][j], wf);
#pragma unroll
                for (int q = 0; q < NC; ++q) {
#pragma unroll
                    for (int e = 0; e < E; e += 2) {
                        acc[r][q][0] = fmaf(wf[e], xv[q][e], acc[r][q][0]);
                        acc[r][q][1] = fmaf(wf[e + 1], xv[q][e + 1], acc[r][q][1]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RPC; ++r) {
            const int rr = c * RPC + r;
            if (rr >= nrows) continue;
            float sums[NC];
#pragma unroll
            for (int q = 0; q < NC; ++q) sums[q] = wave_sum(acc[r][q][0] + acc[r][q][1]);
            out(rr, sums);
        }
    }

    __device__ __forceinline__ int chunks() const { return (nrows + RPC - 1) / RPC; }

    // Before the caller's input wait: issue the first `pre` rows (at most
    // two chunks) of the stream into `a` (chunk 0) and `b` (chunk 1).
    // Returns how many were issued; pass it to finish_prefetch.
    template <class RowFn>
    __device__ __forceinline__ int prefetch(Buf& a, Buf& b, RowFn& row, int pre) const {
        pre = pre < 0 ? 0 : pre > 2 * RPC ? 2 * RPC : pre;
        issue_rows<false>(a, 0, row, 0, pre < RPC ? pre : RPC);
        if (pre > RPC) issue_rows<false>(b, 1, row, 0, pre - RPC);
        return pre;
    }

    // After the wait: the rest of the prefetched chunks.  Returns whether
    // chunk 1 is issued (pass it to run()).
    template <class RowFn>
    __device__ __forceinline__ bool finish_prefetch(Buf& a, Buf& b, RowFn& row, int pre) const {
        if (pre < RPC) issue_rows<false>(a, 0, row, pre, RPC);
        if (pre > RPC) {
            issue_rows<false>(b, 1, row, pre - RPC, RPC);
            return true;
        }
        return false;
    }

    // `a` holds chunk 0, already issued; `b` holds chunk 1 when b_issued.
    //
    // kSplit: four compute sites, a chunk with the next one in flight behind
    // it (one site per buffer) and the final chunk (one per buffer).  Where
    // one site serves both "next chunk issued" and "no next chunk" paths
    // (the compact loop), the compiler assumes the smaller number of loads
    // in flight behind it and waits for the next chunk as well, so a chunk's
    // arithmetic does not overlap the following chunk's loads; the split
    // loop (with every load of a chunk issued, see issue_rows) waits for
    // exactly the chunk it computes, at the price of twice the code and of
    // repeated rows in a partial last chunk.  Callers choose: measured in the
    // decode step, the split loop pays off with several activation columns
    // and costs time with one (where a wave's streams are one or two chunks
    // long and the kernel's instruction footprint grows).
    template <bool kSplit, class RowFn, class OutFn>
    __device__ __forceinline__ void run(Buf& a, Buf& b, RowFn& row, const lds_f32* xs, int ldx, OutFn& out,
                                        bool b_issued = false) const {
        const int nch = chunks();
        if constexpr (kSplit) {
            for (int c = 0; c < nch; c += 2) {
                if (c + 1 >= nch) {
                    compute<true>(a, c, xs, ldx, out);
                    break;
                }
                if (!(c == 0 && b_issued)) issue_rows<true>(b, c + 1, row, 0, RPC);
                compute<true>(a, c, xs, ldx, out);
                if (c + 2 >= nch) {
                    compute<true>(b, c + 1, xs, ldx, out);
                    break;
                }
                issue_rows<true>(a, c + 2, row, 0, RPC);
                compute<true>(b, c + 1, xs, ldx, out);
            }
        } else {
            for (int c = 0; c < nch; c += 2) {
                if (c + 1 < nch && !(c == 0 && b_issued)) issue_rows<false>(b, c + 1, row, 0, RPC);
                compute(a, c, xs, ldx, out);
                if (c + 1 >= nch) break;
                if (c + 2 < nch) issue_rows<false>(a, c + 2, row, 0, RPC);
                compute(b, c + 1, xs, ldx, out);
            }
        }
    }
};

// Segmented variant for rows whose 16-byte vectors do not fill whole 64-lane
// columns (2560-wide rows are 80 vectors in MXFP4 and 160 in FP8: with one
// row per wave instruction a quarter or a half of the lanes of the last
// column idle, yet every instruction costs the whole wave).  A wavefront
// works on P = 64 / LPR rows at once, LPR lanes per row; lane t of a row
// reads its vectors t, t + LPR, ... (NVL = NV / LPR of them, LPR * 16
// contiguous bytes per row and instruction), so every lane does useful work
// in every instruction.  Rows are streamed in chunks of RG row groups (RG * P
// rows) with two chunk buffers in registers, as above; a row's lane sums are
// combined within its LPR lanes by the same order-fixed tree.
//
// row(rr) is called with this lane's row (rows past the end are clamped to
// the last one, so every lane loads a valid address); with RSC, GRow::scale
// points at the row's binary32 scale, which is loaded with the row and
// applied to its sums.  out(rr, sums) is called by every lane, rr being the
// lane's own row (possibly >= nrows: the caller masks) and sums its row's
// results, the same in all LPR lanes of the row.
// Lanes per row for a row of NV vectors: the widest group (64 .. 4 lanes)
// that divides it.
template <int NV>
constexpr int seg_lanes() {
    return NV % 64 == 0 ? 64 : NV % 32 == 0 ? 32 : NV % 16 == 0 ? 16 : NV % 8 == 0 ? 8 : 4;
}

template <int F, int NC, int NV, int LPR, int RG, bool RSC = false>
struct SegStream {
    static constexpr int P = kWave / LPR;
    static constexpr int NVL = NV / LPR;
    static constexpr int E = FmtInfo<F>::kEPV;
    static constexpr int kRowsPerChunk = RG * P;
    static_assert(kWave % LPR == 0 && NV % LPR == 0, "lanes per row divide the wave and the row");

    struct Buf {
        uint4 w[RG][NVL];
        uint32_t s[RG][F == F_MXFP4 ? NVL : 1];
        float rs[RG];
    };

    int nrows, t, p;

    __device__ __forceinline__ SegStream(int nrows_, int lane) : nrows(nrows_), t(lane % LPR), p(lane / LPR) {}

    __device__ __forceinline__ int chunks() const { return (nrows + kRowsPerChunk - 1) / kRowsPerChunk; }

    template <class RowFn>
    __device__ __forceinline__ void issue(Buf& b, int c, RowFn& row) const {
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int rr = (c * RG + g) * P + p;
            const GRow gr = row(rr < nrows ? rr : nrows - 1);
#pragma unroll
            for (int j = 0; j < NVL; ++j) {
                b.w[g][j] = ld_stream_g(gr.data + t + LPR * j);
                if constexpr (F == F_MXFP4) b.s[g][j] = gr.scale[t + LPR * j];
            }
            if constexpr (RSC) b.rs[g] = *reinterpret_cast<const MBG_GLOBAL float*>(gr.scale);
        }
    }

    // (kFence: as in RowStream::compute)
    template <bool kFence = false, class OutFn>
    __device__ __forceinline__ void compute(const Buf& b, int c, const lds_f32* xs, int ldx, OutFn& out) const {
        if constexpr (kFence) asm volatile("" ::: "memory");
        float acc[RG][NC][2];
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int q = 0; q < NC; ++q) acc[g][q][0] = acc[g][q][1] = 0.f;
        // activation slices: all NC columns held at once for NC <= 2 (read
        // once per vector for all RG row groups); for wider windows one
        // column at a time, re-read per row group, to bound live registers
        constexpr int XC = NC <= 2 ? NC : 1;
#pragma unroll
        for (int j = 0; j < NVL; ++j) {
            const int k = (t + LPR * j) * E;
            float xv[XC][E];
            auto load_x = [&](int slot, int q) {
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    const f32x4 v = *reinterpret_cast<const MBG_LDS f32x4*>(xs + q * ldx + k + e);
                    xv[slot][e] = v[0];
                    xv[slot][e + 1] = v[1];
                    xv[slot][e + 2] = v[2];
                    xv[slot][e + 3] = v[3];
                }
            };
            if constexpr (XC == NC) {
#pragma unroll
                for (int q = 0; q < NC; ++q) load_x(q, q);
            }
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                float wf[E];
                decode16<F>(b.w[g][j], b.s[g][F == F_MXFP4 ? j : 0], wf);
#pragma unroll
                for (int q = 0; q < NC; ++q) {
                    if constexpr (XC != NC) load_x(0, q);
                    const int xq = XC == NC ? q : 0;
#pragma unroll
                    for (int e = 0; e < E; e += 2) {
                        acc[g][q][0] = fmaf(wf[e], xv[xq][e], acc[g][q][0]);
                        acc[g][q][1] = fmaf(wf[e + 1], xv[xq][e + 1], acc[g][q][1]);
                    }
                }
            }
            // wider windows: keep the scheduler from hoisting later vectors'
            // LDS reads (their registers would spill)
            if constexpr (NC > 1) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            float sums[NC];
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                sums[q] = group_sum<LPR>(acc[g][q][0] + acc[g][q][1]);
                if constexpr (RSC) sums[q] *= b.rs[g];
            }
            out((c * RG + g) * P + p, sums);
        }
    }

    // Before the caller's input wait: issue up to `pre` (0 .. 2) chunks into
    // a (chunk 0) and b (chunk 1).  Returns how many; pass it to run().
    template <class RowFn>
    __device__ __forceinline__ int prefetch(Buf& a, Buf& b, RowFn& row, int pre) const {
        const int n = min(min(pre, 2), chunks());
        if (n > 0) issue(a, 0, row);
        if (n > 1) issue(b, 1, row);
        return n;
    }

    // kSplit: as in RowStream::run.
    template <bool kSplit, class RowFn, class OutFn>
    __device__ __forceinline__ void run(Buf& a, Buf& b, RowFn& row, const lds_f32* xs, int ldx, OutFn& out,
                                        int issued = 0) const {
        const int nch = chunks();
        if (nch == 0) return;
        if (issued < 1) issue(a, 0, row);
        if constexpr (kSplit) {
            for (int c = 0; c < nch; c += 2) {
                if (c + 1 >= nch) {
                    compute<true>(a, c, xs, ldx, out);
                    break;
                }
                if (!(c == 0 && issued >= 2)) issue(b, c + 1, row);
                compute<true>(a, c, xs, ldx, out);
                if (c + 2 >= nch) {
                    compute<true>(b, c + 1, xs, ldx, out);
                    break;
                }
                issue(a, c + 2, row);
                compute<true>(b, c + 1, xs, ldx, out);
            }
        } else {
            for (int c = 0; c < nch; c += 2) {
                if (c + 1 < nch && !(c == 0 && issued >= 2)) issue(b, c + 1, row);
                compute(a, c, xs, ldx, out);
                if (c + 1 >= nch) break;
                if (c + 2 < nch) issue(a, c + 2, row);
                compute(b, c + 1, xs, ldx, out);
            }
        }
    }
};

}  // namespace mbg
