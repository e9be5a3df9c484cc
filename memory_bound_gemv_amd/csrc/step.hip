// The persistent decode-step kernel: one cooperative launch per token (or
// per verify window) runs every operation of every layer.
//
// Why one launch: a launch plus clean-up costs microseconds, so ten kernels
// per layer over 25 layers would spend over a millisecond per token before
// any useful work (Kog article "Real-time LLM inference on standard GPUs:
// 3k tokens/s per request", section on where standard stacks lose
// microseconds); a resident program removes those boundaries (same article,
// monokernel section; "Muse Spark Open: 1,109 tokens/s" article, sections on
// the launch baseline and the kernel boundary).
//
// Structure:
//   * every workgroup walks its own static task list (built at init); a task
//     is one tile of one operation of one layer;
//   * a task first issues the loads that do not depend on the current step
//     (weight rows, KV history), then waits until the dependency counter of
//     the phase it reads has reached epoch * need, then computes, then adds
//     one to its own phase counter with release semantics.  Counters are
//     never reset: the epoch (launch number) makes them monotonic;
//   * attention history (positions < pos) is loaded before the projections
//     of the same layer finish, because it was written by earlier steps (the
//     Muse Spark Open article's boundary section makes the same observation);
//   * every wait has a deadline on the constant-rate clock; a workgroup whose
//     wait expires latches a timeout and leaves, and all others follow, so a
//     launch always drains;
//   * with tracing on, thread 0 of each workgroup stamps every task (start,
//     wait satisfied, end) into a workspace array: an external profiler sees
//     one long kernel, so the kernel times itself (the Muse Spark Open
//     article describes the same self-profiling, section on where the step
//     time goes).  Stamps do not change any result.
#include <hip/hip_runtime.h>

#include "gemv.h"
#include "layout.h"
#include "mfma.h"
#include "ops.h"

namespace mbg {

constexpr int kThreads = 256;
constexpr int kLogThreads = 8;
static_assert(kThreads == 1 << kLogThreads, "threads per workgroup");
constexpr int kWaves = kThreads / kWave;
// Upper bound of Q/K/V rows one wavefront owns in a step (pairs * 2).
constexpr int kQkvRowsPerWave = 64;

typedef const MBG_CONST StepArgs CArgs;
typedef const MBG_CONST LayerPtrs CLayer;

// Compile-time shape of a model family: hidden, FFN width, query width
// (heads * head_dim), head_dim, query heads per KV head, KV format, MoE.
template <int H_, int F_, int QD_, int HD_, int GQ_, int KVF_, int MOE_, int MF_>
struct Shape {
    static constexpr int H = H_, F = F_, QD = QD_, HD = HD_, GQ = GQ_, KVF = KVF_, MOE = MOE_, MF = MF_;
};

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
__device__ __forceinline__ uint32_t ctr_index(uint32_t layer, uint32_t ph) { return layer * PH_COUNT + ph; }

__shared__ uint64_t s_twait;  // trace: when the current task's wait was satisfied

// The step a workgroup is running within a launch of several greedy steps:
// its epoch (the launch epoch plus the step index) and position.
// One step's view of the launch: the argument block (a->field reads it)
// plus the step this pass runs - its counter epoch, its first position and
// its index within the launch.  The ops take it by value, so the three stay
// in scalar registers (read from LDS at every wait they cost ~1 us per
// layer on the dense 2B step).
struct Ctx {
    CArgs* args;
    uint32_t epoch;   // counter epoch of this step (launch epoch + step)
    int32_t pos;      // position of column 0
    int32_t step;     // index of the step within the launch
    __device__ __forceinline__ CArgs* operator->() const { return args; }
};
// Position of column c and the page-table row it uses: consecutive
// positions of sequence 0 (a step or a verify window) or, in a batch of
// independent sequences, the column's own position and row.
__device__ __forceinline__ int col_pos(Ctx a, int c) { return a->batch ? a->bpos[c] : a.pos + c; }
__device__ __forceinline__ const MBG_CONST int32_t* col_ptab(Ctx a, int c) {
    const MBG_CONST int32_t* p = (const MBG_CONST int32_t*)a->page_table;
    return a->batch ? p + (size_t)a->bseq[c] * a->pt_stride : p;
}

__device__ __forceinline__ uint32_t token_ctr_index(Ctx a) { return (uint32_t)a->n_layers * PH_COUNT; }

// Cross-workgroup data (residual stream, q, new K/V, attention partials and
// output, FFN hidden) is written and read with device-coherent accesses
// (agent-scope relaxed atomics: loads and stores with the device-scope cache
// policy), so no L2 write-back or invalidate is needed between phases: a
// producer waits until its stores have completed, then bumps the phase
// counter; a consumer that has seen the counter reads the data coherently.
__device__ __forceinline__ float ldc(const MBG_GLOBAL float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(MBG_GLOBAL float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void stc_small(MBG_GLOBAL T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ldc16(const MBG_GLOBAL uint4* p) {
    const MBG_GLOBAL uint32_t* q = reinterpret_cast<const MBG_GLOBAL uint32_t*>(p);
    return make_uint4(__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                      __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                      __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                      __hip_atomic_load(q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// 16-byte device-coherent accesses: buffer instructions with the sc1 cache
// policy, which is what a relaxed agent-scope atomic access of 4 bytes
// compiles to on gfx950, four times wider.  Offsets are in bytes.
constexpr int kCohAux = 16;   // sc1
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ f32x4 ldc4(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCohAux));
}
__device__ __forceinline__ void stc4(rsrc_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCohAux);
}
// The same within one XCD: stores reach that XCD's L2 (the per-CU cache
// writes through), loads bypass the per-CU cache (sc0) and read the L2.
// Used only between workgroups that run on the same XCD.
__device__ __forceinline__ f32x4 ldx4(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 1));
}
__device__ __forceinline__ void stx4(rsrc_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

// The kCtrLines lines of counter `lines` (128 bytes apart) and the status
// word, in one batch of scalar loads with the cache-bypass bit.  Counters
// and status live in uncached memory, so these loads return the memory-side
// values; on the scalar path they do not queue behind the vector loads this
// CU has in flight, which under a full HBM stream delay a vector poll by
// about a microsecond.
__device__ __forceinline__ void sload_counter(const uint32_t* lines, const uint32_t* status, uint32_t& sum,
                                              uint32_t& st) {
    static_assert(kCtrLines == 8 && kLineU32 == 32, "counter layout");
    // both addresses are wave-uniform: make them scalar operands
    auto uni = [](const uint32_t* p) {
        const uint64_t v = (uint64_t)(uintptr_t)p;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        return ((uint64_t)hi << 32) | lo;
    };
    const uint64_t la = uni(lines), sa = uni(status);
    uint32_t c0, c1, c2, c3, c4, c5, c6, c7, s;
    asm volatile(
        "s_load_dword %0, %9, 0x0 glc\n\t"
        "s_load_dword %1, %9, 0x80 glc\n\t"
        "s_load_dword %2, %9, 0x100 glc\n\t"
        "s_load_dword %3, %9, 0x180 glc\n\t"
        "s_load_dword %4, %9, 0x200 glc\n\t"
        "s_load_dword %5, %9, 0x280 glc\n\t"
        "s_load_dword %6, %9, 0x300 glc\n\t"
        "s_load_dword %7, %9, 0x380 glc\n\t"
        "s_load_dword %8, %10, 0x0 glc\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(c0), "=&s"(c1), "=&s"(c2), "=&s"(c3), "=&s"(c4), "=&s"(c5), "=&s"(c6), "=&s"(c7), "=&s"(s)
        : "s"(la), "s"(sa)
        : "memory");
    sum = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    st = s;
}

// Wait until counter `idx` (the sum of its kCtrLines lines) reaches
// epoch * need (mod 2^32).  Wave 0 polls; the other waves wait at the
// barrier.  Returns false when the launch is aborting.
__device__ __forceinline__ bool wait_until(Ctx a, uint32_t idx, uint32_t target) {
    __shared__ int s_ok;
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        int ok = 1;
        if (idx != kNoWait) {
            const uint32_t* lines = a->ctr + (size_t)idx * kCtrLines * kLineU32;
            const uint64_t t0 = wall_clock64();
            uint32_t rounds = 0;
            while (true) {
                uint32_t sum, st;
                sload_counter(lines, a->status, sum, st);
                if ((int32_t)(sum - target) >= 0) break;
                if (st != 0u) { ok = 0; break; }
                // the clock is a scalar memory read: consult it every 32nd
                // round (every round under a deadline shorter than a millisecond)
                if ((++rounds & a->clock_mask) == 0u && wall_clock64() - t0 > a->deadline_ticks) {
                    if (lane == 0) latch_error(a->status, kStatusTimeout);
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0) {
            s_ok = ok;
            s_twait = wall_clock64();
        }
    }
    __syncthreads();
    return s_ok != 0;
}

__device__ __forceinline__ bool wait_counter(Ctx a, uint32_t idx, uint32_t need) {
    return wait_until(a, idx, a.epoch * need);
}

// Make this workgroup's stores visible at device scope, then count the task
// on this workgroup's line of the counter.
__device__ __forceinline__ void release_counter(Ctx a, uint32_t idx) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // vmcnt(0): this wave's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        MBG_GLOBAL uint32_t* line = gp(a->ctr) + ((size_t)idx * kCtrLines + (blockIdx.x & (kCtrLines - 1))) * kLineU32;
        __hip_atomic_fetch_add(line, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Token id of column c, clamped into [0, vocab); a clamp raises the range
// flag (reported by mbg_get_status) and the step completes normally.
__device__ __forceinline__ int token_of(Ctx a, int c) {
    // the first step reads the caller's token; a later step of the same
    // launch reads the previous step's argmax (written this launch)
    const int st = a.step;
    int t = st == 0 ? gp(a->tokens)[c]
                    : (int)__hip_atomic_load(gp(a->argmax) + (size_t)(st - 1) * a->ncol + c, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    if (t < 0 || t >= a->vocab) {
        if (threadIdx.x == 0) latch_error(a->flags, kStatusRange);
        t = t < 0 ? 0 : a->vocab - 1;
    }
    return t;
}

// xs[c][i] = src(c, i) / sqrt(mean_i src(c, i)^2 + eps) * gain[i], c < NC,
// i < H, where src4(c, j) returns elements 4j .. 4j+3 of column c.  Sums of
// squares in a fixed order (per thread over its quads, then the wave tree,
// then the four waves in order).
template <int NC, int H, class Src4>
__device__ __forceinline__ void load_normed(Ctx a, Src4 src4, const uint16_t* gain, lds_f32* xs) {
    __shared__ float red[kWaves * 4];
    static_assert(H % 4 == 0, "hidden size");
    constexpr int NV = H / 4;
    constexpr int PER = (NV + kThreads - 1) / kThreads;
    const int tid = threadIdx.x;
    const MBG_GLOBAL u32x2* g2 = gp(reinterpret_cast<const u32x2*>(gain));
    f32x4 v[NC][PER];
    float ss[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        ss[c] = 0.f;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int j = tid + kThreads * p;
            if (NV % kThreads == 0 || j < NV) {
                v[c][p] = src4(c, j);
                ss[c] = fmaf(v[c][p][0], v[c][p][0], ss[c]);
                ss[c] = fmaf(v[c][p][1], v[c][p][1], ss[c]);
                ss[c] = fmaf(v[c][p][2], v[c][p][2], ss[c]);
                ss[c] = fmaf(v[c][p][3], v[c][p][3], ss[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float w = wave_sum(ss[c]);
        if ((tid & 63) == 0) red[(tid >> 6) * 4 + c] = w;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float tot = ((red[c] + red[4 + c]) + red[8 + c]) + red[12 + c];
        const float r = 1.0f / sqrtf(tot / (float)H + a->rms_eps);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int j = tid + kThreads * p;
            if (NV % kThreads == 0 || j < NV) {
                const u32x2 gg = g2[j];
                f32x4 o;
                o[0] = v[c][p][0] * r * bf16_lo(gg.x);
                o[1] = v[c][p][1] * r * bf16_hi(gg.x);
                o[2] = v[c][p][2] * r * bf16_lo(gg.y);
                o[3] = v[c][p][3] * r * bf16_hi(gg.y);
                *reinterpret_cast<MBG_LDS f32x4*>(xs + c * H + 4 * j) = o;
            }
        }
    }
    __syncthreads();
}

// xs[0 .. NC*K) = src[...] (float32, written this step): all 16-byte
// coherent loads issued before any LDS write.
template <int NC, int K>
__device__ __forceinline__ void load_plain(const float* src, lds_f32* xs) {
    static_assert(K % 4 == 0, "row length");
    constexpr int NV = NC * K / 4;
    constexpr int PER = (NV + kThreads - 1) / kThreads;
    const rsrc_t r = make_rsrc(src);
    f32x4 v[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int j = threadIdx.x + kThreads * p;
        if (NV % kThreads == 0 || j < NV) v[p] = ldc4(r, 16u * j);
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int j = threadIdx.x + kThreads * p;
        if (NV % kThreads == 0 || j < NV) *reinterpret_cast<MBG_LDS f32x4*>(xs + 4 * j) = v[p];
    }
    __syncthreads();
}

// xs[0 .. n) = src[0 .. n) (float32 written earlier in this launch, n a
// multiple of 256), copied by wave 0 alone with device-coherent LDS DMA:
// wave 0 is the polling wave and has no weight loads in flight, so the copy
// does not queue behind the other waves' prefetch.  Ends with a barrier.
__device__ __forceinline__ void dma_input(Ctx a, const float* src, int n, lds_f32* xs) {
    if (!a->wave0_input) {   // every wave copies its share through registers
        const rsrc_t r = make_rsrc(src);
        for (int j = threadIdx.x; j < n / 4; j += kThreads)
            *reinterpret_cast<MBG_LDS f32x4*>(xs + 4 * j) = ldc4(r, 16u * j);
        __syncthreads();
        return;
    }
    if (wave_id() == 0) {
        const MBG_GLOBAL float* s = gp(src) + lane_id() * 4;
        for (int i = 0; i < n; i += kWave * 4) lds_dma16_coh(s + i, (MBG_LDS void*)(xs + i));
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __syncthreads();
}

// xs[c][i] (already in LDS) *= 1 / sqrt(mean_i xs[c][i]^2 + eps) * gain[i]:
// the same per-thread quads and reduction order as load_normed.
template <int NC, int H>
__device__ __forceinline__ void norm_in_place(Ctx a, const uint16_t* gain, lds_f32* xs) {
    __shared__ float red[kWaves * 4];
    constexpr int NV = H / 4;
    constexpr int PER = (NV + kThreads - 1) / kThreads;
    const int tid = threadIdx.x;
    const MBG_GLOBAL u32x2* g2 = gp(reinterpret_cast<const u32x2*>(gain));
    float ss[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        ss[c] = 0.f;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int j = tid + kThreads * p;
            if (NV % kThreads == 0 || j < NV) {
                const f32x4 v = *reinterpret_cast<const MBG_LDS f32x4*>(xs + c * H + 4 * j);
                ss[c] = fmaf(v[0], v[0], ss[c]);
                ss[c] = fmaf(v[1], v[1], ss[c]);
                ss[c] = fmaf(v[2], v[2], ss[c]);
                ss[c] = fmaf(v[3], v[3], ss[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float w = wave_sum(ss[c]);
        if ((tid & 63) == 0) red[(tid >> 6) * 4 + c] = w;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float tot = ((red[c] + red[4 + c]) + red[8 + c]) + red[12 + c];
        const float r = 1.0f / sqrtf(tot / (float)H + a->rms_eps);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int j = tid + kThreads * p;
            if (NV % kThreads == 0 || j < NV) {
                const u32x2 gg = g2[j];
                MBG_LDS f32x4* q = reinterpret_cast<MBG_LDS f32x4*>(xs + c * H + 4 * j);
                f32x4 o = *q;
                o[0] = o[0] * r * bf16_lo(gg.x);
                o[1] = o[1] * r * bf16_hi(gg.x);
                o[2] = o[2] * r * bf16_lo(gg.y);
                o[3] = o[3] * r * bf16_hi(gg.y);
                *q = o;
            }
        }
    }
    __syncthreads();
}

// Four BF16 values (8 bytes) as float32.
__device__ __forceinline__ f32x4 bf16x4(const MBG_GLOBAL u32x2* p) {
    const u32x2 u = *p;
    f32x4 o;
    o[0] = bf16_lo(u.x);
    o[1] = bf16_hi(u.x);
    o[2] = bf16_lo(u.y);
    o[3] = bf16_hi(u.y);
    return o;
}

// Rows of its stream a wavefront issues before it waits for its input: the
// prefetch budget (KiB per wavefront) rounded up to whole rows.
template <class RS>
__device__ __forceinline__ int gemv_pre_rows(int kib) {
    return (kib * 1024 + RS::kRowBytes - 1) / RS::kRowBytes;
}
template <class RS>
__device__ __forceinline__ int gemv_pre_rows(Ctx a) {
    return gemv_pre_rows<RS>(a->gemv_pre);
}

__shared__ uint64_t s_stamp[4];  // trace: input loaded, stream finished, two op-specific points
__device__ __forceinline__ void stamp(int k) {
    if (threadIdx.x == 0) s_stamp[k] = wall_clock64();
}

// Residual values of a wavefront's first kResRows output rows (lane c < NC
// holds column c), read before the task's wait: the residual a GEMV adds to
// is final once an earlier wait of the same workgroup has been satisfied, so
// the row epilogue does not wait for a load issued behind the stream.
constexpr int kResRows = 2;
struct ResidPre {
    float v[kResRows];
    template <class LoadFn>
    __device__ __forceinline__ void load(int nrows, bool lane_has, LoadFn f) {
#pragma unroll
        for (int i = 0; i < kResRows; ++i) v[i] = (i < nrows && lane_has) ? f(i) : 0.f;
    }
    // rr is wave-uniform; rows from kResRows on come from fallback()
    template <class LoadFn>
    __device__ __forceinline__ float get(int rr, LoadFn fallback) const {
        if (rr >= kResRows) return fallback();
        float r = v[0];
#pragma unroll
        for (int i = 1; i < kResRows; ++i)
            if (rr == i) r = v[i];
        return r;
    }
};

// ------------------------------------------------------------------ QKV

template <int NC, class S>
__device__ __forceinline__ bool op_qkv(Ctx a, uint32_t layer, uint32_t tile, uint32_t wctr, uint32_t wneed,
                                    lds_f32* xs) {
    constexpr int HD = S::HD, HALF = HD / 2, H = S::H;
    const int lane = lane_id();
    const int wave = wave_id();
    CLayer* L = (CLayer*)a->layers + layer;
    const int Hq = a->n_q_heads, Hkv = a->n_kv_heads;
    const int npairs = (Hq + 2 * Hkv) * HALF;
    const int nw = (int)a->tiles_qkv * kWaves;
    const int gw = (int)tile * kWaves + wave;
    const int nunits = gw < npairs ? (npairs - 1 - gw) / nw + 1 : 0;
    const uint16_t* wq = L->wq;
    const uint16_t* wk = L->wk;
    const uint16_t* wv = L->wv;
    auto rowf = [&](int rr) -> GRow {
        const int u = gw + nw * (rr >> 1);
        const int hh = u / HALF;
        const int i = u - hh * HALF + (rr & 1) * HALF;
        const uint16_t* m;
        int r;
        if (hh < Hq) { m = wq; r = hh * HD + i; }
        else if (hh < Hq + Hkv) { m = wk; r = (hh - Hq) * HD + i; }
        else { m = wv; r = (hh - Hq - Hkv) * HD + i; }
        return GRow{gp(reinterpret_cast<const uint4*>(m + (size_t)r * H)), nullptr};
    };
    using RS = RowStream<F_BF16, NC, H / 8>;
    RS st(2 * nunits, lane);
    typename RS::Buf A, B;
    int pre = 0;
    const bool early = wave != 0 || a->poll_wave_prefetch;   // the polling wave may hold its loads back
    if (early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a));
    // RoPE (cos, sin) of this lane's epilogue items (at most two per lane:
    // nunits * NC <= 2 * kWave), loaded before the wait: positions are known
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const MBG_GLOBAL f32x2* rcs = gp(reinterpret_cast<const f32x2*>(a->rope_cs));
    f32x2 cs_pre[2] = {{1.f, 0.f}, {1.f, 0.f}};
    float ksc_pre[2] = {1.f, 1.f};   // FP8 cache: the scale of the item's (layer, head, K/V)
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = lane + kWave * it;
        if (idx < nunits * NC) {
            const int pu = idx / NC, c = idx - pu * NC;
            const int u = gw + nw * pu;
            const int hh = u / HALF;
            if (hh < Hq + Hkv) cs_pre[it] = rcs[(size_t)col_pos(a, c) * HALF + (u - hh * HALF)];
            if (S::KVF == F_FP8 && hh >= Hq) {
                const int kv = hh < Hq + Hkv ? 0 : 1;
                const int gh = kv == 0 ? hh - Hq : hh - Hq - Hkv;
                ksc_pre[it] = gp(a->kv_scales)[((size_t)layer * Hkv + gh) * 2 + kv];
            }
        }
    }
    // the pages of the columns' positions (scalar loads)
    int page_c[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) page_c[c] = col_ptab(a, c)[col_pos(a, c) >> a->page_shift];
    if (!wait_counter(a, wctr, wneed)) return false;
    if (layer == 0) {
        int tok[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) tok[c] = token_of(a, c);
        const MBG_GLOBAL u32x2* emb = gp(reinterpret_cast<const u32x2*>(a->embed));
        load_normed<NC, H>(a, [&](int c, int j) { return bf16x4(emb + (size_t)tok[c] * (H / 4) + j); }, L->attn_norm,
                           xs);
    } else {
        dma_input(a, a->xres, NC * H, xs);
        norm_in_place<NC, H>(a, L->attn_norm, xs);
    }
    if (!early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a));   // after the input loads, not ahead of them
    stamp(0);
    // row sums -> per-wave LDS slots; RoPE and the cache write run after the stream
    lds_f32* res = xs + NC * H + wave * kQkvRowsPerWave * NC;  // [rows][NC]
    auto out = [&](int rr, const float (&s)[NC]) {
        if (lane == 0) {
#pragma unroll
            for (int c = 0; c < NC; ++c) res[rr * NC + c] = s[c];
        }
    };
    // compact loop: a wave has one or two chunks here, and the split loop (gemv.h) spills in the small model
    st.template run<false>(A, B, rowf, xs, H, out, st.finish_prefetch(A, B, rowf, pre));
    stamp(1);
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = lane + kWave * it;
        if (idx >= nunits * NC) break;
        const int pu = idx / NC;
        const int c = idx - pu * NC;
        float x0 = res[(2 * pu) * NC + c];
        float x1 = res[(2 * pu + 1) * NC + c];
        const int u = gw + nw * pu;
        const int hh = u / HALF;
        const int i = u - hh * HALF;
        const int p = col_pos(a, c);
        if (hh < Hq + Hkv) {
            const float cs = cs_pre[it][0], sn = cs_pre[it][1];
            const float y0 = x0 * cs - x1 * sn;
            const float y1 = x0 * sn + x1 * cs;
            x0 = y0;
            x1 = y1;
        }
        if (hh < Hq) {
            MBG_GLOBAL float* q = gp(a->qbuf) + ((size_t)c * Hq + hh) * HD;
            stc(q + i, x0);
            stc(q + i + HALF, x1);
            continue;
        }
        const int kv = hh < Hq + Hkv ? 0 : 1;
        const int gh = kv == 0 ? hh - Hq : hh - Hq - Hkv;
        int page = page_c[0];
#pragma unroll
        for (int cc = 1; cc < NC; ++cc)
            if (c == cc) page = page_c[cc];
        const int slot = p & (a->page_size - 1);
        const size_t off = (size_t)layer * a->kv_layer_stride +
                           ((((size_t)page * 2 + kv) * Hkv + gh) * a->page_size + slot) * HD + i;
        if constexpr (S::KVF == F_BF16) {
            MBG_GLOBAL uint16_t* pool = gp(reinterpret_cast<uint16_t*>(a->kv_pool));
            stc_small<uint16_t>(pool + off, f32_to_bf16(x0));
            stc_small<uint16_t>(pool + off + HALF, f32_to_bf16(x1));
        } else {
            MBG_GLOBAL uint8_t* pool = gp(reinterpret_cast<uint8_t*>(a->kv_pool));
            const float sc = ksc_pre[it];
            stc_small<uint8_t>(pool + off, f32_to_fp8e4m3(x0 / sc));
            stc_small<uint8_t>(pool + off + HALF, f32_to_fp8e4m3(x1 / sc));
        }
    }
    release_counter(a, ctr_index(layer, PH_QKV));
    return true;
}

// ------------------------------------------------------------ attention

// Merge weights of two softmax states (log2 domain).  Callers combine with
// products first and one commutative add, so merge(x, y) == merge(y, x)
// bit for bit.
__device__ __forceinline__ void merge_weights(float m1, float m2, float& mn, float& w1, float& w2) {
    mn = fmaxf(m1, m2);
    if (mn == -INFINITY) {
        w1 = 0.f;
        w2 = 0.f;
        return;
    }
    w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mn);
    w2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
}

// Query heads one attention task handles: at most two, so that the task's
// online-softmax state stays in registers; larger groups are split.
constexpr int attn_heads(int gq) { return gq < kAttnHeadsPerTask ? gq : kAttnHeadsPerTask; }

// Online-softmax state of one lane: GQ query heads, EPC dims of the output.
// Scores are in the log2 domain (q is pre-scaled by log2(e) / sqrt(d)).
template <int GQ, int EPC, int LPT, int KVF>
struct AttnLane {
    float m[GQ], l[GQ], o[GQ][EPC];

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[h][e] = 0.f;
        }
    }

    // Fold NT tokens (this lane's slices of their K and V rows) into the
    // state.  Every lane of the wave must call it (group reductions).
    template <int NT>
    __device__ __forceinline__ void fold(const float (&q)[GQ][EPC], const uint4 (&K)[NT], const uint4 (&V)[NT],
                                         const bool (&valid)[NT], float ksc) {
        float sc[NT][GQ];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float kf[EPC];
            decode16<KVF>(K[j], 0u, kf);
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                float p0 = 0.f, p1 = 0.f;
#pragma unroll
                for (int e = 0; e < EPC; e += 2) {
                    p0 = fmaf(q[h][e], kf[e], p0);
                    p1 = fmaf(q[h][e + 1], kf[e + 1], p1);
                }
                const float sv = group_sum<LPT>(p0 + p1) * ksc;
                sc[j][h] = valid[j] ? sv : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            float cm = -INFINITY;
#pragma unroll
            for (int j = 0; j < NT; ++j) cm = fmaxf(cm, sc[j][h]);
            const float mn = fmaxf(m[h], cm);
            if (mn == -INFINITY) {  // no valid token yet: weights are 0, state unchanged
#pragma unroll
                for (int j = 0; j < NT; ++j) sc[j][h] = 0.f;
                continue;
            }
            const float al = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - mn);
            m[h] = mn;
            l[h] *= al;
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[h][e] *= al;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                sc[j][h] = sc[j][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[j][h] - mn);
                l[h] += sc[j][h];
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float vf[EPC];
            decode16<KVF>(V[j], 0u, vf);
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
#pragma unroll
                for (int e = 0; e < EPC; ++e) o[h][e] = fmaf(sc[j][h], vf[e], o[h][e]);
            }
        }
    }

    // Merge with the state of lane (this lane ^ MSK): the same slice of the
    // heads over other positions.  Both lanes end with the same state.
    template <int MSK>
    __device__ __forceinline__ void merge_partner() {
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float m2 = xor_lanes<MSK>(m[h]);
            const float l2 = xor_lanes<MSK>(l[h]);
            float mn, w1, w2;
            merge_weights(m[h], m2, mn, w1, w2);
            l[h] = l[h] * w1 + l2 * w2;
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const float o2 = xor_lanes<MSK>(o[h][e]);
                o[h][e] = o[h][e] * w1 + o2 * w2;
            }
            m[h] = mn;
        }
    }
};

// Attention LDS use: per wavefront a ring of kAttnBufs buffers of
// kAttnUnits units; a unit is one wave instruction's worth of K rows (1 KiB)
// plus the same for V.  The cross-wave merge area follows the rings.
constexpr int kAttnUnits = 4;
constexpr int kAttnBufs = 4;
constexpr int kUnitBytes = kWave * 16;
constexpr int kAttnWaveBytes = kAttnBufs * kAttnUnits * 2 * kUnitBytes;
constexpr int kAttnRingBytes = kWaves * kAttnWaveBytes;
// A split's partial result row: o[HD], m, l and two pad words (16-byte rows).
constexpr int kPartPad = 4;

// Wait until at most k ring chunks (2 * kAttnUnits loads each) are in flight.
__device__ __forceinline__ void wait_chunks(int k) {
    static_assert(6 * kAttnUnits < 64, "vmcnt range");
    if (k <= 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    else if (k == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kAttnUnits));
    else if (k == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * kAttnUnits));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(6 * kAttnUnits));
}

// One (KV head, head group, split) task: split-KV attention for GH of the
// query heads that share KV head g (head group hg of the GH / GH groups),
// over positions [t0, t1) of the split, for every column of the window.  History (positions < pos) streams straight from HBM into the
// wave's LDS ring (global_load_lds_dwordx4); up to kAttnBufs chunks are
// requested before the task waits for this step's q and new K/V.
template <int NC, class S>
__device__ __forceinline__ bool op_attn(Ctx a, uint32_t layer, uint32_t tile, uint32_t wctr, uint32_t wneed,
                                        lds_f32* smem) {
    constexpr int HD = S::HD, KVF = S::KVF;
    constexpr int GH = attn_heads(S::GQ);    // query heads per task
    constexpr int HG = S::GQ / GH;           // head groups per KV head
    static_assert(S::GQ % GH == 0, "query-head groups");
    constexpr int EB = KVF == F_BF16 ? 2 : 1;
    constexpr int LPT = HD * EB / 16;        // lanes per token row
    constexpr int EPC = 16 / EB;             // elements per lane
    constexpr int TPI = kWave / LPT;         // tokens per wave instruction
    constexpr int NS = kWaves * TPI;         // token slots per workgroup
    constexpr int NUB = kAttnUnits, NB = kAttnBufs;
    constexpr int stride = HD + kPartPad;
    static_assert(LPT == 4 || LPT == 8 || LPT == 16, "row layout");
    static_assert(EPC % 4 == 0, "lane slice");
    using Lane = AttnLane<GH, EPC, LPT, KVF>;
    const int lane = lane_id();
    const int wave = wave_id();
    const int Hq = a->n_q_heads, Hkv = a->n_kv_heads;
    const int S_ = a->attn_splits;
    const int gg = (int)tile / S_;           // (KV head, head group)
    const int s = (int)tile - gg * S_;
    const int g = gg / HG;
    const int qh0 = g * S::GQ + (gg - g * HG) * GH;   // first query head of the task
    const int pos = a.pos, ncol = a->ncol, page_size = a->page_size;
    // One sequence: column c at pos + c shares the history [0, pos) and sees
    // the window's earlier tokens.  A batch: column c at bpos[c] of its own
    // sequence sees [0, bpos[c]] of that sequence only; the splits then
    // cover the widest column and each column streams its own history.
    const bool batch = a->batch != 0;
    int pmin = pos, pmax = pos + ncol - 1;
    if (batch) {
        pmin = pmax = a->bpos[0];
        for (int c = 1; c < ncol; ++c) {
            pmin = min(pmin, (int)a->bpos[c]);
            pmax = max(pmax, (int)a->bpos[c]);
        }
    }
    const int n_tok = pmax + 1;
    // sliding-window layer: a column at p attends [max(0, p - W + 1), p];
    // the splits cover [lo_al, n_tok), lo_al = the lowest column's first
    // position rounded down to a workgroup token slot
    const int W = ((CLayer*)a->layers + layer)->window;
    const int lo_al = W > 0 ? max(0, pmin - W + 1) / NS * NS : 0;
    // split length: a whole number of workgroup token slots, so that every
    // wave instruction's TPI positions start TPI-aligned and sit in one page
    const int T = ((n_tok - lo_al + S_ - 1) / S_ + NS - 1) / NS * NS;
    const int t0 = lo_al + s * T;
    const int t1 = min(t0 + T, n_tok);
    int th = min(t1, batch ? (int)a->bpos[0] : pos);   // history of column 0: [t0, th)
    const int tl = lane / LPT;                      // token of this lane within an instruction
    const int cidx = lane % LPT;                    // 16-byte slice of the row
    int nu = th > t0 ? (th - t0 + NS - 1) / NS : 0;   // units per wave
    int nch = (nu + NUB - 1) / NUB;
    const bool resident = !batch && nch <= NB;      // whole (shared) history stays in LDS
    const size_t layer_off = (size_t)layer * a->kv_layer_stride;
    const MBG_GLOBAL uint8_t* pool = gp(reinterpret_cast<const uint8_t*>(a->kv_pool));
    MBG_LDS uint8_t* ring = reinterpret_cast<MBG_LDS uint8_t*>(smem) + wave * kAttnWaveBytes;

    auto tok_of = [&](int i) { return t0 + (i * kWaves + wave) * TPI + tl; };
    const MBG_CONST int32_t* ptab_s = col_ptab(a, 0);   // the streamed column's page table
    const size_t lane_off = (size_t)tl * HD * EB + (size_t)cidx * 16;
    const int pshift = a->page_shift, pmask = page_size - 1;
    // Request chunk c of history into ring buffer b: NUB units, each one K and
    // one V instruction.  A unit's TPI positions share a page (a page is a
    // power of two >= 16 positions and units start TPI-aligned), so its page
    // is one scalar load (counted apart from the vector loads the waits
    // count).  Units past the history re-read the split's first unit, so
    // every chunk is the same number of loads.
    // (per task: bytes of a physical page over all KV heads, K -> V within
    // a page, and this KV head's rows in page 0 of the layer)
    const size_t page_bytes = (size_t)2 * Hkv * page_size * HD * EB;
    const size_t vstep = (size_t)Hkv * page_size * HD * EB;
    const MBG_GLOBAL uint8_t* head0 = pool + (layer_off + (size_t)g * page_size * HD) * EB + lane_off;
    auto issue_chunk = [&](int c, int b) {
        // the units' pages first (one wait for all their scalar loads)
        int tbs[NUB], pages[NUB];
#pragma unroll
        for (int u = 0; u < NUB; ++u) {
            const int tb = t0 + ((c * NUB + u) * kWaves + wave) * TPI;
            tbs[u] = __builtin_amdgcn_readfirstlane(tb < th ? tb : t0);
            pages[u] = ptab_s[tbs[u] >> pshift];
        }
#pragma unroll
        for (int u = 0; u < NUB; ++u) {
            const int tb = tbs[u];
            const MBG_GLOBAL uint8_t* kp = head0 + (size_t)pages[u] * page_bytes + (size_t)((tb & pmask) * HD * EB);
            MBG_LDS uint8_t* dst = ring + (b * NUB + u) * 2 * kUnitBytes;
            if (!batch && tb + TPI > a.pos - a.step) {   // rows this launch writes (an earlier step's K/V): coherent loads
                lds_dma16_coh(kp, (MBG_LDS void*)dst);
                lds_dma16_coh(kp + vstep, (MBG_LDS void*)(dst + kUnitBytes));
            } else {
                lds_dma16(kp, (MBG_LDS void*)dst);
                lds_dma16(kp + vstep, (MBG_LDS void*)(dst + kUnitBytes));
            }
        }
    };

    int npre = min(nch, NB);
    // the polling wave (0) may hold its loads back until its wait is over
    const int early = (wave != 0 || a->poll_wave_prefetch) ? min(npre, a->attn_pre) : 0;
    for (int c = 0; c < early; ++c) issue_chunk(c, c);
    // known before the wait, read with scalar loads: the pages of the
    // positions this step writes, the FP8 scales
    int page_new[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) page_new[c] = col_ptab(a, c)[col_pos(a, c) >> pshift];
    const MBG_CONST float* kvs = (const MBG_CONST float*)a->kv_scales;
    const float ksc = KVF == F_FP8 ? kvs[((size_t)layer * Hkv + g) * 2 + 0] : 1.f;
    const float vsc = KVF == F_FP8 ? kvs[((size_t)layer * Hkv + g) * 2 + 1] : 1.f;
    if (!wait_counter(a, wctr, wneed)) return false;
    for (int c = early; c < npre; ++c) issue_chunk(c, c);
    // the positions written this step (at most ncol of them, folded by wave 0
    // after the history): requested now, read coherently
    // (one sequence: lane group tl holds position max(t0, pos) + tl; a batch:
    // lane group tl holds column tl's own new position)
    const bool has_new = wave == 0 && (batch || t1 > pos);   // wave-uniform
    const int tn = batch ? (tl < ncol ? (int)a->bpos[tl] : -1) : max(t0, pos) + tl;   // this lane's position
    const bool ld_new = has_new && tl < ncol && tn >= t0 && tn < t1;
    uint4 Kn = make_uint4(0, 0, 0, 0), Vn = make_uint4(0, 0, 0, 0);
    if (ld_new) {
        int page = page_new[0];
#pragma unroll
        for (int c = 1; c < NC; ++c)
            if ((batch ? tl : tn - pos) == c) page = page_new[c];
        const size_t el =
            layer_off + ((((size_t)page * 2) * Hkv + g) * page_size + (tn & pmask)) * HD;
        const MBG_GLOBAL uint8_t* kp = pool + el * EB + (size_t)cidx * 16;
        Kn = ldc16(reinterpret_cast<const MBG_GLOBAL uint4*>(kp));
        Vn = ldc16(reinterpret_cast<const MBG_GLOBAL uint4*>(kp + (size_t)Hkv * page_size * HD * EB));
    }

    const float qscale = a->attn_scale_log2;
    lds_f32* red = reinterpret_cast<lds_f32*>(reinterpret_cast<MBG_LDS uint8_t*>(smem) + kAttnRingBytes);
    const rsrc_t rq = make_rsrc(a->qbuf);
    const rsrc_t rp = make_rsrc(a->part + (size_t)layer * a->part_layer);
    // this group's splits share an XCD (and its L2); compiled for BF16 caches
    const bool local = KVF == F_BF16 && a->attn_local != 0;
    const bool empty = t0 >= t1;
    // One sequence whose split history does not stay in the ring: the
    // window's columns share that history, so it is streamed once and each
    // chunk is folded into every column's state while it sits in the ring
    // (kJoint columns at a time: all of them, except that four columns over
    // the FP8 cache, whose lane slices are twice as wide, go in pairs, as
    // four states would spill).  The window then reads its history once
    // (twice) instead of once per column.  Compiled for the FP8 cache, the
    // long-context format: in the BF16 kernels, whose histories here stay
    // resident, the joint code's mere presence slowed the routed 4-token
    // window by 4 % (measured), so there a window over a long history is
    // still streamed once per column.  Otherwise one column at a time: a
    // batch column streams its own sequence's history, and a resident
    // history is re-read from LDS.
    constexpr int kJoint = (KVF == F_FP8 && NC > 3) ? 2 : NC;
    bool done_joint = false;
    if constexpr (KVF == F_FP8 && NC >= 2) {
        // q of column col (pre-scaled to the log2 domain)
        auto load_q = [&](float (&q)[GH][EPC], int col) {
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                const uint32_t qo = (uint32_t)((((size_t)col * Hq + qh0 + h) * HD + cidx * EPC) * 4);
#pragma unroll
                for (int e = 0; e < EPC; e += 4) {
                    const f32x4 t = ldc4(rq, qo + 4u * e);
#pragma unroll
                    for (int k = 0; k < 4; ++k) q[h][e + k] = t[k] * qscale;
                }
            }
        };
        // stream the split's history chunks (the first npre already requested)
        // through the ring; fold(K, V, tk) sees each unit's rows and positions
        auto stream = [&](auto fold) {
            for (int c = 0; c < nch; ++c) {
                const int b = c & (NB - 1);
                wait_chunks(min(nch - 1 - c, NB - 1));        // chunk c has landed
                uint4 K[NUB], V[NUB];
                int tk[NUB];
#pragma unroll
                for (int u = 0; u < NUB; ++u) {
                    const MBG_LDS uint8_t* src = ring + (b * NUB + u) * 2 * kUnitBytes + lane * 16;
                    const u32x4 kv4 = *reinterpret_cast<const MBG_LDS u32x4*>(src);
                    const u32x4 vv4 = *reinterpret_cast<const MBG_LDS u32x4*>(src + kUnitBytes);
                    K[u] = make_uint4(kv4.x, kv4.y, kv4.z, kv4.w);
                    V[u] = make_uint4(vv4.x, vv4.y, vv4.z, vv4.w);
                    tk[u] = tok_of(c * NUB + u);
                }
                fold(K, V, tk);
                if (c + NB < nch) {
                    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());  // this buffer's reads are done
                    issue_chunk(c + NB, b);
                }
            }
        };
        // column col after its history: the positions written this step up to
        // its own, the V scale, the merge of the lanes and waves, the split's
        // partial row
        auto finish_column = [&](Lane& st, const float (&q)[GH][EPC], int col, int tlo) {
            const int pc = batch ? (int)a->bpos[col] : pos + col;   // this column's position
            const int te = min(t1, pc + 1);
            if (has_new) {
                const uint4 K[1] = {Kn}, V[1] = {Vn};
                const bool valid[1] = {batch ? ld_new && tl == col : tl < ncol && tn < te && tn >= tlo};
                st.template fold<1>(q, K, V, valid, ksc);
            }
            if constexpr (KVF == F_FP8) {
#pragma unroll
                for (int h = 0; h < GH; ++h)
#pragma unroll
                    for (int e = 0; e < EPC; ++e) st.o[h][e] *= vsc;
            }
            // merge the token slots of a wave (lanes with the same cidx)
            if constexpr (LPT <= 4) st.template merge_partner<4>();
            if constexpr (LPT <= 8) st.template merge_partner<8>();
            if constexpr (LPT <= 16) st.template merge_partner<16>();
            st.template merge_partner<32>();
            // then the waves, through LDS, in wave order
            if (lane < LPT) {
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    lds_f32* r = red + ((size_t)wave * GH + h) * stride;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) r[cidx * EPC + e] = st.o[h][e];
                    if (cidx == 0) {
                        r[HD] = st.m[h];
                        r[HD + 1] = st.l[h];
                    }
                }
            }
            __syncthreads();
            if (wave == 0 && lane < LPT) {
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    float M = red[h * stride + HD], Ls = red[h * stride + HD + 1];
                    float O[EPC];
#pragma unroll
                    for (int e = 0; e < EPC; ++e) O[e] = red[h * stride + cidx * EPC + e];
                    for (int w = 1; w < kWaves; ++w) {
                        const lds_f32* r = red + ((size_t)w * GH + h) * stride;
                        float mn, w1, w2;
                        merge_weights(M, r[HD], mn, w1, w2);
                        Ls = Ls * w1 + r[HD + 1] * w2;
#pragma unroll
                        for (int e = 0; e < EPC; ++e) O[e] = O[e] * w1 + r[cidx * EPC + e] * w2;
                        M = mn;
                    }
                    const uint32_t row = (uint32_t)((((size_t)col * Hq + qh0 + h) * S_ + s) * stride * 4);
#pragma unroll
                    for (int e = 0; e < EPC; e += 4) {
                        f32x4 t;
                        t[0] = O[e];
                        t[1] = O[e + 1];
                        t[2] = O[e + 2];
                        t[3] = O[e + 3];
                        if (local) stx4(rp, row + 4u * (cidx * EPC + e), t);
                        else stc4(rp, row + 4u * (cidx * EPC + e), t);
                    }
                    if (cidx == 0) {
                        f32x4 t;
                        t[0] = M;
                        t[1] = Ls;
                        t[2] = 0.f;
                        t[3] = 0.f;
                        if (local) stx4(rp, row + 4u * HD, t);
                        else stc4(rp, row + 4u * HD, t);
                    }
                }
            }
            __syncthreads();
        };
        if (!batch && !resident && !empty) {
            done_joint = true;
            for (int cg = 0; cg < ncol; cg += kJoint) {
                const int ce = min(ncol, cg + kJoint);
                float q[kJoint][GH][EPC];
                int tlo[kJoint];   // each column's first position (may be < 0)
                Lane st[kJoint];
#pragma unroll
                for (int i = 0; i < kJoint; ++i) {
                    if (cg + i >= ce) continue;
                    load_q(q[i], cg + i);
                    tlo[i] = W > 0 ? pos + cg + i - W + 1 : 0;
                    st[i].init();
                }
                if (cg == 0) stamp(0);
                if (cg > 0) {  // the next group streams the history again
                    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());  // earlier ring reads are done
                    for (int c = 0; c < npre; ++c) issue_chunk(c, c);
                }
                stream([&](const uint4 (&K)[NUB], const uint4 (&V)[NUB], const int (&tk)[NUB]) {
#pragma unroll
                    for (int i = 0; i < kJoint; ++i) {
                        if (cg + i >= ce) continue;
                        bool valid[NUB];
#pragma unroll
                        for (int u = 0; u < NUB; ++u) valid[u] = tk[u] < th && tk[u] >= tlo[i];
                        st[i].template fold<NUB>(q[i], K, V, valid, ksc);
                    }
                });
                if (cg == 0) stamp(2);
#pragma unroll
                for (int i = 0; i < kJoint; ++i)
                    if (cg + i < ce) finish_column(st[i], q[i], cg + i, tlo[i]);
            }
        }
    }
    if (!done_joint) {
        for (int col = 0; col < ncol && !empty; ++col) {
            const int pc = batch ? (int)a->bpos[col] : pos + col;   // this column's position
            const int te = min(t1, pc + 1);
            const int tlo = W > 0 ? pc - W + 1 : 0;   // this column's first position (may be < 0)
            float q[GH][EPC];
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                const uint32_t qo = (uint32_t)((((size_t)col * Hq + qh0 + h) * HD + cidx * EPC) * 4);
#pragma unroll
                for (int e = 0; e < EPC; e += 4) {
                    const f32x4 t = ldc4(rq, qo + 4u * e);
#pragma unroll
                    for (int k = 0; k < 4; ++k) q[h][e + k] = t[k] * qscale;
                }
            }
            if (col == 0) stamp(0);
            Lane st;
            st.init();
            if (col > 0 && !resident) {  // stream the history again for this column
                if (batch) {   // its own sequence's history and pages
                    th = min(t1, pc);
                    ptab_s = col_ptab(a, col);
                    nu = th > t0 ? (th - t0 + NS - 1) / NS : 0;
                    nch = (nu + NUB - 1) / NUB;
                    npre = min(nch, NB);
                }
                __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());  // earlier ring reads are done
                for (int c = 0; c < npre; ++c) issue_chunk(c, c);
            }
            for (int c = 0; c < nch; ++c) {
                const int b = c & (NB - 1);
                wait_chunks(min(nch - 1 - c, NB - 1));        // chunk c has landed
                uint4 K[NUB], V[NUB];
                bool valid[NUB];
#pragma unroll
                for (int u = 0; u < NUB; ++u) {
                    const MBG_LDS uint8_t* src = ring + (b * NUB + u) * 2 * kUnitBytes + lane * 16;
                    const u32x4 kv4 = *reinterpret_cast<const MBG_LDS u32x4*>(src);
                    const u32x4 vv4 = *reinterpret_cast<const MBG_LDS u32x4*>(src + kUnitBytes);
                    K[u] = make_uint4(kv4.x, kv4.y, kv4.z, kv4.w);
                    V[u] = make_uint4(vv4.x, vv4.y, vv4.z, vv4.w);
                    const int tk = tok_of(c * NUB + u);
                    valid[u] = tk < th && tk >= tlo;
                }
                st.template fold<NUB>(q, K, V, valid, ksc);
                if (c + NB < nch) {
                    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());  // this buffer's reads are done
                    issue_chunk(c + NB, b);
                }
            }
            if (col == 0) stamp(2);
            // positions written this step, up to this column's own
            if (has_new) {
                const uint4 K[1] = {Kn}, V[1] = {Vn};
                const bool valid[1] = {batch ? ld_new && tl == col : tl < ncol && tn < te && tn >= tlo};
                st.template fold<1>(q, K, V, valid, ksc);
            }
            if constexpr (KVF == F_FP8) {
#pragma unroll
                for (int h = 0; h < GH; ++h)
#pragma unroll
                    for (int e = 0; e < EPC; ++e) st.o[h][e] *= vsc;
            }
            // merge the token slots of a wave (lanes with the same cidx)
            if constexpr (LPT <= 4) st.template merge_partner<4>();
            if constexpr (LPT <= 8) st.template merge_partner<8>();
            if constexpr (LPT <= 16) st.template merge_partner<16>();
            st.template merge_partner<32>();
            // then the waves, through LDS, in wave order
            if (lane < LPT) {
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    lds_f32* r = red + ((size_t)wave * GH + h) * stride;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) r[cidx * EPC + e] = st.o[h][e];
                    if (cidx == 0) {
                        r[HD] = st.m[h];
                        r[HD + 1] = st.l[h];
                    }
                }
            }
            __syncthreads();
            if (wave == 0 && lane < LPT) {
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    float M = red[h * stride + HD], Ls = red[h * stride + HD + 1];
                    float O[EPC];
#pragma unroll
                    for (int e = 0; e < EPC; ++e) O[e] = red[h * stride + cidx * EPC + e];
                    for (int w = 1; w < kWaves; ++w) {
                        const lds_f32* r = red + ((size_t)w * GH + h) * stride;
                        float mn, w1, w2;
                        merge_weights(M, r[HD], mn, w1, w2);
                        Ls = Ls * w1 + r[HD + 1] * w2;
#pragma unroll
                        for (int e = 0; e < EPC; ++e) O[e] = O[e] * w1 + r[cidx * EPC + e] * w2;
                        M = mn;
                    }
                    const uint32_t row = (uint32_t)((((size_t)col * Hq + qh0 + h) * S_ + s) * stride * 4);
#pragma unroll
                    for (int e = 0; e < EPC; e += 4) {
                        f32x4 t;
                        t[0] = O[e];
                        t[1] = O[e + 1];
                        t[2] = O[e + 2];
                        t[3] = O[e + 3];
                        if (local) stx4(rp, row + 4u * (cidx * EPC + e), t);
                        else stc4(rp, row + 4u * (cidx * EPC + e), t);
                    }
                    if (cidx == 0) {
                        f32x4 t;
                        t[0] = M;
                        t[1] = Ls;
                        t[2] = 0.f;
                        t[3] = 0.f;
                        if (local) stx4(rp, row + 4u * HD, t);
                        else stc4(rp, row + 4u * HD, t);
                    }
                }
            }
            __syncthreads();
        }
    }
    stamp(1);
    // arrival; the last split of this KV head combines all of them
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (threadIdx.x == 0) {
        // within the XCD: an L2 atomic; otherwise a device-scope one
        uint32_t old;
        if (local)
            old = (uint32_t)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(
                1, make_rsrc(a->head_ctr), (int)(((size_t)layer * Hkv * HG + gg) * kLineU32 * 4), 0, 0);
        else
            old = __hip_atomic_fetch_add(gp(a->head_ctr) + ((size_t)layer * Hkv * HG + gg) * kLineU32, 1u,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old + 1u == a.epoch * (uint32_t)S_);
    }
    __syncthreads();
    if (!s_last) return true;
    // Combine: softmax over the column's positions = weights exp2(m_s - M) on the
    // split partials, normalised by their weighted sum.
    const int nsv = min(S_, (n_tok - lo_al + T - 1) / T);   // splits that wrote partials
    const int nch_ = ncol * GH;                      // (column, head) rows
    constexpr int HDV = HD / 4;                      // 16-byte vectors of o
    constexpr int RV = HDV + 1;                      // vectors of a partial row: o, then (m, l, pad)
    // stage 1: in one batch of loads, the whole partial rows of the group when
    // they fit in the (now idle) ring area, else their (m, l) only
    const bool whole = (size_t)nch_ * nsv * RV * 16 + (size_t)nch_ * 65 * 4 <= (size_t)kAttnRingBytes;
    const int vpr = whole ? RV : 1;                  // vectors held per (row, split)
    lds_f32* prt = smem;                             // [nch_][nsv][vpr] vectors
    lds_f32* wts = prt + (size_t)nch_ * nsv * vpr * 4;   // [nch_][64]: weights
    lds_f32* tot = wts + nch_ * 64;                  // [nch_]: weighted sum of l
    lds_f32* accl = smem + kAttnRingBytes / 4;       // [kThreads][4]: group partial sums (merge area)
    const int nload = nch_ * nsv * vpr;
    // rs / nsv as a multiply-high by ceil(2^32 / nsv) (rs itself for one
    // split, where that would not fit 32 bits): exact here (rs < 2^16,
    // nsv <= 64), where a division by a runtime value would cost ~25
    // instructions per load on the combine's critical path
    const uint32_t nsv_inv = nsv > 1 ? 0xFFFFFFFFu / (uint32_t)nsv + 1u : 0u;
    auto stage1 = [&](auto vprc) {
        constexpr int VPR = decltype(vprc)::value;   // the vectors per (row, split): RV or 1
        for (int i0 = 0; i0 < nload; i0 += 8 * kThreads) {
            f32x4 t[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int idx = min(i0 + k * kThreads + (int)threadIdx.x, nload - 1);
                const int rs = idx / VPR, v = idx - rs * VPR;
                const int ch = nsv > 1 ? (int)__umulhi((uint32_t)rs, nsv_inv) : rs, sp = rs - ch * nsv;
                const int col = ch / GH, h = ch - col * GH;
                const int vec = VPR == RV ? v : HDV;
                const uint32_t po = (uint32_t)(((((size_t)col * Hq + qh0 + h) * S_ + sp) * stride + vec * 4) * 4);
                t[k] = local ? ldx4(rp, po) : ldc4(rp, po);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int idx = i0 + k * kThreads + (int)threadIdx.x;
                if (idx < nload) *reinterpret_cast<MBG_LDS f32x4*>(prt + 4 * idx) = t[k];
            }
        }
    };
    if (whole) stage1(std::integral_constant<int, RV>{});
    else stage1(std::integral_constant<int, 1>{});
    __syncthreads();
    // stage 2: one wavefront per row, one lane per split: the maximum, the
    // weights and their l-weighted sum are wavefront reductions
    for (int ch = wave; ch < nch_; ch += kWaves) {
        const bool act = lane < nsv;
        const lds_f32* ml = prt + ((size_t)(ch * nsv + (act ? lane : 0)) * vpr + (whole ? HDV : 0)) * 4;
        const float m = act ? ml[0] : -INFINITY;
        const float M = wave_max(m);
        const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
        const float ls = wave_sum(act ? w * ml[1] : 0.f);
        if (act) wts[ch * 64 + lane] = w;
        if (lane == 0) tot[ch] = ls;
    }
    __syncthreads();
    stamp(3);
    // stage 3: weighted sum of the partial o rows (from LDS, or loaded now).
    // A thread owns one 16-byte slice of a row and every ng-th split; ng
    // thread groups then add up in group order.
    const int pairs = nch_ * HDV;
    // ng = 8, 4, 2 or 1 groups of tpg = kThreads / ng threads: as many as
    // leave every pair a thread (shifts, not runtime divisions)
    const int lng = pairs <= kThreads / 8 ? 3 : pairs <= kThreads / 4 ? 2 : pairs <= kThreads / 2 ? 1 : 0;
    const int ng = 1 << lng;
    const int tpg = kThreads >> lng;
    const int grp = (int)threadIdx.x >> (kLogThreads - lng), pl = (int)threadIdx.x & (tpg - 1);
    const rsrc_t ra = make_rsrc(a->attn);
    for (int base = 0; base < pairs; base += tpg) {
        const int pr = base + pl;
        const int prc = min(pr, pairs - 1);
        const int ch = prc / HDV, vec = prc - ch * HDV;
        const int col = ch / GH, h = ch - col * GH;
        const size_t row0 = ((size_t)col * Hq + qh0 + h) * S_;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int i0 = grp; i0 < nsv; i0 += 8 * ng) {
            f32x4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int sp = min(i0 + k * ng, nsv - 1);
                v[k] = whole ? *reinterpret_cast<const MBG_LDS f32x4*>(prt + ((size_t)(ch * nsv + sp) * RV + vec) * 4)
                             : local ? ldx4(rp, (uint32_t)(((row0 + sp) * stride + vec * 4) * 4))
                                     : ldc4(rp, (uint32_t)(((row0 + sp) * stride + vec * 4) * 4));
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int sp = i0 + k * ng;
                if (sp < nsv) {
                    const float w = wts[ch * 64 + sp];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, v[k][e], acc[e]);
                }
            }
        }
        *reinterpret_cast<MBG_LDS f32x4*>(accl + 4 * threadIdx.x) = acc;
        __syncthreads();
        if (grp == 0 && pr < pairs) {
            f32x4 sum = *reinterpret_cast<const MBG_LDS f32x4*>(accl + 4 * pl);
            for (int q = 1; q < ng; ++q) {
                const f32x4 o = *reinterpret_cast<const MBG_LDS f32x4*>(accl + 4 * (q * tpg + pl));
#pragma unroll
                for (int e = 0; e < 4; ++e) sum[e] += o[e];
            }
            const float tt = tot[ch];
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[e] = sum[e] / tt;
            stc4(ra, (uint32_t)((((size_t)col * Hq + qh0 + h) * HD + vec * 4) * 4), sum);
        }
        __syncthreads();
    }
    release_counter(a, ctr_index(layer, PH_ATTN));
    return true;
}

// --------------------------------------------------- plain row GEMVs

template <int NC, class S>
__device__ __forceinline__ bool op_oproj(Ctx a, uint32_t layer, uint32_t tile, uint32_t wctr, uint32_t wneed,
                                      lds_f32* xs) {
    constexpr int H = S::H, K = S::QD;
    const int lane = lane_id(), wave = wave_id();
    CLayer* L = (CLayer*)a->layers + layer;
    const int nw = (int)a->tiles_o * kWaves, gw = (int)tile * kWaves + wave;
    const int nrows = gw < H ? (H - 1 - gw) / nw + 1 : 0;
    const uint16_t* wo = L->wo;
    auto rowf = [&](int rr) -> GRow {
        return GRow{gp(reinterpret_cast<const uint4*>(wo + (size_t)(gw + nw * rr) * K)), nullptr};
    };
    using RS = RowStream<F_BF16, NC, K / 8>;
    RS st(nrows, lane);
    typename RS::Buf A, B;
    int pre = 0;
    const bool early = wave != 0 || a->poll_wave_prefetch;   // the polling wave may hold its loads back
    if (early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a));
    // the residual: the embedding rows at layer 0, else the stream as the
    // previous layer left it (final since this workgroup's QKV wait)
    int tok[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) tok[c] = layer == 0 ? token_of(a, c) : 0;
    int tk_lane = 0;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
        if (cc == lane) tk_lane = tok[cc];
    MBG_GLOBAL float* x = gp(a->xres);
    const MBG_GLOBAL uint16_t* emb = gp(a->embed);
    auto resid = [&](int rr) -> float {
        const int r = gw + nw * rr;
        return layer == 0 ? bf16_to_f32(emb[(size_t)tk_lane * H + r]) : ldc(x + lane * H + r);
    };
    ResidPre rp;
    rp.load(nrows, lane < NC, resid);
    if (!wait_counter(a, wctr, wneed)) return false;
    dma_input(a, a->attn, NC * K, xs);
    if (!early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a));   // after the input loads, not ahead of them
    stamp(0);
    auto out = [&](int rr, const float (&s)[NC]) {
        if (lane >= NC) return;
        const int c = lane;
        float v = 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
            if (cc == c) v = s[cc];
        const int r = gw + nw * rr;
        stc(x + c * H + r, rp.get(rr, [&] { return resid(rr); }) + v);
    };
    // compact loop: one or two chunks per wave; the split loop spills in the small model
    st.template run<false>(A, B, rowf, xs, K, out, st.finish_prefetch(A, B, rowf, pre));
    stamp(1);
    release_counter(a, ctr_index(layer, PH_OPROJ));
    return true;
}

template <int NC, class S>
__device__ __forceinline__ bool op_gateup(Ctx a, uint32_t layer, uint32_t tile, uint32_t wctr, uint32_t wneed,
                                       lds_f32* xs) {
    constexpr int H = S::H, F = S::F;
    const int lane = lane_id(), wave = wave_id();
    CLayer* L = (CLayer*)a->layers + layer;
    const int nw = (int)a->tiles_gu * kWaves, gw = (int)tile * kWaves + wave;
    const int nunits = gw < F ? (F - 1 - gw) / nw + 1 : 0;
    const uint16_t* wg = L->w_gate;
    const uint16_t* wu = L->w_up;
    auto rowf = [&](int rr) -> GRow {
        const int f = gw + nw * (rr >> 1);
        const uint16_t* m = (rr & 1) ? wu : wg;
        return GRow{gp(reinterpret_cast<const uint4*>(m + (size_t)f * H)), nullptr};
    };
    using RS = RowStream<F_BF16, NC, H / 8>;
    RS st(2 * nunits, lane);
    typename RS::Buf A, B;
    int pre = 0;
    const bool early = wave != 0 || a->poll_wave_prefetch;   // the polling wave may hold its loads back
    if (early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a->gu_pre));
    if (!wait_counter(a, wctr, wneed)) return false;
    dma_input(a, a->xres, NC * H, xs);
    norm_in_place<NC, H>(a, L->ffn_norm, xs);
    if (!early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a->gu_pre));   // after the input loads, not ahead of them
    stamp(0);
    MBG_GLOBAL float* hb = gp(a->hbuf);
    float gate[NC];
    auto out = [&](int rr, const float (&s)[NC]) {
        if ((rr & 1) == 0) {
#pragma unroll
            for (int c = 0; c < NC; ++c) gate[c] = s[c];
            return;
        }
        if (lane >= NC) return;
        const int c = lane;
        float gv = 0.f, uv = 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
            if (cc == c) { gv = gate[cc]; uv = s[cc]; }
        const int f = gw + nw * (rr >> 1);
        stc(hb + (size_t)c * F + f, gv / (1.0f + expf(-gv)) * uv);
    };
    // split loop for several columns (each chunk computed while the next is
    // in flight); for one column the compact loop measured faster in the step
    st.template run<(NC >= 2)>(A, B, rowf, xs, H, out, st.finish_prefetch(A, B, rowf, pre));
    stamp(1);
    release_counter(a, ctr_index(layer, PH_GATEUP));
    return true;
}

template <int NC, class S>
__device__ __forceinline__ bool op_down(Ctx a, uint32_t layer, uint32_t tile, uint32_t wctr, uint32_t wneed,
                                     lds_f32* xs) {
    constexpr int H = S::H, F = S::F;
    const int lane = lane_id(), wave = wave_id();
    CLayer* L = (CLayer*)a->layers + layer;
    const int nw = (int)a->tiles_down * kWaves, gw = (int)tile * kWaves + wave;
    const int nrows = gw < H ? (H - 1 - gw) / nw + 1 : 0;
    const uint16_t* wd = L->w_down;
    auto rowf = [&](int rr) -> GRow {
        return GRow{gp(reinterpret_cast<const uint4*>(wd + (size_t)(gw + nw * rr) * F)), nullptr};
    };
    using RS = RowStream<F_BF16, NC, F / 8>;
    RS st(nrows, lane);
    typename RS::Buf A, B;
    int pre = 0;
    const bool early = wave != 0 || a->poll_wave_prefetch;   // the polling wave may hold its loads back
    if (early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a->down_pre));
    // the residual after this layer's output projection (final since this
    // workgroup's gate/up wait)
    MBG_GLOBAL float* x = gp(a->xres);
    auto resid = [&](int rr) -> float { return ldc(x + lane * H + gw + nw * rr); };
    ResidPre rp;
    rp.load(nrows, lane < NC, resid);
    if (!wait_counter(a, wctr, wneed)) return false;
    dma_input(a, a->hbuf, NC * F, xs);
    if (!early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a->down_pre));   // after the input loads, not ahead of them
    stamp(0);
    auto out = [&](int rr, const float (&s)[NC]) {
        if (lane >= NC) return;
        const int c = lane;
        float v = 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
            if (cc == c) v = s[cc];
        const int r = gw + nw * rr;
        stc(x + c * H + r, rp.get(rr, [&] { return resid(rr); }) + v);
    };
    // split loop for several columns, compact for one (as in op_gateup)
    st.template run<(NC >= 2)>(A, B, rowf, xs, F, out, st.finish_prefetch(A, B, rowf, pre));
    stamp(1);
    release_counter(a, ctr_index(layer, PH_DOWN));
    return true;
}

// ------------------------------------------------------------------- MoE
//
// A routed layer (163.com Ling-3.0-flash article, model and baseline
// configuration: 512 experts, top-8 plus one shared expert; MXFP4 experts
// per its optimisation 1) runs three phases after the output projection:
//   ROUTER  r = W_router rmsnorm(x): BF16 rows, like any GEMV;
//   EXPGU   every workgroup reads the router logits, picks each column's
//           top-k (lower index on ties) and their renormalised softmax
//           weights, and lays the union of the picked experts (by id) and
//           the shared experts out as "slots"; it then streams the MXFP4
//           gate/up rows of the slots and stores h = w * silu(g) * u per
//           column, so only selected experts are read and each is read once
//           for all columns of a verify window (the article's observation
//           that expert activation is the verify cost);
//   EXPDOWN x += sum over slots of D_slot h_slot: an output row is the
//           gather of the slots' row segments, streamed in passes whose h
//           fits in LDS: kSlotsPerPass slots of the step for one column, one
//           pass per column over that column's own slots for a window.

struct RouteLds {
    uint32_t mask[kMaxExperts / 32];
    int nslots, nrouted;
    int slot_exp[kMaxSlots];     // expert id; ids >= n_experts are shared experts
    uint8_t slot_of[kMaxExperts];   // slot of a selected routed expert
    float wt[kMaxSlots][4];      // weight of a slot in each column (0: not selected)
    uint8_t cslot[4][kMaxTopK + kMaxShared];   // each column's own slots, ascending (windows of 2+)
    int sel[4][kMaxTopK];
    float selw[4][kMaxTopK];
    uint32_t layer, epoch;       // the routing these fields hold
};
__shared__ RouteLds s_route;
// The normalised FFN input a ROUTER task left at the start of LDS (layer and
// launch epoch it belongs to; epoch 0: none): the same workgroup's expert
// gate/up task of that layer reuses it instead of loading it again.
__shared__ uint32_t s_xs_layer, s_xs_epoch;

__device__ __forceinline__ float from_ordered_key32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Float -> unsigned key with the same order (negative values reversed).
__device__ __forceinline__ uint32_t ordered_key32(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Routing of this step, from the router logits (float32 [k][E]), into
// s_route.  Wave c < NC picks column c's top-k: lane l holds experts
// 8l .. 8l+7 and k rounds take the largest (value, then lower index) out
// one by one.  One column: each expert as a 64-bit key (the order key of
// its logit above a key of its index, larger for a lower index), a lane's
// eight keys sorted, each round one wave maximum of the lanes' first keys.
// Several columns (kernels at their register limit, where the sorted keys
// would cost registers in the expert streams): a value key and an index key
// per expert, each round a wave maximum of the value keys and one of the
// index keys among the values equal to it.
// Weights are exp(r_j - r_max) / sum over the picked j, which equals the
// picked softmax probabilities renormalised to sum to one.  The slots are
// the union of picked experts, by increasing id, then the shared experts:
// for one column each pick's rank among the picks, for several a prefix sum
// over the 16 words of the selection mask.
// Inlined: as a called function the argument block would reach it through a
// vector register, and every field read would become a vector memory load.
template <int NC>
__device__ __forceinline__ void route_slots(Ctx a, uint32_t layer) {
    RouteLds& R = s_route;
    const int E = a->n_experts, K = a->top_k;
    const int lane = lane_id(), wave = wave_id();
    constexpr int kMaskWords = kMaxExperts / 32;
    static_assert(kMaskWords <= 16, "one row of lanes scans the mask");
    if constexpr (NC > 1) {   // several waves add to the mask: clear it first
        for (int i = threadIdx.x; i < kMaskWords; i += kThreads) R.mask[i] = 0u;
        for (int i = threadIdx.x; i < kMaxSlots * 4; i += kThreads) (&R.wt[0][0])[i] = 0.f;
        __syncthreads();
    } else if (wave == 0) {   // wave 0 alone writes it below
        for (int i = lane; i < kMaxSlots * 4; i += kWave) (&R.wt[0][0])[i] = 0.f;
    }
    if (wave < NC) {
        const int c = wave;
        const rsrc_t rl = make_rsrc(a->rlogits);
        const bool has = 8 * lane < E;
        f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
        if (has) {
            v0 = ldc4(rl, (uint32_t)((c * E + 8 * lane) * 4));
            v1 = ldc4(rl, (uint32_t)((c * E + 8 * lane + 4) * 4));
        }
        if constexpr (NC == 1) {
            // key = (value key << 32) | (2^32 - 1 - index): distinct for every
            // expert, so the largest key is one lane's and the order is by
            // value, then by lower index
            uint64_t s[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = i < 4 ? v0[i] : v1[i - 4];
                const uint32_t hk = has ? ordered_key32(v) : 0u;      // finite logits give keys > 0
                s[i] = ((uint64_t)hk << 32) | (0xFFFFFFFFu - (8u * lane + i));
            }
            if (threadIdx.x == 0) s_stamp[2] = wall_clock64() | (uint32_t)(s[0] >> 32 & 1u);   // logits loaded
            // the lane's keys in descending order (odd-even merge network)
            auto cx = [&](int i, int j) {
                const uint64_t a = s[i], b = s[j];
                s[i] = max_u64(a, b);
                s[j] = a > b ? b : a;
            };
            cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
            cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
            cx(1, 2); cx(5, 6);
            cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
            cx(2, 4); cx(3, 5);
            cx(1, 2); cx(3, 4); cx(5, 6);
            // each round: the wave maximum of the lanes' first keys, which its
            // lane then drops.  The value keys alone decide it unless two lanes
            // hold the largest value (then the full keys do)
            uint64_t mine = 0;   // lane k < K: the k-th pick
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                if (k >= K) break;
                const uint32_t hh = (uint32_t)(s[0] >> 32);
                const uint32_t hm = wave_max_u32(hh);
                const uint64_t at = __builtin_amdgcn_ballot_w64(hh == hm);
                uint64_t m;
                if (__builtin_popcountll(at) == 1)
                    m = ((uint64_t)hm << 32) | (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)s[0], __builtin_ctzll(at));
                else
                    m = wave_max_u64(s[0]);
                const bool win = s[0] == m;
#pragma unroll
                for (int i = 0; i < 7; ++i) s[i] = win ? s[i + 1] : s[i];
                s[7] = win ? 0ull : s[7];
                mine = lane == k ? m : mine;
            }
            // weights in pick order: exp(value - first value), summed from the first
            const float top_v = from_ordered_key32((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), 0));
            const float ex = lane < K ? expf(from_ordered_key32((uint32_t)(mine >> 32)) - top_v) : 0.f;
            float wsum = 0.f;
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                if (k >= K) break;
                wsum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), k));
            }
            // the K picks are distinct experts: a pick's slot is its rank
            // by expert id, and the shared experts follow
            const int esel = (int)(0xFFFFFFFFu - (uint32_t)mine);
            int rank = 0;
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (j >= K) break;
                rank += __builtin_amdgcn_readlane(esel, j) < esel;
            }
            if (lane < K) {
                const float wk = ex / wsum;
                R.sel[0][lane] = esel;
                R.selw[0][lane] = wk;
                R.slot_exp[rank] = esel;
                R.wt[rank][0] = wk;
            }
            const int nsh = a->n_shared;
            if (lane < nsh) {
                R.slot_exp[K + lane] = E + lane;
                R.wt[K + lane][0] = 1.f;
            }
            if (lane == 0) {
                R.nrouted = K;
                R.nslots = K + nsh;
                R.layer = layer;
                R.epoch = a.epoch;
            }
        } else {
            // several columns (one wave each): per lane a value key and an
            // index key per expert; each round a wave maximum of the value
            // keys, then one of the index keys among the values equal to it
            uint32_t hi[8], lo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = i < 4 ? v0[i] : v1[i - 4];
                hi[i] = has ? ordered_key32(v) : 0u;      // finite logits give keys > 0
                lo[i] = 0xFFFFFFFFu - (8u * lane + i);
            }
            if (threadIdx.x == 0) s_stamp[2] = wall_clock64() | (hi[0] & 1u);   // logits loaded
            float top_v = 0.f, wsum = 0.f;
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                if (k >= K) break;
                uint32_t hm = hi[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) hm = max(hm, hi[i]);
                hm = wave_max_u32(hm);
                uint32_t lm = 0u;
#pragma unroll
                for (int i = 0; i < 8; ++i) lm = max(lm, hi[i] == hm ? lo[i] : 0u);
                lm = wave_max_u32(lm);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (hi[i] == hm && lo[i] == lm) hi[i] = 0u;
                const int esel = (int)(0xFFFFFFFFu - lm);
                const float vsel = from_ordered_key32(hm);
                if (k == 0) top_v = vsel;
                const float ex = expf(vsel - top_v);
                wsum += ex;
                if (lane == 0) {
                    R.sel[c][k] = esel;
                    R.selw[c][k] = ex;
                    atomicOr(&R.mask[esel >> 5], 1u << (esel & 31));
                }
            }
            if (lane < K) R.selw[c][lane] = R.selw[c][lane] / wsum;
        }
        if (threadIdx.x == 0) s_stamp[3] = wall_clock64();   // top-k picked
    }
    __syncthreads();
    if constexpr (NC == 1) return;
    if (wave == 0) {
        const uint32_t m = lane < kMaskWords ? R.mask[lane] : 0u;
        const uint32_t cnt = (uint32_t)__builtin_popcount(m);
        const uint32_t incl = row_prefix_sum(cnt);
        int n = (int)(incl - cnt);
        for (uint32_t mm = m; mm; mm &= mm - 1u) {
            const int e = lane * 32 + __builtin_ctz(mm);
            R.slot_of[e] = (uint8_t)n;
            R.slot_exp[n++] = e;
        }
        const int nr = __builtin_amdgcn_readlane((int)incl, kMaskWords - 1);
        if (lane < a->n_shared) R.slot_exp[nr + lane] = E + lane;
        if (lane == 0) {
            R.nrouted = nr;
            R.nslots = nr + a->n_shared;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < NC * K) {
        const int c = threadIdx.x / K, k = threadIdx.x - c * K;
        const int sl = R.slot_of[R.sel[c][k]];
        R.wt[sl][c] = R.selw[c][k];
        if constexpr (NC > 1) {   // rank among the column's (distinct) slots
            int rank = 0;
            for (int k2 = 0; k2 < K; ++k2) rank += R.slot_of[R.sel[c][k2]] < sl;
            R.cslot[c][rank] = (uint8_t)sl;
        }
    }
    if ((int)threadIdx.x < NC * a->n_shared) {
        const int c = threadIdx.x / a->n_shared, sh = threadIdx.x - c * a->n_shared;
        R.wt[R.nrouted + sh][c] = 1.f;
        if constexpr (NC > 1) R.cslot[c][K + sh] = (uint8_t)(R.nrouted + sh);
    }
    if (threadIdx.x == 0) {
        R.layer = layer;
        R.epoch = a.epoch;
    }
    __syncthreads();
}

template <int NC, class S>
__device__ __forceinline__ bool op_router(Ctx a, uint32_t layer, uint32_t tile, uint32_t wctr, uint32_t wneed,
                                       lds_f32* xs) {
    constexpr int H = S::H;
    const int lane = lane_id(), wave = wave_id();
    CLayer* L = (CLayer*)a->layers + layer;
    const int E = a->n_experts;
    const int nw = (int)a->tiles_router * kWaves, gw = (int)tile * kWaves + wave;
    const int nrows = gw < E ? (E - 1 - gw) / nw + 1 : 0;
    const uint16_t* wr = L->w_router;
    auto rowf = [&](int rr) -> GRow {
        return GRow{gp(reinterpret_cast<const uint4*>(wr + (size_t)(gw + nw * rr) * H)), nullptr};
    };
    using RS = RowStream<F_BF16, NC, H / 8>;
    RS st(nrows, lane);
    typename RS::Buf A, B;
    int pre = 0;
    const bool early = wave != 0 || a->poll_wave_prefetch;   // the polling wave may hold its loads back
    if (early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a));
    if (!wait_counter(a, wctr, wneed)) return false;
    dma_input(a, a->xres, NC * H, xs);
    norm_in_place<NC, H>(a, L->ffn_norm, xs);
    if (threadIdx.x == 0) {
        s_xs_layer = layer;
        s_xs_epoch = a.epoch;
    }
    if (!early) pre = st.prefetch(A, B, rowf, gemv_pre_rows<RS>(a));   // after the input loads, not ahead of them
    stamp(0);
    MBG_GLOBAL float* rl = gp(a->rlogits);
    auto out = [&](int rr, const float (&s)[NC]) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (lane == c) stc(rl + (size_t)c * E + gw + nw * rr, s[c]);
    };
    // compact loop: the split one spills in the routed kernel, and a wave has at most one chunk
    st.template run<false>(A, B, rowf, xs, H, out, st.finish_prefetch(A, B, rowf, pre));
    stamp(1);
    release_counter(a, ctr_index(layer, PH_ROUTER));
    return true;
}

template <int NC, class S>
__device__ __forceinline__ bool op_expgu(Ctx a, uint32_t layer, uint32_t tile, uint32_t wctr, uint32_t wneed,
                                      lds_f32* xs) {
    constexpr int H = S::H, MF = S::MF;
    const int lane = lane_id(), wave = wave_id();
    CLayer* L = (CLayer*)a->layers + layer;
    // the input (the stream after the output projection) is complete before
    // the router is: load and normalise it first, then wait for the logits;
    // a workgroup whose router task of this layer left it in LDS keeps it
    if (!(s_xs_layer == layer && s_xs_epoch == a.epoch)) {
        if (!wait_counter(a, ctr_index(layer, PH_OPROJ), a->tiles_o)) return false;
        dma_input(a, a->xres, NC * H, xs);
        norm_in_place<NC, H>(a, L->ffn_norm, xs);
    }
    if (!wait_counter(a, wctr, wneed)) return false;
    route_slots<NC>(a, layer);
    const RouteLds& R = s_route;
    stamp(0);
    const int E = a->n_experts;
    const int U = R.nslots;
    // a workgroup owns a contiguous block of units (rows of one or two
    // experts, so that few experts' pages pass through its address
    // translation cache); its wavefronts interleave within the block
    const int total = U * MF;
    const int per = (total + (int)a->tiles_egu - 1) / (int)a->tiles_egu;
    const int u0 = (int)tile * per, u1 = min(total, u0 + per);
    const int nunits = u0 + wave < u1 ? (u1 - 1 - u0 - wave) / kWaves + 1 : 0;
    const uint8_t* egc = L->eg_codes;
    const uint8_t* egs = L->eg_scales;
    const uint8_t* sgc = L->sg_codes;
    const uint8_t* sgs = L->sg_scales;
    constexpr size_t kMatCodes = (size_t)2 * MF * (H / 2), kMatScales = (size_t)2 * MF * (H / 32);
    auto rowf = [&](int rr) -> GRow {
        const int u = u0 + wave + kWaves * (rr >> 1);
        const int slot = u / MF;
        const int f = u - slot * MF;
        const int e = R.slot_exp[slot];
        const size_t row = (size_t)f + (size_t)(rr & 1) * MF;
        const uint8_t* cb = e < E ? egc + (size_t)e * kMatCodes : sgc + (size_t)(e - E) * kMatCodes;
        const uint8_t* sb = e < E ? egs + (size_t)e * kMatScales : sgs + (size_t)(e - E) * kMatScales;
        return GRow{gp(reinterpret_cast<const uint4*>(cb + row * (H / 2))), gp(sb + row * (H / 32))};
    };
    MBG_GLOBAL float* hb = gp(a->hbuf);
    const int ld = a->hb_ld;
    if constexpr (NC >= 2) {
        if (a->verify_mfma) {
            // matrix-core tile: 16 rows (8 units) per instruction block
            MBG_LDS u32x4* bprep = reinterpret_cast<MBG_LDS u32x4*>(xs + NC * H);
            mfma_prep_b<F_MXFP4, NC, H>(xs, H, bprep, wave, kWaves, lane);
            MfmaStream<F_MXFP4, NC, H> ms(2 * nunits, lane);
            auto outb = [&](int b, const float (&d)[4]) {
                const int n = lane & 15, j = lane >> 4;
                if (n >= NC) return;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int iu = 8 * b + 2 * j + p;   // rows 2 iu (gate) and 2 iu + 1 (up)
                    if (iu >= nunits) continue;
                    const int u = u0 + wave + kWaves * iu;
                    const float gv = d[2 * p], uv = d[2 * p + 1];
                    stc(hb + (size_t)n * ld + u, R.wt[u / MF][n] * (gv / (1.0f + expf(-gv)) * uv));
                }
            };
            ms.run(rowf, bprep, outb);
            stamp(1);
            if (tile == 0 && (int)threadIdx.x < NC * a->top_k) {  // routing record of this step
                const int c = threadIdx.x / a->top_k, k = threadIdx.x - c * a->top_k;
                const size_t o = ((size_t)layer * a->ncol + c) * a->top_k + k;
                gp(a->route_idx)[o] = R.sel[c][k];
                gp(a->route_w)[o] = R.selw[c][k];
            }
            release_counter(a, ctr_index(layer, PH_GATEUP));
            return true;
        }
    }
    // a wave's rows (about 14 of 1.3 KiB for the routed model) are issued at
    // once: the rows are only known after routing, so nothing was prefetched
    // before the wait.  Rows are 80 vectors:
    // for one or two columns the segmented stream keeps every lane busy, and
    // a unit's gate and up rows (rr = 2 iu, 2 iu + 1) sit in neighbouring
    // lane groups; wider windows keep one row per instruction (the segmented
    // buffers would spill)
    if constexpr (NC <= 2) {
        constexpr int LPR = seg_lanes<H / 32>();
        using SS = SegStream<F_MXFP4, NC, H / 32, LPR, (NC == 1 ? 4 : 1)>;
        static_assert(SS::P % 2 == 0, "a unit's two rows share a wave instruction");
        SS st(2 * nunits, lane);
        typename SS::Buf A, B;
        auto out = [&](int rr, const float (&s)[NC]) {
            const int t = lane % LPR;
            float gv = 0.f, uv = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const float other = xor_lanes<LPR>(s[c]);   // the partner row's sums
                if (c == t) { gv = s[c]; uv = other; }
            }
            const int iu = rr >> 1;
            if ((rr & 1) || t >= NC || iu >= nunits) return;
            const int u = u0 + wave + kWaves * iu;
            stc(hb + (size_t)t * ld + u, R.wt[u / MF][t] * (gv / (1.0f + expf(-gv)) * uv));
        };
        // one column: a wave's rows in one chunk; two: the split loop (each
        // chunk computed while the next is in flight)
        st.template run<(NC >= 2)>(A, B, rowf, xs, H, out);
    } else {
        using RS = RowStream<F_MXFP4, NC, H / 32, 4>;
        RS st(2 * nunits, lane);
        typename RS::Buf A, B;
        st.issue(A, 0, rowf);
        float gate[NC];
        auto out = [&](int rr, const float (&s)[NC]) {
            if ((rr & 1) == 0) {
#pragma unroll
                for (int c = 0; c < NC; ++c) gate[c] = s[c];
                return;
            }
            if (lane >= NC) return;
            const int c = lane;
            float gv = 0.f, uv = 0.f;
#pragma unroll
            for (int cc = 0; cc < NC; ++cc)
                if (cc == c) { gv = gate[cc]; uv = s[cc]; }
            const int u = u0 + wave + kWaves * (rr >> 1);
            stc(hb + (size_t)c * ld + u, R.wt[u / MF][c] * (gv / (1.0f + expf(-gv)) * uv));
        };
        // split loop: each chunk computed while the next is in flight
        st.template run<true>(A, B, rowf, xs, H, out);
    }
    stamp(1);
    if (tile == 0 && (int)threadIdx.x < NC * a->top_k) {  // routing record of this step
        const int c = threadIdx.x / a->top_k, k = threadIdx.x - c * a->top_k;
        const size_t o = ((size_t)layer * a->ncol + c) * a->top_k + k;
        gp(a->route_idx)[o] = R.sel[c][k];
        gp(a->route_w)[o] = R.selw[c][k];
    }
    release_counter(a, ctr_index(layer, PH_GATEUP));
    return true;
}

template <int NC, class S>
__device__ __forceinline__ bool op_expdown(Ctx a, uint32_t layer, uint32_t tile, uint32_t wctr, uint32_t wneed,
                                        lds_f32* xs) {
    constexpr int H = S::H, MF = S::MF;
    constexpr int VPS = MF / 32;                     // 16-byte vectors per slot segment of a row
    // One column: passes over the routing's slots in order (the 8 routed +
    // 1 shared experts of the step in one pass).  Several columns: one pass
    // per column over that column's own slots (its h is zero for the other
    // experts of the window, ~70 % of a 4-token window's slot union), the
    // next column's weights in flight while a column is computed; an expert
    // two columns share is read twice.
    constexpr int SPP = NC >= 2 ? kMaxTopK + kMaxShared : kSlotsPerPass;
    constexpr int NV = SPP * VPS;                    // vectors per pass
    constexpr int NJ = (NV + kWave - 1) / kWave;
    constexpr int XLD = SPP * MF;                    // LDS floats per column (one column a pass for NC >= 2)
    const int lane = lane_id(), wave = wave_id();
    CLayer* L = (CLayer*)a->layers + layer;
    const RouteLds& R = s_route;
    const int E = a->n_experts;
    const int nw = (int)a->tiles_edown * kWaves, gw = (int)tile * kWaves + wave;
    const int nrows = gw < H ? min((H - 1 - gw) / nw + 1, kMaxDownRows) : 0;
    const uint8_t* edc = L->ed_codes;
    const uint8_t* eds = L->ed_scales;
    const uint8_t* sdc = L->sd_codes;
    const uint8_t* sds = L->sd_scales;
    constexpr size_t kMatCodes = (size_t)H * (MF / 2), kMatScales = (size_t)H * (MF / 32);
    // every row's gathered vectors of a pass, all in flight at once
    struct PassBuf {
        uint4 w[kMaxDownRows][NJ];
        uint32_t sb[kMaxDownRows][NJ];
    };
    // pass vector v of this lane belongs to slot slot_at(v / VPS)
    auto issue_pass = [&](PassBuf& P, int ns, auto slot_at) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int v = lane + kWave * j;
            const bool act = v < ns * VPS;
            const int slot = slot_at(act ? v / VPS : 0);
            const int vv = v - (v / VPS) * VPS;
            const int e = R.slot_exp[slot];
            const uint8_t* cb = e < E ? edc + (size_t)e * kMatCodes : sdc + (size_t)(e - E) * kMatCodes;
            const uint8_t* scb = e < E ? eds + (size_t)e * kMatScales : sds + (size_t)(e - E) * kMatScales;
#pragma unroll
            for (int i = 0; i < kMaxDownRows; ++i) {
                if (i < nrows && act) {
                    const size_t r = (size_t)(gw + nw * i);
                    P.w[i][j] = ld_stream_g(gp(reinterpret_cast<const uint4*>(cb + r * (MF / 2))) + vv);
                    P.sb[i][j] = gp(scb)[r * (MF / 32) + vv];
                }
            }
        }
    };
    auto col_slot = [&](int c) { return [&R, c](int k) { return (int)R.cslot[c][k]; }; };
    const int ncs = a->top_k + a->n_shared;          // slots of one column
    PassBuf PA, PB;
    // this workgroup's expert gate/up task of the layer left the routing in
    // LDS: then the first pass's weights are requested before the wait
    const bool have_route = R.layer == layer && R.epoch == a.epoch;
    if (have_route) {
        if constexpr (NC == 1) issue_pass(PA, min(SPP, R.nslots), [](int k) { return k; });
        else issue_pass(PA, ncs, col_slot(0));
    }
    // the residual after this layer's output projection (final since this
    // workgroup's expert gate/up wait)
    MBG_GLOBAL float* x = gp(a->xres);
    float res_pre[kMaxDownRows];
#pragma unroll
    for (int i = 0; i < kMaxDownRows; ++i)
        res_pre[i] = (i < nrows && lane < NC) ? ldc(x + lane * H + gw + nw * i) : 0.f;
    if (!wait_counter(a, wctr, wneed)) return false;
    if (!have_route) route_slots<NC>(a, layer);
    stamp(0);
    const int U = R.nslots;
    const rsrc_t hr = make_rsrc(a->hbuf);
    const int ld = a->hb_ld;
    float acc[kMaxDownRows][NC];
#pragma unroll
    for (int i = 0; i < kMaxDownRows; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[i][c] = 0.f;
    // a pass's h into LDS: column c (of cols) of slots slot_at(0 .. ns) ->
    // xs[(c - c0) * XLD + k * MF + f]
    auto load_h = [&](int c0, int cols, int ns, auto slot_at) {
        __syncthreads();
        constexpr int Q = MF / 4;
        const int nvec = ns * Q;
        for (int c = 0; c < cols; ++c)
            for (int j = threadIdx.x; j < nvec; j += kThreads) {
                const int k = j / Q, f4 = j - k * Q;
                *reinterpret_cast<MBG_LDS f32x4*>(xs + c * XLD + 4 * j) =
                    ldc4(hr, (uint32_t)(((size_t)(c0 + c) * ld + (size_t)slot_at(k) * MF + 4 * f4) * 4));
            }
        __syncthreads();
    };
    // acc[i][c0 .. c0 + cols) += the pass's rows against LDS columns 0 .. cols
    auto compute_pass = [&](const PassBuf& P, int ns, auto c0v, auto colsv) {
        constexpr int c0 = decltype(c0v)::value, cols = decltype(colsv)::value;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int v = lane + kWave * j;
            if (v >= ns * VPS) continue;
            float xv[cols][32];
#pragma unroll
            for (int c = 0; c < cols; ++c)
#pragma unroll
                for (int e4 = 0; e4 < 32; e4 += 4) {
                    const f32x4 t = *reinterpret_cast<const MBG_LDS f32x4*>(xs + c * XLD + v * 32 + e4);
                    xv[c][e4] = t[0];
                    xv[c][e4 + 1] = t[1];
                    xv[c][e4 + 2] = t[2];
                    xv[c][e4 + 3] = t[3];
                }
#pragma unroll
            for (int i = 0; i < kMaxDownRows; ++i) {
                if (i >= nrows) continue;
                float wf[32];
                decode16<F_MXFP4>(P.w[i][j], P.sb[i][j], wf);
#pragma unroll
                for (int c = 0; c < cols; ++c) {
                    float p0 = 0.f, p1 = 0.f;
#pragma unroll
                    for (int e2 = 0; e2 < 32; e2 += 2) {
                        p0 = fmaf(wf[e2], xv[c][e2], p0);
                        p1 = fmaf(wf[e2 + 1], xv[c][e2 + 1], p1);
                    }
                    acc[i][c0 + c] += p0 + p1;
                }
            }
        }
    };
    using C0 = std::integral_constant<int, 0>;
    if constexpr (NC == 1) {
        for (int s0 = 0; s0 < U; s0 += SPP) {
            const int ns = min(SPP, U - s0);
            auto seq = [s0](int k) { return s0 + k; };
            load_h(0, 1, ns, seq);
            if (s0 > 0 || !have_route) issue_pass(PA, ns, seq);
            compute_pass(PA, ns, C0{}, std::integral_constant<int, 1>{});
        }
    } else {
        if (!have_route) issue_pass(PA, ncs, col_slot(0));
        // column c: its h into LDS (that wait has also retired its weights),
        // then column c + 1's weights requested, then column c computed
        auto column = [&](auto cv, PassBuf& cur, PassBuf& nxt) {
            constexpr int c = decltype(cv)::value;
            load_h(c, 1, ncs, col_slot(c));
            if constexpr (c + 1 < NC) issue_pass(nxt, ncs, col_slot(c + 1));
            compute_pass(cur, ncs, cv, std::integral_constant<int, 1>{});
        };
        column(C0{}, PA, PB);
        column(std::integral_constant<int, 1>{}, PB, PA);
        if constexpr (NC > 2) column(std::integral_constant<int, 2>{}, PA, PB);
        if constexpr (NC > 3) column(std::integral_constant<int, 3>{}, PB, PA);
    }
    stamp(1);
#pragma unroll
    for (int i = 0; i < kMaxDownRows; ++i) {
        if (i >= nrows) continue;
        const int r = gw + nw * i;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float sum = wave_sum(acc[i][c]);
            if (lane == c) stc(x + c * H + r, res_pre[i] + sum);
        }
    }
    release_counter(a, ctr_index(layer, PH_DOWN));
    return true;
}

// ------------------------------------------------- speculative acceptance

// Greedy prefix acceptance of a verify window (163.com Ling-3.0-flash
// article, optimisation 3: the target checks the draft's tokens in one
// pass and keeps the prefix it agrees with).  The window holds t0 (the last
// emitted token) and the draft's d1 .. d(NC-1); am[j] is the target's argmax
// after window[j].  Draft j + 1 is accepted while am[j] == d(j+1); with m
// accepted, the round emits am[0 .. m] (the accepted drafts and the target's
// own next token) and the next round starts from am[m] at pos + m + 1.  One
// thread; the state words of this round were written by earlier launches.
template <int NC>
__device__ __forceinline__ void spec_accept(Ctx a, const int32_t* am) {
    const MBG_GLOBAL int32_t* cur = gp(a->spec_cur);
    MBG_GLOBAL int32_t* nxt = gp(a->spec_next);
    const MBG_GLOBAL int32_t* win = cur + SPEC_WINDOW;
    int m = 0;
    while (m < NC - 1 && am[m] == win[m + 1]) ++m;
    const int done = cur[SPEC_EMITTED];
    MBG_GLOBAL int32_t* emit = gp(a->spec_emit);
    for (int j = 0; j <= m; ++j)
        if (done + j < a->spec_emit_cap) emit[done + j] = am[j];
    if (done + m + 1 > a->spec_emit_cap) latch_error(a->flags, kStatusRange);
    nxt[SPEC_POS] = a.pos + m + 1;
    nxt[SPEC_EMITTED] = min(done + m + 1, a->spec_emit_cap);
    nxt[SPEC_ACCEPTED] = cur[SPEC_ACCEPTED] + m;
    nxt[SPEC_ROUNDS] = cur[SPEC_ROUNDS] + 1;
    nxt[SPEC_WINDOW] = am[m];
}

// --------------------------------------------------------------- LM head

template <int NC, class S, int F>
__device__ __forceinline__ bool op_lmhead(Ctx a, uint32_t tile, uint32_t wctr, uint32_t wneed, lds_f32* xs) {
    constexpr int H = S::H;
    constexpr int E = FmtInfo<F>::kEPV;
    __shared__ unsigned long long wbest[kWaves * 4];
    const int lane = lane_id(), wave = wave_id();
    const int V = a->vocab;
    // a workgroup owns a contiguous block of rows (few pages per address
    // translation cache); its wavefronts interleave within the block
    const int per = (V + (int)a->tiles_lm - 1) / (int)a->tiles_lm;
    const int r0 = (int)tile * per + wave, r1 = min(V, (int)tile * per + per);
    const int nrows = r0 < r1 ? (r1 - 1 - r0) / kWaves + 1 : 0;
    const MBG_GLOBAL uint4* W = gp(reinterpret_cast<const uint4*>(a->lm_head));
    const MBG_GLOBAL float* lsc = gp(a->lm_scale);
    // rows that do not fill whole 64-lane vector columns (FP8 rows of 2560
    // are 160 vectors): up to two columns the segmented stream (two rows
    // per instruction, the row's FP8 scale loaded with it); wider windows
    // one row per instruction (registers)
    constexpr int NV = H / E;
    constexpr bool kSeg = NC <= 2 && NV % kWave != 0;
    constexpr int SLPR = seg_lanes<NV>();
    constexpr int LPR = kSeg ? SLPR : kWave;   // lanes that share a row
    auto rowf = [&](int rr) -> GRow {
        const size_t r = (size_t)(r0 + kWaves * rr);
        return GRow{W + r * NV, F == F_FP8 ? reinterpret_cast<const MBG_GLOBAL uint8_t*>(lsc + r) : nullptr};
    };
    using SS = SegStream<F, NC, NV, SLPR, (NC == 1 && NV / SLPR <= 8 ? 2 : 1), F == F_FP8>;
    using RS = RowStream<F, NC, NV>;
    SS ss(nrows, lane);
    RS rs(nrows, lane);
    typename SS::Buf SA, SB;
    typename RS::Buf A, B;
    const int pre_kib = a->gemv_pre;
    int pre = 0;
    auto do_prefetch = [&]() {
        if constexpr (kSeg) pre = ss.prefetch(SA, SB, rowf, (pre_kib * 1024 + SS::kRowsPerChunk * NV * 16 - 1) /
                                                                (SS::kRowsPerChunk * NV * 16));
        else pre = rs.prefetch(A, B, rowf, gemv_pre_rows<RS>(pre_kib));
    };
    const bool early = wave != 0 || a->poll_wave_prefetch;   // the polling wave may hold its loads back
    if (early) do_prefetch();
    RowScales rsc;   // FP8 rows of the one-row stream: their scales, requested before the wait
    if constexpr (F == F_FP8 && !kSeg)
        rsc.load(lsc, nrows, lane, [&](int rr) { return (size_t)(r0 + kWaves * rr); });
    if (!wait_counter(a, wctr, wneed)) return false;
    dma_input(a, a->xres, NC * H, xs);
    norm_in_place<NC, H>(a, a->final_norm, xs);
    if (!early) do_prefetch();   // after the input loads, not ahead of them
    stamp(0);
    unsigned long long best[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) best[c] = 0ull;
    MBG_GLOBAL float* logits = a->logits ? gp(a->logits) + (size_t)a.step * NC * a->vocab : nullptr;
    // rr: this lane's row (wave-uniform for the one-row stream); s: its sums
    auto out = [&](int rr, const float (&s)[NC]) {
        if (rr >= nrows) return;
        const uint32_t r = (uint32_t)(r0 + kWaves * rr);
        float sc = 1.0f;
        if constexpr (F == F_FP8 && !kSeg) sc = rsc.get(rr, r);
        const int t = lane % LPR;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float v = s[c] * sc;
            if (logits != nullptr && t == c) logits[(size_t)c * V + r] = v;
            const unsigned long long k = ((unsigned long long)ordered_key32(v) << 32) | (0xFFFFFFFFu - r);
            best[c] = k > best[c] ? k : best[c];
        }
    };
    if constexpr (kSeg) {
        // split loop for several columns, compact for one (measured faster
        // in the step)
        ss.template run<(NC >= 2)>(SA, SB, rowf, xs, H, out, pre);
        // lanes hold the best of their own rows
#pragma unroll
        for (int c = 0; c < NC; ++c) best[c] = wave_max_u64(best[c]);
    } else {
        // compact loop: the split one spills in the dense kernels (BF16 head rows)
        rs.template run<false>(A, B, rowf, xs, H, out, rs.finish_prefetch(A, B, rowf, pre));
    }
    stamp(1);
    if (lane == 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) wbest[wave * 4 + c] = best[c];
    }
    __syncthreads();
    MBG_GLOBAL unsigned long long* keys = gp(a->amax_keys);
    if (threadIdx.x < NC) {
        const int c = threadIdx.x;
        unsigned long long b = wbest[c];
        for (int w = 1; w < kWaves; ++w) b = wbest[w * 4 + c] > b ? wbest[w * 4 + c] : b;
        __hip_atomic_fetch_max(keys + c, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(gp(a->lm_ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old + 1u == a.epoch * a->tiles_lm);
    }
    __syncthreads();
    __shared__ int32_t s_amax[4];
    if (s_last && threadIdx.x < NC) {
        const int c = threadIdx.x;
        const unsigned long long k = __hip_atomic_load(keys + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int32_t am = (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
        // device-coherent: the next step of a multi-step launch reads it as its token
        __hip_atomic_store(gp(a->argmax) + (size_t)a.step * NC + c, am, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(keys + c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_amax[c] = am;
    }
    if (s_last && a->spec_next) {   // wave-uniform: s_last is the workgroup's
        __syncthreads();
        if (threadIdx.x == 0) spec_accept<NC>(a, s_amax);
    }
    if (s_last) release_counter(a, token_ctr_index(a));   // this step's token is written
    return true;
}

// ------------------------------------------------------------------ kernel

template <int NC, class S>
__global__ void __launch_bounds__(kThreads, 1) step_kernel(StepArgs args) {
    (void)args;
    CArgs* ka = (CArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    extern __shared__ __align__(16) float smem_raw[];
    lds_f32* smem = (lds_f32*)smem_raw;
    const uint32_t b = blockIdx.x;
    const MBG_CONST uint32_t* off = (const MBG_CONST uint32_t*)ka->task_off;
    const MBG_CONST u32x4* tasks = (const MBG_CONST u32x4*)ka->tasks;
    const uint32_t end = off[b + 1];
    MBG_GLOBAL unsigned long long* trace = ka->trace ? gp(ka->trace) : nullptr;
    if (threadIdx.x == 0) {
        s_stamp[2] = s_stamp[3] = 0;
        s_route.epoch = 0;   // no routing held yet (epochs start at 1)
        s_xs_epoch = 0;      // no router input held yet
        if (S::KVF == F_BF16 && ka->attn_local) {   // the attention placement assumes workgroup b runs on XCD b % 8
            uint32_t xcc;
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
            if ((xcc & 0xFu) != (blockIdx.x & 7u)) latch_error(ka->status, kStatusPlacement);
        }
    }
    const int nsteps = ka->nsteps;
    int pos0 = ka->pos;
    if (ka->dpos) {   // a speculative round's launch: its position is on the device
        pos0 = *(const MBG_GLOBAL int32_t*)ka->dpos;
        if (pos0 < 0 || pos0 > ka->max_pos - (ka->ncol + nsteps - 1)) {   // every workgroup sees the same value
            if (threadIdx.x == 0 && blockIdx.x == 0) latch_error(ka->status, kStatusPosition);
            return;
        }
    }
    for (int step = 0; step < nsteps; ++step) {
    const Ctx a{ka, ka->epoch + (uint32_t)step, pos0 + step, step};
    // a later step of the launch starts when the previous step's argmax (its
    // token) is written
    if (step > 0 && !wait_until(a, token_ctr_index(a), a.epoch - 1u)) {
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    for (uint32_t ti = off[b]; ti < end; ++ti) {
        const u32x4 tv = tasks[ti];
        const Task tk{tv[0], tv[1], tv[2], tv[3]};
        const uint32_t op = tk.op_layer & 0xFFu;
        const uint32_t layer = tk.op_layer >> 8;
        const uint64_t t_start = trace ? wall_clock64() : 0;
        bool ok = true;
        switch (op) {
            case OP_QKV: ok = op_qkv<NC, S>(a, layer, tk.tile, tk.wait_ctr, tk.wait_need, smem); break;
            case OP_ATTN: ok = op_attn<NC, S>(a, layer, tk.tile, tk.wait_ctr, tk.wait_need, smem); break;
            case OP_OPROJ: ok = op_oproj<NC, S>(a, layer, tk.tile, tk.wait_ctr, tk.wait_need, smem); break;
            case OP_GATEUP:
                if constexpr (!S::MOE) ok = op_gateup<NC, S>(a, layer, tk.tile, tk.wait_ctr, tk.wait_need, smem);
                break;
            case OP_DOWN:
                if constexpr (!S::MOE) ok = op_down<NC, S>(a, layer, tk.tile, tk.wait_ctr, tk.wait_need, smem);
                break;
            case OP_ROUTER:
                if constexpr (S::MOE) ok = op_router<NC, S>(a, layer, tk.tile, tk.wait_ctr, tk.wait_need, smem);
                break;
            case OP_EXPGU:
                if constexpr (S::MOE) ok = op_expgu<NC, S>(a, layer, tk.tile, tk.wait_ctr, tk.wait_need, smem);
                break;
            case OP_EXPDOWN:
                if constexpr (S::MOE) ok = op_expdown<NC, S>(a, layer, tk.tile, tk.wait_ctr, tk.wait_need, smem);
                break;
            case OP_LMHEAD:
                ok = a->lm_dtype == F_FP8 ? op_lmhead<NC, S, F_FP8>(a, tk.tile, tk.wait_ctr, tk.wait_need, smem)
                                          : op_lmhead<NC, S, F_BF16>(a, tk.tile, tk.wait_ctr, tk.wait_need, smem);
                break;
            default: break;
        }
        if (!ok) {
            // the launch is aborting: let every load this wave issued (weight
            // prefetch, LDS DMA) land before the wave ends
            __builtin_amdgcn_s_waitcnt(0);
            return;
        }
        __syncthreads();  // LDS is reused by the next task
        if (trace && threadIdx.x == 0) {
            MBG_GLOBAL unsigned long long* r = trace + (size_t)ti * 8;
            r[0] = t_start;
            r[1] = s_twait;
            r[2] = s_stamp[0];
            r[3] = s_stamp[1];
            r[4] = wall_clock64();
            r[5] = (unsigned long long)tk.op_layer | ((unsigned long long)tk.tile << 32);
            r[6] = s_stamp[2];
            r[7] = s_stamp[3];
            s_stamp[2] = 0;
            s_stamp[3] = 0;
        }
    }
    }
}

// ----------------------------------------------------------- variants

// Model families compiled in: Shape<hidden, ffn, q_heads * head_dim,
// head_dim, q heads per KV head, KV format, MoE, moe_ffn>.  This file is
// compiled once per family (MBG_STEP_SHAPE = 0 .. kStepShapes - 1), so the
// families build in parallel; step_kernel_for (api side) asks each.
#if !defined(MBG_STEP_SHAPE)
#error "compile step.hip with -DMBG_STEP_SHAPE=<0..3>"
#elif MBG_STEP_SHAPE == 0
using ThisShape = Shape<256, 1024, 256, 64, 2, F_BF16, 0, 0>;         // tiny dense
#elif MBG_STEP_SHAPE == 1
using ThisShape = Shape<2048, 8192, 2048, 128, 2, F_BF16, 0, 0>;      // dense 2B, BF16 KV
#elif MBG_STEP_SHAPE == 2
using ThisShape = Shape<2048, 8192, 2048, 128, 2, F_FP8, 0, 0>;       // dense 2B, FP8 KV
#elif MBG_STEP_SHAPE == 3
using ThisShape = Shape<2560, 0, 4096, 128, 8, F_BF16, 1, 768>;       // routed
#else
#error "unknown MBG_STEP_SHAPE"
#endif

template <class S>
static bool matches(const StepVariant& v) {
    return v.hidden == S::H && v.ffn == S::F && v.qdim == S::QD && v.head_dim == S::HD && v.group == S::GQ &&
           v.kv_fmt == S::KVF && v.moe == S::MOE && v.moe_ffn == S::MF;
}

template <class S>
static const void* pick(int ncol) {
    switch (ncol) {
        case 1: return reinterpret_cast<const void*>(&step_kernel<1, S>);
        case 2: return reinterpret_cast<const void*>(&step_kernel<2, S>);
        case 3: return reinterpret_cast<const void*>(&step_kernel<3, S>);
        case 4: return reinterpret_cast<const void*>(&step_kernel<4, S>);
    }
    return nullptr;
}

#define MBG_CAT2(a, b) a##b
#define MBG_CAT(a, b) MBG_CAT2(a, b)

const void* MBG_CAT(step_kernel_shape_, MBG_STEP_SHAPE)(const StepVariant& v, int ncol, int* lds_bytes_out) {
    if (!matches<ThisShape>(v)) return nullptr;
    const void* fn = pick<ThisShape>(ncol);
    if (fn && lds_bytes_out) {
        int kmax = v.hidden;
        if (v.ffn > kmax) kmax = v.ffn;
        if (v.qdim > kmax) kmax = v.qdim;
        if (v.moe_ffn > kmax) kmax = v.moe_ffn;
        const int xs_bytes = ncol * kmax * 4 + kWaves * kQkvRowsPerWave * ncol * 4;
        // attention: rings (reused by the combine), then the cross-wave merge
        // rows or the combine's group sums, whichever is larger
        const int merge_bytes = kWaves * attn_heads(v.group) * (v.head_dim + kPartPad) * 4;
        const int red_bytes = kAttnRingBytes + (merge_bytes > kThreads * 16 ? merge_bytes : kThreads * 16);
        int moe_bytes = v.moe ? ncol * kSlotsPerPass * v.moe_ffn * 4 : 0;
        if (v.moe && ncol >= 2) {   // matrix-core expert gate/up: activations plus prepared B operands
            const int mb = ncol * v.hidden * 4 + (v.hidden / 32) * kWave * 16;
            if (mb > moe_bytes) moe_bytes = mb;
        }
        int m = xs_bytes > red_bytes ? xs_bytes : red_bytes;
        *lds_bytes_out = m > moe_bytes ? m : moe_bytes;
    }
    return fn;
}

}  // namespace mbg
