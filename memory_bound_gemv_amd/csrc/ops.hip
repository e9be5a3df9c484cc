// Standalone kernels: LM-head GEMV fused with argmax, online FP8 row
// quantisation, and the quantising K/V write into the paged cache.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gemv.h"
#include "ops.h"

namespace mbg {

// ---------------------------------------------------------------- argmax

// Order-preserving map of a binary32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_f32(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Packed argmax key: value first, then the lower row index wins ties.
__device__ __forceinline__ unsigned long long argmax_key(float f, uint32_t row) {
    return ((unsigned long long)ordered_f32(f) << 32) | (unsigned long long)(0xFFFFFFFFu - row);
}

// ------------------------------------------------------------- LM head

// Workgroup b owns a contiguous block of rows of the head and its four
// wavefronts take every fourth row of it, streamed back to back; one argmax key per workgroup is merged with
// a 64-bit atomic max, and the last workgroup turns the keys into indices.
template <int F, int NC, int H>
__global__ void __launch_bounds__(256) lm_head_kernel(LmHeadArgs a) {
    extern __shared__ __align__(16) float smem_raw[];
    lds_f32* xs = (lds_f32*)smem_raw;                  // [NC][H]
    __shared__ unsigned long long wbest[4 * 4];
    __shared__ uint32_t last;
    constexpr int E = FmtInfo<F>::kEPV;
    constexpr int NV = H / E;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // a workgroup owns a contiguous block of rows (few pages per address
    // translation cache); its wavefronts interleave within the block
    const int per = (int)((a.V + (int)gridDim.x - 1) / (int)gridDim.x);
    const int r0 = (int)blockIdx.x * per + wave, r1 = min(a.V, (int)blockIdx.x * per + per);
    const int nrows = r0 < r1 ? (r1 - 1 - r0) / 4 + 1 : 0;
    const MBG_GLOBAL uint4* W = gp(reinterpret_cast<const uint4*>(a.w));
    const MBG_GLOBAL uint8_t* Ws = gp(reinterpret_cast<const uint8_t*>(a.wscale));   // MXFP4: E8M0 [V][H/32]
    // rows that do not fill whole 64-lane vector columns (FP8 and MXFP4
    // rows of 2560, ...) go through the segmented stream for one or two
    // columns, the FP8 row scale loaded with its row
    constexpr bool kSeg = NC <= 2 && NV % kWave != 0;
    constexpr int SLPR = seg_lanes<NV>();
    constexpr int LPR = kSeg ? SLPR : kWave;   // lanes that share a row
    const MBG_GLOBAL float* fsc = gp(reinterpret_cast<const float*>(a.wscale));   // FP8: [V]
    auto rowf = [&](int rr) -> GRow {
        const size_t row = (size_t)(r0 + 4 * rr);
        const MBG_GLOBAL uint8_t* sp = F == F_MXFP4 ? Ws + row * NV
                                       : F == F_FP8 ? reinterpret_cast<const MBG_GLOBAL uint8_t*>(fsc + row)
                                                    : nullptr;
        return GRow{W + row * NV, sp};
    };
    using SS = SegStream<F, NC, NV, SLPR, (NC == 1 && NV / SLPR <= 8 ? 2 : 1), F == F_FP8>;
    using RS = RowStream<F, NC, NV>;
    SS ss(nrows, lane);
    RS st(nrows, lane);
    typename SS::Buf SA, SB;
    typename RS::Buf A, B;
    // weights do not depend on x: start streaming first
    int pre = 0;
    if constexpr (kSeg) pre = ss.prefetch(SA, SB, rowf, 1);
    else st.issue(A, 0, rowf);

    RowScales rsc;
    if constexpr (F == F_FP8 && !kSeg) rsc.load(fsc, nrows, lane, [&](int rr) { return (size_t)(r0 + 4 * rr); });
    const MBG_GLOBAL float* x = gp(a.x);
    for (int i = threadIdx.x; i < NC * H; i += blockDim.x) xs[i] = x[i];
    __syncthreads();

    unsigned long long best[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) best[c] = 0ull;
    MBG_GLOBAL float* logits = a.logits ? gp(a.logits) : nullptr;
    // rr: this lane's row (wave-uniform for the one-row stream); s: its sums
    auto out = [&](int rr, const float (&s)[NC]) {
        if (rr >= nrows) return;
        const uint32_t r = (uint32_t)(r0 + 4 * rr);
        float sc = 1.0f;
        if constexpr (F == F_FP8 && !kSeg) sc = rsc.get(rr, r);
        const int t = lane % LPR;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float v = s[c] * sc;
            if (logits != nullptr && t == c) logits[(size_t)c * a.V + r] = v;
            const unsigned long long k = argmax_key(v, r);
            best[c] = k > best[c] ? k : best[c];
        }
    };
    if constexpr (kSeg) {
        ss.template run<true>(SA, SB, rowf, xs, H, out, pre);
#pragma unroll
        for (int c = 0; c < NC; ++c) best[c] = wave_max_u64(best[c]);   // lanes held their own rows' best
    } else {
        st.template run<true>(A, B, rowf, xs, H, out);
    }

    if (lane == 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) wbest[wave * 4 + c] = best[c];
    }
    __syncthreads();
    MBG_GLOBAL unsigned long long* keys = gp(a.keys);
    if (threadIdx.x < NC) {
        const int c = threadIdx.x;
        unsigned long long b = wbest[c];
        for (int w = 1; w < 4; ++w) b = wbest[w * 4 + c] > b ? wbest[w * 4 + c] : b;
        __hip_atomic_fetch_max(keys + c, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (threadIdx.x == 0) {
        fence_release();
        const uint32_t old = __hip_atomic_fetch_add(gp(a.counter), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = (old + 1u == gridDim.x);
        if (last) fence_acquire();
    }
    __syncthreads();
    if (last && threadIdx.x < NC) {
        const unsigned long long k = __hip_atomic_load(keys + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        gp(a.argmax)[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
        __hip_atomic_store(keys + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) __hip_atomic_store(gp(a.counter), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int F, int NC, int H>
static hipError_t launch_lm_head_h(const LmHeadArgs& a, int grid, hipStream_t s) {
    const size_t shm = (size_t)NC * H * sizeof(float);
    hipLaunchKernelGGL((lm_head_kernel<F, NC, H>), dim3(grid), dim3(256), shm, s, a);
    return hipGetLastError();
}

template <int F, int NC>
static hipError_t launch_lm_head_nc(const LmHeadArgs& a, int grid, hipStream_t s) {
    switch (a.H) {
        case 256: return launch_lm_head_h<F, NC, 256>(a, grid, s);
        case 512: return launch_lm_head_h<F, NC, 512>(a, grid, s);
        case 1024: return launch_lm_head_h<F, NC, 1024>(a, grid, s);
        case 2048: return launch_lm_head_h<F, NC, 2048>(a, grid, s);
        case 2560: return launch_lm_head_h<F, NC, 2560>(a, grid, s);
        case 4096: return launch_lm_head_h<F, NC, 4096>(a, grid, s);
        case 8192: return launch_lm_head_h<F, NC, 8192>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

bool lm_head_hidden_supported(int H) {
    return H == 256 || H == 512 || H == 1024 || H == 2048 || H == 2560 || H == 4096 || H == 8192;
}

hipError_t launch_lm_head(const LmHeadArgs& a, int ncol, int fmt, int grid, hipStream_t s) {
    if (fmt == F_BF16) {
        switch (ncol) {
            case 1: return launch_lm_head_nc<F_BF16, 1>(a, grid, s);
            case 2: return launch_lm_head_nc<F_BF16, 2>(a, grid, s);
            case 3: return launch_lm_head_nc<F_BF16, 3>(a, grid, s);
            case 4: return launch_lm_head_nc<F_BF16, 4>(a, grid, s);
        }
    } else if (fmt == F_FP8) {
        switch (ncol) {
            case 1: return launch_lm_head_nc<F_FP8, 1>(a, grid, s);
            case 2: return launch_lm_head_nc<F_FP8, 2>(a, grid, s);
            case 3: return launch_lm_head_nc<F_FP8, 3>(a, grid, s);
            case 4: return launch_lm_head_nc<F_FP8, 4>(a, grid, s);
        }
    } else if (fmt == F_MXFP4) {
        switch (ncol) {
            case 1: return launch_lm_head_nc<F_MXFP4, 1>(a, grid, s);
            case 2: return launch_lm_head_nc<F_MXFP4, 2>(a, grid, s);
            case 3: return launch_lm_head_nc<F_MXFP4, 3>(a, grid, s);
            case 4: return launch_lm_head_nc<F_MXFP4, 4>(a, grid, s);
        }
    }
    return hipErrorInvalidValue;
}

// ------------------------------------------- LM head without allocation
//
// The argmax keys (k <= 4 of 8 bytes at offset 0) and the arrival counter
// (offset 64) of the LM head live in this fixed device array instead of a
// caller workspace, for callers that cannot allocate device memory.  Each
// GPU holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: its device address
// comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kLmScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t lm_head_scratch(hipStream_t s, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        // keys and counter start at zero; every call leaves them at zero
        e = launch_fill_u32(static_cast<uint32_t*>(p), kLmScratchBytes / 4, 0u, s);
        if (e != hipSuccess) return e;
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// ------------------------------------------------- FP8 row quantisation

// One workgroup per row: amax over the row (exact), scale = amax / 448 in
// binary32 (1 for a zero row), codes = E4M3FN(w / scale).
__global__ void __launch_bounds__(256) quantize_fp8_rows_kernel(const uint16_t* __restrict__ w, int64_t cols,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const uint16_t* row = w + r * cols;
    float m = 0.f;
    for (int64_t i = threadIdx.x; i < cols; i += blockDim.x) m = fmaxf(m, fabsf(bf16_to_f32(row[i])));
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
    if (threadIdx.x == 0) scales[r] = scale;
    uint8_t* crow = codes + r * cols;
    for (int64_t i = threadIdx.x; i < cols; i += blockDim.x) crow[i] = f32_to_fp8e4m3(bf16_to_f32(row[i]) / scale);
}

hipError_t launch_quantize_fp8_rows(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* codes, float* scales,
                                    hipStream_t s) {
    hipLaunchKernelGGL(quantize_fp8_rows_kernel, dim3((unsigned)rows), dim3(256), 0, s, w, cols, codes, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------- KV write

__global__ void __launch_bounds__(256) kv_write_kernel(KvWriteArgs a) {
    const int64_t per_pos = (int64_t)a.n_kv_heads * a.head_dim;
    const int64_t total = (int64_t)a.n * per_pos * 2;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int kv = (int)(idx / ((int64_t)a.n * per_pos));
        const int64_t rem = idx - (int64_t)kv * a.n * per_pos;
        const int t = (int)(rem / per_pos);
        const int64_t hd = rem - (int64_t)t * per_pos;
        const int g = (int)(hd / a.head_dim);
        const int e = (int)(hd - (int64_t)g * a.head_dim);
        const int pos = a.pos0 + t;
        const int page = a.page_table[pos / a.page_size];
        const int slot = pos % a.page_size;
        const int64_t off = a.layer_off +
                            ((((int64_t)page * 2 + kv) * a.n_kv_heads + g) * a.page_size + slot) * a.head_dim + e;
        const float v = (kv == 0 ? a.k : a.v)[rem];
        if (a.dtype == F_BF16) {
            reinterpret_cast<uint16_t*>(a.pool)[off] = f32_to_bf16(v);
        } else {
            const float sc = a.scales[(a.layer * a.n_kv_heads + g) * 2 + kv];
            reinterpret_cast<uint8_t*>(a.pool)[off] = f32_to_fp8e4m3(v / sc);
        }
    }
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t s) {
    const int64_t total = (int64_t)a.n * a.n_kv_heads * a.head_dim * 2;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ------------------------------------------------------------ RoPE table

// cs[p][i] = (cos, sin)(p * inv_freq[i]) for every position p < max_pos:
// the angle and its cosine and sine in double precision, rounded once to
// binary32.  Built at init, so a step only loads the pair it needs.
__global__ void rope_table_kernel(const double* __restrict__ inv_freq, int half, int64_t n, float2* __restrict__ cs) {
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = idx / half;
        const int i = (int)(idx - p * half);
        double sd, cd;
        sincos((double)p * inv_freq[i], &sd, &cd);
        cs[idx] = make_float2((float)cd, (float)sd);
    }
}

hipError_t launch_rope_table(const double* inv_freq, int half, int64_t max_pos, float2* cs, hipStream_t s) {
    const int64_t n = max_pos * half;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s, inv_freq, half, n, cs);
    return hipGetLastError();
}

// ---------------------------------------------------------------- fill

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace mbg
