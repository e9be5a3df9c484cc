// C-ABI of the decode library: validation, workspace plan, static task list,
// one cooperative launch per decode step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "mbg.h"
#include "layout.h"
#include "ops.h"

using namespace mbg;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MBG_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(call)                                   \
    do {                                                \
        hipError_t e_ = (call);                         \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

constexpr int kMaxGrid = 1024;   // workgroups of the persistent kernel (upper bound)
constexpr int kMaxStepsPerLaunch = 4096;   // greedy steps one mbg_decode_steps launch may run
constexpr int kMaxSplits = 64;   // split-KV partitions per KV head (upper bound)
constexpr int kBlock = 256;
constexpr int kAttnBufsHost = 4;   // attention ring chunks per wave (step.hip)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace sections, in bytes from the base.
struct Plan {
    size_t keys, head_ctr, task_off, tasks, layers, inv_freq, rope_cs;
    size_t xres, qbuf, part, attn, hbuf, rlogits, route_w, route_idx, trace, total;
    int64_t hb_ld, part_layer;
    size_t n_ctr, max_tasks, zero_bytes;
    size_t uc_bytes;   // caller's uncached counter block: status, LM-head counter, flags, dependency counters
};

// The counter block: one 128-byte line for the status word (word 0), the
// LM-head counter (word 1) and the flag word (word 2), then the dependency
// counters.
constexpr size_t kUcCtrOffset = 128;

Plan make_plan(const mbg_config& c) {
    Plan p{};
    const size_t k = (size_t)c.k_max;
    const size_t L = (size_t)c.n_layers;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    p.keys = take(8 * 4);
    p.n_ctr = L * PH_COUNT + 1;   // the per-(layer, phase) counters and the step-token counter
    p.uc_bytes = kUcCtrOffset + 4 * kLineU32 * kCtrLines * p.n_ctr;
    p.head_ctr = take(4 * kLineU32 * L * (size_t)c.n_q_heads);   // one line per (layer, KV head, head group)
    p.zero_bytes = off;  // everything above starts at zero
    p.task_off = take(4 * (kMaxGrid + 1));
    p.max_tasks = (size_t)kMaxGrid * (8 * L + 1);
    p.tasks = take(sizeof(Task) * p.max_tasks);
    p.layers = take(sizeof(LayerPtrs) * L);
    p.inv_freq = take(8 * (size_t)(c.head_dim / 2));
    p.rope_cs = take(8 * (size_t)c.max_pos * (c.head_dim / 2));
    p.xres = take(4 * k * c.hidden);
    p.qbuf = take(4 * k * (size_t)c.n_q_heads * c.head_dim);
    p.part_layer = (int64_t)k * c.n_q_heads * kMaxSplits * (c.head_dim + 4);   // rows: o, m, l, 2 pad
    p.part = take(4 * L * (size_t)p.part_layer);
    p.attn = take(4 * k * (size_t)c.n_q_heads * c.head_dim);
    // MoE: a window of k tokens uses at most k * top_k routed experts plus the shared ones
    p.hb_ld = c.n_experts > 0 ? (int64_t)(k * c.top_k + c.n_shared) * c.moe_ffn : c.ffn;
    p.hbuf = take(4 * k * (size_t)p.hb_ld);
    p.rlogits = take(4 * k * (size_t)(c.n_experts > 0 ? c.n_experts : 1));
    const size_t nroute = L * k * (size_t)(c.top_k > 0 ? c.top_k : 1);
    p.route_w = take(4 * nroute);
    p.route_idx = take(4 * nroute);
    p.trace = take(64 * p.max_tasks);
    p.total = off;
    return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_tensor(const mbg_tensor& t, const char* name, int dtype, int64_t n, int64_t rows, int64_t cols) {
    if (t.data == nullptr) return fail(MBG_E_INVALID_ARG, "%s: data is NULL", name);
    if (t.dtype != dtype)
        return fail(MBG_E_DTYPE_MISMATCH, "%s: dtype %d, expected %d", name, t.dtype, dtype);
    if (t.n != n || t.rows != rows || t.cols != cols)
        return fail(MBG_E_INVALID_ARG, "%s: shape [%d][%lld][%lld], expected [%lld][%lld][%lld]", name, t.n,
                    (long long)t.rows, (long long)t.cols, (long long)n, (long long)rows, (long long)cols);
    if (!aligned16(t.data)) return fail(MBG_E_INVALID_ARG, "%s: data not 16-byte aligned", name);
    const bool needs_scale = dtype == MBG_FP8_E4M3 || dtype == MBG_MXFP4;
    if (needs_scale && t.scale == nullptr) return fail(MBG_E_DTYPE_MISMATCH, "%s: scale missing", name);
    if (!needs_scale && t.scale != nullptr)
        return fail(MBG_E_DTYPE_MISMATCH, "%s: scale given for a dtype without one", name);
    return MBG_OK;
}

int check_config(const mbg_config* c) {
    if (!c) return fail(MBG_E_INVALID_ARG, "config is NULL");
    if (c->n_layers < 1 || c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->vocab <= 0)
        return fail(MBG_E_INVALID_ARG, "config: non-positive dimension");
    if (c->hidden % 32 != 0) return fail(MBG_E_UNSUPPORTED, "config: hidden %d not a multiple of 32", c->hidden);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(MBG_E_UNSUPPORTED, "config: head_dim %d (64 or 128 supported)", c->head_dim);
    if (c->n_q_heads % c->n_kv_heads != 0)
        return fail(MBG_E_INVALID_ARG, "config: n_q_heads %d not a multiple of n_kv_heads %d", c->n_q_heads,
                    c->n_kv_heads);
    if (c->n_experts < 0 || c->top_k < 0 || c->n_shared < 0 || c->moe_ffn < 0 || c->ffn < 0)
        return fail(MBG_E_INVALID_ARG, "config: negative size");
    if (c->n_experts == 0) {
        if (c->ffn <= 0 || c->ffn % 8 != 0)
            return fail(MBG_E_UNSUPPORTED, "config: ffn %d must be a positive multiple of 8", c->ffn);
    } else {
        if (c->top_k < 1 || c->top_k > kMaxTopK || c->top_k > c->n_experts)
            return fail(MBG_E_UNSUPPORTED, "config: top_k %d (1..%d, <= n_experts)", c->top_k, kMaxTopK);
        if (c->n_experts > kMaxExperts || c->n_experts % 8 != 0)
            return fail(MBG_E_UNSUPPORTED, "config: n_experts %d (a multiple of 8, <= %d)", c->n_experts,
                        kMaxExperts);
        if (c->n_shared > kMaxShared)
            return fail(MBG_E_UNSUPPORTED, "config: n_shared %d (<= %d)", c->n_shared, kMaxShared);
        if (c->k_max * c->top_k + c->n_shared > kMaxSlots)
            return fail(MBG_E_UNSUPPORTED, "config: k_max %d x top_k %d + shared %d experts per window > %d",
                        c->k_max, c->top_k, c->n_shared, kMaxSlots);
        if (c->moe_ffn <= 0 || c->moe_ffn % 32 != 0)
            return fail(MBG_E_UNSUPPORTED, "config: moe_ffn %d must be a positive multiple of 32", c->moe_ffn);
    }
    if (c->page_size <= 0 || c->max_pos <= 0) return fail(MBG_E_INVALID_ARG, "config: page_size/max_pos");
    // an attention instruction reads up to 16 consecutive positions from one
    // page, and the kernels index pages by shifts
    if (c->page_size < 16 || (c->page_size & (c->page_size - 1)) != 0)
        return fail(MBG_E_UNSUPPORTED, "config: page_size %d (a power of two, >= 16)", c->page_size);
    if (c->k_max < 1 || c->k_max > 4) return fail(MBG_E_UNSUPPORTED, "config: k_max %d (1..4)", c->k_max);
    if (c->layer_window)
        for (int l = 0; l < c->n_layers; ++l)
            if (c->layer_window[l] < 0) return fail(MBG_E_INVALID_ARG, "config: layer_window[%d] = %d", l, c->layer_window[l]);
    if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(MBG_E_INVALID_ARG, "config: rope_theta/rms_eps");
    return MBG_OK;
}

StepVariant variant_of(const mbg_config* c, int kv_dtype) {
    StepVariant v;
    v.hidden = c->hidden;
    v.ffn = c->n_experts > 0 ? 0 : c->ffn;
    v.qdim = c->n_q_heads * c->head_dim;
    v.moe_ffn = c->n_experts > 0 ? c->moe_ffn : 0;
    v.head_dim = c->head_dim;
    v.group = c->n_q_heads / c->n_kv_heads;
    v.kv_fmt = kv_dtype == MBG_FP8_E4M3 ? 2 : 1;
    v.moe = c->n_experts > 0 ? 1 : 0;
    return v;
}

}  // namespace

namespace mbg {
const void* step_kernel_for(const StepVariant& v, int ncol, int* lds_bytes_out) {
    using Fn = const void* (*)(const StepVariant&, int, int*);
    static const Fn fns[kStepShapes] = {step_kernel_shape_0, step_kernel_shape_1, step_kernel_shape_2,
                                        step_kernel_shape_3};
    for (Fn f : fns)
        if (const void* k = f(v, ncol, lds_bytes_out)) return k;
    return nullptr;
}
bool step_variant_supported(const StepVariant& v) { return step_kernel_for(v, 1, nullptr) != nullptr; }
}  // namespace mbg

namespace {

int device_cus(int* cus) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev));
    return MBG_OK;
}

}  // namespace

struct mbg_ctx {
    mbg_config cfg;
    StepArgs base;
    hipStream_t stream;
    int grid;
    int lds[5];
    const void* fn[5];
    uint32_t epoch;
    int64_t wall_khz;
    int64_t timeout_us;
    int64_t weight_bytes;
    size_t ws_bytes;
    int lm_dtype, kv_dtype;
    int n_tasks;
    int trace_on;
    int last_ncol;   // columns of the last step/verify call (0: none yet)
    int n_seqs;      // page-table rows (sequences)
    void* uc;        // the caller's uncached counter block
    size_t uc_bytes;
    void* ws_zero;   // start of the workspace region that starts at zero (argmax keys, head counters)
    size_t ws_zero_bytes;
    unsigned long long* trace_buf;
    char variant[64];
};

extern "C" {

const char* mbg_last_error(void) { return g_err.c_str(); }

int mbg_workspace_size(const mbg_config* cfg, size_t* bytes) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!bytes) return fail(MBG_E_INVALID_ARG, "bytes is NULL");
    *bytes = make_plan(*cfg).total;
    return MBG_OK;
}

int mbg_counter_bytes(const mbg_config* cfg, size_t* bytes) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!bytes) return fail(MBG_E_INVALID_ARG, "bytes is NULL");
    *bytes = make_plan(*cfg).uc_bytes;
    return MBG_OK;
}

int mbg_validate(const mbg_config* c, const mbg_weights* w, const mbg_kv* kv) {
    int rc = check_config(c);
    if (rc) return rc;
    const int64_t H = c->hidden, d = c->head_dim, Hq = c->n_q_heads, Hkv = c->n_kv_heads;
    if (kv) {
        if (kv->dtype != MBG_BF16 && kv->dtype != MBG_FP8_E4M3)
            return fail(MBG_E_UNSUPPORTED, "kv: dtype %d (BF16 or FP8 E4M3)", kv->dtype);
        if (!kv->pool || !kv->page_table) return fail(MBG_E_INVALID_ARG, "kv: pool/page_table is NULL");
        if (kv->n_pages <= 0) return fail(MBG_E_INVALID_ARG, "kv: n_pages %d", kv->n_pages);
        if (kv->n_seqs < 0) return fail(MBG_E_INVALID_ARG, "kv: n_seqs %d", kv->n_seqs);
        if (kv->dtype == MBG_FP8_E4M3 && !kv->scales)
            return fail(MBG_E_DTYPE_MISMATCH, "kv: FP8 cache without per-head scales");
        if (kv->dtype == MBG_BF16 && kv->scales)
            return fail(MBG_E_DTYPE_MISMATCH, "kv: BF16 cache given scales");
        if (!aligned16(kv->pool)) return fail(MBG_E_INVALID_ARG, "kv: pool not 16-byte aligned");
        if (!step_variant_supported(variant_of(c, kv->dtype)))
            return fail(MBG_E_UNSUPPORTED,
                        "no compiled kernel for hidden %d, ffn %d, %d x %d query heads, %d per KV head, %s KV, %s",
                        c->hidden, c->n_experts ? c->moe_ffn : c->ffn, c->n_q_heads, c->head_dim, (int)(Hq / Hkv),
                        kv->dtype == MBG_BF16 ? "BF16" : "FP8", c->n_experts ? "MoE" : "dense");
    }
    if (!w) return MBG_OK;
    if (!w->layers) return fail(MBG_E_INVALID_ARG, "weights: layers is NULL");
    if ((rc = check_tensor(w->embed, "embed", MBG_BF16, 1, c->vocab, H))) return rc;
    if ((rc = check_tensor(w->final_norm, "final_norm", MBG_BF16, 1, 1, H))) return rc;
    if (w->lm_head.dtype != MBG_BF16 && w->lm_head.dtype != MBG_FP8_E4M3)
        return fail(MBG_E_UNSUPPORTED, "lm_head: dtype %d (BF16 or FP8 E4M3)", w->lm_head.dtype);
    if ((rc = check_tensor(w->lm_head, "lm_head", w->lm_head.dtype, 1, c->vocab, H))) return rc;
    char nm[64];
    for (int l = 0; l < c->n_layers; ++l) {
        const mbg_layer& L = w->layers[l];
#define CHK(field, dt, n, r, cc)                                   \
    snprintf(nm, sizeof nm, "layers[%d]." #field, l);              \
    if ((rc = check_tensor(L.field, nm, dt, n, r, cc))) return rc;
        CHK(attn_norm, MBG_BF16, 1, 1, H)
        CHK(ffn_norm, MBG_BF16, 1, 1, H)
        CHK(wq, MBG_BF16, 1, Hq * d, H)
        CHK(wk, MBG_BF16, 1, Hkv * d, H)
        CHK(wv, MBG_BF16, 1, Hkv * d, H)
        CHK(wo, MBG_BF16, 1, H, Hq * d)
        if (c->n_experts == 0) {
            CHK(w_gate, MBG_BF16, 1, c->ffn, H)
            CHK(w_up, MBG_BF16, 1, c->ffn, H)
            CHK(w_down, MBG_BF16, 1, H, c->ffn)
        } else {
            CHK(w_router, MBG_BF16, 1, c->n_experts, H)
            CHK(exp_gate_up, MBG_MXFP4, c->n_experts, 2 * (int64_t)c->moe_ffn, H)
            CHK(exp_down, MBG_MXFP4, c->n_experts, H, c->moe_ffn)
            if (c->n_shared > 0) {
                CHK(sh_gate_up, MBG_MXFP4, c->n_shared, 2 * (int64_t)c->moe_ffn, H)
                CHK(sh_down, MBG_MXFP4, c->n_shared, H, c->moe_ffn)
            }
        }
#undef CHK
    }
    return MBG_OK;
}

int mbg_decode_init(const mbg_config* cfg, const mbg_weights* w, const mbg_kv* kv, void* d_ws, size_t ws_bytes,
                    void* d_counters, size_t counter_bytes, void* stream, mbg_ctx** out) {
    if (!out) return fail(MBG_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!w || !kv) return fail(MBG_E_INVALID_ARG, "weights and kv are required");
    int rc = mbg_validate(cfg, w, kv);
    if (rc) return rc;
    const mbg_config& c = *cfg;
    const Plan plan = make_plan(c);
    if (!d_ws || ws_bytes < plan.total)
        return fail(MBG_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, plan.total);
    if (((uintptr_t)d_ws & 255u) != 0) return fail(MBG_E_WORKSPACE, "workspace not 256-byte aligned");
    if (!d_counters || counter_bytes < plan.uc_bytes)
        return fail(MBG_E_WORKSPACE, "counter block %zu bytes, need %zu", counter_bytes, plan.uc_bytes);
    if (((uintptr_t)d_counters & 255u) != 0) return fail(MBG_E_WORKSPACE, "counter block not 256-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    int cus = 0;
    if ((rc = device_cus(&cus))) return rc;
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    int wall_khz = 0;
    HIP_TRY(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev));
    int coop = 0;
    HIP_TRY(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
    if (!coop) return fail(MBG_E_UNSUPPORTED, "device does not support cooperative launches");

    // page table entries (every sequence's row) must address the pool
    const int n_lpages = (c.max_pos + c.page_size - 1) / c.page_size;
    const int n_seqs = std::max(1, (int)kv->n_seqs);
    {
        std::vector<int32_t> pt((size_t)n_seqs * n_lpages);
        HIP_TRY(hipMemcpy(pt.data(), kv->page_table, sizeof(int32_t) * pt.size(), hipMemcpyDeviceToHost));
        for (size_t i = 0; i < pt.size(); ++i)
            if (pt[i] < 0 || pt[i] >= kv->n_pages)
                return fail(MBG_E_RANGE, "page_table[%zu] = %d outside [0, %d)", i, pt[i], kv->n_pages);
    }

    mbg_ctx* x = new mbg_ctx();
    x->cfg = c;
    x->cfg.layer_window = nullptr;   // the caller's array is read during init only
    x->stream = s;
    x->epoch = 0;
    x->wall_khz = wall_khz;
    x->timeout_us = 2000000;
    x->ws_bytes = ws_bytes;
    x->lm_dtype = w->lm_head.dtype;
    x->kv_dtype = kv->dtype;
    const StepVariant v = variant_of(&c, kv->dtype);
    snprintf(x->variant, sizeof x->variant, "step_d%d_g%d_%s_%s", v.head_dim, v.group,
             v.kv_fmt == 1 ? "bf16kv" : "fp8kv", v.moe ? "moe" : "dense");

    StepArgs& a = x->base;
    memset(&a, 0, sizeof a);
    a.n_layers = c.n_layers;
    a.hidden = c.hidden;
    a.n_q_heads = c.n_q_heads;
    a.n_kv_heads = c.n_kv_heads;
    a.head_dim = c.head_dim;
    a.ffn = c.ffn;
    a.vocab = c.vocab;
    a.n_experts = c.n_experts;
    a.top_k = c.top_k;
    a.n_shared = c.n_shared;
    a.moe_ffn = c.moe_ffn;
    a.rms_eps = c.rms_eps;
    a.attn_scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
    a.page_size = c.page_size;
    a.page_shift = __builtin_ctz((unsigned)c.page_size);
    a.max_pos = c.max_pos;

    // kernels, LDS, occupancy -> grid
    int wg_per_cu = 1;   // one 4-wave workgroup per CU (the kernel uses every register of a SIMD)
    for (int k = 1; k <= c.k_max; ++k) {
        x->fn[k] = step_kernel_for(v, k, &x->lds[k]);
        if (!x->fn[k]) {
            delete x;
            return fail(MBG_E_UNSUPPORTED, "no kernel for %d columns", k);
        }
        hipError_t e = hipFuncSetAttribute(x->fn[k], hipFuncAttributeMaxDynamicSharedMemorySize, x->lds[k]);
        if (e != hipSuccess) {
            delete x;
            return hip_fail(e, "hipFuncSetAttribute");
        }
        int nb = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, x->fn[k], kBlock, x->lds[k]);
        if (e != hipSuccess) {
            delete x;
            return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
        }
        if (nb < 1) {
            delete x;
            return fail(MBG_E_UNSUPPORTED, "step kernel (%d columns) cannot be resident", k);
        }
        if (nb < wg_per_cu) wg_per_cu = nb;
    }
    int G = cus * wg_per_cu;
    if (G > kMaxGrid) G = kMaxGrid;
    x->grid = G;

    auto cdiv = [](int64_t n, int64_t d) { return (n + d - 1) / d; };
    auto tiles_for = [&](int64_t units) { return (uint32_t)std::min<int64_t>(G, cdiv(units, 4)); };
    const int HALF = c.head_dim / 2;
    const int64_t npairs = (int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * HALF;
    a.tiles_qkv = tiles_for(npairs);
    if (2 * cdiv(npairs, (int64_t)a.tiles_qkv * 4) > 64) {
        delete x;
        return fail(MBG_E_UNSUPPORTED, "%lld Q/K/V rows exceed the per-wavefront buffer", (long long)(2 * npairs));
    }
    a.tiles_o = tiles_for(c.hidden);
    a.tiles_gu = tiles_for(c.ffn);
    a.tiles_down = tiles_for(c.hidden);
    a.tiles_lm = tiles_for(c.vocab);
    const bool moe = c.n_experts > 0;
    if (moe) {
        a.tiles_router = tiles_for(c.n_experts);
        a.tiles_egu = (uint32_t)G;
        a.tiles_edown = tiles_for(c.hidden);
        if (cdiv(c.hidden, (int64_t)a.tiles_edown * 4) > kMaxDownRows) {
            delete x;
            return fail(MBG_E_UNSUPPORTED, "hidden %d: more than %d expert-down rows per wavefront", c.hidden,
                        kMaxDownRows);
        }
    }
    const uint32_t tiles_last = moe ? a.tiles_edown : a.tiles_down;   // producers of the residual update
    // attention tasks: (KV head, head group of at most kAttnHeadsPerTask
    // query heads, split); the splits fill the grid
    const int gq = c.n_q_heads / c.n_kv_heads;
    const int head_groups = gq / std::min(gq, kAttnHeadsPerTask);
    int S = G / (c.n_kv_heads * head_groups);
    S = std::max(1, std::min(S, kMaxSplits));
    // at least ~176 positions per split: fewer, longer splits than the grid
    // allows shorten the combine, which every layer waits for, and measured
    // best on the dense and routed steps (11 workgroup token slots; 128
    // positions per split or ~40 % more than 176 were slower)
    S = std::min<int>(S, (int)std::max<int64_t>(1, cdiv(c.max_pos, 176)));
    if (S > 4) S -= S % 4;   // whole groups of four splits (the XCD-local placement needs them)
    a.attn_splits = S;
    // prefetch defaults chosen by measurement on the dense 2B step; the
    // environment overrides documented at mbg_decode_init replace them
    a.gemv_pre = 16;
    a.gu_pre = 24;     // dense gate/up and down: deeper than the other phases
    a.down_pre = 32;   // (same-box A/B: +0.9 % on the dense step; 32 for gate/up was slower)
    a.attn_pre = kAttnBufsHost;
    a.poll_wave_prefetch = 1;
    a.wave0_input = 1;
    if (const char* e = getenv("MBG_GEMV_PREFETCH")) a.gemv_pre = std::max(0, std::min(64, atoi(e)));
    if (const char* e = getenv("MBG_GU_PREFETCH")) a.gu_pre = std::max(0, std::min(64, atoi(e)));
    if (const char* e = getenv("MBG_DOWN_PREFETCH")) a.down_pre = std::max(0, std::min(64, atoi(e)));
    if (const char* e = getenv("MBG_ATTN_PREFETCH")) a.attn_pre = std::max(0, std::min(kAttnBufsHost, atoi(e)));
    const uint32_t tiles_attn = (uint32_t)(c.n_kv_heads * head_groups * S);
    // Attention placement: workgroup b runs on XCD b % 8 (the dispatcher
    // deals workgroups round-robin over the 8 XCDs; the kernel checks it).
    // When every group's splits fit on one XCD, XCD x takes the NG / 8
    // consecutive groups x NG / 8 .. (x + 1) NG / 8 - 1: their splits
    // exchange partials and arrivals through that XCD's L2 instead of
    // device-coherent memory, and head groups of one KV head (consecutive
    // group numbers) share the XCD, whose L2 then serves their common
    // history after the first read.  Each group's block of partial rows
    // must then be whole 128-byte lines: (heads per task x splits) % 8 == 0.
    // The kernels for BF16 caches carry this path (the FP8-cache kernels,
    // meant for long contexts, are built without it).  Long contexts keep
    // the default placement: one XCD reading every page
    // of a KV head misses its address translation caches far more often
    // than eight XCDs reading an eighth of the pages each (measured slower
    // at 200,000 positions), and there the combine is a small share.
    const int NG = c.n_kv_heads * head_groups;
    const int gh_task = gq / head_groups;
    a.attn_local = (kv->dtype == MBG_BF16 && G % 8 == 0 && NG % 8 == 0 && (NG / 8) * S <= G / 8 &&
                    (gh_task * S) % 8 == 0 && (int64_t)c.max_pos <= (int64_t)kAttnLocalMaxSplitLen * S)
                       ? 1
                       : 0;
    if (const char* e = getenv("MBG_ATTN_LOCAL")) a.attn_local = a.attn_local && atoi(e) != 0;
    auto attn_tile_of = [&](int wg) -> int {   // the attention tile workgroup wg runs, or -1
        if (!a.attn_local) return wg < (int)tiles_attn ? wg : -1;
        const int x = wg % 8, slot = wg / 8;
        if (slot >= (NG / 8) * S) return -1;
        return (x * (NG / 8) + slot / S) * S + slot % S;
    };

    // task lists
    std::vector<uint32_t> off(G + 1, 0);
    std::vector<Task> tasks;
    auto ci = [](int l, int ph) { return (uint32_t)(l * PH_COUNT + ph); };
    for (int wg = 0; wg < G; ++wg) {
        off[wg] = (uint32_t)tasks.size();
        const uint32_t t = (uint32_t)wg;
        for (int l = 0; l < c.n_layers; ++l) {
            const uint32_t L8 = (uint32_t)l << 8;
            if (t < a.tiles_qkv)
                tasks.push_back(Task{OP_QKV | L8, t, l == 0 ? kNoWait : ci(l - 1, PH_DOWN), l == 0 ? 0u : tiles_last});
            if (attn_tile_of(wg) >= 0)
                tasks.push_back(Task{OP_ATTN | L8, (uint32_t)attn_tile_of(wg), ci(l, PH_QKV), a.tiles_qkv});
            if (t < a.tiles_o)
                tasks.push_back(Task{OP_OPROJ | L8, t, ci(l, PH_ATTN), (uint32_t)(c.n_kv_heads * head_groups)});
            if (!moe) {
                if (t < a.tiles_gu) tasks.push_back(Task{OP_GATEUP | L8, t, ci(l, PH_OPROJ), a.tiles_o});
                if (t < a.tiles_down) tasks.push_back(Task{OP_DOWN | L8, t, ci(l, PH_GATEUP), a.tiles_gu});
            } else {
                if (t < a.tiles_router) tasks.push_back(Task{OP_ROUTER | L8, t, ci(l, PH_OPROJ), a.tiles_o});
                if (t < a.tiles_egu) tasks.push_back(Task{OP_EXPGU | L8, t, ci(l, PH_ROUTER), a.tiles_router});
                if (t < a.tiles_edown) tasks.push_back(Task{OP_EXPDOWN | L8, t, ci(l, PH_GATEUP), a.tiles_egu});
            }
        }
        if (t < a.tiles_lm)
            tasks.push_back(Task{OP_LMHEAD, t, ci(c.n_layers - 1, PH_DOWN), tiles_last});
    }
    off[G] = (uint32_t)tasks.size();
    if (tasks.size() > plan.max_tasks) {
        delete x;
        return fail(MBG_E_WORKSPACE, "task list %zu exceeds plan %zu", tasks.size(), plan.max_tasks);
    }
    x->n_tasks = (int)tasks.size();

    std::vector<LayerPtrs> lp(c.n_layers);
    int64_t per_step = 0;
    for (int l = 0; l < c.n_layers; ++l) {
        const mbg_layer& L = w->layers[l];
        LayerPtrs& p = lp[l];
        memset(&p, 0, sizeof p);
        p.attn_norm = (const uint16_t*)L.attn_norm.data;
        p.ffn_norm = (const uint16_t*)L.ffn_norm.data;
        p.wq = (const uint16_t*)L.wq.data;
        p.wk = (const uint16_t*)L.wk.data;
        p.wv = (const uint16_t*)L.wv.data;
        p.wo = (const uint16_t*)L.wo.data;
        p.w_gate = (const uint16_t*)L.w_gate.data;
        p.w_up = (const uint16_t*)L.w_up.data;
        p.w_down = (const uint16_t*)L.w_down.data;
        p.w_router = (const uint16_t*)L.w_router.data;
        p.eg_codes = (const uint8_t*)L.exp_gate_up.data;
        p.eg_scales = (const uint8_t*)L.exp_gate_up.scale;
        p.ed_codes = (const uint8_t*)L.exp_down.data;
        p.ed_scales = (const uint8_t*)L.exp_down.scale;
        p.sg_codes = (const uint8_t*)L.sh_gate_up.data;
        p.sg_scales = (const uint8_t*)L.sh_gate_up.scale;
        p.sd_codes = (const uint8_t*)L.sh_down.data;
        p.sd_scales = (const uint8_t*)L.sh_down.scale;
        p.window = c.layer_window ? c.layer_window[l] : 0;
        per_step += 2 * ((int64_t)c.hidden * 2 + (int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim * c.hidden +
                         (int64_t)c.hidden * c.n_q_heads * c.head_dim + 3 * (int64_t)c.ffn * c.hidden);
        if (moe) {  // router plus the top_k + shared experts a single token reads (codes and E8M0 scales)
            const int64_t expert = 3 * (int64_t)c.moe_ffn * c.hidden * 17 / 32;
            per_step += 2 * (int64_t)c.n_experts * c.hidden + (int64_t)(c.top_k + c.n_shared) * expert;
        }
    }
    per_step += 2 * (int64_t)c.hidden * 2;  // embedding row + final norm
    per_step += (int64_t)c.vocab * c.hidden * (x->lm_dtype == MBG_FP8_E4M3 ? 1 : 2) +
                (x->lm_dtype == MBG_FP8_E4M3 ? 4 * (int64_t)c.vocab : 0);
    x->weight_bytes = per_step;

    std::vector<double> inv(HALF);
    for (int i = 0; i < HALF; ++i) inv[i] = std::pow((double)c.rope_theta, -2.0 * i / c.head_dim);

    char* base = static_cast<char*>(d_ws);
    void* uc = d_counters;
    x->uc = uc;
    x->uc_bytes = plan.uc_bytes;
    x->ws_zero = base;
    x->ws_zero_bytes = plan.zero_bytes;
    a.status = (uint32_t*)uc;
    a.lm_ctr = a.status + 1;
    a.flags = a.status + 2;
    a.amax_keys = (unsigned long long*)(base + plan.keys);
    a.ctr = (uint32_t*)((char*)uc + kUcCtrOffset);
    a.head_ctr = (uint32_t*)(base + plan.head_ctr);
    a.task_off = (const uint32_t*)(base + plan.task_off);
    a.tasks = (const Task*)(base + plan.tasks);
    a.layers = (const LayerPtrs*)(base + plan.layers);
    a.inv_freq = (const double*)(base + plan.inv_freq);
    a.rope_cs = (const float2*)(base + plan.rope_cs);
    a.xres = (float*)(base + plan.xres);
    a.qbuf = (float*)(base + plan.qbuf);
    a.part = (float*)(base + plan.part);
    a.part_layer = plan.part_layer;
    a.attn = (float*)(base + plan.attn);
    a.hbuf = (float*)(base + plan.hbuf);
    a.hb_ld = (int32_t)plan.hb_ld;
    a.rlogits = (float*)(base + plan.rlogits);
    a.route_w = (float*)(base + plan.route_w);
    a.route_idx = (int32_t*)(base + plan.route_idx);
    x->trace_buf = (unsigned long long*)(base + plan.trace);
    x->trace_on = 0;
    a.trace = nullptr;
    a.embed = (const uint16_t*)w->embed.data;
    a.final_norm = (const uint16_t*)w->final_norm.data;
    a.lm_head = w->lm_head.data;
    a.lm_scale = (const float*)w->lm_head.scale;
    a.lm_dtype = w->lm_head.dtype == MBG_FP8_E4M3 ? 2 : 1;
    a.kv_dtype = kv->dtype == MBG_FP8_E4M3 ? 2 : 1;
    a.kv_pool = kv->pool;
    a.page_table = kv->page_table;
    a.kv_scales = kv->scales;
    a.kv_layer_stride = (int64_t)kv->n_pages * 2 * c.n_kv_heads * c.page_size * c.head_dim;
    a.pt_stride = n_lpages;
    a.batch = 0;
    x->n_seqs = n_seqs;

    hipError_t e = launch_fill_u32((uint32_t*)base, plan.zero_bytes / 4, 0u, s);
    if (e == hipSuccess) e = launch_fill_u32((uint32_t*)uc, plan.uc_bytes / 4, 0u, s);
    if (e == hipSuccess) e = hipMemcpyAsync(base + plan.task_off, off.data(), 4 * off.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(base + plan.tasks, tasks.data(), sizeof(Task) * tasks.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(base + plan.layers, lp.data(), sizeof(LayerPtrs) * lp.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(base + plan.inv_freq, inv.data(), 8 * inv.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = launch_rope_table((const double*)(base + plan.inv_freq), HALF, c.max_pos, (float2*)(base + plan.rope_cs), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete x;
        return hip_fail(e, "workspace upload");
    }
    *out = x;
    return MBG_OK;
}

// Columns of a batch of independent sequences (mbg_decode_batch).
struct BatchCols {
    int n = 0;
    int32_t seq[4] = {0, 0, 0, 0};
    int32_t pos[4] = {0, 0, 0, 0};
};

// A speculative round's launch: position on the device, acceptance outputs.
struct SpecLaunch {
    const int32_t* dpos = nullptr;
    const int32_t* cur = nullptr;
    int32_t* next = nullptr;
    int32_t* emit = nullptr;
    int32_t cap = 0;
};

static int launch_step(mbg_ctx* x, const int32_t* d_tokens, int32_t k, int32_t pos, float* d_logits,
                       int32_t* d_argmax, int32_t nsteps = 1, const BatchCols* batch = nullptr,
                       const SpecLaunch* spec = nullptr) {
    if (!x) return fail(MBG_E_INVALID_ARG, "ctx is NULL");
    if (!d_tokens || !d_argmax) return fail(MBG_E_INVALID_ARG, "tokens/argmax is NULL");
    if (k < 1 || k > x->cfg.k_max) return fail(MBG_E_RANGE, "k %d outside [1, %d]", k, x->cfg.k_max);
    if (nsteps < 1 || nsteps > kMaxStepsPerLaunch)
        return fail(MBG_E_RANGE, "n_steps %d outside [1, %d]", nsteps, kMaxStepsPerLaunch);
    // a batch's positions were checked per column; a device-resident
    // position is checked by the kernel
    const int64_t span = batch ? 1 : (int64_t)k + nsteps - 1;
    if (spec) pos = 0;
    if (pos < 0 || (int64_t)pos + span > x->cfg.max_pos)
        return fail(MBG_E_RANGE, "positions %d..%lld outside [0, %d)", pos, (long long)(pos + span - 1),
                    x->cfg.max_pos);
    StepArgs a = x->base;
    a.tokens = d_tokens;
    a.logits = d_logits;
    a.argmax = d_argmax;
    a.pos = pos;
    a.ncol = k;
    a.nsteps = nsteps;
    if (spec) {
        a.dpos = spec->dpos;
        a.spec_cur = spec->cur;
        a.spec_next = spec->next;
        a.spec_emit = spec->emit;
        a.spec_emit_cap = spec->cap;
    }
    if (batch) {
        a.batch = 1;
        for (int i = 0; i < 4; ++i) {
            a.bseq[i] = i < batch->n ? batch->seq[i] : 0;
            a.bpos[i] = i < batch->n ? batch->pos[i] : 0;
        }
    }
    a.epoch = x->epoch + 1;
    x->epoch += (uint32_t)nsteps;
    a.deadline_ticks = (uint64_t)x->timeout_us * (uint64_t)x->wall_khz / 1000ull;
    a.clock_mask = x->timeout_us < 1000 ? 0u : 31u;
    void* args[] = {&a};
    hipError_t e = hipLaunchCooperativeKernel(x->fn[k], dim3(x->grid), dim3(kBlock), args, (unsigned)x->lds[k],
                                              x->stream);
    if (e != hipSuccess) return hip_fail(e, "hipLaunchCooperativeKernel");
    x->last_ncol = k;
    return MBG_OK;
}

int mbg_decode_step(mbg_ctx* x, const int32_t* d_token, int32_t pos, float* d_logits, int32_t* d_argmax) {
    return launch_step(x, d_token, 1, pos, d_logits, d_argmax);
}

int mbg_decode_verify(mbg_ctx* x, const int32_t* d_tokens, int32_t k, int32_t pos, float* d_logits,
                      int32_t* d_argmax) {
    return launch_step(x, d_tokens, k, pos, d_logits, d_argmax);
}

int mbg_decode_steps(mbg_ctx* x, const int32_t* d_token, int32_t n_steps, int32_t pos, float* d_logits,
                     int32_t* d_argmax) {
    return launch_step(x, d_token, 1, pos, d_logits, d_argmax, n_steps);
}

int mbg_decode_batch(mbg_ctx* x, const int32_t* d_tokens, int32_t n, const int32_t* seq, const int32_t* pos,
                     float* d_logits, int32_t* d_argmax) {
    if (!x) return fail(MBG_E_INVALID_ARG, "ctx is NULL");
    if (!seq || !pos) return fail(MBG_E_INVALID_ARG, "seq/pos is NULL");
    if (n < 1 || n > x->cfg.k_max) return fail(MBG_E_RANGE, "n %d outside [1, %d]", n, x->cfg.k_max);
    BatchCols b;
    for (int i = 0; i < n; ++i) {
        if (seq[i] < 0 || seq[i] >= x->n_seqs)
            return fail(MBG_E_RANGE, "seq[%d] = %d outside [0, %d)", i, seq[i], x->n_seqs);
        if (pos[i] < 0 || pos[i] >= x->cfg.max_pos)
            return fail(MBG_E_RANGE, "pos[%d] = %d outside [0, %d)", i, pos[i], x->cfg.max_pos);
        for (int j = 0; j < i; ++j)
            if (seq[j] == seq[i]) return fail(MBG_E_INVALID_ARG, "sequence %d appears twice", seq[i]);
        b.seq[i] = seq[i];
        b.pos[i] = pos[i];
    }
    b.n = n;
    return launch_step(x, d_tokens, n, pos[0], d_logits, d_argmax, 1, &b);
}

int mbg_spec_round(mbg_ctx* target, mbg_ctx* draft, int32_t k, int32_t* d_state, int32_t* d_next, int32_t* d_emit,
                   int32_t emit_cap, float* d_logits) {
    if (!target || !draft) return fail(MBG_E_INVALID_ARG, "ctx is NULL");
    if (!d_state || !d_next || !d_emit) return fail(MBG_E_INVALID_ARG, "state/next/emit is NULL");
    if (d_state == d_next) return fail(MBG_E_INVALID_ARG, "the next state must be another buffer");
    if (target->stream != draft->stream) return fail(MBG_E_INVALID_ARG, "target and draft must share a stream");
    if (target->cfg.vocab != draft->cfg.vocab) return fail(MBG_E_INVALID_ARG, "target and draft vocabularies differ");
    if (k < 2 || k > target->cfg.k_max) return fail(MBG_E_RANGE, "k %d outside [2, %d]", k, target->cfg.k_max);
    if (emit_cap <= 0) return fail(MBG_E_INVALID_ARG, "emit_cap %d", emit_cap);
    int32_t* win = d_state + SPEC_WINDOW;
    // draft: k greedy steps from window[0] at the state's position; its
    // tokens land in window[1 .. k] (the k-th is only for the draft's own
    // cache: with every draft accepted the next round starts after it)
    SpecLaunch ds;
    ds.dpos = d_state + SPEC_POS;
    int rc = launch_step(draft, win, 1, 0, nullptr, win + 1, k, nullptr, &ds);
    if (rc) return rc;
    // target: the k-token window, then acceptance into the next state
    SpecLaunch vs;
    vs.dpos = d_state + SPEC_POS;
    vs.cur = d_state;
    vs.next = d_next;
    vs.emit = d_emit;
    vs.cap = emit_cap;
    return launch_step(target, win, k, 0, d_logits, d_next + SPEC_WINDOW, 1, nullptr, &vs);
}

int mbg_get_status(mbg_ctx* x) {
    if (!x) return fail(MBG_E_INVALID_ARG, "ctx is NULL");
    HIP_TRY(hipStreamSynchronize(x->stream));
    uint32_t w[3] = {0, 0, 0};   // status, LM-head counter, flags
    HIP_TRY(hipMemcpy(w, x->base.status, sizeof w, hipMemcpyDeviceToHost));
    const uint32_t st = w[0], fl = w[2];
    if (st != 0) {
        // An aborted launch leaves dependency, arrival and LM-head counters
        // short of epoch x need and may leave argmax keys set: start the
        // context over from epoch 0 with every counter and key at zero.
        HIP_TRY(launch_fill_u32((uint32_t*)x->uc, x->uc_bytes / 4, 0u, x->stream));
        HIP_TRY(launch_fill_u32((uint32_t*)x->ws_zero, x->ws_zero_bytes / 4, 0u, x->stream));
        HIP_TRY(hipStreamSynchronize(x->stream));
        x->epoch = 0;
        if (st == kStatusTimeout) return fail(MBG_E_TIMEOUT, "a device wait exceeded its deadline");
        if (st == kStatusPlacement)
            return fail(MBG_E_UNSUPPORTED, "workgroups are not placed on XCD blockIdx %% 8; set MBG_ATTN_LOCAL=0");
        if (st == kStatusPosition) return fail(MBG_E_RANGE, "a speculative round's position was out of range");
        return fail(MBG_E_HIP, "device status %u", st);
    }
    if (fl != 0) {
        HIP_TRY(launch_fill_u32(x->base.flags, 1, 0u, x->stream));
        HIP_TRY(hipStreamSynchronize(x->stream));
        if (fl == kStatusRange) return fail(MBG_E_RANGE, "a token id was outside [0, vocab) and was clamped");
        return fail(MBG_E_HIP, "device flag %u", fl);
    }
    return MBG_OK;
}

int mbg_query(const mbg_ctx* x, mbg_info* info) {
    if (!x || !info) return fail(MBG_E_INVALID_ARG, "ctx/info is NULL");
    memset(info, 0, sizeof *info);
    info->grid = x->grid;
    info->block = kBlock;
    info->n_tasks = x->n_tasks;
    info->launches_per_step = 1;
    info->lm_dtype = x->lm_dtype;
    info->kv_dtype = x->kv_dtype;
    info->expert_dtype = x->cfg.n_experts ? MBG_MXFP4 : 0;
    info->attn_dtype = MBG_BF16;
    info->attn_splits = x->base.attn_splits;
    info->attn_local = x->base.attn_local;
    info->trace = x->trace_on;
    info->verify_path = x->base.verify_mfma ? MBG_PATH_MFMA : MBG_PATH_FMA;
    info->clock_khz = x->wall_khz;
    info->weight_bytes_per_step = x->weight_bytes;
    info->workspace_bytes = (int64_t)x->ws_bytes;
    snprintf(info->variant, sizeof info->variant, "%s", x->variant);
    return MBG_OK;
}

int mbg_set_timeout_us(mbg_ctx* x, int64_t us) {
    if (!x || us <= 0) return fail(MBG_E_INVALID_ARG, "ctx is NULL or timeout <= 0");
    x->timeout_us = us;
    return MBG_OK;
}

int mbg_set_verify_path(mbg_ctx* x, int path) {
    if (!x) return fail(MBG_E_INVALID_ARG, "ctx is NULL");
    if (path != MBG_PATH_FMA && path != MBG_PATH_MFMA) return fail(MBG_E_INVALID_ARG, "verify path %d", path);
    x->base.verify_mfma = path == MBG_PATH_MFMA ? 1 : 0;
    return MBG_OK;
}

int mbg_set_trace(mbg_ctx* x, int on) {
    if (!x) return fail(MBG_E_INVALID_ARG, "ctx is NULL");
    x->trace_on = on ? 1 : 0;
    x->base.trace = on ? x->trace_buf : nullptr;
    return MBG_OK;
}

int mbg_read_trace(mbg_ctx* x, uint64_t* host, size_t max_records, size_t* n_out) {
    if (!x || !host || !n_out) return fail(MBG_E_INVALID_ARG, "NULL pointer");
    if (!x->trace_on) return fail(MBG_E_INVALID_ARG, "tracing is off");
    const size_t n = std::min<size_t>(max_records, (size_t)x->n_tasks);
    HIP_TRY(hipStreamSynchronize(x->stream));
    HIP_TRY(hipMemcpy(host, x->trace_buf, 64 * n, hipMemcpyDeviceToHost));
    *n_out = n;
    return MBG_OK;
}

int mbg_read_routing(mbg_ctx* x, int32_t layer, int32_t* idx, float* weights, int32_t* ncol) {
    if (!x || !idx || !weights || !ncol) return fail(MBG_E_INVALID_ARG, "NULL pointer");
    if (x->cfg.n_experts == 0) return fail(MBG_E_INVALID_ARG, "dense model: no routing");
    if (layer < 0 || layer >= x->cfg.n_layers) return fail(MBG_E_RANGE, "layer %d", layer);
    if (x->last_ncol == 0) return fail(MBG_E_INVALID_ARG, "no step has run");
    const size_t n = (size_t)x->last_ncol * x->cfg.top_k;
    const size_t off = (size_t)layer * n;
    HIP_TRY(hipStreamSynchronize(x->stream));
    HIP_TRY(hipMemcpy(idx, x->base.route_idx + off, 4 * n, hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(weights, x->base.route_w + off, 4 * n, hipMemcpyDeviceToHost));
    *ncol = x->last_ncol;
    return MBG_OK;
}

void mbg_destroy(mbg_ctx* x) {
    if (!x) return;
    // the context's last launch must be done with the caller's buffers
    (void)hipStreamSynchronize(x->stream);
    delete x;
}

// ------------------------------------------------------- standalone ops

int mbg_lm_head_workspace_size(int32_t k, size_t* bytes) {
    if (k < 1 || k > 4) return fail(MBG_E_RANGE, "k %d outside [1, 4]", k);
    if (!bytes) return fail(MBG_E_INVALID_ARG, "bytes is NULL");
    *bytes = 256;
    return MBG_OK;
}

static int lm_head_check(const mbg_tensor* w, const float* d_x, int32_t k, const int32_t* d_argmax) {
    if (!w || !d_x || !d_argmax) return fail(MBG_E_INVALID_ARG, "w/x/argmax is NULL");
    if (k < 1 || k > 4) return fail(MBG_E_RANGE, "k %d outside [1, 4]", k);
    if (w->dtype != MBG_BF16 && w->dtype != MBG_FP8_E4M3 && w->dtype != MBG_MXFP4)
        return fail(MBG_E_UNSUPPORTED, "lm head dtype %d (BF16, FP8 E4M3 or MXFP4)", w->dtype);
    int rc = check_tensor(*w, "lm_head", w->dtype, 1, w->rows, w->cols);
    if (rc) return rc;
    const int align = w->dtype == MBG_MXFP4 ? 32 : 16;
    if (w->rows <= 0 || w->rows > 0x7FFFFFFF || w->cols <= 0 || w->cols % align != 0)
        return fail(MBG_E_UNSUPPORTED, "lm head shape [%lld][%lld]: cols must be a positive multiple of %d",
                    (long long)w->rows, (long long)w->cols, align);
    if (!lm_head_hidden_supported((int)w->cols))
        return fail(MBG_E_UNSUPPORTED, "lm head hidden size %lld not compiled in", (long long)w->cols);
    if ((size_t)k * w->cols * 4 + 256 > 160 * 1024)
        return fail(MBG_E_UNSUPPORTED, "k * cols too large for on-chip activations");
    return MBG_OK;
}

// keys at d_ws, counter at d_ws + 64; both zero on entry and left at zero
static int lm_head_launch(const mbg_tensor* w, const float* d_x, int32_t k, float* d_logits, int32_t* d_argmax,
                          void* d_ws, void* stream) {
    static int cus = 0;
    int rc = 0;
    if (cus == 0 && (rc = device_cus(&cus))) return rc;
    LmHeadArgs a;
    a.w = w->data;
    a.wscale = w->scale;
    a.x = d_x;
    a.logits = d_logits;
    a.argmax = d_argmax;
    a.keys = (unsigned long long*)d_ws;
    a.counter = (uint32_t*)((char*)d_ws + 64);
    a.V = (int32_t)w->rows;
    a.H = (int32_t)w->cols;
    int64_t grid = std::min<int64_t>((a.V + 3) / 4, 2 * (int64_t)cus);
    const int fmt = w->dtype == MBG_FP8_E4M3 ? 2 : w->dtype == MBG_MXFP4 ? 3 : 1;   // kernel format codes (gemv.h)
    hipError_t e = launch_lm_head(a, k, fmt, (int)grid, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "lm_head launch");
    return MBG_OK;
}

int mbg_lm_head(const mbg_tensor* w, const float* d_x, int32_t k, float* d_logits, int32_t* d_argmax,
                void* d_ws, size_t ws_bytes, void* stream) {
    int rc = lm_head_check(w, d_x, k, d_argmax);
    if (rc) return rc;
    if (!d_ws || ws_bytes < 256) return fail(MBG_E_WORKSPACE, "workspace %zu bytes, need 256", ws_bytes);
    return lm_head_launch(w, d_x, k, d_logits, d_argmax, d_ws, stream);
}

int mbg_lm_head_noalloc(const mbg_tensor* w, const float* d_x, int32_t k, float* d_logits, int32_t* d_argmax,
                        void* stream) {
    int rc = lm_head_check(w, d_x, k, d_argmax);
    if (rc) return rc;
    if ((size_t)k * 8 > 64) return fail(MBG_E_RANGE, "k %d: the fixed scratch holds at most 8 argmax keys", k);
    void* p = nullptr;
    hipError_t e = lm_head_scratch((hipStream_t)stream, &p);
    if (e != hipSuccess) return hip_fail(e, "lm_head scratch set-up");
    return lm_head_launch(w, d_x, k, d_logits, d_argmax, p, stream);
}

int mbg_quantize_fp8_rows(const uint16_t* d_w, int64_t rows, int64_t cols, uint8_t* d_codes, float* d_scales,
                          void* stream) {
    if (!d_w || !d_codes || !d_scales) return fail(MBG_E_INVALID_ARG, "NULL pointer");
    if (rows <= 0 || cols <= 0 || rows > 0x7FFFFFFF || cols % 16 != 0)
        return fail(MBG_E_INVALID_ARG, "shape [%lld][%lld]: cols must be a positive multiple of 16",
                    (long long)rows, (long long)cols);
    hipError_t e = launch_quantize_fp8_rows(d_w, rows, cols, d_codes, d_scales, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return MBG_OK;
}

int mbg_kv_write(const mbg_config* cfg, const mbg_kv* kv, int32_t layer, int32_t pos0, int32_t n, const float* d_k,
                 const float* d_v, void* stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!kv || !kv->pool || !kv->page_table || !d_k || !d_v) return fail(MBG_E_INVALID_ARG, "NULL pointer");
    if (kv->dtype != MBG_BF16 && kv->dtype != MBG_FP8_E4M3) return fail(MBG_E_UNSUPPORTED, "kv dtype %d", kv->dtype);
    if (kv->dtype == MBG_FP8_E4M3 && !kv->scales) return fail(MBG_E_DTYPE_MISMATCH, "FP8 cache without scales");
    if (layer < 0 || layer >= cfg->n_layers) return fail(MBG_E_RANGE, "layer %d", layer);
    if (n < 0 || pos0 < 0 || (int64_t)pos0 + n > cfg->max_pos)
        return fail(MBG_E_RANGE, "positions %d..%d outside [0, %d)", pos0, pos0 + n - 1, cfg->max_pos);
    if (n == 0) return MBG_OK;
    {
        const int lp0 = pos0 / cfg->page_size, lp1 = (pos0 + n - 1) / cfg->page_size;
        std::vector<int32_t> pt(lp1 - lp0 + 1);
        HIP_TRY(hipMemcpy(pt.data(), kv->page_table + lp0, 4 * pt.size(), hipMemcpyDeviceToHost));
        for (size_t i = 0; i < pt.size(); ++i)
            if (pt[i] < 0 || pt[i] >= kv->n_pages)
                return fail(MBG_E_RANGE, "page_table[%zu] = %d outside [0, %d)", lp0 + i, pt[i], kv->n_pages);
    }
    KvWriteArgs a;
    a.pool = kv->pool;
    a.page_table = kv->page_table;
    a.scales = kv->scales;
    a.k = d_k;
    a.v = d_v;
    a.layer_off = (int64_t)layer * kv->n_pages * 2 * cfg->n_kv_heads * cfg->page_size * cfg->head_dim;
    a.dtype = kv->dtype == MBG_FP8_E4M3 ? 2 : 1;
    a.layer = layer;
    a.pos0 = pos0;
    a.n = n;
    a.n_kv_heads = cfg->n_kv_heads;
    a.head_dim = cfg->head_dim;
    a.page_size = cfg->page_size;
    hipError_t e = launch_kv_write(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_write launch");
    return MBG_OK;
}

}  // extern "C"
