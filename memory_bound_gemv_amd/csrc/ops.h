// Host-side launch interfaces of the standalone kernels and the decode step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace mbg {

struct LmHeadArgs {
    const void* w;            // [V][H] BF16 or FP8 codes
    const void* wscale;       // FP8: float row scales [V]; MXFP4: E8M0 bytes [V][H/32]
    const float* x;           // [k][H]
    float* logits;            // [k][V] or null
    int32_t* argmax;          // [k]
    unsigned long long* keys; // [k] zeroed between calls
    uint32_t* counter;        // zeroed between calls
    int32_t V, H;
};

struct KvWriteArgs {
    void* pool;
    const int32_t* page_table;
    const float* scales;
    const float* k;
    const float* v;
    int64_t layer_off;  // element offset of the layer in the pool
    int32_t dtype;      // 1 = BF16, 2 = FP8
    int32_t layer, pos0, n, n_kv_heads, head_dim, page_size;
};

hipError_t launch_lm_head(const LmHeadArgs& a, int ncol, int fmt, int grid, hipStream_t s);
// Device address of this device's fixed LM-head scratch array (argmax keys at
// offset 0, arrival counter at offset 64), set up and zeroed on first use.
constexpr size_t kLmScratchBytes = 256;
hipError_t lm_head_scratch(hipStream_t s, void** out);
bool lm_head_hidden_supported(int H);
hipError_t launch_quantize_fp8_rows(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* codes, float* scales,
                                    hipStream_t s);
hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
hipError_t launch_rope_table(const double* inv_freq, int half, int64_t max_pos, float2* cs, hipStream_t s);

// Decode-step kernel family: the compile-time shape a kernel is built for.
struct StepVariant {
    int hidden, ffn, qdim, head_dim;
    int group;     // query heads per KV head
    int kv_fmt;    // 1 BF16, 2 FP8
    int moe;       // 0 dense, 1 MoE
    int moe_ffn;
};
// Returns the kernel entry for ncol columns, or null when not compiled in.
const void* step_kernel_for(const StepVariant& v, int ncol, int* lds_bytes_out);
bool step_variant_supported(const StepVariant& v);
// One per compiled model family (step.hip built with MBG_STEP_SHAPE = i).
constexpr int kStepShapes = 4;
const void* step_kernel_shape_0(const StepVariant& v, int ncol, int* lds_bytes_out);
const void* step_kernel_shape_1(const StepVariant& v, int ncol, int* lds_bytes_out);
const void* step_kernel_shape_2(const StepVariant& v, int ncol, int* lds_bytes_out);
const void* step_kernel_shape_3(const StepVariant& v, int ncol, int* lds_bytes_out);

}  // namespace mbg
