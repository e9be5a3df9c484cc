// Structures shared by the host runtime and the persistent decode kernel:
// the task encoding, per-layer weight pointers and the kernel argument block.
#pragma once

#include <stdint.h>

namespace mbg {

// Operations of the per-step task list.  One task is one tile of one op of
// one layer; a workgroup runs its tasks in list order, each after waiting
// for the counter of the phase it reads.
enum Op : uint32_t {
    OP_QKV = 1,    // RMSNorm(x) -> rows of Wq/Wk/Wv -> RoPE -> q to workspace, k/v to cache
    OP_ATTN = 2,   // one (KV head, split) of single-query attention; last split combines
    OP_OPROJ = 3,  // rows of Wo . attn, residual add
    OP_GATEUP = 4, // RMSNorm(x) -> rows of Wgate/Wup -> silu(g) * u
    OP_DOWN = 5,   // rows of Wdown . h, residual add
    OP_LMHEAD = 6, // final RMSNorm -> rows of the LM head -> logits, argmax
    OP_ROUTER = 7, // MoE: RMSNorm(x) -> router logits (whole row set per task)
    OP_EXPGU = 8,  // MoE: rows of a selected expert's gate/up
    OP_EXPDOWN = 9 // MoE: rows of the experts' down, weighted sum, residual add
};

// Phases: the dependency counters of one layer.
enum Phase : uint32_t {
    PH_QKV = 0,
    PH_ATTN = 1,  // counts finished combines (one per KV head)
    PH_OPROJ = 2,
    PH_GATEUP = 3,
    PH_DOWN = 4,
    PH_ROUTER = 5,
    PH_COUNT = 6
};

// 16-byte task record.
struct Task {
    uint32_t op_layer;  // op | layer << 8
    uint32_t tile;      // tile index within the op
    uint32_t wait_ctr;  // counter to wait on, or kNoWait
    uint32_t wait_need; // per-step count that counter reaches when the producer phase is done
};
constexpr uint32_t kNoWait = 0xFFFFFFFFu;

// A dependency counter is kCtrLines separate 128-byte lines: a producer adds
// to line (workgroup % kCtrLines) and a waiter sums all lines.  Same-address
// atomics from hundreds of workgroups serialise at the memory side; spreading
// them over lines keeps an all-to-all dependency point near two memory round
// trips.  Counters and the status word sit in uncached device memory, where
// a waiter reads all lines with one batch of scalar loads.
constexpr uint32_t kCtrLines = 8;
constexpr uint32_t kLineU32 = 32;

// Query heads per attention task (a KV head's larger group is split into
// several tasks that read the same history).
constexpr int kAttnHeadsPerTask = 2;

// MoE limits of the compiled kernels.
constexpr int kMaxExperts = 512;                 // routed experts (a multiple of 8)
constexpr int kMaxTopK = 8;
constexpr int kMaxShared = 2;
constexpr int kMaxSlots = 4 * kMaxTopK + kMaxShared;   // union over a 4-token window plus shared experts
constexpr int kSlotsPerPass = 9;                 // expert-down slots whose h sits in LDS at once
constexpr int kMaxDownRows = 3;                  // output rows one wavefront owns in the expert down

struct LayerPtrs {
    const uint16_t* attn_norm;
    const uint16_t* ffn_norm;
    const uint16_t* wq;
    const uint16_t* wk;
    const uint16_t* wv;
    const uint16_t* wo;
    const uint16_t* w_gate;
    const uint16_t* w_up;
    const uint16_t* w_down;
    const uint16_t* w_router;
    const uint8_t* eg_codes;   // experts gate/up MXFP4 codes [E][2M][H/2]
    const uint8_t* eg_scales;  // [E][2M][H/32]
    const uint8_t* ed_codes;   // experts down [E][H][M/2]
    const uint8_t* ed_scales;  // [E][H][M/32]
    const uint8_t* sg_codes;   // shared experts gate/up [S][2M][H/2]
    const uint8_t* sg_scales;
    const uint8_t* sd_codes;   // shared experts down [S][H][M/2]
    const uint8_t* sd_scales;
    int32_t window;            // attention window W (0: global): position p reads [p - W + 1, p]
    int32_t pad_;
};

// Everything the persistent kernel reads, by value.
struct StepArgs {
    // model shape
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int32_t n_experts, top_k, n_shared, moe_ffn;
    float rms_eps;
    float attn_scale_log2;  // log2(e) / sqrt(head_dim)
    int32_t page_size, max_pos;
    int32_t page_shift;     // log2(page_size) (a power of two)
    // tiling: tasks (workgroups) per phase; each wavefront of a phase owns
    // the output rows u = wave_id + n_waves * i of that phase
    uint32_t tiles_qkv, tiles_o, tiles_gu, tiles_down, tiles_lm;
    uint32_t tiles_router, tiles_egu, tiles_edown;
    int32_t attn_splits;
    // prefetch before a dependency wait: KiB of weight rows per GEMV
    // wavefront (whole rows, at most two register chunks) and attention ring
    // chunks per wavefront (0 .. kAttnBufs)
    int32_t gemv_pre, attn_pre;
    int32_t gu_pre, down_pre;    // the same budget (KiB) for the dense gate/up and down phases
    int32_t poll_wave_prefetch;  // 1: the polling wave (0) also prefetches before its wait
    int32_t wave0_input;         // 1: inputs copied to LDS by wave 0 alone (coherent DMA); 0: all waves load
    // weights
    const LayerPtrs* layers;
    const uint16_t* embed;
    const uint16_t* final_norm;
    const void* lm_head;
    const float* lm_scale;
    int32_t lm_dtype;
    // KV cache
    int32_t kv_dtype;
    void* kv_pool;
    const int32_t* page_table;  // [n_seqs][pt_stride]
    const float* kv_scales;
    int64_t kv_layer_stride;  // elements per layer = n_pages * 2 * Hkv * page * d
    int32_t pt_stride;        // page-table entries per sequence
    // batch of independent sequences (batch != 0): column c runs at position
    // bpos[c] of page-table row bseq[c]; otherwise column c runs at pos + c
    // of row 0 (one sequence: a step or a verify window)
    int32_t batch;
    int32_t bpos[4];
    int32_t bseq[4];
    // speculative rounds: the launch's first position is read on the device
    // from dpos (range-checked there) instead of pos; a verify launch with
    // spec_next set ends in greedy prefix acceptance (the LM head's last
    // workgroup) that writes the next round's state and the emitted tokens
    const int32_t* dpos;
    const int32_t* spec_cur;   // this round's state (SpecState layout)
    int32_t* spec_next;        // the next round's state, or null
    int32_t* spec_emit;        // emitted tokens [spec_emit_cap]
    int32_t spec_emit_cap;
    // workspace
    const Task* tasks;
    const uint32_t* task_off;  // [grid + 1]
    uint32_t* ctr;             // [n_layers * PH_COUNT + 1][kCtrLines lines], uncached memory; the
                               // last counts steps whose argmax (next token) is written
    uint32_t* head_ctr;        // [n_layers * n_kv_heads] split arrivals
    uint32_t* lm_ctr;          // LM-head tiles finished
    uint32_t* status;          // first device error that ends the launch (uncached memory)
    uint32_t* flags;           // conditions that do not end the launch (a clamped token id)
    float* xres;               // [k][H] residual stream
    float* qbuf;               // [k][Hq][d]
    float* part;               // [L][k][Hq][splits][d + 4] attention partials: each layer has its own
                               // rows, so a partial-row address is written and read once per launch
    int64_t part_layer;        // floats per layer of part
    float* attn;               // [k][Hq * d]
    float* hbuf;               // [k][F] or MoE [k][hb_ld]: column c, slot s, row f at c * hb_ld + s * M + f
    int32_t hb_ld;             // floats per column of hbuf
    float* rlogits;            // [k][n_experts] router logits (MoE)
    float* route_w;            // [L][k][top_k] routing weights of the last step (MoE)
    int32_t* route_idx;        // [L][k][top_k] routed expert ids of the last step
    unsigned long long* amax_keys;  // [k]
    const double* inv_freq;    // [d/2] theta^(-2i/d)
    const float2* rope_cs;     // [max_pos][d/2] (cos, sin) of p * inv_freq[i], from double angles
    unsigned long long* trace; // optional stamps
    // per call
    const int32_t* tokens;
    float* logits;
    int32_t* argmax;
    int32_t pos;               // position of the launch's first step (column 0)
    int32_t ncol;
    uint32_t epoch;            // epoch of the launch's first step; step s runs with epoch + s
    int32_t nsteps;            // greedy steps in this launch (token of step s > 0 = argmax of step s - 1)
    int32_t verify_mfma;       // k >= 2: expert gate/up rows on the matrix cores (mfma.h) instead of FMA
    int32_t attn_local;        // 1: the splits of an attention group run on one XCD (workgroup b on XCD b % 8)
                               //    and exchange partials and arrivals through that XCD's L2
    uint64_t deadline_ticks;   // s_memrealtime ticks a wait may take
    uint32_t clock_mask;       // a spinning wait reads the clock on poll rounds r with (r & mask) == 0
};

// Device status codes (positive on the device, negated at the boundary).
// kStatusTimeout, kStatusPlacement and kStatusPosition end the launch (every wait gives up);
// kStatusRange is a flag: the token id was clamped and the step completes.
constexpr uint32_t kStatusTimeout = 7;
constexpr uint32_t kStatusRange = 4;
constexpr int kAttnLocalMaxSplitLen = 1024;    // XCD-local attention groups only up to this many positions per split
constexpr uint32_t kStatusPlacement = 2;   // a workgroup is not on the XCD its attention placement assumes
constexpr uint32_t kStatusPosition = 5;    // a device-resident position (speculative round) was out of range

// Speculative-round state in device memory (int32 words; mbg_spec_state in
// the public header): position of window[0], tokens emitted, draft tokens
// accepted and rounds run so far, then the window: [0] the last emitted
// token, [1 ..] the draft's tokens.
enum : int { SPEC_POS = 0, SPEC_EMITTED = 1, SPEC_ACCEPTED = 2, SPEC_ROUNDS = 3, SPEC_WINDOW = 4, SPEC_WORDS = 12 };

}  // namespace mbg
