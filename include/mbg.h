/*
 * mbg: batch-1 transformer decode on one MI355X (gfx950), one kernel launch
 * per decode step.
 *
 * What a step computes.  At batch 1 every generated token is a chain of
 * matrix-vector products that streams every active weight byte from HBM
 * once (Kog article "Real-time LLM inference on standard GPUs: 3k tokens/s
 * per request", section on memory bandwidth as the bottleneck).  A step
 * embeds one token, runs every decoder layer (RMSNorm, Q/K/V projections,
 * RoPE, K/V write into a paged cache, grouped single-query attention over
 * positions [0, pos], output projection, RMSNorm, SwiGLU FFN or a routed
 * mixture of experts) and ends with the LM head and an argmax.  The whole
 * chain runs as one persistent kernel instead of a launch per operation
 * (same article, sections on where standard stacks lose microseconds and on
 * the monokernel runtime; the "Muse Spark Open: 1,109 tokens/s" megakernel
 * article, sections on the launch baseline and the kernel boundary).
 *
 * Conventions for every call:
 *   - "device" pointers point into HIP device memory of the current device;
 *     "host" pointers into ordinary process memory.
 *   - Matrices are row-major [rows][cols] with cols contiguous, 16-byte
 *     aligned rows.  BF16 is the top half of an IEEE binary32.  FP8 is OCP
 *     E4M3FN.  MXFP4 is OCP E2M1 (element 2i in the low nibble of byte i)
 *     with one E8M0 scale byte per 32 consecutive elements of a row.
 *   - The caller owns every buffer (weights, KV pool, page table, workspace,
 *     dependency-counter block, outputs).  No call allocates or frees device
 *     memory; an mbg_ctx is a host object.
 *   - Calls that take a stream enqueue work on it and return without
 *     waiting.  A stream is a hipStream_t passed as void* (NULL = the null
 *     stream).
 *   - Return value 0 on success, a negative MBG_E_* code otherwise; no
 *     exception crosses this boundary.  mbg_last_error() gives the text of
 *     the last failure on the calling thread.
 */
#ifndef MBG_H
#define MBG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- errors */
#define MBG_OK 0
#define MBG_E_INVALID_ARG -1     /* null pointer, bad shape, misaligned row  */
#define MBG_E_UNSUPPORTED -2     /* shape/dtype combination not compiled in  */
#define MBG_E_DTYPE_MISMATCH -3  /* tensor dtype or scale not what it must be */
#define MBG_E_RANGE -4           /* pos/k/token outside the configured range */
#define MBG_E_WORKSPACE -5       /* workspace missing or smaller than needed */
#define MBG_E_HIP -6             /* a HIP runtime call failed                */
#define MBG_E_TIMEOUT -7         /* a device wait exceeded its deadline      */

/* ------------------------------------------------- verify-window paths */
#define MBG_PATH_FMA 0   /* k-column FMA GEMV on the vector ALU */
#define MBG_PATH_MFMA 1  /* 16-row blocks on the matrix cores (BF16 hi + lo activations) */

/* ---------------------------------------------------------------- dtypes */
#define MBG_BF16 1
#define MBG_FP8_E4M3 2  /* one binary32 scale per row: value = code * scale[row] */
#define MBG_MXFP4 3     /* scale = E8M0 bytes [rows][cols/32]                   */
#define MBG_FP32 4

/*
 * A weight tensor: `n` stacked matrices of shape [rows][cols] (n = 1 for a
 * plain matrix, n = experts for stacked expert weights).
 *   BF16:  data = uint16 [n][rows][cols];            scale = NULL
 *   FP8:   data = uint8  [n][rows][cols];            scale = float [n][rows]
 *   MXFP4: data = uint8  [n][rows][cols/2];          scale = uint8 [n][rows][cols/32]
 * A 1-D tensor (norm gains) has rows = 1.  data/scale are device pointers.
 */
typedef struct {
    int32_t dtype;
    int32_t n;
    int64_t rows;
    int64_t cols;
    const void *data;
    const void *scale;
} mbg_tensor;

/* One decoder layer.  Dense layers fill w_gate/w_up/w_down; MoE layers fill
 * w_router, exp_gate_up, exp_down and (if n_shared > 0) sh_gate_up, sh_down.
 * Shapes (H hidden, d head_dim, F ffn, E experts, M moe_ffn, S n_shared):
 *   attn_norm, ffn_norm: BF16 [1][H]
 *   wq: BF16 [Hq*d][H]    wk, wv: BF16 [Hkv*d][H]    wo: BF16 [H][Hq*d]
 *   w_gate, w_up: BF16 [F][H]    w_down: BF16 [H][F]
 *   w_router: BF16 [E][H]
 *   exp_gate_up: MXFP4 n=E [2M][H] (rows 0..M-1 gate, M..2M-1 up)
 *   exp_down:    MXFP4 n=E [H][M]
 *   sh_gate_up:  MXFP4 n=S [2M][H]    sh_down: MXFP4 n=S [H][M]
 */
typedef struct {
    mbg_tensor attn_norm, wq, wk, wv, wo, ffn_norm;
    mbg_tensor w_gate, w_up, w_down;
    mbg_tensor w_router, exp_gate_up, exp_down, sh_gate_up, sh_down;
} mbg_layer;

typedef struct {
    const mbg_layer *layers; /* host array [n_layers]; read during init only */
    mbg_tensor embed;        /* BF16 [V][H] */
    mbg_tensor final_norm;   /* BF16 [1][H] */
    mbg_tensor lm_head;      /* BF16 or FP8 [V][H] */
} mbg_weights;

/*
 * Paged KV cache.  pool (device) holds
 *     [n_layers][n_pages][2 (K, V)][n_kv_heads][page_size][head_dim]
 * elements of `dtype` (MBG_BF16 or MBG_FP8_E4M3).  Position t of a layer
 * lives in physical page page_table[t / page_size], slot t % page_size.
 * page_table (device int32 [n_seqs][ceil(max_pos / page_size)]) maps
 * logical to physical pages, one row per sequence (n_seqs 0 counts as 1);
 * the identity table is a contiguous cache.  Sequence 0 is the one that
 * mbg_decode_step/_steps/_verify extend; mbg_decode_batch names the rows it
 * uses.  Rows must not share a physical page that either writes.  scales (device
 * float [n_layers][n_kv_heads][2], FP8 only, NULL for BF16) give
 * value = decode(code) * scale per (layer, KV head, K or V).  Paged FP8 KV
 * with a per-head scale is what the wmrh.cn Kimi-K3 long-context report
 * deploys (test environment table; warnings section, where both engines
 * fell back to a scale of 1.0 because none was supplied).
 */
typedef struct {
    int32_t dtype;
    int32_t n_pages;
    void *pool;
    const int32_t *page_table;
    const float *scales;
    int32_t n_seqs;   /* page-table rows (sequences sharing the pool); 0 or 1: one */
} mbg_kv;

typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int32_t n_experts, top_k, n_shared, moe_ffn; /* n_experts = 0: dense */
    float rope_theta; /* RoPE base; pairs (i, i + d/2) turn by pos * theta^(-2i/d) */
    float rms_eps;    /* RMSNorm: x / sqrt(mean(x^2) + eps) * g */
    int32_t page_size; /* positions per KV page: a power of two, >= 16 */
    int32_t max_pos;  /* KV capacity in positions */
    int32_t k_max;    /* widest verify window, 1..4 */
    /* Sliding-window layers: host array [n_layers], read during init only,
     * or NULL (every layer global).  layer_window[l] = W > 0: the token at
     * position p attends positions [max(0, p - W + 1), p] (its own and the
     * W - 1 before it); 0: [0, p].  The "Muse Spark Open" article (section
     * on how the model is split) describes 46 of 62 layers attending over
     * the last 2,048 tokens and 16 global layers; which layers are which is
     * the caller's.  The cache still holds every position; a windowed layer
     * reads only its window.  Negative values: MBG_E_INVALID_ARG. */
    const int32_t *layer_window;
} mbg_config;

/* What an initialised context runs (the 163.com Ling-3.0-flash article,
 * section on the FP8 LM head and MTP pitfall, reports a silent fallback
 * that read FP8 weights as BF16; this lets a caller check at start-up which
 * path is really active). */
typedef struct {
    int32_t grid;             /* workgroups of the persistent kernel */
    int32_t block;            /* threads per workgroup */
    int32_t n_tasks;          /* tasks per step */
    int32_t launches_per_step;
    int32_t lm_dtype, kv_dtype, expert_dtype, attn_dtype;
    int32_t attn_splits;      /* split-KV partitions per KV head */
    int32_t attn_local;       /* 1: a KV head's splits run on one XCD and exchange partials through its L2 */
    int32_t trace;            /* 1 while in-kernel trace stamps are on (mbg_set_trace) */
    int32_t verify_path;      /* MBG_PATH_FMA or MBG_PATH_MFMA (mbg_set_verify_path) */
    int64_t weight_bytes_per_step; /* bytes of weights one step reads (dense/shared; MoE routed excluded) */
    int64_t workspace_bytes;
    int64_t clock_khz;        /* rate of the device clock the trace stamps count */
    char variant[64];
} mbg_info;

typedef struct mbg_ctx mbg_ctx;

/* ------------------------------------------------------ decode context */

/* Bytes of device workspace a context for `cfg` needs: task lists, RoPE
 * table, the activations that pass between the ops of a step (residual
 * stream, q, split-KV partials, attention output, FFN hidden), argmax keys
 * and the trace buffer.  The step is the persistent one-launch kernel of
 * the Kog article "Real-time LLM inference on standard GPUs: 3k tokens/s
 * per request" (section on co-designing engine, GPU code and model: the
 * monokernel), whose intermediate values never leave device memory.
 * Host-only; errors: MBG_E_INVALID_ARG, MBG_E_UNSUPPORTED for the config. */
int mbg_workspace_size(const mbg_config *cfg, size_t *bytes);

/* Bytes of the dependency-counter block a context for `cfg` needs (one
 * 128-byte line for the status, LM-head counter and flag words, then
 * 8 x 128 bytes per (layer, phase) counter and one more for the step
 * token of multi-step launches; under 1 MiB for 64 layers).
 * The counters replace kernel boundaries with flag polling inside one
 * launch ("Muse Spark Open: 1,109 tokens/s" article, section on the three
 * bills of a kernel this large: synchronisation).  Host-only. */
int mbg_counter_bytes(const mbg_config *cfg, size_t *bytes);

/* Host-only check of a configuration, weight set and KV description: shapes,
 * dtypes, scale presence, alignment, supported combinations.  Makes no HIP
 * call and touches no device memory.  w or kv may be NULL to check less.
 * This is the start-up check the 163.com Ling-3.0-flash article asks for
 * (caveat section and conclusion: an FP8 LM head read as BF16 by a part of
 * the model that did not share the module fell back silently and ran slower
 * than no optimisation); every tensor here carries its own dtype and scale,
 * and a mismatch is MBG_E_DTYPE_MISMATCH rather than a silent fallback.
 * Errors: MBG_E_INVALID_ARG (null data, bad shape, misaligned rows),
 * MBG_E_DTYPE_MISMATCH, MBG_E_UNSUPPORTED (no compiled kernel). */
int mbg_validate(const mbg_config *cfg, const mbg_weights *w, const mbg_kv *kv);

/* Validate, build the static per-step task list in the caller's workspace
 * (device, >= mbg_workspace_size bytes, 256-byte aligned) with copies
 * enqueued on `stream`, zero the caller's counter block, and return a host
 * context (Kog article, monokernel section: the whole step becomes one
 * resident program; the task lists are its schedule).
 *   d_counters: device memory of >= mbg_counter_bytes bytes, 256-byte
 *     aligned, that the L2 does not cache (hipExtMallocWithFlags with
 *     hipDeviceMallocUncached).  The step kernel polls it with
 *     cache-bypassing scalar loads, which see other XCDs' counter updates
 *     only in uncached memory.  The caller keeps it while the context
 *     lives; per the HIP runtime's rules for uncached memory it should
 *     not be freed before the process ends once a kernel has read it, so
 *     a caller reuses it for later contexts.  One context per block.
 * The weights, KV pool, workspace and counter block must outlive the
 * context.  Tuning overrides read from the environment here (defaults are
 * the measured best; the "Muse Spark Open" article's prefetch bill is what
 * they trade): MBG_GEMV_PREFETCH, MBG_GU_PREFETCH, MBG_DOWN_PREFETCH (KiB
 * of weight rows a GEMV wavefront requests before its dependency wait,
 * 0..64; defaults 16, 24, 32), MBG_ATTN_PREFETCH (history ring chunks an
 * attention wave requests before its wait, 0..4), MBG_ATTN_LOCAL=0 (keep
 * the attention splits of a head group off a single XCD's L2).  Results do
 * not depend on them.  Errors: as mbg_validate, MBG_E_WORKSPACE (workspace
 * or counter block missing, small or misaligned), MBG_E_RANGE (a
 * page-table entry outside the pool), MBG_E_HIP. */
int mbg_decode_init(const mbg_config *cfg, const mbg_weights *w, const mbg_kv *kv,
                    void *d_workspace, size_t workspace_bytes, void *d_counters, size_t counter_bytes,
                    void *stream, mbg_ctx **out);

/* One decode step, one kernel launch on the init stream.  Reads the token
 * id at d_token[0] (device int32; may alias the previous step's d_argmax so
 * a greedy loop needs no host round trip), writes K/V of every layer at
 * `pos`, attends over [0, pos], and writes logits (device float [vocab], may
 * be NULL) and the argmax (device int32 [1], lowest index among equal
 * maxima).  What the step computes is the chain of matrix-vector products
 * over every active weight of the Kog article's bandwidth section; one
 * launch per step removes the launch and clean-up costs of its section on
 * where standard stacks lose microseconds.  A token id outside [0, vocab)
 * is clamped on the device, the step completes, and MBG_E_RANGE is
 * reported by the next mbg_get_status.  Returns MBG_E_RANGE if pos is
 * outside [0, max_pos), MBG_E_INVALID_ARG for null pointers, MBG_E_HIP if
 * the launch fails. */
int mbg_decode_step(mbg_ctx *ctx, const int32_t *d_token, int32_t pos,
                    float *d_logits, int32_t *d_argmax);

/* Verify window: k tokens (device int32 [k], 1 <= k <= k_max) at positions
 * pos .. pos+k-1 in one launch, each weight byte read once for all k.
 * Token j attends [0, pos + j], the window's earlier tokens included
 * (163.com Ling-3.0-flash article, section on MTP speculative decoding: the
 * target model checks a 4-token window in one pass).  Writes K/V at all k
 * positions, logits [k][vocab] (may be NULL) and argmax [k].  Accepting a
 * prefix and rolling back is the caller's job: the next call's pos decides
 * which cached positions count. */
int mbg_decode_verify(mbg_ctx *ctx, const int32_t *d_tokens, int32_t k, int32_t pos,
                      float *d_logits, int32_t *d_argmax);

/* Batch of n independent sequences (1 <= n <= k_max) in one launch: column
 * i decodes token d_tokens[i] of sequence seq[i] (a page-table row, host
 * int32 [n], all distinct, each in [0, n_seqs)) at position pos[i] (host
 * int32 [n], each in [0, max_pos)): it writes its K/V at pos[i] in its own
 * pages and attends [0, pos[i]] of its own cache only (its window in a
 * sliding-window layer).  Each weight byte is read once for all n columns,
 * as in a verify window; routed layers read the union of the columns'
 * experts.  The "Muse Spark Open" article (section on what would change the
 * result, first item) names batch > 1 as the next step: more tokens in
 * flight give a throughput figure a serving team can use.  Writes logits
 * [n][vocab] (may be NULL) and argmax [n].  Errors: MBG_E_RANGE for n, a
 * sequence or a position out of range; MBG_E_INVALID_ARG for NULL pointers
 * or a repeated sequence; otherwise as mbg_decode_step. */
int mbg_decode_batch(mbg_ctx *ctx, const int32_t *d_tokens, int32_t n, const int32_t *seq,
                     const int32_t *pos, float *d_logits, int32_t *d_argmax);

/* Speculative decoding state, in device memory (int32 words): the position
 * of window[0]; tokens emitted, draft tokens accepted and rounds run so
 * far; the window: window[0] is the last emitted token, window[1 .. k] the
 * draft's tokens of the round (written by mbg_spec_round). */
typedef struct {
    int32_t pos;
    int32_t n_emitted;
    int32_t n_accepted;
    int32_t n_rounds;
    int32_t window[8];
} mbg_spec_state;

/* One speculative round, enqueued as two launches on the shared stream with
 * no host round trip (163.com Ling-3.0-flash article, optimisation 3: a
 * draft proposes 3 tokens, the target verifies the 4-token window in one
 * pass, and the agreeing prefix is accepted; the "Muse Spark Open" article
 * runs draft, verify and accept as one graph per step).
 *   1. draft: k greedy steps of the draft context (any model with the same
 *      vocabulary, e.g. one layer sharing the target's embedding and LM
 *      head) from state.window[0] at state.pos, its tokens into
 *      state.window[1 .. k];
 *   2. target: the verify window state.window[0 .. k-1] at state.pos, then,
 *      on the device, greedy prefix acceptance: with am[j] the target's
 *      argmax after window[j], draft token j + 1 is accepted while
 *      am[j] == window[j + 1]; with m accepted the round appends
 *      am[0 .. m] to d_emit (int32 [emit_cap], at state.n_emitted) and
 *      writes *d_next: pos + m + 1, window[0] = am[m], the counters + (m + 1),
 *      + m, + 1.
 * Both contexts read the position on the device, so rounds chain: round
 * r + 1 takes round r's d_next as its d_state.  The emitted tokens are
 * those of greedy decoding of the target whatever the draft proposes; the
 * draft's quality only sets how many come per round.  d_logits (may be
 * NULL): the window's target logits [k][vocab].  k in [2, target k_max];
 * d_state and d_next are distinct mbg_spec_state buffers (device); both
 * contexts must have been initialised on the same stream.  A position out of
 * range (state.pos + k > max_pos of either context) ends the launch and
 * makes the next mbg_get_status of that context return MBG_E_RANGE; more
 * emitted tokens than emit_cap are dropped and flagged the same way.
 * Errors here: MBG_E_INVALID_ARG (NULL, shared buffers, different streams
 * or vocabularies), MBG_E_RANGE (k), MBG_E_HIP. */
int mbg_spec_round(mbg_ctx *target, mbg_ctx *draft, int32_t k, int32_t *d_state, int32_t *d_next,
                   int32_t *d_emit, int32_t emit_cap, float *d_logits);

/* n_steps greedy decode steps (1 .. 4096) in ONE kernel launch: step s runs
 * at pos + s; step 0 reads its token at d_token[0], step s > 0 takes the
 * argmax of step s - 1 on the device, and the persistent kernel moves from
 * one step to the next without returning (the Kog article "Real-time LLM
 * inference on standard GPUs: 3k tokens/s per request", section on
 * co-designing engine, GPU code and model: the monokernel keeps the whole
 * generation on the GPU; the "Muse Spark Open" article's step still
 * launches one kernel per layer).  Writes K/V at pos .. pos + n_steps - 1,
 * logits (device float [n_steps][vocab], may be NULL) and the tokens
 * (device int32 d_argmax[n_steps]).  Same arithmetic as n_steps calls of
 * mbg_decode_step with d_token aliasing the previous argmax: results are
 * bitwise equal.  Errors: MBG_E_RANGE if n_steps is outside [1, 4096] or
 * pos + n_steps exceeds max_pos; otherwise as mbg_decode_step. */
int mbg_decode_steps(mbg_ctx *ctx, const int32_t *d_token, int32_t n_steps, int32_t pos,
                     float *d_logits, int32_t *d_argmax);

/* Wait for the init stream, then return the device status of the calls
 * since the last mbg_get_status: 0, MBG_E_TIMEOUT (a dependency wait
 * exceeded its deadline and the launch drained), MBG_E_UNSUPPORTED (the
 * workgroups were not placed on the XCDs the attention placement assumes),
 * or MBG_E_RANGE (a token id was clamped; that step completed).  After
 * MBG_E_TIMEOUT or MBG_E_UNSUPPORTED every counter of the context is reset
 * and its launch count starts over, so the next call runs normally; until
 * mbg_get_status is called, later launches give up at their first wait.
 * The positions an aborted launch was writing hold partial K/V: the caller
 * reruns that step.  The watchdog is the device-side reading of the
 * synchronisation bill ("Muse Spark Open" article, section on the three
 * bills): a polled flag that never arrives must not hang the GPU. */
int mbg_get_status(mbg_ctx *ctx);

/* Describe the active configuration (see mbg_info). */
int mbg_query(const mbg_ctx *ctx, mbg_info *info);

/* Set the device wait deadline in microseconds (default 2,000,000) for
 * later launches.  A wait on a dependency counter that exceeds it makes its
 * workgroup record MBG_E_TIMEOUT and leave; every other wait then ends the
 * same way, so the launch always drains (see mbg_get_status for recovery).
 * A spinning wait reads the clock every 32nd poll, every poll under a
 * deadline below 1,000 us.  The deadline is the watchdog side of the flag
 * polling that replaces kernel boundaries ("Muse Spark Open" article,
 * section on the three bills: synchronisation).  MBG_E_INVALID_ARG for
 * us <= 0. */
int mbg_set_timeout_us(mbg_ctx *ctx, int64_t us);

/* How verify windows and batches (k >= 2 columns) run the routed experts' gate/up
 * rows: MBG_PATH_FMA multiplies every weight with each column on the vector
 * ALU (k multiply-adds per weight); MBG_PATH_MFMA decodes 16 rows at a time
 * to BF16 and runs v_mfma_f32_16x16x32_bf16 against the columns split into
 * BF16 hi and lo parts (the binary32 activations to ~2^-16 relative).  The
 * 163.com Ling-3.0-flash article (optimisation 3) finds expert activation to
 * be what a 4-token verify window costs; the two paths are timed against
 * each other on that window.  Single-token steps always use the FMA path,
 * and so do configurations without routed experts.  The default is
 * MBG_PATH_FMA.  Takes effect for later calls.  MBG_E_INVALID_ARG for another
 * value. */
int mbg_set_verify_path(mbg_ctx *ctx, int path);

/* Per-task self-profiling.  With `on` != 0, every later step makes thread 0
 * of each workgroup record, for each task it runs, eight uint64 words: the
 * device clock at task start, when its dependency wait was satisfied, when
 * its input vector was loaded, when its weight/KV stream finished, and at
 * task end; then (op | layer << 8 | tile << 32) and two op-specific stamps
 * (attention: history folded, split-KV combine weights ready; expert
 * gate/up: router logits loaded, top-k picked; else 0).  An external profiler
 * sees one long kernel per step, so the kernel times itself (the "Muse Spark
 * Open: 1,109 tokens/s" article describes the same in-kernel stamps, section
 * on where the step time goes).  Stamps do not change any result. */
int mbg_set_trace(mbg_ctx *ctx, int on);

/* Wait for the init stream and copy the last step's trace records (n_tasks
 * records of 8 uint64, in task-list order) into host memory; *n_out is the
 * record count.  Fails with MBG_E_INVALID_ARG if tracing is off. */
int mbg_read_trace(mbg_ctx *ctx, uint64_t *host_records, size_t max_records, size_t *n_out);

/* MoE models: wait for the init stream and copy the routing the last
 * step/verify call used in `layer` into host memory: for each of its *ncol
 * columns, the top_k selected expert ids (int32, by decreasing router
 * logit, lower id first on ties) and their renormalised softmax weights
 * (float32), column-major [ncol][top_k].  Both arrays must hold
 * k_max * top_k entries.  The selection rule is the 163.com Ling-3.0-flash
 * article's routed top-8 of 512 experts (model and baseline configuration).
 * MBG_E_INVALID_ARG for a dense model or before the first call. */
int mbg_read_routing(mbg_ctx *ctx, int32_t layer, int32_t *idx, float *weights, int32_t *ncol);

/* Text of the last error on this thread ("" if none). */
const char *mbg_last_error(void);

/* Wait for the context's stream and free the host context.  Does not touch
 * caller memory (the counter block can then serve another context).  The
 * counterpart of mbg_decode_init's set-up of the Kog article's monokernel. */
void mbg_destroy(mbg_ctx *ctx);

/* ------------------------------------------------ standalone operations */

/* Bytes of device workspace mbg_lm_head needs for k columns. */
int mbg_lm_head_workspace_size(int32_t k, size_t *bytes);

/* LM head GEMV fused with argmax: logits[j][v] = sum_i W[v][i] * x[j][i]
 * for j < k (1..4), W BF16, FP8 (row scale applied after accumulation) or
 * MXFP4 (E8M0 scale per 32 elements, applied on decode; cols a multiple of
 * 32), x device float [k][H].  Writes logits (device float [k][V], may be NULL)
 * and argmax (device int32 [k]).  d_workspace (>= the size above) must be
 * zero-filled before its first use; every call leaves it zeroed again.
 * Calls sharing one workspace must not overlap.  The 163.com Ling-3.0-flash
 * article singles the 157,184 x 2,560 LM head out as a block read whole for
 * every token (section "optimisation 2"). */
int mbg_lm_head(const mbg_tensor *w, const float *d_x, int32_t k, float *d_logits,
                int32_t *d_argmax, void *d_workspace, size_t workspace_bytes, void *stream);

/* mbg_lm_head for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc): the
 * same kernel and arguments without the workspace.  Its argmax keys and
 * arrival counter live in a fixed 256-byte device array of the library (one
 * copy per GPU, held until the process ends), set up and zeroed on the
 * first call on each device; every call leaves it zeroed again.  All calls
 * on one GPU share that array, so calls that overlap on one GPU (different
 * streams, or threads) race and must be serialised by the caller.
 * Allocates nothing.  Errors: as mbg_lm_head; k outside [1, 4] (more argmax
 * keys than the array holds) is MBG_E_RANGE; MBG_E_HIP if the array's device
 * address cannot be obtained. */
int mbg_lm_head_noalloc(const mbg_tensor *w, const float *d_x, int32_t k, float *d_logits,
                        int32_t *d_argmax, void *stream);

/* Online FP8 quantisation of a BF16 matrix with one scale per row (163.com
 * Ling-3.0-flash article, "optimisation 2: online FP8 LM head
 * quantisation"): scale[r] = max_i |W[r][i]| / 448 in binary32 (1.0 for an
 * all-zero row), codes[r][i] = E4M3FN(W[r][i] / scale[r]) with the division
 * in binary32, rounded to nearest-even and saturated at +-448.
 * d_w device uint16 [rows][cols]; d_codes device uint8 [rows][cols];
 * d_scales device float [rows].  cols must be a multiple of 16. */
int mbg_quantize_fp8_rows(const uint16_t *d_w, int64_t rows, int64_t cols, uint8_t *d_codes,
                          float *d_scales, void *stream);

/* Write n consecutive positions pos0 .. pos0+n-1 of one layer's K and V
 * into the paged cache in its storage format (BF16 nearest-even, or FP8
 * value / scale in binary32, nearest-even, saturating), the same rounding a
 * decode step applies to the K/V it produces.  d_k, d_v: device float
 * [n][n_kv_heads][head_dim].  Used to fill a cache from a prefill: the
 * paged FP8 cache with per-head scales of the wmrh.cn Kimi-K3 long-context
 * report (test environment and configuration: 64-token pages, fp8_e4m3; its
 * warnings section: a missing scale fell back to 1.0, so an FP8 cache
 * without scales is MBG_E_DTYPE_MISMATCH here).  Errors: MBG_E_RANGE
 * (layer, positions or a page-table entry out of range), MBG_E_INVALID_ARG,
 * MBG_E_UNSUPPORTED, MBG_E_HIP. */
int mbg_kv_write(const mbg_config *cfg, const mbg_kv *kv, int32_t layer, int32_t pos0, int32_t n,
                 const float *d_k, const float *d_v, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MBG_H */
