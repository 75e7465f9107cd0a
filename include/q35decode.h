/*
 * q35decode: single-token (batch-1) decode of Qwen3.5 hybrid decoder layers on
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The calls mirror the problem statement of the `qwen3_5` forward module
 * documented on four pages: the rustdoc index "Module qwen3_5" and the source
 * pages `mod.rs`, `full_attention.rs` and `linear_attention.rs`.  Two layer
 * forwards, `forward_full_attention` and `forward_linear_attention`, each run one
 * decoder layer for one token over a `Qwen35ForwardConfig`, with the layer's
 * weights, state, KV cache and scratch all owned by the caller.
 *
 * Conventions for every call below:
 *  - Pointers named in structs are DEVICE pointers unless the comment says
 *    "host".  The library never frees or retains them past the call.
 *  - The library allocates no device memory.  Calls that take a hipStream_t
 *    only enqueue work on that stream and return; nothing is synchronised
 *    unless stated.  Scratch, state and cache buffers must not be shared by
 *    calls that may run concurrently.
 *  - Every call returns a q35_status, and q35_last_error() then holds a message
 *    (thread-local).  Argument errors are found before anything is enqueued;
 *    Q35_ERR_HIP means a launch failed part way.
 *  - Dtypes: "bf16" buffers hold bfloat16 bit patterns (uint16); "act" buffers
 *    hold the activation dtype of the config (bf16 or fp32); everything else is
 *    fp32 unless stated.
 */
#ifndef Q35DECODE_H
#define Q35DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */

typedef int32_t q35_status;
#define Q35_OK 0
#define Q35_ERR_INVALID_ARG 1   /* bad config, size, alignment or NULL pointer       */
#define Q35_ERR_UNSUPPORTED 2   /* a valid request this build does not implement     */
#define Q35_ERR_OUT_OF_RANGE 3  /* cache position / sequence length out of bounds    */
#define Q35_ERR_HIP 4           /* a HIP runtime call or launch failed               */
#define Q35_ERR_NO_DEVICE 5     /* no device, or the device is not gfx950            */

/* Message for the last non-OK status on this thread ("" if none). */
const char* q35_last_error(void);

/* ------------------------------------------------------------------ config */

#define Q35_ACT_BF16 0u
#define Q35_ACT_F32 1u

/*
 * Qwen35ForwardConfig (mod.rs page, the config struct): the sixteen dimension
 * fields of the pages, in the same order, plus `act_dtype`, the dtype of the
 * residual stream (Q35_ACT_BF16 or Q35_ACT_F32).
 */
typedef struct Qwen35ForwardConfig {
    uint32_t hidden;
    uint32_t intermediate;
    uint32_t num_layers;
    uint32_t vocab;
    uint32_t group_size;
    float rms_eps;
    uint32_t num_heads;
    uint32_t num_kv_heads;
    uint32_t head_dim;
    float rope_theta;
    uint32_t rotary_dim;
    uint32_t num_k_heads_lin;
    uint32_t num_v_heads_lin;
    uint32_t k_head_dim_lin;
    uint32_t v_head_dim_lin;
    uint32_t conv_kernel_size;
    uint32_t act_dtype;
} Qwen35ForwardConfig;

/* Fills *cfg with the Qwen3.5-4B dimensions (mod.rs page, the preset
 * constructor) and act_dtype = Q35_ACT_BF16.  Host pointer. */
q35_status q35_config_qwen3_5_4b(Qwen35ForwardConfig* cfg);

/*
 * Checks that this build supports *cfg (host pointer): group_size 64;
 * hidden, intermediate, q_only, kv_dim and z_dim_lin multiples of 64 and
 * among the GEMV widths compiled in; num_heads % num_kv_heads == 0 with a
 * ratio in {1,2,4,8}; num_v_heads_lin % num_k_heads_lin == 0; head_dim in
 * {64,128,256}; rotary_dim even and <= head_dim; k_head_dim_lin ==
 * v_head_dim_lin in {32,64,128}; conv_kernel_size 4; act_dtype bf16 or f32.
 * Q35_ERR_INVALID_ARG or Q35_ERR_UNSUPPORTED otherwise.
 */
q35_status q35_config_validate(const Qwen35ForwardConfig* cfg);

/* inv_freq[i] = fp32(rope_theta^(-2i/rotary_dim)) for i < rotary_dim/2, computed
 * in double.  This is the caller-built buffer `rope_apply` consumes
 * (full_attention.rs page, the RoPE launches).  host_out: host, rotary_dim/2 floats. */
q35_status q35_rope_inv_freq(const Qwen35ForwardConfig* cfg, float* host_out);

/* ------------------------------------------------------------------ kernels */

/*
 * Qwen35Kernels (mod.rs page, the kernel table and its resolve function):
 * checks once, at start-up, that `device` is a gfx950 GPU and that every
 * kernel of this library loads on it, so nothing is looked up in the hot path.
 * Errors: Q35_ERR_NO_DEVICE (no such device, or not gfx950), Q35_ERR_HIP.
 * The handle is immutable and may be shared by threads; release it with
 * q35_kernels_release.
 */
typedef struct Qwen35Kernels Qwen35Kernels;
q35_status q35_kernels_resolve(int device, Qwen35Kernels** out);
void q35_kernels_release(Qwen35Kernels* k);

/* ------------------------------------------------------------------ weights */

/*
 * One 8-bit affine quantised matrix (the pages' QuantWeights, an MLX-8bit
 * checkpoint with group_size 64): W[n][k] = scale[n][k/64] * code[n][k] +
 * bias[n][k/64].  codes: uint8 [n, k] row-major; scales, biases: bf16 [n, k/64]
 * row-major.  Device pointers, 16-byte aligned, read only.
 */
typedef struct Q35QuantWeight {
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* biases;
    uint32_t n;
    uint32_t k;
} Q35QuantWeight;

/* ------------------------------------------------------------------ KV cache */

#define Q35_KV_BF16 0u
#define Q35_KV_TURBO8 1u
#define Q35_KV_TURBO4 2u
#define Q35_KV_TURBO3 3u
#define Q35_KV_TURBO2 4u
#define Q35_KV_BF16K_TURBO4V 5u
#define Q35_KV_BF16K_TURBO3V 6u
#define Q35_KV_BF16K_TURBO2V 7u

/* Parses a KV storage-format name as the pages' MetalKvDtype FromStr does
 * ("bf16", "turbo8", "turbo4", "turbo3", "turbo2", "bf16k_turbo4v",
 * "bf16k_turbo3v", "bf16k_turbo2v").  Unknown names: Q35_ERR_INVALID_ARG.
 * The per-layer full-attention forward implements every format; the persistent
 * decode path implements Q35_KV_BF16. */
q35_status q35_kv_dtype_from_str(const char* name, uint32_t* dtype);

/*
 * Byte sizes of one layer's cache for `max_seq` tokens, per the page's
 * LayerKvCache::alloc: K data, V data, K scales, V scales (0 where absent).
 * A turbo format with kv_dim % 16 != 0 is Q35_ERR_INVALID_ARG (the page
 * asserts).  Host output pointers.
 */
q35_status q35_kv_cache_bytes(const Qwen35ForwardConfig* cfg, uint32_t dtype, uint32_t max_seq,
                              size_t* k_bytes, size_t* v_bytes, size_t* k_scale_bytes,
                              size_t* v_scale_bytes);

/*
 * LayerKvCache (mod.rs page): token-major, so row `cache_pos` is one
 * contiguous kv_dim vector; capacity is in tokens and IS bounds-checked here.
 *   Q35_KV_BF16:   k, v bf16 [capacity, num_kv_heads, head_dim]; k_scales and
 *                  v_scales NULL.
 *   Q35_KV_TURBO8 (mod.rs: MetalKvDtype::Turbo8, the Turbo branch of
 *                  full_attention.rs): k, v are FP8 E4M3 (OCP) codes, uint8
 *                  [capacity, num_kv_heads, head_dim], of the head vectors
 *                  after the orthonormal Walsh-Hadamard transform; k_scales,
 *                  v_scales bf16 [capacity, num_kv_heads, head_dim / 16], one per
 *                  16 consecutive elements: value = e4m3(code) * scale.  The
 *                  append stores scale = bf16(amax / 448) and codes = E4M3 of
 *                  x / scale, rounded to nearest-even, saturating.
 *   Lloyd-Max formats (mod.rs: MetalKvDtype::Turbo4/3/2 and Bf16KTurbo4V/3V/2V;
 *                  the Turbo branches of full_attention.rs), b = 4, 3 or 2 bits:
 *                  a quantised side holds b-bit indices into the 2^b-level
 *                  codebook of q35_turbo_codebook, uint8 [capacity, num_kv_heads,
 *                  head_dim * b / 8], a little-endian bit stream (element e at
 *                  bits [b e, b e + b)), of the head vectors after the orthonormal
 *                  Walsh-Hadamard transform, with one FP8 E4M3 scale byte per 16
 *                  elements [capacity, num_kv_heads, head_dim / 16]:
 *                  value = e4m3(scale) * level[index].  Q35_KV_TURBO4/3/2 quantise
 *                  K (k_scales) and V (v_scales); Q35_KV_BF16K_TURBO4V/3V/2V keep
 *                  k as bf16 [capacity, num_kv_heads, head_dim], not rotated, with
 *                  k_scales NULL.  The append picks each index as the nearest level
 *                  to x / rms(group) and stores the scale ||x|| / ||level[idx]||.
 * sparse_v: the sparse-V gate of the quantised formats (full_attention.rs: the
 *   Turbo branches pass this threshold to their attention launches; the pages
 *   use 1e-3 unless the caller overrides it, and 0 turns the gate off).  A
 *   position's value row is left out of the weighted sum when its softmax
 *   weight relative to the largest, exp(s_t - max s), is below sparse_v; the
 *   softmax itself still covers every position.  The kernel compares against
 *   its running maximum (never above the final one), so it leaves out a
 *   subset of those rows, and only where every lane of a wave agrees: the
 *   result differs from the exact rule by at most the weight of the rows that
 *   rule drops.  Ignored for Q35_KV_BF16.  Must be finite and >= 0, else
 *   Q35_ERR_INVALID_ARG.
 */
typedef struct LayerKvCache {
    void* k;
    void* v;
    uint32_t capacity;
    uint32_t dtype;
    void* k_scales;
    void* v_scales;
    float sparse_v;
} LayerKvCache;

/* ------------------------------------------------------------------ full-attention layer */

/* FullAttentionLayer (mod.rs page).  Norm weights are bf16 [hidden] (input_ln,
 * post_ln) and bf16 [head_dim] (q_norm, k_norm).  q_proj is [2*num_heads*head_dim,
 * hidden] with each head's rows ordered [Q_h | gate_h]; k_proj and v_proj
 * [kv_dim, hidden]; o_proj [hidden, q_only]; gate_proj and up_proj
 * [intermediate, hidden]; down_proj [hidden, intermediate]. */
typedef struct FullAttentionLayer {
    const uint16_t* input_ln;
    const uint16_t* q_norm;
    const uint16_t* k_norm;
    const uint16_t* post_ln;
    Q35QuantWeight q_proj;
    Q35QuantWeight k_proj;
    Q35QuantWeight v_proj;
    Q35QuantWeight o_proj;
    Q35QuantWeight gate_proj;
    Q35QuantWeight up_proj;
    Q35QuantWeight down_proj;
} FullAttentionLayer;

/*
 * FullAttentionScratch (mod.rs page).  The fused kernels materialise fewer
 * buffers than the page's sixteen.  Required (fp32 unless noted):
 *   q_full [q_total], k [kv_dim], v [kv_dim], gated_attn [q_only],
 *   x_resid [hidden], mlp_act [intermediate] (= silu(gate) * up),
 *   x_out [hidden] (act dtype),
 *   workspace (bytes from q35_full_attention_workspace_bytes: per-chunk
 *   attention partials, rewritten by every call; no initialisation needed).
 * Optional taps, written when non-NULL (fp32): x_norm [hidden],
 *   q_norm_out [q_only] (post-RoPE q), k_norm_out [kv_dim] (post-RoPE k),
 *   attn_out [q_only], o [hidden], x_norm2 [hidden], gate_act [intermediate],
 *   up_act [intermediate].
 * Optional status (device uint32 [1], caller-owned, cleared by the caller):
 *   the device-position entry (q35_forward_full_attention_devpos) ORs
 *   Q35_STATUS_POS_RANGE into it when positions[0] lies outside
 *   [0, capacity) at run time; that call then writes no KV row and its
 *   attention output (gated_attn) is zero, so the step's result is not
 *   the method's.  Without a status word the condition goes unreported.
 */
#define Q35_STATUS_POS_RANGE 2u
/* Error bit of the XCD-split plan: a block read an XCD id outside [0, 8) (its
 * results are invalid). */
#define Q35_STATUS_XCD_MAP 4u
typedef struct FullAttentionScratch {
    float* q_full;
    float* k;
    float* v;
    float* gated_attn;
    float* x_resid;
    float* mlp_act;
    void* x_out;
    void* workspace;
    size_t workspace_bytes;
    float* x_norm;
    float* q_norm_out;
    float* k_norm_out;
    float* attn_out;
    float* o;
    float* x_norm2;
    float* gate_act;
    float* up_act;
    uint32_t* status;
} FullAttentionScratch;

/* Workspace bytes one full-attention layer needs for caches of `capacity` tokens. */
q35_status q35_full_attention_workspace_bytes(const Qwen35ForwardConfig* cfg, uint32_t capacity,
                                              size_t* bytes);

/*
 * forward_full_attention (full_attention.rs page): one token through one gated
 * full-attention layer.  x_in (act [hidden]) is the residual stream; the
 * layer's output residual stream is written to scratch->x_out and *out is set
 * to that pointer.  Steps: input RMSNorm; q/k/v projections; q/gate split;
 * per-head RMSNorm of q and k; partial RoPE at positions[0]; append of k (after
 * RoPE) and v as bf16 at row cache_pos; GQA softmax attention over rows
 * [0, seq_len_attn); sigmoid output gate; o projection plus residual;
 * post-attention RMSNorm; SwiGLU MLP plus residual.
 *   inv_freq: fp32 [rotary_dim/2] (see q35_rope_inv_freq);
 *   positions: int32 [1], must hold cache_pos (RoPE reads it on the device);
 *   cache_pos < kv->capacity and seq_len_attn == cache_pos + 1, else
 *   Q35_ERR_OUT_OF_RANGE; an unknown kv->dtype: Q35_ERR_UNSUPPORTED.  With
 *   Turbo8 and Turbo4/3/2 the query heads, the new key and value are rotated
 *   before the quantising append and the attention output is rotated back; with
 *   Bf16K + TurboNV only the value is rotated (and the output rotated back).
 *   Attention covers all rows; with a quantised format, value rows below the
 *   kv->sparse_v gate are left out of the weighted sum (see LayerKvCache).
 * x_in must not alias any scratch buffer.
 */
q35_status q35_forward_full_attention(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                      const FullAttentionLayer* layer,
                                      const FullAttentionScratch* scratch, const LayerKvCache* kv,
                                      const float* inv_freq, const int32_t* positions,
                                      const void* x_in, uint32_t cache_pos, uint32_t seq_len_attn,
                                      hipStream_t stream, void** out);

/*
 * Same as q35_forward_full_attention, but the cache position is read on the
 * device from positions[0] (seq_len_attn = positions[0] + 1), so one captured
 * HIP graph replays every decode step.  A device position outside
 * [0, capacity) skips the append and the attention: the attention output is
 * zero, no memory outside the buffers is touched, and scratch->status (when
 * given) receives Q35_STATUS_POS_RANGE.
 */
q35_status q35_forward_full_attention_devpos(const Qwen35Kernels* kernels,
                                             const Qwen35ForwardConfig* cfg,
                                             const FullAttentionLayer* layer,
                                             const FullAttentionScratch* scratch,
                                             const LayerKvCache* kv, const float* inv_freq,
                                             const int32_t* positions, const void* x_in,
                                             hipStream_t stream, void** out);

/*
 * Kernel-level export: the attention steps of forward_full_attention alone
 * (full_attention.rs page: the q/gate split, the q/k RMSNorm, partial RoPE, the
 * KV append, attention_decode and sigmoid_gate), on the projections already in
 * scratch->q_full, k and v, with the cache position read from positions[0] as
 * in q35_forward_full_attention_devpos.  Writes the appended row, the
 * attention partials in scratch->workspace, scratch->gated_attn and the
 * optional taps (q_norm_out, k_norm_out, attn_out) and status.  Two launches
 * (per-chunk partials, then the merge with the gate).  Errors as
 * q35_forward_full_attention_devpos.
 */
q35_status q35_attention_devpos(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                const FullAttentionLayer* layer, const FullAttentionScratch* scratch,
                                const LayerKvCache* kv, const float* inv_freq,
                                const int32_t* positions, hipStream_t stream);

/* ------------------------------------------------------------------ GDN layer */

/* LinearAttentionLayer (mod.rs page): input_ln, post_ln bf16 [hidden]; a_log fp32
 * [num_v_heads_lin]; dt_bias bf16 [num_v_heads_lin]; conv1d_weight bf16
 * [qkv_total_lin, conv_kernel_size]; in_proj_a and in_proj_b [num_v_heads_lin,
 * hidden]; in_proj_qkv [qkv_total_lin, hidden] with rows [Q | K | V]; in_proj_z
 * [z_dim_lin, hidden]; norm_weight bf16 [v_head_dim_lin]; out_proj [hidden,
 * z_dim_lin]; gate_proj, up_proj, down_proj as in the full-attention layer. */
typedef struct LinearAttentionLayer {
    const uint16_t* input_ln;
    const float* a_log;
    const uint16_t* dt_bias;
    const uint16_t* conv1d_weight;
    Q35QuantWeight in_proj_a;
    Q35QuantWeight in_proj_b;
    Q35QuantWeight in_proj_qkv;
    Q35QuantWeight in_proj_z;
    const uint16_t* norm_weight;
    Q35QuantWeight out_proj;
    const uint16_t* post_ln;
    Q35QuantWeight gate_proj;
    Q35QuantWeight up_proj;
    Q35QuantWeight down_proj;
} LinearAttentionLayer;

/* LinearAttentionState (mod.rs page): conv1d_state fp32 [qkv_total_lin,
 * conv_kernel_size] (the last conv_kernel_size raw inputs per channel, newest
 * last) and gdn_state fp32 [num_v_heads_lin, k_head_dim_lin, v_head_dim_lin].
 * Carried across tokens and updated in place; the caller allocates and zeroes it. */
typedef struct LinearAttentionState {
    float* conv1d_state;
    float* gdn_state;
} LinearAttentionState;

/*
 * LinearAttentionScratch (mod.rs page).  Required (fp32):
 *   qkv_conv [qkv_total_lin] (conv + SiLU output, before the Q/K L2 norm),
 *   z [z_dim_lin], gate [num_v_heads_lin], beta [num_v_heads_lin],
 *   y [z_dim_lin], x_resid [hidden], mlp_act [intermediate].
 * Optional taps, written when non-NULL (fp32 unless noted): x_norm [hidden],
 *   dt_raw, b_raw [num_v_heads_lin], qkv [qkv_total_lin] (before the conv),
 *   qkv_smooth [qkv_total_lin] (after conv, SiLU and the Q/K L2 norm),
 *   y_norm [z_dim_lin], out [hidden], x_norm2 [hidden], gate_act,
 *   up_act [intermediate], x_final [hidden] (act dtype).
 */
typedef struct LinearAttentionScratch {
    float* qkv_conv;
    float* z;
    float* gate;
    float* beta;
    float* y;
    float* x_resid;
    float* mlp_act;
    float* x_norm;
    float* dt_raw;
    float* b_raw;
    float* qkv;
    float* qkv_smooth;
    float* y_norm;
    float* out;
    float* x_norm2;
    float* gate_act;
    float* up_act;
    void* x_final;
} LinearAttentionScratch;

/* Debug hook (the page's intra_dump): called on the host, after a stream
 * synchronise, once per named intermediate with a device pointer and an element
 * count.  Names: gdn_x_norm, gdn_qkv_pre, gdn_qkv_smooth, gdn_y, gdn_y_norm,
 * gdn_out, gdn_x_resid, gdn_x_final; fp32 buffers except gdn_x_final (act). */
typedef void (*q35_dump_fn)(void* ctx, const char* name, const void* device_ptr, uint32_t count);

/*
 * forward_linear_attention (linear_attention.rs page): one token through one
 * GDN layer.  Steps: input RMSNorm; in_proj a/b/qkv/z projections; causal
 * depthwise conv update with SiLU; decay gate exp(-exp(A_log) *
 * softplus(a + dt_bias)) and beta = sigmoid(b); per-head L2 norm of Q and K;
 * the gated delta-rule recurrence (query scale 1/sqrt(k_head_dim_lin) on the
 * output); per-head RMSNorm times silu(z); out projection plus residual;
 * post-attention RMSNorm; SwiGLU MLP plus residual.  The output residual
 * stream (act [hidden]) is written to x_buf and *out is set to x_buf.
 * x_buf may alias x_in (every read of x_in precedes the write of x_buf).
 * When dump != NULL the stream is synchronised and dump is called for the
 * taps that are non-NULL in scratch.
 */
q35_status q35_forward_linear_attention(const Qwen35Kernels* kernels,
                                        const Qwen35ForwardConfig* cfg,
                                        const LinearAttentionLayer* layer,
                                        const LinearAttentionState* state,
                                        const LinearAttentionScratch* scratch, const void* x_in,
                                        void* x_buf, hipStream_t stream, q35_dump_fn dump,
                                        void* dump_ctx, void** out);

/* ------------------------------------------------------------------ stack tail */

/*
 * Embedding lookup for the caller's layer loop: x_out (act [hidden]) =
 * table[tokens[0]] where table is bf16 [vocab, hidden].  tokens: int32 [1].
 * A token outside [0, vocab) writes zeros.
 */
q35_status q35_embed_lookup(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                            const uint16_t* table, const int32_t* tokens, void* x_out,
                            hipStream_t stream);

/* Workspace bytes q35_lm_head_argmax needs (scratch: no initialisation needed). */
q35_status q35_lm_head_workspace_bytes(const Qwen35ForwardConfig* cfg, size_t* bytes);

/*
 * Caller-owned tail of a decode step: h = RMSNorm(x; final_norm) (x act
 * [hidden], final_norm bf16 [hidden]); logits = lm_head h (lm_head
 * [vocab, hidden]); tokens[0] = argmax (lowest index on ties).  Optional
 * (may be NULL): logits fp32 [vocab]; history int32 [history_len], which
 * receives the token at index positions[0] - history_base when that lies in
 * range; positions int32 [1], incremented by one after the token is chosen;
 * embed_table bf16 [vocab, hidden] with x_next act [hidden] (both 16-byte
 * aligned), which then receives the chosen token's embedding (the next step's
 * input).  Two launches: the GEMV leaves one (max, row) pair per block in the
 * workspace and a one-block kernel reduces them, so no block waits on another.
 */
q35_status q35_lm_head_argmax(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                              const uint16_t* final_norm, const Q35QuantWeight* lm_head,
                              const void* x, float* logits, void* workspace,
                              size_t workspace_bytes, int32_t* tokens, int32_t* positions,
                              int32_t* history, uint32_t history_len, int32_t history_base,
                              const uint16_t* embed_table, void* x_next, hipStream_t stream);

/*
 * q35_lm_head_argmax without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc).  Arguments, layout and results as q35_lm_head_argmax.
 * The per-block partials go to a fixed 64 KiB device array that the library
 * holds on each GPU until the process ends (its address is taken at
 * q35_kernels_resolve); this call allocates nothing.  The partials never need
 * more than 16 KiB (q35_lm_head_workspace_bytes: the launch is capped at a
 * fixed number of blocks; the 248 320 vocabulary needs 15 872 bytes); a
 * configuration that needed more than the array would return
 * Q35_ERR_OUT_OF_RANGE.  Every call on one
 * GPU shares that array: calls that overlap in time on one GPU (different
 * streams without ordering) race and must not be issued.
 */
q35_status q35_lm_head_argmax_noalloc(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                      const uint16_t* final_norm, const Q35QuantWeight* lm_head,
                                      const void* x, float* logits, int32_t* tokens,
                                      int32_t* positions, int32_t* history, uint32_t history_len,
                                      int32_t history_base, const uint16_t* embed_table, void* x_next,
                                      hipStream_t stream);

/* ------------------------------------------------------------------ persistent decode */

/*
 * The same per-token computation as calling q35_forward_linear_attention /
 * q35_forward_full_attention layer by layer and then q35_lm_head_argmax
 * (linear_attention.rs and full_attention.rs pages: every step of both
 * forwards, in the pages' order), run as ONE cooperative launch per token: a
 * persistent kernel with one block per compute unit executes a table of
 * stages (5 per GDN layer, 6 per full-attention layer, 2 for the tail) and
 * synchronises the blocks between stages itself.  Each stage's weight loads
 * are issued before the wait for its inputs, so HBM keeps streaming across
 * stage and layer boundaries.  Results equal the layer-by-layer path up to
 * fp32 summation order (split-K attention chunks follow the block count).
 *
 * Supported shapes: the Qwen3.5-4B layer dimensions with bf16 activations
 * (hidden 2560, intermediate 9216, 16 q heads / 4 kv heads of 256, 16 k / 32 v
 * heads of 128) and the small fp32 test dimensions (hidden 256, intermediate
 * 512, 4 q / 2 kv heads of 64, 2 k / 4 v heads of 32); others return
 * Q35_ERR_UNSUPPORTED (use the per-layer calls).
 */
#define Q35_LAYER_LINEAR 0u
#define Q35_LAYER_FULL 1u

typedef struct Q35StackLayer {
    uint32_t kind;                       /* Q35_LAYER_LINEAR or Q35_LAYER_FULL */
    const LinearAttentionLayer* linear;  /* kind == LINEAR: weights */
    const LinearAttentionState* state;   /* kind == LINEAR: conv and GDN state (updated) */
    const FullAttentionLayer* full;      /* kind == FULL: weights */
    const LayerKvCache* kv;              /* kind == FULL: bf16 cache (row positions[0] written) */
} Q35StackLayer;

/* Host-side description of a stack; every pointer member other than `layers`
 * is a device pointer owned by the caller and must outlive the plan. */
typedef struct Q35DecodeStackDesc {
    uint32_t n_layers;
    const Q35StackLayer* layers;   /* host array [n_layers], read at plan creation */
    const float* inv_freq;         /* fp32 [rotary_dim/2] (q35_rope_inv_freq); any full layer */
    int32_t* positions;            /* int32 [1]: this token's cache position (the tail adds 1) */
    /* Stack tail (final RMSNorm, lm_head, greedy token, next embedding).  With
     * lm_head == NULL the plan is layers only and the caller writes each token's
     * input into q35_decode_layer_input(plan, 0) before the step. */
    const Q35QuantWeight* lm_head; /* [vocab, hidden] (host struct, device arrays) */
    const uint16_t* final_norm;    /* bf16 [hidden] */
    const uint16_t* embed;         /* bf16 [vocab, hidden], 16-byte aligned */
    int32_t* tokens;               /* int32 [1]: current token; receives the next one */
    float* logits;                 /* optional fp32 [vocab] */
    int32_t* history;              /* optional int32 [history_len]: token at positions[0]-history_base */
    uint32_t history_len;
    int32_t history_base;
} Q35DecodeStackDesc;

typedef struct Q35DecodePlan Q35DecodePlan;

/* Device workspace q35_decode_plan_create needs for this stack (per-layer
 * activation buffers, attention partials, the stage table, sync words). */
q35_status q35_decode_workspace_bytes(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                      const Q35DecodeStackDesc* stack, size_t* bytes);

/*
 * Validates the stack (as the per-layer calls do), writes the stage table into
 * the caller's device workspace (256-byte aligned; synchronous copy), clears its
 * sync words, and,
 * with a tail, writes the embedding of tokens[0] into the first layer's input.
 * The workspace must not be used by anything else while the plan lives.  *out
 * is a host object freed with q35_decode_plan_release.  Errors:
 * Q35_ERR_UNSUPPORTED (shape, a KV cache other than bf16, or a device that
 * cannot launch the grid cooperatively), Q35_ERR_INVALID_ARG (as the per-layer calls; workspace too
 * small), Q35_ERR_HIP.
 */
q35_status q35_decode_plan_create(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                  const Q35DecodeStackDesc* stack, void* workspace,
                                  size_t workspace_bytes, Q35DecodePlan** out);
void q35_decode_plan_release(Q35DecodePlan* plan);

/*
 * One token: every layer at cache position positions[0] (read on the device,
 * so one captured graph replays every token), then the tail.  Enqueued on
 * `stream`; capturable.  Steps of one plan must not overlap (one stream).
 */
q35_status q35_decode_step(const Q35DecodePlan* plan, hipStream_t stream);

/*
 * Synchronises the device and reads the plan's error word, a set of bits
 * accumulated over the plan's steps: 0 when every step ran as the method
 * says; bit 0 (1) when an inter-block wait gave up after its time limit (the
 * results of that step are invalid; create a new plan); bit 1
 * (Q35_STATUS_POS_RANGE) when positions[0] lay outside [0, capacity) of a
 * layer's cache, so that layer wrote no KV row and its attention output was
 * zero (the token of that step is not the method's).  The kernel exits
 * normally in both cases.
 */
q35_status q35_decode_check(const Q35DecodePlan* plan, uint32_t* error_word);

/* Device pointer of layer `layer`'s input residual stream (act [hidden]);
 * layer == n_layers gives the last layer's output (the tail's input). */
q35_status q35_decode_layer_input(const Q35DecodePlan* plan, uint32_t layer, void** x);

/* Number of stages, and the first stage of each layer (host array [n_layers + 1]:
 * the last entry is the tail's first stage). */
q35_status q35_decode_stage_layout(const Q35DecodePlan* plan, uint32_t* n_stages,
                                   uint32_t* layer_first_stage);

/*
 * Synchronises and copies, for the last step, block 0's wall-clock time at the
 * start of each stage (after its wait; stage 0 does not wait) into host ticks
 * [n], n <= n_stages, plus the clock rate in Hz.
 */
q35_status q35_decode_stage_times(const Q35DecodePlan* plan, uint64_t* ticks, uint32_t n,
                                  uint64_t* ticks_per_second);

/* ------------------------------------------------------------------ XCD-split decode plan
 *
 * The same token as the per-layer calls and the persistent plan (the layer
 * forwards of the linear_attention.rs and full_attention.rs pages, then the
 * final RMSNorm, lm_head and greedy token), launched so that the steps whose
 * work splits over MI355X's eight XCDs share one launch: a GDN layer is two
 * launches (mixer: in-projection, conv, gate/beta, gated delta rule, gated
 * norm, out-projection; MLP: gate/up, SwiGLU, down), a full-attention layer
 * four (q/k/v; attention; o_proj; MLP).  XCD x takes v-heads
 * [Hv/8 x, Hv/8 (x+1)) of the mixer and intermediate rows
 * [I/8 x, I/8 (x+1)) of the MLP; the out-projection and down then leave
 * eight fp32 partial sums, which the next launch adds to the residual in a
 * fixed order (base, partial 0, ..., partial 7).  The residual stream is
 * rounded to the activation dtype where the per-layer calls store it (each
 * layer's input and the stack's output).  Built for the Qwen3.5-4B shapes with
 * bf16 activations on a device of 8 x 32 compute units whose one-block-per-CU
 * grids place the blocks of one residue class of the block index mod 8 on each
 * XCD (checked at creation; every block takes its share from the XCD id it reads).
 * Any KV format of the per-layer calls.
 */
typedef struct Q35XcdPlan Q35XcdPlan;

/* Device workspace q35_xcd_plan_create needs for this stack. */
q35_status q35_xcd_workspace_bytes(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                   const Q35DecodeStackDesc* stack, size_t* bytes);

/*
 * Validates the stack (as the per-layer calls do), checks the placement of a
 * one-block-per-CU grid, writes the per-XCD stage table into the caller's
 * device workspace (256-byte aligned; synchronous copy), clears the sync words
 * and, with a tail, writes the embedding of tokens[0] into the first layer's
 * input.  `kernels` and the stack's device arrays must outlive the plan; the
 * host structs of the description are copied.  The workspace must not be used
 * by anything else while the plan lives.  Errors: Q35_ERR_UNSUPPORTED (shapes,
 * compute-unit count, placement), Q35_ERR_INVALID_ARG (as the per-layer calls;
 * workspace too small), Q35_ERR_HIP.
 */
q35_status q35_xcd_plan_create(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                               const Q35DecodeStackDesc* stack, void* workspace, size_t workspace_bytes,
                               Q35XcdPlan** out);
void q35_xcd_plan_release(Q35XcdPlan* plan);

/* One token at cache position positions[0] (read on the device): every layer,
 * then the tail.  Enqueued on `stream`; capturable.  Steps of one plan must not
 * overlap (one stream). */
q35_status q35_xcd_step(const Q35XcdPlan* plan, hipStream_t stream);

/*
 * Synchronises the device and reads the plan's error word (bits accumulated
 * over its steps): bit 0 (1) when a wait among the blocks of an XCD gave up
 * after its time limit; Q35_STATUS_POS_RANGE when positions[0] lay outside a
 * layer's cache; Q35_STATUS_XCD_MAP when a block read an XCD id outside [0, 8).  With any bit set the tokens since the plan was created are
 * not the method's; create a new plan.  The kernels exit normally in every case.
 */
q35_status q35_xcd_check(const Q35XcdPlan* plan, uint32_t* error_word);

/* Device pointer (act [hidden]) of the first layer's input (layer 0: without a
 * tail the caller writes each token's input there before the step) or of the
 * last layer's output (layer == n_layers).  Other layers' inputs are not held
 * as whole vectors: Q35_ERR_OUT_OF_RANGE. */
q35_status q35_xcd_layer_input(const Q35XcdPlan* plan, uint32_t layer, void** x);

/* Device buffers of the plan, shared by all layers: after a step they hold the
 * values of the last layer that wrote them (of the only layer, in a one-layer
 * plan).  fp32 unless noted. */
typedef struct Q35XcdBuffers {
    void* x_in;        /* act [hidden]: the layer input, as summed and rounded */
    float* qkv_conv;   /* [qkv_total_lin]: conv + SiLU output (GDN) */
    float* z;          /* [Hv * dv] */
    float* gate;       /* [Hv]: decay gate */
    float* beta;       /* [Hv] */
    float* y;          /* [Hv * dv]: recurrence output, before the gated norm */
    float* out_parts;  /* [8][hidden]: out-projection partial sums (GDN) */
    float* mlp_act;    /* [intermediate]: silu(gate) * up */
    float* mlp_parts;  /* [8][hidden]: down partial sums */
    float* x_mid;      /* [hidden]: x_in + o_proj output (full attention) */
    float* x_resid;    /* [hidden]: the residual after the mixer (the MLP's base) */
} Q35XcdBuffers;
q35_status q35_xcd_buffers(const Q35XcdPlan* plan, Q35XcdBuffers* bufs);

/* ------------------------------------------------------------------ kernel-level export */

/*
 * The first half of the MLP shared by both layer forwards, as one launch:
 * xn2 = RMSNorm(x_resid; post_ln), then gate_proj and up_proj over the same
 * xn2 (the pages' `gemv_gate_up_with`), and mlp_act = silu(gate) * up (the
 * product the pages' `gemv_silu_gate_resid` consumes).  x_resid fp32 [hidden],
 * post_ln bf16 [hidden], gate_proj / up_proj [intermediate, hidden], mlp_act
 * fp32 [intermediate].  This is the largest kernel of a layer; it is exported
 * so that it can be timed on its own.
 */
q35_status q35_gate_up_swiglu(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                              const uint16_t* post_ln, const Q35QuantWeight* gate_proj,
                              const Q35QuantWeight* up_proj, const float* x_resid,
                              float* mlp_act, hipStream_t stream);

/*
 * The Turbo8 group quantiser of the full-attention append, over a plain device
 * vector: for each group of 16 consecutive fp32 values of x [n] (n a multiple
 * of 16), scales[g] = bf16(amax / 448) and codes[16g..16g+15] = E4M3 of
 * x / scale (round to nearest-even, saturating; a zero group gets scale 0 and
 * codes 0).  All device pointers, caller-owned: x fp32 [n] and codes uint8 [n]
 * 16-byte aligned, scales bf16 [n / 16] 2-byte aligned.  n not a multiple of
 * 16, a NULL or misaligned pointer: Q35_ERR_INVALID_ARG; n == 0 launches
 * nothing.  Asynchronous on `stream`.
 */
q35_status q35_turbo8_quantize(const Qwen35Kernels* kernels, const float* x, uint32_t n,
                               uint8_t* codes, uint16_t* scales, hipStream_t stream);

/* The Lloyd-Max codebook of the b-bit formats (mod.rs: the Turbo4/3/2
 * variants' Lloyd-Max indices): the 2^b-level Lloyd-Max quantiser of the
 * standard normal distribution, ascending, computed once by
 * q35_kernels_resolve.  bits 2, 3 or 4; levels: host float [2^bits],
 * caller-owned.  Other bits or NULL: Q35_ERR_INVALID_ARG. */
q35_status q35_turbo_codebook(const Qwen35Kernels* kernels, uint32_t bits, float* levels);

/*
 * The group quantiser of the Lloyd-Max formats' append, over a plain device
 * vector: for each group of 16 fp32 values of x [n] (n a multiple of 16),
 * sigma = sqrt(sum(x^2) / 16) (sum in double, sigma in fp32), each index the
 * number of thresholds (fp32 midpoints of adjacent levels) below x / sigma, and
 * the scale the E4M3 code of ||x|| / ||level[idx]|| (double, rounded to fp32,
 * then round-to-nearest-even, saturating); a zero group gets scale 0 and
 * indices 0.  packed uint8 [n * bits / 8] (little-endian bit stream; aligned
 * to one group's 2 * bits bytes), scales uint8 [n / 16]; x 16-byte aligned;
 * device pointers, caller-owned.  bits other than 2, 3, 4, n not a multiple of
 * 16, a NULL or misaligned pointer: Q35_ERR_INVALID_ARG; n == 0 launches
 * nothing.  Asynchronous on `stream`.
 */
q35_status q35_turbo_quantize(const Qwen35Kernels* kernels, uint32_t bits, const float* x, uint32_t n,
                              uint8_t* packed, uint8_t* scales, hipStream_t stream);

/* The E4M3 decoder of the Turbo8 attention over every code: out fp32 [256]
 * (device, caller-owned, 16-byte aligned), out[c] = value of code c; 0x7F and
 * 0xFF decode to NaN.  NULL or misaligned out: Q35_ERR_INVALID_ARG.
 * Asynchronous on `stream`. */
q35_status q35_fp8_e4m3_table(const Qwen35Kernels* kernels, float* out, hipStream_t stream);

/*
 * Plain GEMV with the library's quantised-weight kernel: y (fp32 [w->n]) =
 * W x (x fp32 [w->k]).  act_dtype picks the arithmetic the layer forwards use
 * for that activation dtype: Q35_ACT_F32, fp32 products; Q35_ACT_BF16, x
 * rounded to f16 after a power-of-two scaling of the whole vector and exact
 * f16 x u8 products summed in fp32.  With x a one-hot vector e_j, y is column
 * j of the dequantised matrix, bit for bit, in both.
 */
q35_status q35_gemv(const Qwen35Kernels* kernels, const Q35QuantWeight* w, const float* x,
                    float* y, uint32_t act_dtype, hipStream_t stream);

/* ------------------------------------------------------------------ prefill */

/*
 * Multi-token prefill of one layer.  The pages define the decode step only
 * (rustdoc index "Module qwen3_5": the module runs one token; the prompt pass
 * is the caller's).  A prefill of n_tokens tokens computes what n_tokens decode
 * calls would, in order: token t runs at cache position cache_pos + t (its RoPE
 * position and its KV row) and attends to rows [0, cache_pos + t]; the conv
 * and GDN states advance token by token.  The results agree with those calls
 * up to rounding (the projections take f16 inputs and f16-rounded weights on
 * the matrix cores, the recurrence runs in chunks of 64 tokens, the attention
 * takes f16 queries and f16 probabilities).
 *
 * Workspace: device memory of at least q35_prefill_workspace_bytes(cfg,
 * n_tokens) bytes, 256-byte aligned, caller-owned, rewritten by every call (no
 * initialisation needed; shared by the two layer kinds, not by concurrent
 * calls).  It includes room for the largest weight set of one projection as
 * f16: from 4096 tokens on, each projection dequantises its weights there
 * once (as q35_prefill_gemm does with a large enough workspace).
 */
q35_status q35_prefill_workspace_bytes(const Qwen35ForwardConfig* cfg, uint32_t max_tokens,
                                       size_t* bytes);

/*
 * n_tokens tokens through one GDN layer (linear_attention.rs page, every step
 * of forward_linear_attention per token).  x_in and x_out: act [n_tokens,
 * hidden], x_out may equal x_in; state: as in q35_forward_linear_attention,
 * updated in place to the state after the last token.  n_tokens == 0 enqueues
 * nothing.  k_head_dim_lin != v_head_dim_lin or not 32, 64 or 128:
 * Q35_ERR_UNSUPPORTED; a small workspace: Q35_ERR_INVALID_ARG.
 */
q35_status q35_prefill_linear_attention(const Qwen35Kernels* kernels,
                                        const Qwen35ForwardConfig* cfg,
                                        const LinearAttentionLayer* layer,
                                        const LinearAttentionState* state, const void* x_in,
                                        uint32_t n_tokens, void* x_out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/*
 * n_tokens tokens through one gated full-attention layer (full_attention.rs
 * page, every step of forward_full_attention per token), the KV rows
 * [cache_pos, cache_pos + n_tokens) appended in the cache's format.  bf16: one
 * causal attention launch over the prompt.  A quantised format (the Turbo
 * branches, kv->sparse_v applied): the result of the decode loop, each token
 * appending its quantised row and attending to the rows [0, its position] as
 * stored; at head_dim 128 and 256 in two launches (every row appended, then
 * one causal attention over the rows as stored), otherwise the decode
 * attention steps once per token in token order.  The projections and the
 * MLP stay batched.  x_in and x_out: act [n_tokens, hidden], x_out may equal
 * x_in; inv_freq as in q35_forward_full_attention.  cache_pos + n_tokens >
 * kv->capacity: Q35_ERR_OUT_OF_RANGE; a head_dim / group the attention kernels
 * do not cover, or (per-token path) a quantised cache whose attention partials
 * exceed the workspace's split-GEMM area (capacities past about four million
 * tokens): Q35_ERR_UNSUPPORTED.  n_tokens == 0 enqueues nothing.
 */
q35_status q35_prefill_full_attention(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                      const FullAttentionLayer* layer, const LayerKvCache* kv,
                                      const float* inv_freq, const void* x_in, uint32_t n_tokens,
                                      uint32_t cache_pos, void* x_out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * The prefill's quantised-weight GEMM: y (fp32 [m, w->n]) = x W^T with x f16
 * [m, w->k] (16-byte aligned rows), W[n, k] = scale * code + bias evaluated in
 * fp32 and rounded to f16, products on the matrix cores with fp32 sums.
 * Exported so that it can be tested and timed on its own.  workspace: NULL, or
 * device memory of at least Q35_PREFILL_GEMM_WORKSPACE_BYTES, 256-byte
 * aligned, caller-owned and rewritten by the call: with it, a last round of
 * tiles that would leave most compute units idle is cut along k into parts
 * whose fp32 sums are added in k order by a second kernel (the result then
 * differs from the NULL case by fp32 rounding only).  With at least
 * Q35_PREFILL_GEMM_WORKSPACE_BYTES + 2 * w->n * w->k bytes, W is first
 * written as f16 after that area and the product reads it from there instead
 * of dequantising each tile of W once per 256 rows of x (the same f16 values,
 * so the same result).  A smaller or misaligned workspace:
 * Q35_ERR_INVALID_ARG.  m == 0 enqueues nothing.
 */
#define Q35_PREFILL_GEMM_WORKSPACE_BYTES ((size_t)32 << 20)
q35_status q35_prefill_gemm(const Qwen35Kernels* kernels, const Q35QuantWeight* w,
                            const uint16_t* x_f16, uint32_t m, float* y, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* Q35DECODE_H */
