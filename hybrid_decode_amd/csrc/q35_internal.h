// Internal interface between the C-ABI host code and the q35decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q35 {

// ------------------------------------------------------------------ GEMV family

constexpr int kMaxSegs = 4;

enum : int32_t {
    kProRmsAct = 0,     // x = RMSNorm(x_act; w)          (x in the activation dtype)
    kProRmsF32 = 1,     // x = RMSNorm(x_f32; w)
    kProGatedNorm = 2,  // x = RMSNorm_per_head(y; w) * silu(z)
    kProLoadF32 = 3,    // x = src
};

enum : int32_t {
    kEpiStore = 0,       // out[n] = y
    kEpiResidActIn = 1,  // out[n] = act(aux0)[n] + y            (tap0 = y)
    kEpiResidToAct = 2,  // out_act[n] = act(f32(aux0)[n] + y)   (out_act2 copy)
    kEpiConv = 3,        // causal conv update + SiLU on channel n (state, aux0 = weights, tap0 = y)
    kEpiGate = 4,        // out[n] = exp(-exp(A_log[n]) softplus(y + dt_bias[n]))   (tap0 = y)
    kEpiBeta = 5,        // out[n] = sigmoid(y)                  (tap0 = y)
    kEpiSwiGLU = 6,      // paired: out[n] = silu(y_a) * y_b     (tap0 = y_a, tap1 = y_b)
    kEpiArgmax = 7,      // logits (optional out) + running argmax
};

struct GemvSeg {
    const uint8_t* codes[2];
    const uint16_t* scales[2];
    const uint16_t* biases[2];
    uint32_t rg_begin, rg_end;  // row-group range of this segment in the launch
    int32_t epi;
    float* out;
    void* out_act;
    void* out_act2;
    float* tap0;
    float* tap1;
    const void* aux0;
    const void* aux1;
    float* state;
};

struct GemvPro {
    int32_t kind;
    int32_t x_f32;  // kProRmsAct: input is fp32 (else bf16)
    const void* x;
    const uint16_t* w;
    const float* z;
    uint32_t head_dim;
    float eps;
    float* tap;  // optional: the normalised x (before the silu(z) factor), block 0 writes it
};

struct GemvArgmax {
    float* part_val;
    int32_t* part_idx;
    uint32_t* counter;  // nullptr: no argmax in this launch
    int32_t* tokens;
    int32_t* positions;
    int32_t* history;
    uint32_t history_len;
    int32_t history_base;
    const uint16_t* embed;
    void* x_next;
    uint32_t hidden;
    uint32_t vocab;
};

struct GemvArgs {
    GemvPro pro;
    GemvSeg seg[kMaxSegs];
    int32_t nseg;
    uint32_t total_rg;
    int32_t act_f32;
    GemvArgmax am;
};

bool gemv_width_supported(uint32_t k);
int gemv_rows_per_group(uint32_t k, bool paired);   // rows per row group
int gemv_rows_per_matrix_group(uint32_t k);         // rows of one matrix per row group
uint32_t gemv_pick_blocks(uint32_t total_rg);
hipError_t gemv_launch(uint32_t k, bool paired, const GemvArgs& a, uint32_t blocks,
                       hipStream_t stream);
const void* gemv_kernel_ptr(uint32_t k, bool paired);

// ------------------------------------------------------------------ GDN recurrence

struct GdnArgs {
    float* state;           // [Hv, dk, dv]
    const float* qkv_conv;  // [2*Hk*dk + Hv*dv], post conv + SiLU, pre L2
    const float* gate;      // [Hv]
    const float* beta;      // [Hv]
    float* y;               // [Hv*dv]
    float* qkv_smooth;      // optional tap [qkv_total]
    uint32_t hk, hv;
    float l2_eps;
    float out_scale;        // 1/sqrt(dk)
};
bool gdn_dims_supported(uint32_t dk, uint32_t dv);
hipError_t gdn_launch(uint32_t dk, uint32_t dv, const GdnArgs& a, hipStream_t stream);
const void* gdn_kernel_ptr(uint32_t dk);

// ------------------------------------------------------------------ attention

struct AttnArgs {
    const float* q_full;     // [Hq, 2D]: per head [Q | gate]
    const float* k;          // [Hkv*D] (pre-norm)
    const float* v;          // [Hkv*D]
    const uint16_t* q_norm;  // bf16 [D]
    const uint16_t* k_norm;  // bf16 [D]
    const float* inv_freq;   // [R/2]
    const int32_t* positions;
    uint16_t* kc;            // bf16 [cap, Hkv, D]
    uint16_t* vc;
    float* gated_attn;       // [Hq*D]
    float* attn_out;         // optional tap
    float* q_norm_out;       // optional tap (post-RoPE)
    float* k_norm_out;       // optional tap (post-RoPE)
    float* part_acc;         // workspace: [Hkv][max_chunks][G][D]
    float* part_ml;          // workspace: [Hkv][max_chunks][G][2]
    uint32_t* counters;      // workspace: [Hkv]
    uint32_t capacity;
    uint32_t hq, hkv, rotary;
    uint32_t chunk;          // positions per block
    uint32_t max_chunks;
    int32_t host_pos;        // >= 0: cache position from the host; < 0: read positions[0]
    float eps;
    float scale;
};
bool attn_dims_supported(uint32_t head_dim, uint32_t group);
uint32_t attn_rows_per_iter(uint32_t head_dim);
hipError_t attn_launch(uint32_t head_dim, uint32_t group, const AttnArgs& a, uint32_t grid_chunks,
                       hipStream_t stream);
const void* attn_kernel_ptr(uint32_t head_dim, uint32_t group);

// ------------------------------------------------------------------ misc

hipError_t embed_launch(const uint16_t* table, const int32_t* tokens, uint32_t vocab,
                        uint32_t hidden, void* x_out, bool act_f32, hipStream_t stream);
const void* embed_kernel_ptr();

}  // namespace q35
