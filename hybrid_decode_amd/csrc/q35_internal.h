// Internal interface between the C-ABI host code and the q35decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q35 {

// ------------------------------------------------------------------ GEMV family

constexpr int kMaxSegs = 6;
constexpr int kGemvThreads = 256;       // threads per block: streaming GEMVs, GDN in-projection
constexpr int kGemvLayerThreads = 640;  // threads per block of the other per-layer GEMVs (one per CU)

enum : int32_t {
    kProRmsAct = 0,     // x = RMSNorm(x_act; w)          (x in the activation dtype)
    kProRmsF32 = 1,     // x = RMSNorm(x_f32; w)
    kProGatedNorm = 2,  // x = RMSNorm_per_head(y; w) * silu(z)
    kProLoadF32 = 3,    // x = src
    kProRmsParts = 4,   // x = RMSNorm(base + sum of nparts fp32 partial vectors; w), the sum optionally
                        //     rounded to bf16 and written out by block 0
};

enum : int32_t {
    kEpiStore = 0,       // out[n] = y
    kEpiResidActIn = 1,  // out[n] = act(pre2|pre4)[n] + y       (tap0 = y)
    kEpiResidToAct = 2,  // out_act[n] = act(f32(pre4)[n] + y)   (out_act2 copy)
    kEpiConv = 3,        // causal conv update + SiLU on channel n (state = pre16, weights = pre8, tap0 = y)
    kEpiGate = 4,        // out[n] = exp(-exp(A_log = pre4[n]) softplus(y + dt_bias = pre2[n]))   (tap0 = y)
    kEpiBeta = 5,        // out[n] = sigmoid(y)                  (tap0 = y)
    kEpiSwiGLU = 6,      // paired: out[n] = silu(y_a) * y_b     (tap0 = y_a, tap1 = y_b)
    kEpiArgmax = 7,      // logits (optional out) + running argmax
};

struct GemvSeg {
    const uint8_t* codes[2];
    const uint16_t* scales[2];
    const uint16_t* biases[2];
    uint32_t rg_begin, rg_end;  // row-group range of this segment in the launch
    uint32_t rows;              // rows of each matrix of the segment
    int32_t epi;
    float* out;
    void* out_act;
    void* out_act2;
    float* tap0;
    float* tap1;
    float* state;
    // Per-row epilogue operands, fetched with the row group's weights: element
    // n of each (16, 8, 4 and 2-byte elements); NULL where the epilogue has none.
    const void* pre16;
    const void* pre8;
    const void* pre4;
    const void* pre2;
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
    // kProRmsParts (x is the base, fp32 when x_f32 else bf16)
    const float* parts;  // [nparts][K] fp32
    uint32_t nparts;     // 0..8
    int32_t sum_bf16;    // round the sum to bf16 before the norm (a layer input held in bf16)
    void* sum_out;       // optional: the sum, bf16 when sum_bf16 else fp32
};

struct GemvArgmax {
    float* part_val;    // [blocks] per-block maximum
    int32_t* part_idx;  // [blocks] its row
};

struct GemvArgs {
    GemvPro pro;
    GemvSeg seg[kMaxSegs];
    int32_t nseg;
    uint32_t total_rg;
    int32_t act_f32;
    GemvArgmax am;
};

// Operations: each GEMV launch is one of these, fixing its prologue and the
// epilogue of every segment.
enum : int32_t {
    kOpPlain = 0,     // x loaded as is; y stored                         (segments: 1)
    kOpInGdn = 1,     // RMSNorm(x_in); qkv->conv, z->store, a->gate, b->beta (4)
    kOpInFull = 2,    // RMSNorm(x_in); q, k, v stored                    (3)
    kOpOutGated = 3,  // gated per-head RMSNorm; out + residual           (1)
    kOpOProj = 4,     // x loaded; o + residual                           (1)
    kOpGateUp = 5,    // RMSNorm(x_resid); paired gate/up -> silu(g) * u  (1)
    kOpDown = 6,      // x loaded; down + residual -> activation dtype    (1)
    kOpLmHead = 7,    // RMSNorm(x); logits + argmax                      (1)
    // Variants of the above for the XCD-split decode: the residual stream
    // arrives as a base plus per-XCD partial sums, and the GEMVs of one XCD
    // cover its share of the rows (or of the columns, as a partial sum).
    kOpInFullP = 8,   // kOpInFull with the kProRmsParts prologue          (3)
    kOpInGdnX = 9,    // kOpInGdn over one XCD's rows: q, k, v (conv), z, a, b (6)
    kOpGateUpX = 10,  // kOpGateUp with the kProRmsParts prologue           (1)
    kOpOutPart = 11,  // gated norm prologue; out_proj column slice, y stored (1)
    kOpDownPart = 12, // x loaded; down column slice, y stored            (1)
};

// GEMV widths compiled in, by role.
#define Q35_W_HIDDEN(X) X(256) X(1024) X(2048) X(2560) X(3072) X(4096) X(5120) X(6144) X(8192)
// Hidden widths of the sum-of-partials prologue: the XCD-split decode, built for K / 4 <= 640 threads.
#define Q35_W_PARTS(X) X(256) X(1024) X(2048) X(2560)
#define Q35_W_PROJ(X) X(128) X(256) X(512) X(1024) X(2048) X(4096) X(6144) X(8192)
#define Q35_W_INTER(X) \
    X(512) X(1024) X(2048) X(3072) X(4096) X(5120) X(6144) X(8192) X(9216) X(12288)
#define Q35_W_ALL(X)                                                                              \
    X(128) X(256) X(512) X(1024) X(2048) X(2560) X(3072) X(4096) X(5120) X(6144) X(8192) X(9216) \
    X(12288)
enum : int { kWidthHidden = 0, kWidthProj = 1, kWidthInter = 2, kWidthAny = 3 };

constexpr int gemv_threads(int op) {
    return (op == kOpPlain || op == kOpLmHead || op == kOpInGdn) ? kGemvThreads : kGemvLayerThreads;
}

bool gemv_width_supported(int role, uint32_t k);
int gemv_rows_per_matrix_group(uint32_t k, bool paired);  // rows of each matrix per row group
uint32_t gemv_row_groups_per_wave(uint32_t total_rg);
uint32_t gemv_pick_blocks(uint32_t total_rg, int op, uint32_t num_cu);
// half: the f16-product variant used for bf16 activations (else exact fp32 products)
hipError_t gemv_launch(int op, uint32_t k, bool half, const GemvArgs& a, uint32_t blocks,
                       hipStream_t stream);
const void* gemv_kernel_ptr(int op, uint32_t k, bool half, bool xreg);

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
    uint32_t* status;        // optional: Q35_STATUS_POS_RANGE is ORed in for a position out of range
    uint16_t* ks;            // Turbo8: bf16 K group scales [cap, Hkv, D/16] (kc then holds E4M3 codes)
    uint16_t* vs;            // Turbo8: bf16 V group scales; Lloyd-Max formats: E4M3 bytes [cap, Hkv, D/16]
                             // (kc/vc of a Lloyd-Max side hold packed indices [cap, Hkv, D*bits/8])
    uint32_t capacity;
    uint32_t hq, hkv, rotary;
    uint32_t chunk;          // positions per block
    uint32_t max_chunks;
    int32_t host_pos;        // >= 0: cache position from the host; < 0: read positions[0]
    float eps;
    float scale;
    float sparse_v_log2;     // quantised formats: log2 of the sparse-V threshold (-inf: gate off)
    float lm_levels[16];     // Lloyd-Max formats: the codebook levels of the format's width
};
bool attn_dims_supported(uint32_t head_dim, uint32_t group);
uint32_t attn_rows_per_iter(uint32_t head_dim);
// Two launches: per-chunk partials, then the log-sum-exp merge with the sigmoid gate.
// kv_dtype: Q35_KV_BF16, Q35_KV_TURBO8 or Q35_KV_BF16K_TURBO4V
hipError_t attn_launch(uint32_t head_dim, uint32_t group, const AttnArgs& a, uint32_t grid_chunks,
                       uint32_t kv_dtype, hipStream_t stream);
// The partial kernel of a shape and KV format; tiles: the matrix-core tile
// variant (the quantised formats at head dimension 128 or 256 only, else null).
const void* attn_kernel_ptr(uint32_t head_dim, uint32_t group, uint32_t kv_dtype, bool tiles = false);
// Turbo8 group quantiser and E4M3 decoder of the attention kernels, over plain buffers.
hipError_t turbo8_quantize_launch(const float* x, uint32_t n, uint8_t* codes, uint16_t* scales,
                                  hipStream_t stream);
hipError_t e4m3_table_launch(float* out256, hipStream_t stream);
struct LmLevels {
    float v[16];
};
hipError_t lm_quantize_launch(uint32_t bits, const float* x, uint32_t n, const LmLevels& levels, uint8_t* packed,
                              uint8_t* scales, hipStream_t stream);
const void* attn_combine_kernel_ptr(uint32_t head_dim, uint32_t group);

// ------------------------------------------------------------------ misc

hipError_t embed_launch(const uint16_t* table, const int32_t* tokens, uint32_t vocab,
                        uint32_t hidden, void* x_out, bool act_f32, hipStream_t stream);
const void* embed_kernel_ptr();
// Device address and size of the fixed workspace (the current device's copy).
hipError_t static_scratch_address(void** ptr, size_t* bytes);

// Greedy token from the lm_head's per-block partials, then the caller's
// bookkeeping: history entry, position increment, next embedding.
struct LmFinishArgs {
    const float* part_val;
    const int32_t* part_idx;
    uint32_t nparts;
    uint32_t vocab;
    int32_t* tokens;
    int32_t* positions;
    int32_t* history;
    uint32_t history_len;
    int32_t history_base;
    const uint16_t* embed;
    void* x_next;
    uint32_t hidden;
    int32_t act_f32;
};
hipError_t lm_finish_launch(const LmFinishArgs& a, hipStream_t stream);
const void* lm_finish_kernel_ptr();

// ------------------------------------------------------------------ persistent decode

// One cooperative launch runs a table of stages (a token through the stack).
constexpr int kPersistThreads = 1024;  // threads per block; one block per CU

enum : int32_t {
    kStInGdn = 1,   // GEMV kOpInGdn
    kStGdn,         // gated delta rule
    kStOutGated,    // GEMV kOpOutGated
    kStInFull,      // GEMV kOpInFull
    kStAttn,        // attention partials (q/k norm, RoPE, KV append)
    kStAttnMerge,   // log-sum-exp merge + sigmoid gate
    kStOProj,       // GEMV kOpOProj
    kStGateUp,      // GEMV kOpGateUp
    kStDown,        // GEMV kOpDown
    kStLmHead,      // GEMV kOpLmHead (per-block argmax partials)
    kStFinish,      // block 0: greedy token, bookkeeping, next embedding
};

struct PStage {
    int32_t kind;
    int32_t pad;
    union {
        GemvArgs g;
        GdnArgs d;
        AttnArgs at;  // max_chunks = chunks per kv head (blocks / Hkv)
        LmFinishArgs f;
    };
};

struct PersistArgs {
    const PStage* stages;  // device, [nstages]
    uint32_t nstages;
    uint32_t* flags;       // [blocks] stages completed (wrapping)
    uint32_t* ctl;         // [0] epoch (launches completed), [1] error (a wait expired)
    uint64_t* stamps;      // optional [nstages]: block 0's time at each stage's start
    uint64_t spin_ticks;   // wall-clock ticks before a wait gives up
};

// 1: Qwen3.5-4B shapes with bf16 activations; 2: the tiny fp32 shapes; 0: none.
int persist_shape_id(uint32_t hidden, uint32_t inter, uint32_t q_only, uint32_t z_dim, uint32_t dk,
                     uint32_t head_dim, uint32_t group, bool half);
size_t persist_lds_bytes(int shape);
const void* persist_kernel_ptr(int shape);
hipError_t persist_launch(int shape, const PersistArgs& a, uint32_t blocks, hipStream_t stream);

// ------------------------------------------------------------------ XCD-split decode

// A launch runs a fixed sequence of stages; block b works for XCD b % 8 (the
// hardware's placement of a one-block-per-CU grid, checked in the kernel) and
// the blocks of one XCD meet at a counter in that XCD's L2 between stages.
constexpr int kXcds = 8;
constexpr int kXcdThreads = 1024;  // threads per block; one block per CU

enum : int32_t {
    kXsInGdn = 1,     // GEMV kOpInGdnX (first stage of a launch)
    kXsGdn = 2,       // gated delta rule tiles of the XCD's v-heads
    kXsOutPart = 3,   // GEMV kOpOutPart: out_proj over the XCD's y columns -> partial
    kXsGateUp = 4,    // GEMV kOpGateUpX (first stage of a launch)
    kXsDownPart = 5,  // GEMV kOpDownPart: down over the XCD's activation columns -> partial
};

struct XStage {  // one XCD's arguments of one stage
    int32_t kind;
    int32_t pad;
    union {
        GemvArgs g;
        GdnArgs d;
    };
};

struct XcdArgs {
    const XStage* table;  // device, [stages of the launch][kXcds]
    uint32_t* sync;       // [kXcds][64]: XCD x's counter at sync[64 x] (monotonic)
    uint32_t* err;        // error word: bit 0 a wait expired, Q35_STATUS_XCD_MAP a block off its XCD
    uint64_t spin_ticks;  // wall-clock ticks before a wait gives up
    uint32_t* probe;      // non-NULL: each block writes its XCD id to probe[blockIdx.x] and exits
};

// The two launches: the GDN mixer (stages kXsInGdn, kXsGdn, kXsOutPart) and
// the MLP (kXsGateUp, kXsDownPart); XcdArgs::table points at the launch's first stage.
enum : int { kXcdMixer = 0, kXcdMlp = 1 };
constexpr uint32_t kXcdStages[2] = {3, 2};

// 1: the Qwen3.5-4B shapes with bf16 activations; 0: not built.
int xcd_shape_id(uint32_t hidden, uint32_t inter, uint32_t z_dim, uint32_t dk, bool half);
const void* xcd_kernel_ptr(int shape, int launch);
hipError_t xcd_launch(int shape, int launch, const XcdArgs& a, uint32_t blocks, hipStream_t stream);
// out = base + parts[0] + ... + parts[nparts-1] (fp32, in that order), stored in
// the activation dtype: the residual stream of the XCD-split decode made whole.
hipError_t xsum_launch(const void* base, bool base_f32, const float* parts, uint32_t nparts, uint32_t n,
                       void* out, bool out_f32, hipStream_t stream);
const void* xsum_kernel_ptr();

// ------------------------------------------------------------------ prefill (T tokens per launch)

enum { kPfF32 = 0, kPfResid = 1, kPfSwiglu = 2 };

// out[m, n] = sum_k x[m, k] W[n, k]: x f16 [M, K]; W 8-bit codes with bf16 scale/bias
// per 64.  kPfF32: W is up to four matrices stacked by rows (segment i holds rows
// [seg_end[i-1], seg_end[i]) and writes fp32 out[i] with row stride ldo[i]).
// kPfResid: one matrix, out[0] = resid + product (resid and out fp32 or bf16 per
// flag).  kPfSwiglu: w[0] gate, w[1] up, out[0] f16 silu(gate) * up.
struct PfGemmArgs {
    const uint16_t* x;
    const uint8_t* w[4];
    const uint16_t* s[4];
    const uint16_t* b[4];
    const uint16_t* wh[4];     // the same matrices already dequantised to f16 [n, K] (NULL: from the codes)
    void* out[4];
    uint32_t ldo[4];
    uint32_t seg_end[4];       // cumulative; unused entries equal N
    const void* resid;
    uint32_t M, N, K;
    uint32_t resid_f32, out_f32;
    float* part;               // fp32 partial tiles of a split last round (NULL: never split)
    uint32_t n_full, split;    // set by the launcher
};
// Most blocks of split k ranges one launch holds: kPfSplitBlocks partial tiles of
// 256 x 128 fp32 (32 MiB).
constexpr uint32_t kPfSplitBlocks = 256;
constexpr size_t kPfSplitBytes = (size_t)kPfSplitBlocks * 256 * 128 * 4;
hipError_t pf_gemm_launch(int mode, const PfGemmArgs& a, uint32_t num_cu, hipStream_t s);
// out (f16 [rows, K]) = scale * code + bias in fp32, rounded once to f16: the
// values the GEMM would build from the codes (K a multiple of 64)
hipError_t pf_dequant_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                             uint32_t rows, uint32_t K, uint16_t* out, hipStream_t s);
// f16 rows of RMSNorm(x) for T rows of H (x fp32 or bf16)
hipError_t pf_rmsnorm_launch(const void* x, bool x_f32, const uint16_t* w, uint16_t* out, uint32_t T,
                             uint32_t H, float eps, hipStream_t s);

struct PfConvArgs {
    const float* qkv;          // [T, C] conv inputs
    const float* conv_state;   // [C, 4] before the first token
    const uint16_t* conv_w;    // bf16 [C, 4]
    const float* a_raw;        // [T, hv]
    const float* b_raw;        // [T, hv]
    const float* a_log;        // [hv]
    const uint16_t* dt_bias;   // bf16 [hv]
    float* qkvs;               // [T, C] conv + SiLU, Q/K heads L2-normalised
    float* lg;                 // [T, hv] log of the decay gate
    float* beta;               // [T, hv]
    uint32_t T, C, nqk, dk, hv;
};
struct PfGdnArgs {
    const float* qkvs;
    const float* lg;
    const float* beta;
    float* Wc;                 // [hv, nch, 64, dk]
    float* Uc;                 // [hv, nch, 64, dv]
    float* Pc;                 // [hv, nch, 64, 64]
    float* Lc;                 // [hv, nch, 64]
    float* y;                  // [T, hv * dv]
    float* state;              // [hv, dk, dv], updated
    uint32_t T, C, hk, hv, dk, dv, nch;
    float out_scale;
};
bool pf_gdn_dims_supported(uint32_t dk, uint32_t dv);
// conv, conv-state advance, chunk build and the state scan
hipError_t pf_gdn_launch(const PfConvArgs& c, const PfGdnArgs& g, float* conv_state_out, hipStream_t s);
hipError_t pf_gdn_out_launch(const float* y, const float* z, const uint16_t* w, uint16_t* yz, uint32_t T,
                             uint32_t hv, uint32_t dv, float eps, hipStream_t s);

struct PfRopeArgs {
    const float* q_full;       // [T, hq * 2D]
    const float* k;            // [T, hkv * D]
    const float* v;            // [T, hkv * D]
    const uint16_t* q_norm;
    const uint16_t* k_norm;
    const float* inv_freq;
    uint16_t* qb;              // f16 [T, hq, D]
    uint16_t* kc;              // bf16 cache [cap, hkv, D]
    uint16_t* vc;
    uint32_t T, cache_pos, hq, hkv, D, rotary;
    float eps;
};
struct PfAttnArgs {
    const uint16_t* qb;
    const float* q_full;       // gate halves
    const uint16_t* kc;
    const uint16_t* vc;
    uint16_t* ga;              // f16 [T, hq * D]
    uint32_t T, cache_pos, hq, hkv;
    float scale_log2;
};
// A prompt into a quantised cache (head dimension 128 or 256): the rows of
// the T tokens appended to the cache as the decode steps would append them,
// then a causal attention of every token over the rows as stored (sparse-V
// gate, sigmoid gate) into ga.  Two launches; qh is f16 scratch [T, hq, D].
struct PfQuantAttnArgs {
    const float* q_full;       // [T, hq * 2D]: q, then the gate, per head
    const float* k;            // [T, hkv * D]
    const float* v;            // [T, hkv * D]
    const uint16_t* q_norm;
    const uint16_t* k_norm;
    const float* inv_freq;
    void* kc;                  // the cache sides (formats as the decode attention's)
    void* vc;
    void* ks;                  // key group scales (null for bf16 keys)
    void* vs;
    uint16_t* qh;              // f16 [T, hq, D]: the prepared query heads
    uint16_t* ga;              // f16 [T, hq * D]: gated attention output
    uint32_t T, cache_pos, hq, hkv, rotary;
    float eps, scale, sparse_v_log2;
    float lm_levels[16];       // Lloyd-Max formats: the codebook levels of the format's width
};
bool pf_quant_attn_supported(uint32_t head_dim, uint32_t group, uint32_t kv_dtype);
hipError_t pf_quant_attn_launch(uint32_t head_dim, uint32_t group, uint32_t kv_dtype, const PfQuantAttnArgs& a,
                                hipStream_t stream);
const void* pf_quant_kernel_ptr(uint32_t head_dim, uint32_t group, uint32_t kv_dtype, bool flash);
bool pf_attn_dims_supported(uint32_t head_dim, uint32_t group);
hipError_t pf_attn_launch(const PfRopeArgs& r, const PfAttnArgs& a, hipStream_t s);
// The prompt's cache positions base + i into out[n], and an fp32 -> f16 cast
// (the per-token attention path of a quantised cache).
hipError_t pf_iota_launch(int32_t* out, uint32_t n, int32_t base, hipStream_t s);
hipError_t pf_cast_f16_launch(const float* x, uint16_t* y, uint32_t n, hipStream_t s);
// the prefill kernels, i = 0, 1, ... until nullptr (for the load check at resolve)
const void* pf_kernel_ptr(int i);

}  // namespace q35
