// C-ABI of q35decode: validation, launch geometry and kernel sequencing for the
// single-token Qwen3.5 layer forwards.  No device memory is allocated here;
// every call enqueues on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <initializer_list>
#include <string>
#include <vector>

#include "../../include/q35decode.h"
#include "q35_internal.h"

using namespace q35;

struct Qwen35Kernels {
    int device;
    int num_cu;
    q35::LmLevels lm[5];  // Lloyd-Max codebooks of 2, 3 and 4 bits (computed at resolve)
    void* scratch;        // this device's copy of the fixed workspace (no-alloc entry points)
    size_t scratch_bytes;
};

namespace {

thread_local std::string g_err;

q35_status fail(q35_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

q35_status ok() {
    g_err.clear();
    return Q35_OK;
}

#define Q35_TRY(expr)                                  \
    do {                                               \
        q35_status st__ = (expr);                      \
        if (st__ != Q35_OK) return st__;               \
    } while (0)

#define Q35_HIP(expr, what)                                                               \
    do {                                                                                  \
        hipError_t e__ = (expr);                                                          \
        if (e__ != hipSuccess) return fail(Q35_ERR_HIP, "%s: %s", what, hipGetErrorString(e__)); \
    } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

uint32_t q_total(const Qwen35ForwardConfig& c) { return 2 * c.num_heads * c.head_dim; }
uint32_t q_only(const Qwen35ForwardConfig& c) { return c.num_heads * c.head_dim; }
uint32_t kv_dim(const Qwen35ForwardConfig& c) { return c.num_kv_heads * c.head_dim; }
uint32_t z_dim(const Qwen35ForwardConfig& c) { return c.num_v_heads_lin * c.v_head_dim_lin; }
uint32_t qkv_total(const Qwen35ForwardConfig& c) {
    return 2 * c.num_k_heads_lin * c.k_head_dim_lin + z_dim(c);
}

q35_status check_rows(const char* what, uint32_t rows, uint32_t k, bool paired = false) {
    const int r = gemv_rows_per_matrix_group(k, paired);
    if (rows == 0 || rows % (uint32_t)r != 0)
        return fail(Q35_ERR_UNSUPPORTED, "%s: %u rows is not a multiple of %d (rows per wave group at K=%u)",
                    what, rows, r, k);
    return Q35_OK;
}

q35_status check_weight(const char* what, const Q35QuantWeight& w, uint32_t n, uint32_t k) {
    if (!w.codes || !w.scales || !w.biases) return fail(Q35_ERR_INVALID_ARG, "%s: NULL pointer", what);
    if (w.n != n || w.k != k)
        return fail(Q35_ERR_INVALID_ARG, "%s: shape [%u, %u], expected [%u, %u]", what, w.n, w.k, n, k);
    if (!aligned16(w.codes)) return fail(Q35_ERR_INVALID_ARG, "%s: codes not 16-byte aligned", what);
    return Q35_OK;
}

q35_status need(const void* p, const char* what, bool vec = true) {
    if (!p) return fail(Q35_ERR_INVALID_ARG, "%s is NULL", what);
    if (vec && !aligned16(p)) return fail(Q35_ERR_INVALID_ARG, "%s not 16-byte aligned", what);
    return Q35_OK;
}

q35_status opt(const void* p, const char* what) {
    if (p && !aligned16(p)) return fail(Q35_ERR_INVALID_ARG, "%s not 16-byte aligned", what);
    return Q35_OK;
}

// Attention split-K geometry: positions per block for a cache length n, and
// the number of per-chunk partial slots a workspace must hold for a capacity.
constexpr uint32_t kAttnTargetBlocks = 512;
constexpr uint32_t kAttnMaxChunk = 2048;

// Rows per block: the share of kAttnTargetBlocks blocks, rounded up to whole
// iterations.  Measured at position 8192 (attention steps of 8 layers): chunks
// of 96 rows (344 blocks) 17.8 us a layer, 64 rows (516 blocks) 21.0 us, 128
// rows (260 blocks) 19.7 us; more blocks repeat the q prologue more often.
uint32_t attn_chunk(const Qwen35ForwardConfig& c, uint32_t n) {
    const uint32_t rpi = attn_rows_per_iter(c.head_dim);
    uint64_t want = ((uint64_t)n * c.num_kv_heads + kAttnTargetBlocks - 1) / kAttnTargetBlocks;
    uint64_t t = ((want + rpi - 1) / rpi) * rpi;
    if (t < rpi) t = rpi;
    if (t > kAttnMaxChunk) t = kAttnMaxChunk;
    return (uint32_t)t;
}

uint32_t attn_max_chunks(const Qwen35ForwardConfig& c, uint32_t capacity) {
    uint32_t a = kAttnTargetBlocks / c.num_kv_heads + 2;
    uint32_t b = (capacity + kAttnMaxChunk - 1) / kAttnMaxChunk + 1;
    return a > b ? a : b;
}

struct AttnWs {
    size_t acc_off, ml_off, total;
};

AttnWs attn_ws_layout(const Qwen35ForwardConfig& c, uint32_t capacity) {
    const uint32_t G = c.num_heads / c.num_kv_heads;
    const size_t mc = attn_max_chunks(c, capacity);
    AttnWs w;
    w.acc_off = 0;
    w.ml_off = (mc * c.num_kv_heads * G * c.head_dim * sizeof(float) + 255) & ~size_t(255);
    w.total = w.ml_off + ((mc * c.num_kv_heads * 2 * G * sizeof(float) + 255) & ~size_t(255));
    return w;
}

struct LmWs {
    size_t val_off, idx_off, total;
    uint32_t blocks;
};

LmWs lm_ws_layout(const Qwen35ForwardConfig& c) {
    LmWs w;
    const uint32_t r = (uint32_t)gemv_rows_per_matrix_group(c.hidden, false);
    w.blocks = gemv_pick_blocks(c.vocab / r, kOpLmHead, 0);  // streaming shape: no CU count needed
    w.val_off = 0;
    w.idx_off = ((size_t)w.blocks * 4 + 255) & ~size_t(255);
    w.total = w.idx_off + (((size_t)w.blocks * 4 + 255) & ~size_t(255));
    return w;
}

// A GEMV launch under construction: segments over one shared x.
struct GemvBuild {
    GemvArgs a;
    int op;
    uint32_t k;
    bool paired;
    uint32_t r;  // rows of one matrix per row group

    GemvBuild(int op_, uint32_t k_, bool act_f32) : op(op_), k(k_), paired(op_ == kOpGateUp) {
        std::memset(&a, 0, sizeof(a));
        a.act_f32 = act_f32 ? 1 : 0;
        r = (uint32_t)gemv_rows_per_matrix_group(k, paired);
    }
    GemvSeg& add(const Q35QuantWeight& w, int32_t epi, const Q35QuantWeight* w2 = nullptr) {
        GemvSeg& s = a.seg[a.nseg++];
        s.codes[0] = w.codes;
        s.scales[0] = w.scales;
        s.biases[0] = w.biases;
        if (w2) {
            s.codes[1] = w2->codes;
            s.scales[1] = w2->scales;
            s.biases[1] = w2->biases;
        }
        s.rg_begin = a.total_rg;
        s.rows = w.n;
        a.total_rg += w.n / r;
        s.rg_end = a.total_rg;
        s.epi = epi;
        return s;
    }
    q35_status launch(uint32_t num_cu, hipStream_t stream, const char* what, uint32_t blocks = 0) {
        if (!blocks) blocks = gemv_pick_blocks(a.total_rg, op, num_cu);
        Q35_HIP(gemv_launch(op, k, a.act_f32 == 0, a, blocks, stream), what);
        return Q35_OK;
    }
};

// gate/up (paired, SwiGLU epilogue) and down (+ residual) shared by both layers.
q35_status launch_mlp(uint32_t num_cu, const Qwen35ForwardConfig& c, const Q35QuantWeight& gate_proj,
                      const Q35QuantWeight& up_proj, const Q35QuantWeight& down_proj,
                      const uint16_t* post_ln, float* x_resid, float* x_norm2, float* mlp_act,
                      float* gate_act, float* up_act, void* x_out, void* x_out2,
                      hipStream_t stream) {
    const bool f32 = c.act_dtype == Q35_ACT_F32;
    {
        GemvBuild b(kOpGateUp, c.hidden, f32);
        b.a.pro.kind = kProRmsF32;
        b.a.pro.x = x_resid;
        b.a.pro.w = post_ln;
        b.a.pro.eps = c.rms_eps;
        b.a.pro.tap = x_norm2;
        GemvSeg& s = b.add(gate_proj, kEpiSwiGLU, &up_proj);
        s.out = mlp_act;
        s.tap0 = gate_act;
        s.tap1 = up_act;
        Q35_TRY(b.launch(num_cu, stream, "gate/up GEMV"));
    }
    {
        GemvBuild b(kOpDown, c.intermediate, f32);
        b.a.pro.kind = kProLoadF32;
        b.a.pro.x = mlp_act;
        GemvSeg& s = b.add(down_proj, kEpiResidToAct);
        s.pre4 = x_resid;
        s.out_act = x_out;
        s.out_act2 = x_out2;
        Q35_TRY(b.launch(num_cu, stream, "down GEMV"));
    }
    return Q35_OK;
}

q35_status check_full_layer(const Qwen35ForwardConfig& c, const FullAttentionLayer& l) {
    Q35_TRY(need(l.input_ln, "input_ln"));
    Q35_TRY(need(l.q_norm, "q_norm"));
    Q35_TRY(need(l.k_norm, "k_norm"));
    Q35_TRY(need(l.post_ln, "post_ln"));
    Q35_TRY(check_weight("q_proj", l.q_proj, q_total(c), c.hidden));
    Q35_TRY(check_weight("k_proj", l.k_proj, kv_dim(c), c.hidden));
    Q35_TRY(check_weight("v_proj", l.v_proj, kv_dim(c), c.hidden));
    Q35_TRY(check_weight("o_proj", l.o_proj, c.hidden, q_only(c)));
    Q35_TRY(check_weight("gate_proj", l.gate_proj, c.intermediate, c.hidden));
    Q35_TRY(check_weight("up_proj", l.up_proj, c.intermediate, c.hidden));
    Q35_TRY(check_weight("down_proj", l.down_proj, c.hidden, c.intermediate));
    return Q35_OK;
}

// The Lloyd-Max codebooks (mod.rs: the Turbo4/3/2 variants' Lloyd-Max indices;
// the level values are not given there): the n-level Lloyd-Max quantiser of
// the standard normal distribution.  Lloyd's iteration in double precision --
// thresholds halfway between adjacent levels, each level moved to the mean of
// N(0, 1) over its cell -- until no level moves, then made exactly symmetric
// and rounded to float.
double normal_cell_mean(double lo, double hi) {
    const double r2 = std::sqrt(2.0), r2pi = std::sqrt(2.0 * 3.14159265358979323846);
    auto pdf = [&](double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) / r2pi; };
    double mass;  // from the tail on the far side of 0, so small cells keep their digits
    if (lo >= 0.0)
        mass = 0.5 * (std::erfc(lo / r2) - std::erfc(hi / r2));
    else if (hi <= 0.0)
        mass = 0.5 * (std::erfc(-hi / r2) - std::erfc(-lo / r2));
    else
        mass = 1.0 - 0.5 * std::erfc(-lo / r2) - 0.5 * std::erfc(hi / r2);
    return (pdf(lo) - pdf(hi)) / mass;
}

void lloyd_max_normal(int n, float* out) {  // n <= 16 levels; out[n..16) = 0
    double c[16] = {};
    for (int i = 0; i < n; ++i) c[i] = -2.5 + 5.0 * i / (n - 1);
    for (int it = 0; it < 20000; ++it) {
        double nc[16] = {}, moved = 0.0;
        for (int i = 0; i < n; ++i) {
            const double lo = i == 0 ? -INFINITY : 0.5 * (c[i - 1] + c[i]);
            const double hi = i == n - 1 ? INFINITY : 0.5 * (c[i] + c[i + 1]);
            nc[i] = normal_cell_mean(lo, hi);
            moved = std::max(moved, std::fabs(nc[i] - c[i]));
        }
        std::memcpy(c, nc, sizeof(c));
        if (moved < 1e-15) break;
    }
    for (int i = 0; i < 16; ++i) out[i] = i < n ? (float)((c[i] - c[n - 1 - i]) / 2.0) : 0.0f;
}

// Index bits of a Lloyd-Max KV format (0 for the others) and whether its K is
// quantised as well.
int kv_lm_bits(uint32_t dt) {
    switch (dt) {
        case Q35_KV_TURBO4: case Q35_KV_BF16K_TURBO4V: return 4;
        case Q35_KV_TURBO3: case Q35_KV_BF16K_TURBO3V: return 3;
        case Q35_KV_TURBO2: case Q35_KV_BF16K_TURBO2V: return 2;
        default: return 0;
    }
}
bool kv_lm_k(uint32_t dt) { return dt == Q35_KV_TURBO4 || dt == Q35_KV_TURBO3 || dt == Q35_KV_TURBO2; }

// bf16 everywhere; in the per-layer forward also Turbo8 (E4M3 codes + bf16
// scales per 16) and the Lloyd-Max formats (packed indices + E4M3 scale bytes
// per 16; K too for the symmetric ones, K bf16 for Bf16K + TurboNV).
q35_status check_kv(const LayerKvCache& kv, bool allow_quantised) {
    if (kv.dtype == Q35_KV_BF16) {
        if (kv.k_scales || kv.v_scales) return fail(Q35_ERR_INVALID_ARG, "bf16 cache with scale buffers");
    } else if (allow_quantised && kv.dtype <= Q35_KV_BF16K_TURBO2V) {
        const bool k_quant = kv.dtype == Q35_KV_TURBO8 || kv_lm_k(kv.dtype);
        if (k_quant) {
            Q35_TRY(need(kv.k_scales, "kv.k_scales", false));
        } else if (kv.k_scales) {
            return fail(Q35_ERR_INVALID_ARG, "KV dtype %u keeps K in bf16: no K scale buffer", kv.dtype);
        }
        Q35_TRY(need(kv.v_scales, "kv.v_scales", false));
        if (kv.dtype == Q35_KV_TURBO8 &&
            ((reinterpret_cast<uintptr_t>(kv.k_scales) | reinterpret_cast<uintptr_t>(kv.v_scales)) & 1u))
            return fail(Q35_ERR_INVALID_ARG, "turbo8 scales not 2-byte aligned");
        if (!(kv.sparse_v >= 0.0f && kv.sparse_v <= 3.0e38f))  // also rejects NaN and +inf
            return fail(Q35_ERR_INVALID_ARG, "sparse_v %g must be finite and >= 0", (double)kv.sparse_v);
    } else {
        return fail(Q35_ERR_UNSUPPORTED, "KV dtype %u is not implemented on this path (%s)", kv.dtype,
                    allow_quantised ? "bf16 | turbo8 | turbo4/3/2 | bf16k_turbo4v/3v/2v" : "bf16");
    }
    Q35_TRY(need(kv.k, "kv.k"));
    Q35_TRY(need(kv.v, "kv.v"));
    if (kv.capacity == 0) return fail(Q35_ERR_OUT_OF_RANGE, "cache capacity is 0");
    return Q35_OK;
}

q35_status check_linear_layer(const Qwen35ForwardConfig& c, const LinearAttentionLayer& l,
                              const LinearAttentionState& st) {
    const uint32_t Hv = c.num_v_heads_lin;
    Q35_TRY(need(st.conv1d_state, "state.conv1d_state"));
    Q35_TRY(need(st.gdn_state, "state.gdn_state"));
    Q35_TRY(need(l.input_ln, "input_ln"));
    Q35_TRY(need(l.post_ln, "post_ln"));
    Q35_TRY(need(l.norm_weight, "norm_weight"));
    Q35_TRY(need(l.a_log, "a_log", false));
    Q35_TRY(need(l.dt_bias, "dt_bias", false));
    if (!l.conv1d_weight || !aligned8(l.conv1d_weight))
        return fail(Q35_ERR_INVALID_ARG, "conv1d_weight NULL or not 8-byte aligned");
    Q35_TRY(check_weight("in_proj_a", l.in_proj_a, Hv, c.hidden));
    Q35_TRY(check_weight("in_proj_b", l.in_proj_b, Hv, c.hidden));
    Q35_TRY(check_weight("in_proj_qkv", l.in_proj_qkv, qkv_total(c), c.hidden));
    Q35_TRY(check_weight("in_proj_z", l.in_proj_z, z_dim(c), c.hidden));
    Q35_TRY(check_weight("out_proj", l.out_proj, c.hidden, z_dim(c)));
    Q35_TRY(check_weight("gate_proj", l.gate_proj, c.intermediate, c.hidden));
    Q35_TRY(check_weight("up_proj", l.up_proj, c.intermediate, c.hidden));
    Q35_TRY(check_weight("down_proj", l.down_proj, c.hidden, c.intermediate));
    return Q35_OK;
}

q35_status check_kernels(const Qwen35Kernels* k) {
    if (!k) return fail(Q35_ERR_INVALID_ARG, "kernels handle is NULL (call q35_kernels_resolve)");
    return Q35_OK;
}

}  // namespace

extern "C" {

const char* q35_last_error(void) { return g_err.c_str(); }

q35_status q35_config_qwen3_5_4b(Qwen35ForwardConfig* cfg) {
    if (!cfg) return fail(Q35_ERR_INVALID_ARG, "cfg is NULL");
    Qwen35ForwardConfig c;
    c.hidden = 2560;
    c.intermediate = 9216;
    c.num_layers = 32;
    c.vocab = 248320;
    c.group_size = 64;
    c.rms_eps = 1e-6f;
    c.num_heads = 16;
    c.num_kv_heads = 4;
    c.head_dim = 256;
    c.rope_theta = 10000000.0f;
    c.rotary_dim = 64;
    c.num_k_heads_lin = 16;
    c.num_v_heads_lin = 32;
    c.k_head_dim_lin = 128;
    c.v_head_dim_lin = 128;
    c.conv_kernel_size = 4;
    c.act_dtype = Q35_ACT_BF16;
    *cfg = c;
    return ok();
}

q35_status q35_config_validate(const Qwen35ForwardConfig* cfg) {
    if (!cfg) return fail(Q35_ERR_INVALID_ARG, "cfg is NULL");
    const Qwen35ForwardConfig& c = *cfg;
    if (c.group_size != 64) return fail(Q35_ERR_UNSUPPORTED, "group_size %u (only 64)", c.group_size);
    if (c.act_dtype != Q35_ACT_BF16 && c.act_dtype != Q35_ACT_F32)
        return fail(Q35_ERR_INVALID_ARG, "act_dtype %u", c.act_dtype);
    if (!(c.rms_eps > 0.0f) || !std::isfinite(c.rms_eps))
        return fail(Q35_ERR_INVALID_ARG, "rms_eps must be positive");
    if (c.num_heads == 0 || c.num_kv_heads == 0 || c.num_heads % c.num_kv_heads)
        return fail(Q35_ERR_INVALID_ARG, "num_heads %u not a multiple of num_kv_heads %u", c.num_heads,
                    c.num_kv_heads);
    if (!attn_dims_supported(c.head_dim, c.num_heads / c.num_kv_heads))
        return fail(Q35_ERR_UNSUPPORTED, "head_dim %u with %u q heads per kv head", c.head_dim,
                    c.num_heads / c.num_kv_heads);
    if (c.rotary_dim == 0 || c.rotary_dim % 2 || c.rotary_dim > c.head_dim)
        return fail(Q35_ERR_INVALID_ARG, "rotary_dim %u (even, <= head_dim)", c.rotary_dim);
    if (c.num_k_heads_lin == 0 || c.num_v_heads_lin % c.num_k_heads_lin)
        return fail(Q35_ERR_INVALID_ARG, "num_v_heads_lin %u not a multiple of num_k_heads_lin %u",
                    c.num_v_heads_lin, c.num_k_heads_lin);
    if (!gdn_dims_supported(c.k_head_dim_lin, c.v_head_dim_lin))
        return fail(Q35_ERR_UNSUPPORTED, "k/v head dims %u/%u (equal, 32/64/128)", c.k_head_dim_lin,
                    c.v_head_dim_lin);
    if (c.conv_kernel_size != 4)
        return fail(Q35_ERR_UNSUPPORTED, "conv_kernel_size %u (only 4)", c.conv_kernel_size);
    const uint32_t widths[4] = {c.hidden, c.intermediate, q_only(c), z_dim(c)};
    const int roles[4] = {kWidthHidden, kWidthInter, kWidthProj, kWidthProj};
    const char* names[4] = {"hidden", "intermediate", "q_only", "z_dim_lin"};
    for (int i = 0; i < 4; ++i) {
        if (widths[i] == 0 || widths[i] % 64)
            return fail(Q35_ERR_INVALID_ARG, "%s %u not a multiple of 64", names[i], widths[i]);
        if (!gemv_width_supported(roles[i], widths[i]))
            return fail(Q35_ERR_UNSUPPORTED, "%s %u is not a compiled GEMV width", names[i], widths[i]);
    }
    // output rows of every GEMV must tile the per-wave row groups
    Q35_TRY(check_rows("q_proj", q_total(c), c.hidden));
    Q35_TRY(check_rows("k_proj/v_proj", kv_dim(c), c.hidden));
    Q35_TRY(check_rows("in_proj_qkv", qkv_total(c), c.hidden));
    Q35_TRY(check_rows("in_proj_z", z_dim(c), c.hidden));
    Q35_TRY(check_rows("in_proj_a/b", c.num_v_heads_lin, c.hidden));
    Q35_TRY(check_rows("gate/up", c.intermediate, c.hidden, true));
    Q35_TRY(check_rows("o_proj", c.hidden, q_only(c)));
    Q35_TRY(check_rows("out_proj", c.hidden, z_dim(c)));
    Q35_TRY(check_rows("down_proj", c.hidden, c.intermediate));
    if (c.vocab) Q35_TRY(check_rows("lm_head", c.vocab, c.hidden));
    return ok();
}

q35_status q35_rope_inv_freq(const Qwen35ForwardConfig* cfg, float* host_out) {
    if (!cfg || !host_out) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    const uint32_t r = cfg->rotary_dim;
    if (r == 0 || r % 2) return fail(Q35_ERR_INVALID_ARG, "rotary_dim %u", r);
    for (uint32_t i = 0; i < r / 2; ++i)
        host_out[i] = (float)std::pow((double)cfg->rope_theta, -2.0 * (double)i / (double)r);
    return ok();
}

q35_status q35_kernels_resolve(int device, Qwen35Kernels** out) {
    if (!out) return fail(Q35_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n == 0) return fail(Q35_ERR_NO_DEVICE, "no HIP device");
    if (device < 0 || device >= n) return fail(Q35_ERR_NO_DEVICE, "device %d of %d", device, n);
    hipDeviceProp_t prop;
    Q35_HIP(hipGetDeviceProperties(&prop, device), "hipGetDeviceProperties");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(Q35_ERR_NO_DEVICE, "device %d is %s, this library is built for gfx950", device,
                    prop.gcnArchName);
    int prev = 0;
    Q35_HIP(hipGetDevice(&prev), "hipGetDevice");
    Q35_HIP(hipSetDevice(device), "hipSetDevice");
    q35_status st = Q35_OK;
    auto probe = [&](const void* fn, const char* name) {
        if (st != Q35_OK) return;
        hipFuncAttributes attr;
        hipError_t e = hipFuncGetAttributes(&attr, fn);
        if (e != hipSuccess) st = fail(Q35_ERR_HIP, "kernel %s does not load: %s", name, hipGetErrorString(e));
    };
    const int ops_hidden[] = {kOpInGdn, kOpInFull, kOpGateUp, kOpLmHead};
    for (bool half : {false, true}) {
#define X(KK)                                                                        \
        probe(gemv_kernel_ptr(kOpPlain, KK, half, false), "gemv");                  \
        probe(gemv_kernel_ptr(kOpPlain, KK, half, true), "gemv (streaming)");
        Q35_W_ALL(X)
#undef X
#define X(KK)                                                                           \
        for (int op : ops_hidden) probe(gemv_kernel_ptr(op, KK, half, false), "gemv");  \
        probe(gemv_kernel_ptr(kOpLmHead, KK, half, true), "lm_head");
        Q35_W_HIDDEN(X)
#undef X
#define X(KK)                                                          \
        probe(gemv_kernel_ptr(kOpOutGated, KK, half, false), "out_proj"); \
        probe(gemv_kernel_ptr(kOpOProj, KK, half, false), "o_proj");
        Q35_W_PROJ(X)
#undef X
#define X(KK) probe(gemv_kernel_ptr(kOpDown, KK, half, false), "down");
        Q35_W_INTER(X)
#undef X
    }
    for (uint32_t dk : {32u, 64u, 128u}) probe(gdn_kernel_ptr(dk), "gated_delta_rule");
    for (uint32_t d : {64u, 128u, 256u})
        for (uint32_t g : {1u, 2u, 4u, 8u})
            for (uint32_t f : {Q35_KV_BF16, Q35_KV_TURBO8, Q35_KV_BF16K_TURBO4V})
                probe(attn_kernel_ptr(d, g, f), "attention");
    for (uint32_t d : {128u, 256u})
        for (uint32_t g : {1u, 2u, 4u, 8u})
            for (uint32_t f : {Q35_KV_TURBO8, Q35_KV_TURBO4, Q35_KV_BF16K_TURBO4V})
                probe(attn_kernel_ptr(d, g, f, true), "attention tiles");
    for (int i = 0; pf_kernel_ptr(i); ++i) probe(pf_kernel_ptr(i), "prefill");
    for (uint32_t d : {128u, 256u})
        for (uint32_t g : {1u, 2u, 4u, 8u})
            for (uint32_t f : {Q35_KV_TURBO8, Q35_KV_TURBO2, Q35_KV_BF16K_TURBO4V})
                for (bool flash : {false, true}) probe(pf_quant_kernel_ptr(d, g, f, flash), "prefill attention (quantised)");
#define X(KK)                                                                  \
    probe(gemv_kernel_ptr(kOpInFullP, KK, false, false), "q/k/v (partial sums)"); \
    probe(gemv_kernel_ptr(kOpInFullP, KK, true, false), "q/k/v (partial sums)");
    Q35_W_PARTS(X)
#undef X
    for (int launch : {kXcdMixer, kXcdMlp}) probe(xcd_kernel_ptr(1, launch), "XCD-split decode");
    probe(xsum_kernel_ptr(), "residual sum");
    probe(embed_kernel_ptr(), "embed");
    probe(lm_finish_kernel_ptr(), "lm_head argmax");
    for (uint32_t d : {64u, 128u, 256u})
        for (uint32_t g : {1u, 2u, 4u, 8u}) probe(attn_combine_kernel_ptr(d, g), "attention merge");
    // the fixed workspace's address on this device (it is current here)
    void* scratch_ptr = nullptr;
    size_t scratch_bytes = 0;
    if (st == Q35_OK) {
        const hipError_t e = static_scratch_address(&scratch_ptr, &scratch_bytes);
        if (e != hipSuccess || !scratch_ptr)
            st = fail(Q35_ERR_HIP, "fixed workspace address: %s", hipGetErrorString(e));
    }
    (void)hipSetDevice(prev);
    if (st != Q35_OK) return st;
    Qwen35Kernels* k = new Qwen35Kernels;
    k->device = device;
    k->num_cu = prop.multiProcessorCount;
    k->scratch = scratch_ptr;
    k->scratch_bytes = scratch_bytes;
    for (int bits = 2; bits <= 4; ++bits) lloyd_max_normal(1 << bits, k->lm[bits].v);
    *out = k;
    return ok();
}

void q35_kernels_release(Qwen35Kernels* k) { delete k; }

q35_status q35_kv_dtype_from_str(const char* name, uint32_t* dtype) {
    if (!name || !dtype) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    static const char* names[] = {"bf16", "turbo8", "turbo4", "turbo3", "turbo2",
                                  "bf16k_turbo4v", "bf16k_turbo3v", "bf16k_turbo2v"};
    for (uint32_t i = 0; i < 8; ++i)
        if (std::strcmp(name, names[i]) == 0) {
            *dtype = i;
            return ok();
        }
    return fail(Q35_ERR_INVALID_ARG,
                "kv dtype \"%s\" unknown (bf16 | turbo8 | turbo4 | turbo3 | turbo2 | bf16k_turbo4v/3v/2v)",
                name);
}

q35_status q35_kv_cache_bytes(const Qwen35ForwardConfig* cfg, uint32_t dtype, uint32_t max_seq,
                              size_t* k_bytes, size_t* v_bytes, size_t* k_scale_bytes,
                              size_t* v_scale_bytes) {
    if (!cfg || !k_bytes || !v_bytes || !k_scale_bytes || !v_scale_bytes)
        return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    const size_t kvd = kv_dim(*cfg);
    if (dtype > Q35_KV_BF16K_TURBO2V) return fail(Q35_ERR_INVALID_ARG, "kv dtype %u", dtype);
    if (dtype != Q35_KV_BF16 && kvd % 16)
        return fail(Q35_ERR_INVALID_ARG, "turbo KV formats need kv_dim divisible by 16 (kv_dim %zu)", kvd);
    const size_t n = (size_t)max_seq * kvd;
    const size_t se = n / 16;  // one scale per 16 elements
    size_t kb = 0, vb = 0, ks = 0, vs = 0;
    switch (dtype) {
        case Q35_KV_BF16: kb = vb = n * 2; break;
        case Q35_KV_TURBO8: kb = vb = n; ks = vs = se * 2; break;
        case Q35_KV_TURBO4: kb = vb = n / 2; ks = vs = se; break;
        case Q35_KV_TURBO3: kb = vb = n * 3 / 8; ks = vs = se; break;
        case Q35_KV_TURBO2: kb = vb = n / 4; ks = vs = se; break;
        case Q35_KV_BF16K_TURBO4V: kb = n * 2; vb = n / 2; vs = se; break;
        case Q35_KV_BF16K_TURBO3V: kb = n * 2; vb = n * 3 / 8; vs = se; break;
        case Q35_KV_BF16K_TURBO2V: kb = n * 2; vb = n / 4; vs = se; break;
    }
    *k_bytes = kb;
    *v_bytes = vb;
    *k_scale_bytes = ks;
    *v_scale_bytes = vs;
    return ok();
}

q35_status q35_full_attention_workspace_bytes(const Qwen35ForwardConfig* cfg, uint32_t capacity,
                                              size_t* bytes) {
    if (!cfg || !bytes) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    *bytes = attn_ws_layout(*cfg, capacity).total;
    return ok();
}

// The attention steps of the full-attention forward (split, q/k norm, RoPE, KV
// append, split-K attention, sigmoid gate) on the projections in the scratch.
static q35_status launch_attention(const Qwen35Kernels* kernels, const Qwen35ForwardConfig& c,
                                   const FullAttentionLayer* layer, const FullAttentionScratch* s,
                                   const LayerKvCache* kv, const AttnWs& ws, const float* inv_freq,
                                   const int32_t* positions, int64_t cache_pos,
                                   uint32_t seq_len_attn, hipStream_t stream) {
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    const uint32_t G = c.num_heads / c.num_kv_heads;
    uint8_t* wsb = static_cast<uint8_t*>(s->workspace);
    a.q_full = s->q_full;
    a.k = s->k;
    a.v = s->v;
    a.q_norm = layer->q_norm;
    a.k_norm = layer->k_norm;
    a.inv_freq = inv_freq;
    a.positions = positions;
    a.kc = static_cast<uint16_t*>(kv->k);
    a.vc = static_cast<uint16_t*>(kv->v);
    a.ks = static_cast<uint16_t*>(kv->k_scales);
    a.vs = static_cast<uint16_t*>(kv->v_scales);
    a.gated_attn = s->gated_attn;
    a.attn_out = s->attn_out;
    a.q_norm_out = s->q_norm_out;
    a.k_norm_out = s->k_norm_out;
    a.part_acc = reinterpret_cast<float*>(wsb + ws.acc_off);
    a.part_ml = reinterpret_cast<float*>(wsb + ws.ml_off);
    a.status = s->status;
    a.capacity = kv->capacity;
    a.hq = c.num_heads;
    a.hkv = c.num_kv_heads;
    a.rotary = c.rotary_dim;
    a.max_chunks = attn_max_chunks(c, kv->capacity);
    a.eps = c.rms_eps;
    a.scale = 1.0f / std::sqrt((float)c.head_dim);
    a.sparse_v_log2 = (kv->dtype == Q35_KV_BF16 || kv->sparse_v <= 0.0f) ? -INFINITY
                                                                          : std::log2(kv->sparse_v);
    if (kv_lm_bits(kv->dtype)) std::memcpy(a.lm_levels, kernels->lm[kv_lm_bits(kv->dtype)].v, sizeof(a.lm_levels));
    uint32_t grid;
    if (cache_pos >= 0) {
        a.host_pos = (int32_t)cache_pos;
        a.chunk = attn_chunk(c, seq_len_attn);
        grid = (seq_len_attn + a.chunk - 1) / a.chunk;
    } else {
        a.host_pos = -1;
        a.chunk = attn_chunk(c, kv->capacity);
        grid = (kv->capacity + a.chunk - 1) / a.chunk;
    }
    if (grid > a.max_chunks) return fail(Q35_ERR_INVALID_ARG, "internal: %u chunks > %u", grid, a.max_chunks);
    Q35_HIP(attn_launch(c.head_dim, G, a, grid, kv->dtype, stream), "attention");
    (void)G;
    return Q35_OK;
}

static q35_status forward_full_impl(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                    const FullAttentionLayer* layer,
                                    const FullAttentionScratch* s, const LayerKvCache* kv,
                                    const float* inv_freq, const int32_t* positions,
                                    const void* x_in, int64_t cache_pos, uint32_t seq_len_attn,
                                    hipStream_t stream, void** out) {
    Q35_TRY(check_kernels(kernels));
    if (!cfg || !layer || !s || !kv || !out) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    const Qwen35ForwardConfig& c = *cfg;
    Q35_TRY(check_kv(*kv, true));
    if (cache_pos >= 0) {
        if ((uint64_t)cache_pos >= kv->capacity)
            return fail(Q35_ERR_OUT_OF_RANGE, "cache_pos %lld >= capacity %u", (long long)cache_pos, kv->capacity);
        if (seq_len_attn != (uint64_t)cache_pos + 1)
            return fail(Q35_ERR_OUT_OF_RANGE, "seq_len_attn %u != cache_pos + 1 (%lld)", seq_len_attn,
                        (long long)cache_pos + 1);
    }
    Q35_TRY(need(inv_freq, "inv_freq", false));
    Q35_TRY(need(positions, "positions", false));
    Q35_TRY(need(x_in, "x_in"));
    Q35_TRY(check_full_layer(c, *layer));
    Q35_TRY(need(s->q_full, "scratch.q_full"));
    Q35_TRY(need(s->k, "scratch.k"));
    Q35_TRY(need(s->v, "scratch.v"));
    Q35_TRY(need(s->gated_attn, "scratch.gated_attn"));
    Q35_TRY(need(s->x_resid, "scratch.x_resid"));
    Q35_TRY(need(s->mlp_act, "scratch.mlp_act"));
    Q35_TRY(need(s->x_out, "scratch.x_out"));
    Q35_TRY(need(s->workspace, "scratch.workspace"));
    Q35_TRY(opt(s->x_norm, "scratch.x_norm"));
    Q35_TRY(opt(s->x_norm2, "scratch.x_norm2"));
    const AttnWs ws = attn_ws_layout(c, kv->capacity);
    if (s->workspace_bytes < ws.total)
        return fail(Q35_ERR_INVALID_ARG, "workspace %zu bytes < %zu required", s->workspace_bytes, ws.total);
    if (x_in == s->x_out) return fail(Q35_ERR_INVALID_ARG, "x_in aliases scratch.x_out");

    const bool f32 = c.act_dtype == Q35_ACT_F32;
    // 1. input RMSNorm + q/k/v projections
    {
        GemvBuild b(kOpInFull, c.hidden, f32);
        b.a.pro.kind = kProRmsAct;
        b.a.pro.x_f32 = f32;
        b.a.pro.x = x_in;
        b.a.pro.w = layer->input_ln;
        b.a.pro.eps = c.rms_eps;
        b.a.pro.tap = s->x_norm;
        b.add(layer->q_proj, kEpiStore).out = s->q_full;
        b.add(layer->k_proj, kEpiStore).out = s->k;
        b.add(layer->v_proj, kEpiStore).out = s->v;
        Q35_TRY(b.launch((uint32_t)kernels->num_cu, stream, "q/k/v GEMV"));
    }
    // 2. split, q/k norm, RoPE, KV append, split-K attention, sigmoid gate
    Q35_TRY(launch_attention(kernels, c, layer, s, kv, ws, inv_freq, positions, cache_pos, seq_len_attn,
                             stream));
    // 3. o projection + residual
    {
        GemvBuild b(kOpOProj, q_only(c), f32);
        b.a.pro.kind = kProLoadF32;
        b.a.pro.x = s->gated_attn;
        GemvSeg& sg = b.add(layer->o_proj, kEpiResidActIn);
        sg.out = s->x_resid;
        (f32 ? sg.pre4 : sg.pre2) = x_in;
        sg.tap0 = s->o;
        Q35_TRY(b.launch((uint32_t)kernels->num_cu, stream, "o_proj GEMV"));
    }
    // 4-5. post-attention norm, SwiGLU MLP, residual
    Q35_TRY(launch_mlp((uint32_t)kernels->num_cu, c, layer->gate_proj, layer->up_proj, layer->down_proj, layer->post_ln,
                       s->x_resid, s->x_norm2, s->mlp_act, s->gate_act, s->up_act, s->x_out,
                       nullptr, stream));
    *out = s->x_out;
    return ok();
}

q35_status q35_forward_full_attention(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                      const FullAttentionLayer* layer,
                                      const FullAttentionScratch* scratch, const LayerKvCache* kv,
                                      const float* inv_freq, const int32_t* positions,
                                      const void* x_in, uint32_t cache_pos, uint32_t seq_len_attn,
                                      hipStream_t stream, void** out) {
    return forward_full_impl(kernels, cfg, layer, scratch, kv, inv_freq, positions, x_in,
                             (int64_t)cache_pos, seq_len_attn, stream, out);
}

q35_status q35_forward_full_attention_devpos(const Qwen35Kernels* kernels,
                                             const Qwen35ForwardConfig* cfg,
                                             const FullAttentionLayer* layer,
                                             const FullAttentionScratch* scratch,
                                             const LayerKvCache* kv, const float* inv_freq,
                                             const int32_t* positions, const void* x_in,
                                             hipStream_t stream, void** out) {
    return forward_full_impl(kernels, cfg, layer, scratch, kv, inv_freq, positions, x_in, -1, 0,
                             stream, out);
}

q35_status q35_attention_devpos(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                const FullAttentionLayer* layer, const FullAttentionScratch* s,
                                const LayerKvCache* kv, const float* inv_freq,
                                const int32_t* positions, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (!cfg || !layer || !s || !kv) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    const Qwen35ForwardConfig& c = *cfg;
    Q35_TRY(check_kv(*kv, true));
    Q35_TRY(need(inv_freq, "inv_freq", false));
    Q35_TRY(need(positions, "positions", false));
    Q35_TRY(check_full_layer(c, *layer));
    Q35_TRY(need(s->q_full, "scratch.q_full"));
    Q35_TRY(need(s->k, "scratch.k"));
    Q35_TRY(need(s->v, "scratch.v"));
    Q35_TRY(need(s->gated_attn, "scratch.gated_attn"));
    Q35_TRY(need(s->workspace, "scratch.workspace"));
    const AttnWs ws = attn_ws_layout(c, kv->capacity);
    if (s->workspace_bytes < ws.total)
        return fail(Q35_ERR_INVALID_ARG, "workspace %zu bytes < %zu required", s->workspace_bytes, ws.total);
    Q35_TRY(launch_attention(kernels, c, layer, s, kv, ws, inv_freq, positions, -1, 0, stream));
    return ok();
}

q35_status q35_forward_linear_attention(const Qwen35Kernels* kernels,
                                        const Qwen35ForwardConfig* cfg,
                                        const LinearAttentionLayer* layer,
                                        const LinearAttentionState* state,
                                        const LinearAttentionScratch* s, const void* x_in,
                                        void* x_buf, hipStream_t stream, q35_dump_fn dump,
                                        void* dump_ctx, void** out) {
    Q35_TRY(check_kernels(kernels));
    if (!cfg || !layer || !state || !s || !out) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    const Qwen35ForwardConfig& c = *cfg;
    const uint32_t Hv = c.num_v_heads_lin;
    Q35_TRY(need(x_in, "x_in"));
    Q35_TRY(need(x_buf, "x_buf"));
    Q35_TRY(check_linear_layer(c, *layer, *state));
    Q35_TRY(need(s->qkv_conv, "scratch.qkv_conv"));
    Q35_TRY(need(s->z, "scratch.z"));
    Q35_TRY(need(s->gate, "scratch.gate", false));
    Q35_TRY(need(s->beta, "scratch.beta", false));
    Q35_TRY(need(s->y, "scratch.y"));
    Q35_TRY(need(s->x_resid, "scratch.x_resid"));
    Q35_TRY(need(s->mlp_act, "scratch.mlp_act"));
    Q35_TRY(opt(s->x_norm, "scratch.x_norm"));
    Q35_TRY(opt(s->y_norm, "scratch.y_norm"));
    Q35_TRY(opt(s->x_norm2, "scratch.x_norm2"));

    const bool f32 = c.act_dtype == Q35_ACT_F32;
    // 1. input RMSNorm + in_proj qkv (conv epilogue) / z / a (gate) / b (beta)
    {
        GemvBuild b(kOpInGdn, c.hidden, f32);
        b.a.pro.kind = kProRmsAct;
        b.a.pro.x_f32 = f32;
        b.a.pro.x = x_in;
        b.a.pro.w = layer->input_ln;
        b.a.pro.eps = c.rms_eps;
        b.a.pro.tap = s->x_norm;
        GemvSeg& sq = b.add(layer->in_proj_qkv, kEpiConv);
        sq.out = s->qkv_conv;
        sq.state = state->conv1d_state;
        sq.pre16 = state->conv1d_state;
        sq.pre8 = layer->conv1d_weight;
        sq.tap0 = s->qkv;
        b.add(layer->in_proj_z, kEpiStore).out = s->z;
        GemvSeg& sa = b.add(layer->in_proj_a, kEpiGate);
        sa.out = s->gate;
        sa.pre2 = layer->dt_bias;
        sa.pre4 = layer->a_log;
        sa.tap0 = s->dt_raw;
        GemvSeg& sb = b.add(layer->in_proj_b, kEpiBeta);
        sb.out = s->beta;
        sb.tap0 = s->b_raw;
        Q35_TRY(b.launch((uint32_t)kernels->num_cu, stream, "in_proj GEMV"));
    }
    // 2. L2 norm of q/k + gated delta rule
    {
        GdnArgs g;
        std::memset(&g, 0, sizeof(g));
        g.state = state->gdn_state;
        g.qkv_conv = s->qkv_conv;
        g.gate = s->gate;
        g.beta = s->beta;
        g.y = s->y;
        g.qkv_smooth = s->qkv_smooth;
        g.hk = c.num_k_heads_lin;
        g.hv = Hv;
        g.l2_eps = 1e-6f;
        g.out_scale = 1.0f / std::sqrt((float)c.k_head_dim_lin);
        Q35_HIP(gdn_launch(c.k_head_dim_lin, c.v_head_dim_lin, g, stream), "gated delta rule");
    }
    // 3. gated RMSNorm + out projection + residual
    {
        GemvBuild b(kOpOutGated, z_dim(c), f32);
        b.a.pro.kind = kProGatedNorm;
        b.a.pro.x = s->y;
        b.a.pro.w = layer->norm_weight;
        b.a.pro.z = s->z;
        b.a.pro.head_dim = c.v_head_dim_lin;
        b.a.pro.eps = c.rms_eps;
        b.a.pro.tap = s->y_norm;
        GemvSeg& so = b.add(layer->out_proj, kEpiResidActIn);
        so.out = s->x_resid;
        (f32 ? so.pre4 : so.pre2) = x_in;
        so.tap0 = s->out;
        Q35_TRY(b.launch((uint32_t)kernels->num_cu, stream, "out_proj GEMV"));
    }
    // 4-5. MLP; output residual stream straight into x_buf
    Q35_TRY(launch_mlp((uint32_t)kernels->num_cu, c, layer->gate_proj, layer->up_proj, layer->down_proj, layer->post_ln,
                       s->x_resid, s->x_norm2, s->mlp_act, s->gate_act, s->up_act, x_buf,
                       s->x_final, stream));
    if (dump) {
        Q35_HIP(hipStreamSynchronize(stream), "hipStreamSynchronize");
        const uint32_t qt = qkv_total(c), zd = z_dim(c);
        if (s->x_norm) dump(dump_ctx, "gdn_x_norm", s->x_norm, c.hidden);
        if (s->qkv) dump(dump_ctx, "gdn_qkv_pre", s->qkv, qt);
        if (s->qkv_smooth) dump(dump_ctx, "gdn_qkv_smooth", s->qkv_smooth, qt);
        dump(dump_ctx, "gdn_y", s->y, zd);
        if (s->y_norm) dump(dump_ctx, "gdn_y_norm", s->y_norm, zd);
        if (s->out) dump(dump_ctx, "gdn_out", s->out, c.hidden);
        dump(dump_ctx, "gdn_x_resid", s->x_resid, c.hidden);
        dump(dump_ctx, "gdn_x_final", s->x_final ? s->x_final : x_buf, c.hidden);
    }
    *out = x_buf;
    return ok();
}

q35_status q35_embed_lookup(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                            const uint16_t* table, const int32_t* tokens, void* x_out,
                            hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (!cfg || !table || !tokens || !x_out) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    if (cfg->vocab == 0 || cfg->hidden == 0) return fail(Q35_ERR_INVALID_ARG, "vocab/hidden is 0");
    Q35_HIP(embed_launch(table, tokens, cfg->vocab, cfg->hidden, x_out, cfg->act_dtype == Q35_ACT_F32,
                         stream), "embed");
    return ok();
}

q35_status q35_lm_head_workspace_bytes(const Qwen35ForwardConfig* cfg, size_t* bytes) {
    if (!cfg || !bytes) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    if (cfg->vocab == 0) return fail(Q35_ERR_INVALID_ARG, "vocab is 0");
    *bytes = lm_ws_layout(*cfg).total;
    return ok();
}

q35_status q35_lm_head_argmax(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                              const uint16_t* final_norm, const Q35QuantWeight* lm_head,
                              const void* x, float* logits, void* workspace,
                              size_t workspace_bytes, int32_t* tokens, int32_t* positions,
                              int32_t* history, uint32_t history_len, int32_t history_base,
                              const uint16_t* embed_table, void* x_next, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (!cfg || !lm_head) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    const Qwen35ForwardConfig& c = *cfg;
    if (c.vocab == 0) return fail(Q35_ERR_INVALID_ARG, "vocab is 0");
    Q35_TRY(check_weight("lm_head", *lm_head, c.vocab, c.hidden));
    Q35_TRY(need(final_norm, "final_norm"));
    Q35_TRY(need(x, "x"));
    Q35_TRY(need(tokens, "tokens", false));
    Q35_TRY(need(workspace, "workspace"));
    if ((embed_table == nullptr) != (x_next == nullptr))
        return fail(Q35_ERR_INVALID_ARG, "embed_table and x_next go together");
    if (x_next && x_next == x) return fail(Q35_ERR_INVALID_ARG, "x_next aliases x");
    Q35_TRY(opt(embed_table, "embed_table"));
    Q35_TRY(opt(x_next, "x_next"));
    const LmWs ws = lm_ws_layout(c);
    if (workspace_bytes < ws.total)
        return fail(Q35_ERR_INVALID_ARG, "workspace %zu bytes < %zu required", workspace_bytes, ws.total);
    const bool f32 = c.act_dtype == Q35_ACT_F32;
    GemvBuild b(kOpLmHead, c.hidden, f32);
    b.a.pro.kind = kProRmsAct;
    b.a.pro.x_f32 = f32;
    b.a.pro.x = x;
    b.a.pro.w = final_norm;
    b.a.pro.eps = c.rms_eps;
    b.add(*lm_head, kEpiArgmax).out = logits;
    uint8_t* wsb = static_cast<uint8_t*>(workspace);
    b.a.am.part_val = reinterpret_cast<float*>(wsb + ws.val_off);
    b.a.am.part_idx = reinterpret_cast<int32_t*>(wsb + ws.idx_off);
    Q35_TRY(b.launch((uint32_t)kernels->num_cu, stream, "lm_head GEMV", ws.blocks));
    LmFinishArgs f;
    std::memset(&f, 0, sizeof(f));
    f.part_val = b.a.am.part_val;
    f.part_idx = b.a.am.part_idx;
    f.nparts = ws.blocks;
    f.vocab = c.vocab;
    f.tokens = tokens;
    f.positions = positions;
    f.history = history;
    f.history_len = history ? history_len : 0;
    f.history_base = history_base;
    f.embed = embed_table;
    f.x_next = x_next;
    f.hidden = c.hidden;
    f.act_f32 = f32 ? 1 : 0;
    Q35_HIP(lm_finish_launch(f, stream), "lm_head argmax");
    return ok();
}

q35_status q35_lm_head_argmax_noalloc(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                      const uint16_t* final_norm, const Q35QuantWeight* lm_head,
                                      const void* x, float* logits, int32_t* tokens,
                                      int32_t* positions, int32_t* history, uint32_t history_len,
                                      int32_t history_base, const uint16_t* embed_table, void* x_next,
                                      hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (!cfg) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    if (cfg->vocab == 0) return fail(Q35_ERR_INVALID_ARG, "vocab is 0");
    const size_t need_bytes = lm_ws_layout(*cfg).total;
    if (need_bytes > kernels->scratch_bytes)
        return fail(Q35_ERR_OUT_OF_RANGE,
                    "vocab %u needs %zu bytes of workspace, more than the fixed %zu bytes "
                    "(use q35_lm_head_argmax with a caller workspace)",
                    cfg->vocab, need_bytes, kernels->scratch_bytes);
    // the per-block partials are written before they are read: nothing to clear
    return q35_lm_head_argmax(kernels, cfg, final_norm, lm_head, x, logits, kernels->scratch,
                              kernels->scratch_bytes, tokens, positions, history, history_len,
                              history_base, embed_table, x_next, stream);
}

q35_status q35_gate_up_swiglu(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                              const uint16_t* post_ln, const Q35QuantWeight* gate_proj,
                              const Q35QuantWeight* up_proj, const float* x_resid,
                              float* mlp_act, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (!cfg || !gate_proj || !up_proj) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    const Qwen35ForwardConfig& c = *cfg;
    Q35_TRY(check_weight("gate_proj", *gate_proj, c.intermediate, c.hidden));
    Q35_TRY(check_weight("up_proj", *up_proj, c.intermediate, c.hidden));
    Q35_TRY(need(post_ln, "post_ln"));
    Q35_TRY(need(x_resid, "x_resid"));
    Q35_TRY(need(mlp_act, "mlp_act"));
    GemvBuild b(kOpGateUp, c.hidden, c.act_dtype == Q35_ACT_F32);
    b.a.pro.kind = kProRmsF32;
    b.a.pro.x = x_resid;
    b.a.pro.w = post_ln;
    b.a.pro.eps = c.rms_eps;
    b.add(*gate_proj, kEpiSwiGLU, up_proj).out = mlp_act;
    Q35_TRY(b.launch((uint32_t)kernels->num_cu, stream, "gate/up GEMV"));
    return ok();
}

q35_status q35_turbo8_quantize(const Qwen35Kernels* kernels, const float* x, uint32_t n,
                               uint8_t* codes, uint16_t* scales, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (n % 16) return fail(Q35_ERR_INVALID_ARG, "n = %u is not a multiple of 16", n);
    if (n == 0) return ok();
    Q35_TRY(need(x, "x"));
    Q35_TRY(need(codes, "codes"));
    Q35_TRY(need(scales, "scales", false));
    if (reinterpret_cast<uintptr_t>(scales) & 1u) return fail(Q35_ERR_INVALID_ARG, "scales not 2-byte aligned");
    Q35_HIP(turbo8_quantize_launch(x, n, codes, scales, stream), "turbo8 quantise");
    return ok();
}

q35_status q35_turbo_codebook(const Qwen35Kernels* kernels, uint32_t bits, float* levels) {
    Q35_TRY(check_kernels(kernels));
    if (bits < 2 || bits > 4) return fail(Q35_ERR_INVALID_ARG, "bits = %u (2, 3 or 4)", bits);
    if (!levels) return fail(Q35_ERR_INVALID_ARG, "levels is NULL");
    std::memcpy(levels, kernels->lm[bits].v, (1u << bits) * sizeof(float));
    return ok();
}

q35_status q35_turbo_quantize(const Qwen35Kernels* kernels, uint32_t bits, const float* x, uint32_t n,
                              uint8_t* packed, uint8_t* scales, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (bits < 2 || bits > 4) return fail(Q35_ERR_INVALID_ARG, "bits = %u (2, 3 or 4)", bits);
    if (n % 16) return fail(Q35_ERR_INVALID_ARG, "n = %u is not a multiple of 16", n);
    if (n == 0) return ok();
    Q35_TRY(need(x, "x"));
    Q35_TRY(need(packed, "packed", false));
    const uintptr_t align = bits == 4 ? 8u : bits == 2 ? 4u : 2u;  // one group's indices
    if (reinterpret_cast<uintptr_t>(packed) & (align - 1))
        return fail(Q35_ERR_INVALID_ARG, "packed not %u-byte aligned", (unsigned)align);
    Q35_TRY(need(scales, "scales", false));
    Q35_HIP(lm_quantize_launch(bits, x, n, kernels->lm[bits], packed, scales, stream), "turbo quantise");
    return ok();
}

q35_status q35_fp8_e4m3_table(const Qwen35Kernels* kernels, float* out, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    Q35_TRY(need(out, "out"));
    Q35_HIP(e4m3_table_launch(out, stream), "e4m3 table");
    return ok();
}

q35_status q35_gemv(const Qwen35Kernels* kernels, const Q35QuantWeight* w, const float* x,
                    float* y, uint32_t act_dtype, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (!w) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    if (!gemv_width_supported(kWidthAny, w->k))
        return fail(Q35_ERR_UNSUPPORTED, "K = %u is not a compiled width", w->k);
    Q35_TRY(check_weight("w", *w, w->n, w->k));
    Q35_TRY(check_rows("w", w->n, w->k));
    Q35_TRY(need(x, "x"));
    Q35_TRY(need(y, "y", false));
    if (act_dtype != Q35_ACT_BF16 && act_dtype != Q35_ACT_F32)
        return fail(Q35_ERR_INVALID_ARG, "act_dtype %u", act_dtype);
    GemvBuild b(kOpPlain, w->k, act_dtype == Q35_ACT_F32);
    b.a.pro.kind = kProLoadF32;
    b.a.pro.x = x;
    b.add(*w, kEpiStore).out = y;
    Q35_TRY(b.launch((uint32_t)kernels->num_cu, stream, "GEMV"));
    return ok();
}

// ------------------------------------------------------------------ prefill

}  // extern "C"

namespace {

// Prefill workspace: the buffers of one layer kind for T tokens, each
// 256-byte aligned; the two kinds share one region.
struct PfWs {
    size_t xh, qkv, z, fa, fb, qkvs, lg, beta, wc, uc, pc, lc, y, yz, r, h;  // GDN
    size_t qf, kf, vf, qb, ga;                                               // full (xh, r, h shared)
    size_t gaf, pos;                                                         // full, quantised caches
    size_t part;                                                             // split GEMM partial tiles
    size_t wh;                                                               // a GEMM's weights as f16
    uint32_t nch;
    size_t bytes;
};

// Bytes of the largest weight set one prefill GEMM launch reads (every
// matrix of the launch, stacked), as f16.
size_t pf_wh_bytes(const Qwen35ForwardConfig& c) {
    const size_t H = c.hidden, I = c.intermediate;
    const size_t in_gdn = (size_t)qkv_total(c) + z_dim(c) + 2 * (size_t)c.num_v_heads_lin;
    const size_t in_full = (size_t)q_total(c) + 2 * (size_t)kv_dim(c);
    const size_t elems = std::max({in_gdn * H, H * z_dim(c), 2 * I * H, H * I, in_full * H, H * q_only(c)});
    return elems * 2;
}

// From this many prompt rows (sixteen row tiles) a prefill GEMM dequantises its
// weights to f16 once, in the workspace, instead of once per row tile: the
// pass over every weight costs a 4B stack about 3 ms per prompt, which the
// faster GEMMs save back at 4096 tokens (measured) and more beyond.
constexpr uint32_t kPfF16MinRows = 4096;

PfWs pf_ws_layout(const Qwen35ForwardConfig& c, uint32_t T) {
    PfWs w{};
    auto take = [](size_t& off, size_t n) {
        const size_t o = off;
        off += (n + 255) & ~(size_t)255;
        return o;
    };
    const size_t t = T, H = c.hidden, I = c.intermediate, C = qkv_total(c), Z = z_dim(c);
    const size_t hv = c.num_v_heads_lin, dk = c.k_head_dim_lin, dv = c.v_head_dim_lin;
    w.nch = (T + 63) / 64;
    size_t o = 0;
    w.xh = take(o, t * H * 2);
    w.r = take(o, t * H * 4);
    w.h = take(o, t * I * 2);
    const size_t shared = o;
    w.qkv = take(o, t * C * 4);
    w.z = take(o, t * Z * 4);
    w.fa = take(o, t * hv * 4);
    w.fb = take(o, t * hv * 4);
    w.qkvs = take(o, t * C * 4);
    w.lg = take(o, t * hv * 4);
    w.beta = take(o, t * hv * 4);
    w.wc = take(o, hv * w.nch * 64 * dk * 4);
    w.uc = take(o, hv * w.nch * 64 * dv * 4);
    w.pc = take(o, hv * w.nch * 64 * 64 * 4);
    w.lc = take(o, hv * w.nch * 64 * 4);
    w.y = take(o, t * Z * 4);
    w.yz = take(o, t * Z * 2);
    const size_t gdn = o;
    o = shared;
    w.qf = take(o, t * q_total(c) * 4);
    w.kf = take(o, t * kv_dim(c) * 4);
    w.vf = take(o, t * kv_dim(c) * 4);
    w.qb = take(o, t * q_only(c) * 2);
    w.ga = take(o, t * q_only(c) * 2);
    w.gaf = take(o, t * q_only(c) * 4);
    w.pos = take(o, t * 4);
    o = gdn > o ? gdn : o;
    w.part = take(o, T ? kPfSplitBytes : 0);
    w.wh = take(o, T ? pf_wh_bytes(c) : 0);
    w.bytes = o;
    return w;
}

template <class T>
T* at_off(void* base, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// Where a GEMM launch may leave the partial tiles of a split last round (part
// NULL: never split), the compute units it plans the rounds for, and where it
// may write its weights dequantised to f16 first (wh NULL: the GEMM
// dequantises them from the codes as it goes; same values either way).
struct PfSplit {
    float* part;
    uint32_t num_cu;
    uint16_t* wh;
};

// One prefill GEMM launch.  F32 mode: up to four matrices stacked by rows, each
// writing its own fp32 output (row stride = its rows); RESID and SWIGLU: ws[0]
// (and ws[1] = up_proj for SWIGLU) into out with row stride ldo.
q35_status pf_gemm(const PfSplit& sp, const char* what, int mode, const uint16_t* x, uint32_t M,
                   std::initializer_list<const Q35QuantWeight*> ws, std::initializer_list<void*> outs,
                   uint32_t ldo, const void* resid, bool resid_f32, bool out_f32, hipStream_t stream) {
    PfGemmArgs g{};
    g.x = x;
    uint32_t i = 0, rows = 0;
    size_t wh_off = 0;
    for (const Q35QuantWeight* w : ws) {
        g.w[i] = w->codes;
        g.s[i] = w->scales;
        g.b[i] = w->biases;
        if (sp.wh) {
            g.wh[i] = sp.wh + wh_off;
            Q35_HIP(pf_dequant_launch(w->codes, w->scales, w->biases, w->n, w->k, sp.wh + wh_off, stream), what);
            wh_off += (size_t)w->n * w->k;
        }
        if (mode == kPfF32 || i == 0) rows += w->n;
        g.seg_end[i] = rows;
        g.ldo[i] = mode == kPfF32 ? w->n : ldo;
        ++i;
    }
    for (uint32_t k = i; k < 4; ++k) g.seg_end[k] = rows;
    uint32_t o = 0;
    for (void* p : outs) g.out[o++] = p;
    g.resid = resid;
    g.M = M;
    g.N = rows;
    g.K = (*ws.begin())->k;
    g.resid_f32 = resid_f32 ? 1 : 0;
    g.out_f32 = out_f32 ? 1 : 0;
    g.part = sp.part;
    Q35_HIP(pf_gemm_launch(mode, g, sp.num_cu, stream), what);
    return Q35_OK;
}

q35_status pf_check_ws(const Qwen35ForwardConfig& c, uint32_t T, const void* ws, size_t bytes,
                       PfWs* out) {
    *out = pf_ws_layout(c, T);
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(Q35_ERR_INVALID_ARG, "workspace NULL or not 256-byte aligned");
    if (bytes < out->bytes)
        return fail(Q35_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed for %u tokens", bytes,
                    out->bytes, T);
    return Q35_OK;
}

// the MLP half shared by both kinds: xn2 = RMSNorm(r), gate/up SwiGLU, down + r -> x_out
template <class L>
q35_status pf_mlp(const PfSplit& sp, const Qwen35ForwardConfig& c, const L& l, const PfWs& w, void* ws,
                  uint32_t T, void* x_out, hipStream_t stream) {
    uint16_t* xh = at_off<uint16_t>(ws, w.xh);
    float* r = at_off<float>(ws, w.r);
    uint16_t* h = at_off<uint16_t>(ws, w.h);
    Q35_HIP(pf_rmsnorm_launch(r, true, l.post_ln, xh, T, c.hidden, c.rms_eps, stream), "prefill post norm");
    Q35_TRY(pf_gemm(sp, "prefill gate/up", kPfSwiglu, xh, T, {&l.gate_proj, &l.up_proj}, {h}, c.intermediate,
                    nullptr, false, false, stream));
    Q35_TRY(pf_gemm(sp, "prefill down", kPfResid, h, T, {&l.down_proj}, {x_out}, c.hidden, r, true,
                    c.act_dtype == Q35_ACT_F32, stream));
    return Q35_OK;
}

}  // namespace

extern "C" {

q35_status q35_prefill_workspace_bytes(const Qwen35ForwardConfig* cfg, uint32_t max_tokens,
                                       size_t* bytes) {
    Q35_TRY(q35_config_validate(cfg));
    if (!bytes) return fail(Q35_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = pf_ws_layout(*cfg, max_tokens).bytes;
    return ok();
}

q35_status q35_prefill_linear_attention(const Qwen35Kernels* kernels,
                                        const Qwen35ForwardConfig* cfg,
                                        const LinearAttentionLayer* layer,
                                        const LinearAttentionState* state, const void* x_in,
                                        uint32_t n_tokens, void* x_out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    Q35_TRY(q35_config_validate(cfg));
    if (!layer || !state) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    const Qwen35ForwardConfig& c = *cfg;
    Q35_TRY(check_linear_layer(c, *layer, *state));
    Q35_TRY(need(x_in, "x_in", false));
    Q35_TRY(need(x_out, "x_out", false));
    const uint32_t dk = c.k_head_dim_lin, dv = c.v_head_dim_lin, hv = c.num_v_heads_lin;
    if (!pf_gdn_dims_supported(dk, dv))
        return fail(Q35_ERR_UNSUPPORTED, "prefill GDN head dims %u x %u (32, 64 or 128, equal)", dk, dv);
    PfWs w;
    Q35_TRY(pf_check_ws(c, n_tokens, workspace, workspace_bytes, &w));
    if (n_tokens == 0) return ok();
    const uint32_t T = n_tokens, C = qkv_total(c);
    const bool f32 = c.act_dtype == Q35_ACT_F32;
    void* ws = workspace;
    const PfSplit sp{at_off<float>(ws, w.part), (uint32_t)kernels->num_cu,
                     T >= kPfF16MinRows ? at_off<uint16_t>(ws, w.wh) : nullptr};
    const LinearAttentionLayer& l = *layer;
    uint16_t* xh = at_off<uint16_t>(ws, w.xh);
    float* qkv = at_off<float>(ws, w.qkv);
    float* z = at_off<float>(ws, w.z);
    float* fa = at_off<float>(ws, w.fa);
    float* fb = at_off<float>(ws, w.fb);

    Q35_HIP(pf_rmsnorm_launch(x_in, f32, l.input_ln, xh, T, c.hidden, c.rms_eps, stream), "prefill input norm");
    Q35_TRY(pf_gemm(sp, "prefill in_proj", kPfF32, xh, T,
                    {&l.in_proj_qkv, &l.in_proj_z, &l.in_proj_a, &l.in_proj_b}, {qkv, z, fa, fb}, 0, nullptr,
                    false, true, stream));

    PfConvArgs cv{};
    cv.qkv = qkv;
    cv.conv_state = state->conv1d_state;
    cv.conv_w = l.conv1d_weight;
    cv.a_raw = fa;
    cv.b_raw = fb;
    cv.a_log = l.a_log;
    cv.dt_bias = l.dt_bias;
    cv.qkvs = at_off<float>(ws, w.qkvs);
    cv.lg = at_off<float>(ws, w.lg);
    cv.beta = at_off<float>(ws, w.beta);
    cv.T = T;
    cv.C = C;
    cv.nqk = 2 * c.num_k_heads_lin * dk;
    cv.dk = dk;
    cv.hv = hv;
    PfGdnArgs g{};
    g.qkvs = cv.qkvs;
    g.lg = cv.lg;
    g.beta = cv.beta;
    g.Wc = at_off<float>(ws, w.wc);
    g.Uc = at_off<float>(ws, w.uc);
    g.Pc = at_off<float>(ws, w.pc);
    g.Lc = at_off<float>(ws, w.lc);
    g.y = at_off<float>(ws, w.y);
    g.state = state->gdn_state;
    g.T = T;
    g.C = C;
    g.hk = c.num_k_heads_lin;
    g.hv = hv;
    g.dk = dk;
    g.dv = dv;
    g.nch = w.nch;
    g.out_scale = 1.0f / std::sqrt((float)dk);
    Q35_HIP(pf_gdn_launch(cv, g, state->conv1d_state, stream), "prefill gated delta rule");
    uint16_t* yz = at_off<uint16_t>(ws, w.yz);
    Q35_HIP(pf_gdn_out_launch(g.y, z, l.norm_weight, yz, T, hv, dv, c.rms_eps, stream), "prefill gated norm");
    Q35_TRY(pf_gemm(sp, "prefill out_proj", kPfResid, yz, T, {&l.out_proj}, {at_off<float>(ws, w.r)}, c.hidden,
                    x_in, f32, true, stream));
    Q35_TRY(pf_mlp(sp, c, l, w, ws, T, x_out, stream));
    return ok();
}

q35_status q35_prefill_full_attention(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                      const FullAttentionLayer* layer, const LayerKvCache* kv,
                                      const float* inv_freq, const void* x_in, uint32_t n_tokens,
                                      uint32_t cache_pos, void* x_out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    Q35_TRY(q35_config_validate(cfg));
    if (!layer || !kv) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    const Qwen35ForwardConfig& c = *cfg;
    Q35_TRY(check_full_layer(c, *layer));
    Q35_TRY(check_kv(*kv, true));
    Q35_TRY(need(inv_freq, "inv_freq", false));
    Q35_TRY(need(x_in, "x_in", false));
    Q35_TRY(need(x_out, "x_out", false));
    const uint32_t G = c.num_heads / c.num_kv_heads;
    const bool quant = kv->dtype != Q35_KV_BF16;
    if (!quant && !pf_attn_dims_supported(c.head_dim, G))
        return fail(Q35_ERR_UNSUPPORTED, "prefill attention head_dim %u, group %u", c.head_dim, G);
    if (quant && !attn_dims_supported(c.head_dim, G))
        return fail(Q35_ERR_UNSUPPORTED, "attention head_dim %u, group %u", c.head_dim, G);
    if ((uint64_t)cache_pos + n_tokens > kv->capacity)
        return fail(Q35_ERR_OUT_OF_RANGE, "cache_pos %u + %u tokens > capacity %u", cache_pos, n_tokens,
                    kv->capacity);
    PfWs w;
    Q35_TRY(pf_check_ws(c, n_tokens, workspace, workspace_bytes, &w));
    if (n_tokens == 0) return ok();
    // a quantised cache the batched attention does not cover: the per-token
    // attention's partials use the split-GEMM area
    const bool quant_batched = quant && pf_quant_attn_supported(c.head_dim, G, kv->dtype);
    const AttnWs aws = attn_ws_layout(c, kv->capacity);
    if (quant && !quant_batched && aws.total > kPfSplitBytes)
        return fail(Q35_ERR_UNSUPPORTED, "capacity %u: attention partials exceed the prefill workspace",
                    kv->capacity);
    const uint32_t T = n_tokens;
    const bool f32 = c.act_dtype == Q35_ACT_F32;
    void* ws = workspace;
    const PfSplit sp{at_off<float>(ws, w.part), (uint32_t)kernels->num_cu,
                     T >= kPfF16MinRows ? at_off<uint16_t>(ws, w.wh) : nullptr};
    const FullAttentionLayer& l = *layer;
    uint16_t* xh = at_off<uint16_t>(ws, w.xh);
    float* qf = at_off<float>(ws, w.qf);
    float* kf = at_off<float>(ws, w.kf);
    float* vf = at_off<float>(ws, w.vf);
    Q35_HIP(pf_rmsnorm_launch(x_in, f32, l.input_ln, xh, T, c.hidden, c.rms_eps, stream), "prefill input norm");
    Q35_TRY(pf_gemm(sp, "prefill q/k/v", kPfF32, xh, T, {&l.q_proj, &l.k_proj, &l.v_proj}, {qf, kf, vf}, 0, nullptr,
                    false, true, stream));
    uint16_t* ga = at_off<uint16_t>(ws, w.ga);
    if (quant_batched) {
        // A quantised cache at head dimension 128 or 256: the prompt's rows are
        // appended as its decode steps would append them, then every token
        // attends to the rows as stored (two launches; see pfq_flash_kernel)
        PfQuantAttnArgs qa;
        std::memset(&qa, 0, sizeof(qa));
        qa.q_full = qf;
        qa.k = kf;
        qa.v = vf;
        qa.q_norm = l.q_norm;
        qa.k_norm = l.k_norm;
        qa.inv_freq = inv_freq;
        qa.kc = kv->k;
        qa.vc = kv->v;
        qa.ks = kv->k_scales;
        qa.vs = kv->v_scales;
        qa.qh = at_off<uint16_t>(ws, w.qb);
        qa.ga = ga;
        qa.T = T;
        qa.cache_pos = cache_pos;
        qa.hq = c.num_heads;
        qa.hkv = c.num_kv_heads;
        qa.rotary = c.rotary_dim;
        qa.eps = c.rms_eps;
        qa.scale = 1.0f / std::sqrt((float)c.head_dim);
        qa.sparse_v_log2 = kv->sparse_v <= 0.0f ? -INFINITY : std::log2(kv->sparse_v);
        if (kv_lm_bits(kv->dtype)) std::memcpy(qa.lm_levels, kernels->lm[kv_lm_bits(kv->dtype)].v, sizeof(qa.lm_levels));
        Q35_HIP(pf_quant_attn_launch(c.head_dim, G, kv->dtype, qa, stream), "prefill attention (quantised cache)");
        Q35_TRY(pf_gemm(sp, "prefill o_proj", kPfResid, ga, T, {&l.o_proj}, {at_off<float>(ws, w.r)}, c.hidden,
                        x_in, f32, true, stream));
        Q35_TRY(pf_mlp(sp, c, l, w, ws, T, x_out, stream));
        return ok();
    }
    if (quant) {
        // A quantised cache at the other head dimensions: each prompt token runs
        // the decode attention steps (q/k norm, RoPE, the quantising append of its
        // row, attention over the rows as stored, sparse-V gate, sigmoid gate), in
        // token order; the projections around them stay batched.
        int32_t* pos = at_off<int32_t>(ws, w.pos);
        float* gaf = at_off<float>(ws, w.gaf);
        Q35_HIP(pf_iota_launch(pos, T, (int32_t)cache_pos, stream), "prefill positions");
        FullAttentionScratch s{};
        s.workspace = at_off<void>(ws, w.part);
        s.workspace_bytes = kPfSplitBytes;
        for (uint32_t t = 0; t < T; ++t) {
            s.q_full = qf + (size_t)t * q_total(c);
            s.k = kf + (size_t)t * kv_dim(c);
            s.v = vf + (size_t)t * kv_dim(c);
            s.gated_attn = gaf + (size_t)t * q_only(c);
            Q35_TRY(launch_attention(kernels, c, layer, &s, kv, aws, inv_freq, pos + t, (int64_t)cache_pos + t,
                                     cache_pos + t + 1, stream));
        }
        Q35_HIP(pf_cast_f16_launch(gaf, ga, T * q_only(c), stream), "prefill attention output");
        Q35_TRY(pf_gemm(sp, "prefill o_proj", kPfResid, ga, T, {&l.o_proj}, {at_off<float>(ws, w.r)}, c.hidden,
                        x_in, f32, true, stream));
        Q35_TRY(pf_mlp(sp, c, l, w, ws, T, x_out, stream));
        return ok();
    }
    PfRopeArgs rp{};
    rp.q_full = qf;
    rp.k = kf;
    rp.v = vf;
    rp.q_norm = l.q_norm;
    rp.k_norm = l.k_norm;
    rp.inv_freq = inv_freq;
    rp.qb = at_off<uint16_t>(ws, w.qb);
    rp.kc = static_cast<uint16_t*>(kv->k);
    rp.vc = static_cast<uint16_t*>(kv->v);
    rp.T = T;
    rp.cache_pos = cache_pos;
    rp.hq = c.num_heads;
    rp.hkv = c.num_kv_heads;
    rp.D = c.head_dim;
    rp.rotary = c.rotary_dim;
    rp.eps = c.rms_eps;
    PfAttnArgs at{};
    at.qb = rp.qb;
    at.q_full = qf;
    at.kc = rp.kc;
    at.vc = rp.vc;
    at.ga = ga;
    at.T = T;
    at.cache_pos = cache_pos;
    at.hq = c.num_heads;
    at.hkv = c.num_kv_heads;
    at.scale_log2 = 1.4426950408889634f / std::sqrt((float)c.head_dim);
    Q35_HIP(pf_attn_launch(rp, at, stream), "prefill attention");
    Q35_TRY(pf_gemm(sp, "prefill o_proj", kPfResid, at.ga, T, {&l.o_proj}, {at_off<float>(ws, w.r)}, c.hidden,
                    x_in, f32, true, stream));
    Q35_TRY(pf_mlp(sp, c, l, w, ws, T, x_out, stream));
    return ok();
}

static_assert(Q35_PREFILL_GEMM_WORKSPACE_BYTES == kPfSplitBytes, "split workspace size");

q35_status q35_prefill_gemm(const Qwen35Kernels* kernels, const Q35QuantWeight* w, const uint16_t* x_f16,
                            uint32_t m, float* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Q35_TRY(check_kernels(kernels));
    if (!w) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(check_weight("w", *w, w->n, w->k));
    if (w->n == 0 || w->k == 0 || w->k % 64 != 0)
        return fail(Q35_ERR_INVALID_ARG, "w: shape [%u, %u] (k a nonzero multiple of 64)", w->n, w->k);
    Q35_TRY(need(x_f16, "x_f16"));
    Q35_TRY(need(y, "y", false));
    if (workspace && ((reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < kPfSplitBytes))
        return fail(Q35_ERR_INVALID_ARG, "workspace: %zu bytes, 256-byte aligned, needed (or NULL)", kPfSplitBytes);
    if (m == 0) return ok();
    // with room for the weights as f16 after the split area, they are dequantised once first
    uint16_t* wh = workspace && workspace_bytes >= kPfSplitBytes + (size_t)2 * w->n * w->k
                       ? reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + kPfSplitBytes)
                       : nullptr;
    const PfSplit sp{static_cast<float*>(workspace), (uint32_t)kernels->num_cu, wh};
    Q35_TRY(pf_gemm(sp, "prefill GEMM", kPfF32, x_f16, m, {w}, {y}, 0, nullptr, false, true, stream));
    return ok();
}

// ------------------------------------------------------------------ persistent decode

}  // extern "C"

struct Q35DecodePlan {
    int device;
    int shape;
    uint32_t blocks;
    PersistArgs args;
    uint32_t n_layers;
    std::vector<uint32_t> first_stage;  // [n_layers + 1]
    std::vector<void*> x_in;            // [n_layers + 1]
    uint64_t clock_hz;
};

namespace {

// Bump allocation of the plan's workspace sections (256-byte aligned, so no two
// buffers share a cache line); base == nullptr only counts.
struct Bump {
    uint8_t* base;
    size_t off = 0;
    void* take(size_t bytes) {
        void* p = base ? base + off : nullptr;
        off += (bytes + 255) & ~size_t(255);
        return p;
    }
    float* f32(size_t n) { return static_cast<float*>(take(n * sizeof(float))); }
};

constexpr uint32_t kStagesGdn = 5, kStagesFull = 6, kStagesTail = 2;
constexpr double kWaitLimitSeconds = 0.2;  // a wait longer than this is an error

// Validates the stack, lays out the workspace and (when ws != nullptr) fills
// the stage table and the plan's host view.
q35_status plan_build(const Qwen35Kernels* k, const Qwen35ForwardConfig* cfg,
                      const Q35DecodeStackDesc* d, uint8_t* ws, size_t* total,
                      std::vector<PStage>* stages, Q35DecodePlan* plan) {
    Q35_TRY(check_kernels(k));
    if (!cfg || !d) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    const Qwen35ForwardConfig& c = *cfg;
    const bool f32 = c.act_dtype == Q35_ACT_F32;
    const uint32_t G = c.num_heads / c.num_kv_heads;
    const int shape = persist_shape_id(c.hidden, c.intermediate, q_only(c), z_dim(c), c.k_head_dim_lin,
                                       c.head_dim, G, !f32);
    if (!shape)
        return fail(Q35_ERR_UNSUPPORTED, "the persistent kernel is not built for these dimensions "
                                         "(use the per-layer calls)");
    if (d->n_layers == 0 || !d->layers) return fail(Q35_ERR_INVALID_ARG, "empty stack");
    const uint32_t blocks = (uint32_t)k->num_cu;
    if (blocks < c.num_kv_heads || blocks > 1024)
        return fail(Q35_ERR_UNSUPPORTED, "%u compute units", blocks);
    const uint32_t cpb = blocks / c.num_kv_heads;  // attention chunks per kv head
    if (c.num_v_heads_lin * (c.v_head_dim_lin / 16) > blocks)
        return fail(Q35_ERR_UNSUPPORTED, "more recurrence tiles than blocks");
    Q35_TRY(need(d->positions, "positions", false));
    const bool tail = d->lm_head != nullptr;
    bool any_full = false;
    for (uint32_t l = 0; l < d->n_layers; ++l) {
        const Q35StackLayer& L = d->layers[l];
        if (L.kind == Q35_LAYER_LINEAR) {
            if (!L.linear || !L.state) return fail(Q35_ERR_INVALID_ARG, "layer %u: NULL weights/state", l);
            Q35_TRY(check_linear_layer(c, *L.linear, *L.state));
        } else if (L.kind == Q35_LAYER_FULL) {
            if (!L.full || !L.kv) return fail(Q35_ERR_INVALID_ARG, "layer %u: NULL weights/cache", l);
            Q35_TRY(check_full_layer(c, *L.full));
            Q35_TRY(check_kv(*L.kv, false));
            any_full = true;
        } else {
            return fail(Q35_ERR_INVALID_ARG, "layer %u: kind %u", l, L.kind);
        }
    }
    if (any_full) Q35_TRY(need(d->inv_freq, "inv_freq", false));
    if (tail) {
        if (c.vocab == 0) return fail(Q35_ERR_INVALID_ARG, "vocab is 0");
        Q35_TRY(check_weight("lm_head", *d->lm_head, c.vocab, c.hidden));
        Q35_TRY(need(d->final_norm, "final_norm"));
        Q35_TRY(need(d->tokens, "tokens", false));
        if (!d->embed || !aligned16(d->embed) || c.hidden % 8 != 0)
            return fail(Q35_ERR_INVALID_ARG, "embed NULL or not 16-byte aligned, or hidden %% 8 != 0");
        Q35_TRY(opt(d->logits, "logits"));
    }

    const uint32_t nst = [&] {
        uint32_t n = tail ? kStagesTail : 0;
        for (uint32_t l = 0; l < d->n_layers; ++l)
            n += d->layers[l].kind == Q35_LAYER_LINEAR ? kStagesGdn : kStagesFull;
        return n;
    }();
    const size_t act = f32 ? 4 : 2;
    Bump b{ws};
    uint32_t* ctl = static_cast<uint32_t*>(b.take(256));
    uint32_t* flags = static_cast<uint32_t*>(b.take(4u * blocks));
    uint64_t* stamps = static_cast<uint64_t*>(b.take(8u * nst));
    PStage* table = static_cast<PStage*>(b.take(sizeof(PStage) * nst));
    std::vector<void*> X(d->n_layers + 1);
    for (auto& x : X) x = b.take(act * c.hidden);
    std::vector<PStage> st;
    std::vector<uint32_t> first;
    auto gemv_stage = [&](int kind, const GemvBuild& gb) {
        PStage ps;
        std::memset(&ps, 0, sizeof(ps));
        ps.kind = kind;
        ps.g = gb.a;
        st.push_back(ps);
    };
    auto mlp = [&](const Q35QuantWeight& gp, const Q35QuantWeight& up, const Q35QuantWeight& dp,
                   const uint16_t* post_ln, float* x_resid, void* x_out) {
        float* h = b.f32(c.intermediate);
        GemvBuild g1(kOpGateUp, c.hidden, f32);
        g1.a.pro.kind = kProRmsF32;
        g1.a.pro.x = x_resid;
        g1.a.pro.w = post_ln;
        g1.a.pro.eps = c.rms_eps;
        g1.add(gp, kEpiSwiGLU, &up).out = h;
        gemv_stage(kStGateUp, g1);
        GemvBuild g2(kOpDown, c.intermediate, f32);
        g2.a.pro.kind = kProLoadF32;
        g2.a.pro.x = h;
        GemvSeg& sd = g2.add(dp, kEpiResidToAct);
        sd.pre4 = x_resid;
        sd.out_act = x_out;
        gemv_stage(kStDown, g2);
    };
    for (uint32_t l = 0; l < d->n_layers; ++l) {
        const Q35StackLayer& L = d->layers[l];
        first.push_back((uint32_t)st.size());
        float* x_resid = b.f32(c.hidden);
        if (L.kind == Q35_LAYER_LINEAR) {
            const LinearAttentionLayer& w = *L.linear;
            const uint32_t qt = qkv_total(c), zd = z_dim(c), Hv = c.num_v_heads_lin;
            float* qkv = b.f32(qt);
            float* z = b.f32(zd);
            float* gate = b.f32(Hv);
            float* beta = b.f32(Hv);
            float* y = b.f32(zd);
            GemvBuild g(kOpInGdn, c.hidden, f32);
            g.a.pro.kind = kProRmsAct;
            g.a.pro.x_f32 = f32;
            g.a.pro.x = X[l];
            g.a.pro.w = w.input_ln;
            g.a.pro.eps = c.rms_eps;
            GemvSeg& sq = g.add(w.in_proj_qkv, kEpiConv);
            sq.out = qkv;
            sq.state = L.state->conv1d_state;
            sq.pre16 = L.state->conv1d_state;
            sq.pre8 = w.conv1d_weight;
            g.add(w.in_proj_z, kEpiStore).out = z;
            GemvSeg& sa = g.add(w.in_proj_a, kEpiGate);
            sa.out = gate;
            sa.pre2 = w.dt_bias;
            sa.pre4 = w.a_log;
            g.add(w.in_proj_b, kEpiBeta).out = beta;
            gemv_stage(kStInGdn, g);
            PStage ps;
            std::memset(&ps, 0, sizeof(ps));
            ps.kind = kStGdn;
            ps.d.state = L.state->gdn_state;
            ps.d.qkv_conv = qkv;
            ps.d.gate = gate;
            ps.d.beta = beta;
            ps.d.y = y;
            ps.d.hk = c.num_k_heads_lin;
            ps.d.hv = Hv;
            ps.d.l2_eps = 1e-6f;
            ps.d.out_scale = 1.0f / std::sqrt((float)c.k_head_dim_lin);
            st.push_back(ps);
            GemvBuild go(kOpOutGated, zd, f32);
            go.a.pro.kind = kProGatedNorm;
            go.a.pro.x = y;
            go.a.pro.w = w.norm_weight;
            go.a.pro.z = z;
            go.a.pro.head_dim = c.v_head_dim_lin;
            go.a.pro.eps = c.rms_eps;
            GemvSeg& so = go.add(w.out_proj, kEpiResidActIn);
            so.out = x_resid;
            (f32 ? so.pre4 : so.pre2) = X[l];
            gemv_stage(kStOutGated, go);
            mlp(w.gate_proj, w.up_proj, w.down_proj, w.post_ln, x_resid, X[l + 1]);
        } else {
            const FullAttentionLayer& w = *L.full;
            float* qf = b.f32(q_total(c));
            float* kk = b.f32(kv_dim(c));
            float* vv = b.f32(kv_dim(c));
            float* ga = b.f32(q_only(c));
            float* pacc = b.f32((size_t)c.num_kv_heads * cpb * G * c.head_dim);
            float* pml = b.f32((size_t)c.num_kv_heads * cpb * 2 * G);
            GemvBuild g(kOpInFull, c.hidden, f32);
            g.a.pro.kind = kProRmsAct;
            g.a.pro.x_f32 = f32;
            g.a.pro.x = X[l];
            g.a.pro.w = w.input_ln;
            g.a.pro.eps = c.rms_eps;
            g.add(w.q_proj, kEpiStore).out = qf;
            g.add(w.k_proj, kEpiStore).out = kk;
            g.add(w.v_proj, kEpiStore).out = vv;
            gemv_stage(kStInFull, g);
            PStage ps;
            std::memset(&ps, 0, sizeof(ps));
            ps.kind = kStAttn;
            AttnArgs& a = ps.at;
            a.q_full = qf;
            a.k = kk;
            a.v = vv;
            a.q_norm = w.q_norm;
            a.k_norm = w.k_norm;
            a.inv_freq = d->inv_freq;
            a.positions = d->positions;
            a.kc = static_cast<uint16_t*>(L.kv->k);
            a.vc = static_cast<uint16_t*>(L.kv->v);
            a.gated_attn = ga;
            a.part_acc = pacc;
            a.part_ml = pml;
            a.capacity = L.kv->capacity;
            a.hq = c.num_heads;
            a.hkv = c.num_kv_heads;
            a.rotary = c.rotary_dim;
            a.max_chunks = cpb;
            a.host_pos = -1;
            a.eps = c.rms_eps;
            a.scale = 1.0f / std::sqrt((float)c.head_dim);
            st.push_back(ps);
            ps.kind = kStAttnMerge;
            st.push_back(ps);
            GemvBuild go(kOpOProj, q_only(c), f32);
            go.a.pro.kind = kProLoadF32;
            go.a.pro.x = ga;
            GemvSeg& so = go.add(w.o_proj, kEpiResidActIn);
            so.out = x_resid;
            (f32 ? so.pre4 : so.pre2) = X[l];
            gemv_stage(kStOProj, go);
            mlp(w.gate_proj, w.up_proj, w.down_proj, w.post_ln, x_resid, X[l + 1]);
        }
    }
    first.push_back((uint32_t)st.size());
    if (tail) {
        float* pval = b.f32(blocks);
        int32_t* pidx = reinterpret_cast<int32_t*>(b.f32(blocks));
        GemvBuild g(kOpLmHead, c.hidden, f32);
        g.a.pro.kind = kProRmsAct;
        g.a.pro.x_f32 = f32;
        g.a.pro.x = X[d->n_layers];
        g.a.pro.w = d->final_norm;
        g.a.pro.eps = c.rms_eps;
        g.add(*d->lm_head, kEpiArgmax).out = d->logits;
        g.a.am.part_val = pval;
        g.a.am.part_idx = pidx;
        gemv_stage(kStLmHead, g);
        PStage ps;
        std::memset(&ps, 0, sizeof(ps));
        ps.kind = kStFinish;
        LmFinishArgs& f = ps.f;
        f.part_val = pval;
        f.part_idx = pidx;
        f.nparts = blocks;
        f.vocab = c.vocab;
        f.tokens = d->tokens;
        f.positions = d->positions;
        f.history = d->history;
        f.history_len = d->history ? d->history_len : 0;
        f.history_base = d->history_base;
        f.embed = d->embed;
        f.x_next = X[0];
        f.hidden = c.hidden;
        f.act_f32 = f32 ? 1 : 0;
        st.push_back(ps);
    }
    if (st.size() != nst) return fail(Q35_ERR_INVALID_ARG, "internal: %zu stages != %u", st.size(), nst);
    *total = b.off;
    if (stages) *stages = std::move(st);
    if (plan) {
        plan->shape = shape;
        plan->blocks = blocks;
        plan->args.stages = table;
        plan->args.nstages = nst;
        plan->args.flags = flags;
        plan->args.ctl = ctl;
        plan->args.stamps = stamps;
        plan->n_layers = d->n_layers;
        plan->first_stage = first;
        plan->x_in = X;
    }
    return Q35_OK;
}

// Runs f with the plan's device current, restoring the caller's.
template <class F>
q35_status on_device(int dev, F&& f) {
    int prev = 0;
    Q35_HIP(hipGetDevice(&prev), "hipGetDevice");
    if (prev != dev) Q35_HIP(hipSetDevice(dev), "hipSetDevice");
    const q35_status st = f();
    if (prev != dev) (void)hipSetDevice(prev);
    return st;
}

}  // namespace

extern "C" {

q35_status q35_decode_workspace_bytes(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                      const Q35DecodeStackDesc* stack, size_t* bytes) {
    if (!bytes) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    size_t total = 0;
    Q35_TRY(plan_build(kernels, cfg, stack, nullptr, &total, nullptr, nullptr));
    *bytes = total;
    return ok();
}

q35_status q35_decode_plan_create(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                  const Q35DecodeStackDesc* stack, void* workspace,
                                  size_t workspace_bytes, Q35DecodePlan** out) {
    if (!out) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    *out = nullptr;
    size_t total = 0;
    Q35_TRY(plan_build(kernels, cfg, stack, nullptr, &total, nullptr, nullptr));
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(Q35_ERR_INVALID_ARG, "workspace NULL or not 256-byte aligned");
    if (workspace_bytes < total)
        return fail(Q35_ERR_INVALID_ARG, "workspace %zu bytes < %zu required", workspace_bytes, total);
    Q35DecodePlan* plan = new Q35DecodePlan();
    plan->device = kernels->device;
    std::vector<PStage> stages;
    q35_status st = plan_build(kernels, cfg, stack, static_cast<uint8_t*>(workspace), &total, &stages, plan);
    if (st == Q35_OK) {
        st = on_device(plan->device, [&]() -> q35_status {
            int coop = 0, khz = 0;
            Q35_HIP(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, plan->device),
                    "hipDeviceGetAttribute");
            if (!coop) return fail(Q35_ERR_UNSUPPORTED, "device %d cannot launch cooperatively", plan->device);
            Q35_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, plan->device),
                    "hipDeviceGetAttribute");
            if (khz <= 0) return fail(Q35_ERR_UNSUPPORTED, "no device wall clock");
            plan->clock_hz = (uint64_t)khz * 1000u;
            plan->args.spin_ticks = (uint64_t)(kWaitLimitSeconds * (double)plan->clock_hz);
            int per_cu = 0;
            Q35_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &per_cu, persist_kernel_ptr(plan->shape), kPersistThreads,
                        persist_lds_bytes(plan->shape)),
                    "hipOccupancyMaxActiveBlocksPerMultiprocessor");
            if (per_cu < 1) return fail(Q35_ERR_UNSUPPORTED, "the persistent kernel does not fit on a CU");
            Q35_HIP(hipMemcpy(const_cast<PStage*>(plan->args.stages), stages.data(),
                              stages.size() * sizeof(PStage), hipMemcpyHostToDevice),
                    "stage table upload");
            Q35_HIP(hipMemset(plan->args.ctl, 0, 256), "sync word clear");
            Q35_HIP(hipMemset(plan->args.flags, 0, 4u * plan->blocks), "sync word clear");
            Q35_HIP(hipMemset(plan->args.stamps, 0, 8u * plan->args.nstages), "stamp clear");
            if (stack->lm_head) {
                Q35_HIP(embed_launch(stack->embed, stack->tokens, cfg->vocab, cfg->hidden, plan->x_in[0],
                                     cfg->act_dtype == Q35_ACT_F32, nullptr),
                        "first embedding");
            }
            Q35_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
            return Q35_OK;
        });
    }
    if (st != Q35_OK) {
        delete plan;
        return st;
    }
    *out = plan;
    return ok();
}

void q35_decode_plan_release(Q35DecodePlan* plan) { delete plan; }

q35_status q35_decode_step(const Q35DecodePlan* plan, hipStream_t stream) {
    if (!plan) return fail(Q35_ERR_INVALID_ARG, "NULL plan");
    Q35_HIP(persist_launch(plan->shape, plan->args, plan->blocks, stream), "persistent decode launch");
    return ok();
}

q35_status q35_decode_check(const Q35DecodePlan* plan, uint32_t* error_word) {
    if (!plan || !error_word) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(on_device(plan->device, [&]() -> q35_status {
        Q35_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
        Q35_HIP(hipMemcpy(error_word, plan->args.ctl + 1, 4, hipMemcpyDeviceToHost), "error word read");
        return Q35_OK;
    }));
    return ok();
}

q35_status q35_decode_layer_input(const Q35DecodePlan* plan, uint32_t layer, void** x) {
    if (!plan || !x) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    if (layer > plan->n_layers) return fail(Q35_ERR_OUT_OF_RANGE, "layer %u > %u", layer, plan->n_layers);
    *x = plan->x_in[layer];
    return ok();
}

q35_status q35_decode_stage_layout(const Q35DecodePlan* plan, uint32_t* n_stages,
                                   uint32_t* layer_first_stage) {
    if (!plan) return fail(Q35_ERR_INVALID_ARG, "NULL plan");
    if (n_stages) *n_stages = plan->args.nstages;
    if (layer_first_stage)
        std::memcpy(layer_first_stage, plan->first_stage.data(), plan->first_stage.size() * sizeof(uint32_t));
    return ok();
}

q35_status q35_decode_stage_times(const Q35DecodePlan* plan, uint64_t* ticks, uint32_t n,
                                  uint64_t* ticks_per_second) {
    if (!plan || !ticks) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    if (n > plan->args.nstages) return fail(Q35_ERR_OUT_OF_RANGE, "%u > %u stages", n, plan->args.nstages);
    Q35_TRY(on_device(plan->device, [&]() -> q35_status {
        Q35_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
        Q35_HIP(hipMemcpy(ticks, plan->args.stamps, 8u * n, hipMemcpyDeviceToHost), "stamp read");
        return Q35_OK;
    }));
    if (ticks_per_second) *ticks_per_second = plan->clock_hz;
    return ok();
}

}  // extern "C"

// ------------------------------------------------------------------ XCD-split decode plan

struct Q35XcdPlan {
    int device;
    int shape;
    uint32_t blocks;
    uint32_t n_layers;
    uint32_t* ctl;  // [0] unused, [1] error word
    uint32_t* sync;
    uint32_t* probe;
    uint64_t spin_ticks;
    XStage* table;                                       // device copy of `stages`
    std::vector<XStage> stages;                          // [launch stages][kXcds], in step order
    std::vector<std::function<q35_status(hipStream_t)>> ops;  // one token's launches
    void* x_first;
    void* x_last;
    Q35XcdBuffers bufs;
};

namespace {

// The residual stream between launches: base + partial sums (fp32, in order).
struct XRes {
    const void* base;
    bool base_f32;
    const float* parts;
    uint32_t nparts;
};

// Segment over rows [row0, row0 + rows) of w (and w2), columns from col0 on;
// r rows per row group at the launch's K.
GemvSeg& xseg(GemvArgs& a, const Q35QuantWeight& w, uint32_t row0, uint32_t rows, uint32_t col0, uint32_t r,
              int32_t epi, const Q35QuantWeight* w2 = nullptr) {
    GemvSeg& s = a.seg[a.nseg++];
    const size_t kg = w.k / 64;
    s.codes[0] = w.codes + (size_t)row0 * w.k + col0;
    s.scales[0] = w.scales + row0 * kg + col0 / 64;
    s.biases[0] = w.biases + row0 * kg + col0 / 64;
    if (w2) {
        s.codes[1] = w2->codes + (size_t)row0 * w2->k + col0;
        s.scales[1] = w2->scales + row0 * kg + col0 / 64;
        s.biases[1] = w2->biases + row0 * kg + col0 / 64;
    }
    s.rg_begin = a.total_rg;
    s.rows = rows;
    a.total_rg += rows / r;
    s.rg_end = a.total_rg;
    s.epi = epi;
    return s;
}

void parts_pro(GemvPro& p, const XRes& in, const uint16_t* norm, float eps, bool round_bf16, void* sum_out) {
    p.kind = kProRmsParts;
    p.x = in.base;
    p.x_f32 = in.base_f32 ? 1 : 0;
    p.parts = in.parts;
    p.nparts = in.nparts;
    p.w = norm;
    p.eps = eps;
    p.sum_bf16 = round_bf16 ? 1 : 0;
    p.sum_out = sum_out;
}

// Validates the stack for the XCD-split plan, lays out the workspace and (when
// plan != nullptr) fills the plan.
q35_status xcd_build(const Qwen35Kernels* k, const Qwen35ForwardConfig* cfg, const Q35DecodeStackDesc* d,
                     uint8_t* ws, size_t* total, Q35XcdPlan* plan) {
    Q35_TRY(check_kernels(k));
    if (!cfg || !d) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(q35_config_validate(cfg));
    const Qwen35ForwardConfig& c = *cfg;
    const bool f32 = c.act_dtype == Q35_ACT_F32;
    const int shape = xcd_shape_id(c.hidden, c.intermediate, z_dim(c), c.k_head_dim_lin, !f32);
    if (!shape) return fail(Q35_ERR_UNSUPPORTED, "the XCD-split kernels are not built for these dimensions");
    const uint32_t blocks = (uint32_t)k->num_cu;
    const uint32_t nb = blocks / kXcds;
    const uint32_t Hk = c.num_k_heads_lin, Hv = c.num_v_heads_lin, dk = c.k_head_dim_lin, dv = c.v_head_dim_lin;
    if (blocks % kXcds != 0 || Hk % kXcds != 0 || Hv % kXcds != 0 || (Hv / kXcds) * (dv / 16) != nb ||
        c.intermediate % kXcds != 0)
        return fail(Q35_ERR_UNSUPPORTED, "%u compute units, %u/%u linear heads: no even split over %d XCDs",
                    blocks, Hk, Hv, kXcds);
    if (d->n_layers == 0 || !d->layers) return fail(Q35_ERR_INVALID_ARG, "empty stack");
    Q35_TRY(need(d->positions, "positions", false));
    const bool tail = d->lm_head != nullptr;
    uint32_t max_cap = 0;
    bool any_full = false;
    for (uint32_t l = 0; l < d->n_layers; ++l) {
        const Q35StackLayer& L = d->layers[l];
        if (L.kind == Q35_LAYER_LINEAR) {
            if (!L.linear || !L.state) return fail(Q35_ERR_INVALID_ARG, "layer %u: NULL weights/state", l);
            Q35_TRY(check_linear_layer(c, *L.linear, *L.state));
        } else if (L.kind == Q35_LAYER_FULL) {
            if (!L.full || !L.kv) return fail(Q35_ERR_INVALID_ARG, "layer %u: NULL weights/cache", l);
            Q35_TRY(check_full_layer(c, *L.full));
            Q35_TRY(check_kv(*L.kv, true));
            max_cap = std::max(max_cap, L.kv->capacity);
            any_full = true;
        } else {
            return fail(Q35_ERR_INVALID_ARG, "layer %u: kind %u", l, L.kind);
        }
    }
    if (any_full) Q35_TRY(need(d->inv_freq, "inv_freq", false));
    if (tail) {
        if (c.vocab == 0) return fail(Q35_ERR_INVALID_ARG, "vocab is 0");
        Q35_TRY(check_weight("lm_head", *d->lm_head, c.vocab, c.hidden));
        Q35_TRY(need(d->final_norm, "final_norm"));
        Q35_TRY(need(d->tokens, "tokens", false));
        if (!d->embed || !aligned16(d->embed) || c.hidden % 8 != 0)
            return fail(Q35_ERR_INVALID_ARG, "embed NULL or not 16-byte aligned, or hidden %% 8 != 0");
        Q35_TRY(opt(d->logits, "logits"));
    }

    const size_t act = f32 ? 4 : 2;
    const uint32_t H = c.hidden, I = c.intermediate, qt = qkv_total(c), zd = z_dim(c);
    uint32_t nxst = 0;
    for (uint32_t l = 0; l < d->n_layers; ++l)
        nxst += (d->layers[l].kind == Q35_LAYER_LINEAR ? kXcdStages[kXcdMixer] : 0) + kXcdStages[kXcdMlp];
    Bump b{ws};
    uint32_t* ctl = static_cast<uint32_t*>(b.take(256));
    uint32_t* sync = static_cast<uint32_t*>(b.take(kXcds * 256));
    // the placement probe's output: its own lines, never the counters' (another
    // XCD's cached copy of a counter line could outlive the clear)
    uint32_t* probe = static_cast<uint32_t*>(b.take(4u * blocks));
    XStage* table = static_cast<XStage*>(b.take(sizeof(XStage) * kXcds * nxst));
    void* x_first = b.take(act * H);
    void* x_in = b.take(act * H);
    void* x_last = b.take(act * H);
    float* x_mid = b.f32(H);
    float* x_res = b.f32(H);
    float* pmix = b.f32((size_t)kXcds * H);
    float* pmlp = b.f32((size_t)kXcds * H);
    float* qkv = b.f32(qt);
    float* z = b.f32(zd);
    float* gate = b.f32(Hv);
    float* beta = b.f32(Hv);
    float* y = b.f32(zd);
    float* h = b.f32(I);
    FullAttentionScratch fs;
    std::memset(&fs, 0, sizeof(fs));
    AttnWs aws{};
    if (any_full) {
        fs.q_full = b.f32(q_total(c));
        fs.k = b.f32(kv_dim(c));
        fs.v = b.f32(kv_dim(c));
        fs.gated_attn = b.f32(q_only(c));
        aws = attn_ws_layout(c, max_cap);
        fs.workspace = b.take(aws.total);
        fs.workspace_bytes = aws.total;
        fs.status = ctl ? ctl + 1 : nullptr;  // a position out of range is reported by q35_xcd_check
    }
    LmWs lws{};
    void* lm_ws = nullptr;
    if (tail) {
        lws = lm_ws_layout(c);
        lm_ws = b.take(lws.total);
    }
    *total = b.off;
    if (!plan) return Q35_OK;

    plan->shape = shape;
    plan->blocks = blocks;
    plan->n_layers = d->n_layers;
    plan->ctl = ctl;
    plan->sync = sync;
    plan->probe = probe;
    plan->table = table;
    plan->x_first = x_first;
    plan->x_last = x_last;
    Q35XcdBuffers& bf = plan->bufs;
    bf.x_in = x_in;
    bf.qkv_conv = qkv;
    bf.z = z;
    bf.gate = gate;
    bf.beta = beta;
    bf.y = y;
    bf.out_parts = pmix;
    bf.mlp_act = h;
    bf.mlp_parts = pmlp;
    bf.x_mid = x_mid;
    bf.x_resid = x_res;

    std::vector<XStage>& tab = plan->stages;
    auto& ops = plan->ops;
    const uint32_t num_cu = blocks;
    const uint32_t r_h = (uint32_t)gemv_rows_per_matrix_group(H, false);
    const uint32_t r_gu = (uint32_t)gemv_rows_per_matrix_group(H, true);
    const uint32_t r_z8 = (uint32_t)gemv_rows_per_matrix_group(zd / kXcds, false);
    const uint32_t r_i8 = (uint32_t)gemv_rows_per_matrix_group(I / kXcds, false);
    auto new_stage = [&](int kind) -> std::vector<XStage*> {
        std::vector<XStage*> v;
        const size_t at = tab.size();
        tab.resize(at + kXcds);
        for (int x = 0; x < kXcds; ++x) {
            XStage& s = tab[at + x];
            std::memset(&s, 0, sizeof(s));
            s.kind = kind;
            v.push_back(&s);
        }
        return v;
    };
    auto xcd_op = [&](int launch, size_t first_entry) {
        XcdArgs a;
        std::memset(&a, 0, sizeof(a));
        a.table = table + first_entry;
        a.sync = sync;
        a.err = ctl + 1;
        ops.push_back([plan, launch, a](hipStream_t s) mutable -> q35_status {
            a.spin_ticks = plan->spin_ticks;
            Q35_HIP(xcd_launch(plan->shape, launch, a, plan->blocks, s),
                    launch == kXcdMixer ? "XCD mixer launch" : "XCD MLP launch");
            return Q35_OK;
        });
    };
    // gate/up over XCD x's rows from the residual `in`, its sum written to x_res;
    // down over the matching columns into pmlp[x]
    auto mlp = [&](const Q35QuantWeight& gp, const Q35QuantWeight& up, const Q35QuantWeight& dp,
                   const uint16_t* post_ln, const XRes& in) {
        const size_t first = tab.size();
        const uint32_t i8 = I / kXcds;
        auto s0 = new_stage(kXsGateUp);
        for (int x = 0; x < kXcds; ++x) {
            GemvArgs& g = s0[x]->g;
            g.act_f32 = f32;
            parts_pro(g.pro, in, post_ln, c.rms_eps, false, x_res);
            xseg(g, gp, i8 * x, i8, 0, r_gu, kEpiSwiGLU, &up).out = h + i8 * x;
        }
        auto s1 = new_stage(kXsDownPart);
        for (int x = 0; x < kXcds; ++x) {
            GemvArgs& g = s1[x]->g;
            g.act_f32 = f32;
            g.pro.kind = kProLoadF32;
            g.pro.x = h + i8 * x;
            xseg(g, dp, 0, H, i8 * x, r_i8, kEpiStore).out = pmlp + (size_t)H * x;
        }
        xcd_op(kXcdMlp, first);
    };

    XRes in{x_first, f32, nullptr, 0};
    for (uint32_t l = 0; l < d->n_layers; ++l) {
        const Q35StackLayer& L = d->layers[l];
        if (L.kind == Q35_LAYER_LINEAR) {
            const LinearAttentionLayer& w = *L.linear;
            const size_t first = tab.size();
            const uint32_t qh = Hk * dk / kXcds, vh = Hv * dv / kXcds, ah = Hv / kXcds;
            auto s0 = new_stage(kXsInGdn);
            for (int x = 0; x < kXcds; ++x) {
                GemvArgs& g = s0[x]->g;
                g.act_f32 = f32;
                parts_pro(g.pro, in, w.input_ln, c.rms_eps, !f32, x_in);
                // q, k and v channels of the XCD's heads: conv + SiLU
                const uint32_t ch[3] = {qh * x, Hk * dk + qh * x, 2 * Hk * dk + vh * x};
                const uint32_t nch[3] = {qh, qh, vh};
                for (int j = 0; j < 3; ++j) {
                    GemvSeg& sq = xseg(g, w.in_proj_qkv, ch[j], nch[j], 0, r_h, kEpiConv);
                    sq.out = qkv + ch[j];
                    sq.state = L.state->conv1d_state + (size_t)ch[j] * 4;
                    sq.pre16 = sq.state;
                    sq.pre8 = w.conv1d_weight + (size_t)ch[j] * 4;
                }
                xseg(g, w.in_proj_z, vh * x, vh, 0, r_h, kEpiStore).out = z + vh * x;
                GemvSeg& sa = xseg(g, w.in_proj_a, ah * x, ah, 0, r_h, kEpiGate);
                sa.out = gate + ah * x;
                sa.pre2 = w.dt_bias + ah * x;
                sa.pre4 = w.a_log + ah * x;
                xseg(g, w.in_proj_b, ah * x, ah, 0, r_h, kEpiBeta).out = beta + ah * x;
            }
            auto s1 = new_stage(kXsGdn);
            for (int x = 0; x < kXcds; ++x) {
                GdnArgs& g = s1[x]->d;
                g.state = L.state->gdn_state;
                g.qkv_conv = qkv;
                g.gate = gate;
                g.beta = beta;
                g.y = y;
                g.hk = Hk;
                g.hv = Hv;
                g.l2_eps = 1e-6f;
                g.out_scale = 1.0f / std::sqrt((float)dk);
            }
            auto s2 = new_stage(kXsOutPart);
            for (int x = 0; x < kXcds; ++x) {
                GemvArgs& g = s2[x]->g;
                g.act_f32 = f32;
                g.pro.kind = kProGatedNorm;
                g.pro.x = y + vh * x;
                g.pro.z = z + vh * x;
                g.pro.w = w.norm_weight;
                g.pro.head_dim = dv;
                g.pro.eps = c.rms_eps;
                xseg(g, w.out_proj, 0, H, vh * x, r_z8, kEpiStore).out = pmix + (size_t)H * x;
            }
            xcd_op(kXcdMixer, first);
            mlp(w.gate_proj, w.up_proj, w.down_proj, w.post_ln, XRes{x_in, f32, pmix, (uint32_t)kXcds});
        } else {
            const FullAttentionLayer& w = *L.full;
            const LayerKvCache* kv = L.kv;
            {
                GemvBuild g(kOpInFullP, H, f32);
                parts_pro(g.a.pro, in, w.input_ln, c.rms_eps, !f32, x_in);
                g.add(w.q_proj, kEpiStore).out = fs.q_full;
                g.add(w.k_proj, kEpiStore).out = fs.k;
                g.add(w.v_proj, kEpiStore).out = fs.v;
                ops.push_back([g, num_cu](hipStream_t s) mutable -> q35_status {
                    return g.launch(num_cu, s, "q/k/v GEMV");
                });
            }
            {
                // the layer and cache descriptions are host structs read at creation: copied
                const Qwen35Kernels* kk = k;
                const Qwen35ForwardConfig cc = c;
                const FullAttentionLayer wl = w;
                const LayerKvCache kvc = *kv;
                const float* inv = d->inv_freq;
                const int32_t* pos = d->positions;
                ops.push_back([kk, cc, wl, fs, kvc, aws, inv, pos](hipStream_t s) -> q35_status {
                    return launch_attention(kk, cc, &wl, &fs, &kvc, aws, inv, pos, -1, 0, s);
                });
            }
            {
                GemvBuild g(kOpOProj, q_only(c), f32);
                g.a.pro.kind = kProLoadF32;
                g.a.pro.x = fs.gated_attn;
                GemvSeg& so = g.add(w.o_proj, kEpiResidActIn);
                so.out = x_mid;
                (f32 ? so.pre4 : so.pre2) = x_in;
                ops.push_back([g, num_cu](hipStream_t s) mutable -> q35_status {
                    return g.launch(num_cu, s, "o_proj GEMV");
                });
            }
            mlp(w.gate_proj, w.up_proj, w.down_proj, w.post_ln, XRes{x_mid, true, nullptr, 0});
        }
        in = XRes{x_res, true, pmlp, (uint32_t)kXcds};
    }
    // the last layer's output, whole, in the activation dtype
    ops.push_back([x_res, pmlp, H, x_last, f32](hipStream_t s) -> q35_status {
        Q35_HIP(xsum_launch(x_res, true, pmlp, kXcds, H, x_last, f32, s), "residual sum");
        return Q35_OK;
    });
    if (tail) {
        GemvBuild g(kOpLmHead, H, f32);
        g.a.pro.kind = kProRmsAct;
        g.a.pro.x_f32 = f32;
        g.a.pro.x = x_last;
        g.a.pro.w = d->final_norm;
        g.a.pro.eps = c.rms_eps;
        g.add(*d->lm_head, kEpiArgmax).out = d->logits;
        uint8_t* wsb = static_cast<uint8_t*>(lm_ws);
        g.a.am.part_val = reinterpret_cast<float*>(wsb + lws.val_off);
        g.a.am.part_idx = reinterpret_cast<int32_t*>(wsb + lws.idx_off);
        LmFinishArgs f;
        std::memset(&f, 0, sizeof(f));
        f.part_val = g.a.am.part_val;
        f.part_idx = g.a.am.part_idx;
        f.nparts = lws.blocks;
        f.vocab = c.vocab;
        f.tokens = d->tokens;
        f.positions = d->positions;
        f.history = d->history;
        f.history_len = d->history ? d->history_len : 0;
        f.history_base = d->history_base;
        f.embed = d->embed;
        f.x_next = x_first;
        f.hidden = H;
        f.act_f32 = f32 ? 1 : 0;
        const uint32_t lm_blocks = lws.blocks;
        ops.push_back([g, f, num_cu, lm_blocks](hipStream_t s) mutable -> q35_status {
            Q35_TRY(g.launch(num_cu, s, "lm_head GEMV", lm_blocks));
            Q35_HIP(lm_finish_launch(f, s), "lm_head argmax");
            return Q35_OK;
        });
    }
    if (tab.size() != (size_t)nxst * kXcds)
        return fail(Q35_ERR_INVALID_ARG, "internal: %zu stage entries != %u", tab.size(), nxst * kXcds);
    return Q35_OK;
}

}  // namespace

extern "C" {

q35_status q35_xcd_workspace_bytes(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                                   const Q35DecodeStackDesc* stack, size_t* bytes) {
    if (!bytes) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    size_t total = 0;
    Q35_TRY(xcd_build(kernels, cfg, stack, nullptr, &total, nullptr));
    *bytes = total;
    return ok();
}

q35_status q35_xcd_plan_create(const Qwen35Kernels* kernels, const Qwen35ForwardConfig* cfg,
                               const Q35DecodeStackDesc* stack, void* workspace, size_t workspace_bytes,
                               Q35XcdPlan** out) {
    if (!out) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    *out = nullptr;
    size_t total = 0;
    Q35_TRY(xcd_build(kernels, cfg, stack, nullptr, &total, nullptr));
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(Q35_ERR_INVALID_ARG, "workspace NULL or not 256-byte aligned");
    if (workspace_bytes < total)
        return fail(Q35_ERR_INVALID_ARG, "workspace %zu bytes < %zu required", workspace_bytes, total);
    Q35XcdPlan* plan = new Q35XcdPlan();
    plan->device = kernels->device;
    q35_status st = xcd_build(kernels, cfg, stack, static_cast<uint8_t*>(workspace), &total, plan);
    if (st == Q35_OK) {
        st = on_device(plan->device, [&]() -> q35_status {
            int khz = 0;
            Q35_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, plan->device),
                    "hipDeviceGetAttribute");
            if (khz <= 0) return fail(Q35_ERR_UNSUPPORTED, "no device wall clock");
            plan->spin_ticks = (uint64_t)(kWaitLimitSeconds * (double)khz * 1000.0);
            for (int launch : {kXcdMixer, kXcdMlp}) {
                int per_cu = 0;
                Q35_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, xcd_kernel_ptr(plan->shape, launch),
                                                                     kXcdThreads, 0),
                        "hipOccupancyMaxActiveBlocksPerMultiprocessor");
                if (per_cu != 1)
                    return fail(Q35_ERR_UNSUPPORTED, "the XCD kernels fit %d blocks per CU, not one", per_cu);
            }
            // placement: XCD of block b = (b + c) % 8 for one c (the dispatcher's
            // turn order; c may differ from launch to launch)
            XcdArgs pa;
            std::memset(&pa, 0, sizeof(pa));
            pa.probe = plan->probe;
            Q35_HIP(xcd_launch(plan->shape, kXcdMixer, pa, plan->blocks, nullptr), "XCD placement probe");
            std::vector<uint32_t> where(plan->blocks);
            Q35_HIP(hipMemcpy(where.data(), plan->probe, 4u * plan->blocks, hipMemcpyDeviceToHost), "probe read");
            for (uint32_t i = 0; i < plan->blocks; ++i)
                if (where[i] >= (uint32_t)kXcds || (where[i] + kXcds - i % kXcds) % kXcds != where[0])
                    return fail(Q35_ERR_UNSUPPORTED, "block %u ran on XCD %u, block 0 on %u: not one residue "
                                                     "class of the block index per XCD", i, where[i], where[0]);
            Q35_HIP(hipMemcpy(plan->table, plan->stages.data(), plan->stages.size() * sizeof(XStage),
                              hipMemcpyHostToDevice),
                    "stage table upload");
            Q35_HIP(hipMemset(plan->ctl, 0, 256), "sync word clear");
            Q35_HIP(hipMemset(plan->sync, 0, kXcds * 256), "sync word clear");
            if (stack->lm_head) {
                Q35_HIP(embed_launch(stack->embed, stack->tokens, cfg->vocab, cfg->hidden, plan->x_first,
                                     cfg->act_dtype == Q35_ACT_F32, nullptr),
                        "first embedding");
            }
            Q35_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
            return Q35_OK;
        });
    }
    if (st != Q35_OK) {
        delete plan;
        return st;
    }
    *out = plan;
    return ok();
}

void q35_xcd_plan_release(Q35XcdPlan* plan) { delete plan; }

q35_status q35_xcd_step(const Q35XcdPlan* plan, hipStream_t stream) {
    if (!plan) return fail(Q35_ERR_INVALID_ARG, "NULL plan");
    for (const auto& op : plan->ops) Q35_TRY(op(stream));
    return ok();
}

q35_status q35_xcd_check(const Q35XcdPlan* plan, uint32_t* error_word) {
    if (!plan || !error_word) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    Q35_TRY(on_device(plan->device, [&]() -> q35_status {
        Q35_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
        Q35_HIP(hipMemcpy(error_word, plan->ctl + 1, 4, hipMemcpyDeviceToHost), "error word read");
        return Q35_OK;
    }));
    return ok();
}

q35_status q35_xcd_layer_input(const Q35XcdPlan* plan, uint32_t layer, void** x) {
    if (!plan || !x) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    if (layer != 0 && layer != plan->n_layers)
        return fail(Q35_ERR_OUT_OF_RANGE, "layer %u: only the first input (0) and the last output (%u) are whole vectors",
                    layer, plan->n_layers);
    *x = layer == 0 ? plan->x_first : plan->x_last;
    return ok();
}

q35_status q35_xcd_buffers(const Q35XcdPlan* plan, Q35XcdBuffers* bufs) {
    if (!plan || !bufs) return fail(Q35_ERR_INVALID_ARG, "NULL argument");
    *bufs = plan->bufs;
    return ok();
}

}  // extern "C"
