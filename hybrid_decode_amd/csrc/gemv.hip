// Int8 group-64 affine-dequant GEMV family for batch-1 decode (gfx950).
//
// y[n] = sum_k (scale[n][k/64] * code[n][k] + bias[n][k/64]) * x[k]
//      = sum_g scale[n][g] * (sum_{k in g} code[n][k] x[k]) + bias[n][g] * (sum_{k in g} x[k])
//
// This is the weight trait of the pages (the `gemv`, `gemv_gate_up_with`,
// `gemv_silu_gate` and `gemv_silu_gate_resid` calls of both layer forwards)
// for MLX-style 8-bit weights with 64-wide groups.
//
// Work decomposition.  Each wave streams whole "row groups": GR consecutive
// rows (GR*K bytes of codes), chosen so that GR*K/16 is a multiple of 64.
// Lane l then owns the 16-byte chunks c = l + 64*i (i < NC), loads each with
// one 128-bit load, and the chunk->(row, column) map is the same for every row
// group, so every wave-wide load is one fully coalesced 1 KB stream segment.
// Several matrices that read the same x (q/k/v; qkv/z/a/b; gate+up) run in one
// launch as consecutive "segments" of the row-group space.  A paired segment
// (gate+up) puts R gate rows and the same R up rows into one row group so the
// SwiGLU product can be formed in the epilogue.
//
// x (after a fused prologue: RMSNorm, gated per-head RMSNorm, or a plain load)
// lives in LDS as fp32, laid out [4][K/16] float4 so that the lanes of a wave
// read consecutive 16-byte words (no bank conflicts), plus the 16-element chunk
// sums needed by the bias term.  The first row group's weight loads are issued
// before the prologue so their latency overlaps it; after that each wave keeps
// one row group in flight and occupancy (several waves per SIMD) hides the
// memory latency.
#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {

namespace {

constexpr int kNT = 256;  // threads per block (4 waves)

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

template <int K, bool PAIRED>
struct Geo {
    static constexpr int KC = K / 16;                      // 16-byte chunks per row
    static constexpr int R = 64 / gcd_c(64, KC);           // rows of one matrix per row group
    static constexpr int GR = PAIRED ? 2 * R : R;          // rows per row group
    static constexpr int NC = GR * KC / 64;                // chunks per lane per row group
    static constexpr int MC = (KC + kNT - 1) / kNT;        // prologue chunks per thread
    static constexpr int NCH = PAIRED ? NC / 2 : NC;       // distinct x chunks per lane
    static constexpr bool XREG = NCH <= 5;                 // keep x in registers across row groups
    static_assert(K % 64 == 0, "K must be a multiple of the group size");
    static_assert((GR * KC) % 64 == 0, "row group must tile the wave");
};

struct Regs1 {
    uint4 w;
    uint32_t s, b;
};

Q35_DEV float dot16(const uint4& w, const float4& x0, const float4& x1, const float4& x2,
                    const float4& x3) {
    float a0 = (float)(w.x & 0xFFu) * x0.x;
    float a1 = (float)((w.x >> 8) & 0xFFu) * x0.y;
    float a2 = (float)((w.x >> 16) & 0xFFu) * x0.z;
    float a3 = (float)(w.x >> 24) * x0.w;
    a0 = fmaf((float)(w.y & 0xFFu), x1.x, a0);
    a1 = fmaf((float)((w.y >> 8) & 0xFFu), x1.y, a1);
    a2 = fmaf((float)((w.y >> 16) & 0xFFu), x1.z, a2);
    a3 = fmaf((float)(w.y >> 24), x1.w, a3);
    a0 = fmaf((float)(w.z & 0xFFu), x2.x, a0);
    a1 = fmaf((float)((w.z >> 8) & 0xFFu), x2.y, a1);
    a2 = fmaf((float)((w.z >> 16) & 0xFFu), x2.z, a2);
    a3 = fmaf((float)(w.z >> 24), x2.w, a3);
    a0 = fmaf((float)(w.w & 0xFFu), x3.x, a0);
    a1 = fmaf((float)((w.w >> 8) & 0xFFu), x3.y, a1);
    a2 = fmaf((float)((w.w >> 16) & 0xFFu), x3.z, a2);
    a3 = fmaf((float)(w.w >> 24), x3.w, a3);
    return (a0 + a1) + (a2 + a3);
}

// Find the segment that owns row group rg (segments are sorted, contiguous).
Q35_DEV int find_seg(const GemvArgs& a, uint32_t rg) {
    int s = 0;
#pragma unroll
    for (int i = 1; i < kMaxSegs; ++i)
        if (i < a.nseg && rg >= a.seg[i].rg_begin) s = i;
    return s;
}

// ---------------------------------------------------------------- prologue

template <int K>
Q35_DEV void write_chunk(float4* xq, float* xs, int cc, const float v[16]) {
    constexpr int KC = K / 16;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        xq[j * KC + cc] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    xs[cc] = s;
}

Q35_DEV void load16(const void* src, bool is_f32, uint32_t base, float v[16]) {
    if (is_f32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + base);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4 t = p[j];
            v[4 * j] = t.x;
            v[4 * j + 1] = t.y;
            v[4 * j + 2] = t.z;
            v[4 * j + 3] = t.w;
        }
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + base);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            uint4 t = p[j];
            v[8 * j + 0] = bf16_lo(t.x);
            v[8 * j + 1] = bf16_hi(t.x);
            v[8 * j + 2] = bf16_lo(t.y);
            v[8 * j + 3] = bf16_hi(t.y);
            v[8 * j + 4] = bf16_lo(t.z);
            v[8 * j + 5] = bf16_hi(t.z);
            v[8 * j + 6] = bf16_lo(t.w);
            v[8 * j + 7] = bf16_hi(t.w);
        }
    }
}

template <int K>
Q35_DEV void prologue(const GemvPro& p, float4* xq, float* xs, float* red) {
    using G = Geo<K, false>;
    constexpr int KC = G::KC, MC = G::MC;
    const int t = threadIdx.x;
    const bool tap = (p.tap != nullptr) && blockIdx.x == 0;

    if (p.kind == kProLoadF32) {
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            int cc = t + kNT * m;
            if (cc < KC) {
                float v[16];
                load16(p.x, true, 16u * cc, v);
                write_chunk<K>(xq, xs, cc, v);
            }
        }
        return;
    }

    if (p.kind == kProRmsAct || p.kind == kProRmsF32) {
        const bool f32 = (p.kind == kProRmsF32) || p.x_f32;
        float v[MC][16];
        float ss = 0.f;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            int cc = t + kNT * m;
            if (cc < KC) {
                load16(p.x, f32, 16u * cc, v[m]);
#pragma unroll
                for (int j = 0; j < 16; ++j) ss = fmaf(v[m][j], v[m][j], ss);
            }
        }
        ss = block_sum<kNT>(ss, red);
        const float rs = 1.0f / sqrtf(ss / (float)K + p.eps);
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            int cc = t + kNT * m;
            if (cc < KC) {
                const uint4* wp = reinterpret_cast<const uint4*>(p.w + 16u * cc);
                uint4 w0 = wp[0], w1 = wp[1];
                uint32_t wr[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    v[m][2 * j] = v[m][2 * j] * rs * bf16_lo(wr[j]);
                    v[m][2 * j + 1] = v[m][2 * j + 1] * rs * bf16_hi(wr[j]);
                }
                if (tap) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) p.tap[16 * cc + j] = v[m][j];
                }
                write_chunk<K>(xq, xs, cc, v[m]);
            }
        }
        return;
    }

    // kProGatedNorm: x = RMSNorm_head(y; w) * silu(z); heads of p.head_dim.
    const int per_head = (int)p.head_dim / 16;  // chunks per head: 2, 4 or 8
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        int cc = t + kNT * m;
        float v[16];
        float ss = 0.f;
        if (cc < KC) {
            load16(p.x, true, 16u * cc, v);
#pragma unroll
            for (int j = 0; j < 16; ++j) ss = fmaf(v[j], v[j], ss);
        }
        for (int o = 1; o < per_head; o <<= 1) ss += __shfl_xor(ss, o);
        if (cc < KC) {
            const float rs = 1.0f / sqrtf(ss / (float)p.head_dim + p.eps);
            const uint32_t d0 = (16u * cc) % p.head_dim;
            const uint4* wp = reinterpret_cast<const uint4*>(p.w + d0);
            uint4 w0 = wp[0], w1 = wp[1];
            uint32_t wr[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            float zz[16];
            load16(p.z, true, 16u * cc, zz);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[2 * j] = v[2 * j] * rs * bf16_lo(wr[j]);
                v[2 * j + 1] = v[2 * j + 1] * rs * bf16_hi(wr[j]);
            }
            if (tap) {
#pragma unroll
                for (int j = 0; j < 16; ++j) p.tap[16 * cc + j] = v[j];
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] *= siluf_(zz[j]);
            write_chunk<K>(xq, xs, cc, v);
        }
    }
}

// ---------------------------------------------------------------- epilogue (one row)

Q35_DEV void epilogue(const GemvArgs& a, const GemvSeg& s, uint32_t n, float v, float v2,
                      float& best_v, int& best_i) {
    switch (s.epi) {
        case kEpiStore:
            s.out[n] = v;
            break;
        case kEpiResidActIn: {
            if (s.tap0) s.tap0[n] = v;
            s.out[n] = load_act(s.aux0, n, a.act_f32) + v;
            break;
        }
        case kEpiResidToAct: {
            float r = static_cast<const float*>(s.aux0)[n] + v;
            store_act(s.out_act, n, r, a.act_f32);
            if (s.out_act2) store_act(s.out_act2, n, r, a.act_f32);
            break;
        }
        case kEpiConv: {
            if (s.tap0) s.tap0[n] = v;
            float4* st = reinterpret_cast<float4*>(s.state) + n;
            float4 o = *st;
            uint2 w = reinterpret_cast<const uint2*>(s.aux0)[n];
            float u = bf16_lo(w.x) * o.y;
            u = fmaf(bf16_hi(w.x), o.z, u);
            u = fmaf(bf16_lo(w.y), o.w, u);
            u = fmaf(bf16_hi(w.y), v, u);
            *st = make_float4(o.y, o.z, o.w, v);
            s.out[n] = siluf_(u);
            break;
        }
        case kEpiGate: {
            if (s.tap0) s.tap0[n] = v;
            float dtb = bf16_to_f32(static_cast<const uint16_t*>(s.aux0)[n]);
            float al = static_cast<const float*>(s.aux1)[n];
            s.out[n] = expf(-expf(al) * softplusf_(v + dtb));
            break;
        }
        case kEpiBeta:
            if (s.tap0) s.tap0[n] = v;
            s.out[n] = sigmoidf_(v);
            break;
        case kEpiSwiGLU:
            if (s.tap0) s.tap0[n] = v;
            if (s.tap1) s.tap1[n] = v2;
            s.out[n] = siluf_(v) * v2;
            break;
        case kEpiArgmax:
            if (s.out) s.out[n] = v;
            if (v > best_v || (v == best_v && (int)n < best_i)) {
                best_v = v;
                best_i = (int)n;
            }
            break;
        default:
            break;
    }
}

// ---------------------------------------------------------------- argmax finish

Q35_DEV bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

Q35_DEV void argmax_finish(const GemvArgs& a, float best_v, int best_i, float* red) {
    int* redi = reinterpret_cast<int*>(red + 8);
    __shared__ int is_last;
    // wave reduce
    for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(best_v, o);
        int oi = __shfl_xor(best_i, o);
        if (better(ov, oi, best_v, best_i)) {
            best_v = ov;
            best_i = oi;
        }
    }
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
        red[wid] = best_v;
        redi[wid] = best_i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float bv = red[0];
        int bi = redi[0];
        for (int w = 1; w < kNT / 64; ++w)
            if (better(red[w], redi[w], bv, bi)) {
                bv = red[w];
                bi = redi[w];
            }
        a.am.part_val[blockIdx.x] = bv;
        a.am.part_idx[blockIdx.x] = bi;
        __threadfence();
        unsigned prev = __hip_atomic_fetch_add(a.am.counter, 1u, __ATOMIC_ACQ_REL,
                                               __HIP_MEMORY_SCOPE_AGENT);
        is_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (uint32_t b = threadIdx.x; b < gridDim.x; b += kNT) {
        float v = __hip_atomic_load(a.am.part_val + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int i = __hip_atomic_load(a.am.part_idx + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (better(v, i, bv, bi)) {
            bv = v;
            bi = i;
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o);
        int oi = __shfl_xor(bi, o);
        if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    __syncthreads();
    if (lane == 0) {
        red[wid] = bv;
        redi[wid] = bi;
    }
    __syncthreads();
    __shared__ int tok_sh;
    if (threadIdx.x == 0) {
        bv = red[0];
        bi = redi[0];
        for (int w = 1; w < kNT / 64; ++w)
            if (better(red[w], redi[w], bv, bi)) {
                bv = red[w];
                bi = redi[w];
            }
        int tok = (bi >= 0 && (uint32_t)bi < a.am.vocab) ? bi : 0;
        tok_sh = tok;
        a.am.tokens[0] = tok;
        int pos = a.am.positions ? a.am.positions[0] : 0;
        if (a.am.history) {
            int hidx = pos - a.am.history_base;
            if (hidx >= 0 && (uint32_t)hidx < a.am.history_len) a.am.history[hidx] = tok;
        }
        if (a.am.positions) a.am.positions[0] = pos + 1;
        __hip_atomic_store(a.am.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (a.am.embed) {
        const uint16_t* row = a.am.embed + (size_t)tok_sh * a.am.hidden;
        for (uint32_t k = threadIdx.x; k < a.am.hidden; k += kNT)
            store_act(a.am.x_next, k, bf16_to_f32(row[k]), a.act_f32);
    }
}

// ---------------------------------------------------------------- the kernel

template <int K, bool PAIRED>
__global__ __launch_bounds__(kNT) void gemv_kernel(GemvArgs a) {
    using G = Geo<K, PAIRED>;
    constexpr int KC = G::KC, R = G::R, GR = G::GR, NC = G::NC;
    constexpr int KG = K / 64;  // scale groups per row

    extern __shared__ float4 smem4[];
    float4* xq = smem4;
    float* xs = reinterpret_cast<float*>(smem4 + 4 * KC);
    float* red = xs + KC;

    const int lane = threadIdx.x & 63;
    const uint32_t nw = gridDim.x * (kNT / 64);
    uint32_t rg = blockIdx.x * (kNT / 64) + (threadIdx.x >> 6);
    const uint32_t total = a.total_rg;

    // chunk i of this lane: c = lane + 64 i, in row slot c / KC, column chunk c % KC
    auto load_rg = [&](uint32_t g, Regs1 (&r)[NC]) {
        const GemvSeg& s = a.seg[find_seg(a, g)];
        const uint32_t row0 = (g - s.rg_begin) * R;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
            const int sl = c / KC, cc = c - sl * KC;
            const int m = (PAIRED && sl >= R) ? 1 : 0;
            const uint32_t row = row0 + (uint32_t)(sl - m * R);
            const uint8_t* cp = m ? s.codes[1] : s.codes[0];
            const uint16_t* sp = m ? s.scales[1] : s.scales[0];
            const uint16_t* bp = m ? s.biases[1] : s.biases[0];
            r[i].w = *reinterpret_cast<const uint4*>(cp + (size_t)row * K + 16u * cc);
            r[i].s = sp[(size_t)row * KG + (cc >> 2)];
            r[i].b = bp[(size_t)row * KG + (cc >> 2)];
        }
    };

    // the first row group's weights are requested before the prologue runs
    Regs1 cur[NC];
    if (rg < total) load_rg(rg, cur);

    prologue<K>(a.pro, xq, xs, red);
    __syncthreads();

    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;

    while (rg < total) {
        // Wide rows: keep x in LDS (an opaque zero offset stops the compiler from
        // hoisting all NC chunks of x into registers, which would cost occupancy).
        // Narrow rows: the hoisted copy of x stays in registers across row groups.
        int xo = 0;
        if constexpr (!G::XREG) asm volatile("" : "+v"(xo));
        float acc[GR];
#pragma unroll
        for (int j = 0; j < GR; ++j) acc[j] = 0.f;
#pragma unroll
        for (int i = 0; i < G::NCH; ++i) {
            const int c = lane + 64 * i;
            const int sl = c / KC, cc = c - sl * KC + xo;
            const float4 x0 = xq[cc], x1 = xq[KC + cc], x2 = xq[2 * KC + cc], x3 = xq[3 * KC + cc];
            const float xsum = xs[cc];
#pragma unroll
            for (int m = 0; m < (PAIRED ? 2 : 1); ++m) {
                const Regs1& w = cur[i + m * G::NCH];
                float p = dot16(w.w, x0, x1, x2, x3);
                p = fmaf(bf16_to_f32(w.s), p, bf16_to_f32(w.b) * xsum);
                // chunk i + m*NCH lies in row slot sl + m*R (paired: the same columns of B)
                const int lo = (64 * i) / KC, hi = (64 * i + 63) / KC;
#pragma unroll
                for (int j = lo; j <= hi; ++j) acc[j + m * R] += (sl == j) ? p : 0.f;
            }
        }
        float tot[GR];
#pragma unroll
        for (int j = 0; j < GR; ++j) tot[j] = wave_sum(acc[j]);

        const GemvSeg& s = a.seg[find_seg(a, rg)];
        const uint32_t row0 = (rg - s.rg_begin) * R;
        if (lane < R) {
            float v = 0.f, v2 = 0.f;
#pragma unroll
            for (int j = 0; j < R; ++j)
                if (lane == j) {
                    v = tot[j];
                    if constexpr (PAIRED) v2 = tot[j + R];
                }
            epilogue(a, s, row0 + lane, v, v2, best_v, best_i);
        }
        rg += nw;
        if (rg < total) load_rg(rg, cur);
    }

    if (a.am.counter != nullptr) argmax_finish(a, best_v, best_i, red);
}

template <int K, bool PAIRED>
hipError_t launch_t(const GemvArgs& a, uint32_t blocks, hipStream_t stream) {
    using G = Geo<K, PAIRED>;
    const size_t lds = (size_t)G::KC * (4 * sizeof(float4) + sizeof(float)) + 16 * sizeof(float);
    hipLaunchKernelGGL((gemv_kernel<K, PAIRED>), dim3(blocks), dim3(kNT), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

int gemv_rows_per_group(uint32_t k, bool paired) {
    const int kc = (int)k / 16;
    const int r = 64 / gcd_c(64, kc);
    return paired ? 2 * r : r;
}

int gemv_rows_per_matrix_group(uint32_t k) { return 64 / gcd_c(64, (int)k / 16); }

uint32_t gemv_pick_blocks(uint32_t total_rg) {
    // ~8 waves per CU on 256 CUs, with the row groups spread evenly over waves
    const uint32_t target_waves = 256u * 8u;
    uint32_t per_wave = (total_rg + target_waves - 1) / target_waves;
    if (per_wave == 0) per_wave = 1;
    uint32_t waves = (total_rg + per_wave - 1) / per_wave;
    uint32_t blocks = (waves + 3) / 4;
    return blocks ? blocks : 1;
}

// K values compiled in.  Paired (gate+up) launches only ever use K = hidden.
#define Q35_GEMV_WIDTHS(X) \
    X(128) X(256) X(512) X(1024) X(2048) X(2560) X(3072) X(4096) X(5120) X(6144) X(8192) \
    X(9216) X(12288)
#define Q35_PAIRED_MAX_K 8192

bool gemv_width_supported(uint32_t k) {
#define X(KK) if (k == KK) return true;
    Q35_GEMV_WIDTHS(X)
#undef X
    return false;
}

hipError_t gemv_launch(uint32_t k, bool paired, const GemvArgs& a, uint32_t blocks,
                       hipStream_t stream) {
#define X(KK)                                                                        \
    if (k == KK) {                                                                   \
        if constexpr (KK <= Q35_PAIRED_MAX_K)                                        \
            if (paired) return launch_t<KK, true>(a, blocks, stream);                \
        return paired ? hipErrorInvalidValue : launch_t<KK, false>(a, blocks, stream); \
    }
    Q35_GEMV_WIDTHS(X)
#undef X
    return hipErrorInvalidValue;
}

const void* gemv_kernel_ptr(uint32_t k, bool paired) {
#define X(KK)                                                                   \
    if (k == KK) {                                                              \
        if constexpr (KK <= Q35_PAIRED_MAX_K)                                   \
            if (paired) return (const void*)&gemv_kernel<KK, true>;             \
        return paired ? nullptr : (const void*)&gemv_kernel<KK, false>;         \
    }
    Q35_GEMV_WIDTHS(X)
#undef X
    return nullptr;
}

}  // namespace q35
