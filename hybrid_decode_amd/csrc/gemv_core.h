// Int8 group-64 affine-dequant GEMV family for batch-1 decode (gfx950).
//
// y[n] = sum_k (scale[n][k/64] * code[n][k] + bias[n][k/64]) * x[k]
//      = sum_g scale[n][g] * (sum_{k in g} code[n][k] x[k]) + bias[n][g] * (sum_{k in g} x[k])
//
// This is the weight trait of the pages (the `gemv`, `gemv_gate_up_with`,
// `gemv_silu_gate` and `gemv_silu_gate_resid` calls of both layer forwards)
// for MLX-style 8-bit weights with 64-wide groups.  Each kernel is specialised
// by its operation: the prologue that forms x (RMSNorm, gated per-head RMSNorm,
// or a plain load) and, per matrix segment, the epilogue that consumes each
// output row (store, residual add, conv update, decay gate, beta, SwiGLU,
// argmax) are compiled in, so a launch runs only its own code.
//
// Work decomposition.  A launch covers several matrices that read the same x
// (q/k/v; qkv/z/a/b; gate+up) as consecutive "segments" of one row-group space.
// A row group is 64/LR rows; LR = gcd(64, K/16) lanes of a wave share one row
// and each lane streams K/(16 LR) 16-byte chunks of it, so every lane works on
// exactly one row and every wave-wide load covers LR*16 contiguous bytes per
// row.  For the paired gate+up segment LR = gcd(32, K/16) and the row slots of
// a wave alternate gate row / up row of the same index, so the SwiGLU product
// is formed in the epilogue.  Loads go through buffer resources: one SGPR
// descriptor per matrix, a lane-constant 32-bit offset, and the row group's
// offset as the scalar offset, so a load is one instruction with no per-load
// address arithmetic; code loads are marked non-temporal (streamed once).
//
// Ordering.  A wave first issues the loads of its share of x (and the norm
// weights), then the loads of its first row group of weights, then builds x in
// LDS: vector loads complete in order, so waiting for x does not wait for the
// weights, and the weights stream in while the prologue runs.  Row groups are
// spread so that the resident waves cover the whole matrix in one or a few row
// groups each; occupancy hides the rest.
//
// Arithmetic.  Two variants, chosen by the activation dtype of the layer:
//  * fp32 (HALF = false): codes -> fp32 (v_cvt_f32_ubyteN), fp32 FMAs.
//  * HALF: x is held as f16 after a power-of-two scaling of the whole vector
//    (11 significant bits: finer than the bf16 the activations are stored in,
//    and the scaling keeps it clear of f16 overflow).  One v_perm_b32 turns two
//    code bytes into the exact f16 pair (1024 + q0, 1024 + q1) and one
//    v_dot2_f32_f16 multiplies it into an fp32 sum, so sum (1024+q) x =
//    sum q x + 1024 sum x; the 1024 sum x term is folded into the bias:
//    y = s * dot' + (b - 1024 s) * sum x.  Products of f16 inputs are exact in
//    fp32 and accumulation is fp32, so the only extra rounding is that of x.
// x (and its 16-element chunk sums, needed by the bias term) lives in LDS,
// laid out so that the lanes of a wave read consecutive 16-byte words.
#pragma once

#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace gemv {

constexpr int kNT = 256;  // threads per block (4 waves)

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- operations

template <int OP>
struct Op;
template <>
struct Op<kOpPlain> {
    static constexpr bool PAIRED = false;
    static constexpr int PRO = kProLoadF32, NSEG = 1;
};
template <>
struct Op<kOpInGdn> {  // segments: qkv (conv), z, a (gate), b (beta)
    static constexpr bool PAIRED = false;
    static constexpr int PRO = kProRmsAct, NSEG = 4;
};
template <>
struct Op<kOpInFull> {  // segments: q, k, v
    static constexpr bool PAIRED = false;
    static constexpr int PRO = kProRmsAct, NSEG = 3;
};
template <>
struct Op<kOpOutGated> {
    static constexpr bool PAIRED = false;
    static constexpr int PRO = kProGatedNorm, NSEG = 1;
};
template <>
struct Op<kOpOProj> {
    static constexpr bool PAIRED = false;
    static constexpr int PRO = kProLoadF32, NSEG = 1;
};
template <>
struct Op<kOpGateUp> {
    static constexpr bool PAIRED = true;
    static constexpr int PRO = kProRmsF32, NSEG = 1;
};
template <>
struct Op<kOpDown> {
    static constexpr bool PAIRED = false;
    static constexpr int PRO = kProLoadF32, NSEG = 1;
};
template <>
struct Op<kOpLmHead> {
    static constexpr bool PAIRED = false;
    static constexpr int PRO = kProRmsAct, NSEG = 1;
};

template <int K, bool PAIRED>
struct Geo {
    static constexpr int KC = K / 16;                                  // 16-byte chunks per row
    static constexpr int LR = PAIRED ? gcd_c(32, KC) : gcd_c(64, KC);  // lanes per row
    static constexpr int SLOTS = 64 / LR;                              // rows per row group
    static constexpr int R = PAIRED ? SLOTS / 2 : SLOTS;               // rows of each matrix per row group
    static constexpr int NC = KC / LR;                                 // chunks per lane
    static constexpr int MC = (KC + kNT - 1) / kNT;                    // prologue chunks per thread
    static_assert(K % 64 == 0, "K must be a multiple of the group size");
    static_assert(LR >= 8, "rows must span at least 8 lanes");
};

// ---------------------------------------------------------------- dot products

// fp32 variant: 16 codes times 16 fp32 x values
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

// HALF variant: returns sum_j (1024 + q_j) * x_j for 16 codes and 16 f16 x values
// (xa holds x0..x7, xb x8..x15, each dword an f16 pair).
constexpr uint32_t kF16Exp1024 = 0x64646464u;  // 0x64 is the high byte of f16 1024.0
constexpr uint32_t kSelLo = 0x04010400u;       // bytes [q0, 0x64, q1, 0x64]
constexpr uint32_t kSelHi = 0x04030402u;       // bytes [q2, 0x64, q3, 0x64]

Q35_DEV float fdot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
}

Q35_DEV float dot16h(const uint4& w, const uint4& xa, const uint4& xb) {
    float a0 = fdot2(__builtin_amdgcn_perm(kF16Exp1024, w.x, kSelLo), xa.x, 0.0f);
    float a1 = fdot2(__builtin_amdgcn_perm(kF16Exp1024, w.x, kSelHi), xa.y, 0.0f);
    a0 = fdot2(__builtin_amdgcn_perm(kF16Exp1024, w.y, kSelLo), xa.z, a0);
    a1 = fdot2(__builtin_amdgcn_perm(kF16Exp1024, w.y, kSelHi), xa.w, a1);
    a0 = fdot2(__builtin_amdgcn_perm(kF16Exp1024, w.z, kSelLo), xb.x, a0);
    a1 = fdot2(__builtin_amdgcn_perm(kF16Exp1024, w.z, kSelHi), xb.y, a1);
    a0 = fdot2(__builtin_amdgcn_perm(kF16Exp1024, w.w, kSelLo), xb.z, a0);
    a1 = fdot2(__builtin_amdgcn_perm(kF16Exp1024, w.w, kSelHi), xb.w, a1);
    return a0 + a1;
}

Q35_DEV uint32_t pack_f16x2(float lo, float hi) {
    _Float16 l = (_Float16)lo, h = (_Float16)hi;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

Q35_DEV float f16_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu)); }
Q35_DEV float f16_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// ---------------------------------------------------------------- segments

// Segment of row group g, with segment boundaries read at compile-time offsets.
template <int NSEG>
Q35_DEV int find_seg(const GemvArgs& a, uint32_t g) {
    int s = 0;
#pragma unroll
    for (int i = 1; i < NSEG; ++i)
        if (g >= a.seg[i].rg_begin) s = i;
    return s;
}

// Calls f(seg, integral_constant<I>) for the segment of row group g; every field
// access inside f uses a compile-time segment index.
template <int I>
struct SegIdx {
    static constexpr int value = I;
};

template <int NSEG, class F>
Q35_DEV void with_seg(const GemvArgs& a, uint32_t g, F&& f) {
    if constexpr (NSEG == 1) {
        f(a.seg[0], SegIdx<0>{});
    } else {
        const int si = find_seg<NSEG>(a, g);
        if (si == 0) f(a.seg[0], SegIdx<0>{});
        if constexpr (NSEG > 1) if (si == 1) f(a.seg[1], SegIdx<1>{});
        if constexpr (NSEG > 2) if (si == 2) f(a.seg[2], SegIdx<2>{});
        if constexpr (NSEG > 3) if (si == 3) f(a.seg[3], SegIdx<3>{});
    }
}

// ---------------------------------------------------------------- prologue

// The prologue's global loads for one thread: x (and z) chunks and norm-weight
// chunks, raw, issued before the weights.
template <int K, int PRO>
struct ProRegs {
    static constexpr int MC = Geo<K, false>::MC;
    uint4 x[MC][4];  // 16 fp32 (4 uint4) or 16 bf16 (2 uint4)
    uint4 z[MC][4];  // gated norm: 16 fp32 of z
    uint4 w[MC][2];  // 16 bf16 norm weights
};

template <int K, int PRO, bool HALF>
Q35_DEV void prologue_issue(const GemvPro& p, ProRegs<K, PRO>& r) {
    constexpr int KC = K / 16, MC = Geo<K, false>::MC;
    constexpr bool X_BF16 = (PRO == kProRmsAct) && HALF;  // the residual stream is bf16 for HALF
    const int t = threadIdx.x;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int cc = t + kNT * m;
        if (cc < KC) {
            if constexpr (X_BF16) {
                const uint4* px = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x) + 16u * cc);
                r.x[m][0] = px[0];
                r.x[m][1] = px[1];
            } else {
                const uint4* px = reinterpret_cast<const uint4*>(static_cast<const float*>(p.x) + 16u * cc);
#pragma unroll
                for (int j = 0; j < 4; ++j) r.x[m][j] = px[j];
            }
            if constexpr (PRO == kProRmsAct || PRO == kProRmsF32) {
                const uint4* pw = reinterpret_cast<const uint4*>(p.w + 16u * cc);
                r.w[m][0] = pw[0];
                r.w[m][1] = pw[1];
            }
            if constexpr (PRO == kProGatedNorm) {
                const uint4* pz = reinterpret_cast<const uint4*>(p.z + 16u * cc);
#pragma unroll
                for (int j = 0; j < 4; ++j) r.z[m][j] = pz[j];
                const uint4* pw = reinterpret_cast<const uint4*>(p.w + (16u * cc) % p.head_dim);
                r.w[m][0] = pw[0];
                r.w[m][1] = pw[1];
            }
        }
    }
}

Q35_DEV void unpack_f32x16(const uint4 (&u)[4], float v[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[4 * j] = __uint_as_float(u[j].x);
        v[4 * j + 1] = __uint_as_float(u[j].y);
        v[4 * j + 2] = __uint_as_float(u[j].z);
        v[4 * j + 3] = __uint_as_float(u[j].w);
    }
}

Q35_DEV void unpack_bf16x16(const uint4* u, float v[16]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t d[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[8 * j + 2 * e] = bf16_lo(d[e]);
            v[8 * j + 2 * e + 1] = bf16_hi(d[e]);
        }
    }
}

// Stage a 16-element chunk of fp32 values in LDS slots {cc, KC+cc, 2KC+cc, 3KC+cc}.
template <int K>
Q35_DEV void stage_chunk(float4* xq, int cc, const float v[16]) {
    constexpr int KC = K / 16;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        xq[j * KC + cc] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
}

template <int K>
Q35_DEV void unstage_chunk(const float4* xq, int cc, float v[16]) {
    constexpr int KC = K / 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 t = xq[j * KC + cc];
        v[4 * j] = t.x;
        v[4 * j + 1] = t.y;
        v[4 * j + 2] = t.z;
        v[4 * j + 3] = t.w;
    }
}

// LDS image of x.  fp32: xq float4 [4][KC]; HALF: xq viewed as uint4 [2][KC] of f16
// pairs.  xs[KC]: per-chunk sums of the values actually multiplied.
template <int K, bool HALF>
Q35_DEV void write_chunk(float4* xq, float* xs, int cc, const float v[16], float scale) {
    constexpr int KC = K / 16;
    if constexpr (HALF) {
        uint4* xh = reinterpret_cast<uint4*>(xq);
        uint32_t p[8];
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = pack_f16x2(v[2 * j] * scale, v[2 * j + 1] * scale);
            s += f16_lo(p[j]) + f16_hi(p[j]);
        }
        xh[cc] = make_uint4(p[0], p[1], p[2], p[3]);
        xh[KC + cc] = make_uint4(p[4], p[5], p[6], p[7]);
        xs[cc] = s;
    } else {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) s += v[j];
        stage_chunk<K>(xq, cc, v);
        xs[cc] = s;
    }
}

// Power of two s with max|x| * s in [2^13, 2^14): f16 keeps 11 significant bits
// for the large entries and nothing can overflow.  1 for an all-zero vector.
Q35_DEV float half_scale(float amax) {
    if (!(amax > 0.0f) || !isfinite(amax)) return 1.0f;
    int e;
    frexpf(amax, &e);  // amax in [2^(e-1), 2^e)
    return ldexpf(1.0f, 14 - e);
}

// Builds x in LDS from the registers prologue_issue filled; returns the factor
// x was multiplied by (HALF only).  Pass 1 forms the values chunk by chunk and
// stages them in LDS as fp32 (gathering the block-wide statistics it needs);
// pass 2 turns each thread's own staged chunk into the final image in place:
// the image of chunk cc only covers LDS slots of chunk cc.
template <int K, int PRO, bool HALF>
Q35_DEV float prologue_finish(const GemvPro& p, const ProRegs<K, PRO>& r, float4* xq, float* xs,
                              float* red) {
    constexpr int KC = K / 16, MC = Geo<K, false>::MC;
    constexpr bool X_BF16 = (PRO == kProRmsAct) && HALF;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const bool tap = (p.tap != nullptr) && blockIdx.x == 0;
    float amax = 0.f, ss = 0.f;

#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int cc = t + kNT * m;
        float v[16];
        for (int j = 0; j < 16; ++j) v[j] = 0.f;
        if (cc < KC) {
            if constexpr (X_BF16) {
                unpack_bf16x16(r.x[m], v);
            } else {
                unpack_f32x16(r.x[m], v);
            }
        }
        if constexpr (PRO == kProRmsAct || PRO == kProRmsF32) {
            // x * w staged; sum of squares of x and max |x * w| reduced together
            if (cc < KC) {
                float wv[16];
                unpack_bf16x16(r.w[m], wv);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    ss = fmaf(v[j], v[j], ss);
                    v[j] *= wv[j];
                    amax = fmaxf(amax, fabsf(v[j]));
                }
                stage_chunk<K>(xq, cc, v);
            }
        } else if constexpr (PRO == kProGatedNorm) {
            // RMSNorm over each head of p.head_dim, times the norm weight, times silu(z)
            const int per_head = (int)p.head_dim / 16;  // chunks per head: 2, 4 or 8
            float hs = 0.f;
            if (cc < KC) {
#pragma unroll
                for (int j = 0; j < 16; ++j) hs = fmaf(v[j], v[j], hs);
            }
            for (int o = 1; o < per_head; o <<= 1) hs += __shfl_xor(hs, o);
            if (cc < KC) {
                const float rs = 1.0f / sqrtf(hs / (float)p.head_dim + p.eps);
                float wv[16], zv[16];
                unpack_bf16x16(r.w[m], wv);
                unpack_f32x16(r.z[m], zv);
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = v[j] * rs * wv[j];
                if (tap) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) p.tap[16 * cc + j] = v[j];
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    v[j] *= siluf_(zv[j]);
                    amax = fmaxf(amax, fabsf(v[j]));
                }
                stage_chunk<K>(xq, cc, v);
            }
        } else {  // kProLoadF32
            if (cc < KC) {
#pragma unroll
                for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
                stage_chunk<K>(xq, cc, v);
            }
        }
    }

    float post = 1.0f;
    constexpr bool RMS = (PRO == kProRmsAct || PRO == kProRmsF32);
    if constexpr (RMS || HALF) {
        // one block reduction: sum of squares (RMS) and max magnitude (HALF scaling)
        const float s_w = RMS ? wave_sum(ss) : 0.f;
        const float m_w = HALF ? wave_max(amax) : 0.f;
        if (lane == 0) {
            red[wid] = s_w;
            red[4 + wid] = m_w;
        }
        __syncthreads();
        float ss_t = 0.f, am_t = 0.f;
#pragma unroll
        for (int i = 0; i < kNT / 64; ++i) {
            ss_t += red[i];
            am_t = fmaxf(am_t, red[4 + i]);
        }
        if constexpr (RMS) post = 1.0f / sqrtf(ss_t / (float)K + p.eps);
        amax = am_t * post;
    }
    float scale = 1.0f;
    if constexpr (HALF) scale = half_scale(amax);
    if constexpr (!RMS && !HALF) return scale;  // the staged fp32 chunks are already the image

#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int cc = t + kNT * m;
        if (cc < KC) {
            float v[16];
            unstage_chunk<K>(xq, cc, v);
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] *= post;
            if (RMS && tap) {
#pragma unroll
                for (int j = 0; j < 16; ++j) p.tap[16 * cc + j] = v[j];
            }
            write_chunk<K, HALF>(xq, xs, cc, v, scale);
        }
    }
    return scale;
}

// The !RMS && !HALF path stages fp32 values without chunk sums; fill them.
template <int K>
Q35_DEV void chunk_sums_f32(const float4* xq, float* xs) {
    constexpr int KC = K / 16;
    for (int cc = threadIdx.x; cc < KC; cc += kNT) {
        float v[16];
        unstage_chunk<K>(xq, cc, v);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) s += v[j];
        xs[cc] = s;
    }
}

// ---------------------------------------------------------------- epilogues

template <int OP, int SI>
Q35_DEV void epilogue(const GemvArgs& a, const GemvSeg& s, uint32_t n, float v, float v2,
                      float& best_v, int& best_i) {
    if constexpr (OP == kOpPlain || OP == kOpInFull || (OP == kOpInGdn && SI == 1)) {
        s.out[n] = v;
    } else if constexpr (OP == kOpInGdn && SI == 0) {
        // causal depthwise conv update of channel n (window: state[1..3] + new input), SiLU
        if (s.tap0) s.tap0[n] = v;
        float4* st = reinterpret_cast<float4*>(s.state) + n;
        const float4 o = *st;
        const uint2 w = reinterpret_cast<const uint2*>(s.aux0)[n];
        float u = bf16_lo(w.x) * o.y;
        u = fmaf(bf16_hi(w.x), o.z, u);
        u = fmaf(bf16_lo(w.y), o.w, u);
        u = fmaf(bf16_hi(w.y), v, u);
        *st = make_float4(o.y, o.z, o.w, v);
        s.out[n] = siluf_(u);
    } else if constexpr (OP == kOpInGdn && SI == 2) {
        // decay gate exp(-exp(A_log) * softplus(a + dt_bias))
        if (s.tap0) s.tap0[n] = v;
        const float dtb = bf16_to_f32(static_cast<const uint16_t*>(s.aux0)[n]);
        const float al = static_cast<const float*>(s.aux1)[n];
        s.out[n] = expf(-expf(al) * softplusf_(v + dtb));
    } else if constexpr (OP == kOpInGdn && SI == 3) {
        if (s.tap0) s.tap0[n] = v;
        s.out[n] = sigmoidf_(v);
    } else if constexpr (OP == kOpOutGated || OP == kOpOProj) {
        // residual from the layer input (activation dtype)
        if (s.tap0) s.tap0[n] = v;
        s.out[n] = load_act(s.aux0, n, a.act_f32) + v;
    } else if constexpr (OP == kOpGateUp) {
        if (s.tap0) s.tap0[n] = v;
        if (s.tap1) s.tap1[n] = v2;
        s.out[n] = siluf_(v) * v2;
    } else if constexpr (OP == kOpDown) {
        const float r = static_cast<const float*>(s.aux0)[n] + v;
        store_act(s.out_act, n, r, a.act_f32);
        if (s.out_act2) store_act(s.out_act2, n, r, a.act_f32);
    } else if constexpr (OP == kOpLmHead) {
        if (s.out) s.out[n] = v;
        if (v > best_v || (v == best_v && (int)n < best_i)) {
            best_v = v;
            best_i = (int)n;
        }
    }
}

// ---------------------------------------------------------------- argmax partials

Q35_DEV bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Per-block partial argmax (lowest index on ties), stored plainly; a follow-up
// kernel reduces the partials, so no block needs a device-wide fence.
Q35_DEV void argmax_partial(const GemvArgs& a, float best_v, int best_i, float* red) {
    int* redi = reinterpret_cast<int*>(red + 8);
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best_v, o);
        const int oi = __shfl_xor(best_i, o);
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
    }
}

// ---------------------------------------------------------------- the kernel

template <int K, int OP, bool HALF, bool XREG>
__global__ __launch_bounds__(kNT) void gemv_kernel(GemvArgs a) {
    using T = Op<OP>;
    constexpr bool PAIRED = T::PAIRED;
    using G = Geo<K, PAIRED>;
    constexpr int KC = G::KC, LR = G::LR, R = G::R, NC = G::NC;
    constexpr int KG = K / 64;  // scale groups per row

    extern __shared__ float4 smem4[];
    float4* xq = smem4;
    float* xs = reinterpret_cast<float*>(smem4 + 4 * KC);
    float* red = xs + KC;
    const uint4* xh = reinterpret_cast<const uint4*>(smem4);

    const int lane = threadIdx.x & 63;
    const int slot = lane / LR, li = lane % LR;
    const int m = PAIRED ? (slot & 1) : 0;  // paired: odd slots are up rows
    const uint32_t rloc = PAIRED ? (uint32_t)(slot >> 1) : (uint32_t)slot;
    const uint32_t nw = gridDim.x * (kNT / 64);
    const uint32_t total = a.total_rg;

    u32x4_t w[NC];
    uint32_t sv[NC], bv[NC];
    auto load_rg = [&](uint32_t g) {
        with_seg<T::NSEG>(a, g, [&](const GemvSeg& s, auto) {
            const uint32_t row0 = (g - s.rg_begin) * R;
            const uint32_t cbytes = s.rows * (uint32_t)K, sbytes = s.rows * (uint32_t)KG * 2u;
            const uint32_t coff = row0 * (uint32_t)K, soff = row0 * (uint32_t)KG * 2u;
            auto issue = [&](const void* c, const void* sc, const void* bi) {
                const auto rc = rsrc(c, cbytes), rs = rsrc(sc, sbytes), rb = rsrc(bi, sbytes);
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    const uint32_t cc = (uint32_t)li + LR * i;
                    w[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, rloc * K + 16u * cc, coff, kAuxStream);
                    sv[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, (rloc * KG + (cc >> 2)) * 2u, soff, 0);
                    bv[i] = __builtin_amdgcn_raw_buffer_load_b16(rb, (rloc * KG + (cc >> 2)) * 2u, soff, 0);
                }
            };
            if (!PAIRED || m == 0)
                issue(s.codes[0], s.scales[0], s.biases[0]);
            else
                issue(s.codes[1], s.scales[1], s.biases[1]);
        });
    };

    // x loads first, then the first row group's weights (vector loads complete in order)
    ProRegs<K, T::PRO> pr;
    prologue_issue<K, T::PRO, HALF>(a.pro, pr);
    asm volatile("" ::: "memory");
    uint32_t rg = blockIdx.x * (kNT / 64) + (threadIdx.x >> 6);
    if (rg < total) load_rg(rg);
    asm volatile("" ::: "memory");

    const float scale = prologue_finish<K, T::PRO, HALF>(a.pro, pr, xq, xs, red);
    if constexpr (T::PRO != kProRmsAct && T::PRO != kProRmsF32 && !HALF) {
        __syncthreads();
        chunk_sums_f32<K>(xq, xs);   // fp32 x was staged as-is: add its chunk sums
    }
    const float inv_scale = 1.0f / scale;
    __syncthreads();

    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;

    while (rg < total) {
        // Short streams keep x in LDS (an opaque zero offset stops the compiler
        // from hoisting every chunk of x into registers, which costs occupancy);
        // long streams (XREG) keep the hoisted copy in registers.
        int xo = 0;
        if constexpr (!XREG) asm volatile("" : "+v"(xo));
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int cc = li + LR * i + xo;
            const float xsum = xs[cc];
            const float sc = bf16_to_f32(sv[i]), bi = bf16_to_f32(bv[i]);
            const uint4 wi = make_uint4(w[i].x, w[i].y, w[i].z, w[i].w);
            float p;
            if constexpr (HALF) {
                p = fmaf(sc, dot16h(wi, xh[cc], xh[KC + cc]), fmaf(-1024.0f, sc, bi) * xsum);
            } else {
                p = fmaf(sc, dot16(wi, xq[cc], xq[KC + cc], xq[2 * KC + cc], xq[3 * KC + cc]), bi * xsum);
            }
            acc += p;
        }
        // row sums land in the last lane of each group of LR lanes
        const float v = group_sum_last<LR>(acc) * inv_scale;
        with_seg<T::NSEG>(a, rg, [&](const GemvSeg& s, auto si) {
            constexpr int SI = decltype(si)::value;
            const uint32_t n = (rg - s.rg_begin) * R + rloc;
            if constexpr (PAIRED) {
                const float gate = __shfl_up(v, LR, 64);  // the gate row sum sits LR lanes below
                if (li == LR - 1 && m == 1) epilogue<OP, SI>(a, s, n, gate, v, best_v, best_i);
            } else {
                if (li == LR - 1) epilogue<OP, SI>(a, s, n, v, 0.f, best_v, best_i);
            }
        });
        rg += nw;
        if (rg < total) load_rg(rg);
    }

    if constexpr (OP == kOpLmHead) argmax_partial(a, best_v, best_i, red);
}

template <int K, int OP, bool HALF, bool XREG>
hipError_t launch_t(const GemvArgs& a, uint32_t blocks, hipStream_t stream) {
    constexpr int KC = K / 16;
    const size_t lds = (size_t)KC * (4 * sizeof(float4) + sizeof(float)) + 16 * sizeof(float);
    hipLaunchKernelGGL((gemv_kernel<K, OP, HALF, XREG>), dim3(blocks), dim3(kNT), lds, stream, a);
    return hipGetLastError();
}

template <int K, int OP, bool HALF, bool XREG>
const void* kernel_ptr_t() {
    return (const void*)&gemv_kernel<K, OP, HALF, XREG>;
}

}  // namespace gemv
}  // namespace q35
