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
// row.  For the paired gate+up segment a wave loads the row group of each
// matrix (same rows, same lanes) and forms both dot products from one read of
// x, so the SwiGLU product is formed in the epilogue of the lane holding both
// sums.  Loads go through buffer resources: one SGPR descriptor per matrix
// (wave-uniform, so no load needs a per-lane descriptor loop), a lane-constant
// 32-bit offset, and the row group's offset as the scalar offset, so a load is
// one instruction with no per-load address arithmetic; code loads are marked
// non-temporal (streamed once).
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
//  * HALF: x is held as f16 after a power-of-two scaling of each 16-element
//    chunk (11 significant bits: finer than the bf16 the activations are
//    stored in, and the scaling keeps it clear of f16 overflow).  One
//    v_perm_b32 turns two code bytes into the exact f16 pair (1024 + q0,
//    1024 + q1) and one v_dot2_f32_f16 multiplies it into an fp32 sum, so
//    sum (1024+q) x = sum q x + 1024 sum x; the 1024 sum x term is folded into
//    the bias: chunk term = s * dot' + (b - 1024 s) * sum x.  Products of f16
//    inputs are exact in fp32 and accumulation is fp32, so the only extra
//    rounding is that of x.
// x (with per-chunk factors and sums, needed by the bias term) lives in LDS,
// laid out so that the lanes of a wave read consecutive 16-byte words.  Every
// block builds it in one pass with a single barrier: the RMS factor of the
// norm prologues multiplies each row's dot product instead of x, so no step
// waits for a block-wide reduction before the image is written.
#pragma once

#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace gemv {

constexpr int kRedSlots = 64;  // LDS floats for block reductions (two per wave, 16 waves max)

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- operations

template <int OP>
struct Op;
// PRO: the prologue; NSEG: segments; EPI: the operation whose epilogues the
// segments run, segment SI running that operation's segment esi(SI).
template <int EPI_, int PRO_, int NSEG_, bool PAIRED_ = false>
struct OpT {
    static constexpr bool PAIRED = PAIRED_;
    static constexpr int PRO = PRO_, NSEG = NSEG_, EPI = EPI_;
    static constexpr int esi(int si) { return si; }
};
template <> struct Op<kOpPlain> : OpT<kOpPlain, kProLoadF32, 1> {};
template <> struct Op<kOpInGdn> : OpT<kOpInGdn, kProRmsAct, 4> {};  // qkv (conv), z, a (gate), b (beta)
template <> struct Op<kOpInFull> : OpT<kOpInFull, kProRmsAct, 3> {};  // q, k, v
template <> struct Op<kOpOutGated> : OpT<kOpOutGated, kProGatedNorm, 1> {};
template <> struct Op<kOpOProj> : OpT<kOpOProj, kProLoadF32, 1> {};
template <> struct Op<kOpGateUp> : OpT<kOpGateUp, kProRmsF32, 1, true> {};
template <> struct Op<kOpDown> : OpT<kOpDown, kProLoadF32, 1> {};
template <> struct Op<kOpLmHead> : OpT<kOpLmHead, kProRmsAct, 1> {};
template <> struct Op<kOpInFullP> : OpT<kOpInFull, kProRmsParts, 3> {};
template <> struct Op<kOpInGdnX> : OpT<kOpInGdn, kProRmsParts, 6> {  // q, k, v (conv), z, a, b
    static constexpr int esi(int si) { return si < 3 ? 0 : si - 2; }
};
template <> struct Op<kOpGateUpX> : OpT<kOpGateUp, kProRmsParts, 1, true> {};
template <> struct Op<kOpOutPart> : OpT<kOpPlain, kProGatedNorm, 1> {};
template <> struct Op<kOpDownPart> : OpT<kOpPlain, kProLoadF32, 1> {};

template <int K, bool PAIRED>
struct Geo {
    static constexpr int KC = K / 16;                                  // 16-byte chunks per row
    static constexpr int LR = gcd_c(64, KC);                           // lanes per row
    static constexpr int SLOTS = 64 / LR;                              // rows per row group
    static constexpr int R = SLOTS;                                    // rows of each matrix per row group
    static constexpr int NC = KC / LR;                                 // chunks per lane
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
        if constexpr (NSEG > 4) if (si == 4) f(a.seg[4], SegIdx<4>{});
        if constexpr (NSEG > 5) if (si == 5) f(a.seg[5], SegIdx<5>{});
    }
}

// A field of the segment with (wave-uniform) index si, picked with scalar
// selects rather than branches.
template <int NSEG, class F>
Q35_DEV auto pick(int si, F&& f) {
    auto v = f(0);
#pragma unroll
    for (int i = 1; i < NSEG; ++i)
        if (si == i) v = f(i);
    return v;
}

// ---------------------------------------------------------------- prologue

// The prologue's global loads for one thread: x (and z) chunks and norm-weight
// chunks, raw, issued before the weights.
template <int K, int NT>
constexpr int pro_chunks() { return (K / 16 + NT - 1) / NT; }  // prologue chunks per thread

template <int K, int PRO, int NT>
struct ProRegs {
    static constexpr int MC = pro_chunks<K, NT>();
    uint4 x[MC][4];  // 16 fp32 (4 uint4) or 16 bf16 (2 uint4)
    uint4 z[MC][4];  // gated norm: 16 fp32 of z
    uint4 w[MC][2];  // 16 bf16 norm weights
};

// COH: x (and z) were written by other blocks of the same launch and are read
// with cache policy XAUX (device-coherent, or L2 for blocks of one XCD).
template <int K, int PRO, bool HALF, int NT, bool COH = false, int XAUX = kAuxCoherent>
Q35_DEV void prologue_issue(const GemvPro& p, ProRegs<K, PRO, NT>& r) {
    constexpr int KC = K / 16, MC = pro_chunks<K, NT>();
    constexpr bool X_BF16 = (PRO == kProRmsAct) && HALF;  // the residual stream is bf16 for HALF
    const int t = tid_x();
    if constexpr (COH) {
        // x (and z) were written by other blocks of the same launch: device-coherent
        // buffer loads over a wave-uniform resource, per-lane offsets
        const auto rx = rsrc(p.x, K * (X_BF16 ? 2u : 4u));
        const auto rz = rsrc(p.z, PRO == kProGatedNorm ? K * 4u : 0u);
        const auto rw = rsrc(p.w, (PRO == kProGatedNorm ? p.head_dim : K) * 2u);
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int cc = t + NT * m;
            if (cc < KC) {
                if constexpr (X_BF16) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        r.x[m][j] = ld_b128<XAUX>(rx, 32u * cc + 16u * j);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        r.x[m][j] = ld_b128<XAUX>(rx, 64u * cc + 16u * j);
                }
                if constexpr (PRO == kProRmsAct || PRO == kProRmsF32) {
                    r.w[m][0] = ld_b128<0>(rw, 32u * cc);
                    r.w[m][1] = ld_b128<0>(rw, 32u * cc + 16u);
                }
                if constexpr (PRO == kProGatedNorm) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        r.z[m][j] = ld_b128<XAUX>(rz, 64u * cc + 16u * j);
                    const uint32_t wo = ((16u * cc) % p.head_dim) * 2u;
                    r.w[m][0] = ld_b128<0>(rw, wo);
                    r.w[m][1] = ld_b128<0>(rw, wo + 16u);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int cc = t + NT * m;
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

// Power of two s with max|x| * s in [2^13, 2^14): f16 keeps 11 significant bits
// for the large entries and nothing can overflow.  Built from the exponent
// field: amax in [2^(E-127), 2^(E-126)) gives s = 2^(140-E); E is clamped so s
// stays a normal float (a chunk below 2^-114 keeps its tiny values as they
// are), and zero, inf and NaN chunks get s = 1.
Q35_DEV float half_scale(float amax) {
    const uint32_t E = (__float_as_uint(amax) >> 23) & 0xFFu;
    if (E == 0u || E == 0xFFu) return 1.0f;
    const uint32_t Ec = E < 13u ? 13u : E;
    return __uint_as_float((267u - Ec) << 23);
}

// silu(z) with the hardware exp and reciprocal (about 1 ulp each): cheap
// enough for a prologue that every block runs over all of x.
Q35_DEV float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

constexpr uint32_t kF16OnePair = 0x3C003C00u;  // (1.0, 1.0) in f16

// LDS image of x, built once per block in one pass.
//   HALF: xh  uint4 [2][KC]  f16 pairs of x_k * s_c, s_c a power of two per 16-element
//                            chunk (so no block-wide maximum is needed);
//         xab float2 [KC]    A_c = f_c / s_c and B_c = A_c * (sum of the chunk's f16 values),
//                            so a row's chunk term is sc * A_c * dot' + (b - 1024 sc) * B_c.
//   fp32: xq  float4 [4][KC] x_k * f_c;  xab[cc].y = the chunk sum.
// f_c is the per-head RMS factor of the gated norm (constant over a chunk), else
// 1.  The RMS prologues leave the global 1/rms factor out of x: it multiplies
// every row's dot product instead, so x does not wait for that reduction.
template <int K, bool HALF>
Q35_DEV void write_chunk(uint4* ximg, float2* xab, int cc, const float v[16], float f) {
    constexpr int KC = K / 16;
    if constexpr (HALF) {
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
        const float sc = half_scale(amax);
        uint32_t p[8];
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = pack_f16x2(v[2 * j] * sc, v[2 * j + 1] * sc);
            sum = fdot2(p[j], kF16OnePair, sum);  // sum of the f16 values as multiplied
        }
        ximg[cc] = make_uint4(p[0], p[1], p[2], p[3]);
        ximg[KC + cc] = make_uint4(p[4], p[5], p[6], p[7]);
        const float A = f / sc;
        xab[cc] = make_float2(A, A * sum);
    } else {
        float4* xq = reinterpret_cast<float4*>(ximg);
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 q = make_float4(v[4 * j] * f, v[4 * j + 1] * f, v[4 * j + 2] * f, v[4 * j + 3] * f);
            sum += (q.x + q.y) + (q.z + q.w);
            xq[j * KC + cc] = q;
        }
        xab[cc] = make_float2(f, sum);
    }
}

// The value of x_k * f_c (times `post`) as held in the image (for the RMS tap).
template <int K, bool HALF>
Q35_DEV void read_chunk(const uint4* ximg, const float2* xab, int cc, float v[16]) {
    constexpr int KC = K / 16;
    if constexpr (HALF) {
        const uint4 lo = ximg[cc], hi = ximg[KC + cc];
        const float A = xab[cc].x;
        const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[2 * j] = f16_lo(d[j]) * A;
            v[2 * j + 1] = f16_hi(d[j]) * A;
        }
    } else {
        const float4* xq = reinterpret_cast<const float4*>(ximg);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 q = xq[j * KC + cc];
            v[4 * j] = q.x;
            v[4 * j + 1] = q.y;
            v[4 * j + 2] = q.z;
            v[4 * j + 3] = q.w;
        }
    }
}

// Builds the image from the registers prologue_issue filled; returns the factor
// every row's dot product is multiplied by (1/rms for the RMS prologues, else 1).
template <int K, int PRO, bool HALF, int NT>
Q35_DEV float prologue_build(const GemvPro& p, const ProRegs<K, PRO, NT>& r, uint4* ximg,
                             float2* xab, float* red, bool lead) {
    constexpr int KC = K / 16, MC = pro_chunks<K, NT>(), NW = NT / 64;
    constexpr bool X_BF16 = (PRO == kProRmsAct) && HALF;
    constexpr bool RMS = (PRO == kProRmsAct || PRO == kProRmsF32);
    const int t = tid_x(), lane = t & 63, wid = t >> 6;
    const bool tap = (p.tap != nullptr) && lead;
    float ss = 0.f;

#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int cc = t + NT * m;
        float v[16];
        for (int j = 0; j < 16; ++j) v[j] = 0.f;
        if (cc < KC) {
            if constexpr (X_BF16) {
                unpack_bf16x16(r.x[m], v);
            } else {
                unpack_f32x16(r.x[m], v);
            }
        }
        float f = 1.0f;
        if constexpr (RMS) {
            if (cc < KC) {
                float wv[16];
                unpack_bf16x16(r.w[m], wv);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    ss = fmaf(v[j], v[j], ss);
                    v[j] *= wv[j];
                }
            }
        } else if constexpr (PRO == kProGatedNorm) {
            // RMSNorm over each head of p.head_dim (2, 4 or 8 chunks held by
            // consecutive threads), times the norm weight, times silu(z)
            const int per_head = (int)p.head_dim / 16;
            float hs = 0.f;
            if (cc < KC) {
#pragma unroll
                for (int j = 0; j < 16; ++j) hs = fmaf(v[j], v[j], hs);
            }
            for (int o = 1; o < per_head; o <<= 1) hs += __shfl_xor(hs, o);
            f = 1.0f / sqrtf(hs / (float)p.head_dim + p.eps);
            if (cc < KC) {
                float wv[16], zv[16];
                unpack_bf16x16(r.w[m], wv);
                unpack_f32x16(r.z[m], zv);
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] *= wv[j];
                if (tap) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) p.tap[16 * cc + j] = v[j] * f;
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] *= silu_fast(zv[j]);
            }
        }
        if (cc < KC) write_chunk<K, HALF>(ximg, xab, cc, v, f);
    }

    float post = 1.0f;
    if constexpr (RMS) {
        const float s_w = wave_sum(ss);
        if (lane == 0) red[wid] = s_w;
    }
    __syncthreads();
    if constexpr (RMS) {
        float ss_t = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) ss_t += red[i];
        post = 1.0f / sqrtf(ss_t / (float)K + p.eps);
        if (tap) {
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const int cc = t + NT * m;
                if (cc < KC) {
                    float v[16];
                    read_chunk<K, HALF>(ximg, xab, cc, v);
#pragma unroll
                    for (int j = 0; j < 16; ++j) p.tap[16 * cc + j] = v[j] * post;
                }
            }
        }
    }
    return post;
}

// ---------------------------------------------------------------- sum-of-partials prologue

// kProRmsParts.  The residual stream arrives as a base vector plus up to eight
// fp32 partial vectors (one per XCD of a column-split GEMV); x is their sum,
// added in a fixed order (base, then partial 0, 1, ...), so every block forms
// the same values.  Thread t owns quads (4 elements) t, t + NT, ...; the first
// round of quads is loaded with the other early loads and later rounds (K/4 >
// NT) where they are summed.  Out-of-range offsets (quads past the end,
// partials past nparts) read zero through the buffer ranges, so the loads are
// branch-free.  The sum goes to an fp32 staging area in LDS, then the image is
// built from it as in the RMS prologues; block 0 writes the sum out.
constexpr int kMaxParts = 8;

template <int K, int NT>
struct PartsRegs {
    static constexpr int NQ = K / 4, MQ = (NQ + NT - 1) / NT, MC = pro_chunks<K, NT>();
    uint4 b;              // base quad: 4 fp32, or 4 bf16 in .x/.y
    uint4 p[kMaxParts];   // the partials' quads
    uint4 w[MC][2];       // 16 bf16 norm weights per chunk
};

template <int K>
Q35_DEV void parts_load(const GemvPro& p, int q, uint4& b, uint4 (&pp)[kMaxParts]) {
    constexpr uint32_t NQ = K / 4, kPast = 0xFFFFFFF0u;
    const bool live = (uint32_t)q < NQ;
    if (p.x_f32) {
        b = ld_b128<0>(rsrc(p.x, K * 4u), live ? 16u * q : kPast);
    } else {
        const uint2 h = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                      rsrc(p.x, K * 2u), live ? 8u * q : kPast, 0, 0));
        b = make_uint4(h.x, h.y, 0u, 0u);
    }
    const auto rp = rsrc(p.parts, p.parts ? p.nparts * K * 4u : 0u);
#pragma unroll
    for (int i = 0; i < kMaxParts; ++i) pp[i] = ld_b128<0>(rp, live ? (i * K + 4u * q) * 4u : kPast);
}

template <int K, int NT>
Q35_DEV void parts_issue(const GemvPro& p, PartsRegs<K, NT>& r) {
    constexpr int KC = K / 16;
    const int t = tid_x();
    parts_load<K>(p, t, r.b, r.p);
    const auto rw = rsrc(p.w, K * 2u);
#pragma unroll
    for (int m = 0; m < PartsRegs<K, NT>::MC; ++m) {
        const int cc = t + NT * m;
        const uint32_t off = cc < KC ? 32u * cc : 0xFFFFFFF0u;
        r.w[m][0] = ld_b128<0>(rw, off);
        r.w[m][1] = ld_b128<0>(rw, off + 16u);
    }
}

template <int K, bool HALF, int NT>
Q35_DEV float parts_build(const GemvPro& p, const PartsRegs<K, NT>& r, uint4* ximg, float2* xab,
                          float* red, float* xs, bool lead) {
    using PR = PartsRegs<K, NT>;
    constexpr int KC = K / 16, NW = NT / 64;
    const int t = tid_x(), lane = t & 63, wid = t >> 6;
#pragma unroll
    for (int m = 0; m < PR::MQ; ++m) {
        const int q = t + NT * m;
        uint4 b = r.b;
        uint4 pp[kMaxParts];
#pragma unroll
        for (int i = 0; i < kMaxParts; ++i) pp[i] = r.p[i];
        if (m > 0) parts_load<K>(p, q, b, pp);
        if (q < PR::NQ) {
            float v[4];
            if (p.x_f32) {
                v[0] = __uint_as_float(b.x);
                v[1] = __uint_as_float(b.y);
                v[2] = __uint_as_float(b.z);
                v[3] = __uint_as_float(b.w);
            } else {
                v[0] = bf16_lo(b.x);
                v[1] = bf16_hi(b.x);
                v[2] = bf16_lo(b.y);
                v[3] = bf16_hi(b.y);
            }
#pragma unroll
            for (int i = 0; i < kMaxParts; ++i) {
                v[0] += __uint_as_float(pp[i].x);
                v[1] += __uint_as_float(pp[i].y);
                v[2] += __uint_as_float(pp[i].z);
                v[3] += __uint_as_float(pp[i].w);
            }
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[j] = f32_to_bf16(v[j]);
                if (p.sum_bf16) v[j] = bf16_to_f32(h[j]);
            }
            reinterpret_cast<float4*>(xs)[q] = make_float4(v[0], v[1], v[2], v[3]);
            if (p.sum_out && blockIdx.x == 0) {
                if (p.sum_bf16)
                    reinterpret_cast<uint2*>(p.sum_out)[q] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                else
                    reinterpret_cast<float4*>(p.sum_out)[q] = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
    __syncthreads();
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < PR::MC; ++m) {
        const int cc = t + NT * m;
        if (cc < KC) {
            float v[16], wv[16];
            const float4* x4 = reinterpret_cast<const float4*>(xs) + 4 * cc;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 u = x4[j];
                v[4 * j] = u.x;
                v[4 * j + 1] = u.y;
                v[4 * j + 2] = u.z;
                v[4 * j + 3] = u.w;
            }
            unpack_bf16x16(r.w[m], wv);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                ss = fmaf(v[j], v[j], ss);
                v[j] *= wv[j];
            }
            write_chunk<K, HALF>(ximg, xab, cc, v, 1.0f);
        }
    }
    const float s_w = wave_sum(ss);
    if (lane == 0) red[wid] = s_w;
    __syncthreads();
    float ss_t = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) ss_t += red[i];
    const float post = 1.0f / sqrtf(ss_t / (float)K + p.eps);
    if (p.tap && lead) {
#pragma unroll
        for (int m = 0; m < PR::MC; ++m) {
            const int cc = t + NT * m;
            if (cc < KC) {
                float v[16];
                read_chunk<K, HALF>(ximg, xab, cc, v);
#pragma unroll
                for (int j = 0; j < 16; ++j) p.tap[16 * cc + j] = v[j] * post;
            }
        }
    }
    return post;
}

// ---------------------------------------------------------------- epilogues

// Operands an epilogue reads from memory (GemvSeg::pre16/8/4/2, element n),
// loaded with the row group's weights: a load issued in the epilogue would
// wait, in order, for the next row group's weight loads issued before it.
// Every segment of an operation issues the same loads (a NULL operand gets an
// empty buffer range and reads zero), so the compiler's count of outstanding
// loads is the same on every path and its waits stay exact.
struct EpiPre {
    uint4 q16;    // conv state of channel n (4 fp32)
    uint2 q8;     // conv weights of channel n (4 bf16)
    uint32_t q4;  // fp32: residual, A_log
    uint32_t q2;  // bf16: residual, dt_bias
};

template <int OP_, bool HALF>
constexpr int pre_mask() {  // which of the 16/8/4/2-byte operands the op's epilogues read
    constexpr int OP = Op<OP_>::EPI;
    return OP == kOpInGdn ? (16 | 8 | 4 | 2)
         : (OP == kOpOutGated || OP == kOpOProj) ? (HALF ? 2 : 4)
         : OP == kOpDown ? 4
         : 0;
}

template <int OP_, int SI_, bool COH>
Q35_DEV void epilogue(const GemvArgs& a, const GemvSeg& s, uint32_t n, float v, float v2,
                      const EpiPre& e, float& best_v, int& best_i) {
    constexpr int OP = Op<OP_>::EPI, SI = Op<OP_>::esi(SI_);
    if constexpr (OP == kOpPlain || OP == kOpInFull || (OP == kOpInGdn && SI == 1)) {
        st_f32<COH>(s.out, n, v);
    } else if constexpr (OP == kOpInGdn && SI == 0) {
        // causal depthwise conv update of channel n (window: state[1..3] + new input), SiLU
        if (s.tap0) s.tap0[n] = v;
        const float4 o = make_float4(__uint_as_float(e.q16.x), __uint_as_float(e.q16.y),
                                     __uint_as_float(e.q16.z), __uint_as_float(e.q16.w));
        const uint2 w = e.q8;
        float u = bf16_lo(w.x) * o.y;
        u = fmaf(bf16_hi(w.x), o.z, u);
        u = fmaf(bf16_lo(w.y), o.w, u);
        u = fmaf(bf16_hi(w.y), v, u);
        // the conv state row is read and written by this lane only
        reinterpret_cast<float4*>(s.state)[n] = make_float4(o.y, o.z, o.w, v);
        st_f32<COH>(s.out, n, siluf_(u));
    } else if constexpr (OP == kOpInGdn && SI == 2) {
        // decay gate exp(-exp(A_log) * softplus(a + dt_bias))
        if (s.tap0) s.tap0[n] = v;
        st_f32<COH>(s.out, n, expf(-expf(__uint_as_float(e.q4)) * softplusf_(v + bf16_to_f32(e.q2))));
    } else if constexpr (OP == kOpInGdn && SI == 3) {
        if (s.tap0) s.tap0[n] = v;
        st_f32<COH>(s.out, n, sigmoidf_(v));
    } else if constexpr (OP == kOpOutGated || OP == kOpOProj) {
        // residual from the layer input (activation dtype)
        if (s.tap0) s.tap0[n] = v;
        st_f32<COH>(s.out, n, (a.act_f32 ? __uint_as_float(e.q4) : bf16_to_f32(e.q2)) + v);
    } else if constexpr (OP == kOpGateUp) {
        if (s.tap0) s.tap0[n] = v;
        if (s.tap1) s.tap1[n] = v2;
        st_f32<COH>(s.out, n, siluf_(v) * v2);
    } else if constexpr (OP == kOpDown) {
        const float r = __uint_as_float(e.q4) + v;
        st_act_t<COH>(s.out_act, n, r, a.act_f32);
        if (s.out_act2) st_act_t<COH>(s.out_act2, n, r, a.act_f32);
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
template <int NT, bool COH>
Q35_DEV void argmax_partial(const GemvArgs& a, float best_v, int best_i, float* red) {
    int* redi = reinterpret_cast<int*>(red + kRedSlots / 2);
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best_v, o);
        const int oi = __shfl_xor(best_i, o);
        if (better(ov, oi, best_v, best_i)) {
            best_v = ov;
            best_i = oi;
        }
    }
    const int lane = tid_x() & 63, wid = tid_x() >> 6;
    __syncthreads();
    if (lane == 0) {
        red[wid] = best_v;
        redi[wid] = best_i;
    }
    __syncthreads();
    if (tid_x() == 0) {
        float bv = red[0];
        int bi = redi[0];
        for (int w = 1; w < NT / 64; ++w)
            if (better(red[w], redi[w], bv, bi)) {
                bv = red[w];
                bi = redi[w];
            }
        st_f32<COH>(a.am.part_val, blockIdx.x, bv);
        st_i32<COH>(a.am.part_idx, blockIdx.x, bi);
    }
}

// ---------------------------------------------------------------- the kernel

// The registers of one row group in flight: codes, scales and biases of each
// matrix, and the epilogue operands.
template <int NC, int NC2>
struct RgBuf {
    u32x4_t w[NC], w2[NC2];  // paired: w2 holds the second matrix's rows of the same index
    uint32_t sv[NC], bv[NC], sv2[NC2], bv2[NC2];
    EpiPre pre;
};

// The body shared by the standalone kernels, the stages of the persistent
// decode kernel and those of the XCD-split kernel.  rg: this wave's first row
// group; nw: the stride between its row groups; lead: this block writes the
// prologue's tap; smem4: the block's LDS.
// SYNC 0: standalone (or the first stage of a launch): x loads, then weights.
// SYNC 1 (persistent stages): x, the epilogue operands and the outputs are
// exchanged with other blocks of the launch through device-coherent loads and
// stores.  SYNC 2 (XCD stages): x was written by blocks of the same XCD with
// plain stores and is read with device-coherent loads.  With
// SYNC 1 or 2 the wave's first row group of weights is issued before wait()
// (which returns once the stage's inputs are published), and a wave with no
// row group issues no loads.
// KS: the row stride of the matrices in elements; K < KS reads a column slice
// (the segment pointers then point at the slice's first column).
template <int K, int OP, bool HALF, bool XREG, int NT, int SYNC, int KS = K, class Wait>
Q35_DEV void gemv_body(const GemvArgs& a, uint32_t rg, uint32_t nw, Wait&& wait, bool lead, uint4* smem4) {
    using T = Op<OP>;
    constexpr bool PAIRED = T::PAIRED;
    using G = Geo<K, PAIRED>;
    constexpr int KC = G::KC, LR = G::LR, R = G::R, NC = G::NC;
    constexpr int KGS = KS / 64;  // scale groups per row of the matrix
    constexpr bool COH = SYNC == 1;
    constexpr bool PARTS = T::PRO == kProRmsParts;
    static_assert(KS % 64 == 0 && KS >= K, "row stride");

    uint4* ximg = smem4;                                         // x image (f16: 2*KC, fp32: 4*KC)
    float2* xab = reinterpret_cast<float2*>(smem4 + (HALF ? 2 : 4) * KC);  // per-chunk (A, B)
    float* red = reinterpret_cast<float*>(xab + KC);
    float* xs = red + kRedSlots;                                 // kProRmsParts: fp32 sum [K]
    const float4* xq = reinterpret_cast<const float4*>(smem4);

    const int lane = tid_x() & 63;
    const int li = lane % LR;
    const uint32_t rloc = (uint32_t)(lane / LR);  // row of the row group
    const uint32_t total = a.total_rg;
    constexpr int PRE_AUX = COH ? kAuxCoherent : 0;

    constexpr int NC2 = PAIRED ? NC : 1;
    using Buf = RgBuf<NC, NC2>;
    static_assert(!PAIRED || T::NSEG == 1, "a paired launch has one segment");
    constexpr int PM = pre_mask<OP, HALF>();
    // Branch-free in the segment: the same loads are issued whatever the row
    // group.  A row group past the end (live == false) gets empty buffer
    // ranges: its loads return zero without touching memory, so they can be
    // issued unconditionally and the compiler's count of loads in flight stays
    // exact on every path.
    auto load_rg = [&](uint32_t g, bool live, Buf& b) {
        if (!live) g = total - 1;
        const int si = find_seg<T::NSEG>(a, g);
        const uint32_t rows = live ? pick<T::NSEG>(si, [&](int i) { return a.seg[i].rows; }) : 0u;
        const uint32_t row0 = (g - pick<T::NSEG>(si, [&](int i) { return a.seg[i].rg_begin; })) * R;
        const uint32_t n = row0 + rloc;
        // epilogue operands first: they have landed once the weights have
        auto pre_rsrc = [&](const void* p, uint32_t elt) { return rsrc(p, p ? rows * elt : 0u); };
        if constexpr (PM & 16)
            b.pre.q16 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                pre_rsrc(pick<T::NSEG>(si, [&](int i) { return a.seg[i].pre16; }), 16u), n * 16u, 0, PRE_AUX));
        if constexpr (PM & 8)
            b.pre.q8 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                pre_rsrc(pick<T::NSEG>(si, [&](int i) { return a.seg[i].pre8; }), 8u), n * 8u, 0, PRE_AUX));
        if constexpr (PM & 4)
            b.pre.q4 = __builtin_amdgcn_raw_buffer_load_b32(
                pre_rsrc(pick<T::NSEG>(si, [&](int i) { return a.seg[i].pre4; }), 4u), n * 4u, 0, PRE_AUX);
        if constexpr (PM & 2)
            b.pre.q2 = __builtin_amdgcn_raw_buffer_load_b16(
                pre_rsrc(pick<T::NSEG>(si, [&](int i) { return a.seg[i].pre2; }), 2u), n * 2u, 0, PRE_AUX);
        const uint32_t cbytes = rows * (uint32_t)KS, sbytes = rows * (uint32_t)KGS * 2u;
        const uint32_t coff = row0 * (uint32_t)KS, soff = row0 * (uint32_t)KGS * 2u;
        auto issue = [&](const void* c, const void* sc, const void* bi, u32x4_t* wd, uint32_t* sd,
                         uint32_t* bd) {
            const auto rc = rsrc(c, cbytes), rs = rsrc(sc, sbytes), rb = rsrc(bi, sbytes);
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const uint32_t cc = (uint32_t)li + LR * i;
                wd[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, rloc * KS + 16u * cc, coff, kAuxStream);
                sd[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, (rloc * KGS + (cc >> 2)) * 2u, soff, 0);
                bd[i] = __builtin_amdgcn_raw_buffer_load_b16(rb, (rloc * KGS + (cc >> 2)) * 2u, soff, 0);
            }
        };
        issue(pick<T::NSEG>(si, [&](int i) { return a.seg[i].codes[0]; }),
              pick<T::NSEG>(si, [&](int i) { return a.seg[i].scales[0]; }),
              pick<T::NSEG>(si, [&](int i) { return a.seg[i].biases[0]; }), b.w, b.sv, b.bv);
        if constexpr (PAIRED)
            issue(a.seg[0].codes[1], a.seg[0].scales[1], a.seg[0].biases[1], b.w2, b.sv2, b.bv2);
    };

    Buf b0;
    ProRegs<K, PARTS ? kProLoadF32 : T::PRO, NT> pr;
    PartsRegs<K, NT> prp;
    if constexpr (PARTS) {
        static_assert(SYNC == 0, "the partial sums come from an earlier launch");
        parts_issue<K, NT>(a.pro, prp);
        asm volatile("" ::: "memory");
        load_rg(rg, rg < total, b0);
    } else if constexpr (SYNC != 0) {
        // weights first (they do not depend on this launch), then the wait for
        // the stage's inputs, then x
        if (rg < total) load_rg(rg, true, b0);
        asm volatile("" ::: "memory");
        wait();
        prologue_issue<K, T::PRO, HALF, NT, true, kAuxCoherent>(a.pro, pr);
    } else {
        // x loads first, then the first row groups' weights (vector loads complete in order)
        prologue_issue<K, T::PRO, HALF, NT>(a.pro, pr);
        asm volatile("" ::: "memory");
        load_rg(rg, rg < total, b0);
    }
    asm volatile("" ::: "memory");

    float post;
    if constexpr (PARTS)
        post = parts_build<K, HALF, NT>(a.pro, prp, ximg, xab, red, xs, lead);
    else
        post = prologue_build<K, T::PRO, HALF, NT>(a.pro, pr, ximg, xab, red, lead);

    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;

    // One row group: dot products from buffer b, then (before this row group's
    // epilogue stores: on this ISA the vector memory counter also counts stores,
    // so a store issued first would make the next wait include its write
    // latency) the request for the wave's next row group into b.
    auto step = [&](Buf& b) {
        // Short streams keep x in LDS (an opaque zero offset stops the compiler
        // from hoisting every chunk of x into registers, which costs occupancy);
        // long streams (XREG) keep the hoisted copy in registers.
        int xo = 0;
        if constexpr (!XREG) asm volatile("" : "+v"(xo));
        float acc = 0.f, acc2 = 0.f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int cc = li + LR * i + xo;
            const float2 ab = xab[cc];
            auto term = [&](const u32x4_t& wv, uint32_t sb, uint32_t bb) {
                const float sc = bf16_to_f32(sb), bi = bf16_to_f32(bb);
                const uint4 wi = make_uint4(wv.x, wv.y, wv.z, wv.w);
                if constexpr (HALF)
                    return fmaf(sc * ab.x, dot16h(wi, ximg[cc], ximg[KC + cc]), fmaf(-1024.0f, sc, bi) * ab.y);
                else
                    return fmaf(sc, dot16(wi, xq[cc], xq[KC + cc], xq[2 * KC + cc], xq[3 * KC + cc]), bi * ab.y);
            };
            acc += term(b.w[i], b.sv[i], b.bv[i]);
            if constexpr (PAIRED) acc2 += term(b.w2[i % NC2], b.sv2[i % NC2], b.bv2[i % NC2]);
        }
        // row sums land in the last lane of each group of LR lanes
        const float v = group_sum_last<LR>(acc) * post;
        const float v2 = PAIRED ? group_sum_last<LR>(acc2) * post : 0.f;
        const uint32_t cur = rg;
        const EpiPre cpre = b.pre;
        rg += nw;
        if (rg < total) load_rg(rg, true, b);
        with_seg<T::NSEG>(a, cur, [&](const GemvSeg& s, auto si) {
            constexpr int SI = decltype(si)::value;
            const uint32_t n = (cur - s.rg_begin) * R + rloc;
            if (li == LR - 1) epilogue<OP, SI, COH>(a, s, n, v, v2, cpre, best_v, best_i);
        });
    };

    while (rg < total) step(b0);

    if constexpr (OP == kOpLmHead) argmax_partial<NT, COH>(a, best_v, best_i, red);
}

template <int K, int OP, bool HALF, bool XREG, int NT>
__global__ __launch_bounds__(NT) void gemv_kernel(GemvArgs a) {
    extern __shared__ uint4 smem4[];
    // wave-uniform by construction; readfirstlane lets the compiler keep the row
    // group (and so every buffer load's scalar offset) in SGPRs
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
    gemv_body<K, OP, HALF, XREG, NT, 0>(a, blockIdx.x * (NT / 64) + wave, gridDim.x * (NT / 64), [] {},
                                        blockIdx.x == 0, smem4);
}

// x image + per-chunk (A, B) + reduction slots (+ the fp32 sum of kProRmsParts)
template <int K, bool HALF, bool PARTS = false>
constexpr size_t lds_bytes() {
    return (size_t)(K / 16) * ((HALF ? 2 : 4) * 16 + 8) + kRedSlots * sizeof(float) + (PARTS ? K * 4 : 0);
}

template <int K, int OP, bool HALF, bool XREG>
hipError_t launch_t(const GemvArgs& a, uint32_t blocks, hipStream_t stream) {
    constexpr int NT = gemv_threads(OP);
    const size_t lds = lds_bytes<K, HALF, Op<OP>::PRO == kProRmsParts>();
    hipLaunchKernelGGL((gemv_kernel<K, OP, HALF, XREG, NT>), dim3(blocks), dim3(NT), lds, stream, a);
    return hipGetLastError();
}

template <int K, int OP, bool HALF, bool XREG>
const void* kernel_ptr_t() {
    return (const void*)&gemv_kernel<K, OP, HALF, XREG, gemv_threads(OP)>;
}

}  // namespace gemv
}  // namespace q35
