// Gated GQA decode attention over a bf16 KV cache (gfx950), one token.
//
// Covers the middle of the pages' full-attention forward (full_attention.rs
// page: the q/gate split, the per-head q/k RMSNorm, partial RoPE, the KV
// append, `attention_decode`, then the `sigmoid_gate` launch):
//     q_h  = RoPE(RMSNorm(q_full[h, :D]; q_norm))        h in kv group g
//     k    = RoPE(RMSNorm(k_g; k_norm)),  v = v_g         appended as bf16 at row pos
//     s_t  = q_h . K[t, g] / sqrt(D),  p = softmax(s),  a_h = sum_t p_t V[t, g]
//     out  = a_h * sigmoid(q_full[h, D:])
//
// Two launches, no inter-block synchronisation inside either (an agent-scope
// fence per block costs an L2 write-back per XCD on this part):
//   attn_partial_kernel  grid (chunk of positions, kv head g), 256 threads.
//       The first batch of K/V row loads is issued before anything else (it
//       does not depend on this token), then the block builds the G query
//       heads of its group and the new key in LDS; the block whose chunk holds
//       `pos` also stores the new K/V row.  A row of the cache is D/8 lanes
//       (16 bytes each); the block's row slots each run an online softmax over
//       their rows (base-2 exponent), then merge in LDS and the block writes
//       one (max, sum, unnormalised output) triple per query head.  Each K/V
//       row is read once for all G heads of its group (the GQA reuse).
//   attn_merge_kernel    grid (q head, D/32), 256 threads: log-sum-exp merge
//       of the chunk partials, the division by the total, the sigmoid gate.
//
// Layouts: K/V caches bf16 [capacity, Hkv, D] (token-major).
#include <type_traits>

#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace {

constexpr int kNT = 256;
constexpr int kUnroll = 4;                    // rows per row slot per batch
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct AGeo {
    static constexpr int LPR = D / 8;         // lanes per cache row
    static constexpr int RPI = kNT / LPR;     // row slots per block
    static constexpr int B = RPI * kUnroll;   // rows per batch
};

Q35_DEV void unpack8(const uint4& u, float v[8]) {
    v[0] = bf16_lo(u.x);
    v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y);
    v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z);
    v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w);
    v[7] = bf16_hi(u.w);
}

Q35_DEV int32_t attn_pos(const AttnArgs& a) {
    return a.host_pos >= 0 ? a.host_pos : a.positions[0];
}

// T8: Turbo8 cache (E4M3 codes [capacity, Hkv, D] with bf16 scales per 16
// [capacity, Hkv, D/16], in the orthonormal Walsh-Hadamard basis of a head).
// The prologue also rotates the G query heads and the new k and v, the block
// holding `pos` quantises the rotated k and v in groups of 16, rows are
// dequantised in the loop, and the block's unnormalised per-head accumulators
// are rotated back before they are written (the transform is linear and its
// own inverse, so the merge is unchanged).
template <int D, int G, bool T8>
__global__ __launch_bounds__(kNT) void attn_partial_kernel(AttnArgs a) {
    static_assert(D <= kNT && D % 32 == 0, "one new-v element per thread; merge blocks of 32 dims");
    using Geo = AGeo<D>;
    constexpr int LPR = Geo::LPR, RPI = Geo::RPI, B = Geo::B;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int j = t % LPR;   // dim slice [8j, 8j+8)
    const int rs = t / LPR;  // row slot
    const uint32_t g = blockIdx.y;
    const uint32_t c = blockIdx.x;
    const uint32_t T = a.chunk;

    __shared__ float qs[(G + 1) * D];  // q heads of the group, then the new k
    __shared__ float vn[D];            // new v, bf16-rounded
    __shared__ float rsq[G + 1];
    __shared__ float2 rot[D / 2];      // (cos, sin) of pos * inv_freq[d], d < rotary / 2
    __shared__ float mls[RPI][2 * G];  // per-slot (max, sum)
    __shared__ float red[RPI * D];     // per-slot outputs of one head
    __shared__ float ov[T8 ? G * D : 1];  // Turbo8: merged accumulators, rotated back in place
    constexpr float kInvSqrtD = D == 64 ? 0.125f : D == 256 ? 0.0625f : 0.08838834764831845f;

    const int32_t pos = attn_pos(a);
    if (pos < 0 || (uint32_t)pos >= a.capacity) return;
    const uint32_t L = (uint32_t)pos + 1;
    const uint32_t nch = (L + T - 1) / T;
    if (c >= nch) return;
    const uint32_t t0 = c * T;
    const uint32_t t1 = min(t0 + T, L);
    const bool has_new = (uint32_t)pos >= t0 && (uint32_t)pos < t1;
    const int32_t rope_pos = a.positions[0];

    // ---------------- first batch of K/V loads, in flight during the prologue
    const uint32_t row_bytes = a.hkv * D * (T8 ? 1u : 2u);      // one token's row of K (or V) data
    const uint32_t span = (t1 - t0) * row_bytes;
    const uint32_t srow_bytes = a.hkv * (D / 16) * 2u;          // Turbo8: one token's scales
    const uint32_t sspan = T8 ? (t1 - t0) * srow_bytes : 0u;

    // ---------------- the prologue's own loads go out first (vector loads
    // complete in order, so the prologue then waits for them alone)
    constexpr int PQ = ((G + 1) * D + kNT - 1) / kNT;  // q/k elements per thread
    float qv[PQ], nv[PQ];
#pragma unroll
    for (int r = 0; r < PQ; ++r) {
        const int e = min(t + kNT * r, (G + 1) * D - 1);  // clamped: no branch around the loads
        const int i = e / D, d = e % D;
        qv[r] = (i < G) ? a.q_full[(size_t)(g * G + i) * 2 * D + d] : a.k[g * D + d];
        nv[r] = bf16_to_f32((i < G) ? a.q_norm[d] : a.k_norm[d]);
    }
    const float vnew = a.v[g * D + min(t, D - 1)];
    const float invf = a.inv_freq[min(t, (int)a.rotary / 2 - 1)];
    asm volatile("" ::: "memory");

    const size_t row0 = ((size_t)t0 * a.hkv + g) * D;  // element offset of the chunk's first row
    const auto rk = rsrc(T8 ? (const void*)(reinterpret_cast<const uint8_t*>(a.kc) + row0)
                            : (const void*)(a.kc + row0), span);
    const auto rv = rsrc(T8 ? (const void*)(reinterpret_cast<const uint8_t*>(a.vc) + row0)
                            : (const void*)(a.vc + row0), span);
    const size_t srow0 = ((size_t)t0 * a.hkv + g) * (D / 16);
    const auto rks = rsrc(a.ks + (T8 ? srow0 : 0), sspan);
    const auto rvs = rsrc(a.vs + (T8 ? srow0 : 0), sspan);
    // two batches in flight: the next batch's rows load while this one computes
    using KT = std::conditional_t<T8, uint2, uint4>;  // 8 elements of one row per lane
    KT kr[2][kUnroll], vr[2][kUnroll];
    uint32_t ksr[2][kUnroll], vsr[2][kUnroll];  // Turbo8: the lane's group scale (bf16 bits)
    auto load_batch = [&](KT (&kd)[kUnroll], KT (&vd)[kUnroll], uint32_t (&ksd)[kUnroll],
                          uint32_t (&vsd)[kUnroll], uint32_t tb) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI + rs;
            const bool live = tt < t1 && tt != (uint32_t)pos;
            if constexpr (T8) {
                const uint32_t off = live ? (tt - t0) * row_bytes + 8u * j : span;  // past the end: zero
                const uint32_t soff = live ? (tt - t0) * srow_bytes + 2u * (j / 2) : sspan;
                kd[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, kAuxStream));
                vd[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, kAuxStream));
                ksd[u] = __builtin_amdgcn_raw_buffer_load_b16(rks, soff, 0, kAuxStream);
                vsd[u] = __builtin_amdgcn_raw_buffer_load_b16(rvs, soff, 0, kAuxStream);
            } else {
                const uint32_t off = live ? (tt - t0) * row_bytes + 16u * j : span;  // past the end: zero
                kd[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kAuxStream));
                vd[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kAuxStream));
            }
        }
    };
    load_batch(kr[0], vr[0], ksr[0], vsr[0], t0);
    load_batch(kr[1], vr[1], ksr[1], vsr[1], t0 + B);  // loads past the chunk return zero, unused

    // ---------------- prologue: q heads of this group and the new k, v
#pragma unroll
    for (int r = 0; r < PQ; ++r)
        if (t + kNT * r < (G + 1) * D) qs[t + kNT * r] = qv[r];
    if (t < D) vn[t] = T8 ? vnew : bf16_to_f32(f32_to_bf16(vnew));
    if (t < (int)a.rotary / 2) {
        float sn, cs;
        sincosf((float)rope_pos * invf, &sn, &cs);
        rot[t] = make_float2(cs, sn);
    }
    __syncthreads();
    for (int i = wid; i < G + 1; i += kNT / 64) {
        float ss = 0.f;
        for (int d = lane; d < D; d += 64) ss = fmaf(qs[i * D + d], qs[i * D + d], ss);
        ss = wave_sum(ss);
        if (lane == 0) rsq[i] = 1.0f / sqrtf(ss / (float)D + a.eps);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < PQ; ++r) {
        const int e = t + kNT * r;
        if (e < (G + 1) * D) qs[e] = qs[e] * rsq[e / D] * nv[r];
    }
    __syncthreads();
    {
        const int half = (int)a.rotary / 2;
        for (int e = t; e < (G + 1) * half; e += kNT) {
            const int i = e / half, d = e % half;
            const float cs = rot[d].x, sn = rot[d].y;
            const float x1 = qs[i * D + d], x2 = qs[i * D + d + half];
            qs[i * D + d] = x1 * cs - x2 * sn;
            qs[i * D + d + half] = x2 * cs + x1 * sn;
        }
    }
    __syncthreads();
    if (a.q_norm_out && c == 0)
        for (int e = t; e < G * D; e += kNT) a.q_norm_out[(size_t)g * G * D + e] = qs[e];
    if constexpr (T8) {
        if (has_new && a.k_norm_out)
            for (int d = t; d < D; d += kNT) a.k_norm_out[g * D + d] = qs[G * D + d];
        __syncthreads();  // the taps read qs before the rotation rewrites it
        // orthonormal Walsh-Hadamard transform of the G query heads, the new k and
        // the new v: butterflies of doubling width, 1/sqrt(D) in the last stage
        auto vec = [&](int vi) { return vi <= G ? qs + vi * D : vn; };
        for (int h = 1; h < D; h <<= 1) {
            const float f = 2 * h == D ? kInvSqrtD : 1.0f;
            for (int e = t; e < (G + 2) * (D / 2); e += kNT) {
                const int vi = e / (D / 2), p = e % (D / 2);
                const int i = (p / h) * 2 * h + p % h;
                float* x = vec(vi);
                const float u = x[i], w = x[i + h];
                x[i] = (u + w) * f;
                x[i + h] = (u - w) * f;
            }
            __syncthreads();
        }
        if (has_new) {
            // quantising append: one thread per group of 16 of the rotated k or v;
            // the block then attends to the dequantised row, as stored
            if (t < 2 * (D / 16)) {
                const int side = t / (D / 16), grp = t % (D / 16);
                float* src = (side ? vn : qs + G * D) + 16 * grp;
                float v16[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) v16[e] = src[e];
                uint32_t cw[4];
                const uint32_t sb = turbo8_quantize16(v16, cw);
                uint8_t* dst = reinterpret_cast<uint8_t*>(side ? a.vc : a.kc) + ((size_t)pos * a.hkv + g) * D + 16 * grp;
                *reinterpret_cast<uint4*>(dst) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
                (side ? a.vs : a.ks)[((size_t)pos * a.hkv + g) * (D / 16) + grp] = (uint16_t)sb;
                const float sc = bf16_to_f32(sb);
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                    const q35_float2_t lo = e4m3x2_to_f32<false>(cw[w4]), hi = e4m3x2_to_f32<true>(cw[w4]);
                    src[4 * w4] = lo.x * sc;
                    src[4 * w4 + 1] = lo.y * sc;
                    src[4 * w4 + 2] = hi.x * sc;
                    src[4 * w4 + 3] = hi.y * sc;
                }
            }
            __syncthreads();
        }
    } else if (has_new) {
        if (a.k_norm_out)
            for (int d = t; d < D; d += kNT) a.k_norm_out[g * D + d] = qs[G * D + d];
        uint16_t* krow = a.kc + ((size_t)pos * a.hkv + g) * D;
        uint16_t* vrow = a.vc + ((size_t)pos * a.hkv + g) * D;
        for (int d = t; d < D; d += kNT) {
            const uint32_t kb = f32_to_bf16(qs[G * D + d]);
            krow[d] = (uint16_t)kb;
            vrow[d] = (uint16_t)f32_to_bf16(vn[d]);  // vn is already bf16-exact
            qs[G * D + d] = bf16_to_f32(kb);  // attend to the row as stored
        }
        __syncthreads();
    }

    // ---------------- batches of B rows: scores, online softmax, p V
    float qr[G][8];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[i][e] = qs[i * D + 8 * j + e];
    const float sscale = a.scale * kLog2e;  // scores in the base-2 exponent domain

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    }

    // 8 elements of a row: bf16 pairs, or Turbo8 codes times the group scale
    auto unpack = [&](const KT& w, uint32_t sbits, float v[8]) {
        if constexpr (T8) {
            const float sc = bf16_to_f32(sbits & 0xFFFFu);
            const q35_float2_t p0 = e4m3x2_to_f32<false>(w.x), p1 = e4m3x2_to_f32<true>(w.x);
            const q35_float2_t p2 = e4m3x2_to_f32<false>(w.y), p3 = e4m3x2_to_f32<true>(w.y);
            v[0] = p0.x * sc;
            v[1] = p0.y * sc;
            v[2] = p1.x * sc;
            v[3] = p1.y * sc;
            v[4] = p2.x * sc;
            v[5] = p2.y * sc;
            v[6] = p3.x * sc;
            v[7] = p3.y * sc;
        } else {
            (void)sbits;
            unpack8(w, v);
        }
    };
    auto batch = [&](const KT (&kd)[kUnroll], const KT (&vd)[kUnroll], const uint32_t (&ksd)[kUnroll],
                     const uint32_t (&vsd)[kUnroll], uint32_t tb) {
        float s[kUnroll][G];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI + rs;
            float kv[8];
            if (tt == (uint32_t)pos) {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = qs[G * D + 8 * j + e];
            } else {
                unpack(kd[u], ksd[u], kv);
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qr[i][e], kv[e], d);
                d = group_sum_all<LPR>(d);
                s[u][i] = tt < t1 ? d * sscale : -INFINITY;
            }
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float mx = m[i];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, s[u][i]);
            const float mref = mx == -INFINITY ? 0.f : mx;  // slot with no rows yet
            const float corr = exp2f(m[i] - mref);
            m[i] = mx;
            l[i] *= corr;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][e] *= corr;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) s[u][i] = exp2f(s[u][i] - mref);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI + rs;
            float vv[8];
            if (tt == (uint32_t)pos) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vv[e] = vn[8 * j + e];
            } else {
                unpack(vd[u], vsd[u], vv);
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                l[i] += s[u][i];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(s[u][i], vv[e], acc[i][e]);
            }
        }
    };
    // Reloads are unconditional (rows past the chunk read zero and move no
    // data), so the count of loads in flight is the same on every path and
    // each wait is for the batch about to be used alone.
    for (uint32_t tb = t0;; tb += 2 * B) {
        batch(kr[0], vr[0], ksr[0], vsr[0], tb);
        if (tb + B >= t1) break;
        load_batch(kr[0], vr[0], ksr[0], vsr[0], tb + 2 * B);
        batch(kr[1], vr[1], ksr[1], vsr[1], tb + B);
        if (tb + 2 * B >= t1) break;
        load_batch(kr[1], vr[1], ksr[1], vsr[1], tb + 3 * B);
    }

    // ---------------- merge the row slots, write this chunk's partials
    if (j == 0)
#pragma unroll
        for (int i = 0; i < G; ++i) {
            mls[rs][2 * i] = m[i];
            mls[rs][2 * i + 1] = l[i];
        }
    __syncthreads();
    float* pacc = a.part_acc + ((size_t)g * a.max_chunks + c) * G * D;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        float M = -INFINITY;
        for (int r = 0; r < RPI; ++r) M = fmaxf(M, mls[r][2 * i]);  // slot 0 always has a row
        const float w = exp2f(m[i] - M);
#pragma unroll
        for (int e = 0; e < 8; ++e) red[rs * D + 8 * j + e] = acc[i][e] * w;
        __syncthreads();
        for (int d = t; d < D; d += kNT) {
            float o = 0.f;
#pragma unroll 8
            for (int r = 0; r < RPI; ++r) o += red[r * D + d];
            if constexpr (T8)
                ov[i * D + d] = o;
            else
                pacc[i * D + d] = o;
        }
        if (t == 0) {
            float tot = 0.f;
            for (int r = 0; r < RPI; ++r) tot = fmaf(exp2f(mls[r][2 * i] - M), mls[r][2 * i + 1], tot);
            float* pml = a.part_ml + ((size_t)g * a.max_chunks + c) * 2 * G;
            pml[2 * i] = M;
            pml[2 * i + 1] = tot;
        }
        __syncthreads();
    }
    if constexpr (T8) {
        // each head's merged accumulator back to the original basis (the
        // orthonormal transform is its own inverse; the merge is linear)
        for (int h = 1; h < D; h <<= 1) {
            const float f = 2 * h == D ? kInvSqrtD : 1.0f;
            for (int e = t; e < G * (D / 2); e += kNT) {
                const int vi = e / (D / 2), p = e % (D / 2);
                const int i = (p / h) * 2 * h + p % h;
                float* x = ov + vi * D;
                const float u = x[i], w = x[i + h];
                x[i] = (u + w) * f;
                x[i + h] = (u - w) * f;
            }
            __syncthreads();
        }
        for (int e = t; e < G * D; e += kNT) pacc[e] = ov[e];
    }
}

// grid (Hq, D/32); thread t: dim d0 + t % 32, chunk lane t / 32.  Each thread
// issues its first kPrefetch partial loads before the weights are known, so the
// partials and the (max, sum) pairs arrive together.
constexpr int kMergeDims = 32;
constexpr int kMergeLanes = kNT / kMergeDims;
constexpr int kPrefetch = 16;

template <int D, int G>
__global__ __launch_bounds__(kNT) void attn_merge_kernel(AttnArgs a) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int dl = t % kMergeDims, cl = t / kMergeDims;
    const uint32_t h = blockIdx.x, g = h / G, i = h % G;
    const uint32_t d = blockIdx.y * kMergeDims + dl;
    extern __shared__ float wsh[];  // [max_chunks] chunk weights
    __shared__ float red[kNT];
    __shared__ float stat[kNT / 64];

    const int32_t pos = attn_pos(a);
    if (pos < 0 || (uint32_t)pos >= a.capacity) return;
    const uint32_t nch = ((uint32_t)pos + a.chunk) / a.chunk;

    // partials of head h, dim d: part_acc[g][cc][i][d], chunk stride G*D floats
    const uint32_t cstride = (uint32_t)(G * D) * 4u;
    const auto racc = rsrc(a.part_acc + ((size_t)g * a.max_chunks * G + i) * D, nch * cstride);
    float pa[kPrefetch];
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
        const uint32_t cc = (uint32_t)(cl + kMergeLanes * k);
        pa[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(racc, cc * cstride + d * 4u, 0, 0));
    }
    const float* pml = a.part_ml + (size_t)g * a.max_chunks * 2 * G + 2 * i;

    float mx = -INFINITY;
    for (uint32_t cc = t; cc < nch; cc += kNT) mx = fmaxf(mx, pml[cc * 2 * G]);
    mx = wave_max(mx);
    if (lane == 0) red[wid] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < kNT / 64; ++w) M = fmaxf(M, red[w]);
    float tot = 0.f;
    for (uint32_t cc = t; cc < nch; cc += kNT) {
        const float w = exp2f(pml[cc * 2 * G] - M);
        wsh[cc] = w;
        tot = fmaf(w, pml[cc * 2 * G + 1], tot);
    }
    tot = block_sum<kNT>(tot, stat);  // its barriers also publish wsh (and free red)

    float o = 0.f;
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
        const uint32_t cc = (uint32_t)(cl + kMergeLanes * k);
        if (cc < nch) o = fmaf(wsh[cc], pa[k], o);
    }
    for (uint32_t cc = cl + kMergeLanes * kPrefetch; cc < nch; cc += kMergeLanes)
        o = fmaf(wsh[cc], __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(racc, cc * cstride + d * 4u, 0, 0)), o);
    red[t] = o;
    __syncthreads();
    if (cl == 0) {
        o = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < kMergeLanes; ++c2) o += red[c2 * kMergeDims + dl];
        o /= tot;
        if (a.attn_out) a.attn_out[h * D + d] = o;
        const float gate = a.q_full[(size_t)h * 2 * D + D + d];
        a.gated_attn[h * D + d] = o * sigmoidf_(gate);
    }
}

template <int D, int G>
hipError_t launch_t(const AttnArgs& a, uint32_t grid_chunks, bool t8, hipStream_t stream) {
    if (t8)
        hipLaunchKernelGGL((attn_partial_kernel<D, G, true>), dim3(grid_chunks, a.hkv), dim3(kNT), 0, stream, a);
    else
        hipLaunchKernelGGL((attn_partial_kernel<D, G, false>), dim3(grid_chunks, a.hkv), dim3(kNT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_merge_kernel<D, G>), dim3(a.hq, D / kMergeDims), dim3(kNT),
                       (size_t)a.max_chunks * sizeof(float), stream, a);
    return hipGetLastError();
}

// Turbo8 group quantiser over a plain vector (kernel-level export): one thread
// per group of 16.
__global__ __launch_bounds__(256) void turbo8_quantize_kernel(const float* x, uint32_t groups,
                                                              uint8_t* codes, uint16_t* scales) {
    const uint32_t gi = blockIdx.x * 256u + threadIdx.x;
    if (gi >= groups) return;
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = x[16u * gi + e];
    uint32_t cw[4];
    scales[gi] = (uint16_t)turbo8_quantize16(v, cw);
    *reinterpret_cast<uint4*>(codes + 16u * gi) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
}

// Every E4M3 code through the decoder the attention loop uses (kernel-level export).
__global__ __launch_bounds__(64) void e4m3_table_kernel(float* out) {
    const uint32_t t = threadIdx.x;  // codes 4t..4t+3
    const uint32_t w = (4u * t) | ((4u * t + 1u) << 8) | ((4u * t + 2u) << 16) | ((4u * t + 3u) << 24);
    const q35_float2_t lo = e4m3x2_to_f32<false>(w), hi = e4m3x2_to_f32<true>(w);
    out[4 * t] = lo.x;
    out[4 * t + 1] = lo.y;
    out[4 * t + 2] = hi.x;
    out[4 * t + 3] = hi.y;
}

}  // namespace

uint32_t attn_rows_per_iter(uint32_t head_dim) { return (kNT / (head_dim / 8)) * kUnroll; }

#define Q35_ATTN_SHAPES(X) \
    X(64, 1) X(64, 2) X(64, 4) X(64, 8) X(128, 1) X(128, 2) X(128, 4) X(128, 8) \
    X(256, 1) X(256, 2) X(256, 4) X(256, 8)

bool attn_dims_supported(uint32_t head_dim, uint32_t group) {
#define X(DD, GG) if (head_dim == DD && group == GG) return true;
    Q35_ATTN_SHAPES(X)
#undef X
    return false;
}

hipError_t attn_launch(uint32_t head_dim, uint32_t group, const AttnArgs& a, uint32_t grid_chunks,
                       bool turbo8, hipStream_t stream) {
#define X(DD, GG) \
    if (head_dim == DD && group == GG) return launch_t<DD, GG>(a, grid_chunks, turbo8, stream);
    Q35_ATTN_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

const void* attn_kernel_ptr(uint32_t head_dim, uint32_t group, bool turbo8) {
#define X(DD, GG)                                                                             \
    if (head_dim == DD && group == GG)                                                        \
        return turbo8 ? (const void*)&attn_partial_kernel<DD, GG, true>                       \
                      : (const void*)&attn_partial_kernel<DD, GG, false>;
    Q35_ATTN_SHAPES(X)
#undef X
    return nullptr;
}

const void* attn_combine_kernel_ptr(uint32_t head_dim, uint32_t group) {
#define X(DD, GG) \
    if (head_dim == DD && group == GG) return (const void*)&attn_merge_kernel<DD, GG>;
    Q35_ATTN_SHAPES(X)
#undef X
    return nullptr;
}

hipError_t turbo8_quantize_launch(const float* x, uint32_t n, uint8_t* codes, uint16_t* scales,
                                  hipStream_t stream) {
    const uint32_t groups = n / 16;
    if (groups == 0) return hipSuccess;
    hipLaunchKernelGGL(turbo8_quantize_kernel, dim3((groups + 255) / 256), dim3(256), 0, stream, x,
                       groups, codes, scales);
    return hipGetLastError();
}

hipError_t e4m3_table_launch(float* out256, hipStream_t stream) {
    hipLaunchKernelGGL(e4m3_table_kernel, dim3(1), dim3(64), 0, stream, out256);
    return hipGetLastError();
}

}  // namespace q35
