// Gated GQA decode attention over a bf16 KV cache (gfx950), one token.
//
// Fuses the middle of the pages' full-attention forward (full_attention.rs
// page: the q/gate split, the per-head q/k RMSNorm, partial RoPE, the KV
// append and `attention_decode`, then the `sigmoid_gate` launch):
//     q_h  = RoPE(RMSNorm(q_full[h, :D]; q_norm))        h in the kv group
//     k    = RoPE(RMSNorm(k_g; k_norm)),  v = v_g         appended as bf16 at row pos
//     s_t  = q_h . K[t, g] / sqrt(D),  p = softmax(s),  a_h = sum_t p_t V[t, g]
//     out  = a_h * sigmoid(q_full[h, D:])
// Grid: (chunk of positions, kv head g).  One block reads each K/V row of its
// chunk once for all G = Hq/Hkv query heads of the group (the GQA reuse), and
// writes a partial (max, sum, unnormalised output) per head.  The last block
// of each kv head to finish (an atomic ticket) merges the partials with the
// usual log-sum-exp rescaling and applies the sigmoid gate, then resets the
// ticket to zero so the next call (or graph replay) starts clean.
//
// Layouts: K/V caches bf16 [capacity, Hkv, D] (token-major); a lane holds 8
// consecutive dims (one 16-byte load), D/8 lanes cover one row.
#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace {

constexpr int kNT = 256;
constexpr int kUnroll = 4;

template <int D>
struct AGeo {
    static constexpr int LPR = D / 8;        // lanes per cache row
    static constexpr int RPI = kNT / LPR;    // rows per block iteration
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

template <int D, int G>
__global__ __launch_bounds__(kNT) void attn_kernel(AttnArgs a) {
    using Geo = AGeo<D>;
    constexpr int LPR = Geo::LPR, RPI = Geo::RPI;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int j = t % LPR;   // dim slice [8j, 8j+8)
    const int rs = t / LPR;  // row slot
    const uint32_t g = blockIdx.y;
    const uint32_t c = blockIdx.x;
    const uint32_t T = a.chunk;

    extern __shared__ float smem[];
    float* qs = smem;                       // [G+1][D]: q heads, then k
    float* vn = qs + (G + 1) * D;           // [D] new v (bf16-rounded)
    float* rsq = vn + D;                    // [G+1] rms factors
    float* ml = rsq + (G + 1);              // [G][2] max, sum
    float* sc = ml + 2 * G + 2;             // union: [G][T] scores, or [RPI][G][D] partial outputs
    __shared__ int last_flag;

    const int32_t pos = a.host_pos >= 0 ? a.host_pos : a.positions[0];
    if (pos < 0 || (uint32_t)pos >= a.capacity) return;
    const uint32_t L = (uint32_t)pos + 1;
    const uint32_t nch = (L + T - 1) / T;
    if (c >= nch) return;
    const uint32_t t0 = c * T;
    const uint32_t t1 = min(t0 + T, L);
    const bool has_new = (uint32_t)pos >= t0 && (uint32_t)pos < t1;
    const int32_t rope_pos = a.positions[0];

    // ---------------- prologue: q heads of this group and the new k, v
    for (int e = t; e < (G + 1) * D; e += kNT) {
        const int i = e / D, d = e % D;
        qs[e] = (i < G) ? a.q_full[(size_t)(g * G + i) * 2 * D + d] : a.k[g * D + d];
    }
    for (int d = t; d < D; d += kNT) vn[d] = bf16_to_f32(f32_to_bf16(a.v[g * D + d]));
    __syncthreads();
    for (int i = wid; i < G + 1; i += kNT / 64) {
        float ss = 0.f;
        for (int d = lane; d < D; d += 64) ss = fmaf(qs[i * D + d], qs[i * D + d], ss);
        ss = wave_sum(ss);
        if (lane == 0) rsq[i] = 1.0f / sqrtf(ss / (float)D + a.eps);
    }
    __syncthreads();
    for (int e = t; e < (G + 1) * D; e += kNT) {
        const int i = e / D, d = e % D;
        const uint16_t* w = (i < G) ? a.q_norm : a.k_norm;
        qs[e] = qs[e] * rsq[i] * bf16_to_f32(w[d]);
    }
    __syncthreads();
    {
        const int half = (int)a.rotary / 2;
        for (int e = t; e < (G + 1) * half; e += kNT) {
            const int i = e / half, d = e % half;
            const float ang = (float)rope_pos * a.inv_freq[d];
            float sn, cs;
            sincosf(ang, &sn, &cs);
            const float x1 = qs[i * D + d], x2 = qs[i * D + d + half];
            qs[i * D + d] = x1 * cs - x2 * sn;
            qs[i * D + d + half] = x2 * cs + x1 * sn;
        }
    }
    __syncthreads();
    if (a.q_norm_out && c == 0)
        for (int e = t; e < G * D; e += kNT) a.q_norm_out[(size_t)g * G * D + e] = qs[e];
    if (has_new) {
        if (a.k_norm_out)
            for (int d = t; d < D; d += kNT) a.k_norm_out[g * D + d] = qs[G * D + d];
        uint16_t* krow = a.kc + ((size_t)pos * a.hkv + g) * D;
        uint16_t* vrow = a.vc + ((size_t)pos * a.hkv + g) * D;
        for (int d = t; d < D; d += kNT) {
            const uint32_t kb = f32_to_bf16(qs[G * D + d]);
            krow[d] = (uint16_t)kb;
            vrow[d] = (uint16_t)f32_to_bf16(a.v[g * D + d]);
            qs[G * D + d] = bf16_to_f32(kb);  // the row this block attends to is the stored one
        }
        __syncthreads();
    }

    // ---------------- pass 1: scores for rows [t0, t1)
    float qr[G][8];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[i][e] = qs[i * D + 8 * j + e];

    const size_t row_stride = (size_t)a.hkv * D;
    const uint16_t* kbase = a.kc + (size_t)g * D + 8 * j;
    const uint16_t* vbase = a.vc + (size_t)g * D + 8 * j;

    for (uint32_t tb = t0 + rs; tb < t1; tb += RPI * kUnroll) {
        uint4 kr[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI;
            kr[u] = make_uint4(0u, 0u, 0u, 0u);
            if (tt < t1 && tt != (uint32_t)pos)
                kr[u] = *reinterpret_cast<const uint4*>(kbase + (size_t)tt * row_stride);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI;
            float kv[8];
            if (tt == (uint32_t)pos) {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = qs[G * D + 8 * j + e];
            } else {
                unpack8(kr[u], kv);
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) s = fmaf(qr[i][e], kv[e], s);
                s = group_sum_last<LPR>(s);
                if (j == LPR - 1 && tt < t1) sc[i * T + (tt - t0)] = s * a.scale;
            }
        }
    }
    __syncthreads();

    // ---------------- softmax over the chunk, per head
    const uint32_t n = t1 - t0;
    for (int i = wid; i < G; i += kNT / 64) {
        float m = -INFINITY;
        for (uint32_t e = lane; e < n; e += 64) m = fmaxf(m, sc[i * T + e]);
        m = wave_max(m);
        float l = 0.f;
        for (uint32_t e = lane; e < n; e += 64) {
            const float p = expf(sc[i * T + e] - m);
            sc[i * T + e] = p;
            l += p;
        }
        l = wave_sum(l);
        if (lane == 0) {
            ml[2 * i] = m;
            ml[2 * i + 1] = l;
        }
    }
    __syncthreads();

    // ---------------- pass 2: unnormalised p V
    float acc[G][8];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    for (uint32_t tb = t0 + rs; tb < t1; tb += RPI * kUnroll) {
        uint4 vr[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI;
            vr[u] = make_uint4(0u, 0u, 0u, 0u);
            if (tt < t1 && tt != (uint32_t)pos)
                vr[u] = *reinterpret_cast<const uint4*>(vbase + (size_t)tt * row_stride);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI;
            if (tt >= t1) break;
            float vv[8];
            if (tt == (uint32_t)pos) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vv[e] = vn[8 * j + e];
            } else {
                unpack8(vr[u], vv);
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float p = sc[i * T + (tt - t0)];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(p, vv[e], acc[i][e]);
            }
        }
    }
    __syncthreads();  // everyone is done with the probabilities: reuse sc
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[(rs * G + i) * D + 8 * j + e] = acc[i][e];
    __syncthreads();

    float* pacc = a.part_acc + ((size_t)g * a.max_chunks + c) * G * D;
    for (int e = t; e < G * D; e += kNT) {
        float s = 0.f;
#pragma unroll 4
        for (int r = 0; r < RPI; ++r) s += sc[r * G * D + e];
        pacc[e] = s;
    }
    if (t < 2 * G) a.part_ml[((size_t)g * a.max_chunks + c) * 2 * G + t] = ml[t];

    // ---------------- last block of this kv head merges the partials
    __threadfence();
    __syncthreads();
    if (t == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + g, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (prev == nch - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // per (chunk, head) weights exp(m_c - M) in sc[c*G + i]; M and the total in ml
    const float* pml = a.part_ml + (size_t)g * a.max_chunks * 2 * G;
    for (int i = wid; i < G; i += kNT / 64) {
        float m = -INFINITY;
        for (uint32_t cc = lane; cc < nch; cc += 64) m = fmaxf(m, pml[cc * 2 * G + 2 * i]);
        m = wave_max(m);
        float l = 0.f;
        for (uint32_t cc = lane; cc < nch; cc += 64) {
            const float w = expf(pml[cc * 2 * G + 2 * i] - m);
            sc[cc * G + i] = w;
            l = fmaf(w, pml[cc * 2 * G + 2 * i + 1], l);
        }
        l = wave_sum(l);
        if (lane == 0) rsq[i] = 1.0f / l;
    }
    __syncthreads();
    const float* pa = a.part_acc + (size_t)g * a.max_chunks * G * D;
    for (int e = t; e < G * D; e += kNT) {
        const int i = e / D, d = e % D;
        float o = 0.f;
        for (uint32_t cc = 0; cc < nch; ++cc) o = fmaf(sc[cc * G + i], pa[(size_t)cc * G * D + e], o);
        o *= rsq[i];
        const uint32_t h = g * G + i;
        if (a.attn_out) a.attn_out[h * D + d] = o;
        const float gate = a.q_full[(size_t)h * 2 * D + D + d];
        a.gated_attn[h * D + d] = o * sigmoidf_(gate);
    }
    if (t == 0) __hip_atomic_store(a.counters + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int G>
hipError_t launch_t(const AttnArgs& a, uint32_t grid_chunks, hipStream_t stream) {
    constexpr int RPI = AGeo<D>::RPI;
    size_t uni = (size_t)G * a.chunk;
    if ((size_t)RPI * G * D > uni) uni = (size_t)RPI * G * D;
    if ((size_t)a.max_chunks * G > uni) uni = (size_t)a.max_chunks * G;
    const size_t lds = ((G + 1) * D + D + (G + 1) + 2 * G + 2 + uni) * sizeof(float);
    hipLaunchKernelGGL((attn_kernel<D, G>), dim3(grid_chunks, a.hkv), dim3(kNT), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

uint32_t attn_rows_per_iter(uint32_t head_dim) { return kNT / (head_dim / 8); }

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
                       hipStream_t stream) {
#define X(DD, GG) \
    if (head_dim == DD && group == GG) return launch_t<DD, GG>(a, grid_chunks, stream);
    Q35_ATTN_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

const void* attn_kernel_ptr(uint32_t head_dim, uint32_t group) {
#define X(DD, GG) \
    if (head_dim == DD && group == GG) return (const void*)&attn_kernel<DD, GG>;
    Q35_ATTN_SHAPES(X)
#undef X
    return nullptr;
}

}  // namespace q35
