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

template <int D, int G>
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
    const uint32_t row_bytes = a.hkv * D * 2u;
    const uint32_t span = (t1 - t0) * row_bytes;

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

    const auto rk = rsrc(a.kc + ((size_t)t0 * a.hkv + g) * D, span);
    const auto rv = rsrc(a.vc + ((size_t)t0 * a.hkv + g) * D, span);
    // two batches in flight: the next batch's rows load while this one computes
    uint4 kr[2][kUnroll], vr[2][kUnroll];
    auto load_batch = [&](uint4 (&kd)[kUnroll], uint4 (&vd)[kUnroll], uint32_t tb) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI + rs;
            const bool live = tt < t1 && tt != (uint32_t)pos;
            const uint32_t off = live ? (tt - t0) * row_bytes + 16u * j : span;  // past the end: zero
            kd[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kAuxStream));
            vd[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kAuxStream));
        }
    };
    load_batch(kr[0], vr[0], t0);
    load_batch(kr[1], vr[1], t0 + B);  // loads past the chunk return zero and are never used

    // ---------------- prologue: q heads of this group and the new k, v
#pragma unroll
    for (int r = 0; r < PQ; ++r)
        if (t + kNT * r < (G + 1) * D) qs[t + kNT * r] = qv[r];
    if (t < D) vn[t] = bf16_to_f32(f32_to_bf16(vnew));
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
    if (has_new) {
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

    auto batch = [&](const uint4 (&kd)[kUnroll], const uint4 (&vd)[kUnroll], uint32_t tb) {
        float s[kUnroll][G];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI + rs;
            float kv[8];
            if (tt == (uint32_t)pos) {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = qs[G * D + 8 * j + e];
            } else {
                unpack8(kd[u], kv);
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
                unpack8(vd[u], vv);
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
        batch(kr[0], vr[0], tb);
        if (tb + B >= t1) break;
        load_batch(kr[0], vr[0], tb + 2 * B);
        batch(kr[1], vr[1], tb + B);
        if (tb + 2 * B >= t1) break;
        load_batch(kr[1], vr[1], tb + 3 * B);
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
hipError_t launch_t(const AttnArgs& a, uint32_t grid_chunks, hipStream_t stream) {
    hipLaunchKernelGGL((attn_partial_kernel<D, G>), dim3(grid_chunks, a.hkv), dim3(kNT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_merge_kernel<D, G>), dim3(a.hq, D / kMergeDims), dim3(kNT),
                       (size_t)a.max_chunks * sizeof(float), stream, a);
    return hipGetLastError();
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
                       hipStream_t stream) {
#define X(DD, GG) \
    if (head_dim == DD && group == GG) return launch_t<DD, GG>(a, grid_chunks, stream);
    Q35_ATTN_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

const void* attn_kernel_ptr(uint32_t head_dim, uint32_t group) {
#define X(DD, GG) \
    if (head_dim == DD && group == GG) return (const void*)&attn_partial_kernel<DD, GG>;
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

}  // namespace q35
