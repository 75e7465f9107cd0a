// Gated delta-rule decode recurrence (gfx950), one token, fp32 state.
//
// Per v-head h with k-head i = h / (Hv/Hk), state S_h in [dk, dv] orientation
// (linear_attention.rs page: the `gated_delta_rule_decode` launch; the state
// shape is given by LinearAttentionState in mod.rs):
//     q, k  <- L2-normalised Q and K heads (eps 1e-6)
//     S     <- g S
//     delta  = beta (v - S^T k)
//     S     <- S + k delta^T
//     y      = S^T q / sqrt(dk)
// Columns of S are independent, so the grid splits each head into tiles of
// 32 columns.  With a = S_old^T k and b = S_old^T q the step is
//     delta = beta (v - g a),   y = (g b + (k.q) delta) / sqrt(dk),
//     S'    = g S_old + k delta^T,
// so one pass over the state computes both dot products, and one more writes
// the new state from registers: the state is read and written exactly once.
// The L2 norms of q and k (the tail of the pages' conv kernel) are computed
// here, where q and k are consumed.
#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace {

constexpr int kNT = 256;
constexpr int kCT = 32;  // state columns per block

template <int DK>
__global__ __launch_bounds__(kNT) void gdn_kernel(GdnArgs a) {
    constexpr int DV = DK;
    constexpr int RJ = DK / 32;  // state rows per thread
    __shared__ float qs[DK], ks[DK], vs[kCT], dl[kCT];
    __shared__ float red[3][kNT / 64];
    __shared__ float part[kNT / 64][8][8];

    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int cq = t & 7, rgp = t >> 3;
    const uint32_t h = blockIdx.y;
    const uint32_t col0 = blockIdx.x * kCT;
    const uint32_t rep = a.hv / a.hk;
    const uint32_t i = h / rep;

    // 1. state tile -> registers (issued first: the longest-latency loads)
    float4 S[RJ];
    float* sbase = a.state + (size_t)h * DK * DV + col0 + 4 * cq;
#pragma unroll
    for (int j = 0; j < RJ; ++j) S[j] = *reinterpret_cast<const float4*>(sbase + (size_t)(rgp + 32 * j) * DV);

    // 2. q, k of k-head i; v slice of v-head h; gate, beta
    float qv = 0.f, kv = 0.f;
    if (t < DK) {
        qv = a.qkv_conv[i * DK + t];
        kv = a.qkv_conv[a.hk * DK + i * DK + t];
    }
    if (t < kCT) vs[t] = a.qkv_conv[2 * a.hk * DK + h * DV + col0 + t];
    const float g = a.gate[h];
    const float beta = a.beta[h];

    float r0 = wave_sum(qv * qv), r1 = wave_sum(kv * kv), r2 = wave_sum(kv * qv);
    if (lane == 0) {
        red[0][wid] = r0;
        red[1][wid] = r1;
        red[2][wid] = r2;
    }
    __syncthreads();
    float qq = 0.f, kk = 0.f, kq = 0.f;
#pragma unroll
    for (int w = 0; w < kNT / 64; ++w) {
        qq += red[0][w];
        kk += red[1][w];
        kq += red[2][w];
    }
    const float rq = 1.0f / sqrtf(qq + a.l2_eps);
    const float rk = 1.0f / sqrtf(kk + a.l2_eps);
    kq *= rq * rk;
    if (t < DK) {
        qs[t] = qv * rq;
        ks[t] = kv * rk;
    }
    if (a.qkv_smooth) {
        if (blockIdx.x == 0 && (h % rep) == 0 && t < DK) {
            a.qkv_smooth[i * DK + t] = qv * rq;
            a.qkv_smooth[a.hk * DK + i * DK + t] = kv * rk;
        }
        if (t < kCT) a.qkv_smooth[2 * a.hk * DK + h * DV + col0 + t] = vs[t];
    }
    __syncthreads();

    // 3. a = S^T k, b = S^T q over this thread's rows, for its 4 columns
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const float kr = ks[rgp + 32 * j], qr = qs[rgp + 32 * j];
        pa[0] = fmaf(S[j].x, kr, pa[0]);
        pa[1] = fmaf(S[j].y, kr, pa[1]);
        pa[2] = fmaf(S[j].z, kr, pa[2]);
        pa[3] = fmaf(S[j].w, kr, pa[3]);
        pb[0] = fmaf(S[j].x, qr, pb[0]);
        pb[1] = fmaf(S[j].y, qr, pb[1]);
        pb[2] = fmaf(S[j].z, qr, pb[2]);
        pb[3] = fmaf(S[j].w, qr, pb[3]);
    }
    // sum over the 8 row groups of this wave that share cq (lane bits 3..5)
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pa[c] += __shfl_xor(pa[c], o);
            pb[c] += __shfl_xor(pb[c], o);
        }
    }
    if (lane < 8) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            part[wid][lane][c] = pa[c];
            part[wid][lane][4 + c] = pb[c];
        }
    }
    __syncthreads();

    // 4. per column: delta and y
    if (t < kCT) {
        const int q4 = t >> 2, c = t & 3;
        float av = 0.f, bv = 0.f;
#pragma unroll
        for (int w = 0; w < kNT / 64; ++w) {
            av += part[w][q4][c];
            bv += part[w][q4][4 + c];
        }
        const float d = beta * (vs[t] - g * av);
        dl[t] = d;
        a.y[h * DV + col0 + t] = (g * bv + kq * d) * a.out_scale;
    }
    __syncthreads();

    // 5. S' = g S + k delta^T
    const float d0 = dl[4 * cq], d1 = dl[4 * cq + 1], d2 = dl[4 * cq + 2], d3 = dl[4 * cq + 3];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const float kr = ks[rgp + 32 * j];
        float4 o;
        o.x = fmaf(kr, d0, g * S[j].x);
        o.y = fmaf(kr, d1, g * S[j].y);
        o.z = fmaf(kr, d2, g * S[j].z);
        o.w = fmaf(kr, d3, g * S[j].w);
        *reinterpret_cast<float4*>(sbase + (size_t)(rgp + 32 * j) * DV) = o;
    }
}

}  // namespace

bool gdn_dims_supported(uint32_t dk, uint32_t dv) {
    return dk == dv && (dk == 32 || dk == 64 || dk == 128);
}

hipError_t gdn_launch(uint32_t dk, uint32_t dv, const GdnArgs& a, hipStream_t stream) {
    dim3 grid(dv / kCT, a.hv);
    switch (dk) {
        case 32: hipLaunchKernelGGL(gdn_kernel<32>, grid, dim3(kNT), 0, stream, a); break;
        case 64: hipLaunchKernelGGL(gdn_kernel<64>, grid, dim3(kNT), 0, stream, a); break;
        case 128: hipLaunchKernelGGL(gdn_kernel<128>, grid, dim3(kNT), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

const void* gdn_kernel_ptr(uint32_t dk) {
    switch (dk) {
        case 32: return (const void*)&gdn_kernel<32>;
        case 64: return (const void*)&gdn_kernel<64>;
        case 128: return (const void*)&gdn_kernel<128>;
        default: return nullptr;
    }
}

}  // namespace q35
