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
// 32 columns: a tile row is one 128-byte line, so every line of the state is
// read and written by exactly one block (a 16-column tile left each line half
// to a block on another XCD, and both XCDs' L2s fetched all of it).  With
// a = S_old^T k and b = S_old^T q the step is
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

constexpr int kCT = 32;  // state columns per block (one 128-byte line per row)

// Threads: 2*DK.  Thread t holds state rows {2r, 2r+1} (r = t / 4) for the 8
// columns 8c..8c+7 (c = t % 4) of the block's tile: four float4 per thread, all
// issued before any arithmetic.
template <int DK>
__global__ __launch_bounds__(2 * DK) void gdn_kernel(GdnArgs a) {
    constexpr int DV = DK;
    constexpr int NT = 2 * DK, NW = (NT + 63) / 64;
    constexpr int NPR = NT / 16;  // 16-lane DPP rows; each sums 4 row pairs (8 state rows)
    static_assert(NT >= 64 && kCT == 32 && DV % kCT == 0, "at least one wave; 4 lanes cover a tile row");
    __shared__ float dl[kCT];
    __shared__ float red[3][NW];
    __shared__ float part[NPR][2][kCT];  // per DPP row: a and b partials of the tile's columns

    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int cq = t & 3, r = t >> 2;
    const uint32_t h = blockIdx.y;
    const uint32_t col0 = blockIdx.x * kCT;
    const uint32_t rep = a.hv / a.hk;
    const uint32_t i = h / rep;
    const uint32_t row0 = 2 * r;

    // 1. every load is issued up front: the state tile, this thread's two q and
    //    k entries (raw; the L2 norms become two scalar factors), v, gate, beta
    float* sbase = a.state + (size_t)h * DK * DV + col0 + 8 * cq;
    float S[2][8];
    {
        const float4* p0 = reinterpret_cast<const float4*>(sbase + (size_t)row0 * DV);
        const float4* p1 = reinterpret_cast<const float4*>(sbase + (size_t)(row0 + 1) * DV);
        const float4 u0 = p0[0], u1 = p0[1], u2 = p1[0], u3 = p1[1];
        S[0][0] = u0.x; S[0][1] = u0.y; S[0][2] = u0.z; S[0][3] = u0.w;
        S[0][4] = u1.x; S[0][5] = u1.y; S[0][6] = u1.z; S[0][7] = u1.w;
        S[1][0] = u2.x; S[1][1] = u2.y; S[1][2] = u2.z; S[1][3] = u2.w;
        S[1][4] = u3.x; S[1][5] = u3.y; S[1][6] = u3.z; S[1][7] = u3.w;
    }
    const float2 qr = *reinterpret_cast<const float2*>(a.qkv_conv + i * DK + row0);
    const float2 kr = *reinterpret_cast<const float2*>(a.qkv_conv + a.hk * DK + i * DK + row0);
    const float vv = a.qkv_conv[2 * a.hk * DK + h * DV + col0 + min(t, kCT - 1)];
    const float g = a.gate[h];
    const float beta = a.beta[h];

    // 2. partial a = S^T k, b = S^T q (raw q, k) and the norms' sums, reduced
    //    over the rows of each 16-lane DPP row (lanes of equal column octet)
    float pa[8], pb[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        pa[c] = fmaf(S[0][c], kr.x, S[1][c] * kr.y);
        pb[c] = fmaf(S[0][c], qr.x, S[1][c] * qr.y);
    }
    // rotating a 16-lane row by 4 and then 8 keeps lane & 3 (the column octet):
    // every lane ends with the sum over the row's 4 row pairs for its columns
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        pa[c] += dpp<0x124>(pa[c]);  // row_ror:4
        pb[c] += dpp<0x124>(pb[c]);
        pa[c] += dpp<0x128>(pa[c]);  // row_ror:8
        pb[c] += dpp<0x128>(pb[c]);
    }
    const bool own = cq == 0;  // one thread per row pair feeds the norms
    float r0 = wave_sum(own ? fmaf(qr.x, qr.x, qr.y * qr.y) : 0.f);
    float r1 = wave_sum(own ? fmaf(kr.x, kr.x, kr.y * kr.y) : 0.f);
    float r2 = wave_sum(own ? fmaf(kr.x, qr.x, kr.y * qr.y) : 0.f);
    if (lane == 0) {
        red[0][wid] = r0;
        red[1][wid] = r1;
        red[2][wid] = r2;
    }
    if ((lane & 15) < 4) {  // lanes 0..3 of each DPP row: column octets 0..3
        const int pr = t >> 4;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            part[pr][0][8 * cq + c] = pa[c];
            part[pr][1][8 * cq + c] = pb[c];
        }
    }
    __syncthreads();
    float qq = 0.f, kk = 0.f, kq = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        qq += red[0][w];
        kk += red[1][w];
        kq += red[2][w];
    }
    const float rq = 1.0f / sqrtf(qq + a.l2_eps);
    const float rk = 1.0f / sqrtf(kk + a.l2_eps);
    kq *= rq * rk;

    // 3. per column: delta and y (y is stored after the state: a store issued
    //    here would make the wait before the state stores include its latency,
    //    the vector memory counter counting stores as well as loads)
    float yv = 0.f;
    if (t < kCT) {
        float av = 0.f, bv = 0.f;
#pragma unroll
        for (int w = 0; w < NPR; ++w) {
            av += part[w][0][t];
            bv += part[w][1][t];
        }
        const float d = beta * (vv - g * av * rk);
        dl[t] = d;
        yv = (g * bv * rq + kq * d) * a.out_scale;
    }
    __syncthreads();

    // 4. S' = g S + k delta^T (k normalised)
    const float k0 = kr.x * rk, k1 = kr.y * rk;
    float o[2][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float d = dl[8 * cq + c];
        o[0][c] = fmaf(k0, d, g * S[0][c]);
        o[1][c] = fmaf(k1, d, g * S[1][c]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float4* p = reinterpret_cast<float4*>(sbase + (size_t)(row0 + j) * DV);
        p[0] = make_float4(o[j][0], o[j][1], o[j][2], o[j][3]);
        p[1] = make_float4(o[j][4], o[j][5], o[j][6], o[j][7]);
    }
    if (t < kCT) a.y[h * DV + col0 + t] = yv;
    if (a.qkv_smooth) {
        if (blockIdx.x == 0 && (h % rep) == 0 && own) {
            a.qkv_smooth[i * DK + row0] = qr.x * rq;
            a.qkv_smooth[i * DK + row0 + 1] = qr.y * rq;
            a.qkv_smooth[a.hk * DK + i * DK + row0] = kr.x * rk;
            a.qkv_smooth[a.hk * DK + i * DK + row0 + 1] = kr.y * rk;
        }
        if (t < kCT) a.qkv_smooth[2 * a.hk * DK + h * DV + col0 + t] = vv;
    }
}

}  // namespace

bool gdn_dims_supported(uint32_t dk, uint32_t dv) {
    return dk == dv && (dk == 32 || dk == 64 || dk == 128);
}

hipError_t gdn_launch(uint32_t dk, uint32_t dv, const GdnArgs& a, hipStream_t stream) {
    dim3 grid(dv / kCT, a.hv);
    switch (dk) {
        case 32: hipLaunchKernelGGL(gdn_kernel<32>, grid, dim3(64), 0, stream, a); break;
        case 64: hipLaunchKernelGGL(gdn_kernel<64>, grid, dim3(128), 0, stream, a); break;
        case 128: hipLaunchKernelGGL(gdn_kernel<128>, grid, dim3(256), 0, stream, a); break;
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
