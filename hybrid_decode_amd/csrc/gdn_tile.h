// Tile of the gated delta rule for the multi-stage decode kernels (the
// persistent one and the XCD-split one): the linear_attention.rs page's
// recurrence step on 16 state columns of one v-head per block.
#pragma once

#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {

// One tile of 16 state columns of one v-head per block (threads [0, 2*DK)), the
// same arithmetic as the standalone recurrence kernel: with a = S^T k and
// b = S^T q of the old state, delta = beta (v - g a), y = (g b + (k.q) delta)/sqrt(dk),
// S' = g S + k delta^T.  The state tile is loaded before wait(), which returns
// once q, k, v, the gate and beta of this launch are published.  SYNC 1: they
// were written by any block of the launch (device-coherent loads and y
// stores); SYNC 2: by blocks of the same XCD (device-coherent loads, plain
// stores).
constexpr int kCT = 16;

template <int SYNC>
Q35_DEV float ld_stage_f32(const float* p, uint32_t i) {
    if constexpr (SYNC == 1)
        return ld_coh_f32(p, i);
    else
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(p, 0xFFFFFFFFu), 4u * i, 0, kAuxCoherent));
}

template <int DK, int SYNC, class Wait>
Q35_DEV void gdn_tile(const GdnArgs& a, uint32_t tile, uint8_t* lds, Wait&& wait) {
    static_assert(SYNC == 1 || SYNC == 2, "a stage of a multi-stage launch");
    constexpr int DV = DK, TT = 2 * DK, NW = (TT + 63) / 64, NPR = TT / 16;
    float* dl = reinterpret_cast<float*>(lds);  // [kCT]
    float* red = dl + kCT;                      // [3][NW]
    float* part = red + 3 * NW;                 // [NPR][2][kCT]

    const int t = tid_x(), lane = t & 63, wid = t >> 6;
    const int cq = t & 3, r = t >> 2;
    const uint32_t tiles_per_head = DV / kCT;
    const bool tile_ok = tile < a.hv * tiles_per_head;  // block-uniform
    const bool act = tile_ok && t < TT;                 // wave-uniform
    const uint32_t h = tile / tiles_per_head;
    const uint32_t col0 = (tile % tiles_per_head) * kCT;
    const uint32_t rep = a.hv / a.hk;
    const uint32_t i = h / rep;
    const uint32_t row0 = 2 * r;

    float* sbase = a.state + (size_t)h * DK * DV + col0 + 4 * cq;
    float4 S0 = make_float4(0.f, 0.f, 0.f, 0.f), S1 = S0;
    if (act) {  // the state is this launch's own input: no wait needed
        S0 = *reinterpret_cast<const float4*>(sbase + (size_t)row0 * DV);
        S1 = *reinterpret_cast<const float4*>(sbase + (size_t)(row0 + 1) * DV);
    }
    wait();
    if (tile_ok) {
        float2 qr = make_float2(0.f, 0.f), kr = qr;
        float vv = 0.f, g = 0.f, beta = 0.f;
        if (act) {
            qr = make_float2(ld_stage_f32<SYNC>(a.qkv_conv, i * DK + row0), ld_stage_f32<SYNC>(a.qkv_conv, i * DK + row0 + 1));
            const uint32_t ko = a.hk * DK + i * DK + row0;
            kr = make_float2(ld_stage_f32<SYNC>(a.qkv_conv, ko), ld_stage_f32<SYNC>(a.qkv_conv, ko + 1));
            vv = ld_stage_f32<SYNC>(a.qkv_conv, 2 * a.hk * DK + h * DV + col0 + min(t, kCT - 1));
            g = ld_stage_f32<SYNC>(a.gate, h);
            beta = ld_stage_f32<SYNC>(a.beta, h);

            float pa[4], pb[4];
            pa[0] = fmaf(S0.x, kr.x, S1.x * kr.y);
            pa[1] = fmaf(S0.y, kr.x, S1.y * kr.y);
            pa[2] = fmaf(S0.z, kr.x, S1.z * kr.y);
            pa[3] = fmaf(S0.w, kr.x, S1.w * kr.y);
            pb[0] = fmaf(S0.x, qr.x, S1.x * qr.y);
            pb[1] = fmaf(S0.y, qr.x, S1.y * qr.y);
            pb[2] = fmaf(S0.z, qr.x, S1.z * qr.y);
            pb[3] = fmaf(S0.w, qr.x, S1.w * qr.y);
#pragma unroll
            for (int c = 0; c < 4; ++c) {  // rotate each 16-lane row by 4 and 8: column quad kept
                pa[c] += dpp<0x124>(pa[c]);
                pb[c] += dpp<0x124>(pb[c]);
                pa[c] += dpp<0x128>(pa[c]);
                pb[c] += dpp<0x128>(pb[c]);
            }
            const bool own = cq == 0;
            const float r0 = wave_sum(own ? fmaf(qr.x, qr.x, qr.y * qr.y) : 0.f);
            const float r1 = wave_sum(own ? fmaf(kr.x, kr.x, kr.y * kr.y) : 0.f);
            const float r2 = wave_sum(own ? fmaf(kr.x, qr.x, kr.y * qr.y) : 0.f);
            if (lane == 0) {
                red[0 * NW + wid] = r0;
                red[1 * NW + wid] = r1;
                red[2 * NW + wid] = r2;
            }
            if ((lane & 15) < 4) {
                const int pr = t >> 4;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    part[(pr * 2 + 0) * kCT + 4 * cq + c] = pa[c];
                    part[(pr * 2 + 1) * kCT + 4 * cq + c] = pb[c];
                }
            }
        }
        __syncthreads();
        float rk = 0.f;
        if (act) {
            float qq = 0.f, kk = 0.f, kq = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                qq += red[0 * NW + w];
                kk += red[1 * NW + w];
                kq += red[2 * NW + w];
            }
            const float rq = 1.0f / sqrtf(qq + a.l2_eps);
            rk = 1.0f / sqrtf(kk + a.l2_eps);
            kq *= rq * rk;
            if (t < kCT) {
                float av = 0.f, bv = 0.f;
#pragma unroll
                for (int w = 0; w < NPR; ++w) {
                    av += part[(w * 2 + 0) * kCT + t];
                    bv += part[(w * 2 + 1) * kCT + t];
                }
                const float d = beta * (vv - g * av * rk);
                dl[t] = d;
                st_f32<SYNC == 1>(a.y, h * DV + col0 + t, (g * bv * rq + kq * d) * a.out_scale);
            }
        }
        __syncthreads();
        if (act) {
            const float d0 = dl[4 * cq], d1 = dl[4 * cq + 1], d2 = dl[4 * cq + 2], d3 = dl[4 * cq + 3];
            const float k0 = kr.x * rk, k1 = kr.y * rk;
            float4 o0, o1;
            o0.x = fmaf(k0, d0, g * S0.x);
            o0.y = fmaf(k0, d1, g * S0.y);
            o0.z = fmaf(k0, d2, g * S0.z);
            o0.w = fmaf(k0, d3, g * S0.w);
            o1.x = fmaf(k1, d0, g * S1.x);
            o1.y = fmaf(k1, d1, g * S1.y);
            o1.z = fmaf(k1, d2, g * S1.z);
            o1.w = fmaf(k1, d3, g * S1.w);
            *reinterpret_cast<float4*>(sbase + (size_t)row0 * DV) = o0;
            *reinterpret_cast<float4*>(sbase + (size_t)(row0 + 1) * DV) = o1;
        }
    }
}

}  // namespace q35
