// Gated GQA decode attention (gfx950), one token, over a bf16 or quantised KV
// cache; and the attention of a prompt into a quantised cache.
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
//       row is read once for all G heads of its group (the GQA reuse).  For
//       the quantised formats the pages' sparse-V gate leaves out the value
//       rows whose weight is below a threshold (see the loop).
//       At head dimension 128 and 256 the quantised formats take the
//       matrix-core variant instead (MFT: 64-row tiles decoded once into
//       LDS, scores and p V as MFMAs; same partials).
//   attn_merge_kernel    grid (q head, D/32), 256 threads: log-sum-exp merge
//       of the chunk partials, the division by the total, the sigmoid gate.
// A prompt into a quantised cache (head dimension 128 and 256): the rows
// appended (pfq_prep_kernel), then one causal attention over the rows as
// stored in the same tiles (pfq_flash_kernel).
//
// Layouts: K/V caches token-major [capacity, Hkv, D] (bf16), with the
// quantised formats' data and group scales in the same row order.
#include <type_traits>

#include "q35decode.h"
#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace {

constexpr int kNT = 256;
constexpr int kUnroll = 4;                    // rows per row slot per batch
constexpr int kMfRows = 64;                   // matrix-core path: rows per LDS tile
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

// Row reductions.  A cache row spans LPR lanes; lane j of a row holds G
// partial dot products, one per query head of the group.  Lane j keeps them in
// its own order: slot p holds head p ^ hl(j), hl(j) = head_of_lane<G>(j).
// The first log2(G) exchange steps each halve what a lane carries: it keeps
// the lower half of its slots and adds the partner's upper half, which holds
// the same heads (the partner differs in the one bit of hl that the step
// retires).  Lane j ends with head hl(j) alone in slot 0 after about
// G + log2(LPR) exchanges instead of G * log2(LPR), with no selects.
//   bit 0, 1: quad permutations; bit 2: rotate a 16-lane row by 4 (a cache
//   row fills whole 16-lane rows when LPR >= 16), else a swizzle of lane ^ 4;
//   bit 3: rotate by 8; bit 4: swizzle of lane ^ 16.  A rotation pairs each
//   lane with one whose bit differs and whose lower bits agree, and two of
//   them cover the four quads of a row.
template <int B, int LPR>
Q35_DEV float row_partner(float v) {
    if constexpr (B == 0) return dpp<0xB1>(v);        // quad_perm [1,0,3,2]
    else if constexpr (B == 1) return dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    else if constexpr (B == 2 && LPR >= 16) return dpp<0x124>(v);  // row_ror:4
    else if constexpr (B == 2)
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x101F));
    else if constexpr (B == 3) return dpp<0x128>(v);  // row_ror:8
    else return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// Lane bit b (b < log2 G) carries head bit log2(G) - 1 - b.
template <int G>
Q35_DEV int head_of_lane(int j) {
    int h = 0;
#pragma unroll
    for (int b = 0; b < ilog2c(G); ++b) h |= ((j >> b) & 1) << (ilog2c(G) - 1 - b);
    return h;
}

template <int G, int LPR>
Q35_DEV float row_reduce(float (&x)[G]) {
    constexpr int LG = ilog2c(G), LL = ilog2c(LPR);
    static_assert(LG <= LL && LL <= 5, "rows of G to 32 lanes");
#pragma unroll
    for (int i = 0; i < G / 2; ++i) x[i] += row_partner<0, LPR>(x[i + G / 2]);
    if constexpr (G >= 4)
#pragma unroll
        for (int i = 0; i < G / 4; ++i) x[i] += row_partner<1, LPR>(x[i + G / 4]);
    if constexpr (G >= 8) x[0] += row_partner<2, LPR>(x[1]);
    float v = x[0];
    if constexpr (LG <= 0 && LL > 0) v += row_partner<0, LPR>(v);
    if constexpr (LG <= 1 && LL > 1) v += row_partner<1, LPR>(v);
    if constexpr (LG <= 2 && LL > 2) v += row_partner<2, LPR>(v);
    if constexpr (LL > 3) v += row_partner<3, LPR>(v);
    if constexpr (LL > 4) v += row_partner<4, LPR>(v);
    return v;
}

// For slot p: the value of the lane (in this lane's group of G lanes) whose
// own head is this lane's head in slot p, i.e. lane q ^ rev(p).  Slot 0 is the
// lane itself.
template <int G>
Q35_DEV float slot_bcast(float v, int p) {
    if constexpr (G == 1) {
        (void)p;
        return v;
    } else {
        int r = 0;  // p with its log2(G) bits reversed
#pragma unroll
        for (int b = 0; b < ilog2c(G); ++b) r |= ((p >> b) & 1) << (ilog2c(G) - 1 - b);
        if constexpr (G <= 4) {
            switch (r) {  // quad_perm: lane q reads lane q ^ r
                case 0: return v;
                case 1: return dpp<0xB1>(v);   // [1,0,3,2]
                case 2: return dpp<0x4E>(v);   // [2,3,0,1]
                default: return dpp<0x1B>(v);  // [3,2,1,0]
            }
        } else {
            return __shfl_xor(v, r);
        }
    }
}

// Value of lane (lane ^ LB) of the wave.
template <int LB>
Q35_DEV float lane_xor(float v) {
    if constexpr (LB == 1) return dpp<0xB1>(v);       // quad_perm [1,0,3,2]
    else if constexpr (LB == 2) return dpp<0x4E>(v);  // quad_perm [2,3,0,1]
    else if constexpr (LB < 32)                       // swizzle, bitmask mode: xor LB
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F | (LB << 10)));
    else return __shfl_xor(v, 32);
}

// Orthonormal Walsh-Hadamard transform of one D-vector held by a wave, lane l
// holding elements [E l, E l + E), E = D / 64: butterflies of doubling width h
// ((x_i, x_i+h) -> (x_i + x_i+h, x_i - x_i+h)), inside the lane while h < E,
// then between lanes l and l ^ (h / E); 1/sqrt(D) applied in the last stage.
template <int D>
Q35_DEV void wht_regs(float (&x)[D / 64], int lane) {
    constexpr int E = D / 64;
    constexpr float f = D == 64 ? 0.125f : D == 256 ? 0.0625f : 0.08838834764831845f;
#pragma unroll
    for (int h = 1; h < E; h <<= 1)
#pragma unroll
        for (int i = 0; i < E; ++i)
            if ((i & h) == 0) {
                const float u = x[i], w = x[i + h];
                x[i] = u + w;
                x[i + h] = u - w;
            }
    auto stage = [&](auto lbc) {
        constexpr int LB = decltype(lbc)::value;
        const bool hi = (lane & LB) != 0;
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float p = lane_xor<LB>(x[i]);
            const float y = hi ? p - x[i] : x[i] + p;
            x[i] = LB == 32 ? y * f : y;
        }
    };
    stage(std::integral_constant<int, 1>{});
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 4>{});
    stage(std::integral_constant<int, 8>{});
    stage(std::integral_constant<int, 16>{});
    stage(std::integral_constant<int, 32>{});
}

// Lloyd-Max row formats: index bits of a format (0: not one), and whether K
// is stored in it too.
constexpr int lm_bits(int f) {
    return (f == Q35_KV_TURBO4 || f == Q35_KV_BF16K_TURBO4V)   ? 4
           : (f == Q35_KV_TURBO3 || f == Q35_KV_BF16K_TURBO3V) ? 3
           : (f == Q35_KV_TURBO2 || f == Q35_KV_BF16K_TURBO2V) ? 2
                                                               : 0;
}
constexpr bool lm_k(int f) { return f == Q35_KV_TURBO4 || f == Q35_KV_TURBO3 || f == Q35_KV_TURBO2; }

// Quantises one group of 16 rotated values into the cache (2 * BITS bytes of
// indices at group index gi, one E4M3 scale byte) and writes the dequantised
// values, as stored, to out[16].
template <int BITS>
Q35_DEV void lm_append_group(const float v[16], const float* levels, const float* lut, uint8_t* data,
                             uint8_t* scales, size_t gi, float* out) {
    uint32_t idx[2];
    const uint32_t sc = lm_quantize16<BITS>(v, levels, idx);
    if constexpr (BITS == 4) {
        reinterpret_cast<uint2*>(data)[gi] = make_uint2(idx[0], idx[1]);
    } else if constexpr (BITS == 2) {
        reinterpret_cast<uint32_t*>(data)[gi] = idx[0];
    } else {  // 6 bytes, 2-byte aligned
        uint16_t* d16 = reinterpret_cast<uint16_t*>(data + gi * 6);
        d16[0] = (uint16_t)idx[0];
        d16[1] = (uint16_t)(idx[0] >> 16);
        d16[2] = (uint16_t)idx[1];
    }
    scales[gi] = (uint8_t)sc;
    const float s = e4m3x2_to_f32<false>(sc).x;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int b0 = BITS * e;  // bit offset in the group's stream (idx[0]: bits 0-31)
        const uint64_t w = ((uint64_t)idx[1] << 32) | idx[0];
        out[e] = s * lut[(uint32_t)(w >> b0) & ((1u << BITS) - 1u)];
    }
}

// Matrix-core tiles of a KV cache (head dimension 128 or 256; the attention
// kernels use them for the quantised formats): kMfRows rows of one kv head loaded by the decoders (thread
// t < 16 D/16, 4 rows of one group of 16 each: data and scale of K and of V)
// into registers, then decoded into LDS as f16: K row-major (KTS halves per
// row), V in quads of rows (element 16 i + e of a row at slot (D/16) e + i of
// its quad, position row % 4), so a quad's 4 values of one element form one
// 8-byte word and the decoders' stores spread over the banks.
typedef _Float16 tile_h8 __attribute__((ext_vector_type(8)));
typedef _Float16 tile_h4 __attribute__((ext_vector_type(4)));
typedef _Float16 tile_h2 __attribute__((ext_vector_type(2)));

template <int D, int F>
struct KvTile {
    static constexpr bool T8 = F == Q35_KV_TURBO8;
    static constexpr int LMB = lm_bits(F);
    static constexpr bool LMK = lm_k(F), LMV = LMB > 0;
    static constexpr int NG = D / 16;              // scale groups of 16 per row
    static constexpr int ND = 16 * NG;             // decoder threads
    static constexpr int KTS = D + 8;              // f16 per K row in LDS (8 of padding)
    static constexpr int VQS = 4 * (D + 16);       // f16 per quad of V rows (16 slots of padding)
    static constexpr int KT_HALVES = kMfRows * KTS, VT_HALVES = kMfRows / 4 * VQS;
    // bits per element of K and V data, bytes per group scale
    static constexpr uint32_t KBITS = T8 ? 8u : LMK ? (uint32_t)LMB : 16u;
    static constexpr uint32_t VBITS = T8 ? 8u : LMV ? (uint32_t)LMB : 16u;
    // words of data per row and group (E4M3 codes: 4; 4- and 3-bit indices: 2,
    // the 3-bit group's 6 bytes from the word boundary below them; 2-bit: 1;
    // bf16 keys: 8)
    static constexpr int KW = T8 ? 4 : LMK ? (LMB == 2 ? 1 : 2) : 8;
    static constexpr int VW = T8 ? 4 : LMV ? (LMB == 2 ? 1 : 2) : 8;
    // Lloyd-Max formats: the levels as f16, by pairs (4-bit: one index byte,
    // 256 pairs; 3-bit: 6 index bits, 64 pairs) or by fours (2-bit: one index
    // byte, 256 entries of two words); the first element in the low half
    static constexpr int PTW = LMV ? (LMB == 2 ? 512 : LMB == 4 ? 256 : 64) : 1;

    __amdgpu_buffer_rsrc_t rk, rv, rks, rvs;     // the sides from the first row of the range
    uint32_t krow, vrow, ksrow, vsrow;           // bytes per cache row of each side
    int gi, rq;                                  // decoder: group gi of the tile's rows 4 rq .. 4 rq + 3
    bool dec;
    uint32_t lsh;                                // 3-bit groups: bits below the group in its first word
    uint32_t kc4[4][KW], vc4[4][VW], ks4[4], vs4[4];

    Q35_DEV void init(int t, __amdgpu_buffer_rsrc_t k_, __amdgpu_buffer_rsrc_t v_, __amdgpu_buffer_rsrc_t ks_,
                      __amdgpu_buffer_rsrc_t vs_, uint32_t hkv) {
        rk = k_, rv = v_, rks = ks_, rvs = vs_;
        krow = hkv * D * KBITS / 8u;
        vrow = hkv * D * VBITS / 8u;
        ksrow = hkv * (uint32_t)NG * (T8 ? 2u : LMK ? 1u : 0u);
        vsrow = hkv * (uint32_t)NG * (T8 ? 2u : LMV ? 1u : 0u);
        gi = t % NG;
        rq = t / NG;
        dec = ND == kNT || t < ND;
        lsh = 8u * ((uint32_t)LMB * 2u * (uint32_t)gi & 3u);
    }

    template <int N>
    static Q35_DEV void load_words(__amdgpu_buffer_rsrc_t rr, uint32_t off, uint32_t* w) {
        if constexpr (N == 8) {
            const uint4 a0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, kAuxStream));
            const uint4 a1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, off + 16u, 0, kAuxStream));
            w[0] = a0.x, w[1] = a0.y, w[2] = a0.z, w[3] = a0.w, w[4] = a1.x, w[5] = a1.y, w[6] = a1.z, w[7] = a1.w;
        } else if constexpr (N == 4) {
            const uint4 a0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, kAuxStream));
            w[0] = a0.x, w[1] = a0.y, w[2] = a0.z, w[3] = a0.w;
        } else if constexpr (N == 2) {
            const uint2 a0 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rr, off, 0, kAuxStream));
            w[0] = a0.x, w[1] = a0.y;
        } else {
            w[0] = __builtin_amdgcn_raw_buffer_load_b32(rr, off, 0, kAuxStream);
        }
    }

    // the rows tr .. tr + kMfRows - 1 of the range into registers (rows past
    // the range read zero)
    Q35_DEV void load(uint32_t tr) {
        if (!dec) return;
        const uint32_t kg = (KBITS * 2u * (uint32_t)gi) & ~3u, vg = (VBITS * 2u * (uint32_t)gi) & ~3u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t r = tr + 4u * rq + u;
            load_words<KW>(rk, r * krow + kg, kc4[u]);
            if constexpr (T8) ks4[u] = __builtin_amdgcn_raw_buffer_load_b16(rks, r * ksrow + 2u * gi, 0, kAuxStream);
            else if constexpr (LMK) ks4[u] = __builtin_amdgcn_raw_buffer_load_b8(rks, r * ksrow + gi, 0, kAuxStream);
            else ks4[u] = 0;
            load_words<VW>(rv, r * vrow + vg, vc4[u]);
            if constexpr (T8) vs4[u] = __builtin_amdgcn_raw_buffer_load_b16(rvs, r * vsrow + 2u * gi, 0, kAuxStream);
            else if constexpr (LMV) vs4[u] = __builtin_amdgcn_raw_buffer_load_b8(rvs, r * vsrow + gi, 0, kAuxStream);
            else vs4[u] = 0;
        }
    }

    static Q35_DEV void fill_ptab(uint32_t* ptab, const float* levels, int t) {
        if constexpr (LMV) {
            auto lv16 = [&](uint32_t i) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)levels[i]); };
            if constexpr (LMB == 4) {
                ptab[t] = lv16(t & 15u) | (lv16((uint32_t)t >> 4) << 16);
            } else if constexpr (LMB == 3) {
                if (t < 64) ptab[t] = lv16(t & 7u) | (lv16((uint32_t)t >> 3) << 16);
            } else {
                ptab[2 * t] = lv16(t & 3u) | (lv16((t >> 2) & 3u) << 16);
                ptab[2 * t + 1] = lv16((t >> 4) & 3u) | (lv16((uint32_t)t >> 6) << 16);
            }
        }
    }

    // elements 4 c .. 4 c + 3 of a row's group of 16: E4M3 codes times the
    // bf16 group scale, or bf16 keys as they are
    template <int NW>
    static Q35_DEV void dec4(const uint32_t* w, uint32_t sbits, int c, float f[4]) {
        if constexpr (NW == 8) {
            f[0] = bf16_lo(w[2 * c]);
            f[1] = bf16_hi(w[2 * c]);
            f[2] = bf16_lo(w[2 * c + 1]);
            f[3] = bf16_hi(w[2 * c + 1]);
        } else {
            const float sc = bf16_to_f32(sbits & 0xFFFFu);
            const q35_float2_t p0 = e4m3x2_to_f32<false>(w[c]), p1 = e4m3x2_to_f32<true>(w[c]);
            f[0] = p0.x * sc;
            f[1] = p0.y * sc;
            f[2] = p1.x * sc;
            f[3] = p1.y * sc;
        }
    }

    // a row's group of 16 in a Lloyd-Max format as 8 f16 pairs (elements
    // 2 p, 2 p + 1 in word p): levels from the pair table times the E4M3 group
    // scale, in packed f16 (the level and the product each rounded to f16)
    Q35_DEV void dec_lm(const uint32_t* w, uint32_t sbyte, const uint32_t* ptab, uint32_t o[8]) const {
        const _Float16 sh = (_Float16)e4m3x2_to_f32<false>(sbyte & 0xFFu).x;  // exact: E4M3 is a subset of f16
        const tile_h2 s2 = {sh, sh};
        auto scaled = [&](uint32_t x) { return __builtin_bit_cast(uint32_t, __builtin_bit_cast(tile_h2, x) * s2); };
        if constexpr (LMB == 4) {
#pragma unroll
            for (int p = 0; p < 8; ++p) o[p] = scaled(ptab[(w[p / 4] >> (8 * (p % 4))) & 0xFFu]);
        } else if constexpr (LMB == 2) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint2 v = reinterpret_cast<const uint2*>(ptab)[(w[0] >> (8 * k)) & 0xFFu];
                o[2 * k] = scaled(v.x);
                o[2 * k + 1] = scaled(v.y);
            }
        } else {
            const uint64_t bits = (((uint64_t)w[1] << 32) | w[0]) >> lsh;
#pragma unroll
            for (int p = 0; p < 8; ++p) o[p] = scaled(ptab[(uint32_t)(bits >> (6 * p)) & 0x3Fu]);
        }
    }

    // The loaded rows into the LDS tiles.  Rows past the range (nrows): the
    // first tile decodes them (their loads read zero); a later tile leaves a
    // decoder's 4 rows as the previous tile left them when all 4 are past the
    // range (finite values, which the callers mask out of the scores and give
    // weight 0).
    Q35_DEV void store(uint32_t tr, uint32_t nrows, _Float16* kt, _Float16* vt, const uint32_t* ptab) const {
        if (!dec || (tr > 0 && tr + 4u * rq >= nrows)) return;
        // K: row by row, 16 elements as two 16-byte stores
        if constexpr (LMK) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t o[8];
                dec_lm(kc4[u], ks4[u], ptab, o);
                _Float16* kd = kt + (4 * rq + u) * KTS + 16 * gi;
                *reinterpret_cast<uint4*>(kd) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(kd + 8) = make_uint4(o[4], o[5], o[6], o[7]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float kf[16];
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) dec4<KW>(kc4[u], ks4[u], w4, kf + 4 * w4);
                tile_h8 k0, k1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    k0[e] = (_Float16)kf[e];
                    k1[e] = (_Float16)kf[8 + e];
                }
                _Float16* kd = kt + (4 * rq + u) * KTS + 16 * gi;
                *reinterpret_cast<tile_h8*>(kd) = k0;
                *reinterpret_cast<tile_h8*>(kd + 8) = k1;
            }
        }
        // V: one 8-byte store per element (its 4 rows)
        if constexpr (LMV) {
            uint32_t o[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) dec_lm(vc4[u], vs4[u], ptab, o[u]);
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                // low halves: element 2 p of rows 0..3; high halves: element 2 p + 1
                const uint2 lo = make_uint2(__builtin_amdgcn_perm(o[1][p], o[0][p], 0x05040100u),
                                            __builtin_amdgcn_perm(o[3][p], o[2][p], 0x05040100u));
                const uint2 hi = make_uint2(__builtin_amdgcn_perm(o[1][p], o[0][p], 0x07060302u),
                                            __builtin_amdgcn_perm(o[3][p], o[2][p], 0x07060302u));
                *reinterpret_cast<uint2*>(vt + rq * VQS + (NG * (2 * p) + gi) * 4) = lo;
                *reinterpret_cast<uint2*>(vt + rq * VQS + (NG * (2 * p + 1) + gi) * 4) = hi;
            }
        } else {
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                float vf[4][4];
#pragma unroll
                for (int u = 0; u < 4; ++u) dec4<VW>(vc4[u], vs4[u], w4, vf[u]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<tile_h4*>(vt + rq * VQS + (NG * (4 * w4 + e) + gi) * 4) =
                        tile_h4{(_Float16)vf[0][e], (_Float16)vf[1][e], (_Float16)vf[2][e], (_Float16)vf[3][e]};
            }
        }
    }
};

// T8: Turbo8 cache (E4M3 codes [capacity, Hkv, D] with bf16 scales per 16
// [capacity, Hkv, D/16], in the orthonormal Walsh-Hadamard basis of a head).
// The prologue also rotates the G query heads and the new k and v, the block
// holding `pos` quantises the rotated k and v in groups of 16, rows are
// dequantised in the loop, and the block's unnormalised per-head accumulators
// are rotated back before they are written (the transform is linear and its
// own inverse, so the merge is unchanged).
template <int D, int G, int F, bool MFT = false>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2))) void attn_partial_kernel(AttnArgs a) {
    static_assert(D <= kNT && D % 32 == 0, "one new-v element per thread; merge blocks of 32 dims");
    // row formats (F = a Q35_KV_* value): bf16; Turbo8 (K and V rotated, E4M3
    // with a bf16 scale per 16); the Lloyd-Max formats (LMB-bit codebook
    // indices with an E4M3 scale per 16, rotated): K and V for Turbo4/3/2, V
    // only (K bf16, not rotated) for Bf16K + Turbo4V/3V/2V
    constexpr bool T8 = F == Q35_KV_TURBO8;
    constexpr int LMB = lm_bits(F);
    constexpr bool LMK = lm_k(F);      // K in a Lloyd-Max format
    constexpr bool LMV = LMB > 0;      // V in a Lloyd-Max format
    constexpr bool ROTQK = T8 || LMK;  // query and key rotated
    constexpr bool ROTV = T8 || LMV;
    // MFT: the quantised formats at head dimension 128 or 256 through the
    // matrix cores (tiles of 64 rows decoded once into LDS as f16; see the
    // tile loop)
    constexpr bool MF = MFT;
    static_assert(!MF || ((T8 || LMV) && (D == 128 || D == 256)), "matrix-core tiles: quantised V at D 128 or 256");
    constexpr int NG = D / 16;              // scale groups of 16 per row
    constexpr int KTS = D + 8;              // MF: f16 per K row in LDS (8 of padding)
    constexpr int VQS = 4 * (D + 16);       // MF: f16 per quad of V rows in LDS (16 slots of padding)
    using Geo = AGeo<D>;
    constexpr int LPR = Geo::LPR, RPI = Geo::RPI, B = Geo::B;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int j = t % LPR;   // dim slice [8j, 8j+8)
    const int rs = t / LPR;  // row slot
    // MF: the kv heads of a chunk run on one XCD (block b on XCD b % 8), so the
    // group scales of a token, one 128-byte line for all heads, are fetched once
    // into that XCD's L2; the grid is padded to whole groups of 8 chunks
    uint32_t g = blockIdx.y, c = blockIdx.x;
    if constexpr (MF) {
        const uint32_t b = blockIdx.x + blockIdx.y * gridDim.x, q = b / 8u;
        c = 8u * (q / a.hkv) + b % 8u;
        g = q % a.hkv;
    }
    const uint32_t T = a.chunk;

    __shared__ __align__(16) float qs[(G + 1) * D];  // q heads of the group, then the new k
    __shared__ float vn[D];            // new v, bf16-rounded
    __shared__ float rsq[G + 1];
    __shared__ float2 rot[D / 2];      // (cos, sin) of pos * inv_freq[d], d < rotary / 2
    __shared__ float mls[RPI][2 * G];  // per-slot (max, sum)
    __shared__ float red[MF ? 1 : (G < 4 ? G : 4) * RPI * D];  // per-slot outputs of up to 4 heads
    __shared__ float ov[(ROTV && !MF) ? G * D : 1];  // rotated V: merged accumulators, rotated back
    // MF: the K tile, row-major, and the V tile in quads of rows: element
    // 16 i + e of row r (group i, element e of the group) at slot NG e + i of
    // quad r / 4, position r % 4, so a quad's 4 rows of one element are one
    // 8-byte word and the decoders' stores spread over the banks.  After the
    // loop the two hold the per-wave (max, sum) pairs and accumulators.
    __shared__ __align__(16) _Float16 kt_s[MF ? kMfRows * KTS : 1];
    __shared__ __align__(16) _Float16 vt_s[MF ? kMfRows / 4 * VQS : 1];
    __shared__ float lut[LMV ? 16 : 1];     // Lloyd-Max formats: the codebook levels
    __shared__ __align__(8) uint32_t ptab[MF ? KvTile<D, F>::PTW : 1];  // MF, Lloyd-Max formats: the level pair table
    __shared__ float bmax[G];               // sparse-V gate: running max of each head over the block

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
    // bytes of one token's row: K data, V data, K scales, V scales
    // bits per element of K and V data, bytes per group scale of K and V
    constexpr uint32_t KBITS = T8 ? 8u : LMK ? (uint32_t)LMB : 16u;
    constexpr uint32_t VBITS = T8 ? 8u : LMV ? (uint32_t)LMB : 16u;
    constexpr uint32_t KSB = T8 ? 2u : LMK ? 1u : 0u, VSB = T8 ? 2u : LMV ? 1u : 0u;
    const uint32_t krow_bytes = a.hkv * D * KBITS / 8u;
    const uint32_t vrow_bytes = a.hkv * D * VBITS / 8u;
    const uint32_t ksrow_bytes = a.hkv * (D / 16) * KSB;
    const uint32_t vsrow_bytes = a.hkv * (D / 16) * VSB;
    const uint32_t nrows = t1 - t0;

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
    const size_t srow0 = ((size_t)t0 * a.hkv + g) * (D / 16);
    const auto rk = rsrc(reinterpret_cast<const uint8_t*>(a.kc) + row0 * KBITS / 8, nrows * krow_bytes);
    const auto rv = rsrc(reinterpret_cast<const uint8_t*>(a.vc) + row0 * VBITS / 8, nrows * vrow_bytes);
    const auto rks = rsrc(reinterpret_cast<const uint8_t*>(a.ks) + srow0 * KSB, nrows * ksrow_bytes);
    const auto rvs = rsrc(reinterpret_cast<const uint8_t*>(a.vs) + srow0 * VSB, nrows * vsrow_bytes);
    // two batches in flight: the next batch's rows load while this one
    // computes (three, or smaller batches at higher occupancy, measured no
    // faster).  A lane holds 8 elements of a row.
    using KT = std::conditional_t<T8, uint2, std::conditional_t<LMK, uint32_t, uint4>>;
    using VT = std::conditional_t<T8, uint2, std::conditional_t<LMV, uint32_t, uint4>>;
    // a lane's 8 Lloyd-Max indices: LMB bytes at byte LMB * j of the row (3
    // bytes for 3-bit indices: two aligned words and a byte shift)
    auto load_lm = [&](__amdgpu_buffer_rsrc_t rr, uint32_t off) -> uint32_t {
        if constexpr (LMB == 4) {
            return __builtin_amdgcn_raw_buffer_load_b32(rr, off, 0, kAuxStream);
        } else if constexpr (LMB == 2) {
            return __builtin_amdgcn_raw_buffer_load_b16(rr, off, 0, kAuxStream);
        } else {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rr, off & ~3u, 0, kAuxStream);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(rr, (off & ~3u) + 4u, 0, kAuxStream);
            return __builtin_amdgcn_alignbyte(hi, lo, off & 3u) & 0xFFFFFFu;
        }
    };
    KT kr[2][kUnroll];
    VT vr[2][kUnroll];
    uint32_t ksr[2][kUnroll], vsr[2][kUnroll];  // the lane's group scale, raw bits
    auto load_batch = [&](KT (&kd)[kUnroll], VT (&vd)[kUnroll], uint32_t (&ksd)[kUnroll],
                          uint32_t (&vsd)[kUnroll], uint32_t tb) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI + rs;
            const bool live = tt < t1 && tt != (uint32_t)pos;
            const uint32_t r = live ? tt - t0 : nrows;  // past the end: loads return zero
            if constexpr (T8) {
                kd[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, r * krow_bytes + 8u * j, 0, kAuxStream));
                ksd[u] = __builtin_amdgcn_raw_buffer_load_b16(rks, r * ksrow_bytes + 2u * (j / 2), 0, kAuxStream);
            } else if constexpr (LMK) {
                kd[u] = load_lm(rk, r * krow_bytes + (uint32_t)LMB * j);
                ksd[u] = __builtin_amdgcn_raw_buffer_load_b8(rks, r * ksrow_bytes + (j / 2), 0, kAuxStream);
            } else {
                kd[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, r * krow_bytes + 16u * j, 0, kAuxStream));
                ksd[u] = 0;
            }
            if constexpr (T8) {
                vd[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, r * vrow_bytes + 8u * j, 0, kAuxStream));
                vsd[u] = __builtin_amdgcn_raw_buffer_load_b16(rvs, r * vsrow_bytes + 2u * (j / 2), 0, kAuxStream);
            } else if constexpr (LMV) {
                vd[u] = load_lm(rv, r * vrow_bytes + (uint32_t)LMB * j);
                vsd[u] = __builtin_amdgcn_raw_buffer_load_b8(rvs, r * vsrow_bytes + (j / 2), 0, kAuxStream);
            } else {
                vd[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, r * vrow_bytes + 16u * j, 0, kAuxStream));
                vsd[u] = 0;
            }
        }
    };
    // MF: the tile loader; the first tile's loads go out now
    [[maybe_unused]] KvTile<D, F> tio;
    if constexpr (MF) {
        tio.init(t, rk, rv, rks, rvs, a.hkv);
        tio.load(0);
    } else {
        load_batch(kr[0], vr[0], ksr[0], vsr[0], t0);
        load_batch(kr[1], vr[1], ksr[1], vsr[1], t0 + B);  // loads past the chunk return zero, unused
    }

    // ---------------- prologue: q heads of this group and the new k, v
#pragma unroll
    for (int r = 0; r < PQ; ++r)
        if (t + kNT * r < (G + 1) * D) qs[t + kNT * r] = qv[r];
    if (t < D) vn[t] = ROTV ? vnew : bf16_to_f32(f32_to_bf16(vnew));
    if constexpr (LMV)
        if (t < 16) lut[t] = a.lm_levels[t];
    if constexpr (MF && LMV) KvTile<D, F>::fill_ptab(ptab, a.lm_levels, t);
    if (t < G) bmax[t] = -INFINITY;
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
    uint16_t new_k = 0, new_v = 0;  // bf16 formats: this thread's element of the new row
    if constexpr (ROTQK) {
        if (has_new && a.k_norm_out)
            for (int d = t; d < D; d += kNT) a.k_norm_out[g * D + d] = qs[G * D + d];
        __syncthreads();  // the taps read qs before the rotation rewrites it
        // orthonormal Walsh-Hadamard transform of the G query heads, the new k and
        // the new v, one vector per wave
        for (int vi = wid; vi < G + 2; vi += kNT / 64) {
            float* xv = vi <= G ? qs + vi * D : vn;
            float x[D / 64];
#pragma unroll
            for (int i = 0; i < D / 64; ++i) x[i] = xv[lane * (D / 64) + i];
            wht_regs<D>(x, lane);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) xv[lane * (D / 64) + i] = x[i];
        }
        __syncthreads();
        if (has_new) {
            // quantising append: one thread per group of 16 of the rotated k or v;
            // the block then attends to the dequantised row, as stored
            if (t < 2 * (D / 16)) {
                const int side = t / (D / 16), grp = t % (D / 16);
                float* src = (side ? vn : qs + G * D) + 16 * grp;
                float v16[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) v16[e] = src[e];
                const size_t gi = ((size_t)pos * a.hkv + g) * (D / 16) + grp;  // group index in the cache
                if constexpr (T8) {
                    uint32_t cw[4];
                    const uint32_t sb = turbo8_quantize16(v16, cw);
                    uint8_t* dst = reinterpret_cast<uint8_t*>(side ? a.vc : a.kc) + gi * 16;
                    *reinterpret_cast<uint4*>(dst) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
                    (side ? a.vs : a.ks)[gi] = (uint16_t)sb;
                    const float sc = bf16_to_f32(sb);
#pragma unroll
                    for (int w4 = 0; w4 < 4; ++w4) {
                        const q35_float2_t lo = e4m3x2_to_f32<false>(cw[w4]), hi = e4m3x2_to_f32<true>(cw[w4]);
                        src[4 * w4] = lo.x * sc;
                        src[4 * w4 + 1] = lo.y * sc;
                        src[4 * w4 + 2] = hi.x * sc;
                        src[4 * w4 + 3] = hi.y * sc;
                    }
                } else {
                    lm_append_group<LMB>(v16, a.lm_levels, lut, reinterpret_cast<uint8_t*>(side ? a.vc : a.kc),
                                         reinterpret_cast<uint8_t*>(side ? a.vs : a.ks), gi, src);
                }
            }
            __syncthreads();
        }
    } else if (has_new) {
        if (a.k_norm_out)
            for (int d = t; d < D; d += kNT) a.k_norm_out[g * D + d] = qs[G * D + d];
        // the bf16 row is stored at the end of the kernel (the loop below attends
        // to it from LDS): stores issued here would be counted by every later
        // wait for the batch loads
        if (t < D) {
            new_k = (uint16_t)f32_to_bf16(qs[G * D + t]);
            new_v = (uint16_t)f32_to_bf16(vn[t]);  // vn is already bf16-exact
            qs[G * D + t] = bf16_to_f32(new_k);    // attend to the row as stored
        }
        if constexpr (LMV) {
            // the new v: rotated by wave 0, then quantised in groups of 16 (one
            // thread each); the block attends to the dequantised row, as stored
            if (wid == 0) {
                float x[D / 64];
#pragma unroll
                for (int i = 0; i < D / 64; ++i) x[i] = vn[lane * (D / 64) + i];
                wht_regs<D>(x, lane);
#pragma unroll
                for (int i = 0; i < D / 64; ++i) vn[lane * (D / 64) + i] = x[i];
            }
            __syncthreads();
            if (t < D / 16) {
                float v16[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) v16[e] = vn[16 * t + e];
                lm_append_group<LMB>(v16, a.lm_levels, lut, reinterpret_cast<uint8_t*>(a.vc),
                                     reinterpret_cast<uint8_t*>(a.vs), ((size_t)pos * a.hkv + g) * (D / 16) + t,
                                     vn + 16 * t);
            }
        }
        __syncthreads();
    }

    if constexpr (MF) {
        // ---------------- matrix-core tiles of kMfRows rows
        // Per tile: the decoders turn the codes into f16 values (code times the
        // group scale, rounded to nearest) in LDS, the row at `pos` from the
        // values as stored in LDS; the next tile's loads then go out.  Wave w
        // takes the tile's rows 16 w .. 16 w + 15: scores S (16 rows x 16
        // columns, column h = query head h, zero for h >= G) as 16x16x32 MFMAs
        // of K rows with q split into two f16 parts (high, then the rounding
        // rest: products carry about 22 bits of q), an online softmax per head,
        // and p V as 16x16x16 MFMAs with p in A (row = head, k = row of the
        // tile), whose lane layout is the scores' output layout, so p stays in
        // registers.  Lane L holds scores of rows 4 (L/16) + i, head L % 16,
        // and accumulators of heads 4 (L/16) + i, V slot 16 dt + L % 16.
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        typedef float f4 __attribute__((ext_vector_type(4)));
        const int hq = lane & 15, lq = lane >> 4;
        // the B operands of the scores: q of head hq (columns h >= G repeat
        // head h % G, never read back), elements 32 ks + 8 lq .. + 7, in f16
        h8 qb[D / 32];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) qb[ks][e] = (_Float16)qs[(hq & (G - 1)) * D + 32 * ks + 8 * lq + e];
        const float sscale = a.scale * kLog2e;  // scores in the base-2 exponent domain
        const float lt = a.sparse_v_log2;
        const uint32_t prow = (uint32_t)pos - t0;  // chunk-relative row of pos (out of range if not here)
        float m = -INFINITY, l = 0.f, mrun = -INFINITY;
        f4 O[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) O[dt] = f4{0.f, 0.f, 0.f, 0.f};

        auto compute_tile = [&](uint32_t tr) {
            if (tr + 16u * wid >= nrows) return;  // none of the wave's rows is in the chunk
            f4 S = {0.f, 0.f, 0.f, 0.f};
            const _Float16* ka = kt_s + (16 * wid + hq) * KTS + 8 * lq;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const h8 kv = *reinterpret_cast<const h8*>(ka + 32 * ks);
                S = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qb[ks], S, 0, 0, 0);
            }
            const uint32_t rb = tr + 16u * wid + 4u * lq;  // chunk-relative row of S[0]
            float s[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] = rb + i < nrows ? S[i] * sscale : -INFINITY;
            float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            mx = fmaxf(mx, lane_xor<16>(mx));
            mx = fmaxf(mx, lane_xor<32>(mx));  // the wave's max over the tile, head hq
            mrun = fmaxf(mrun, mx);
            // lazy rescale, as in the row-slot loop: only when some head's max
            // grows by more than 8 (weights stay below 2^8, also in f16)
            if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f) != 0) {
                const float mn = fmaxf(m, mx);
                const float corr = mn == -INFINITY ? 1.0f : exp2f(m - mn);
                m = mn;
                l *= corr;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ci = __shfl(corr, 4 * lq + i);  // head 4 lq + i lives in lane 4 lq + i
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt) O[dt][i] *= ci;
                }
            }
            // every row's weight enters the sum; its value only if s - mrun >= lt
            // (mrun: the exact running max of this wave's rows, never above
            // the block's final max, so a dropped row's weight relative to the
            // largest is below the threshold)
            const float mref = m == -INFINITY ? 0.f : m;
            h4 P;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = exp2f(s[i] - mref);
                l += p;
                P[i] = (_Float16)(s[i] - mrun >= lt ? p : 0.f);
            }
            const _Float16* vb = vt_s + (4 * wid + lq) * VQS + 4 * hq;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const h4 vv = *reinterpret_cast<const h4*>(vb + 64 * dt);
                O[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(P, vv, O[dt], 0, 0, 0);
            }
        };

        // the next tile's loads go out once this one is decoded (two tiles
        // in flight measured slower, also without spills)
        for (uint32_t tr = 0; tr < nrows; tr += kMfRows) {
            __syncthreads();  // the previous tile is read
            tio.store(tr, nrows, kt_s, vt_s, ptab);
            if (tr + kMfRows < nrows) tio.load(tr + kMfRows);
            if (has_new && prow - tr < (uint32_t)kMfRows) {
                // the row at pos, from its values as stored (its codes in memory
                // are being written by this block)
                __syncthreads();
                const uint32_t r = prow - tr;
                for (int d = t; d < D; d += kNT) {
                    const int sl = NG * (d % 16) + d / 16;  // V slot of element d
                    kt_s[r * KTS + d] = (_Float16)qs[G * D + d];
                    vt_s[(r / 4) * VQS + sl * 4 + r % 4] = (_Float16)vn[d];
                }
            }
            __syncthreads();
            compute_tile(tr);
        }

        // ---------------- merge the four waves, write this chunk's partials
        l += lane_xor<16>(l);
        l += lane_xor<32>(l);  // head hq's sum over the wave's rows
        static_assert(4 * G * 2 * sizeof(float) <= sizeof(kt_s) && 4 * G * D * sizeof(float) <= sizeof(vt_s),
                      "per-wave results fit the tiles");
        float* wml = reinterpret_cast<float*>(kt_s);  // [wave][head] (max, sum)
        float* wo = reinterpret_cast<float*>(vt_s);   // [wave][head][D] accumulators, scaled to the block max
        __syncthreads();  // every wave is done with the tiles
        if (lane < G) {
            wml[(wid * G + lane) * 2] = m;
            wml[(wid * G + lane) * 2 + 1] = l;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * lq + i;
            if (h < G) {
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < kNT / 64; ++w) M = fmaxf(M, wml[(w * G + h) * 2]);  // wave 0 has a row
                const float f = exp2f(wml[(wid * G + h) * 2] - M);
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) {
                    const int sl = 16 * dt + hq;              // V slot
                    const int d = 16 * (sl % NG) + sl / NG;   // its element
                    wo[(wid * G + h) * D + d] = O[dt][i] * f;
                }
            }
        }
        float* pacc = a.part_acc + ((size_t)g * a.max_chunks + c) * G * D;
        float* pml = a.part_ml + ((size_t)g * a.max_chunks + c) * 2 * G;
        if (t < G) {
            float M = -INFINITY, tot = 0.f;
#pragma unroll
            for (int w = 0; w < kNT / 64; ++w) M = fmaxf(M, wml[(w * G + t) * 2]);
#pragma unroll
            for (int w = 0; w < kNT / 64; ++w) tot = fmaf(exp2f(wml[(w * G + t) * 2] - M), wml[(w * G + t) * 2 + 1], tot);
            pml[2 * t] = M;
            pml[2 * t + 1] = tot;
        }
        __syncthreads();
        // each head's merged accumulator back to the original basis, one head per wave
        for (int h = wid; h < G; h += kNT / 64) {
            float x[D / 64];
#pragma unroll
            for (int i = 0; i < D / 64; ++i) {
                const int d = lane * (D / 64) + i;
                float o = 0.f;
#pragma unroll
                for (int w = 0; w < kNT / 64; ++w) o += wo[(w * G + h) * D + d];
                x[i] = o;
            }
            wht_regs<D>(x, lane);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) pacc[h * D + lane * (D / 64) + i] = x[i];
        }
        if constexpr (!ROTQK)  // bf16 keys: the new row's key, stored last as in the row-slot path
            if (has_new && t < D) a.kc[((size_t)pos * a.hkv + g) * D + t] = new_k;
        return;
    }

    // ---------------- batches of B rows: scores, online softmax, p V
    // Rows at `pos` are left out here (their loads read zero and their scores
    // are masked) and attended after the loop from LDS, as stored.
    // Lane slots: slot p is head p ^ hl (see row_reduce); after the reduction
    // the lane holds head hl's score, and m, l are that head's running max and
    // sum for the lane's row slot.
    const int hl = head_of_lane<G>(j);
    // bf16 keys: q as a bf16 pair (hi + lo, 16 significant bits) for the
    // two-element bf16 dot instruction, so the keys need no unpacking
    using Q2 = std::conditional_t<ROTQK, float, uint32_t>;
    constexpr int QN = ROTQK ? 8 : 4;
    Q2 qh[G][QN], ql[G][ROTQK ? 1 : 4];
#pragma unroll
    for (int p = 0; p < G; ++p) {
        const float* qp = qs + (p ^ hl) * D + 8 * j;
        if constexpr (ROTQK) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qh[p][e] = qp[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = qp[2 * e], x1 = qp[2 * e + 1];
                const uint32_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
                const uint32_t l0 = f32_to_bf16(x0 - bf16_to_f32(h0)), l1 = f32_to_bf16(x1 - bf16_to_f32(h1));
                qh[p][e] = h0 | (h1 << 16);
                ql[p][e] = l0 | (l1 << 16);
            }
        }
    }
    const float sscale = a.scale * kLog2e;  // scores in the base-2 exponent domain

    float m = -INFINITY, l = 0.f, acc[G][8];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;

    // 8 elements of a row: bf16 pairs, Turbo8 codes or Turbo4 levels (the
    // group scale is applied to the partial dot products and to the weights
    // instead)
    auto unpack_e4m3x8 = [](const uint2& w, float v[8]) {
        const q35_float2_t p0 = e4m3x2_to_f32<false>(w.x), p1 = e4m3x2_to_f32<true>(w.x);
        const q35_float2_t p2 = e4m3x2_to_f32<false>(w.y), p3 = e4m3x2_to_f32<true>(w.y);
        v[0] = p0.x;
        v[1] = p0.y;
        v[2] = p1.x;
        v[3] = p1.y;
        v[4] = p2.x;
        v[5] = p2.y;
        v[6] = p3.x;
        v[7] = p3.y;
    };
    auto unpack_v = [&](const VT& w, float v[8]) {
        if constexpr (T8) {
            unpack_e4m3x8(w, v);
        } else if constexpr (LMV) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = lut[(w >> (LMB * e)) & ((1u << LMB) - 1u)];
        } else {
            unpack8(w, v);
        }
    };
    auto vscale_of = [](uint32_t bits) {
        if constexpr (T8) return bf16_to_f32(bits & 0xFFFFu);
        else if constexpr (LMV) return e4m3x2_to_f32<false>(bits & 0xFFu).x;
        else return 1.0f;
    };
    // one row's score for head hl from the lane's 8 key elements
    auto score = [&](const KT& w, float kscale) {
        float d[G];
        if constexpr (ROTQK) {
            float kv[8];
            if constexpr (T8)
                unpack_e4m3x8(w, kv);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = lut[(w >> (LMB * e)) & ((1u << LMB) - 1u)];
#pragma unroll
            for (int p = 0; p < G; ++p) {
                float x = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) x = fmaf(qh[p][e], kv[e], x);
                d[p] = x * kscale;
            }
        } else {
            (void)kscale;
            const uint32_t kw[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int p = 0; p < G; ++p) {
                float x = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) x = bf16_dot2(qh[p][e], kw[e], x);
#pragma unroll
                for (int e = 0; e < 4; ++e) x = bf16_dot2(ql[p][e], kw[e], x);
                d[p] = x;
            }
        }
        return row_reduce<G, LPR>(d) * sscale;
    };
    // the appended row (fp32 values in LDS)
    auto score_f32 = [&](const float kv[8]) {
        float d[G];
#pragma unroll
        for (int p = 0; p < G; ++p) {
            const float* qp = qs + (p ^ hl) * D + 8 * j;
            float x = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) x = fmaf(qp[e], kv[e], x);
            d[p] = x;
        }
        return row_reduce<G, LPR>(d) * sscale;
    };
    // Online-softmax rescale towards the new max mx of head hl.  It runs only
    // when some lane's max grows by more than 8 (base 2; weights stay below
    // 2^8, the result is the same up to rounding), and then in every lane of
    // the wave: lanes of one head sum the same values in different orders, so
    // their maxima can differ in the last bit, and a per-lane decision could
    // leave two of them 2^8 apart.
    auto rescale_to = [&](float mx) {
        if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f) != 0) {
            const float mn = fmaxf(m, mx);
            const float corr = mn == -INFINITY ? 1.0f : exp2f(m - mn);
            m = mn;
            l *= corr;
#pragma unroll
            for (int p = 0; p < G; ++p) {
                const float cp = slot_bcast<G>(corr, p);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[p][e] *= cp;
            }
        }
    };
    auto add_value = [&](float pw, const float vv[8], float vscale) {
#pragma unroll
        for (int p = 0; p < G; ++p) {
            float pp = slot_bcast<G>(pw, p);
            if constexpr (ROTV) pp *= vscale;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[p][e] = fmaf(pp, vv[e], acc[p][e]);
        }
    };
    auto accumulate = [&](float pw, const float vv[8], float vscale) {
        l += pw;
        add_value(pw, vv, vscale);
    };
    // Sparse-V gate of the quantised formats: the weight of every row enters the
    // softmax sum, but a row's value is decoded and added only if some lane of
    // the wave has s - r >= log2(sparse_v) for it.  r is the larger of the
    // exact running maximum of the lane's row slot and the block's running
    // maximum of its head, which the slots share through an LDS atomic max
    // (m above is raised lazily and can lag by 8, which would weaken the gate
    // by up to 2^8; a slot alone sees too few rows of a chunk).  Every value r
    // can take is the maximum of rows already scored, never above the final
    // maximum, so a row left out here has exp(s - max s) < sparse_v: the
    // pages' rule would drop it too.
    constexpr bool GATE = T8 || LMV;
    const float lt = GATE ? a.sparse_v_log2 : -INFINITY;
    float mrun = -INFINITY;
    auto batch = [&](const KT (&kd)[kUnroll], const VT (&vd)[kUnroll], const uint32_t (&ksd)[kUnroll],
                     const uint32_t (&vsd)[kUnroll], uint32_t tb) {
        float s[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t tt = tb + u * RPI + rs;
            const float r = score(kd[u], T8    ? bf16_to_f32(ksd[u] & 0xFFFFu)
                                         : LMK ? e4m3x2_to_f32<false>(ksd[u] & 0xFFu).x
                                               : 1.0f);
            s[u] = (tt < t1 && tt != (uint32_t)pos) ? r : -INFINITY;
        }
        float mx = m;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, s[u]);
        rescale_to(mx);
        float gref = -INFINITY;
        if constexpr (GATE) {
            mrun = fmaxf(mrun, mx);
            if (j < G && mrun > -INFINITY)  // one lane per head of each row slot publishes
                __hip_atomic_fetch_max(&bmax[hl], mrun, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            gref = fmaxf(mrun, __hip_atomic_load(&bmax[hl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        }
        const float mref = m == -INFINITY ? 0.f : m;  // slot with no rows yet
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float pw = exp2f(s[u] - mref);
            l += pw;
            if (!GATE || __builtin_amdgcn_ballot_w64(s[u] - gref >= lt) != 0) {
                float vv[8];
                unpack_v(vd[u], vv);
                add_value(pw, vv, vscale_of(vsd[u]));
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
    if (has_new) {
        // the appended row, as stored (dequantised for Turbo8), in row slot 0
        float kv[8], vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kv[e] = qs[G * D + 8 * j + e];
            vv[e] = vn[8 * j + e];
        }
        const float r = score_f32(kv);
        const float sn = rs == 0 ? r : -INFINITY;
        rescale_to(fmaxf(m, sn));
        const float mref = m == -INFINITY ? 0.f : m;
        accumulate(exp2f(sn - mref), vv, 1.0f);
    }

    // ---------------- merge the row slots, write this chunk's partials
    if (j < G) {  // one lane per head in each row slot
        mls[rs][2 * hl] = m;
        mls[rs][2 * hl + 1] = l;
    }
    __syncthreads();
    float* pacc = a.part_acc + ((size_t)g * a.max_chunks + c) * G * D;
    float* pml = a.part_ml + ((size_t)g * a.max_chunks + c) * 2 * G;
    if (t < G) {
        float M = -INFINITY, tot = 0.f;
        for (int r = 0; r < RPI; ++r) M = fmaxf(M, mls[r][2 * t]);  // slot 0 always has a row
        for (int r = 0; r < RPI; ++r) tot = fmaf(exp2f(mls[r][2 * t] - M), mls[r][2 * t + 1], tot);
        pml[2 * t] = M;
        pml[2 * t + 1] = tot;
    }
    // heads in rounds of HM: each slot writes its weighted accumulators, then
    // every thread sums the slots for HM * D / 256 outputs
    constexpr int HM = G < 4 ? G : 4;
#pragma unroll
    for (int h0 = 0; h0 < G; h0 += HM) {
#pragma unroll
        for (int p = 0; p < G; ++p) {
            const int h = p ^ hl;
            if (h >= h0 && h < h0 + HM) {
                float M = -INFINITY;
                for (int r = 0; r < RPI; ++r) M = fmaxf(M, mls[r][2 * h]);
                const float w = exp2f(mls[rs][2 * h] - M);
                float* dst = red + ((h - h0) * RPI + rs) * D + 8 * j;
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[e] = acc[p][e] * w;
            }
        }
        __syncthreads();
        for (int e = t; e < HM * D; e += kNT) {
            const int hh = e / D, d = e % D;
            float o = 0.f;
#pragma unroll 8
            for (int r = 0; r < RPI; ++r) o += red[(hh * RPI + r) * D + d];
            if constexpr (ROTV)
                ov[(h0 + hh) * D + d] = o;
            else
                pacc[(h0 + hh) * D + d] = o;
        }
        __syncthreads();
    }
    if constexpr (ROTV) {
        // each head's merged accumulator back to the original basis (the
        // orthonormal transform is its own inverse; the merge is linear), one
        // head per wave
        for (int vi = wid; vi < G; vi += kNT / 64) {
            float x[D / 64];
#pragma unroll
            for (int i = 0; i < D / 64; ++i) x[i] = ov[vi * D + lane * (D / 64) + i];
            wht_regs<D>(x, lane);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) pacc[vi * D + lane * (D / 64) + i] = x[i];
        }
    }
    if constexpr (!ROTQK) {
        if (has_new && t < D) {
            const size_t row = ((size_t)pos * a.hkv + g) * D;
            a.kc[row + t] = new_k;
            if constexpr (!LMV) a.vc[row + t] = new_v;
        }
    }
}

// grid (Hq, D/32); thread t: dim d0 + t % 32, chunk lane t / 32.  Each thread
// issues its first kPrefetch partial loads before the weights are known, so the
// partials and the (max, sum) pairs arrive together; the pairs are read from
// memory once (kept in LDS for the weights) and the gate is requested with
// them, so no load waits on an earlier result.
constexpr int kMergeDims = 32;
constexpr int kMergeLanes = kNT / kMergeDims;
constexpr int kPrefetch = 16;

template <int D, int G>
__global__ __launch_bounds__(kNT) void attn_merge_kernel(AttnArgs a) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int dl = t % kMergeDims, cl = t / kMergeDims;
    const uint32_t h = blockIdx.x, g = h / G, i = h % G;
    const uint32_t d = blockIdx.y * kMergeDims + dl;
    extern __shared__ float wsh[];  // [max_chunks] chunk maxima, then weights; then [max_chunks] sums
    __shared__ float red[kNT];
    __shared__ float stat[kNT / 64];

    const int32_t pos = attn_pos(a);
    if (pos < 0 || (uint32_t)pos >= a.capacity) {
        // no attention for a position outside the cache: a zero output, and the
        // caller's status word says so (the partial kernel wrote nothing)
        if (cl == 0) {
            a.gated_attn[h * D + d] = 0.f;
            if (a.attn_out) a.attn_out[h * D + d] = 0.f;
        }
        if (a.status && blockIdx.x == 0 && blockIdx.y == 0 && t == 0)
            __hip_atomic_fetch_or(a.status, Q35_STATUS_POS_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
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
    float* lsh = wsh + a.max_chunks;

    float mx = -INFINITY;
    for (uint32_t cc = t; cc < nch; cc += kNT) {
        const float2 ml = *reinterpret_cast<const float2*>(pml + cc * 2 * G);
        wsh[cc] = ml.x;
        lsh[cc] = ml.y;
        mx = fmaxf(mx, ml.x);
    }
    const float gate = a.q_full[(size_t)h * 2 * D + D + d];
    mx = wave_max(mx);
    if (lane == 0) red[wid] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < kNT / 64; ++w) M = fmaxf(M, red[w]);
    float tot = 0.f;
    for (uint32_t cc = t; cc < nch; cc += kNT) {  // this thread's own chunks: no barrier needed
        const float w = exp2f(wsh[cc] - M);
        wsh[cc] = w;
        tot = fmaf(w, lsh[cc], tot);
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
        a.gated_attn[h * D + d] = o * sigmoidf_(gate);
    }
}

// The quantised formats at head dimension 128 or 256 take the matrix-core
// tiles once a chunk holds a whole tile.
template <int D, int F>
constexpr bool kHasMfTiles = (F == Q35_KV_TURBO8 || lm_bits(F) > 0) && (D == 128 || D == 256);

template <int D, int G, int F>
void launch_partial(const AttnArgs& a, uint32_t grid_chunks, hipStream_t stream) {
    if constexpr (kHasMfTiles<D, F>) {
        if (a.chunk >= (uint32_t)kMfRows) {
            hipLaunchKernelGGL((attn_partial_kernel<D, G, F, true>), dim3((grid_chunks + 7) / 8 * 8, a.hkv), dim3(kNT),
                               0, stream, a);
            return;
        }
    }
    hipLaunchKernelGGL((attn_partial_kernel<D, G, F>), dim3(grid_chunks, a.hkv), dim3(kNT), 0, stream, a);
}

#define Q35_KV_FORMATS(X)                                                                          \
    X(Q35_KV_BF16) X(Q35_KV_TURBO8) X(Q35_KV_TURBO4) X(Q35_KV_TURBO3) X(Q35_KV_TURBO2)             \
    X(Q35_KV_BF16K_TURBO4V) X(Q35_KV_BF16K_TURBO3V) X(Q35_KV_BF16K_TURBO2V)

template <int D, int G>
hipError_t launch_t(const AttnArgs& a, uint32_t grid_chunks, uint32_t fmt, hipStream_t stream) {
    bool known = false;
#define X(FF)                                                   \
    if (fmt == FF) {                                            \
        launch_partial<D, G, FF>(a, grid_chunks, stream);       \
        known = true;                                           \
    }
    Q35_KV_FORMATS(X)
#undef X
    if (!known) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_merge_kernel<D, G>), dim3(a.hq, D / kMergeDims), dim3(kNT),
                       (size_t)a.max_chunks * 2 * sizeof(float), stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prompt into a quantised cache (head dimension 128 or 256), two launches in
// place of the decode steps of every prompt token: each token's row is
// appended as the decode step would append it, then every token attends to the
// rows [0, its position] as stored, so each sees the earlier prompt rows
// quantised, as in token order.
//
// pfq_prep_kernel   grid (token, kv head g), 256 threads: the decode step's
//     prologue for one token: RMSNorm and RoPE of the G query heads and the
//     key, the Walsh-Hadamard rotation (query and key for the formats with
//     rotated keys, the value always), the query heads as f16 into qh, the row
//     quantised in groups of 16 into the cache (bf16 keys stored as bf16).
template <int D, int G, int F>
__global__ __launch_bounds__(kNT) void pfq_prep_kernel(PfQuantAttnArgs a) {
    constexpr bool T8 = F == Q35_KV_TURBO8;
    constexpr int LMB = lm_bits(F);
    constexpr bool ROTQK = T8 || lm_k(F);
    static_assert(T8 || LMB > 0, "quantised value rows");
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const uint32_t tok = blockIdx.x, g = blockIdx.y;
    const uint32_t pos = a.cache_pos + tok;
    __shared__ float qs[(G + 1) * D];  // q heads of the group, then the key
    __shared__ float vn[D];
    __shared__ float rsq[G + 1];
    __shared__ float2 rot[D / 2];
    __shared__ float lut[16];
    const float* qf = a.q_full + (size_t)tok * a.hq * 2u * D;
    const float* kf = a.k + (size_t)tok * a.hkv * D;
    const float* vf = a.v + (size_t)tok * a.hkv * D;
    for (int e = t; e < (G + 1) * D; e += kNT) {
        const int i = e / D, d = e % D;
        qs[e] = i < G ? qf[(size_t)(g * G + i) * 2 * D + d] : kf[g * D + d];
    }
    for (int d = t; d < D; d += kNT) vn[d] = vf[g * D + d];
    if constexpr (LMB > 0)
        if (t < 16) lut[t] = a.lm_levels[t];
    if (t < (int)a.rotary / 2) {
        float sn, cs;
        sincosf((float)pos * a.inv_freq[t], &sn, &cs);
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
    for (int e = t; e < (G + 1) * D; e += kNT) {
        const int i = e / D, d = e % D;
        qs[e] = qs[e] * rsq[i] * bf16_to_f32(i < G ? a.q_norm[d] : a.k_norm[d]);
    }
    __syncthreads();
    const int half = (int)a.rotary / 2;
    for (int e = t; e < (G + 1) * half; e += kNT) {
        const int i = e / half, d = e % half;
        const float cs = rot[d].x, sn = rot[d].y;
        const float x1 = qs[i * D + d], x2 = qs[i * D + d + half];
        qs[i * D + d] = x1 * cs - x2 * sn;
        qs[i * D + d + half] = x2 * cs + x1 * sn;
    }
    __syncthreads();
    // rotations, one vector per wave: the G query heads and the key (rotated
    // keys only), then the value
    for (int vi = (ROTQK ? 0 : G + 1) + wid; vi < G + 2; vi += kNT / 64) {
        float* xv = vi <= G ? qs + vi * D : vn;
        float x[D / 64];
#pragma unroll
        for (int i = 0; i < D / 64; ++i) x[i] = xv[lane * (D / 64) + i];
        wht_regs<D>(x, lane);
#pragma unroll
        for (int i = 0; i < D / 64; ++i) xv[lane * (D / 64) + i] = x[i];
    }
    __syncthreads();
    for (int e = t; e < G * D; e += kNT)
        a.qh[((size_t)tok * a.hq + (size_t)g * G) * D + e] = __builtin_bit_cast(uint16_t, (_Float16)qs[e]);
    const size_t gi0 = ((size_t)pos * a.hkv + g) * (D / 16);  // group index of the row in the cache
    if constexpr (!ROTQK)
        if (t < D) static_cast<uint16_t*>(a.kc)[((size_t)pos * a.hkv + g) * D + t] = (uint16_t)f32_to_bf16(qs[G * D + t]);
    constexpr int SIDES = ROTQK ? 2 : 1;  // groups of the key (rotated formats), then of the value
    if (t < SIDES * (D / 16)) {
        const int side = SIDES == 2 ? t / (D / 16) : 1, grp = t % (D / 16);
        const float* src = (side ? vn : qs + G * D) + 16 * grp;
        float v16[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v16[e] = src[e];
        if constexpr (T8) {
            uint32_t cw[4];
            const uint32_t sb = turbo8_quantize16(v16, cw);
            uint8_t* dst = static_cast<uint8_t*>(side ? a.vc : a.kc) + (gi0 + grp) * 16;
            *reinterpret_cast<uint4*>(dst) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
            static_cast<uint16_t*>(side ? a.vs : a.ks)[gi0 + grp] = (uint16_t)sb;
        } else {
            float out16[16];
            lm_append_group<LMB>(v16, a.lm_levels, lut, static_cast<uint8_t*>(side ? a.vc : a.kc),
                                 static_cast<uint8_t*>(side ? a.vs : a.ks), gi0 + grp, out16);
        }
    }
}

// pfq_flash_kernel   grid (block of 64/G prompt tokens, kv head g), 256
//     threads: causal attention of the block's tokens over the cache rows as
//     stored, in the matrix-core tiles of the decode kernel (KvTile): each
//     64-row tile is decoded once for all the block's tokens.  Wave w owns
//     the 16 (token, head) columns 16 w .. 16 w + 15 (token 16 w / G + c / G,
//     head c % G) across all tiles: scores S^T (16 rows x 16 columns) as
//     16x16x32 f16 MFMAs of K rows against the f16 query heads, an online
//     softmax per column (lazy rescale by 8 in base 2, the sparse-V gate
//     against the column's exact running maximum), p V as 16x16x16 MFMAs with
//     p in registers.  Then each column is divided by its sum, rotated back
//     and multiplied by the sigmoid of its gate into ga (f16).  Blocks of the
//     last tokens (the most rows) start first.
template <int D, int G, int F>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2))) void pfq_flash_kernel(PfQuantAttnArgs a) {
    using Tile = KvTile<D, F>;
    constexpr int QB = 64 / G;  // prompt tokens per block
    constexpr int NG = D / 16, KTS = Tile::KTS, VQS = Tile::VQS;
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int hq = lane & 15, lq = lane >> 4;
    const uint32_t g = blockIdx.y;
    const uint32_t tq0 = (gridDim.x - 1 - blockIdx.x) * QB;
    const uint32_t tq1 = min(tq0 + (uint32_t)QB, a.T);
    const uint32_t kend = a.cache_pos + tq1;  // rows [0, kend) are visible to some token of the block

    // the K tile, then the V tile; after the loop the per-wave outputs
    __shared__ __align__(16) _Float16 tiles[Tile::KT_HALVES + Tile::VT_HALVES];
    __shared__ __align__(8) uint32_t ptab[Tile::PTW];
    _Float16* kt_s = tiles;
    _Float16* vt_s = tiles + Tile::KT_HALVES;

    // head g's sides from cache row 0; each tile's loads go through buffer
    // resources based at the tile's first row (32-bit offsets within 64 rows
    // for any cache length), over the tile's rows below kend
    constexpr uint32_t SB = Tile::T8 ? 2u : 1u;  // bytes per group scale
    const uint8_t* kb0 = static_cast<const uint8_t*>(a.kc) + (size_t)g * D * Tile::KBITS / 8;
    const uint8_t* vb0 = static_cast<const uint8_t*>(a.vc) + (size_t)g * D * Tile::VBITS / 8;
    const uint8_t* ksb0 = Tile::T8 || Tile::LMK ? static_cast<const uint8_t*>(a.ks) + (size_t)g * NG * SB : nullptr;
    const uint8_t* vsb0 = static_cast<const uint8_t*>(a.vs) + (size_t)g * NG * SB;
    Tile tio;
    tio.init(t, rsrc(kb0, 0u), rsrc(vb0, 0u), rsrc(vsb0, 0u), rsrc(vsb0, 0u), a.hkv);
    auto load_from = [&](uint32_t tr) {
        const uint32_t n = min(kend - tr, (uint32_t)kMfRows);
        tio.rk = rsrc(kb0 + (size_t)tr * tio.krow, n * tio.krow);
        tio.rv = rsrc(vb0 + (size_t)tr * tio.vrow, n * tio.vrow);
        if constexpr (Tile::T8 || Tile::LMK) tio.rks = rsrc(ksb0 + (size_t)tr * tio.ksrow, n * tio.ksrow);
        tio.rvs = rsrc(vsb0 + (size_t)tr * tio.vsrow, n * tio.vsrow);
        tio.load(0);
    };
    load_from(0);
    if constexpr (Tile::LMV) Tile::fill_ptab(ptab, a.lm_levels, t);

    // this lane's column: prompt token tok, head hh of the group
    const int col = 16 * wid + hq;
    const uint32_t tok = tq0 + (uint32_t)(col / G);
    const int hh = col % G;
    const bool live = tok < a.T;
    const uint32_t last = a.cache_pos + (live ? tok : tq1 - 1);  // the column's last visible row
    h8 qb[D / 32];
    {
        const uint16_t* qp = a.qh + ((size_t)(live ? tok : tq0) * a.hq + (size_t)g * G + hh) * D + 8 * lq;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) qb[ks] = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(qp + 32 * ks));
    }
    const float sscale = a.scale * kLog2e;
    const float lt = a.sparse_v_log2;
    float m = -INFINITY, l = 0.f, mrun = -INFINITY;
    f4 O[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) O[dt] = f4{0.f, 0.f, 0.f, 0.f};

    for (uint32_t tr = 0; tr < kend; tr += kMfRows) {
        __syncthreads();  // the previous tile is read
        tio.store(tr, kend, kt_s, vt_s, ptab);
        if (tr + kMfRows < kend) load_from(tr + kMfRows);
        __syncthreads();
        // scores of the tile's 4 sub-tiles of 16 rows (lane: rows 4 lq + i of each)
        float s[4][4];
        float mx = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            f4 S = {0.f, 0.f, 0.f, 0.f};
            if (tr + 16u * sub < kend) {
                const _Float16* ka = kt_s + (16 * sub + hq) * KTS + 8 * lq;
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
                    S = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const h8*>(ka + 32 * ks), qb[ks], S, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t r = tr + 16u * sub + 4u * lq + i;
                s[sub][i] = r <= last ? S[i] * sscale : -INFINITY;
                mx = fmaxf(mx, s[sub][i]);
            }
        }
        mx = fmaxf(mx, lane_xor<16>(mx));
        mx = fmaxf(mx, lane_xor<32>(mx));  // the column's max over the tile
        mrun = fmaxf(mrun, mx);
        if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f) != 0) {
            const float mn = fmaxf(m, mx);
            const float corr = mn == -INFINITY ? 1.0f : exp2f(m - mn);
            m = mn;
            l *= corr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ci = __shfl(corr, 4 * lq + i);  // column 4 lq + i lives in lane 4 lq + i
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) O[dt][i] *= ci;
            }
        }
        const float mref = m == -INFINITY ? 0.f : m;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
            if (tr + 16u * sub >= kend) break;
            h4 P;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = exp2f(s[sub][i] - mref);
                l += p;
                P[i] = (_Float16)(s[sub][i] - mrun >= lt ? p : 0.f);
            }
            const _Float16* vb = vt_s + (4 * sub + lq) * VQS + 4 * hq;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                O[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(P, *reinterpret_cast<const h4*>(vb + 64 * dt), O[dt], 0, 0, 0);
        }
    }

    // ---------------- each column divided by its sum, rotated back, gated
    l += lane_xor<16>(l);
    l += lane_xor<32>(l);  // column hq's sum
    static_assert(4 * 16 * D * sizeof(float) <= sizeof(tiles), "per-wave outputs fit the tiles");
    float* wo = reinterpret_cast<float*>(tiles) + wid * 16 * D;  // [column][D]
    __syncthreads();  // every wave is done with the tiles
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float inv = 1.0f / __shfl(l, 4 * lq + i);  // column 4 lq + i
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const int sl = 16 * dt + hq;
            wo[(4 * lq + i) * D + 16 * (sl % NG) + sl / NG] = O[dt][i] * inv;
        }
    }
    __syncthreads();
    for (int c = 0; c < 16; ++c) {
        const int cc = 16 * wid + c;
        const uint32_t tc = tq0 + (uint32_t)(cc / G);
        if (tc >= a.T) break;
        const uint32_t h = g * G + (uint32_t)(cc % G);
        float x[D / 64];
#pragma unroll
        for (int i = 0; i < D / 64; ++i) x[i] = wo[c * D + lane * (D / 64) + i];
        wht_regs<D>(x, lane);
        const float* gate = a.q_full + ((size_t)tc * a.hq + h) * 2 * D + D;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const int d = lane * (D / 64) + i;
            a.ga[((size_t)tc * a.hq + h) * D + d] = __builtin_bit_cast(uint16_t, (_Float16)(x[i] * sigmoidf_(gate[d])));
        }
    }
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

// Lloyd-Max group quantiser over a plain vector (kernel-level export): one
// thread per group of 16; the levels go to LDS for the dequantised copy the
// append path also writes (not kept here).
template <int BITS>
__global__ __launch_bounds__(256) void lm_quantize_kernel(const float* x, uint32_t groups, LmLevels lv,
                                                          uint8_t* packed, uint8_t* scales) {
    __shared__ float lut[16];
    if (threadIdx.x < 16) lut[threadIdx.x] = lv.v[threadIdx.x];
    __syncthreads();
    const uint32_t gi = blockIdx.x * 256u + threadIdx.x;
    if (gi >= groups) return;
    float v[16], out[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = x[16u * gi + e];
    lm_append_group<BITS>(v, lv.v, lut, packed, scales, gi, out);
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
                       uint32_t kv_dtype, hipStream_t stream) {
#define X(DD, GG) \
    if (head_dim == DD && group == GG) return launch_t<DD, GG>(a, grid_chunks, kv_dtype, stream);
    Q35_ATTN_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

template <int D, int G>
const void* partial_ptr(uint32_t fmt, bool tiles) {
    if (tiles) {
#define X(FF)                                 \
    if constexpr (kHasMfTiles<D, FF>)         \
        if (fmt == FF) return (const void*)&attn_partial_kernel<D, G, FF, true>;
        Q35_KV_FORMATS(X)
#undef X
        return nullptr;
    }
#define X(FF) \
    if (fmt == FF) return (const void*)&attn_partial_kernel<D, G, FF>;
    Q35_KV_FORMATS(X)
#undef X
    return nullptr;
}

const void* attn_kernel_ptr(uint32_t head_dim, uint32_t group, uint32_t kv_dtype, bool tiles) {
#define X(DD, GG) \
    if (head_dim == DD && group == GG) return partial_ptr<DD, GG>(kv_dtype, tiles);
    Q35_ATTN_SHAPES(X)
#undef X
    return nullptr;
}

namespace {
template <int D, int G, int F>
void pfq_launch(const PfQuantAttnArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((pfq_prep_kernel<D, G, F>), dim3(a.T, a.hkv), dim3(kNT), 0, stream, a);
    constexpr uint32_t QB = 64 / G;
    hipLaunchKernelGGL((pfq_flash_kernel<D, G, F>), dim3((a.T + QB - 1) / QB, a.hkv), dim3(kNT), 0, stream, a);
}
#define Q35_PFQ_SHAPES(X) X(128, 1) X(128, 2) X(128, 4) X(128, 8) X(256, 1) X(256, 2) X(256, 4) X(256, 8)
#define Q35_QUANT_FORMATS(X)                                                                       \
    X(Q35_KV_TURBO8) X(Q35_KV_TURBO4) X(Q35_KV_TURBO3) X(Q35_KV_TURBO2) X(Q35_KV_BF16K_TURBO4V) \
    X(Q35_KV_BF16K_TURBO3V) X(Q35_KV_BF16K_TURBO2V)
}  // namespace

bool pf_quant_attn_supported(uint32_t head_dim, uint32_t group, uint32_t kv_dtype) {
    bool fmt = false;
#define X(FF) fmt |= kv_dtype == FF;
    Q35_QUANT_FORMATS(X)
#undef X
#define X(DD, GG) if (fmt && head_dim == DD && group == GG) return true;
    Q35_PFQ_SHAPES(X)
#undef X
    return false;
}

hipError_t pf_quant_attn_launch(uint32_t head_dim, uint32_t group, uint32_t kv_dtype, const PfQuantAttnArgs& a,
                                hipStream_t stream) {
    if (!pf_quant_attn_supported(head_dim, group, kv_dtype)) return hipErrorInvalidValue;
    if (a.T == 0) return hipSuccess;
#define XF(DD, GG, FF) \
    if (head_dim == DD && group == GG && kv_dtype == FF) pfq_launch<DD, GG, FF>(a, stream);
#define X(DD, GG)                   \
    XF(DD, GG, Q35_KV_TURBO8)         \
    XF(DD, GG, Q35_KV_TURBO4)         \
    XF(DD, GG, Q35_KV_TURBO3)         \
    XF(DD, GG, Q35_KV_TURBO2)         \
    XF(DD, GG, Q35_KV_BF16K_TURBO4V)  \
    XF(DD, GG, Q35_KV_BF16K_TURBO3V)  \
    XF(DD, GG, Q35_KV_BF16K_TURBO2V)
    Q35_PFQ_SHAPES(X)
#undef X
#undef XF
    return hipGetLastError();
}

const void* pf_quant_kernel_ptr(uint32_t head_dim, uint32_t group, uint32_t kv_dtype, bool flash) {
#define XF(DD, GG, FF)                                                                           \
    if (head_dim == DD && group == GG && kv_dtype == FF)                                          \
        return flash ? (const void*)&pfq_flash_kernel<DD, GG, FF> : (const void*)&pfq_prep_kernel<DD, GG, FF>;
#define X(DD, GG)                   \
    XF(DD, GG, Q35_KV_TURBO8)         \
    XF(DD, GG, Q35_KV_TURBO4)         \
    XF(DD, GG, Q35_KV_TURBO3)         \
    XF(DD, GG, Q35_KV_TURBO2)         \
    XF(DD, GG, Q35_KV_BF16K_TURBO4V)  \
    XF(DD, GG, Q35_KV_BF16K_TURBO3V)  \
    XF(DD, GG, Q35_KV_BF16K_TURBO2V)
    Q35_PFQ_SHAPES(X)
#undef X
#undef XF
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

hipError_t lm_quantize_launch(uint32_t bits, const float* x, uint32_t n, const LmLevels& levels, uint8_t* packed,
                              uint8_t* scales, hipStream_t stream) {
    const uint32_t groups = n / 16;
    if (groups == 0) return hipSuccess;
    const dim3 grid((groups + 255) / 256), block(256);
    if (bits == 4)
        hipLaunchKernelGGL(lm_quantize_kernel<4>, grid, block, 0, stream, x, groups, levels, packed, scales);
    else if (bits == 3)
        hipLaunchKernelGGL(lm_quantize_kernel<3>, grid, block, 0, stream, x, groups, levels, packed, scales);
    else if (bits == 2)
        hipLaunchKernelGGL(lm_quantize_kernel<2>, grid, block, 0, stream, x, groups, levels, packed, scales);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t e4m3_table_launch(float* out256, hipStream_t stream) {
    hipLaunchKernelGGL(e4m3_table_kernel, dim3(1), dim3(64), 0, stream, out256);
    return hipGetLastError();
}

}  // namespace q35
