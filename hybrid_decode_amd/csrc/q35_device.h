// Device helpers shared by the q35decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define Q35_DEV __device__ __forceinline__

namespace q35 {

constexpr int kWave = 64;

// ------------------------------------------------------------------ dtypes

Q35_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
Q35_DEV float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
Q35_DEV float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 bits; NaN -> canonical quiet NaN.
Q35_DEV uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Read element i of an activation vector (bf16 bits or fp32).
Q35_DEV float load_act(const void* p, uint32_t i, bool is_f32) {
    return is_f32 ? static_cast<const float*>(p)[i]
                  : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

Q35_DEV void store_act(void* p, uint32_t i, float v, bool is_f32) {
    if (is_f32)
        static_cast<float*>(p)[i] = v;
    else
        static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16(v));
}

typedef __bf16 q35_bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c over two bf16 pairs (exact products, fp32 sum).
Q35_DEV float bf16_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(q35_bf16x2_t, a),
                                           __builtin_bit_cast(q35_bf16x2_t, b), c, false);
}

// ------------------------------------------------------------------ FP8 E4M3 (OCP "fn")

// fp32 -> E4M3 code: round to nearest-even, saturating to +-448 (the largest
// finite magnitude; infinities and NaN saturate too).  Below the smallest
// normal 2^-6 the step is 2^-9; a subnormal that rounds up to 8 steps lands on
// the smallest normal, whose code follows on.  Normals round the fp32 mantissa
// to three bits; a carry moves into the exponent field.
Q35_DEV uint32_t e4m3_encode(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    uint32_t code;
    if (!(a < 448.0f)) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        const uint32_t ab = __float_as_uint(a);
        const uint32_t e = (ab >> 23) - 120u;  // exponent field: unbiased + 7
        const uint32_t m = ab & 0x7FFFFFu;
        const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;
        code = (e << 3) + r;
    }
    return code | sign;
}

typedef float q35_float2_t __attribute__((ext_vector_type(2)));

// Two E4M3 codes (bytes 0-1 of w, or 2-3 when HI) -> two fp32 values, exactly.
template <bool HI>
Q35_DEV q35_float2_t e4m3x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// Turbo8 group of 16 rotated values: scale = bf16(amax / 448), codes = E4M3 of
// x / scale (a zero group keeps scale 0 and codes 0).  codes[w] holds elements
// 4w..4w+3, element i in byte i % 4.  Returns the scale's bf16 bits.
Q35_DEV uint32_t turbo8_quantize16(const float v[16], uint32_t codes[4]) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sb = f32_to_bf16(amax / 448.0f);
    const float s = bf16_to_f32(sb);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t c = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (s != 0.0f) c |= e4m3_encode(v[4 * w + b] / s) << (8 * b);
        codes[w] = c;
    }
    return sb;
}

// Lloyd-Max group of 16 rotated values over a 2^BITS-level codebook
// (ascending): each index is the number of thresholds (fp32 midpoints of
// adjacent levels) below x / sigma, sigma = sqrt(sum(x^2) / 16) with the sum in
// double and sigma in fp32 (the nearest level, ties to the lower); packed as a
// little-endian bit stream, element e at bits [BITS e, BITS e + BITS) of
// idx[0] (bits 0-31) : idx[1] (bits 32-63).  Returns the E4M3 code of the
// scale ||x|| / ||levels[idx]|| (double, rounded to fp32, then E4M3), which
// keeps the group's norm up to that rounding.  A zero group: scale 0 and
// indices 0.
template <int BITS>
Q35_DEV uint32_t lm_quantize16(const float v[16], const float* levels, uint32_t idx[2]) {
    constexpr int NL = 1 << BITS;
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss += (double)v[e] * (double)v[e];
    idx[0] = idx[1] = 0u;
    if (ss == 0.0) return 0u;
    const float sigma = sqrtf((float)ss / 16.0f);
    float th[NL - 1];
#pragma unroll
    for (int k = 0; k < NL - 1; ++k) th[k] = (levels[k] + levels[k + 1]) * 0.5f;
    double cn = 0.0;
    uint64_t w = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float y = v[e] / sigma;
        uint32_t n = 0;
#pragma unroll
        for (int k = 0; k < NL - 1; ++k) n += y > th[k] ? 1u : 0u;
        w |= (uint64_t)n << (BITS * e);
        const double l = levels[n];
        cn += l * l;
    }
    idx[0] = (uint32_t)w;
    idx[1] = (uint32_t)(w >> 32);
    return e4m3_encode((float)(sqrt(ss) / sqrt(cn)));
}

// ------------------------------------------------------------------ activations

Q35_DEV float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
Q35_DEV float siluf_(float x) { return x / (1.0f + expf(-x)); }
Q35_DEV float softplusf_(float x) { return x > 20.0f ? x : log1pf(expf(x)); }

// ------------------------------------------------------------------ cross-lane sums

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
Q35_DEV float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                           BANK_MASK, false));
}

// Sum over aligned groups of W lanes (W in {2,...,64}), returned in EVERY lane
// of the group (butterfly: each step pairs lanes whose partial sums cover
// disjoint halves, so all lanes end with the same value).
template <int W>
Q35_DEV float group_sum_all(float v) {
    static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "W");
    v += dpp<0xB1>(v);                          // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp<0x141>(v);   // row_half_mirror: quad 0 <-> quad 1
    if constexpr (W >= 16) v += dpp<0x140>(v);  // row_mirror: half-row 0 <-> half-row 1
    if constexpr (W >= 32)                      // ds_swizzle bitmask mode, lane ^ 16
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    if constexpr (W >= 64) v += __shfl_xor(v, 32);
    return v;
}

// ------------------------------------------------------------------ buffer loads

constexpr int kBufWord3 = 0x00020000;  // raw buffer resource, gfx9 family
constexpr int kAuxStream = 2;          // non-temporal: data streamed once per call

// Device-coherent access (the sc1 cache-policy bit): what agent-scope atomic
// loads and stores use.  Data one block writes and another block of the same
// launch reads later goes through these, so no stage needs an L2 write-back
// or invalidate.
constexpr int kAuxCoherent = 16;

// Raw buffer resource over [p, p + bytes): loads past the end return zero.
Q35_DEV __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufWord3);
}

template <int AUX>
Q35_DEV uint4 ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}

// Stores of values another block reads in the same launch (COH), else plain.
template <bool COH>
Q35_DEV void st_f32(float* p, uint32_t i, float v) {
    if constexpr (COH)
        __hip_atomic_store(p + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        p[i] = v;
}

template <bool COH>
Q35_DEV void st_i32(int32_t* p, uint32_t i, int32_t v) {
    if constexpr (COH)
        __hip_atomic_store(p + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        p[i] = v;
}

template <bool COH>
Q35_DEV void st_act_t(void* p, uint32_t i, float v, bool is_f32) {
    if (is_f32) {
        st_f32<COH>(static_cast<float*>(p), i, v);
    } else {
        const uint16_t b = static_cast<uint16_t>(f32_to_bf16(v));
        if constexpr (COH)
            __hip_atomic_store(static_cast<uint16_t*>(p) + i, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            static_cast<uint16_t*>(p)[i] = b;
    }
}

// Loads of values another block wrote earlier in the same launch.
Q35_DEV float ld_coh_f32(const float* p, uint32_t i) {
    return __hip_atomic_load(const_cast<float*>(p) + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
Q35_DEV int32_t ld_coh_i32(const int32_t* p, uint32_t i) {
    return __hip_atomic_load(const_cast<int32_t*>(p) + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum over aligned groups of W lanes (W in {2,4,8,16,32,64}).  The result is
// valid in the LAST lane of each group (other lanes hold partial sums).
template <int W>
Q35_DEV float group_sum_last(float v) {
    static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "W");
    v += dpp<0xB1>(v);                         // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: all quad lanes hold the quad sum
    if constexpr (W >= 8) v += dpp<0x124>(v);  // row_ror:4: odd quads hold their 8-lane sum
    if constexpr (W >= 16) v += dpp<0x128>(v); // row_ror:8: every lane holds its 16-lane row sum
    if constexpr (W >= 32) v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    if constexpr (W >= 64) v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Full wave sum, returned wave-uniform in every lane.
Q35_DEV float wave_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x124>(v);
    v += dpp<0x128>(v);  // every lane: its row (16 lanes) sum
    float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
    float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
    float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    return (a + b) + (c + d);
}

Q35_DEV float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x124>(v));
    v = fmaxf(v, dpp<0x128>(v));  // every lane: its row (16 lanes) maximum
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Block-wide sum for blockDim.x == NT (multiple of 64); every thread gets the
// total.  `red` must hold NT/64 floats of shared memory.
template <int NT>
Q35_DEV float block_sum(float v, float* red) {
    constexpr int NW = NT / kWave;
    float w = wave_sum(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();  // protect `red` from a previous use
    if (lane == 0) red[wid] = w;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += red[i];
    return t;
}

Q35_DEV float uniform_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

Q35_DEV uint32_t lane_id() { return threadIdx.x & 63u; }

// threadIdx.x through an opaque copy.  In a kernel that runs many stages in a
// loop, the compiler would otherwise compute every stage's thread-derived
// values once, before the loop, and hold them all in registers for the whole
// launch; the opaque copy makes each use site compute its own.
Q35_DEV int tid_x() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

}  // namespace q35
