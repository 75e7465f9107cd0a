// Multi-token prefill of the two Qwen3.5 layer kinds (gfx950).
//
// The pages' forward module runs one token (rustdoc index "Module qwen3_5",
// first paragraph; the prompt pass is left to the caller).  A prefill of T
// tokens is defined as T decode steps in order, token t at cache position
// cache_pos + t; here the T tokens go through each step together:
//
//  * every projection is one GEMM over the T rows (MFMA 32x32x16 f16: the
//    8-bit codes are dequantised to f16 on their way into LDS, the inputs are
//    the f16 rows the norm kernels write);
//  * the causal conv1d, the gates and the per-head L2 norm run per token, the
//    conv state then advances by T inputs at once;
//  * the gated delta rule runs in chunks of 64 tokens: a chunk's corrections
//    solve a unit lower-triangular system built from its own keys (no state
//    needed, all chunks in parallel), and one pass per head then carries the
//    state across the chunks (linear_attention.rs page, the recurrence
//    kernel's update order);
//  * the causal attention is a flash-style pass over K/V tiles of the bf16
//    cache (MFMA 32x32x16 f16) with the online softmax, output gate fused.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "q35decode.h"
#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace pf {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

Q35_DEV float silu(float x) { return x / (1.0f + expf(-x)); }

Q35_DEV uint32_t pack_h2(float a, float b) {
    half2v h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

Q35_DEV uint16_t to_h(float a) { return __builtin_bit_cast(uint16_t, (_Float16)a); }

// two bf16 (low half first) -> two f16, through fp32 (exact for normal bf16 values
// of magnitude up to 65504; smaller than 2^-14 they keep f16's subnormal step)
Q35_DEV uint32_t bf2_to_h2(uint32_t w) { return pack_h2(bf16_lo(w), bf16_hi(w)); }

// ====================================================================== GEMM
//
// out[m, n] = sum_k x[m, k] * W[n, k], W[n, k] = s[n, k/64] * code[n, k] + b[n, k/64]
// (weights dequantised in fp32, rounded once to f16).  Block tile 256 (rows of
// x) x 128 (rows of W) x 64 (one quantisation group); 512 threads in waves of
// 64 x 64 as 2 x 2 MFMA tiles, so each dequantised weight serves 256 rows.  k
// tiles pass through two register stages and two LDS buffers: a tile's loads
// are waited for only where it is written to LDS, a k step after they were
// issued.  SwiGLU mode: the 128 W rows are 64 gate rows and the same 64 up
// rows; a wave holds a gate tile and its up tile, so the epilogue is
// elementwise in registers.
//
// W16: the weights arrive already dequantised (f16 [n, K], the same values
// built the same way by dequant_kernel once per launch), and the stash copies
// them: each weight tile is otherwise dequantised once for every 256-row tile
// of x, which at T = 4096 cost the k loop about a fifth of its rate.
//
// Wave quantisation.  A launch of n tiles on C compute units (one block each)
// runs ceil(n / C) rounds; when the last round would be at most a quarter full,
// its tiles are cut into `split` ranges of k tiles, one block each, so that
// round takes about 1/split of the time.  Those blocks leave fp32 partial tiles
// in a workspace and gemm_reduce_kernel adds the parts in order and applies the
// epilogue.

constexpr int kBN = 128, kBK = 64, kRow = kBK + 8;  // LDS row: 144 bytes

// Tile t of a launch -> (row tile, column tile).  Consecutive blocks go to the 8
// XCDs in turn, so block b runs on XCD b % 8.  When the row tiles divide evenly,
// XCD x takes the row tiles x, x + 8, ... and sweeps all column tiles of one row
// tile before the next: the blocks an XCD runs at once share their x tile in
// that XCD's L2.
Q35_DEV void tile_of(uint32_t t, uint32_t n_mt, uint32_t n_nt, uint32_t& mt, uint32_t& nt) {
    if (n_mt % 8 == 0) {
        const uint32_t slot = t / 8;
        mt = t % 8 + 8 * (slot / n_nt);
        nt = slot % n_nt;
    } else {
        mt = t / n_nt;
        nt = t % n_nt;
    }
}

// BM = 256 rows of x per block, 512 threads: waves of 64 x 64; each thread stages
// one 16-code chunk of W per k tile.
template <int MODE, int BM, bool W16 = false>
__global__ __launch_bounds__(2 * BM, 1) void gemm_kernel(PfGemmArgs a) {
    static_assert(BM == 256, "one W chunk per thread per k tile");
    constexpr int kBM = BM, kGemmThreads = 2 * BM;
    __shared__ __align__(16) _Float16 xs[2][kBM * kRow];
    __shared__ __align__(16) _Float16 ws[2][kBN * kRow];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const uint32_t bn = MODE == kPfSwiglu ? kBN / 2 : kBN;
    const uint32_t n_nt = (a.N + bn - 1) / bn, n_mt = (a.M + kBM - 1) / kBM, b = blockIdx.x;
    // blocks [0, n_full) take whole tiles; block n_full + split j + p takes k range
    // p of tail tile n_full + j
    const bool whole = b < a.n_full;
    const uint32_t pb = whole ? 0 : b - a.n_full;
    uint32_t mt, nt;
    tile_of(whole ? b : a.n_full + pb / a.split, n_mt, n_nt, mt, nt);
    const uint32_t m0 = mt * kBM;
    const uint32_t n0 = nt * bn;
    const uint32_t nk_all = a.K / kBK, ng = a.K / 64;
    const uint32_t k_lo = whole ? 0 : (pb % a.split) * nk_all / a.split;
    const uint32_t nk = whole ? nk_all : (pb % a.split + 1) * nk_all / a.split - k_lo;

    // global -> register staging of one k tile (two stages in flight).  Named
    // members, not arrays: a staged array may be moved to LDS by the compiler,
    // which then waits for every load where it is issued.
    struct Stage {
        uint4 x0, x1, x2, x3;  // four x chunks
        uint4 w;               // sixteen weight codes (W16: the first eight f16 weights)
        uint4 w2;              // W16: the last eight f16 weights
        uint32_t sc, bi;       // raw bf16 bits (unused with W16)
    };
    // This thread's W row (fixed for the whole k loop): rows 64..127 of a SwiGLU
    // tile are the up rows of n0..n0+63; otherwise the row's segment picks the
    // matrix.  A row past the last one reads row 0 of the first matrix (always
    // present) and is masked to zero at the stash.
    const int wrow_t = tid >> 2, wcol_t = (tid & 3) * 16;
    const uint8_t* wrow_p;
    const uint16_t* srow_p;
    const uint16_t* brow_p;
    uint32_t wmsk;
    {
        const uint32_t gn = n0 + wrow_t;
        uint32_t q = 0, n = gn;
        if constexpr (MODE == kPfSwiglu) {
            q = wrow_t >= kBN / 2 ? 1 : 0;
            n = n0 + (q ? wrow_t - kBN / 2 : wrow_t);
        } else if constexpr (MODE == kPfF32) {
            q = (gn >= a.seg_end[0]) + (gn >= a.seg_end[1]) + (gn >= a.seg_end[2]);
            n = gn - (q == 0 ? 0 : q == 1 ? a.seg_end[0] : q == 2 ? a.seg_end[1] : a.seg_end[2]);
        }
        const bool live = (MODE == kPfSwiglu ? n : gn) < a.N;
        if (!live) q = 0;
        const size_t nn = live ? n : 0;
        if constexpr (W16)
            wrow_p = reinterpret_cast<const uint8_t*>((q == 0 ? a.wh[0] : q == 1 ? a.wh[1] : q == 2 ? a.wh[2] : a.wh[3]) +
                                                      nn * a.K + wcol_t);
        else
            wrow_p = (q == 0 ? a.w[0] : q == 1 ? a.w[1] : q == 2 ? a.w[2] : a.w[3]) + nn * a.K + wcol_t;
        srow_p = (q == 0 ? a.s[0] : q == 1 ? a.s[1] : q == 2 ? a.s[2] : a.s[3]) + nn * ng;
        brow_p = (q == 0 ? a.b[0] : q == 1 ? a.b[1] : q == 2 ? a.b[2] : a.b[3]) + nn * ng;
        wmsk = live ? 0xFFFFFFFFu : 0u;
    }
    // x rows past the last one repeat it: they feed only output rows that are never
    // stored, and loads without a condition keep the compiler's wait counts exact
    const uint16_t* xrow_p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + kGemmThreads * i;
        xrow_p[i] = a.x + (size_t)min(m0 + (c >> 3), a.M - 1) * a.K + (c & 7) * 8;
    }
    auto load = [&](Stage& g, uint32_t kt) {
        kt += k_lo;
        const uint32_t ko = kt * kBK;
        g.x0 = *reinterpret_cast<const uint4*>(xrow_p[0] + ko);
        g.x1 = *reinterpret_cast<const uint4*>(xrow_p[1] + ko);
        g.x2 = *reinterpret_cast<const uint4*>(xrow_p[2] + ko);
        g.x3 = *reinterpret_cast<const uint4*>(xrow_p[3] + ko);
        if constexpr (W16) {
            g.w = *reinterpret_cast<const uint4*>(wrow_p + 2 * ko);
            g.w2 = *reinterpret_cast<const uint4*>(wrow_p + 2 * ko + 16);
        } else {
            g.w = *reinterpret_cast<const uint4*>(wrow_p + ko);
            g.sc = srow_p[kt];
            g.bi = brow_p[kt];
        }
    };
    // part q (0..3) of moving a staged tile into LDS: one x chunk, and four weights
    // dequantised (fp32 fma, one f16 rounding); spread over the MFMA steps
    // (q is a compile-time constant throughout, so every member is picked statically)
    auto stash_part = [&](const Stage& g, int buf, auto q_c) {
        constexpr int q = decltype(q_c)::value;
        uint4 xv;
        uint32_t v;
        if constexpr (q == 0) xv = g.x0, v = g.w.x;
        if constexpr (q == 1) xv = g.x1, v = g.w.y;
        if constexpr (q == 2) xv = g.x2, v = g.w.z;
        if constexpr (q == 3) xv = g.x3, v = g.w.w;
        {
            const int c = tid + kGemmThreads * q, row = c >> 3, col = (c & 7) * 8;
            *reinterpret_cast<uint4*>(&xs[buf][row * kRow + col]) = xv;
        }
        if constexpr (W16) {
            uint2 h;
            if constexpr (q == 0) h = make_uint2(g.w.x, g.w.y);
            if constexpr (q == 1) h = make_uint2(g.w.z, g.w.w);
            if constexpr (q == 2) h = make_uint2(g.w2.x, g.w2.y);
            if constexpr (q == 3) h = make_uint2(g.w2.z, g.w2.w);
            *reinterpret_cast<uint2*>(&ws[buf][wrow_t * kRow + wcol_t + 4 * q]) = make_uint2(h.x & wmsk, h.y & wmsk);
        } else {
            v &= wmsk;
            const float sc = __uint_as_float((g.sc << 16) & wmsk);
            const float bi = __uint_as_float((g.bi << 16) & wmsk);
            *reinterpret_cast<uint2*>(&ws[buf][wrow_t * kRow + wcol_t + 4 * q]) =
                make_uint2(pack_h2(fmaf(sc, (float)(v & 0xFFu), bi), fmaf(sc, (float)((v >> 8) & 0xFFu), bi)),
                           pack_h2(fmaf(sc, (float)((v >> 16) & 0xFFu), bi), fmaf(sc, (float)(v >> 24), bi)));
        }
    };
    using c0 = std::integral_constant<int, 0>;
    using c1 = std::integral_constant<int, 1>;
    using c2 = std::integral_constant<int, 2>;
    using c3 = std::integral_constant<int, 3>;
    auto stash = [&](const Stage& g, int buf) {
        stash_part(g, buf, c0{});
        stash_part(g, buf, c1{});
        stash_part(g, buf, c2{});
        stash_part(g, buf, c3{});
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // LDS rows this wave reads: x rows 64 wm + 32 mi + lane%32; W rows per mode
    int wrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        wrow[j] = (MODE == kPfSwiglu ? j * 64 + 32 * wn : 64 * wn + 32 * j) + (lane & 31);
    const int koff = 8 * (lane >> 5);

    // MFMAs on LDS buffer CUR; with do_stash, the stash of the stage that feeds the
    // other buffer is interleaved, a quarter per k step
    Stage g0, g1;
    auto kstep = [&](auto cur_c, auto ks_c, bool do_stash) {
        constexpr int cur = decltype(cur_c)::value, ks = decltype(ks_c)::value;
        {
            half8 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = *reinterpret_cast<const half8*>(
                    &xs[cur][(64 * wm + 32 * i + (lane & 31)) * kRow + ks * 16 + koff]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *reinterpret_cast<const half8*>(&ws[cur][wrow[j] * kRow + ks * 16 + koff]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
            if (do_stash) {
                if constexpr (cur == 0) stash_part(g1, 1, ks_c);
                else stash_part(g0, 0, ks_c);
            }
        }
    };
    auto compute = [&](auto cur_c, bool do_stash) {
        kstep(cur_c, c0{}, do_stash);
        kstep(cur_c, c1{}, do_stash);
        kstep(cur_c, c2{}, do_stash);
        kstep(cur_c, c3{}, do_stash);
    };

    // k tile kt sits in LDS buffer kt % 2 while tile kt + 1 waits in registers and
    // tile kt + 2 is being fetched.  Loads past the last tile repeat it (in bounds,
    // never stashed), so every iteration issues the same loads, and the loop body
    // stashes at every step (a straight line the scheduler can interleave); the
    // last one or two tiles run after it.  A scheduling barrier after each load
    // keeps the loads at the head of their half: left free, the compiler sank
    // them behind three of the four k steps, so the stash of the next half
    // waited for them (the prefill GEMMs ran about 3 % slower).
    const c0 lds0;
    const c1 lds1;
    load(g0, 0);
    load(g1, min(1u, nk - 1));
    stash(g0, 0);
    __syncthreads();
    uint32_t kt = 0;
    for (; kt + 2 < nk; kt += 2) {
        load(g0, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(lds0, true);
        __syncthreads();
        load(g1, min(kt + 3, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(lds1, true);
        __syncthreads();
    }
    if (kt + 1 < nk) {  // tiles kt (LDS buffer 0) and kt + 1 (stage g1)
        compute(lds0, true);
        __syncthreads();
        compute(lds1, false);
    } else {            // tile kt
        compute(lds0, false);
    }

    // epilogue: acc[i][j][r] is (row 8 (r/4) + 4 (lane/32) + r%4, column lane%32) of its tile
    if (!whole) {
        // partial tile [kBM][kBN] in fp32, columns as the tile's W rows (SwiGLU:
        // gate rows 0..63, up rows 64..127); rows past the last one of x are not
        // written (the reduction skips them), columns past the matrix hold zeros
        float* pp = a.part + (size_t)pb * (kBM * kBN);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = (MODE == kPfSwiglu ? 64 * j + 32 * wn : 64 * wn + 32 * j) + (lane & 31);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t row = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (m0 + row < a.M) pp[row * kBN + col] = acc[i][j][r];
                }
        }
    } else if constexpr (MODE == kPfSwiglu) {
        const uint32_t n = n0 + 32 * wn + (lane & 31);
        if (n < a.N) {
            uint16_t* out = static_cast<uint16_t*>(a.out[0]) + n;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (m < a.M) out[(size_t)m * a.ldo[0]] = to_h(silu(acc[i][0][r]) * acc[i][1][r]);
                }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t n = n0 + 64 * wn + 32 * j + (lane & 31);
            if (n >= a.N) continue;
            uint32_t q = 0, n1 = n;
            if constexpr (MODE == kPfF32) {
                q = (n >= a.seg_end[0]) + (n >= a.seg_end[1]) + (n >= a.seg_end[2]);
                n1 = n - (q == 0 ? 0 : q == 1 ? a.seg_end[0] : q == 2 ? a.seg_end[1] : a.seg_end[2]);
            }
            void* out = q == 0 ? a.out[0] : q == 1 ? a.out[1] : q == 2 ? a.out[2] : a.out[3];
            const uint32_t ld = q == 0 ? a.ldo[0] : q == 1 ? a.ldo[1] : q == 2 ? a.ldo[2] : a.ldo[3];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (m >= a.M) continue;
                    const size_t o = (size_t)m * ld + n1;
                    if constexpr (MODE == kPfF32) {
                        static_cast<float*>(out)[o] = acc[i][j][r];
                    } else {
                        store_act(out, o, acc[i][j][r] + load_act(a.resid, o, a.resid_f32), a.out_f32);
                    }
                }
        }
    }
}

// The tail tiles of a split launch: out = epilogue(sum of the `split` fp32 parts,
// added in k order).  One thread per four consecutive columns of a tile row.
template <int MODE, int BM>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(PfGemmArgs a) {
    constexpr uint32_t kTile = BM * kBN, kPerTile = kTile / 4;
    const uint32_t bn = MODE == kPfSwiglu ? kBN / 2 : kBN;
    const uint32_t n_nt = (a.N + bn - 1) / bn, n_mt = (a.M + BM - 1) / BM;
    const uint32_t g = blockIdx.x * 256 + threadIdx.x, j = g / kPerTile, e = g % kPerTile;
    const uint32_t row = e / (kBN / 4), c4 = (e % (kBN / 4)) * 4;
    if (MODE == kPfSwiglu && c4 >= kBN / 2) return;  // the up half is read with its gate half
    uint32_t mt, nt;
    tile_of(a.n_full + j, n_mt, n_nt, mt, nt);
    const uint32_t m = mt * BM + row;
    if (m >= a.M) return;
    const float* pp = a.part + (size_t)j * a.split * kTile + row * kBN + c4;
    float4 v = *reinterpret_cast<const float4*>(pp), u = make_float4(0.f, 0.f, 0.f, 0.f);
    if (MODE == kPfSwiglu) u = *reinterpret_cast<const float4*>(pp + kBN / 2);
    for (uint32_t p = 1; p < a.split; ++p) {
        const float4 w = *reinterpret_cast<const float4*>(pp + (size_t)p * kTile);
        v.x += w.x, v.y += w.y, v.z += w.z, v.w += w.w;
        if (MODE == kPfSwiglu) {
            const float4 w2 = *reinterpret_cast<const float4*>(pp + (size_t)p * kTile + kBN / 2);
            u.x += w2.x, u.y += w2.y, u.z += w2.z, u.w += w2.w;
        }
    }
    const float vv[4] = {v.x, v.y, v.z, v.w}, uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t n = nt * bn + c4 + c;
        if (n >= a.N) break;
        if constexpr (MODE == kPfSwiglu) {
            static_cast<uint16_t*>(a.out[0])[(size_t)m * a.ldo[0] + n] = to_h(silu(vv[c]) * uu[c]);
        } else if constexpr (MODE == kPfF32) {
            const uint32_t q = (n >= a.seg_end[0]) + (n >= a.seg_end[1]) + (n >= a.seg_end[2]);
            const uint32_t n1 = n - (q == 0 ? 0 : q == 1 ? a.seg_end[0] : q == 2 ? a.seg_end[1] : a.seg_end[2]);
            float* out = static_cast<float*>(q == 0 ? a.out[0] : q == 1 ? a.out[1] : q == 2 ? a.out[2] : a.out[3]);
            out[(size_t)m * (q == 0 ? a.ldo[0] : q == 1 ? a.ldo[1] : q == 2 ? a.ldo[2] : a.ldo[3]) + n1] = vv[c];
        } else {
            const size_t o = (size_t)m * a.ldo[0] + n;
            store_act(a.out[0], o, vv[c] + load_act(a.resid, o, a.resid_f32), a.out_f32);
        }
    }
}

// out = f16(scale * code + bias) (fp32 fma, one rounding), 16 codes per thread:
// element for element what gemm_kernel's stash builds from the codes.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* codes, const uint16_t* scales,
                                                      const uint16_t* biases, uint16_t* out,
                                                      uint32_t n16, uint32_t K) {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n16) return;
    const uint32_t per_row = K / 16, row = i / per_row, g = (i % per_row) / 4;
    const uint4 c = reinterpret_cast<const uint4*>(codes)[i];
    const float sc = bf16_to_f32(scales[(size_t)row * (K / 64) + g]);
    const float bi = bf16_to_f32(biases[(size_t)row * (K / 64) + g]);
    auto deq4 = [&](uint32_t v) {
        return make_uint2(pack_h2(fmaf(sc, (float)(v & 0xFFu), bi), fmaf(sc, (float)((v >> 8) & 0xFFu), bi)),
                          pack_h2(fmaf(sc, (float)((v >> 16) & 0xFFu), bi), fmaf(sc, (float)(v >> 24), bi)));
    };
    const uint2 a0 = deq4(c.x), a1 = deq4(c.y), a2 = deq4(c.z), a3 = deq4(c.w);
    uint4* o = reinterpret_cast<uint4*>(out) + 2 * (size_t)i;
    o[0] = make_uint4(a0.x, a0.y, a1.x, a1.y);
    o[1] = make_uint4(a2.x, a2.y, a3.x, a3.y);
}

// ====================================================================== row norms

// out[t, :] = f16(x[t, :] * w / sqrt(mean(x[t, :]^2) + eps)); one block per row.
// PER >= H / 256 values per thread, all loaded before the sum and kept in
// registers for the scaling (one read of the row).
template <int PER>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const void* x, uint32_t x_f32,
                                                           const uint16_t* w, uint16_t* out,
                                                           uint32_t H, float eps) {
    __shared__ float red[4];
    const size_t base = (size_t)blockIdx.x * H;
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const uint32_t i = threadIdx.x + 256 * u;
        v[u] = i < H ? load_act(x, base + i, x_f32) : 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < PER; ++u) ss = fmaf(v[u], v[u], ss);
    ss = block_sum<256>(ss, red);
    const float rs = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const uint32_t i = threadIdx.x + 256 * u;
        if (i < H) out[base + i] = to_h(v[u] * rs * bf16_to_f32(w[i]));
    }
}

// ====================================================================== GDN: conv, gates

// One block per token: causal depthwise conv over the last K raw inputs (the
// conv state supplies those before the first token), SiLU, the L2 norm of each
// Q and K head, and the token's decay (as log g) and beta.
__global__ __launch_bounds__(256) void gdn_conv_kernel(PfConvArgs a) {
    extern __shared__ float sq[];  // [nqk]
    // The blocks of a launch go to the eight XCDs in turn, so block b's XCD is
    // fixed by b mod 8: that class takes a contiguous run of tokens, and the
    // input rows that neighbouring tokens' windows share stay in its L2.  The
    // grid is 8 ceil(T / 8) blocks; those past the last token return at once.
    const uint32_t per = (a.T + 7) / 8;
    const uint32_t t = (blockIdx.x % 8) * per + blockIdx.x / 8;
    if (t >= a.T) return;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const size_t row = (size_t)t * a.C;
    // four channels per pass: all their loads first (channels past the last
    // one repeat it, unused), then the sums and stores
    for (uint32_t c0 = tid; c0 < a.C; c0 += 4 * 256) {
        uint2 wv[4];
        float in[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t c = min(c0 + 256 * k, a.C - 1);
            wv[k] = *reinterpret_cast<const uint2*>(a.conv_w + (size_t)c * 4);  // 4 bf16 taps
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tau = (int)t - 3 + j;
                in[k][j] = tau >= 0 ? a.qkv[(size_t)tau * a.C + c] : a.conv_state[c * 4 + 4 + tau];
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t c = c0 + 256 * k;
            if (c >= a.C) break;
            const float w[4] = {bf16_lo(wv[k].x), bf16_hi(wv[k].x), bf16_lo(wv[k].y), bf16_hi(wv[k].y)};
            float u = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) u = fmaf(w[j], in[k][j], u);
            const float sv = silu(u);
            if (c < a.nqk)
                sq[c] = sv;
            else
                a.qkvs[row + c] = sv;
        }
    }
    if (tid < (int)a.hv) {
        const float av = a.a_raw[(size_t)t * a.hv + tid] + bf16_to_f32(a.dt_bias[tid]);
        const float sp = av > 20.0f ? av : log1pf(expf(av));
        a.lg[(size_t)t * a.hv + tid] = -expf(a.a_log[tid]) * sp;
        a.beta[(size_t)t * a.hv + tid] = 1.0f / (1.0f + expf(-a.b_raw[(size_t)t * a.hv + tid]));
    }
    __syncthreads();
    const uint32_t nh = a.nqk / a.dk;
    for (uint32_t h = wid; h < nh; h += 4) {
        float ss = 0.f;
        for (uint32_t i = lane; i < a.dk; i += 64) ss = fmaf(sq[h * a.dk + i], sq[h * a.dk + i], ss);
        ss = wave_sum(ss);
        const float inv = 1.0f / sqrtf(ss + 1e-6f);
        for (uint32_t i = lane; i < a.dk; i += 64) a.qkvs[row + h * a.dk + i] = sq[h * a.dk + i] * inv;
    }
}

// The conv state after T tokens: the last four raw inputs per channel (older
// state entries where T < 4).
__global__ __launch_bounds__(256) void gdn_conv_state_kernel(const float* qkv, float* state,
                                                             uint32_t T, uint32_t C) {
    const uint32_t c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tau = (int)T - 4 + j;
        v[j] = tau >= 0 ? qkv[(size_t)tau * C + c] : state[c * 4 + 4 + tau];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) state[c * 4 + j] = v[j];
}

// ====================================================================== GDN: chunks
//
// Within a chunk of 64 tokens (L_r = running sum of log g from the chunk
// start), the recurrence S_r = g_r S_{r-1} + k_r d_r^T with
// d_r = beta_r (v_r - g_r S_{r-1}^T k_r) gives, for the corrections D = [d_r],
//   (I + A) D = beta V - beta e^L (K S0),  A[r][s] = beta_r e^(L_r - L_s) k_r.k_s  (s < r)
// so D = U - W S0 with U = (I + A)^-1 beta V and W = (I + A)^-1 beta e^L K,
// both free of the state.  The outputs and the state at the chunk end are
//   y_r = e^(L_r) S0^T q_r + sum_{s <= r} e^(L_r - L_s) (q_r.k_s) d_s
//   S_end = e^(L_end) S0 + sum_s e^(L_end - L_s) k_s d_s^T.
// gdn_chunk_kernel builds U, W, P[r][s] = e^(L_r - L_s) q_r.k_s (s <= r) and L
// for every (head, chunk); gdn_scan_kernel carries the state.

constexpr int kC = 64;

// LDS holds at most 67 KB (DK = DV = 128), so two blocks share a CU: the Gram
// products stream k and q through LDS in two halves of the head dimension, the
// forward substitution reuses that space for its solved rows, A is kept once
// (transposed), and the K columns of the right-hand side are read from memory.
template <int DK, int DV>
__global__ __launch_bounds__(256) void gdn_chunk_kernel(PfGdnArgs a) {
    static_assert(DK + DV <= 256 && DK % 8 == 0, "chunk kernel: one thread per column of [V | K]");
    constexpr int DH = DK / 2, KR = DH + 4;
    constexpr int kGram = 2 * kC * KR, kSol = (kC - 16) * (DK + DV);
    __shared__ __align__(16) float lds[kGram > kSol ? kGram : kSol];
    __shared__ __align__(16) float at[kC * 68];   // A, transposed: at[s][r] = A[r][s]
    __shared__ float L[kC], bt[kC];
    float* ks = lds;                 // Gram phase: half of k and q per pass
    float* qs = lds + kC * KR;
    float* xsol = lds;               // substitution: solved rows of the first three blocks
    const int tid = threadIdx.x;
    const uint32_t ch = blockIdx.x, j = blockIdx.y, nch = gridDim.x;
    const uint32_t i = j / (a.hv / a.hk);
    const uint32_t t0 = ch * kC;
    const int n = (int)min((uint32_t)kC, a.T - t0);
    const uint32_t qoff = i * DK, koff = a.hk * DK + i * DK, voff = 2 * a.hk * DK + j * DV;

    // this thread's column of the right-hand side [V | K] for the substitution
    // below, 16 rows at a time: the first 16 are fetched now, behind the Gram
    // products, and each row block fetches the next one's while it is solved
    // (a resource over the chunk's rows returns zero past the last token;
    // threads past the last column read values they never use)
    const auto rX = rsrc(a.qkvs + (size_t)t0 * a.C, (uint32_t)n * a.C * 4u);
    const uint32_t rcol = tid < DV ? voff + tid : koff + (tid - DV);
    auto fetch16 = [&](float (&dst)[16], int rb) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
            dst[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rX, ((rb + u) * a.C + rcol) * 4u, 0, 0));
    };
    // one half of the head dimension of k and q for the Gram products: NH float4
    // of each per thread, loaded into registers and then stashed in LDS; the
    // second half is fetched while the first half's products run
    constexpr int NH = kC * DH / 4 / 256;
    static_assert(NH * 256 * 4 == kC * DH, "whole float4 per thread per half");
    struct Half {
        float4 k[NH], q[NH];
    };
    auto load_half = [&](Half& g, int h) {
#pragma unroll
        for (int e = 0; e < NH; ++e) {
            const int c = tid + 256 * e, r = c / (DH / 4), d = (c % (DH / 4)) * 4;
            g.k[e] = __builtin_bit_cast(float4, ld_b128<0>(rX, (r * a.C + koff + h * DH + d) * 4u));
            g.q[e] = __builtin_bit_cast(float4, ld_b128<0>(rX, (r * a.C + qoff + h * DH + d) * 4u));
        }
    };
    auto stash_half = [&](const Half& g) {
#pragma unroll
        for (int e = 0; e < NH; ++e) {
            const int c = tid + 256 * e, r = c / (DH / 4), d = (c % (DH / 4)) * 4;
            *reinterpret_cast<float4*>(&ks[r * KR + d]) = g.k[e];
            *reinterpret_cast<float4*>(&qs[r * KR + d]) = g.q[e];
        }
    };

    float lg = 0.f;
    if (tid < 64) {
        lg = tid < n ? a.lg[(size_t)(t0 + tid) * a.hv + j] : 0.f;
        bt[tid] = tid < n ? a.beta[(size_t)(t0 + tid) * a.hv + j] : 0.f;
    }
    Half h0, h1;
    load_half(h0, 0);
    float rhs[16];
    fetch16(rhs, 0);
    if (tid < 64) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {  // inclusive scan over the wave
            const float u = __shfl_up(lg, o);
            if (tid >= o) lg += u;
        }
        L[tid] = lg;
    }

    // Gram blocks: thread (rb, sb) -> rows 4 rb.., columns 4 sb..
    {
        const int rb = tid >> 4, sb = tid & 15;
        float kk[4][4] = {}, qk[4][4] = {};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            stash_half(h == 0 ? h0 : h1);
            __syncthreads();
            if (h == 0) load_half(h1, 1);
            for (int d = 0; d < DH; d += 4) {
                float4 kr[4], qr[4], kc[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    kr[u] = *reinterpret_cast<const float4*>(&ks[(4 * rb + u) * KR + d]);
                    qr[u] = *reinterpret_cast<const float4*>(&qs[(4 * rb + u) * KR + d]);
                    kc[u] = *reinterpret_cast<const float4*>(&ks[(4 * sb + u) * KR + d]);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        kk[u][v] = fmaf(kr[u].x, kc[v].x, fmaf(kr[u].y, kc[v].y,
                                   fmaf(kr[u].z, kc[v].z, fmaf(kr[u].w, kc[v].w, kk[u][v]))));
                        qk[u][v] = fmaf(qr[u].x, kc[v].x, fmaf(qr[u].y, kc[v].y,
                                   fmaf(qr[u].z, kc[v].z, fmaf(qr[u].w, kc[v].w, qk[u][v]))));
                    }
            }
            __syncthreads();
        }
        float* P = a.Pc + ((size_t)j * nch + ch) * kC * kC;
        float av[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * rb + u;
            float pv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int s = 4 * sb + v;
                const float e = s <= r ? expf(L[r] - L[s]) : 0.f;
                av[u][v] = s < r ? bt[r] * e * kk[u][v] : 0.f;
                pv[v] = e * qk[u][v];
            }
            *reinterpret_cast<float4*>(&P[r * kC + 4 * sb]) = make_float4(pv[0], pv[1], pv[2], pv[3]);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
            *reinterpret_cast<float4*>(&at[(4 * sb + v) * 68 + 4 * rb]) =
                make_float4(av[0][v], av[1][v], av[2][v], av[3][v]);
    }
    __syncthreads();

    // forward substitution, one thread per column of the right-hand side
    // [beta V | beta e^L K], in blocks of 16 rows: a block first takes the
    // contributions of the rows solved before it (kept in LDS), then solves its
    // own 16 x 16 triangle in registers
    if (tid < DK + DV) {
        const int c = tid;
        const size_t blk = (size_t)j * nch + ch;
        float* out = c < DV ? a.Uc + blk * kC * DV + c : a.Wc + blk * kC * DK + (c - DV);
        const int ld = c < DV ? DV : DK;
        for (int rb = 0; rb < kC; rb += 16) {
            float x[16], nxt[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int r = rb + u;
                x[u] = c < DV ? bt[r] * rhs[u] : bt[r] * expf(L[r]) * rhs[u];
            }
            fetch16(nxt, min(rb + 16, kC - 16));  // the last block refetches its own rows, unused
            for (int s = 0; s < rb; ++s) {
                const float xv = xsol[s * (DK + DV) + c];
                const float4* ar = reinterpret_cast<const float4*>(&at[s * 68 + rb]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 w = ar[q];
                    x[4 * q] = fmaf(-w.x, xv, x[4 * q]);
                    x[4 * q + 1] = fmaf(-w.y, xv, x[4 * q + 1]);
                    x[4 * q + 2] = fmaf(-w.z, xv, x[4 * q + 2]);
                    x[4 * q + 3] = fmaf(-w.w, xv, x[4 * q + 3]);
                }
            }
#pragma unroll
            for (int u = 1; u < 16; ++u)
#pragma unroll
                for (int v = 0; v < u; ++v) x[u] = fmaf(-at[(rb + v) * 68 + rb + u], x[v], x[u]);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                out[(size_t)(rb + u) * ld] = x[u];
                if (rb + 16 < kC) xsol[(rb + u) * (DK + DV) + c] = x[u];
                rhs[u] = nxt[u];
            }
        }
    }
    if (tid < kC) a.Lc[((size_t)j * nch + ch) * kC + tid] = L[tid];
}

// One block per (v-head, 16 state columns): the state slice S0 [DK, 16] is
// carried through the chunks in order.  The products run on the fp32 matrix
// cores (16x16x4: A row i = lane % 16, B column j = lane % 16, both with
// k = lane / 16; D row 4 (lane / 16) + r, column lane % 16).  Within each
// 16-wide k block, lane group g supplies k = 4 g + s to step s, so a lane reads
// its four k values as one float4.  Every wave holds all of S0 as B operands;
// S0 and D are kept transposed in LDS for those float4 reads.
constexpr int kSL = 16;

template <int DK>
__global__ __launch_bounds__(256, 1) void gdn_scan_kernel(PfGdnArgs a) {
    constexpr int KR = DK + 4, TR = kC + 4, NB = DK / 16;
    __shared__ __align__(16) float wl[kC * KR];   // W rows
    __shared__ __align__(16) float ql[kC * KR];   // Q rows
    __shared__ __align__(16) float kl[kC * KR];   // K rows
    __shared__ __align__(16) float pl[kC * TR];   // P rows
    __shared__ __align__(16) float dlt[kSL * TR]; // D transposed [column][token]
    __shared__ __align__(16) float st[kSL * KR];  // S transposed [column][d]
    __shared__ __align__(16) float L[kC], ef[kC], el[kC];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;      // MFMA row/column, k group
    const uint32_t j = blockIdx.x, c0 = blockIdx.y * kSL, nch = a.nch;
    const uint32_t dv = a.dv, i = j / (a.hv / a.hk);
    const uint32_t qoff = i * DK, koff = a.hk * DK + i * DK;
    float* gst = a.state + (size_t)j * DK * dv;

    for (int e = tid; e < DK * kSL; e += 256) st[(e % kSL) * KR + e / kSL] = gst[(e / kSL) * dv + c0 + (e % kSL)];

    // chunk ch + 1's operands are fetched into registers while chunk ch computes
    // (buffer loads: a resource over the chunk's own token rows returns zero past
    // the last token)
    constexpr int NW4 = kC * DK / 4 / 256;
    struct Regs {
        float4 w[NW4], q[NW4], k[NW4], p[4];
        float u[4];
        float l;
    } R;
    auto gload = [&](Regs& g, uint32_t ch) {
        const uint32_t t0 = ch * kC;
        const uint32_t n = min((uint32_t)kC, a.T - t0);
        const size_t blk = (size_t)j * nch + ch;
        const auto rW = rsrc(a.Wc + blk * kC * DK, kC * DK * 4);
        const auto rP = rsrc(a.Pc + blk * kC * kC, kC * kC * 4);
        const auto rX = rsrc(a.qkvs + (size_t)t0 * a.C, n * a.C * 4);
#pragma unroll
        for (int e = 0; e < NW4; ++e) {
            const uint32_t c = tid + 256 * e, rr = c / (DK / 4), d = (c % (DK / 4)) * 4;
            g.w[e] = __builtin_bit_cast(float4, ld_b128<0>(rW, (rr * DK + d) * 4));
            g.q[e] = __builtin_bit_cast(float4, ld_b128<0>(rX, (rr * a.C + qoff + d) * 4));
            g.k[e] = __builtin_bit_cast(float4, ld_b128<0>(rX, (rr * a.C + koff + d) * 4));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t c = tid + 256 * e, rr = c / (kC / 4), s4 = (c % (kC / 4)) * 4;
            g.p[e] = __builtin_bit_cast(float4, ld_b128<0>(rP, (rr * kC + s4) * 4));
        }
        const auto rU = rsrc(a.Uc + blk * kC * dv, kC * dv * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)  // U at (token 16 wid + 4 lg + r, column c0 + li)
            g.u[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rU, ((16 * wid + 4 * lg + r) * dv + c0 + li) * 4, 0, 0));
        g.l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.Lc + blk * kC, kC * 4),
                                                                            (uint32_t)lane * 4, 0, 0));
    };
    typedef float f4 __attribute__((ext_vector_type(4)));
    auto mfma = [](float x, float y, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c, 0, 0, 0); };
    auto f4z = []() { f4 z = {0.f, 0.f, 0.f, 0.f}; return z; };

    gload(R, 0);
    __syncthreads();  // st filled
    for (uint32_t ch = 0; ch < nch; ++ch) {
        const uint32_t t0 = ch * kC;
        const int n = (int)min((uint32_t)kC, a.T - t0);
#pragma unroll
        for (int e = 0; e < NW4; ++e) {
            const int c = tid + 256 * e, rr = c / (DK / 4), d = (c % (DK / 4)) * 4;
            *reinterpret_cast<float4*>(&wl[rr * KR + d]) = R.w[e];
            *reinterpret_cast<float4*>(&ql[rr * KR + d]) = R.q[e];
            *reinterpret_cast<float4*>(&kl[rr * KR + d]) = R.k[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = tid + 256 * e, rr = c / (kC / 4), s4 = (c % (kC / 4)) * 4;
            *reinterpret_cast<float4*>(&pl[rr * TR + s4]) = R.p[e];
        }
        if (tid < kC) L[tid] = R.l;
        float u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = R.u[r];
        __syncthreads();
        if (ch + 1 < nch) gload(R, ch + 1);
        if (tid < kC) {
            ef[tid] = expf(L[kC - 1] - L[tid]);
            el[tid] = expf(L[tid]);
        }

        // S0 as B operands: sb[b] holds S0[16 b + 4 lg + s][li], s = 0..3
        float4 sb[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) sb[b] = *reinterpret_cast<const float4*>(&st[li * KR + 16 * b + 4 * lg]);

        // W S0 and Q S0 for rows 16 wid .. 16 wid + 15
        f4 ws = f4z(), qs = f4z();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float4 wa = *reinterpret_cast<const float4*>(&wl[(16 * wid + li) * KR + 16 * b + 4 * lg]);
            const float4 qa = *reinterpret_cast<const float4*>(&ql[(16 * wid + li) * KR + 16 * b + 4 * lg]);
            ws = mfma(wa.x, sb[b].x, ws);
            ws = mfma(wa.y, sb[b].y, ws);
            ws = mfma(wa.z, sb[b].z, ws);
            ws = mfma(wa.w, sb[b].w, ws);
            qs = mfma(qa.x, sb[b].x, qs);
            qs = mfma(qa.y, sb[b].y, qs);
            qs = mfma(qa.z, sb[b].z, qs);
            qs = mfma(qa.w, sb[b].w, qs);
        }
        // D = U - W S0 at (token 16 wid + 4 lg + r, column li), stored transposed
        *reinterpret_cast<float4*>(&dlt[li * TR + 16 * wid + 4 * lg]) =
            make_float4(u[0] - ws[0], u[1] - ws[1], u[2] - ws[2], u[3] - ws[3]);
        __syncthreads();

        // y = e^L (Q S0) + P D; P is lower triangular, so k blocks past this wave's rows add nothing
        {
            const float4 e4 = *reinterpret_cast<const float4*>(&el[16 * wid + 4 * lg]);
            f4 y = {e4.x * qs[0], e4.y * qs[1], e4.z * qs[2], e4.w * qs[3]};
            // every k block's operands read first (in bounds for all four), then the chain
            float4 pa[kC / 16], db[kC / 16];
#pragma unroll
            for (int b = 0; b < kC / 16; ++b) {
                pa[b] = *reinterpret_cast<const float4*>(&pl[(16 * wid + li) * TR + 16 * b + 4 * lg]);
                db[b] = *reinterpret_cast<const float4*>(&dlt[li * TR + 16 * b + 4 * lg]);
            }
#pragma unroll
            for (int b = 0; b < kC / 16; ++b) {
                if (b > wid) break;  // wave-uniform
                y = mfma(pa[b].x, db[b].x, y);
                y = mfma(pa[b].y, db[b].y, y);
                y = mfma(pa[b].z, db[b].z, y);
                y = mfma(pa[b].w, db[b].w, y);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * wid + 4 * lg + r;
                if (row < n) a.y[(size_t)(t0 + row) * a.hv * dv + (size_t)j * dv + c0 + li] = y[r] * a.out_scale;
            }
        }

        // S <- e^(L_end) S0 + K^T (ef D): this wave's d tiles t = wid, wid + 4, ...
        f4 sn[(NB + 3) / 4];
        const float ge = expf(L[kC - 1]);
#pragma unroll
        for (int tt = 0; tt < (NB + 3) / 4; ++tt) {
            const int t = wid + 4 * tt;
            if (t >= NB) break;
            const float4 s0 = *reinterpret_cast<const float4*>(&st[li * KR + 16 * t + 4 * lg]);
            f4 acc = {ge * s0.x, ge * s0.y, ge * s0.z, ge * s0.w};
            // A = K^T: (d 16 t + li, token 16 b + 4 lg + s), scalar reads of K rows;
            // all sixteen operand pairs are read before the chain, so one wait covers them
            float ka[kC / 16][4];
            float4 bb[kC / 16];
#pragma unroll
            for (int b = 0; b < kC / 16; ++b) {
                const float* kr = &kl[(16 * b + 4 * lg) * KR + 16 * t + li];
                ka[b][0] = kr[0];
                ka[b][1] = kr[KR];
                ka[b][2] = kr[2 * KR];
                ka[b][3] = kr[3 * KR];
                const float4 db = *reinterpret_cast<const float4*>(&dlt[li * TR + 16 * b + 4 * lg]);
                const float4 fb = *reinterpret_cast<const float4*>(&ef[16 * b + 4 * lg]);
                bb[b] = make_float4(fb.x * db.x, fb.y * db.y, fb.z * db.z, fb.w * db.w);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < kC / 16; ++b) {
                acc = mfma(ka[b][0], bb[b].x, acc);
                acc = mfma(ka[b][1], bb[b].y, acc);
                acc = mfma(ka[b][2], bb[b].z, acc);
                acc = mfma(ka[b][3], bb[b].w, acc);
            }
            sn[tt] = acc;
        }
        __syncthreads();  // every read of S0 is done
#pragma unroll
        for (int tt = 0; tt < (NB + 3) / 4; ++tt) {
            const int t = wid + 4 * tt;
            if (t >= NB) break;
            *reinterpret_cast<float4*>(&st[li * KR + 16 * t + 4 * lg]) =
                make_float4(sn[tt][0], sn[tt][1], sn[tt][2], sn[tt][3]);
        }
        __syncthreads();
    }
    for (int e = tid; e < DK * kSL; e += 256) gst[(e / kSL) * dv + c0 + (e % kSL)] = st[(e % kSL) * KR + e / kSL];
}

// yz[t, j, :] = f16(RMSNorm(y[t, j, :]; w) * silu(z[t, j, :])); one block per token.
// Wave wid takes heads wid, wid + 4, ...: eight of them at a time, with every
// y and z value of the eight loaded before the sums (dv <= 128: two per lane).
__global__ __launch_bounds__(256) void gdn_out_kernel(const float* y, const float* z,
                                                      const uint16_t* w, uint16_t* yz, uint32_t hv,
                                                      uint32_t dv, float eps) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const size_t row = (size_t)blockIdx.x * hv * dv;
    for (uint32_t j0 = wid; j0 < hv; j0 += 4 * 8) {
        float yv[8][2], zv[8][2];
#pragma unroll
        for (int h = 0; h < 8; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t j = j0 + 4 * h, d = lane + 64 * e;
                const bool in = j < hv && d < dv;
                const size_t o = row + (size_t)(in ? j : 0) * dv + (in ? d : 0);
                yv[h][e] = in ? y[o] : 0.f;
                zv[h][e] = in ? z[o] : 0.f;
            }
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const uint32_t j = j0 + 4 * h;
            if (j >= hv) break;  // wave-uniform
            const float ss = wave_sum(fmaf(yv[h][0], yv[h][0], yv[h][1] * yv[h][1]));
            const float rs = 1.0f / sqrtf(ss / (float)dv + eps);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t d = lane + 64 * e;
                if (d < dv) yz[row + j * dv + d] = to_h(yv[h][e] * rs * bf16_to_f32(w[d]) * silu(zv[h][e]));
            }
        }
    }
}

// ====================================================================== attention

// One block per token: q and k per-head RMSNorm, RoPE at cache_pos + t, q to an
// f16 row for the attention, k and v appended to the bf16 cache.
__global__ __launch_bounds__(256) void qk_rope_append_kernel(PfRopeArgs a) {
    extern __shared__ float buf[];  // [(hq + hkv) * D] then rsq[hq + hkv], rot[2 * R/2]
    const uint32_t t = blockIdx.x, D = a.D, nh = a.hq + a.hkv, half = a.rotary / 2;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    float* rsq = buf + nh * D;
    float* rot = rsq + nh;
    const uint32_t pos = a.cache_pos + t;
    const float* qrow = a.q_full + (size_t)t * a.hq * 2 * D;
    for (uint32_t e = tid; e < nh * D; e += 256) {
        const uint32_t h = e / D, d = e % D;
        buf[e] = h < a.hq ? qrow[h * 2 * D + d] : a.k[(size_t)t * a.hkv * D + (h - a.hq) * D + d];
    }
    if (tid < (int)half) {
        float sn, cs;
        sincosf((float)pos * a.inv_freq[tid], &sn, &cs);
        rot[2 * tid] = cs;
        rot[2 * tid + 1] = sn;
    }
    __syncthreads();
    for (uint32_t h = wid; h < nh; h += 4) {
        float ss = 0.f;
        for (uint32_t d = lane; d < D; d += 64) ss = fmaf(buf[h * D + d], buf[h * D + d], ss);
        ss = wave_sum(ss);
        if (lane == 0) rsq[h] = 1.0f / sqrtf(ss / (float)D + a.eps);
    }
    __syncthreads();
    for (uint32_t e = tid; e < nh * D; e += 256) {
        const uint32_t h = e / D, d = e % D;
        const uint16_t* nw = h < a.hq ? a.q_norm : a.k_norm;
        float x = buf[e] * rsq[h] * bf16_to_f32(nw[d]);
        if (d < a.rotary) {
            const uint32_t pd = d < half ? d + half : d - half;
            const float xp = buf[h * D + pd] * rsq[h] * bf16_to_f32(nw[pd]);
            const float cs = rot[2 * (d % half)], sn = rot[2 * (d % half) + 1];
            x = d < half ? x * cs - xp * sn : x * cs + xp * sn;
        }
        if (h < a.hq)
            a.qb[((size_t)t * a.hq + h) * D + d] = to_h(x);
        else
            a.kc[((size_t)pos * a.hkv + (h - a.hq)) * D + d] = (uint16_t)f32_to_bf16(x);
    }
    for (uint32_t e = tid; e < a.hkv * D; e += 256)
        a.vc[(size_t)pos * a.hkv * D + e] = (uint16_t)f32_to_bf16(a.v[(size_t)t * a.hkv * D + e]);
}

// Causal GQA attention over the bf16 cache for 32 tokens x G heads of one kv
// head per block (one wave per q-head), key tiles of 64.  The tiles go to LDS
// as f16 (a bf16 value of the cache's range is exact in f16), the query is an
// f16 row and the probabilities are rounded to f16, so the products are f16 x
// f16 on the matrix cores with fp32 sums.  S^T = K Q^T puts one query per lane:
// the softmax statistics are per lane (plus the partner lane l ^ 32), and the
// probabilities in registers are already the B operand of O^T += V^T P^T.
// Output: f16(attention * sigmoid(gate)).  With D = 256 (and G <= 4) two waves
// share a query head, each computing the scores (the same in both) and half of the output
// columns: eight 32 x 32 accumulators per lane left too few registers for the
// next key tile's loads to stay in flight.
constexpr int kKT = 64;  // keys per tile

template <int D, int G>
constexpr int flash_wph() { return D == 256 && G <= 4 ? 2 : 1; }  // waves per query head

template <int D, int G>
__global__ __launch_bounds__((64 * G * flash_wph<D, G>())) void flash_kernel(PfAttnArgs a) {
    constexpr int WPH = flash_wph<D, G>(), NT = 64 * G * WPH, KRW = D + 8, VRW = kKT + 4, DT = D / 32;
    constexpr int DTW = DT / WPH;  // output column tiles of this wave
    __shared__ __align__(16) uint16_t kt_s[kKT * KRW];
    __shared__ __align__(16) uint16_t vt_s[D * VRW];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, h2 = lane >> 5;
    const int half = wid % WPH;  // this wave's output columns: tiles half * DTW ..
    const uint32_t g = blockIdx.y, h = g * G + wid / WPH;
    const uint32_t t0 = (gridDim.x - 1 - blockIdx.x) * 32;  // longest blocks first
    const uint32_t tq = t0 + (lane & 31);
    const uint32_t kend = a.cache_pos + min(t0 + 32, a.T);  // rows any query here may read
    const size_t rs = (size_t)a.hkv * D;                     // cache row stride (elements)

    half8 qv[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (tq < a.T)
            w = *reinterpret_cast<const uint4*>(a.qb + ((size_t)tq * a.hq + h) * D + ks * 16 + 8 * h2);
        qv[ks] = __builtin_bit_cast(half8, w);
    }
    f32x16 o[DTW];
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    // tile kt + 1 is fetched into registers while tile kt is in LDS
    constexpr int KL = (kKT * D / 8 + NT - 1) / NT;          // K: 16-byte chunks per thread
    constexpr int VTASK = kKT / 4 * (D / 8);                  // V: (key quad, column octet) tasks
    constexpr int VL = (VTASK + NT - 1) / NT;
    // Loads without a condition keep the compiler's wait counts exact, so tile
    // kt + 1 stays in flight while tile kt is used: rows past kend (in the last
    // tile only) repeat row kend - 1, finite values that the causal mask removes
    // (keys past every query of the block) and that meet zero probabilities in
    // P V; a thread whose chunk index is past the tile's loads a repeat of an
    // earlier chunk and does not store it.
    uint4 kr[KL], vr[VL][4];
    auto gload = [&](uint32_t k0) {
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const int c = (tid + NT * i) % (kKT * D / 8), row = c / (D / 8), col = (c % (D / 8)) * 8;
            const uint32_t key = min(k0 + row, kend - 1);
            kr[i] = *reinterpret_cast<const uint4*>(a.kc + key * rs + g * D + col);
        }
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            // key quads vary fastest across lanes: the transposed LDS writes of a wave
            // then fall on distinct banks but for one 2-way overlap
            const int c = (tid + NT * i) % VTASK, q4 = c % (kKT / 4), b = c / (kKT / 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t key = min(k0 + 4 * q4 + u, kend - 1);
                vr[i][u] = *reinterpret_cast<const uint4*>(a.vc + key * rs + g * D + 8 * b);
            }
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const int c = tid + NT * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
            if (c < kKT * D / 8)
                *reinterpret_cast<uint4*>(&kt_s[row * KRW + col]) =
                    make_uint4(bf2_to_h2(kr[i].x), bf2_to_h2(kr[i].y), bf2_to_h2(kr[i].z), bf2_to_h2(kr[i].w));
        }
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            const int c = tid + NT * i, q4 = c % (kKT / 4), b = c / (kKT / 4);
            if (c >= VTASK) continue;
            const uint32_t* p0 = reinterpret_cast<const uint32_t*>(&vr[i][0]);
            const uint32_t* p1 = reinterpret_cast<const uint32_t*>(&vr[i][1]);
            const uint32_t* p2 = reinterpret_cast<const uint32_t*>(&vr[i][2]);
            const uint32_t* p3 = reinterpret_cast<const uint32_t*>(&vr[i][3]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sh = (e & 1) * 16;
                const uint32_t v0 = (p0[e >> 1] >> sh) & 0xFFFFu, v1 = (p1[e >> 1] >> sh) & 0xFFFFu;
                const uint32_t v2 = (p2[e >> 1] >> sh) & 0xFFFFu, v3 = (p3[e >> 1] >> sh) & 0xFFFFu;
                *reinterpret_cast<uint2*>(&vt_s[(8 * b + e) * VRW + 4 * q4]) =
                    make_uint2(bf2_to_h2(v0 | (v1 << 16)), bf2_to_h2(v2 | (v3 << 16)));
            }
        }
    };
    const uint32_t nkt = (kend + kKT - 1) / kKT;
    gload(0);
    for (uint32_t kt = 0; kt < nkt; ++kt) {
        const uint32_t k0 = kt * kKT;
        lstore();
        __syncthreads();
        gload(min(k0 + kKT, (nkt - 1) * kKT));  // past the last tile: repeats it, unused

        // S^T for two 32-key halves: s[hf][r] is key k0 + 32 hf + 8 (r/4) + 4 h2 + r%4, query tq
        // (the two halves' MFMA chains interleave, so no MFMA waits on the previous one)
        f32x16 s[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[hf][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const half8 kv = *reinterpret_cast<const half8*>(
                    &kt_s[(32 * hf + (lane & 31)) * KRW + ks * 16 + 8 * h2]);
                s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kv, qv[ks], s[hf], 0, 0, 0);
            }
        // scale to base 2; only a tile reaching past the block's first query (the
        // diagonal, block-uniform) needs the causal mask
        float mx = -INFINITY;
        if (k0 + kKT - 1 <= a.cache_pos + t0 && k0 + kKT <= kend) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[hf][r] *= a.scale_log2;
                    mx = fmaxf(mx, s[hf][r]);
                }
        } else {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t key = k0 + 32 * hf + 8 * (r >> 2) + 4 * h2 + (r & 3);
                    const bool ok = key <= a.cache_pos + tq && key < kend;
                    s[hf][r] = ok ? s[hf][r] * a.scale_log2 : -INFINITY;
                    mx = fmaxf(mx, s[hf][r]);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // the running maximum moves (and the accumulators are rescaled) only when
        // some query's tile maximum exceeds it by more than 2^8: probabilities stay
        // below 256, far inside f16 and fp32 range, and the rescale is skipped for
        // most tiles; the decision is wave-uniform
        if (__ballot(mx > m + 8.0f)) {
            const float mn = fmaxf(m, mx);
            const float al = __builtin_amdgcn_exp2f(m - mn);
            m = mn;
            l *= al;
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= al;
        }
        float ps = 0.f;
        half8 pb[4];  // k steps of 16 keys: step kk holds s[kk / 2][8 (kk % 2) + e]
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[hf][r] - m);
                ps += p;
                pb[2 * hf + (r >> 3)][r & 7] = (_Float16)p;
            }
        l += ps;
        // k steps outer, the DT independent accumulators inner
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) {
                // keys 16 kk + 4 h2 + 0..3 and 16 kk + 8 + 4 h2 + 0..3, the order of pb[kk]
                const int dg = half * DTW + dt;
                const uint16_t* vrow = &vt_s[(32 * dg + (lane & 31)) * VRW + 4 * h2 + 16 * kk];
                const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
                const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
                const half8 vv = __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv, pb[kk], o[dt], 0, 0, 0);
            }
        __syncthreads();
    }
    l += __shfl_xor(l, 32);
    if (tq >= a.T) return;
    const float inv = 1.0f / l;
    const float* gate = a.q_full + (size_t)tq * a.hq * 2 * D + (size_t)h * 2 * D + D;
    uint16_t* out = a.ga + ((size_t)tq * a.hq + h) * D;
    // every gate value first: a store between two loads would make the second
    // load's wait include the store (the vector memory counter counts both)
    float4 gv[DTW][4];
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            gv[dt][r4] = *reinterpret_cast<const float4*>(gate + 32 * (half * DTW + dt) + 8 * r4 + 4 * h2);
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * (half * DTW + dt) + 8 * r4 + 4 * h2;
            const float gt[4] = {gv[dt][r4].x, gv[dt][r4].y, gv[dt][r4].z, gv[dt][r4].w};
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = o[dt][4 * r4 + u] * inv / (1.0f + expf(-gt[u]));
            *reinterpret_cast<uint2*>(out + d) = make_uint2(pack_h2(v[0], v[1]), pack_h2(v[2], v[3]));
        }
}

// ---------------------------------------------------------------------- quantised caches

// Cache positions base, base + 1, ... of the prompt's tokens (the per-token
// attention of a quantised cache reads its RoPE position from memory).
__global__ __launch_bounds__(256) void iota_kernel(int32_t* out, uint32_t n, int32_t base) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i < n) out[i] = base + (int32_t)i;
}

// fp32 -> f16 (round to nearest even), the o-projection GEMM's operand.
__global__ __launch_bounds__(256) void cast_f16_kernel(const float* x, uint16_t* y, uint32_t n) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i < n) y[i] = __builtin_bit_cast(uint16_t, (_Float16)x[i]);
}

}  // namespace pf

// ====================================================================== launchers

hipError_t pf_iota_launch(int32_t* out, uint32_t n, int32_t base, hipStream_t s) {
    if (n == 0) return hipSuccess;
    pf::iota_kernel<<<(n + 255) / 256, 256, 0, s>>>(out, n, base);
    return hipGetLastError();
}

hipError_t pf_cast_f16_launch(const float* x, uint16_t* y, uint32_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    pf::cast_f16_kernel<<<(n + 255) / 256, 256, 0, s>>>(x, y, n);
    return hipGetLastError();
}

const void* pf_kernel_ptr(int i) {
    static const void* const k[] = {
        reinterpret_cast<const void*>(pf::gemm_kernel<kPfF32, 256>),
        reinterpret_cast<const void*>(pf::gemm_kernel<kPfResid, 256>),
        reinterpret_cast<const void*>(pf::gemm_kernel<kPfSwiglu, 256>),
        reinterpret_cast<const void*>(pf::gemm_reduce_kernel<kPfF32, 256>),
        reinterpret_cast<const void*>(pf::gemm_reduce_kernel<kPfResid, 256>),
        reinterpret_cast<const void*>(pf::gemm_reduce_kernel<kPfSwiglu, 256>),
        reinterpret_cast<const void*>(pf::rmsnorm_rows_kernel<4>),
        reinterpret_cast<const void*>(pf::rmsnorm_rows_kernel<8>),
        reinterpret_cast<const void*>(pf::rmsnorm_rows_kernel<16>),
        reinterpret_cast<const void*>(pf::rmsnorm_rows_kernel<32>),
        reinterpret_cast<const void*>(pf::gdn_conv_kernel),
        reinterpret_cast<const void*>(pf::gdn_conv_state_kernel),
        reinterpret_cast<const void*>(pf::gdn_chunk_kernel<32, 32>),
        reinterpret_cast<const void*>(pf::gdn_chunk_kernel<64, 64>),
        reinterpret_cast<const void*>(pf::gdn_chunk_kernel<128, 128>),
        reinterpret_cast<const void*>(pf::gdn_scan_kernel<32>),
        reinterpret_cast<const void*>(pf::gdn_scan_kernel<64>),
        reinterpret_cast<const void*>(pf::gdn_scan_kernel<128>),
        reinterpret_cast<const void*>(pf::gdn_out_kernel),
        reinterpret_cast<const void*>(pf::qk_rope_append_kernel),
        reinterpret_cast<const void*>(pf::flash_kernel<64, 2>),
        reinterpret_cast<const void*>(pf::flash_kernel<256, 4>),
        reinterpret_cast<const void*>(pf::iota_kernel),
        reinterpret_cast<const void*>(pf::cast_f16_kernel),
        reinterpret_cast<const void*>(pf::gemm_kernel<kPfF32, 256, true>),
        reinterpret_cast<const void*>(pf::gemm_kernel<kPfResid, 256, true>),
        reinterpret_cast<const void*>(pf::gemm_kernel<kPfSwiglu, 256, true>),
        reinterpret_cast<const void*>(pf::dequant_kernel),
    };
    return i >= 0 && i < (int)(sizeof(k) / sizeof(k[0])) ? k[i] : nullptr;
}

// The split plan: with n tiles on num_cu compute units (one block each), a last
// round of t = n % num_cu tiles with 4 t <= min(num_cu, kPfSplitBlocks) is cut
// into split = min(that / t, 8, k tiles) ranges of k tiles.  (A last round over
// a quarter full was measured faster whole: its tiles run faster than a full
// round's, and the parts add partial-tile traffic and a second kernel.)
template <int BM>
static void gemm_plan(PfGemmArgs& a, uint32_t bn, uint32_t num_cu) {
    const uint32_t n_tiles = ((a.N + bn - 1) / bn) * ((a.M + BM - 1) / BM);
    a.n_full = n_tiles;
    a.split = 1;
    if (!a.part || num_cu == 0) return;
    const uint32_t slots = num_cu < kPfSplitBlocks ? num_cu : kPfSplitBlocks, tail = n_tiles % num_cu;
    if (tail == 0 || 4 * tail > slots) return;
    uint32_t split = slots / tail;
    if (split > 8) split = 8;
    if (split > a.K / pf::kBK) split = a.K / pf::kBK;
    if (split < 2) return;
    a.n_full = n_tiles - tail;
    a.split = split;
}

template <int MODE, int BM>
static hipError_t gemm_launch_mode(PfGemmArgs a, uint32_t num_cu, hipStream_t s) {
    const uint32_t bn = MODE == kPfSwiglu ? pf::kBN / 2 : pf::kBN;
    gemm_plan<BM>(a, bn, num_cu);
    const uint32_t n_tiles = ((a.N + bn - 1) / bn) * ((a.M + BM - 1) / BM), tail = n_tiles - a.n_full;
    if (a.wh[0])
        pf::gemm_kernel<MODE, BM, true><<<a.n_full + tail * a.split, 2 * BM, 0, s>>>(a);
    else
        pf::gemm_kernel<MODE, BM, false><<<a.n_full + tail * a.split, 2 * BM, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || tail == 0) return e;
    pf::gemm_reduce_kernel<MODE, BM><<<tail * (BM * pf::kBN / 4 / 256), 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t pf_gemm_launch(int mode, const PfGemmArgs& a, uint32_t num_cu, hipStream_t s) {
    if (a.M == 0) return hipSuccess;
    switch (mode) {
        case kPfF32: return gemm_launch_mode<kPfF32, 256>(a, num_cu, s);
        case kPfResid: return gemm_launch_mode<kPfResid, 256>(a, num_cu, s);
        case kPfSwiglu: return gemm_launch_mode<kPfSwiglu, 256>(a, num_cu, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t pf_dequant_launch(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                             uint32_t rows, uint32_t K, uint16_t* out, hipStream_t s) {
    const uint32_t n16 = rows * (K / 16);
    if (n16 == 0) return hipSuccess;
    pf::dequant_kernel<<<(n16 + 255) / 256, 256, 0, s>>>(codes, scales, biases, out, n16, K);
    return hipGetLastError();
}

hipError_t pf_rmsnorm_launch(const void* x, bool x_f32, const uint16_t* w, uint16_t* out, uint32_t T,
                             uint32_t H, float eps, hipStream_t s) {
    if (H <= 4 * 256)
        pf::rmsnorm_rows_kernel<4><<<T, 256, 0, s>>>(x, x_f32, w, out, H, eps);
    else if (H <= 8 * 256)
        pf::rmsnorm_rows_kernel<8><<<T, 256, 0, s>>>(x, x_f32, w, out, H, eps);
    else if (H <= 16 * 256)
        pf::rmsnorm_rows_kernel<16><<<T, 256, 0, s>>>(x, x_f32, w, out, H, eps);
    else if (H <= 32 * 256)
        pf::rmsnorm_rows_kernel<32><<<T, 256, 0, s>>>(x, x_f32, w, out, H, eps);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

bool pf_gdn_dims_supported(uint32_t dk, uint32_t dv) {
    return dk == dv && (dk == 32 || dk == 64 || dk == 128);
}

hipError_t pf_gdn_launch(const PfConvArgs& c, const PfGdnArgs& g, float* conv_state_out,
                         hipStream_t s) {
    pf::gdn_conv_kernel<<<8 * ((c.T + 7) / 8), 256, c.nqk * sizeof(float), s>>>(c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    pf::gdn_conv_state_kernel<<<(c.C + 255) / 256, 256, 0, s>>>(c.qkv, conv_state_out, c.T, c.C);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dim3 gc(g.nch, g.hv), gs(g.hv, g.dv / pf::kSL);
    switch (g.dk) {
        case 32:
            pf::gdn_chunk_kernel<32, 32><<<gc, 256, 0, s>>>(g);
            pf::gdn_scan_kernel<32><<<gs, 256, 0, s>>>(g);
            break;
        case 64:
            pf::gdn_chunk_kernel<64, 64><<<gc, 256, 0, s>>>(g);
            pf::gdn_scan_kernel<64><<<gs, 256, 0, s>>>(g);
            break;
        case 128:
            pf::gdn_chunk_kernel<128, 128><<<gc, 256, 0, s>>>(g);
            pf::gdn_scan_kernel<128><<<gs, 256, 0, s>>>(g);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t pf_gdn_out_launch(const float* y, const float* z, const uint16_t* w, uint16_t* yz,
                             uint32_t T, uint32_t hv, uint32_t dv, float eps, hipStream_t s) {
    if (dv > 128) return hipErrorInvalidValue;  // two values per lane
    pf::gdn_out_kernel<<<T, 256, 0, s>>>(y, z, w, yz, hv, dv, eps);
    return hipGetLastError();
}

bool pf_attn_dims_supported(uint32_t d, uint32_t g) {
    return (d == 64 || d == 128 || d == 256) && (g == 1 || g == 2 || g == 4 || g == 8);
}

hipError_t pf_attn_launch(const PfRopeArgs& r, const PfAttnArgs& a, hipStream_t s) {
    const size_t lds = ((size_t)(r.hq + r.hkv) * r.D + (r.hq + r.hkv) + r.rotary) * sizeof(float);
    pf::qk_rope_append_kernel<<<r.T, 256, lds, s>>>(r);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint32_t G = a.hq / a.hkv;
    dim3 grid((a.T + 31) / 32, a.hkv);
#define Q35_PF_FLASH(DD, GG)                                                  \
    if (r.D == DD && G == GG) {                                               \
        pf::flash_kernel<DD, GG><<<grid, 64 * GG * pf::flash_wph<DD, GG>(), 0, s>>>(a); \
        return hipGetLastError();                                             \
    }
    Q35_PF_FLASH(64, 1) Q35_PF_FLASH(64, 2) Q35_PF_FLASH(64, 4) Q35_PF_FLASH(64, 8)
    Q35_PF_FLASH(128, 1) Q35_PF_FLASH(128, 2) Q35_PF_FLASH(128, 4) Q35_PF_FLASH(128, 8)
    Q35_PF_FLASH(256, 1) Q35_PF_FLASH(256, 2) Q35_PF_FLASH(256, 4) Q35_PF_FLASH(256, 8)
#undef Q35_PF_FLASH
    return hipErrorInvalidValue;
}

}  // namespace q35
