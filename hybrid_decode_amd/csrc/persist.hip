// Persistent decode kernel (gfx950): one cooperative launch runs a whole token
// through the layer stack, stage after stage, with no kernel boundary between
// the steps of the pages' two layer forwards (linear_attention.rs and
// full_attention.rs pages: the in-projection, conv, gate/beta, gated delta
// rule, gated norm + out-projection; the q/k/v projections, q/k norm, RoPE,
// KV append, attention_decode, sigmoid_gate, o-projection; then the shared
// SwiGLU MLP) nor between layers, then the lm_head and greedy token.
//
// Why.  At batch 1 every step is a short HBM stream (a few to 50 MB) and a
// launch per step pays a ramp-up and a tail of several microseconds each.
// Here one block runs on each CU for the whole token.  Stage s of every block
// first issues the loads that do not depend on this token (its first row group
// of weights, the GDN state tile, the first K/V rows), then waits until every
// block has finished stage s-1, then reads its inputs and computes: the wait
// overlaps with weight streaming instead of leaving HBM idle.
//
// Synchronisation.  Each block owns one flag word; after a stage it waits for
// its own stores to complete (s_waitcnt), meets its waves at a barrier and
// stores base + s + 1 into its flag.  A waiting block's first wave polls all
// flags with one coherent load per lane until each is >= base + s (wrapping
// comparison).  base = epoch * nstages, and the epoch word advances by one per
// launch (block 0 bumps it after the last stage), so flags never need
// clearing.  Every exchange between blocks goes through device-coherent loads
// and stores (the sc1 policy of agent-scope atomics), so no stage pays an L2
// write-back or invalidate.  Every wait is bounded in time: on expiry the
// block records an error word and stops waiting, so the grid always drains;
// the host reports the error.  The grid is one block per CU and launched
// cooperatively, so all blocks are resident together.
#include "gdn_tile.h"
#include "gemv_core.h"
#include "q35decode.h"
#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace {

constexpr int kPT = kPersistThreads;  // threads per block
constexpr int kPW = kPT / 64;         // waves per block

// ------------------------------------------------------------------ grid sync

// Only a few words live across stages; everything else is re-read from the
// kernel arguments where it is used (few registers stay occupied across the
// stage switch).
//
// The flag is stored as soon as the block's stores of a stage are complete,
// before any of the next stage's weight loads are issued: a CU's vector memory
// requests are served in order, so a flag store or poll issued behind a large
// prefetch would wait for it.
struct PSync {
    const PersistArgs* p;
    uint32_t base;
    bool failed;

    Q35_DEV void init(const PersistArgs& args) {
        p = &args;
        failed = false;
        const uint32_t e = __hip_atomic_load(args.ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        base = __builtin_amdgcn_readfirstlane(e * args.nstages);
    }

    // All blocks have finished stage s - 1 (stage 0 reads only what earlier
    // launches wrote).
    Q35_DEV void wait(uint32_t s) {
        if (s > 0 && tid_x() < 64 && !failed) {
            const uint32_t target = base + s;
            const uint32_t nblocks = gridDim.x;
            const auto rf = rsrc(p->flags, nblocks * 4u);
            const uint32_t lane = tid_x();
            const uint64_t t0 = wall_clock64();
            for (;;) {
                bool ok = true;
                for (uint32_t b0 = 0; b0 < nblocks; b0 += 256) {
                    // flags past nblocks read as zero and are skipped
                    const uint4 f = ld_b128<kAuxCoherent>(rf, (b0 + 4u * lane) * 4u);
                    const uint32_t b = b0 + 4u * lane;
                    ok &= b + 0 >= nblocks || (int32_t)(f.x - target) >= 0;
                    ok &= b + 1 >= nblocks || (int32_t)(f.y - target) >= 0;
                    ok &= b + 2 >= nblocks || (int32_t)(f.z - target) >= 0;
                    ok &= b + 3 >= nblocks || (int32_t)(f.w - target) >= 0;
                }
                if (__ballot(!ok) == 0) break;
                if (wall_clock64() - t0 > p->spin_ticks) {
                    failed = true;
                    if (lane == 0) __hip_atomic_fetch_or(p->ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        if (p->stamps && blockIdx.x == 0 && tid_x() == 0) p->stamps[s] = wall_clock64();
        __syncthreads();
    }

    // This block has finished stage s: its stores are complete, then its flag moves.
    Q35_DEV void arrive(uint32_t s) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid_x() == 0)
            __hip_atomic_store(p->flags + blockIdx.x, base + s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

// ------------------------------------------------------------------ GEMV stages

template <int K, int OP, bool HALF, bool XREG>
Q35_DEV void st_gemv(const GemvArgs& a, PSync& sy, uint32_t s, uint8_t* lds) {
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
    // row group r goes to wave r / gridDim.x of block r % gridDim.x: every CU gets
    // the same share of every stage
    gemv::gemv_body<K, OP, HALF, XREG, kPT, 1>(a, wave * gridDim.x + blockIdx.x, gridDim.x * kPW,
                                               [&] { sy.wait(s); }, blockIdx.x == 0,
                                               reinterpret_cast<uint4*>(lds));
    sy.arrive(s);
}

// ------------------------------------------------------------------ gated delta rule (gdn_tile.h)

template <int DK>
Q35_DEV void st_gdn(const GdnArgs& a, PSync& sy, uint32_t s, uint8_t* lds) {
    gdn_tile<DK, 1>(a, blockIdx.x, lds, [&] { sy.wait(s); });
    sy.arrive(s);
}

// ------------------------------------------------------------------ attention

// Split-K decode attention for one (chunk, kv head) item per block, as the
// standalone partial kernel: each block reads its K/V rows once for the G query
// heads of its group (GQA reuse), row slots of D/4 lanes run an online softmax
// in the base-2 exponent and merge in LDS; the block holding the new position
// builds q and k (RMSNorm, RoPE), stores the bf16 K/V row and attends to it from
// LDS.  The chunk length follows the live length: chunks per head = blocks / Hkv.
constexpr int kAU = 2;   // rows per row slot per batch (two batches in flight)
constexpr int kEPL = 4;  // dims per lane: a 256-dim row is one wave (1024 threads leave 128 VGPRs)
constexpr float kLog2e = 1.4426950408889634f;

Q35_DEV void unpack4(const uint2& u, float v[4]) {
    v[0] = bf16_lo(u.x);
    v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y);
    v[3] = bf16_hi(u.y);
}

struct AttnSplit {
    uint32_t L, T, nch;
    bool valid;
};

Q35_DEV AttnSplit attn_split(const AttnArgs& a) {
    AttnSplit sp;
    const int32_t pos = a.positions[0];  // written by an earlier launch
    sp.valid = pos >= 0 && (uint32_t)pos < a.capacity;
    sp.L = sp.valid ? (uint32_t)pos + 1 : 1u;
    const uint32_t cpb = a.max_chunks;  // chunks per kv head
    sp.T = (sp.L + cpb - 1) / cpb;
    sp.nch = (sp.L + sp.T - 1) / sp.T;
    return sp;
}

template <int D, int G>
Q35_DEV void st_attn(const AttnArgs& a, PSync& sy, uint32_t s, uint8_t* lds) {
    constexpr int LPR = D / kEPL, RPI = kPT / LPR, B = RPI * kAU;
    static_assert(LPR <= 64 && 64 % LPR == 0, "a row spans a power-of-two lane group of one wave");
    static_assert(D <= kPT, "one new-v element per thread");
    float* qs = reinterpret_cast<float*>(lds);  // [(G+1)*D] q heads, then the new k
    float* vn = qs + (G + 1) * D;               // [D]
    float* rsq = vn + D;                        // [8]
    float2* rot = reinterpret_cast<float2*>(rsq + 8);  // [D/2]
    float* mls = reinterpret_cast<float*>(rot + D / 2);  // [RPI][2G]
    float* red = mls + RPI * 2 * G;                      // [RPI][D]

    const int t = tid_x(), lane = t & 63, wid = t >> 6;
    const int j = t % LPR, rs = t / LPR;
    const AttnSplit sp = attn_split(a);
    const int32_t pos = a.positions[0];
    const uint32_t g = blockIdx.x % a.hkv;
    const uint32_t c = blockIdx.x / a.hkv;
    const bool work = sp.valid && c < sp.nch;  // block-uniform
    const uint32_t t0 = c * sp.T;
    const uint32_t t1 = min(t0 + sp.T, sp.L);
    const bool has_new = work && (uint32_t)pos >= t0 && (uint32_t)pos < t1;

    const uint32_t row_bytes = a.hkv * D * 2u;
    const uint32_t span = work ? (t1 - t0) * row_bytes : 0u;
    const auto rk = rsrc(a.kc + ((size_t)t0 * a.hkv + g) * D, span);
    const auto rv = rsrc(a.vc + ((size_t)t0 * a.hkv + g) * D, span);
    uint2 kr[2][kAU], vr[2][kAU];
    auto load_batch = [&](uint2 (&kd)[kAU], uint2 (&vd)[kAU], uint32_t tb) {
#pragma unroll
        for (int u = 0; u < kAU; ++u) {
            const uint32_t tt = tb + u * RPI + rs;
            const bool live = tt < t1 && tt != (uint32_t)pos;
            const uint32_t off = live ? (tt - t0) * row_bytes + 2u * kEPL * j : span;  // past the end: zero
            kd[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, kAuxStream));
            vd[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, kAuxStream));
        }
    };
    if (work) {  // cache rows of earlier positions: ready before this token's inputs
        load_batch(kr[0], vr[0], t0);
        load_batch(kr[1], vr[1], t0 + B);
    }
    sy.wait(s);
    if (work) {
        constexpr int PQ = ((G + 1) * D + kPT - 1) / kPT;
        float qv[PQ], nv[PQ];
#pragma unroll
        for (int r = 0; r < PQ; ++r) {
            const int e = min(t + kPT * r, (G + 1) * D - 1);
            const int i = e / D, d = e % D;
            qv[r] = (i < G) ? ld_coh_f32(a.q_full, (g * G + i) * 2 * D + d) : ld_coh_f32(a.k, g * D + d);
            nv[r] = bf16_to_f32((i < G) ? a.q_norm[d] : a.k_norm[d]);
        }
        const float vnew = ld_coh_f32(a.v, g * D + min(t, D - 1));
        const float invf = a.inv_freq[min(t, (int)a.rotary / 2 - 1)];
#pragma unroll
        for (int r = 0; r < PQ; ++r)
            if (t + kPT * r < (G + 1) * D) qs[t + kPT * r] = qv[r];
        if (t < D) vn[t] = bf16_to_f32(f32_to_bf16(vnew));
        if (t < (int)a.rotary / 2) {
            float sn, cs;
            sincosf((float)pos * invf, &sn, &cs);
            rot[t] = make_float2(cs, sn);
        }
        __syncthreads();
        for (int i = wid; i < G + 1; i += kPW) {
            float ss = 0.f;
            for (int d = lane; d < D; d += 64) ss = fmaf(qs[i * D + d], qs[i * D + d], ss);
            ss = wave_sum(ss);
            if (lane == 0) rsq[i] = 1.0f / sqrtf(ss / (float)D + a.eps);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PQ; ++r) {
            const int e = t + kPT * r;
            if (e < (G + 1) * D) qs[e] = qs[e] * rsq[e / D] * nv[r];
        }
        __syncthreads();
        {
            const int half = (int)a.rotary / 2;
            for (int e = t; e < (G + 1) * half; e += kPT) {
                const int i = e / half, d = e % half;
                const float cs = rot[d].x, sn = rot[d].y;
                const float x1 = qs[i * D + d], x2 = qs[i * D + d + half];
                qs[i * D + d] = x1 * cs - x2 * sn;
                qs[i * D + d + half] = x2 * cs + x1 * sn;
            }
        }
        __syncthreads();
        if (has_new) {
            // the new row, as stored, is attended to from LDS; later launches read it
            uint16_t* krow = a.kc + ((size_t)pos * a.hkv + g) * D;
            uint16_t* vrow = a.vc + ((size_t)pos * a.hkv + g) * D;
            for (int d = t; d < D; d += kPT) {
                const uint32_t kb = f32_to_bf16(qs[G * D + d]);
                krow[d] = (uint16_t)kb;
                vrow[d] = (uint16_t)f32_to_bf16(vn[d]);
                qs[G * D + d] = bf16_to_f32(kb);
            }
            __syncthreads();
        }

        float qr[G][kEPL];
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int e = 0; e < kEPL; ++e) qr[i][e] = qs[i * D + kEPL * j + e];
        const float sscale = a.scale * kLog2e;
        float m[G], l[G], acc[G][kEPL];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            m[i] = -INFINITY;
            l[i] = 0.f;
#pragma unroll
            for (int e = 0; e < kEPL; ++e) acc[i][e] = 0.f;
        }
        auto batch = [&](const uint2 (&kd)[kAU], const uint2 (&vd)[kAU], uint32_t tb) {
            float sc[kAU][G];
#pragma unroll
            for (int u = 0; u < kAU; ++u) {
                const uint32_t tt = tb + u * RPI + rs;
                float kv[kEPL];
                if (tt == (uint32_t)pos) {
#pragma unroll
                    for (int e = 0; e < kEPL; ++e) kv[e] = qs[G * D + kEPL * j + e];
                } else {
                    unpack4(kd[u], kv);
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < kEPL; ++e) d = fmaf(qr[i][e], kv[e], d);
                    d = group_sum_all<LPR>(d);
                    sc[u][i] = tt < t1 ? d * sscale : -INFINITY;
                }
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                float mx = m[i];
#pragma unroll
                for (int u = 0; u < kAU; ++u) mx = fmaxf(mx, sc[u][i]);
                const float mref = mx == -INFINITY ? 0.f : mx;
                const float corr = exp2f(m[i] - mref);
                m[i] = mx;
                l[i] *= corr;
#pragma unroll
                for (int e = 0; e < kEPL; ++e) acc[i][e] *= corr;
#pragma unroll
                for (int u = 0; u < kAU; ++u) sc[u][i] = exp2f(sc[u][i] - mref);
            }
#pragma unroll
            for (int u = 0; u < kAU; ++u) {
                const uint32_t tt = tb + u * RPI + rs;
                float vv[kEPL];
                if (tt == (uint32_t)pos) {
#pragma unroll
                    for (int e = 0; e < kEPL; ++e) vv[e] = vn[kEPL * j + e];
                } else {
                    unpack4(vd[u], vv);
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    l[i] += sc[u][i];
#pragma unroll
                    for (int e = 0; e < kEPL; ++e) acc[i][e] = fmaf(sc[u][i], vv[e], acc[i][e]);
                }
            }
        };
        for (uint32_t tb = t0;; tb += 2 * B) {
            batch(kr[0], vr[0], tb);
            if (tb + B >= t1) break;
            load_batch(kr[0], vr[0], tb + 2 * B);
            batch(kr[1], vr[1], tb + B);
            if (tb + 2 * B >= t1) break;
            load_batch(kr[1], vr[1], tb + 3 * B);
        }

        if (j == 0)
#pragma unroll
            for (int i = 0; i < G; ++i) {
                mls[rs * 2 * G + 2 * i] = m[i];
                mls[rs * 2 * G + 2 * i + 1] = l[i];
            }
        __syncthreads();
        float* pacc = a.part_acc + ((size_t)g * a.max_chunks + c) * G * D;
        float* pml = a.part_ml + ((size_t)g * a.max_chunks + c) * 2 * G;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float M = -INFINITY;
            for (int r = 0; r < RPI; ++r) M = fmaxf(M, mls[r * 2 * G + 2 * i]);  // slot 0 always has a row
            const float w = exp2f(m[i] - M);
#pragma unroll
            for (int e = 0; e < kEPL; ++e) red[rs * D + kEPL * j + e] = acc[i][e] * w;
            __syncthreads();
            for (int d = t; d < D; d += kPT) {
                float o = 0.f;
#pragma unroll 8
                for (int r = 0; r < RPI; ++r) o += red[r * D + d];
                st_f32<true>(pacc, i * D + d, o);
            }
            if (t == 0) {
                float tot = 0.f;
                for (int r = 0; r < RPI; ++r)
                    tot = fmaf(exp2f(mls[r * 2 * G + 2 * i] - M), mls[r * 2 * G + 2 * i + 1], tot);
                st_f32<true>(pml, 2 * i, M);
                st_f32<true>(pml, 2 * i + 1, tot);
            }
            __syncthreads();
        }
    }
    sy.arrive(s);
}

// Log-sum-exp merge of the chunk partials and the sigmoid gate: one wave per
// output element (q head h, dim d), its lanes over the chunks.
template <int D, int G>
Q35_DEV void st_merge(const AttnArgs& a, PSync& sy, uint32_t s) {
    sy.wait(s);
    const AttnSplit sp = attn_split(a);
    const int lane = tid_x() & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
    const uint32_t nout = a.hq * D;
    if (sp.valid) {
        for (uint32_t o = wave * gridDim.x + blockIdx.x; o < nout; o += gridDim.x * kPW) {
            const uint32_t h = o / D, d = o % D, g = h / G, i = h % G;
            float m = -INFINITY, l = 0.f, acc = 0.f;
            for (uint32_t c = lane; c < sp.nch; c += 64) {
                const size_t pi = (size_t)g * a.max_chunks + c;
                const float mc = ld_coh_f32(a.part_ml, pi * 2 * G + 2 * i);
                const float lc = ld_coh_f32(a.part_ml, pi * 2 * G + 2 * i + 1);
                const float ac = ld_coh_f32(a.part_acc, pi * G * D + i * D + d);
                const float mn = fmaxf(m, mc);
                const float f0 = m == -INFINITY ? 0.f : exp2f(m - mn);
                const float f1 = exp2f(mc - mn);
                l = l * f0 + lc * f1;
                acc = acc * f0 + ac * f1;
                m = mn;
            }
            const float M = wave_max(m);
            const float f = m == -INFINITY ? 0.f : exp2f(m - M);
            const float lt = wave_sum(l * f);
            const float at = wave_sum(acc * f);
            if (lane == 0) {
                const float out = at / lt;
                if (a.attn_out) a.attn_out[h * D + d] = out;
                const float gate = ld_coh_f32(a.q_full, h * 2 * D + D + d);
                st_f32<true>(a.gated_attn, h * D + d, out * sigmoidf_(gate));
            }
        }
    } else {
        // positions[0] outside the cache: no attention this step.  The output is
        // zero and the error word records it (q35_decode_check reports it).
        for (uint32_t o = wave * gridDim.x + blockIdx.x; o < nout; o += gridDim.x * kPW)
            if (lane == 0) {
                if (a.attn_out) a.attn_out[o] = 0.f;
                st_f32<true>(a.gated_attn, o, 0.f);
            }
        if (blockIdx.x == 0 && tid_x() == 0)
            __hip_atomic_fetch_or(sy.p->ctl + 1, Q35_STATUS_POS_RANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sy.arrive(s);
}

// ------------------------------------------------------------------ token finish

Q35_DEV bool better_tok(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Block 0: greedy token from the lm_head's per-block partials, history entry,
// position increment, next token's embedding row into the first layer's input.
Q35_DEV void st_finish(const LmFinishArgs& a, PSync& sy, uint32_t s, uint8_t* lds) {
    if (blockIdx.x != 0) return;
    sy.wait(s);
    float* sv = reinterpret_cast<float*>(lds);
    int* si = reinterpret_cast<int*>(sv + kPW);
    int* tok_sh = si + kPW;
    const int t = tid_x();
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (uint32_t b = t; b < a.nparts; b += kPT) {
        const float v = ld_coh_f32(a.part_val, b);
        const int ix = ld_coh_i32(a.part_idx, b);
        if (better_tok(v, ix, bv, bi)) {
            bv = v;
            bi = ix;
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (better_tok(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    const int lane = t & 63, wid = t >> 6;
    if (lane == 0) {
        sv[wid] = bv;
        si[wid] = bi;
    }
    __syncthreads();
    if (t == 0) {
        for (int w = 1; w < kPW; ++w)
            if (better_tok(sv[w], si[w], sv[0], si[0])) {
                sv[0] = sv[w];
                si[0] = si[w];
            }
        const int tok = (si[0] >= 0 && (uint32_t)si[0] < a.vocab) ? si[0] : 0;
        *tok_sh = tok;
        a.tokens[0] = tok;
        const int pos = a.positions[0];
        if (a.history) {
            const int hidx = pos - a.history_base;
            if (hidx >= 0 && (uint32_t)hidx < a.history_len) a.history[hidx] = tok;
        }
        a.positions[0] = pos + 1;
    }
    __syncthreads();
    const uint4* row = reinterpret_cast<const uint4*>(a.embed + (size_t)(*tok_sh) * a.hidden);
    const bool f32 = a.act_f32 != 0;
    for (uint32_t c = t; c < a.hidden / 8; c += kPT) {
        const uint4 u = row[c];
        if (f32) {
            float4* o = reinterpret_cast<float4*>(a.x_next) + 2 * c;
            o[0] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
            o[1] = make_float4(bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w));
        } else {
            reinterpret_cast<uint4*>(a.x_next)[c] = u;
        }
    }
}

// ------------------------------------------------------------------ the kernel

// Compile-time shapes the persistent kernel is built for (GEMV widths, head sizes).
struct Shape4B {  // hidden 2560, intermediate 9216, q_only = z_dim 4096, dk 128, D 256, G 4, bf16
    static constexpr int H = 2560, I = 9216, QO = 4096, ZD = 4096, DK = 128, D = 256, G = 4;
    static constexpr bool HALF = true;
};
struct ShapeTiny {  // hidden 256, intermediate 512, q_only 256, z_dim 128, dk 32, D 64, G 2, fp32
    static constexpr int H = 256, I = 512, QO = 256, ZD = 128, DK = 32, D = 64, G = 2;
    static constexpr bool HALF = false;
};

template <class Sh>
__global__ __launch_bounds__(kPT) void persist_kernel(PersistArgs p) {
    extern __shared__ uint4 psmem[];
    uint8_t* lds = reinterpret_cast<uint8_t*>(psmem);
    PSync sy;
    sy.init(p);
    // The stage table is read-only for the whole launch: reading it through the
    // constant address space lets the compiler use scalar loads and re-load
    // fields where they are used instead of holding them in registers.
    typedef const __attribute__((address_space(4))) PStage CStage;
    CStage* cst = (CStage*)p.stages;
    for (uint32_t s = 0; s < p.nstages; ++s) {
        const PStage& st = *(const PStage*)(cst + s);
        const int kind = __builtin_amdgcn_readfirstlane(st.kind);
        switch (kind) {
            case kStInGdn: st_gemv<Sh::H, kOpInGdn, Sh::HALF, false>(st.g, sy, s, lds); break;
            case kStGdn: st_gdn<Sh::DK>(st.d, sy, s, lds); break;
            case kStOutGated: st_gemv<Sh::ZD, kOpOutGated, Sh::HALF, false>(st.g, sy, s, lds); break;
            case kStInFull: st_gemv<Sh::H, kOpInFull, Sh::HALF, false>(st.g, sy, s, lds); break;
            case kStAttn: st_attn<Sh::D, Sh::G>(st.at, sy, s, lds); break;
            case kStAttnMerge: st_merge<Sh::D, Sh::G>(st.at, sy, s); break;
            case kStOProj: st_gemv<Sh::QO, kOpOProj, Sh::HALF, false>(st.g, sy, s, lds); break;
            case kStGateUp: st_gemv<Sh::H, kOpGateUp, Sh::HALF, false>(st.g, sy, s, lds); break;
            case kStDown: st_gemv<Sh::I, kOpDown, Sh::HALF, false>(st.g, sy, s, lds); break;
            case kStLmHead: st_gemv<Sh::H, kOpLmHead, Sh::HALF, true>(st.g, sy, s, lds); break;
            case kStFinish: st_finish(st.f, sy, s, lds); break;
            default: break;
        }
    }
    // every block read the epoch before its first arrival, and block 0 has seen
    // all blocks arrive at least once since: the next launch may use the next one
    if (blockIdx.x == 0 && tid_x() == 0) {
        const uint32_t e = __hip_atomic_load(p.ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ctl, e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <class Sh>
constexpr size_t persist_lds() {
    constexpr size_t g1 = gemv::lds_bytes<Sh::H, Sh::HALF>(), g2 = gemv::lds_bytes<Sh::I, Sh::HALF>(),
                     g3 = gemv::lds_bytes<Sh::QO, Sh::HALF>(), g4 = gemv::lds_bytes<Sh::ZD, Sh::HALF>();
    constexpr int RPI = kPT / (Sh::D / kEPL);
    constexpr size_t at = sizeof(float) * ((Sh::G + 1) * Sh::D + Sh::D + 8 + Sh::D + RPI * 2 * Sh::G + RPI * Sh::D);
    constexpr size_t gd = sizeof(float) * (kCT + 3 * 4 + 32 * kCT);
    size_t m = g1;
    m = m > g2 ? m : g2;
    m = m > g3 ? m : g3;
    m = m > g4 ? m : g4;
    m = m > at ? m : at;
    m = m > gd ? m : gd;
    return (m + 255) & ~size_t(255);
}

}  // namespace

int persist_shape_id(uint32_t hidden, uint32_t inter, uint32_t q_only, uint32_t z_dim, uint32_t dk,
                     uint32_t head_dim, uint32_t group, bool half) {
    if (hidden == Shape4B::H && inter == Shape4B::I && q_only == Shape4B::QO && z_dim == Shape4B::ZD &&
        dk == Shape4B::DK && head_dim == Shape4B::D && group == Shape4B::G && half == Shape4B::HALF)
        return 1;
    if (hidden == ShapeTiny::H && inter == ShapeTiny::I && q_only == ShapeTiny::QO &&
        z_dim == ShapeTiny::ZD && dk == ShapeTiny::DK && head_dim == ShapeTiny::D &&
        group == ShapeTiny::G && half == ShapeTiny::HALF)
        return 2;
    return 0;
}

size_t persist_lds_bytes(int shape) {
    return shape == 1 ? persist_lds<Shape4B>() : shape == 2 ? persist_lds<ShapeTiny>() : 0;
}

const void* persist_kernel_ptr(int shape) {
    return shape == 1 ? (const void*)&persist_kernel<Shape4B>
         : shape == 2 ? (const void*)&persist_kernel<ShapeTiny>
                      : nullptr;
}

hipError_t persist_launch(int shape, const PersistArgs& a, uint32_t blocks, hipStream_t stream) {
    const void* f = persist_kernel_ptr(shape);
    if (!f) return hipErrorInvalidValue;
    void* args[] = {const_cast<PersistArgs*>(&a)};
    return hipLaunchCooperativeKernel(f, dim3(blocks), dim3(kPT), args,
                                      (unsigned int)persist_lds_bytes(shape), stream);
}

}  // namespace q35
