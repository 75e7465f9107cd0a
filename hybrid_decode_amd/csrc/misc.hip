// Small stack-plumbing kernels (gfx950).
#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace {

// x_out = table[tokens[0]] (bf16 row -> activation dtype); zeros for an invalid token.
__global__ __launch_bounds__(256) void embed_kernel(const uint16_t* table, const int32_t* tokens,
                                                    uint32_t vocab, uint32_t hidden, void* x_out,
                                                    int act_f32) {
    const int32_t tok = tokens[0];
    const bool ok = tok >= 0 && (uint32_t)tok < vocab;
    const uint16_t* row = table + (size_t)(ok ? tok : 0) * hidden;
    for (uint32_t k = blockIdx.x * blockDim.x + threadIdx.x; k < hidden; k += gridDim.x * blockDim.x)
        store_act(x_out, k, ok ? bf16_to_f32(row[k]) : 0.0f, act_f32 != 0);
}

Q35_DEV bool better_tok(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

constexpr int kFinishThreads = 256;
constexpr int kFinishPer = 16;  // partials each thread loads before comparing

__global__ __launch_bounds__(kFinishThreads) void lm_finish_kernel(LmFinishArgs a) {
    __shared__ float sv[kFinishThreads / 64];
    __shared__ int si[kFinishThreads / 64];
    __shared__ int tok_sh;
    const int t = threadIdx.x;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    // all loads of a round are issued before any comparison
    for (uint32_t base = 0; base < a.nparts; base += kFinishThreads * kFinishPer) {
        float v[kFinishPer];
        int ix[kFinishPer];
#pragma unroll
        for (int r = 0; r < kFinishPer; ++r) {
            const uint32_t b = base + t + kFinishThreads * r;
            const bool in = b < a.nparts;
            v[r] = in ? a.part_val[b] : -INFINITY;
            ix[r] = in ? a.part_idx[b] : 0x7FFFFFFF;
        }
#pragma unroll
        for (int r = 0; r < kFinishPer; ++r)
            if (better_tok(v[r], ix[r], bv, bi)) {
                bv = v[r];
                bi = ix[r];
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
        for (int w = 1; w < kFinishThreads / 64; ++w)
            if (better_tok(sv[w], si[w], sv[0], si[0])) {
                sv[0] = sv[w];
                si[0] = si[w];
            }
        const int tok = (si[0] >= 0 && (uint32_t)si[0] < a.vocab) ? si[0] : 0;
        tok_sh = tok;
        a.tokens[0] = tok;
        const int pos = a.positions ? a.positions[0] : 0;
        if (a.history) {
            const int hidx = pos - a.history_base;
            if (hidx >= 0 && (uint32_t)hidx < a.history_len) a.history[hidx] = tok;
        }
        if (a.positions) a.positions[0] = pos + 1;
    }
    __syncthreads();
    if (a.embed) {
        // the next token's embedding row, 8 elements (16 bytes) per thread and step
        const uint4* row = reinterpret_cast<const uint4*>(a.embed + (size_t)tok_sh * a.hidden);
        const bool f32 = a.act_f32 != 0;
        for (uint32_t c = t; c < a.hidden / 8; c += kFinishThreads) {
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
}

}  // namespace

hipError_t lm_finish_launch(const LmFinishArgs& a, hipStream_t stream) {
    if (a.embed && (a.hidden % 8 != 0 || (reinterpret_cast<uintptr_t>(a.embed) & 15) ||
                    (reinterpret_cast<uintptr_t>(a.x_next) & 15)))
        return hipErrorInvalidValue;  // the row copy moves 16-byte words
    hipLaunchKernelGGL(lm_finish_kernel, dim3(1), dim3(kFinishThreads), 0, stream, a);
    return hipGetLastError();
}

const void* lm_finish_kernel_ptr() { return (const void*)&lm_finish_kernel; }

hipError_t embed_launch(const uint16_t* table, const int32_t* tokens, uint32_t vocab,
                        uint32_t hidden, void* x_out, bool act_f32, hipStream_t stream) {
    const uint32_t blocks = (hidden + 255) / 256;
    hipLaunchKernelGGL(embed_kernel, dim3(blocks), dim3(256), 0, stream, table, tokens, vocab,
                       hidden, x_out, act_f32 ? 1 : 0);
    return hipGetLastError();
}

const void* embed_kernel_ptr() { return (const void*)&embed_kernel; }

// Fixed workspace of the entry points that allocate nothing: each GPU the
// library runs on holds one copy until the process ends.  Host code never
// passes this name to a kernel (on the host it is a stand-in, not a device
// address); static_scratch_address gives the device address, once per device,
// with that device current.
constexpr size_t kStaticScratchBytes = 64 * 1024;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch_address(void** ptr, size_t* bytes) {
    *ptr = nullptr;
    *bytes = kStaticScratchBytes;
    return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch));
}

}  // namespace q35
