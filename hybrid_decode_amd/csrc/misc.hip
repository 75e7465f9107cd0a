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

__global__ __launch_bounds__(256) void lm_finish_kernel(LmFinishArgs a) {
    __shared__ float sv[4];
    __shared__ int si[4];
    __shared__ int tok_sh;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (uint32_t b = threadIdx.x; b < a.nparts; b += blockDim.x) {
        const float v = a.part_val[b];
        const int i = a.part_idx[b];
        if (better_tok(v, i, bv, bi)) {
            bv = v;
            bi = i;
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
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wid] = bv;
        si[wid] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w)
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
        const uint16_t* row = a.embed + (size_t)tok_sh * a.hidden;
        for (uint32_t k = threadIdx.x; k < a.hidden; k += blockDim.x)
            store_act(a.x_next, k, bf16_to_f32(row[k]), a.act_f32 != 0);
    }
}

}  // namespace

hipError_t lm_finish_launch(const LmFinishArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(lm_finish_kernel, dim3(1), dim3(256), 0, stream, a);
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

}  // namespace q35
