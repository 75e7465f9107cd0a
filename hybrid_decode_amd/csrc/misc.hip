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

}  // namespace

hipError_t embed_launch(const uint16_t* table, const int32_t* tokens, uint32_t vocab,
                        uint32_t hidden, void* x_out, bool act_f32, hipStream_t stream) {
    const uint32_t blocks = (hidden + 255) / 256;
    hipLaunchKernelGGL(embed_kernel, dim3(blocks), dim3(256), 0, stream, table, tokens, vocab,
                       hidden, x_out, act_f32 ? 1 : 0);
    return hipGetLastError();
}

const void* embed_kernel_ptr() { return (const void*)&embed_kernel; }

}  // namespace q35
