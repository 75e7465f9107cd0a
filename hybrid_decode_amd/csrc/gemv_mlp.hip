// GEMV instantiations: kOpGateUp, kOpDown.
#include "gemv_core.h"

namespace q35 {

hipError_t gemv_launch_mlp(int op, uint32_t k, bool half, bool xreg, const GemvArgs& a,
                          uint32_t blocks, hipStream_t stream) {
    (void)xreg;
    if (op == kOpGateUp) {
#define X(KK)                                                                              \
        if (k == KK) return half ? gemv::launch_t<KK, kOpGateUp, true, false>(a, blocks, stream) \
                                 : gemv::launch_t<KK, kOpGateUp, false, false>(a, blocks, stream);
        Q35_W_HIDDEN(X)
#undef X
    }
    if (op == kOpDown) {
#define X(KK)                                                                              \
        if (k == KK) return half ? gemv::launch_t<KK, kOpDown, true, false>(a, blocks, stream) \
                                 : gemv::launch_t<KK, kOpDown, false, false>(a, blocks, stream);
        Q35_W_INTER(X)
#undef X
    }
    return hipErrorInvalidValue;
}

const void* gemv_ptr_mlp(int op, uint32_t k, bool half, bool xreg) {
    (void)xreg;
    if (op == kOpGateUp) {
#define X(KK)                                                                           \
        if (k == KK) return half ? gemv::kernel_ptr_t<KK, kOpGateUp, true, false>()          \
                                 : gemv::kernel_ptr_t<KK, kOpGateUp, false, false>();
        Q35_W_HIDDEN(X)
#undef X
    }
    if (op == kOpDown) {
#define X(KK)                                                                           \
        if (k == KK) return half ? gemv::kernel_ptr_t<KK, kOpDown, true, false>()          \
                                 : gemv::kernel_ptr_t<KK, kOpDown, false, false>();
        Q35_W_INTER(X)
#undef X
    }
    return nullptr;
}

}  // namespace q35
