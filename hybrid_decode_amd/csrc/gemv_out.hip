// GEMV instantiations: kOpOutGated, kOpOProj.
#include "gemv_core.h"

namespace q35 {

hipError_t gemv_launch_out(int op, uint32_t k, bool half, bool xreg, const GemvArgs& a,
                          uint32_t blocks, hipStream_t stream) {
    (void)xreg;
    if (op == kOpOutGated) {
#define X(KK)                                                                              \
        if (k == KK) return half ? gemv::launch_t<KK, kOpOutGated, true, false>(a, blocks, stream) \
                                 : gemv::launch_t<KK, kOpOutGated, false, false>(a, blocks, stream);
        Q35_W_PROJ(X)
#undef X
    }
    if (op == kOpOProj) {
#define X(KK)                                                                              \
        if (k == KK) return half ? gemv::launch_t<KK, kOpOProj, true, false>(a, blocks, stream) \
                                 : gemv::launch_t<KK, kOpOProj, false, false>(a, blocks, stream);
        Q35_W_PROJ(X)
#undef X
    }
    return hipErrorInvalidValue;
}

const void* gemv_ptr_out(int op, uint32_t k, bool half, bool xreg) {
    (void)xreg;
    if (op == kOpOutGated) {
#define X(KK)                                                                           \
        if (k == KK) return half ? gemv::kernel_ptr_t<KK, kOpOutGated, true, false>()          \
                                 : gemv::kernel_ptr_t<KK, kOpOutGated, false, false>();
        Q35_W_PROJ(X)
#undef X
    }
    if (op == kOpOProj) {
#define X(KK)                                                                           \
        if (k == KK) return half ? gemv::kernel_ptr_t<KK, kOpOProj, true, false>()          \
                                 : gemv::kernel_ptr_t<KK, kOpOProj, false, false>();
        Q35_W_PROJ(X)
#undef X
    }
    return nullptr;
}

}  // namespace q35
