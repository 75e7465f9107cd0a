// GEMV instantiations: kOpInGdn, kOpInFull, kOpInFullP.
#include "gemv_core.h"

namespace q35 {

hipError_t gemv_launch_in(int op, uint32_t k, bool half, bool xreg, const GemvArgs& a,
                          uint32_t blocks, hipStream_t stream) {
    (void)xreg;
    if (op == kOpInGdn) {
#define X(KK)                                                                              \
        if (k == KK) return half ? gemv::launch_t<KK, kOpInGdn, true, false>(a, blocks, stream) \
                                 : gemv::launch_t<KK, kOpInGdn, false, false>(a, blocks, stream);
        Q35_W_HIDDEN(X)
#undef X
    }
    if (op == kOpInFull) {
#define X(KK)                                                                              \
        if (k == KK) return half ? gemv::launch_t<KK, kOpInFull, true, false>(a, blocks, stream) \
                                 : gemv::launch_t<KK, kOpInFull, false, false>(a, blocks, stream);
        Q35_W_HIDDEN(X)
#undef X
    }
    if (op == kOpInFullP) {
#define X(KK)                                                                              \
        if (k == KK) return half ? gemv::launch_t<KK, kOpInFullP, true, false>(a, blocks, stream) \
                                 : gemv::launch_t<KK, kOpInFullP, false, false>(a, blocks, stream);
        Q35_W_PARTS(X)
#undef X
    }
    return hipErrorInvalidValue;
}

const void* gemv_ptr_in(int op, uint32_t k, bool half, bool xreg) {
    (void)xreg;
    if (op == kOpInGdn) {
#define X(KK)                                                                           \
        if (k == KK) return half ? gemv::kernel_ptr_t<KK, kOpInGdn, true, false>()          \
                                 : gemv::kernel_ptr_t<KK, kOpInGdn, false, false>();
        Q35_W_HIDDEN(X)
#undef X
    }
    if (op == kOpInFull) {
#define X(KK)                                                                           \
        if (k == KK) return half ? gemv::kernel_ptr_t<KK, kOpInFull, true, false>()          \
                                 : gemv::kernel_ptr_t<KK, kOpInFull, false, false>();
        Q35_W_HIDDEN(X)
#undef X
    }
    if (op == kOpInFullP) {
#define X(KK)                                                                           \
        if (k == KK) return half ? gemv::kernel_ptr_t<KK, kOpInFullP, true, false>()          \
                                 : gemv::kernel_ptr_t<KK, kOpInFullP, false, false>();
        Q35_W_PARTS(X)
#undef X
    }
    return nullptr;
}

}  // namespace q35
