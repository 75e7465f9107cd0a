// GEMV instantiations: kOpPlain.
#include "gemv_core.h"

namespace q35 {

hipError_t gemv_launch_plain(int op, uint32_t k, bool half, bool xreg, const GemvArgs& a,
                          uint32_t blocks, hipStream_t stream) {
    (void)xreg;
    if (op == kOpPlain) {
#define X(KK)                                                                                   \
        if (k == KK) {                                                                          \
            if (xreg) return half ? gemv::launch_t<KK, kOpPlain, true, true>(a, blocks, stream)     \
                                  : gemv::launch_t<KK, kOpPlain, false, true>(a, blocks, stream);   \
            return half ? gemv::launch_t<KK, kOpPlain, true, false>(a, blocks, stream)              \
                        : gemv::launch_t<KK, kOpPlain, false, false>(a, blocks, stream);            \
        }
        Q35_W_ALL(X)
#undef X
    }
    return hipErrorInvalidValue;
}

const void* gemv_ptr_plain(int op, uint32_t k, bool half, bool xreg) {
    (void)xreg;
    if (op == kOpPlain) {
#define X(KK)                                                                                   \
        if (k == KK) {                                                                          \
            if (xreg) return half ? gemv::kernel_ptr_t<KK, kOpPlain, true, true>()                  \
                                  : gemv::kernel_ptr_t<KK, kOpPlain, false, true>();                \
            return half ? gemv::kernel_ptr_t<KK, kOpPlain, true, false>()                           \
                        : gemv::kernel_ptr_t<KK, kOpPlain, false, false>();                         \
        }
        Q35_W_ALL(X)
#undef X
    }
    return nullptr;
}

}  // namespace q35
