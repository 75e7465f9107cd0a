// GEMV launch geometry and dispatch to the per-operation instantiations.
#include "q35_internal.h"

namespace q35 {

namespace {
constexpr int gcd_i(int a, int b) { return b == 0 ? a : gcd_i(b, a % b); }
}  // namespace

hipError_t gemv_launch_plain(int, uint32_t, bool, bool, const GemvArgs&, uint32_t, hipStream_t);
hipError_t gemv_launch_in(int, uint32_t, bool, bool, const GemvArgs&, uint32_t, hipStream_t);
hipError_t gemv_launch_out(int, uint32_t, bool, bool, const GemvArgs&, uint32_t, hipStream_t);
hipError_t gemv_launch_mlp(int, uint32_t, bool, bool, const GemvArgs&, uint32_t, hipStream_t);
hipError_t gemv_launch_lm(int, uint32_t, bool, bool, const GemvArgs&, uint32_t, hipStream_t);
const void* gemv_ptr_plain(int, uint32_t, bool, bool);
const void* gemv_ptr_in(int, uint32_t, bool, bool);
const void* gemv_ptr_out(int, uint32_t, bool, bool);
const void* gemv_ptr_mlp(int, uint32_t, bool, bool);
const void* gemv_ptr_lm(int, uint32_t, bool, bool);

int gemv_rows_per_matrix_group(uint32_t k, bool paired) {
    const int kc = (int)k / 16;
    return paired ? 32 / gcd_i(32, kc) : 64 / gcd_i(64, kc);
}

// Row groups per wave: one while the whole launch fits in the resident waves
// (all of its weights requested at once), more for long streams (the lm_head).
uint32_t gemv_row_groups_per_wave(uint32_t total_rg) {
    const uint32_t resident = 256u * 32u;
    return total_rg <= resident ? 1u : (total_rg + resident - 1) / resident;
}

uint32_t gemv_pick_blocks(uint32_t total_rg) {
    const uint32_t rgw = gemv_row_groups_per_wave(total_rg);
    const uint32_t waves = (total_rg + rgw - 1) / rgw;
    const uint32_t blocks = (waves + 3) / 4;
    return blocks ? blocks : 1;
}

bool gemv_width_supported(int role, uint32_t k) {
    switch (role) {
        case kWidthHidden:
#define X(KK) if (k == KK) return true;
            Q35_W_HIDDEN(X)
            return false;
        case kWidthProj:
            Q35_W_PROJ(X)
            return false;
        case kWidthInter:
            Q35_W_INTER(X)
            return false;
        default:
            Q35_W_ALL(X)
#undef X
            return false;
    }
}

static bool op_xreg(int op, uint32_t total_rg) {
    return (op == kOpPlain || op == kOpLmHead) && gemv_row_groups_per_wave(total_rg) >= 4;
}

hipError_t gemv_launch(int op, uint32_t k, bool half, const GemvArgs& a, uint32_t blocks,
                       hipStream_t stream) {
    const bool xreg = op_xreg(op, a.total_rg);
    switch (op) {
        case kOpPlain: return gemv_launch_plain(op, k, half, xreg, a, blocks, stream);
        case kOpInGdn:
        case kOpInFull: return gemv_launch_in(op, k, half, xreg, a, blocks, stream);
        case kOpOutGated:
        case kOpOProj: return gemv_launch_out(op, k, half, xreg, a, blocks, stream);
        case kOpGateUp:
        case kOpDown: return gemv_launch_mlp(op, k, half, xreg, a, blocks, stream);
        case kOpLmHead: return gemv_launch_lm(op, k, half, xreg, a, blocks, stream);
        default: return hipErrorInvalidValue;
    }
}

const void* gemv_kernel_ptr(int op, uint32_t k, bool half, bool xreg) {
    switch (op) {
        case kOpPlain: return gemv_ptr_plain(op, k, half, xreg);
        case kOpInGdn:
        case kOpInFull: return gemv_ptr_in(op, k, half, xreg);
        case kOpOutGated:
        case kOpOProj: return gemv_ptr_out(op, k, half, xreg);
        case kOpGateUp:
        case kOpDown: return gemv_ptr_mlp(op, k, half, xreg);
        case kOpLmHead: return gemv_ptr_lm(op, k, half, xreg);
        default: return nullptr;
    }
}

}  // namespace q35
