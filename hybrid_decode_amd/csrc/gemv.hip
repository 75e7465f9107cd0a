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
    (void)paired;  // a paired row group holds the same rows of both matrices
    return 64 / gcd_i(64, (int)k / 16);
}

// Launch shape.  The streaming GEMVs (plain, lm_head) and the GDN
// in-projection get about three waves per four row groups of 256-thread blocks
// when they fit in the chip's resident waves: every wave has its first row
// group in flight from the start and a third of them stream a second one;
// long streams (the lm_head) use all resident waves with many row groups
// each.  The other per-layer GEMVs run one 640-thread block per compute unit,
// each wave taking about two row groups in turn.  Measured on MI355X inside
// the 32-layer stack (us per launch, 256-thread shape -> per-CU shape):
// gate/up 11.55 -> 10.5-10.8, out_proj 5.39 -> 4.66, o_proj 4.67 -> 4.43,
// down and q/k/v unchanged, GDN in-projection 9.43 -> 10.43 (6176 row groups:
// some waves run three in turn), so it keeps the 256-thread shape.  Row groups
// stay contiguous within a block: interleaving them over the CUs balances the
// rounds but measured slower for every GEMV (DRAM page and TLB locality).
constexpr uint32_t kResidentWaves = 256u * 32u;

uint32_t gemv_row_groups_per_wave(uint32_t total_rg) {
    return total_rg <= kResidentWaves ? 1u : (total_rg + kResidentWaves - 1) / kResidentWaves;
}

uint32_t gemv_pick_blocks(uint32_t total_rg, int op, uint32_t num_cu) {
    const uint32_t wpb = (uint32_t)gemv_threads(op) / 64;
    uint32_t blocks;
    if (gemv_threads(op) == kGemvLayerThreads) {
        blocks = (total_rg + wpb - 1) / wpb;  // fewer blocks than CUs only for small matrices
        if (blocks > num_cu) blocks = num_cu;
    } else {
        const uint32_t rgw = gemv_row_groups_per_wave(total_rg);
        const uint32_t waves = rgw == 1u ? (3u * total_rg + 3u) / 4u : (total_rg + rgw - 1) / rgw;
        blocks = (waves + wpb - 1) / wpb;
    }
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
        case kOpInFull:
        case kOpInFullP: return gemv_launch_in(op, k, half, xreg, a, blocks, stream);
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
        case kOpInFull:
        case kOpInFullP: return gemv_ptr_in(op, k, half, xreg);
        case kOpOutGated:
        case kOpOProj: return gemv_ptr_out(op, k, half, xreg);
        case kOpGateUp:
        case kOpDown: return gemv_ptr_mlp(op, k, half, xreg);
        case kOpLmHead: return gemv_ptr_lm(op, k, half, xreg);
        default: return nullptr;
    }
}

}  // namespace q35
