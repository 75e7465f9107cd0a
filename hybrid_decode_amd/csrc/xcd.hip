// XCD-split decode kernel (gfx950).
//
// MI355X has 8 XCDs of 32 CUs, each with its own L2.  The workgroups of a
// dispatch go to the XCDs in turn: block b of a grid of one block per CU runs
// on XCD (b + c) % 8, c depending on earlier dispatches, so each XCD holds the
// 32 blocks of one residue class of b mod 8.  A block takes its share of the
// work from the XCD it finds itself on (the hardware register XCC_ID) and its
// rank b / 8 within it, and the 32 blocks of one XCD meet at a counter in their
// shared L2, where a grid-wide signal or a kernel boundary costs more.  This kernel runs the steps of a layer
// whose work splits by XCD without any exchange between XCDs inside one launch:
//   * the GDN mixer (linear_attention.rs page: input RMSNorm, in-projection,
//     conv + SiLU, decay gate and beta, the gated delta rule, the gated
//     RMSNorm, out-projection): XCD x owns v-heads [Hv/8 x, Hv/8 (x+1)) and
//     the k-heads they read, i.e. their rows of q, k, v, z, a, b, their conv
//     channels, their recurrence state, and the out-projection's input columns
//     of those heads, whose product is a partial sum of the output;
//   * the SwiGLU MLP: XCD x owns rows [I/8 x, I/8 (x+1)) of gate and up, and
//     the matching input columns of down (a partial sum again).
// A stage's output that the next stage reads comes from blocks of the same
// XCD: plain stores, then, after the counter, device-coherent loads (the sc1
// policy).  Measured on MI355X: loads with only the L1-bypass hint (sc0), or
// plain loads after an L1 invalidate, can return stale data here; sc1 loads of
// plainly stored data do not.  The eight partial sums go to
// the next launch, whose prologue adds them to the residual base (kernel
// boundaries make them visible to every XCD).
//
// Synchronisation.  After a stage each block waits for its stores
// (s_waitcnt), meets its waves at a barrier, and one thread adds 1 to its
// XCD's counter with a workgroup-scope atomic (performed in the XCD's L2).
// Before the next stage's inputs are read that thread polls the counter (with
// atomics, see XSync::wait) until
// it reaches the next multiple of the XCD's block count; the counter is never
// cleared, and every launch adds the same number per block to it, so a
// multiple of the block count separates launches.  The next stage's first
// weights are requested before the poll, so the wait overlaps their transfer.
// Every wait is bounded in time; on expiry the error word records it and the
// block stops waiting, so the grid always drains.  A block that finds itself on
// The placement (one residue class of b mod 8 per XCD) is checked when a plan
// is created; a block that reads an XCD id past the eighth records
// Q35_STATUS_XCD_MAP and works as block b % 8 would.
#include "gdn_tile.h"
#include "gemv_core.h"
#include "q35decode.h"
#include "q35_device.h"
#include "q35_internal.h"

namespace q35 {
namespace {

constexpr int kXT = kXcdThreads;
constexpr int kXW = kXT / 64;
constexpr int kPoll = (kXW - 1) * 64;  // the polling thread: lane 0 of the last wave
// More than half of a CU's 160 KB of LDS: at most one block per CU.
constexpr int kXcdLds = 84 * 1024;

Q35_DEV uint32_t xcc_id() {
    // s_getreg_b32 of HW_REG_XCC_ID (hardware register 20), bits [3:0]
    return __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (15 << 11)) & 0xFu;
}

struct XSync {
    uint32_t* ctr;
    uint32_t* err;
    uint64_t spin;
    uint32_t nb;
    uint32_t old;
    bool failed;

    // This block has finished a stage: its stores are complete, then it counts in.
    Q35_DEV void arrive() {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid_x() == kPoll) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    // Every block of the XCD has counted in.
    Q35_DEV void wait() {
        if (tid_x() == kPoll && !failed) {
            const uint32_t target = (old / nb + 1u) * nb;
            const uint64_t t0 = wall_clock64();
            for (;;) {
                // read the counter with an atomic (an opaque zero added), performed in the
                // XCD's L2 like the increments: a plain or L1-bypass-hinted load can keep
                // returning the CU's cached copy
                uint32_t zero = 0;
                asm volatile("" : "+v"(zero));
                const uint32_t v = __hip_atomic_fetch_add(ctr, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if ((int32_t)(v - target) >= 0) break;
                if (wall_clock64() - t0 > spin) {
                    failed = true;
                    __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
    }
};

struct Shape4B {  // hidden 2560, intermediate 9216, z_dim 4096, dk = dv 128, bf16 activations
    static constexpr int H = 2560, I = 9216, ZD = 4096, DK = 128;
    static constexpr bool HALF = true;
};

// Common start of both launches: the placement probe, the XCD check, the sync state.
struct XBlock {
    uint32_t x, r, nb, rg, nw;
    XSync sy;

    Q35_DEV bool init(const XcdArgs& p) {
        const uint32_t hw = __builtin_amdgcn_readfirstlane(xcc_id());
        x = hw < kXcds ? hw : blockIdx.x % kXcds;
        r = blockIdx.x / kXcds;
        nb = gridDim.x / kXcds;
        if (p.probe) {  // placement probe: the same grid, no stages
            if (tid_x() == 0) p.probe[blockIdx.x] = hw;
            return false;
        }
        if (tid_x() == 0 && hw >= kXcds)
            __hip_atomic_fetch_or(p.err, Q35_STATUS_XCD_MAP, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sy.ctr = p.sync + 64u * x;
        sy.err = p.err;
        sy.spin = p.spin_ticks;
        sy.nb = nb;
        sy.old = 0u;
        sy.failed = false;
        // row group g of the XCD's share goes to wave g / nb of the XCD's block g % nb
        const uint32_t wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
        rg = wave * nb + r;
        nw = nb * kXW;
        return true;
    }

    // stage s's arguments for this block's XCD; the table is read-only for the
    // launch, so its fields are read with scalar loads where they are used
    Q35_DEV const XStage& stage(const XcdArgs& p, uint32_t s) const {
        typedef const __attribute__((address_space(4))) XStage CStage;
        return *(const XStage*)((CStage*)p.table + s * kXcds + x);
    }
};

// The GDN mixer: in-projection (kXsInGdn), recurrence (kXsGdn), out-projection
// partial (kXsOutPart).
template <class Sh>
__global__ __launch_bounds__(kXT) void xcd_mixer_kernel(XcdArgs p) {
    __shared__ __align__(16) uint4 xlds[kXcdLds / 16];
    XBlock b;
    if (!b.init(p)) return;
    auto w = [&] { b.sy.wait(); };
    gemv::gemv_body<Sh::H, kOpInGdnX, Sh::HALF, false, kXT, 0>(b.stage(p, 0).g, b.rg, b.nw, [] {},
                                                             blockIdx.x == 0, xlds);
    b.sy.arrive();
    gdn_tile<Sh::DK, 2>(b.stage(p, 1).d, b.x * b.nb + b.r, reinterpret_cast<uint8_t*>(xlds), w);
    b.sy.arrive();
    gemv::gemv_body<Sh::ZD / kXcds, kOpOutPart, Sh::HALF, false, kXT, 2, Sh::ZD>(b.stage(p, 2).g, b.rg, b.nw, w,
                                                                               b.r == 0, xlds);
}

// The MLP: gate/up (kXsGateUp), down partial (kXsDownPart).
template <class Sh>
__global__ __launch_bounds__(kXT) void xcd_mlp_kernel(XcdArgs p) {
    __shared__ __align__(16) uint4 xlds[kXcdLds / 16];
    XBlock b;
    if (!b.init(p)) return;
    auto w = [&] { b.sy.wait(); };
    gemv::gemv_body<Sh::H, kOpGateUpX, Sh::HALF, false, kXT, 0>(b.stage(p, 0).g, b.rg, b.nw, [] {},
                                                              blockIdx.x == 0, xlds);
    b.sy.arrive();
    gemv::gemv_body<Sh::I / kXcds, kOpDownPart, Sh::HALF, false, kXT, 2, Sh::I>(b.stage(p, 1).g, b.rg, b.nw, w,
                                                                              b.r == 0, xlds);
}

__global__ __launch_bounds__(256) void xsum_kernel(const void* base, int base_f32, const float* parts,
                                                   uint32_t nparts, uint32_t n, void* out, int out_f32) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    float v = load_act(base, i, base_f32 != 0);
    for (uint32_t k = 0; k < nparts; ++k) v += parts[(size_t)k * n + i];
    store_act(out, i, v, out_f32 != 0);
}

}  // namespace

int xcd_shape_id(uint32_t hidden, uint32_t inter, uint32_t z_dim, uint32_t dk, bool half) {
    return (hidden == Shape4B::H && inter == Shape4B::I && z_dim == Shape4B::ZD && dk == Shape4B::DK &&
            half == Shape4B::HALF)
               ? 1
               : 0;
}

const void* xcd_kernel_ptr(int shape, int launch) {
    if (shape != 1) return nullptr;
    return launch == kXcdMixer ? (const void*)&xcd_mixer_kernel<Shape4B>
         : launch == kXcdMlp   ? (const void*)&xcd_mlp_kernel<Shape4B>
                               : nullptr;
}

hipError_t xcd_launch(int shape, int launch, const XcdArgs& a, uint32_t blocks, hipStream_t stream) {
    if (shape != 1) return hipErrorInvalidValue;
    if (launch == kXcdMixer)
        hipLaunchKernelGGL(xcd_mixer_kernel<Shape4B>, dim3(blocks), dim3(kXT), 0, stream, a);
    else if (launch == kXcdMlp)
        hipLaunchKernelGGL(xcd_mlp_kernel<Shape4B>, dim3(blocks), dim3(kXT), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}


hipError_t xsum_launch(const void* base, bool base_f32, const float* parts, uint32_t nparts, uint32_t n,
                       void* out, bool out_f32, hipStream_t stream) {
    hipLaunchKernelGGL(xsum_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, base, base_f32 ? 1 : 0, parts,
                       nparts, n, out, out_f32 ? 1 : 0);
    return hipGetLastError();
}

const void* xsum_kernel_ptr() { return (const void*)&xsum_kernel; }

}  // namespace q35
