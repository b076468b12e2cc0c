// cconv_fwd.hip -- the plain forward in every launch variant, and the forward's dispatch.
// Packed batches and the epilogue variants are instantiated in cconv_fwd_extra.hip.
#include "cconv_fwd_body.hpp"

namespace cconv {

namespace {

template <int VEC, int G, int W>
hipError_t launch_fwd_f(int F, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
#define CCONV_FWD_CASE(f, vl)                                                                        \
    case f: hipLaunchKernelGGL((cconv_fwd_kernel<VEC, G, W, f, vl>), grid, block, 0, s, a); break;     \
    case f + kSolo: hipLaunchKernelGGL((cconv_fwd_kernel_solo<VEC, G, W, f, vl>), grid, block, 0, s, a); break;
    switch (F) {
        CCONV_FWD_CASE(0, false)
        CCONV_FWD_CASE(1, false)
        CCONV_FWD_CASE(2, false)
        CCONV_FWD_CASE(3, false)
        CCONV_FWD_CASE(4, false)
        CCONV_FWD_CASE(5, false)
        CCONV_FWD_CASE(6, false)
        CCONV_FWD_CASE(7, false)
        default: return hipErrorInvalidValue;
    }
#undef CCONV_FWD_CASE
    return hipGetLastError();
}

template <int VEC, int G>
hipError_t launch_fwd_w(int W, int F, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    switch (W) {
        case 1: return launch_fwd_f<VEC, G, 1>(F, grid, block, a, s);
        case 2: return launch_fwd_f<VEC, G, 2>(F, grid, block, a, s);
        case 3: return launch_fwd_f<VEC, G, 3>(F, grid, block, a, s);
        case 4: return launch_fwd_f<VEC, G, 4>(F, grid, block, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool fwd_variant_exists(int vec, int group) {
    return (vec == 8 && (group == 4 || group == 8)) || (vec == 4 && (group == 4 || group == 8 || group == 16)) ||
           ((vec == 1 || vec == 2) && group == 16);
}

hipError_t launch_fwd(const Plan& p, int W, const FwdArgs& a, hipStream_t s) {
    if (a.cu || p.vec <= 2 || (p.options & (kLinear | kResidual))) return launch_fwd_extra(p, W, a, s);
    const dim3 grid(static_cast<uint32_t>(p.blocks)), block(static_cast<uint32_t>(p.waves * kWave));
    const int F = p.options;
    if (p.vec == 8) {
        if (p.group == 4) return launch_fwd_w<8, 4>(W, F, grid, block, a, s);
        if (p.group == 8) return launch_fwd_w<8, 8>(W, F, grid, block, a, s);
    } else if (p.vec == 4) {
        if (p.group == 4) return launch_fwd_w<4, 4>(W, F, grid, block, a, s);
        if (p.group == 8) return launch_fwd_w<4, 8>(W, F, grid, block, a, s);
        if (p.group == 16) return launch_fwd_w<4, 16>(W, F, grid, block, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace cconv
