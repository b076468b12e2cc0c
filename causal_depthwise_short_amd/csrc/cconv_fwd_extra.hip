// cconv_fwd_extra.hip -- the forward's packed-batch kernels (every (vec, group) pair, streaming
// options), its epilogue variants (no activation, residual; the default launch only: 4
// channels per lane, 16-row groups, one-wave solo blocks), and the element-granular paths (two
// channels per lane for D = 2 mod 4, one for any D), fixed-length and packed.
#include "cconv_fwd_body.hpp"

namespace cconv {

namespace {

template <int VEC, int G, int W, int F, bool VL, bool SOLO>
hipError_t launch_k(dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    if constexpr (SOLO)
        hipLaunchKernelGGL((cconv_fwd_kernel_solo<VEC, G, W, F, VL>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((cconv_fwd_kernel<VEC, G, W, F, VL>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int VEC, int G, int W, int F, bool VL>
hipError_t launch_k2(bool solo, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    return solo ? launch_k<VEC, G, W, F, VL, true>(grid, block, a, s) : launch_k<VEC, G, W, F, VL, false>(grid, block, a, s);
}

// packed, plain epilogue: both kernels for every (vec, group)
template <int VEC, int G>
hipError_t launch_vl(int W, bool solo, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    constexpr int F = kVarlenFwdOptions;
    switch (W) {
        case 1: return launch_k2<VEC, G, 1, F, true>(solo, grid, block, a, s);
        case 2: return launch_k2<VEC, G, 2, F, true>(solo, grid, block, a, s);
        case 3: return launch_k2<VEC, G, 3, F, true>(solo, grid, block, a, s);
        case 4: return launch_k2<VEC, G, 4, F, true>(solo, grid, block, a, s);
        default: return hipErrorInvalidValue;
    }
}

// epilogue variants: the default launch, solo kernel only
template <int W, bool VL>
hipError_t launch_epi_w(int epi, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    constexpr int B0 = kVarlenFwdOptions;
    switch (epi) {
        case kLinear: return launch_k<4, 16, W, B0 | kLinear, VL, true>(grid, block, a, s);
        case kResidual: return launch_k<4, 16, W, B0 | kResidual, VL, true>(grid, block, a, s);
        case kLinear | kResidual: return launch_k<4, 16, W, B0 | kLinear | kResidual, VL, true>(grid, block, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool VL>
hipError_t launch_epi(int W, int epi, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    switch (W) {
        case 1: return launch_epi_w<1, VL>(epi, grid, block, a, s);
        case 2: return launch_epi_w<2, VL>(epi, grid, block, a, s);
        case 3: return launch_epi_w<3, VL>(epi, grid, block, a, s);
        case 4: return launch_epi_w<4, VL>(epi, grid, block, a, s);
        default: return hipErrorInvalidValue;
    }
}

// element-granular D: one or two channels per lane, 16-row groups, the general kernel, plain
// loads and stores, every epilogue, fixed-length or packed
template <int VEC, int W, bool VL>
hipError_t launch_narrow_w(int epi, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    constexpr int B0 = kNarrowOptions;
    switch (epi) {
        case 0: return launch_k<VEC, 16, W, B0, VL, false>(grid, block, a, s);
        case kLinear: return launch_k<VEC, 16, W, B0 | kLinear, VL, false>(grid, block, a, s);
        case kResidual: return launch_k<VEC, 16, W, B0 | kResidual, VL, false>(grid, block, a, s);
        case kLinear | kResidual: return launch_k<VEC, 16, W, B0 | kLinear | kResidual, VL, false>(grid, block, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int VEC, bool VL>
hipError_t launch_narrow(int W, int epi, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    switch (W) {
        case 1: return launch_narrow_w<VEC, 1, VL>(epi, grid, block, a, s);
        case 2: return launch_narrow_w<VEC, 2, VL>(epi, grid, block, a, s);
        case 3: return launch_narrow_w<VEC, 3, VL>(epi, grid, block, a, s);
        case 4: return launch_narrow_w<VEC, 4, VL>(epi, grid, block, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool fwd_launch_exists(int vec, int group, int options, bool packed) {
    if (!fwd_variant_exists(vec, group) || options < 0) return false;
    const int epi = options & (kLinear | kResidual);
    const int base = options & ~(kSolo | kLinear | kResidual);
    if (options & ~(kSolo | kLinear | kResidual | kNtLoad | kNtStore | kPrefetch)) return false;
    if (vec <= 2) return !(options & kSolo) && base == kNarrowOptions;
    if (epi == 0) return packed ? base == kVarlenFwdOptions : true;
    return vec == 4 && group == 16 && (options & kSolo) && base == kVarlenFwdOptions;
}

hipError_t launch_fwd_extra(const Plan& p, int W, const FwdArgs& a, hipStream_t s) {
    const bool vl = a.cu != nullptr;
    if (!fwd_launch_exists(p.vec, p.group, p.options, vl)) return hipErrorInvalidValue;
    const dim3 grid(static_cast<uint32_t>(p.blocks)), block(static_cast<uint32_t>(p.waves * kWave));
    const int epi = p.options & (kLinear | kResidual);
    const bool solo = (p.options & kSolo) != 0;
    if (p.vec == 1)
        return vl ? launch_narrow<1, true>(W, epi, grid, block, a, s) : launch_narrow<1, false>(W, epi, grid, block, a, s);
    if (p.vec == 2)
        return vl ? launch_narrow<2, true>(W, epi, grid, block, a, s) : launch_narrow<2, false>(W, epi, grid, block, a, s);
    if (epi) return vl ? launch_epi<true>(W, epi, grid, block, a, s) : launch_epi<false>(W, epi, grid, block, a, s);
    if (p.vec == 8) {
        if (p.group == 4) return launch_vl<8, 4>(W, solo, grid, block, a, s);
        if (p.group == 8) return launch_vl<8, 8>(W, solo, grid, block, a, s);
    } else if (p.vec == 4) {
        if (p.group == 4) return launch_vl<4, 4>(W, solo, grid, block, a, s);
        if (p.group == 8) return launch_vl<4, 8>(W, solo, grid, block, a, s);
        if (p.group == 16) return launch_vl<4, 16>(W, solo, grid, block, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace cconv
