// cconv_bwd_extra.hip -- the backward's packed-batch kernels (every (vec, group) pair,
// streaming options), its variant without an activation (g = dy; the default launch only: 4
// channels per lane, 16-row groups, one-wave solo blocks), and the element-granular paths (two
// channels per lane for D = 2 mod 4, one for any D), fixed-length and packed.
#include "cconv_bwd_body.hpp"

namespace cconv {

namespace {

template <int VEC, int G, int W, int F, bool VL, bool SOLO>
hipError_t launch_k(dim3 grid, dim3 block, size_t lds, const BwdArgs& a, hipStream_t s) {
    if constexpr (SOLO)
        hipLaunchKernelGGL((cconv_bwd_kernel_solo<VEC, G, W, F, VL>), grid, block, lds, s, a);
    else
        hipLaunchKernelGGL((cconv_bwd_kernel<VEC, G, W, F, VL>), grid, block, lds, s, a);
    return hipGetLastError();
}

// packed, with SiLU: both kernels for every (vec, group)
template <int VEC, int G>
hipError_t launch_vl(int W, bool solo, dim3 grid, dim3 block, size_t lds, const BwdArgs& a, hipStream_t s) {
    constexpr int F = kVarlenBwdOptions;
    switch (W) {
#define CCONV_VL(w)                                                                                \
    case w:                                                                                        \
        return solo ? launch_k<VEC, G, w, F, true, true>(grid, block, lds, a, s)                  \
                    : launch_k<VEC, G, w, F, true, false>(grid, block, lds, a, s);
        CCONV_VL(1)
        CCONV_VL(2)
        CCONV_VL(3)
        CCONV_VL(4)
#undef CCONV_VL
        default: return hipErrorInvalidValue;
    }
}

// no activation: the default launch, solo kernel only
template <bool VL>
hipError_t launch_lin(int W, dim3 grid, dim3 block, size_t lds, const BwdArgs& a, hipStream_t s) {
    constexpr int F = kVarlenBwdOptions | kLinear;
    switch (W) {
        case 1: return launch_k<4, 16, 1, F, VL, true>(grid, block, lds, a, s);
        case 2: return launch_k<4, 16, 2, F, VL, true>(grid, block, lds, a, s);
        case 3: return launch_k<4, 16, 3, F, VL, true>(grid, block, lds, a, s);
        case 4: return launch_k<4, 16, 4, F, VL, true>(grid, block, lds, a, s);
        default: return hipErrorInvalidValue;
    }
}

// element-granular D: one or two channels per lane, 16-row groups, the general kernel, plain
// loads and stores
template <int VEC, bool VL>
hipError_t launch_narrow(int W, bool lin, dim3 grid, dim3 block, size_t lds, const BwdArgs& a, hipStream_t s) {
    constexpr int F = kNarrowOptions;
    switch (W) {
#define CCONV_NARROW(w)                                                                            \
    case w:                                                                                        \
        return lin ? launch_k<VEC, 16, w, F | kLinear, VL, false>(grid, block, lds, a, s)         \
                   : launch_k<VEC, 16, w, F, VL, false>(grid, block, lds, a, s);
        CCONV_NARROW(1)
        CCONV_NARROW(2)
        CCONV_NARROW(3)
        CCONV_NARROW(4)
#undef CCONV_NARROW
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool bwd_launch_exists(int vec, int group, int options, bool packed) {
    if (!bwd_variant_exists(vec, group) || options < 0) return false;
    if (options & ~(kSolo | kLinear | kNtLoad | kNtStore | kPrefetch)) return false;
    const int base = options & ~(kSolo | kLinear);
    if (vec <= 2) return !(options & kSolo) && base == kNarrowOptions;
    if (!(options & kLinear)) return packed ? base == kVarlenBwdOptions : true;
    return vec == 4 && group == 16 && (options & kSolo) && base == kVarlenBwdOptions;
}

hipError_t launch_bwd_extra(const Plan& p, int W, const BwdArgs& a, hipStream_t s) {
    const bool vl = a.cu != nullptr;
    if (!bwd_launch_exists(p.vec, p.group, p.options, vl)) return hipErrorInvalidValue;
    const dim3 grid(static_cast<uint32_t>(p.blocks)), block(static_cast<uint32_t>(p.waves * kWave));
    const size_t lds = static_cast<size_t>(p.waves) * p.vec * kWave * sizeof(float);
    const bool solo = (p.options & kSolo) != 0;
    if (p.vec <= 2) {
        const bool lin = (p.options & kLinear) != 0;
        if (p.vec == 2)
            return vl ? launch_narrow<2, true>(W, lin, grid, block, lds, a, s)
                      : launch_narrow<2, false>(W, lin, grid, block, lds, a, s);
        return vl ? launch_narrow<1, true>(W, lin, grid, block, lds, a, s) : launch_narrow<1, false>(W, lin, grid, block, lds, a, s);
    }
    if (p.options & kLinear)
        return vl ? launch_lin<true>(W, grid, block, lds, a, s) : launch_lin<false>(W, grid, block, lds, a, s);
    if (p.vec == 8) {
        if (p.group == 4) return launch_vl<8, 4>(W, solo, grid, block, lds, a, s);
        if (p.group == 8) return launch_vl<8, 8>(W, solo, grid, block, lds, a, s);
    } else if (p.vec == 4) {
        if (p.group == 4) return launch_vl<4, 4>(W, solo, grid, block, lds, a, s);
        if (p.group == 8) return launch_vl<4, 8>(W, solo, grid, block, lds, a, s);
        if (p.group == 16) return launch_vl<4, 16>(W, solo, grid, block, lds, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace cconv
