// cconv_bwd.hip -- the plain backward in every launch variant, the backward's dispatch, and
// the fixed-order reduction of the dw/dbias partials. Packed batches and the variant without
// an activation are instantiated in cconv_bwd_extra.hip.
#include "cconv_bwd_body.hpp"

namespace cconv {

// dw[d, j] = sum_p partial[p, j, d] (j < W), dbias[d] = sum_p partial[p, W, d]. A block
// handles 64 consecutive (j, d) entries; its 4 waves each sum a contiguous quarter of the
// partials in ascending order, then the four sums are added in wave order. Loads are issued
// in batches of kBatch before they are summed, so a quarter of up to kBatch partials costs one
// memory latency. P == 0 writes zeros (an empty batch or sequence).
__global__ __launch_bounds__(256) void cconv_dw_reduce_kernel(const ReduceArgs a) {
    constexpr int kBatch = 16;
    __shared__ float part[4][kWave];
    if (a.status && *a.status != 0) return;  // the offset check failed: write nothing
    const int lane = threadIdx.x % kWave, q = threadIdx.x / kWave;
    const int64_t E = static_cast<int64_t>(a.W + 1) * a.D;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kWave + lane;
    float s = 0.0f;
    if (e < E) {
        const int64_t chunk = (a.P + 3) / 4;
        const int64_t p0 = q * chunk, p1 = min(a.P, p0 + chunk);
        const float* __restrict__ src = a.partial + e;
        for (int64_t p = p0; p < p1; p += kBatch) {
            float v[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) v[i] = (p + i < p1) ? src[(p + i) * E] : 0.0f;
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                if (p + i < p1) s += v[i];
        }
    }
    part[q][lane] = s;
    __syncthreads();
    if (q == 0 && e < E) {
        const float tot = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        const int64_t j = e / a.D, d = e % a.D;
        if (j < a.W) {
            if (a.dw_f32) {
                static_cast<float*>(a.dw)[d * a.W + j] = tot;
            } else {
                static_cast<uint16_t*>(a.dw)[d * a.W + j] = static_cast<uint16_t>(pack_bf16x2(tot, 0.0f) & 0xffffu);
            }
        } else if (a.dbias) {
            a.dbias[d] = tot;
        }
    }
}

namespace {

template <int VEC, int G, int W>
hipError_t launch_bwd_f(int F, dim3 grid, dim3 block, size_t lds, const BwdArgs& a, hipStream_t s) {
#define CCONV_BWD_CASE(f, vl)                                                                              \
    case f: hipLaunchKernelGGL((cconv_bwd_kernel<VEC, G, W, f, vl>), grid, block, lds, s, a); break;        \
    case f + kSolo: hipLaunchKernelGGL((cconv_bwd_kernel_solo<VEC, G, W, f, vl>), grid, block, lds, s, a); break;
    switch (F) {
        CCONV_BWD_CASE(0, false)
        CCONV_BWD_CASE(1, false)
        CCONV_BWD_CASE(2, false)
        CCONV_BWD_CASE(3, false)
        CCONV_BWD_CASE(4, false)
        CCONV_BWD_CASE(5, false)
        CCONV_BWD_CASE(6, false)
        CCONV_BWD_CASE(7, false)
        default: return hipErrorInvalidValue;
    }
#undef CCONV_BWD_CASE
    return hipGetLastError();
}

template <int VEC, int G>
hipError_t launch_bwd_w(int W, int F, dim3 grid, dim3 block, size_t lds, const BwdArgs& a, hipStream_t s) {
    switch (W) {
        case 1: return launch_bwd_f<VEC, G, 1>(F, grid, block, lds, a, s);
        case 2: return launch_bwd_f<VEC, G, 2>(F, grid, block, lds, a, s);
        case 3: return launch_bwd_f<VEC, G, 3>(F, grid, block, lds, a, s);
        case 4: return launch_bwd_f<VEC, G, 4>(F, grid, block, lds, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool bwd_variant_exists(int vec, int group) {
    return (vec == 8 && (group == 4 || group == 8)) || (vec == 4 && (group == 4 || group == 8 || group == 16)) ||
           ((vec == 1 || vec == 2) && group == 16);
}

hipError_t launch_bwd(const Plan& p, int W, const BwdArgs& a, hipStream_t s) {
    if (a.cu || p.vec <= 2 || (p.options & kLinear)) return launch_bwd_extra(p, W, a, s);
    const dim3 grid(static_cast<uint32_t>(p.blocks)), block(static_cast<uint32_t>(p.waves * kWave));
    const size_t lds = static_cast<size_t>(p.waves) * p.vec * kWave * sizeof(float);
    const int F = p.options;
    if (p.vec == 8) {
        if (p.group == 4) return launch_bwd_w<8, 4>(W, F, grid, block, lds, a, s);
        if (p.group == 8) return launch_bwd_w<8, 8>(W, F, grid, block, lds, a, s);
    } else if (p.vec == 4) {
        if (p.group == 4) return launch_bwd_w<4, 4>(W, F, grid, block, lds, a, s);
        if (p.group == 8) return launch_bwd_w<4, 8>(W, F, grid, block, lds, a, s);
        if (p.group == 16) return launch_bwd_w<4, 16>(W, F, grid, block, lds, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
    const int64_t E = static_cast<int64_t>(a.W + 1) * a.D;
    const int64_t blocks = (E + kWave - 1) / kWave;
    hipLaunchKernelGGL(cconv_dw_reduce_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace cconv
