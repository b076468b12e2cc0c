// roofline_copy.hip -- flat streaming copies used as the measured bandwidth roofline.
// Each thread moves `U` 16-byte vectors; a block covers a contiguous span of
// threads*U vectors, so every load and store instruction of a wave is one coalesced 1 KB.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cconv_roofline.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 ld(const uint4* p) {
    if constexpr (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st(uint4* p, uint4 v) {
    if constexpr (NT) {
        const u32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    } else {
        *p = v;
    }
}

template <int U, bool TWO, bool NT>
__global__ __launch_bounds__(1024) void copy_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                    uint4* __restrict__ dst, int64_t n) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x * U + threadIdx.x;
    uint4 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * blockDim.x;
        if (i < n) {
            va[u] = ld<NT>(a + i);
            if constexpr (TWO) vb[u] = ld<NT>(b + i);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * blockDim.x;
        if (i < n) {
            uint4 v = va[u];
            if constexpr (TWO) v = make_uint4(v.x ^ vb[u].x, v.y ^ vb[u].y, v.z ^ vb[u].z, v.w ^ vb[u].w);
            st<NT>(dst + i, v);
        }
    }
}

// Persistent grid-stride copy: a fixed grid (a few blocks per CU) walks the buffer in chunks of
// blockDim*U vectors, each thread with U 16-byte loads in flight before its stores, so the
// bytes in flight per wave are set by U rather than by how many blocks the hardware has
// dispatched.
template <int U, bool TWO, bool NT>
__global__ __launch_bounds__(1024) void copy_persistent_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                               uint4* __restrict__ dst, int64_t n) {
    const int64_t chunk = static_cast<int64_t>(blockDim.x) * U;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * chunk + threadIdx.x; base < n;
         base += static_cast<int64_t>(gridDim.x) * chunk) {
        uint4 va[U], vb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * blockDim.x;
            if (i < n) {
                va[u] = ld<NT>(a + i);
                if constexpr (TWO) vb[u] = ld<NT>(b + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * blockDim.x;
            if (i < n) {
                uint4 v = va[u];
                if constexpr (TWO) v = make_uint4(v.x ^ vb[u].x, v.y ^ vb[u].y, v.z ^ vb[u].z, v.w ^ vb[u].w);
                st<NT>(dst + i, v);
            }
        }
    }
}

template <int U, bool TWO>
void launch_persistent(dim3 g, dim3 blk, bool nt, const uint4* a, const uint4* b, uint4* d, int64_t n, hipStream_t s) {
    if (nt)
        hipLaunchKernelGGL((copy_persistent_kernel<U, TWO, true>), g, blk, 0, s, a, b, d, n);
    else
        hipLaunchKernelGGL((copy_persistent_kernel<U, TWO, false>), g, blk, 0, s, a, b, d, n);
}

template <int U, bool TWO>
void launch(dim3 g, dim3 blk, bool nt, const uint4* a, const uint4* b, uint4* d, int64_t n, hipStream_t s) {
    if (nt)
        hipLaunchKernelGGL((copy_kernel<U, TWO, true>), g, blk, 0, s, a, b, d, n);
    else
        hipLaunchKernelGGL((copy_kernel<U, TWO, false>), g, blk, 0, s, a, b, d, n);
}

}  // namespace

extern "C" int cconv_roofline_copy(int kind, const void* a, const void* b, void* dst, int64_t bytes, int unroll,
                                   int threads, int nontemporal, struct ihipStream_t* stream) {
    if ((kind != 1 && kind != 2) || !a || !dst || (kind == 2 && !b)) return 1;
    if (bytes < 0 || bytes % 16 != 0) return 1;
    if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(dst) |
         (kind == 2 ? reinterpret_cast<uintptr_t>(b) : 0)) % 16 != 0)
        return 1;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return 1;
    if (threads != 256 && threads != 512 && threads != 1024) return 1;
    const int64_t n = bytes / 16;
    if (n == 0) return 0;
    const int64_t per_block = static_cast<int64_t>(threads) * unroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > INT32_MAX) return 1;
    const dim3 g(static_cast<uint32_t>(blocks)), blk(threads);
    const auto* pa = static_cast<const uint4*>(a);
    const auto* pb = static_cast<const uint4*>(b);
    auto* pd = static_cast<uint4*>(dst);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool nt = nontemporal != 0;
    const bool two = kind == 2;
    switch (unroll) {
        case 1: two ? launch<1, true>(g, blk, nt, pa, pb, pd, n, s) : launch<1, false>(g, blk, nt, pa, pb, pd, n, s); break;
        case 2: two ? launch<2, true>(g, blk, nt, pa, pb, pd, n, s) : launch<2, false>(g, blk, nt, pa, pb, pd, n, s); break;
        case 4: two ? launch<4, true>(g, blk, nt, pa, pb, pd, n, s) : launch<4, false>(g, blk, nt, pa, pb, pd, n, s); break;
        case 8: two ? launch<8, true>(g, blk, nt, pa, pb, pd, n, s) : launch<8, false>(g, blk, nt, pa, pb, pd, n, s); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int cconv_roofline_copy_persistent(int kind, const void* a, const void* b, void* dst, int64_t bytes,
                                              int blocks, int unroll, int threads, int nontemporal,
                                              struct ihipStream_t* stream) {
    if ((kind != 1 && kind != 2) || !a || !dst || (kind == 2 && !b)) return 1;
    if (bytes < 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65536) return 1;
    if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(dst) |
         (kind == 2 ? reinterpret_cast<uintptr_t>(b) : 0)) % 16 != 0)
        return 1;
    if (unroll != 2 && unroll != 4 && unroll != 8) return 1;
    if (threads != 256 && threads != 512 && threads != 1024) return 1;
    const int64_t n = bytes / 16;
    if (n == 0) return 0;
    const dim3 g(static_cast<uint32_t>(blocks)), blk(threads);
    const auto* pa = static_cast<const uint4*>(a);
    const auto* pb = static_cast<const uint4*>(b);
    auto* pd = static_cast<uint4*>(dst);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool nt = nontemporal != 0;
    const bool two = kind == 2;
    switch (unroll) {
        case 2: two ? launch_persistent<2, true>(g, blk, nt, pa, pb, pd, n, s) : launch_persistent<2, false>(g, blk, nt, pa, pb, pd, n, s); break;
        case 4: two ? launch_persistent<4, true>(g, blk, nt, pa, pb, pd, n, s) : launch_persistent<4, false>(g, blk, nt, pa, pb, pd, n, s); break;
        case 8: two ? launch_persistent<8, true>(g, blk, nt, pa, pb, pd, n, s) : launch_persistent<8, false>(g, blk, nt, pa, pb, pd, n, s); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
