// cconv_seq.hip -- bookkeeping kernels for packed variable-length batches (fla's cu_seqlens
// parameter, kernel-fun wheel, _common/compat.py FLA_KWARGS row for causal_conv1d).
//
// The offsets live on the device, so the host cannot check them: one block checks
// cu[0] = 0 <= cu[1] <= ... <= cu[n] = total and writes the verdict to a status word, which
// every later kernel of the call reads before it writes anything. Empty sequences hold no row,
// so no streaming wave meets them: the same block then gives them their final state (the
// history, or zeros) and a zero history gradient.
#include "../../include/cconv.h"
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

namespace cconv {

// One block: the verdict on the offsets, then (when it is good and states are asked for) the
// empty sequences' state rows: their final state is their history (or zeros), their history
// gradient zero. The second pass gathers a chunk's empty sequences into an LDS list and writes
// each one's [D, L] rows with all threads; its order does not matter, the rows being disjoint.
__global__ __launch_bounds__(1024) void cconv_offsets_kernel(const int32_t* cu, int64_t n, int64_t total,
                                                             int32_t* status, const uint16_t* h0, uint16_t* hT,
                                                             uint16_t* dh0, int64_t D, int L) {
    __shared__ int32_t list[1024];
    __shared__ int count;
    bool bad = false;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x)
        if (cu[i] > cu[i + 1]) bad = true;
    if (threadIdx.x == 0 && (cu[0] != 0 || static_cast<int64_t>(cu[n]) != total)) bad = true;
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) status[0] = bad ? CCONV_ERR_INDEX : CCONV_OK;
    if (bad || (!hT && !dh0) || D <= 0 || L <= 0) return;
    const int64_t E = D * L;
    for (int64_t base = 0; base < n; base += blockDim.x) {
        if (threadIdx.x == 0) count = 0;
        __syncthreads();
        const int64_t i = base + threadIdx.x;
        if (i < n && cu[i] == cu[i + 1]) list[atomicAdd(&count, 1)] = static_cast<int32_t>(threadIdx.x);
        __syncthreads();
        const int c = count;
        for (int j = 0; j < c; ++j) {
            const int64_t q = base + list[j];
            for (int64_t e = threadIdx.x; e < E; e += blockDim.x) {
                if (hT) hT[q * E + e] = h0 ? h0[q * E + e] : static_cast<uint16_t>(0);
                if (dh0) dh0[q * E + e] = 0;
            }
        }
        __syncthreads();
    }
}

hipError_t launch_offsets(const int32_t* cu, int64_t nseq, int64_t total, int32_t* status, const uint16_t* h0,
                          uint16_t* hT, uint16_t* dh0, int64_t D, int L, hipStream_t s) {
    hipLaunchKernelGGL(cconv_offsets_kernel, dim3(1), dim3(1024), 0, s, cu, nseq, total, status, h0, hT, dh0, D, L);
    return hipGetLastError();
}

}  // namespace cconv
