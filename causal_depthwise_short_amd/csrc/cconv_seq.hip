// cconv_seq.hip -- bookkeeping kernels for packed variable-length batches (fla's cu_seqlens
// parameter, kernel-fun wheel, _common/compat.py FLA_KWARGS row for causal_conv1d).
//
// The offsets live on the device, so the host cannot check them: one block checks
// cu[0] = 0 <= cu[1] <= ... <= cu[n] = total and writes the verdict to a status word, which
// every later kernel of the call reads before it writes anything. Empty sequences hold no row,
// so no streaming wave meets them: a small grid gives them their final state (the history, or
// zeros) and a zero history gradient.
#include "../../include/cconv.h"
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

namespace cconv {

__global__ __launch_bounds__(1024) void cconv_offsets_kernel(const int32_t* cu, int64_t n, int64_t total,
                                                             int32_t* status) {
    bool bad = false;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x)
        if (cu[i] > cu[i + 1]) bad = true;
    if (threadIdx.x == 0 && (cu[0] != 0 || static_cast<int64_t>(cu[n]) != total)) bad = true;
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) status[0] = bad ? CCONV_ERR_INDEX : CCONV_OK;
}

// Blocks stride over the sequences; a block that meets an empty one writes its [D, L] state
// rows with all its threads.
__global__ __launch_bounds__(256) void cconv_empty_seq_kernel(const int32_t* cu, int64_t n, const uint16_t* h0,
                                                              uint16_t* hT, uint16_t* dh0, int64_t D, int L,
                                                              const int32_t* status) {
    if (*status != 0) return;
    const int64_t E = D * L;
    for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
        if (cu[i] != cu[i + 1]) continue;
        for (int64_t e = threadIdx.x; e < E; e += blockDim.x) {
            if (hT) hT[i * E + e] = h0 ? h0[i * E + e] : static_cast<uint16_t>(0);
            if (dh0) dh0[i * E + e] = 0;
        }
    }
}

hipError_t launch_offsets(const int32_t* cu, int64_t nseq, int64_t total, int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(cconv_offsets_kernel, dim3(1), dim3(1024), 0, s, cu, nseq, total, status);
    return hipGetLastError();
}

hipError_t launch_empty_seqs(const int32_t* cu, int64_t nseq, const uint16_t* h0, uint16_t* hT, uint16_t* dh0,
                             int64_t D, int L, const int32_t* status, hipStream_t s) {
    if (nseq <= 0 || D <= 0 || L <= 0 || (!hT && !dh0)) return hipSuccess;
    const int64_t blocks = nseq < 1024 ? nseq : 1024;
    hipLaunchKernelGGL(cconv_empty_seq_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, cu, nseq, h0, hT,
                       dh0, D, L, status);
    return hipGetLastError();
}

}  // namespace cconv
