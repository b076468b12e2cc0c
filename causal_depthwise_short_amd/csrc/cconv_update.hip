// cconv_update.hip -- one-token decode update of the causal depthwise short convolution +
// SiLU on gfx950 [cudnn-frontend PR #797 "Add experimental causal conv1d decode update",
// PR description: API and semantics].
//
// A thread owns 8 consecutive channels of a run of rows: per row it gathers the slot
// s = state_indices[n] (or n), reads x[n, d..d+7] (16 B) and state[s, d..d+7, 0..W-2]
// (8*(W-1) contiguous bf16, 16*(W-1) B), forms z = bias + sum_j w[d, j] state_j + w[d, W-1] x
// in the forward's tap order, writes y = silu(z) and the shifted state (bit copies: the
// oldest value drops out and x becomes the newest).
//
// Fail-closed validation without a device trap: every block reads all N indices and checks
// them against an S-bit set in LDS (range [-1, S) and no repeated non-negative slot), so all
// blocks reach the same verdict. If any index is invalid no block writes state; block 0
// reports the verdict in *status. The page's kernel scans all earlier rows per row (quadratic
// in N) and traps; here a block pays O(N + S/32) and the grid is sized so that the number of
// blocks stays near a constant, keeping the total linear in N.
#include "../../include/cconv.h"
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

namespace cconv {

// The tokens 1 .. W-1 steps back, from the L state entries a thread loaded (h[v*L + e] is
// entry e of channel d+v), in the forward's ring order: ring[k-1] = x[t-k]. Shift mode
// (ROT < 0): entry L-k. Circular mode with rotation ROT = c mod L: entry (ROT - k) mod L.
template <int VEC, int W, int L, int ROT>
__device__ __forceinline__ void ring_from_state(const uint16_t (&h)[VEC * (L > 0 ? L : 1)],
                                                float (&ring)[W > 1 ? W - 1 : 1][VEC]) {
    for (int k = 1; k < W; ++k) {
        const int e = ROT < 0 ? L - k : ((ROT - k) % L + L) % L;
        for (int v = 0; v < VEC; ++v) ring[k - 1][v] = __uint_as_float(static_cast<uint32_t>(h[v * L + e]) << 16);
    }
}

// Circular mode, VEC = 8: the thread's whole state run (8 channels x L entries, 16*L bytes)
// stored as L 16-byte vectors, entry ROT of each channel replaced by the token and the other
// entries rewritten with the values just read (the memory changes only at entry ROT).
template <int L, int ROT>
__device__ __forceinline__ void store_run_circ(uint16_t* __restrict__ sp, const uint16_t (&h)[8 * L], const Row<8>& rx) {
    uint16_t nh[8 * L];
#pragma unroll
    for (int i = 0; i < 8 * L; ++i) nh[i] = h[i];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const uint32_t xw = rx.u[v / 2];
        nh[v * L + ROT] = static_cast<uint16_t>((v & 1) ? (xw >> 16) : (xw & 0xffffu));
    }
#pragma unroll
    for (int q = 0; q < L; ++q) {
        uint32_t u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = static_cast<uint32_t>(nh[q * 8 + 2 * i]) | (static_cast<uint32_t>(nh[q * 8 + 2 * i + 1]) << 16);
        reinterpret_cast<uint4*>(sp)[q] = make_uint4(u[0], u[1], u[2], u[3]);
    }
}

// VEC = 8: a thread owns 8 channels (16-byte x rows, 16*L-byte state runs); VEC = 1: one channel
// (any D, any row stride).
// The thread's channels of one row: x (VEC values) and the state entries of slot s (VEC x L
// values, entry e of channel d+v at 16-bit position v*L + e).
template <int L, int VEC>
__device__ __forceinline__ void gather_row(const UpdateArgs& a, int64_t n, int64_t s, int64_t d, Row<VEC>& rx,
                                           uint16_t (&h)[VEC * (L > 0 ? L : 1)]) {
    rx = load_row<VEC>(a.x + n * a.x_ld + d);
    const uint16_t* __restrict__ sp = a.state + (s * a.D + d) * L;
    if constexpr (L > 0 && VEC == 1) {
        for (int e = 0; e < L; ++e) h[e] = sp[e];
    } else if constexpr (L > 0) {
#pragma unroll
        for (int q = 0; q < L; ++q) {
            const uint4 v4 = reinterpret_cast<const uint4*>(sp)[q];
            const uint32_t u[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[q * 8 + 2 * i] = static_cast<uint16_t>(u[i] & 0xffffu);
                h[q * 8 + 2 * i + 1] = static_cast<uint16_t>(u[i] >> 16);
            }
        }
    }
}

// VEC = 8: a thread owns 8 channels (16-byte x rows, 16*L-byte state runs); VEC = 1: one channel
// (any D, any row stride).
template <int W, int L, bool CIRC, int VEC>
__global__ __launch_bounds__(256) void cconv_update_kernel(const UpdateArgs a) {
    constexpr int R = W > 1 ? W - 1 : 1;
    extern __shared__ uint32_t seen[];

    const int64_t d = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * VEC;
    const bool lane = d < a.D;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * a.rows_per_block;
    const int64_t n1 = min(n0 + a.rows_per_block, a.N);

    // The block's first row is gathered before the slot check, so its loads overlap the check;
    // a slot outside [0, S) is not read, and nothing is stored before the verdict.
    Row<VEC> rx0 = zero_row<VEC>();
    uint16_t h0[VEC * (L > 0 ? L : 1)];
    int64_t s0 = -1;
    int64_t cs0 = 0;  // circular: the first row's cache_seqlens entry, loaded with its slot
    if (lane && n0 < n1) {
        s0 = a.idx ? static_cast<int64_t>(a.idx[n0]) : n0;
        if constexpr (CIRC) cs0 = a.cs[n0];
        if (s0 >= 0 && s0 < a.S) gather_row<L, VEC>(a, n0, s0, d, rx0, h0);
    }

    // circular: every cache_seqlens entry must be >= 0. The thread's first entry is loaded
    // before the slot check and compared after it, so that its load overlaps the check; the
    // two verdicts meet in one block-wide OR.
    int32_t c0 = 0;
    if (CIRC && static_cast<int64_t>(threadIdx.x) < a.N) c0 = a.cs[threadIdx.x];
    bool bad = a.idx ? block_slots_bad(a.idx, a.N, a.S, seen) : false;
    if (CIRC) {
        bool neg = c0 < 0;
        for (int64_t i = static_cast<int64_t>(threadIdx.x) + blockDim.x; i < a.N; i += blockDim.x)
            if (a.cs[i] < 0) neg = true;
        bad = __syncthreads_or(neg || bad);
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && a.status)
        a.status[0] = bad ? CCONV_ERR_INDEX : CCONV_OK;
    if (bad || !lane) return;

    float tap[W][VEC];
    load_taps<VEC, W>(a.w, a.w_f32, d, tap);
    float bs[VEC];
    load_bias<VEC>(a.bias, d, bs);

    for (int64_t n = n0; n < n1; ++n) {
        const bool first = (n == n0);
        const int64_t s = first ? s0 : (a.idx ? static_cast<int64_t>(a.idx[n]) : n);
        const int64_t cn = CIRC ? (first ? cs0 : static_cast<int64_t>(a.cs[n])) : 0;  // before the gather
        uint16_t* __restrict__ yp = a.y + n * a.D + d;
        if (s < 0) {  // padding row: no state access, output 0
            store_row<VEC>(yp, zero_row<VEC>());
            continue;
        }
        Row<VEC> rx = rx0;
        uint16_t h[VEC * (L > 0 ? L : 1)];
        if (first) {
#pragma unroll
            for (int i = 0; i < VEC * (L > 0 ? L : 1); ++i) h[i] = h0[i];
        } else {
            gather_row<L, VEC>(a, n, s, d, rx, h);
        }
        float xt[VEC];
        widen(rx, xt);
        uint16_t* __restrict__ sp = a.state + (s * a.D + d) * L;
        float ring[R][VEC];
        int rot = 0;  // circular: the entry that takes the token (block-uniform: one row at a time)
        if constexpr (W > 1) {
            if constexpr (!CIRC) {
                ring_from_state<VEC, W, L, -1>(h, ring);
            } else {
                rot = static_cast<int>(cn % L);
                if (rot == 0) ring_from_state<VEC, W, L, 0>(h, ring);
                if constexpr (L > 1) if (rot == 1) ring_from_state<VEC, W, L, (L > 1 ? 1 : 0)>(h, ring);
                if constexpr (L > 2) if (rot == 2) ring_from_state<VEC, W, L, (L > 2 ? 2 : 0)>(h, ring);
                if constexpr (L > 3) if (rot == 3) ring_from_state<VEC, W, L, (L > 3 ? 3 : 0)>(h, ring);
            }
        } else if constexpr (CIRC) {
            rot = static_cast<int>(cn % L);
        }
        float y[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float z = conv_z<VEC, W>(tap, bs, xt, ring, v);
            y[v] = z * sigmoid(z);
        }
        store_row<VEC>(yp, narrow<VEC>(y));
        if constexpr (L > 0) {
            if constexpr (CIRC && VEC == 8) {  // the token's entry changes; whole runs are stored
                if (rot == 0) store_run_circ<L, 0>(sp, h, rx);
                if constexpr (L > 1) if (rot == 1) store_run_circ<L, (L > 1 ? 1 : 0)>(sp, h, rx);
                if constexpr (L > 2) if (rot == 2) store_run_circ<L, (L > 2 ? 2 : 0)>(sp, h, rx);
                if constexpr (L > 3) if (rot == 3) store_run_circ<L, (L > 3 ? 3 : 0)>(sp, h, rx);
            } else if constexpr (CIRC) {  // one channel: write only the token's entry
                sp[rot] = static_cast<uint16_t>(rx.u[0] & 0xffffu);
            } else if constexpr (VEC == 1) {  // shift, one channel
                for (int j = 0; j + 1 < L; ++j) sp[j] = h[j + 1];
                sp[L - 1] = static_cast<uint16_t>(rx.u[0] & 0xffffu);
            } else {  // shift: drop the oldest entry, append the token
                uint16_t nh[VEC * L];
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
#pragma unroll
                    for (int j = 0; j + 1 < L; ++j) nh[v * L + j] = h[v * L + j + 1];
                    const uint32_t xw = rx.u[v / 2];
                    nh[v * L + L - 1] = static_cast<uint16_t>((v & 1) ? (xw >> 16) : (xw & 0xffffu));
                }
#pragma unroll
                for (int q = 0; q < L; ++q) {
                    uint32_t u[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        u[i] = static_cast<uint32_t>(nh[q * 8 + 2 * i]) | (static_cast<uint32_t>(nh[q * 8 + 2 * i + 1]) << 16);
                    reinterpret_cast<uint4*>(sp)[q] = make_uint4(u[0], u[1], u[2], u[3]);
                }
            }
        }
    }
}

// The slot check alone, for the prefill into a pool: one block writes the verdict, which the
// forward's waves read before they write anything.
__global__ __launch_bounds__(1024) void cconv_slots_kernel(const int32_t* idx, int64_t N, int64_t S,
                                                           int32_t* status) {
    extern __shared__ uint32_t seen[];
    const bool bad = block_slots_bad(idx, N, S, seen);
    if (threadIdx.x == 0) status[0] = bad ? CCONV_ERR_INDEX : CCONV_OK;
}

__global__ void cconv_status_kernel(int32_t* status, int32_t value) {
    if (threadIdx.x == 0 && blockIdx.x == 0) status[0] = value;
}

namespace {

template <int W, int L, bool CIRC>
void launch_update_k(bool narrow, dim3 grid, dim3 block, size_t lds, const UpdateArgs& a, hipStream_t s) {
    if (narrow)
        hipLaunchKernelGGL((cconv_update_kernel<W, L, CIRC, 1>), grid, block, lds, s, a);
    else
        hipLaunchKernelGGL((cconv_update_kernel<W, L, CIRC, 8>), grid, block, lds, s, a);
}

template <int W>
hipError_t launch_update_w(int L, bool circ, bool narrow, dim3 grid, dim3 block, size_t lds, const UpdateArgs& a,
                           hipStream_t s) {
    if (L == W - 1) {
        if (!circ) {
            launch_update_k<W, W - 1, false>(narrow, grid, block, lds, a, s);
        } else if constexpr (W > 1) {
            launch_update_k<W, W - 1, true>(narrow, grid, block, lds, a, s);
        } else {
            return hipErrorInvalidValue;  // a circular state needs at least one entry
        }
    } else if (L == W) {
        if (circ)
            launch_update_k<W, W, true>(narrow, grid, block, lds, a, s);
        else
            launch_update_k<W, W, false>(narrow, grid, block, lds, a, s);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_update(int W, int L, bool narrow, const UpdateArgs& a, int block_threads, int64_t grid_x,
                         int64_t grid_y, size_t lds, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(grid_x), static_cast<uint32_t>(grid_y)), block(block_threads);
    const bool circ = a.cs != nullptr;
    switch (W) {
        case 1: return launch_update_w<1>(L, circ, narrow, grid, block, lds, a, s);
        case 2: return launch_update_w<2>(L, circ, narrow, grid, block, lds, a, s);
        case 3: return launch_update_w<3>(L, circ, narrow, grid, block, lds, a, s);
        case 4: return launch_update_w<4>(L, circ, narrow, grid, block, lds, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_slots(const int32_t* idx, int64_t N, int64_t S, int32_t* status, hipStream_t s) {
    const size_t lds = static_cast<size_t>((S + 31) / 32) * 4;
    hipLaunchKernelGGL(cconv_slots_kernel, dim3(1), dim3(1024), lds, s, idx, N, S, status);
    return hipGetLastError();
}

hipError_t launch_status(int32_t* status, int32_t value, hipStream_t s) {
    hipLaunchKernelGGL(cconv_status_kernel, dim3(1), dim3(64), 0, s, status, value);
    return hipGetLastError();
}

}  // namespace cconv
