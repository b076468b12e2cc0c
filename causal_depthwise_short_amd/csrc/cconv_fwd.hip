// cconv_fwd.hip -- forward of the depthwise causal short convolution + SiLU on gfx950.
//
// Work decomposition (after the channel-strip, time-sequential scheme of the kernel-fun
// wheel's strip.py module docstring, re-cut for wave64): a lane owns VEC consecutive
// channels; a wave owns a strip of 64*VEC channels for one time segment of one batch row and
// walks the segment's rows in order. The W-1 previous rows of x stay in VGPRs as a ring, so
// each element costs one coalesced load, one sigmoid and one store. Rows are loaded G at a
// time (all G loads issued before the group's arithmetic) to keep bytes in flight.
//
// y[b,t,d] = silu(bias[d] + sum_k w[d, W-1-k] * x[b, t-k, d]), x = 0 before t = 0
// [strip.py: `_tap`, `_ld_ring`, `_silu`, `_fwd4`].
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

namespace cconv {

template <int VEC, int W>
__device__ __forceinline__ Row<VEC> fwd_row(const float (&tap)[W][VEC], const float (&b)[VEC],
                                            const Row<VEC>& raw,
                                            float (&ring)[W > 1 ? W - 1 : 1][VEC]) {
    float xt[VEC];
    widen(raw, xt);
    float y[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        const float z = conv_z<VEC, W>(tap, b, xt, ring, v);
        y[v] = z * sigmoid(z);
    }
    // rotate: ring[k] holds x[t-1-k]
#pragma unroll
    for (int k = W - 2; k > 0; --k)
#pragma unroll
        for (int v = 0; v < VEC; ++v) ring[k][v] = ring[k - 1][v];
    if constexpr (W > 1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) ring[0][v] = xt[v];
    }
    return narrow<VEC>(y);
}

template <int VEC, int G, int W, int F>
__device__ __forceinline__ void fwd_body(const FwdArgs& a) {
    constexpr int R = W > 1 ? W - 1 : 1;
    constexpr bool NTL = (F & kNtLoad) != 0, NTS = (F & kNtStore) != 0, PF = (F & kPrefetch) != 0;
    const WaveTile wt = wave_tile<VEC>(a.strip_groups, a.seg_groups, a.ws, a.seg_rows, a.T);
    const int64_t t0 = wt.t0, t1 = wt.t1;
    if (t0 >= a.T) return;    // a trailing wave of the last segment group
    if (wt.d >= a.D) return;  // lanes past the last channel (D is a multiple of VEC)
    if (a.status && *a.status != 0) return;  // pool mode: the slot check failed, write nothing

    // Row bases are wave-uniform (scalar registers); a lane adds its 32-bit channel offset,
    // so a row load is one global_load with a scalar base and no per-row VALU address math.
    const uint32_t lo = static_cast<uint32_t>(wt.d) * 2u;  // byte offset of the lane's channels
    const uint16_t* __restrict__ xb = a.x + wt.b * a.x_sb;
    uint16_t* __restrict__ yb = a.y + wt.b * a.T * a.D;
    const int64_t xs = a.x_st, ys = a.D;

    float tap[W][VEC];
    load_taps<VEC, W>(a.w, a.w_f32, wt.d, tap);
    float bs[VEC];
    load_bias<VEC>(a.bias, wt.d, bs);

    // ring prologue: x[t0-1-k]; before the sequence start, the history (or zeros). Only the
    // first segment's wave reaches t < 0, and only it reads the history and writes the final
    // state, so the two may share one buffer.
    float hist[R][VEC];
    const bool first = (t0 == 0);
    // the sequence's state row: its batch row, or in pool mode its slot (-1: none)
    int64_t hrow = wt.b;
    const uint16_t* h0 = a.h0;
    if (a.sidx && first) {
        hrow = a.sidx[wt.b];
        if (hrow < 0 || !(a.has_init && a.has_init[wt.b])) h0 = nullptr;
    }
    if (first) load_history<VEC, W>(h0, hrow, a.D, wt.d, hist);
    float ring[R][VEC];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int64_t t = t0 - 1 - k;
        if (W > 1 && t >= 0) {
            widen(load_row<VEC>(at(xb + t * xs, lo)), ring[k]);
        } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) ring[k][v] = (W > 1 && first) ? hist[R - 1 - k][v] : 0.0f;
        }
    }

    int64_t t = t0;
    if constexpr (PF) {
        // Software pipeline: while a group is computed, the next group's loads are in flight.
        // The look-ahead row index is clamped into the segment, so the last iteration re-reads
        // valid rows instead of running past them.
        if (t + G <= t1) {
            Row<VEC> cur[G];
#pragma unroll
            for (int g = 0; g < G; ++g) cur[g] = load_row<VEC, NTL>(at(xb + (t + g) * xs, lo));
            for (; t + G <= t1; t += G) {
                Row<VEC> nxt[G];
#pragma unroll
                for (int g = 0; g < G; ++g) nxt[g] = load_row<VEC, NTL>(at(xb + min(t + G + g, t1 - 1) * xs, lo));
#pragma unroll
                for (int g = 0; g < G; ++g)
                    store_row<VEC, NTS>(at(yb + (t + g) * ys, lo), fwd_row<VEC, W>(tap, bs, cur[g], ring));
#pragma unroll
                for (int g = 0; g < G; ++g) cur[g] = nxt[g];
            }
        }
    } else {
        for (; t + G <= t1; t += G) {
            Row<VEC> raw[G];
#pragma unroll
            for (int g = 0; g < G; ++g) raw[g] = load_row<VEC, NTL>(at(xb + (t + g) * xs, lo));
#pragma unroll
            for (int g = 0; g < G; ++g)
                store_row<VEC, NTS>(at(yb + (t + g) * ys, lo), fwd_row<VEC, W>(tap, bs, raw[g], ring));
        }
    }
    for (; t < t1; ++t)
        store_row<VEC, NTS>(at(yb + t * ys, lo), fwd_row<VEC, W>(tap, bs, load_row<VEC, NTL>(at(xb + t * xs, lo)), ring));

    // final state: the last W-1 values of the extended sequence (history, then x)
    if constexpr (W > 1) {
        if (first && a.hT && hrow >= 0) {
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int64_t tt = a.T - R + j;
                float v8[VEC];
                if (tt >= 0) {
                    widen(load_row<VEC>(at(xb + tt * xs, lo)), v8);
                } else {  // T < W-1: part of the history survives (re-read: slot T+j > j is not written yet)
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        v8[v] = h0 ? __uint_as_float(static_cast<uint32_t>(h0[(hrow * a.D + wt.d + v) * R + (tt + R)]) << 16)
                                   : 0.0f;
                }
#pragma unroll
                for (int v = 0; v < VEC; ++v) store_state_bf16(a.hT, hrow, a.D, wt.d + v, R, j, v8[v]);
            }
        }
    }
}

// A general kernel (blocks of up to 8 waves) and a "solo" one for one-wave blocks run one wave
// per SIMD, which may use the whole register file (256 VGPRs + 256 AGPRs).
template <int VEC, int G, int W, int F>
__global__ __launch_bounds__(512) void cconv_fwd_kernel(const FwdArgs a) {
    fwd_body<VEC, G, W, F>(a);
}

template <int VEC, int G, int W, int F>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void cconv_fwd_kernel_solo(const FwdArgs a) {
    fwd_body<VEC, G, W, F>(a);
}

namespace {

template <int VEC, int G, int W>
hipError_t launch_fwd_f(int F, dim3 grid, dim3 block, const FwdArgs& a, hipStream_t s) {
    switch (F) {
#define CCONV_FWD_CASE(f)                                                                  \
    case f: hipLaunchKernelGGL((cconv_fwd_kernel<VEC, G, W, f>), grid, block, 0, s, a); break; \
    case f + kSolo: hipLaunchKernelGGL((cconv_fwd_kernel_solo<VEC, G, W, f>), grid, block, 0, s, a); break;
        CCONV_FWD_CASE(0)
        CCONV_FWD_CASE(1)
        CCONV_FWD_CASE(2)
        CCONV_FWD_CASE(3)
        CCONV_FWD_CASE(4)
        CCONV_FWD_CASE(5)
        CCONV_FWD_CASE(6)
        CCONV_FWD_CASE(7)
#undef CCONV_FWD_CASE
        default: return hipErrorInvalidValue;
    }
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
    return (vec == 8 && (group == 4 || group == 8)) || (vec == 4 && (group == 4 || group == 8 || group == 16));
}

hipError_t launch_fwd(const Plan& p, int W, const FwdArgs& a, hipStream_t s) {
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
