// cconv_fwd_body.hpp -- the forward kernels' bodies and kernel templates, instantiated by
// cconv_fwd.hip (the plain forward in every launch variant) and cconv_fwd_extra.hip (packed
// batches and the epilogue variants, for the default launch only).
//
// Work decomposition (after the channel-strip, time-sequential scheme of the kernel-fun
// wheel's strip.py module docstring, re-cut for wave64): a lane owns VEC consecutive
// channels; a wave owns a strip of 64*VEC channels for one time segment of one batch row and
// walks the segment's rows in order. The W-1 previous rows of x stay in VGPRs as a ring, so
// each element costs one coalesced load, one sigmoid and one store. Rows are loaded G at a
// time (all G loads issued before the group's arithmetic) to keep bytes in flight.
//
// y[b,t,d] = silu(bias[d] + sum_k w[d, W-1-k] * x[b, t-k, d]), x = 0 before t = 0
// [strip.py: `_tap`, `_ld_ring`, `_silu`, `_fwd4`]; without an activation y = z, and a residual
// is added after the activation [fla's activation and residual parameters, _common/compat.py].
#pragma once
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

namespace cconv {

// One row: z from the ring, then the epilogue: SiLU (or none with LIN), plus the residual row
// (RES) after the activation.
template <int VEC, int W, bool LIN, bool RES>
__device__ __forceinline__ Row<VEC> fwd_row(const float (&tap)[W][VEC], const float (&b)[VEC],
                                            const Row<VEC>& raw, const Row<VEC>& res,
                                            float (&ring)[W > 1 ? W - 1 : 1][VEC]) {
    float xt[VEC];
    widen(raw, xt);
    float y[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        const float z = conv_z<VEC, W>(tap, b, xt, ring, v);
        y[v] = LIN ? z : z * sigmoid(z);
    }
    if constexpr (RES) {
        float rt[VEC];
        widen(res, rt);
#pragma unroll
        for (int v = 0; v < VEC; ++v) y[v] += rt[v];
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

// Rows [t, e) of one sequence: per row one coalesced load (two with a residual), the
// convolution over the ring, the epilogue, one store. Rows are loaded G at a time; with PF the
// next group's loads are in flight while the current group is computed (the look-ahead row is
// clamped into [t, e), so the last iteration re-reads valid rows instead of running past them).
template <int VEC, int G, int W, int F>
__device__ __forceinline__ void fwd_run(const float (&tap)[W][VEC], const float (&bs)[VEC],
                                        float (&ring)[W > 1 ? W - 1 : 1][VEC], const uint16_t* __restrict__ xb,
                                        int64_t xs, const uint16_t* __restrict__ rb, int64_t rs,
                                        uint16_t* __restrict__ yb, int64_t ys, uint32_t lo, int64_t t,
                                        const int64_t e) {
    constexpr bool NTL = (F & kNtLoad) != 0, NTS = (F & kNtStore) != 0, PF = (F & kPrefetch) != 0;
    constexpr bool LIN = (F & kLinear) != 0, RES = (F & kResidual) != 0;
    auto ldr = [&](int64_t row) { return RES ? load_row<VEC, NTL>(at(rb + row * rs, lo)) : zero_row<VEC>(); };
    if constexpr (PF) {
        if (t + G <= e) {
            Row<VEC> cur[G], cres[G];
#pragma unroll
            for (int g = 0; g < G; ++g) cur[g] = load_row<VEC, NTL>(at(xb + (t + g) * xs, lo));
#pragma unroll
            for (int g = 0; g < G; ++g) cres[g] = ldr(t + g);
            for (; t + G <= e; t += G) {
                Row<VEC> nxt[G], nres[G];
#pragma unroll
                for (int g = 0; g < G; ++g) nxt[g] = load_row<VEC, NTL>(at(xb + min(t + G + g, e - 1) * xs, lo));
#pragma unroll
                for (int g = 0; g < G; ++g) nres[g] = ldr(min(t + G + g, e - 1));
#pragma unroll
                for (int g = 0; g < G; ++g)
                    store_row<VEC, NTS>(at(yb + (t + g) * ys, lo), fwd_row<VEC, W, LIN, RES>(tap, bs, cur[g], cres[g], ring));
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    cur[g] = nxt[g];
                    cres[g] = nres[g];
                }
            }
        }
    } else {
        for (; t + G <= e; t += G) {
            Row<VEC> raw[G], res[G];
#pragma unroll
            for (int g = 0; g < G; ++g) raw[g] = load_row<VEC, NTL>(at(xb + (t + g) * xs, lo));
#pragma unroll
            for (int g = 0; g < G; ++g) res[g] = ldr(t + g);
            // the group's G rows of y go out together after its math (as the backward's dx)
            Row<VEC> out[G];
#pragma unroll
            for (int g = 0; g < G; ++g) out[g] = fwd_row<VEC, W, LIN, RES>(tap, bs, raw[g], res[g], ring);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < G; ++g) store_row<VEC, NTS>(at(yb + (t + g) * ys, lo), out[g]);
        }
    }
    if (t < e) {
        // the run's last rows, fewer than G: all loaded at once (row indices clamped into the
        // run) instead of one dependent load per row
        Row<VEC> raw[G], res[G];
#pragma unroll
        for (int g = 0; g < G; ++g) raw[g] = load_row<VEC, NTL>(at(xb + min(t + g, e - 1) * xs, lo));
#pragma unroll
        for (int g = 0; g < G; ++g) res[g] = ldr(min(t + g, e - 1));
#pragma unroll
        for (int g = 0; g < G; ++g)
            if (t + g < e)
                store_row<VEC, NTS>(at(yb + (t + g) * ys, lo), fwd_row<VEC, W, LIN, RES>(tap, bs, raw[g], res[g], ring));
    }
}

// One wave: a strip of 64*VEC channels over the rows [t0, t1) of its segment. A batch row is
// one sequence. In a packed batch (VL) the segment may cross sequence boundaries: it is cut
// into runs, and at each sequence start the ring restarts from that sequence's history.
template <int VEC, int G, int W, int F, bool VL>
__device__ __forceinline__ void fwd_body(const FwdArgs& a) {
    constexpr int R = W > 1 ? W - 1 : 1;
    const WaveTile wt = wave_tile<VEC>(a.strip_groups, a.seg_groups, a.ws, a.seg_rows, a.T, a.lane_groups, a.strips, a.D);
    const int64_t t0 = wt.t0, t1 = wt.t1;
    if (t0 >= a.T) return;    // a trailing wave of the last segment group
    if (!wt.active) return;   // lanes past the strip's channels
    if (a.status && *a.status != 0) return;  // the slot or offset check failed: write nothing

    // Row bases are wave-uniform; a lane adds its 32-bit byte offset to reach its channels.
    const uint32_t lo = static_cast<uint32_t>(wt.d) * 2u;  // byte offset of the lane's channels
    const uint16_t* __restrict__ xb = a.x + wt.b * a.x_sb;
    uint16_t* __restrict__ yb = a.y + wt.b * a.y_sb;
    const uint16_t* __restrict__ rb = a.r ? a.r + wt.b * a.r_sb : nullptr;
    const int64_t xs = a.x_st, ys = a.y_st, rs = a.r_st;

    float tap[W][VEC];
    load_taps<VEC, W>(a.w, a.w_f32, wt.d, tap);
    float bs[VEC];
    load_bias<VEC>(a.bias, wt.d, bs);

    // the sequence holding row t0: its rows [start, end) and its state row
    int64_t s = wt.b, start = 0, end = a.T;
    if constexpr (VL) {
        s = seq_of(a.cu, a.nseq, t0);
        start = a.cu[s];
        end = a.cu[s + 1];
    }
    // Fixed-length batches: only the first segment's wave reaches rows before t = 0, and only
    // it reads the history and writes the final state, so the two may share one buffer. In
    // pool mode the state row is the sequence's slot (-1: none), its history used only where
    // flagged.
    const bool first = (t0 == start);
    int64_t hrow = s;
    const uint16_t* h0 = a.h0;
    if (!VL && a.sidx && first) {
        hrow = a.sidx[wt.b];
        if (hrow < 0 || !(a.has_init && a.has_init[wt.b])) h0 = nullptr;
    }
    float ring[R][VEC];
    ring_at<VEC, W>(ring, t0, start, xb, xs, lo, h0, hrow, a.D, wt.d);

    int64_t t = t0;
    for (;;) {
        const int64_t e = VL ? min(t1, end) : t1;
        fwd_run<VEC, G, W, F>(tap, bs, ring, xb, xs, rb, rs, yb, ys, lo, t, e);
        if constexpr (!VL) {
            break;
        } else {
            // the sequence ends in this wave: its final state is the ring
            if (W > 1 && e == end && a.hT) {
#pragma unroll
                for (int j = 0; j < R; ++j)
#pragma unroll
                    for (int v = 0; v < VEC; ++v) store_state_bf16(a.hT, s, a.D, wt.d + v, R, j, ring[R - 1 - j][v]);
            }
            if (e >= t1) break;
            // the next non-empty sequence starts at row e
            do {
                ++s;
            } while (a.cu[s + 1] <= e);
            start = e;
            end = a.cu[s + 1];
            ring_at<VEC, W>(ring, e, start, xb, xs, lo, a.h0, s, a.D, wt.d);
            t = e;
        }
    }

    // fixed-length final state: the last W-1 values of the extended sequence (history, then x)
    if constexpr (W > 1 && !VL) {
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
template <int VEC, int G, int W, int F, bool VL>
__global__ __launch_bounds__(512) void cconv_fwd_kernel(const FwdArgs a) {
    fwd_body<VEC, G, W, F, VL>(a);
}

template <int VEC, int G, int W, int F, bool VL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void cconv_fwd_kernel_solo(const FwdArgs a) {
    fwd_body<VEC, G, W, F, VL>(a);
}

}  // namespace cconv
