// cconv_bwd_body.hpp -- the backward kernels' bodies and kernel templates, instantiated by
// cconv_bwd.hip (the plain backward in every launch variant) and cconv_bwd_extra.hip (packed
// batches and the variant without an activation, for the default launch only).
//
// Same decomposition as the forward (lane = VEC channels, wave = channel strip x time
// segment x batch row). Each row recomputes z from the x ring (the forward is never re-run),
// forms g = dy * s * (1 + z(1-s)), s = sigmoid(z) [strip.py: `_dsilu`], accumulates the tap
// gradients dw_k += g[t] * x[t-k] and dbias += g[t] in fp32, and keeps the W-1 previous
// rows of g in a second ring: dx[u] = sum_k w[:, W-1-k] * g[u+k] is complete W-1 rows after u
// [strip.py: `_bwd4` docstring]. A segment does not own dx for its first W-1 rows' lag
// window: the previous segment finishes those from a right halo of W-1 rows whose g it
// recomputes without accumulating dw [strip.py: `cconv_bwd_strip` halo].
//
// dw/dbias partials: the waves of a block (consecutive segments of one strip and batch row)
// are summed through LDS in wave order, and the block writes one fp32 partial row
// [W+1][D] (columns 0..W-1 dw, column W dbias). A second kernel sums the partials over
// blocks in a fixed order and casts dw to its dtype [strip.py: host `cconv_bwd`, the
// deterministic reduction with no atomics]. Both orders are fixed, so dw/dbias are bitwise
// reproducible.
//
// Without an activation (kLinear, y = z) g is dy itself and no z is formed.
#pragma once
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

namespace cconv {


// One backward row t. `acc_on`: the row belongs to this segment (accumulate dw/dbias);
// `emit`: dx of row t-(W-1) is this segment's: it is stored at dxrow (or into the history's
// gradient when hist_grad is given), or, with `defer`, handed back for the caller to store.
template <int VEC, int W, int F>
__device__ __forceinline__ void bwd_row(const float (&tap)[W][VEC], const float (&b)[VEC],
                                        const Row<VEC>& rx, const Row<VEC>& rdy,
                                        float (&xr)[W > 1 ? W - 1 : 1][VEC],
                                        float (&gr)[W > 1 ? W - 1 : 1][VEC], float (&acc)[W][VEC],
                                        float (&db)[VEC], bool acc_on, bool emit,
                                        uint16_t* __restrict__ dxrow, uint32_t lo, uint16_t* hist_grad = nullptr,
                                        int64_t hb = 0, int64_t D = 0, int64_t d = 0, int hj = 0,
                                        Row<VEC>* defer = nullptr) {
    constexpr bool NTS = (F & kNtStore) != 0, LIN = (F & kLinear) != 0;
    float xt[VEC], dyt[VEC], g[VEC];
    widen(rx, xt);
    widen(rdy, dyt);
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        if constexpr (LIN) {  // y = z: g = dy
            g[v] = dyt[v];
        } else {
            // g = dy * s * (1 + z(1-s)) as a + a*m with a = dy*s and m = z - z*s: three VALU ops
            const float z = conv_z<VEC, W>(tap, b, xt, xr, v);
            const float s = sigmoid(z);
            const float a = dyt[v] * s;
            g[v] = __builtin_fmaf(a, __builtin_fmaf(-z, s, z), a);
        }
    }
    if (acc_on) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            acc[0][v] = __builtin_fmaf(g[v], xt[v], acc[0][v]);
#pragma unroll
            for (int k = 1; k < W; ++k) acc[k][v] = __builtin_fmaf(g[v], xr[k - 1][v], acc[k][v]);
            db[v] += g[v];
        }
    }
    if (emit) {
        // dx[u], u = t-(W-1): sum over k ascending of tap[k] * g[u+k]; g[u+k] is g (k = W-1)
        // or the ring entry gr[W-2-k] = g[t-(W-1-k)].
        float dx[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            float s = tap[0][v] * (W == 1 ? g[v] : gr[W > 1 ? W - 2 : 0][v]);
#pragma unroll
            for (int k = 1; k < W; ++k) s = __builtin_fmaf(tap[k][v], k == W - 1 ? g[v] : gr[W - 2 - k][v], s);
            dx[v] = s;
        }
        if (hist_grad) {  // a row before t = 0: the history's gradient, slot hj of [B, D, W-1]
#pragma unroll
            for (int v = 0; v < VEC; ++v) store_state_bf16(hist_grad, hb, D, d + v, W - 1, hj, dx[v]);
        } else if (defer) {
            *defer = narrow<VEC>(dx);
        } else {
            store_row<VEC, NTS>(at(dxrow, lo), narrow<VEC>(dx));
        }
    }
#pragma unroll
    for (int k = W - 2; k > 0; --k)
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            xr[k][v] = xr[k - 1][v];
            gr[k][v] = gr[k - 1][v];
        }
    if constexpr (W > 1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            xr[0][v] = xt[v];
            gr[0][v] = g[v];
        }
    }
}

// Where a run's dx rows go. Row u's dx is emitted when row u+W-1 is processed. Rows u >= own
// are this wave's; with hg set (the wave holds the sequence's first row), the W-1 rows before
// `start` give the history gradient of state row s instead.
struct DxSink {
    uint16_t* dxb;
    int64_t dxs;
    uint32_t lo;
    int64_t own, start;
    uint16_t* hg;
    int64_t s, D, d;
};

// One row t of a run. GEN: the general emission rule (the first W-1 rows of a run, the tail
// and the halo); otherwise row t-(W-1) is known to be this wave's own dx row (its dx goes to
// *defer when given).
template <int VEC, int W, int F, bool GEN>
__device__ __forceinline__ void bwd_step(const float (&tap)[W][VEC], const float (&bs)[VEC], const Row<VEC>& rx,
                                         const Row<VEC>& rdy, float (&xr)[W > 1 ? W - 1 : 1][VEC],
                                         float (&gr)[W > 1 ? W - 1 : 1][VEC], float (&acc)[W][VEC], float (&db)[VEC],
                                         const DxSink& k, int64_t t, bool acc_on, Row<VEC>* defer = nullptr) {
    const int64_t u = t - (W - 1);
    if constexpr (GEN) {
        const bool emit = u >= k.own || (k.hg && u >= k.start - (W - 1));
        bwd_row<VEC, W, F>(tap, bs, rx, rdy, xr, gr, acc, db, acc_on, emit, k.dxb + u * k.dxs, k.lo,
                             u < k.start ? k.hg : nullptr, k.s, k.D, k.d, static_cast<int>(u - k.start + (W - 1)));
    } else {
        bwd_row<VEC, W, F>(tap, bs, rx, rdy, xr, gr, acc, db, acc_on, true, k.dxb + u * k.dxs, k.lo, nullptr, 0, 0,
                             0, 0, defer);
    }
}

// G consecutive rows of x, then of dy, from row pointers xp and dyp (the lane's channels at
// byte offset lo). One tensor's rows go out back to back (x rows together, then dy rows):
// measured faster than alternating the two tensors row by row.
//
// With 4 or 8 channels per lane the rows go through one buffer resource per tensor at the
// group's first row: row g is the scalar byte offset g * stride * 2 (loop-invariant), the
// lane's channel offset the vector offset, so no address arithmetic is done per row. The host
// keeps these plans to row strides of at most kMaxGroupStride elements.
template <int VEC, int G, bool NT>
__device__ __forceinline__ void load_group(Row<VEC> (&rx)[G], Row<VEC> (&rdy)[G], const uint16_t* __restrict__ xp,
                                           int64_t xs, const uint16_t* __restrict__ dyp, int64_t dys, uint32_t lo) {
    if constexpr (VEC == 4 || VEC == 8) {
        const __amdgpu_buffer_rsrc_t r1 = row_rsrc(xp), r2 = row_rsrc(dyp);
#pragma unroll
        for (int g = 0; g < G; ++g) rx[g] = load_row_rs<VEC, NT>(r1, lo, static_cast<uint32_t>(g * xs * 2));
#pragma unroll
        for (int g = 0; g < G; ++g) rdy[g] = load_row_rs<VEC, NT>(r2, lo, static_cast<uint32_t>(g * dys * 2));
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) rx[g] = load_row<VEC, NT>(at(xp + g * xs, lo));
#pragma unroll
        for (int g = 0; g < G; ++g) rdy[g] = load_row<VEC, NT>(at(dyp + g * dys, lo));
    }
}

// Rows t .. t+G-1 of a run, already loaded. Outside the general rule every row's dx (row
// t+g-(W-1)) is this wave's own, and the group's G dx rows are stored together after its math
// (a scheduling barrier keeps the compiler from moving them back between the rows): a run of
// G row stores measured 2.5-3.5% faster than one store per row as it is formed (268-274 vs
// 276-278 us at [8,8192,4096], 320 vs 326 us at [8,8192,4100], interleaved; dx bit-identical).
template <int VEC, int G, int W, int F, bool GEN>
__device__ __forceinline__ void bwd_group(const float (&tap)[W][VEC], const float (&bs)[VEC], const Row<VEC> (&rx)[G],
                                          const Row<VEC> (&rdy)[G], float (&xr)[W > 1 ? W - 1 : 1][VEC],
                                          float (&gr)[W > 1 ? W - 1 : 1][VEC], float (&acc)[W][VEC], float (&db)[VEC],
                                          const DxSink& k, int64_t t) {
    if constexpr (GEN) {
#pragma unroll
        for (int g = 0; g < G; ++g) bwd_step<VEC, W, F, GEN>(tap, bs, rx[g], rdy[g], xr, gr, acc, db, k, t + g, true);
    } else {
        constexpr bool NTS = (F & kNtStore) != 0;
        Row<VEC> out[G];
#pragma unroll
        for (int g = 0; g < G; ++g)
            bwd_step<VEC, W, F, GEN>(tap, bs, rx[g], rdy[g], xr, gr, acc, db, k, t + g, true, &out[g]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (VEC == 4 || VEC == 8) {  // dx rows as scalar offsets, as the loads
            const __amdgpu_buffer_rsrc_t rd = row_rsrc(k.dxb + (t - (W - 1)) * k.dxs);
#pragma unroll
            for (int g = 0; g < G; ++g) store_row_rs<VEC, NTS>(rd, k.lo, static_cast<uint32_t>(g * k.dxs * 2), out[g]);
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) store_row<VEC, NTS>(at(k.dxb + (t + g - (W - 1)) * k.dxs, k.lo), out[g]);
        }
    }
}

// Rows [t, e) of one sequence, t being the first row whose dx this wave owns in it (k.own).
// Only the first G >= W-1 rows can emit a row before k.own, so the first group takes the
// general rule and the steady groups none. A group's loads are all issued before its math
// (a scheduling barrier keeps the compiler from sinking them into it).
//
// With PF the groups are double-buffered: buffers A and B alternate, and the loads of the
// next group are issued before the current group's math, so they are in flight while it
// computes. The two buffers are separate register sets (the loop is unrolled by two): a
// copy of the prefetched rows would need them to have landed first, and since loads and
// stores share one in-order counter that wait would also cover the current group's dx
// stores. The group that has no successor to prefetch takes the general rule.
template <int VEC, int G, int W, int F>
__device__ __forceinline__ void bwd_run(const float (&tap)[W][VEC], const float (&bs)[VEC],
                                        float (&xr)[W > 1 ? W - 1 : 1][VEC], float (&gr)[W > 1 ? W - 1 : 1][VEC],
                                        float (&acc)[W][VEC], float (&db)[VEC], const uint16_t* __restrict__ xb,
                                        int64_t xs, const uint16_t* __restrict__ dyb, int64_t dys, const DxSink& k,
                                        int64_t t, const int64_t e) {
    static_assert(G >= W - 1, "the first group must cover the rows that need the general rule");
    constexpr bool NTL = (F & kNtLoad) != 0, PF = (F & kPrefetch) != 0;
    const uint32_t lo = k.lo;
    if (t + G <= e) {
        // the first group: general rule
        Row<VEC> ax[G], ady[G];
        load_group<VEC, G, NTL>(ax, ady, xb + t * xs, xs, dyb + t * dys, dys, lo);
        if constexpr (PF) {
            Row<VEC> bx[G], bdy[G];
            const bool more = t + 2 * G <= e;
            if (more) {
                load_group<VEC, G, NTL>(bx, bdy, xb + (t + G) * xs, xs, dyb + (t + G) * dys, dys, lo);
            }
            __builtin_amdgcn_sched_barrier(0);
            bwd_group<VEC, G, W, F, true>(tap, bs, ax, ady, xr, gr, acc, db, k, t);
            t += G;
            if (more) {
                // B holds rows [t, t+G); A is free
                for (;;) {
                    if (t + 2 * G > e) {
                        __builtin_amdgcn_sched_barrier(0);
                        bwd_group<VEC, G, W, F, true>(tap, bs, bx, bdy, xr, gr, acc, db, k, t);
                        t += G;
                        break;
                    }
                    load_group<VEC, G, NTL>(ax, ady, xb + (t + G) * xs, xs, dyb + (t + G) * dys, dys, lo);
                    __builtin_amdgcn_sched_barrier(0);
                    bwd_group<VEC, G, W, F, false>(tap, bs, bx, bdy, xr, gr, acc, db, k, t);
                    t += G;
                    // A holds rows [t, t+G); B is free
                    if (t + 2 * G > e) {
                        __builtin_amdgcn_sched_barrier(0);
                        bwd_group<VEC, G, W, F, true>(tap, bs, ax, ady, xr, gr, acc, db, k, t);
                        t += G;
                        break;
                    }
                    load_group<VEC, G, NTL>(bx, bdy, xb + (t + G) * xs, xs, dyb + (t + G) * dys, dys, lo);
                    __builtin_amdgcn_sched_barrier(0);
                    bwd_group<VEC, G, W, F, false>(tap, bs, ax, ady, xr, gr, acc, db, k, t);
                    t += G;
                }
            }
        } else {
            __builtin_amdgcn_sched_barrier(0);
            bwd_group<VEC, G, W, F, true>(tap, bs, ax, ady, xr, gr, acc, db, k, t);
            for (t += G; t + G <= e; t += G) {
                Row<VEC> rx[G], rdy[G];
                load_group<VEC, G, NTL>(rx, rdy, xb + t * xs, xs, dyb + t * dys, dys, lo);
                __builtin_amdgcn_sched_barrier(0);
                bwd_group<VEC, G, W, F, false>(tap, bs, rx, rdy, xr, gr, acc, db, k, t);
            }
        }
    }
    if (t < e) {
        // the run's last rows, fewer than G (a run cut by a sequence start, or a segment that
        // is not a whole number of groups): all loaded at once, with the row indices clamped
        // into the run, instead of one dependent load per row
        Row<VEC> rx[G], rdy[G];
#pragma unroll
        for (int g = 0; g < G; ++g) rx[g] = load_row<VEC, NTL>(at(xb + min(t + g, e - 1) * xs, lo));
#pragma unroll
        for (int g = 0; g < G; ++g) rdy[g] = load_row<VEC, NTL>(at(dyb + min(t + g, e - 1) * dys, lo));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < G; ++g)
            if (t + g < e) bwd_step<VEC, W, F, true>(tap, bs, rx[g], rdy[g], xr, gr, acc, db, k, t + g, true);
    }
}

// The halo after a run ending at row e: rows e .. e+W-2 finish dx of the run's last W-1 rows.
// Rows before the sequence end are read (the next segment's first rows: g only, no dw); rows
// at or past it have g = 0 for this sequence.
template <int VEC, int W, int F>
__device__ __forceinline__ void bwd_halo(const float (&tap)[W][VEC], const float (&bs)[VEC],
                                         float (&xr)[W > 1 ? W - 1 : 1][VEC], float (&gr)[W > 1 ? W - 1 : 1][VEC],
                                         float (&acc)[W][VEC], float (&db)[VEC], const uint16_t* __restrict__ xb,
                                         int64_t xs, const uint16_t* __restrict__ dyb, int64_t dys, const DxSink& k,
                                         int64_t e, int64_t end) {
    if constexpr (W > 1) {
        // all W-1 rows' loads first (indices clamped to the sequence's last row; rows at or
        // past its end are then replaced by zeros), so the halo costs one memory latency
        Row<VEC> hx[W - 1], hdy[W - 1];
#pragma unroll
        for (int h = 0; h < W - 1; ++h) {
            const int64_t th = min(e + h, end - 1);
            hx[h] = load_row<VEC>(at(xb + th * xs, k.lo));
            hdy[h] = load_row<VEC>(at(dyb + th * dys, k.lo));
        }
#pragma unroll
        for (int h = 0; h < W - 1; ++h) {
            if (e + h >= end) {
                hx[h] = zero_row<VEC>();
                hdy[h] = zero_row<VEC>();
            }
            bwd_step<VEC, W, F, true>(tap, bs, hx[h], hdy[h], xr, gr, acc, db, k, e + h, false);
        }
    }
}

template <int VEC, int G, int W, int F, bool VL>
__device__ __forceinline__ void bwd_body(const BwdArgs& a) {
    constexpr int R = W > 1 ? W - 1 : 1;
    extern __shared__ float red[];  // [waves][VEC][64], one column at a time
    const WaveTile wt = wave_tile<VEC>(a.strip_groups, a.seg_groups, a.ws, a.seg_rows, a.T, a.lane_groups, a.strips, a.D);
    const int64_t t0 = wt.t0, t1 = wt.t1;
    const int wave = wave_id();
    const int lane = threadIdx.x % kWave;
    const bool active = wt.active;
    const bool valid = !(a.status && *a.status != 0);  // the offset check passed (or there is none)
    const uint32_t lo = static_cast<uint32_t>(wt.d) * 2u;  // byte offset of the lane's channels

    float acc[W][VEC], db[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        db[v] = 0.0f;
#pragma unroll
        for (int k = 0; k < W; ++k) acc[k][v] = 0.0f;
    }

    if (active && valid && t0 < a.T) {
        // wave-uniform row bases plus the lane's 32-bit channel offset
        const uint16_t* __restrict__ xb = a.x + wt.b * a.x_sb;
        const uint16_t* __restrict__ dyb = a.dy + wt.b * a.dy_sb;
        const int64_t xs = a.x_st, dys = a.dy_st;

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
        // ring prologue as in the forward; the g ring starts at zero (rows before t0 are not
        // this wave's, and history rows have no g)
        float xr[R][VEC], gr[R][VEC];
        ring_at<VEC, W>(xr, t0, start, xb, xs, lo, a.h0, s, a.D, wt.d);
        for (auto& row : gr)
            for (float& g : row) g = 0.0f;
        DxSink k{a.dx + wt.b * a.dx_sb, a.dx_st, lo, t0, start, (t0 == start) ? a.dh0 : nullptr, s, a.D, wt.d};

        int64_t t = t0;
        for (;;) {
            const int64_t e = VL ? min(t1, end) : t1;
            bwd_run<VEC, G, W, F>(tap, bs, xr, gr, acc, db, xb, xs, dyb, dys, k, t, e);
            bwd_halo<VEC, W, F>(tap, bs, xr, gr, acc, db, xb, xs, dyb, dys, k, e, end);
            if constexpr (!VL) {
                break;
            } else {
                if (e >= t1) break;
                // the next non-empty sequence starts at row e: this wave holds its first row
                do {
                    ++s;
                } while (a.cu[s + 1] <= e);
                start = e;
                end = a.cu[s + 1];
                ring_at<VEC, W>(xr, e, start, xb, xs, lo, a.h0, s, a.D, wt.d);
                for (auto& row : gr)
                    for (float& g : row) g = 0.0f;
                k.own = e;
                k.start = e;
                k.hg = a.dh0;
                k.s = s;
                t = e;
            }
        }
    }

    // The waves that share a strip (same ws_i, consecutive segments) are summed through LDS in
    // segment order, one column at a time; the first of them stores the block's partial.
    const int64_t p = wt.b * a.seg_groups + wt.sg;
    float* __restrict__ out = a.partial + p * (W + 1) * a.D;
#pragma unroll
    for (int j = 0; j <= W; ++j) {
        // column j < W is dw[:, j], the gradient of tap k = W-1-j; column W is dbias
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            red[(wave * VEC + v) * kWave + lane] = (j < W) ? acc[W - 1 - j][v] : db[v];
        __syncthreads();
        if (wt.wt_i == 0 && active && valid) {
            float s[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                s[v] = red[(wt.ws_i * VEC + v) * kWave + lane];
                for (int i = 1; i < wt.wt; ++i) s[v] += red[((i * a.ws + wt.ws_i) * VEC + v) * kWave + lane];
            }
            float* o = at(out + j * a.D, lo * 2u);  // fp32 partials: twice the bf16 byte offset
            if constexpr (VEC == 1) {
                o[0] = s[0];
            } else if constexpr (VEC == 2) {
                reinterpret_cast<float2*>(o)[0] = make_float2(s[0], s[1]);
            } else if constexpr (VEC == 8) {
                reinterpret_cast<float4*>(o)[0] = make_float4(s[0], s[1], s[2], s[3]);
                reinterpret_cast<float4*>(o)[1] = make_float4(s[4], s[5], s[6], s[7]);
            } else {  // 4 channels: 8-byte aligned when D = 2 (mod 4)
                const f32x4a q = {s[0], s[1], s[2], s[3]};
                *reinterpret_cast<f32x4a*>(o) = q;
            }
        }
        __syncthreads();
    }
}

// The kernels: a general one (blocks of up to 8 waves, at most 256 VGPRs per wave so two
// waves fit a SIMD), and a "solo" one for one-wave blocks run one wave per SIMD, which may use
// the whole register file (256 VGPRs + 256 AGPRs): deeper row groups then fit without scratch
// spills (the compiler parks values in AGPRs).
template <int VEC, int G, int W, int F, bool VL>
__global__ __launch_bounds__(512) void cconv_bwd_kernel(const BwdArgs a) {
    bwd_body<VEC, G, W, F, VL>(a);
}

template <int VEC, int G, int W, int F, bool VL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void cconv_bwd_kernel_solo(const BwdArgs a) {
    bwd_body<VEC, G, W, F, VL>(a);
}

}  // namespace cconv
