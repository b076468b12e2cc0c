// cconv_bwd.hip -- backward of the depthwise causal short convolution + SiLU on gfx950.
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
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

namespace cconv {

// One backward row t. `acc_on`: the row belongs to this segment (accumulate dw/dbias);
// `emit`: dx of row t-(W-1) is this segment's and gets stored.
template <int VEC, int W, bool NTS>
__device__ __forceinline__ void bwd_row(const float (&tap)[W][VEC], const float (&b)[VEC],
                                        const Row<VEC>& rx, const Row<VEC>& rdy,
                                        float (&xr)[W > 1 ? W - 1 : 1][VEC],
                                        float (&gr)[W > 1 ? W - 1 : 1][VEC], float (&acc)[W][VEC],
                                        float (&db)[VEC], bool acc_on, bool emit,
                                        uint16_t* __restrict__ dxrow, uint32_t lo, uint16_t* hist_grad = nullptr,
                                        int64_t hb = 0, int64_t D = 0, int64_t d = 0, int hj = 0) {
    float xt[VEC], dyt[VEC], g[VEC];
    widen(rx, xt);
    widen(rdy, dyt);
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        // g = dy * s * (1 + z(1-s)) as a + a*m with a = dy*s and m = z - z*s: three VALU ops
        const float z = conv_z<VEC, W>(tap, b, xt, xr, v);
        const float s = sigmoid(z);
        const float a = dyt[v] * s;
        g[v] = __builtin_fmaf(a, __builtin_fmaf(-z, s, z), a);
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

template <int VEC, int G, int W, int F>
__device__ __forceinline__ void bwd_body(const BwdArgs& a) {
    constexpr int R = W > 1 ? W - 1 : 1;
    constexpr bool NTL = (F & kNtLoad) != 0, NTS = (F & kNtStore) != 0, PF = (F & kPrefetch) != 0;
    extern __shared__ float red[];  // [waves][VEC][64], one column at a time
    const WaveTile wt = wave_tile<VEC>(a.strip_groups, a.seg_groups, a.ws, a.seg_rows, a.T);
    const int64_t t0 = wt.t0, t1 = wt.t1;
    const int wave = wave_id();
    const int lane = threadIdx.x % kWave;
    const bool active = wt.d < a.D;
    const uint32_t lo = static_cast<uint32_t>(wt.d) * 2u;  // byte offset of the lane's channels

    float acc[W][VEC], db[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        db[v] = 0.0f;
#pragma unroll
        for (int k = 0; k < W; ++k) acc[k][v] = 0.0f;
    }

    if (active && t0 < a.T) {
        // wave-uniform row bases plus the lane's 32-bit channel offset
        const uint16_t* __restrict__ xb = a.x + wt.b * a.x_sb;
        const uint16_t* __restrict__ dyb = a.dy + wt.b * a.dy_sb;
        uint16_t* __restrict__ dxb = a.dx + wt.b * a.T * a.D;
        const int64_t xs = a.x_st, dys = a.dy_st, dxs = a.D;

        float tap[W][VEC];
        load_taps<VEC, W>(a.w, a.w_f32, wt.d, tap);
        float bs[VEC];
        load_bias<VEC>(a.bias, wt.d, bs);

        // ring prologue as in the forward; before t = 0, the history (or zeros)
        const bool first = (t0 == 0);
        float hist[R][VEC];
        if (first) load_history<VEC, W>(a.h0, wt.b, a.D, wt.d, hist);
        float xr[R][VEC], gr[R][VEC];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t t = t0 - 1 - k;
            if (W > 1 && t >= 0) {
                widen(load_row<VEC>(at(xb + t * xs, lo)), xr[k]);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) xr[k][v] = (W > 1 && first) ? hist[R - 1 - k][v] : 0.0f;
            }
#pragma unroll
            for (int v = 0; v < VEC; ++v) gr[k][v] = 0.0f;  // rows before t0 are not ours (history rows have g = 0)
        }
        // With a history gradient requested, the first segment also emits "dx" for the W-1
        // rows before t = 0, into dh0; elsewhere rows before t0 belong to the previous segment.
        uint16_t* const hg = (first && a.dh0) ? a.dh0 : nullptr;

        int64_t t = t0;
        if constexpr (PF) {
            // Software pipeline: the next group's x and dy loads are in flight while this
            // group is computed. The look-ahead row is clamped into the segment.
            if (t + G <= t1) {
                Row<VEC> cx[G], cdy[G];
#pragma unroll
                for (int g = 0; g < G; ++g) cx[g] = load_row<VEC, NTL>(at(xb + (t + g) * xs, lo));
#pragma unroll
                for (int g = 0; g < G; ++g) cdy[g] = load_row<VEC, NTL>(at(dyb + (t + g) * dys, lo));
                for (; t + G <= t1; t += G) {
                    Row<VEC> nx[G], ndy[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) nx[g] = load_row<VEC, NTL>(at(xb + min(t + G + g, t1 - 1) * xs, lo));
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        ndy[g] = load_row<VEC, NTL>(at(dyb + min(t + G + g, t1 - 1) * dys, lo));
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int64_t u = t + g - (W - 1);
                        bwd_row<VEC, W, NTS>(tap, bs, cx[g], cdy[g], xr, gr, acc, db, true, u >= t0 || (hg && u >= -R),
                                             dxb + u * dxs, lo, u < 0 ? hg : nullptr, wt.b, a.D, wt.d,
                                             static_cast<int>(u + R));
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        cx[g] = nx[g];
                        cdy[g] = ndy[g];
                    }
                }
            }
        } else {
            for (; t + G <= t1; t += G) {
                Row<VEC> rx[G], rdy[G];
#pragma unroll
                for (int g = 0; g < G; ++g) rx[g] = load_row<VEC, NTL>(at(xb + (t + g) * xs, lo));
#pragma unroll
                for (int g = 0; g < G; ++g) rdy[g] = load_row<VEC, NTL>(at(dyb + (t + g) * dys, lo));
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int64_t u = t + g - (W - 1);
                    bwd_row<VEC, W, NTS>(tap, bs, rx[g], rdy[g], xr, gr, acc, db, true, u >= t0 || (hg && u >= -R),
                                         dxb + u * dxs, lo, u < 0 ? hg : nullptr, wt.b, a.D, wt.d,
                                         static_cast<int>(u + R));
                }
            }
        }
        for (; t < t1; ++t) {
            const int64_t u = t - (W - 1);
            bwd_row<VEC, W, NTS>(tap, bs, load_row<VEC, NTL>(at(xb + t * xs, lo)), load_row<VEC, NTL>(at(dyb + t * dys, lo)),
                                 xr, gr, acc, db, true, u >= t0 || (hg && u >= -R), dxb + u * dxs, lo,
                                 u < 0 ? hg : nullptr, wt.b, a.D, wt.d, static_cast<int>(u + R));
        }
        // right halo: rows t1 .. t1+W-2 finish dx of this segment's last W-1 rows; rows at or
        // past T have g = 0 (their x and dy read as zero).
#pragma unroll
        for (int h = 0; h < W - 1; ++h) {
            const int64_t th = t1 + h;
            const int64_t u = th - (W - 1);
            Row<VEC> hx = zero_row<VEC>(), hdy = zero_row<VEC>();
            if (th < a.T) {
                hx = load_row<VEC>(at(xb + th * xs, lo));
                hdy = load_row<VEC>(at(dyb + th * dys, lo));
            }
            bwd_row<VEC, W, NTS>(tap, bs, hx, hdy, xr, gr, acc, db, false, u >= t0 || (hg && u >= -R), dxb + u * dxs,
                                 lo, u < 0 ? hg : nullptr, wt.b, a.D, wt.d, static_cast<int>(u + R));
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
        if (wt.wt_i == 0 && active) {
            float s[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                s[v] = red[(wt.ws_i * VEC + v) * kWave + lane];
                for (int i = 1; i < wt.wt; ++i) s[v] += red[((i * a.ws + wt.ws_i) * VEC + v) * kWave + lane];
            }
            float* o = at(out + j * a.D, lo * 2u);  // fp32 partials: twice the bf16 byte offset
            if constexpr (VEC == 8) {
                reinterpret_cast<float4*>(o)[0] = make_float4(s[0], s[1], s[2], s[3]);
                reinterpret_cast<float4*>(o)[1] = make_float4(s[4], s[5], s[6], s[7]);
            } else {
                reinterpret_cast<float4*>(o)[0] = make_float4(s[0], s[1], s[2], s[3]);
            }
        }
        __syncthreads();
    }
}

// The kernels: a general one (blocks of up to 8 waves, at most 256 VGPRs per wave so two
// waves fit a SIMD), and a "solo" one for one-wave blocks run one wave per SIMD, which may use
// the whole register file (256 VGPRs + 256 AGPRs): deeper row groups then fit without scratch
// spills (the compiler parks values in AGPRs).
template <int VEC, int G, int W, int F>
__global__ __launch_bounds__(512) void cconv_bwd_kernel(const BwdArgs a) {
    bwd_body<VEC, G, W, F>(a);
}

template <int VEC, int G, int W, int F>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void cconv_bwd_kernel_solo(const BwdArgs a) {
    bwd_body<VEC, G, W, F>(a);
}

// dw[d, j] = sum_p partial[p, j, d] (j < W), dbias[d] = sum_p partial[p, W, d]. A block
// handles 64 consecutive (j, d) entries; its 4 waves each sum a contiguous quarter of the
// partials in ascending order, then the four sums are added in wave order. Loads are issued
// in batches of kBatch before they are summed, so a quarter of up to kBatch partials costs one
// memory latency. P == 0 writes zeros (an empty batch or sequence).
__global__ __launch_bounds__(256) void cconv_dw_reduce_kernel(const ReduceArgs a) {
    constexpr int kBatch = 16;
    __shared__ float part[4][kWave];
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
    switch (F) {
#define CCONV_BWD_CASE(f)                                                                                \
    case f: hipLaunchKernelGGL((cconv_bwd_kernel<VEC, G, W, f>), grid, block, lds, s, a); break;         \
    case f + kSolo: hipLaunchKernelGGL((cconv_bwd_kernel_solo<VEC, G, W, f>), grid, block, lds, s, a); break;
        CCONV_BWD_CASE(0)
        CCONV_BWD_CASE(1)
        CCONV_BWD_CASE(2)
        CCONV_BWD_CASE(3)
        CCONV_BWD_CASE(4)
        CCONV_BWD_CASE(5)
        CCONV_BWD_CASE(6)
        CCONV_BWD_CASE(7)
#undef CCONV_BWD_CASE
        default: return hipErrorInvalidValue;
    }
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
    return (vec == 8 && (group == 4 || group == 8)) || (vec == 4 && (group == 4 || group == 8 || group == 16));
}

hipError_t launch_bwd(const Plan& p, int W, const BwdArgs& a, hipStream_t s) {
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
