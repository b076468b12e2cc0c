// cconv_device.hpp -- gfx950 device helpers for the causal depthwise short convolution.
//
// Data movement is in whole rows of a lane's VEC contiguous channels: one 16-byte (VEC = 8)
// or 8-byte (VEC = 4) global load or store per row, so a wave64 moves 1 KB (or 512 B) of a
// bf16 row per instruction, fully coalesced. VEC = 2 (4 bytes per lane) serves rows that are
// only 4-byte aligned (D = 2 mod 4), VEC = 1 (2 bytes per lane) any D and any row alignment.
// bf16 values stay packed two to a dword until
// they are used; widening is a shift or a mask, narrowing is gfx950's packed
// round-to-nearest-even convert (v_cvt_pk_bf16_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace cconv {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// VEC bf16 values of one row, packed two per dword (element 2i in the low half of u[i]); with
// VEC = 1 (the element-granular path for any D) the one value is the low half of u[0].
template <int VEC>
struct Row {
    uint32_t u[VEC >= 2 ? VEC / 2 : 1];
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
// A lane's 8-byte row chunk of 4 channels needs only 4-byte alignment: CDNA's vector memory
// instructions ask dword alignment of an access of a dword or more, so the 4-byte aligned rows
// of a width D = 2 (mod 4) take the same one-instruction 8-byte loads and stores.
typedef unsigned int u32x2a __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4a __attribute__((ext_vector_type(4), aligned(4)));

// NT selects non-temporal loads/stores (streamed data that is not re-read soon).
template <int VEC, bool NT = false>
__device__ __forceinline__ Row<VEC> load_row(const uint16_t* __restrict__ p) {
    static_assert(VEC == 1 || VEC == 2 || VEC == 4 || VEC == 8, "VEC is 1, 2, 4 or 8");
    Row<VEC> r;
    if constexpr (VEC == 1) {
        if constexpr (NT) {
            r.u[0] = __builtin_nontemporal_load(p);
        } else {
            r.u[0] = *p;
        }
    } else if constexpr (VEC == 2) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        if constexpr (NT) {
            r.u[0] = __builtin_nontemporal_load(q);
        } else {
            r.u[0] = *q;
        }
    } else if constexpr (VEC == 8) {
        u32x4 v;
        if constexpr (NT) {
            v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        } else {
            v = *reinterpret_cast<const u32x4*>(p);
        }
        r.u[0] = v.x;
        r.u[1] = v.y;
        r.u[2] = v.z;
        r.u[3] = v.w;
    } else {
        u32x2a v;
        if constexpr (NT) {
            v = __builtin_nontemporal_load(reinterpret_cast<const u32x2a*>(p));
        } else {
            v = *reinterpret_cast<const u32x2a*>(p);
        }
        r.u[0] = v.x;
        r.u[1] = v.y;
    }
    return r;
}

template <int VEC>
__device__ __forceinline__ Row<VEC> zero_row() {
    Row<VEC> r;
#pragma unroll
    for (int i = 0; i < (VEC >= 2 ? VEC / 2 : 1); ++i) r.u[i] = 0u;
    return r;
}

template <int VEC, bool NT = false>
__device__ __forceinline__ void store_row(uint16_t* __restrict__ p, const Row<VEC>& r) {
    if constexpr (VEC == 1) {
        const uint16_t v = static_cast<uint16_t>(r.u[0]);
        if constexpr (NT) {
            __builtin_nontemporal_store(v, p);
        } else {
            *p = v;
        }
    } else if constexpr (VEC == 2) {
        uint32_t* q = reinterpret_cast<uint32_t*>(p);
        if constexpr (NT) {
            __builtin_nontemporal_store(r.u[0], q);
        } else {
            *q = r.u[0];
        }
    } else if constexpr (VEC == 8) {
        const u32x4 v = {r.u[0], r.u[1], r.u[2], r.u[3]};
        if constexpr (NT) {
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
        } else {
            *reinterpret_cast<u32x4*>(p) = v;
        }
    } else {
        const u32x2a v = {r.u[0], r.u[1]};
        if constexpr (NT) {
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2a*>(p));
        } else {
            *reinterpret_cast<u32x2a*>(p) = v;
        }
    }
}

// A row of a lane through a buffer resource: the resource holds the row's wave-uniform base
// (built with scalar instructions), `voff` the lane's byte offset. No per-lane 64-bit address
// arithmetic per row. The range is the whole 32-bit offset space.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(0xffffffffu), 0x00020000);
}

template <int VEC, bool NT = false>
__device__ __forceinline__ Row<VEC> load_row_rs(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    static_assert(VEC == 4 || VEC == 8, "buffer rows: 4 or 8 channels per lane");
    constexpr int aux = NT ? 2 : 0;  // 2: non-temporal
    Row<VEC> row;
    if constexpr (VEC == 8) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), aux);
        row.u[0] = v.x, row.u[1] = v.y, row.u[2] = v.z, row.u[3] = v.w;
    } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voff), static_cast<int>(soff), aux);
        row.u[0] = v.x, row.u[1] = v.y;
    }
    return row;
}

template <int VEC, bool NT = false>
__device__ __forceinline__ void store_row_rs(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                             const Row<VEC>& row) {
    static_assert(VEC == 4 || VEC == 8, "buffer rows: 4 or 8 channels per lane");
    constexpr int aux = NT ? 2 : 0;  // 2: non-temporal
    if constexpr (VEC == 8) {
        const u32x4 v = {row.u[0], row.u[1], row.u[2], row.u[3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(voff), static_cast<int>(soff), aux);
    } else {
        const u32x2 v = {row.u[0], row.u[1]};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(voff), static_cast<int>(soff), aux);
    }
}

// The backward's 4- and 8-channel kernels address a row group from one buffer resource at its
// first row, row g at the scalar byte offset g * stride * 2. The offsets are 32-bit: with row
// strides of at most kMaxGroupStride elements, 15 strides plus a row's bytes stay below 2^32.
constexpr int64_t kMaxGroupStride = int64_t(1) << 26;

// Option bits of the row kernels (a template parameter).
constexpr int kNtLoad = 1;    // non-temporal loads of x (and dy)
constexpr int kNtStore = 2;   // non-temporal stores of y (dx)
constexpr int kPrefetch = 4;  // next group's loads issued before the current group's math
constexpr int kSolo = 8;      // one-wave blocks, one wave per SIMD, whole register file (launch-time)
// Packed batches (and the epilogue and element-granular variants) are compiled for the
// streaming options only, with or without kSolo: non-temporal loads and stores, no software
// prefetch (the backward is issue-bound, and the prefetch's extra live rows cost more
// register moves than the latency they hide).
constexpr int kVarlenFwdOptions = kNtLoad | kNtStore;
constexpr int kVarlenBwdOptions = kNtLoad | kNtStore;
// The element-granular paths (one channel per lane for odd D, two for D = 2) are
// compiled with plain loads and stores: their rows never start on a 128-byte cache line, and
// non-temporal hints then keep the L2 from merging the lines two neighbouring strips share.
constexpr int kNarrowOptions = 0;
// Epilogue variants (compile-time, default launch only): no activation (y = z, g = dy), and a
// residual added to the forward's output after the activation.
constexpr int kLinear = 16;
constexpr int kResidual = 32;
// Option bits of the decode update: non-temporal stores of y and the state; non-temporal loads
// of x and the state.
constexpr int kUpdNtStore = 1;
constexpr int kUpdNtLoad = 2;
// Option bit of the decode update (8 channels per thread): the state runs move between memory
// and registers through the wave's LDS region, so that every load and store instruction covers
// contiguous bytes (lane i takes 16-byte chunk q*64 + i of the wave's run) instead of 16 bytes
// at a 16*L-byte lane stride.
constexpr int kUpdStaged = 4;

// The wave's index in its block, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

// A row element at a wave-uniform base plus a lane's byte offset (a 32-bit byte count). In the
// row loops the compiler keeps each lane's 64-bit row address in vector registers and steps it
// by the row stride: one 64-bit vector add per load or store. The backward's row groups go
// through buffer resources instead (load_row_rs / store_row_rs: one resource per tensor at the
// group's first row, the rows as loop-invariant scalar offsets), which takes the 16 dx-store
// adds and the scalar row-base arithmetic of the 32 loads off each 16-row group (1629 -> 1531
// instructions, 1458 -> 1442 of them vector; backward 1-2% faster).
template <typename P>
__device__ __forceinline__ P* at(P* base, uint32_t off_bytes) {
    using C = typename std::conditional<std::is_const<P>::value, const char, char>::type;
    return reinterpret_cast<P*>(reinterpret_cast<C*>(base) + off_bytes);
}

// bf16 -> fp32 is exact: the bf16 pattern is the high half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int VEC>
__device__ __forceinline__ void widen(const Row<VEC>& r, float (&f)[VEC]) {
    if constexpr (VEC == 1) f[0] = bf16_lo(r.u[0]);
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
        f[2 * i] = bf16_lo(r.u[i]);
        f[2 * i + 1] = bf16_hi(r.u[i]);
    }
}

// Two fp32 -> two bf16 (round to nearest even), packed: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    const bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

template <int VEC>
__device__ __forceinline__ Row<VEC> narrow(const float (&f)[VEC]) {
    Row<VEC> r;
    if constexpr (VEC == 1) r.u[0] = pack_bf16x2(f[0], 0.0f) & 0xffffu;
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) r.u[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return r;
}

// sigma(z) = 1 / (1 + e^-z) = 1 / (1 + 2^(-z log2 e)): one v_exp_f32 and one v_rcp_f32 (each
// accurate to about 1 ulp). Saturates correctly: e^-z -> inf gives 0, e^-z -> 0 gives 1.
__device__ __forceinline__ float sigmoid(float z) {
    const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// Taps of VEC consecutive channels d .. d+VEC-1 in the tap-major order the ring uses:
// tap[k][v] multiplies x[t-k] of channel d+v, i.e. tap[k][v] = w[d+v, W-1-k]; taps k >= W
// are zero. w is [D, W] row-major, bf16 (w_f32 == 0) or fp32.
template <int VEC, int W>
__device__ __forceinline__ void load_taps(const void* __restrict__ w, int w_f32, int64_t d,
                                          float (&tap)[W][VEC]) {
    if (w_f32) {
        const float* wf = static_cast<const float*>(w) + d * W;
#pragma unroll
        for (int v = 0; v < VEC; ++v)
#pragma unroll
            for (int k = 0; k < W; ++k) tap[k][v] = wf[v * W + (W - 1 - k)];
    } else {
        const uint16_t* wb = static_cast<const uint16_t*>(w) + d * W;
#pragma unroll
        for (int v = 0; v < VEC; ++v)
#pragma unroll
            for (int k = 0; k < W; ++k)
                tap[k][v] = __uint_as_float(static_cast<uint32_t>(wb[v * W + (W - 1 - k)]) << 16);
    }
}

template <int VEC>
__device__ __forceinline__ void load_bias(const float* __restrict__ bias, int64_t d,
                                          float (&b)[VEC]) {
    if (bias) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) b[v] = bias[d + v];
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) b[v] = 0.0f;
    }
}

// z = bias + sum_k tap[k] * x[t-k], accumulated newest tap first (x[t], then x[t-1], ...).
// Every kernel uses this one order, so y, dx and the decode output do not depend on the
// launch shape, and zero taps appended on the oldest side leave z unchanged.
template <int VEC, int W>
__device__ __forceinline__ float conv_z(const float (&tap)[W][VEC], const float (&b)[VEC],
                                        const float (&xt)[VEC], const float (&ring)[W > 1 ? W - 1 : 1][VEC],
                                        int v) {
    float z = __builtin_fmaf(tap[0][v], xt[v], b[v]);
#pragma unroll
    for (int k = 1; k < W; ++k) z = __builtin_fmaf(tap[k][v], ring[k - 1][v], z);
    return z;
}

// Workgroup -> logical tile, so that the contiguous logical range [x*q, (x+1)*q) runs on one
// XCD. Workgroups are handed to the 8 XCDs round-robin by id; neighbouring tiles (adjacent
// time segments of one channel strip) then share an L2 for the rows they both read.
__device__ __forceinline__ int64_t xcd_tile(int64_t pid, int64_t n) {
    constexpr int64_t kXcd = 8;
    const int64_t xcd = pid % kXcd, k = pid / kXcd;
    const int64_t q = n / kXcd, r = n % kXcd;
    return xcd * q + (xcd < r ? xcd : r) + k;
}

// The W-1 inputs before row t of a sequence whose first row is `start`, newest first:
// ring[k] = X[t-1-k] for VEC consecutive channels d... Rows at or after `start` are read from
// x; earlier ones come from the sequence's history, state row `hrow` of h0 ([rows, D, W-1],
// slot row - start + W - 1, oldest first), or are zero without a history (h0 null).
//
// Every load is issued first (the x rows with their indices clamped into the sequence, and the
// lane's whole history run when the sequence started fewer than W-1 rows back), and only then
// are the entries picked: one memory round trip. How many of the W-1 rows lie inside the
// sequence (m = t - start, capped at W-1) is wave-uniform, so a uniform switch picks a
// compile-time entry map (no dynamic register indexing).
template <int VEC, int R, int M>
__device__ __forceinline__ void ring_pick(float (&ring)[R][VEC], const Row<VEC> (&rx)[R],
                                          const uint16_t (&hv)[VEC * R]) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
        if (k < M) {
            widen(rx[k], ring[k]);
        } else {
            const int slot = R - 1 - (k - M);  // row t-1-k = start - (k - M) - 1
#pragma unroll
            for (int v = 0; v < VEC; ++v) ring[k][v] = __uint_as_float(static_cast<uint32_t>(hv[v * R + slot]) << 16);
        }
    }
}

template <int VEC, int W>
__device__ __forceinline__ void ring_at(float (&ring)[W > 1 ? W - 1 : 1][VEC], int64_t t, int64_t start,
                                        const uint16_t* __restrict__ xb, int64_t xs, uint32_t lo,
                                        const uint16_t* h0, int64_t hrow, int64_t D, int64_t d) {
    if constexpr (W == 1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) ring[0][v] = 0.0f;
    } else {
        constexpr int R = W - 1;
        Row<VEC> rx[R];
#pragma unroll
        for (int k = 0; k < R; ++k) rx[k] = load_row<VEC>(at(xb + max(t - 1 - k, start) * xs, lo));
        const int64_t m = t - start;
        uint16_t hv[VEC * R];
        if (h0 && m < R) {
            const uint16_t* __restrict__ hp = h0 + (hrow * D + d) * R;
#pragma unroll
            for (int i = 0; i < VEC * R; ++i) hv[i] = hp[i];
        } else {
#pragma unroll
            for (int i = 0; i < VEC * R; ++i) hv[i] = 0;
        }
        if (m >= R) {
            ring_pick<VEC, R, R>(ring, rx, hv);
        } else if (m == 0) {
            ring_pick<VEC, R, 0>(ring, rx, hv);
        } else if constexpr (R > 1) {
            if (m == 1) {
                ring_pick<VEC, R, (R > 1 ? 1 : 0)>(ring, rx, hv);
            } else if constexpr (R > 2) {
                ring_pick<VEC, R, (R > 2 ? 2 : 0)>(ring, rx, hv);
            }
        }
    }
}

// The sequence of a packed batch that holds row t: the largest s < n with cu[s] <= t, so empty
// sequences are passed over (the offsets were checked first: cu[0] = 0 <= t < cu[n]). Called
// by the active lanes of a wave, all with the same t. They probe P = (active lanes) positions
// at once, strictly inside the range [lo, hi) so that it splits into P + 1 parts; a ballot
// counts the probes at or before t (a prefix of them, cu being nondecreasing), and the range
// shrinks to one part. One round of loads for up to 64 sequences, 4 for 2^24; every round
// shrinks the range, even with a single active lane.
__device__ __forceinline__ int64_t seq_of(const int32_t* cu, int64_t n, int64_t t) {
    const uint64_t act = __ballot(1);
    const int64_t P = __popcll(act);
    const int64_t rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(act >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(act), 0u));
    int64_t lo = 0, hi = n;
    while (hi - lo > 1) {
        const int64_t step = (hi - lo + P) / (P + 1);
        const int64_t p = lo + (rank + 1) * step;
        const int64_t k = __popcll(__ballot(p < hi && cu[p] <= t));
        hi = min(hi, lo + (k + 1) * step);
        lo += k * step;
    }
    return lo;
}

// One bf16 value of channel d+v, slot j, of a [B, D, W-1] state.
__device__ __forceinline__ void store_state_bf16(uint16_t* st, int64_t b, int64_t D, int64_t d, int L, int j,
                                                 float val) {
    st[(b * D + d) * L + j] = static_cast<uint16_t>(pack_bf16x2(val, 0.0f) & 0xffffu);
}

// A workgroup barrier that orders LDS accesses only: the waves' global loads in flight are not
// waited for (a plain __syncthreads() would also wait for every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The decode slot rule, checked by one block: true (in every thread of the block) when some
// idx[n] lies outside [-1, S), a non-negative slot appears twice, or (cs non-null) some cs[n]
// is negative. idx may be null (no slots to check). `seen` is an LDS bit set of (S + 31) / 32
// words followed by one verdict word ((S + 31) / 32 + 1 words with idx, 1 without).
// O(N + S/32) per block, no device trap; the two barriers order LDS only, so global loads
// the block issued before the check stay in flight through it.
//
// `first` holds the thread's entries of row threadIdx.x (v = -1, c = 0 past N), loaded by the
// caller before its other loads: vector loads complete in issue order, so waiting for an
// entry issued after them would also wait for them. Rows threadIdx.x + k * blockDim.x (N
// larger than the block) are loaded here.
struct SlotEntry {
    int32_t v, c;
};

__device__ __forceinline__ bool block_slots_bad(const int32_t* __restrict__ idx, const int32_t* __restrict__ cs,
                                                int64_t N, int64_t S, uint32_t* seen, SlotEntry first) {
    const int64_t words = idx ? (S + 31) / 32 : 0;
    const int64_t i0 = threadIdx.x;
    for (int64_t i = i0; i <= words; i += blockDim.x) seen[i] = 0u;
    lds_barrier();
    bool bad = false;
    auto take = [&](int32_t v, int32_t c) {
        if (c < 0) bad = true;
        if (v < -1 || static_cast<int64_t>(v) >= S) {
            bad = true;
        } else if (v >= 0) {
            const uint32_t bit = 1u << (v & 31);
            const uint32_t old = atomicOr(&seen[v >> 5], bit);
            if (old & bit) bad = true;
        }
    };
    take(first.v, first.c);
    for (int64_t i = i0 + blockDim.x; i < N; i += blockDim.x) take(idx ? idx[i] : -1, cs ? cs[i] : 0);
    if (bad) seen[words] = 1u;  // every writer stores the same value
    lds_barrier();
    return seen[words] != 0u;
}

// Where a wave works. The block id (XCD-remapped) selects a (strip group, segment group,
// batch row); the wave's index selects its strip within the group (ws_i) and its segment
// within the group (wt_i). The strip holds lane groups floor(s*L/strips) .. floor((s+1)*L/
// strips) - 1 of the L = lane_groups (as equal widths as integers allow, at most 64: no strip
// is left nearly empty); `active` marks the lanes that own one. All fields are wave-uniform
// except `d`, the lane's first channel, and `active`.
//
// Lane group g starts at channel g*VEC, except that the last one of a width D that is not a
// multiple of VEC (4 channels per lane at D = 2 (mod 4)) starts at D - VEC: it overlaps its
// neighbour by VEC - D % VEC channels. Both lanes compute those channels from the same inputs
// in the same order, so what they store there (y, dx, states, the dw/dbias partials) is the
// same bits, and no lane reads or writes past channel D - 1.
struct WaveTile {
    int64_t b, sg, t0, t1, d;
    int ws_i, wt_i, wt;
    bool active;
};

template <int VEC>
__device__ __forceinline__ WaveTile wave_tile(int64_t strip_groups, int64_t seg_groups, int ws, int64_t seg_rows,
                                              int64_t T, int64_t lane_groups, int64_t strips, int64_t D) {
    WaveTile w;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t sgrp = tile % strip_groups;
    const int64_t rest = tile / strip_groups;
    w.sg = rest % seg_groups;
    w.b = rest / seg_groups;
    const int wave = wave_id();
    w.wt = (blockDim.x / kWave) / ws;
    w.ws_i = wave % ws;
    w.wt_i = wave / ws;
    w.t0 = (w.sg * w.wt + w.wt_i) * seg_rows;
    w.t1 = min(w.t0 + seg_rows, T);
    const int64_t strip = sgrp * ws + w.ws_i;
    const int64_t g0 = strip * lane_groups / strips, g1 = (strip + 1) * lane_groups / strips;
    const int64_t lane = threadIdx.x % kWave;
    w.active = strip < strips && lane < g1 - g0;
    w.d = min((g0 + lane) * VEC, D - VEC);
    return w;
}

}  // namespace cconv
