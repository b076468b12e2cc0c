// cconv_update.hip -- one-token decode update of the causal depthwise short convolution +
// SiLU on gfx950 [cudnn-frontend PR #797 "Add experimental causal conv1d decode update",
// PR description: API and semantics].
//
// A thread owns VEC consecutive channels (VEC = 8: 16-byte x rows and 16*L-byte state runs;
// VEC = 1: one channel, any D and any row stride) of the rows a block walks. Per row it takes
// the slot s = state_indices[n] (or n), reads x[n, d..] and state[s, d.., 0..L-1], forms
// z = bias + sum_j w[d, j] state_j + w[d, W-1] x in the forward's tap order, writes
// y = silu(z) and the new state (bit copies: shift mode drops the oldest entry and appends x;
// circular mode writes x into entry c mod L).
//
// The call is latency-bound (16.8 MB at the 256-row, 4096-channel shape), so the kernel is
// laid out as one chain of memory round trips, as short as it can be:
//   * every access goes through a buffer resource whose base is the row (x, y), the slot's
//     run (state) or the whole operand (taps, bias): lanes past D, a padding or invalid slot
//     and an absent bias get a zero-sized range, so the hardware returns zeros for their
//     loads and drops their stores. No lane branches, so nothing splits the loads into
//     separate blocks, and all of them are issued before the first wait;
//   * the row's slot is a block-uniform scalar load; the loads are issued in the order they
//     are needed (vector loads complete in issue order): the slot check's entries, the taps
//     and bias (L2-resident: every row reads them), the x row, the state run;
//   * fail-closed validation without a device trap: every block reads all N indices and checks
//     them against an S-bit set in LDS (range [-1, S), no repeated non-negative slot; circular
//     mode also rejects a negative cache_seqlens entry), so all blocks reach the same verdict.
//     Its two barriers order LDS only (no wait on the gathers in flight), so the check runs in
//     the shadow of the gathers. If any entry is invalid no block writes state; block 0
//     reports the verdict in *status. The page's kernel scans all earlier rows per row
//     (quadratic in N) and traps; here a block pays O(N + S/32) and the grid is sized so that
//     the number of blocks stays near a constant, keeping the total linear in N;
//   * a block that walks several rows issues the next row's loads before the current row's
//     arithmetic (its slot differs from every other row's, which the verdict guarantees
//     before anything is stored).
#include "../../include/cconv.h"
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

namespace cconv {

// Word 3 of a raw gfx9 buffer descriptor (32-bit data format; untyped loads and stores).
constexpr int kRawBufferWord3 = 0x00020000;

// A buffer resource over `bytes` bytes at `base` (bytes < 2^31; 0: every access is out of
// range, loads return zero and stores are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRawBufferWord3);
}

// cache policy of a buffer access: non-temporal or default
template <bool NT>
constexpr int cpol() {
    return NT ? 2 : 0;
}

template <bool NT>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, cpol<NT>());
}

template <bool NT>
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, cpol<NT>());
}

template <bool NT>
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t a, uint32_t b, uint32_t c,
                                         uint32_t d) {
    const u32x4 v = {a, b, c, d};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, cpol<NT>());
}

template <bool NT>
__device__ __forceinline__ void bstore2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(v & 0xffffu), r, static_cast<int>(off), 0,
                                          cpol<NT>());
}

// VEC/2 dwords (a chunk of VEC bf16 values: 16 bytes for VEC = 8, 8 for VEC = 4) at byte
// offset `off`.
template <int VEC, bool NT>
__device__ __forceinline__ void bload_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* dst) {
    static_assert(VEC == 4 || VEC == 8, "chunks of 4 or 8 bf16 values");
    if constexpr (VEC == 8) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, cpol<NT>());
        dst[0] = v.x, dst[1] = v.y, dst[2] = v.z, dst[3] = v.w;
    } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, cpol<NT>());
        dst[0] = v.x, dst[1] = v.y;
    }
}

template <int VEC, bool NT>
__device__ __forceinline__ void bstore_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint32_t* src) {
    static_assert(VEC == 4 || VEC == 8, "chunks of 4 or 8 bf16 values");
    if constexpr (VEC == 8) {
        const u32x4 v = {src[0], src[1], src[2], src[3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, cpol<NT>());
    } else {
        const u32x2 v = {src[0], src[1]};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(off), 0, cpol<NT>());
    }
}

// 16-bit entry `i` of a packed run of dwords (entry 2q in the low half of word q).
template <int N>
__device__ __forceinline__ uint32_t half_at(const uint32_t (&u)[N], int i) {
    return (i & 1) ? (u[i >> 1] >> 16) : (u[i >> 1] & 0xffffu);
}

// The thread's taps and bias, raw (converted once they are used). Taps: the VEC*W values
// w[d..d+VEC-1, 0..W-1], contiguous in w[D, W] (for VEC = 8 they start at a multiple of 16
// bytes: d is a multiple of 8 and w is 16-byte aligned), as bf16 pairs or fp32 words; bias:
// VEC fp32 words (zeros when absent).
template <int VEC, int W, bool WF32>
struct Params {
    uint32_t w[WF32 ? VEC * W : (VEC * W + 1) / 2];
    uint32_t b[VEC];
};

template <int VEC, int W, bool WF32>
__device__ __forceinline__ void load_params(const UpdateArgs& a, int64_t d, Params<VEC, W, WF32>& p) {
    constexpr int E = WF32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, a.D * W * E);
    const uint32_t ow = static_cast<uint32_t>(d * W * E);
    if constexpr (VEC == 8 || (VEC == 4 && WF32)) {
        // 16-byte chunks: the run starts at d*W*E, a multiple of 16 (d a multiple of 8, or of 4
        // with 4-byte taps)
        constexpr int Q = (VEC * W * E) / 16;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const u32x4 v = bload16<false>(rw, ow + 16 * q);
            p.w[4 * q] = v.x;
            p.w[4 * q + 1] = v.y;
            p.w[4 * q + 2] = v.z;
            p.w[4 * q + 3] = v.w;
        }
    } else if constexpr (VEC == 4) {
        // bf16 taps of 4 channels: W 8-byte chunks (the run starts at a multiple of 8)
#pragma unroll
        for (int q = 0; q < W; ++q) bload_chunk<4, false>(rw, ow + 8 * q, &p.w[2 * q]);
    } else if constexpr (WF32) {
#pragma unroll
        for (int k = 0; k < W; ++k)
            p.w[k] = __builtin_amdgcn_raw_buffer_load_b32(rw, static_cast<int>(ow + 4 * k), 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < (W + 1) / 2; ++i) p.w[i] = 0u;
#pragma unroll
        for (int k = 0; k < W; ++k) p.w[k >> 1] |= bload2<false>(rw, ow + 2 * k) << ((k & 1) * 16);
    }
    const __amdgpu_buffer_rsrc_t rb = rsrc(a.bias, a.bias ? a.D * 4 : 0);
    if constexpr (VEC >= 4) {
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
            const u32x4 v = bload16<false>(rb, static_cast<uint32_t>(d * 4 + 16 * q));
            p.b[4 * q] = v.x, p.b[4 * q + 1] = v.y, p.b[4 * q + 2] = v.z, p.b[4 * q + 3] = v.w;
        }
    } else {
        p.b[0] = __builtin_amdgcn_raw_buffer_load_b32(rb, static_cast<int>(d * 4), 0, 0);
    }
}

// tap[k][v] = w[d+v, W-1-k] (the ring's order, as load_taps), bias as floats.
template <int VEC, int W, bool WF32>
__device__ __forceinline__ void unpack_params(const Params<VEC, W, WF32>& p, float (&tap)[W][VEC], float (&bs)[VEC]) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const int e = v * W + (W - 1 - k);
            tap[k][v] = WF32 ? __uint_as_float(p.w[e]) : __uint_as_float(half_at(p.w, e) << 16);
        }
        bs[v] = __uint_as_float(p.b[v]);
    }
}

// One row's inputs for a thread: the slot, the circular position, the x values and the state
// entries (entry e of channel d+v is 16-bit entry v*L + e of `h`; zeros for a slot outside
// [0, S), which is not read).
template <int VEC, int LL>
struct DecIn {
    int64_t s;  // the slot; -1 for a padding row and for a row past the block's last
    int64_t c;
    bool valid;  // the row exists (n < the block's end): its y is stored
    Row<VEC> rx;
    uint32_t h[(VEC * LL + 1) / 2];
};

// The buffer over a row's state run: slot s's [D, L] entries, or nothing for a slot outside
// [0, S) (a padding row, or an invalid index that the verdict rejects).
template <int L>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_rsrc(const UpdateArgs& a, int64_t s) {
    const bool ok = s >= 0 && s < a.S;
    return rsrc(a.state + (ok ? s : 0) * a.D * L, ok ? a.D * L * 2 : 0);
}

// The slots and circular positions of rows n .. n+R-1 (those before `end` exist), one vector
// load each for all R rows: lane i mod R reads row n + (i mod R), and readlane makes each
// value block-uniform. One load, so one wait, whatever R is (a scalar load per row would
// each be waited for before the next is issued). Entries past `end` read as 0 (the buffer
// range ends there); such rows are marked invalid.
struct RowSlots {
    int32_t s, c;  // this lane's entries
};

template <bool CIRC, bool IDX, int R>
__device__ __forceinline__ RowSlots dec_slots(const int32_t* __restrict__ idx, const int32_t* __restrict__ cs,
                                              int64_t n, int64_t end) {
    const int64_t m = max<int64_t>(0, min<int64_t>(R, end - n));
    const uint32_t off = static_cast<uint32_t>((threadIdx.x % R) * 4);
    RowSlots r{0, 0};
    if constexpr (IDX) r.s = __builtin_amdgcn_raw_buffer_load_b32(rsrc(idx + n, m * 4), static_cast<int>(off), 0, 0);
    if constexpr (CIRC) r.c = __builtin_amdgcn_raw_buffer_load_b32(rsrc(cs + n, m * 4), static_cast<int>(off), 0, 0);
    return r;
}

template <bool CIRC, bool IDX, int R, int VEC, int LL>
__device__ __forceinline__ void dec_take_slots(const RowSlots& r, int64_t n, int64_t end, DecIn<VEC, LL> (&in)[R]) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
        in[i].valid = n + i < end;
        in[i].s = !in[i].valid ? -1 : (IDX ? static_cast<int64_t>(__builtin_amdgcn_readlane(r.s, i)) : n + i);
        in[i].c = CIRC ? static_cast<int64_t>(__builtin_amdgcn_readlane(r.c, i)) : 0;
    }
}

// Issue the gathers of row n: the x row and the slot's state run (empty ranges for a row past
// the block's end and for a slot outside [0, S)).
template <int VEC, int L, bool NTL, bool STG = false>
__device__ __forceinline__ void dec_gather(const UpdateArgs& a, int64_t n, int64_t d, DecIn<VEC, (L > 0 ? L : 1)>& in) {
    constexpr int LL = L > 0 ? L : 1;
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + (in.valid ? n : 0) * a.x_ld, in.valid ? a.D * 2 : 0);
    const uint32_t ox = static_cast<uint32_t>(d * 2);
    if constexpr (VEC >= 4) {
        bload_chunk<VEC, NTL>(rx, ox, in.rx.u);
    } else {
        in.rx.u[0] = bload2<NTL>(rx, ox);
    }
#pragma unroll
    for (int i = 0; i < (VEC * LL + 1) / 2; ++i) in.h[i] = 0u;
    if constexpr (L > 0) {
        const __amdgpu_buffer_rsrc_t rs = state_rsrc<L>(a, in.s);
        const uint32_t os = static_cast<uint32_t>(d * L * 2);
        if constexpr (STG) {
            // the wave's run, chunk q*64 + lane in this lane (stage_in puts the lane's own
            // chunks in place once they have landed)
            const uint32_t lane = threadIdx.x % kWave;
            const uint32_t wb = os - lane * (VEC * L * 2);
#pragma unroll
            for (int q = 0; q < L; ++q) bload_chunk<VEC, NTL>(rs, wb + (q * kWave + lane) * 16, &in.h[4 * q]);
        } else if constexpr (VEC >= 4) {
            // the run is L chunks of VEC values (chunk q: flat entries q*VEC .. q*VEC+VEC-1)
#pragma unroll
            for (int q = 0; q < L; ++q) bload_chunk<VEC, NTL>(rs, os + VEC * 2 * q, &in.h[(VEC / 2) * q]);
        } else {
#pragma unroll
            for (int e = 0; e < L; ++e) in.h[e >> 1] |= bload2<NTL>(rs, os + 2 * e) << ((e & 1) * 16);
        }
    }
}

// The loads of rows n .. n+R-1 (those before `end` exist): slots, then gathers.
template <int VEC, int L, bool CIRC, bool IDX, bool NTL, int R, bool STG = false>
__device__ __forceinline__ void dec_load(const UpdateArgs& a, const int32_t* __restrict__ idx,
                                         const int32_t* __restrict__ cs, int64_t n, int64_t end, int64_t d,
                                         DecIn<VEC, (L > 0 ? L : 1)> (&in)[R]) {
    dec_take_slots<CIRC, IDX, R>(dec_slots<CIRC, IDX, R>(idx, cs, n, end), n, end, in);
#pragma unroll
    for (int i = 0; i < R; ++i) dec_gather<VEC, L, NTL, STG>(a, n + i, d, in[i]);
}

// The wave's LDS staging region: 64 * L 16-byte chunks. Only this wave touches it; the
// fences order its LDS writes before the reads of other lanes of the same wave, and those
// reads before the region's next writes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Chunk-major (chunk q*64 + lane in this lane's h[4q..4q+3]) -> lane-major (the lane's own
// run, chunk k in h[4k..4k+3]).
template <int L, int NH>
__device__ __forceinline__ void stage_in(u32x4* __restrict__ stg, uint32_t (&h)[NH]) {
    const uint32_t lane = threadIdx.x % kWave;
#pragma unroll
    for (int q = 0; q < L; ++q) stg[q * kWave + lane] = u32x4{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const u32x4 v = stg[lane * L + k];
        h[4 * k] = v.x, h[4 * k + 1] = v.y, h[4 * k + 2] = v.z, h[4 * k + 3] = v.w;
    }
    wave_lds_sync();
}

// The tokens 1 .. W-1 steps back, from the L state entries, in the forward's ring order:
// ring[k-1] = x[t-k]. Shift mode (ROT < 0): entry L-k. Circular mode with rotation
// ROT = c mod L: entry (ROT - k) mod L.
template <int VEC, int W, int L, int ROT, int NH>
__device__ __forceinline__ void ring_from_state(const uint32_t (&h)[NH], float (&ring)[W > 1 ? W - 1 : 1][VEC]) {
#pragma unroll
    for (int k = 1; k < W; ++k) {
        const int e = ROT < 0 ? L - k : ((ROT - k) % L + L) % L;
#pragma unroll
        for (int v = 0; v < VEC; ++v) ring[k - 1][v] = __uint_as_float(half_at(h, v * L + e) << 16);
    }
}

// The state run after the row: shift mode (ROT < 0) drops entry 0 and appends x; circular
// mode replaces entry ROT by x and keeps the others (the whole run is stored: 16-byte stores
// beat 2-byte ones at decode sizes). VEC = 8 stores L 16-byte vectors; VEC = 1 stores entry
// by entry (shift) or the one changed entry (circular).
template <int VEC, int L, int ROT, bool NTS, int NH>
__device__ __forceinline__ void store_state(__amdgpu_buffer_rsrc_t rs, uint32_t os, const uint32_t (&h)[NH],
                                            const Row<VEC>& rx, u32x4* __restrict__ stg = nullptr) {
    if constexpr (VEC >= 4) {
        uint32_t nu[(VEC / 2) * L];
#pragma unroll
        for (int i = 0; i < (VEC / 2) * L; ++i) {
            uint32_t half[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int p = 2 * i + j, v = p / L, e = p % L;
                const bool tok = ROT < 0 ? (e == L - 1) : (e == ROT);
                half[j] = tok ? half_at(rx.u, v) : half_at(h, ROT < 0 ? p + 1 : p);
            }
            nu[i] = half[0] | (half[1] << 16);
        }
        if constexpr (VEC == 8) {
            if (stg) {
                // lane-major -> chunk-major through the wave's region: lane i stores chunk
                // q*64 + i of the wave's run
                const uint32_t lane = threadIdx.x % kWave;
                const uint32_t wb = os - lane * (VEC * L * 2);
#pragma unroll
                for (int k = 0; k < L; ++k) stg[lane * L + k] = u32x4{nu[4 * k], nu[4 * k + 1], nu[4 * k + 2], nu[4 * k + 3]};
                wave_lds_sync();
#pragma unroll
                for (int q = 0; q < L; ++q) {
                    const u32x4 v = stg[q * kWave + lane];
                    const uint32_t c[4] = {v.x, v.y, v.z, v.w};
                    bstore_chunk<8, NTS>(rs, wb + (q * kWave + lane) * 16, c);
                }
                wave_lds_sync();
                return;
            }
        }
#pragma unroll
        for (int q = 0; q < L; ++q) bstore_chunk<VEC, NTS>(rs, os + VEC * 2 * q, &nu[(VEC / 2) * q]);
    } else if constexpr (ROT < 0) {
#pragma unroll
        for (int e = 0; e + 1 < L; ++e) bstore2<NTS>(rs, os + 2 * e, half_at(h, e + 1));
        bstore2<NTS>(rs, os + 2 * (L - 1), rx.u[0]);
    } else {
        bstore2<NTS>(rs, os + 2 * ROT, rx.u[0]);
    }
}

// y and the new state of one row whose inputs have landed. A padding row (s < 0) stores
// y = 0 and, its state range being empty, no state.
template <int W, int L, int VEC, bool NTS, int ROT>
__device__ __forceinline__ void dec_finish(const UpdateArgs& a, const float (&tap)[W][VEC], const float (&bs)[VEC],
                                           const DecIn<VEC, (L > 0 ? L : 1)>& in, int64_t n, int64_t d,
                                           u32x4* __restrict__ stg) {
    constexpr int R = W > 1 ? W - 1 : 1;
    float xt[VEC];
    widen(in.rx, xt);
    float ring[R][VEC];
    if constexpr (W > 1) {
        ring_from_state<VEC, W, L, ROT>(in.h, ring);
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) ring[0][v] = 0.0f;
    }
    float y[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        const float z = conv_z<VEC, W>(tap, bs, xt, ring, v);
        y[v] = z * sigmoid(z);
    }
    Row<VEC> ry = narrow<VEC>(y);
    if (in.s < 0) ry = zero_row<VEC>();
    const __amdgpu_buffer_rsrc_t rr = rsrc(a.y + (in.valid ? n : 0) * a.D, in.valid ? a.D * 2 : 0);
    const uint32_t oy = static_cast<uint32_t>(d * 2);
    if constexpr (VEC >= 4) {
        bstore_chunk<VEC, NTS>(rr, oy, ry.u);
    } else {
        bstore2<NTS>(rr, oy, ry.u[0]);
    }
    if constexpr (L > 0)
        store_state<VEC, L, ROT, NTS>(state_rsrc<L>(a, in.s), static_cast<uint32_t>(d * L * 2), in.h, in.rx, stg);
}

template <int W, int L, bool CIRC, int VEC, bool NTS, bool STG = false>
__device__ __forceinline__ void dec_row(const UpdateArgs& a, const float (&tap)[W][VEC], const float (&bs)[VEC],
                                        DecIn<VEC, (L > 0 ? L : 1)>& in, int64_t n, int64_t d, u32x4* __restrict__ stg) {
    if constexpr (STG && L > 0) stage_in<L>(stg, in.h);
    u32x4* const sp = STG ? stg : nullptr;
    if constexpr (!CIRC || L == 0) {
        dec_finish<W, L, VEC, NTS, -1>(a, tap, bs, in, n, d, sp);
    } else {
        // the rotation is block-uniform: a uniform switch picks a compile-time entry map
        const int rot = static_cast<int>(in.c % L);
        if (rot == 0) dec_finish<W, L, VEC, NTS, 0>(a, tap, bs, in, n, d, sp);
        if constexpr (L > 1) if (rot == 1) dec_finish<W, L, VEC, NTS, (L > 1 ? 1 : 0)>(a, tap, bs, in, n, d, sp);
        if constexpr (L > 2) if (rot == 2) dec_finish<W, L, VEC, NTS, (L > 2 ? 2 : 0)>(a, tap, bs, in, n, d, sp);
        if constexpr (L > 3) if (rot == 3) dec_finish<W, L, VEC, NTS, (L > 3 ? 3 : 0)>(a, tap, bs, in, n, d, sp);
    }
}

// R: rows a thread carries at once (their loads are all in flight together, and the taps and
// bias are loaded once for them).
template <int W, int L, bool CIRC, int VEC, bool IDX, bool WF32, int OPT, int R>
__global__ __launch_bounds__(update_max_threads(R)) void cconv_update_kernel(const UpdateArgs a, const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ cs) {
    constexpr int LL = L > 0 ? L : 1;
    constexpr bool NTS = (OPT & kUpdNtStore) != 0, NTL = (OPT & kUpdNtLoad) != 0;
    constexpr bool STG = (OPT & kUpdStaged) != 0 && VEC == 8 && L > 0;
    constexpr bool CHECK = IDX || CIRC;
    extern __shared__ uint32_t seen[];
    // the staging regions follow the slot check's words, 16-byte aligned, one per wave
    u32x4* stg = nullptr;
    if constexpr (STG) {
        const int64_t words = IDX ? (a.S + 31) / 32 + 1 : (CIRC ? 1 : 0);
        stg = reinterpret_cast<u32x4*>(seen + ((words + 3) & ~int64_t(3))) + (threadIdx.x / kWave) * (kWave * LL);
    }

    const int64_t d = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * VEC;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * a.rows_per_block;
    const int64_t n1 = min(n0 + a.rows_per_block, a.N);

    // Issue order: the slot check's entries (row threadIdx.x; -1 and 0 past N), the first rows'
    // slots, the taps and bias, the first rows' x and state.
    SlotEntry first{-1, 0};
    if constexpr (CHECK) {
        const int64_t i0 = threadIdx.x;
        if constexpr (IDX) {
            const int32_t v = __builtin_amdgcn_raw_buffer_load_b32(rsrc(idx, a.N * 4), static_cast<int>(i0 * 4), 0, 0);
            first.v = i0 < a.N ? v : -1;
        }
        if constexpr (CIRC) first.c = __builtin_amdgcn_raw_buffer_load_b32(rsrc(cs, a.N * 4), static_cast<int>(i0 * 4), 0, 0);
    }
    const RowSlots rs0 = dec_slots<CIRC, IDX, R>(idx, cs, n0, n1);
    Params<VEC, W, WF32> prm;
    load_params<VEC, W, WF32>(a, d, prm);
    DecIn<VEC, LL> cur[R];
    dec_take_slots<CIRC, IDX, R>(rs0, n0, n1, cur);
#pragma unroll
    for (int i = 0; i < R; ++i) dec_gather<VEC, L, NTL, STG>(a, n0 + i, d, cur[i]);

    if constexpr (CHECK) {
        const bool bad = block_slots_bad(IDX ? idx : nullptr, CIRC ? cs : nullptr, a.N, a.S, seen, first);
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && a.status)
            a.status[0] = bad ? CCONV_ERR_INDEX : CCONV_OK;
        if (bad) return;
    } else if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && a.status) {
        a.status[0] = CCONV_OK;
    }

    float tap[W][VEC], bs[VEC];
    unpack_params<VEC, W, WF32>(prm, tap, bs);
    for (int64_t g = n0; g < n1; g += R) {
        DecIn<VEC, LL> nxt[R];
        if (g + R < n1) dec_load<VEC, L, CIRC, IDX, NTL, R, STG>(a, idx, cs, g + R, n1, d, nxt);
#pragma unroll
        for (int i = 0; i < R; ++i) dec_row<W, L, CIRC, VEC, NTS, STG>(a, tap, bs, cur[i], g + i, d, stg);
#pragma unroll
        for (int i = 0; i < R; ++i) cur[i] = nxt[i];
    }
}

// The slot check alone, for the prefill into a pool: one block writes the verdict, which the
// forward's waves read before they write anything.
__global__ __launch_bounds__(1024) void cconv_slots_kernel(const int32_t* __restrict__ idx, int64_t N, int64_t S,
                                                           int32_t* status) {
    extern __shared__ uint32_t seen[];
    const int64_t i0 = threadIdx.x;
    const SlotEntry first{i0 < N ? idx[i0] : -1, 0};
    const bool bad = block_slots_bad(idx, nullptr, N, S, seen, first);
    if (threadIdx.x == 0) status[0] = bad ? CCONV_ERR_INDEX : CCONV_OK;
}

__global__ void cconv_status_kernel(int32_t* status, int32_t value) {
    if (threadIdx.x == 0 && blockIdx.x == 0) status[0] = value;
}

namespace {

struct UpdLaunch {
    dim3 grid, block;
    size_t lds;
    hipStream_t s;
};

template <int W, int L, bool CIRC, int VEC, bool IDX, bool WF32, int OPT, int R>
void launch_one(const UpdLaunch& l, const UpdateArgs& a) {
    hipLaunchKernelGGL((cconv_update_kernel<W, L, CIRC, VEC, IDX, WF32, OPT, R>), l.grid, l.block, l.lds, l.s, a, a.idx,
                       a.cs);
}

template <int W, int L, bool CIRC, int VEC, bool IDX, bool WF32>
void launch_opt(int options, int rows_per_thread, const UpdLaunch& l, const UpdateArgs& a) {
    if constexpr (VEC == 1) {
        launch_one<W, L, CIRC, 1, IDX, WF32, 0, 1>(l, a);
    } else {
        constexpr int S = kUpdNtStore, N = kUpdNtLoad, G = kUpdStaged;
        const bool two = rows_per_thread != 1;
#define CCONV_UPD_OPT(o) \
    case o: two ? launch_one<W, L, CIRC, VEC, IDX, WF32, o, 2>(l, a) : launch_one<W, L, CIRC, VEC, IDX, WF32, o, 1>(l, a); break;
        // staging (8 channels per thread only) with or without non-temporal stores
        switch (options & (VEC == 8 ? (S | N | G) : (S | N))) {
            CCONV_UPD_OPT(0)
            CCONV_UPD_OPT(S)
            CCONV_UPD_OPT(N)
            CCONV_UPD_OPT(S | N)
            CCONV_UPD_OPT(G)
            default: CCONV_UPD_OPT(G | S)
        }
#undef CCONV_UPD_OPT
    }
}

template <int W, int L, bool CIRC, int VEC>
void launch_vec(int o, int r, const UpdLaunch& l, const UpdateArgs& a) {
    const bool idx = a.idx != nullptr, f32 = a.w_f32 != 0;
    if (idx)
        f32 ? launch_opt<W, L, CIRC, VEC, true, true>(o, r, l, a) : launch_opt<W, L, CIRC, VEC, true, false>(o, r, l, a);
    else
        f32 ? launch_opt<W, L, CIRC, VEC, false, true>(o, r, l, a) : launch_opt<W, L, CIRC, VEC, false, false>(o, r, l, a);
}

template <int W, int L, bool CIRC>
void launch_update_k(int vec, int o, int r, const UpdLaunch& l, const UpdateArgs& a) {
    if (vec == 8)
        launch_vec<W, L, CIRC, 8>(o, r, l, a);
    else if (vec == 4)
        launch_vec<W, L, CIRC, 4>(o, r, l, a);
    else
        launch_vec<W, L, CIRC, 1>(o, r, l, a);
}

template <int W>
hipError_t launch_update_w(int L, bool circ, int vec, int o, int r, const UpdLaunch& l, const UpdateArgs& a) {
    if (L == W - 1) {
        if (!circ) {
            launch_update_k<W, W - 1, false>(vec, o, r, l, a);
        } else if constexpr (W > 1) {
            launch_update_k<W, W - 1, true>(vec, o, r, l, a);
        } else {
            return hipErrorInvalidValue;  // a circular state needs at least one entry
        }
    } else if (L == W) {
        if (circ)
            launch_update_k<W, W, true>(vec, o, r, l, a);
        else
            launch_update_k<W, W, false>(vec, o, r, l, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_update(int W, int L, int vec, int options, int rows_per_thread, const UpdateArgs& a,
                         int block_threads, int64_t grid_x, int64_t grid_y, size_t lds, hipStream_t s) {
    const UpdLaunch l{dim3(static_cast<uint32_t>(grid_x), static_cast<uint32_t>(grid_y)), dim3(block_threads), lds, s};
    const bool circ = a.cs != nullptr;
    const int o = options, r = rows_per_thread;
    switch (W) {
        case 1: return launch_update_w<1>(L, circ, vec, o, r, l, a);
        case 2: return launch_update_w<2>(L, circ, vec, o, r, l, a);
        case 3: return launch_update_w<3>(L, circ, vec, o, r, l, a);
        case 4: return launch_update_w<4>(L, circ, vec, o, r, l, a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_slots(const int32_t* idx, int64_t N, int64_t S, int32_t* status, hipStream_t s) {
    const size_t lds = static_cast<size_t>((S + 31) / 32 + 1) * 4;
    hipLaunchKernelGGL(cconv_slots_kernel, dim3(1), dim3(1024), lds, s, idx, N, S, status);
    return hipGetLastError();
}

hipError_t launch_status(int32_t* status, int32_t value, hipStream_t s) {
    hipLaunchKernelGGL(cconv_status_kernel, dim3(1), dim3(64), 0, s, status, value);
    return hipGetLastError();
}

}  // namespace cconv
