// cconv_internal.hpp -- launch plans and kernel launchers shared by the C ABI (cconv_api.hip)
// and the kernels (cconv_fwd.hip, cconv_bwd.hip, cconv_update.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cconv {

// How a forward or backward call is cut into work.
//   A lane owns `vec` consecutive channels (a lane group); the D/vec lane groups are split into
//   `strips` channel strips of as equal a width as integers allow (strip s holds lane groups
//   floor(s*L/strips) .. floor((s+1)*L/strips) - 1, at most 64), and a wave owns one strip for
//   one time segment of `seg_rows` rows of one batch row. A block holds `waves` waves arranged
//   as `ws` adjacent strips x `waves/ws` consecutive segments of one batch row. `group` rows
//   are loaded together.
struct Plan {
    int vec;
    int group;
    int waves;
    int ws;  // strips per block
    int64_t seg_rows;
    int options;  // kNtLoad | kNtStore | kPrefetch | kSolo, plus the epilogue bits kLinear | kResidual
    // derived
    int64_t lane_groups;   // ceil(D / vec)
    int64_t strips;        // ceil(lane_groups / 64)
    int64_t strip_groups;  // ceil(strips / ws)
    int64_t segs;          // ceil(T / seg_rows)
    int64_t seg_groups;    // ceil(segs / (waves/ws))
    int64_t blocks;        // strip_groups * seg_groups * B
    int64_t partials;      // backward: B * seg_groups fp32 partial rows of [W+1, D]
};

struct FwdArgs {
    const uint16_t* x;
    int64_t x_sb, x_st;
    const void* w;
    int w_f32;
    const float* bias;
    uint16_t* y;
    const uint16_t* h0;  // [B, D, W-1] history before t = 0, or null (zeros)
    uint16_t* hT;        // [B, D, W-1] final state out, or null; may equal h0
    // Pool mode (sidx non-null): h0 and hT are a decode pool [S, D, W-1] and sequence b uses
    // slot sidx[b] (-1: zero history, no final state); its history is read only where
    // has_init[b] is set (null: nowhere). Every wave first reads *status, the verdict of the
    // slot check, and writes nothing unless it is CCONV_OK.
    const int32_t* sidx;
    const uint8_t* has_init;
    const int32_t* status;
    // Packed mode (cu non-null): B = 1, T = total rows; sequence i is rows cu[i] .. cu[i+1]-1
    // with its own history h0[i] and final state hT[i] (written by the wave holding its last
    // row, so hT must not share h0's memory). *status holds the offset check's verdict.
    const int32_t* cu;
    int64_t nseq;
    // residual added after the activation (kResidual): bf16 rows like x's, strides r_sb, r_st
    const uint16_t* r;
    int64_t r_sb, r_st;
    // y's batch and row strides in elements (y_st >= D; y_sb ignored for packed batches)
    int64_t y_sb, y_st;
    int64_t B, T, D;
    int64_t seg_rows, strip_groups, seg_groups;
    int ws;
    int64_t lane_groups, strips;  // the channel split (see Plan)
};

struct BwdArgs {
    const uint16_t* x;
    int64_t x_sb, x_st;
    const uint16_t* dy;
    int64_t dy_sb, dy_st;
    const void* w;
    int w_f32;
    const float* bias;
    uint16_t* dx;
    int64_t dx_sb, dx_st;  // dx's batch and row strides in elements (dx_st >= D)
    float* partial;      // [partials, W+1, D]
    const uint16_t* h0;  // [B, D, W-1] history before t = 0, or null (zeros)
    uint16_t* dh0;       // [B, D, W-1] gradient of the history out, or null
    // Packed mode as in FwdArgs: h0 and dh0 are [nseq, D, W-1]; sequence i's history gradient
    // is written by the wave holding its first row. Waves skip everything unless *status
    // (when given) is CCONV_OK, and then leave their partials unwritten.
    const int32_t* cu;
    int64_t nseq;
    const int32_t* status;
    int64_t B, T, D;
    int64_t seg_rows, strip_groups, seg_groups;
    int ws;
    int64_t lane_groups, strips;  // the channel split (see Plan)
};

struct ReduceArgs {
    const float* partial;  // [P, W+1, D]
    int64_t P, D;
    int W;
    void* dw;  // [D, W]
    int dw_f32;
    float* dbias;  // [D] or null
    const int32_t* status;  // when given, nothing is written unless *status is CCONV_OK
};

struct UpdateArgs {
    const uint16_t* x;
    int64_t x_ld;
    uint16_t* state;  // [S, D, L], L = W-1 or W
    int64_t S;
    const int32_t* idx;  // [N] or null
    const int32_t* cs;   // [N] cache_seqlens (circular state) or null (shift)
    const void* w;
    int w_f32;
    const float* bias;
    uint16_t* y;  // [N, D]
    int64_t N, D;
    int64_t rows_per_block;  // rows of N each block walks
    int32_t* status;
};

// Largest block of the decode update when a thread carries R rows at once: each row in flight
// holds up to 16 registers (x and the state run), so R = 2 needs more than the 128 VGPRs a
// lane of a 1024-thread block may use.
constexpr int update_max_threads(int R) { return R >= 2 ? 512 : 1024; }

// Launchers: enqueue on `stream`, return hipGetLastError() after the launch.
hipError_t launch_fwd(const Plan& p, int W, const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const Plan& p, int W, const BwdArgs& a, hipStream_t stream);
// Packed batches and epilogue variants (their own translation units).
hipError_t launch_fwd_extra(const Plan& p, int W, const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_extra(const Plan& p, int W, const BwdArgs& a, hipStream_t stream);
// Whether a kernel is compiled for this launch: (vec, group), options (kernel option bits,
// kSolo and the epilogue bits included), packed or not.
bool fwd_launch_exists(int vec, int group, int options, bool packed);
bool bwd_launch_exists(int vec, int group, int options, bool packed);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_update(int W, int L, int vec, int options, int rows_per_thread, const UpdateArgs& a,
                         int block_threads, int64_t grid_x, int64_t grid_y, size_t lds_bytes, hipStream_t stream);
hipError_t launch_status(int32_t* status, int32_t value, hipStream_t stream);
hipError_t launch_slots(const int32_t* idx, int64_t N, int64_t S, int32_t* status, hipStream_t stream);
// Packed batches: the offset check (one block writes *status), then, when it passes, the
// states of empty sequences (final state hT = history or zeros, history gradient dh0 = 0;
// either may be null), which no streaming wave holds.
hipError_t launch_offsets(const int32_t* cu, int64_t nseq, int64_t total, int32_t* status, const uint16_t* h0,
                          uint16_t* hT, uint16_t* dh0, int64_t D, int L, hipStream_t stream);

// Which (vec, group) pairs are compiled.
bool fwd_variant_exists(int vec, int group);
bool bwd_variant_exists(int vec, int group);

}  // namespace cconv
