// cconv_api.hip -- the C ABI declared in include/cconv.h: host-side validation, launch
// planning and dispatch. Nothing here allocates device memory, synchronises, or reads device
// memory; every check that can fail happens before the first launch, so an error leaves all
// outputs untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/cconv.h"
#include "cconv_device.hpp"
#include "cconv_internal.hpp"

using cconv::Plan;

// ---- the backward without a caller workspace ----------------------------------------------
// The dw/dbias partials of cconv_bwd_noalloc live in this file-scope device array: each GPU the
// library runs on holds its own copy from the first call until the process ends. In host code
// `scratch` is only a stand-in for the symbol; the array's device address on each GPU comes
// from hipGetSymbolAddress, looked up once per device (with that device current) and kept.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on its first use on that device).
cconv_status_t scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return CCONV_ERR_LAUNCH;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CCONV_ERR_LAUNCH;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return CCONV_OK;
}

}  // namespace


namespace {

constexpr int64_t kMaxDim = int64_t(1) << 40;        // any one size or stride
constexpr int64_t kMaxDecodeRows = int64_t(1) << 24;  // N
constexpr int64_t kMaxChannels = int64_t(1) << 30;    // D: lane channel offsets are 32-bit
// S with state_indices: the slot check's S-bit set and its verdict word fill at most 64 KB of LDS
constexpr int64_t kMaxIndexedSlots = (int64_t(1) << 19) - 32;
// LDS of a decode block with staged state runs (the slot check's words plus the regions)
constexpr size_t kMaxUpdateLds = size_t(64) << 10;
constexpr int64_t kMaxSequences = int64_t(1) << 24;     // packed sequences per call
constexpr int64_t kTargetWaves = 1024;  // wave slots of the solo kernels: one per SIMD (256 CUs x 4 SIMDs)
// wave slots of the narrow path (one channel per lane): three waves per SIMD for the forward,
// two for the backward (interleaved sweeps at [8,8192,D] for D = 4098, 2050, 1003 and at
// [4,4096,4098]: 6-9% faster forwards, 4-8% faster backwards than four waves per SIMD)
constexpr int64_t kNarrowFwdTargetWaves = 3072;
constexpr int64_t kNarrowBwdTargetWaves = 2048;
// wave slots of the two-channel lanes (the default at D = 2; an explicit option at other
// D = 2 (mod 4)): two waves per SIMD (interleaved sweeps of 1024 to 4096 at [8,8192,4098] and
// [4,8192,2050]: best or within 3% of the best for both passes)
constexpr int64_t kPairFwdTargetWaves = 2048;
constexpr int64_t kPairBwdTargetWaves = 2048;
// forward and backward: non-temporal loads and stores, solo kernel (no software prefetch)
constexpr int kFwdOptions = cconv::kNtLoad | cconv::kNtStore | cconv::kSolo;
constexpr int kBwdOptions = cconv::kNtLoad | cconv::kNtStore | cconv::kSolo;
// calls that stream at most this many bytes (the 256 MB Infinity Cache) keep non-temporal hints
// even on rows that miss the 128-byte lines
constexpr int64_t kSmallStreamBytes = int64_t(256) << 20;
constexpr int64_t kUpdateTargetBlocks = 1024;
// D of the decode update: its buffer ranges (a slot's [D, L] state run, fp32 taps [D, W]) stay
// below 2^31 bytes
constexpr int64_t kMaxDecodeChannels = int64_t(1) << 26;
// Decode launch (kernel-trace sweeps of block size x rows per thread x channels per thread x
// store hints at N = 256, D = 4096, W = 4, from HBM: 256-thread blocks, two rows per thread,
// 8 channels per thread and non-temporal stores took 5.3 us per call, the other 33 shapes
// 5.3-8.0 us; non-temporal loads and 4-channel threads did not help). With 8 channels per
// thread the state runs also pass through LDS (contiguous loads and stores): 5.53 -> 5.33 us
// a call in graph replays from HBM (the 16*L-byte lane stride had kept the texture
// addresser's queues full). Without room in LDS (a very large S) the plan drops that bit.
constexpr int64_t kUpdateThreads = 256;
constexpr int kUpdateOptions = cconv::kUpdNtStore;
constexpr int kUpdateOptions8 = cconv::kUpdNtStore | cconv::kUpdStaged;
constexpr int64_t kUpdateRowsPerThread = 2;
constexpr int kUpdateVec8 = 8;  // channels per thread when D % 8 == 0

struct Span {
    uintptr_t lo, hi;
};

// The byte range of an operand; an absent (NULL) operand occupies nothing.
Span span(const void* p, __int128 bytes) {
    if (!p) return {0, 0};
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlap(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Bytes spanned by a [B, T, D] tensor with strides (sb, st, 1).
__int128 extent3(int64_t B, int64_t T, int64_t D, int64_t sb, int64_t st, int esize) {
    if (B == 0 || T == 0 || D == 0) return 0;
    return (static_cast<__int128>(B - 1) * sb + static_cast<__int128>(T - 1) * st + D) * esize;
}

int esize(cconv_dtype_t t) { return t == CCONV_F32 ? 4 : 2; }
bool dtype_ok(cconv_dtype_t t) { return t == CCONV_BF16 || t == CCONV_F32; }

bool config_ok(const cconv_config_t& c, bool bwd) {
    if (bwd ? !cconv::bwd_variant_exists(c.vec, c.rows_per_group)
            : !cconv::fwd_variant_exists(c.vec, c.rows_per_group))
        return false;
    if (c.waves_per_block != 1 && c.waves_per_block != 2 && c.waves_per_block != 4 && c.waves_per_block != 8)
        return false;
    if (c.strips_per_block < 1 || c.waves_per_block % c.strips_per_block != 0) return false;
    if (c.seg_rows < 8 || c.seg_rows > kMaxDim || c.seg_rows % c.rows_per_group != 0) return false;
    if (c.options < 0 || c.options > 15) return false;
    if ((c.options & cconv::kSolo) && c.waves_per_block != 1) return false;  // solo kernels run one-wave blocks
    return true;
}

// The static launch table (from sweeps on MI355X at 8x8192x4096, W=4, and at D = 4100, 4104
// and 4160). Each wave owns one (channel strip, time segment, batch row) and streams its rows:
// fewer, longer-running waves beat more, shorter ones, and a wave alone on its SIMD may use the
// whole register file (the "solo" kernels), which is what lets deep row groups stay in flight
// without scratch spills.
//   * Shape: 4 channels per lane and 16-row groups (the backward loads 16 rows of x and 16 of
//     dy per group: 16 KiB in flight per wave), also for D = 4 (mod 8), whose rows are
//     8-byte aligned (at D = 4100 this halves the one-channel plan's time), and for D = 2
//     (mod 4), D >= 6, whose rows are 4-byte aligned (8-byte accesses need only dword
//     alignment) and whose last lane group overlaps its neighbour by two channels (at
//     [8,8192,4098] forward 261 -> 210 us, backward 386 -> 328 us against two channels per
//     lane). D = 2: two channels per lane; odd D: one; both with 16-row groups and the general
//     kernel.
//   * Strips: the D/vec lane groups are dealt to ceil(D/(64*vec)) strips of near-equal width
//     (strip s takes groups floor(s*L/n) .. floor((s+1)*L/n) - 1). At D = 4100 and 4104 the 17
//     strips carry 60 or 61 lane groups each instead of sixteen full strips and one holding one
//     or two: forward 238 -> 208 us and 247 -> 210 us at [8,8192,D] (the backward, whose waves
//     are bound by their own instruction stream, is unchanged at 323-326 us).
//   * Segments: each batch row is cut into as many segments as the wave slots allow (1024
//     solo waves, one per SIMD; kNarrow*TargetWaves for the narrow path) and no more. A grid
//     slightly larger than the slots (17 strips x 8 segments x 8 rows = 1088 waves at D = 4160)
//     leaves the extra waves sharing a SIMD with another, and the kernel waits for them: about
//     twice the time. Segments shrink to a single row group (16 rows) when the problem is
//     too small to fill the slots otherwise: the W-1 rows each segment re-reads then cost
//     less than idle SIMDs (graph-timed, from HBM: [1,256,512] forward 9.9 -> 4.3 us and
//     backward 20.4 -> 11.0 us with 16- instead of 64-row segments; [3,1000,2000] W=2 forward
//     12.9 -> 8.9 us and backward 22.6 -> 17.3 us with 32-row ones).
//   * Cache hints: non-temporal loads and stores when every streamed row starts on a 128-byte
//     cache line (for contiguous operands, 2D a multiple of 128), or when the call streams at
//     most kSmallStreamBytes; otherwise plain ones, so that the L2 merges the lines two
//     neighbouring strips share (at D = 4104: 214 vs 254 us forward, 332 vs 387 us backward;
//     at [3,1000,2000], whose rows miss the lines too, the non-temporal hints are the faster:
//     8.9 vs 10.1 us forward, 17.3 vs 19.2 us backward). The narrow path always runs plain
//     ones. Packed batches and the epilogue variants keep the streaming hints (their kernels
//     are compiled for those only).
//   `line_rows_in` (-1: from D alone, as for contiguous operands on 128-byte aligned bases)
//   says whether every streamed row of the call starts on a 128-byte line.
//   `lanes` says whether the call's activations meet the rule of the shape's lane width: for
//   D = 4 (mod 8), 8-byte aligned, strides multiples of 4; for D = 2 (mod 4), 4-byte aligned,
//   even strides. When they do not, the plan
//   runs one channel per lane with that lane width's segments: the dw/dbias partials (their
//   count, so the workspace and what a finishing stage reads) stay those of the shape,
//   whatever the layout.
cconv_config_t default_config(bool bwd, int64_t B, int64_t T, int64_t D, int W, bool streaming_only = false,
                              int line_rows_in = -1, bool lanes = true) {
    (void)W;
    cconv_config_t c;
    // odd D: one channel per lane; D = 2: two; every other even D: four (at D = 2 (mod 4) the
    // last lane group overlaps its neighbour by two channels)
    const bool narrow = (D % 2 != 0);
    const bool pair = (D == 2);
    c.vec = pair ? 2 : (narrow ? 1 : 4);
    c.rows_per_group = 16;
    c.waves_per_block = 1;
    c.strips_per_block = 1;
    const bool line_rows = line_rows_in < 0 ? (2 * D) % 128 == 0 : line_rows_in != 0;
    const bool small = static_cast<__int128>(B) * T * D * (bwd ? 6 : 4) <= kSmallStreamBytes;
    if (narrow || pair)
        c.options = cconv::kNarrowOptions;
    else if (line_rows || streaming_only || small)
        c.options = bwd ? kBwdOptions : kFwdOptions;
    else
        c.options = cconv::kSolo;
    // segment length: a multiple of the row group (and of 8), at least one group, at most T
    // rounded up
    const int64_t align = std::max<int64_t>(8, c.rows_per_group);
    const int64_t lane_groups = (D + c.vec - 1) / c.vec;
    const int64_t strips = std::max<int64_t>(1, (lane_groups + cconv::kWave - 1) / cconv::kWave);
    const int64_t slots = pair     ? (bwd ? kPairBwdTargetWaves : kPairFwdTargetWaves)
                          : narrow ? (bwd ? kNarrowBwdTargetWaves : kNarrowFwdTargetWaves)
                                   : kTargetWaves;
    // (batch row, strip) pairs; the product is formed only when both factors are within the
    // slot count (no overflow at the largest sizes the API accepts)
    const int64_t b1 = std::max<int64_t>(B, 1);
    const int64_t per_row = (b1 > slots || strips > slots) ? 1 : std::max<int64_t>(1, slots / (b1 * strips));
    const int64_t t = std::max<int64_t>(T, 1);
    int64_t ts = (t + per_row - 1) / per_row;
    ts = std::max(align, ((ts + align - 1) / align) * align);
    const int64_t tcap = ((t + align - 1) / align) * align;
    c.seg_rows = std::min(ts, tcap);
    if (!narrow && D % 8 != 0 && !lanes) {
        c.vec = 1;
        c.options = cconv::kNarrowOptions;
    }
    return c;
}

bool make_plan(const cconv_config_t& c, int64_t B, int64_t T, int64_t D, Plan* p) {
    p->vec = c.vec;
    p->group = c.rows_per_group;
    p->waves = c.waves_per_block;
    p->ws = c.strips_per_block;
    p->seg_rows = c.seg_rows;
    p->options = c.options;
    p->lane_groups = (D + c.vec - 1) / c.vec;
    p->strips = (p->lane_groups + cconv::kWave - 1) / cconv::kWave;
    p->strip_groups = (p->strips + p->ws - 1) / p->ws;
    p->segs = (T + c.seg_rows - 1) / c.seg_rows;
    const int64_t wt = c.waves_per_block / c.strips_per_block;
    p->seg_groups = (p->segs + wt - 1) / wt;
    const __int128 blocks = static_cast<__int128>(p->strip_groups) * p->seg_groups * B;
    if (blocks > INT32_MAX) return false;
    p->blocks = static_cast<int64_t>(blocks);
    p->partials = B * p->seg_groups;
    return true;
}

// Whether every row of a [B, T, D] operand with strides (sb, st, 1) starts on a 128-byte line.
bool on_lines(const void* p, int64_t sb, int64_t st) {
    return aligned(p, 128) && (2 * st) % 128 == 0 && (2 * sb) % 128 == 0;
}

// Whether a [B, T, D] operand meets the rule of v channels per lane: 2v-byte aligned, strides
// multiples of v.
bool on_lanes(const void* p, int64_t sb, int64_t st, int v) {
    return aligned(p, static_cast<uintptr_t>(2 * v)) && sb % v == 0 && st % v == 0;
}

// The operand rule (channels of alignment) the default plan of D asks for: 4 for D = 0 (mod 4)
// (also for D = 0 mod 8, whose plans check the 8-channel granule instead), 2 for D = 2 (mod 4)
// (four channels per lane on 4-byte aligned rows), 1 for odd D.
int lane_width(int64_t D) { return D % 4 == 0 ? 4 : (D % 4 == 2 ? 2 : 1); }

// Whether a plan's lane width fits D: whole lane groups, or four channels per lane over an
// even D >= 6 whose last group overlaps its neighbour.
bool width_ok(const cconv_config_t& c, int64_t D) {
    return D % c.vec == 0 || (c.vec == 4 && D % 4 == 2 && D > 4);
}

// Checks shared by the forward and backward before a plan exists: sizes, width, tap dtype.
cconv_status_t check_train_common(cconv_dtype_t w_dtype, int64_t B, int64_t T, int64_t D, int W) {
    if (B < 0 || T < 0 || D < 0 || B > kMaxDim || T > kMaxDim || D > kMaxDim) return CCONV_ERR_BAD_SHAPE;
    if (W < 1 || W > 4) return CCONV_ERR_BAD_SHAPE;
    if (D > kMaxChannels) return CCONV_ERR_BAD_SHAPE;
    if (!dtype_ok(w_dtype)) return CCONV_ERR_UNSUPPORTED_DTYPE;
    return CCONV_OK;
}

// The channel granule of a plan: the operand rules follow from it. 8 for a vector plan over
// whole 8-channel groups (16-byte aligned rows, strides multiples of 8, 16-byte aligned taps,
// bias, dw and states); 4 for a 4-channel plan with D = 4 (mod 8) (8-byte aligned rows, strides
// multiples of 4; the taps, bias, dw and states are read and written per element, so element
// alignment); 2 for a 2-channel plan, and for a 4-channel plan with D = 2 (mod 4) (4-byte
// aligned rows, even strides, element alignment elsewhere); 1 for the element-granular plan
// (one channel per lane: any stride, element alignment everywhere).
int granule(const cconv_config_t& c, int64_t D) {
    return c.vec <= 2 ? c.vec : (D % 8 == 0 ? 8 : (D % 4 == 0 ? 4 : 2));
}

// Alignment of the taps and bias: 16 bytes for granule 8; the element size otherwise.
cconv_status_t check_params(const void* w, cconv_dtype_t w_dtype, const float* bias, int gran) {
    const bool wide = (gran == 8);
    const uintptr_t wa = wide ? 16 : static_cast<uintptr_t>(esize(w_dtype)), ba = wide ? 16 : 4;
    if (!aligned(w, wa) || (bias && !aligned(bias, ba))) return CCONV_ERR_MISALIGNED;
    return CCONV_OK;
}

// A bf16 [B, T, D] operand with strides (sb, st, 1): strides multiples of the plan's granule
// and 2 * granule bytes of alignment (granule 8: 16 bytes; 4: 8 bytes, whole 8-byte rows per
// lane; 2: 4 bytes; 1: any strides, 2-byte alignment).
cconv_status_t check_act(const void* p, int64_t sb, int64_t st, int64_t D, int gran) {
    if (sb < 0 || st < D || sb > kMaxDim || st > kMaxDim) return CCONV_ERR_BAD_STRIDE;
    if (sb % gran != 0 || st % gran != 0) return CCONV_ERR_BAD_STRIDE;
    if (!aligned(p, static_cast<uintptr_t>(2 * gran))) return CCONV_ERR_MISALIGNED;
    return CCONV_OK;
}

// An output [B, T, D] with strides (sb, st, 1) given by the caller: the operand rules of
// check_act, and rows that do not overlap (st >= D and, for B > 1, each batch row's rows end
// before the next batch row starts).
cconv_status_t check_out(const void* p, int64_t sb, int64_t st, int64_t B, int64_t T, int64_t D, int gran) {
    const cconv_status_t s = check_act(p, sb, st, D, gran);
    if (s != CCONV_OK) return s;
    if (B > 1 && T > 0 && static_cast<__int128>(sb) < static_cast<__int128>(T - 1) * st + D) return CCONV_ERR_BAD_STRIDE;
    return CCONV_OK;
}

size_t bwd_workspace(const Plan& p, int64_t D, int W) {
    return static_cast<size_t>(p.partials) * static_cast<size_t>(W + 1) * static_cast<size_t>(D) * sizeof(float);
}

// What a call adds to the plain forward or backward: a history and its output (the final
// state, or the history's gradient), and the mode those live in.
//   kPerSeq  one state row per batch row, [B, D, W-1] (the forward may advance it in place);
//   kPool    rows of a decode pool [S, D, W-1], addressed by slot indices, under the slot rule;
//   kPacked  one row per packed sequence, [nseq, D, W-1], sequences given by device offsets.
// Pool and packed calls report through a device status word, written by every call that
// returns CCONV_OK; the streaming kernels write nothing unless it reads CCONV_OK.
enum Mode { kPerSeq, kPool, kPacked };
struct Extra {
    Mode mode = kPerSeq;
    const void* h0 = nullptr;
    void* out = nullptr;
    int64_t rows = 0;                   // state rows for kPool (S) and kPacked (nseq)
    const int32_t* sidx = nullptr;      // kPool
    const uint8_t* has_init = nullptr;  // kPool
    const int32_t* cu = nullptr;        // kPacked
    int32_t* status = nullptr;          // kPool, kPacked
    // epilogue: no activation (y = z; the backward's g = dy), and the forward's residual
    bool linear = false;
    const void* r = nullptr;
    int64_t r_sb = 0, r_st = 0;
    // the output's (y's, dx's) batch and row strides; o_st == 0: contiguous [B, T, D]
    int64_t o_sb = 0, o_st = 0;
    // backward: the partials go to the library's static scratch (no caller workspace)
    bool scratch = false;
};

// Checks of the states and of the pool/packed metadata against the call's other operands.
// `ins` and `outs` are the call's own tensors; returns CCONV_OK or the error.
cconv_status_t check_extra(const Extra& ex, int64_t B, int64_t D, int W, bool fwd, const Span* ins, int n_in,
                           const Span* outs, int n_out, Span* sh0_out, uintptr_t state_align) {
    const void* h0 = ex.h0;
    const void* out = ex.out;
    if (!aligned(h0, state_align) || !aligned(out, state_align)) return CCONV_ERR_MISALIGNED;
    const int64_t rows = ex.mode == kPerSeq ? B : ex.rows;
    const __int128 state_bytes = static_cast<__int128>(rows) * D * (W - 1) * 2;
    const Span sh0 = span(h0, state_bytes), so = span(out, state_bytes);
    *sh0_out = sh0;
    // the output state against every operand; in place only for a forward's per-sequence
    // states or pool (the packed final state is written while other waves still read h0)
    for (int i = 0; i < n_in; ++i)
        if (overlap(so, ins[i])) return CCONV_ERR_ALIASING;
    for (int i = 0; i < n_out; ++i)
        if (overlap(so, outs[i]) || overlap(sh0, outs[i])) return CCONV_ERR_ALIASING;
    const bool in_place_ok = fwd && ex.mode != kPacked && out == h0;
    if (!in_place_ok && overlap(so, sh0)) return CCONV_ERR_ALIASING;
    if (ex.mode == kPerSeq) return CCONV_OK;
    if (!ex.status) return CCONV_ERR_NULL_POINTER;
    if (!aligned(ex.status, 4) || !aligned(ex.sidx, 4) || !aligned(ex.cu, 4)) return CCONV_ERR_MISALIGNED;
    const Span meta[3] = {span(ex.sidx, static_cast<__int128>(B) * 4), span(ex.has_init, B),
                          span(ex.cu, ex.mode == kPacked ? static_cast<__int128>(ex.rows + 1) * 4 : 0)};
    const Span ss = span(ex.status, 4);
    for (int i = 0; i < n_in; ++i)
        if (overlap(ss, ins[i])) return CCONV_ERR_ALIASING;
    for (int i = 0; i < n_out; ++i)
        if (overlap(ss, outs[i])) return CCONV_ERR_ALIASING;
    if (overlap(ss, sh0) || overlap(ss, so)) return CCONV_ERR_ALIASING;
    for (const Span& m : meta) {
        if (overlap(ss, m) || overlap(so, m)) return CCONV_ERR_ALIASING;
        for (int i = 0; i < n_out; ++i)
            if (overlap(m, outs[i])) return CCONV_ERR_ALIASING;
    }
    return CCONV_OK;
}

// The first launches of a pool or packed call: the check that writes the status word, and for
// packed batches the states of empty sequences.
cconv_status_t launch_checks(const Extra& ex, int64_t B, int64_t T, int64_t D, int W, bool fwd, hipStream_t s) {
    if (ex.mode == kPool && cconv::launch_slots(ex.sidx, B, ex.rows, ex.status, s) != hipSuccess)
        return CCONV_ERR_LAUNCH;
    if (ex.mode == kPacked) {
        const uint16_t* h0 = static_cast<const uint16_t*>(ex.h0);
        uint16_t* o = static_cast<uint16_t*>(ex.out);
        if (cconv::launch_offsets(ex.cu, ex.rows, T, ex.status, h0, fwd ? o : nullptr, fwd ? nullptr : o, D, W - 1,
                                  s) != hipSuccess)
            return CCONV_ERR_LAUNCH;
    }
    return CCONV_OK;
}

cconv_status_t fwd_impl(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                        const float* bias, void* y, int64_t B, int64_t T, int64_t D, int W,
                        const cconv_config_t* cfg, cconv_stream_t stream, Extra ex = Extra{}) {
    // a pointer may be NULL only when its tensor is empty
    const bool act_empty = (B == 0 || T == 0 || D == 0);
    if ((!x && !act_empty) || (!w && D > 0) || (!y && !act_empty)) return CCONV_ERR_NULL_POINTER;
    cconv_status_t st = check_train_common(w_dtype, B, T, D, W);
    if (st != CCONV_OK) return st;
    const int epi = (ex.linear ? cconv::kLinear : 0) | (ex.r ? cconv::kResidual : 0);
    // packed batches and the epilogue variants are compiled for the streaming hints only
    // the default plan's cache hints follow where the call's rows actually start
    const bool lines = on_lines(x, x_sb, x_st) &&
                       (ex.o_st ? on_lines(y, ex.mode == kPacked ? 0 : ex.o_sb, ex.o_st) : on_lines(y, T * D, D)) &&
                       (!ex.r || on_lines(ex.r, ex.r_sb, ex.r_st));
    const int lv = lane_width(D);
    const bool lanes = on_lanes(x, x_sb, x_st, lv) &&
                       (ex.o_st ? on_lanes(y, ex.mode == kPacked ? 0 : ex.o_sb, ex.o_st, lv) : on_lanes(y, T * D, D, lv)) &&
                       (!ex.r || on_lanes(ex.r, ex.r_sb, ex.r_st, lv));
    const cconv_config_t c =
        cfg ? *cfg : default_config(false, B, T, D, W, ex.mode == kPacked || epi != 0, lines, lanes);
    if (!config_ok(c, false)) return CCONV_ERR_BAD_CONFIG;
    if (!width_ok(c, D)) return CCONV_ERR_BAD_CONFIG;
    const int gran = granule(c, D);
    if ((st = check_params(w, w_dtype, bias, gran)) != CCONV_OK) return st;
    if ((st = check_act(x, x_sb, x_st, D, gran)) != CCONV_OK) return st;
    int64_t y_sb = T * D, y_st = D;  // contiguous unless the general entry point gives strides
    if (ex.o_st != 0) {
        y_st = ex.o_st;
        y_sb = ex.mode == kPacked ? 0 : ex.o_sb;
        if ((st = check_out(y, y_sb, y_st, B, T, D, gran)) != CCONV_OK) return st;
    } else if (!aligned(y, static_cast<uintptr_t>(2 * gran))) {
        return CCONV_ERR_MISALIGNED;
    }
    if (!cconv::fwd_launch_exists(c.vec, c.rows_per_group, c.options | epi, ex.mode == kPacked))
        return CCONV_ERR_BAD_CONFIG;
    if (ex.r && (st = check_act(ex.r, ex.r_sb, ex.r_st, D, gran)) != CCONV_OK) return st;
    const Span sy = span(y, extent3(B, T, D, y_sb, y_st, 2));
    const Span sx = span(x, extent3(B, T, D, x_sb, x_st, 2));
    const Span sw = span(w, static_cast<__int128>(D) * W * esize(w_dtype));
    const Span sb = bias ? span(bias, static_cast<__int128>(D) * 4) : Span{0, 0};
    const Span sr = ex.r ? span(ex.r, extent3(B, T, D, ex.r_sb, ex.r_st, 2)) : Span{0, 0};
    if (overlap(sy, sx) || overlap(sy, sw) || overlap(sy, sb) || overlap(sy, sr)) return CCONV_ERR_ALIASING;
    // history in, final state out (W == 1 has none)
    if (W == 1) ex.h0 = ex.out = nullptr;
    const Span ins[4] = {sx, sw, sb, sr};
    Span sh0;
    if ((st = check_extra(ex, B, D, W, true, ins, 4, &sy, 1, &sh0, gran == 8 ? 16 : 2)) != CCONV_OK) return st;
    Plan p;
    if (!make_plan(c, B, T, D, &p)) return CCONV_ERR_BAD_SHAPE;
    p.options |= epi;
    // a per-sequence or pool final state needs at least one token
    if (ex.out && ex.mode != kPacked && T == 0 && B > 0 && D > 0) return CCONV_ERR_BAD_SHAPE;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    if ((st = launch_checks(ex, B, T, D, W, true, hs)) != CCONV_OK) return st;
    if (B == 0 || T == 0 || D == 0) return CCONV_OK;
    cconv::FwdArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.x_sb = x_sb;
    a.x_st = x_st;
    a.w = w;
    a.w_f32 = (w_dtype == CCONV_F32);
    a.bias = bias;
    a.y = static_cast<uint16_t*>(y);
    a.y_sb = y_sb;
    a.y_st = y_st;
    a.h0 = static_cast<const uint16_t*>(ex.h0);
    a.hT = static_cast<uint16_t*>(ex.out);
    a.sidx = ex.sidx;
    a.has_init = ex.has_init;
    a.status = ex.status;
    a.cu = ex.cu;
    a.nseq = ex.mode == kPacked ? ex.rows : 0;
    a.r = static_cast<const uint16_t*>(ex.r);
    a.r_sb = ex.r_sb;
    a.r_st = ex.r_st;
    a.B = B;
    a.T = T;
    a.D = D;
    a.seg_rows = p.seg_rows;
    a.strip_groups = p.strip_groups;
    a.seg_groups = p.seg_groups;
    a.ws = p.ws;
    a.lane_groups = p.lane_groups;
    a.strips = p.strips;
    return cconv::launch_fwd(p, W, a, hs) == hipSuccess ? CCONV_OK : CCONV_ERR_LAUNCH;
}

// Stages of the backward: kMain computes dx and the fp32 partials in the workspace, kFinish
// reduces the partials into dw and dbias. cconv_bwd runs both.
constexpr int kMain = 1, kFinish = 2;

cconv_status_t bwd_impl(int stages, const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb,
                        int64_t dy_st, const void* w, cconv_dtype_t w_dtype, const float* bias, void* dx, void* dw,
                        cconv_dtype_t dw_dtype, float* dbias, void* workspace, size_t workspace_bytes, int64_t B,
                        int64_t T, int64_t D, int W, const cconv_config_t* cfg, cconv_stream_t stream,
                        Extra ex = Extra{}) {
    const bool act_empty = (B == 0 || T == 0 || D == 0);
    const bool main = (stages & kMain) != 0, finish = (stages & kFinish) != 0;
    if (main && (((!x || !dy || !dx) && !act_empty) || (!w && D > 0))) return CCONV_ERR_NULL_POINTER;
    if (finish && !dw && D > 0) return CCONV_ERR_NULL_POINTER;
    if (!main) {  // the finishing stage reads only the workspace: treat the inputs as absent
        x = dy = w = nullptr;
        dx = nullptr;
        bias = nullptr;
        x_sb = dy_sb = 0;
        x_st = dy_st = D;
        w_dtype = CCONV_BF16;
    }
    if (!finish) {
        dw = nullptr;
        dbias = nullptr;
        dw_dtype = CCONV_BF16;
    }
    cconv_status_t st = check_train_common(w_dtype, B, T, D, W);
    if (st != CCONV_OK) return st;
    if (!dtype_ok(dw_dtype)) return CCONV_ERR_UNSUPPORTED_DTYPE;
    const int epi = ex.linear ? cconv::kLinear : 0;
    // packed batches and the variant without an activation are compiled for the streaming
    // hints only
    // the default plan's cache hints follow where the call's rows actually start (the plan's
    // segments, and so the partials a finishing stage reads, do not depend on them)
    const bool lines = on_lines(x, x_sb, x_st) && on_lines(dy, dy_sb, dy_st) &&
                       (ex.o_st && main ? on_lines(dx, ex.mode == kPacked ? 0 : ex.o_sb, ex.o_st) : on_lines(dx, T * D, D));
    const int lv = lane_width(D);
    const bool lanes = on_lanes(x, x_sb, x_st, lv) && on_lanes(dy, dy_sb, dy_st, lv) &&
                       (ex.o_st && main ? on_lanes(dx, ex.mode == kPacked ? 0 : ex.o_sb, ex.o_st, lv)
                                        : on_lanes(dx, T * D, D, lv));
    cconv_config_t c = cfg ? *cfg : default_config(true, B, T, D, W, ex.mode == kPacked || epi != 0, lines, lanes);
    // the 4- and 8-channel kernels address a row group as 32-bit scalar offsets from its first
    // row: row strides up to kMaxGroupStride; beyond that the default plan runs one channel per
    // lane with the same segments (so the same partials and workspace)
    const int64_t dx_row = ex.o_st && main ? ex.o_st : D;
    if (c.vec >= 4 && (x_st > cconv::kMaxGroupStride || dy_st > cconv::kMaxGroupStride ||
                       dx_row > cconv::kMaxGroupStride)) {
        if (cfg) return CCONV_ERR_BAD_STRIDE;
        c.vec = 1;
        c.options = cconv::kNarrowOptions;
    }
    if (!config_ok(c, true)) return CCONV_ERR_BAD_CONFIG;
    if (!width_ok(c, D)) return CCONV_ERR_BAD_CONFIG;
    const int gran = granule(c, D);
    if ((st = check_params(w, w_dtype, bias, gran)) != CCONV_OK) return st;
    if ((st = check_act(x, x_sb, x_st, D, gran)) != CCONV_OK) return st;
    if ((st = check_act(dy, dy_sb, dy_st, D, gran)) != CCONV_OK) return st;
    int64_t dx_sb = T * D, dx_st = D;  // contiguous unless the general entry point gives strides
    if (ex.o_st != 0 && main) {
        dx_st = ex.o_st;
        dx_sb = ex.mode == kPacked ? 0 : ex.o_sb;
        if ((st = check_out(dx, dx_sb, dx_st, B, T, D, gran)) != CCONV_OK) return st;
    } else if (!aligned(dx, static_cast<uintptr_t>(2 * gran))) {
        return CCONV_ERR_MISALIGNED;
    }
    if (!aligned(dw, gran == 8 ? 16 : static_cast<uintptr_t>(esize(dw_dtype))) || (dbias && !aligned(dbias, gran == 8 ? 16 : 4)))
        return CCONV_ERR_MISALIGNED;
    if (!cconv::bwd_launch_exists(c.vec, c.rows_per_group, c.options | epi, ex.mode == kPacked))
        return CCONV_ERR_BAD_CONFIG;
    Plan p;
    if (!make_plan(c, B, T, D, &p)) return CCONV_ERR_BAD_SHAPE;
    p.options |= epi;
    const size_t need = (B == 0 || T == 0 || D == 0) ? 0 : bwd_workspace(p, D, W);
    if (ex.scratch) {
        workspace = nullptr;  // resolved after every check has passed
        workspace_bytes = kScratchBytes;
    } else if (need > 0 && (!workspace || !aligned(workspace, 16))) {
        return workspace ? CCONV_ERR_MISALIGNED : CCONV_ERR_NULL_POINTER;
    }

    const Span in_x = span(x, extent3(B, T, D, x_sb, x_st, 2));
    const Span in_dy = span(dy, extent3(B, T, D, dy_sb, dy_st, 2));
    const Span in_w = span(w, static_cast<__int128>(D) * W * esize(w_dtype));
    const Span in_b = bias ? span(bias, static_cast<__int128>(D) * 4) : Span{0, 0};
    const Span o_dx = span(dx, extent3(B, T, D, dx_sb, dx_st, 2));
    const Span o_dw = span(dw, static_cast<__int128>(D) * W * esize(dw_dtype));
    const Span o_db = dbias ? span(dbias, static_cast<__int128>(D) * 4) : Span{0, 0};
    const Span o_ws = span(workspace, need);
    if (W == 1 || !main) ex.h0 = ex.out = nullptr;
    const Span outs[4] = {o_dx, o_dw, o_db, o_ws};
    const Span ins[4] = {in_x, in_dy, in_w, in_b};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j)
            if (overlap(outs[i], ins[j])) return CCONV_ERR_ALIASING;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return CCONV_ERR_ALIASING;
    }
    Span sh0;
    if ((st = check_extra(ex, B, D, W, false, ins, 4, outs, 4, &sh0, gran == 8 ? 16 : 2)) != CCONV_OK) return st;
    if (workspace_bytes < need) return CCONV_ERR_WORKSPACE;
    // a per-sequence history gradient needs at least one token
    if (ex.out && ex.mode != kPacked && T == 0 && B > 0 && D > 0) return CCONV_ERR_BAD_SHAPE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (ex.scratch && need > 0 && (st = scratch_ptr(&workspace)) != CCONV_OK) return st;
    if ((st = launch_checks(ex, B, T, D, W, false, s)) != CCONV_OK) return st;
    if (D == 0) return CCONV_OK;

    const bool empty = (B == 0 || T == 0);
    if (main && !empty) {
        cconv::BwdArgs a;
        a.x = static_cast<const uint16_t*>(x);
        a.x_sb = x_sb;
        a.x_st = x_st;
        a.dy = static_cast<const uint16_t*>(dy);
        a.dy_sb = dy_sb;
        a.dy_st = dy_st;
        a.w = w;
        a.w_f32 = (w_dtype == CCONV_F32);
        a.bias = bias;
        a.dx = static_cast<uint16_t*>(dx);
        a.dx_sb = dx_sb;
        a.dx_st = dx_st;
        a.partial = static_cast<float*>(workspace);
        a.h0 = static_cast<const uint16_t*>(ex.h0);
        a.dh0 = static_cast<uint16_t*>(ex.out);
        a.cu = ex.cu;
        a.nseq = ex.mode == kPacked ? ex.rows : 0;
        a.status = ex.status;
        a.B = B;
        a.T = T;
        a.D = D;
        a.seg_rows = p.seg_rows;
        a.strip_groups = p.strip_groups;
        a.seg_groups = p.seg_groups;
        a.ws = p.ws;
        a.lane_groups = p.lane_groups;
        a.strips = p.strips;
        if (cconv::launch_bwd(p, W, a, s) != hipSuccess) return CCONV_ERR_LAUNCH;
    }
    if (!finish) return CCONV_OK;
    cconv::ReduceArgs r;
    r.partial = static_cast<const float*>(workspace);
    r.P = empty ? 0 : p.partials;
    r.D = D;
    r.W = W;
    r.dw = dw;
    r.dw_f32 = (dw_dtype == CCONV_F32);
    r.dbias = dbias;
    r.status = ex.status;
    return cconv::launch_reduce(r, s) == hipSuccess ? CCONV_OK : CCONV_ERR_LAUNCH;
}

// The packed entry points: B = 1 and T = total rows, with the offsets, states and status word
// in the packed-mode descriptor.
cconv_status_t packed_extra(const int32_t* cu_seqlens, int64_t nseq, int64_t total, const void* h0, void* out,
                            int32_t* status, Extra* ex) {
    if (!status || !cu_seqlens) return CCONV_ERR_NULL_POINTER;
    if (nseq < 0 || nseq > kMaxSequences || total < 0 || total > INT32_MAX) return CCONV_ERR_BAD_SHAPE;
    ex->mode = kPacked;
    ex->h0 = h0;
    ex->out = out;
    ex->rows = nseq;
    ex->cu = cu_seqlens;
    ex->status = status;
    return CCONV_OK;
}

cconv_status_t fwd_varlen_impl(const void* x, int64_t x_st, const int32_t* cu_seqlens, int64_t nseq, int64_t total,
                               const void* w, cconv_dtype_t w_dtype, const float* bias, const void* init_state,
                               void* final_state, int32_t* status, void* y, int64_t D, int W,
                               const cconv_config_t* cfg, cconv_stream_t stream) {
    Extra ex;
    const cconv_status_t st = packed_extra(cu_seqlens, nseq, total, init_state, final_state, status, &ex);
    if (st != CCONV_OK) return st;
    return fwd_impl(x, 0, x_st, w, w_dtype, bias, y, 1, total, D, W, cfg, stream, ex);
}

cconv_status_t bwd_varlen_impl(const void* x, int64_t x_st, const void* dy, int64_t dy_st, const int32_t* cu_seqlens,
                               int64_t nseq, int64_t total, const void* w, cconv_dtype_t w_dtype, const float* bias,
                               const void* init_state, void* dx, void* dw, cconv_dtype_t dw_dtype, float* dbias,
                               void* d_init_state, void* workspace, size_t workspace_bytes, int32_t* status,
                               int64_t D, int W, const cconv_config_t* cfg, cconv_stream_t stream) {
    Extra ex;
    const cconv_status_t st = packed_extra(cu_seqlens, nseq, total, init_state, d_init_state, status, &ex);
    if (st != CCONV_OK) return st;
    return bwd_impl(kMain | kFinish, x, 0, x_st, dy, 0, dy_st, w, w_dtype, bias, dx, dw, dw_dtype, dbias, workspace,
                    workspace_bytes, 1, total, D, W, cfg, stream, ex);
}

// The decode update's launch rule: a thread per `vec` channels (8 when D % 8 == 0, 4 when
// D % 4 == 0, else 1); blocks of up to kUpdateThreads threads across a row's channel groups;
// rows per block chosen so that the grid holds about kUpdateTargetBlocks blocks (each block
// pays the O(N) slot check, so their number is kept near a constant).
cconv_update_config_t update_config_for(int64_t N, int64_t D, int vec) {
    cconv_update_config_t c;
    c.vec = vec;
    const int64_t dv = D / c.vec;
    c.block_threads = static_cast<int>(std::min<int64_t>(kUpdateThreads, std::max<int64_t>(64, ((dv + 63) / 64) * 64)));
    const int64_t grid_x = std::max<int64_t>(1, (dv + c.block_threads - 1) / c.block_threads);
    c.rows_per_block = std::max<int64_t>(1, (std::max<int64_t>(N, 1) * grid_x + kUpdateTargetBlocks - 1) / kUpdateTargetBlocks);
    c.rows_per_thread = 1;
    c.options = 0;
    if (c.vec > 1) {
        c.options = c.vec == 8 ? kUpdateOptions8 : kUpdateOptions;
        c.rows_per_thread = static_cast<int>(kUpdateRowsPerThread);
        c.rows_per_block = ((c.rows_per_block + c.rows_per_thread - 1) / c.rows_per_thread) * c.rows_per_thread;
        c.block_threads = std::min(c.block_threads, cconv::update_max_threads(c.rows_per_thread));
    }
    return c;
}

cconv_update_config_t default_update_config(int64_t N, int64_t D) {
    return update_config_for(N, D, (D % 8 == 0) ? kUpdateVec8 : (D % 4 == 0 ? 4 : 1));
}

// The decode update: state of L entries (L = W-1 or W), shift or (with cache_seqlens)
// circular addressing.
cconv_status_t update_impl(const void* x, int64_t x_ld, void* state, int64_t S, int L, const int32_t* state_indices,
                           const int32_t* cache_seqlens, const void* w, cconv_dtype_t w_dtype, const float* bias,
                           void* y, int64_t N, int64_t D, int W, int32_t* status, const cconv_update_config_t* cfg,
                           cconv_stream_t stream) {
    if (N < 0 || S < 0 || D < 0 || W < 1 || W > 4) return CCONV_ERR_BAD_SHAPE;
    if (L != W - 1 && L != W) return CCONV_ERR_BAD_SHAPE;
    if (cache_seqlens && L < 1) return CCONV_ERR_BAD_SHAPE;  // a circular state needs entries
    if (((!x || !y) && N > 0 && D > 0) || (!w && D > 0) || (!state && S > 0 && D > 0 && L > 0))
        return CCONV_ERR_NULL_POINTER;
    // what only the device can check is reported through the status word, so a call that has
    // such entries needs one
    if ((state_indices || cache_seqlens) && !status && N > 0) return CCONV_ERR_NULL_POINTER;
    if (N > kMaxDecodeRows || S > kMaxDim || D > kMaxDecodeChannels) return CCONV_ERR_BAD_SHAPE;
    if (state_indices && S > kMaxIndexedSlots) return CCONV_ERR_BAD_SHAPE;
    if (!state_indices && N > S) return CCONV_ERR_BAD_SHAPE;
    if (!dtype_ok(w_dtype)) return CCONV_ERR_UNSUPPORTED_DTYPE;
    // Rows: D a multiple of 8 needs a row stride that is one too and 16-byte aligned operands;
    // any other D takes compact rows (x_ld == D) or a stride that is a multiple of 8 [the
    // decode PR's row-stride contract], with element alignment.
    const bool wide = (D % 8 == 0);
    if (x_ld < D || x_ld > kMaxDim || (x_ld % 8 != 0 && !(!wide && x_ld == D))) return CCONV_ERR_BAD_STRIDE;
    const uintptr_t va = wide ? 16 : 2;
    if (!aligned(x, va) || !aligned(state, va) || !aligned(w, wide ? 16 : static_cast<uintptr_t>(esize(w_dtype))) ||
        !aligned(y, va) || (bias && !aligned(bias, wide ? 16 : 4)) || (state_indices && !aligned(state_indices, 4)) ||
        (cache_seqlens && !aligned(cache_seqlens, 4)) || (status && !aligned(status, 4)))
        return CCONV_ERR_MISALIGNED;
    // 4 channels per thread: 8-byte rows and state runs, taps and bias in 8/16-byte chunks
    const bool quad_ok = D % 4 == 0 && x_ld % 4 == 0 && aligned(x, 8) && aligned(y, 8) && aligned(state, 8) &&
                         aligned(w, w_dtype == CCONV_F32 ? 16 : 8) && (!bias || aligned(bias, 16));
    const Span in_x = span(x, N == 0 || D == 0 ? 0 : (static_cast<__int128>(N - 1) * x_ld + D) * 2);
    const Span in_w = span(w, static_cast<__int128>(D) * W * esize(w_dtype));
    const Span in_b = bias ? span(bias, static_cast<__int128>(D) * 4) : Span{0, 0};
    const Span in_i = state_indices ? span(state_indices, static_cast<__int128>(N) * 4) : Span{0, 0};
    const Span in_c = cache_seqlens ? span(cache_seqlens, static_cast<__int128>(N) * 4) : Span{0, 0};
    const Span o_st = span(state, static_cast<__int128>(S) * D * L * 2);
    const Span o_y = span(y, static_cast<__int128>(N) * D * 2);
    const Span o_s = status ? span(status, 4) : Span{0, 0};
    const Span outs[3] = {o_st, o_y, o_s};
    const Span ins[5] = {in_x, in_w, in_b, in_i, in_c};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlap(outs[i], ins[j])) return CCONV_ERR_ALIASING;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return CCONV_ERR_ALIASING;
    }
    cconv_update_config_t c;
    if (cfg) {
        c = *cfg;
        if (c.vec == 4 && D % 4 == 0 && x_ld % 4 == 0 && !quad_ok) return CCONV_ERR_MISALIGNED;
    } else {
        c = default_update_config(N, D);
        if (c.vec == 4 && !quad_ok) c = update_config_for(N, D, 1);  // operands off the 4-channel rule
    }
    if (c.block_threads < 64 || c.block_threads > 1024 || c.block_threads % 64 != 0 || c.rows_per_block < 1 ||
        c.rows_per_block > kMaxDecodeRows || c.options < 0 || c.options > 5 ||
        ((c.options & cconv::kUpdStaged) && (c.vec != 8 || (c.options & cconv::kUpdNtLoad))) ||
        (c.rows_per_thread != 1 && c.rows_per_thread != 2) || c.block_threads > cconv::update_max_threads(c.rows_per_thread) ||
        (c.vec != 1 && c.vec != 4 && c.vec != 8) || D % c.vec != 0 || (c.vec == 4 && x_ld % 4 != 0) ||
        (c.vec == 1 && (c.options != 0 || c.rows_per_thread != 1)))
        return CCONV_ERR_BAD_CONFIG;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (N == 0 || D == 0) {
        if (status) return cconv::launch_status(status, CCONV_OK, s) == hipSuccess ? CCONV_OK : CCONV_ERR_LAUNCH;
        return CCONV_OK;
    }
    const int64_t dv = D / c.vec;  // channel groups per row (one thread each)
    const int64_t grid_x = (dv + c.block_threads - 1) / c.block_threads;
    const int64_t grid_y = (N + c.rows_per_block - 1) / c.rows_per_block;
    if (grid_x > INT32_MAX || grid_y > 65535) return CCONV_ERR_BAD_CONFIG;
    // the slot check's bit set and verdict word (a verdict word alone for cache_seqlens only),
    // then, when staged, one region of 64 * L 16-byte chunks per wave
    const int64_t words = state_indices ? (S + 31) / 32 + 1 : (cache_seqlens ? 1 : 0);
    size_t lds = static_cast<size_t>(words) * 4;
    if ((c.options & cconv::kUpdStaged) && L > 0) {
        const size_t staged = static_cast<size_t>((words + 3) & ~int64_t(3)) * 4 +
                              static_cast<size_t>(c.block_threads / cconv::kWave) * cconv::kWave * 16 * L;
        if (staged <= kMaxUpdateLds)
            lds = staged;
        else if (cfg)
            return CCONV_ERR_BAD_CONFIG;
        else
            c.options &= ~cconv::kUpdStaged;  // the default plan without the staging
    }
    cconv::UpdateArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.x_ld = x_ld;
    a.state = static_cast<uint16_t*>(state);
    a.S = S;
    a.idx = state_indices;
    a.cs = cache_seqlens;
    a.w = w;
    a.w_f32 = (w_dtype == CCONV_F32);
    a.bias = bias;
    a.y = static_cast<uint16_t*>(y);
    a.N = N;
    a.D = D;
    a.rows_per_block = c.rows_per_block;
    a.status = status;
    return cconv::launch_update(W, L, c.vec, c.options, c.rows_per_thread, a, c.block_threads, grid_x, grid_y, lds, s) ==
                   hipSuccess
               ? CCONV_OK
               : CCONV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

cconv_status_t cconv_fwd(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                         const float* bias, void* y, int64_t B, int64_t T, int64_t D, int W,
                         cconv_stream_t stream) {
    return fwd_impl(x, x_sb, x_st, w, w_dtype, bias, y, B, T, D, W, nullptr, stream);
}

cconv_status_t cconv_fwd_state(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                               const float* bias, const void* init_state, void* final_state, void* y, int64_t B,
                               int64_t T, int64_t D, int W, cconv_stream_t stream) {
    Extra ex;
    ex.h0 = init_state;
    ex.out = final_state;
    return fwd_impl(x, x_sb, x_st, w, w_dtype, bias, y, B, T, D, W, nullptr, stream, ex);
}

cconv_status_t cconv_fwd_pool(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                              const float* bias, void* state, int64_t S, const int32_t* state_indices,
                              const uint8_t* has_initial_state, int32_t* status, void* y, int64_t B, int64_t T,
                              int64_t D, int W, cconv_stream_t stream) {
    if (!status || (!state_indices && B > 0)) return CCONV_ERR_NULL_POINTER;
    if (W >= 2 && W <= 4 && !state && S > 0 && D > 0) return CCONV_ERR_NULL_POINTER;
    if (S < 0 || S > kMaxIndexedSlots || B > kMaxDecodeRows) return CCONV_ERR_BAD_SHAPE;
    Extra ex;
    ex.mode = kPool;
    ex.h0 = has_initial_state ? state : nullptr;
    ex.out = state;
    ex.rows = S;
    ex.sidx = state_indices;
    ex.has_init = has_initial_state;
    ex.status = status;
    return fwd_impl(x, x_sb, x_st, w, w_dtype, bias, y, B, T, D, W, nullptr, stream, ex);
}

cconv_status_t cconv_bwd_state(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb,
                               int64_t dy_st, const void* w, cconv_dtype_t w_dtype, const float* bias,
                               const void* init_state, void* dx, void* dw, cconv_dtype_t dw_dtype, float* dbias,
                               void* d_init_state, void* workspace, size_t workspace_bytes, int64_t B, int64_t T,
                               int64_t D, int W, cconv_stream_t stream) {
    Extra ex;
    ex.h0 = init_state;
    ex.out = d_init_state;
    return bwd_impl(kMain | kFinish, x, x_sb, x_st, dy, dy_sb, dy_st, w, w_dtype, bias, dx, dw, dw_dtype, dbias,
                    workspace, workspace_bytes, B, T, D, W, nullptr, stream, ex);
}

cconv_status_t cconv_fwd_ex(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                            const float* bias, void* y, int64_t B, int64_t T, int64_t D, int W,
                            const cconv_fwd_opts_t* o, cconv_stream_t stream) {
    Extra ex;
    if (o) {
        if (o->activation != CCONV_ACT_SILU && o->activation != CCONV_ACT_NONE) return CCONV_ERR_BAD_CONFIG;
        ex.linear = (o->activation == CCONV_ACT_NONE);
        ex.r = o->residual;
        ex.r_sb = o->residual_sb;
        ex.r_st = o->residual_st;
        ex.o_sb = o->y_sb;
        ex.o_st = o->y_st;
        if (o->cu_seqlens) {
            if (B != 1) return CCONV_ERR_BAD_SHAPE;
            const cconv_status_t st =
                packed_extra(o->cu_seqlens, o->nseq, T, o->init_state, o->final_state, o->status, &ex);
            if (st != CCONV_OK) return st;
            x_sb = 0;
            ex.r_sb = 0;
        } else {
            ex.h0 = o->init_state;
            ex.out = o->final_state;
        }
    }
    return fwd_impl(x, x_sb, x_st, w, w_dtype, bias, y, B, T, D, W, nullptr, stream, ex);
}

cconv_status_t cconv_bwd_ex(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb, int64_t dy_st,
                            const void* w, cconv_dtype_t w_dtype, const float* bias, void* dx, void* dw,
                            cconv_dtype_t dw_dtype, float* dbias, void* workspace, size_t workspace_bytes, int64_t B,
                            int64_t T, int64_t D, int W, const cconv_bwd_opts_t* o, cconv_stream_t stream) {
    Extra ex;
    if (o) {
        if (o->activation != CCONV_ACT_SILU && o->activation != CCONV_ACT_NONE) return CCONV_ERR_BAD_CONFIG;
        ex.linear = (o->activation == CCONV_ACT_NONE);
        ex.o_sb = o->dx_sb;
        ex.o_st = o->dx_st;
        if (o->cu_seqlens) {
            if (B != 1) return CCONV_ERR_BAD_SHAPE;
            const cconv_status_t st =
                packed_extra(o->cu_seqlens, o->nseq, T, o->init_state, o->d_init_state, o->status, &ex);
            if (st != CCONV_OK) return st;
            x_sb = dy_sb = 0;
        } else {
            ex.h0 = o->init_state;
            ex.out = o->d_init_state;
        }
    }
    return bwd_impl(kMain | kFinish, x, x_sb, x_st, dy, dy_sb, dy_st, w, w_dtype, bias, dx, dw, dw_dtype, dbias,
                    workspace, workspace_bytes, B, T, D, W, nullptr, stream, ex);
}

cconv_status_t cconv_fwd_varlen(const void* x, int64_t x_st, const int32_t* cu_seqlens, int64_t nseq, int64_t total,
                                const void* w, cconv_dtype_t w_dtype, const float* bias, const void* init_state,
                                void* final_state, int32_t* status, void* y, int64_t D, int W,
                                cconv_stream_t stream) {
    return fwd_varlen_impl(x, x_st, cu_seqlens, nseq, total, w, w_dtype, bias, init_state, final_state, status, y, D,
                           W, nullptr, stream);
}

cconv_status_t cconv_fwd_varlen_config(const void* x, int64_t x_st, const int32_t* cu_seqlens, int64_t nseq,
                                       int64_t total, const void* w, cconv_dtype_t w_dtype, const float* bias,
                                       const void* init_state, void* final_state, int32_t* status, void* y,
                                       int64_t D, int W, const cconv_config_t* config, cconv_stream_t stream) {
    if (!config) return CCONV_ERR_NULL_POINTER;
    return fwd_varlen_impl(x, x_st, cu_seqlens, nseq, total, w, w_dtype, bias, init_state, final_state, status, y, D,
                           W, config, stream);
}

cconv_status_t cconv_bwd_varlen(const void* x, int64_t x_st, const void* dy, int64_t dy_st, const int32_t* cu_seqlens,
                                int64_t nseq, int64_t total, const void* w, cconv_dtype_t w_dtype, const float* bias,
                                const void* init_state, void* dx, void* dw, cconv_dtype_t dw_dtype, float* dbias,
                                void* d_init_state, void* workspace, size_t workspace_bytes, int32_t* status,
                                int64_t D, int W, cconv_stream_t stream) {
    return bwd_varlen_impl(x, x_st, dy, dy_st, cu_seqlens, nseq, total, w, w_dtype, bias, init_state, dx, dw, dw_dtype,
                           dbias, d_init_state, workspace, workspace_bytes, status, D, W, nullptr, stream);
}

cconv_status_t cconv_bwd_varlen_config(const void* x, int64_t x_st, const void* dy, int64_t dy_st,
                                       const int32_t* cu_seqlens, int64_t nseq, int64_t total, const void* w,
                                       cconv_dtype_t w_dtype, const float* bias, const void* init_state, void* dx,
                                       void* dw, cconv_dtype_t dw_dtype, float* dbias, void* d_init_state,
                                       void* workspace, size_t workspace_bytes, int32_t* status, int64_t D, int W,
                                       const cconv_config_t* config, cconv_stream_t stream) {
    if (!config) return CCONV_ERR_NULL_POINTER;
    return bwd_varlen_impl(x, x_st, dy, dy_st, cu_seqlens, nseq, total, w, w_dtype, bias, init_state, dx, dw, dw_dtype,
                           dbias, d_init_state, workspace, workspace_bytes, status, D, W, config, stream);
}

cconv_status_t cconv_fwd_config(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                                const float* bias, void* y, int64_t B, int64_t T, int64_t D, int W,
                                const cconv_config_t* cfg, cconv_stream_t stream) {
    if (!cfg) return CCONV_ERR_NULL_POINTER;
    return fwd_impl(x, x_sb, x_st, w, w_dtype, bias, y, B, T, D, W, cfg, stream);
}

size_t cconv_bwd_workspace_bytes_config(int64_t B, int64_t T, int64_t D, int W, const cconv_config_t* cfg) {
    if (B <= 0 || T <= 0 || D <= 0 || W < 1 || W > 4 || B > kMaxDim || T > kMaxDim || D > kMaxDim) return 0;
    const cconv_config_t c = cfg ? *cfg : default_config(true, B, T, D, W);
    if (!config_ok(c, true)) return 0;
    Plan p;
    if (!make_plan(c, B, T, D, &p)) return 0;
    return bwd_workspace(p, D, W);
}

size_t cconv_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int W) {
    return cconv_bwd_workspace_bytes_config(B, T, D, W, nullptr);
}

cconv_status_t cconv_bwd(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb, int64_t dy_st,
                         const void* w, cconv_dtype_t w_dtype, const float* bias, void* dx, void* dw,
                         cconv_dtype_t dw_dtype, float* dbias, void* workspace, size_t workspace_bytes, int64_t B,
                         int64_t T, int64_t D, int W, cconv_stream_t stream) {
    return bwd_impl(kMain | kFinish, x, x_sb, x_st, dy, dy_sb, dy_st, w, w_dtype, bias, dx, dw, dw_dtype, dbias,
                    workspace, workspace_bytes, B, T, D, W, nullptr, stream);
}

cconv_status_t cconv_bwd_noalloc(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb,
                                 int64_t dy_st, const void* w, cconv_dtype_t w_dtype, const float* bias, void* dx,
                                 void* dw, cconv_dtype_t dw_dtype, float* dbias, int64_t B, int64_t T, int64_t D,
                                 int W, cconv_stream_t stream) {
    Extra ex;
    ex.scratch = true;
    return bwd_impl(kMain | kFinish, x, x_sb, x_st, dy, dy_sb, dy_st, w, w_dtype, bias, dx, dw, dw_dtype, dbias,
                    nullptr, 0, B, T, D, W, nullptr, stream, ex);
}

size_t cconv_bwd_noalloc_max_workspace(void) { return kScratchBytes; }

cconv_status_t cconv_bwd_main(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb,
                              int64_t dy_st, const void* w, cconv_dtype_t w_dtype, const float* bias, void* dx,
                              void* workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t D, int W,
                              cconv_stream_t stream) {
    return bwd_impl(kMain, x, x_sb, x_st, dy, dy_sb, dy_st, w, w_dtype, bias, dx, nullptr, CCONV_BF16, nullptr,
                    workspace, workspace_bytes, B, T, D, W, nullptr, stream);
}

cconv_status_t cconv_bwd_finish(const void* workspace, size_t workspace_bytes, void* dw, cconv_dtype_t dw_dtype,
                                float* dbias, int64_t B, int64_t T, int64_t D, int W, cconv_stream_t stream) {
    return bwd_impl(kFinish, nullptr, 0, D, nullptr, 0, D, nullptr, CCONV_BF16, nullptr, nullptr, dw, dw_dtype,
                    dbias, const_cast<void*>(workspace), workspace_bytes, B, T, D, W, nullptr, stream);
}

cconv_status_t cconv_bwd_config(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb,
                                int64_t dy_st, const void* w, cconv_dtype_t w_dtype, const float* bias, void* dx,
                                void* dw, cconv_dtype_t dw_dtype, float* dbias, void* workspace,
                                size_t workspace_bytes, int64_t B, int64_t T, int64_t D, int W,
                                const cconv_config_t* cfg, cconv_stream_t stream) {
    if (!cfg) return CCONV_ERR_NULL_POINTER;
    return bwd_impl(kMain | kFinish, x, x_sb, x_st, dy, dy_sb, dy_st, w, w_dtype, bias, dx, dw, dw_dtype, dbias,
                    workspace, workspace_bytes, B, T, D, W, cfg, stream);
}

cconv_status_t cconv_default_config(int which, int64_t B, int64_t T, int64_t D, int W, cconv_config_t* out) {
    if (!out) return CCONV_ERR_NULL_POINTER;
    if (which != 0 && which != 1) return CCONV_ERR_BAD_CONFIG;
    if (B < 0 || T < 0 || D < 0 || W < 1 || W > 4) return CCONV_ERR_BAD_SHAPE;
    *out = default_config(which == 1, B, T, D, W);
    return CCONV_OK;
}

cconv_status_t cconv_update(const void* x, int64_t x_ld, void* state, int64_t S, const int32_t* state_indices,
                            const void* w, cconv_dtype_t w_dtype, const float* bias, void* y, int64_t N, int64_t D,
                            int W, int32_t* status, cconv_stream_t stream) {
    return update_impl(x, x_ld, state, S, W - 1, state_indices, nullptr, w, w_dtype, bias, y, N, D, W, status, nullptr,
                       stream);
}

cconv_status_t cconv_update_ex(const void* x, int64_t x_ld, void* state, int64_t S, int L,
                               const int32_t* state_indices, const int32_t* cache_seqlens, const void* w,
                               cconv_dtype_t w_dtype, const float* bias, void* y, int64_t N, int64_t D, int W,
                               int32_t* status, cconv_stream_t stream) {
    return update_impl(x, x_ld, state, S, L, state_indices, cache_seqlens, w, w_dtype, bias, y, N, D, W, status,
                       nullptr, stream);
}

cconv_status_t cconv_update_config(const void* x, int64_t x_ld, void* state, int64_t S, int L,
                                   const int32_t* state_indices, const int32_t* cache_seqlens, const void* w,
                                   cconv_dtype_t w_dtype, const float* bias, void* y, int64_t N, int64_t D, int W,
                                   int32_t* status, const cconv_update_config_t* cfg, cconv_stream_t stream) {
    if (!cfg) return CCONV_ERR_NULL_POINTER;
    return update_impl(x, x_ld, state, S, L, state_indices, cache_seqlens, w, w_dtype, bias, y, N, D, W, status, cfg,
                       stream);
}

cconv_status_t cconv_default_update_config(int64_t N, int64_t D, cconv_update_config_t* out) {
    if (!out) return CCONV_ERR_NULL_POINTER;
    if (N < 0 || D < 0 || N > kMaxDecodeRows || D > kMaxDecodeChannels) return CCONV_ERR_BAD_SHAPE;
    *out = default_update_config(N, D);
    return CCONV_OK;
}

const char* cconv_status_string(cconv_status_t status) {
    switch (status) {
        case CCONV_OK: return "ok";
        case CCONV_ERR_NULL_POINTER: return "a required pointer is NULL";
        case CCONV_ERR_BAD_SHAPE: return "unsupported shape (negative size, W outside [1,4], D not a multiple of 8, or above a limit)";
        case CCONV_ERR_BAD_STRIDE: return "unsupported stride (negative, row stride below D, or not a multiple of 8)";
        case CCONV_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype (weights and dw must be bf16 or fp32)";
        case CCONV_ERR_MISALIGNED: return "misaligned pointer (tensors need 16 bytes, indices and status 4)";
        case CCONV_ERR_ALIASING: return "an output overlaps an input or another output";
        case CCONV_ERR_WORKSPACE: return "workspace smaller than cconv_bwd_workspace_bytes()";
        case CCONV_ERR_INDEX: return "state_indices out of [-1, S) or repeated, or cu_seqlens not a valid partition";
        case CCONV_ERR_LAUNCH: return "kernel launch failed";
        case CCONV_ERR_BAD_CONFIG: return "invalid launch configuration";
    }
    return "unknown status";
}

const char* cconv_version(void) { return "cconv 0.1.0 for gfx950, built with " __VERSION__; }

}  // extern "C"
