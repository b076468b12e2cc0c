/*
 * cconv.h -- C ABI of libcconv.so: the depthwise causal short convolution (width W <= 4,
 * one set of taps per channel, optional bias) fused with SiLU, on AMD Instinct MI355X
 * (gfx950).
 *
 * The operation. For activations x[B, T, D] (channel dimension contiguous) and taps w[D, W]:
 *
 *     z[b, t, d] = bias[d] + sum_{j=0}^{W-1} w[d, j] * x[b, t-(W-1)+j, d]    (x = 0 for t < 0)
 *     y[b, t, d] = z * sigmoid(z)
 *
 * i.e. the tap that multiplies x[t-k] is w[:, W-1-k] [kernel-fun 0.2.0.dev1 wheel, page 2,
 * strip.py: `_tap`], the history before the sequence start is zero [strip.py: `_ld_ring`],
 * and SiLU is fused [kernel-fun wheel, cconv/__init__.py docstring; strip.py: `_silu`]. The
 * backward returns dx, dw and dbias through SiLU's derivative without re-running the
 * forward [strip.py: module docstring and `_bwd4`; `_dsilu`]. The decode update advances a
 * per-sequence state of the last W-1 inputs by one token [cudnn-frontend PR #797 "Add
 * experimental causal conv1d decode update", PR description: API and semantics].
 *
 * Conventions shared by every entry point:
 *  - Every pointer is caller-owned device memory. It may be NULL where stated, and any
 *    pointer may be NULL when the tensor it points to is empty (torch hands out NULL data
 *    pointers for empty tensors). The library
 *    allocates nothing, keeps no pointer beyond the call and owns no output (outputs are
 *    never cached; compare the kernel-fun wheel's _common/cache.py docstring on outputs).
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL is the null stream):
 *    no host synchronisation, no device-to-host read. Calls are reentrant and may be
 *    captured into a HIP graph from the first call.
 *  - bf16 tensors are passed as raw 16-bit patterns; fp32 as IEEE binary32. Outputs in
 *    bf16 are rounded to nearest-even [strip.py: `_st`].
 *  - Alignment and D. When D is a multiple of 8 (the vector path: each lane moves whole 16- or
 *    8-byte groups of channels), every tensor pointer must be 16-byte aligned, except
 *    state_indices, cache_seqlens, cu_seqlens and status (4 bytes) [PR #797 review thread:
 *    alignment contract], and every row and batch stride a multiple of 8 elements. The
 *    training calls (forward and backward, every variant) also run 4 channels per lane when
 *    D = 4 (mod 8), their default then: the bf16 activations (x, dy, y, dx, residual) 8-byte
 *    aligned with strides that are multiples of 4, the taps, bias, dw, dbias and states with
 *    element alignment (they are read and written per element). When D = 2 (mod 4) they run
 *    4 channels per lane by default from D = 6 on (8-byte accesses need only 4-byte alignment;
 *    the last lane group starts at channel D - 4 and overlaps the one before by two channels,
 *    which both write with the same bits) and 2 channels per lane at D = 2, the activations
 *    then 4-byte aligned with even strides. The backward's 4- and 8-channel plans address a
 *    group of rows as 32-bit offsets from its first row, so they take row strides (x_st,
 *    dy_st and dx's) of at most 2^26 elements: beyond that the default backward plan runs one
 *    channel per lane (the same segments and workspace) and an explicit vec >= 4
 *    configuration returns CCONV_ERR_BAD_STRIDE.
 *    Any other D (the element-granular path [strip.py's masked loads handle any D]: one
 *    channel per lane) needs only element alignment (2 bytes for bf16, 4 for fp32) and
 *    strides >= D; an explicit configuration with vec = 1 takes that path for any D. When
 *    D = 4 (mod 8) or D = 2 (mod 4) and the activations miss the rule of that lane width,
 *    the default plan runs one channel per lane too, with the segments (so the dw/dbias
 *    partials and the workspace) of the wider plan; an explicit vec = 4 or vec = 2
 *    configuration is checked against its rule (vec = 4 with D = 2 (mod 4): 4-byte aligned,
 *    even strides). The decode update runs 8
 *    channels per lane when D is a multiple of 8 and one otherwise, taking compact rows
 *    (x_ld == D) or a row stride that is a multiple of 8 [the decode PR's row-stride
 *    contract]. The element-granular paths (1 or 2 channels per lane) run with plain loads
 *    and stores only (options 0; 16-row groups, one-wave blocks by default); a
 *    configuration whose vec does not divide D is CCONV_ERR_BAD_CONFIG, except vec = 4 with
 *    D = 2 (mod 4) and D >= 6. The alignments
 *    stated below are those of the vector path with D a multiple of 8.
 *  - Errors fail closed. A problem visible on the host returns its code before anything is
 *    enqueued, leaving every output untouched: NULL required pointer, negative size, W
 *    outside [1, 4] (the pages' kernels are written for at most 4 taps, strip.py module
 *    docstring), bad stride, unsupported dtype, misalignment, an output overlapping another
 *    operand, a workspace that is too small. A failed launch returns CCONV_ERR_LAUNCH.
 *  - An empty problem (B*T*D == 0, N*D == 0) is CCONV_OK; the backward still writes its
 *    zero dw/dbias when D > 0, and the decode update still writes *status when given.
 *  - Performance: at a fixed D the time depends on the pitch of the rows (x_st, dy_st and
 *    the output strides of the general entry points) by up to 25% on MI355X, with no simple
 *    rule: D = 4096 contiguous and D = 6144 in rows of 8192 stream at 94-95% of a flat copy,
 *    D = 4096 in rows of 8192 and D = 6144 contiguous at ~78%. Only the D channels of a row
 *    are read or written, so a padded pitch costs memory, not bandwidth.
 */
#ifndef CCONV_H
#define CCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
/* A hipStream_t. NULL means the null stream. */
typedef struct ihipStream_t* cconv_stream_t;

typedef enum { CCONV_BF16 = 0, CCONV_F32 = 1 } cconv_dtype_t;

typedef enum {
    CCONV_OK = 0,
    CCONV_ERR_NULL_POINTER = 1,
    CCONV_ERR_BAD_SHAPE = 2,
    CCONV_ERR_BAD_STRIDE = 3,
    CCONV_ERR_UNSUPPORTED_DTYPE = 4,
    CCONV_ERR_MISALIGNED = 5,
    CCONV_ERR_ALIASING = 6,
    CCONV_ERR_WORKSPACE = 7,
    CCONV_ERR_INDEX = 8, /* device-side: bad state_indices, or cu_seqlens that are not a partition */
    CCONV_ERR_LAUNCH = 9,
    CCONV_ERR_BAD_CONFIG = 10
} cconv_status_t;

/*
 * Forward [strip.py: `cconv_fwd`, `cconv_fwd_strip`; bias as in fla's parameter list,
 * kernel-fun wheel _common/compat.py FLA_KWARGS].
 *   x     bf16 [B, T, D]: element (b, t, d) at x[b*x_sb + t*x_st + d]; x_st >= D.
 *   w     [D, W] contiguous, dtype w_dtype (CCONV_BF16 or CCONV_F32).
 *   bias  fp32 [D], or NULL for none.
 *   y     bf16 [B, T, D] contiguous (written; must not overlap x, w or bias).
 *   B, T >= 0; 0 <= D <= 2^30; 1 <= W <= 4.
 * Channels are independent, so the q, k and v convolutions of a fused projection
 * [B, T, Dq + Dk + Dv] are one call over all its channels with the three taps and biases
 * concatenated; y (and, in cconv_bwd, dx) is bit for bit that of three calls on the channel
 * slices with row stride Dq + Dk + Dv [kernel-fun wheel, cconv/__init__.py docstring: a KDA
 * layer convolves q, k and v separately, v twice as wide].
 */
cconv_status_t cconv_fwd(const void* x, int64_t x_sb, int64_t x_st, const void* w,
                         cconv_dtype_t w_dtype, const float* bias, void* y, int64_t B,
                         int64_t T, int64_t D, int W, cconv_stream_t stream);

/* Bytes of device workspace cconv_bwd needs for this problem (fp32 dw/dbias partials). */
size_t cconv_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int W);

/*
 * Backward [strip.py: `cconv_bwd`, `cconv_bwd_strip`, `_bwd4`, `_dsilu`]. With
 * g = dy * s * (1 + z*(1-s)), s = sigmoid(z) recomputed from x:
 *   dx[b, u, d] = sum_j w[d, j] * g[b, u+(W-1)-j, d]            (g = 0 at or past T)
 *   dw[d, j]    = sum_{b,t} g[b, t, d] * x[b, t-(W-1)+j, d]      (x = 0 before t = 0)
 *   dbias[d]    = sum_{b,t} g[b, t, d]
 *   x, dy    bf16 [B, T, D] with strides (x_sb, x_st, 1) and (dy_sb, dy_st, 1).
 *   w, bias  as in cconv_fwd (bias only enters z; NULL = no bias).
 *   dx       bf16 [B, T, D] contiguous, written.
 *   dw       [D, W] in dw_dtype (CCONV_BF16 or CCONV_F32), overwritten (not accumulated).
 *   dbias    fp32 [D], overwritten, or NULL when not wanted.
 *   workspace, workspace_bytes: caller-provided device scratch of at least
 *            cconv_bwd_workspace_bytes(B, T, D, W) bytes (may be NULL when that is 0).
 * dw and dbias are summed in a fixed order with no atomics, so they are bitwise
 * reproducible run to run [strip.py: host `cconv_bwd`, comment on the reduction].
 */
cconv_status_t cconv_bwd(const void* x, int64_t x_sb, int64_t x_st, const void* dy,
                         int64_t dy_sb, int64_t dy_st, const void* w, cconv_dtype_t w_dtype,
                         const float* bias, void* dx, void* dw, cconv_dtype_t dw_dtype,
                         float* dbias, void* workspace, size_t workspace_bytes, int64_t B,
                         int64_t T, int64_t D, int W, cconv_stream_t stream);

/*
 * cconv_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the dw/dbias partials go to a
 * static scratch array inside the library instead of a caller workspace. Arguments,
 * results and errors as cconv_bwd, with no workspace: dx, dw and dbias are bit for bit those
 * of cconv_bwd. The call allocates nothing and calls no allocating routine.
 *   Limit: cconv_bwd_workspace_bytes(B, T, D, W) <= cconv_bwd_noalloc_max_workspace()
 *   (16 MiB; the B8 T8192 D4096 W4 backward needs 10.5 MB); larger problems return
 *   CCONV_ERR_WORKSPACE before anything is enqueued.
 *   Each GPU holds its own copy of the array from the first call on it until the process
 *   ends; that first call looks up the copy's device address (a host-side runtime query,
 *   made with the calling thread's current device). Every call on one GPU uses the same
 *   array, so calls that overlap on one GPU (on different streams, or from several threads
 *   without ordering) race and give wrong dw/dbias; calls ordered on one stream are safe.
 */
cconv_status_t cconv_bwd_noalloc(const void* x, int64_t x_sb, int64_t x_st, const void* dy,
                                 int64_t dy_sb, int64_t dy_st, const void* w, cconv_dtype_t w_dtype,
                                 const float* bias, void* dx, void* dw, cconv_dtype_t dw_dtype,
                                 float* dbias, int64_t B, int64_t T, int64_t D, int W,
                                 cconv_stream_t stream);

/* Bytes of the static scratch cconv_bwd_noalloc uses: its largest workspace. */
size_t cconv_bwd_noalloc_max_workspace(void);

/*
 * Forward and backward with a history before t = 0: the prefill <-> decode state handoff
 * (fla's initial_state and output_final_state parameters, in the kernel-fun wheel's
 * _common/compat.py FLA_KWARGS table; the decode PR's description names a direct
 * full-sequence-to-decode state handoff as the next step). States use the decode layout:
 * bf16 [B, D, W-1] contiguous, oldest first, 16-byte aligned; for W == 1 they hold nothing
 * and are ignored.
 *   init_state   history of each sequence before t = 0 (NULL = zeros, i.e. cconv_fwd/bwd).
 *   final_state  out: the last W-1 values of the extended sequence (history, then x) -- the
 *                state a cconv_update continues from. May be init_state's own buffer (an
 *                in-place advance); must not overlap anything else. Needs T >= 1.
 *   d_init_state out (backward): the gradient of each history value (dx at the W-1 rows before
 *                t = 0), bf16; NULL when not wanted. Needs T >= 1.
 * The backward's dw includes the history's products; dx is unchanged in meaning.
 */
cconv_status_t cconv_fwd_state(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                               const float* bias, const void* init_state, void* final_state, void* y, int64_t B,
                               int64_t T, int64_t D, int W, cconv_stream_t stream);

cconv_status_t cconv_bwd_state(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb,
                               int64_t dy_st, const void* w, cconv_dtype_t w_dtype, const float* bias,
                               const void* init_state, void* dx, void* dw, cconv_dtype_t dw_dtype, float* dbias,
                               void* d_init_state, void* workspace, size_t workspace_bytes, int64_t B, int64_t T,
                               int64_t D, int W, cconv_stream_t stream);

/*
 * Prefill straight into the decode state pool: the forward of B sequences whose histories
 * and final states live in slots of the pool cconv_update advances (the follow-up scope in
 * the decode PR's discussion: a direct full-sequence-to-decode state handoff).
 *   state              bf16 [S, D, W-1] pool, the cconv_update layout (16-byte aligned); read
 *                      and written in place. May be NULL when it holds no element.
 *   state_indices      int32 [B] on the device: sequence b uses slot state_indices[b]; -1 marks
 *                      a padding sequence (zero history, y computed, no slot written). The
 *                      decode slot rule applies: every index in [-1, S), no slot named twice.
 *   has_initial_state  uint8 [B] on the device or NULL (= all zero): sequence b starts from the
 *                      history in its slot when nonzero, from zeros otherwise.
 *   status             int32 on the device, required: receives CCONV_OK, or CCONV_ERR_INDEX
 *                      when the slot rule fails -- then nothing else is written (neither y nor
 *                      any slot). Written by every call that returns CCONV_OK.
 * After the call, slot state_indices[b] holds the last W-1 values of history-then-x of
 * sequence b (as cconv_fwd_state's final state). x, w, bias, y as in cconv_fwd. Limits:
 * S <= 2^19, B <= 2^24; T >= 1 when B > 0 and W > 1. W == 1: no state; the slot rule is still
 * checked.
 */
cconv_status_t cconv_fwd_pool(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                              const float* bias, void* state, int64_t S, const int32_t* state_indices,
                              const uint8_t* has_initial_state, int32_t* status, void* y, int64_t B, int64_t T,
                              int64_t D, int W, cconv_stream_t stream);

/*
 * Packed variable-length batches (fla's cu_seqlens parameter: kernel-fun wheel,
 * _common/compat.py, FLA_KWARGS row for causal_conv1d). Sequences of different lengths are
 * packed along time into one [total, D] tensor; sequence i is rows cu_seqlens[i] ..
 * cu_seqlens[i+1]-1 and is convolved on its own: it starts from its own history (zeros
 * without one) and nothing crosses a boundary.
 *   x, dy         bf16 [total, D], channels contiguous, row stride x_st / dy_st (elements, a
 *                 multiple of 8, >= D), 16-byte aligned. y, dx: bf16 [total, D] contiguous.
 *   cu_seqlens    int32 [nseq+1] on the device. Checked on the device: cu[0] == 0, never
 *                 decreasing, cu[nseq] == total; empty sequences are allowed.
 *   init_state    bf16 [nseq, D, W-1] (decode layout) or NULL (zeros).
 *   final_state   out, bf16 [nseq, D, W-1] or NULL: the last W-1 values of each sequence's
 *                 history-then-rows (an empty sequence's is its history). Must not overlap
 *                 init_state (no in-place advance for packed batches).
 *   d_init_state  out (backward), bf16 [nseq, D, W-1] or NULL: each history's gradient.
 *   status        int32 on the device, required: receives CCONV_OK, or CCONV_ERR_INDEX when
 *                 the offsets break the rule -- then nothing else is written (y, dx, dw,
 *                 dbias and the states keep their contents). Written by every call that
 *                 returns CCONV_OK.
 *   workspace     as for cconv_bwd with B = 1, T = total: cconv_bwd_workspace_bytes(1, total,
 *                 D, W), or cconv_bwd_workspace_bytes_config(1, total, D, W, config).
 * Limits: total <= 2^31 - 1, nseq <= 2^24. dw and dbias sum over all sequences. The _config
 * variants take a launch configuration as for one batch row of total rows; only the streaming
 * options (options & ~8 == 3: non-temporal loads and stores, no prefetch) are compiled for
 * packed batches, others
 * give CCONV_ERR_BAD_CONFIG.
 */
cconv_status_t cconv_fwd_varlen(const void* x, int64_t x_st, const int32_t* cu_seqlens, int64_t nseq, int64_t total,
                                const void* w, cconv_dtype_t w_dtype, const float* bias, const void* init_state,
                                void* final_state, int32_t* status, void* y, int64_t D, int W,
                                cconv_stream_t stream);

cconv_status_t cconv_bwd_varlen(const void* x, int64_t x_st, const void* dy, int64_t dy_st, const int32_t* cu_seqlens,
                                int64_t nseq, int64_t total, const void* w, cconv_dtype_t w_dtype, const float* bias,
                                const void* init_state, void* dx, void* dw, cconv_dtype_t dw_dtype, float* dbias,
                                void* d_init_state, void* workspace, size_t workspace_bytes, int32_t* status,
                                int64_t D, int W, cconv_stream_t stream);

/*
 * The general forward and backward [fla's causal_conv1d parameter list, kernel-fun wheel,
 * _common/compat.py FLA_KWARGS: activation, residual, initial_state, output_final_state,
 * cu_seqlens]: one entry point each combining the epilogue variants with a history and with
 * packed batches. opts == NULL is SiLU and nothing else (cconv_fwd / cconv_bwd).
 *   activation   CCONV_ACT_SILU (y = silu(z)) or CCONV_ACT_NONE (y = z; the backward's g = dy).
 *                Anything else: CCONV_ERR_BAD_CONFIG.
 *   residual     bf16 rows like x (batch stride residual_sb, row stride residual_st elements,
 *                multiples of 8, residual_st >= D; 16-byte aligned) added to y after the
 *                activation, or NULL. Its gradient is dy itself: the backward has nothing to do.
 *   init_state, final_state, d_init_state
 *                as cconv_fwd_state / cconv_bwd_state ([B, D, W-1]), or per packed sequence
 *                ([nseq, D, W-1]) with cu_seqlens.
 *   cu_seqlens, nseq, status
 *                a packed batch as cconv_fwd_varlen / cconv_bwd_varlen: then B must be 1 and
 *                T is the packed row count; x_sb, dy_sb and residual_sb are ignored.
 *   y_sb, y_st (forward), dx_sb, dx_st (backward)
 *                the output's batch and row strides in elements; y_st == 0 (dx_st == 0)
 *                means contiguous [B, T, D]. Otherwise the rules of the inputs' strides
 *                (multiples of 8 on the vector path, row stride >= D), and rows that do not
 *                overlap (for B > 1, batch stride >= (T-1)*row stride + D); the batch stride
 *                is ignored for a packed batch. Only the D channels of each row are written.
 *                A power-of-two row pitch streams fastest (see the performance note above):
 *                an output of width 3072 or 6144 written into rows of 4096 or 8192 elements
 *                cuts the forward's time by 12-14%. The aliasing check treats the output as
 *                the whole byte range it spans, padding included.
 * The variants without an activation or with a residual run the default launch (no
 * configuration entry point).
 */
typedef enum { CCONV_ACT_NONE = 0, CCONV_ACT_SILU = 1 } cconv_activation_t;

typedef struct {
    int activation;
    const void* residual;
    int64_t residual_sb, residual_st;
    const void* init_state;
    void* final_state;
    const int32_t* cu_seqlens;
    int64_t nseq;
    int32_t* status;
    int64_t y_sb, y_st;
} cconv_fwd_opts_t;

typedef struct {
    int activation;
    const void* init_state;
    void* d_init_state;
    const int32_t* cu_seqlens;
    int64_t nseq;
    int32_t* status;
    int64_t dx_sb, dx_st;
} cconv_bwd_opts_t;

cconv_status_t cconv_fwd_ex(const void* x, int64_t x_sb, int64_t x_st, const void* w, cconv_dtype_t w_dtype,
                            const float* bias, void* y, int64_t B, int64_t T, int64_t D, int W,
                            const cconv_fwd_opts_t* opts, cconv_stream_t stream);

cconv_status_t cconv_bwd_ex(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb, int64_t dy_st,
                            const void* w, cconv_dtype_t w_dtype, const float* bias, void* dx, void* dw,
                            cconv_dtype_t dw_dtype, float* dbias, void* workspace, size_t workspace_bytes, int64_t B,
                            int64_t T, int64_t D, int W, const cconv_bwd_opts_t* opts, cconv_stream_t stream);

/*
 * The backward's two stages, for callers that want the fp32 partials themselves (a
 * data-parallel caller can sum them across ranks before the final cast) or that time the
 * stages apart. cconv_bwd_main writes dx and fills the workspace with fp32 dw/dbias partial
 * sums; cconv_bwd_finish sums the partials in a fixed order into dw (dw_dtype) and dbias
 * (fp32, or NULL). Both take the same B, T, D, W as the cconv_bwd call they split, and
 * cconv_bwd == cconv_bwd_main followed by cconv_bwd_finish, bit for bit.
 */
cconv_status_t cconv_bwd_main(const void* x, int64_t x_sb, int64_t x_st, const void* dy, int64_t dy_sb,
                              int64_t dy_st, const void* w, cconv_dtype_t w_dtype, const float* bias, void* dx,
                              void* workspace, size_t workspace_bytes, int64_t B, int64_t T, int64_t D, int W,
                              cconv_stream_t stream);

cconv_status_t cconv_bwd_finish(const void* workspace, size_t workspace_bytes, void* dw, cconv_dtype_t dw_dtype,
                                float* dbias, int64_t B, int64_t T, int64_t D, int W, cconv_stream_t stream);

/*
 * One-token decode update [PR #797 description: `CausalConv1dUpdate` API and semantics].
 *   x       bf16 [N, D], row n at x + n*x_ld, x_ld >= D (a slice of a wider projection).
 *   state   bf16 [S, D, W-1] contiguous, in/out, oldest first: state[s, d, j] holds the
 *           input that came W-1-j tokens before the one being added. Updated in place by
 *           bit copies: the oldest value drops out and x[n, d] becomes the newest.
 *   state_indices  int32 [N]: the slot of row n; -1 marks a padding row that reads and
 *           writes no state and whose y row is 0. NULL means slot n for row n (needs N <= S).
 *   w, bias as in cconv_fwd; y bf16 [N, D] contiguous, written.
 *   z = bias + sum_{j<W-1} w[d, j] * state[s, d, j] + w[d, W-1] * x[n, d];  y = silu(z).
 *   status  device int32: receives CCONV_OK or CCONV_ERR_INDEX. Required (non-NULL) when
 *           state_indices is given and N > 0, since only the device sees the verdict
 *           (CCONV_ERR_NULL_POINTER otherwise); may be NULL without indices.
 * Index validation happens on the device, inside the one kernel: an index outside [-1, S),
 * or a non-negative index that appears twice, makes the whole call invalid. Then no state
 * row is written (bitwise unchanged), y is unspecified, and *status = CCONV_ERR_INDEX.
 * No device trap is raised, so the process stays usable. Limits: N <= 2^24, D <= 2^26; with
 * indices, S <= 2^19 - 32 (the duplicate check keeps an S-bit set and a verdict word in 64 KB
 * of LDS).
 */
cconv_status_t cconv_update(const void* x, int64_t x_ld, void* state, int64_t S,
                            const int32_t* state_indices, const void* w, cconv_dtype_t w_dtype,
                            const float* bias, void* y, int64_t N, int64_t D, int W,
                            int32_t* status, cconv_stream_t stream);

/*
 * Decode variants [the decode PR's API: conv_state [S, D, L] with L in {3, 4} for W = 4, and
 * reserved cache_seqlens circular-buffer metadata].
 *   L              entries per channel in the state: W-1 (as cconv_update) or W (the oldest
 *                  entry is carried but not used: a shift drops it).
 *   state          bf16 [S, D, L], 16-byte aligned, updated in place.
 *   cache_seqlens  int32 [N] on the device, or NULL. NULL: shift mode (drop the oldest entry,
 *                  append the token: L entries rewritten). Given: circular mode, nothing
 *                  moves: for row n with c = cache_seqlens[n] >= 0 the token k steps back is
 *                  entry (c - k) mod L and the new token goes to entry c mod L; no other
 *                  entry changes value (on the vector path the kernel stores each slot's whole
 *                  16*L-byte run, the other entries with the values it just read: 16-byte
 *                  stores beat 2-byte ones at decode sizes). The caller advances
 *                  cache_seqlens. A state written by a prefill (oldest first) is a circular
 *                  state with c = 0 (mod L). Needs L >= 1.
 * Everything else as cconv_update; a negative cache_seqlens entry fails the call like an
 * invalid index (CCONV_ERR_INDEX in *status, nothing written), so status is required when
 * cache_seqlens is given too.
 */
cconv_status_t cconv_update_ex(const void* x, int64_t x_ld, void* state, int64_t S, int L,
                               const int32_t* state_indices, const int32_t* cache_seqlens, const void* w,
                               cconv_dtype_t w_dtype, const float* bias, void* y, int64_t N, int64_t D, int W,
                               int32_t* status, cconv_stream_t stream);

/*
 * Launch configuration of the decode update, for sweeps and for tests of invariance to the
 * launch shape: y and the state do not depend on it (bit for bit).
 *   vec              channels per thread: 8 (D % 8 == 0), 4 (D % 4 == 0, row stride a
 *                    multiple of 4, x, y and the state 8-byte aligned, w 8-byte aligned (16
 *                    for fp32 taps), bias 16-byte aligned; CCONV_ERR_MISALIGNED otherwise)
 *                    or 1 (any D)
 *   block_threads    threads per block, a multiple of 64 in [64, 1024]; a thread owns vec
 *                    channels of every row its block walks
 *   rows_per_thread  rows a thread carries at once, their loads in flight together and the
 *                    taps loaded once for them: 1 or 2 (1 when vec = 1); blocks of at most
 *                    512 threads for 2 (registers)
 *   options          bit 0: non-temporal stores of y and the state; bit 1: non-temporal
 *                    loads of x and the state; bit 2 (vec = 8, not with bit 1): the state
 *                    runs pass through LDS so that each load and store instruction covers
 *                    contiguous bytes (the block's LDS, slot check included, must stay
 *                    within 64 KiB); 0 when vec = 1
 *   rows_per_block   rows of N each block walks (>= 1; the grid's row dimension,
 *                    ceil(N / rows_per_block), must stay <= 65535)
 * An invalid configuration is CCONV_ERR_BAD_CONFIG.
 */
typedef struct {
    int vec;
    int block_threads;
    int rows_per_thread;
    int options;
    int64_t rows_per_block;
} cconv_update_config_t;

/* The configuration cconv_update and cconv_update_ex use for N rows of D channels (with
 * operands that meet the vec rule above; a call whose operands miss the 4-channel rule runs
 * one channel per thread): 8 channels per thread with options 5 (non-temporal stores, state
 * runs staged through LDS; the call drops the staging when S is too large for the LDS), 4
 * with options 1, 1 with options 0; 256-thread blocks, 2 rows per thread. */
cconv_status_t cconv_default_update_config(int64_t N, int64_t D, cconv_update_config_t* out);

/* cconv_update_ex with an explicit launch configuration (cfg must not be NULL). */
cconv_status_t cconv_update_config(const void* x, int64_t x_ld, void* state, int64_t S, int L,
                                   const int32_t* state_indices, const int32_t* cache_seqlens,
                                   const void* w, cconv_dtype_t w_dtype, const float* bias, void* y,
                                   int64_t N, int64_t D, int W, int32_t* status,
                                   const cconv_update_config_t* cfg, cconv_stream_t stream);

/* A short English description of a status code (static storage). */
const char* cconv_status_string(cconv_status_t status);

/* Library version and build string (static storage). */
const char* cconv_version(void);

/*
 * Launch configuration, for sweeps and for tests of invariance to the launch shape. The
 * entry points above pick one from a static table; these take it explicitly. y and dx do
 * not depend on the configuration (bitwise); dw and dbias depend on it only through the
 * order of their fixed-order sum.
 *   vec              channels per lane: 4 or 8 (8 or 16 bytes per row per lane); 2 (4 bytes)
 *                    or 1 (2 bytes) on the element-granular paths (16-row groups, plain
 *                    loads and stores, the general kernel: options 0)
 *   rows_per_group   rows whose loads are issued together: 4 or 8 (and 16 with vec 4)
 *   waves_per_block  1, 2, 4 or 8 waves per block
 *   strips_per_block a divisor of waves_per_block: the block's waves cover this many
 *                    adjacent channel strips (64*vec channels each) times
 *                    waves_per_block/strips_per_block consecutive time segments of one batch
 *                    row; the backward sums the dw partials of a strip's segments in LDS
 *   seg_rows         rows per wave segment: a multiple of rows_per_group, >= 8
 *   options          bit 0: non-temporal loads of x (and dy); bit 1: non-temporal stores of
 *                    y (dx); bit 2: issue the next row group's loads before the current
 *                    group's arithmetic (software prefetch); bit 3: "solo" kernels for
 *                    one-wave blocks (waves_per_block must be 1) that run one wave per SIMD
 *                    and may use the whole register file. Results do not depend on them.
 * The lane groups (ceil(D / vec) of them; with vec = 4 and D = 2 (mod 4) the last one starts
 * at channel D - 4) are split into ceil(D / (64 * vec)) channel strips of as equal widths as
 * integers allow.
 */
typedef struct {
    int vec;
    int rows_per_group;
    int waves_per_block;
    int strips_per_block;
    int options;
    int64_t seg_rows;
} cconv_config_t;

/*
 * The configuration cconv_fwd (which = 0) or cconv_bwd (which = 1) uses for this shape: 4
 * channels per lane (2 when D == 2, 1 for odd D), 16-row groups, one-wave blocks, each
 * batch row cut into as many segments as the wave slots hold (1024 waves, one per SIMD; 2048
 * with 2 channels per lane; 3072 for the forward and 2048 for the backward with one), down
 * to one 16-row group;
 * non-temporal hints (options 11) when 2D is a multiple of 128 or the call streams at most
 * 256 MB, plain loads and stores (options 8; 0 on the element-granular path) otherwise.
 * Packed batches and the epilogue variants use the same plan with the streaming hints. The
 * segments depend on the shape alone, so the workspace cconv_bwd_workspace_bytes reports
 * holds for every layout of the operands.
 */
cconv_status_t cconv_default_config(int which, int64_t B, int64_t T, int64_t D, int W,
                                    cconv_config_t* out);

cconv_status_t cconv_fwd_config(const void* x, int64_t x_sb, int64_t x_st, const void* w,
                                cconv_dtype_t w_dtype, const float* bias, void* y, int64_t B,
                                int64_t T, int64_t D, int W, const cconv_config_t* cfg,
                                cconv_stream_t stream);

/* Workspace for cconv_bwd_config with this configuration; 0 for an invalid one. */
size_t cconv_bwd_workspace_bytes_config(int64_t B, int64_t T, int64_t D, int W,
                                        const cconv_config_t* cfg);

cconv_status_t cconv_bwd_config(const void* x, int64_t x_sb, int64_t x_st, const void* dy,
                                int64_t dy_sb, int64_t dy_st, const void* w,
                                cconv_dtype_t w_dtype, const float* bias, void* dx, void* dw,
                                cconv_dtype_t dw_dtype, float* dbias, void* workspace,
                                size_t workspace_bytes, int64_t B, int64_t T, int64_t D, int W,
                                const cconv_config_t* cfg, cconv_stream_t stream);

/* Packed batches with an explicit launch configuration (see cconv_fwd_varlen). */
cconv_status_t cconv_fwd_varlen_config(const void* x, int64_t x_st, const int32_t* cu_seqlens, int64_t nseq,
                                       int64_t total, const void* w, cconv_dtype_t w_dtype, const float* bias,
                                       const void* init_state, void* final_state, int32_t* status, void* y,
                                       int64_t D, int W, const cconv_config_t* config, cconv_stream_t stream);

cconv_status_t cconv_bwd_varlen_config(const void* x, int64_t x_st, const void* dy, int64_t dy_st,
                                       const int32_t* cu_seqlens, int64_t nseq, int64_t total, const void* w,
                                       cconv_dtype_t w_dtype, const float* bias, const void* init_state, void* dx,
                                       void* dw, cconv_dtype_t dw_dtype, float* dbias, void* d_init_state,
                                       void* workspace, size_t workspace_bytes, int32_t* status, int64_t D, int W,
                                       const cconv_config_t* config, cconv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CCONV_H */
