/*
 * ssm.h -- C ABI of libssm.so, the selective state-space scan for AMD
 * Instinct MI355X (gfx950).
 *
 * Per (sequence i, head h, channel p, state n) the scan computes
 *
 *     h_t[n] = exp(dt_t * A_hn) * h_{t-1}[n] + dt_t * B_t[n] * u_t
 *     y_t    = sum_n C_t[n] * h_t[n] + D_h * u_t
 *
 * ("mambazip mamba1/model.rs", forward_impl and selective_scan_state16),
 * where u is the scan input x, or -- with the fused conv -- SiLU of the
 * causal depthwise convolution of x ("ggmlR tests/testthat/test-ssm-rwkv.R",
 * the ssm_conv reference computation).  Operand shapes follow the ggml
 * ssm_scan contract of that ggmlR page (make_scan): every tensor below is
 * row-major, slowest axis first, i.e. ggml's ne list read backwards.
 *
 *   s          [n_state_rows][n_head][head_dim][d_state]  f32   state pool
 *   x          [n_seqs][n_tokens][n_head][head_dim]         io
 *   dt         [n_seqs][n_tokens][n_head]                   io
 *   A          [n_head][d_state] (a_per_state=1) or [n_head] (a_per_state=0)  f32
 *   B, C       [n_seqs][n_tokens][n_group][d_state]         io
 *   D          [n_head]                                     f32  (SSM_HAS_D)
 *   ids        [n_seqs]                                     i32
 *   conv_w     [n_head][d_conv]                             f32  (d_conv > 0)
 *   conv_state [n_state_rows][n_head][d_conv-1]             f32  (optional)
 *
 * The Mamba-1 form is head_dim = 1, n_head = d_inner, a_per_state = 1,
 * n_group = 1.  The Mamba-2 form is a_per_state = 0 (one scalar A per head)
 * with B/C shared by the heads of a group: head h reads group
 * h / (n_head / n_group).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  A pointer to
 *    a tensor with no elements may be NULL.  The library
 *    never allocates, frees or synchronises on the compute calls; they are
 *    enqueued on `stream` (a hipStream_t; NULL is the default stream) and
 *    return as soon as the launches are queued.
 *  - Arguments are checked on the host before anything is launched: a
 *    failed check returns a non-zero ssm_status and launches nothing.  The
 *    checks never read device memory.
 *  - Outputs must not alias inputs (not checked).
 *  - Calls on different streams are independent as long as their outputs
 *    and workspaces differ; the library keeps no mutable global state.
 *  - io is the element type of x, dt, B, C, y and dy (SSM_F32 or
 *    SSM_BF16); everything else is f32.  bf16 results are rounded to
 *    nearest even.
 */
#ifndef SSM_H_
#define SSM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *ssm_stream_t; /* a hipStream_t */

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL = 1,        /* a required pointer is NULL */
    SSM_ERR_SHAPE = 2,       /* a dimension is out of range or inconsistent */
    SSM_ERR_DTYPE = 3,       /* unknown io dtype */
    SSM_ERR_UNSUPPORTED = 4, /* a valid combination the library has no kernel for */
    SSM_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
    SSM_ERR_ALIGN = 6,       /* a pointer is not aligned to its element size (workspace: 256 B) */
    SSM_ERR_HIP = 7          /* a HIP launch reported an error */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

enum {
    SSM_HAS_D = 1u,       /* add D_h * u_t to y_t */
    SSM_DT_SOFTPLUS = 2u  /* use softplus(dt) (x > 20 ? x : log(1 + e^x), "mambazip
                             mamba1/model.rs" softplus) instead of dt as given */
};

/* Device-side error bits, read back with ssm_get_device_error(). */
enum {
    SSM_DEVERR_IDS = 1u,     /* an ids[i] was outside [0, n_state_rows) */
    SSM_DEVERR_SEQLENS = 2u, /* a cu_seqlens span was invalid (selective_scan_fwd_ext) */
    SSM_DEVERR_RELAY = 4u    /* a workgroup of a split grid gave up waiting for the
                                values of the time piece before its own (only if the
                                device stalls for seconds); that call's results are
                                unreliable */
};

typedef struct ssm_scan_desc {
    int64_t n_seqs;       /* sequences (>= 0)                                  */
    int64_t n_tokens;     /* tokens per sequence (>= 0), equal for all        */
    int64_t n_head;       /* heads (Mamba-1: d_inner) (>= 1)                  */
    int64_t head_dim;     /* channels per head (Mamba-1: 1) (>= 1)            */
    int64_t d_state;      /* states per channel, 1..256                       */
    int64_t n_group;      /* B/C groups, divides n_head                       */
    int64_t n_state_rows; /* rows of s and conv_state (>= 1)                  */
    int32_t a_per_state;  /* 1: A[n_head][d_state]; 0: A[n_head]              */
    int32_t d_conv;       /* 0: u = x; 2..8: u = SiLU(causal conv of x), head_dim 1 */
    int32_t chunk;        /* time chunk in tokens, 0 = library's choice; results
                             do not depend on it beyond rounding               */
    int32_t io_dtype;     /* ssm_dtype                                        */
    uint32_t flags;       /* SSM_HAS_D | SSM_DT_SOFTPLUS                      */
    uint32_t reserved;    /* must be 0                                        */
} ssm_scan_desc;

/* Human-readable name of a status code (static storage). */
const char *ssm_status_str(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int ssm_version(void);

/* ---- sizes and offsets of the packed buffers (host only) ----------------
 * Packed forward result (ggmlR page, "ggml_ssm_scan packs outputs and
 * states into one flat tensor"): y [n_seqs][n_tokens][n_head][head_dim] in
 * io, immediately followed by the final states [n_seqs][n_head][head_dim]
 * [d_state] in f32.  Row i of the state block is sequence i's final state.
 * For f32 io the state block starts at element nelements(x), as in ggml.
 * Each returns 0 if the descriptor is invalid. */
size_t ssm_scan_out_bytes(const ssm_scan_desc *desc);
size_t ssm_scan_state_offset_bytes(const ssm_scan_desc *desc);

/* Packed gradient of selective_scan_bwd, all f32, in the order of ggml's
 * ssm_scan_back ("ggml_ssm_scan_back packs all six input gradients"):
 * d_s (shape of s) | d_x | d_dt | d_A | d_B | d_C, then d_D [n_head] when
 * SSM_HAS_D, then with d_conv > 0 (selective_scan_bwd_conv) d_conv_w
 * [n_head][d_conv] and d_conv_state [n_state_rows][n_head][d_conv-1].
 * offsets[k] (k = 0..6) receives the byte offset of block k (d_D's offset
 * is the end of d_C; the conv blocks follow d_D, or d_C without D); returns
 * the total size in bytes, 0 if the descriptor is invalid. */
size_t ssm_scan_dgrad_layout(const ssm_scan_desc *desc, size_t offsets[7]);

/* Workspace the compute calls need (bytes, a multiple of 256).  backward = 0
 * for selective_scan_fwd, 1 for selective_scan_bwd.  The first 256 bytes of
 * a workspace hold the device-error word: zero the workspace once after
 * allocating it; the library sets bits and never clears them.  The rest may
 * hold flags of the relay split (see ssm_scan_fwd_plan) and of the backward's
 * split of the Mamba-2 form (selective_scan_bwd) that every finished
 * call leaves at zero; after SSM_DEVERR_RELAY, zero the workspace again. */
size_t ssm_scan_workspace_bytes(const ssm_scan_desc *desc, int backward);

/* ---- compute -------------------------------------------------------------
 * ssm_conv_fwd: the ggml ssm_conv operator ("ggml_ssm_conv matches a
 * depthwise convolution computed in R"):
 *   out[s][t][c] = sum_{j<d_conv} sx[s][c][t + j] * w[c][j]
 * then SiLU when apply_silu != 0.  sx [n_s][d_inner][d_conv-1+n_t] (time
 * fastest, carrying the d_conv-1 earlier inputs) and out [n_s][n_t][d_inner]
 * have dtype io; w [d_inner][d_conv] is f32.  The last tap w[c][d_conv-1]
 * multiplies the newest input.  One sequence's tensors are addressed with
 * 32-bit byte offsets: (d_inner + 64) * (d_conv - 1 + n_t + 128) must not
 * exceed 2^29 - 1, else SSM_ERR_SHAPE. */
int ssm_conv_fwd(const void *sx, const float *w, void *out, int64_t n_s, int64_t n_t,
                 int64_t d_inner, int32_t d_conv, int32_t io_dtype, int32_t apply_silu,
                 ssm_stream_t stream);

/* ssm_conv_bwd: backward of ssm_conv_fwd, the ggmlR extension's ssm_conv
 * backward ("ggmlR tests/testthat/test-ssm-rwkv.R", the ssm_conv backward
 * block; ggml_ssm_conv_back).  With z = sum_j sx[s][c][t + j] * w[c][j]:
 *   g[s][t][c] = dout[s][t][c]                       (apply_silu == 0)
 *   g[s][t][c] = dout[s][t][c] * d/dz (z * sigmoid(z))  (apply_silu != 0,
 *                 at the pre-activation recomputed from sx and w)
 *   d_sx[s][c][tau] = sum_j w[c][j] * g[s][tau - j][c]   (0 <= tau - j < n_t)
 *   d_w[c][j]       = sum_{s,t} g[s][t][c] * sx[s][c][t + j]
 *  - sx [n_s][d_inner][d_conv-1+n_t] has dtype io_dtype; w [d_inner][d_conv],
 *    dout [n_s][n_t][d_inner] (the gradient of ssm_conv_fwd's out, e.g. the
 *    d_x of selective_scan_bwd when the scan consumed that output) are f32.
 *  - dgrad (f32, caller-owned) receives d_sx [n_s][d_inner][d_conv-1+n_t]
 *    followed by d_w [d_inner][d_conv], the page's packed order; every
 *    element is written.
 *  - workspace (device, caller-owned, at least ssm_conv_bwd_workspace_bytes
 *    bytes, 4-byte aligned; may be NULL when that is 0) holds per-tile
 *    partial weight gradients; its contents need no initialisation.  d_w is
 *    summed in a fixed order, so results repeat bitwise.
 *  - sx and dout may be NULL when they have no elements (n_t = 0 for dout).
 *  - One sequence's tensors are addressed with 32-bit byte offsets:
 *    (d_inner + 64) * (d_conv - 1 + n_t + 128) must not exceed 2^29 - 1, else
 *    SSM_ERR_SHAPE.
 *  - Errors as ssm_conv_fwd, plus SSM_ERR_WORKSPACE for a short workspace;
 *    nothing is launched on error.  Asynchronous on stream. */
size_t ssm_conv_bwd_workspace_bytes(int64_t n_s, int64_t n_t, int64_t d_inner, int32_t d_conv);
int ssm_conv_bwd(const void *sx, const float *w, const float *dout, float *dgrad, int64_t n_s,
                 int64_t n_t, int64_t d_inner, int32_t d_conv, int32_t io_dtype,
                 int32_t apply_silu, void *workspace, size_t workspace_bytes,
                 ssm_stream_t stream);

/* selective_scan_fwd: the scan over n_tokens tokens for every sequence.
 *  - Sequence i starts from state row ids[i] of s.  An id outside
 *    [0, n_state_rows) is not read: that sequence's y and state are written
 *    as NaN and SSM_DEVERR_IDS is set in the workspace's error word.
 *  - With d_conv > 0, the conv for token t reads x at t-d_conv+1..t; inputs
 *    before token 0 come from conv_state row ids[i] (oldest first), or are
 *    zero when conv_state is NULL.  conv_state_out (may be NULL) receives
 *    the last d_conv-1 inputs of each sequence, [n_seqs][n_head][d_conv-1].
 *  - out receives the packed result (see ssm_scan_out_bytes).
 *  - D may be NULL only without SSM_HAS_D; conv_w only when d_conv = 0.
 *  - workspace: ssm_scan_workspace_bytes(desc, 0) bytes, 256-byte aligned. */
int selective_scan_fwd(const ssm_scan_desc *desc, const float *s, const void *x,
                       const void *dt, const float *A, const void *B, const void *C,
                       const float *D, const int32_t *ids, const float *conv_w,
                       const float *conv_state, void *out, float *conv_state_out,
                       void *workspace, size_t workspace_bytes, ssm_stream_t stream);

/* selective_scan_fwd_static: selective_scan_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It takes no workspace: its scratch (the
 * time-chunk carries of the chunked kernels and the device-error word) is a
 * 32 MiB array of static device memory inside the library, which each GPU
 * holds from the first call on it until the process ends.  It calls no
 * hipMalloc, hipFree or other allocating routine.
 *  - Arguments, results and kernels are those of selective_scan_fwd.
 *  - err (nullable): a caller-owned device word that receives the
 *    SSM_DEVERR_* bits (set, never cleared); without it they are dropped.
 *  - A call whose ssm_scan_workspace_bytes(desc, 0) exceeds 32 MiB returns
 *    SSM_ERR_WORKSPACE before anything is launched.
 *  - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *    time on one GPU (on different streams, or from several host threads
 *    without ordering) race on it.  Calls queued on one stream are ordered
 *    and safe.  The scratch starts at zero (static storage) and every
 *    finished call leaves its relay flags at zero again. */
int selective_scan_fwd_static(const ssm_scan_desc *desc, const float *s, const void *x,
                              const void *dt, const float *A, const void *B, const void *C,
                              const float *D, const int32_t *ids, const float *conv_w,
                              const float *conv_state, void *out, float *conv_state_out,
                              uint32_t *err, ssm_stream_t stream);

/* Extras of selective_scan_fwd_ext.  Every pointer may be NULL (feature off).
 *  - dt_bias [n_head] f32: added to dt before softplus, as the step of
 *    "mambazip mamba1/model.rs" (forward_impl) does: dt = softplus(dt_raw +
 *    dt_bias) with SSM_DT_SOFTPLUS, dt_raw + dt_bias without it.
 *  - z, shaped like x in io dtype: the output gate of that step,
 *    y = (sum_n C h + D u) * SiLU(z), applied before y is rounded to io.
 *  - cu_seqlens [n_seqs + 1] int32, DEVICE: variable-length sequences packed
 *    along one token axis.  Sequence i is tokens cu_seqlens[i] ..
 *    cu_seqlens[i+1]-1 and starts from state row ids[i] (and conv_state row
 *    ids[i]), as the flattened sequences of "ggmlR tests/testthat/test-ssm-rwkv.R"
 *    (its RWKV-6/7 shapes) start a fresh state at each sequence; lengths may differ and may be 0.
 *    x, z, y are then [total_tokens][n_head][head_dim], dt [total_tokens]
 *    [n_head], B and C [total_tokens][n_group][d_state], and desc->n_tokens
 *    is an upper bound on every length (it sizes chunking and workspace).
 *    A span with cu_seqlens[i] < 0, cu_seqlens[i+1] < cu_seqlens[i],
 *    cu_seqlens[i+1] > total_tokens or a length above desc->n_tokens is not
 *    scanned: its final state is written as NaN, its y rows are left as they
 *    were, and SSM_DEVERR_SEQLENS is set.
 *  - total_tokens: with cu_seqlens, the length of the packed token axis
 *    (>= 0); without, it must be 0 and the layout is that of
 *    selective_scan_fwd. */
typedef struct ssm_scan_ext {
    const float *dt_bias;
    const void *z;
    const int32_t *cu_seqlens;
    int64_t total_tokens;
} ssm_scan_ext;

/* Size of the packed result of selective_scan_fwd_ext: y (total_tokens x
 * n_head x head_dim io elements with cu_seqlens, else as ssm_scan_out_bytes)
 * followed by the n_seqs final states in f32.  *state_offset (may be NULL)
 * receives the state block's byte offset.  Returns 0 if desc or ext is
 * invalid (ext may be NULL: no extras). */
size_t ssm_scan_ext_out_bytes(const ssm_scan_desc *desc, const ssm_scan_ext *ext,
                              size_t *state_offset);

/* selective_scan_fwd_ext: selective_scan_fwd with the extras above (ext may
 * be NULL, which equals selective_scan_fwd).  Same arguments, checks and
 * workspace (ssm_scan_workspace_bytes(desc, 0)); z must be aligned like x.
 * Kernels: every shape selective_scan_fwd runs, with the extras fused into
 * the scan (dt_bias where dt is read, the gate where y is written, the
 * spans in each workgroup's token range). */
int selective_scan_fwd_ext(const ssm_scan_desc *desc, const ssm_scan_ext *ext, const float *s,
                           const void *x, const void *dt, const float *A, const void *B,
                           const void *C, const float *D, const int32_t *ids,
                           const float *conv_w, const float *conv_state, void *out,
                           float *conv_state_out, void *workspace, size_t workspace_bytes,
                           ssm_stream_t stream);

/* ssm_scan_fwd_plan: the kernel family a selective_scan_fwd(_ext) call with
 * this descriptor and extras (ext may be NULL; only which of its pointers
 * are non-NULL matters) would run, taking every tensor as present and
 * 256-byte aligned: "none" (nothing to compute), "time_split" (few
 * (sequence, channel) rows: tokens split across the waves of a workgroup),
 * "quad" or "quad_chunked" (the Mamba-1 form, d_state <= 16, without or with
 * time chunks), "quad_relay" (as "quad", with the last jobs of an uneven grid
 * cut into time pieces that hand their state on, on the current device; the
 * results are bitwise those of "quad", and the environment variable
 * SSM_RELAY=0 turns the split off),
 * "ssd" (the Mamba-2 form on MFMA) or "rows" (every other shape).  NULL if
 * the descriptor or ext is invalid.  Host only; reads no device memory (it
 * may query the current device's properties).  For profiling and tests. */
const char *ssm_scan_fwd_plan(const ssm_scan_desc *desc, const ssm_scan_ext *ext);

/* selective_scan_bwd: reverse-time adjoint of selective_scan_fwd without the
 * fused conv (d_conv must be 0; selective_scan_bwd_conv takes the fused
 * layer).  dout is packed like the forward result (dy in io, then dstate in
 * f32).  dgrad receives the packed f32 gradient (see ssm_scan_dgrad_layout).
 * Rows of d_s no id refers to are zero; repeated ids accumulate.  A sequence
 * whose id is outside [0, n_state_rows) sets SSM_DEVERR_IDS, adds nothing to
 * d_s, and has its d_x and d_dt written as NaN; sums it takes part in that
 * depend on its initial state (d_A, d_C) are NaN as well.
 * Every shape selective_scan_fwd takes is supported.  The adjoint is the one
 * of "kizzasi-model backprop_ssm.rs" (ssm_backward): dL/dh_{t-1} = a_t dL/dh_t +
 * C_{t-1} dy_{t-1}, with the per-element terms of "mambazip mamba1/model.rs"
 * (accumulate_token_step_gradients).  Kernels:
 *  - the Mamba-1 form with d_state <= 16 and one group: a checkpointed
 *    recompute in the forward's four-lanes-per-channel layout;
 *  - the Mamba-2 form with bf16 io, head_dim 32 or 64, d_state 64 or 128 and
 *    16-byte aligned x, dout, B, C, s and dgrad: chunked products on bf16
 *    MFMA operands (the carried gradient and the checkpointed state as bf16
 *    pairs) with fp32 accumulation; when the (sequence, head) jobs exceed
 *    the compute units unevenly, each is cut into pieces of whole chunks
 *    that hand the carried gradient on (bitwise the same results;
 *    SSM_RELAY=0 turns the split off);
 *  - every other shape: one lane group per (sequence, channel) row with
 *    fp32 arithmetic.
 * Every sum over channels, heads, tokens or sequences is taken in a fixed
 * order, so results are bitwise repeatable.
 * workspace: ssm_scan_workspace_bytes(desc, 1) bytes, 256-byte aligned. */
int selective_scan_bwd(const ssm_scan_desc *desc, const float *s, const void *x,
                       const void *dt, const float *A, const void *B, const void *C,
                       const float *D, const int32_t *ids, const void *dout, float *dgrad,
                       void *workspace, size_t workspace_bytes, ssm_stream_t stream);

/* selective_scan_bwd_conv: the backward of the fused layer, causal conv +
 * SiLU + scan (selective_scan_fwd with d_conv > 0): the chain rule through
 * the scan (as selective_scan_bwd), SiLU (derivative sigma(c)(1 + c(1 -
 * sigma(c))) at the pre-activation recomputed from x, conv_state and conv_w)
 * and the depthwise conv in ggml's tap order ("ggmlR
 * tests/testthat/test-ssm-rwkv.R", ssm_conv and its backward block, which
 * packs the gradient of the inputs before that of the weights).
 *  - Arguments as selective_scan_bwd plus the forward's conv_w [n_head]
 *    [d_conv] (required when d_conv > 0) and conv_state [n_state_rows]
 *    [n_head][d_conv-1] (NULL: zeros).  With d_conv = 0 it equals
 *    selective_scan_bwd.
 *  - d_x in dgrad is the gradient of the pre-conv input x.  After d_D the
 *    packed gradient holds d_conv_w [n_head][d_conv] and d_conv_state
 *    [n_state_rows][n_head][d_conv-1]: the gradient of the conv-state row
 *    each sequence gathered (rows no id names are zero, repeated ids
 *    accumulate).  The gradient of the forward's conv_state_out output is
 *    not an input (taken as zero).
 *  - d_conv 2..4.  A bad id also makes d_conv_w NaN (its inputs are unknown).
 * workspace: ssm_scan_workspace_bytes(desc, 1) bytes, 256-byte aligned. */
int selective_scan_bwd_conv(const ssm_scan_desc *desc, const float *s, const void *x,
                            const void *dt, const float *A, const void *B, const void *C,
                            const float *D, const int32_t *ids, const float *conv_w,
                            const float *conv_state, const void *dout, float *dgrad,
                            void *workspace, size_t workspace_bytes, ssm_stream_t stream);

/* selective_state_update: one decode token of every sequence of a batch,
 * with the states updated in place ("mambazip mamba1/model.rs", forward_impl's
 * single-token step: the conv window of depthwise_conv_step, SiLU,
 * dt = softplus(dt_raw + dt_bias), the state update of selective_scan_state16,
 * and the output times SiLU(z); the conv taps in ggml's order as in
 * ssm_conv_fwd, the last weight on the newest input).  For sequence i with
 * state row r = ids[i], head h, channel p:
 *   u = SiLU(sum_j w[h][j] win[j]) with win = conv_state[r][h][0..K-2], x[i][h]
 *       when d_conv = K > 0 (head_dim 1), after which conv_state[r][h] holds
 *       the last K-1 entries of win; otherwise u = x[i][h][p];
 *   d = dt[i][h] (+ dt_bias[h]), then softplus with SSM_DT_SOFTPLUS;
 *   s[r][h][p][n] = exp(d A) s[r][h][p][n] + d B[i][g][n] u   (g = h / (n_head / n_group));
 *   y[i][h][p] = (sum_n C[i][g][n] s[r][h][p][n] + D[h] u) * SiLU(z[i][h][p]).
 *  - desc->n_tokens must be 1; chunk is ignored.  Shapes (row-major): s
 *    [n_state_rows][n_head][head_dim][d_state] f32 (in/out); x, z, y
 *    [n_seqs][n_head][head_dim] and dt [n_seqs][n_head] in io_dtype; B, C
 *    [n_seqs][n_group][d_state] in io_dtype; A, D, dt_bias, conv_w as in
 *    selective_scan_fwd (dt_bias [n_head] f32); conv_state
 *    [n_state_rows][n_head][d_conv-1] f32 (in/out).
 *  - dt_bias, z and err may be NULL; D may be NULL only without SSM_HAS_D;
 *    conv_w and conv_state must be given when d_conv > 0.
 *  - ids must be distinct: two sequences naming one row race on it.  An id
 *    outside [0, n_state_rows) leaves every row untouched, writes that
 *    sequence's y as NaN and, when err is given, sets SSM_DEVERR_IDS in *err
 *    (a device word the caller owns and clears).
 *  - Outputs must not alias inputs (s and conv_state are updated in place).
 *  - No workspace.  Asynchronous on stream; nothing is launched on error. */
int selective_state_update(const ssm_scan_desc *desc, float *s, const void *x, const void *dt,
                           const float *dt_bias, const float *A, const void *B, const void *C,
                           const float *D, const void *z, const int32_t *ids,
                           const float *conv_w, float *conv_state, void *y, uint32_t *err,
                           ssm_stream_t stream);

/* Copies the device-error word of a workspace to *bits (synchronises the
 * stream; for tests and debugging, not for the hot path). */
int ssm_get_device_error(const void *workspace, ssm_stream_t stream, uint32_t *bits);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H_ */
