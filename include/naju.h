/*
 * naju.h -- C ABI of libnaju.so, the MI355X (gfx950) implementation of the
 * Naju native-discrete selective state scan and of the mixer-block pieces
 * fused around it.
 *
 * The operation (Naju reproduction README of arXiv 2607.21000, section
 * "Core equations"): for each batch row and channel c, with state row
 * x[c, 0..N-1] (N = d_state),
 *
 *     x_n[c,s] = f_n[c] x_{n-1}[c,s] + i_n[c] h_n[c] B_n[s],
 *     f_n = sigma(a_n),  i_n = sigma(b_n)            (retain / write gates)
 *     ys_n[c]  = (1/sqrt(N)) sum_s x_n[c,s] C_n[s] + D[c] h_n[c]
 *
 * using the post-update state in the readout.  The gates and h are given per
 * (token, channel); B_n and C_n are one N-vector per (batch, token), shared by
 * every channel (the page's "token-dependent B/C directions").
 *
 * The block entry points add the front end and the output modulation of the
 * same page's block flowchart: h = SiLU(causal depthwise conv1d(u)) with
 * d_conv taps and no bias, and y = ys * SiLU(z).  The convolution is a
 * cross-correlation whose last tap multiplies the current token:
 *     pre_n[c] = sum_{k<K} conv_w[c,k] u_{n-K+1+k}[c]
 * with u_m for m < 0 taken from conv_state (zeros if conv_state is NULL).
 *
 * The backward entry points are the reverse mode of these definitions.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layouts   row-major, contiguous, no strides:
 *              per (token, channel) tensors: [batch][seqlen][d_inner]
 *              per token tensors B, C, dB, dC: [batch][seqlen][d_state]
 *              states x0, x_final, dx_final, dx0: [batch][d_inner][d_state] fp32
 *              D, dD: [d_inner] fp32;  conv_w, dconv_w: [d_inner][d_conv] fp32
 *              conv_state, conv_state_out, dconv_state: [batch][d_conv-1][d_inner]
 *                (the d_conv-1 inputs that precede u_0, oldest first), io dtype
 *  Dtypes    activations and their gradients use dims->io (fp32 or bf16);
 *            parameters, states, checkpoints and dD/dconv_w are fp32.  Device
 *            arithmetic is fp32; bf16 results are rounded to nearest even.
 *  Pointers  every data pointer is a device pointer (hipMalloc'd or a torch
 *            tensor), aligned to its element size; outputs must not alias
 *            inputs.  `dims` is a host pointer.  Optional pointers may be NULL
 *            as documented per argument.
 *  Ownership the caller owns every buffer.  The library never allocates device
 *            memory; it uses only the caller's workspace.
 *  Stream    `stream` is a hipStream_t (NULL = the default stream).  Every call
 *            only enqueues work on that stream and returns; nothing is
 *            synchronised.
 *  Workspace `ws` of at least naju_workspace_bytes(op, dims) bytes, zero-filled
 *            before its first use (naju_workspace_init, or any zero fill).
 *            Each call leaves it in a reusable state when its work completes,
 *            for further calls of the same entry point with the same dims.
 *            Zero-fill it again before using it for another entry point or
 *            other dims.  Calls that share one workspace must be ordered (same
 *            stream or explicit dependencies); concurrent calls need separate
 *            workspaces.
 *  Errors    arguments are validated before anything is enqueued: any status
 *            other than NAJU_OK and NAJU_EHIP means nothing was enqueued.
 *            NAJU_EHIP reports a HIP launch error.  naju_last_error() returns a
 *            thread-local message describing the last failure.
 *  Sizes     batch, seqlen, d_inner >= 0 (any zero makes the call a no-op
 *            except for the state outputs: with seqlen == 0, x_final = x0 and
 *            conv_state_out = conv_state).  d_state in {16, 64}; d_conv == 4
 *            for the block entry points.
 */
#ifndef NAJU_H
#define NAJU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NAJU_OK = 0,
    NAJU_EINVAL = 1,       /* bad argument: NULL pointer, bad size, misalignment */
    NAJU_EUNSUPPORTED = 2, /* valid but not built: d_state or d_conv not instantiated */
    NAJU_EWORKSPACE = 3,   /* ws NULL or smaller than naju_workspace_bytes() */
    NAJU_EHIP = 4          /* the HIP runtime reported an error */
} naju_status_t;

typedef enum { NAJU_F32 = 0, NAJU_BF16 = 1 } naju_dtype_t;

typedef enum {
    NAJU_OP_SCAN_FWD = 0,
    NAJU_OP_SCAN_BWD = 1,
    NAJU_OP_BLOCK_FWD = 2,
    NAJU_OP_BLOCK_BWD = 3
} naju_op_t;

typedef struct {
    int64_t batch;   /* Bt */
    int64_t seqlen;  /* L */
    int64_t d_inner; /* Di: channels */
    int64_t d_state; /* N: 16 or 64 */
    int32_t d_conv;  /* K: 4 (block entry points; ignored by the scan ones) */
    int32_t io;      /* naju_dtype_t of activations and their gradients */
} naju_dims_t;

/* Bytes of workspace the entry point `op` needs for `dims` (0 if dims invalid). */
size_t naju_workspace_bytes(naju_op_t op, const naju_dims_t *dims);

/* Bytes of the optional forward checkpoint buffer (fp32 chunk-boundary states
 * written by the forward and read by the backward).  Its layout is private to
 * the library; it is valid only for the same dims. */
size_t naju_ckpt_bytes(const naju_dims_t *dims);

/* Zero-fills a workspace on `stream` (with a kernel, so it may be captured). */
naju_status_t naju_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Synchronises `stream`, then reads the workspace's device-side error word:
 * *flags = 0 if every cross-workgroup wait of the previous calls completed,
 * nonzero if one gave up after its bounded spin (results are then invalid).
 * Every kernel that waits on another workgroup takes its work items from an
 * in-order counter (the matrix-core forward by default), so a
 * wait is always on an item already held by a running workgroup and ends
 * however many workgroups the device runs at once; the bound (about 0.4 s of
 * polling) only catches a device stalled for longer than that. */
naju_status_t naju_workspace_check(const void *ws, size_t ws_bytes, void *stream,
                                   uint32_t *flags);

/*
 * Scan forward: y = ys (readout + feedthrough), x_final = x_L.
 *   h, a, b   [Bt][L][Di] io          token activations, forget and write
 *                                     gate pre-activations
 *   B, C      [Bt][L][N]  io          write / read directions
 *   D         [Di] fp32               direct feedthrough
 *   x0        [Bt][Di][N] fp32 or NULL (= zeros)  initial state
 *   y         [Bt][L][Di] io          output (written)
 *   x_final   [Bt][Di][N] fp32 or NULL            final state (written)
 *   ckpt      naju_ckpt_bytes() or NULL           checkpoints for the backward
 */
naju_status_t naju_scan_fwd(const naju_dims_t *dims, const void *h, const void *a,
                            const void *b, const void *B, const void *C, const float *D,
                            const float *x0, void *y, float *x_final, float *ckpt, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * Scan backward.  Inputs are the forward's inputs plus
 *   ckpt      from naju_scan_fwd on the same inputs, or NULL (recomputed)
 *   dy        [Bt][L][Di] io          dLoss/dy
 *   dx_final  [Bt][Di][N] fp32 or NULL (= zeros)  dLoss/dx_final
 * Outputs (written, not accumulated):
 *   dh, da, db [Bt][L][Di] io;  dB, dC [Bt][L][N] io;  dD [Di] fp32;
 *   dx0 [Bt][Di][N] fp32 or NULL (skipped)
 */
naju_status_t naju_scan_bwd(const naju_dims_t *dims, const void *h, const void *a,
                            const void *b, const void *B, const void *C, const float *D,
                            const float *x0, const float *ckpt, const void *dy,
                            const float *dx_final, void *dh, void *da, void *db, void *dB,
                            void *dC, float *dD, float *dx0, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Block forward: y = ScanReadout(SiLU(conv(u)), a, b, B, C, D) * SiLU(z).
 *   u, z          [Bt][L][Di] io      conv input and modulation input
 *   conv_w        [Di][K] fp32        depthwise taps (no bias)
 *   conv_state    [Bt][K-1][Di] io or NULL (= zeros)  inputs preceding u_0
 *   a, b, B, C, D, x0                 as naju_scan_fwd
 *   y             [Bt][L][Di] io      output (written)
 *   x_final       [Bt][Di][N] fp32 or NULL
 *   conv_state_out [Bt][K-1][Di] io or NULL: last K-1 rows of [conv_state; u]
 *   ckpt          naju_ckpt_bytes() or NULL
 */
naju_status_t naju_block_fwd(const naju_dims_t *dims, const void *u, const void *z,
                             const float *conv_w, const void *conv_state, const void *a,
                             const void *b, const void *B, const void *C, const float *D,
                             const float *x0, void *y, float *x_final, void *conv_state_out,
                             float *ckpt, void *ws, size_t ws_bytes, void *stream);

/*
 * Block backward.  Inputs: the block forward's inputs, ckpt (or NULL), dy and
 * dx_final (or NULL).  Outputs (written):
 *   du, dz, da, db [Bt][L][Di] io;  dB, dC [Bt][L][N] io;
 *   dconv_w [Di][K] fp32;  dD [Di] fp32;
 *   dconv_state [Bt][K-1][Di] io or NULL;  dx0 [Bt][Di][N] fp32 or NULL
 */
naju_status_t naju_block_bwd(const naju_dims_t *dims, const void *u, const void *z,
                             const float *conv_w, const void *conv_state, const void *a,
                             const void *b, const void *B, const void *C, const float *D,
                             const float *x0, const float *ckpt, const void *dy,
                             const float *dx_final, void *du, void *dz, float *dconv_w,
                             void *dconv_state, void *da, void *db, void *dB, void *dC,
                             float *dD, float *dx0, void *ws, size_t ws_bytes, void *stream);

/*
 * Decode step: one token of the scan for every batch row, with the state
 * carried in place -- the streaming-generation form of the same recurrence
 * and readout (naju_scan_fwd on one token with x0 = x, x_final written back
 * to x).  dims->seqlen is not used; no workspace.
 *   h, a, b   [Bt][Di] io         this token's activation and gate pre-activations
 *   B, C      [Bt][N]  io
 *   D         [Di] fp32
 *   x         [Bt][Di][N] fp32, 16-byte aligned: the state before the token on
 *             entry, after it on return (read and written by the call)
 *   y         [Bt][Di] io         output (written)
 * batch <= 65535.
 */
naju_status_t naju_scan_step(const naju_dims_t *dims, const void *h, const void *a,
                             const void *b, const void *B, const void *C, const float *D,
                             float *x, void *y, void *stream);

/*
 * Block decode step: one token of the block (naju_block_fwd on one token with
 * x0 = x and conv_state, both updated in place).
 *   u, z          [Bt][Di] io
 *   conv_w        [Di][K] fp32
 *   conv_state    [Bt][K-1][Di] io: the K-1 inputs before u (oldest first) on
 *                 entry; shifted by one token (u appended) on return
 *   a, b, B, C, D, x, y   as naju_scan_step
 */
naju_status_t naju_block_step(const naju_dims_t *dims, const void *u, const void *z,
                              const float *conv_w, void *conv_state, const void *a,
                              const void *b, const void *B, const void *C, const float *D,
                              float *x, void *y, void *stream);

/*
 * Mixer layer forward (bf16 io only): the block flowchart of the same page
 * ("Background and main changes") around the scan -- input projection, causal
 * depthwise conv + SiLU, forget / write gate and B/C projections, the block
 * scan with readout, feedthrough and SiLU(z) modulation, output projection and
 * residual.  Per token, with row vectors and weights stored [in][out]:
 *     u = xn W_u;  z = xn W_z;  h = SiLU(conv(u))             (conv as naju_block_fwd)
 *     a = h W_a + a_bias;  b = h W_b + b_bias;  B = h W_B;  C = h W_C
 *     y = naju_block_fwd(u, z, conv_w, conv_state, a, b, B, C, D)
 *     out = y W_out + res
 * u, z, h, a, b, B, C and y are bf16 intermediates in the workspace (each
 * rounded to nearest even from fp32); the projections read the bf16 h, the
 * scan recomputes h from u in fp32.  The projections run through hipBLASLt
 * (fp32 accumulation); its handle is created on a device's first call and
 * kept for the process.
 *   dims          batch, seqlen, d_inner, d_state as elsewhere; d_conv == 4;
 *                 io == NAJU_BF16; d_inner % 8 == 0
 *   d_model       width of the layer's input and output, % 8 == 0
 *   xn            [Bt][L][d_model] bf16     normalized tokens
 *   res           [Bt][L][d_model] bf16 or NULL (= no residual)
 *   W_u, W_z      [d_model][d_inner] bf16   input projection (conv branch, gate branch)
 *   conv_w        [d_inner][4] fp32;  conv_state [Bt][3][d_inner] bf16 or NULL
 *   W_a, W_b      [d_inner][d_inner] bf16;  a_bias, b_bias [d_inner] fp32
 *   W_B, W_C      [d_inner][d_state] bf16
 *   D             [d_inner] fp32
 *   W_out         [d_inner][d_model] bf16
 *   out           [Bt][L][d_model] bf16 (written)
 *   ws            naju_mixer_workspace_bytes() bytes, 256-byte aligned, zero-filled
 *                 before first use (as for the other entry points)
 * Matrices, conv_w and conv_state must be 16-byte aligned; batch <= 65535,
 * seqlen <= 16 * 65535.  The first call for a shape asks hipBLASLt's heuristic
 * for each projection's algorithm (host work only) and caches it.  A hipBLASLt
 * failure returns NAJU_EHIP; work already enqueued is not undone.
 */
size_t naju_mixer_workspace_bytes(const naju_dims_t *dims, int64_t d_model);
naju_status_t naju_mixer_fwd(const naju_dims_t *dims, int64_t d_model, const void *xn,
                             const void *res, const void *W_u, const void *W_z,
                             const float *conv_w, const void *conv_state, const void *W_a,
                             const float *a_bias, const void *W_b, const float *b_bias,
                             const void *W_B, const void *W_C, const float *D,
                             const void *W_out, void *out, void *ws, size_t ws_bytes,
                             void *stream);

/*
 * Mixer layer backward: the reverse mode of naju_mixer_fwd for the upstream
 * gradient d_out = dLoss/dout.  The call recomputes the layer's forward
 * intermediates (u, z, h, a, b, B, C, y and the scan checkpoints) in its
 * workspace, then runs the output projection's, the block scan's (the
 * naju_block_bwd kernels), the gate / B / C projections', the projection
 * path's conv + SiLU and the input projections' reverse modes.  The stored
 * bf16 intermediates pass gradients unchanged (rounding taken as the
 * identity); dy and the block backward's gradients are kept in bf16, the
 * projections' sums in fp32.  The residual's gradient is d_out itself.
 *   inputs        as naju_mixer_fwd (no res), and
 *   d_out         [Bt][L][d_model] bf16
 * outputs (written, fp32 unless noted):
 *   dxn [Bt][L][d_model];  dW_u, dW_z [d_model][d_inner];  dconv_w [d_inner][4];
 *   dconv_state [Bt][3][d_inner] bf16 or NULL (needs conv_state);
 *   dW_a, dW_b [d_inner][d_inner];  da_bias, db_bias [d_inner];
 *   dW_B, dW_C [d_inner][d_state];  dD [d_inner];  dW_out [d_inner][d_model]
 *   fwd_ws        NULL (the forward intermediates are recomputed), or the workspace
 *                 of the naju_mixer_fwd call on the same inputs, untouched since
 *                 (it holds u, z, h, a, b, B, C, y and the scan's checkpoints, so
 *                 the recomputation is skipped); fwd_ws_bytes its size
 *   ws            naju_mixer_bwd_workspace_bytes() bytes, as for the forward
 * Output buffers must be 16-byte aligned (dD 4-byte).
 */
size_t naju_mixer_bwd_workspace_bytes(const naju_dims_t *dims, int64_t d_model);
naju_status_t naju_mixer_bwd(const naju_dims_t *dims, int64_t d_model, const void *xn,
                             const void *W_u, const void *W_z, const float *conv_w,
                             const void *conv_state, const void *W_a, const float *a_bias,
                             const void *W_b, const float *b_bias, const void *W_B,
                             const void *W_C, const float *D, const void *W_out,
                             const void *d_out, float *dxn, float *dW_u, float *dW_z,
                             float *dconv_w, void *dconv_state, float *dW_a, float *da_bias,
                             float *dW_b, float *db_bias, float *dW_B, float *dW_C, float *dD,
                             float *dW_out, const void *fwd_ws, size_t fwd_ws_bytes, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * Scan forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, outputs and results as
 * naju_scan_fwd; it allocates nothing, neither itself nor through a library.
 * Its scratch is a 64 MiB device array inside the library, one per GPU, zero
 * at load and held until the process ends; shapes whose forward workspace
 * (naju_workspace_bytes(NAJU_OP_SCAN_FWD, dims)) exceeds it return
 * NAJU_EWORKSPACE before anything is enqueued.  Every call on a GPU shares that
 * GPU's scratch: calls that overlap on one GPU (different streams, or host
 * threads) race and must not be issued.
 *   flags  device uint32 or NULL: receives the call's error word (0: every
 *          cross-workgroup wait completed; nonzero: one gave up and the
 *          results are invalid), which the call then clears in the scratch
 */
naju_status_t naju_scan_fwd_noalloc(const naju_dims_t *dims, const void *h, const void *a,
                                    const void *b, const void *B, const void *C, const float *D,
                                    const float *x0, void *y, float *x_final, float *ckpt,
                                    uint32_t *flags, void *stream);

/* Thread-local description of the last non-OK status ("" if none). */
const char *naju_last_error(void);

/* Library version string. */
const char *naju_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NAJU_H */
