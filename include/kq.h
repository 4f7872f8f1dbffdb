/*
 * kq.h -- C ABI of libkq, the k-quant decode matvec library for AMD MI355X
 * (gfx950).
 *
 * The operations come from "How to Write an Inference Engine -- the Muser
 * book":
 *   - the decode matvec y = W x over quantized weight rows (Ch 1 "The problem:
 *     why inference is a memory problem", section 1.3; Ch 19 "The down
 *     projection + residual", section 19.1, operation 1);
 *   - the Q4_K and Q6_K 256-weight superblocks of 144 and 210 bytes (Ch 19,
 *     section 19.3) with per-block scale (and min) (Ch 5 "Quantization from
 *     scratch", section 5.5);
 *   - the speculative-verify batch of up to 16 activation rows (Ch 10 "The
 *     forward pass at a glance", section 10.1; Ch 36 "Prefill vs decode",
 *     section 36.4, Y = W X);
 *   - the SiLU-gated FFN product (Ch 10, section 10.3, box 11);
 *   - the fused dual-epsilon residual tail (Ch 19, sections 19.1 and 19.4;
 *     Ch 10, section 10.4, Figure 10.2).
 *
 * Superblock layouts (the pages give only the sizes; this library adopts the
 * common k-quant packing):
 *   Q4_K, 144 B: d f16 @0, dmin f16 @2, 12 B of packed 6-bit scales and mins
 *     for 8 sub-blocks of 32 @4, 128 B of 4-bit quants @16.
 *     weight = d * scale_s * q - dmin * min_s.
 *   Q6_K, 210 B: low 4 bits @0 (128 B), high 2 bits @128 (64 B), 16 int8
 *     scales for sub-blocks of 16 @192, d f16 @208.
 *     weight = d * scale_s * (q - 32).
 *   Q5_K, 176 B: d f16 @0, dmin f16 @2, the 12 bytes of 6-bit scales and mins
 *     of Q4_K @4, 32 B of fifth bits @16 (byte j: bit 2c for weight 64c + j,
 *     bit 2c+1 for weight 64c + 32 + j), 128 B of low 4 bits @48 laid out as
 *     Q4_K's quants.  weight = d * scale_s * q - dmin * min_s, q = 0..31.
 *     (The pages name Q5_K among the pinned decode kernels, Ch 4 "Pipeline
 *     state objects and the three kernel sources", section 4.4.)
 *   A weight matrix with n_rows outputs and k inputs is stored row-major:
 *   row r is k/256 consecutive superblocks starting at byte
 *   r * (k/256) * block_bytes, and superblock b of a row covers inputs
 *   256b .. 256b+255.
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer (hipMalloc or a PyTorch ROCm
 *     tensor).  The caller owns every buffer; the library allocates nothing.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  They enqueue kernels and return; they do
 *     no host<->device copy and no synchronization.
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     any error the call returns a negative kq_status and enqueues nothing, so
 *     outputs are left untouched.  A failed kernel launch returns
 *     KQ_ERR_LAUNCH.  Unsupported shapes return KQ_ERR_UNSUPPORTED; there is no
 *     slower fallback path.
 *   - Outputs must not overlap inputs (KQ_ERR_ALIAS), except that the tail
 *     updates `residual` in place.
 *   - Results are deterministic: every reduction runs in a fixed order and no
 *     output is written with atomics, so identical inputs give identical bits.
 *   - Accuracy of the M = 1 matvecs (f32 or staged input).  Each input enters
 *     as x_i + e_i with |e_i| <= 2^-22 * max|x_j| over its scale group (32
 *     consecutive inputs for a Q4_K matrix, 16 for Q6_K; a group whose largest
 *     magnitude is below 2^-100 uses the fixed step of such a group instead,
 *     |e_i| <= 2^-123).  Integer dot products are exact; the scales, the Q4_K
 *     min term, the Q6_K -32 offset and the fixed-order sums are f32.  Row r
 *     then satisfies
 *       |y_r - exact_r| <= 2^-22 * sum_g max_g|x| * sum_{i in g} |w_ri|
 *                          + 2^-17 * C_r,
 *     with C_r = sum_i (|a_ri| + |b_ri|) |x_i| for the weight written as
 *     w = a - b before the min or offset cancels (Q4_K a = d*sc*q, b =
 *     dmin*m; Q6_K a = d*sc*q, b = 32*d*sc).  This meets the tolerance
 *     1e-3 * S_r, S_r = sum_i |w_ri x_i|, whenever every group satisfies
 *     max_g|x| * sum_{i in g}|w_ri| <= 2000 * sum_{i in g}|w_ri x_i| and
 *     C_r <= 60 * S_r: activations whose in-group spread is moderate (about
 *     3 for N(0,1) inputs).  One input thousands of times larger than the
 *     rest of its group, on a near-zero weight, can exceed 1e-3 * S_r; the
 *     bound above still holds.
 *     kq_matmul_small_m (M >= 2) on the matrix cores: each input enters as
 *     x_i + e_i with |e_i| <= 2^-22 |x_i| + 2^-39 * max|x| over its
 *     256-input superblock of its activation row.  On the matvec's dot path
 *     (Q4_K at M = 2; the verify gate+up at M = 2 and 3) every row is
 *     computed as the M = 1 matvec computes it, with the bound above.  The
 *     tail's outputs agree within 2e-3 absolute.
 *   - Calls hold no per-call state between them.  Process-wide state: the
 *     device attributes each launcher caches, the kernel attribute set on
 *     first use, the launch-shape override of kq_tune.h (benchmarks only; it
 *     changes the split of the work, never the definition of the result),
 *     the small-M path switches of kq_tune.h (they choose between two
 *     kernels that both meet the bounds above), and the scratch array of
 *     kq_matmul_small_m_noalloc.  Calls are safe from several host threads
 *     on different streams, except concurrently with the kq_tune_set_*
 *     calls.
 */
#ifndef KQ_H
#define KQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int kq_status;

#define KQ_OK 0
#define KQ_ERR_NULL (-1)        /* a required pointer is NULL */
#define KQ_ERR_SHAPE (-2)       /* a size is out of range or inconsistent */
#define KQ_ERR_ALIGN (-3)       /* a pointer is not aligned as required */
#define KQ_ERR_ALIAS (-4)       /* an output overlaps an input */
#define KQ_ERR_UNSUPPORTED (-5) /* valid but not supported (e.g. k too large) */
#define KQ_ERR_LAUNCH (-6)      /* the HIP runtime refused the launch */
#define KQ_ERR_DEVICE (-7)      /* the current device is not usable */

#define KQ_QTYPE_Q4K 1
#define KQ_QTYPE_Q6K 2
#define KQ_QTYPE_Q5K 3

#define KQ_QK 256           /* weights per superblock */
#define KQ_Q4K_BLOCK_BYTES 144
#define KQ_Q6K_BLOCK_BYTES 210
#define KQ_Q5K_BLOCK_BYTES 176
#define KQ_MAX_K 40960      /* largest k (inputs per row) any matvec accepts */
#define KQ_MAX_M 16         /* largest activation batch of kq_matmul_small_m */
#define KQ_MAX_TAIL_N 32768 /* largest row width of kq_fused_residual_norm */
#define KQ_STAGED_LIMBS 3   /* byte limbs per input in a staged activation */
#define KQ_MAX_FUSED_TAIL_K 8192 /* largest k of kq_ffn_tail_gate_up_q4k */

/*
 * Q4_K decode matvec: y[r] = sum_i w[r,i] * x[i] for r < n_rows, with an
 * optional SiLU-gated epilogue y[r] = silu(silu_gate[r]) * (W x)[r] where
 * silu(z) = z / (1 + exp(-z)).
 *   W          [n_rows * (k/256) * 144] bytes, 16-byte aligned.
 *   x          [k] f32, 16-byte aligned.
 *   y          [n_rows] f32 output, 4-byte aligned; must not overlap W, x or
 *              silu_gate.
 *   n_rows     >= 0 (0 enqueues nothing and returns KQ_OK), < 2^31.
 *   k          multiple of 256, 256 <= k <= KQ_MAX_K.
 *   silu_gate  NULL, or [n_rows] f32 (4-byte aligned).
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_ALIAS,
 * KQ_ERR_UNSUPPORTED, KQ_ERR_LAUNCH, KQ_ERR_DEVICE.
 */
kq_status kq_matvec_q4k(const void *W, const float *x, float *y, int64_t n_rows, int64_t k,
                        const float *silu_gate, void *stream);

/*
 * FFN entry in one launch (Ch 10 "The forward pass at a glance", section 10.3:
 * gate and up read the same normed input and meet in the SiLU product):
 *   mid[r] = silu((W_gate x)[r]) * (W_up x)[r],  silu(z) = z / (1 + exp(-z)),
 * for r < n_rows.  Both matrices are Q4_K with the layout and alignment of
 * kq_matvec_q4k, n_rows x k each; x is read and staged once.
 *   mid [n_rows] f32 output, 4-byte aligned; must not overlap W_gate, W_up or x.
 * Errors as kq_matvec_q4k.
 */
kq_status kq_ffn_gate_up_q4k(const void *W_gate, const void *W_up, const float *x, float *mid,
                             int64_t n_rows, int64_t k, void *stream);

/*
 * Q5_K decode matvec: kq_matvec_q4k for Q5_K weights (same arguments,
 * alignment, epilogue, errors and accuracy contract; W is
 * n_rows * (k/256) * 176 bytes, 16-byte aligned).
 */
kq_status kq_matvec_q5k(const void *W, const float *x, float *y, int64_t n_rows, int64_t k,
                        const float *silu_gate, void *stream);

/*
 * Embedding lookup (Ch 10 "The forward pass at a glance", section 10.3, box 1:
 * the token's row of the [vocab x hidden] table becomes the residual stream):
 * for t < n_tokens, out[t * hidden + i] = weight i of row tokens[t] of E,
 * dequantized.  Each value is the f32 nearest the exact weight (the products
 * d * scale * q and dmin * min are exact in f32; only their difference
 * rounds), so the result is exact up to that one rounding.
 *   qtype     KQ_QTYPE_Q4K or KQ_QTYPE_Q5K.
 *   E         [vocab * (hidden/256) * block bytes], 16-byte aligned; row v is
 *             token v.
 *   vocab     1 .. 2^31 - 1.   hidden  multiple of 256, <= KQ_MAX_K.
 *   tokens    [n_tokens] int32 (DEVICE memory), 4-byte aligned.  A token
 *             outside [0, vocab) is not an error: its output row is all NaN
 *             and no row of E is read for it.
 *   n_tokens  0 .. 2^31 - 1 (0 enqueues nothing).
 *   out       [n_tokens][hidden] f32, 16-byte aligned; must not overlap E or
 *             tokens.
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_ALIAS,
 * KQ_ERR_UNSUPPORTED, KQ_ERR_LAUNCH, KQ_ERR_DEVICE.
 */
kq_status kq_embedding(int qtype, const void *E, int64_t vocab, int64_t hidden,
                       const int32_t *tokens, int64_t n_tokens, float *out, void *stream);

/*
 * Several matvecs on one input in one launch: the attention projections of a
 * decode layer (Q, K, V and the output gate) read the same normed input and
 * write disjoint outputs, issued as one concurrent group (Ch 10 "The forward
 * pass at a glance", section 10.3, box 4 and fusion (e); Q [6656->4096],
 * K and V [6656->256], gate [6656->4096]).  For i < count and r < n_rows[i]:
 *   y[i][r] = sum_j w_i[r,j] * x[j],
 * with every matrix of weight type qtype and k inputs.  The input is staged
 * once per workgroup for all of them, and rows of all matrices are spread
 * over the GPU together, so a 256-row matrix in the group does not leave most
 * of the GPU idle.  Each y[i] equals, bit for bit, the single-matrix matvec
 * of that qtype on the same x launched with the same shape (the launch shape
 * follows the total row count, so it may differ from a lone call's, and the
 * result then agrees within the tolerance).
 *   qtype    KQ_QTYPE_Q4K, KQ_QTYPE_Q5K or KQ_QTYPE_Q6K.
 *   count    1 .. KQ_MAX_GROUP.
 *   W, y, n_rows  HOST arrays of `count` entries: device pointers to each
 *            matrix (alignment as for the matvec of qtype) and to its output
 *            [n_rows[i]] f32 (4-byte aligned), and the row counts (>= 0;
 *            their sum < 2^31).  A member with 0 rows is skipped; its W and
 *            y may be NULL.
 *   x        [k] f32, 16-byte aligned; k as for the matvecs.
 * No output may overlap an input or another output.
 * Errors as kq_matvec_q4k; count out of range is KQ_ERR_SHAPE.
 */
#define KQ_MAX_GROUP 4
kq_status kq_matvec_group(int qtype, int count, const void *const *W, float *const *y,
                          const int64_t *n_rows, const float *x, int64_t k, void *stream);

/*
 * kq_matvec_group on a staged input: xs = kq_staged_bytes(qtype, k) bytes,
 * 16-byte aligned (same results, bit for bit, as on the f32 vector the stage
 * was made from).
 */
kq_status kq_matvec_group_staged(int qtype, int count, const void *const *W, float *const *y,
                                 const int64_t *n_rows, const void *xs, int64_t k, void *stream);

/*
 * Q6_K decode matvec: y[r] = sum_i w[r,i] * x[i] for r < n_rows.
 *   W   [n_rows * (k/256) * 210] bytes, 4-byte aligned (a 210-byte superblock
 *       keeps only 2-byte alignment, and rows keep 4-byte alignment).
 *   x   [k] f32, 16-byte aligned.   y [n_rows] f32 output, 4-byte aligned,
 *       must not overlap W or x.
 *   n_rows >= 0, k multiple of 256 with 256 <= k <= KQ_MAX_K.
 * Errors as kq_matvec_q4k.
 */
kq_status kq_matvec_q6k(const void *W, const float *x, float *y, int64_t n_rows, int64_t k,
                        void *stream);

/*
 * Small-M matmul for the verify batch (Ch 36 "Prefill vs decode: the two
 * graphs", section 36.4 "Projections: from matvec to GEMM": each weight row is
 * read once and used for every input column; Ch 19 "The down projection +
 * residual", section 19.7, times M = 16): for m < M and r < n_rows,
 *   Y[m * ldy + r] = sum_i w[r,i] * X[m * ldx + i].
 * Each weight is read from memory once and applied to all M rows.  M = 1 runs
 * the matvec of that qtype (identical results).  Q4_K at M = 2 runs the
 * matvec's integer dot path on both rows (no workspace); other M >= 2 run the
 * matrix-core kernel, whose partial sums over ranges of k may pass through
 * `workspace` (kq_tune_set_small_m_rows moves the boundary).
 *   qtype   KQ_QTYPE_Q4K or KQ_QTYPE_Q6K.
 *   W       weight bytes as for the matvec of that qtype (same alignment).
 *   X       [M][ldx] f32, ldx >= k and ldx % 4 == 0, 16-byte aligned.
 *   Y       [M][ldy] f32 output, ldy >= n_rows, 4-byte aligned; must not
 *           overlap W, X or the workspace.
 *   n_rows  >= 0; k as for the matvec; 1 <= m <= KQ_MAX_M.
 *   workspace, workspace_bytes
 *           caller-owned device memory of at least
 *           kq_matmul_small_m_workspace_bytes(qtype, n_rows, k, m) bytes,
 *           256-byte aligned and zero-filled before its first use; every call
 *           leaves it zero-filled where it matters (its counters), so it can
 *           be reused without clearing.  May be NULL when that size is 0.
 *           Calls sharing a workspace must be ordered (same stream, or
 *           synchronised); concurrent calls need separate workspaces.
 * Results are deterministic for a given shape and device.
 * Errors as kq_matvec_q4k; a workspace that is too small is KQ_ERR_SHAPE.
 */
kq_status kq_matmul_small_m(int qtype, const void *W, const float *X, int64_t ldx, float *Y,
                            int64_t ldy, int64_t n_rows, int64_t k, int m, void *workspace,
                            int64_t workspace_bytes, void *stream);

/*
 * The FFN entry for the verify batch (Ch 10 "The forward pass at a glance",
 * section 10.3, box 11, for M rows: Ch 36 "Prefill vs decode", section 36.4):
 * for m < M and r < n_rows,
 *   Mid[m * ldm + r] = silu((W_gate X[m])[r]) * (W_up X[m])[r],
 * silu(z) = z / (1 + exp(-z)); both matrices Q4_K, n_rows x k.  M = 1 runs the
 * one-launch gate+up kernel (the result of kq_ffn_gate_up_q4k).  M = 2 and 3
 * run gate and up through the matvec's integer dot path in one launch, and
 * each row of Mid is then kq_ffn_gate_up_q4k of that row of X, bit for bit
 * (kq_tune_set_gate_up_rows moves this boundary).  Larger M run
 * kq_matmul_small_m twice (gate into Mid, then up with the SiLU product
 * applied as each output is stored), each within the kq_matmul_small_m
 * accuracy of its own matvec.
 *   X, ldx, m, workspace, workspace_bytes  as for kq_matmul_small_m with
 *          qtype KQ_QTYPE_Q4K (the same workspace size serves both launches;
 *          the one-launch dot path uses none).
 *   Mid    [M][ldm] f32 output, ldm >= n_rows, 4-byte aligned; must not
 *          overlap W_gate, W_up, X or the workspace.
 * A layer of the verify batch is this call, kq_matmul_small_m on Mid (the
 * down projection) and kq_fused_residual_norm over the M rows.
 * Errors as kq_matmul_small_m.
 */
kq_status kq_ffn_gate_up_q4k_small_m(const void *W_gate, const void *W_up, const float *X,
                                     int64_t ldx, float *Mid, int64_t ldm, int64_t n_rows,
                                     int64_t k, int m, void *workspace, int64_t workspace_bytes,
                                     void *stream);

/*
 * kq_matmul_small_m without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * kq_matmul_small_m (bit for bit: the same kernels on the same grid), except
 * that the partial tiles and counters of the split over k live in a
 * library-owned device array of KQ_SMALL_M_SCRATCH_BYTES (16 KiB of counters,
 * one per 256-row group, then 16 MiB of partial tiles), one per GPU, held
 * until the process ends.  The call allocates nothing.  Where
 * kq_matmul_small_m takes the matvec's dot path (Q4_K at M = 2 by default),
 * so does this call, and it uses none of the array.
 *   Returns KQ_ERR_UNSUPPORTED when the shape needs more than that array
 *   holds (more than 4096 row groups of 256 rows, or a split over more than
 *   512 workgroups; kq_matmul_small_m with a workspace takes any shape).
 *   KQ_ERR_DEVICE if the array's device address cannot be obtained.
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or different host threads without ordering)
 * race and may return wrong results; calls ordered on one stream do not.
 * The counters start at zero (cleared by the first call on each GPU that
 * needs them) and every completed call leaves them at zero.
 */
#define KQ_SMALL_M_SCRATCH_BYTES (16 * 1024 + 16 * 1024 * 1024)
kq_status kq_matmul_small_m_noalloc(int qtype, const void *W, const float *X, int64_t ldx,
                                    float *Y, int64_t ldy, int64_t n_rows, int64_t k, int m,
                                    void *stream);

/*
 * Workspace bytes kq_matmul_small_m needs for this shape on the current
 * device (0 if none), or a negative kq_status for arguments it would reject
 * (KQ_ERR_SHAPE, KQ_ERR_UNSUPPORTED, KQ_ERR_DEVICE).  Synchronous, no GPU work.
 */
int64_t kq_matmul_small_m_workspace_bytes(int qtype, int64_t n_rows, int64_t k, int m);

/*
 * Fused dual-epsilon residual tail, rows independent:
 *   residual[r] += rms_norm(projected[r], eps_post) * g_post
 *   next_in[r]   = rms_norm(residual[r], eps_next) * g_next
 * with rms_norm(v, eps)_i = v_i / sqrt(mean_j(v_j^2) + eps).  The second norm
 * sees the f32 residual after the add, which is also what is stored.
 *   residual   [rows][n] f32, updated in place, 16-byte aligned.
 *   projected  [rows][n] f32, 16-byte aligned.
 *   next_in    [rows][n] f32 output, 16-byte aligned; must not overlap
 *              residual, projected, g_post or g_next.
 *   g_post, g_next  [n] f32 gains shared by all rows, 16-byte aligned.
 *   rows >= 0; n % 4 == 0 with 4 <= n <= KQ_MAX_TAIL_N; eps >= 0 and finite.
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_ALIAS,
 * KQ_ERR_UNSUPPORTED, KQ_ERR_LAUNCH, KQ_ERR_DEVICE.
 */
kq_status kq_fused_residual_norm(float *residual, const float *projected, float *next_in,
                                 const float *g_post, const float *g_next, int64_t rows,
                                 int64_t n, float eps_post, float eps_next, void *stream);

/*
 * Staged activations.  Every matvec workgroup converts its f32 input into a
 * block-floating-point form in on-chip memory before the weight stream: per
 * scale group (32 inputs for a Q4_K consumer, 16 for Q6_K) a power-of-two
 * scale and the group sum, and each input as KQ_STAGED_LIMBS signed byte
 * limbs.  A producer that already holds the values can write that form once
 * (a "staged" vector), and every consumer workgroup then copies it instead of
 * converting x again.  This fuses dispatches without moving a rounding point
 * (Ch 19 "The down projection + residual", section 19.7): a matvec on a
 * staged vector returns bit for bit what it returns on the f32 vector the
 * stage was made from.  The layout is internal to this library: KQ_STAGED_LIMBS
 * byte planes of k + k/8 bytes (the inputs in order, 16 bytes of padding after
 * every 128, so that lanes reading units 128 inputs apart use different LDS
 * banks), then k/G f32 scales, then k/G f32 group sums.
 *
 * kq_staged_bytes: bytes of the staged form of a k-vector for a consumer of
 * weight type qtype (KQ_QTYPE_Q4K or KQ_QTYPE_Q6K); k as for the matvecs.
 * Returns the size (> 0), or a negative kq_status for a bad qtype or k.
 */
int64_t kq_staged_bytes(int qtype, int64_t k);

/*
 * Staged form of x for a consumer of type qtype.
 *   x   [k] f32, 16-byte aligned; k as for the matvecs.
 *   xs  kq_staged_bytes(qtype, k) bytes output, 16-byte aligned, must not
 *       overlap x.
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_ALIAS,
 * KQ_ERR_UNSUPPORTED, KQ_ERR_LAUNCH, KQ_ERR_DEVICE.
 */
kq_status kq_stage_activation(int qtype, const float *x, void *xs, int64_t k, void *stream);

/*
 * kq_matvec_q4k / kq_matvec_q6k on a staged input (same results, bit for bit,
 * as on the f32 vector the stage was made from).
 *   qtype      weight type of W; xs must have been staged for that type.
 *   W, y, n_rows, k, silu_gate  as for the matvec of that type (silu_gate
 *              only for Q4_K: KQ_ERR_UNSUPPORTED otherwise).
 *   xs         kq_staged_bytes(qtype, k) bytes, 16-byte aligned; y must not
 *              overlap it.
 * Errors as kq_matvec_q4k.
 */
kq_status kq_matvec_staged(int qtype, const void *W, const void *xs, float *y, int64_t n_rows,
                           int64_t k, const float *silu_gate, void *stream);

/*
 * kq_ffn_gate_up_q4k on a staged input (xs, staged for Q4_K), optionally also
 * writing mid in staged form for the next matvec (the down projection,
 * Ch 10 section 10.3, weight type mid_qtype).
 *   xs     kq_staged_bytes(KQ_QTYPE_Q4K, k) bytes, 16-byte aligned.
 *   mid    [n_rows] f32 output, as for kq_ffn_gate_up_q4k.
 *   mid_s  NULL, or kq_staged_bytes(mid_qtype, n_rows) bytes output, 16-byte
 *          aligned; then n_rows must be a multiple of 256 (it is the next
 *          matvec's k).  No output may overlap an input or the other output.
 * Errors as kq_matvec_q4k.
 */
kq_status kq_ffn_gate_up_q4k_staged(const void *W_gate, const void *W_up, const void *xs,
                                    float *mid, void *mid_s, int mid_qtype, int64_t n_rows,
                                    int64_t k, void *stream);

/*
 * One layer boundary in one launch: the previous layer's dual-eps tail
 * (Ch 19 "The down projection + residual", section 19.3) followed by this
 * layer's gate, up and SiLU product (Ch 10 "The forward pass at a glance",
 * section 10.3: the tail's second output is the next layer's input):
 *   residual_out = residual_in + rms_norm(projected, eps_post) * g_post
 *   x            = rms_norm(residual_out, eps_next) * g_next
 *   next_in      = x                                  (if next_in != NULL)
 *   mid[r]       = silu((W_gate x)[r]) * (W_up x)[r]  for r < n_rows
 *   mid_s        = staged form of mid for a consumer of mid_qtype (if non-NULL)
 * x has k elements (the tail's row width is the gate and up matrices' k).
 * Every workgroup runs the tail itself, in the order of kq_fused_residual_norm,
 * so residual_out, next_in and mid equal, bit for bit, kq_fused_residual_norm
 * followed by kq_ffn_gate_up_q4k.
 *   residual_in, projected, g_post, g_next  [k] f32, 16-byte aligned.
 *   residual_out  [k] f32 output, 16-byte aligned; must not overlap
 *                 residual_in (every workgroup reads it while one writes).
 *   next_in       NULL or [k] f32 output, 16-byte aligned.
 *   W_gate, W_up, mid, mid_s, mid_qtype  as for kq_ffn_gate_up_q4k_staged.
 *   n_rows        >= 1 (the tail's outputs need a launch), < 2^31.
 *   k             multiple of 256, <= KQ_MAX_FUSED_TAIL_K.
 *   eps_post, eps_next  >= 0 and finite.
 * No output may overlap an input or another output.
 * Errors as kq_matvec_q4k.
 */
kq_status kq_ffn_tail_gate_up_q4k(const float *residual_in, const float *projected,
                                  const float *g_post, const float *g_next, float *residual_out,
                                  float *next_in, const void *W_gate, const void *W_up, float *mid,
                                  void *mid_s, int mid_qtype, int64_t n_rows, int64_t k,
                                  float eps_post, float eps_next, void *stream);

/*
 * The decode FFN pass of a whole layer stack in one call (Ch 10 "The forward
 * pass at a glance", section 10.3: each layer's SiLU-gated FFN on the normed
 * input, then the tail, whose second output is the next layer's input;
 * Ch 19 "The down projection + residual", sections 19.1 and 19.4).  From the
 * residual r_0, for l = 0 .. n_layers-1:
 *   x_0     = rms_norm(r_0, eps_next) * g_entry      (unit gain if g_entry is NULL)
 *   mid_l   = silu(W_gate[l] x_l) * (W_up[l] x_l)    (Q4_K, ffn x hidden)
 *   p_l     = W_down[l] mid_l                        (Q6_K, hidden x ffn)
 *   r_{l+1} = r_l + rms_norm(p_l, eps_post) * g_post[l]
 *   x_{l+1} = rms_norm(r_{l+1}, eps_next) * g_next[l]
 * and residual <- r_L, x_out <- x_L.  rms_norm(v, eps) = v / sqrt(mean(v^2) + eps).
 * It enqueues two launches per layer and one more: kq_ffn_tail_gate_up_q4k
 * (layer l's gate, up and SiLU with layer l-1's tail in front; layer 0's
 * tail is the entry norm) writing mid staged for Q6_K, then kq_matvec_staged
 * on the Q6_K down matrix; then the last kq_fused_residual_norm.  Results
 * equal those calls made one by one, bit for bit.
 *   layers     HOST array of n_layers kq_ffn_layer records holding device
 *              pointers: W_gate and W_up (Q4_K [ffn][hidden], 16-byte
 *              aligned), W_down (Q6_K [hidden][ffn], 4-byte aligned), g_post
 *              and g_next ([hidden] f32, 16-byte aligned).  Read during the
 *              call only.
 *   n_layers   >= 1.
 *   residual   [hidden] f32, 16-byte aligned: r_0 in, r_L out.
 *   x_out      [hidden] f32 output, 16-byte aligned.
 *   g_entry    NULL or [hidden] f32, 16-byte aligned.
 *   workspace, workspace_bytes
 *              caller-owned device memory of at least
 *              kq_ffn_pass_workspace_bytes(hidden, ffn) bytes, 256-byte
 *              aligned, for the relay buffers (the residual's second buffer,
 *              the down output, mid and its staged form); no initial contents
 *              needed.
 *              Calls sharing a workspace must be ordered.
 *   hidden     multiple of 256, <= KQ_MAX_FUSED_TAIL_K.
 *   ffn        multiple of 256, <= KQ_MAX_K.
 *   eps_post, eps_next  >= 0 and finite.
 * No output (residual, x_out, workspace) may overlap another argument's
 * buffer (weights, gains, g_entry, or another output).
 * Errors as kq_ffn_tail_gate_up_q4k; a workspace that is too small is
 * KQ_ERR_SHAPE.
 */
typedef struct kq_ffn_layer {
    const void *W_gate, *W_up, *W_down;
    const float *g_post, *g_next;
} kq_ffn_layer;

kq_status kq_ffn_pass_q4k_q6k(const kq_ffn_layer *layers, int n_layers, float *residual,
                              float *x_out, const float *g_entry, void *workspace,
                              int64_t workspace_bytes, int64_t hidden, int64_t ffn,
                              float eps_post, float eps_next, void *stream);

/*
 * Workspace bytes kq_ffn_pass_q4k_q6k needs, or a negative kq_status for
 * shapes it would reject.  Host arithmetic only.
 */
int64_t kq_ffn_pass_workspace_bytes(int64_t hidden, int64_t ffn);

/*
 * kq_fused_residual_norm that also writes next_in in staged form, for a
 * consumer of type next_qtype (the next layer's gate and up: Q4_K).
 *   next_in_s  rows * kq_staged_bytes(next_qtype, n) bytes output (row r at
 *              r * kq_staged_bytes(next_qtype, n)), 16-byte aligned, must not
 *              overlap any other argument.
 *   n          multiple of 256 (it is the next matvec's k), <= KQ_MAX_TAIL_N.
 *   The other arguments and the f32 outputs as for kq_fused_residual_norm.
 * Errors as kq_fused_residual_norm.
 */
kq_status kq_fused_residual_norm_staged(float *residual, const float *projected, float *next_in,
                                        void *next_in_s, int next_qtype, const float *g_post,
                                        const float *g_next, int64_t rows, int64_t n,
                                        float eps_post, float eps_next, void *stream);

/* Static text for a status code (never NULL). */
const char *kq_status_string(kq_status s);

/* Static text naming the build: kernel variants, gfx target, HIP version. */
const char *kq_build_info(void);

/*
 * Name of the HIP error behind the last KQ_ERR_LAUNCH returned to the
 * calling thread ("hipSuccess" if there was none): the detail the status
 * code does not carry.  The string is static.
 */
const char *kq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
