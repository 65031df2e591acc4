/*
 * gq.h — C ABI of libgq.so: grouped Fisher accumulation (GuidedQuant) and the
 * LNQ alternating optimisation on one AMD Instinct MI355X (gfx950).
 *
 * Sources (the "GuidedQuant" blog page, jinukkim.me/blog/guidedquant):
 *   - GuidedQuant objective equation: || dl/dZ (.) (XW - XW_hat) ||_F^2
 *     = n sum_j (w_j - w_hat_j)^T F_j (w_j - w_hat_j), with block-diagonal
 *     Fisher blocks F_j that are grouped and averaged within each group.
 *   - Section "LNQ": per-row problem over a one-hot assignment P^(j)
 *     (P 1_m = 1) and a codebook c^(j) in R^m; the algorithm box alternates
 *     "(codebook)" c <- (P^T F P)^{-1} P^T F w and "(assignment)" over
 *     i = 1..d_in, each coordinate taking the codebook entry that minimises
 *     (w_hat - w)^T F (w_hat - w).
 *
 * Conventions shared by every entry point
 *   Layout.   Row-major, contiguous.  X [n][d_in] (calibration activations,
 *             one token per row), G [n][d_out] (end-loss gradients dl/dZ),
 *             W [d_out][d_in] (row j is the page's column w_j), F
 *             [groups][d_in][d_in] float32 symmetric, C [d_out][m] float32,
 *             P [d_out][d_in] uint8 codes in [0, m).  m = 2^bits.
 *   Groups.   Output channel j belongs to group j / (d_out / groups); groups
 *             are contiguous equal blocks (d_out % groups == 0).
 *   F_g.      X^T diag(s_g) X with s_g[t] = mean_{j in g} G[t, j]^2 (the
 *             1/n of the objective equation is not applied; LNQ does not
 *             depend on the scale of F).
 *   Damping.  Every LNQ call works with F'_g = F_g + lambda_g I,
 *             lambda_g = ridge_rel * mean(diag F_g) (+ ridge_abs, see
 *             gq_lnq_options), formed on the fly.
 *   Memory.   Every array argument is a device pointer (HIP global memory)
 *             unless stated otherwise.  The caller owns all buffers; the
 *             library keeps no pointer after a call returns.
 *   Alignment. X, G, W, F and P must be 16-byte aligned, ws 256-byte aligned
 *             (GQ_EINVAL otherwise).  F must be exactly symmetric, as
 *             gq_fisher_accumulate writes it.
 *   Workspace. ws/ws_bytes is caller-owned device scratch of at least the
 *             size the matching *_workspace_size() returns.  ws == NULL asks
 *             the library to allocate it stream-ordered (hipMallocAsync /
 *             hipFreeAsync on `stream`).
 *   Streams.  `stream` is a hipStream_t (NULL = default stream).  Calls only
 *             enqueue work; outputs are valid once the stream is synchronised.
 *             Calls on one stream are ordered.  A checked call (check_finite,
 *             GQ_FISHER_CHECK_FINITE) synchronises its stream before returning.
 *   State.    Calls on different streams may run concurrently: the library's
 *             only state shared between calls is (a) the cache of kernel LDS
 *             limits already raised on each device (set once, under a lock),
 *             (b) the per-stage timing record (diagnostics, off unless
 *             gq_timing_enable is called; its marks are kept per stream), (c)
 *             the per-device scratch array of lnq_quantize_static, and the
 *             thread-local error string.
 *   Errors.   Arguments are validated before anything is enqueued; on a
 *             non-OK status no output has been touched and gq_last_error()
 *             (thread-local) says why.  GQ_EHIP reports a failed HIP call.
 *             The one exception is GQ_ENOTPD from a checked call: the run has
 *             completed and its outputs are written (see gq_lnq_options).
 *   Precision. Fisher: bfloat16 inputs, MFMA with float32 accumulation; the
 *             gradient-square scale is applied to one operand, rounded to
 *             bfloat16.  float32 inputs take a float64-accumulating path.
 *             LNQ: F' is split into bfloat16 planes (hi + lo) for the matrix
 *             cores, residuals and codebook systems are accumulated in
 *             float32, the m x m solve and all objectives are float64.
 */
#ifndef GQ_H
#define GQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQ_ABI_VERSION 8

typedef enum {
    GQ_OK = 0,
    GQ_EINVAL = 1,    /* bad argument value (null pointer, bits, block, iters, workspace too small) */
    GQ_ESHAPE = 2,    /* inconsistent sizes (d_out % groups, d_in % 32 or 64, empty shapes) */
    GQ_EDTYPE = 3,    /* unsupported dtype code */
    GQ_ENOMEM = 4,    /* library-side workspace allocation failed */
    GQ_EHIP = 5,      /* a HIP runtime call or kernel launch failed */
    GQ_ENOTPD = 6,    /* checked call: some codebook system P^T F' P (or GANQ's F') was not
                         positive definite, so the closed form of the "(codebook)" step (or the
                         Cholesky factor) does not exist there; those rows kept their codebook
                         (codes).  Outputs are written. */
    GQ_ENONFINITE = 7, /* checked call: an input holds NaN or +-Inf; nothing was written */
    GQ_ENOTIMPL = 8,  /* valid request outside what the library supports */
    GQ_ECHECK = 9     /* debug check (option check_residual) failed: an assignment pass's
                         running residual disagreed with a fresh F'(C[P] - W); outputs are
                         written, but they come from a faulty pass */
} gq_status;

typedef enum { GQ_F32 = 0, GQ_BF16 = 1 } gq_dtype;

typedef enum { GQ_INIT_QUANTILE = 0, GQ_INIT_GIVEN = 1, GQ_INIT_UNIFORM = 2 } gq_lnq_init;

typedef enum { GQ_GRAM_AUTO = 0, GQ_GRAM_DENSE = 1 } gq_gram_update;

typedef struct {
    int32_t block;      /* assignment block B: 64, 128, 256 or 512 coordinates.  Inside a block
                           the pass decides 64 coordinates at a time exactly in registers (one per
                           lane of a 64-wide wavefront) and carries their moves to the block's
                           later coordinates on the matrix cores; at the end of a block the
                           deferred update R[:, later] += Delta_B F'[B, later] of all its moves is
                           pushed into the residual array on the matrix cores.  B changes only
                           the float32 summation order, never the order in which coordinates
                           are visited or the tie rule.  d_in must be a multiple of 64 (the
                           last block may be shorter than B).  Default 512. */
    float ridge_rel;    /* rho in lambda_g = rho * mean(diag F_g) + ridge_abs: the relative
                           ("adaptive") ridge, scaling with F.  Default 1e-6. */
    int32_t init;       /* gq_lnq_init.  QUANTILE: c_j = m quantiles of w_j at levels
                           (q + 1/2)/m (linear interpolation between order statistics),
                           codes = nearest entry (lowest index on ties).  UNIFORM: the
                           row's uniform grid c_q = lo + q (hi - lo)/(m - 1), lo and hi the
                           row's minimum and maximum, formed in float64 and stored float32,
                           codes = nearest entry (lowest index on ties).  GIVEN: start from
                           the C and P passed in.  Default QUANTILE (grid_quantize: UNIFORM
                           when opt is NULL; it rejects QUANTILE). */
    int32_t gram_update; /* gq_gram_update: how each codebook step after the first obtains
                           A_j = P_j^T F' P_j and the residual F'(C[P] - W).  DENSE:
                           recomputed from scratch on the matrix cores.  AUTO: when the
                           previous assignment pass changed at most a set share of the
                           codes (see lnq_quantize), updated from the changed coordinates
                           only (equal up to float rounding), else recomputed.
                           Default AUTO. */
    float ridge_abs;    /* fixed ridge added to lambda_g whatever F is (ridge_rel = 0 and
                           ridge_abs = lambda is the fixed-lambda preconditioning of the GANQ
                           summary page's ablation).  Finite, >= 0.  Default 0. */
    int32_t check_finite; /* 1: a checked call.  Before anything is written, W and F are
                           scanned for NaN and +-Inf (GQ_ENONFINITE if any, outputs
                           untouched); after the run, GQ_ENOTPD if any codebook system (GANQ:
                           any group's F') was not positive definite.  The call synchronises
                           its stream.  0: no data checks, fully asynchronous.  Default 0. */
    int32_t check_residual; /* 1: debug check of the coordinate-descent pass (lnq_quantize,
                           grid_quantize; GQ_EINVAL for ganq_quantize and
                           lnq_quantize_static).  The pass decides every coordinate from a
                           running residual r = F'(w_hat - w) that it updates move by move;
                           after each pass, every row's objective is recomputed from scratch
                           with a residual array of its own and compared with the objective
                           the pass reached through r (its start plus the accepted changes).
                           Rows differing by more than 1e-4 of their objective at the pass
                           start are counted, and the call returns GQ_ECHECK if there are any.
                           Costs one residual product per pass and d_out * d_in * 4 + d_out * 8
                           bytes allocated stream-ordered for the call; the run's results are
                           unchanged; the call synchronises its stream.  Default 0. */
} gq_lnq_options;

/* The options under the name the problem statement uses. */
typedef gq_lnq_options lnq_options;

/* ABI version of the loaded library (GQ_ABI_VERSION). */
int gq_abi_version(void);

/* Message for the most recent non-OK status on this thread ("" if none).
   Owned by the library; valid until the next call on this thread. */
const char* gq_last_error(void);

/* Fills *opt with the defaults listed in gq_lnq_options.  opt: host pointer.
   lnq_options_default is the same function under the problem statement's name. */
void gq_lnq_options_default(gq_lnq_options* opt);
void lnq_options_default(lnq_options* opt);

/* Workspace bytes gq_fisher_accumulate needs for these sizes. */
size_t gq_fisher_workspace_size(int64_t n, int64_t d_in, int64_t d_out, int32_t groups,
                                gq_dtype x_dt);

/*
 * Grouped Fisher blocks (GuidedQuant objective equation and the grouping
 * sentence after it):  F[g] (=|+=) X^T diag(s_g) X,
 *   s_g[t] = (1/|g|) sum_{j in g} G[t, j]^2.
 * X [n][d_in] of dtype x_dt, G [n][d_out] of dtype g_dt, F [groups][d_in][d_in]
 * float32 output; accumulate = 0 overwrites F, 1 adds to it (token chunks can be
 * streamed through repeated calls, F being a sum over tokens).  OR-ing
 * GQ_FISHER_CHECK_FINITE into `accumulate` makes the call checked: X and G are
 * scanned for NaN and +-Inf first (GQ_ENONFINITE, F untouched) and the call
 * synchronises its stream.  The result is exactly symmetric (the upper triangle is
 * computed and mirrored).
 * Requires n >= 1, d_in >= 1, d_out >= 1, 1 <= groups, d_out % groups == 0,
 * x_dt == g_dt.
 */
#define GQ_FISHER_CHECK_FINITE 2
gq_status gq_fisher_accumulate(const void* X, gq_dtype x_dt, int64_t n, int64_t d_in,
                               const void* G, gq_dtype g_dt, int64_t d_out, int32_t groups,
                               float* F, int32_t accumulate,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * The grouped Fisher of gq_fisher_accumulate for calibration data held in host
 * memory (a token count beyond what device memory holds): X [n][d_in] and
 * G [n][d_out] are HOST pointers (pinned, e.g. hipHostMalloc, for the copies to
 * run asynchronously; pageable memory works but each copy then blocks the
 * caller).  The tokens are taken in chunks of chunk_tokens (the last may be
 * shorter); each chunk is copied to device memory on a library-created copy
 * stream while the previous chunk's Fisher runs on `stream`, and every chunk adds
 * into F (the first with `accumulate`).  Since F is a sum over tokens, the result
 * is the Fisher of all n tokens, with float32 sums of the per-chunk partials.
 * F, ws: device memory; ws of at least gq_fisher_stream_workspace_size(chunk_tokens
 * or n if smaller, ...) bytes (NULL: allocated stream-ordered).  The host arrays
 * must stay valid and unchanged until `stream` has passed this call's work.
 */
size_t gq_fisher_stream_workspace_size(int64_t chunk_tokens, int64_t d_in, int64_t d_out,
                                       int32_t groups, gq_dtype x_dt);
gq_status gq_fisher_accumulate_host(const void* X_host, gq_dtype x_dt, int64_t n, int64_t d_in,
                                    const void* G_host, gq_dtype g_dt, int64_t d_out,
                                    int32_t groups, float* F, int32_t accumulate,
                                    int64_t chunk_tokens, void* ws, size_t ws_bytes,
                                    void* stream);

/* Workspace bytes every lnq_* call below needs for these sizes and W dtype
   (lnq_workspace_size: the same function under the problem statement's name). */
size_t gq_lnq_workspace_size(int64_t d_out, int64_t d_in, int32_t groups, int32_t bits,
                             gq_dtype w_dt);
size_t lnq_workspace_size(int64_t d_out, int64_t d_in, int32_t groups, int32_t bits,
                          gq_dtype w_dt);

/*
 * One "(codebook)" step of the LNQ algorithm box for every row j:
 *   c_j <- (P_j^T F' P_j)^{-1} P_j^T F' w_j   on the codes that own at least one
 * coordinate; codes that own none keep their value.  F' = F_g(j) + lambda I.
 * F [groups][d_in][d_in], W [d_out][d_in] (w_dt), P [d_out][d_in] (read),
 * C [d_out][m] (read, then overwritten).  A row whose m x m system is not
 * positive definite keeps its codebook and is counted in *n_not_pd (device
 * int64, may be NULL; incremented, not reset).  This happens for every row of a
 * group whose Fisher is zero (all its output gradients vanish, so lambda = 0 and
 * F' = 0), and can happen with ridge_rel == 0.
 * Shape limits shared by every lnq_* call: 1 <= bits <= 4, d_out % groups == 0,
 * d_in % 32 == 0, 32 <= d_in <= 32768, ridge_rel finite and >= 0 (GQ_EINVAL /
 * GQ_ESHAPE otherwise); the assignment pass (lnq_assign_sweep, lnq_quantize,
 * grid_quantize) and ganq_* also need d_in % 64 == 0.  bits 5..8 (codebooks of
 * 32..256 entries, which the uint8 codes could hold) are valid requests that this
 * library does not build: GQ_ENOTIMPL (bits outside 1..8: GQ_EINVAL).  The pages'
 * LNQ runs use 2..4 bits; larger codebooks would grow the Gram partials as m^2 and
 * exceed the one-row-per-lane solve at m > 64.
 */
gq_status lnq_codebook_update(const float* F, int32_t groups, int64_t d_in,
                              const void* W, gq_dtype w_dt, int64_t d_out,
                              const uint8_t* P, int32_t bits, float* C, float ridge_rel,
                              int64_t* n_not_pd, void* ws, size_t ws_bytes, void* stream);

/*
 * One "(assignment)" pass of the LNQ algorithm box for every row j: for
 * i = 0..d_in-1 in ascending order, coordinate i takes the codebook entry
 * that minimises (w_hat - w)^T F' (w_hat - w) with every other coordinate
 * fixed; the current entry is kept unless another strictly lowers the
 * objective, and among equal minimisers the lowest index wins.
 * P [d_out][d_in] is read and overwritten; C [d_out][m] is read.  The number of
 * coordinates that changed is added to *n_changed (device int64, may be NULL).
 * block: as gq_lnq_options.block (64, 128, 256 or 512).
 */
gq_status lnq_assign_sweep(const float* F, int32_t groups, int64_t d_in,
                           const void* W, gq_dtype w_dt, int64_t d_out,
                           const float* C, int32_t bits, uint8_t* P, float ridge_rel,
                           int32_t block, int64_t* n_changed,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Per-row objective (LNQ problem statement with F' in place of X^T X, i.e.
 * the GuidedQuant objective of the row):  obj_rows[j] = e_j^T F' e_j,
 * e_j = C[j][P[j]] - w_j, as float64 (device, [d_out]).  obj_total (device
 * float64, may be NULL) receives sum_j obj_rows[j].
 */
gq_status lnq_objective(const float* F, int32_t groups, int64_t d_in,
                        const void* W, gq_dtype w_dt, int64_t d_out,
                        const float* C, const uint8_t* P, int32_t bits, float ridge_rel,
                        double* obj_rows, double* obj_total,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Whole LNQ on a layer: initialise (opt->init), then `iters` times
 * (codebook step, assignment pass), as in the LNQ algorithm box.
 * W [d_out][d_in] (w_dt), F [groups][d_in][d_in]; C [d_out][2^bits] and
 * P [d_out][d_in] are outputs (inputs too when opt->init == GQ_INIT_GIVEN).
 * obj_trace (device float64 [2*iters+1], may be NULL): layer objective
 * sum_j e_j^T F' e_j at the start and after every half-step, from the residual
 * F'(C[P] - W) each step uses: recomputed from (C, P), except that under
 * GQ_GRAM_AUTO the entry before a codebook step that follows a pass with at most
 * d_out * d_in * (2^bits + 3) * 17 / 10000 changes comes from the residual updated
 * by the changed coordinates (equal up to float rounding).  The last entry is
 * always recomputed.  n_changed (device int64 [iters], may be NULL): coordinates
 * changed by each assignment pass (overwritten).
 * opt == NULL means the defaults.  Requires 1 <= bits <= 4, iters >= 0.
 */
gq_status lnq_quantize(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in,
                       const float* F, int32_t groups, int32_t bits, int32_t iters,
                       const gq_lnq_options* opt, float* C, uint8_t* P,
                       double* obj_trace, int64_t* n_changed,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * lnq_quantize for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * results as lnq_quantize without ws / ws_bytes: the call's scratch is a fixed array of
 * GQ_STATIC_SCRATCH_BYTES (64 MiB) per device inside the library (lnq_static_scratch_bytes
 * returns it), held until the process ends, and the call itself allocates nothing.
 * Layers whose gq_lnq_workspace_size exceeds it (e.g. beyond about 1536 x 1536 with
 * m = 8) get GQ_ENOTIMPL before anything is enqueued.  Every call on one device shares
 * that device's array, which keeps the previous call's contents (each call initialises
 * what it reads): calls that overlap on one device, on any streams, race and corrupt
 * each other's results, so serialise them.
 */
#define GQ_STATIC_SCRATCH_BYTES (64u << 20)
size_t lnq_static_scratch_bytes(void);
gq_status lnq_quantize_static(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in,
                              const float* F, int32_t groups, int32_t bits, int32_t iters,
                              const gq_lnq_options* opt, float* C, uint8_t* P,
                              double* obj_trace, int64_t* n_changed, void* stream);

/*
 * Fixed-grid scalar backend with the GuidedQuant objective.  The blog page says
 * its objective can be used by any layer-wise quantizer; this entry point is
 * the plainest such backend: each row keeps a fixed uniform grid (opt->init ==
 * GQ_INIT_UNIFORM, the min-max grid described under gq_lnq_options.init, or
 * GQ_INIT_GIVEN: the C and P passed in) and only the "(assignment)" pass of the
 * LNQ algorithm box is run, `iters` times; there is no codebook step.
 * Arguments as for lnq_quantize: W [d_out][d_in] (w_dt), F [groups][d_in][d_in];
 * C [d_out][2^bits] and P [d_out][d_in] outputs (inputs too under GIVEN).
 * obj_trace (device float64 [iters+1], may be NULL): layer objective
 * sum_j e_j^T F' e_j before each pass and after the last, each recomputed
 * from (C, P); it never increases.  n_changed (device int64 [iters], may be
 * NULL): coordinates changed by each pass (overwritten).  opt == NULL means the
 * defaults with init UNIFORM; opt->gram_update is ignored.  Requires
 * 1 <= bits <= 4, iters >= 0; GQ_EINVAL for init == GQ_INIT_QUANTILE.  Workspace:
 * gq_lnq_workspace_size.
 */
gq_status grid_quantize(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in,
                        const float* F, int32_t groups, int32_t bits, int32_t iters,
                        const gq_lnq_options* opt, float* C, uint8_t* P,
                        double* obj_trace, int64_t* n_changed,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Lookup-table dequantisation product for the (C, P) format.  Section "LNQ" of
 * the blog page keeps per row j a codebook c^(j) and b-bit indices P^(j), and
 * notes that the result runs on the same lookup-table kernel as SqueezeLLM; the
 * product is y[b][j] = sum_i c^(j)[P[j][i]] x[b][i].
 *
 * Packed layout (this library's own; the pages fix none): codes are taken in
 * pairs (i, i + 1), a pair being the 2b-bit index code_i | code_{i+1} << b; a
 * 32-bit word holds 16 / b pairs (integer division), the first pair in the low
 * bits, i.e. 32, 16, 10 or 8 codes per word for b = 1, 2, 3, 4; each row is
 * lut_packed_row_words(d_in, bits) words (a multiple of 4), code slots past
 * d_in are 0.  lut_packed_row_words returns 0 for d_in < 1 or bits outside 1..4.
 */
int64_t lut_packed_row_words(int64_t d_in, int32_t bits);

/*
 * P [d_out][d_in] uint8 codes (each taken modulo 2^bits) -> Q [d_out][row words]
 * uint32 in the layout above.  Q 16-byte aligned.  1 <= bits <= 4.
 */
gq_status lut_pack_codes(const uint8_t* P, int64_t d_out, int64_t d_in, int32_t bits,
                         uint32_t* Q, void* stream);

/*
 * y [batch][d_out] float32 = the product above for x [batch][d_in] (x_dt),
 * 1 <= batch <= 8, Q from lut_pack_codes, C [d_out][2^bits] float32.
 * bfloat16 x: the codebook enters as bfloat16 (rounded to nearest even, as a
 * 16-bit lookup table holds it), each product of two bfloat16 values is exact
 * and the sums are float32.  The activations are staged in LDS, a whole row's worth
 * when it fits, else in segments of a multiple of 512 packed words; one chunk of them
 * must fit: batch * (min(row words, 512) + 1) * X * 4 + 8 * 4^bits * 4 <= 160 KiB with
 * X = 16 / bits for bits 1, 2, 4 and X = 5 for bits 3, else GQ_ENOTIMPL.  With segments
 * each output is the float32 sum of the segments' sums.  float32 x: float32 codebook and
 * float32 fused multiply-adds.
 */
gq_status lut_gemv(const uint32_t* Q, const float* C, int64_t d_out, int64_t d_in, int32_t bits,
                   const void* x, gq_dtype x_dt, int32_t batch, float* y, void* stream);

/*
 * GANQ-style alternation.  The GANQ summary page ("Approach") solves each row by
 * alternating a closed-form least-squares codebook update with an assignment of
 * the indices by Cholesky / back-substitution.  Here: F'_g = L L^T (float64
 * factorization on the GPU); the row objective is ||L^T e||^2 with
 * e = w_hat - w, and the assignment visits j = d_in - 1 down to 0, giving
 * coordinate j the codebook entry nearest to w_j - s_j / L_jj,
 * s_j = sum_{k>j} L_kj e_k (lowest index on ties; the targets are float32).  The
 * codebook step is LNQ's (lnq_codebook_update).  Unlike LNQ's coordinate pass,
 * the assignment does not start from the current codes and need not lower the
 * objective.
 *
 * ganq_quantize: init as opt->init (QUANTILE, UNIFORM or GIVEN), then `iters`
 * times (codebook step, assignment).  Arguments as for lnq_quantize; obj_trace
 * [2*iters+1] holds the objective before and after every half-step, each
 * recomputed from (C, P).  not_pd (device int32 [groups], may be NULL): 1 where
 * F'_g has a non-positive pivot (e.g. all-zero gradients with ridge 0); those
 * groups keep their codes through every assignment.  opt->gram_update is
 * ignored.  Requires d_in % 64 == 0, 1 <= bits <= 4.  Workspace:
 * ganq_workspace_size (the LNQ workspace plus groups * d_in^2 * 8 bytes for the
 * float64 factor and the bf16 planes of L^T).
 *
 * ganq_factor_damped: the factor alone, L [groups][d_in][d_in] float32 (lower
 * triangle, zeros above) of F'_g = F_g + ridge_rel * mean(diag F_g) I, and the
 * not_pd flags (may be NULL).  Workspace: ganq_workspace_size(groups, d_in,
 * groups, 1, ...).
 */
size_t ganq_workspace_size(int64_t d_out, int64_t d_in, int32_t groups, int32_t bits,
                           gq_dtype w_dt);
gq_status ganq_quantize(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in,
                        const float* F, int32_t groups, int32_t bits, int32_t iters,
                        const gq_lnq_options* opt, float* C, uint8_t* P,
                        double* obj_trace, int64_t* n_changed, int32_t* not_pd,
                        void* ws, size_t ws_bytes, void* stream);
gq_status ganq_factor_damped(const float* F, int32_t groups, int64_t d_in, float ridge_rel,
                             float* L, int32_t* not_pd, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * Diagnostics: per-stage kernel timing with HIP events.
 * gq_timing_enable(mask) makes every later call bracket each launch sequence of
 * the stages whose bit (1 << gq_stage) is set in `mask` with two events recorded
 * on the call's stream (events are created on first use and kept in a pool);
 * mask 0 turns timing off, -1 times every stage.  gq_timing_read synchronises
 * the recorded events, writes the summed milliseconds and the number of timed
 * launch sequences per stage into ms[GQ_STAGE_COUNT] and
 * launches[GQ_STAGE_COUNT] (host arrays), and clears the record.  Each timed
 * stage boundary adds one event record to the stream; results of the
 * computation do not change.  GQ_EHIP if an event call failed.
 */
typedef enum {
    GQ_STAGE_GROUP_SCALE = 0,   /* s_g from G */
    GQ_STAGE_FISHER_MFMA,       /* the matrix-core Fisher contraction */
    GQ_STAGE_FISHER_FINALIZE,   /* split-K sum + mirror write of F */
    GQ_STAGE_FISHER_PLAIN,      /* float32-input Fisher */
    GQ_STAGE_LNQ_PREPARE,       /* ridge and F' planes */
    GQ_STAGE_LNQ_RESID,         /* residual R = F'(C[P] - W) on the matrix cores */
    GQ_STAGE_LNQ_INIT,          /* quantile codebooks and nearest codes */
    GQ_STAGE_LNQ_GRAM,          /* P_j^T F' P_j on the matrix cores */
    GQ_STAGE_LNQ_SOLVE,         /* codebook solves and row objectives */
    GQ_STAGE_LNQ_SWEEP,         /* the assignment pass */
    GQ_STAGE_LNQ_SMALL,         /* sums and counters */
    GQ_STAGE_FISHER_PACK,       /* feature-major bf16 operands of the Fisher contraction */
    GQ_STAGE_LNQ_DELTA,         /* Gram and residual updates from the changed coordinates */
    GQ_STAGE_LUT_PACK,          /* code packing for the lookup-table product */
    GQ_STAGE_LUT_GEMV,          /* the lookup-table product */
    GQ_STAGE_FISHER_H2D,        /* host-to-device copies of the streamed Fisher (copy stream) */
    GQ_STAGE_GANQ_CHOL,         /* Cholesky factor of F' for the back-substitution assignment */
    GQ_STAGE_GANQ_PASS,         /* the back-substitution assignment */
    GQ_STAGE_COUNT
} gq_stage;

void gq_timing_enable(int mask);
gq_status gq_timing_read(double* ms, int64_t* launches);
/* Short name of a stage ("" for an unknown id); static storage. */
const char* gq_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
