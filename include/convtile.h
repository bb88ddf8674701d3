/*
 * convtile -- NCHW 2-D convolution (implicit GEMM on CDNA4 matrix cores) and
 * per-channel broadcast for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (TVM tutorial "Tuning High Performance Convolution on NVIDIA
 * GPUs", Step 1, the conv2d_nchw compute of the template):
 *
 *   y[n][f][oy][ox] = sum_{c<CI} sum_{ky<KH} sum_{kx<KW}
 *                     xp[n][c][oy*stride+ky][ox*stride+kx] * w[f][c][ky][kx]
 *
 *   xp = x zero-padded by `pad` on every side (never materialised: padding is
 *   applied inline while gathering), dilation 1, no kernel flip, and
 *   OH = (H + 2 pad - KH) / stride + 1, OW likewise (integer division).
 *   Output is always fp32 (the template's out_dtype='float32'), also for fp16 /
 *   bf16 inputs, which are multiplied exactly and accumulated in fp32.
 *
 * Optional per-channel epilogue (Paddle PR "[CINN] Add the TileBroadcastTactic
 * for NCHW broadcast", Performance Impact: per-channel div/exp/rsqrt chains,
 * with the channel bound to a grid axis so its value is computed once per
 * workgroup):
 *   CT_EPI_NONE            out = y
 *   CT_EPI_BIAS            out = y + bias[f]
 *   CT_EPI_EXP_BIAS_RSQRT  out = exp(y + bias[f]) * rsqrt(var[f] + eps)
 *
 * Layouts (all contiguous, row-major, device memory owned by the caller):
 *   x    [N][CI][H][W]      dtype CT_F32 (float), CT_F16 (IEEE half), CT_BF16
 *   w    [CO][CI][KH][KW]   same dtype as x
 *   y    [N][CO][OH][OW]    float; must not alias x, w, bias or var
 *   bias [CO], var [CO]     float (NULL when the epilogue does not read them)
 *
 * Conventions
 *   - Every entry point returns a status (CT_OK = 0, negative on error) and
 *     never throws across the ABI.  ct_last_error() gives a message for the
 *     last failure on the calling thread.
 *   - Argument errors are reported with CT_ERR_INVALID_ARG before any HIP call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Launch calls are
 *     asynchronous on that stream.  Once a device is set up (ct_init, or the
 *     first launch on it) and a stream's workspace has grown to what a shape
 *     needs (the first split-reduction launch of that size on the stream),
 *     a launch neither synchronises nor allocates, so it may be captured into
 *     a HIP graph.  A launch that would need either step while its stream is
 *     capturing returns CT_ERR_UNSUPPORTED and captures nothing.
 *   - The library owns: the compiled kernels, a process-wide tile-config cache
 *     (mutex-protected), a launch plan per (device, shape) derived from it,
 *     and per-(device, stream) split-reduction workspaces.  A workspace grows
 *     by allocating a larger buffer; the buffer it replaces stays allocated
 *     until ct_release(), because a graph captured earlier on that stream may
 *     still use it.  Two launches that use split reduction on the same stream
 *     are ordered by the stream; launches on different streams get different
 *     workspaces.  A captured launch keeps the workspace of the stream it was
 *     captured on: replays of such graphs must not overlap one another or
 *     other launches on that stream.
 */
#ifndef CONVTILE_H
#define CONVTILE_H

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define CT_OK 0
#define CT_ERR_INVALID_ARG (-1)  /* bad shape, NULL pointer, unknown enum      */
#define CT_ERR_UNSUPPORTED (-2)  /* legal arguments no kernel here can run    */
#define CT_ERR_HIP (-3)          /* a HIP runtime call failed                 */
#define CT_ERR_NO_MEMORY (-4)    /* workspace / scratch allocation failed     */
#define CT_ERR_IO (-5)           /* cache file could not be read or written   */
#define CT_ERR_TUNE_FAILED (-6)  /* no candidate of the search ran correctly  */

/* ---- enums ------------------------------------------------------------ */
enum ct_dtype { CT_F32 = 0, CT_F16 = 1, CT_BF16 = 2 };
enum ct_epilogue { CT_EPI_NONE = 0, CT_EPI_BIAS = 1, CT_EPI_EXP_BIAS_RSQRT = 2 };
enum ct_bcast_op { CT_BC_EXP = 0 };
enum ct_bcast_mode {
    CT_BC_AUTO = 0,    /* channel-bound when it applies, else flat            */
    CT_BC_CHANNEL = 1, /* channel index on a grid axis; value computed once   */
    CT_BC_FLAT = 2     /* all axes fused; value loaded and computed per element */
};

/* Measurement outcome codes of a tuning trial (the meanings of the autotvm
 * MeasureResult error_no values printed in the tutorial's tuning log). */
enum ct_trial_error {
    CT_TRIAL_OK = 0,
    CT_TRIAL_ILLEGAL = 1,  /* rejected by the legality check, never launched */
    CT_TRIAL_RUNTIME = 4,  /* HIP error, or output differs from the reference */
    CT_TRIAL_TIMEOUT = 6   /* exceeded the per-trial time limit               */
};

/* One point of a shape's tile-config space. */
typedef struct ct_tile_config {
    int variant;     /* kernel variant id (see ct_variant_info)               */
    int split_k;     /* S: workgroups that share one output tile's reduction  */
    int stages;      /* LDS stages each workgroup runs                        */
    int kc;          /* input channels per LDS stage                          */
    long long index; /* flat index in the shape's space; -1 = not from space  */
    float us;        /* mean microseconds per launch when measured, else 0    */
    int error_no;    /* ct_trial_error of the measurement, 0 if never timed   */
} ct_tile_config;

/* A compiled kernel variant (one instantiation of the tiled template). */
typedef struct ct_variant_desc {
    char name[48];
    int dtype;        /* ct_dtype it accepts                                   */
    int kind;         /* 0 = direct (one lane per output), 1 = implicit GEMM   */
    int mfma_m, mfma_n, mfma_k; /* matrix-core instruction shape (0 for direct) */
    int waves_m, waves_n, waves_k; /* waves per workgroup along CO, P, K       */
    int reps_m, reps_n;  /* MFMA tiles per wave along CO and P                 */
    int tile_m, tile_n;  /* workgroup output tile: CO x P                      */
    int kc_max;          /* most input channels one LDS stage holds            */
    int threads;         /* workgroup size                                     */
} ct_variant_desc;

/* One timed candidate of ct_conv2d_tune (autotvm MeasureResult analogue). */
typedef struct ct_tune_record {
    ct_tile_config cfg;
    float costs_us[3];   /* mean us per launch of each repeat                  */
    int n_costs;
    int error_no;        /* ct_trial_error                                     */
    double all_cost_s;   /* wall seconds spent on this trial                   */
    double timestamp;    /* seconds since the epoch when the trial ended       */
} ct_tune_record;

/* ---- convolution ----------------------------------------------------- */

/* Forward convolution with the cached tile config for this shape (or the
 * built-in default when none is cached; with the environment variable
 * CT_TUNE=1, a shape with no cached config is first searched with
 * ct_conv2d_tune on `stream`, once per process -- CT_TUNE_TRIALS bounds the
 * trials, CT_TUNE_MS sets min_repeat_ms (default 20) -- unless the stream is
 * capturing).  Shapes/layouts as above; `eps` is
 * used only by CT_EPI_EXP_BIAS_RSQRT.  Errors: CT_ERR_INVALID_ARG for any
 * dimension <= 0, stride <= 0, pad < 0, OH or OW <= 0, NULL x/w/y, unknown
 * dtype/epilogue, or bias/var missing when the epilogue reads them;
 * CT_ERR_UNSUPPORTED when the device is not set up or the stream's workspace
 * must grow while the stream is capturing (see Conventions);
 * CT_ERR_NO_MEMORY if the split workspace cannot grow; CT_ERR_HIP on a launch
 * failure. */
int ct_conv2d_nchw_fwd(const void* x, const void* w, float* y,
                       int N, int CI, int H, int W, int CO, int KH, int KW,
                       int stride, int pad, int dtype, int epilogue,
                       const float* bias, const float* var, float eps,
                       void* stream);

/* Half-precision filters in the layout the kernels stage from.  The
 * half-precision kernels read the filter as 16-byte records of 8 input
 * channels at one tap:
 *
 *   wp[co][g][t][j] = w[co][8g + j][t]   (t = ky*KW + kx; 0 when 8g + j >= CI)
 *
 * wp is [CO][CI64/8][KH*KW][8] halves with CI64 = CI rounded up to a multiple
 * of 64 (every stage of the kernels' reduction then lies inside a row),
 * ct_conv2d_filter_prepared_bytes bytes.  ct_conv2d_nchw_fwd reorders the caller's filter into its scratch
 * on every call (one small kernel before the convolution); a caller whose
 * filter does not change between calls (inference) prepares it once with
 * ct_conv2d_prepare_filter (asynchronous on `stream`, wp caller-owned device
 * memory, 16-byte aligned) and calls ct_conv2d_nchw_fwd_prepared, which
 * takes the same arguments as ct_conv2d_nchw_fwd with wp in place of w and
 * gives the same bits, without the reorder.  The prepared entry point uses
 * the cached tile config when its variant reads a prepared filter, else the
 * best such default.  Errors: CT_ERR_INVALID_ARG for dtype CT_F32 (fp32
 * kernels read the caller's layout directly) or a NULL pointer, and those of
 * ct_conv2d_nchw_fwd; CT_ERR_UNSUPPORTED when no tile config of the shape
 * reads a prepared filter. */
long long ct_conv2d_filter_prepared_bytes(int CO, int CI, int KH, int KW, int dtype);
int ct_conv2d_prepare_filter(const void* w, void* wp, int CO, int CI, int KH, int KW, int dtype,
                             void* stream);
int ct_conv2d_nchw_fwd_prepared(const void* x, const void* wp, float* y,
                                int N, int CI, int H, int W, int CO, int KH, int KW,
                                int stride, int pad, int dtype, int epilogue,
                                const float* bias, const float* var, float eps,
                                void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * convolution as ct_conv2d_nchw_fwd (same arguments, config, kernel and
 * bits), but a launch's scratch -- the split partials, their arrival
 * counters and the half-precision kernels' reordered filter -- lives in a
 * fixed array inside the library instead of a per-stream workspace:
 * CT_NOALLOC_SCRATCH_BYTES for partials plus filter and 16384 counters (at
 * most 512 split tiles), held by every device the library runs on until the
 * process ends.  Never calls hipMalloc or hipFree.  Errors: those of
 * ct_conv2d_nchw_fwd, and CT_ERR_UNSUPPORTED when the config needs more
 * scratch than that (the message says how much).  Every call on a device
 * shares that device's array, which keeps the last call's contents: calls
 * that overlap in time on one device (launches on different streams, or
 * concurrent graph replays) race and give wrong results. */
#define CT_NOALLOC_SCRATCH_BYTES (16LL << 20)
int ct_conv2d_nchw_fwd_noalloc(const void* x, const void* w, float* y,
                               int N, int CI, int H, int W, int CO, int KH, int KW,
                               int stride, int pad, int dtype, int epilogue,
                               const float* bias, const float* var, float eps,
                               void* stream);

/* The same with an explicit tile config (cfg->variant, split_k, stages, kc);
 * cfg->index is ignored.  Returns CT_ERR_UNSUPPORTED when the config is not
 * legal for the shape (the check of ct_conv2d_space_entity). */
int ct_conv2d_nchw_fwd_config(const void* x, const void* w, float* y,
                              int N, int CI, int H, int W, int CO, int KH, int KW,
                              int stride, int pad, int dtype, int epilogue,
                              const float* bias, const float* var, float eps,
                              const ct_tile_config* cfg, void* stream);

/* Reference kernel: one lane per output, fp32 fused multiply-add over the
 * taps in definition order.  Slow; used as the on-device check of every
 * tuning candidate.  Same arguments and errors as ct_conv2d_nchw_fwd. */
int ct_conv2d_nchw_direct(const void* x, const void* w, float* y,
                          int N, int CI, int H, int W, int CO, int KH, int KW,
                          int stride, int pad, int dtype, int epilogue,
                          const float* bias, const float* var, float eps,
                          void* stream);

/* ---- matrix product (the 1x1-convolution view) -----------------------
 * The TVM tutorial notes, in its opening, that the same tiled template also
 * serves a matrix product.  Here that is literal:
 *
 *   C[m][n] = sum_{k<K} A[m][k] * B[k][n]      (row-major, all contiguous)
 *
 * is the batch-1 convolution with a 1x1 filter, CO = M, CI = K and H*W = N:
 * w = A as [M][K][1][1], x = B as [1][K][H][W], y = C as [1][M][H][W] (a 1x1
 * filter sees pixels only as a flat index, so every split of N has the same
 * layout; W is the largest divisor of N not above 256).  A and B
 * have dtype `dtype` (CT_F32 / CT_F16 / CT_BF16), C is float.  The epilogue is
 * per row m (bias[m], var[m]).  Tuned configs are cached under that
 * convolution's shape, so ct_conv2d_tune and ct_gemm_tune share records.
 * Errors: CT_ERR_INVALID_ARG for M, N or K <= 0; otherwise those of
 * ct_conv2d_nchw_fwd / ct_conv2d_tune / ct_conv2d_query. */
int ct_gemm_fwd(const void* A, const void* B, float* C, int M, int N, int K,
                int dtype, int epilogue, const float* bias, const float* var,
                float eps, void* stream);
int ct_gemm_tune(int M, int N, int K, int dtype, int epilogue,
                 int max_trials, float min_repeat_ms, void* stream,
                 ct_tile_config* best_out,
                 ct_tune_record* records, int max_records, int* n_records);
int ct_gemm_query(int M, int N, int K, int dtype, int epilogue,
                  ct_tile_config* cfg_out, int* from_cache);

/* ---- general per-channel broadcast -----------------------------------
 * The Paddle PR's Introduction generalises its tactic, by axis fusion, to
 * [1,P,1] => [B,P,B] with the last axis a broadcast axis, and its
 * Performance Impact section names div / exp / rsqrt chains as the work the
 * tactic saves.  Here: out is [outer][P][inner] (inner contiguous) and a
 * program of three chains, each at most CT_CHAIN_MAX_OPS steps applied in
 * order to a value that starts at 0, is evaluated in fp32 per element:
 *
 *   chain 0 -> c0   operands: immediates, arrays a0..a3 at [p]
 *   chain 1 -> c1   operands: the same, and c0
 *   chain 2 -> v    operands: the same, c0, c1, and x[o][p][i]
 *   out[o][p][i] = v, or c0 when chain 2 is empty
 *
 * A step is (op, src, imm): CT_OP_SET v = a; ADD v + a; SUB v - a; MUL v * a;
 * DIV v / a; RSUB a - v; RDIV a / v; EXP exp(v); RSQRT 1/sqrt(v); SQRT
 * sqrt(v) (the unary steps ignore their operand); a is imm, x, c0, c1 or
 * a_k[p] by `src`.  exp and rsqrt run on the hardware units (about 1 ulp
 * each), division and sqrt are correctly rounded, nothing is contracted into
 * a fused multiply-add, and fp16 output is rounded to nearest even. */
#define CT_CHAIN_MAX_OPS 8
#define CT_OP_SET 0
#define CT_OP_ADD 1
#define CT_OP_SUB 2
#define CT_OP_MUL 3
#define CT_OP_DIV 4
#define CT_OP_RSUB 5
#define CT_OP_RDIV 6
#define CT_OP_EXP 7
#define CT_OP_RSQRT 8
#define CT_OP_SQRT 9
#define CT_SRC_IMM 0
#define CT_SRC_X 1
#define CT_SRC_C0 2
#define CT_SRC_C1 3
#define CT_SRC_A0 4  /* CT_SRC_A0 + k for array a_k, k < 4 */

typedef struct ct_chain_op {
    int op;      /* CT_OP_* */
    int src;     /* CT_SRC_* */
    float imm;   /* the operand when src == CT_SRC_IMM */
} ct_chain_op;

typedef struct ct_bcast_program {
    int n_ops[3];                             /* steps in chains 0, 1, 2 */
    ct_chain_op ops[3][CT_CHAIN_MAX_OPS];
} ct_bcast_program;

/* Evaluate `prog` into out ([outer][P][inner], out_dtype CT_F32 or CT_F16).
 * a0..a3: per-channel fp32 arrays of P floats on the device (NULL when no
 * step reads them); x: the producer's fp32 output, same [outer][P][inner]
 * layout (NULL when no step reads it; x == out is allowed for fp32 output,
 * any other overlap is not).  mode: CT_BC_CHANNEL (channel-bound: c0 and c1
 * once per block), CT_BC_FLAT (everything per element) or CT_BC_AUTO, which
 * takes the channel-bound form when inner >= 32, each row is a whole number
 * of 16-byte vectors of out (and x), both are 16-byte aligned and the grid
 * fits, and the flat form otherwise.  Both forms give identical bits.
 * Errors: CT_ERR_INVALID_ARG for a NULL prog or out, outer, P or inner < 1,
 * more than 2^46 elements, a step count outside [0, CT_CHAIN_MAX_OPS], an
 * unknown op or source, a source a chain may not read, a NULL array or x
 * that a step reads, an unknown dtype or mode, or x == out with fp16 output;
 * CT_ERR_UNSUPPORTED for CT_BC_CHANNEL when the channel-bound conditions
 * fail; CT_ERR_HIP on a launch failure.  Asynchronous on `stream`. */
int ct_broadcast_chain(const ct_bcast_program* prog, const float* a0, const float* a1,
                       const float* a2, const float* a3, const float* x, void* out,
                       int out_dtype, long long outer, int P, long long inner, int mode,
                       void* stream);

/* ---- depthwise convolution -------------------------------------------
 * The TVM tutorial names, in its opening, depthwise convolution as another
 * operator its template covers.  Each channel is convolved with its own
 * filter:
 *
 *   y[n][c][oy][ox] = sum_{ky<KH} sum_{kx<KW} xp[n][c][oy*s+ky][ox*s+kx] * w[c][0][ky][kx]
 *
 * x [N][C][H][W] and w [C][1][KH][KW] (contiguous, dtype `dtype`), y
 * [N][C][OH][OW] float with OH, OW as for ct_conv2d_nchw_fwd, xp x padded with
 * `pad` zeros, fp32 accumulation, and the per-channel epilogue (bias[c],
 * var[c]).  No channel reduction, so no tile config: one LDS-tiled kernel.
 * Errors: those of ct_conv2d_nchw_fwd for the arguments, and
 * CT_ERR_UNSUPPORTED for more than 256 taps (KH*KW), N*C or H*W above 2^31 - 1, or
 * an output row too wide for one workgroup's LDS window (about
 * ((3*stride + KH) * ((OW-1)*stride + KW)) > 40960); CT_ERR_HIP on a launch
 * failure.  Asynchronous on `stream`. */
int ct_conv2d_nchw_depthwise(const void* x, const void* w, float* y,
                             int N, int C, int H, int W, int KH, int KW,
                             int stride, int pad, int dtype, int epilogue,
                             const float* bias, const float* var, float eps,
                             void* stream);

/* ---- tile-config search ----------------------------------------------
 * The space of a shape follows the TVM tutorial's template (Step 1): ordered
 * knobs, each a split (all ordered factorizations of an extent, the
 * "policy=all" of the gist's ConfigSpace dump) or an option list, and a flat
 * index that is mixed radix over the knobs with the first knob least
 * significant.  Knobs here, in order:
 *   tile_ci = split(CI, 3) -> [split_k, stages, kc]
 *   variant = option(ids of the compiled variants for the dtype)
 */

/* Number of points in the space of this shape (legal or not); < 0 on error. */
long long ct_conv2d_space_size(int N, int CI, int H, int W, int CO, int KH, int KW,
                               int stride, int pad, int dtype, int epilogue);

/* Decode flat `index` into *cfg_out and report in *legal (1/0) whether the
 * point passes the legality check (LDS bytes within 160 KiB, workgroup size
 * within 1024, channels per stage within the variant's limit, ...).  The
 * check never launches anything.  CT_ERR_INVALID_ARG for an index outside
 * [0, size). */
int ct_conv2d_space_entity(int N, int CI, int H, int W, int CO, int KH, int KW,
                           int stride, int pad, int dtype, int epilogue,
                           long long index, ct_tile_config* cfg_out, int* legal);

/* Enumerate the legal points, time up to `max_trials` of them on `stream`
 * (0 = all legal points), keep the fastest whose output matches the direct
 * reference kernel, store it in the cache and in *best_out.  Timing follows
 * the TVM tutorial's runner (Step 2): a warm-up, then `repeat` (3)
 * measurements each of at least `min_repeat_ms` milliseconds of back-to-back
 * launches, and a per-trial limit of 4 s (CT_TUNE_TIMEOUT_S overrides it),
 * checked while the launches run: a trial past it records error 6 and issues
 * no more launches.  Scratch inputs are allocated and filled on the device
 * by the library.  `records` (may be NULL) receives up to `max_records` trial
 * records and *n_records their count.
 * Tuning log (the tutorial's log_to_file): when the environment variable
 * CT_CACHE_PATH names a file, every trial record is appended to it as one
 * JSON line when the trial ends (error_no 1/4/6 included), and a search of a
 * shape first reads the file: points already logged for the shape are not
 * measured again (resume), and their logged results take part in choosing
 * the winner; `records` lists only the trials measured by this call.
 * Synchronises the stream; may take seconds.  Returns CT_ERR_TUNE_FAILED if
 * no candidate ran correctly, CT_ERR_IO if the log cannot be appended. */
int ct_conv2d_tune(int N, int CI, int H, int W, int CO, int KH, int KW,
                   int stride, int pad, int dtype, int epilogue,
                   int max_trials, float min_repeat_ms, void* stream,
                   ct_tile_config* best_out,
                   ct_tune_record* records, int max_records, int* n_records);

/* The flat indices ct_conv2d_tune would time for this shape, in order (legal
 * points by the analytic time estimate, then the illegal ones), leaving out
 * the points already recorded in the CT_CACHE_PATH log (resume), at most
 * `max_trials` (0 = all).  Writes up to `max_out` of them to order_out and
 * their full count to *n_out.  Host-only: launches nothing. */
int ct_conv2d_tune_order(int N, int CI, int H, int W, int CO, int KH, int KW,
                         int stride, int pad, int dtype, int epilogue, int max_trials,
                         long long* order_out, int max_out, int* n_out);

/* Guided search for spaces too large to time exhaustively (the role of the
 * TVM tutorial's cost-model tuner, XGBTuner, in Step 2).  Times at most
 * `max_trials` legal configs (0 = all), `batch` at a time: the first batch
 * drawn uniformly (SplitMix64 on `seed`), each later one the lowest
 * predictions of a ridge regression of log(time) on 11 features of a config
 * (ct_ridge_fit, lambda 1e-3, refitted after every batch) plus max(1,
 * batch/4) uniform draws among the untimed configs.  Trials, records, the
 * cache entry and errors as ct_conv2d_tune; CT_ERR_INVALID_ARG also for
 * batch < 1.  The CT_CACHE_PATH log is written and resumed from as for
 * ct_conv2d_tune. */
int ct_conv2d_tune_guided(int N, int CI, int H, int W, int CO, int KH, int KW,
                          int stride, int pad, int dtype, int epilogue,
                          int max_trials, int batch, unsigned long long seed,
                          float min_repeat_ms, void* stream,
                          ct_tile_config* best_out,
                          ct_tune_record* records, int max_records, int* n_records);

/* The guided search's parts on host data (no device): ct_ridge_fit solves
 * min |X w - y|^2 + lambda |w|^2 (X row-major n x d, 1 <= d <= 64) by a
 * Cholesky factorisation, CT_ERR_INVALID_ARG when X^T X + lambda I is
 * singular; ct_guided_search_table runs the search of ct_conv2d_tune_guided
 * over n points with features feats (n x d) whose costs are given (cost <= 0
 * or not finite = a failed trial, left out of the fit), with n_explore
 * draws a batch after the first, and writes the order in which it would time
 * them (at most max_trials) to order_out, their count to *n_order. */
int ct_ridge_fit(const double* X, const double* y, int n, int d, double lambda, double* w);
int ct_guided_search_table(const double* feats, const double* costs, int n, int d,
                           int max_trials, int batch, int n_explore,
                           unsigned long long seed, double lambda,
                           int* order_out, int* n_order);

/* The config ct_conv2d_nchw_fwd would use for this shape; *from_cache = 1
 * when it came from a tuning record, 0 when it is the built-in default.  The
 * TVM tutorial's closing step looks the tuned config of a workload up in its
 * log this way (apply_history_best, then query of the best record) before it
 * builds the kernel.  Errors: those of ct_conv2d_space_size, CT_ERR_INVALID_ARG
 * for a NULL cfg_out. */
int ct_conv2d_query(int N, int CI, int H, int W, int CO, int KH, int KW,
                    int stride, int pad, int dtype, int epilogue,
                    ct_tile_config* cfg_out, int* from_cache);

/* Compiled variants. */
int ct_variant_count(void);
int ct_variant_info(int variant, ct_variant_desc* out);

/* Ordered factorizations of n into k factors ("policy=all" split): count, and
 * the i-th one written to out[0..k-1] in the space's order (ascending by
 * (x_k, ..., x_2)).  Count < 0 for n <= 0 or k outside [1, 8]. */
long long ct_split_count(long long n, int k);
int ct_split_entity(long long n, int k, long long i, long long* out);

/* ---- the tutorial template's own space ---------------------------------
 * The conv2d_nchw schedule of the TVM tutorial "Tuning High Performance
 * Convolution on NVIDIA GPUs" (Step 1) has eight knobs, in declaration order:
 *   tile_f = split(CO, 4), tile_y = split(OH, 4), tile_x = split(OW, 4),
 *   tile_rc = split(CI, 3), tile_ry = split(KH, 3), tile_rx = split(KW, 3)
 *   (each in ct_split_entity's order), auto_unroll_max_step in {0, 512,
 *   1500}, unroll_explicit in {0, 1};
 * the flat index is mixed radix over them, tile_f least significant: the
 * space the gist's run prints for the last ResNet layer (10,454,400 points)
 * and the index beside each record of its tuning log.  This library does not
 * build that schedule (its kernels are the MFMA variants above); the space
 * and the check below reproduce which of the tutorial's candidates its run
 * rejected before timing them (error_no 1, "invalid gpu kernel"). */
typedef struct {
    int tile_f[4], tile_y[4], tile_x[4];
    int tile_rc[3], tile_ry[3], tile_rx[3];
    int auto_unroll_max_step;
    int unroll_explicit;
} ct_tvm_config;

/* Points of the template's space for this shape; < 0 on a bad shape. */
long long ct_tvm_space_size(int N, int CI, int H, int W, int CO, int KH, int KW,
                            int stride, int pad);
/* Decode flat `index` into *out.  CT_ERR_INVALID_ARG for a bad shape, a NULL
 * out or an index outside [0, size). */
int ct_tvm_space_entity(int N, int CI, int H, int W, int CO, int KH, int KW,
                        int stride, int pad, long long index, ct_tvm_config* out);
/* The flat index of *cfg in the space (the inverse of ct_tvm_space_entity);
 * CT_ERR_INVALID_ARG for a bad shape or a NULL cfg, -1 (with no error
 * recorded) when *cfg is not a point of the space. */
long long ct_tvm_space_index(int N, int CI, int H, int W, int CO, int KH, int KW,
                             int stride, int pad, const ct_tvm_config* cfg);

#define CT_TVM_LIMITS_PAGE 0    /* the tutorial run's GPU: 48 KiB shared memory, 1024 threads per block */
#define CT_TVM_LIMITS_GFX950 1  /* this device: 160 KiB LDS, 1024 threads per workgroup */

/* The tutorial schedule's block resources under *cfg, without building it.
 * The schedule stages the padded input (AA) and the filter (WW) in shared
 * memory at the outer rx loop, inside the outer rc, ry and rx loops, so each
 * holds one block's output tile against the middle x inner reduction
 * extents, in fp32:
 *   AA = RC_s * ((Y_b - 1) * stride + RY_s) * ((X_b - 1) * stride + RX_s)
 *   WW = F_b * RC_s * RY_s * RX_s
 * with F_b = tile_f[1] * tile_f[2] * tile_f[3] (vthread, thread and inner
 * factors; Y_b and X_b alike), RC_s = tile_rc[1] * tile_rc[2] and, as the
 * schedule is printed, the ry axis split by tile_rx's factors and rx by
 * tile_ry's: RY_s = tile_rx[1] * tile_rx[2], RX_s = tile_ry[1] * tile_ry[2].
 * Threads per block = tile_f[2] * tile_y[2] * tile_x[2].  Writes
 * *shared_bytes = 4 * (AA + WW) and *threads (either may be NULL); returns
 * 1 when both fit the limits of `mode`, 0 when not, CT_ERR_INVALID_ARG for a
 * NULL cfg, a factor < 1, stride < 1 or an unknown mode. */
int ct_tvm_config_check(const ct_tvm_config* cfg, int stride, int mode,
                        long long* shared_bytes, int* threads);

/* ---- per-channel broadcast --------------------------------------------
 * out[n][c][h][w] = exp(var[c])  (Paddle PR, Introduction and Example:
 * [1,C,1,1] => [N,C,H,W]).  var: C floats on the device; out: N*C*H*W
 * elements of out_dtype (CT_F32 or CT_F16, rounded to nearest even).  The
 * channel-bound form needs H*W % 32 == 0 and a 16-byte aligned `out`;
 * CT_BC_AUTO falls back to the flat form otherwise, CT_BC_CHANNEL returns
 * CT_ERR_UNSUPPORTED.  Results are identical in every mode. */
int ct_broadcast_nchw(const float* var, void* out, int N, int C, int H, int W,
                      int out_dtype, int op, int mode, void* stream);

/* ---- cache, lifetime, errors ----------------------------------------- */

/* Append-only JSON-lines tuning log: the TVM tutorial's Step 2 writes every
 * measure record to a log file (log_to_file), and its closing step picks the
 * best record per workload from that log (apply_history_best).  Here a record
 * is one line with the shape key, the config, its costs, error_no and a
 * timestamp.  load merges the file into memory, keeping per shape the fastest
 * successful record (lines that do not parse, name an unknown variant or are
 * not legal for their shape are skipped); save appends every in-memory
 * winner to the file.  CT_ERR_INVALID_ARG for a NULL path, CT_ERR_IO when the
 * file cannot be opened or written.  clear empties the in-memory cache; size
 * is its number of shapes. */
int ct_cache_load(const char* path);
int ct_cache_save(const char* path);
int ct_cache_clear(void);
int ct_cache_size(void);

/* Free the library's device workspaces, and every buffer a workspace
 * outgrew (all devices, all streams).  Synchronises each stream that owns a
 * workspace first.  No graph that captured a launch may be replayed after
 * this. */
int ct_release(void);

/* Set up `device` for launches: the zero page's device address and the
 * workgroup-placement probe of the XCD-local variants (which launches and
 * synchronises a private stream).  Idempotent.  Call it before capturing
 * the first launch on a device into a HIP graph.  CT_ERR_INVALID_ARG for a
 * device that does not exist, CT_ERR_HIP when a HIP call fails. */
int ct_init(int device);

/* How many times ct_conv2d_nchw_fwd resolved a launch plan (a first call for
 * a (device, shape), or the first after the config cache changed); every
 * other call reused a plan.  For tests and diagnostics. */
long long ct_plan_misses(void);

const char* ct_status_string(int status);
const char* ct_last_error(void);
const char* ct_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CONVTILE_H */
