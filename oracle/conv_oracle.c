/*
 * Oracle for the NCHW convolution / per-channel broadcast path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library (tensor_compiler_tiling_amd)
 * may include, link or call this file.  Only tests/, __graft_entry__.smoke()
 * and bench.py's cpu_baseline leg use it.  It shares no code, header, table or
 * helper with the HIP path.
 *
 * Everything is computed in IEEE double precision, with the loops written in
 * the order of the plain mathematical definition and no blocking, fusion or
 * reordering.  The inputs are double arrays that already hold the exact values
 * the GPU sees (fp32, or fp16/bf16 values widened exactly).
 *
 * Sources (the pages this reproduces):
 *  - TVM tutorial "Tuning High Performance Convolution on NVIDIA GPUs",
 *    Step 1 (search-space definition): data [N,CI,H,W], kernel [CO,CI,KH,KW],
 *    conv2d_nchw with stride, padding, dilation 1, float32 output; the
 *    padded input is inlined ("inline padding"), never materialised.
 *    The formula itself is not printed on the page; the reading taken is the
 *    deep-learning convention: cross-correlation (no kernel flip), symmetric
 *    zero padding, dilation 1.
 *  - Paddle PR "[CINN] Add the TileBroadcastTactic for NCHW broadcast",
 *    Introduction / Example: [1,C,1,1] => [N,C,H,W] with value exp(var[c]);
 *    Performance Impact: per-channel div/exp/rsqrt chains.
 */
#include <math.h>
#include <stddef.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)

/* Output extent of a strided, zero-padded correlation with dilation 1:
 * floor((in + 2*pad - k) / stride) + 1, or 0 when the kernel does not fit. */
static long oracle_out_extent(long in, long k, long stride, long pad)
{
    long span = in + 2 * pad - k;
    if (span < 0 || stride <= 0) return 0;
    return span / stride + 1;
}

long oracle_out_extent_api(long in, long k, long stride, long pad)
{
    return oracle_out_extent(in, k, stride, pad);
}

/* Value of the zero-padded input xp[n][c][i][j] = x[n][c][i-pad][j-pad]
 * inside the image, 0 outside (TVM tutorial, Step 1, "inline padding"). */
static double oracle_padded(const double *x, long CI, long H, long W,
                            long n, long c, long i, long j, long pad)
{
    long r = i - pad, q = j - pad;
    if (r < 0 || r >= H || q < 0 || q >= W) return 0.0;
    return x[((n * CI + c) * H + r) * W + q];
}

/*
 * y[n][f][oy][ox] = sum_{c<CI} sum_{ky<KH} sum_{kx<KW}
 *                   xp[n][c][oy*s+ky][ox*s+kx] * w[f][c][ky][kx]
 * absacc[...]     = the same sum over |xp * w|   (scale for the tolerance)
 *
 * Seven nested loops in the order n, f, oy, ox, c, ky, kx; fp64 accumulation.
 * absacc may be NULL.  Parallel over (n, f) only, so each output is still one
 * sequential sum in the definition's order.
 */
int oracle_conv2d_nchw(const double *x, const double *w, double *y, double *absacc,
                       long N, long CI, long H, long W, long CO, long KH, long KW,
                       long stride, long pad)
{
    if (!x || !w || !y || N <= 0 || CI <= 0 || H <= 0 || W <= 0 || CO <= 0 ||
        KH <= 0 || KW <= 0 || stride <= 0 || pad < 0)
        return ORACLE_BAD_ARG;
    long OH = oracle_out_extent(H, KH, stride, pad);
    long OW = oracle_out_extent(W, KW, stride, pad);
    if (OH <= 0 || OW <= 0) return ORACLE_BAD_ARG;

    long nf_total = N * CO;
#pragma omp parallel for schedule(dynamic, 1)
    for (long nf = 0; nf < nf_total; ++nf) {
        long n = nf / CO, f = nf % CO;
        for (long oy = 0; oy < OH; ++oy) {
            for (long ox = 0; ox < OW; ++ox) {
                double acc = 0.0, aacc = 0.0;
                for (long c = 0; c < CI; ++c) {
                    for (long ky = 0; ky < KH; ++ky) {
                        for (long kx = 0; kx < KW; ++kx) {
                            double xv = oracle_padded(x, CI, H, W, n, c,
                                                      oy * stride + ky, ox * stride + kx, pad);
                            double prod = xv * w[((f * CI + c) * KH + ky) * KW + kx];
                            acc += prod;
                            aacc += fabs(prod);
                        }
                    }
                }
                long o = ((n * CO + f) * OH + oy) * OW + ox;
                y[o] = acc;
                if (absacc) absacc[o] = aacc;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * The same sum as oracle_conv2d_nchw, for a list of output coordinates only
 * (idx holds npts quadruples n, f, oy, ox).  Used to check sampled outputs of
 * workloads too large for the full seven-loop pass.
 */
int oracle_conv2d_points(const double *x, const double *w, const long *idx, long npts,
                         double *y, double *absacc,
                         long N, long CI, long H, long W, long CO, long KH, long KW,
                         long stride, long pad)
{
    if (!x || !w || !idx || !y || npts < 0 || N <= 0 || CI <= 0 || H <= 0 ||
        W <= 0 || CO <= 0 || KH <= 0 || KW <= 0 || stride <= 0 || pad < 0)
        return ORACLE_BAD_ARG;
    long OH = oracle_out_extent(H, KH, stride, pad);
    long OW = oracle_out_extent(W, KW, stride, pad);
    if (OH <= 0 || OW <= 0) return ORACLE_BAD_ARG;
    for (long t = 0; t < npts; ++t) {
        long n = idx[4 * t], f = idx[4 * t + 1], oy = idx[4 * t + 2], ox = idx[4 * t + 3];
        if (n < 0 || n >= N || f < 0 || f >= CO || oy < 0 || oy >= OH || ox < 0 || ox >= OW)
            return ORACLE_BAD_ARG;
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (long t = 0; t < npts; ++t) {
        long n = idx[4 * t], f = idx[4 * t + 1], oy = idx[4 * t + 2], ox = idx[4 * t + 3];
        double acc = 0.0, aacc = 0.0;
        for (long c = 0; c < CI; ++c)
            for (long ky = 0; ky < KH; ++ky)
                for (long kx = 0; kx < KW; ++kx) {
                    double xv = oracle_padded(x, CI, H, W, n, c,
                                              oy * stride + ky, ox * stride + kx, pad);
                    double prod = xv * w[((f * CI + c) * KH + ky) * KW + kx];
                    acc += prod;
                    aacc += fabs(prod);
                }
        y[t] = acc;
        if (absacc) absacc[t] = aacc;
    }
    return ORACLE_OK;
}

/*
 * Per-channel epilogue applied to a conv result y[N][C][HW]:
 *   kind 0: out = y
 *   kind 1: out = y + b[c]
 *   kind 2: out = exp(y + b[c]) * (v[c] + eps)^(-1/2)
 * The exp / rsqrt chain over a per-channel operand is the case the Paddle PR's
 * "Performance Impact" section targets; bias, mean and eps follow the plain
 * normalisation reading.  Computed with libm exp and 1/sqrt in fp64.
 */
int oracle_channel_epilogue(const double *y, const double *b, const double *v, double eps,
                            long N, long C, long HW, int kind, double *out)
{
    if (!y || !out || N <= 0 || C <= 0 || HW <= 0 || kind < 0 || kind > 2) return ORACLE_BAD_ARG;
    if (kind >= 1 && !b) return ORACLE_BAD_ARG;
    if (kind == 2 && !v) return ORACLE_BAD_ARG;
    for (long n = 0; n < N; ++n)
        for (long c = 0; c < C; ++c)
            for (long i = 0; i < HW; ++i) {
                long o = (n * C + c) * HW + i;
                double t = y[o];
                if (kind == 1) t = t + b[c];
                else if (kind == 2) t = exp(t + b[c]) * (1.0 / sqrt(v[c] + eps));
                out[o] = t;
            }
    return ORACLE_OK;
}

/*
 * Broadcast [1,C,1,1] => [N,C,H,W]: out[n][c][h][w] = exp(var[c])
 * (Paddle PR, Example section: the loop nest over N, C, H, W writing exp(var[j])).
 */
int oracle_broadcast_exp(const double *var, long N, long C, long H, long W, double *out)
{
    if (!var || !out || N <= 0 || C <= 0 || H <= 0 || W <= 0) return ORACLE_BAD_ARG;
    for (long n = 0; n < N; ++n)
        for (long c = 0; c < C; ++c)
            for (long h = 0; h < H; ++h)
                for (long q = 0; q < W; ++q)
                    out[((n * C + c) * H + h) * W + q] = exp(var[c]);
    return ORACLE_OK;
}
