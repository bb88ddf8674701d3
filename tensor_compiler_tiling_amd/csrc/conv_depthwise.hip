// Depthwise NCHW convolution: every channel convolved with its own filter
// (the TVM tutorial "Tuning High Performance Convolution on NVIDIA GPUs"
// names depthwise convolution, in its opening, as another use of its
// template):
//
//   y[n][c][oy][ox] = sum_{ky<KH} sum_{kx<KW} xp[n][c][oy*s+ky][ox*s+kx] * w[c][0][ky][kx]
//
// with xp the input zero-padded by `pad` (inline), fp32 accumulation and
// output, and the per-channel epilogue of the convolution path.
//
// There is no reduction over channels, so nothing here is a dense
// contraction: each input is read KH*KW times from LDS but once from HBM and
// the kernel is bound by HBM (x read once, y written once).  The planes
// (n, c) are contiguous in both x and y, so they are numbered pl = n*C + c.
// One workgroup computes RB output rows (a multiple of 4) of PPW consecutive
// planes (PPW > 1 only when a whole plane is smaller than a workgroup's work):
//   - it stages the receptive field, RIN = (RB-1)*s + KH input rows of the
//     padded row width per plane, in LDS as fp32, zeros outside the image, so
//     the inner loop has no bounds tests.  The image rows a block needs are
//     one contiguous range of x (rows of consecutive planes follow each
//     other), read with 16-byte loads at 16-byte aligned addresses, up to
//     eight a lane in flight at once, plus a scalar head and tail; the zero
//     border goes to LDS words no load writes, so the two need no barrier
//     between them;
//   - the planes' taps and epilogue values follow the windows in LDS, loaded
//     together with the window (no load waits on another);
//   - each lane computes one output column over 4 consecutive rows, so the
//     lanes of a wave read consecutive LDS words (no bank conflicts at
//     stride 1) and, for the filter sizes compiled in, input rows shared by
//     the 4 outputs are read once;
//   - a workgroup takes up to about 2048 strips (8192 outputs) within 32 KB
//     of LDS, so that five fit a CU with all of their loads in flight;
//     consecutive workgroups of one XCD take neighbouring row blocks, whose
//     halo rows then meet in one L2.
// Small planes (3x3, stride 1, pad 0 or 1, rows of at most 32 pixels, 32 rows
// of output at most) take a second kernel: there the first one's index
// arithmetic (a division per staged element when a row is not a whole number
// of 16-byte vectors, two per 4-row strip) costs more than the data moves.
// A workgroup holds PPW whole planes; each staging lane copies one input row
// with 4-byte loads, and each compute lane walks one output column top to
// bottom with the filter and a 3-row window in registers (3 LDS reads and 9
// FMAs an output).  The planes' outputs are one contiguous run of y: they go
// through LDS and out in 16-byte non-temporal stores (whole lines, not read
// again by the launch).
#include "ct_device.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

namespace ct {

namespace {

constexpr int kDwThreads = 256;
constexpr int kDwMaxTaps = 256;         // KH*KW
constexpr int kDwMaxLds = 160 * 1024;   // bytes of LDS per workgroup on gfx950
constexpr int kDwPrefLds = 32 * 1024;   // plans above this only when nothing smaller fits (5 workgroups a CU)
constexpr int kDwTargetItems = 2048;    // 4-row strips a workgroup aims at

struct DwParams {
    const void* x;
    const void* w;
    float* y;
    const float* bias;
    const float* var;
    float eps;
    int NC, C, H, W, KH, KW, stride, pad, OH, OW;
    int RB;      // output rows a workgroup computes (a multiple of 4)
    int RIN;     // input rows it stages per plane: (RB-1)*stride + KH
    int WPAD;    // staged row width: (OW-1)*stride + KW
    int LDSW;    // LDS row pitch (floats): WPAD rounded up to odd
    int PPW;     // planes a workgroup computes
    int TAPS;    // LDS word of the first tap (after the PPW windows)
    int EPIW;    // LDS word of the planes' epilogue values (after the taps)
    int blocks;  // row blocks per plane: ceil(OH / RB)
    int tiles;   // workgroups with work: blocks * ceil(NC / PPW)
    int tiles8;  // tiles rounded up to a multiple of 8 (the grid)
    int epilogue;
    int vec;      // x is 16-byte aligned: vector loads
    int rowvec;   // ... and W is a multiple of the elements of a load: one row each
    double rW;    // 1 / W and 1 / (H*W), for the divisions of the staging loop
    double rHW;
    double rOW;   // 1 / OW and 1 / (RB/4 * OW), for the strip index of an item
    double rPPI;
};

// q = n / d for 0 <= n < 2^31, d > 0, rd = 1/d rounded to double: the
// product's error is far below one, so the truncated estimate is the
// quotient or one off, and one correction step fixes it.
__device__ __forceinline__ int fdiv(int n, int d, double rd) {
    int q = (int)((double)n * rd);
    const int r = n - q * d;
    q += r < 0 ? -1 : (r >= d ? 1 : 0);
    return q;
}

// Elements of one 16-byte load and their conversion to fp32.
template <int DT> struct Vec16;
template <> struct Vec16<DT_F32> {
    static constexpr int N = 4;
    static __device__ __forceinline__ float at(const uint4& u, int i) {
        return __uint_as_float(i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w);
    }
};
template <> struct Vec16<DT_F16> {
    static constexpr int N = 8;
    static __device__ __forceinline__ float at(const uint4& u, int i) {
        const unsigned w = (i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w;
        const unsigned short h = (unsigned short)((i & 1) ? (w >> 16) : (w & 0xffffu));
        return (float)__builtin_bit_cast(_Float16, h);
    }
};
template <> struct Vec16<DT_BF16> {
    static constexpr int N = 8;
    static __device__ __forceinline__ float at(const uint4& u, int i) {
        const unsigned w = (i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w;
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// One workgroup's share of the output: PPW planes from pl0 (np of them in
// the last group), output rows [oy0, oy0 + RB); image rows [iy_lo, iy_hi)
// of each plane land in the window, which in x is the local range [lo, hi)
// counted from plane pl0's first element; 16-byte vectors [va, vb) of that
// range, vector v holding local elements v*VE - m .. v*VE - m + VE - 1.
struct DwTile {
    int pl0, np, oy0, iy0, iy_lo, iy_hi, lo, hi, m, va, vb;
};

template <int DT>
__device__ __forceinline__ DwTile dw_tile(const DwParams& p, int tile, int S) {
    constexpr int VE = Vec16<DT>::N;
    DwTile t;
    const int blk = tile % p.blocks;
    t.pl0 = (tile / p.blocks) * p.PPW;
    t.np = min(p.PPW, p.NC - t.pl0);
    t.oy0 = blk * p.RB;
    t.iy0 = t.oy0 * S - p.pad;
    t.iy_lo = min(max(t.iy0, 0), p.H);
    t.iy_hi = max(min(t.iy0 + p.RIN, p.H), t.iy_lo);
    const int HW = p.H * p.W;  // < 2^31: checked by the host
    t.lo = t.iy_lo * p.W;
    t.hi = (t.np - 1) * HW + t.iy_hi * p.W;
    t.m = 0;
    t.va = t.vb = 0;
    if (p.vec) {
        t.m = (int)(((long long)t.pl0 * HW) % VE);
        t.va = (t.lo + t.m + VE - 1) / VE;
        t.vb = (t.hi + t.m) / VE;
        if (t.va > t.vb) t.va = t.vb = 0;
    }
    return t;
}

template <int DT>
__device__ __forceinline__ const uint4* dw_vectors(const DwParams& p, const DwTile& t) {
    using T = typename Elem<DT>::T;
    return reinterpret_cast<const uint4*>(static_cast<const T*>(p.x) + (long long)t.pl0 * p.H * p.W - t.m);
}

// What a tile's staging reads from global memory ahead of time: the first
// batch of 16-byte loads (vectors va + k*256 + tid, clamped to va past the
// end: in bounds, not stored), the lane's tap (tap tid of the tile's planes)
// and, for lanes below np, its plane's bias and var.
struct DwPrefetch {
    uint4 u[8];
    float tw, eb, ev;
};

template <int DT>
__device__ __forceinline__ void dw_issue(const DwParams& p, const DwTile& t, DwPrefetch& f, int TT, int tid) {
    using T = typename Elem<DT>::T;
    if (t.va < t.vb) {
        const uint4* xv = dw_vectors<DT>(p, t);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int v = t.va + k * kDwThreads + tid;
            f.u[k] = xv[v < t.vb ? v : t.va];
        }
    }
    // clamped indices: every lane loads, lanes past the end load a valid word
    const T* w = static_cast<const T*>(p.w);
    const int i = min(tid, t.np * TT - 1);
    const int pp = i / TT;
    f.tw = Elem<DT>::to_f32(w[(long long)((t.pl0 + pp) % p.C) * TT + (i - pp * TT)]);
    // bias and var always point at C readable floats (the host substitutes
    // what the epilogue does not read), so these loads need no branch
    const int c = (t.pl0 + min(tid, t.np - 1)) % p.C;
    f.eb = p.bias[c];
    f.ev = p.var[c];
}

// Write one batch of loaded vectors (from v0) into the window.
template <int DT>
__device__ __forceinline__ void dw_scatter(const DwParams& p, const DwTile& t, const uint4 (&u)[8], int v0,
                                           float* lds, int tid) {
    constexpr int VE = Vec16<DT>::N;
    const int HW = p.H * p.W;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int v = v0 + k * kDwThreads + tid;
        if (v < t.vb) {
            if (p.rowvec) {
                // m = 0 and the VE elements share a row: one slot, VE words
                const int e = v * VE;
                const int pp = fdiv(e, HW, p.rHW);
                const int rem = e - pp * HW;
                const int iy = fdiv(rem, p.W, p.rW);
                const int j = rem - iy * p.W + p.pad;
                if (iy >= t.iy_lo && iy < t.iy_hi) {
                    float* dst = lds + (pp * p.RIN + iy - t.iy0) * p.LDSW + j;
#pragma unroll
                    for (int i = 0; i < VE; ++i)
                        if (j + i < p.WPAD) dst[i] = Vec16<DT>::at(u[k], i);
                }
            } else {
                // the first element's (plane, row, column), then one step at a
                // time with carries (a vector may cross rows and planes)
                const int e = v * VE - t.m;
                int pp = fdiv(e, HW, p.rHW);
                const int rem = e - pp * HW;
                int iy = fdiv(rem, p.W, p.rW);
                int ix = rem - iy * p.W;
#pragma unroll
                for (int i = 0; i < VE; ++i) {
                    const int j = ix + p.pad;
                    if (iy >= t.iy_lo && iy < t.iy_hi && j < p.WPAD)
                        lds[(pp * p.RIN + iy - t.iy0) * p.LDSW + j] = Vec16<DT>::at(u[k], i);
                    if (++ix == p.W) {
                        ix = 0;
                        if (++iy == p.H) {
                            iy = 0;
                            ++pp;
                        }
                    }
                }
            }
        }
    }
}

// Stage a tile's windows and taps: the zero border (rows outside the image,
// then the padding columns of image rows: words no load writes), the scalar
// head and tail of the range (all of it without vectors), the first batch of
// vectors from u (already in flight) and any further batches.
template <int DT>
__device__ __forceinline__ void dw_stage(const DwParams& p, const DwTile& t, DwPrefetch& f, int TT,
                                         float* lds, int tid) {
    using T = typename Elem<DT>::T;
    constexpr int VE = Vec16<DT>::N;
    const int HW = p.H * p.W;
    const int drows = t.iy_hi - t.iy_lo;
    const int zr_top = drows > 0 ? t.iy_lo - t.iy0 : p.RIN;
    const int zr_bot = drows > 0 ? t.iy0 + p.RIN - t.iy_hi : 0;
    const int zrows = zr_top + zr_bot;
    const int nz = t.np * zrows * p.WPAD;
    const double rWPAD = 1.0 / (double)p.WPAD, rZ = 1.0 / (double)max(zrows, 1);
    for (int e = tid; e < nz; e += kDwThreads) {
        const int row = fdiv(e, p.WPAD, rWPAD);
        const int j = e - row * p.WPAD;
        const int pp = fdiv(row, zrows, rZ);
        const int k = row - pp * zrows;
        const int r = k < zr_top ? k : p.RIN - zr_bot + (k - zr_top);
        lds[(pp * p.RIN + r) * p.LDSW + j] = 0.0f;
    }
    const int left = min(p.pad, p.WPAD);             // columns before the image
    const int right = max(p.WPAD - p.pad - p.W, 0);  // columns past the image
    const int pc = left + right;
    const int nc = t.np * drows * pc;
    const double rPC = 1.0 / (double)max(pc, 1), rD = 1.0 / (double)max(drows, 1);
    for (int e = tid; e < nc; e += kDwThreads) {
        const int row = fdiv(e, pc, rPC);
        const int k = e - row * pc;
        const int pp = fdiv(row, drows, rD);
        const int r = zr_top + (row - pp * drows);
        const int j = k < left ? k : p.pad + p.W + (k - left);
        lds[(pp * p.RIN + r) * p.LDSW + j] = 0.0f;
    }
    const T* xb = static_cast<const T*>(p.x) + (long long)t.pl0 * HW;
    const bool vecs = t.va < t.vb;
    const int head_end = vecs ? t.va * VE - t.m : t.hi;
    const int tail_beg = vecs ? t.vb * VE - t.m : t.hi;
    auto put = [&](int e) {
        const int pp = fdiv(e, HW, p.rHW);
        const int rem = e - pp * HW;
        const int iy = fdiv(rem, p.W, p.rW);
        const int j = rem - iy * p.W + p.pad;
        if (iy >= t.iy_lo && iy < t.iy_hi && j < p.WPAD)
            lds[(pp * p.RIN + iy - t.iy0) * p.LDSW + j] = Elem<DT>::to_f32(xb[e]);
    };
    // the prefetched words first, then what still has to be loaded
    float* tap = lds + p.TAPS;
    if (tid < t.np * TT) tap[tid] = f.tw;
    if (tid < t.np) {
        lds[p.EPIW + 2 * tid] = p.epilogue != EPI_NONE ? f.eb : 0.0f;
        lds[p.EPIW + 2 * tid + 1] = p.epilogue == EPI_EXP_BIAS_RSQRT ? dev_rsqrt(f.ev + p.eps) : 1.0f;
    }
    if (vecs) dw_scatter<DT>(p, t, f.u, t.va, lds, tid);
    if (vecs) {
        const uint4* xv = dw_vectors<DT>(p, t);
        for (int v0 = t.va + 8 * kDwThreads; v0 < t.vb; v0 += 8 * kDwThreads) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int v = v0 + k * kDwThreads + tid;
                f.u[k] = xv[v < t.vb ? v : t.va];
            }
            dw_scatter<DT>(p, t, f.u, v0, lds, tid);
        }
    }
    for (int e = t.lo + tid; e < head_end; e += kDwThreads) put(e);
    for (int e = tail_beg + tid; e < t.hi; e += kDwThreads) put(e);
    const T* w = static_cast<const T*>(p.w);
    for (int i = kDwThreads + tid; i < t.np * TT; i += kDwThreads) {
        const int pp = i / TT;
        const int c = (t.pl0 + pp) % p.C;
        tap[i] = Elem<DT>::to_f32(w[(long long)c * TT + (i - pp * TT)]);
    }
}

// One workgroup per tile.  Workgroup b runs on XCD b % 8, and XCD x takes
// tiles [x*TX, (x+1)*TX), so neighbouring row blocks, which share halo rows,
// meet in one L2.  The tile's loads (window vectors, taps, epilogue values)
// are all issued before any of them is used.
template <int DT, int KH_, int KW_, int S_>
__global__ __launch_bounds__(kDwThreads) void conv_depthwise_kernel(DwParams p) {
    extern __shared__ float lds[];  // PPW x [RIN][LDSW] windows, taps, epilogue values
    const int tid = threadIdx.x;
    const int KH = KH_ > 0 ? KH_ : p.KH;
    const int KW = KW_ > 0 ? KW_ : p.KW;
    const int S = S_ > 0 ? S_ : p.stride;
    const int TT = KH * KW;
    const int tile = (blockIdx.x & 7) * (p.tiles8 >> 3) + (blockIdx.x >> 3);
    if (tile >= p.tiles) return;

    DwPrefetch f;
    const DwTile t = dw_tile<DT>(p, tile, S);
    dw_issue<DT>(p, t, f, TT, tid);
    dw_stage<DT>(p, t, f, TT, lds, tid);
    __syncthreads();

    // 4-row strips: item = (plane, strip g, column ox)
    const int strips = p.RB / 4;
    const int per_plane_items = strips * p.OW;
    const float* tap = lds + p.TAPS;
    for (int item = tid; item < t.np * per_plane_items; item += kDwThreads) {
        const int pp = fdiv(item, per_plane_items, p.rPPI);
        const int rem = item - pp * per_plane_items;
        const int g = fdiv(rem, p.OW, p.rOW);
        const int ox = rem - g * p.OW;
        const float* win = lds + (pp * p.RIN + 4 * g * S) * p.LDSW + ox * S;
        const float* tp = tap + pp * TT;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (KH_ > 0) {
            float tr[KH_ * KW_];
#pragma unroll
            for (int i = 0; i < KH_ * KW_; ++i) tr[i] = tp[i];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int ky = 0; ky < KH_; ++ky)
#pragma unroll
                    for (int kx = 0; kx < KW_; ++kx)
                        acc[i] = __builtin_fmaf(win[(i * S_ + ky) * p.LDSW + kx], tr[ky * KW_ + kx], acc[i]);
        } else {
            for (int ky = 0; ky < KH; ++ky)
                for (int kx = 0; kx < KW; ++kx) {
                    const float wv = tp[ky * KW + kx];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i] = __builtin_fmaf(win[(i * S + ky) * p.LDSW + kx], wv, acc[i]);
                }
        }
        const int pl = t.pl0 + pp;
        const float e_b = lds[p.EPIW + 2 * pp], e_r = lds[p.EPIW + 2 * pp + 1];
        const int oy = t.oy0 + 4 * g;
        float* yp = p.y + (long long)pl * p.OH * p.OW + (long long)oy * p.OW + ox;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (oy + i < p.OH) yp[(long long)i * p.OW] = apply_epilogue(p.epilogue, acc[i], e_b, e_r);
    }
}

// ---- small planes ----------------------------------------------------------
typedef float floatv4 __attribute__((ext_vector_type(4)));  // for the non-temporal 16-byte stores

struct DwSmallParams {
    const void* x;
    const void* w;
    float* y;
    const float* bias;
    const float* var;
    float eps;
    int NC, C, H, W, pad, OH, OW;
    int HP;       // staged rows per plane: H + 2*pad
    int LDSW;     // LDS row pitch (floats): W + 2*pad rounded up to odd
    int PPW;      // planes a workgroup holds
    int groups;   // workgroups with work: ceil(NC / PPW)
    int epilogue;
    double rHP, rOW;  // 1 / HP and 1 / OW for the lane-to-(plane, row/column) divisions
};

constexpr int kDwSmallMaxW = 32;
constexpr int kDwSmallMaxOH = 32;
constexpr int kDwSmallLds = 32 * 1024;

// One input row of plane pl, image row iy, into LDS row `dst` (WPAD = W +
// 2*pad floats, the padding columns zero); rows outside the image or past
// the last plane are all zeros.  16-bit rows are read as 4-byte words (W even,
// x 4-byte aligned), fp32 rows as words, all of a row's loads in flight
// before its writes.
template <int DT>
__device__ __forceinline__ void dws_stage_row(const DwSmallParams& p, int pl, int iy, float* dst) {
    using T = typename Elem<DT>::T;
    constexpr bool H16 = DT != DT_F32;
    constexpr int MAXD = H16 ? kDwSmallMaxW / 2 : kDwSmallMaxW;  // words of the widest row
    const int WPAD = p.W + 2 * p.pad;
    if (pl < p.NC && iy >= 0 && iy < p.H) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(static_cast<const T*>(p.x) +
                                                                ((long long)pl * p.H + iy) * p.W);
        const int nd = H16 ? p.W / 2 : p.W;
        uint32_t v[MAXD];
#pragma unroll
        for (int i = 0; i < MAXD; ++i) v[i] = i < nd ? src[i] : 0u;
        if (p.pad) {
            dst[0] = 0.0f;
            dst[WPAD - 1] = 0.0f;
        }
        float* d = dst + p.pad;
#pragma unroll
        for (int i = 0; i < MAXD; ++i) {
            if (i < nd) {
                if constexpr (H16) {
                    d[2 * i] = Elem<DT>::to_f32(__builtin_bit_cast(T, (uint16_t)(v[i] & 0xffffu)));
                    d[2 * i + 1] = Elem<DT>::to_f32(__builtin_bit_cast(T, (uint16_t)(v[i] >> 16)));
                } else {
                    d[i] = __uint_as_float(v[i]);
                }
            }
        }
    } else {
        for (int j = 0; j < WPAD; ++j) dst[j] = 0.0f;
    }
}

template <int DT>
__global__ __launch_bounds__(kDwThreads) void conv_depthwise_small_kernel(DwSmallParams p) {
    using T = typename Elem<DT>::T;
    extern __shared__ float lds[];  // PPW x [HP][LDSW]
    const int tid = threadIdx.x;
    const int grp = blockIdx.x;
    if (grp >= p.groups) return;
    const int pl0 = grp * p.PPW;

    // this lane's output column and its filter and epilogue values, loaded
    // first (their latency overlaps the staging)
    const int pp = fdiv(tid, p.OW, p.rOW);
    const int ox = tid - pp * p.OW;
    const int pl = pl0 + pp;
    const bool active = pp < p.PPW && pl < p.NC;
    const int c = (active ? pl : pl0) % p.C;
    float tw[9];
    const T* w = static_cast<const T*>(p.w) + (long long)c * 9;
#pragma unroll
    for (int i = 0; i < 9; ++i) tw[i] = Elem<DT>::to_f32(w[i]);
    // bias and var always point at C readable floats (the host substitutes
    // what the epilogue does not read)
    const float e_b = p.epilogue != EPI_NONE ? p.bias[c] : 0.0f;
    const float e_v = p.var[c];

    // staging: row r = (plane r / HP, row r % HP) of the workgroup's planes,
    // one row a lane
    for (int r = tid; r < p.PPW * p.HP; r += kDwThreads) {
        const int q = fdiv(r, p.HP, p.rHP);
        const int rr = r - q * p.HP;
        dws_stage_row<DT>(p, pl0 + q, rr - p.pad, lds + r * p.LDSW);
    }
    __syncthreads();

    // the column, top to bottom, into registers
    float res[kDwSmallMaxOH];
    if (active) {
        const float e_r = p.epilogue == EPI_EXP_BIAS_RSQRT ? dev_rsqrt(e_v + p.eps) : 1.0f;
        const float* col = lds + pp * p.HP * p.LDSW + ox;
        float a0 = col[0], a1 = col[1], a2 = col[2];
        float b0 = col[p.LDSW], b1 = col[p.LDSW + 1], b2 = col[p.LDSW + 2];
#pragma unroll
        for (int oy = 0; oy < kDwSmallMaxOH; ++oy) {
            if (oy < p.OH) {
                const float* r2 = col + (oy + 2) * p.LDSW;
                const float c0 = r2[0], c1 = r2[1], c2 = r2[2];
                float acc = a0 * tw[0];
                acc = __builtin_fmaf(a1, tw[1], acc);
                acc = __builtin_fmaf(a2, tw[2], acc);
                acc = __builtin_fmaf(b0, tw[3], acc);
                acc = __builtin_fmaf(b1, tw[4], acc);
                acc = __builtin_fmaf(b2, tw[5], acc);
                acc = __builtin_fmaf(c0, tw[6], acc);
                acc = __builtin_fmaf(c1, tw[7], acc);
                acc = __builtin_fmaf(c2, tw[8], acc);
                res[oy] = apply_epilogue(p.epilogue, acc, e_b, e_r);
                a0 = b0; a1 = b1; a2 = b2;
                b0 = c0; b1 = c1; b2 = c2;
            }
        }
    }
    // The workgroup's output, planes pl0 .. pl0+np-1, is one contiguous run
    // of y in y's own layout: it goes through LDS (over the windows, no longer
    // read) and out in 16-byte stores (4-byte ones when y's run is not
    // 16-byte aligned).
    __syncthreads();
    const int OHW = p.OH * p.OW;
    if (active) {
        float* o = lds + pp * OHW + ox;
#pragma unroll
        for (int oy = 0; oy < kDwSmallMaxOH; ++oy)
            if (oy < p.OH) o[oy * p.OW] = res[oy];
    }
    __syncthreads();
    const int np = min(p.PPW, p.NC - pl0);
    const int total = np * OHW;  // <= PPW * HP * LDSW floats: within the windows
    float* yb = p.y + (long long)pl0 * OHW;
    if (reinterpret_cast<uintptr_t>(yb) % 16 == 0) {
        const int n4 = total >> 2;
        for (int i = tid; i < n4; i += kDwThreads)
            __builtin_nontemporal_store(reinterpret_cast<const floatv4*>(lds)[i], &reinterpret_cast<floatv4*>(yb)[i]);
        for (int i = 4 * n4 + tid; i < total; i += kDwThreads) yb[i] = lds[i];
    } else {
        for (int i = tid; i < total; i += kDwThreads) yb[i] = lds[i];
    }
}

}  // namespace

namespace {

int plan_within(int NC, int OH, int OW, int KH, int KW, int stride, int budget, int* RB, int* RIN,
                int* WPAD, int* LDSW, int* PPW, int* TAPS) {
    *WPAD = (OW - 1) * stride + KW;
    *LDSW = *WPAD | 1;  // odd pitch: the rows of a strip start on different banks
    const int strips_plane = (OH + 3) / 4;
    int g = OW >= kDwTargetItems ? 1 : kDwTargetItems / OW;
    if (g > strips_plane) g = strips_plane;
    int ppw = 1;
    if (g == strips_plane) {
        ppw = kDwTargetItems / (g * OW);
        if (ppw < 1) ppw = 1;
        if (ppw > NC) ppw = NC;
    }
    const int taps = KH * KW;
    for (;;) {
        const long long rin = (long long)(4 * g - 1) * stride + KH;
        const long long words = (long long)ppw * rin * (*LDSW);
        const long long bytes = (words + (long long)ppw * (taps + 2)) * 4;
        if (bytes <= budget) {
            *RB = 4 * g;
            *RIN = (int)rin;
            *PPW = ppw;
            *TAPS = (int)words;
            return (int)bytes;
        }
        if (ppw > 1) ppw /= 2;
        else if (g > 1) --g;
        else return -1;
    }
}

}  // namespace

// Work split of a depthwise launch: RB rows (a multiple of 4) of PPW planes a
// workgroup, about kDwTargetItems 4-row strips, within 32 KB of LDS (five
// workgroups a CU, as many as the registers allow) or, when four output rows
// of one plane need more, within the 160 KB a workgroup may hold.  Returns
// the LDS bytes, or -1 if four output rows of one plane do not fit even
// there.
int depthwise_plan(int NC, int OH, int OW, int KH, int KW, int stride, int* RB, int* RIN, int* WPAD,
                   int* LDSW, int* PPW, int* TAPS) {
    const int b = plan_within(NC, OH, OW, KH, KW, stride, kDwPrefLds, RB, RIN, WPAD, LDSW, PPW, TAPS);
    if (b >= 0) return b;
    return plan_within(NC, OH, OW, KH, KW, stride, kDwMaxLds, RB, RIN, WPAD, LDSW, PPW, TAPS);
}

namespace {

template <int DT, int KH_, int KW_, int S_>
hipError_t launch_dw(const DwParams& p, int bytes, hipStream_t stream) {
    auto kern = conv_depthwise_kernel<DT, KH_, KW_, S_>;
    static std::atomic<int> lds_limit{65536};
    if (bytes > lds_limit.load(std::memory_order_relaxed)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e;
        }
        lds_limit.store(bytes, std::memory_order_relaxed);
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)p.tiles8), dim3(kDwThreads), bytes, stream, p);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const DwParams& p, int bytes, hipStream_t stream) {
    const int k = p.KH == p.KW ? p.KH : 0;
    if (k == 3 && p.stride == 1) return launch_dw<DT, 3, 3, 1>(p, bytes, stream);
    if (k == 3 && p.stride == 2) return launch_dw<DT, 3, 3, 2>(p, bytes, stream);
    if (k == 5 && p.stride == 1) return launch_dw<DT, 5, 5, 1>(p, bytes, stream);
    if (k == 5 && p.stride == 2) return launch_dw<DT, 5, 5, 2>(p, bytes, stream);
    if (k == 7 && p.stride == 1) return launch_dw<DT, 7, 7, 1>(p, bytes, stream);
    if (k == 7 && p.stride == 2) return launch_dw<DT, 7, 7, 2>(p, bytes, stream);
    return launch_dw<DT, 0, 0, 0>(p, bytes, stream);
}

}  // namespace

// Shapes are checked by the caller (positive sizes, output not empty, the
// plan fits); this returns hipErrorInvalidValue for what it cannot launch.
hipError_t launch_depthwise(const void* x, const void* w, float* y, int N, int C, int H, int W, int KH, int KW,
                            int stride, int pad, int dtype, int epilogue, const float* bias, const float* var,
                            float eps, hipStream_t stream) {
    DwParams p{};
    p.x = x; p.w = w; p.y = y; p.bias = bias; p.var = var; p.eps = eps;
    // stand-ins for the per-channel arrays the epilogue does not read: the
    // kernel loads both unconditionally and discards them (y holds at least
    // C floats)
    if (epilogue == EPI_NONE) p.bias = y;
    if (epilogue != EPI_EXP_BIAS_RSQRT) p.var = p.bias;
    p.NC = N * C; p.C = C; p.H = H; p.W = W; p.KH = KH; p.KW = KW; p.stride = stride; p.pad = pad;
    p.OH = (H + 2 * pad - KH) / stride + 1;
    p.OW = (W + 2 * pad - KW) / stride + 1;
    p.epilogue = epilogue;
    if (KH * KW > kDwMaxTaps || p.OH <= 0 || p.OW <= 0) return hipErrorInvalidValue;
    if (KH == 3 && KW == 3 && stride == 1 && pad <= 1 && W <= kDwSmallMaxW && p.OH <= kDwSmallMaxOH &&
        reinterpret_cast<uintptr_t>(x) % 4 == 0 && (dtype == DT_F32 || W % 2 == 0)) {
        // small planes: whole planes a workgroup, one output column a lane
        DwSmallParams q{};
        q.x = x; q.w = w; q.y = y; q.bias = p.bias; q.var = p.var; q.eps = eps;
        q.NC = p.NC; q.C = C; q.H = H; q.W = W; q.pad = pad; q.OH = p.OH; q.OW = p.OW;
        q.HP = H + 2 * pad;
        q.LDSW = (W + 2 * pad) | 1;  // odd pitch: a wave's rows start on different banks
        q.PPW = std::min(kDwThreads / q.OW, kDwSmallLds / (q.HP * q.LDSW * 4));
        // a power of two: with N*C one too, the grid is whole rounds of
        // workgroups (18 planes of 14x14 left the last round 78% full)
        while (q.PPW & (q.PPW - 1)) q.PPW &= q.PPW - 1;
        q.groups = (q.NC + q.PPW - 1) / q.PPW;
        q.epilogue = epilogue;
        q.rHP = 1.0 / (double)q.HP;
        q.rOW = 1.0 / (double)q.OW;
        const int bytes = q.PPW * q.HP * q.LDSW * 4;
        (void)hipGetLastError();
        switch (dtype) {
            case DT_F32:
                hipLaunchKernelGGL(conv_depthwise_small_kernel<DT_F32>, dim3((unsigned)q.groups), dim3(kDwThreads),
                                   bytes, stream, q);
                break;
            case DT_F16:
                hipLaunchKernelGGL(conv_depthwise_small_kernel<DT_F16>, dim3((unsigned)q.groups), dim3(kDwThreads),
                                   bytes, stream, q);
                break;
            case DT_BF16:
                hipLaunchKernelGGL(conv_depthwise_small_kernel<DT_BF16>, dim3((unsigned)q.groups), dim3(kDwThreads),
                                   bytes, stream, q);
                break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if ((long long)H * W >= (1LL << 31)) return hipErrorInvalidValue;
    const int bytes = depthwise_plan(p.NC, p.OH, p.OW, KH, KW, stride, &p.RB, &p.RIN, &p.WPAD, &p.LDSW,
                                     &p.PPW, &p.TAPS);
    if (bytes < 0) return hipErrorInvalidValue;
    // the local element offsets of a workgroup's planes stay below 2^31
    if ((long long)p.PPW * H * W >= (1LL << 31)) p.PPW = 1;
    p.EPIW = p.TAPS + p.PPW * KH * KW;
    p.blocks = (p.OH + p.RB - 1) / p.RB;
    const long long tiles = (long long)p.blocks * ((p.NC + p.PPW - 1) / p.PPW);
    if (tiles > 0x7ffffff0LL) return hipErrorInvalidValue;
    p.tiles = (int)tiles;
    p.tiles8 = (p.tiles + 7) & ~7;
    p.vec = (reinterpret_cast<uintptr_t>(x) % 16) == 0;
    p.rowvec = p.vec && W % (dtype == DT_F32 ? 4 : 8) == 0;
    p.rW = 1.0 / (double)W;
    p.rHW = 1.0 / (double)((long long)H * W);
    p.rOW = 1.0 / (double)p.OW;
    p.rPPI = 1.0 / (double)((long long)(p.RB / 4) * p.OW);
    switch (dtype) {
        case DT_F32: return launch_dt<DT_F32>(p, bytes, stream);
        case DT_F16: return launch_dt<DT_F16>(p, bytes, stream);
        case DT_BF16: return launch_dt<DT_BF16>(p, bytes, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ct
