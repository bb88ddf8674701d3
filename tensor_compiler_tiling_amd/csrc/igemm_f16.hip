// fp16 / bf16 implicit-GEMM convolution on CDNA4 matrix cores
// (v_mfma_f32_32x32x16_f16 / _bf16: 16-bit inputs multiplied exactly and
// accumulated in fp32), with split reduction across workgroups and the fused
// per-channel epilogue.  Output is fp32, as the TVM tutorial's template
// declares it ("Tuning High Performance Convolution on NVIDIA GPUs", Step 1:
// out_dtype float32).
//
// The half-precision instruction takes 8 consecutive reduction values per
// lane, while NCHW data is contiguous along pixels, not along the reduction.
// The reduction of a stage (kc channels x T taps) is therefore ordered in
// groups of 8 channels at one tap, g = tap * (kc/8) + channel/8, and both
// operands are stored channel-fastest in LDS:
//   W tile  [tile_m][group][8]        (transposed from [co][c][tap] while staged)
//   window  [row][col][channel]       (transposed from NCHW while staged)
// so an A or B fragment of one instruction is one 16-byte LDS read.  Global
// loads of the next stage are issued into registers before the current
// stage's matrix instructions, and written to LDS after them.
#include "ct_device.hpp"
#include "igemm_common.hpp"

#include <atomic>

namespace ct {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

template <int DT> struct HMfma;
template <> struct HMfma<DT_F16> {
    static __device__ __forceinline__ floatx16 mma(uint4v a, uint4v b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                     __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
    }
};
template <> struct HMfma<DT_BF16> {
    static __device__ __forceinline__ floatx16 mma(uint4v a, uint4v b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

// LDS carve-up in 16-bit units (host and kernel share it).
struct HLayout {
    int kcp;      // channels per stage rounded up to 8
    int cgs;      // channel groups of 8 per stage
    int groups;   // T * cgs
    int gp;       // groups rounded up to 2 (one instruction = 2 groups)
    int wst;      // W row stride: (gp + 1) * 8, odd multiple of 16 bytes
    int kcs;      // window pixel stride: odd multiple of 8 halves >= kcp + 8
    int xs_off;   // window [R*Wp][kcs]
    int ktab_off; // (in 16-bit units; 4-byte aligned) per-group offsets [gp]
    int epi_off;  // bias, rsqrt [2][tile_m] floats
    int red_off;  // unused (no cross-wave reduction)
    int halves;
};

__host__ __device__ inline HLayout h_layout(int tile_m, int kc, int T, int R, int Wp) {
    HLayout L;
    L.kcp = round_up(kc, 8);
    L.cgs = L.kcp / 8;
    L.groups = T * L.cgs;
    L.gp = round_up(L.groups, 2);
    L.wst = (L.gp + 1) * 8;
    L.kcs = (L.cgs + 1 + (L.cgs & 1)) * 8;
    L.xs_off = tile_m * L.wst;
    L.ktab_off = L.xs_off + R * Wp * L.kcs;
    L.epi_off = L.ktab_off + 2 * L.gp;
    L.red_off = 0;
    L.halves = L.epi_off + 4 * tile_m;
    return L;
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

template <int DT, int WM, int WN, int RM, int RN, int WTM, int XTM>
struct HCfg {
    static constexpr int TILE_M = WM * RM * 32;
    static constexpr int TILE_N = WN * RN * 32;
    static constexpr int THREADS = WM * WN * 64;
};

// Staging plans.  W: a task is (row m, channel group cg): 8 channels x T taps
// of one W row, contiguous in global memory.  Fast when T is 9 or 1 and the
// run is 16-byte aligned (16*T bytes -> T vector loads); otherwise element by
// element.  Window: a task is (pixel, channel group): 8 channel values of one
// padded-window pixel (8 loads of 2 bytes, zero outside the image).
template <int DT, int WM, int WN, int RM, int RN, int WTM, int XTM>
__global__ __launch_bounds__(WM * WN * 64) void igemm_h_kernel(ConvParams p) {
    fetch_kernargs(p);
    using Cfg = HCfg<DT, WM, WN, RM, RN, WTM, XTM>;
    constexpr int TILE_M = Cfg::TILE_M, TILE_N = Cfg::TILE_N, THREADS = Cfg::THREADS;
    extern __shared__ __align__(16) uint16_t hs[];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int lj = lane & 31;
    const int lh = lane >> 5;

    const HLayout L = h_layout(TILE_M, p.kc, p.T, p.R, p.Wp);
    uint16_t* Ws = hs;
    uint16_t* Xs = hs + L.xs_off;
    int* ktab = reinterpret_cast<int*>(hs + L.ktab_off);
    float* e_bias = reinterpret_cast<float*>(hs + L.epi_off);
    float* e_rs = e_bias + TILE_M;

    const int tiles = p.tiles_m * p.tiles_n;
    const int tile = blockIdx.x % tiles;
    const int split = blockIdx.x / tiles;
    const int tm = tile % p.tiles_m;
    const int tn = tile / p.tiles_m;
    const int co0 = tm * TILE_M;
    const long long p0 = (long long)tn * TILE_N;
    const long long n_first = p0 / p.OHW;
    const int oy_first = (int)((p0 % p.OHW) / p.OW);
    const long long vr_first = n_first * p.Hp + (long long)oy_first * p.stride;
    const long long HW = (long long)p.H * p.W;

    const uint16_t* __restrict__ xg = static_cast<const uint16_t*>(p.x);
    const uint16_t* __restrict__ wg = static_cast<const uint16_t*>(p.w);

    // ---- per-lane B columns --------------------------------------------------
    int pbase[RN];       // window pixel index of the column's (0,0) tap
    long long yoff[RN];  // y offset of (n, 0, oy, ox); -1 past P
#pragma unroll
    for (int rn = 0; rn < RN; ++rn) {
        const long long pc = p0 + (long long)(wn * RN + rn) * 32 + lj;
        pbase[rn] = 0;
        yoff[rn] = -1;
        if (pc < p.P) {
            const long long n = pc / p.OHW;
            const int rem = (int)(pc - n * p.OHW);
            const int oy = rem / p.OW;
            const int ox = rem - oy * p.OW;
            pbase[rn] = (int)(n * p.Hp + (long long)oy * p.stride - vr_first) * p.Wp + ox * p.stride;
            yoff[rn] = n * (long long)p.CO * p.OHW + rem;
        }
    }

    // ---- tables: group offsets, epilogue; zero the W padding groups ----------
    for (int g = tid; g < L.gp; g += THREADS) {
        int off = -1;
        if (g < L.groups) {
            const int t = g / L.cgs;
            const int cg = g - t * L.cgs;
            const int ky = t / p.KW;
            const int kx = t - ky * p.KW;
            off = (ky * p.Wp + kx) * L.kcs + cg * 8;
        }
        ktab[g] = off;
    }
    for (int m = tid; m < TILE_M; m += THREADS) {
        const int co = co0 + m;
        float b = 0.0f, r = 1.0f;
        if (co < p.CO) {
            if (p.epilogue != EPI_NONE) b = p.bias[co];
            if (p.epilogue == EPI_EXP_BIAS_RSQRT) r = dev_rsqrt(p.var[co] + p.eps);
        }
        e_bias[m] = b;
        e_rs[m] = r;
    }
    if (L.gp > L.groups)  // the odd group's A fragment must read zeros
        for (int m = tid; m < TILE_M; m += THREADS)
            *reinterpret_cast<uint4v*>(Ws + m * L.wst + L.groups * 8) = uint4v{0u, 0u, 0u, 0u};

    floatx16 acc[RM][RN];
#pragma unroll
    for (int rm = 0; rm < RM; ++rm)
#pragma unroll
        for (int rn = 0; rn < RN; ++rn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rm][rn][r] = 0.0f;

    // ---- staging ---------------------------------------------------------------
    // Task assignment is fixed for the whole kernel, so each task's source
    // offset (without the stage's channel base) and LDS destination are
    // computed once.
    const int n_wtasks = TILE_M * L.cgs;
    const int n_xtasks = p.R * p.Wp * L.cgs;
    const bool w_fast = (p.T == 9 || p.T == 1) && ((p.K & 7) == 0) &&
                        ((reinterpret_cast<uintptr_t>(wg) & 15) == 0);
    long long wsrc[WTM];  // W run start without c0*T; -1: row past CO or no task
    int wdst[WTM];        // LDS offset of the task's group 0 (tap 0)
    int wcb[WTM];         // first channel of the task's group within the stage
#pragma unroll
    for (int j = 0; j < WTM; ++j) {
        const int task = tid + j * THREADS;
        wsrc[j] = -1;
        wdst[j] = 0;
        wcb[j] = 0;
        if (task < n_wtasks) {
            const int m = task / L.cgs;
            const int cg = task - m * L.cgs;
            wdst[j] = m * L.wst + cg * 8;
            wcb[j] = cg * 8;
            if (co0 + m < p.CO) wsrc[j] = (long long)(co0 + m) * p.K + (long long)cg * 8 * p.T;
        }
    }
    long long xsrc[XTM];  // element offset of channel (cg*8) at the pixel, without c0*HW; -1: zero
    int xdst[XTM];        // LDS offset; -1: no task
    int xcg[XTM];
#pragma unroll
    for (int j = 0; j < XTM; ++j) {
        const int task = tid + j * THREADS;
        xsrc[j] = -1;
        xdst[j] = -1;
        xcg[j] = 0;
        if (task < n_xtasks) {
            const int cg = task / (p.R * p.Wp);
            const int pix = task - cg * (p.R * p.Wp);
            const int r = pix / p.Wp;
            const int col = pix - r * p.Wp;
            const long long vr = vr_first + r;
            const long long n = vr / p.Hp;
            const int iy = (int)(vr - n * p.Hp) - p.pad;
            const int ix = col - p.pad;
            xdst[j] = pix * L.kcs + cg * 8;
            xcg[j] = cg;
            if (n < p.N && iy >= 0 && iy < p.H && ix >= 0 && ix < p.W)
                xsrc[j] = (n * p.CI + cg * 8) * HW + (long long)iy * p.W + ix;
        }
    }
    uint4v wreg[WTM][9];  // fast W path: T 16-byte loads per task
    uint32_t xreg[XTM][4];

    // the fast W path copies whole 8-channel groups, so it needs the stage's
    // channel base and count to be multiples of 8
    auto w_fast_stage = [&](int c0, int cvalid) {
        return w_fast && ((c0 & 7) == 0) && ((cvalid & 7) == 0);
    };

    auto load_stage = [&](int c0, int cvalid) {
        if (w_fast_stage(c0, cvalid)) {
#pragma unroll
            for (int j = 0; j < WTM; ++j) {
                const bool ok = wsrc[j] >= 0 && wcb[j] + 8 <= cvalid;
                const uint4v* src = reinterpret_cast<const uint4v*>(
                    wg + (ok ? wsrc[j] + (long long)c0 * p.T : 0));
                if (p.T == 9) {
#pragma unroll
                    for (int q = 0; q < 9; ++q) wreg[j][q] = ok ? src[q] : uint4v{0u, 0u, 0u, 0u};
                } else {
                    wreg[j][0] = ok ? src[0] : uint4v{0u, 0u, 0u, 0u};
                }
            }
        }
#pragma unroll
        for (int j = 0; j < XTM; ++j) {
            uint16_t v[8];
            const bool in = xsrc[j] >= 0;
            const long long base = in ? xsrc[j] + (long long)c0 * HW : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = (in && xcg[j] * 8 + i < cvalid) ? xg[base + i * HW] : (uint16_t)0;
#pragma unroll
            for (int i = 0; i < 4; ++i) xreg[j][i] = pack2(v[2 * i], v[2 * i + 1]);
        }
    };

    auto store_stage = [&](int c0, int cvalid) {
        if (w_fast_stage(c0, cvalid)) {
#pragma unroll
            for (int j = 0; j < WTM; ++j) {
                if (tid + j * THREADS >= n_wtasks) continue;
                uint16_t* dst = Ws + wdst[j];
                if (p.T == 9) {
                    // element c*9 + t of the run goes to group t*cgs + cg, lane c
                    const uint32_t* in = reinterpret_cast<const uint32_t*>(&wreg[j][0]);
#pragma unroll
                    for (int t = 0; t < 9; ++t) {
                        uint16_t e[8];
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const int idx = c * 9 + t;
                            const uint32_t wrd = in[idx >> 1];
                            e[c] = (idx & 1) ? (uint16_t)(wrd >> 16) : (uint16_t)(wrd & 0xffffu);
                        }
                        uint4v o;
                        o.x = pack2(e[0], e[1]);
                        o.y = pack2(e[2], e[3]);
                        o.z = pack2(e[4], e[5]);
                        o.w = pack2(e[6], e[7]);
                        *reinterpret_cast<uint4v*>(dst + t * L.cgs * 8) = o;
                    }
                } else {
                    *reinterpret_cast<uint4v*>(dst) = wreg[j][0];
                }
            }
        } else {
            // element by element: W[co][c0 + c][t] -> row m, group t*cgs + c/8, lane c%8
            const int n_el = TILE_M * L.kcp * p.T;
            for (int i = tid; i < n_el; i += THREADS) {
                const int m = i / (L.kcp * p.T);
                const int rest = i - m * (L.kcp * p.T);
                const int c = rest / p.T;
                const int t = rest - c * p.T;
                const int co = co0 + m;
                uint16_t v = 0;
                if (co < p.CO && c < cvalid) v = wg[(long long)co * p.K + (long long)(c0 + c) * p.T + t];
                Ws[m * L.wst + (t * L.cgs + (c >> 3)) * 8 + (c & 7)] = v;
            }
        }
#pragma unroll
        for (int j = 0; j < XTM; ++j) {
            if (xdst[j] < 0) continue;
            *reinterpret_cast<uint4v*>(Xs + xdst[j]) = uint4v{xreg[j][0], xreg[j][1], xreg[j][2], xreg[j][3]};
        }
    };

    const int first_c0 = split * p.stages * p.kc;
    if (first_c0 < p.CI) load_stage(first_c0, min(p.kc, p.CI - first_c0));
    for (int st = 0; st < p.stages; ++st) {
        const int c0 = (split * p.stages + st) * p.kc;
        if (c0 >= p.CI) break;
        const int cvalid = min(p.kc, p.CI - c0);
        __syncthreads();  // previous stage's fragments consumed (and tables visible)
        store_stage(c0, cvalid);
        __syncthreads();
        const int c1 = c0 + p.kc;
        if (st + 1 < p.stages && c1 < p.CI) load_stage(c1, min(p.kc, p.CI - c1));

        // every group of the stage: groups are tap-major, so channel groups
        // past cvalid sit between real ones; they hold zeros in both tiles
        const int nsteps = L.gp >> 1;
        for (int s = 0; s < nsteps; ++s) {
            const int g = 2 * s + lh;
            const int koff = ktab[g];
            uint4v a[RM], b[RN];
#pragma unroll
            for (int rm = 0; rm < RM; ++rm)
                a[rm] = *reinterpret_cast<const uint4v*>(Ws + ((wm * RM + rm) * 32 + lj) * L.wst + g * 8);
#pragma unroll
            for (int rn = 0; rn < RN; ++rn)
                b[rn] = koff >= 0 ? *reinterpret_cast<const uint4v*>(Xs + pbase[rn] * L.kcs + koff)
                                  : uint4v{0u, 0u, 0u, 0u};
#pragma unroll
            for (int rm = 0; rm < RM; ++rm)
#pragma unroll
                for (int rn = 0; rn < RN; ++rn) acc[rm][rn] = HMfma<DT>::mma(a[rm], b[rn], acc[rm][rn]);
        }
    }

    // ---- split reduction across workgroups (device-scope atomics) -------------
    const int wslot = wm + wn * WM;
    if (p.S > 1) {
        const long long tile_words = (long long)TILE_M * TILE_N;
        float* part = p.ws + ((long long)tile * p.S) * tile_words;
        const int base = wslot * RM * RN * 16;
        float* mine = part + (long long)split * tile_words;
        #pragma unroll
        for (int rm = 0; rm < RM; ++rm)
            #pragma unroll
            for (int rn = 0; rn < RN; ++rn)
                #pragma unroll
                for (int r = 0; r < 16; ++r)
                    __hip_atomic_store(&mine[(base + (rm * RN + rn) * 16 + r) * 64 + lane],
                                       acc[rm][rn][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const unsigned old = __hip_atomic_fetch_add(&p.tickets[tile * kTicketStride], 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = (old == (unsigned)(p.S - 1)) ? 1 : 0;
        }
        __syncthreads();
        if (!s_last) return;
        #pragma unroll
        for (int rm = 0; rm < RM; ++rm)
            #pragma unroll
            for (int rn = 0; rn < RN; ++rn)
                #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // every split's partial from memory, this one's too (its
                    // registers hold the same values; a per-split choice
                    // between registers and memory is a form the compiler
                    // has mistranslated in the second fp16 kernel)
                    const int o = (base + (rm * RN + rn) * 16 + r) * 64 + lane;
                    float sum = 0.0f;
                    for (int s2 = 0; s2 < p.S; ++s2) {
                        const float v = __hip_atomic_load(&part[(long long)s2 * tile_words + o], __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                        sum = (s2 == 0) ? v : sum + v;
                    }
                    acc[rm][rn][r] = sum;
                }
        if (tid == 0)
            __hip_atomic_store(&p.tickets[tile * kTicketStride], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue and store (C: row 8*(r/4) + 4*(lane/32) + r%4, col lane%32)
    #pragma unroll
    for (int rm = 0; rm < RM; ++rm) {
        #pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = (wm * RM + rm) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            const int co = co0 + row;
            if (co >= p.CO) continue;
            const float eb = e_bias[row], er = e_rs[row];
            #pragma unroll
            for (int rn = 0; rn < RN; ++rn) {
                if (yoff[rn] < 0) continue;
                p.y[yoff[rn] + (long long)co * p.OHW] = apply_epilogue(p.epilogue, acc[rm][rn][r], eb, er);
            }
        }
    }
}

template <int DT, int WM, int WN, int RM, int RN, int WTM, int XTM>
int h_lds_bytes(const ConvParams& p) {
    using Cfg = HCfg<DT, WM, WN, RM, RN, WTM, XTM>;
    const HLayout L = h_layout(Cfg::TILE_M, p.kc, p.T, p.R, p.Wp);
    // staging tasks must fit the per-thread register slots
    if ((long long)p.R * p.Wp * L.cgs > (long long)XTM * Cfg::THREADS) return 1 << 30;
    const bool w_fast_shape = (p.T == 9 || p.T == 1) && (p.K % 8 == 0);
    if (w_fast_shape && Cfg::TILE_M * L.cgs > WTM * Cfg::THREADS) return 1 << 30;
    if ((long long)p.N * p.Hp >= (1LL << 31)) return 1 << 30;
    return 2 * L.halves;
}

template <int DT, int WM, int WN, int RM, int RN, int WTM, int XTM>
hipError_t h_launch(const ConvParams& p, hipStream_t stream) {
    using Cfg = HCfg<DT, WM, WN, RM, RN, WTM, XTM>;
    const int bytes = h_lds_bytes<DT, WM, WN, RM, RN, WTM, XTM>(p);
    if (bytes > 163840 - 64) return hipErrorInvalidValue;
    auto kern = igemm_h_kernel<DT, WM, WN, RM, RN, WTM, XTM>;
    static std::atomic<int> lds_limit{65536};
    if (bytes > lds_limit.load(std::memory_order_relaxed)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e;
        }
        lds_limit.store(bytes, std::memory_order_relaxed);
    }
    const long long grid = (long long)p.tiles_m * p.tiles_n * p.S;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::THREADS), bytes, stream, p);
    return hipGetLastError();
}

#define CT_H_VARIANT(NAME, DT, WM, WN, RM, RN, WTM, XTM, KCMAX)                                 \
    {NAME, DT, 32, 32, 16, WM, WN, 1, RM, RN, KCMAX, &h_lds_bytes<DT, WM, WN, RM, RN, WTM, XTM>, \
     &h_launch<DT, WM, WN, RM, RN, WTM, XTM>}

const IgemmVariant kHVariants[] = {
    CT_H_VARIANT("f16_m128n128_w2x2_r2x2", DT_F16, 2, 2, 2, 2, 1, 4, 64),
    CT_H_VARIANT("f16_m128n256_w2x2_r2x4", DT_F16, 2, 2, 2, 4, 1, 6, 64),
    CT_H_VARIANT("f16_m256n128_w4x2_r2x2", DT_F16, 4, 2, 2, 2, 1, 3, 64),
    CT_H_VARIANT("f16_m64n64_w2x2_r1x1", DT_F16, 2, 2, 1, 1, 1, 4, 64),
    CT_H_VARIANT("bf16_m128n128_w2x2_r2x2", DT_BF16, 2, 2, 2, 2, 1, 4, 64),
    CT_H_VARIANT("bf16_m128n256_w2x2_r2x4", DT_BF16, 2, 2, 2, 4, 1, 6, 64),
    CT_H_VARIANT("bf16_m64n64_w2x2_r1x1", DT_BF16, 2, 2, 1, 1, 1, 4, 64),
};

}  // namespace

const IgemmVariant* igemm_f16_variants(int* count) {
    *count = (int)(sizeof(kHVariants) / sizeof(kHVariants[0]));
    return kHVariants;
}

}  // namespace ct
