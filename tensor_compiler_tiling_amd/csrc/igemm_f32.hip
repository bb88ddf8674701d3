// fp32 implicit-GEMM convolution on CDNA4 fp32 matrix cores
// (v_mfma_f32_32x32x2_f32 / v_mfma_f32_16x16x4_f32), with split reduction
// across workgroups and a fused per-channel epilogue.
//
// Tiling follows the levels of the TVM tutorial's template ("Tuning High
// Performance Convolution on NVIDIA GPUs", Step 1); see igemm_common.hpp for
// the mapping.  Split reduction (split_k = S > 1): the S workgroups of an
// output tile each reduce 1/S of the input channels, write an fp32 partial
// tile, then take a ticket; the last to arrive sums the S partials in split
// order 0..S-1 (so the result does not depend on arrival order), applies the
// epilogue, stores y and resets the ticket.  Nobody waits on anybody.
//
// Fused epilogue: a workgroup's output channels are fixed by its grid index,
// so bias[c] and rsqrt(var[c] + eps) are loaded and computed once per
// workgroup into LDS (the per-channel binding of the Paddle PR "[CINN] Add
// the TileBroadcastTactic for NCHW broadcast", Performance Impact).
#include "ct_device.hpp"
#include "igemm_common.hpp"

#include <atomic>

namespace ct {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

template <int M> struct MfmaF32;

// 32x32 output, K = 2 per instruction.
//  A[i][k]: lane i + 32 k.  B[k][j]: lane j + 32 k.
//  C[i][j]: lane j + 32 * ((i / 4) % 2), register 4 * (i / 8) + i % 4.
template <> struct MfmaF32<32> {
    static constexpr int M = 32, N = 32, KPI = 2, NACC = 16;
    using acc_t = floatx16;
    static __device__ __forceinline__ acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int ab_idx(int lane) { return lane & 31; }
    static __device__ __forceinline__ int k_idx(int lane) { return lane >> 5; }
    static __device__ __forceinline__ int c_row(int r, int lane) {
        return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    }
};

// 16x16 output, K = 4 per instruction.
//  A[i][k]: lane i + 16 k.  B[k][j]: lane j + 16 k.
//  C[i][j]: lane j + 16 * (i / 4), register i % 4.
template <> struct MfmaF32<16> {
    static constexpr int M = 16, N = 16, KPI = 4, NACC = 4;
    using acc_t = floatx4;
    static __device__ __forceinline__ acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int ab_idx(int lane) { return lane & 15; }
    static __device__ __forceinline__ int k_idx(int lane) { return lane >> 4; }
    static __device__ __forceinline__ int c_row(int r, int lane) { return 4 * (lane >> 4) + r; }
};

// LDS carve-up of one workgroup, in 4-byte words.  Shared by the host
// (legality, launch size) and the kernel so the two cannot disagree.
struct F32Layout {
    int ksp;       // stage reduction extent kc*T rounded up to the MFMA K
    int wstr;      // W tile row stride (odd, spreads rows over banks)
    int xs_off;    // window tile [kc][R][Wp]
    int ktab_off;  // per-k window offset table [ksp]
    int epi_off;   // per-channel bias and rsqrt [2][tile_m]
    int words;
};

__host__ __device__ inline F32Layout f32_layout(int tile_m, int kpi, int kc, int T, int R, int Wp,
                                                int red_words) {
    F32Layout L;
    L.ksp = round_up(kc * T, kpi);
    L.wstr = L.ksp + 1;
    L.xs_off = tile_m * L.wstr;
    int stage = L.xs_off + kc * R * Wp;
    int region = stage > red_words ? stage : red_words;
    L.ktab_off = region;
    L.epi_off = L.ktab_off + L.ksp;
    L.words = L.epi_off + 2 * tile_m;
    return L;
}

template <int MF, int WM, int WN, int WK, int RM, int RN>
struct F32Cfg {
    using Mf = MfmaF32<MF>;
    static constexpr int TILE_M = WM * RM * Mf::M;
    static constexpr int TILE_N = WN * RN * Mf::N;
    static constexpr int THREADS = WM * WN * WK * 64;
    // LDS words for the cross-wave reduction when WK > 1
    static constexpr int RED_WORDS = (WK - 1) * WM * WN * RM * RN * Mf::NACC * 64;
};

template <int MF, int WM, int WN, int WK, int RM, int RN>
__global__ __launch_bounds__(WM * WN * WK * 64) void igemm_f32_kernel(ConvParams p) {
    using Cfg = F32Cfg<MF, WM, WN, WK, RM, RN>;
    using Mf = typename Cfg::Mf;
    using acc_t = typename Mf::acc_t;
    constexpr int M = Mf::M, N = Mf::N, KPI = Mf::KPI, NACC = Mf::NACC;
    constexpr int TILE_M = Cfg::TILE_M, TILE_N = Cfg::TILE_N, THREADS = Cfg::THREADS;

    extern __shared__ float lds[];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM;
    const int wn = (wave / WM) % WN;
    const int wk = wave / (WM * WN);

    const F32Layout L = f32_layout(TILE_M, KPI, p.kc, p.T, p.R, p.Wp, Cfg::RED_WORDS);
    float* Ws = lds;
    float* Xs = lds + L.xs_off;
    int* ktab = reinterpret_cast<int*>(lds + L.ktab_off);
    float* e_bias = lds + L.epi_off;
    float* e_rs = e_bias + TILE_M;

    // ---- which tile and which slice of the reduction --------------------
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

    // ---- per-lane output columns -----------------------------------------
    int pbase[RN];          // window offset of the column's (0,0) tap
    long long yoff[RN];     // y offset of (n, 0, oy, ox); -1 if past P
    for (int rn = 0; rn < RN; ++rn) {
        const long long pc = p0 + (long long)(wn * RN + rn) * N + Mf::ab_idx(lane);
        if (pc < p.P) {
            const long long n = pc / p.OHW;
            const int rem = (int)(pc - n * p.OHW);
            const int oy = rem / p.OW;
            const int ox = rem - oy * p.OW;
            const long long vr = n * p.Hp + (long long)oy * p.stride;
            pbase[rn] = (int)(vr - vr_first) * p.Wp + ox * p.stride;
            yoff[rn] = n * (long long)p.CO * p.OHW + rem;
        } else {
            pbase[rn] = 0;
            yoff[rn] = -1;
        }
    }

    // ---- per-stage tables (same for every stage) ---------------------------
    for (int kk = tid; kk < L.ksp; kk += THREADS) {
        const int c = kk / p.T;
        const int t = kk - c * p.T;
        const int ky = t / p.KW;
        const int kx = t - ky * p.KW;
        ktab[kk] = (c * p.R + ky) * p.Wp + kx;
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

    __syncthreads();  // tables visible to every wave

    acc_t acc[RM][RN];
    for (int rm = 0; rm < RM; ++rm)
        for (int rn = 0; rn < RN; ++rn)
            for (int r = 0; r < NACC; ++r) acc[rm][rn][r] = 0.0f;

    const float* __restrict__ xg = static_cast<const float*>(p.x);
    const float* __restrict__ wg = static_cast<const float*>(p.w);
    const int RWp = p.R * p.Wp;
    const int stage_words_x = p.kc * RWp;

    for (int st = 0; st < p.stages; ++st) {
        const int c0 = (split * p.stages + st) * p.kc;
        if (c0 >= p.CI) break;
        const int cvalid = min(p.kc, p.CI - c0);
        const int kvalid = cvalid * p.T;
        __syncthreads();  // previous stage fully consumed
        // W tile: rows co0.., columns c0*T .. c0*T + ksp (zero past kvalid)
        for (int i = tid; i < TILE_M * L.ksp; i += THREADS) {
            const int m = i / L.ksp;
            const int kk = i - m * L.ksp;
            const int co = co0 + m;
            float v = 0.0f;
            if (co < p.CO && kk < kvalid) v = wg[(long long)co * p.K + (long long)c0 * p.T + kk];
            Ws[m * L.wstr + kk] = v;
        }
        // padded-input window: channels c0.., virtual rows vr_first..
        for (int i = tid; i < stage_words_x; i += THREADS) {
            const int c = i / RWp;
            const int rem = i - c * RWp;
            const int r = rem / p.Wp;
            const int col = rem - r * p.Wp;
            float v = 0.0f;
            if (c < cvalid) {
                const long long vr = vr_first + r;
                const long long n = vr / p.Hp;
                const int iy = (int)(vr - n * p.Hp) - p.pad;
                const int ix = col - p.pad;
                if (n < p.N && iy >= 0 && iy < p.H && ix >= 0 && ix < p.W)
                    v = xg[((n * p.CI + c0 + c) * p.H + iy) * (long long)p.W + ix];
            }
            Xs[i] = v;
        }
        __syncthreads();
        const int nsteps = (kvalid + KPI - 1) / KPI;
        for (int j = wk; j < nsteps; j += WK) {
            const int k = j * KPI + Mf::k_idx(lane);
            const bool kok = k < kvalid;
            const int koff = ktab[k];
            float a[RM], b[RN];
            for (int rm = 0; rm < RM; ++rm)
                a[rm] = Ws[((wm * RM + rm) * M + Mf::ab_idx(lane)) * L.wstr + k];
            for (int rn = 0; rn < RN; ++rn) b[rn] = kok ? Xs[pbase[rn] + koff] : 0.0f;
            for (int rm = 0; rm < RM; ++rm)
                for (int rn = 0; rn < RN; ++rn) acc[rm][rn] = Mf::mma(a[rm], b[rn], acc[rm][rn]);
        }
    }

    // ---- reduce the waves_k partial accumulators inside the workgroup ------
    const int wslot = wm + wn * WM;
    if constexpr (WK > 1) {
        __syncthreads();
        float* red = lds;
        if (wk > 0) {
            const int base = ((wk - 1) * WM * WN + wslot) * RM * RN * NACC;
            for (int rm = 0; rm < RM; ++rm)
                for (int rn = 0; rn < RN; ++rn)
                    for (int r = 0; r < NACC; ++r)
                        red[(base + (rm * RN + rn) * NACC + r) * 64 + lane] = acc[rm][rn][r];
        }
        __syncthreads();
        if (wk == 0) {
            for (int w2 = 1; w2 < WK; ++w2) {
                const int base = ((w2 - 1) * WM * WN + wslot) * RM * RN * NACC;
                for (int rm = 0; rm < RM; ++rm)
                    for (int rn = 0; rn < RN; ++rn)
                        for (int r = 0; r < NACC; ++r)
                            acc[rm][rn][r] += red[(base + (rm * RN + rn) * NACC + r) * 64 + lane];
            }
        }
    }

    // ---- split reduction across workgroups ---------------------------------
    if (p.S > 1) {
        const long long tile_words = (long long)TILE_M * TILE_N;
        float* part = p.ws + ((long long)tile * p.S) * tile_words;
        const int base = wslot * RM * RN * NACC;
        if (wk == 0) {
            float* mine = part + (long long)split * tile_words;
            for (int rm = 0; rm < RM; ++rm)
                for (int rn = 0; rn < RN; ++rn)
                    for (int r = 0; r < NACC; ++r)
                        mine[(base + (rm * RN + rn) * NACC + r) * 64 + lane] = acc[rm][rn][r];
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const unsigned old = atomicAdd(&p.tickets[tile], 1u);
            s_last = (old == (unsigned)(p.S - 1)) ? 1 : 0;
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        if (wk == 0) {
            for (int rm = 0; rm < RM; ++rm)
                for (int rn = 0; rn < RN; ++rn)
                    for (int r = 0; r < NACC; ++r) {
                        const int o = (base + (rm * RN + rn) * NACC + r) * 64 + lane;
                        float sum = (split == 0) ? acc[rm][rn][r] : part[o];
                        for (int s2 = 1; s2 < p.S; ++s2)
                            sum += (s2 == split) ? acc[rm][rn][r] : part[(long long)s2 * tile_words + o];
                        acc[rm][rn][r] = sum;
                    }
        }
        if (tid == 0) p.tickets[tile] = 0u;
    }

    // ---- epilogue and store ------------------------------------------------
    if (wk != 0) return;
    for (int rm = 0; rm < RM; ++rm) {
        for (int r = 0; r < NACC; ++r) {
            const int row = (wm * RM + rm) * M + Mf::c_row(r, lane);
            const int co = co0 + row;
            if (co >= p.CO) continue;
            const float eb = e_bias[row], er = e_rs[row];
            for (int rn = 0; rn < RN; ++rn) {
                if (yoff[rn] < 0) continue;
                p.y[yoff[rn] + (long long)co * p.OHW] =
                    apply_epilogue(p.epilogue, acc[rm][rn][r], eb, er);
            }
        }
    }
}

template <int MF, int WM, int WN, int WK, int RM, int RN>
int f32_lds_bytes(int kc, int R, int Wp, int T) {
    using Cfg = F32Cfg<MF, WM, WN, WK, RM, RN>;
    return 4 * f32_layout(Cfg::TILE_M, MfmaF32<MF>::KPI, kc, T, R, Wp, Cfg::RED_WORDS).words;
}

template <int MF, int WM, int WN, int WK, int RM, int RN>
hipError_t f32_launch(const ConvParams& p, hipStream_t stream) {
    using Cfg = F32Cfg<MF, WM, WN, WK, RM, RN>;
    const int bytes = f32_lds_bytes<MF, WM, WN, WK, RM, RN>(p.kc, p.R, p.Wp, p.T);
    auto kern = igemm_f32_kernel<MF, WM, WN, WK, RM, RN>;
    // raise the dynamic-LDS limit once per instantiation (process-wide)
    static std::atomic<int> lds_limit{0};
    if (bytes > lds_limit.load(std::memory_order_relaxed)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
        if (e != hipSuccess) return e;
        lds_limit.store(163840, std::memory_order_relaxed);
    }
    const long long grid = (long long)p.tiles_m * p.tiles_n * p.S;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::THREADS), bytes, stream, p);
    return hipGetLastError();
}

#define CT_F32_VARIANT(NAME, MF, WM, WN, WK, RM, RN, KCMAX)                                     \
    {NAME, DT_F32, MF, MF, MfmaF32<MF>::KPI, WM, WN, WK, RM, RN, KCMAX,                          \
     &f32_lds_bytes<MF, WM, WN, WK, RM, RN>, &f32_launch<MF, WM, WN, WK, RM, RN>}

const IgemmVariant kF32Variants[] = {
    CT_F32_VARIANT("f32_m16n64_w1x1x4_r1x4", 16, 1, 1, 4, 1, 4, 64),
    CT_F32_VARIANT("f32_m32n64_w1x1x4_r1x2", 32, 1, 1, 4, 1, 2, 64),
    CT_F32_VARIANT("f32_m64n64_w2x2x1_r1x1", 32, 2, 2, 1, 1, 1, 64),
    CT_F32_VARIANT("f32_m64n128_w2x2x1_r1x2", 32, 2, 2, 1, 1, 2, 64),
    CT_F32_VARIANT("f32_m128n128_w2x2x1_r2x2", 32, 2, 2, 1, 2, 2, 64),
    CT_F32_VARIANT("f32_m64n256_w1x4x1_r2x2", 32, 1, 4, 1, 2, 2, 64),
};

}  // namespace

const IgemmVariant* igemm_f32_variants(int* count) {
    *count = (int)(sizeof(kF32Variants) / sizeof(kF32Variants[0]));
    return kF32Variants;
}

}  // namespace ct
