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
// (legality, launch size) and the kernel so the two cannot disagree.  The W
// and window regions are whole 64-word chunks: each chunk is filled by one
// direct-to-LDS load instruction of one wave.
struct F32Layout {
    int ksp;       // stage reduction extent kc*T rounded up to the MFMA K
    int wstr;      // W tile row stride; = KPI mod 64 so a fragment read of
                   // rows i and k-lanes q hits 64 distinct banks
    int w_words;   // W region [tile_m][wstr], rounded up to 64
    int xs_off;    // window region [kc][R][Wp]
    int x_words;   // rounded up to 64
    int ktab_off;  // per-k window offset table [ksp]
    int epi_off;   // per-channel bias and rsqrt [2][tile_m]
    int words;
};

__host__ __device__ inline F32Layout f32_layout(int tile_m, int kpi, int kc, int T, int R, int Wp,
                                                int red_words) {
    F32Layout L;
    L.ksp = round_up(kc * T, kpi);
    L.wstr = round_up(L.ksp - kpi, 64) + kpi;
    L.w_words = round_up(tile_m * L.wstr, 64);
    L.xs_off = L.w_words;
    L.x_words = round_up(kc * R * Wp, 64);
    int stage = L.xs_off + L.x_words;
    int region = stage > red_words ? stage : red_words;
    L.ktab_off = region;
    L.epi_off = L.ktab_off + L.ksp;
    L.words = L.epi_off + 2 * tile_m;
    return L;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// One wave fills 64 consecutive LDS words; lane l's word comes from src.
__device__ __forceinline__ void load_word_to_lds(const float* src, float* lds_chunk) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_chunk, 4, 0, 0);
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)__umulhi(n, f.mul) + n) >> f.shift);
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
    fetch_kernargs(p);
    using Cfg = F32Cfg<MF, WM, WN, WK, RM, RN>;
    using Mf = typename Cfg::Mf;
    using acc_t = typename Mf::acc_t;
    constexpr int M = Mf::M, N = Mf::N, KPI = Mf::KPI, NACC = Mf::NACC;
    constexpr int TILE_M = Cfg::TILE_M, TILE_N = Cfg::TILE_N, THREADS = Cfg::THREADS;
    constexpr int NWAVES = THREADS / 64;

    extern __shared__ __align__(16) float lds[];  // 16-byte LDS accesses need a 16-byte aligned base
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
    const float* zero = static_cast<const float*>(p.zero);
    const int RWp = p.R * p.Wp;

    for (int st = 0; st < p.stages; ++st) {
        const int c0 = (split * p.stages + st) * p.kc;
        if (c0 >= p.CI) break;
        const int cvalid = min(p.kc, p.CI - c0);
        const int kvalid = cvalid * p.T;
        __syncthreads();  // previous stage fully consumed
        // Every load of the stage is issued before any is waited for: the
        // loads write LDS directly, so nothing waits on a register.
        // W tile: rows co0.., columns c0*T .. c0*T + ksp (zero past kvalid)
        for (int ch = wave; ch < L.w_words / 64; ch += NWAVES) {
            const uint32_t q = (uint32_t)(ch * 64 + lane);
            const uint32_t m = fdiv(q, p.fd_wstr);
            const int kk = (int)(q - m * (uint32_t)L.wstr);
            const int co = co0 + (int)m;
            const float* src = zero;
            if ((int)m < TILE_M && co < p.CO && kk < kvalid)
                src = wg + (long long)co * p.K + (long long)c0 * p.T + kk;
            load_word_to_lds(src, Ws + ch * 64);
        }
        // padded-input window: channels c0.., virtual rows vr_first..
        for (int ch = wave; ch < L.x_words / 64; ch += NWAVES) {
            const uint32_t i = (uint32_t)(ch * 64 + lane);
            const uint32_t c = fdiv(i, p.fd_rwp);
            const uint32_t rem = i - c * (uint32_t)RWp;
            const uint32_t r = fdiv(rem, p.fd_wp);
            const int col = (int)(rem - r * (uint32_t)p.Wp);
            const float* src = zero;
            if ((int)c < cvalid) {
                const long long vr = vr_first + r;
                const long long n = fdiv((uint32_t)vr, p.fd_hp);
                const int iy = (int)(vr - n * p.Hp) - p.pad;
                const int ix = col - p.pad;
                if (n < p.N && iy >= 0 && iy < p.H && ix >= 0 && ix < p.W)
                    src = xg + ((n * p.CI + c0 + c) * p.H + iy) * (long long)p.W + ix;
            }
            load_word_to_lds(src, Xs + ch * 64);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have landed
        __syncthreads();                // and everybody else's
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
    // Partials and tickets are accessed only with device-scope atomics.  On
    // gfx950 a device-scope store is written through to the device's point
    // of coherence and a device-scope load reads from it, so no cache-wide
    // write-back or invalidate (what a device-scope fence costs) is needed:
    // each wave waits for its stores to complete before the workgroup
    // barrier, and the ticket is taken after the barrier.
    if (p.S > 1) {
        const long long tile_words = (long long)TILE_M * TILE_N;
        float* part = p.ws + ((long long)tile * p.S) * tile_words;
        const int base = wslot * RM * RN * NACC;
        if (wk == 0) {
            float* mine = part + (long long)split * tile_words;
            for (int rm = 0; rm < RM; ++rm)
                for (int rn = 0; rn < RN; ++rn)
                    for (int r = 0; r < NACC; ++r)
                        __hip_atomic_store(&mine[(base + (rm * RN + rn) * NACC + r) * 64 + lane],
                                           acc[rm][rn][r], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
        __syncthreads();
        if (tid == 0) {
            const unsigned old = __hip_atomic_fetch_add(&p.tickets[tile * kTicketStride], 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            s_last = (old == (unsigned)(p.S - 1)) ? 1 : 0;
        }
        __syncthreads();
        if (!s_last) return;
        // Last to arrive: every thread of the workgroup reduces a share of
        // the tile, with its loads issued in batches of OB outputs x SB
        // splits before any is consumed.  Summation order is 0..S-1.
        constexpr int OB = 4, SB = 8;
        constexpr int TILE_WORDS = TILE_M * TILE_N;
        for (int o0 = tid; o0 < TILE_WORDS; o0 += THREADS * OB) {
            float sum[OB];
            for (int u = 0; u < OB; ++u) sum[u] = 0.0f;
            for (int s0 = 0; s0 < p.S; s0 += SB) {
                float v[OB][SB];
#pragma unroll
                for (int u = 0; u < OB; ++u)
#pragma unroll
                    for (int j = 0; j < SB; ++j) {
                        const int o = o0 + u * THREADS;
                        v[u][j] = 0.0f;
                        if (o < TILE_WORDS && s0 + j < p.S)
                            v[u][j] = __hip_atomic_load(&part[(long long)(s0 + j) * tile_words + o],
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                for (int u = 0; u < OB; ++u)
#pragma unroll
                    for (int j = 0; j < SB; ++j)
                        if (s0 + j < p.S) sum[u] = (s0 + j == 0) ? v[u][j] : sum[u] + v[u][j];
            }
#pragma unroll
            for (int u = 0; u < OB; ++u) {
                const int o = o0 + u * THREADS;
                if (o >= TILE_WORDS) continue;
                // o = ((slot * RM + rm) * RN + rn) * NACC + r) * 64 + lane
                const int ln = o & 63;
                int t = o >> 6;
                const int r = t % NACC;
                t /= NACC;
                const int rn = t % RN;
                t /= RN;
                const int rm = t % RM;
                const int slot = t / RM;
                const int row = ((slot % WM) * RM + rm) * M + Mf::c_row(r, ln);
                const int co = co0 + row;
                const long long pc = p0 + (long long)((slot / WM) * RN + rn) * N + Mf::ab_idx(ln);
                if (co >= p.CO || pc >= p.P) continue;
                const long long n = pc / p.OHW;
                const long long rem = pc - n * p.OHW;
                p.y[(n * p.CO + co) * p.OHW + rem] =
                    apply_epilogue(p.epilogue, sum[u], e_bias[row], e_rs[row]);
            }
        }
        if (tid == 0) __hip_atomic_store(&p.tickets[tile * kTicketStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
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
int f32_lds_bytes(const ConvParams& p) {
    using Cfg = F32Cfg<MF, WM, WN, WK, RM, RN>;
    return 4 * f32_layout(Cfg::TILE_M, MfmaF32<MF>::KPI, p.kc, p.T, p.R, p.Wp, Cfg::RED_WORDS).words;
}

template <int MF, int WM, int WN, int WK, int RM, int RN>
hipError_t f32_launch(const ConvParams& p, hipStream_t stream) {
    using Cfg = F32Cfg<MF, WM, WN, WK, RM, RN>;
    const int bytes = f32_lds_bytes<MF, WM, WN, WK, RM, RN>(p);
    auto kern = igemm_f32_kernel<MF, WM, WN, WK, RM, RN>;
    const F32Layout L = f32_layout(Cfg::TILE_M, MfmaF32<MF>::KPI, p.kc, p.T, p.R, p.Wp,
                                   Cfg::RED_WORDS);
    ConvParams q = p;
    q.fd_wstr = make_fastdiv((uint32_t)L.wstr);
    q.fd_rwp = make_fastdiv((uint32_t)(p.R * p.Wp));
    q.fd_wp = make_fastdiv((uint32_t)p.Wp);
    q.fd_hp = make_fastdiv((uint32_t)p.Hp);
    // raise the dynamic-LDS limit (64 KiB by default) once per instantiation
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
    (void)hipGetLastError();  // report only this launch's error
    const long long grid = (long long)p.tiles_m * p.tiles_n * p.S;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::THREADS), bytes, stream, q);
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
