// fp32 matrix product, equivalently the batch-1 1x1 convolution, on
// v_mfma_f32_32x32x2_f32:
//   C[M][N] = A[M][K] * B[K][N]  (+ the per-row epilogue)
// The TVM tutorial "Tuning High Performance Convolution on NVIDIA GPUs"
// opens by noting that its tiling template also serves a matrix product;
// here that product is the 1x1 stride-1 unpadded convolution at batch 1:
// A = w [CO][CI], B = x [CI][H*W], C = y [CO][H*W].
//
// One workgroup of 4 waves computes a 128 x 128 tile of C over the whole
// reduction, each wave a 64 x 64 block (2 x 2 instruction tiles of 32 x 32),
// in stages of 32 k:
//  - both operand tiles of a stage go from memory straight into LDS (loads
//    that write LDS: 16 bytes a lane when both operands are 16-byte aligned
//    and K and N are multiples of 4, 4 bytes otherwise); the next stage's are
//    issued as the current stage starts, into the other of two LDS copies,
//    and one barrier ends a stage;
//  - A is held [m][32 k] with the eight 16-byte chunks of row m rotated by
//    XOR with ((m / 2) mod 8): a lane's 4 consecutive k of its row are one
//    16-byte read, and the 16 lanes on consecutive rows that one LDS cycle
//    serves (64 banks, 256 bytes: two 128-byte rows a bank line) read 16
//    different 16-byte bank groups (no bank conflicts).  B is held [k][128 n] and read one word a lane, lanes on
//    consecutive n;
//  - the instruction's two k slots are the wave's two lane halves: in group
//    g of 8 k, instruction i gives half h the k = 8g + 4h + i, so a lane's A
//    operands for a whole group are one 16-byte read.
// The reduction is not split: a workgroup owns its tile's every k, so the
// output is stored once with no partials or counters.
#include "ct_device.hpp"
#include "igemm_common.hpp"

#include <atomic>
#include <type_traits>

namespace ct {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBufRaw = 0x00020000;        // raw buffer descriptor, 32-bit elements
constexpr unsigned kBufOut = 0x80000000u;  // an offset past every buffer (all are < 2 GiB): reads zeros
constexpr int kTM = 128, kTN = 128, kKS = 32;  // tile rows, columns, k per stage
constexpr int kNT = 256;                        // 4 waves
constexpr int kCopy = kTM * kKS + kKS * kTN;    // floats of one LDS copy (A then B)
constexpr int kLdsBytes = (2 * kCopy + 2 * kTM) * 4;

struct GemmParams {
    const float* a;  // [M][K]
    const float* b;  // [K][N]
    float* c;        // [M][N]
    const float* bias;
    const float* var;
    float eps;
    int M, N, K;
    int epilogue;
    int tiles_m, tiles_n;
    int cgl;         // log2 of the XCD column groups; -1: column blocks per XCD
    FastDiv fd_lm;   // row tiles of one XCD's rectangle (all of them without XCD groups)
};
static_assert(sizeof(GemmParams) <= 128, "two argument lines");

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (uint32_t)(((uint64_t)__umulhi(n, f.mul) + n) >> f.shift);
}

// One wave fills 64 consecutive LDS slots of CS floats from lane_off (bytes)
// within r, lane l the l-th; lds is wave-uniform.
template <int CS>
__device__ __forceinline__ void load_slots(__amdgpu_buffer_rsrc_t r, float* lds, unsigned lane_off) {
    if constexpr (CS == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, lane_off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, lane_off, 0, 0, 0);
}

// V16: 16-byte slots (4 floats), else 4-byte slots.
template <bool V16>
__global__ __launch_bounds__(kNT) void igemm_f32_gemm_kernel(GemmParams p) {
    asm volatile("" ::"s"(p.a), "s"(p.fd_lm.d));  // both argument lines in one batch
    constexpr int CS = V16 ? 4 : 1;               // floats a slot
    constexpr int LPW = kTM * kKS / CS / 64 / 4;  // loads a wave per operand tile
    extern __shared__ __align__(16) float ls[];
    float* e_bias = ls + 2 * kCopy;
    float* e_rs = e_bias + kTM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int lj = lane & 31, lh = lane >> 5;

    // ---- workgroup -> tile.  Workgroup b runs on XCD b % 8; with XCD groups
    // (cgl >= 0) the XCDs split the tile grid into rectangles of
    // fd_lm.d row tiles x (tiles_n >> cgl) column tiles, row tiles fastest,
    // so that each XCD's L2 holds a few A row blocks and B column blocks;
    // otherwise each XCD takes a block of whole columns and workgroups past
    // the last column exit at once.
    const uint32_t bx = blockIdx.x;
    const uint32_t x = bx & 7, l = bx >> 3;
    const uint32_t lq = fdiv(l, p.fd_lm);
    const int lr = (int)(l - lq * p.fd_lm.d);
    int tm, tn;
    if (p.cgl >= 0) {
        tm = (int)(x >> p.cgl) * (int)p.fd_lm.d + lr;
        tn = (int)(x & ((1u << p.cgl) - 1)) * (p.tiles_n >> p.cgl) + (int)lq;
    } else {
        tm = lr;
        tn = (int)x * (((p.tiles_n + 7) & ~7) >> 3) + (int)lq;
        if (tn >= p.tiles_n) return;  // padding of the grid: uniform over the workgroup
    }
    const int m0 = tm * kTM, n0 = tn * kTN;

    // ---- epilogue values of row tid, loaded first (written to LDS once the
    //      first stage's loads are out)
    float e_b = 0.0f, e_v = 0.0f;
    const bool e_row = tid < kTM && m0 + tid < p.M;
    if (e_row && p.epilogue != EPI_NONE) e_b = p.bias[m0 + tid];
    if (e_row && p.epilogue == EPI_EXP_BIAS_RSQRT) e_v = p.var[m0 + tid];

    // ---- per-lane load offsets (bytes, without the stage term) -------------
    // A slot s of a stage: row r = s / (32/CS), position pos: the slot holds
    // the CS floats of global k = ((chunk(pos) ^ ((r / 2) % 8)) * 4) | (element % 4).
    // B slot s: k = s / (128/CS), columns n = (s % (128/CS)) * CS ...
    unsigned aoff[LPW], boff[LPW];
    int akk[LPW];  // the slot's k within the stage (for the k tail)
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int s = (wave + 4 * j) * 64 + lane;
        {
            const int r = s / (kKS / CS);
            const int e = (s - r * (kKS / CS)) * CS;  // element of the row in LDS
            const int k = (((e >> 2) ^ ((r >> 1) & 7)) << 2) | (e & 3);
            akk[j] = k;
            aoff[j] = (m0 + r < p.M) ? (unsigned)((r * p.K + k) * 4) : kBufOut;
        }
        {
            const int k = s / (kTN / CS);
            const int n = (s - k * (kTN / CS)) * CS;
            boff[j] = (n0 + n < p.N) ? (unsigned)((k * p.N + n) * 4) : kBufOut;
        }
    }
    const long long a_bytes = (long long)p.M * p.K * 4, b_bytes = (long long)p.K * p.N * 4;
    const int NS = (p.K + kKS - 1) / kKS;

    // issue stage st's tiles into LDS copy buf
    auto load_stage = [&](int st, int buf) {
        const int k0 = st * kKS;
        const long long abase = (long long)m0 * p.K + k0, bbase = (long long)k0 * p.N + n0;
        const int anrec = __builtin_amdgcn_readfirstlane((int)(a_bytes - 4 * abase));
        const int bnrec = __builtin_amdgcn_readfirstlane((int)(b_bytes > 4 * bbase ? b_bytes - 4 * bbase : 0));
        const __amdgpu_buffer_rsrc_t ar =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.a + abase), 0, anrec, kBufRaw);
        const __amdgpu_buffer_rsrc_t br =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.b + bbase), 0, bnrec, kBufRaw);
        float* As = ls + buf * kCopy;
        float* Bs = As + kTM * kKS;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            // a slot past K (the last stage of a K that is not a multiple of
            // 32) would read the next row: zeros instead
            const unsigned ao = (k0 + akk[j] < p.K) ? aoff[j] : kBufOut;
            load_slots<CS>(ar, As + (wave + 4 * j) * 64 * CS, ao);
            load_slots<CS>(br, Bs + (wave + 4 * j) * 64 * CS, boff[j]);
        }
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // fragment addresses (floats within a copy)
    int arow[2], ar7[2], bcol[2];
#pragma unroll
    for (int rm = 0; rm < 2; ++rm) {
        const int row = wm * 64 + rm * 32 + lj;
        arow[rm] = row * kKS;
        ar7[rm] = (row >> 1) & 7;
    }
#pragma unroll
    for (int rn = 0; rn < 2; ++rn) bcol[rn] = kTM * kKS + 4 * lh * kTN + wn * 64 + rn * 32 + lj;

    load_stage(0, 0);
    if (tid < kTM) {
        e_bias[tid] = e_b;
        e_rs[tid] = (e_row && p.epilogue == EPI_EXP_BIAS_RSQRT) ? dev_rsqrt(e_v + p.eps) : 1.0f;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int st = 0; st < NS; ++st) {
        if (st + 1 < NS) load_stage(st + 1, (st + 1) & 1);
        const float* Ls = ls + (st & 1) * kCopy;
        floatx4 a[2][2];
        float b[2][2][4];
        auto frag = [&](int g, floatx4 (&af)[2], float (&bf)[2][4]) {
#pragma unroll
            for (int rm = 0; rm < 2; ++rm)
                af[rm] = *reinterpret_cast<const floatx4*>(Ls + arow[rm] + (((2 * g + lh) ^ ar7[rm]) << 2));
#pragma unroll
            for (int rn = 0; rn < 2; ++rn)
#pragma unroll
                for (int i = 0; i < 4; ++i) bf[rn][i] = Ls[bcol[rn] + (8 * g + i) * kTN];
        };
        frag(0, a[0], b[0]);
#pragma unroll
        for (int g = 0; g < kKS / 8; ++g) {
            if (g + 1 < kKS / 8) frag(g + 1, a[(g + 1) & 1], b[(g + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int rm = 0; rm < 2; ++rm)
#pragma unroll
                    for (int rn = 0; rn < 2; ++rn)
                        acc[rm][rn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[g & 1][rm][i], b[g & 1][rn][i],
                                                                            acc[rm][rn], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next stage are in LDS
        __syncthreads();                // and everybody's; this stage's reads are done
    }

    // ---- epilogue and store (C: row 8*(r/4) + 4*(lane/32) + r%4, col lane%32).
    // A lane's rows are m0 + wm*64 + 4*(lane/32) + (a wave-uniform offset),
    // its columns n0 + wn*64 + lane%32 + 32 rn: one per-lane base address,
    // a uniform row offset and an immediate column offset per store.
    const int lrow = m0 + wm * 64 + 4 * lh;
    const int lcol = n0 + wn * 64 + lj;
    float* const cl = p.c + (long long)lrow * p.N + lcol;
    // One branch-free store loop for every epilogue: the tables hold bias 0
    // and scale 1 where the epilogue has none, and exp is selected by a
    // uniform flag (a branch on the epilogue around the stores made the
    // compiler copy accumulators out of their registers and spill).
    const bool ex = p.epilogue == EPI_EXP_BIAS_RSQRT;
#pragma unroll
    for (int rm = 0; rm < 2; ++rm) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ro = rm * 32 + 8 * (r >> 2) + (r & 3);  // wave-uniform
            if (lrow + ro >= p.M) continue;
            const int row = lrow - m0 + ro;
            const float eb = e_bias[row], er = e_rs[row];
            float* const crow = cl + (long long)ro * p.N;
#pragma unroll
            for (int rn = 0; rn < 2; ++rn) {
                if (lcol + rn * 32 >= p.N) continue;
                const float v = acc[rm][rn][r] + eb;
                // streamed out: the results are not read again by this launch
                __builtin_nontemporal_store(ex ? dev_exp(v) * er : v, crow + rn * 32);
            }
            __builtin_amdgcn_sched_barrier(0);  // one row's values at a time
        }
    }
}

// The shapes the kernel serves: batch 1, 1x1, stride 1, no padding, fp32,
// one split, 32 channels a stage; offsets of both operands within 32 bits.
int gemm_lds_bytes(const ConvParams& p) {
    if (p.N != 1 || p.KH != 1 || p.KW != 1 || p.stride != 1 || p.pad != 0) return 1 << 30;
    if (p.kc != kKS || p.S != 1) return 1 << 30;
    if ((long long)p.stages * kKS < p.CI) return 1 << 30;
    if (p.P >= (1LL << 31)) return 1 << 30;
    // byte offsets of A, B and C rows (and the tile past the last) fit 31 bits
    const long long tiles_m = (p.CO + kTM - 1) / kTM, tiles_n = (p.P + kTN - 1) / kTN;
    if (tiles_m * kTM * (long long)p.CI * 4 >= (1LL << 31)) return 1 << 30;
    if ((long long)(p.CI + kKS) * (tiles_n * kTN) * 4 >= (1LL << 31)) return 1 << 30;
    return kLdsBytes;
}

template <bool V16>
hipError_t gemm_launch_v(const GemmParams& q, int grid, hipStream_t stream) {
    auto kern = igemm_f32_gemm_kernel<V16>;
    static std::atomic<int> lds_set{0};
    if (!lds_set.load(std::memory_order_relaxed)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e;
        }
        lds_set.store(1, std::memory_order_relaxed);
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kNT), kLdsBytes, stream, q);
    return hipGetLastError();
}

hipError_t gemm_launch(const ConvParams& p, hipStream_t stream) {
    if (gemm_lds_bytes(p) > 163840) return hipErrorInvalidValue;
    GemmParams q{};
    q.a = static_cast<const float*>(p.w);
    q.b = static_cast<const float*>(p.x);
    q.c = p.y;
    q.bias = p.bias;
    q.var = p.var;
    q.eps = p.eps;
    q.M = p.CO;
    q.N = (int)p.P;
    q.K = p.CI;
    q.epilogue = p.epilogue;
    q.tiles_m = (p.CO + kTM - 1) / kTM;
    q.tiles_n = (int)((p.P + kTN - 1) / kTN);
    // XCD row groups ga: the one that minimises the estimate of the operand
    // bytes the XCDs fetch, (8/ga) * |A| + ga * |B| (a tile row block of A is
    // read by the 8/ga XCDs of its row group, a column block of B by ga),
    // among those that divide the grid
    q.cgl = -1;
    int lm = q.tiles_m;
    if ((q.tiles_n & 7) == 0) {
        const double abytes = (double)q.tiles_m * kTM * q.K, bbytes = (double)q.tiles_n * kTN * q.K;
        int ga = 1;
        double best = 8.0 * abytes + bbytes;
        for (int g = 2; g <= 8; g *= 2) {
            const double cost = (8 / g) * abytes + g * bbytes;
            if (q.tiles_m % g == 0 && q.tiles_n % (8 / g) == 0 && cost < best) {
                best = cost;
                ga = g;
            }
        }
        q.cgl = ga == 1 ? 3 : ga == 2 ? 2 : ga == 4 ? 1 : 0;
        lm = q.tiles_m / ga;
    }
    q.fd_lm = make_fastdiv((uint32_t)lm);
    const int grid = q.tiles_m * ((q.tiles_n + 7) & ~7);
    const bool v16 = reinterpret_cast<uintptr_t>(p.x) % 16 == 0 && reinterpret_cast<uintptr_t>(p.w) % 16 == 0 &&
                     q.K % 4 == 0 && q.N % 4 == 0;
    return v16 ? gemm_launch_v<true>(q, grid, stream) : gemm_launch_v<false>(q, grid, stream);
}

const IgemmVariant kGemmVariants[] = {
    // name, dtype, mfma m/n/k, waves m/n/k, reps m/n, kc_max, lds, launch, aux, xcd_local, tile_n, prepared
    {"f32g_m128n128_w2x2_r2x2_k32", DT_F32, 32, 32, 2, 2, 2, 1, 2, 2, kKS, &gemm_lds_bytes, &gemm_launch,
     nullptr, 0, 0, 0},
};

}  // namespace

const IgemmVariant* igemm_f32_gemm_variants(int* count) {
    *count = (int)(sizeof(kGemmVariants) / sizeof(kGemmVariants[0]));
    return kGemmVariants;
}

}  // namespace ct
