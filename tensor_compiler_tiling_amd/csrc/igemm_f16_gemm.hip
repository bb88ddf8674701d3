// fp16 / bf16 matrix product, equivalently the batch-1 1x1 convolution, on
// v_mfma_f32_32x32x16_f16 / _bf16 with fp32 accumulation and output:
//   C[M][N] = A[M][K] * B[K][N]  (+ the per-row epilogue)
// The TVM tutorial "Tuning High Performance Convolution on NVIDIA GPUs"
// opens by noting that its tiling template also serves a matrix product;
// here that product is the 1x1 stride-1 unpadded convolution at batch 1:
// A = w [CO][CI], B = x [CI][H*W], C = y [CO][H*W].
//
// One workgroup of 4 waves computes a 256 x 256 tile of C over the whole
// reduction, each wave a 128 x 128 block (4 x 4 instruction tiles of 32 x
// 32): each instruction then reads half a KB of operand fragments from LDS,
// half of what a 64 x 64 wave block needs.  The reduction runs in stages of
// KS halves, through two LDS copies.  Two forms stage the operand tiles:
//  - with 16-byte aligned operands, K and N multiples of 8 and KS = 64, the
//    register-staged form below (plain loads into registers, LDS writes by
//    the waves, spread between the matrix instructions);
//  - otherwise the first form: loads that write LDS directly (16 or 4 bytes
//    a lane, the widest the operands' alignment and K, N allow; with 2-byte
//    aligned operands or an odd K or N through registers, since a 2-byte
//    load that writes LDS fills 4 bytes of it a lane).  The compiler waits
//    for every such load in flight before a transposing LDS read of the
//    same LDS object, so a stage first reads all its B fragments (the
//    transposing reads), then issues the next stage's loads, which thus have
//    the whole stage to land, and reads its A fragments (plain 16-byte
//    reads) through two register sets, step t+1's while step t's
//    instructions run; one barrier ends a stage.
// Layouts, shared by both forms:
//  - A is held [m][KS] in 16-byte chunks (8 k), chunk q of row m stored at
//    q ^ rot(m) (below): a lane's A operand (8 consecutive k of its row) is
//    one 16-byte read, and the 16 lanes an LDS cycle serves hit 16 different
//    bank groups;
//  - B is held [k][256 n] in 16-byte chunks (8 n), chunk c of row k stored at
//    c ^ (2 (k mod 4)).  The instruction wants 8 consecutive k of one column
//    per lane: two transposing reads (ds_read_b64_tr_b16) give them, 4 k
//    each.  Within 16 lanes that read returns to lane i its element r from
//    the 8 bytes lane 4r + i/4 addresses (element i mod 4), so lane L
//    addresses row k0 + L/4, columns n0 + 4 (L mod 4) .. + 3, and lane i
//    receives B[k0 .. k0+3][n0 + i].  The rotation puts those four rows'
//    32-byte pieces in four different bank groups.
// The reduction is not split: a workgroup owns its tile's every k, so the
// output is stored once with no partials or counters.
#include "ct_device.hpp"
#include "igemm_common.hpp"

#include <atomic>
#include <type_traits>

namespace ct {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4v lds_short4v;

constexpr int kBufRaw = 0x00020000;        // raw buffer descriptor, 32-bit elements
constexpr unsigned kBufOut = 0x80000000u;  // an offset past every buffer (all are < 2 GiB): reads zeros
constexpr int kTM = 256, kTN = 256;        // tile rows and columns
constexpr int kNT = 256;                   // 4 waves, 2 x 2

template <int DT> struct GMma;
template <> struct GMma<DT_F16> {
    static __device__ __forceinline__ floatx16 mma(uint4v a, uint4v b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                     __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
    }
};
template <> struct GMma<DT_BF16> {
    static __device__ __forceinline__ floatx16 mma(uint4v a, uint4v b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct HGemmParams {
    const uint16_t* a;  // [M][K]
    const uint16_t* b;  // [K][N]
    float* c;           // [M][N]
    const float* bias;
    const float* var;
    float eps;
    int M, N, K;
    int epilogue;
    int tiles_m, tiles_n;
    int cgl;        // log2 of the XCD column groups; -1: column blocks per XCD
    FastDiv fd_lm;  // row tiles of one XCD's rectangle (all of them without XCD groups)
};
static_assert(sizeof(HGemmParams) <= 128, "two argument lines");

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (uint32_t)(((uint64_t)__umulhi(n, f.mul) + n) >> f.shift);
}

template <int KS>
struct HG {
    static constexpr int ACH = KS / 8;                // 16-byte chunks of an A row
    static constexpr int A_H = kTM * KS;              // halves of an A tile
    static constexpr int B_H = KS * kTN;              // halves of a B tile
    static constexpr int COPY = A_H + B_H;            // halves of one LDS copy
    static constexpr int LDS = 2 * COPY * 2 + 2 * kTM * 4;  // bytes
    static_assert(KS == 32 || KS == 64, "the chunk rotations below");
    // A row m's rotation of its chunks.  LDS serves 16 lanes of a 16-byte
    // read a cycle from 64 banks (256 bytes): the 16 rows m .. m+15 of one
    // read sit at 256/(2 KS) row offsets a bank line, and the rotation gives
    // rows with the same offset different chunks.
    static __device__ __forceinline__ int rot(int m) { return KS == 32 ? (m >> 2) & 3 : (m >> 1) & 7; }
};

// The tile of this workgroup: XCD x = blockIdx % 8 takes one rectangle of
// tiles (row tiles fastest), or, without XCD groups, a run of column tiles.
// False for the padding of the grid (uniform over the workgroup).
__device__ __forceinline__ bool block_tile(const HGemmParams& p, int& m0, int& n0) {
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
        if (tn >= p.tiles_n) return false;
    }
    m0 = tm * kTM;
    n0 = tn * kTN;
    return true;
}

// Epilogue and store of a wave's 128 x 128 block (C: row 8*(r/4) +
// 4*(lane/32) + r%4, column lane%32 of each 32 x 32 instruction tile).  A
// lane's rows are m0 + wm*128 + 4*(lane/32) + (a wave-uniform offset), its
// columns n0 + wn*128 + lane%32 + 32 rn: one per-lane base address, a uniform
// row offset and an immediate column offset per store.  One branch-free store
// loop serves every epilogue: the tables hold bias 0 and scale 1 where the
// epilogue has none, and exp is selected by a uniform flag (a branch on the
// epilogue around the stores made the compiler copy accumulators out of
// their registers and spill).
__device__ __forceinline__ void store_block(const HGemmParams& p, floatx16 (&acc)[4][4], int m0, int n0, int wm,
                                            int wn, int lane, const float* e_bias, const float* e_rs) {
    const int lj = lane & 31, lh = lane >> 5;
    const int lrow = m0 + wm * 128 + 4 * lh;
    const int lcol = n0 + wn * 128 + lj;
    float* const cl = p.c + (long long)lrow * p.N + lcol;
    const bool ex = p.epilogue == EPI_EXP_BIAS_RSQRT;
#pragma unroll
    for (int rm = 0; rm < 4; ++rm) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ro = rm * 32 + 8 * (r >> 2) + (r & 3);  // wave-uniform
            if (lrow + ro >= p.M) continue;
            const int row = lrow - m0 + ro;
            const float eb = e_bias[row], er = e_rs[row];
            float* const crow = cl + (long long)ro * p.N;
#pragma unroll
            for (int rn = 0; rn < 4; ++rn) {
                if (lcol + rn * 32 >= p.N) continue;
                const float v = acc[rm][rn][r] + eb;
                // streamed out: the results are not read again by this launch
                __builtin_nontemporal_store(ex ? dev_exp(v) * er : v, crow + rn * 32);
            }
            __builtin_amdgcn_sched_barrier(0);  // one row's values at a time
        }
    }
}

// One wave fills 64 consecutive LDS slots of CB (16 or 4) bytes from
// lane_off (bytes) within r, lane l the l-th; lds is wave-uniform.
template <int CB>
__device__ __forceinline__ void load_slots(__amdgpu_buffer_rsrc_t r, uint16_t* lds, unsigned lane_off) {
    static_assert(CB == 16 || CB == 4, "loads that write LDS fill 4 bytes a lane at least");
    if constexpr (CB == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, lane_off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, lane_off, 0, 0, 0);
}

// The same for 2-byte slots, through registers: n slots a lane, loaded in
// batches of 16 and written once each batch has arrived.
template <int N>
__device__ __forceinline__ void load_halves(__amdgpu_buffer_rsrc_t r, uint16_t* lds, int wave, int lane,
                                            const unsigned (&off)[N]) {
    static_assert(N % 16 == 0, "whole batches");
#pragma unroll
    for (int j0 = 0; j0 < N; j0 += 16) {
        uint16_t v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b16(r, off[j0 + j], 0, 0);
#pragma unroll
        for (int j = 0; j < 16; ++j) lds[(wave + 4 * (j0 + j)) * 64 + lane] = v[j];
    }
}

template <int DT, int KS, int CB>
__global__ __launch_bounds__(kNT) void igemm_h_gemm_kernel(HGemmParams p) {
    asm volatile("" ::"s"(p.a), "s"(p.fd_lm.d));  // both argument lines in one batch
    using C = HG<KS>;
    constexpr int SH = CB / 2;                    // halves a slot
    constexpr int ALPW = C::A_H / SH / 64 / 4;    // A loads a wave
    constexpr int BLPW = C::B_H / SH / 64 / 4;    // B loads a wave
    constexpr int STEPS = KS / 16;                // instruction steps a stage
    extern __shared__ __align__(16) uint16_t hs[];
    float* e_bias = reinterpret_cast<float*>(hs + 2 * C::COPY);
    float* e_rs = e_bias + kTM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int lj = lane & 31, lh = lane >> 5;

    int m0, n0;
    if (!block_tile(p, m0, n0)) return;

    // ---- epilogue values of row tid, loaded first
    float e_b = 0.0f, e_v = 0.0f;
    const bool e_row = m0 + tid < p.M;
    if (e_row && p.epilogue != EPI_NONE) e_b = p.bias[m0 + tid];
    if (e_row && p.epilogue == EPI_EXP_BIAS_RSQRT) e_v = p.var[m0 + tid];

    // ---- per-lane load offsets (bytes, without the stage term) -------------
    // A slot s: row m = s / (KS/SH), LDS element e of the row; LDS chunk
    // e/8 holds global chunk (e/8) ^ rot(m).
    unsigned aoff[ALPW];
#pragma unroll
    for (int j = 0; j < ALPW; ++j) {
        const int s = (wave + 4 * j) * 64 + lane;
        const int m = s / (KS / SH);
        const int e = (s - m * (KS / SH)) * SH;
        const int k = (((e >> 3) ^ C::rot(m)) << 3) | (e & 7);
        aoff[j] = (m0 + m < p.M) ? (unsigned)((m * p.K + k) * 2) : kBufOut;
    }
    // B slot s: row k = s / (256/SH), LDS element e of the row; LDS chunk e/8
    // holds global chunk (e/8) ^ (2 (k % 4)).
    unsigned boff[BLPW];
#pragma unroll
    for (int j = 0; j < BLPW; ++j) {
        const int s = (wave + 4 * j) * 64 + lane;
        const int k = s / (kTN / SH);
        const int e = (s - k * (kTN / SH)) * SH;
        const int n = ((((e >> 3) ^ (2 * (k & 3)))) << 3) | (e & 7);
        boff[j] = (n0 + n < p.N) ? (unsigned)((k * p.N + n) * 2) : kBufOut;
    }
    const long long a_bytes = (long long)p.M * p.K * 2, b_bytes = (long long)p.K * p.N * 2;
    const int NS = p.K / KS;

    auto load_stage = [&](int st, int buf) {
        const int k0 = st * KS;
        const long long abase = (long long)m0 * p.K + k0, bbase = (long long)k0 * p.N + n0;
        const int anrec = __builtin_amdgcn_readfirstlane((int)(a_bytes - 2 * abase));
        const int bnrec = __builtin_amdgcn_readfirstlane((int)(b_bytes - 2 * bbase));
        const __amdgpu_buffer_rsrc_t ar =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.a + abase), 0, anrec, kBufRaw);
        const __amdgpu_buffer_rsrc_t br =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.b + bbase), 0, bnrec, kBufRaw);
        uint16_t* As = hs + buf * C::COPY;
        uint16_t* Bs = As + C::A_H;
        if constexpr (CB == 2) {
            load_halves(ar, As, wave, lane, aoff);
            load_halves(br, Bs, wave, lane, boff);
        } else {
#pragma unroll
            for (int j = 0; j < ALPW; ++j) load_slots<CB>(ar, As + (wave + 4 * j) * 64 * SH, aoff[j]);
#pragma unroll
            for (int j = 0; j < BLPW; ++j) load_slots<CB>(br, Bs + (wave + 4 * j) * 64 * SH, boff[j]);
        }
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // fragment addresses (halves within a copy).  A: row wm*128 + rm*32 + lj,
    // chunk 2 t + lh of step t (rotated).  B: lane L = lane % 16 of its
    // 16-lane group addresses row 8 lh + L/4 (+4 for the second read) of
    // the step, column n = wn*128 + rn*32 + 16 (lj/16) + 4 (L % 4).
    int arow[4], arot[4];
#pragma unroll
    for (int rm = 0; rm < 4; ++rm) {
        const int row = wm * 128 + rm * 32 + lj;
        arow[rm] = row * KS;
        arot[rm] = C::rot(row);
    }
    const int L = lane & 15;
    const int brow = 8 * lh + (L >> 2);  // rows brow and brow + 4 of a step; brow % 4 = L/4
    int bcol[4];
#pragma unroll
    for (int rn = 0; rn < 4; ++rn) {
        const int n = wn * 128 + rn * 32 + 16 * (lj >> 4) + 4 * (L & 3);
        // rows brow and brow + 4 have the same k % 4, hence the same rotation
        bcol[rn] = ((((n >> 3) ^ (2 * (brow & 3)))) << 3) | (n & 7);
    }

    load_stage(0, 0);
    e_bias[tid] = e_b;
    e_rs[tid] = (e_row && p.epilogue == EPI_EXP_BIAS_RSQRT) ? dev_rsqrt(e_v + p.eps) : 1.0f;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int st = 0; st < NS; ++st) {
        const uint16_t* As = hs + (st & 1) * C::COPY;
        const uint16_t* Bs = As + C::A_H;
        // A fragments of step t: row wm*128 + rm*32 + lj, chunk 2t + lh (rotated)
        uint4v a[2][4];
        auto frag_a = [&](int t, uint4v (&af)[4]) {
#pragma unroll
            for (int rm = 0; rm < 4; ++rm)
                af[rm] = *reinterpret_cast<const uint4v*>(As + arow[rm] + (((2 * t + lh) ^ arot[rm]) << 3));
        };
        // step 0's A fragments first (LDS reads complete in order: the first
        // instructions then wait for them and step 0's B only), then the B
        // fragments of every step (transposing reads)
        frag_a(0, a[0]);
        uint4v b[STEPS][4];
#pragma unroll
        for (int t = 0; t < STEPS; ++t)
#pragma unroll
            for (int rn = 0; rn < 4; ++rn) {
                const uint16_t* q = Bs + (16 * t + brow) * kTN + bcol[rn];
                const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)q);
                const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(q + 4 * kTN));
                const uint2v l2 = __builtin_bit_cast(uint2v, lo), h2 = __builtin_bit_cast(uint2v, hi);
                b[t][rn] = uint4v{l2.x, l2.y, h2.x, h2.y};
            }
        __builtin_amdgcn_sched_barrier(0);
        // no transposing read follows: the next stage's loads go out now
        if (st + 1 < NS) load_stage(st + 1, (st + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            if (t + 1 < STEPS) frag_a(t + 1, a[(t + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rm = 0; rm < 4; ++rm)
#pragma unroll
                for (int rn = 0; rn < 4; ++rn)
                    acc[rm][rn] = GMma<DT>::mma(a[t & 1][rm], b[t][rn], acc[rm][rn]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next stage are in LDS
        __syncthreads();                // and everybody's; this stage's reads are done
    }

    store_block(p, acc, m0, n0, wm, wn, lane, e_bias, e_rs);
}

// Register-staged form, for 16-byte aligned operands with K and N multiples
// of 8 (every 16-byte chunk of a tile row either wholly inside or wholly
// past the matrix) and stages of 64 channels.  Loads that write LDS
// directly hold up the wave that issues them (on this chip each costs the
// issuing wave about as long as the whole CU's queue of them ahead of it),
// and with one wave a SIMD that wave is the one that issues the matrix
// instructions.  Plain 16-byte loads into registers and 16-byte LDS writes
// by the waves themselves cost the matrix pipe almost nothing, so this form
// stages through registers:
//  - a thread holds 2 KS/8 chunks of 16 bytes (KS/8 of A, KS/8 of B) of the
//    next stage;
//  - a stage's STEPS steps each run 16 instructions with one LDS access or
//    load between consecutive instructions: the fragment reads of the next
//    step (12 reads: 4 of A, 8 transposing of B), and in the two steps before
//    the last, each held chunk is written to the other copy and its register
//    at once reloaded with the matching chunk of the stage after next (so a
//    load has a whole stage to land, and the writes are spread over two
//    steps);
//  - one barrier a stage, after the writes: the last step then already reads
//    the next stage's first fragments from the other copy, so no step waits
//    for its fragments after a barrier;
//  - past the last stage the loads read zeros (an empty buffer range) into a
//    copy that is no longer read, which keeps the loop free of branches.
template <int DT, int KS>
__global__ __launch_bounds__(kNT) void igemm_h_gemm_rs_kernel(HGemmParams p) {
    asm volatile("" ::"s"(p.a), "s"(p.fd_lm.d));  // both argument lines in one batch
    using C = HG<KS>;
    constexpr int LPO = KS / 8;       // 16-byte chunks a thread holds, per operand
    constexpr int STEPS = KS / 16;    // instruction steps a stage
    constexpr int AMJ = 2048 / KS;    // A rows between a thread's chunks
    static_assert(STEPS >= 3, "the writes take the two steps before the last");
    // two LDS copies as two objects, named statically by the stage loop
    __shared__ __align__(16) uint16_t lds0[C::COPY];
    __shared__ __align__(16) uint16_t lds1[C::COPY];
    __shared__ float e_bias[kTM], e_rs[kTM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int lj = lane & 31, lh = lane >> 5;

    int m0, n0;
    if (!block_tile(p, m0, n0)) return;

    // ---- epilogue values of row tid, loaded first
    float e_b = 0.0f, e_v = 0.0f;
    const bool e_row = m0 + tid < p.M;
    if (e_row && p.epilogue != EPI_NONE) e_b = p.bias[m0 + tid];
    if (e_row && p.epilogue == EPI_EXP_BIAS_RSQRT) e_v = p.var[m0 + tid];

    // ---- a thread's chunks.  A chunk j: row am + j*AMJ, chunk aq of the
    // row's KS/8, stored at chunk aq ^ rot(row) (rot(row) = rot(am): AMJ is
    // a multiple of the rotation's period).  B chunk j: row bk + 8 j of the
    // stage, chunk bc of the row's 32, stored at bc ^ (2 (row % 4)).
    const int aq = tid % (KS / 8), am = tid / (KS / 8);
    const int bc = tid & 31, bk = tid >> 5;
    unsigned aoff[LPO], boff[LPO];  // bytes from the stage's tile origin; past the matrix: kBufOut
#pragma unroll
    for (int j = 0; j < LPO; ++j) {
        aoff[j] = (m0 + am + j * AMJ < p.M) ? (unsigned)(((am + j * AMJ) * p.K + aq * 8) * 2) : kBufOut;
        boff[j] = (n0 + bc * 8 < p.N) ? (unsigned)(((bk + 8 * j) * p.N + bc * 8) * 2) : kBufOut;
    }
    const int aw = am * KS + ((aq ^ C::rot(am)) << 3);            // + j * AMJ * KS halves
    const int bw = C::A_H + bk * kTN + ((bc ^ (2 * (bk & 3))) << 3);  // + j * 8 * kTN halves
    const long long a_bytes = (long long)p.M * p.K * 2, b_bytes = (long long)p.K * p.N * 2;
    const int NS = p.K / KS;

    uint4v g[2 * LPO];
    __amdgpu_buffer_rsrc_t ar, br;
    auto stage_rsrc = [&](int st) {
        const bool live = st < NS;
        const long long abase = live ? (long long)m0 * p.K + (long long)st * KS : 0;
        const long long bbase = live ? (long long)st * KS * p.N + n0 : 0;
        const int anrec = __builtin_amdgcn_readfirstlane(live ? (int)(a_bytes - 2 * abase) : 0);
        const int bnrec = __builtin_amdgcn_readfirstlane(live ? (int)(b_bytes - 2 * bbase) : 0);
        ar = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.a + abase), 0, anrec, kBufRaw);
        br = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.b + bbase), 0, bnrec, kBufRaw);
    };
    auto load_one = [&](int i) {
        if (i < LPO) g[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[i], 0, 0);
        else g[i] = __builtin_amdgcn_raw_buffer_load_b128(br, boff[i - LPO], 0, 0);
    };
    auto write_one = [&](uint16_t* cp, int i) {
        if (i < LPO) *reinterpret_cast<uint4v*>(cp + aw + i * AMJ * KS) = g[i];
        else *reinterpret_cast<uint4v*>(cp + bw + (i - LPO) * 8 * kTN) = g[i];
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // fragment addresses (halves within a copy), as in the first form
    int arow[4], arot[4];
#pragma unroll
    for (int rm = 0; rm < 4; ++rm) {
        const int row = wm * 128 + rm * 32 + lj;
        arow[rm] = row * KS;
        arot[rm] = C::rot(row);
    }
    const int L = lane & 15;
    const int brow = 8 * lh + (L >> 2);
    int bcol[4];
#pragma unroll
    for (int rn = 0; rn < 4; ++rn) {
        const int n = wn * 128 + rn * 32 + 16 * (lj >> 4) + 4 * (L & 3);
        bcol[rn] = ((((n >> 3) ^ (2 * (brow & 3)))) << 3) | (n & 7);
    }
    // read r (0..11) of step t's fragments from copy cp: A rows first, then
    // the two transposing reads of each B column block
    uint4v a[2][4];
    uint2v bl[2][4], bh[2][4];
    auto read_one = [&](const uint16_t* cp, int t, int set, int r) {
        if (r < 4) {
            a[set][r] = *reinterpret_cast<const uint4v*>(cp + arow[r] + (((2 * t + lh) ^ arot[r]) << 3));
        } else {
            const int rn = (r - 4) >> 1;
            const uint16_t* q = cp + C::A_H + (16 * t + brow + 4 * ((r - 4) & 1)) * kTN + bcol[rn];
            const uint2v v = __builtin_bit_cast(uint2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)q));
            if ((r & 1) == 0) bl[set][rn] = v;
            else bh[set][rn] = v;
        }
    };

    // ---- prologue: stage 0 into copy 0, stage 1 into registers
    stage_rsrc(0);
#pragma unroll
    for (int i = 0; i < 2 * LPO; ++i) load_one(i);
    e_bias[tid] = e_b;
    e_rs[tid] = (e_row && p.epilogue == EPI_EXP_BIAS_RSQRT) ? dev_rsqrt(e_v + p.eps) : 1.0f;
#pragma unroll
    for (int i = 0; i < 2 * LPO; ++i) write_one(lds0, i);
    stage_rsrc(1);
#pragma unroll
    for (int i = 0; i < 2 * LPO; ++i) load_one(i);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 12; ++r) read_one(lds0, 0, 0, r);

    auto stage = [&](int st, const uint16_t* cur, uint16_t* oth) {
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            const int c = t & 1, n = c ^ 1;
            uint4v bf[4];
#pragma unroll
            for (int rn = 0; rn < 4; ++rn)
                bf[rn] = uint4v{bl[c][rn].x, bl[c][rn].y, bh[c][rn].x, bh[c][rn].y};
            if (t == STEPS - 3) stage_rsrc(st + 2);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc[i >> 2][i & 3] = GMma<DT>::mma(a[c][i >> 2], bf[i & 3], acc[i >> 2][i & 3]);
                if (i < 12) {
                    if (t + 1 < STEPS) read_one(cur, t + 1, n, i);
                    else read_one(oth, 0, n, i);  // the next stage's first step (written before the barrier)
                }
                // steps STEPS-3 and STEPS-2: write a held chunk, then load its successor into it
                if (t == STEPS - 3 && i < LPO) { write_one(oth, i); load_one(i); }
                if (t == STEPS - 2 && i < LPO) { write_one(oth, LPO + i); load_one(LPO + i); }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (t == STEPS - 2) __syncthreads();  // the other copy is whole; this copy's reads are done
        }
    };
    static_assert(2 * LPO <= 16, "one load or write between instructions");
    int st = 0;
    for (; st + 1 < NS; st += 2) {
        stage(st, lds0, lds1);
        stage(st + 1, lds1, lds0);
    }
    if (st < NS) stage(st, lds0, lds1);

    store_block(p, acc, m0, n0, wm, wn, lane, e_bias, e_rs);
}

// The shapes the kernel serves: batch 1, 1x1, stride 1, no padding, one
// split, KS channels a stage (K a multiple of KS); byte offsets of both
// operands within 31 bits.
template <int KS>
int hgemm_lds_bytes(const ConvParams& p) {
    if (p.N != 1 || p.KH != 1 || p.KW != 1 || p.stride != 1 || p.pad != 0) return 1 << 30;
    if (p.kc != KS || p.S != 1 || (long long)p.stages * KS != p.CI) return 1 << 30;
    if (p.P >= (1LL << 31)) return 1 << 30;
    const long long tiles_m = (p.CO + kTM - 1) / kTM, tiles_n = (p.P + kTN - 1) / kTN;
    if (tiles_m * kTM * (long long)p.CI * 2 >= (1LL << 31)) return 1 << 30;
    if ((long long)p.CI * (tiles_n * kTN) * 2 >= (1LL << 31)) return 1 << 30;
    return HG<KS>::LDS;
}

template <int DT, int KS, int CB>
hipError_t hgemm_launch_v(const HGemmParams& q, int grid, hipStream_t stream) {
    auto kern = igemm_h_gemm_kernel<DT, KS, CB>;
    static std::atomic<int> lds_set{0};
    if (!lds_set.load(std::memory_order_relaxed)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, HG<KS>::LDS);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e;
        }
        lds_set.store(1, std::memory_order_relaxed);
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kNT), HG<KS>::LDS, stream, q);
    return hipGetLastError();
}

template <int DT, int KS>
hipError_t hgemm_launch_rs(const HGemmParams& q, int grid, hipStream_t stream) {
    (void)hipGetLastError();
    // all LDS is static (HG<KS>::LDS bytes)
    hipLaunchKernelGGL((igemm_h_gemm_rs_kernel<DT, KS>), dim3((unsigned)grid), dim3(kNT), 0, stream, q);
    return hipGetLastError();
}

template <int DT, int KS>
hipError_t hgemm_launch(const ConvParams& p, hipStream_t stream) {
    if (hgemm_lds_bytes<KS>(p) > 163840) return hipErrorInvalidValue;
    HGemmParams q{};
    q.a = static_cast<const uint16_t*>(p.w);
    q.b = static_cast<const uint16_t*>(p.x);
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
    // bytes the XCDs fetch, (8/ga) * |A| + ga * |B|, among those that divide
    // the grid
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
    // the widest load every slot of both operands allows
    const uintptr_t al = reinterpret_cast<uintptr_t>(p.x) | reinterpret_cast<uintptr_t>(p.w);
    if (al % 16 == 0 && q.K % 8 == 0 && q.N % 8 == 0) {
        // the register-staged form needs at least three steps a stage
        if constexpr (KS == 64) return hgemm_launch_rs<DT, KS>(q, grid, stream);
        else return hgemm_launch_v<DT, KS, 16>(q, grid, stream);
    }
    if (al % 4 == 0 && q.K % 2 == 0 && q.N % 2 == 0) return hgemm_launch_v<DT, KS, 4>(q, grid, stream);
    return hgemm_launch_v<DT, KS, 2>(q, grid, stream);
}

#define CT_HGEMM_VARIANT(NAME, DT, KS)                                                               \
    {NAME, DT, 32, 32, 16, 2, 2, 1, 4, 4, KS, &hgemm_lds_bytes<KS>, &hgemm_launch<DT, KS>, nullptr, 0, 0, 0}

const IgemmVariant kHGemmVariants[] = {
    CT_HGEMM_VARIANT("hgf16_m256n256_w2x2_r4x4_k32", DT_F16, 32),
    CT_HGEMM_VARIANT("hgf16_m256n256_w2x2_r4x4_k64", DT_F16, 64),
    CT_HGEMM_VARIANT("hgbf16_m256n256_w2x2_r4x4_k32", DT_BF16, 32),
    CT_HGEMM_VARIANT("hgbf16_m256n256_w2x2_r4x4_k64", DT_BF16, 64),
};

}  // namespace

const IgemmVariant* igemm_f16_gemm_variants(int* count) {
    *count = (int)(sizeof(kHGemmVariants) / sizeof(kHGemmVariants[0]));
    return kHGemmVariants;
}

}  // namespace ct
