// fp32 implicit-GEMM convolution for batch-1 layers with very few input
// channels and a large filter: the 3-channel 7x7 stride-2 first layer of the
// ResNet-18-style sweep (1 x 3 x 224 x 224 -> 64, 7x7, stride 2, pad 3).
// Layer geometry and channel count are template arguments.
//
// Why a separate kernel.  The reduction is CI*KH*KW = 147 long.  Giving each
// of the 16x16x4 instruction's four lane groups its own input channel (the
// shape-specialised kernel's mapping) would leave 13 of every 16 channel
// slots empty at CI = 3.  Here the lane groups split the filter rows instead:
// lane group g takes filter rows ky = g + 4a (a = 0, 1; row 7 does not exist
// and gets a zero filter value), and matrix step (c, kx) feeds it the
// reduction index (c, g + 4a, kx).  The lane group's row g + 4a is folded
// into the lane's LDS base address, so every B read is one ds_read_b32 with a
// compile-time displacement c*XCS + kx.
//
// Workgroup = MT x 16 output channels x one column tile of 4 output rows x 16
// output columns (one 16-column matrix block per output row; whole rows of 64
// bytes, so the results leave as aligned 16-byte stores).  Waves: MT channel
// tiles x WC channel groups x 2 row sets; a wave loops over its group's
// CI / WC channels.  The whole reduction fits one workgroup: no split, no
// workspace.  The 2*WC partial tiles of a channel tile are summed in LDS in
// wave order.  Each workgroup stages its tile's receptive field once for all
// its channel tiles: (OTH-1)*STR + 8 rows (the eighth filter row's inputs are
// read with a zero filter value) x (OTW-1)*STR + KW columns per channel, zeros
// for padding.
//
// XM: with G tiles rounded up to G8 = 8*ceil(G/8) workgroups, workgroup b
// computes tile (b % 8) * (G8 / 8) + b / 8 (and exits if that is >= G), so
// with workgroups placed round-robin over the 8 XCDs each XCD writes whole
// bands of output rows and reads one band of the input.  The mapping is a
// permutation whatever the placement: only the speed depends on it.
#include "ct_device.hpp"
#include "igemm_common.hpp"

namespace ct {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRowsT = 16;  // output channels per channel tile
constexpr int kTileT = 64;  // pixels of a column tile (4 x 16)
constexpr int kRST = 68;    // reduction row: 64 columns + 4, 16-byte rows that start on different banks
constexpr int kQuads = 16;  // 16-byte column groups of a reduction row

// Workgroup barrier for LDS traffic only: loads into registers may still be
// in flight (the compiler waits for each where its value is used).
__device__ __forceinline__ void lds_sync_t() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: lgkmcnt(0) only
    asm volatile("s_barrier" ::: "memory");
}

// channel slot: >= the window's words, a multiple of 4, not a multiple of 32
// banks apart
constexpr int slot_t(int words) {
    int x = (words + 3) / 4 * 4;
    while ((x % 32) < 8 || (x % 32) > 24) x += 4;
    return x;
}

template <int H_, int W_, int K_, int STR_, int PAD_, int CI_>
struct StemShape {
    static constexpr int H = H_, W = W_, KH = K_, KW = K_, STR = STR_, PAD = PAD_, CI = CI_;
    static constexpr int OH = (H + 2 * PAD - KH) / STR + 1;
    static constexpr int OW = (W + 2 * PAD - KW) / STR + 1;
    static constexpr int P = OH * OW;
    static constexpr int OTH = 4, OTW = 16, PT = OTH * OTW;
    static constexpr int TQW = OW / OTW, NQ = (OH / OTH) * TQW;
    static constexpr int NA = (KH + 3) / 4;              // row sets: filter rows per lane group
    static constexpr int WR = (OTH - 1) * STR + 4 * NA;  // window rows: every row a lane group reads
    static constexpr int WP = (OTW - 1) * STR + KW;      // window row pitch
    static constexpr int RC = WR * WP;
    static constexpr int XCS = slot_t(RC);
    static_assert(OH % OTH == 0 && OW % OTW == 0, "whole 4 x 16 tiles");
    static_assert(PT == kTileT && OTW == 16, "one matrix block per output row");
};

template <class SH, int MT, int WC>
struct SktCfg {
    static constexpr int CPW = SH::CI / WC;  // channels per wave
    static constexpr int NW = MT * WC * SH::NA;
    static constexpr int NT = NW * 64;
    static constexpr int XE = (SH::CI * SH::RC + NT - 1) / NT;
    static constexpr int NPART = WC * SH::NA;  // partial tiles per channel tile
    static constexpr int RED_OFF = SH::CI * SH::XCS;
    static constexpr int WORDS = RED_OFF + NW * kRowsT * kRST + 1;  // + a word for stores past the window
    static constexpr int ITEMS = MT * kRowsT * kQuads;        // output items: (row, column group)
    static_assert(SH::CI % WC == 0, "channel groups divide the channels");
    static_assert(NT <= 1024, "workgroup size");
};

struct SktParams {
    const float* x;
    const float* w;
    float* y;
    const float* bias;
    const float* var;
    float eps;
    int CO, epilogue, tiles, tiles8;  // tiles8: tiles rounded up to a multiple of 8
    int y16;                          // y is 16-byte aligned
};

template <class SH, int MT, int WC, bool XM>
__global__ __launch_bounds__((SktCfg<SH, MT, WC>::NT)) void igemm_f32_skt_kernel(SktParams p) {
    using C = SktCfg<SH, MT, WC>;
    constexpr int NT = C::NT, XE = C::XE, KW = SH::KW, KH = SH::KH, CPW = C::CPW;
    constexpr int HW = SH::H * SH::W;
    extern __shared__ __align__(16) float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;
    int tile = blockIdx.x;
    if constexpr (XM) {
        tile = (tile & 7) * (p.tiles8 >> 3) + (tile >> 3);
        if (tile >= p.tiles) return;  // workgroup-uniform, before any barrier
    }
    const int tm = tile / SH::NQ;
    const int tq = tile - tm * SH::NQ;
    const int qy0 = (tq / SH::TQW) * SH::OTH, qx0 = (tq % SH::TQW) * SH::OTW;
    const int co0 = tm * (MT * kRowsT);
    // wave = ((m * WC) + cg) * NA + a
    const int wa = wave % SH::NA;
    const int wcg = (wave / SH::NA) % WC;
    const int wm = wave / (SH::NA * WC);
    const int co_a = co0 + wm * kRowsT + li;

    // ---- loads first: the tile's receptive field, then A -------------------
    // Every load reads a valid address (an out-of-range element reads element
    // 0) and the value is zeroed afterwards: no branches around the loads.
    float xr[XE];
    int xdst[XE];
    unsigned xok = 0;
#pragma unroll
    for (int j = 0; j < XE; ++j) {
        const int e = j * NT + tid;
        const int c = e / SH::RC;
        const int rem = e - c * SH::RC;
        const int r = rem / SH::WP;
        const int iy = qy0 * SH::STR - SH::PAD + r;
        const int ix = qx0 * SH::STR - SH::PAD + rem - r * SH::WP;
        const bool in = e < SH::CI * SH::RC;
        const bool ok = in && iy >= 0 && iy < SH::H && ix >= 0 && ix < SH::W;
        xr[j] = p.x[ok ? c * HW + iy * SH::W + ix : 0];
        xok |= (ok ? 1u : 0u) << j;
        xdst[j] = in ? c * SH::XCS + rem : C::WORDS - 1;
    }
    // A for step (cc, kx): W[co_a][wcg*CPW + cc][lg + 4*wa][kx]; zero past the filter
    float a[CPW][KW];
    const int ky = lg + 4 * wa;
    const bool aok = co_a < p.CO && ky < KH;
    {
        const float* src = p.w + (aok ? (co_a * SH::CI + wcg * CPW) * (KH * KW) + ky * KW : 0);
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
            for (int t = 0; t < KW; ++t) a[cc][t] = src[cc * KH * KW + t];
    }
    __builtin_amdgcn_sched_barrier(0);

    // B read base: channel group, lane group's filter row, column li's (0,0)
    // tap; block nb (output row nb) adds nb*STR*WP
    constexpr int NB = SH::OTH;
    const float* bptr = lds + wcg * CPW * SH::XCS + ky * SH::WP + li * SH::STR;

#pragma unroll
    for (int j = 0; j < XE; ++j) lds[xdst[j]] = (xok >> j) & 1 ? xr[j] : 0.0f;
    lds_sync_t();
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
        for (int t = 0; t < KW; ++t) a[cc][t] = aok ? a[cc][t] : 0.0f;

    // ---- matrix steps (cc, kx), B read one step ahead ----------------------
    constexpr int NS = CPW * KW;
    floatx4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float b[2][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[0][nb] = bptr[nb * SH::STR * SH::WP];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int cc = s / KW, kx = s % KW;
        const int nd = (s + 1) / KW * SH::XCS + (s + 1) % KW;  // next step's displacement
        float(&cur)[NB] = b[s & 1];
        float(&nxt)[NB] = b[(s + 1) & 1];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[cc][kx], cur[nb], acc[nb], 0, 0, 0);
            if (s + 1 < NS) nxt[nb] = bptr[nb * SH::STR * SH::WP + nd];
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- sum the partial tiles in LDS, epilogue, store ----------------------
    float* red = lds + C::RED_OFF + wave * kRowsT * kRST;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(4 * lg + r) * kRST + nb * 16 + li] = acc[nb][r];
    lds_sync_t();
#pragma unroll
    for (int it = 0; it < (C::ITEMS + NT - 1) / NT; ++it) {
        const int item = it * NT + tid;
        if (item >= C::ITEMS) break;
        const int row = item / kQuads;  // the workgroup's channel row
        const int oq = item - row * kQuads;
        const int oco = co0 + row;
        if (oco >= p.CO) break;  // later items have later rows
        const int m = row / kRowsT, rr = row - m * kRowsT;
        floatx4 sum = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < C::NPART; ++w)
            sum += *reinterpret_cast<const floatx4*>(lds + C::RED_OFF + ((m * C::NPART + w) * kRowsT + rr) * kRST +
                                                     4 * oq);
        float e_b = 0.0f, e_r = 1.0f;
        if (p.epilogue != EPI_NONE) {
            e_b = p.bias[oco];
            if (p.epilogue == EPI_EXP_BIAS_RSQRT) e_r = dev_rsqrt(p.var[oco] + p.eps);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] = apply_epilogue(p.epilogue, sum[i], e_b, e_r);
        // pixels 4*oq .. 4*oq+3 of the tile: one output row, 16-byte aligned
        const int py = qy0 + oq / (SH::OTW / 4), px = qx0 + 4 * (oq % (SH::OTW / 4));
        if (p.y16)
            *reinterpret_cast<floatx4*>(p.y + (long long)oco * SH::P + py * SH::OW + px) = sum;
        else
#pragma unroll
            for (int i = 0; i < 4; ++i) p.y[(long long)oco * SH::P + py * SH::OW + px + i] = sum[i];
    }
}

template <class SH, int MT, int WC, bool XM>
int skt_lds_bytes(const ConvParams& p) {
    if (p.N != 1 || p.H != SH::H || p.W != SH::W || p.KH != SH::KH || p.KW != SH::KW ||
        p.stride != SH::STR || p.pad != SH::PAD || p.CI != SH::CI)
        return 1 << 30;  // compiled for one layer geometry and channel count
    // the whole reduction in one workgroup: one split, one stage of all channels
    if (p.S != 1 || p.stages != 1 || p.kc != SH::CI) return 1 << 30;
    if ((p.P + kTileT - 1) / kTileT != SH::NQ) return 1 << 30;
    static_assert(SH::OW % 4 == 0 && SH::P % 4 == 0, "16-byte output rows");
    return 4 * SktCfg<SH, MT, WC>::WORDS;
}

template <class SH, int MT, int WC, bool XM>
hipError_t skt_launch(const ConvParams& p, hipStream_t stream) {
    const int bytes = skt_lds_bytes<SH, MT, WC, XM>(p);
    if (bytes > 163840 - 64) return hipErrorInvalidValue;
    // the runtime's channel tiles are MT x 16 rows: tiles_m = ceil(CO / (16 MT))
    if (p.tiles_m != (p.CO + MT * kRowsT - 1) / (MT * kRowsT)) return hipErrorInvalidValue;
    SktParams q{};
    q.x = static_cast<const float*>(p.x);
    q.w = static_cast<const float*>(p.w);
    q.y = p.y;
    q.bias = p.bias;
    q.var = p.var;
    q.eps = p.eps;
    q.CO = p.CO;
    q.epilogue = p.epilogue;
    q.tiles = p.tiles_m * SH::NQ;
    q.tiles8 = (q.tiles + 7) / 8 * 8;
    q.y16 = (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;
    (void)hipGetLastError();
    hipLaunchKernelGGL((igemm_f32_skt_kernel<SH, MT, WC, XM>), dim3((unsigned)(XM ? q.tiles8 : q.tiles)),
                       dim3(SktCfg<SH, MT, WC>::NT),
                       bytes, stream, q);
    return hipGetLastError();
}

using Stem224 = StemShape<224, 224, 7, 2, 3, 3>;  // 3 x 224 x 224, 7x7, stride 2, pad 3

// descriptor: 16x16x4 instruction, waves MT x 1 x (WC * row sets) (CO x P x K),
// reps 1 x 4 (column tiles of 64 pixels), kc = CI (the whole reduction in one
// stage)
#define CT_SKT_VARIANT(NAME, SH, MT, WC, XM)                                                                 \
    {NAME, DT_F32, 16, 16, 4, MT, 1, WC * SH::NA, 1, 4, SH::CI, &skt_lds_bytes<SH, MT, WC, XM>, \
     &skt_launch<SH, MT, WC, XM>, nullptr, 0, 0}

const IgemmVariant kSktVariants[] = {
    CT_SKT_VARIANT("f32skt224_m1_g3", Stem224, 1, 3, false),
    CT_SKT_VARIANT("f32skt224_m2_g1", Stem224, 2, 1, false),
    CT_SKT_VARIANT("f32skt224_m4_g1", Stem224, 4, 1, false),
    CT_SKT_VARIANT("f32skt224_m2_g3", Stem224, 2, 3, false),
    CT_SKT_VARIANT("f32skt224x_m1_g3", Stem224, 1, 3, true),
    CT_SKT_VARIANT("f32skt224x_m2_g1", Stem224, 2, 1, true),
    CT_SKT_VARIANT("f32skt224x_m4_g1", Stem224, 4, 1, true),
    CT_SKT_VARIANT("f32skt224x_m2_g3", Stem224, 2, 3, true),
};

}  // namespace

const IgemmVariant* igemm_f32_skt_variants(int* count) {
    *count = (int)(sizeof(kSktVariants) / sizeof(kSktVariants[0]));
    return kSktVariants;
}

}  // namespace ct
