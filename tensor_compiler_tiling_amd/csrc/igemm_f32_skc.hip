// fp32 implicit-GEMM convolution, split-K across workgroups, for batch-1
// layers whose whole output is 49 pixels (7 x 7): the final ResNet layer of
// the TVM tutorial "Tuning High Performance Convolution on NVIDIA GPUs"
// (Step 1: 1 x 512 x 7 x 7 -> 512, 3 x 3, stride 1, pad 1) and the stride-2
// layer that produces the same output size.  The layer geometry is a
// template argument, so every index below is compile-time arithmetic.
//
// Why a shape-specialised kernel.  At this size a workgroup does about 50
// matrix instructions per wave between one HBM round trip and the split
// reduction, so instruction count on the critical path is the cost:
//  - B operand: a lane's LDS address is a per-lane base plus a compile-time
//    displacement per matrix step, so each B value is one ds_read_b32 with an
//    immediate offset (no address arithmetic inside the matrix loop), and
//    the reads of step s+2 are placed between the matrix instructions of
//    step s, where they issue while the matrix core is busy.
//  - Columns: 49 = 3 x 16 + 1.  Three 16-column blocks run on
//    v_mfma_f32_16x16x4_f32 and the 49th column is a VALU FMA per step,
//    instead of a fourth, 15/16-empty matrix block (a quarter of the matrix
//    time at this size).
//  - Prologue: the window and filter loads are issued first; LDS zeroing and
//    every address computation run while they are in flight.
//
// Reduction index k = (c, tap) with c the input channel and tap = ky*KW+kx.
// Stage: KC = 4*NW*CPL channels.  Wave w, lane group g = lane/16 owns the
// channels cl = w*4*CPL + 4*j + g (j < CPL) of the stage; matrix step
// s = j*T + tap feeds lane group g with k = (c0 + cl, tap).  A lane's A values
// for a channel are the T consecutive floats of its filter row; its B value
// for pixel column col is the zero-padded window word
//     Xs[cl*XCS + (oy*STR + ky)*WP + ox*STR + kx]
//   = Xs[lane base + pbase(col)] displaced by 4*j*XCS + ky*WP + kx.
// (Any assignment of k to (step, lane group) is valid when A and B share it.)
//
// Split reduction: as in the other split-K kernels -- the waves' partial
// tiles are summed in LDS in wave order, each workgroup stores its partial
// tile with device-coherent 16-byte stores and takes a ticket, and the last
// to arrive sums the S partials in split order 0..S-1 (run-to-run
// identical), applies the epilogue and stores y.  Workgroup b handles split
// b % S of output-channel tile b / S.
//
// XCD-local form (XL).  Each round trip of that protocol at device scope --
// the coherent partial store, the ticket, the reducer's loads -- goes past
// the L2 of the workgroup's XCD and costs about half a microsecond.  On an
// MI355X workgroup b runs on XCD b % 8, and each XCD's L2 is the coherence
// point of its CUs.  The XL form gives all S workgroups of a tile the same
// b % 8 (tile = b%8 + 8*((b/8)/S), split = (b/8) % S), so the protocol runs
// through that one L2: plain stores, a workgroup-scope atomic (executed in
// L2), loads that skip the CU's L1.  Kernel boundaries write the L2 back.
// The runtime enables XL variants only on a device where a probe launch
// has observed the b % 8 placement.
#include "ct_device.hpp"
#include "igemm_common.hpp"

#include <atomic>

namespace ct {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit elements
constexpr int kCoherent = 16;          // cache policy: device-coherent (sc1)
constexpr int kSkipL1 = 1;             // cache policy: sc0, the load misses the CU's L1
constexpr int kRowsM = 16;             // output channels per tile
constexpr int kRS = 52;                // reduction / partial row: 49 columns, 16-byte rows
constexpr int kSlab = kRowsM * kRS;    // floats per partial tile
constexpr int kTileP = 49;             // pixels of a column tile (7 x 7), the runtime's tile width
static_assert(kRS == (kTileP + 3) / 4 * 4, "partial rows are the runtime's 16-byte padded tile rows");

// Workgroup barrier for LDS traffic only: loads into registers may still be
// in flight (the compiler waits for each where its value is used).
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: lgkmcnt(0) only
    asm volatile("s_barrier" ::: "memory");
}

constexpr int cround4(int v) { return (v + 3) / 4 * 4; }
// channel slot of the LDS window: >= R*WP words, a multiple of 4, and not a
// multiple of 32 banks apart, so the lane groups' slots start on different
// banks
constexpr int window_slot(int words) {
    int x = cround4(words);
    while ((x % 32) < 8 || (x % 32) > 24) x += 4;
    return x;
}

// TQ: the output is cut into TQ x TQ column tiles of (OH/TQ) x (OW/TQ)
// pixels (a 14 x 14 output into four 7 x 7 quadrants).
// WIN = false: the LDS window holds the whole zero-padded image (staged with
// 16-byte loads of the channels' contiguous data, padding zeroed once), and a
// tile reads it at its own offset.  WIN = true: the window holds only the
// tile's receptive field, (OTH-1)*STR+KH rows x (OTW-1)*STR+KW columns,
// staged word by word with zeros for padding (large images).
template <int H_, int W_, int KH_, int KW_, int STR_, int PAD_, int TQ_ = 1, bool WIN_ = false>
struct LayerShape {
    static constexpr int H = H_, W = W_, KH = KH_, KW = KW_, STR = STR_, PAD = PAD_, TQ = TQ_;
    static constexpr bool WIN = WIN_;
    static constexpr int OH = (H + 2 * PAD - KH) / STR + 1;
    static constexpr int OW = (W + 2 * PAD - KW) / STR + 1;
    static constexpr int P = OH * OW;  // batch 1
    static constexpr int OTH = OH / TQ, OTW = OW / TQ;  // a column tile's output rows, columns
    static constexpr int PT = OTH * OTW;                // pixels of a column tile
    static constexpr int NQ = TQ * TQ;                  // column tiles
    static constexpr int T = KH * KW;
    static constexpr int HW = H * W;
    static constexpr int WR = WIN ? (OTH - 1) * STR + KH : (OH - 1) * STR + KH;  // window rows
    static constexpr int WP = WIN ? (OTW - 1) * STR + KW : W + 2 * PAD;          // window row pitch
    static constexpr int RC = WR * WP;               // window words per channel
    static constexpr int XCS = window_slot(RC);      // words per channel slot
    static constexpr int NBM = PT / 16;              // 16-column matrix blocks
    static constexpr int VT = PT - 16 * NBM;         // VALU tail columns
    static_assert(OH % TQ == 0 && OW % TQ == 0, "whole column tiles");
    static_assert(VT <= 1, "at most one VALU tail column");
    static_assert(WIN || (PAD + H <= WR && PAD + W <= WP), "the window holds the whole image");
    static_assert(PT <= kRS, "partial rows hold every column");
};

// Kernel arguments: two 64-byte lines, all loaded at entry.
struct SkcParams {
    const float* x;
    const float* w;
    float* y;
    float* ws;
    unsigned* tickets;
    const float* zero;  // >= 256 zero bytes
    const float* bias;
    const float* var;
    float eps;
    int CI, CO, S, stages, epilogue;
    int tiles;  // output-channel tiles
    int pad_;
};
static_assert(sizeof(SkcParams) <= 128, "two kernel-argument lines");

template <class SH, int NW, int CPL>
struct SkcCfg {
    static constexpr int NT = NW * 64;
    static constexpr int KC = 4 * NW * CPL;        // channels per stage
    static constexpr int KSTEP = CPL * SH::T;      // matrix steps per wave per stage
    // window words per thread: whole-image form, the stage's KC*H*W floats in
    // 16-byte groups; windowed form, the KC*RC window words one by one
    static constexpr int XE = SH::WIN ? (KC * SH::RC + NT - 1) / NT : cround4((KC * SH::HW + NT - 1) / NT);
    // LDS words: windows | reduction | tail | one word that takes the stores
    // of staged words past the stage's data.  The window zeroing covers whole
    // rounds of the threads' 16-byte stores (it may run into the reduction
    // area, which is written only after the matrix steps).
    static constexpr int RED_OFF = KC * SH::XCS;
    static constexpr int TAIL_OFF = RED_OFF + NW * kSlab;
    static constexpr int DUMMY = TAIL_OFF + NW * kRowsM;
    static constexpr int ZERO_ROUNDS = SH::WIN ? 0 : (KC * SH::XCS / 4 + NT - 1) / NT;
    static constexpr int WORDS = (DUMMY + 1 > ZERO_ROUNDS * NT * 4) ? DUMMY + 1 : ZERO_ROUNDS * NT * 4;
    static constexpr int NB = SH::NBM + SH::VT;    // B reads per step
    static constexpr int D = 2;                    // B reads run D steps ahead
    static_assert(NT >= 256, "the reduction uses 16 x 16 threads");
    static_assert(SH::WIN || (KC * SH::HW) % 4 == 0, "a stage is whole 16-byte groups");
    static_assert(SH::T <= 64, "a filter run of the zero block");
};

// XV: x is 16-byte aligned, so the window loads are 16-byte loads.
// XL: XCD-local split reduction (see above).
template <class SH, int NW, int CPL, bool XV, bool XL>
__global__ __launch_bounds__(NW * 64) void igemm_f32_skc_kernel(SkcParams p) {
    using C = SkcCfg<SH, NW, CPL>;
    constexpr int NT = C::NT, KC = C::KC, KSTEP = C::KSTEP, XE = C::XE, NB = C::NB, D = C::D;
    constexpr int T = SH::T, HW = SH::HW;
    extern __shared__ __align__(16) float lds[];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;
    int tile, split;
    if constexpr (XL) {
        const int idx = blockIdx.x >> 3;
        const int q = idx / p.S;
        tile = (blockIdx.x & 7) + 8 * q;
        split = idx - q * p.S;
        if (tile >= p.tiles) return;  // the last XCD rounds may be short
    } else {
        tile = blockIdx.x / p.S;
        split = blockIdx.x - tile * p.S;
    }
    const int tm = tile / SH::NQ;  // output-channel tile
    const int tq = tile - tm * SH::NQ;  // column tile
    const int qy0 = (tq / SH::TQ) * SH::OTH, qx0 = (tq % SH::TQ) * SH::OTW;  // its first output row, column
    const int co0 = tm * kRowsM;
    const int co_a = co0 + li;
    const bool row_ok = co_a < p.CO;
    const int K = p.CI * T;

    // output-side constants: thread (orow, oq) owns columns 4*oq .. 4*oq+3
    const int orow = (tid & 255) >> 4;
    const int oq = tid & 15;
    const bool out_thread = tid < 256 && oq * 4 < SH::PT;
    const int oco = co0 + orow;
    float e_b = 0.0f, e_v = 1.0f;
    if (out_thread && oco < p.CO && p.epilogue != EPI_NONE) {
        e_b = p.bias[oco];
        if (p.epilogue == EPI_EXP_BIAS_RSQRT) e_v = p.var[oco];
    }

    float xr[XE];
    float a[KSTEP];
    const int cl_lane = wave * 4 * CPL + lg;  // stage-local channel of j = 0

    // Register loads of stage st: this thread's XE window words (flat order
    // of the stage's KC*H*W contiguous floats), then its A values.
    auto issue_loads = [&](int st) {
        const int c0 = (split * p.stages + st) * KC;
        const int E = min(KC, p.CI - c0) * HW;  // valid words of the stage (<= 0: none)
        const float* xblk = p.x + (long long)c0 * HW;
        if constexpr (SH::WIN) {
            // word e = c*RC + r*WP + col of the tile's receptive field: image
            // row qy0*STR - PAD + r, column qx0*STR - PAD + col; zero outside
            const int cv = min(KC, p.CI - c0);
#pragma unroll
            for (int j = 0; j < XE; ++j) {
                const int e = j * NT + tid;
                const int c = e / SH::RC;
                const int rem = e - c * SH::RC;
                const int r = rem / SH::WP;
                const int iy = qy0 * SH::STR - SH::PAD + r;
                const int ix = qx0 * SH::STR - SH::PAD + rem - r * SH::WP;
                const bool ok = e < KC * SH::RC && c < cv && iy >= 0 && iy < SH::H && ix >= 0 && ix < SH::W;
                xr[j] = ok ? xblk[c * HW + iy * SH::W + ix] : 0.0f;
            }
        } else if constexpr (XV) {
#pragma unroll
            for (int j = 0; j < XE / 4; ++j) {
                const int f = 4 * (j * NT + tid);
                // E is a multiple of 4 (the host checks CI*H*W and KC*H*W)
                const floatx4 v = *reinterpret_cast<const floatx4*>(f < E ? xblk + f : p.zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) xr[4 * j + i] = v[i];
            }
        } else {
#pragma unroll
            for (int j = 0; j < XE / 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int f = 4 * (j * NT + tid) + i;
                    xr[4 * j + i] = f < E ? xblk[f] : 0.0f;
                }
        }
        // window loads first in issue order: they are needed first
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = c0 + cl_lane + 4 * j;
            const float* src = (row_ok && c < p.CI) ? p.w + (long long)co_a * K + (long long)c * T : p.zero;
#pragma unroll
            for (int t = 0; t < T; ++t) a[j * T + t] = src[t];
        }
    };
    issue_loads(0);

    // ---- set-up while the first loads are in flight -----------------------
    // window destination of each staged word (past the stage's data: the
    // dummy word)
    int xdst[XE];
    if constexpr (SH::WIN) {
#pragma unroll
        for (int j = 0; j < XE; ++j) {
            const int e = j * NT + tid;
            const int c = e / SH::RC;
            xdst[j] = e < KC * SH::RC ? c * SH::XCS + e - c * SH::RC : C::DUMMY;
        }
    } else {
#pragma unroll
        for (int j = 0; j < XE / 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = 4 * (j * NT + tid) + i;
                const int c = f / HW;
                const int r = f - c * HW;
                const int iy = r / SH::W;
                const int ix = r - iy * SH::W;
                xdst[4 * j + i] = f < KC * HW ? c * SH::XCS + (iy + SH::PAD) * SH::WP + ix + SH::PAD : C::DUMMY;
            }
    }
    // B read bases: lane slot plus the column's (0,0)-tap offset
    const float* bptr[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int px = nb < SH::NBM ? nb * 16 + li : 16 * SH::NBM;  // tail: the one extra column
        // window row / column of the pixel's (0,0) tap: the whole-image window
        // starts at padded row and column 0, the tile window at the tile
        const int oy = (SH::WIN ? 0 : qy0) + px / SH::OTW;
        const int ox = (SH::WIN ? 0 : qx0) + px % SH::OTW;
        bptr[nb] = lds + cl_lane * SH::XCS + oy * SH::STR * SH::WP + ox * SH::STR;
    }
    // whole-image form: padding words are the same in every stage, zero the
    // windows once (the tile-window form stages its zeros with the data)
    if constexpr (!SH::WIN) {
        floatx4* xz = reinterpret_cast<floatx4*>(lds);
#pragma unroll
        for (int i = 0; i < C::ZERO_ROUNDS; ++i) xz[i * NT + tid] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        lds_sync();
    }

    floatx4 acc[SH::NBM];
#pragma unroll
    for (int nb = 0; nb < SH::NBM; ++nb) acc[nb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float acc_t = 0.0f;  // VALU tail column, this lane group's k only

    for (int st = 0; st < p.stages; ++st) {
        if (st > 0) {
            // registers are free: load this stage, then wait until every
            // wave is done reading the previous windows
            issue_loads(st);
            lds_sync();
        }
        // window data into LDS (waits for the window loads only)
#pragma unroll
        for (int e = 0; e < XE; ++e) lds[xdst[e]] = xr[e];
        lds_sync();

        // ---- matrix steps: B reads of step s+D between the instructions of
        //      step s; compile-time displacements (immediate offsets)
        float b[D + 1][NB];
        auto read_b = [&](int s, float (&dst)[NB]) {
            const int j = s / T, t = s - (s / T) * T;
            const int disp = 4 * j * SH::XCS + (t / SH::KW) * SH::WP + (t % SH::KW);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) dst[nb] = bptr[nb][disp];
        };
#pragma unroll
        for (int s = 0; s < D && s < KSTEP; ++s) read_b(s, b[s]);
#pragma unroll
        for (int s = 0; s < KSTEP; ++s) {
            float(&cur)[NB] = b[s % (D + 1)];
            float(&nxt)[NB] = b[(s + D) % (D + 1)];
            const int sn = s + D;
            const int jn = sn / T, tn = sn - (sn / T) * T;
            const int dn = 4 * jn * SH::XCS + (tn / SH::KW) * SH::WP + (tn % SH::KW);
#pragma unroll
            for (int nb = 0; nb < SH::NBM; ++nb) {
                acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], cur[nb], acc[nb], 0, 0, 0);
                if (sn < KSTEP) nxt[nb] = bptr[nb][dn];
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (SH::VT == 1) {
                acc_t = __builtin_fmaf(a[s], cur[SH::NBM], acc_t);
                if (sn < KSTEP) nxt[SH::NBM] = bptr[SH::NBM][dn];
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // ---- sum the waves' accumulators in LDS --------------------------------
    // C layout of v_mfma_f32_16x16x4_f32: row 4*(lane/16) + r, column lane%16.
    float* red = lds + C::RED_OFF + wave * kSlab;
#pragma unroll
    for (int nb = 0; nb < SH::NBM; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(4 * lg + r) * kRS + nb * 16 + li] = acc[nb][r];
    if constexpr (SH::VT == 1) {
        // the tail column of row li: sum the four lane groups' k
        acc_t += __shfl_xor(acc_t, 16);
        acc_t += __shfl_xor(acc_t, 32);
        if (lg == 0) lds[C::TAIL_OFF + wave * kRowsM + li] = acc_t;
    }
    lds_sync();
    floatx4 sum = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (out_thread) {
        if (oq < SH::NBM * 4) {
#pragma unroll
            for (int w = 0; w < NW; ++w)
                sum += *reinterpret_cast<const floatx4*>(lds + C::RED_OFF + w * kSlab + orow * kRS + 4 * oq);
        } else {
#pragma unroll
            for (int w = 0; w < NW; ++w) sum[0] += lds[C::TAIL_OFF + w * kRowsM + orow];
        }
    }
    const float e_r = p.epilogue == EPI_EXP_BIAS_RSQRT ? dev_rsqrt(e_v + p.eps) : 1.0f;
    auto store_out = [&](const floatx4& v) {
        if (!(out_thread && oco < p.CO)) return;
        float* yrow = p.y + (long long)oco * SH::P;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * oq + i;  // pixel of the column tile
            if (c < SH::PT)
                yrow[(qy0 + c / SH::OTW) * SH::OW + qx0 + c % SH::OTW] = apply_epilogue(p.epilogue, v[i], e_b, e_r);
        }
    };
    if (p.S == 1) {
        store_out(sum);
        return;
    }

    // ---- split reduction across workgroups ---------------------------------
    float* part = p.ws + (long long)tile * p.S * kSlab;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(part, 0, p.S * kSlab * 4, kBufWord3);
    const int fo = orow * kRS + 4 * oq;
    if (out_thread) {
        uint4v v;
        v.x = __float_as_uint(sum[0]);
        v.y = __float_as_uint(sum[1]);
        v.z = __float_as_uint(sum[2]);
        v.w = __float_as_uint(sum[3]);
        __builtin_amdgcn_raw_buffer_store_b128(v, prs, (split * kSlab + fo) * 4, 0, XL ? 0 : kCoherent);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial store is complete
    __syncthreads();
    if (tid == 0) {
        const unsigned old = XL ? __hip_atomic_fetch_add(&p.tickets[tile * kTicketStride], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_WORKGROUP)
                                : __hip_atomic_fetch_add(&p.tickets[tile * kTicketStride], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (unsigned)(p.S - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;

    // last arriver: sum the S partials in split order, 16 loads in flight
    if (out_thread) {
        constexpr int SB = 16;
        floatx4 tot = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = 0; s0 < p.S; s0 += SB) {
            floatx4 v[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j)
                v[j] = (s0 + j < p.S) ? __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                       prs, ((s0 + j) * kSlab + fo) * 4, 0,
                                                                       XL ? kSkipL1 : kCoherent))
                                      : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < SB; ++j)
                if (s0 + j < p.S) tot = (s0 + j == 0) ? v[j] : tot + v[j];
        }
        store_out(tot);
    }
    if (tid == 0) {
        if constexpr (XL)
            __hip_atomic_store(&p.tickets[tile * kTicketStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        else
            __hip_atomic_store(&p.tickets[tile * kTicketStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <class SH, int NW, int CPL, bool XL>
int skc_lds_bytes(const ConvParams& p) {
    using C = SkcCfg<SH, NW, CPL>;
    if (p.N != 1 || p.H != SH::H || p.W != SH::W || p.KH != SH::KH || p.KW != SH::KW ||
        p.stride != SH::STR || p.pad != SH::PAD)
        return 1 << 30;  // compiled for one layer geometry
    if (p.kc != C::KC) return 1 << 30;  // a stage is exactly the lanes' channels
    // whole 16-byte groups per stage, also at the end of the input
    if (!SH::WIN && ((long long)p.CI * SH::HW) % 4 != 0) return 1 << 30;
    if ((long long)p.S * kSlab * 4 >= (1LL << 31)) return 1 << 30;
    // the runtime's column tiles (kTileP columns each) must be the kernel's
    if ((p.P + kTileP - 1) / kTileP != SH::NQ) return 1 << 30;
    return 4 * C::WORDS;
}

template <class SH, int NW, int CPL, bool XL>
hipError_t skc_launch(const ConvParams& p, hipStream_t stream) {
    using C = SkcCfg<SH, NW, CPL>;
    const int bytes = skc_lds_bytes<SH, NW, CPL, XL>(p);
    if (bytes > 163840 - 64) return hipErrorInvalidValue;
    const bool xv = (reinterpret_cast<uintptr_t>(p.x) & 15) == 0;
    auto kern = xv ? igemm_f32_skc_kernel<SH, NW, CPL, true, XL> : igemm_f32_skc_kernel<SH, NW, CPL, false, XL>;
    static std::atomic<int> lds_limit[2] = {65536, 65536};
    if (bytes > lds_limit[xv].load(std::memory_order_relaxed)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 163840 - 64);
        if (e != hipSuccess) return e;
        lds_limit[xv].store(163840 - 64, std::memory_order_relaxed);
    }
    SkcParams q{};
    q.x = static_cast<const float*>(p.x);
    q.w = static_cast<const float*>(p.w);
    q.y = p.y;
    q.ws = p.ws;
    q.tickets = p.tickets;
    q.zero = static_cast<const float*>(p.zero);
    q.bias = p.bias;
    q.var = p.var;
    q.eps = p.eps;
    q.CI = p.CI;
    q.CO = p.CO;
    q.S = p.S;
    q.stages = p.stages;
    q.epilogue = p.epilogue;
    q.tiles = p.tiles_m * SH::NQ;
    const long long grid = XL ? 8LL * ((q.tiles + 7) / 8) * p.S : (long long)q.tiles * p.S;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), bytes, stream, q);
    return hipGetLastError();
}

using Layer7s1 = LayerShape<7, 7, 3, 3, 1, 1>;    // 7x7 -> 7x7, 3x3, stride 1, pad 1
using Layer14s2 = LayerShape<14, 14, 3, 3, 2, 1>;  // 14x14 -> 7x7, 3x3, stride 2, pad 1
using Layer14q = LayerShape<14, 14, 3, 3, 1, 1, 2>;  // 14x14 -> 14x14 in four 7x7 quadrants
using Layer14q1 = LayerShape<14, 14, 1, 1, 1, 0, 2>;  // 1x1 filter, 14x14, in four 7x7 quadrants
using Layer28s2q = LayerShape<28, 28, 3, 3, 2, 1, 2>;  // 28x28 -> 14x14 stride 2, in four 7x7 quadrants
using Layer56w = LayerShape<56, 56, 3, 3, 1, 1, 8, true>;   // 56x56, 64 tiles of 7x7, tile windows
// tile-window forms of the smaller geometries
using Layer7w = LayerShape<7, 7, 3, 3, 1, 1, 1, true>;
using Layer14qw = LayerShape<14, 14, 3, 3, 1, 1, 2, true>;
using Layer14q1w = LayerShape<14, 14, 1, 1, 1, 0, 2, true>;
using Layer28s2w = LayerShape<28, 28, 3, 3, 2, 1, 2, true>;
using Layer56s2w = LayerShape<56, 56, 3, 3, 2, 1, 4, true>; // 56x56 -> 28x28 stride 2, 16 tiles, tile windows

// descriptor: 16x16x4 instruction, waves 1 x 1 x NW (CO x P x K), reps 1 x 4,
// column tiles of kTileP = 49 pixels, a stage of exactly 4*NW*CPL channels
#define CT_SKC_VARIANT(NAME, SH, NW, CPL, XL)                                                 \
    {NAME, DT_F32, 16, 16, 4, 1, 1, NW, 1, 4, 4 * NW * CPL, &skc_lds_bytes<SH, NW, CPL, XL>, \
     &skc_launch<SH, NW, CPL, XL>, nullptr, XL, kTileP}

const IgemmVariant kSkcVariants[] = {
    CT_SKC_VARIANT("f32skc7_w8_c2", Layer7s1, 8, 2, false),
    CT_SKC_VARIANT("f32skc7_w4_c2", Layer7s1, 4, 2, false),
    CT_SKC_VARIANT("f32skc7_w4_c4", Layer7s1, 4, 4, false),
    CT_SKC_VARIANT("f32skc7_w8_c1", Layer7s1, 8, 1, false),
    CT_SKC_VARIANT("f32skc14s2_w8_c1", Layer14s2, 8, 1, false),
    CT_SKC_VARIANT("f32skc14s2_w4_c2", Layer14s2, 4, 2, false),
    CT_SKC_VARIANT("f32skc7x_w8_c2", Layer7s1, 8, 2, true),
    CT_SKC_VARIANT("f32skc7x_w4_c2", Layer7s1, 4, 2, true),
    CT_SKC_VARIANT("f32skc7x_w8_c1", Layer7s1, 8, 1, true),
    CT_SKC_VARIANT("f32skc14s2x_w8_c1", Layer14s2, 8, 1, true),
    CT_SKC_VARIANT("f32skc14s2x_w4_c2", Layer14s2, 4, 2, true),
    CT_SKC_VARIANT("f32skc14q_w8_c2", Layer14q, 8, 2, false),
    CT_SKC_VARIANT("f32skc14q_w4_c4", Layer14q, 4, 4, false),
    CT_SKC_VARIANT("f32skc14q_w4_c2", Layer14q, 4, 2, false),
    CT_SKC_VARIANT("f32skc14q_w4_c1", Layer14q, 4, 1, false),
    CT_SKC_VARIANT("f32skc14qx_w4_c2", Layer14q, 4, 2, true),
    CT_SKC_VARIANT("f32skc14qx_w4_c1", Layer14q, 4, 1, true),
    CT_SKC_VARIANT("f32skc14q1_w4_c4", Layer14q1, 4, 4, false),
    CT_SKC_VARIANT("f32skc14q1x_w4_c4", Layer14q1, 4, 4, true),
    CT_SKC_VARIANT("f32skc14q1x_w4_c8", Layer14q1, 4, 8, true),
    CT_SKC_VARIANT("f32skc14q1x_w8_c4", Layer14q1, 8, 4, true),
    CT_SKC_VARIANT("f32skc28s2q_w4_c1", Layer28s2q, 4, 1, false),
    CT_SKC_VARIANT("f32skc28s2qx_w4_c1", Layer28s2q, 4, 1, true),
    CT_SKC_VARIANT("f32skc28s2qx_w8_c1", Layer28s2q, 8, 1, true),
    CT_SKC_VARIANT("f32skc56w_w8_c2", Layer56w, 8, 2, false),
    CT_SKC_VARIANT("f32skc56w_w4_c4", Layer56w, 4, 4, false),
    CT_SKC_VARIANT("f32skc56w_w4_c2", Layer56w, 4, 2, false),
    CT_SKC_VARIANT("f32skc56wx_w4_c2", Layer56w, 4, 2, true),
    CT_SKC_VARIANT("f32skc56s2w_w8_c2", Layer56s2w, 8, 2, false),
    CT_SKC_VARIANT("f32skc56s2w_w4_c2", Layer56s2w, 4, 2, false),
    CT_SKC_VARIANT("f32skc56s2wx_w4_c2", Layer56s2w, 4, 2, true),
    CT_SKC_VARIANT("f32skc56s2wx_w8_c1", Layer56s2w, 8, 1, true),
    CT_SKC_VARIANT("f32skc7wx_w8_c1", Layer7w, 8, 1, true),
    CT_SKC_VARIANT("f32skc7wx_w8_c2", Layer7w, 8, 2, true),
    CT_SKC_VARIANT("f32skc14qwx_w4_c1", Layer14qw, 4, 1, true),
    CT_SKC_VARIANT("f32skc14qw_w8_c2", Layer14qw, 8, 2, false),
    CT_SKC_VARIANT("f32skc14q1wx_w4_c4", Layer14q1w, 4, 4, true),
    CT_SKC_VARIANT("f32skc28s2wx_w4_c1", Layer28s2w, 4, 1, true),
    CT_SKC_VARIANT("f32skc28s2wx_w8_c1", Layer28s2w, 8, 1, true),
    CT_SKC_VARIANT("f32skc28s2w_w8_c2", Layer28s2w, 8, 2, false),
};

}  // namespace

const IgemmVariant* igemm_f32_skc_variants(int* count) {
    *count = (int)(sizeof(kSkcVariants) / sizeof(kSkcVariants[0]));
    return kSkcVariants;
}

}  // namespace ct
