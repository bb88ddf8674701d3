// fp32 implicit-GEMM convolution with a 16-channel output tile, for layers
// whose output pixels are too few to occupy 256 compute units (the final
// ResNet layer of the TVM tutorial "Tuning High Performance Convolution on
// NVIDIA GPUs": 7x7 outputs, CI*KH*KW = 4608), so the reduction is split
// across workgroups.
//
// Why a 16-row tile: the workgroup that finishes a tile's split reduction
// last reads S partial tiles, and with T tiles sharing 256 workgroups
// S * tile bytes = 256 * (CO*P*4) / T^2.  Sixteen output channels per tile
// double T against a 32-row tile and quarter that serial read; the
// 16x16x4 fp32 instruction issues at the same matrix rate as 32x32x2 on
// gfx950 (32 cycles for 1024 MACs), even as one dependent chain.
//
// Workgroup: NW waves, tile 16 output channels x 64 pixels = four 16x16
// blocks of v_mfma_f32_16x16x4_f32 per wave.  The waves split the stage's
// reduction range: wave w owns k in [w*KPW, (w+1)*KPW), KPW = 4*KSTEP, and at
// instruction step s the lane group g = lane/16 feeds
//     k = w*KPW + 16*(s/4) + 4*g + s%4
// (a last group of only 2 steps covers 8 values, g feeding 2g and 2g+1)
// (any assignment of k to (step, lane group) is valid when A and B share
// it), so a lane's A values for steps 4t..4t+3 are four consecutive floats
// of its filter row: one 16-byte load from global memory per four steps.
//
// Input windows, two compiled forms:
//  - staged ("f32sk16s", batch-1 layers whose one 64-column tile covers the
//    whole output and whose window reads every image row, like the 7x7 and
//    14x14-stride-2 layers): a stage's data is kc*H*W contiguous floats.  It
//    is loaded with coalesced 16-byte loads into registers, the filter loads
//    are issued, and only then is the data written into the zero-padded LDS
//    window (the padding was zeroed once at kernel start).  Everything is an
//    ordinary register load, so the compiler's in-order wait counting lets
//    the first matrix steps start while the rest of the filter arrives.
//  - direct ("f32sk16", any shape): each window word is a direct-to-LDS load
//    (padding lanes read a zeroed block), and the stage waits for all loads.
//
// Split reduction: the waves' accumulators are summed in LDS by all
// threads; each workgroup writes its partial tile with 16-byte
// device-coherent stores, takes a ticket, and the last to arrive sums the S
// partials in split order 0..S-1 (run-to-run identical) and applies the
// epilogue.  Workgroup b handles split b % S of tile b / S, so with eight
// splits the round-robin placement of workgroups on the 8 XCDs puts every
// tile of one split -- all readers of the same input channels -- on one XCD.
#include "ct_device.hpp"
#include "igemm_common.hpp"

#include <atomic>
#include <type_traits>

namespace ct {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kTileM = 16, kTileN = 64, kNB = 4;  // 4 column blocks of 16
constexpr int kRedStride = 68;                     // padded row of the reduction area
constexpr int kChMax = 4;                          // window words per lane kept as offsets: 4*64
constexpr int kBufWord3 = 0x00020000;              // raw buffer, 32-bit elements
constexpr int kCoherent = 16;                      // cache policy: device-coherent (sc1)
constexpr int kSkipL1 = 1;                         // cache policy: sc0, the load misses the CU's L1

__device__ __forceinline__ uint32_t fdiv16(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)__umulhi(n, f.mul) + n) >> f.shift);
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then the waves meet.  Unlike __syncthreads (whose acquire fence
// waits for every outstanding vector-memory load), loads into registers may
// still be in flight; the compiler waits for each where its value is used.
// The asm statement's memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // gfx9 encoding: lgkmcnt(0), vmcnt / expcnt not waited
    asm volatile("s_barrier" ::: "memory");
}


// LDS words: windows [kc][XCS] | k table [KS]; the cross-wave reduction
// [NW][16][68] aliases the windows.
struct Sk16Layout {
    int xcs, x_words, ktab_off, words;
};

__host__ __device__ inline Sk16Layout sk16_layout(int kc, int RWp, int KS, int NW) {
    Sk16Layout L;
    L.xcs = round_up(RWp, 64) <= 64 * kChMax ? round_up(RWp, 64) : RWp;
    L.x_words = round_up(kc * L.xcs, 64);
    const int red = NW * kTileM * kRedStride;
    L.ktab_off = L.x_words > red ? L.x_words : red;
    L.words = L.ktab_off + KS;
    return L;
}

// Divisors in ConvParams: fd_wstr = OH*OW, fd_wp = Wp, fd_rwp = XCS,
// fd_hp = Hp, fd_ow = OW, fd_t = KH*KW, fd_kw = KW, fd_w = W, fd_hw = H*W.
// XL: XCD-local split reduction -- every split of a tile has the same
// workgroup index mod 8, so on an MI355X (workgroup b on XCD b % 8) the
// partial stores, the ticket and the partial loads complete in that XCD's
// L2 rather than at device scope; legal only where the runtime has observed
// that placement.
template <int NW, int KSTEP, bool STAGED, bool XL>
__global__ __launch_bounds__(NW * 64) void igemm_f32_sk16_kernel(ConvParams p) {
    fetch_kernargs(p);
    constexpr int XE = 16;  // staged window words per thread
    static_assert(KSTEP % 2 == 0, "steps per wave come in pairs");
    constexpr int KT = (KSTEP + 3) / 4;       // 4-step groups; the last may hold 2 steps
    constexpr int LE = KSTEP - 4 * (KT - 1);  // steps of the last group: 2 or 4
    constexpr int KPW = 4 * KSTEP;            // reduction values per wave
    constexpr int KS = NW * KPW;
    constexpr int NT = NW * 64;
    extern __shared__ __align__(16) float lds[];  // 16-byte LDS accesses need a 16-byte aligned base
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;  // A row, B / C column inside a 16x16 block
    const int lg = lane >> 4;  // lane group: which k of the instruction's four
    const int RWp = p.R * p.Wp;

    const Sk16Layout L = sk16_layout(p.kc, RWp, KS, NW);
    const int xcs = L.xcs;
    float* Xs = lds;
    int* ktab = reinterpret_cast<int*>(lds + L.ktab_off);

    int tile, split;
    if constexpr (XL) {
        const int idx = blockIdx.x >> 3;
        const int q = idx / p.S;
        tile = (blockIdx.x & 7) + 8 * q;
        split = idx - q * p.S;
        if (tile >= p.tiles_m * p.tiles_n) return;  // the last XCD rounds may be short
    } else {
        tile = blockIdx.x / p.S;
        split = blockIdx.x - tile * p.S;
    }
    const int tm = tile % p.tiles_m;
    const int tn = tile / p.tiles_m;
    const int co0 = tm * kTileM;
    const int p0 = tn * kTileN;  // P < 2^31 for this kernel (checked on the host)
    const int n_first = (int)fdiv16((uint32_t)p0, p.fd_wstr);
    const int oy_first = (int)fdiv16((uint32_t)(p0 - n_first * p.OHW), p.fd_ow);
    const int vr_first = n_first * p.Hp + oy_first * p.stride;
    const long long HW = (long long)p.H * p.W;

    const float* __restrict__ xg = static_cast<const float*>(p.x);
    const float* __restrict__ wg = static_cast<const float*>(p.w);
    const float* zero = static_cast<const float*>(p.zero);

    // ---- output-side constants: this thread's 4 outputs after the reduction
    //      are row `orow`, columns ocol .. ocol+3 of the tile
    const bool out_thread = tid < 256;
    const int orow = (tid & 255) >> 4;
    const int ocol = 4 * (tid & 15);
    const int oco = co0 + orow;
    float e_b = 0.0f, e_v = 1.0f;
    if (out_thread && oco < p.CO && p.epilogue != EPI_NONE) {
        // requested first: these loads retire before everything below
        e_b = p.bias[oco];
        if (p.epilogue == EPI_EXP_BIAS_RSQRT) e_v = p.var[oco];
    }

    const int co_a = co0 + li;
    const int kw0 = wave * KPW + 4 * lg;  // k of step 0; step s adds 16*(s/4) + s%4
    // a last group of 2 steps covers 8 values: lane group g takes 2g, 2g+1
    const int kw_last = LE == 4 ? kw0 + 16 * (KT - 1) : wave * KPW + 16 * (KT - 1) + 2 * lg;
    const bool w_vec = ((p.K & 3) == 0) && ((reinterpret_cast<uintptr_t>(wg) & 15) == 0);
    const bool lane_offsets = xcs <= 64 * kChMax;

    // ---- staged windows: the tile's image rows 0..H-1 of image 0 -----------
    // (the host allows this form only for one tile per image whose window
    // reads every image row, so a stage's data is kc*H*W contiguous floats)
    const int wr0 = oy_first * p.stride;  // padded image row of window row 0
    float xr[XE];
    floatx4 a4[KT];
    const bool row_ok = co_a < p.CO;
    // Register loads of stage st: the window data (staged form: this thread's
    // XE words, 16-byte groups in flat order) and then A, steps 4t..4t+3 =
    // W[co_a][c0*T + kw0 + 16t + (0..3)] (a last group of 2 steps =
    // W[co_a][c0*T + kw_last + (0, 1)]).  Issued before anything that waits,
    // so the memory latency overlaps the set-up below.
    auto issue_loads = [&](int st) {
        const int c0 = (split * p.stages + st) * p.kc;
        const int cvalid = min(p.kc, p.CI - c0);
        const int kvalid = cvalid * p.T;
        if constexpr (STAGED) {
            // the launcher runs this form only with 16-byte aligned x and w and
            // kc*H*W, CI*H*W, KH*KW*kc multiples of 4: every load below is a
            // whole 16-byte group, issued unconditionally (past the end: the
            // zero block)
            const int E = cvalid * (int)HW;
            const float* xblk = xg + (long long)c0 * HW;
#pragma unroll
            for (int j = 0; j < XE / 4; ++j) {
                const int f = 4 * (j * NT + tid);
                const float* src = f < E ? xblk + f : zero;
                const floatx4 v = *reinterpret_cast<const floatx4*>(src);
                xr[4 * j] = v[0];
                xr[4 * j + 1] = v[1];
                xr[4 * j + 2] = v[2];
                xr[4 * j + 3] = v[3];
            }
            // window loads first in issue order: they retire first
            __builtin_amdgcn_sched_barrier(0);
        }
        const float* wrow = wg + (long long)co_a * p.K + (long long)c0 * p.T + kw0;
        // whole 16-byte groups only: every group is then all valid or all past
        // kvalid, and a group past it (or past CO) reads the zero block
        const bool vec_stage = STAGED || (w_vec && (((c0 * p.T) & 3) == 0) && ((kvalid & 3) == 0));
        const float* wlast = wrow - kw0 + kw_last;
        if (vec_stage) {
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                if (t < KT - 1 || LE == 4) {
                    const int k = kw0 + 16 * t;
                    const float* src = (row_ok && k < kvalid) ? wrow + 16 * t : zero;
                    a4[t] = *reinterpret_cast<const floatx4*>(src);
                } else {
                    const float* src = (row_ok && kw_last < kvalid) ? wlast : zero;
                    const float2 v = *reinterpret_cast<const float2*>(src);
                    a4[t] = floatx4{v.x, v.y, 0.0f, 0.0f};
                }
            }
        } else if constexpr (!STAGED) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool last2 = t == KT - 1 && LE == 2;
                    const int k = last2 ? kw_last + e : kw0 + 16 * t + e;
                    a4[t][e] = (row_ok && k < kvalid && (!last2 || e < 2))
                                   ? (last2 ? wlast[e] : wrow[16 * t + e])
                                   : 0.0f;
                }
        }
    };
    // k -> window offset of every k lane of a stage
    auto build_ktab = [&]() {
        for (int k = tid; k < KS; k += NT) {
            const int c = (int)fdiv16((uint32_t)k, p.fd_t);
            const int t = k - c * p.T;
            const int ky = (int)fdiv16((uint32_t)t, p.fd_kw);
            const int kx = t - ky * p.KW;
            ktab[k] = (c < p.kc) ? c * xcs + ky * p.Wp + kx : 0;
        }
    };
    // the first stage's register loads go out before any other set-up
    if constexpr (STAGED) issue_loads(0);


    floatx4 acc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[nb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // window offset of each B column's (0,0) tap; columns past P read 0
    int pbase[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        const int pc = p0 + nb * 16 + li;
        pbase[nb] = 0;
        if (pc < p.P) {
            const int n = (int)fdiv16((uint32_t)pc, p.fd_wstr);
            const int rem = pc - n * p.OHW;
            const int oy = (int)fdiv16((uint32_t)rem, p.fd_ow);
            const int ox = rem - oy * p.OW;
            pbase[nb] = (n * p.Hp + oy * p.stride - vr_first) * p.Wp + ox * p.stride;
        }
    }
    // source offset (within one channel, image included) of window word
    // h*64 + lane; -1 = padding or past the window
    long long xoff[kChMax];
#pragma unroll
    for (int h = 0; h < kChMax; ++h) {
        xoff[h] = -1;
        const int pos = h * 64 + lane;
        if (!STAGED && lane_offsets && pos < RWp) {
            const int r = (int)fdiv16((uint32_t)pos, p.fd_wp);
            const int col = pos - r * p.Wp;
            const int vr = vr_first + r;
            const int n = (int)fdiv16((uint32_t)vr, p.fd_hp);
            const int iy = vr - n * p.Hp - p.pad;
            const int ix = col - p.pad;
            if (n < p.N && iy >= 0 && iy < p.H && ix >= 0 && ix < p.W)
                xoff[h] = (long long)n * p.CI * HW + (long long)iy * p.W + ix;
        }
    }

    if constexpr (STAGED) {
        // padding words are the same in every stage: zero the windows once,
        // and build the k table, while the first stage's loads are in flight
        floatx4* xz = reinterpret_cast<floatx4*>(Xs);
        for (int i = tid; i < L.x_words / 4; i += NT) xz[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        build_ktab();
        lds_barrier();
    }
    for (int st = 0; st < p.stages; ++st) {
        const int c0 = (split * p.stages + st) * p.kc;
        if (c0 >= p.CI) break;
        const int cvalid = min(p.kc, p.CI - c0);
        const int kvalid = cvalid * p.T;

        if (st > 0) {
            // the previous stage's registers are free: load this stage's, then
            // wait until every wave is done reading the previous windows
            if constexpr (STAGED) issue_loads(st);
            lds_barrier();
        }
        if constexpr (!STAGED) issue_loads(st);

        if constexpr (STAGED) {
            // (3) window data into LDS from the registers loaded above (the
            // host allows this form only when a stage's data fits NT*XE words)
            const int E = cvalid * (int)HW;
#pragma unroll
            for (int j = 0; j < XE / 4; ++j) {
                const int f = 4 * (j * NT + tid);
                if (f < E) {
                    // four consecutive words: step the column, wrapping rows
                    // and channels
                    const int c = (int)fdiv16((uint32_t)f, p.fd_hw);
                    const int off = f - c * (int)HW;
                    int iy = (int)fdiv16((uint32_t)off, p.fd_w);
                    int ix = off - iy * p.W;
                    int cb = c * xcs;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        Xs[cb + (iy + p.pad - wr0) * p.Wp + ix + p.pad] = xr[4 * j + i];
                        if (++ix == p.W) {
                            ix = 0;
                            if (++iy == p.H) {
                                iy = 0;
                                cb += xcs;
                            }
                        }
                    }
                }
            }
        } else {
            // (3) zero-padded windows of channels c0 .. c0+cvalid, straight to LDS
            if (lane_offsets) {
                const int per_c = xcs / 64;
                for (int ch = wave; ch < cvalid * per_c; ch += NW) {
                    const int c = ch / per_c;
                    const int h = ch - c * per_c;
                    long long off = -1;
#pragma unroll
                    for (int hh = 0; hh < kChMax; ++hh)
                        if (hh == h) off = xoff[hh];
                    const float* src = off >= 0 ? xg + off + (long long)(c0 + c) * HW : zero;
                    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(Xs + ch * 64), 4, 0, 0);
                }
            } else {
                for (int ch = wave; ch < L.x_words / 64; ch += NW) {
                    const uint32_t i = (uint32_t)(ch * 64 + lane);
                    const uint32_t c = fdiv16(i, p.fd_rwp);
                    const uint32_t rem = i - c * (uint32_t)xcs;
                    const uint32_t r = fdiv16(rem, p.fd_wp);
                    const int col = (int)(rem - r * (uint32_t)p.Wp);
                    const float* src = zero;
                    if ((int)c < cvalid) {
                        const int vr = vr_first + (int)r;
                        const int n = (int)fdiv16((uint32_t)vr, p.fd_hp);
                        const int iy = vr - n * p.Hp - p.pad;
                        const int ix = col - p.pad;
                        if (n < p.N && iy >= 0 && iy < p.H && ix >= 0 && ix < p.W)
                            src = xg + ((long long)n * p.CI + c0 + (int)c) * HW + (long long)iy * p.W + ix;
                    }
                    __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(Xs + ch * 64), 4, 0, 0);
                }
            }
            // (4) k -> window offset, once, while the loads are in flight
            if (st == 0) build_ktab();
        }
        // the windows and the k table are complete and visible to every wave;
        // direct-to-LDS loads are waited for here, register loads by the
        // compiler where their values are used
        if constexpr (STAGED) {
            lds_barrier();
        } else {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }

        // (5) matrix-core steps; B of group t+1 is read while group t runs.
        // The wave's k -> window offsets live in registers, so a group's
        // reads depend on nothing but the window; in a full stage no k is
        // past the data and the reads feed the instructions unmasked.
        int4 kt[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            if (t < KT - 1 || LE == 4) {
                kt[t] = *reinterpret_cast<const int4*>(ktab + kw0 + 16 * t);
            } else {
                const int2 v = *reinterpret_cast<const int2*>(ktab + kw_last);
                kt[t] = int4{v.x, v.y, 0, 0};
            }
        }
        auto steps = [&](auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            float bcur[4][kNB], bnext[4][kNB];
            auto fetch = [&](int t, float (&b)[4][kNB]) {
                const int ne = (t == KT - 1) ? LE : 4;
                const int kb = (t == KT - 1) ? kw_last : kw0 + 16 * t;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (e >= ne) break;
                    const int koff = e == 0 ? kt[t].x : e == 1 ? kt[t].y : e == 2 ? kt[t].z : kt[t].w;
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb) {
                        const float v = Xs[pbase[nb] + koff];
                        b[e][nb] = (!MASKED || kb + e < kvalid) ? v : 0.0f;
                    }
                }
            };
            fetch(0, bcur);
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                if (t + 1 < KT) fetch(t + 1, bnext);
                // keep the next group's reads ahead of this group's instructions
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (e >= ((t == KT - 1) ? LE : 4)) break;
#pragma unroll
                    for (int nb = 0; nb < kNB; ++nb)
                        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[t][e], bcur[e][nb], acc[nb], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (t + 1 < KT) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int nb = 0; nb < kNB; ++nb) bcur[e][nb] = bnext[e][nb];
                }
            }
        };
        if (kvalid >= KS)
            steps(std::false_type{});
        else
            steps(std::true_type{});
    }

    // ---- sum the waves' accumulators in LDS (all threads take part) -------
    // C layout of v_mfma_f32_16x16x4_f32: row 4*(lane/16) + r, column lane%16.
    __syncthreads();  // every wave is done reading the windows
    float* red = lds;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            red[(wave * kTileM + 4 * lg + r) * kRedStride + nb * 16 + li] = acc[nb][r];
    __syncthreads();
    floatx4 sum = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (out_thread) {
#pragma unroll
        for (int w = 0; w < NW; ++w)
            sum += *reinterpret_cast<const floatx4*>(red + (w * kTileM + orow) * kRedStride + ocol);
    }
    const bool ocol_any = p0 + ocol < p.P;
    const float e_r = p.epilogue == EPI_EXP_BIAS_RSQRT ? dev_rsqrt(e_v + p.eps) : 1.0f;

    auto store_out = [&](const floatx4& v) {
        if (!(out_thread && ocol_any && oco < p.CO)) return;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pc = p0 + ocol + j;
            if (pc >= p.P) break;
            const int n = (int)fdiv16((uint32_t)pc, p.fd_wstr);
            const int rem = pc - n * p.OHW;
            p.y[((long long)n * p.CO + oco) * p.OHW + rem] = apply_epilogue(p.epilogue, v[j], e_b, e_r);
        }
    };

    if (p.S == 1) {
        store_out(sum);
        return;
    }

    // ---- split reduction across workgroups --------------------------------
    // Partial tile: [row 16][col 64] floats; tile t's S partials are slabs
    // t*S .. t*S+S-1 of the workspace.
    constexpr int TILE_F = kTileM * kTileN;
    float* part = p.ws + (long long)tile * p.S * TILE_F;
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(part, 0, p.S * TILE_F * 4, kBufWord3);
    const int fo = orow * kTileN + ocol;  // this thread's float offset in a slab
    if (out_thread && ocol_any) {
        uint4v v;
        v.x = __float_as_uint(sum[0]);
        v.y = __float_as_uint(sum[1]);
        v.z = __float_as_uint(sum[2]);
        v.w = __float_as_uint(sum[3]);
        __builtin_amdgcn_raw_buffer_store_b128(v, prs, (split * TILE_F + fo) * 4, 0, XL ? 0 : kCoherent);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial store is complete
    __syncthreads();
    if (tid == 0) {
        const unsigned old = XL ? __hip_atomic_fetch_add(&p.tickets[tile * kTicketStride], 1u,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                                : __hip_atomic_fetch_add(&p.tickets[tile * kTicketStride], 1u,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (unsigned)(p.S - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;

    // last arriver: each thread sums its 4 outputs over the S slabs, in
    // split order, with up to 16 loads in flight
    if (out_thread && ocol_any) {
        constexpr int SB = 16;
        floatx4 tot = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = 0; s0 < p.S; s0 += SB) {
            floatx4 v[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j)
                v[j] = (s0 + j < p.S) ? __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                       prs, ((s0 + j) * TILE_F + fo) * 4, 0,
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

template <int NW, int KSTEP, bool STAGED>
int sk16_lds_bytes(const ConvParams& p) {
    constexpr int KS = NW * 4 * KSTEP;
    if (p.kc * p.T > KS) return 1 << 30;  // the stage must fit the k lanes
    if (STAGED) {
        // one tile, one image, and its window reads every image row
        if (p.N != 1 || p.P > kTileN) return 1 << 30;
        if ((long long)(p.OH - 1) * p.stride + p.KH - 1 - p.pad < p.H - 1) return 1 << 30;
        // one round of staged registers: kc*H*W <= threads * 16
        if ((long long)p.kc * p.H * p.W > (long long)NW * 64 * 16) return 1 << 30;
    }
    if (p.P >= (1LL << 31) || (long long)p.N * p.Hp >= (1LL << 31)) return 1 << 30;
    if ((long long)p.kc * p.R * p.Wp >= (1LL << 24)) return 1 << 30;
    // partial slabs are addressed with 32-bit byte offsets per tile
    if ((long long)p.S * kTileM * kTileN * 4 >= (1LL << 31)) return 1 << 30;
    return 4 * sk16_layout(p.kc, p.R * p.Wp, KS, NW).words;
}

template <int NW, int KSTEP, bool STAGED, bool XL>
hipError_t sk16_launch(const ConvParams& p, hipStream_t stream) {
    if (STAGED) {
        const long long HW = (long long)p.H * p.W;
        const bool aligned = (reinterpret_cast<uintptr_t>(p.x) & 15) == 0 &&
                             (reinterpret_cast<uintptr_t>(p.w) & 15) == 0 && (p.K & 3) == 0 &&
                             ((p.kc * HW) & 3) == 0 && ((p.CI * HW) & 3) == 0 &&
                             ((p.kc * p.T) & 3) == 0;
        // same tile config, same result: the direct-window form takes any layout
        if (!aligned) return sk16_launch<NW, KSTEP, false, XL>(p, stream);
    }
    const int bytes = sk16_lds_bytes<NW, KSTEP, STAGED>(p);
    if (bytes > 163840 - 64) return hipErrorInvalidValue;
    auto kern = igemm_f32_sk16_kernel<NW, KSTEP, STAGED, XL>;
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
    const Sk16Layout L = sk16_layout(p.kc, p.R * p.Wp, NW * 4 * KSTEP, NW);
    ConvParams q = p;
    q.fd_wstr = make_fastdiv((uint32_t)p.OHW);
    q.fd_wp = make_fastdiv((uint32_t)p.Wp);
    q.fd_rwp = make_fastdiv((uint32_t)L.xcs);
    q.fd_hp = make_fastdiv((uint32_t)p.Hp);
    q.fd_ow = make_fastdiv((uint32_t)p.OW);
    q.fd_t = make_fastdiv((uint32_t)p.T);
    q.fd_kw = make_fastdiv((uint32_t)p.KW);
    q.fd_w = make_fastdiv((uint32_t)p.W);
    q.fd_hw = make_fastdiv((uint32_t)(p.H * p.W));
    const long long tiles = (long long)p.tiles_m * p.tiles_n;
    const long long grid = XL ? 8 * ((tiles + 7) / 8) * p.S : tiles * p.S;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), bytes, stream, q);
    return hipGetLastError();
}

// descriptor: 16x16x4 instruction, waves 1 x 1 x NW (CO x P x K), reps 1 x 4;
// NW waves of KSTEP steps hold a stage of up to NW*4*KSTEP reduction values
#define CT_SK16_VARIANT(NAME, NW, KSTEP, STAGED, XL)                                             \
    {NAME, DT_F32, 16, 16, 4, 1, 1, NW, 1, 4, NW * 4 * KSTEP, &sk16_lds_bytes<NW, KSTEP, STAGED>, \
     &sk16_launch<NW, KSTEP, STAGED, XL>, nullptr, XL}

const IgemmVariant kSk16Variants[] = {
    CT_SK16_VARIANT("f32sk16_m16n64_w4_kt9", 4, 36, false, false),
    CT_SK16_VARIANT("f32sk16_m16n64_w4_kt5", 4, 20, false, false),
    CT_SK16_VARIANT("f32sk16_m16n64_w4_kt3", 4, 12, false, false),
    CT_SK16_VARIANT("f32sk16s_m16n64_w4_kt9", 4, 36, true, false),
    CT_SK16_VARIANT("f32sk16s_m16n64_w4_kt5", 4, 20, true, false),
    CT_SK16_VARIANT("f32sk16s_m16n64_w4_kt3", 4, 12, true, false),
    CT_SK16_VARIANT("f32sk16_m16n64_w8_s18", 8, 18, false, false),
    CT_SK16_VARIANT("f32sk16s_m16n64_w8_s18", 8, 18, true, false),
    CT_SK16_VARIANT("f32sk16s_m16n64_w8_s10", 8, 10, true, false),
    CT_SK16_VARIANT("f32sk16x_m16n64_w4_kt9", 4, 36, false, true),
    CT_SK16_VARIANT("f32sk16x_m16n64_w4_kt5", 4, 20, false, true),
    CT_SK16_VARIANT("f32sk16x_m16n64_w4_kt3", 4, 12, false, true),
    CT_SK16_VARIANT("f32sk16x_m16n64_w8_s18", 8, 18, false, true),
    CT_SK16_VARIANT("f32sk16sx_m16n64_w8_s10", 8, 10, true, true),
};

}  // namespace

const IgemmVariant* igemm_f32_sk16_variants(int* count) {
    *count = (int)(sizeof(kSk16Variants) / sizeof(kSk16Variants[0]));
    return kSk16Variants;
}

}  // namespace ct
