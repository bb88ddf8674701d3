// fp32 implicit-GEMM convolution for layers with few output pixels and a
// long reduction (the final ResNet layer of the TVM tutorial "Tuning High
// Performance Convolution on NVIDIA GPUs": 7x7 outputs, CI*KH*KW = 4608),
// where the output tiles alone cannot fill 256 compute units and the
// reduction is split across workgroups.
//
// Workgroup: 4 waves, output tile 32 channels x 64 pixels (two 32x32 blocks
// of v_mfma_f32_32x32x2_f32, the fp32 instruction that runs at the matrix
// peak on gfx950).  A stage holds KS = 8*KL reduction values; wave w owns
// [w*2KL, (w+1)*2KL) and, inside it, the k value that lane half q feeds at
// instruction step s is
//     w*2KL + 8*(s/4) + 4*q + s%4
// (any assignment of k to (step, lane half) is valid when A and B share it).
// With this one a lane's A values for steps 4t..4t+3 are four consecutive
// floats of its W row: one 16-byte load per four steps, straight from
// global memory into registers.
//
// B operand: the stage's input channels are staged in LDS as zero-padded
// windows (the rows of the padded input the tile's 64 pixels read), filled
// by direct-to-LDS loads whose out-of-image lanes read a zeroed block, so a
// B value is one LDS read at (pixel base + per-k offset) with no masking.
// When a channel's window fits 256 words each lane computes the source
// offsets of its window words once and reuses them for every channel.
//
// Split reduction: the four waves' accumulators are summed in LDS; each
// workgroup writes its partial tile with 16-byte device-coherent stores
// (columns past P skipped), takes a ticket, and the last to arrive sums the
// S partials in split order 0..S-1 with 16-byte device-coherent loads, all
// of a thread's loads in flight together, then applies the epilogue.
#include "ct_device.hpp"
#include "igemm_common.hpp"

#include <atomic>

namespace ct {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kSkWaves = 4;
constexpr int kSkThreads = kSkWaves * 64;
constexpr int kSkTileM = 32, kSkTileN = 64, kSkRN = 2;

__device__ __forceinline__ uint32_t fdiv_sk(uint32_t n, FastDiv f) {
    return (uint32_t)(((uint64_t)__umulhi(n, f.mul) + n) >> f.shift);
}

// LDS words: windows [kc][XCS] | k table [KS] | epilogue [2][32]; the
// cross-wave reduction [3][RN*16][64] aliases the windows.  XCS is R*Wp
// rounded up to 64 when that is at most kSkChMax*64 words (per-lane offsets),
// else R*Wp.
constexpr int kSkChMax = 4;

struct SkLayout {
    int xcs;
    int x_words;
    int ktab_off;
    int epi_off;
    int words;
};

__host__ __device__ inline SkLayout sk_layout(int kc, int RWp, int KS) {
    SkLayout L;
    L.xcs = round_up(RWp, 64) <= 64 * kSkChMax ? round_up(RWp, 64) : RWp;
    L.x_words = round_up(kc * L.xcs, 64);
    const int red = (kSkWaves - 1) * kSkRN * 16 * 64;
    const int region = L.x_words > red ? L.x_words : red;
    L.ktab_off = region;
    L.epi_off = L.ktab_off + KS;
    L.words = L.epi_off + 2 * kSkTileM;
    return L;
}

typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit elements
constexpr int kCoherent = 16;          // cache policy: device-coherent (sc1)
constexpr int kSkipL1 = 1;             // cache policy: sc0, the load misses the CU's L1

// Divisors the kernel needs arrive in ConvParams' FastDiv slots:
//   fd_wstr = OH*OW, fd_wp = Wp, fd_rwp = XCS, fd_hp = Hp, fd_ow = OW,
//   fd_t = KH*KW, fd_kw = KW.
// XL: XCD-local split reduction -- every split of a tile has the same
// workgroup index mod 8, so on an MI355X (workgroup b on XCD b % 8) the
// partial stores, the ticket and the partial loads complete in that XCD's
// L2 rather than at device scope; legal only where the runtime has observed
// that placement.
template <int KL, bool XL>
__global__ __launch_bounds__(kSkThreads) void igemm_f32_sk_kernel(ConvParams p) {
    fetch_kernargs(p);
    constexpr int KS = 8 * KL;
    constexpr int KT = KL / 4;
    static_assert(KL % 4 == 0, "KL must be a multiple of 4");
    extern __shared__ __align__(16) float lds[];  // 16-byte LDS accesses need a 16-byte aligned base
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lj = lane & 31;  // A row, B / C column inside a 32x32 block
    const int lq = lane >> 5;  // lane half: which k of the instruction's pair
    const int RWp = p.R * p.Wp;

    const SkLayout L = sk_layout(p.kc, RWp, KS);
    const int xcs = L.xcs;
    float* Xs = lds;
    int* ktab = reinterpret_cast<int*>(lds + L.ktab_off);
    float* e_bias = lds + L.epi_off;
    float* e_rs = e_bias + kSkTileM;

    const int tiles = p.tiles_m * p.tiles_n;
    int tile, split;
    if constexpr (XL) {
        const int idx = blockIdx.x >> 3;
        const int q = idx / p.S;
        tile = (blockIdx.x & 7) + 8 * q;
        split = idx - q * p.S;
        if (tile >= tiles) return;  // the last XCD rounds may be short
    } else {
        tile = blockIdx.x % tiles;
        split = blockIdx.x / tiles;
    }
    const int tm = tile % p.tiles_m;
    const int tn = tile / p.tiles_m;
    const int co0 = tm * kSkTileM;
    const int p0 = tn * kSkTileN;  // P < 2^31 for this kernel
    const int n_first = (int)fdiv_sk((uint32_t)p0, p.fd_wstr);
    const int oy_first = (int)fdiv_sk((uint32_t)(p0 - n_first * p.OHW), p.fd_ow);
    const int vr_first = n_first * p.Hp + oy_first * p.stride;  // < 2^31 (checked on the host)
    const long long HW = (long long)p.H * p.W;

    const float* __restrict__ xg = static_cast<const float*>(p.x);
    const float* __restrict__ wg = static_cast<const float*>(p.w);
    const float* zero = static_cast<const float*>(p.zero);

    const int co_a = co0 + lj;
    const int kw0 = wave * 2 * KL + 4 * lq;  // k of step 0; step s adds 8*(s/4) + s%4
    const bool w_vec = ((p.K & 3) == 0) && ((reinterpret_cast<uintptr_t>(wg) & 15) == 0);
    const bool lane_offsets = xcs <= 64 * kSkChMax;

    floatx16 acc[kSkRN];
    for (int rn = 0; rn < kSkRN; ++rn)
        for (int r = 0; r < 16; ++r) acc[rn][r] = 0.0f;

    // window offset of each B column's (0,0) tap; columns past P read 0
    int pbase[kSkRN];
    for (int rn = 0; rn < kSkRN; ++rn) {
        const int pc = p0 + rn * 32 + lj;
        pbase[rn] = 0;
        if (pc < p.P) {
            const int n = (int)fdiv_sk((uint32_t)pc, p.fd_wstr);
            const int rem = pc - n * p.OHW;
            const int oy = (int)fdiv_sk((uint32_t)rem, p.fd_ow);
            const int ox = rem - oy * p.OW;
            pbase[rn] = (n * p.Hp + oy * p.stride - vr_first) * p.Wp + ox * p.stride;
        }
    }
    // source offset (within one channel, image included) of window word
    // h*64 + lane; -1 = padding or past the window
    long long xoff[kSkChMax];
    for (int h = 0; h < kSkChMax; ++h) {
        xoff[h] = -1;
        const int pos = h * 64 + lane;
        if (lane_offsets && pos < RWp) {
            const int r = (int)fdiv_sk((uint32_t)pos, p.fd_wp);
            const int col = pos - r * p.Wp;
            const int vr = vr_first + r;
            const int n = (int)fdiv_sk((uint32_t)vr, p.fd_hp);
            const int iy = vr - n * p.Hp - p.pad;
            const int ix = col - p.pad;
            if (n < p.N && iy >= 0 && iy < p.H && ix >= 0 && ix < p.W)
                xoff[h] = (long long)n * p.CI * HW + (long long)iy * p.W + ix;
        }
    }
    bool ktab_done = false;

    for (int st = 0; st < p.stages; ++st) {
        const int c0 = (split * p.stages + st) * p.kc;
        if (c0 >= p.CI) break;
        const int cvalid = min(p.kc, p.CI - c0);
        const int kvalid = cvalid * p.T;

        // (1) A: steps 4t..4t+3 = W[co_a][c0*T + kw0 + 8t + (0..3)]
        floatx4 a4[KT];
        const float* wrow = wg + (long long)co_a * p.K + (long long)c0 * p.T + kw0;
        const bool row_ok = co_a < p.CO;
        const bool vec_stage = w_vec && (((c0 * p.T) & 3) == 0);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int k = kw0 + 8 * t;
            if (row_ok && vec_stage && k + 3 < kvalid) {
                a4[t] = *reinterpret_cast<const floatx4*>(wrow + 8 * t);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) a4[t][e] = (row_ok && k + e < kvalid) ? wrow[8 * t + e] : 0.0f;
            }
        }

        // (2) zero-padded windows of channels c0 .. c0+cvalid
        if (st > 0) __syncthreads();  // previous stage's windows consumed
        if (lane_offsets) {
            const int per_c = xcs / 64;
            for (int ch = wave; ch < cvalid * per_c; ch += kSkWaves) {
                const int c = ch / per_c;
                const int h = ch - c * per_c;
                long long off = -1;
#pragma unroll
                for (int hh = 0; hh < kSkChMax; ++hh)
                    if (hh == h) off = xoff[hh];
                const float* src = off >= 0 ? xg + off + (long long)(c0 + c) * HW : zero;
                __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(Xs + ch * 64), 4, 0, 0);
            }
        } else {
            for (int ch = wave; ch < L.x_words / 64; ch += kSkWaves) {
                const uint32_t i = (uint32_t)(ch * 64 + lane);
                const uint32_t c = fdiv_sk(i, p.fd_rwp);
                const uint32_t rem = i - c * (uint32_t)xcs;
                const uint32_t r = fdiv_sk(rem, p.fd_wp);
                const int col = (int)(rem - r * (uint32_t)p.Wp);
                const float* src = zero;
                if ((int)c < cvalid) {
                    const int vr = vr_first + (int)r;
                    const int n = (int)fdiv_sk((uint32_t)vr, p.fd_hp);
                    const int iy = vr - n * p.Hp - p.pad;
                    const int ix = col - p.pad;
                    if (n < p.N && iy >= 0 && iy < p.H && ix >= 0 && ix < p.W)
                        src = xg + ((long long)n * p.CI + c0 + (int)c) * HW + (long long)iy * p.W + ix;
                }
                __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)(Xs + ch * 64), 4, 0, 0);
            }
        }

        // (3) k -> window offset, once, while the loads are in flight
        if (!ktab_done) {
            ktab_done = true;
            for (int k = tid; k < KS; k += kSkThreads) {
                const int c = (int)fdiv_sk((uint32_t)k, p.fd_t);
                const int t = k - c * p.T;
                const int ky = (int)fdiv_sk((uint32_t)t, p.fd_kw);
                const int kx = t - ky * p.KW;
                ktab[k] = (c < p.kc) ? c * xcs + ky * p.Wp + kx : 0;
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        // (4) matrix-core steps: B for group t+1 is read from LDS while the
        // instructions of group t run
        int4 kt[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) kt[t] = *reinterpret_cast<const int4*>(ktab + kw0 + 8 * t);
        const bool full = kvalid >= KS;
        float bcur[4][kSkRN], bnext[4][kSkRN];
        auto fetch = [&](int t, float (&b)[4][kSkRN]) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int koff = e == 0 ? kt[t].x : e == 1 ? kt[t].y : e == 2 ? kt[t].z : kt[t].w;
                const bool kok = full || (kw0 + 8 * t + e < kvalid);
#pragma unroll
                for (int rn = 0; rn < kSkRN; ++rn) {
                    const float v = Xs[pbase[rn] + koff];
                    b[e][rn] = kok ? v : 0.0f;
                }
            }
        };
        fetch(0, bcur);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            if (t + 1 < KT) fetch(t + 1, bnext);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int rn = 0; rn < kSkRN; ++rn)
                    acc[rn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[t][e], bcur[e][rn], acc[rn], 0, 0, 0);
            if (t + 1 < KT) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int rn = 0; rn < kSkRN; ++rn) bcur[e][rn] = bnext[e][rn];
            }
        }
    }

    // ---- per-channel epilogue values (read after the loads above landed) ----
    __syncthreads();
    for (int m = tid; m < kSkTileM; m += kSkThreads) {
        const int co = co0 + m;
        float b = 0.0f, r = 1.0f;
        if (co < p.CO) {
            if (p.epilogue != EPI_NONE) b = p.bias[co];
            if (p.epilogue == EPI_EXP_BIAS_RSQRT) r = dev_rsqrt(p.var[co] + p.eps);
        }
        e_bias[m] = b;
        e_rs[m] = r;
    }

    // ---- sum the four waves' accumulators in LDS ------------------------------
    float* red = lds;
    if (wave > 0)
        for (int rn = 0; rn < kSkRN; ++rn)
            for (int r = 0; r < 16; ++r) red[(((wave - 1) * kSkRN + rn) * 16 + r) * 64 + lane] = acc[rn][r];
    __syncthreads();
    if (wave == 0)
        for (int w2 = 1; w2 < kSkWaves; ++w2)
            for (int rn = 0; rn < kSkRN; ++rn)
                for (int r = 0; r < 16; ++r) acc[rn][r] += red[(((w2 - 1) * kSkRN + rn) * 16 + r) * 64 + lane];

    // C layout of v_mfma_f32_32x32x2_f32: row 8*(r/4) + 4*(lane/32) + r%4,
    // column lane%32.
    if (p.S == 1) {
        if (wave != 0) return;
        for (int rn = 0; rn < kSkRN; ++rn) {
            const int pc = p0 + rn * 32 + lj;
            if (pc >= p.P) continue;
            const int n = (int)fdiv_sk((uint32_t)pc, p.fd_wstr);
            const int rem = pc - n * p.OHW;
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r >> 2) + 4 * lq + (r & 3);
                const int co = co0 + row;
                if (co < p.CO)
                    p.y[((long long)n * p.CO + co) * p.OHW + rem] =
                        apply_epilogue(p.epilogue, acc[rn][r], e_bias[row], e_rs[row]);
            }
        }
        return;
    }

    // ---- split reduction across workgroups ------------------------------------
    // Partial layout: float4 f = (rn*4 + r4)*64 + lane holds accumulator
    // registers 4*r4 .. 4*r4+3 of that lane (rows 8*r4 + 4*(lane/32) + 0..3,
    // column rn*32 + lane%32).
    constexpr int TILE_F4 = kSkTileM * kSkTileN / 4;
    float* part = p.ws + (long long)tile * p.S * (TILE_F4 * 4);
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        part, 0, p.S * TILE_F4 * 16, kBufWord3);
    if (wave == 0) {
        for (int rn = 0; rn < kSkRN; ++rn) {
            if (p0 + rn * 32 + lj >= p.P) continue;  // nobody reads padding columns
            for (int r4 = 0; r4 < 4; ++r4) {
                uint4v v;
                v.x = __float_as_uint(acc[rn][4 * r4 + 0]);
                v.y = __float_as_uint(acc[rn][4 * r4 + 1]);
                v.z = __float_as_uint(acc[rn][4 * r4 + 2]);
                v.w = __float_as_uint(acc[rn][4 * r4 + 3]);
                const int f = split * TILE_F4 + (rn * 4 + r4) * 64 + lane;
                __builtin_amdgcn_raw_buffer_store_b128(v, prs, f * 16, 0, XL ? 0 : kCoherent);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
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
    // last arriver: thread t owns float4s t and t + 256 of every partial
    constexpr int OB = TILE_F4 / kSkThreads, SB = 16;
    static_assert(TILE_F4 % kSkThreads == 0, "tile float4s per thread");
    floatx4 sum[OB];
    bool col_ok[OB];
#pragma unroll
    for (int u = 0; u < OB; ++u) {
        const int f = tid + u * kSkThreads;
        col_ok[u] = p0 + (f >> 8) * 32 + (f & 31) < p.P;
        sum[u] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int s0 = 0; s0 < p.S; s0 += SB) {
        floatx4 v[OB][SB];
#pragma unroll
        for (int u = 0; u < OB; ++u)
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int f = (s0 + j) * TILE_F4 + tid + u * kSkThreads;
                v[u][j] = (col_ok[u] && s0 + j < p.S)
                              ? __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                prs, f * 16, 0, XL ? kSkipL1 : kCoherent))
                              : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
        for (int u = 0; u < OB; ++u)
#pragma unroll
            for (int j = 0; j < SB; ++j)
                if (s0 + j < p.S) sum[u] = (s0 + j == 0) ? v[u][j] : sum[u] + v[u][j];
    }
#pragma unroll
    for (int u = 0; u < OB; ++u) {
        if (!col_ok[u]) continue;
        const int f = tid + u * kSkThreads;
        const int ln = f & 63;
        const int r4 = (f >> 6) & 3;
        const int rn = f >> 8;
        const int pc = p0 + rn * 32 + (ln & 31);
        const int n = (int)fdiv_sk((uint32_t)pc, p.fd_wstr);
        const int rem = pc - n * p.OHW;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 8 * r4 + 4 * (ln >> 5) + i;
            const int co = co0 + row;
            if (co < p.CO)
                p.y[((long long)n * p.CO + co) * p.OHW + rem] =
                    apply_epilogue(p.epilogue, sum[u][i], e_bias[row], e_rs[row]);
        }
    }
    if (tid == 0) {
        if constexpr (XL)
            __hip_atomic_store(&p.tickets[tile * kTicketStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        else
            __hip_atomic_store(&p.tickets[tile * kTicketStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int KL>
int sk_lds_bytes(const ConvParams& p) {
    if (p.kc * p.T > 8 * KL) return 1 << 30;  // the stage must fit the k-lanes
    if (p.P >= (1LL << 31) || (long long)p.N * p.Hp >= (1LL << 31)) return 1 << 30;
    if ((long long)p.kc * p.R * p.Wp >= (1LL << 24)) return 1 << 30;
    // partial tiles are addressed with 32-bit byte offsets per tile
    if ((long long)p.S * kSkTileM * kSkTileN * 4 >= (1LL << 31)) return 1 << 30;
    return 4 * sk_layout(p.kc, p.R * p.Wp, 8 * KL).words;
}

template <int KL, bool XL>
hipError_t sk_launch(const ConvParams& p, hipStream_t stream) {
    const int bytes = sk_lds_bytes<KL>(p);
    if (bytes > 163840 - 64) return hipErrorInvalidValue;
    auto kern = igemm_f32_sk_kernel<KL, XL>;
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
    const SkLayout L = sk_layout(p.kc, p.R * p.Wp, 8 * KL);
    ConvParams q = p;
    q.fd_wstr = make_fastdiv((uint32_t)p.OHW);
    q.fd_wp = make_fastdiv((uint32_t)p.Wp);
    q.fd_rwp = make_fastdiv((uint32_t)L.xcs);
    q.fd_hp = make_fastdiv((uint32_t)p.Hp);
    q.fd_ow = make_fastdiv((uint32_t)p.OW);
    q.fd_t = make_fastdiv((uint32_t)p.T);
    q.fd_kw = make_fastdiv((uint32_t)p.KW);
    const long long tiles = (long long)p.tiles_m * p.tiles_n;
    const long long grid = XL ? 8 * ((tiles + 7) / 8) * p.S : tiles * p.S;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kSkThreads), bytes, stream, q);
    return hipGetLastError();
}

// descriptor: 32x32x2 instruction, waves 1 x 1 x 4 (CO x P x K), reps 1 x 2
#define CT_SK_VARIANT(NAME, KL, XL) \
    {NAME, DT_F32, 32, 32, 2, 1, 1, 4, 1, 2, 8 * KL, &sk_lds_bytes<KL>, &sk_launch<KL, XL>, nullptr, XL}

const IgemmVariant kSkVariants[] = {
    CT_SK_VARIANT("f32sk_m32n64_kl72", 72, false),
    CT_SK_VARIANT("f32sk_m32n64_kl36", 36, false),
    CT_SK_VARIANT("f32sk_m32n64_kl20", 20, false),
    CT_SK_VARIANT("f32skx_m32n64_kl72", 72, true),
    CT_SK_VARIANT("f32skx_m32n64_kl36", 36, true),
    CT_SK_VARIANT("f32skx_m32n64_kl20", 20, true),
};

}  // namespace

const IgemmVariant* igemm_f32_sk_variants(int* count) {
    *count = (int)(sizeof(kSkVariants) / sizeof(kSkVariants[0]));
    return kSkVariants;
}

}  // namespace ct
