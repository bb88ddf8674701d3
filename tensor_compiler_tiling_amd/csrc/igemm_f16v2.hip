// fp16 / bf16 implicit-GEMM convolution for 3x3 (and 1x1) filters, second form
// (v_mfma_f32_32x32x16_f16 / _bf16, fp32 accumulation and output, as the
// TVM tutorial "Tuning High Performance Convolution on NVIDIA GPUs", Step 1,
// declares the output).
//
// The half-precision instruction takes 8 consecutive reduction values per
// lane.  The reduction of a stage (KC channels x 9 taps) is ordered in groups
// of 8 channels at one tap, g = tap * (KC/8) + channel/8, and both operands
// sit channel-fastest in LDS, so a fragment is one 16-byte LDS read:
//   filter tile  [m][cg][tap][8]     window  [pixel][channel]
// What differs from the first form is where the reordering happens:
//  - the filter is reordered by a small kernel into the prepared layout
//    [CO][CI64/8][T][8] (CI64 = CI rounded up to 64, zeros past CI): 8
//    channels at one tap per 16 bytes, so one stage of one filter row (KC/8
//    groups x T taps, KC = 16, 32 or 64, a divisor of 64) is 9*KC contiguous
//    halves inside the row, whatever KC is, and staging the filter tile is a
//    stream of 16-byte copies with no arithmetic and no range checks.  A caller with a
//    static filter prepares it once (ct_conv2d_prepare_filter); otherwise
//    each launch reorders into its scratch first;
//  - the window is staged with vector loads of PX consecutive pixels of one
//    channel (PX = 8, 4, 2 or 1, the largest the row width and alignment
//    allow), 8 channels per task, transposed in registers into PX 16-byte
//    pixel records;
//  - LDS holds two copies of (filter tile, window).  The next stage's filter
//    tile goes from memory straight into the other copy (16-byte loads that
//    write LDS, no registers), all issued as the current stage starts; the
//    window loads (from HBM) go out two stages ahead into a second register
//    set and are transposed into the other copy after the stage's matrix
//    steps; one barrier per stage;
//  - a stage's 9*KC/16 matrix steps are unrolled, each reading the next
//    step's fragments before issuing its own instructions;
//  - in the variants with staging waves (names ending _x1, _x2), one or two
//    further waves take every window task and no matrix work: they write
//    stage st+1's window as stage st starts and then load stage st+3's, so
//    that the register transposes run beside the matrix waves' steps rather
//    than between their last step and the barrier.
// The window's padding is zeroed once at kernel start and never written
// again (only in-image pixels are staged).
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

constexpr int kBufRaw = 0x00020000;       // raw buffer descriptor, 32-bit elements
constexpr unsigned kBufOut = 0x80000000u;  // an offset past every buffer (all are < 2 GiB): reads zeros
typedef __attribute__((address_space(3))) void lds_void_t;

// One wave fills 64 consecutive 16-byte LDS slots from lane_off (bytes)
// within r, lane l the l-th; lds is wave-uniform.
__device__ __forceinline__ void load_chunk_to_lds(__amdgpu_buffer_rsrc_t r, uint16_t* lds, unsigned lane_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, lane_off, 0, 0, 0);
}

// s_waitcnt immediates that wait for the memory-load counter only (vmcnt in
// bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kVmcnt0 = vmcnt_imm(0);
template <int XPT> constexpr int kVmcnt8Xpt = vmcnt_imm(8 * XPT);

template <int DT> struct HMma2;
template <> struct HMma2<DT_F16> {
    static __device__ __forceinline__ floatx16 mma(uint4v a, uint4v b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                     __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
    }
};
template <> struct HMma2<DT_BF16> {
    static __device__ __forceinline__ floatx16 mma(uint4v a, uint4v b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

// Record t of a prepared-filter unit: `in` holds one filter row's 8 channels
// x T taps in the caller's layout (half h = c*T + t, channel-major); the
// record is the 8 channels at tap t, each output word two halves picked by
// one byte permute (v_perm_b32: bytes 0-3 of its second operand, 4-7 of its
// first).
template <int T>
__device__ __forceinline__ uint4v tap_record(const uint4v* in, int t) {
    uint4v o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ia = 2 * j * T + t, ib = (2 * j + 1) * T + t;
        const uint32_t wa = in[ia / 8][(ia % 8) / 2];
        const uint32_t wb = in[ib / 8][(ib % 8) / 2];
        const uint32_t sel = ((ib & 1) ? 0x07060000u : 0x05040000u) | ((ia & 1) ? 0x0302u : 0x0100u);
        o[j] = __builtin_amdgcn_perm(wb, wa, sel);
    }
    return o;
}

// w [CO][CI][T] -> wp [CO][CGP][T][8], one thread per (row, 8-channel group)
// unit: T 16-byte loads of the unit's contiguous run, T 16-byte records out
// (zeros for the groups past CI).  Needs CI % 8 == 0 and a 16-byte aligned w.
template <int T>
__global__ __launch_bounds__(64) void h2_prepare_vec_kernel(const uint4v* __restrict__ w, uint4v* __restrict__ wp,
                                                            int CO, int CG, int CGP) {
    const long long u = (long long)blockIdx.x * 64 + threadIdx.x;  // unit (co, g), g < CGP
    if (u >= (long long)CO * CGP) return;
    const long long co = u / CGP;
    const int g = (int)(u - co * CGP);
    uint4v in[T];
#pragma unroll
    for (int i = 0; i < T; ++i) in[i] = g < CG ? w[(co * CG + g) * T + i] : uint4v{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < T; ++t) wp[u * T + t] = T == 1 ? in[0] : tap_record<T>(in, t);
}

// The same for any CI and alignment, one element at a time.
__global__ __launch_bounds__(256) void h2_prepare_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wp,
                                                         int CO, int CI, int T) {
    const int CG8 = (CI + 63) / 64 * 8;  // groups of a prepared row
    const long long total = (long long)CO * CG8 * T * 8;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const int j = (int)(i & 7);
        const long long r1 = i >> 3;
        const int t = (int)(r1 % T);
        const long long r2 = r1 / T;
        const int g = (int)(r2 % CG8);
        const long long co = r2 / CG8;
        const int c = 8 * g + j;
        wp[i] = c < CI ? w[(co * CI + c) * T + t] : (uint16_t)0;
    }
}

// NXW: waves that only stage the window (0: the matrix waves stage it).
template <int WM, int WN, int RM, int RN, int KC, int T, int NXW = 0>
struct H2 {
    static constexpr int TM = WM * RM * 32;
    static constexpr int TN = WN * RN * 32;
    static constexpr int NTM = WM * WN * 64;   // threads of the matrix waves
    static constexpr int NT = NTM + NXW * 64;  // threads of the workgroup
    static constexpr int CG = KC / 8;          // channel groups per stage
    static constexpr int G = T * CG;           // groups per stage
    static constexpr int NSTEP = G / 2;        // instruction steps per stage
    static constexpr int WST = (G + 1) * 8;    // halves per filter row in LDS (odd x 16 B)
    static constexpr int KCS = (CG + 1) * 8;   // halves per window pixel (odd x 16 B)
    static constexpr int NW = WM * WN;         // matrix waves
    // the filter tile of a stage as 16-byte LDS slots [TM][G + 1] (the last
    // slot of a row is padding), filled 64 slots (one load per wave) at a time
    static constexpr int WSL = TM * (G + 1);
    static constexpr int WCK = WSL / 64;       // 64-slot chunks
    static constexpr int WLD = (WCK + NW - 1) / NW;  // chunk loads per wave
    static_assert(WSL % 64 == 0, "whole chunks");
    // window tasks per staging thread and the task stride: with staging
    // waves, as many tasks as 32 registers of one set hold (8 loads of PX
    // halves a task, a 1- or 2-pixel load in one register)
    static constexpr int xpt(int px) {
        return NXW == 0 ? (NTM >= 256 ? 1 : 2) : (px >= 8 ? 1 : px == 4 ? 2 : 4);
    }
    static constexpr int XT = NXW == 0 ? NTM : NXW * 64;
    static constexpr int WB = TM * WST;        // halves per filter copy
    static_assert(G % 2 == 0, "a step takes two groups");
};

__host__ __device__ inline int h2_xb(int R, int Wp, int kcs) { return round_up(R * Wp * kcs, 8); }

// Vector of PX halves.
template <int PX> struct PxVec;
template <> struct PxVec<8> { typedef uint4v T; };
template <> struct PxVec<4> { typedef uint2v T; };
template <> struct PxVec<2> { typedef uint32_t T; };
template <> struct PxVec<1> { typedef uint16_t T; };

__device__ __forceinline__ uint32_t pack2h(uint16_t lo, uint16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Pixel u of two channels' vectors a and b, packed as (a[u], b[u]): for
// PX >= 2 one byte permute (v_perm_b32: bytes 0-3 of its second operand,
// 4-7 of its first) of the two 32-bit words that hold pixel u.
template <int PX>
__device__ __forceinline__ uint32_t pack_px(const typename PxVec<PX>::T& a, const typename PxVec<PX>::T& b, int u) {
    if constexpr (PX == 1) {
        return pack2h(a, b);
    } else {
        uint32_t da, db;
        if constexpr (PX == 2) {
            da = a;
            db = b;
        } else {
            da = a[u >> 1];
            db = b[u >> 1];
        }
        return __builtin_amdgcn_perm(db, da, (u & 1) ? 0x07060302u : 0x05040100u);
    }
}

// Raw buffer load of PX halves at byte offset off.
template <int PX> struct BufLoad;
template <> struct BufLoad<8> {
    static __device__ __forceinline__ uint4v load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
};
template <> struct BufLoad<4> {
    static __device__ __forceinline__ uint2v load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
};
template <> struct BufLoad<2> {
    static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
};
template <> struct BufLoad<1> {
    static __device__ __forceinline__ uint16_t load(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
};

// Column tiles of the grid: tiles_n rounded up to a multiple of 8, so that
// every XCD (workgroup b runs on XCD b % 8) takes a block of whole columns.
__host__ __device__ inline int h2_col_tiles(int tiles_n) { return (tiles_n + 7) & ~7; }

// The kernel's arguments: the convolution's plus the divisors of its index
// set-up, so that the set-up runs on 32-bit multiply-high divisions (a
// 64-bit or runtime 32-bit division is a long instruction sequence, and the
// set-up precedes every load of the workgroup).
struct H2Params : ConvParams {
    FastDiv fd_ohw;    // OH * OW
    FastDiv fd_tiles;  // workgroups per split: tiles_m * h2_col_tiles(tiles_n)
    FastDiv fd_lm;     // row tiles of one XCD's rectangle (all of them without XCD groups)
    FastDiv fd_rn;     // window tasks per channel group: R * runs per row
    FastDiv fd_run;    // runs per window row: W / PX
    int cgl;           // log2 of the XCD column groups; -1: column blocks per XCD
};
// also fd_kw = KW, fd_ow = OW, fd_hp = Hp (filled by the launcher)

__device__ __forceinline__ void fetch_h2_kernargs(const H2Params& p) {
    fetch_kernargs(p);
    asm volatile("" ::"s"(p.fd_lm.d));  // the sixth 64-byte line
}
// (the derived fields follow the base's: fd_lm starts the sixth line)
static_assert((sizeof(ConvParams) + 2 * sizeof(FastDiv)) / 64 == 5 && sizeof(H2Params) <= 384,
              "six argument lines");

// n / d for any 32-bit n (the divisor's round-up multiplier and shift)
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (uint32_t)(((uint64_t)__umulhi(n, f.mul) + n) >> f.shift);
}

template <int DT, int WM, int WN, int RM, int RN, int KC, int T, int PX, int NXW>
__global__ __launch_bounds__((WM * WN + NXW) * 64) void igemm_h2_kernel(H2Params p) {
    fetch_h2_kernargs(p);
    using C = H2<WM, WN, RM, RN, KC, T, NXW>;
    constexpr int TM = C::TM, TN = C::TN, NT = C::NT, CG = C::CG, G = C::G;
    constexpr int NSTEP = C::NSTEP, WST = C::WST, KCS = C::KCS, XPT = C::xpt(PX);
    constexpr int NW = C::NW, WCK = C::WCK, WLD = C::WLD;
    extern __shared__ __align__(16) uint16_t hs[];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform, and known to be: branches on it are not divergent
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // waves NW.. (when NXW > 0) only stage the window
    const bool mma_wave = wave < NW;
    const int wm = wave % WM;
    const int wn = wave / WM;
    const int lj = lane & 31;
    const int lh = lane >> 5;

    const int RWp = p.R * p.Wp;
    const int XB = h2_xb(p.R, p.Wp, KCS);
    uint16_t* Wsb = hs;                // [2][TM][WST]
    uint16_t* Xsb = hs + 2 * C::WB;    // [2][R*Wp][KCS]
    float* e_bias = reinterpret_cast<float*>(hs + 2 * C::WB + 2 * XB);
    float* e_rs = e_bias + TM;

    // workgroup -> (split, tile).  When the column tiles come in multiples
    // of 8, workgroup b runs on XCD x = b % 8 (round-robin placement) and the
    // XCDs split the tile grid into ga row groups x 8/ga column groups
    // (2^cgl = 8/ga): XCD x takes one rectangle, row tiles fastest (the
    // readers of one window run together).  Each filter row block is then
    // read by 8/ga XCDs and each window by ga; the launcher picks ga.
    // Otherwise (cgl < 0) the grid holds column tiles rounded up to a
    // multiple of 8 (h2_col_tiles) and each XCD takes a block of whole
    // columns; workgroups past the last column exit at once.
    const int split = (int)fdiv(blockIdx.x, p.fd_tiles);
    const uint32_t b = blockIdx.x - (uint32_t)split * p.fd_tiles.d;
    const uint32_t x = b & 7, l = b >> 3;
    const uint32_t lq = fdiv(l, p.fd_lm);
    const int lr = (int)(l - lq * p.fd_lm.d);
    int tm, tn;
    if (p.cgl >= 0) {
        tm = (int)(x >> p.cgl) * (int)p.fd_lm.d + lr;
        tn = (int)(x & ((1u << p.cgl) - 1)) * (p.tiles_n >> p.cgl) + (int)lq;
    } else {
        tm = lr;
        tn = (int)x * (h2_col_tiles(p.tiles_n) >> 3) + (int)lq;
        if (tn >= p.tiles_n) return;  // padding of the grid: uniform over the workgroup
    }
    const int tile = tm + tn * p.tiles_m;
    const int co0 = tm * TM;
    // column indices fit 32 bits (P < 2^31, checked by the launcher)
    const uint32_t p0 = (uint32_t)tn * TN;
    const uint32_t n_first = fdiv(p0, p.fd_ohw);
    const uint32_t oy_first = fdiv(p0 - n_first * p.fd_ohw.d, p.fd_ow);
    const int vr_first = (int)(n_first * p.Hp + oy_first * p.stride);
    const long long HW = (long long)p.H * p.W;

    const uint16_t* __restrict__ xg = static_cast<const uint16_t*>(p.x);
    // the prepared filter: the caller's (p.w) or this launch's copy (p.aux)
    const uint16_t* __restrict__ wpk = static_cast<const uint16_t*>(p.aux ? p.aux : p.w);
    const int CG8 = (p.CI + 63) / 64 * 8;  // 8-channel groups of a prepared filter row
    const int NS = (p.CI + KC - 1) / KC;  // stages of the whole reduction

    // ---- per-lane B columns --------------------------------------------------
    int pbase[RN];       // window pixel of the column's (0,0) tap
    long long yoff[RN];  // y offset of (n, 0, oy, ox); -1 past P
#pragma unroll
    for (int rn = 0; rn < RN; ++rn) {
        const uint32_t pc = p0 + (uint32_t)((wn * RN + rn) * 32 + lj);
        pbase[rn] = 0;
        yoff[rn] = -1;
        if ((long long)pc < p.P) {
            const uint32_t n = fdiv(pc, p.fd_ohw);
            const int rem = (int)(pc - n * p.fd_ohw.d);
            const int oy = (int)fdiv((uint32_t)rem, p.fd_ow);
            const int ox = rem - oy * p.OW;
            pbase[rn] = ((int)n * p.Hp + oy * p.stride - vr_first) * p.Wp + ox * p.stride;
            yoff[rn] = (long long)n * p.CO * p.OHW + rem;
        }
    }
    // Window offset of this lane's group 2s + lh at step s.  With an even
    // number of channel groups the two groups of a step share one tap, so
    // the offset is a wave-uniform step part (tap and group 2s) plus the
    // lane part lh*8, which goes into the lane's base address.
    static_assert(CG % 2 == 0, "the two groups of a step share a tap");
    int koff[NSTEP];
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        const int t = (2 * s) / CG;
        const int cg = 2 * s - t * CG;
        const int ky = (int)fdiv((uint32_t)t, p.fd_kw);
        const int kx = t - ky * p.KW;
        koff[s] = __builtin_amdgcn_readfirstlane((ky * p.Wp + kx) * KCS + cg * 8);
    }
    int xlane[RN];
#pragma unroll
    for (int rn = 0; rn < RN; ++rn) xlane[rn] = pbase[rn] * KCS + lh * 8;

    // ---- epilogue values of row m = tid, loaded now (ahead of the stage
    //      loads, so that waiting for them never waits for those) and written
    //      to the LDS tables once the first stage's loads are out; zero both
    //      windows -------------------------------------------------------------
    static_assert(TM <= C::NTM, "one epilogue row per matrix thread");
    float e_b = 0.0f, e_v = 0.0f;
    const bool e_row = tid < TM && co0 + tid < p.CO;
    if (e_row && p.epilogue != EPI_NONE) e_b = p.bias[co0 + tid];
    if (e_row && p.epilogue == EPI_EXP_BIAS_RSQRT) e_v = p.var[co0 + tid];
    auto write_tables = [&]() {
        if (tid < TM) {
            e_bias[tid] = e_b;
            e_rs[tid] = (e_row && p.epilogue == EPI_EXP_BIAS_RSQRT) ? dev_rsqrt(e_v + p.eps) : 1.0f;
        }
    };
    {
        uint4v* xz = reinterpret_cast<uint4v*>(Xsb);
        for (int i = tid; i < XB / 4; i += NT) xz[i] = uint4v{0u, 0u, 0u, 0u};  // 2*XB halves
    }

    // ---- staging tasks (fixed for the kernel) ----------------------------------
    // filter slot q = (m, r) of chunk wave + j*NW: record r = cg*T + tap of
    // row co0+m's stage, in the prepared row's order (r = G: padding)
    int wsrc[WLD];  // halves, without the stage term; -1: padding
#pragma unroll
    for (int j = 0; j < WLD; ++j) {
        const int q = (wave + j * NW) * 64 + lane;
        const int m = q / (G + 1);
        const int r = q - m * (G + 1);
        wsrc[j] = (q < C::WSL && r < G) ? (co0 + m) * CG8 * (T * 8) + r * 8 : -1;
    }
    // window task q = (cg, window row r, run u): 8 channels x PX pixels, for
    // thread tid - xt0 (the staging waves' threads with NXW > 0)
    constexpr int xt0 = NXW == 0 ? 0 : C::NTM;
    const int nrun = p.W / PX;
    const int n_xt = CG * p.R * nrun;
    long long xsrc[XPT];  // halves, channel cg*8 without the stage term; -1: none
    int xdst[XPT];
    int xch[XPT];         // channel of the task's first lane within a stage
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
        const int q = tid - xt0 + j * C::XT;
        xsrc[j] = -1;
        xdst[j] = 0;
        xch[j] = 0;
        if (q >= 0 && q < n_xt) {
            const int cg = (int)fdiv((uint32_t)q, p.fd_rn);
            const int rem = q - cg * (int)p.fd_rn.d;
            const int r = (int)fdiv((uint32_t)rem, p.fd_run);
            const int u = rem - r * nrun;
            const uint32_t vr = (uint32_t)vr_first + (uint32_t)r;
            const int n = (int)fdiv(vr, p.fd_hp);
            const int iy = (int)(vr - (uint32_t)n * p.Hp) - p.pad;
            if (n < p.N && iy >= 0 && iy < p.H) {
                xsrc[j] = ((n * p.CI + cg * 8) * p.H + iy) * (long long)p.W + u * PX;
                xdst[j] = (r * p.Wp + p.pad + u * PX) * KCS + cg * 8;
                xch[j] = cg * 8;
            }
        }
    }

    using XV = typename PxVec<PX>::T;
    // Staging registers.  The filter tile (from the small reordered copy,
    // an L2 hit) is loaded one stage ahead; the input window (from HBM) two
    // stages ahead, into two register sets, so each window load has two
    // stages of matrix work to arrive.
    struct XRegs {
        XV v[XPT][8];
    };
    // Loads are raw buffer loads with no condition around them.  A stage's
    // descriptors start at that stage (x at its first channel, the reordered
    // filter at its block), so a lane's byte offsets are fixed for the
    // kernel: the filter chunk's, and the window task's plus i*HW*2 for its
    // channel i.  A lane with no chunk or task passes an offset past the
    // buffer and reads zeros.  (A load under a condition, or with a zero
    // default, compiles to code on which the compiler must wait for every
    // load in flight, the prefetches included.)
    const long long x_bytes = (long long)p.N * p.CI * HW * 2;
    const long long w_bytes = (long long)p.CO * CG8 * T * 16;
    unsigned wvo[WLD], xvo[XPT];
#pragma unroll
    for (int j = 0; j < WLD; ++j) wvo[j] = wsrc[j] >= 0 ? (unsigned)wsrc[j] * 2u : kBufOut;
#pragma unroll
    for (int j = 0; j < XPT; ++j) xvo[j] = xsrc[j] >= 0 ? (unsigned)xsrc[j] * 2u : kBufOut;

    floatx16 acc[RM][RN];
#pragma unroll
    for (int rm = 0; rm < RM; ++rm)
#pragma unroll
        for (int rn = 0; rn < RN; ++rn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rm][rn][r] = 0.0f;

    // issue(s): the loads to issue between the fragment reads and the
    // instructions of matrix step s
    auto mfma_stage = [&](int buf, auto&& issue) {
        const uint16_t* Wb = Wsb + buf * C::WB;
        const uint16_t* Xb = Xsb + buf * XB;
        uint4v a[2][RM], bf[2][RN];
        auto frag = [&](int s, uint4v (&ar)[RM], uint4v (&br)[RN]) {
#pragma unroll
            // groups 2s and 2s+1 of the step (tap-major) are records
            // (cg*T + tap) of the filter tile: channel groups cg and cg+1 of
            // one tap, T records apart
            for (int rm = 0; rm < RM; ++rm)
                ar[rm] = *reinterpret_cast<const uint4v*>(Wb + ((wm * RM + rm) * 32 + lj) * WST + lh * (T * 8) +
                                                          (((2 * s) % CG) * T + (2 * s) / CG) * 8);
#pragma unroll
            for (int rn = 0; rn < RN; ++rn)
                br[rn] = *reinterpret_cast<const uint4v*>(Xb + xlane[rn] + koff[s]);
        };
        frag(0, a[0], bf[0]);
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            if (s + 1 < NSTEP) frag(s + 1, a[(s + 1) & 1], bf[(s + 1) & 1]);
            issue(s);
            // the next step's reads stay ahead of this step's instructions
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rm = 0; rm < RM; ++rm)
#pragma unroll
                for (int rn = 0; rn < RN; ++rn)
                    acc[rm][rn] = HMma2<DT>::mma(a[s & 1][rm], bf[s & 1][rn], acc[rm][rn]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- stages of this split: loads two stages ahead, multiply, store the
    //      next stage, one barrier per stage
    const int s_first = split * p.stages;
    int nst = p.stages;
    if (s_first + nst > NS) nst = NS - s_first;
    __syncthreads();  // windows zeroed before any stage writes into them
    // Stage indices past the split's last stage are clamped to it: the loads
    // and LDS writes of every step are unconditional (the extra ones load the
    // last stage again and write the buffer no later stage reads).  The loop
    // comes in two copies, for the waves that stage window tasks (HX) and for
    // those that do not, so that in each the number of loads issued per step
    // is fixed and the compiler waits for exactly the ones a step consumes
    // (mode 1 and mode 0; mode 2 is a staging wave's loop: window staging
    // and no matrix work).
    const int last = nst - 1;
    auto run_stages = [&](auto mode_tag) {
        constexpr int MODE = decltype(mode_tag)::value;
        constexpr bool HX = MODE != 0;
        XRegs xa, xb;
        // Load units: filter chunk j of stage s_abs (into LDS copy buf), and
        // window channel i of every task of the stage starting at channel c0.
        // Channels past CI in the last image read zeros; those past CI inside
        // the tensor are zeroed by store_stage.
        // (descriptor fields pass through readfirstlane: they are uniform,
        // and a descriptor the compiler cannot prove uniform costs a loop
        // over the lanes around each load)
        // The descriptor starts at the stage's first group of row 0 (a stage
        // never runs past its row: rows hold a multiple of 64 channels), so
        // only rows past CO fall outside it and read zeros.
        // Each load writes the 64 consecutive 16-byte LDS slots of one chunk,
        // lane l the l-th (the LDS address is the chunk's, a wave-uniform
        // value).
        auto load_w = [&](int s_abs, int buf) {
            const int sb = __builtin_amdgcn_readfirstlane(s_abs * CG * (T * 8));  // halves
            const int nrec = __builtin_amdgcn_readfirstlane((int)(w_bytes - 2LL * sb));
            const __amdgpu_buffer_rsrc_t wrs =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wpk + sb), 0, nrec, kBufRaw);
            auto one = [&](int j) { load_chunk_to_lds(wrs, Wsb + buf * C::WB + (wave + j * NW) * 512, wvo[j]); };
            // only a wave's last chunk can lie past the tile
#pragma unroll
            for (int j = 0; j + 1 < WLD; ++j) one(j);
            if (WCK % NW == 0 || wave + (WLD - 1) * NW < WCK) one(WLD - 1);
            // loads issued later stay later (wait_filter counts on it)
            __builtin_amdgcn_sched_barrier(0);
        };
        auto load_x1 = [&](XRegs& rg, int i, int c0) {
            // one descriptor per channel (scalar work only)
            const int cb = __builtin_amdgcn_readfirstlane((int)((long long)(c0 + i) * HW));  // halves
            // a descriptor at a channel past the whole tensor (batch 1, the
            // last stage's channels past CI) gets an empty range: every load
            // through it is padding and reads zeros, and none reaches memory
            const long long left = x_bytes - 2LL * cb;
            const int nrec = __builtin_amdgcn_readfirstlane((int)(left > 0 ? left : 0));
            const __amdgpu_buffer_rsrc_t xrs =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xg + cb), 0, nrec, kBufRaw);
#pragma unroll
            for (int j = 0; j < XPT; ++j) rg.v[j][i] = BufLoad<PX>::load(xrs, xvo[j]);
        };
        auto load_x = [&](XRegs& rg, int c0) {
            if constexpr (HX) {
#pragma unroll
                for (int i = 0; i < 8; ++i) load_x1(rg, i, c0);
            }
        };
        // The next stages' loads: the filter chunks as the stage's first
        // matrix step issues, the window channels spread over the later
        // steps (channel i at step 1 + i * (NSTEP - 1) / 8; all at the first
        // when a stage is one step), so that no wave
        // stalls on a full memory queue with its matrix work waiting.  Every
        // filter load precedes every window load of the stage.
        auto spread_loads = [&](int s, int s_w, int buf_w, XRegs& rg, int c0) {
            if (s == 0) load_w(s_w, buf_w);
            if constexpr (HX) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if ((NSTEP > 1 ? 1 + i * (NSTEP - 1) / 8 : 0) == s) load_x1(rg, i, c0);
            }
        };
        // Wait for this wave's filter loads: the window loads issued after
        // them may stay in flight (memory loads complete in order).
        auto wait_filter = [&]() {
            if constexpr (HX)
                __builtin_amdgcn_s_waitcnt(kVmcnt8Xpt<XPT>);
            else
                __builtin_amdgcn_s_waitcnt(kVmcnt0);
        };
        // LDS writes of a stage's window: its pixel records (channels past
        // CI zeroed first).  c0: the stage's first channel.
        auto store_stage = [&](XRegs& rg, int buf, int c0) {
            uint16_t* Xb = Xsb + buf * XB;
            if constexpr (HX) {
                auto& xreg = rg.v;
                // only a last stage that runs past CI has channels to zero
                // (a uniform test: the selects cost as much as the packing)
                const bool tail = c0 + KC > p.CI;
#pragma unroll
                for (int j = 0; j < XPT; ++j) {
                    if (xvo[j] == kBufOut) continue;
                    if (tail) {
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            if (c0 + xch[j] + i >= p.CI) xreg[j][i] = XV{};
                    }
#pragma unroll
                    for (int u = 0; u < PX; ++u) {
                        uint4v o;
                        o.x = pack_px<PX>(xreg[j][0], xreg[j][1], u);
                        o.y = pack_px<PX>(xreg[j][2], xreg[j][3], u);
                        o.z = pack_px<PX>(xreg[j][4], xreg[j][5], u);
                        o.w = pack_px<PX>(xreg[j][6], xreg[j][7], u);
                        *reinterpret_cast<uint4v*>(Xb + xdst[j] + u * KCS) = o;
                    }
                }
            }
        };
        if constexpr (MODE == 2) {
            // A staging wave stores stage st+1's window (loaded two stages
            // earlier) as soon as stage st starts (its copy was last read in
            // stage st-1), then loads stage st+3's into the freed registers;
            // its register transposes run beside the matrix waves' steps.
            // (The compiler waits for each register's own loads: the newer
            // set stays in flight.)
            if (nst > 0) {
                load_x(xa, s_first * KC);
                load_x(xb, (s_first + min(1, last)) * KC);
                store_stage(xa, 0, s_first * KC);
                load_x(xa, (s_first + min(2, last)) * KC);
            }
            __syncthreads();
            auto sstep = [&](int st, XRegs& held) {
                store_stage(held, (st + 1) & 1, (s_first + min(st + 1, last)) * KC);
                load_x(held, (s_first + min(st + 3, last)) * KC);
                __syncthreads();
            };
            int st = 0;
            for (; st + 1 < nst; st += 2) {
                sstep(st, xb);
                sstep(st + 1, xa);
            }
            if (st < nst) sstep(st, xb);
            return;
        }
        if (nst > 0) {
            load_w(s_first, 0);
            load_x(xa, s_first * KC);
            load_x(xb, (s_first + min(1, last)) * KC);
            store_stage(xa, 0, s_first * KC);
        }
        write_tables();
        if (nst > 0) wait_filter();
        __syncthreads();
        // stage st: `held` has stage st+1's window, `free` takes stage st+2's
        auto step = [&](int st, XRegs& held, XRegs& free) {
            const int s_w = s_first + min(st + 1, last);
            const int c0x = (s_first + min(st + 2, last)) * KC;
            mfma_stage(st & 1, [&](int s) { spread_loads(s, s_w, (st + 1) & 1, free, c0x); });
            // LDS writes after the matrix steps: interleaved with them, the
            // window's register transposes lengthen the matrix phase by as
            // much as they take
            store_stage(held, (st + 1) & 1, (s_first + min(st + 1, last)) * KC);
            wait_filter();
            __syncthreads();
        };
        int st = 0;
        for (; st + 1 < nst; st += 2) {
            step(st, xb, xa);
            step(st + 1, xa, xb);
        }
        if (st < nst) step(st, xb, xa);
    };
    if constexpr (NXW > 0) {
        if (mma_wave)
            run_stages(std::integral_constant<int, 0>{});
        else
            run_stages(std::integral_constant<int, 2>{});
    } else {
        // wave-uniform: does this wave hold any window task (q = tid + j*NT)?
        if (wave * 64 < n_xt)
            run_stages(std::integral_constant<int, 1>{});
        else
            run_stages(std::integral_constant<int, 0>{});
    }

    // ---- split reduction across workgroups (device-scope atomics) -------------
    const int wslot = wm + wn * WM;
    if (p.S > 1) {
        const long long tile_words = (long long)TM * TN;
        float* part = p.ws + ((long long)tile * p.S) * tile_words;
        const int base = wslot * RM * RN * 16;
        float* mine = part + (long long)split * tile_words;
        // (staging waves hold no results: they only take the barriers)
        if (mma_wave) {
#pragma unroll
            for (int rm = 0; rm < RM; ++rm)
#pragma unroll
                for (int rn = 0; rn < RN; ++rn)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        __hip_atomic_store(&mine[(base + (rm * RN + rn) * 16 + r) * 64 + lane], acc[rm][rn][r],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const unsigned old = __hip_atomic_fetch_add(&p.tickets[tile * kTicketStride], 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = (old == (unsigned)(p.S - 1)) ? 1 : 0;
        }
        __syncthreads();
        if (!s_last || !mma_wave) return;
#pragma unroll
        for (int rm = 0; rm < RM; ++rm)
#pragma unroll
            for (int rn = 0; rn < RN; ++rn)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // every split's partial from memory, this one's too (the
                    // same value as its registers, so the sum is unchanged):
                    // selecting the registers for s2 == split compiled, in
                    // some of the forms with staging waves, to code that read
                    // a wrong value for the first element of each block
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

    if (!mma_wave) return;
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
                // streamed out: the results are not read again by this launch
                __builtin_nontemporal_store(apply_epilogue(p.epilogue, acc[rm][rn][r], eb, er),
                                            &p.y[yoff[rn] + (long long)co * p.OHW]);
            }
        }
    }
}

// Pixels per window task for this shape: the widest vector that divides W.
inline int h2_px_for_shape(int W) {
    if (W % 8 == 0) return 8;
    if (W % 4 == 0) return 4;
    if (W % 2 == 0) return 2;
    return 1;
}

template <int WM, int WN, int RM, int RN, int KC, int T, int NXW>
int h2_bytes_for(const ConvParams& p, int px) {
    using C = H2<WM, WN, RM, RN, KC, T, NXW>;
    if (p.T != T || p.kc != KC) return 1 << 30;
    if (p.P >= (1LL << 31) || (long long)p.N * p.Hp >= (1LL << 31)) return 1 << 30;
    // x and the prepared filter are read through buffer descriptors with
    // 32-bit byte offsets; offset 2^31 must lie past both, also for the rows
    // of the last tile past CO
    const long long tiles_m = (p.CO + C::TM - 1) / C::TM;
    if (tiles_m * C::TM * round_up(p.CI, 64) * T * 2 >= (1LL << 31)) return 1 << 30;
    static_assert(64 % KC == 0, "a stage divides a prepared row's 64-channel blocks");
    if ((long long)p.N * p.CI * p.H * p.W * 2 >= (1LL << 31)) return 1 << 30;
    // the window tasks must fit the per-thread slots
    if ((long long)C::CG * p.R * (p.W / px) > (long long)C::xpt(px) * C::XT) return 1 << 30;
    if ((long long)p.R * p.Wp * C::KCS >= (1LL << 28)) return 1 << 30;
    return 2 * (2 * C::WB + 2 * h2_xb(p.R, p.Wp, C::KCS) + 4 * C::TM);
}

template <int WM, int WN, int RM, int RN, int KC, int T, int NXW>
int h2_lds_bytes(const ConvParams& p) {
    return h2_bytes_for<WM, WN, RM, RN, KC, T, NXW>(p, h2_px_for_shape(p.W));
}

// The launch's own prepared copy of the filter (none when the caller passes
// a prepared filter).
template <int WM, int WN, int RM, int RN, int KC, int T>
long long h2_aux_bytes(const ConvParams& p) {
    if (p.w_prepared) return 0;
    return 2LL * p.CO * round_up(p.CI, 64) * T;
}

template <int DT, int WM, int WN, int RM, int RN, int KC, int T, int NXW, int PX>
hipError_t h2_launch_px(const ConvParams& base, int bytes, hipStream_t stream) {
    using C = H2<WM, WN, RM, RN, KC, T, NXW>;
    auto kern = igemm_h2_kernel<DT, WM, WN, RM, RN, KC, T, PX, NXW>;
    H2Params q;
    static_cast<ConvParams&>(q) = base;
    q.fd_kw = make_fastdiv((uint32_t)base.KW);
    q.fd_ow = make_fastdiv((uint32_t)base.OW);
    q.fd_hp = make_fastdiv((uint32_t)base.Hp);
    q.fd_ohw = make_fastdiv((uint32_t)base.OHW);
    const int cols = h2_col_tiles(base.tiles_n);
    q.fd_tiles = make_fastdiv((uint32_t)(base.tiles_m * cols));
    // XCD row groups ga: the one that minimises the estimate of the bytes
    // the XCDs fetch, (8/ga) * tiles_m*TM*K + ga * tiles_n*TN*CI (1 for
    // convolutions, whose filters are small; 2 or 4 for large matrix
    // products), among those that divide the grid
    q.cgl = -1;
    int lm = base.tiles_m;
    if ((base.tiles_n & 7) == 0) {
        const double wbytes = (double)base.tiles_m * C::TM * base.K;
        const double xbytes = (double)base.tiles_n * C::TN * base.CI;
        int ga = 1;
        double best = 8.0 * wbytes + xbytes;
        for (int g = 2; g <= 8; g *= 2) {
            const double cost = (8 / g) * wbytes + g * xbytes;
            if (base.tiles_m % g == 0 && base.tiles_n % (8 / g) == 0 && cost < best) {
                best = cost;
                ga = g;
            }
        }
        q.cgl = ga == 1 ? 3 : ga == 2 ? 2 : ga == 4 ? 1 : 0;
        lm = base.tiles_m / ga;
    }
    q.fd_lm = make_fastdiv((uint32_t)lm);
    const int nrun = base.W / PX;
    q.fd_rn = make_fastdiv((uint32_t)(base.R * nrun));
    q.fd_run = make_fastdiv((uint32_t)nrun);
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
    const long long grid = (long long)q.tiles_m * h2_col_tiles(q.tiles_n) * q.S;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), bytes, stream, q);
    return hipGetLastError();
}

template <int DT, int WM, int WN, int RM, int RN, int KC, int T, int NXW>
hipError_t h2_launch(const ConvParams& p, hipStream_t stream) {
    // the widest window vector the shape and the pointer's alignment allow
    // (every run starts at a multiple of PX pixels of a row)
    int px = h2_px_for_shape(p.W);
    const uintptr_t xa = reinterpret_cast<uintptr_t>(p.x);
    while (px > 1 && (xa % (2u * px) != 0 || (p.H * (long long)p.W) % px != 0)) px >>= 1;
    const int bytes = h2_bytes_for<WM, WN, RM, RN, KC, T, NXW>(p, px);
    if (bytes > 163840 - 64) return hipErrorInvalidValue;

    ConvParams pp = p;
    if (!p.w_prepared) {
        // reorder the filter into this launch's prepared copy
        if (!p.aux) return hipErrorInvalidValue;
        const hipError_t e = h2_prepare_filter(p.w, p.aux, p.CO, p.CI, T, stream);
        if (e != hipSuccess) return e;
    } else {
        pp.aux = nullptr;  // the caller's filter is prepared: stage from p.w
    }
    switch (px) {
        case 8: return h2_launch_px<DT, WM, WN, RM, RN, KC, T, NXW, 8>(pp, bytes, stream);
        case 4: return h2_launch_px<DT, WM, WN, RM, RN, KC, T, NXW, 4>(pp, bytes, stream);
        case 2: return h2_launch_px<DT, WM, WN, RM, RN, KC, T, NXW, 2>(pp, bytes, stream);
        default: return h2_launch_px<DT, WM, WN, RM, RN, KC, T, NXW, 1>(pp, bytes, stream);
    }
}

}  // namespace

// wp [CO][CI64/8][T][8] = w [CO][CI][T] regrouped, zeros past CI (CI64 = CI
// rounded up to 64).
hipError_t h2_prepare_filter(const void* w, void* wp, int CO, int CI, int T, hipStream_t stream) {
    (void)hipGetLastError();
    const int CGP = (CI + 63) / 64 * 8;
    const long long units = (long long)CO * CGP;
    if (CI % 8 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0 && (T == 9 || T == 1)) {
        // one wave per 64 units: small filters still spread over many CUs
        const long long blocks = (units + 63) / 64;
        if (T == 9)
            hipLaunchKernelGGL(h2_prepare_vec_kernel<9>, dim3((unsigned)blocks), dim3(64), 0, stream,
                               static_cast<const uint4v*>(w), static_cast<uint4v*>(wp), CO, CI / 8, CGP);
        else
            hipLaunchKernelGGL(h2_prepare_vec_kernel<1>, dim3((unsigned)blocks), dim3(64), 0, stream,
                               static_cast<const uint4v*>(w), static_cast<uint4v*>(wp), CO, CI / 8, CGP);
    } else {
        long long blocks = (units * T * 8 + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(h2_prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(w), static_cast<uint16_t*>(wp), CO, CI, T);
    }
    return hipGetLastError();
}

namespace {

// descriptor: 32x32x16 instruction, waves WM x WN x 1, reps RM x RN; kc fixed
// at KC (kc_max = KC); filters of T taps (3x3, and 1x1 for the matrix-product
// view)
#define CT_H2_VARIANT_X(NAME, DT, WM, WN, RM, RN, KC, T, NXW)                                   \
    {NAME, DT, 32, 32, 16, WM, WN, 1, RM, RN, KC, &h2_lds_bytes<WM, WN, RM, RN, KC, T, NXW>,     \
     &h2_launch<DT, WM, WN, RM, RN, KC, T, NXW>, &h2_aux_bytes<WM, WN, RM, RN, KC, T>, 0, 0, 1}
#define CT_H2_VARIANT_T(NAME, DT, WM, WN, RM, RN, KC, T) CT_H2_VARIANT_X(NAME, DT, WM, WN, RM, RN, KC, T, 0)
#define CT_H2_VARIANT(NAME, DT, WM, WN, RM, RN, KC) CT_H2_VARIANT_T(NAME, DT, WM, WN, RM, RN, KC, 9)

const IgemmVariant kH2Variants[] = {
    CT_H2_VARIANT("h2f16_m128n256_w2x4_r2x2_kc16", DT_F16, 2, 4, 2, 2, 16),
    CT_H2_VARIANT("h2f16_m128n128_w2x2_r2x2_kc16", DT_F16, 2, 2, 2, 2, 16),
    CT_H2_VARIANT("h2f16_m128n256_w2x2_r2x4_kc16", DT_F16, 2, 2, 2, 4, 16),
    CT_H2_VARIANT("h2f16_m64n256_w1x4_r2x2_kc32", DT_F16, 1, 4, 2, 2, 32),
    CT_H2_VARIANT("h2f16_m64n256_w1x4_r2x2_kc16", DT_F16, 1, 4, 2, 2, 16),
    CT_H2_VARIANT("h2f16_m64n128_w1x2_r2x2_kc16", DT_F16, 1, 2, 2, 2, 16),
    CT_H2_VARIANT("h2bf16_m128n256_w2x4_r2x2_kc16", DT_BF16, 2, 4, 2, 2, 16),
    CT_H2_VARIANT("h2bf16_m128n128_w2x2_r2x2_kc16", DT_BF16, 2, 2, 2, 2, 16),
    // 1x1 filters (T = 1: the matrix-product view): 32 or 64 channels a stage
    CT_H2_VARIANT_T("h2f16_m128n256_w2x4_r2x2_kc64_t1", DT_F16, 2, 4, 2, 2, 64, 1),
    CT_H2_VARIANT_T("h2f16_m128n256_w2x4_r2x2_kc32_t1", DT_F16, 2, 4, 2, 2, 32, 1),
    CT_H2_VARIANT_T("h2f16_m128n128_w2x2_r2x2_kc64_t1", DT_F16, 2, 2, 2, 2, 64, 1),
    CT_H2_VARIANT_T("h2bf16_m128n256_w2x4_r2x2_kc64_t1", DT_BF16, 2, 4, 2, 2, 64, 1),
};

// the same with waves that only stage the window (the matrix waves never
// pack it), and the number of those waves: registered after every other table
const IgemmVariant kH2XVariants[] = {
    CT_H2_VARIANT_X("h2f16_m128n256_w2x4_r2x2_kc16_x2", DT_F16, 2, 4, 2, 2, 16, 9, 2),
    CT_H2_VARIANT_X("h2f16_m128n128_w2x2_r2x2_kc16_x2", DT_F16, 2, 2, 2, 2, 16, 9, 2),
    CT_H2_VARIANT_X("h2f16_m128n128_w2x2_r2x2_kc16_x1", DT_F16, 2, 2, 2, 2, 16, 9, 1),
    CT_H2_VARIANT_X("h2bf16_m128n128_w2x2_r2x2_kc16_x2", DT_BF16, 2, 2, 2, 2, 16, 9, 2),
};
const int kH2XExtraWaves[] = {2, 2, 1, 2};
static_assert(sizeof(kH2XExtraWaves) / sizeof(int) == sizeof(kH2XVariants) / sizeof(kH2XVariants[0]),
              "one wave count per variant");

}  // namespace

const IgemmVariant* igemm_f16v2_variants(int* count) {
    *count = (int)(sizeof(kH2Variants) / sizeof(kH2Variants[0]));
    return kH2Variants;
}

const IgemmVariant* igemm_f16v2x_variants(int* count, const int** extra_waves) {
    *count = (int)(sizeof(kH2XVariants) / sizeof(kH2XVariants[0]));
    *extra_waves = kH2XExtraWaves;
    return kH2XVariants;
}

}  // namespace ct
