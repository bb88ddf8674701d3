// Host-visible declarations shared by the C-ABI runtime and the HIP kernel
// files.  No torch types anywhere: plain pointers and sizes.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ct {

// Division by a runtime constant d (1 <= d < 2^31) with a multiply-high and a
// shift (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): q = (umulhi(n, mul) + n) >> shift, exact for every
// 32-bit n.
struct FastDiv {
    uint32_t d, mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

// Arrival counters of the split reduction sit one per 128-byte line
// (tickets[tile * kTicketStride]), so the workgroups of different tiles do
// not contend for one cache line.
constexpr int kTicketStride = 32;

// Everything a convolution launch needs, resolved on the host.
struct ConvParams {
    const void* x;
    const void* w;
    float* y;
    const float* bias;
    const float* var;
    float eps;
    int N, CI, H, W, CO, KH, KW, stride, pad, OH, OW;
    int T;          // KH * KW taps
    int K;          // CI * T, the GEMM reduction length
    long long P;    // N * OH * OW, the GEMM column count
    int OHW;        // OH * OW
    int epilogue;   // ct_epilogue
    // implicit-GEMM tiling (resolved from a ct_tile_config)
    int kc;         // input channels per LDS stage
    int stages;     // LDS stages per workgroup
    int S;          // workgroups sharing one output tile's reduction
    int tiles_m;    // ceil(CO / tile_m)
    int tiles_n;    // ceil(P / tile_n)
    int R;          // padded-input window rows held in LDS per stage
    int Hp, Wp;     // padded input height / width (H + 2 pad, W + 2 pad)
    float* ws;      // S partial tiles per output tile (S > 1 only)
    unsigned* tickets;  // one arrival counter per output tile (S > 1 only)
    const void* zero;   // >= 256 zero bytes: the source of every padded tap
    FastDiv fd_wstr, fd_rwp, fd_wp, fd_hp;  // filled by the variant's launcher
    FastDiv fd_ow, fd_t, fd_kw;
    FastDiv fd_w, fd_hw;                    // W, H*W (register-staged windows)
    void* aux;          // variant-specific scratch (a reordered filter copy), or null
    int w_prepared;     // 1: w is already in the prepared layout of the variant (prepared_filter)
};

// Static description of one compiled implicit-GEMM instantiation.
struct IgemmVariant {
    const char* name;
    int dtype;
    int mfma_m, mfma_n, mfma_k;
    int waves_m, waves_n, waves_k;
    int reps_m, reps_n;
    int kc_max;
    // LDS bytes the variant needs for this shape and tiling (p has the shape
    // plus kc, stages, S and R filled in); > 163840 means "cannot run".
    int (*lds_bytes)(const ConvParams& p);
    hipError_t (*launch)(const ConvParams& p, hipStream_t stream);
    // bytes of ConvParams::aux the launch needs (null: none); p.w may be
    // null (the legality check), then the bytes for a 16-byte aligned w
    long long (*aux_bytes)(const ConvParams& p);
    // nonzero: the variant keeps each tile's split reduction inside one XCD,
    // relying on workgroup b running on XCD b % 8; legal only where the
    // runtime has observed that placement
    int xcd_local;
    // nonzero: the width (output pixels) of the variant's column tiles, when
    // it is not waves_n * reps_n * mfma_n
    int tile_n;
    // nonzero: the launch also accepts a filter already in the prepared
    // layout (ConvParams::w_prepared), the one h2_prepare_filter writes
    int prepared_filter;
};

// Kernel-file registries.
const IgemmVariant* igemm_f32_variants(int* count);
const IgemmVariant* igemm_f32_sk_variants(int* count);
const IgemmVariant* igemm_f32_sk16_variants(int* count);
const IgemmVariant* igemm_f32_skc_variants(int* count);
const IgemmVariant* igemm_f32_skt_variants(int* count);
const IgemmVariant* igemm_f16_variants(int* count);
const IgemmVariant* igemm_f16v2_variants(int* count);
const IgemmVariant* igemm_f32_gemm_variants(int* count);
const IgemmVariant* igemm_f16_gemm_variants(int* count);

// Half-precision prepared filter: wp [CO][CI64/8][T][8] = w [CO][CI][T]
// regrouped into 16-byte records of 8 channels at one tap, zeros past CI
// (CI64 = CI rounded up to 64).
hipError_t h2_prepare_filter(const void* w, void* wp, int CO, int CI, int T, hipStream_t stream);

// Direct (one lane per output) reference kernel.
hipError_t launch_conv_direct(const ConvParams& p, int dtype, hipStream_t stream);

// Broadcast out[n][c][hw] = exp(var[c]).
//   channel-bound: grid axis over channels, rows_per_block images per block.
//   flat: fused index, value recomputed per element.
hipError_t launch_bcast_channel(const float* var, void* out, int N, int C, int HW,
                                int out_dtype, hipStream_t stream);
hipError_t launch_bcast_flat(const float* var, void* out, int N, int C, int HW,
                             int out_dtype, hipStream_t stream);

// out[b] = the XCD that workgroup b of a `blocks`-workgroup launch ran on.
hipError_t launch_xcc_probe(int* out, int blocks, hipStream_t stream);

// Deterministic device fill used by the tuner's scratch inputs:
// v[i] = lo + (hi - lo) * u(i, seed), u a counter-based hash in [0, 1).
hipError_t launch_fill_uniform(void* dst, long long n, int dtype, float lo, float hi,
                               unsigned seed, hipStream_t stream);

// dst[0..n) = v, as a kernel on `stream`.
hipError_t launch_fill_u32(unsigned* dst, long long n, unsigned v, hipStream_t stream);

// max over i of |a[i] - b[i]| / (atol + rtol * |b[i]|) > 1 ?  writes a flag.
hipError_t launch_compare(const float* a, const float* b, long long n, float atol,
                          float rtol, unsigned* bad_count, hipStream_t stream);

}  // namespace ct
