// Per-channel broadcast [1,C,1,1] => [N,C,H,W] of exp(var[c]) (Paddle PR
// "[CINN] Add the TileBroadcastTactic for NCHW broadcast": Introduction,
// Performance Impact and Example sections).
//
// Two forms:
//  * channel-bound -- the channel index is a grid axis, so every lane loads
//    var[c] and evaluates exp once (a uniform value), then streams 16-byte
//    non-temporal stores over the contiguous H*W runs of the (n, c) rows its
//    block owns (about 32 KiB per block).  This is the PR's tactic, re-tiled
//    for 64-wide waves and 16-byte stores.
//  * flat -- all four axes fused into one index, the channel recovered per
//    element with a divide and modulo, var[c] loaded and exp evaluated per
//    element: the PR's description of the general tactic, kept as the
//    ablation baseline (same 16-byte non-temporal stores).
#include "ct_device.hpp"
#include "ct_kernels.hpp"

namespace ct {

namespace {

constexpr int kBcastThreads = 256;

typedef float vf4 __attribute__((ext_vector_type(4)));

template <int ODT> struct OutT;
template <> struct OutT<DT_F32> {
    using T = float;
    static constexpr int kVec = 4;  // elements per 16-byte store
    static __device__ __forceinline__ float4 splat(float v) { return make_float4(v, v, v, v); }
    static __device__ __forceinline__ T conv(float v) { return v; }
};
template <> struct OutT<DT_F16> {
    using T = _Float16;
    static constexpr int kVec = 8;
    static __device__ __forceinline__ float4 splat(float v) {
        _Float16 h = (_Float16)v;  // round to nearest even
        uint32_t u = (uint32_t)__builtin_bit_cast(uint16_t, h);
        uint32_t two = u | (u << 16);
        return make_float4(__uint_as_float(two), __uint_as_float(two), __uint_as_float(two),
                           __uint_as_float(two));
    }
    static __device__ __forceinline__ T conv(float v) { return (_Float16)v; }
};

// grid: (C, row_blocks) or, when swap, (row_blocks, C).  Each block writes
// rows n in [n0, n0 + rows) of channel c; a row is HW contiguous elements.
template <int ODT>
__global__ __launch_bounds__(kBcastThreads) void bcast_channel_kernel(
    const float* __restrict__ var, typename OutT<ODT>::T* __restrict__ out, int N, int C,
    int HW, int rows, int swap) {
    const int c = swap ? blockIdx.y : blockIdx.x;
    const int rb = swap ? blockIdx.x : blockIdx.y;
    const int n0 = rb * rows;
    const int n_end = min(N, n0 + rows);
    // one load and one exp per lane for the whole block
    const float4 v4 = OutT<ODT>::splat(dev_exp(var[c]));
    const vf4 v = {v4.x, v4.y, v4.z, v4.w};
    constexpr int VEC = OutT<ODT>::kVec;
    const int vpr = HW / VEC;  // 16-byte vectors per row
    const int total = (n_end - n0) * vpr;
    // vector i of the block is (row r, position q), i = r * vpr + q; every
    // thread steps i by the block size, so (r, q) advance by a fixed
    // (dr, dq) with one carry instead of a divide per store
    int r = threadIdx.x / vpr;
    int q = threadIdx.x - r * vpr;
    const int dr = kBcastThreads / vpr;
    const int dq = kBcastThreads - dr * vpr;
    for (int i = threadIdx.x; i < total; i += kBcastThreads) {
        vf4* dst = reinterpret_cast<vf4*>(out + ((long long)(n0 + r) * C + c) * HW) + q;
        // streaming store: the output is not read back by this kernel
        __builtin_nontemporal_store(v, dst);
        q += dq;
        r += dr;
        if (q >= vpr) {
            q -= vpr;
            ++r;
        }
    }
}

template <int ODT>
__global__ __launch_bounds__(kBcastThreads) void bcast_flat_kernel(
    const float* __restrict__ var, typename OutT<ODT>::T* __restrict__ out, long long total,
    int C, int HW, int vec_ok) {
    using T = typename OutT<ODT>::T;
    constexpr int VEC = OutT<ODT>::kVec;
    const long long stride = (long long)gridDim.x * kBcastThreads * VEC;
    for (long long i0 = ((long long)blockIdx.x * kBcastThreads + threadIdx.x) * VEC; i0 < total;
         i0 += stride) {
        if (vec_ok && i0 + VEC <= total) {
            T vals[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const int c = (int)(((i0 + j) / HW) % C);
                vals[j] = OutT<ODT>::conv(dev_exp(var[c]));
            }
            __builtin_nontemporal_store(*reinterpret_cast<const vf4*>(vals),
                                        reinterpret_cast<vf4*>(out + i0));
        } else {
            const long long i_end = (i0 + VEC < total) ? i0 + VEC : total;
            for (long long i = i0; i < i_end; ++i) {
                const int c = (int)((i / HW) % C);
                out[i] = OutT<ODT>::conv(dev_exp(var[c]));
            }
        }
    }
}

}  // namespace

hipError_t launch_bcast_channel(const float* var, void* out, int N, int C, int HW, int out_dtype,
                                hipStream_t stream) {
    const int esize = out_dtype == DT_F16 ? 2 : 4;
    // about 32 KiB of output per block, whole rows
    const long long row_bytes = (long long)HW * esize;
    int rows = (int)(32768 / row_bytes);
    if (rows < 1) rows = 1;
    if (rows > N) rows = N;
    const int row_blocks = (N + rows - 1) / rows;
    // blockIdx.y / z are limited to 65535 here; put the larger count on x
    const int swap = (row_blocks > 65535) ? 1 : 0;
    if ((swap ? C : row_blocks) > 65535) return hipErrorInvalidValue;
    dim3 grid = swap ? dim3(row_blocks, C) : dim3(C, row_blocks);
    if (out_dtype == DT_F16) {
        (void)hipGetLastError();
        hipLaunchKernelGGL(bcast_channel_kernel<DT_F16>, grid, dim3(kBcastThreads), 0, stream, var,
                           static_cast<_Float16*>(out), N, C, HW, rows, swap);
    } else if (out_dtype == DT_F32) {
        (void)hipGetLastError();
        hipLaunchKernelGGL(bcast_channel_kernel<DT_F32>, grid, dim3(kBcastThreads), 0, stream, var,
                           static_cast<float*>(out), N, C, HW, rows, swap);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bcast_flat(const float* var, void* out, int N, int C, int HW, int out_dtype,
                             hipStream_t stream) {
    const long long total = (long long)N * C * HW;
    const int vec = out_dtype == DT_F16 ? 8 : 4;
    long long blocks = (total + (long long)kBcastThreads * vec - 1) / ((long long)kBcastThreads * vec);
    if (blocks > 65536LL * 16) blocks = 65536LL * 16;  // grid-stride beyond this
    if (blocks < 1) blocks = 1;
    const int vec_ok = (reinterpret_cast<uintptr_t>(out) % 16) == 0 ? 1 : 0;
    if (out_dtype == DT_F16) {
        (void)hipGetLastError();
        hipLaunchKernelGGL(bcast_flat_kernel<DT_F16>, dim3((unsigned)blocks), dim3(kBcastThreads),
                           0, stream, var, static_cast<_Float16*>(out), total, C, HW, vec_ok);
    } else if (out_dtype == DT_F32) {
        (void)hipGetLastError();
        hipLaunchKernelGGL(bcast_flat_kernel<DT_F32>, dim3((unsigned)blocks), dim3(kBcastThreads),
                           0, stream, var, static_cast<float*>(out), total, C, HW, vec_ok);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ct
