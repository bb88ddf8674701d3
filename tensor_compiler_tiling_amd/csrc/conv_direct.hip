// Direct convolution: one lane per output element, fp32 fused multiply-add
// over the taps in the definition's order (c, ky, kx), zero padding applied
// inline while reading (TVM tutorial "Tuning High Performance Convolution on
// NVIDIA GPUs", Step 1: the conv2d_nchw compute with inlined padding).
//
// This is the slow, simple kernel: the on-device reference the tile-config
// search checks every candidate against, and the fallback for shapes no
// tiled variant accepts.
#include "ct_device.hpp"
#include "ct_kernels.hpp"

namespace ct {

template <int DT>
__global__ __launch_bounds__(256) void conv_direct_kernel(ConvParams p) {
    using T = typename Elem<DT>::T;
    const long long total = p.P * (long long)p.CO;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int ox = (int)(idx % p.OW);
    long long t = idx / p.OW;
    const int oy = (int)(t % p.OH);
    t /= p.OH;
    const int f = (int)(t % p.CO);
    const int n = (int)(t / p.CO);

    const T* x = static_cast<const T*>(p.x);
    const T* w = static_cast<const T*>(p.w);
    const T* xn = x + (long long)n * p.CI * p.H * p.W;
    const T* wf = w + (long long)f * p.K;
    float acc = 0.0f;
    for (int c = 0; c < p.CI; ++c) {
        const T* xc = xn + (long long)c * p.H * p.W;
        const T* wc = wf + c * p.T;
        for (int ky = 0; ky < p.KH; ++ky) {
            const int iy = oy * p.stride + ky - p.pad;
            const bool row_ok = (iy >= 0) && (iy < p.H);
            for (int kx = 0; kx < p.KW; ++kx) {
                const int ix = ox * p.stride + kx - p.pad;
                float xv = 0.0f;
                if (row_ok && ix >= 0 && ix < p.W) xv = Elem<DT>::to_f32(xc[iy * p.W + ix]);
                acc = __builtin_fmaf(xv, Elem<DT>::to_f32(wc[ky * p.KW + kx]), acc);
            }
        }
    }
    float b = 0.0f, r = 1.0f;
    if (p.epilogue != EPI_NONE) b = p.bias[f];
    if (p.epilogue == EPI_EXP_BIAS_RSQRT) r = dev_rsqrt(p.var[f] + p.eps);
    p.y[idx] = apply_epilogue(p.epilogue, acc, b, r);
}

hipError_t launch_conv_direct(const ConvParams& p, int dtype, hipStream_t stream) {
    const long long total = p.P * (long long)p.CO;
    const int block = 256;
    const long long grid = (total + block - 1) / block;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    switch (dtype) {
        case DT_F32:
            (void)hipGetLastError();
            hipLaunchKernelGGL(conv_direct_kernel<DT_F32>, dim3((unsigned)grid), dim3(block), 0,
                               stream, p);
            break;
        case DT_F16:
            (void)hipGetLastError();
            hipLaunchKernelGGL(conv_direct_kernel<DT_F16>, dim3((unsigned)grid), dim3(block), 0,
                               stream, p);
            break;
        case DT_BF16:
            (void)hipGetLastError();
            hipLaunchKernelGGL(conv_direct_kernel<DT_BF16>, dim3((unsigned)grid), dim3(block), 0,
                               stream, p);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ct
