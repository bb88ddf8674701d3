// Small device utilities: deterministic scratch fills and an on-device output
// comparison for the tile-config search, a word fill (kernel, not a memset, so
// it may sit in a captured graph), and the workgroup-placement probe.
#include "ct_device.hpp"
#include "ct_kernels.hpp"

namespace ct {

namespace {

// 32-bit finaliser of MurmurHash3 (Appleby), used as a counter-based generator.
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

template <int DT>
__global__ __launch_bounds__(256) void fill_uniform_kernel(void* dst, long long n, float lo,
                                                           float hi, uint32_t seed) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t h = mix32((uint32_t)i ^ mix32(seed ^ (uint32_t)(i >> 32)));
        const float u = (float)(h >> 8) * (1.0f / 16777216.0f);
        const float v = lo + (hi - lo) * u;
        if (DT == DT_F32) {
            static_cast<float*>(dst)[i] = v;
        } else if (DT == DT_F16) {
            static_cast<_Float16*>(dst)[i] = (_Float16)v;
        } else {
            // round to nearest even into bfloat16
            uint32_t b = __float_as_uint(v);
            b += 0x7fffu + ((b >> 16) & 1u);
            static_cast<uint16_t*>(dst)[i] = (uint16_t)(b >> 16);
        }
    }
}

__global__ __launch_bounds__(256) void compare_kernel(const float* a, const float* b, long long n,
                                                      float atol, float rtol, unsigned* bad) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    unsigned local = 0;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float d = fabsf(a[i] - b[i]);
        // NaN in either side fails (the comparison is false)
        if (!(d <= atol + rtol * fabsf(b[i]))) ++local;
    }
    if (local) atomicAdd(bad, local);
}

__global__ __launch_bounds__(256) void fill_u32_kernel(unsigned* dst, long long n, unsigned v) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = v;
}

// Which XCD (accelerator complex die) each workgroup ran on: the XCC_ID
// hardware register (id 20), bits 3:0.
__global__ __launch_bounds__(64) void xcc_probe_kernel(int* out) {
    if (threadIdx.x == 0) out[blockIdx.x] = (int)(__builtin_amdgcn_s_getreg(20 | (3 << 11)) & 15);
}

}  // namespace

hipError_t launch_xcc_probe(int* out, int blocks, hipStream_t stream) {
    if (blocks < 1) return hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(xcc_probe_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, out);
    return hipGetLastError();
}

hipError_t launch_fill_uniform(void* dst, long long n, int dtype, float lo, float hi,
                               unsigned seed, hipStream_t stream) {
    long long blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    switch (dtype) {
        case DT_F32:
            (void)hipGetLastError();
            hipLaunchKernelGGL(fill_uniform_kernel<DT_F32>, dim3((unsigned)blocks), dim3(256), 0,
                               stream, dst, n, lo, hi, seed);
            break;
        case DT_F16:
            (void)hipGetLastError();
            hipLaunchKernelGGL(fill_uniform_kernel<DT_F16>, dim3((unsigned)blocks), dim3(256), 0,
                               stream, dst, n, lo, hi, seed);
            break;
        case DT_BF16:
            (void)hipGetLastError();
            hipLaunchKernelGGL(fill_uniform_kernel<DT_BF16>, dim3((unsigned)blocks), dim3(256), 0,
                               stream, dst, n, lo, hi, seed);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fill_u32(unsigned* dst, long long n, unsigned v, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    long long blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    (void)hipGetLastError();
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, n, v);
    return hipGetLastError();
}

hipError_t launch_compare(const float* a, const float* b, long long n, float atol, float rtol,
                          unsigned* bad_count, hipStream_t stream) {
    long long blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(compare_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, b, n, atol,
                       rtol, bad_count);
    return hipGetLastError();
}

}  // namespace ct
