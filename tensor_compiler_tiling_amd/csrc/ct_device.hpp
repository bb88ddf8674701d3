// Device-side helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ct {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum { EPI_NONE = 0, EPI_BIAS = 1, EPI_EXP_BIAS_RSQRT = 2 };

// exp(x) = 2^(x * log2 e) on the v_exp_f32 unit (2^x to about 1 ulp); the
// product x * log2 e adds a relative error of about |x| * 2^-24 * ln 2.
__device__ __forceinline__ float dev_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// 1 / sqrt(x) on v_rsq_f32 (about 1 ulp).
__device__ __forceinline__ float dev_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

template <int DT> struct Elem;
template <> struct Elem<DT_F32> {
    using T = float;
    static __device__ __forceinline__ float to_f32(T v) { return v; }
};
template <> struct Elem<DT_F16> {
    using T = _Float16;
    static __device__ __forceinline__ float to_f32(T v) { return (float)v; }
};
template <> struct Elem<DT_BF16> {
    using T = uint16_t;
    static __device__ __forceinline__ float to_f32(T v) {
        return __uint_as_float(((uint32_t)v) << 16);
    }
};

// Per-channel epilogue on an fp32 accumulator.  `r` is rsqrt(var + eps),
// precomputed once per channel by the caller for EPI_EXP_BIAS_RSQRT.
__device__ __forceinline__ float apply_epilogue(int epi, float acc, float b, float r) {
    if (epi == EPI_BIAS) return acc + b;
    if (epi == EPI_EXP_BIAS_RSQRT) return dev_exp(acc + b) * r;
    return acc;
}

}  // namespace ct
