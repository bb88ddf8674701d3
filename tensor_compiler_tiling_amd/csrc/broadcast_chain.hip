// General per-channel broadcast [1,P,1] => [B,P,B] with a chain of
// elementwise operations (Paddle PR "[CINN] Add the TileBroadcastTactic for
// NCHW broadcast": the Introduction's axis-fusion form, where the preserved
// axis P sits between fused broadcast axes and the last axis is a broadcast
// axis, and Performance Impact's div / exp / rsqrt chains).
//
// The output is [outer][P][inner] (inner contiguous).  A program of three
// chains of at most 8 steps is evaluated per output element:
//   c0 = chain 0 (immediates, per-channel arrays a_k[p])
//   c1 = chain 1 (the same, and c0)
//   v  = chain 2 (the same, c0, c1, and x[o][p][i], the producer's element)
//   out[o][p][i] = v  (or c0 when chain 2 is empty)
//
// Two forms, both evaluating every step with the same device code (no FMA
// contraction anywhere in this file), so they give identical bits:
//  * channel-bound -- p is a grid axis; c0 and c1 are evaluated once per
//    lane for the whole block (uniform values), and each element only runs
//    chain 2, four 16-byte vectors of x a lane at a time (loads issued
//    together, each step decoded once for all their elements);
//  * flat -- one fused index; p recovered per element, all three chains
//    evaluated per element (the PR's picture of the general tactic, kept as
//    the fallback: any shape, any alignment).
#include "ct_device.hpp"
#include "../../include/convtile.h"

#include <hip/hip_runtime.h>

#include <cstring>

#pragma clang fp contract(off)

namespace ct {

namespace {

constexpr int kChainThreads = 256;

struct ChainArgs {
    ct_bcast_program prog;
    const float* a[4];
    const float* x;      // producer's fp32 output, or null when no step reads it
    void* out;
    long long outer;
    long long inner;
    int P;
    int rows;            // channel-bound: (o) rows of `inner` elements a block owns
    int swap;            // channel-bound: grid axes swapped (P on y)
    int vec_ok;          // flat: out (and x) 16-byte aligned
};

// One chain, steps in order from v = 0.
__device__ __forceinline__ float run_chain(const ChainArgs& g, int c, float x, float c0, float c1, int p) {
    float v = 0.0f;
    const int n = g.prog.n_ops[c];
    for (int k = 0; k < n; ++k) {
        const ct_chain_op o = g.prog.ops[c][k];
        float a;
        switch (o.src) {
            case CT_SRC_IMM: a = o.imm; break;
            case CT_SRC_X: a = x; break;
            case CT_SRC_C0: a = c0; break;
            case CT_SRC_C1: a = c1; break;
            default: a = g.a[o.src - CT_SRC_A0][p]; break;
        }
        switch (o.op) {
            case CT_OP_SET: v = a; break;
            case CT_OP_ADD: v = v + a; break;
            case CT_OP_SUB: v = v - a; break;
            case CT_OP_MUL: v = v * a; break;
            case CT_OP_DIV: v = v / a; break;
            case CT_OP_RSUB: v = a - v; break;
            case CT_OP_RDIV: v = a / v; break;
            case CT_OP_EXP: v = dev_exp(v); break;
            case CT_OP_RSQRT: v = dev_rsqrt(v); break;
            default: v = __builtin_sqrtf(v); break;
        }
    }
    return v;
}

__device__ __forceinline__ float element(const ChainArgs& g, float x, float c0, float c1, int p) {
    return g.prog.n_ops[2] > 0 ? run_chain(g, 2, x, c0, c1, p) : c0;
}

// Chain 2 on M elements of one channel at once: each step is decoded once
// and applied to all M (the same operations per element as run_chain, so
// the same bits).
template <int M>
__device__ __forceinline__ void element_m(const ChainArgs& g, float (&v)[M], const float (&x)[M], float c0, float c1,
                                          int p) {
    const int n = g.prog.n_ops[2];
    if (n == 0) {
#pragma unroll
        for (int j = 0; j < M; ++j) v[j] = c0;
        return;
    }
#pragma unroll
    for (int j = 0; j < M; ++j) v[j] = 0.0f;
    for (int k = 0; k < n; ++k) {
        const ct_chain_op o = g.prog.ops[2][k];
        const bool ax = o.src == CT_SRC_X;
        float a = 0.0f;
        switch (o.src) {
            case CT_SRC_IMM: a = o.imm; break;
            case CT_SRC_X: break;
            case CT_SRC_C0: a = c0; break;
            case CT_SRC_C1: a = c1; break;
            default: a = g.a[o.src - CT_SRC_A0][p]; break;
        }
        switch (o.op) {
#define CT_STEP(expr)                                                   \
    _Pragma("unroll") for (int j = 0; j < M; ++j) {                     \
        const float aj = ax ? x[j] : a;                                 \
        (void)aj;                                                       \
        v[j] = (expr);                                                  \
    }                                                                   \
    break;
            case CT_OP_SET: CT_STEP(aj)
            case CT_OP_ADD: CT_STEP(v[j] + aj)
            case CT_OP_SUB: CT_STEP(v[j] - aj)
            case CT_OP_MUL: CT_STEP(v[j] * aj)
            case CT_OP_DIV: CT_STEP(v[j] / aj)
            case CT_OP_RSUB: CT_STEP(aj - v[j])
            case CT_OP_RDIV: CT_STEP(aj / v[j])
            case CT_OP_EXP: CT_STEP(dev_exp(v[j]))
            case CT_OP_RSQRT: CT_STEP(dev_rsqrt(v[j]))
            default: CT_STEP(__builtin_sqrtf(v[j]))
#undef CT_STEP
        }
    }
}

template <int ODT> struct ChainOut;
template <> struct ChainOut<DT_F32> {
    using T = float;
    static constexpr int kVec = 4;
};
template <> struct ChainOut<DT_F16> {
    using T = _Float16;
    static constexpr int kVec = 8;
};

typedef float cvf4 __attribute__((ext_vector_type(4)));

// grid (P, row blocks) or, swapped, (row blocks, P).  A block owns rows
// [o0, o0 + rows) of channel p; a row is `inner` contiguous elements, a
// multiple of the vector width (checked by the host).
template <int ODT, bool HASX>
__global__ __launch_bounds__(kChainThreads) void chain_channel_kernel(ChainArgs g) {
    using T = typename ChainOut<ODT>::T;
    constexpr int VEC = ChainOut<ODT>::kVec;
    const int p = g.swap ? blockIdx.y : blockIdx.x;
    const long long rb = g.swap ? blockIdx.x : blockIdx.y;
    const long long o0 = rb * g.rows;
    const long long o_end = min(g.outer, o0 + g.rows);
    // the channel values: once per lane for the whole block
    const float c0 = run_chain(g, 0, 0.0f, 0.0f, 0.0f, p);
    const float c1 = run_chain(g, 1, 0.0f, c0, 0.0f, p);
    const float cst = HASX ? 0.0f : element(g, 0.0f, c0, c1, p);  // no element input: one value
    const long long vpr = g.inner / VEC;
    const long long total = (o_end - o0) * vpr;
    // U vectors a lane per round: all their loads go out before any is used
    constexpr int U = 4;
    for (long long i0 = threadIdx.x; i0 < total; i0 += U * kChainThreads) {
        long long base[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long i = min(i0 + (long long)u * kChainThreads, total - 1);  // in bounds; not stored
            const long long r = i / vpr;
            base[u] = ((o0 + r) * g.P + p) * g.inner + (i - r * vpr) * VEC;
        }
        float v[U * VEC];
        if constexpr (HASX) {
            float xin[U * VEC];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const cvf4* xs = reinterpret_cast<const cvf4*>(g.x + base[u]);
#pragma unroll
                for (int h = 0; h < VEC / 4; ++h) {
                    const cvf4 xv = __builtin_nontemporal_load(xs + h);
#pragma unroll
                    for (int j = 0; j < 4; ++j) xin[u * VEC + 4 * h + j] = xv[j];
                }
            }
            element_m<U * VEC>(g, v, xin, c0, c1, p);
        } else {
#pragma unroll
            for (int j = 0; j < U * VEC; ++j) v[j] = cst;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + (long long)u * kChainThreads < total) {
                T o[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) o[j] = (T)v[u * VEC + j];
                __builtin_nontemporal_store(*reinterpret_cast<const cvf4*>(o),
                                            reinterpret_cast<cvf4*>(static_cast<T*>(g.out) + base[u]));
            }
        }
    }
}

template <int ODT, bool HASX>
__global__ __launch_bounds__(kChainThreads) void chain_flat_kernel(ChainArgs g) {
    using T = typename ChainOut<ODT>::T;
    constexpr int VEC = ChainOut<ODT>::kVec;
    const long long total = g.outer * g.P * g.inner;
    const long long stride = (long long)gridDim.x * kChainThreads * VEC;
    T* out = static_cast<T*>(g.out);
    for (long long i0 = ((long long)blockIdx.x * kChainThreads + threadIdx.x) * VEC; i0 < total;
         i0 += stride) {
        const long long i_end = i0 + VEC < total ? i0 + VEC : total;
        T o[VEC];
        for (long long i = i0; i < i_end; ++i) {
            const int p = (int)((i / g.inner) % g.P);
            const float c0 = run_chain(g, 0, 0.0f, 0.0f, 0.0f, p);
            const float c1 = run_chain(g, 1, 0.0f, c0, 0.0f, p);
            const float x = HASX ? g.x[i] : 0.0f;
            o[i - i0] = (T)element(g, x, c0, c1, p);
        }
        if (g.vec_ok && i_end - i0 == VEC) {
            __builtin_nontemporal_store(*reinterpret_cast<const cvf4*>(o), reinterpret_cast<cvf4*>(out + i0));
        } else {
            for (long long i = i0; i < i_end; ++i) out[i] = o[i - i0];
        }
    }
}

template <int ODT, bool HASX>
hipError_t launch_chain(const ChainArgs& g, bool channel, hipStream_t stream) {
    (void)hipGetLastError();
    if (channel) {
        const long long row_blocks = (g.outer + g.rows - 1) / g.rows;
        const dim3 grid = g.swap ? dim3((unsigned)row_blocks, (unsigned)g.P) : dim3((unsigned)g.P, (unsigned)row_blocks);
        hipLaunchKernelGGL((chain_channel_kernel<ODT, HASX>), grid, dim3(kChainThreads), 0, stream, g);
    } else {
        constexpr int VEC = ChainOut<ODT>::kVec;
        const long long total = g.outer * g.P * g.inner;
        long long blocks = (total + (long long)kChainThreads * VEC - 1) / ((long long)kChainThreads * VEC);
        if (blocks > 65536LL * 16) blocks = 65536LL * 16;  // grid-stride beyond this
        if (blocks < 1) blocks = 1;
        hipLaunchKernelGGL((chain_flat_kernel<ODT, HASX>), dim3((unsigned)blocks), dim3(kChainThreads), 0, stream, g);
    }
    return hipGetLastError();
}

// Channel-bound rows per block: about 32 KiB of output, whole rows.
long long chain_rows(long long outer, long long inner, int out_dtype) {
    long long rows = 32768 / (inner * (out_dtype == DT_F16 ? 2 : 4));
    if (rows < 1) rows = 1;
    if (rows > outer) rows = outer;
    return rows;
}

}  // namespace

// The tactic rule: channel-bound when every row of `inner` elements is a
// whole number of 16-byte vectors of out (and of x when it is read), both
// 16-byte aligned, inner is at least 32 (a row keeps a wave busy), and the
// (P, row blocks) grid fits (65535 on its second axis); otherwise flat.
bool chain_channel_ok(long long outer, int P, long long inner, int out_dtype, const void* out, const void* x) {
    const int vec = out_dtype == DT_F16 ? 8 : 4;
    if (inner < 32 || inner % vec != 0) return false;
    if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return false;
    if (x && reinterpret_cast<uintptr_t>(x) % 16 != 0) return false;
    const long long rows = chain_rows(outer, inner, out_dtype);
    const long long row_blocks = (outer + rows - 1) / rows;
    const bool swap = row_blocks > 65535;
    if ((swap ? (long long)P : row_blocks) > 65535) return false;
    if (swap && row_blocks > 0x7fffffffLL) return false;
    return true;
}

// Arguments are checked by the caller; `channel` is the chosen form, which
// the caller has checked with chain_channel_ok.  `x` is null when no step
// reads the producer's element.
hipError_t launch_broadcast_chain(const ct_bcast_program* prog, const float* const a[4], const float* x, void* out,
                                  int out_dtype, long long outer, int P, long long inner, bool channel,
                                  hipStream_t stream) {
    ChainArgs g{};
    std::memcpy(&g.prog, prog, sizeof(ct_bcast_program));
    for (int k = 0; k < 4; ++k) g.a[k] = a[k];
    g.x = x;
    g.out = out;
    g.outer = outer;
    g.P = P;
    g.inner = inner;
    const long long rows = chain_rows(outer, inner, out_dtype);
    g.rows = (int)rows;
    g.swap = (outer + rows - 1) / rows > 65535 ? 1 : 0;
    g.vec_ok = (reinterpret_cast<uintptr_t>(out) % 16 == 0) ? 1 : 0;
    const bool hasx = x != nullptr;
    if (out_dtype == DT_F32)
        return hasx ? launch_chain<DT_F32, true>(g, channel, stream) : launch_chain<DT_F32, false>(g, channel, stream);
    if (out_dtype == DT_F16)
        return hasx ? launch_chain<DT_F16, true>(g, channel, stream) : launch_chain<DT_F16, false>(g, channel, stream);
    return hipErrorInvalidValue;
}

}  // namespace ct
