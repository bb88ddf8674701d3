// Shared pieces of the implicit-GEMM convolution kernels.
//
// GEMM view of the convolution (TVM tutorial "Tuning High Performance
// Convolution on NVIDIA GPUs", Step 1 -- output axes f, y, x and reduction
// axes rc, ry, rx of conv2d_nchw):
//   Y[CO x P] = W[CO x K] * Xcol[K x P],  K = CI*KH*KW,  P = N*OH*OW
//   Xcol[(c,ky,kx)][(n,oy,ox)] = xp[n][c][oy*s+ky][ox*s+kx]  (never stored)
//
// The template's tiling levels map onto the MI355X this way:
//   output axes    block      -> workgroup tile (tile_m x tile_n), grid axis
//                  vthread    -> MFMA tiles repeated per wave (reps_m, reps_n)
//                  thread     -> waves per workgroup (waves_m, waves_n)
//                  inner      -> the matrix-core instruction's own tile
//   reduction rc   outer      -> split across workgroups (split_k, new here)
//                  middle     -> LDS stage loop (stages)
//                  inner      -> channels per LDS stage (kc), all taps inside;
//                                within a stage the waves_k waves interleave
//                                over the instruction K steps
//   "shared" cache -> LDS tiles of W and of a padded-input window
//   "local" cache  -> VGPR operand fragments and accumulators
//
// Padded-input window.  Images are stacked along rows in a virtual padded
// tensor of N*Hp rows (Hp = H + 2 pad) and Wp = W + 2 pad columns; output
// (n, oy, ox) reads virtual rows n*Hp + oy*s + ky and columns ox*s + kx.
// A workgroup's output columns are a contiguous range of P, so the rows it
// reads form one contiguous range of virtual rows: that range (R rows, full
// padded width, kc channels) is one LDS stage.  Rows that fall in padding or
// past the last image are written as zeros, so padding is applied inline.
#pragma once

#include <cstddef>

#include "ct_kernels.hpp"

namespace ct {

// Kernel arguments arrive in a buffer no cache holds yet.  Left alone, the
// compiler loads the fields of ConvParams in several batches where they are
// first needed, and each batch that touches a new 64-byte line is a full
// memory round trip (about a microsecond).  Naming one field of every line at
// kernel entry makes the first batch bring in all five lines together; later
// loads of any field then hit the scalar cache.
static_assert(sizeof(ConvParams) <= 320, "ConvParams spans more than five 64-byte lines");
static_assert(offsetof(ConvParams, x) < 64 && offsetof(ConvParams, KH) / 64 == 1 &&
                  offsetof(ConvParams, tiles_n) / 64 == 2 && offsetof(ConvParams, fd_wp) / 64 == 3 &&
                  offsetof(ConvParams, fd_hw) / 64 == 4,
              "one touched field per 64-byte line of ConvParams");
__device__ __forceinline__ void fetch_kernargs(const ConvParams& p) {
    asm volatile("" ::"s"(p.x), "s"(p.KH), "s"(p.tiles_n), "s"(p.fd_wp.d), "s"(p.fd_hw.d));
}

// Round up to a multiple.
__host__ __device__ inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Number of window rows a tile of columns [p0, p1) needs.
__host__ __device__ inline long long window_rows_for(long long p0, long long p1, int OHW, int OW,
                                                     int Hp, int stride, int KH) {
    const long long nA = p0 / OHW, nB = (p1 - 1) / OHW;
    const long long oyA = (p0 % OHW) / OW, oyB = ((p1 - 1) % OHW) / OW;
    const long long vrA = nA * Hp + oyA * stride, vrB = nB * Hp + oyB * stride;
    return vrB - vrA + KH;
}

}  // namespace ct
