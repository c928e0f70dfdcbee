// MFMA shrink core shared by the LoRA apply kernels and the router's first layer (both are
// row-gathered products of bf16 activations with a [rows][d] bf16 weight held transposed).
#pragma once

#include "molora_dev.h"

namespace molora {

// --------------------------------------------------------------------------------------
// shrink core
// Each step consumes 128 reduction elements: lane (row n = lane%16, group G = lane/16) reads
// 64 contiguous bytes x[row][off + 32G .. off + 32G + 31] and the same 32 elements of A^T rows
// (one row per rank column n of each 16-wide rank block).  MFMA c (c = 0..3) takes the c-th
// 8-element piece from both, so k-slot 8G+i of MFMA c is reduction index off + 32G + 8c + i
// on both operands.
template <int RB>
__device__ __forceinline__ void shrink_steps(f32x4_t (&acc)[RB], const uint16_t* __restrict__ xrow,
                                             const uint16_t* __restrict__ At, int d_in, int s0,
                                             int s1, int lane) {
  const int n = lane & 15, G = lane >> 4;
  const uint16_t* xp = xrow + G * 32;
  const uint16_t* ap = At + (size_t)n * d_in + G * 32;
  const size_t ublk = (size_t)16 * d_in;

  for (int s = s0; s < s1; ++s) {
    const int off = s * kStepK;
    u32x4_t xv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[c] = ld16(xp + off + c * 8);
    u32x4_t av[RB][4];
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) av[u][c] = ld16(ap + u * ublk + off + c * 8);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int u = 0; u < RB; ++u)
        acc[u] = mfma16x16x32(as_bf16x8(xv[c]), as_bf16x8(av[u][c]), acc[u]);
  }
}

template <int RB>
struct RedLds {
  static constexpr int RS = RB * 16 + 4;  // row stride (floats), keeps 16-byte alignment
  static constexpr int kFloats = 4 * 16 * RS;
};

// acc[u] lane (n, G) holds h[row 4G+i][rank 16u + n]; park the wave's partial in LDS.
template <int RB>
__device__ __forceinline__ void shrink_to_lds(const f32x4_t (&acc)[RB], float* red, int wave, int lane) {
  constexpr int RS = RedLds<RB>::RS;
  const int n = lane & 15, G = lane >> 4;
  float* base = red + wave * 16 * RS;
#pragma unroll
  for (int u = 0; u < RB; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) base[(4 * G + i) * RS + u * 16 + n] = acc[u][i];
}

}  // namespace molora
