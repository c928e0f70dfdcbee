// MFMA cores shared by the LoRA apply kernels and the router's first layer.
//
// Shrink (D = x * A, rows = 16 tokens, columns = 16 ranks per block u):
//   one step consumes 128 reduction elements in 4 MFMAs (c = 0..3).  In MFMA c, k-slot 8G+i
//   (lane group G = lane/16) is reduction index 128s + 32c + 8G + i on both operands, so the
//   four lanes G of a token read 64 contiguous bytes of its x row per load instruction.
//   The A operand comes either from the hot-set slab, pre-swizzled so that the 64 lanes of a
//   wave read 1 KB contiguously per instruction, or from a row-major [rows][d] matrix (the
//   router weight W1, nn.Linear layout).
// Expand (D = h * B, rows = 16 tokens, columns = 16 output columns per MFMA j):
//   the A operand is h as a bf16 hi/lo pair stacked along k (k-slots 0..15 carry hi of ranks
//   16u + 0..15, 16..31 carry lo); the B operand is read from the slab's B^T, whose columns
//   are permuted inside each 128-column block so that MFMA j, lane n reads slab row
//   128b + 16j + n, which holds output column 128b + 8n + j.  The D fragment of lane (n, G)
//   then holds, for tokens 4G..4G+3, the 8 contiguous columns 128b + 8n .. 128b + 8n + 7:
//   a load or store instruction covers 4 token rows x 256 contiguous bytes (bf16).
#pragma once

#include "molora_dev.h"

namespace molora {

// Slab index of A element (rank j = 16u + n, reduction index 128s + 32c + 8G + i).
__host__ __device__ __forceinline__ size_t a_swz_index(int RB, int s, int c, int u, int n, int G, int i) {
  return (((((size_t)(s * 4 + c) * RB + u) * 16 + n) * 4 + G) * 8 + i);
}
// Output column held by slab row `row` of B^T (column permutation inside 128-column blocks).
__host__ __device__ __forceinline__ int b_perm_col(int row) {
  const int blk = row >> 7, w = row & 127;
  return (blk << 7) + ((w & 15) << 3) + (w >> 4);
}

template <int RB, bool SWZ>
__device__ __forceinline__ const uint16_t* a_piece(const uint16_t* A, int d, int s, int c, int u, int n, int G) {
  if constexpr (SWZ) return A + a_swz_index(RB, s, c, u, n, G, 0);
  else return A + (size_t)(u * 16 + n) * d + s * kStepK + c * 32 + G * 8;
}

// Steps per register batch: every load of a batch is issued before its MFMAs.
template <int RB>
struct ShrinkBatch {
  static constexpr int SB = RB == 1 ? 4 : 2;
};

// SB: steps whose loads are issued together (more loads in flight, more registers).
template <int RB, bool SWZ, int SB = ShrinkBatch<RB>::SB>
__device__ __forceinline__ void shrink_steps_batched(f32x4_t (&acc)[RB], const uint16_t* __restrict__ xrow,
                                                     const uint16_t* __restrict__ A, int d_in, int s0,
                                                     int s1, int lane) {
  const int n = lane & 15, G = lane >> 4;
  const uint16_t* xp = xrow + G * 8;
  for (int sb = s0; sb < s1; sb += SB) {
    const int nb = min(SB, s1 - sb);  // wave-uniform
    u32x4_t xv[SB][4];
    u32x4_t av[SB][RB][4];
    // steps past the end re-read the last step (their results are not used)
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int s = min(sb + i, s1 - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[i][c] = ld16(xp + s * kStepK + c * 32);
    }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int s = min(sb + i, s1 - 1);
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) av[i][u][c] = ld16(a_piece<RB, SWZ>(A, d_in, s, c, u, n, G));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its MFMAs
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if (i < nb) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int u = 0; u < RB; ++u)
            acc[u] = mfma16x16x32(as_bf16x8(xv[i][c]), as_bf16x8(av[i][u][c]), acc[u]);
      }
    }
  }
}

// Shrink of one token tile against up to U adapters: each batch of x steps is loaded once and
// contracted with the A of every adapter j < nU in turn (acc[j]); the A loads of one adapter
// are issued together, ahead of its MFMAs.
template <int RB, int U>
__device__ __forceinline__ void shrink_multi(f32x4_t (&acc)[U][RB], const uint16_t* __restrict__ xrow,
                                             const uint16_t* const (&At)[U], int nU, int d_in, int s0, int s1,
                                             int lane) {
  constexpr int SB = ShrinkBatch<RB>::SB;
  const int n = lane & 15, G = lane >> 4;
  const uint16_t* xp = xrow + G * 8;
  for (int sb = s0; sb < s1; sb += SB) {
    const int nb = min(SB, s1 - sb);  // wave-uniform
    u32x4_t xv[SB][4];
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int s = min(sb + i, s1 - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[i][c] = ld16(xp + s * kStepK + c * 32);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (j < nU) {
        u32x4_t av[SB][RB][4];
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const int s = min(sb + i, s1 - 1);
#pragma unroll
          for (int u = 0; u < RB; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) av[i][u][c] = ld16(a_piece<RB, true>(At[j], d_in, s, c, u, n, G));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          if (i < nb) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int u = 0; u < RB; ++u)
                acc[j][u] = mfma16x16x32(as_bf16x8(xv[i][c]), as_bf16x8(av[i][u][c]), acc[j][u]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <int RB, int NW = 4>
struct RedLds {
  static constexpr int RS = RB * 16 + 4;  // row stride (floats), keeps 16-byte alignment
  static constexpr int kFloats = NW * 16 * RS;
};

// acc[u] lane (n, G) holds h[token 4G+i][rank 16u + n]; park the wave's partial in LDS.
template <int RB, int NW = 4>
__device__ __forceinline__ void shrink_to_lds(const f32x4_t (&acc)[RB], float* red, int wave, int lane) {
  constexpr int RS = RedLds<RB, NW>::RS;
  const int n = lane & 15, G = lane >> 4;
  float* base = red + wave * 16 * RS;
#pragma unroll
  for (int u = 0; u < RB; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) base[(4 * G + i) * RS + u * 16 + n] = acc[u][i];
}

// hi/lo split of 8 fp32 values: groups G = 0, 1 carry hi = bf16(v) of ranks 16u + 8(G&1) + i,
// groups 2, 3 the remainder lo = bf16(v - hi).
__device__ __forceinline__ bf16x8_t split_hilo(const float (&v)[8], bool lo_part) {
  bf16x8_t out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 hi = (__bf16)v[i];
    out[i] = lo_part ? (__bf16)(v[i] - (float)hi) : hi;
  }
  return out;
}

// Sum the NW waves' partials of the lane's token n (fixed order), scale by wgt, split.
template <int RB, int NW>
__device__ __forceinline__ void h_operand_from_lds(bf16x8_t (&hb)[RB], const float* red, float wgt, int lane) {
  constexpr int RS = RedLds<RB, NW>::RS;
  const int n = lane & 15, G = lane >> 4;
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    const int col = u * 16 + (G & 1) * 8;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* p = red + (w * 16 + n) * RS + col;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += p[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= wgt;
    hb[u] = split_hilo(v, G >= 2);
  }
}

// Expand of one 128-column block at colbase (a multiple of 128) of the slab's B^T.  All of
// the block's B pieces are requested before the first MFMA (8 * RB loads in flight).
template <int RB>
__device__ __forceinline__ void expand_load_b(u32x4_t (&bv)[8][RB], const uint16_t* __restrict__ Bt, int r_pad,
                                              int colbase, int lane) {
  const int n = lane & 15, G = lane >> 4;
  const uint16_t* bp = Bt + (size_t)(colbase + n) * r_pad + (G & 1) * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int u = 0; u < RB; ++u) bv[j][u] = ld16(bp + (size_t)j * 16 * r_pad + u * 16);
}
template <int RB>
__device__ __forceinline__ void expand_mfma_regs(f32x4_t (&acc)[8], const bf16x8_t (&hb)[RB], const u32x4_t (&bv)[8][RB]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int u = 0; u < RB; ++u) acc[j] = mfma16x16x32(hb[u], as_bf16x8(bv[j][u]), acc[j]);
}
template <int RB>
__device__ __forceinline__ void expand_mfma(f32x4_t (&acc)[8], const bf16x8_t (&hb)[RB],
                                            const uint16_t* __restrict__ Bt, int r_pad, int colbase, int lane) {
  u32x4_t bv[8][RB];
  expand_load_b<RB>(bv, Bt, r_pad, colbase, lane);
  __builtin_amdgcn_sched_barrier(0);  // keep every load of the block ahead of the MFMAs
  expand_mfma_regs<RB>(acc, hb, bv);
}

// 8 contiguous columns (colbase + 8n ..) of the 4 token rows 4G..4G+3 of one block.
template <bool F32>
struct RowChunk;
template <>
struct RowChunk<false> {
  u32x4_t v[4];
};
template <>
struct RowChunk<true> {
  u32x4_t v[8];
};

// rows[i]: base address of token row 4G+i (bytes); colbase in elements.
template <bool F32>
__device__ __forceinline__ void load_row_chunk(RowChunk<F32>& r, const char* const (&rows)[4], int colbase, int n) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (F32) {
      const float* p = reinterpret_cast<const float*>(rows[i]) + colbase + n * 8;
      r.v[2 * i] = ld16_nt(p);
      r.v[2 * i + 1] = ld16_nt(p + 4);
    } else {
      r.v[i] = ld16_nt(reinterpret_cast<const uint16_t*>(rows[i]) + colbase + n * 8);
    }
  }
}

// y[row 4G+i][colbase + 8n + j] = y0 + acc[j][i], for the rows whose bit i is set in `valid`.
template <bool Y0F32, bool YF32>
__device__ __forceinline__ void epilogue_store(const f32x4_t (&acc)[8], const RowChunk<Y0F32>& y0c,
                                               char* const (&rows)[4], int colbase, int n, unsigned valid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!((valid >> i) & 1u)) continue;
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = acc[j][i];
    if constexpr (Y0F32) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        o[t] += __uint_as_float(y0c.v[2 * i][t]);
        o[t + 4] += __uint_as_float(y0c.v[2 * i + 1][t]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t wv = y0c.v[i][t];
        o[2 * t] += bf16_to_f32(wv & 0xffffu);
        o[2 * t + 1] += bf16_to_f32(wv >> 16);
      }
    }
    if constexpr (YF32) {
      float* p = reinterpret_cast<float*>(rows[i]) + colbase + n * 8;
      u32x4_t a, b;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = __float_as_uint(o[t]);
        b[t] = __float_as_uint(o[t + 4]);
      }
      st16_nt(p, a);
      st16_nt(p + 4, b);
    } else {
      u32x4_t a;
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = pack_bf16x2(o[2 * t], o[2 * t + 1]);
      st16_nt(reinterpret_cast<uint16_t*>(rows[i]) + colbase + n * 8, a);
    }
  }
}

}  // namespace molora
