// Grouped LoRA application on gfx950: shrink h = x_t A_e (d_in -> r), expand
// delta = h B_e (r -> d_out), and the gate-weighted, alpha/r-scaled add into y.
//
// MoLoRA pages (thelatestinai.com): Figure 2 (tokens grouped by selected adapter, a grouped
// GEMM, outputs combined by a weighted sum), Table 10 (A is (K, d, r), B is (K, r, d)),
// Figure 4 / Table 2 (hot-set adapters at fixed addresses, direct or indirect layout),
// Figure 5 / Figure 9 (a matrix-core kernel for large batches, a skinny kernel for small ones).
//
// Kernels:
//   apply_fused_k1     one routed adapter per token: a workgroup owns 16 grouped rows of one
//                      adapter and a slice of the output columns; it gathers the 16 x rows,
//                      shrinks with MFMA (the 4 waves split d_in and meet in LDS), then
//                      streams y0 -> y for its columns with MFMA expands.  Each token is
//                      written by exactly one tile, so no combine is needed.
//   shrink_grouped     the same shrink, written as fp32 partials (optionally split over d_in)
//                      into a workspace, already multiplied by gate weight and alpha/r.
//   expand_grouped_k1  one adapter per token, expand from those partials (small batches).
//   expand_tokens      k > 1: a workgroup owns 16 consecutive tokens; for every adapter any of
//                      them uses (ascending), an MFMA expand with the other tokens' rows zeroed,
//                      summed in registers; y0 is read and y written once per token, in a fixed
//                      order, so the result is deterministic.
//   copy_unrouted      y = y0 for tokens that no adapter was applied to (out-of-place calls).
//
// The shrink result h is kept in fp32 and enters the expand MFMA as a bf16 hi/lo pair
// (h = hi + lo to about 2^-17 relative), stacked along the reduction dimension.
#include <algorithm>
#include <cstdlib>

#include "molora_launch.h"
#include "molora_mfma.h"

namespace molora {

// hi/lo split of 8 fp32 values into the expand's B operand: groups G = 0, 1 carry the bf16
// rounding hi of ranks 16u + 8(G&1) + i, groups 2, 3 the remainder lo = bf16(v - hi).
__device__ __forceinline__ bf16x8_t split_hilo(const float (&v)[8], bool lo_part) {
  bf16x8_t out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 hi = (__bf16)v[i];
    out[i] = lo_part ? (__bf16)(v[i] - (float)hi) : hi;
  }
  return out;
}

// Sum the four waves' partials of the lane's row n (fixed order), scale, split.
template <int RB>
__device__ __forceinline__ void h_operand_from_lds(bf16x8_t (&hb)[RB], const float* red, float wgt,
                                                   int lane) {
  constexpr int RS = RedLds<RB>::RS;
  const int n = lane & 15, G = lane >> 4;
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    const int col = u * 16 + (G & 1) * 8;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* p = red + (w * 16 + n) * RS + col;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += p[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= wgt;
    hb[u] = split_hilo(v, G >= 2);
  }
}

// --------------------------------------------------------------------------------------
// expand core
// Output column permutation: within a block of 128 columns at colbase, MFMA j (0..7) row m
// is column colbase + 32(j/2) + 8(m/4) + 4(j%2) + m%4.  The D fragment of lane (n, G) then
// covers, for c = 0..3, the 8 contiguous columns colbase + 32c + 8G .. +7 of token n, so the
// four lanes G = 0..3 of a token read/write 64 contiguous bytes (bf16) per c.
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

template <bool F32>
__device__ __forceinline__ void load_row_chunk(RowChunk<F32>& r, const void* row, int colbase, int G) {
  if constexpr (F32) {
    const float* p = reinterpret_cast<const float*>(row) + colbase + G * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r.v[2 * c] = ld16_nt(p + c * 32);
      r.v[2 * c + 1] = ld16_nt(p + c * 32 + 4);
    }
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + colbase + G * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c) r.v[c] = ld16_nt(p + c * 32);
  }
}

template <int RB>
__device__ __forceinline__ void expand_mfma(f32x4_t (&acc)[8], const bf16x8_t (&hb)[RB],
                                            const uint16_t* __restrict__ Bt, int r_pad, int colbase,
                                            int lane) {
  const int n = lane & 15, G = lane >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int col = colbase + (j >> 1) * 32 + (n >> 2) * 8 + (j & 1) * 4 + (n & 3);
    const uint16_t* bp = Bt + (size_t)col * r_pad + (G & 1) * 8;
#pragma unroll
    for (int u = 0; u < RB; ++u) acc[j] = mfma16x16x32(as_bf16x8(ld16(bp + u * 16)), hb[u], acc[j]);
  }
}

template <bool Y0F32, bool YF32>
__device__ __forceinline__ void epilogue_store(const f32x4_t (&acc)[8], const RowChunk<Y0F32>& y0c,
                                               void* yrow, int colbase, int G) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = acc[2 * c + (t >> 2)][t & 3];
    if constexpr (Y0F32) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        o[t] += __uint_as_float(y0c.v[2 * c][t]);
        o[t + 4] += __uint_as_float(y0c.v[2 * c + 1][t]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t wv = y0c.v[c][t];
        o[2 * t] += bf16_to_f32(wv & 0xffffu);
        o[2 * t + 1] += bf16_to_f32(wv >> 16);
      }
    }
    if constexpr (YF32) {
      float* p = reinterpret_cast<float*>(yrow) + colbase + c * 32 + G * 8;
      u32x4_t a, b;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = __float_as_uint(o[t]);
        b[t] = __float_as_uint(o[t + 4]);
      }
      st16_nt(p, a);
      st16_nt(p + 4, b);
    } else {
      uint16_t* p = reinterpret_cast<uint16_t*>(yrow) + colbase + c * 32 + G * 8;
      u32x4_t a;
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = pack_bf16x2(o[2 * t], o[2 * t + 1]);
      st16_nt(p, a);
    }
  }
}

// --------------------------------------------------------------------------------------
// y = y0 for rows no tile writes (k = 1, out of place).  Token t is unrouted iff inv[t] < 0.
template <bool Y0F32, bool YF32>
__device__ void copy_unrouted(const void* y0, void* y, const int32_t* __restrict__ inv, int N,
                              int d_out, int cb, int ncb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = (cb * 4 + wave) * kWave; base < N; base += ncb * 4 * kWave) {
    const int t = base + lane;
    uint64_t m = __ballot(t < N && inv[t] < 0);
    while (m) {
      const int tt = base + __builtin_ctzll(m);
      m &= m - 1;
      for (int c = lane * 4; c < d_out; c += kWave * 4) {
        float v[4];
        if constexpr (Y0F32) {
          const float* p = reinterpret_cast<const float*>(y0) + (size_t)tt * d_out + c;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = p[i];
        } else {
          const uint16_t* p = reinterpret_cast<const uint16_t*>(y0) + (size_t)tt * d_out + c;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = bf16_to_f32(p[i]);
        }
        if constexpr (YF32) {
          float* p = reinterpret_cast<float*>(y) + (size_t)tt * d_out + c;
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = v[i];
        } else {
          uint32_t* p = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(y) + (size_t)tt * d_out + c);
          p[0] = pack_bf16x2(v[0], v[1]);
          p[1] = pack_bf16x2(v[2], v[3]);
        }
      }
    }
  }
}

// --------------------------------------------------------------------------------------
struct FusedArgs {
  TargetDev tgt;
  const uint16_t* x;
  const void* y0;
  void* y;
  const int32_t* offsets;
  const int32_t* perm;
  const float* perm_w;
  const int32_t* inv;
  int N, K;
  float scale;
  int col_groups;     // output-column slices per tile
  int tiles_per_xcd;  // tile slots per XCD (grid main part = 8 * tiles_per_xcd * col_groups)
  int copy_blocks;    // trailing blocks that copy unrouted rows (0 when in place)
};

// Block b -> (XCD b%8, slot b/8).  Slots of one XCD enumerate (tile, column group) with the
// column group fastest, so the col_groups workgroups of a tile run back to back on the same
// XCD and share its L2 for the gathered x rows.
template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(256) void apply_fused_k1(FusedArgs a) {
  __shared__ float red[RedLds<RB>::kFloats];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int main_blocks = 8 * a.tiles_per_xcd * a.col_groups;
  if (b >= main_blocks) {
    copy_unrouted<Y0F32, YF32>(a.y0, a.y, a.inv, a.N, a.tgt.d_out, b - main_blocks, a.copy_blocks);
    return;
  }
  const int xcd = b & 7, slot = b >> 3;
  const int g = slot % a.col_groups;
  const int T = (slot / a.col_groups) * 8 + xcd;
  int e, row0, nrows;
  if (!find_tile(a.offsets, a.K, T, lane, e, row0, nrows)) return;
  const int n = lane & 15, G = lane >> 4;
  const bool valid = n < nrows;
  const int q = row0 + (valid ? n : 0);
  const int tok = a.perm[q];
  const float wgt = valid ? a.perm_w[q] * a.scale : 0.f;
  const uint16_t* At = adapter_A<INDIRECT>(a.tgt, e);
  const uint16_t* Bt = adapter_B<INDIRECT>(a.tgt, e);
  const int d_in = a.tgt.d_in, d_out = a.tgt.d_out;
  const int cols = d_out / a.col_groups;
  const int c0 = g * cols;
  const int nblk = cols / kColBlock;
  const char* y0row = reinterpret_cast<const char*>(a.y0) + (size_t)tok * d_out * (Y0F32 ? 4 : 2);
  char* yrow = reinterpret_cast<char*>(a.y) + (size_t)tok * d_out * (YF32 ? 4 : 2);

  // y0 of the first block is independent of the shrink: start fetching it now.
  RowChunk<Y0F32> cur;
  int blk = wave;
  if (blk < nblk) load_row_chunk<Y0F32>(cur, y0row, c0 + blk * kColBlock, G);

  f32x4_t acc[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int S = d_in / kStepK;
  shrink_steps<RB>(acc, a.x + (size_t)tok * d_in, At, d_in, (S * wave) / 4, (S * (wave + 1)) / 4, lane);
  shrink_to_lds<RB>(acc, red, wave, lane);
  __syncthreads();
  bf16x8_t hb[RB];
  h_operand_from_lds<RB>(hb, red, wgt, lane);

  for (; blk < nblk; blk += 4) {
    RowChunk<Y0F32> nxt;
    const int nb = blk + 4;
    if (nb < nblk) load_row_chunk<Y0F32>(nxt, y0row, c0 + nb * kColBlock, G);
    f32x4_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    expand_mfma<RB>(o, hb, Bt, a.tgt.r_pad, c0 + blk * kColBlock, lane);
    if (valid) epilogue_store<Y0F32, YF32>(o, cur, yrow, c0 + blk * kColBlock, G);
    cur = nxt;
  }
}

// --------------------------------------------------------------------------------------
struct ShrinkArgs {
  TargetDev tgt;
  const uint16_t* x;
  const int32_t* offsets;
  const int32_t* perm;
  const float* perm_w;
  int K, k;
  float scale;
  float* hpart;     // [nsplit][P][r_pad] fp32, row q = grouped position
  long long P;      // rows per split slice
  int nsplit;
};

// grid (tile slots, nsplit).  Writes perm_w * scale * (partial h) for valid rows only.
template <int RB, bool INDIRECT>
__global__ __launch_bounds__(256) void shrink_grouped(ShrinkArgs a) {
  __shared__ float red[RedLds<RB>::kFloats];
  constexpr int RS = RedLds<RB>::RS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = blockIdx.x, sp = blockIdx.y;
  int e, row0, nrows;
  if (!find_tile(a.offsets, a.K, T, lane, e, row0, nrows)) return;
  const int n = lane & 15, G = lane >> 4;
  const bool valid = n < nrows;
  const int q = row0 + (valid ? n : 0);
  const int tok = a.perm[q] / a.k;
  const uint16_t* At = adapter_A<INDIRECT>(a.tgt, e);
  const int d_in = a.tgt.d_in;
  const int S = d_in / kStepK;
  const int sa = (S * sp) / a.nsplit, sb = (S * (sp + 1)) / a.nsplit;
  const int len = sb - sa;
  f32x4_t acc[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  shrink_steps<RB>(acc, a.x + (size_t)tok * d_in, At, d_in, sa + (len * wave) / 4,
                   sa + (len * (wave + 1)) / 4, lane);
  shrink_to_lds<RB>(acc, red, wave, lane);
  __syncthreads();
  // lane (n, G) writes ranks [G * RB * 4, (G + 1) * RB * 4) of row n
  if (valid) {
    const float wgt = a.perm_w[q] * a.scale;
    float* dst = a.hpart + ((long long)sp * a.P + q) * (RB * 16) + G * RB * 4;
#pragma unroll
    for (int i = 0; i < RB * 4; i += 4) {
      u32x4_t v;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int col = G * RB * 4 + i + t;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) s += red[(w * 16 + n) * RS + col];
        v[t] = __float_as_uint(s * wgt);
      }
      st16(dst + i, v);
    }
  }
}

// Sum the nsplit partials of grouped row q for the lane's rank pieces and split hi/lo.
template <int RB>
__device__ __forceinline__ void h_operand_from_ws(bf16x8_t (&hb)[RB], const float* __restrict__ hpart,
                                                  long long P, int nsplit, int q, bool valid, int lane) {
  const int G = lane >> 4;
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
    if (valid) {
      for (int sp = 0; sp < nsplit; ++sp) {
        const float* p = hpart + ((long long)sp * P + q) * (RB * 16) + u * 16 + (G & 1) * 8;
        const u32x4_t a = ld16(p), b = ld16(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] += __uint_as_float(a[i]);
          v[i + 4] += __uint_as_float(b[i]);
        }
      }
    }
    hb[u] = split_hilo(v, G >= 2);
  }
}

struct ExpandArgs {
  TargetDev tgt;
  const void* y0;
  void* y;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* inv;
  const float* hpart;
  long long P;
  int nsplit;
  int N, K, k;
  int col_groups;
  int copy_blocks;
  int main_blocks;
};

// k = 1, small batches: grid = tile slots * col_groups (+ copy blocks).
template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(256) void expand_grouped_k1(ExpandArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  if (b >= a.main_blocks) {
    copy_unrouted<Y0F32, YF32>(a.y0, a.y, a.inv, a.N, a.tgt.d_out, b - a.main_blocks, a.copy_blocks);
    return;
  }
  const int g = b % a.col_groups, T = b / a.col_groups;
  int e, row0, nrows;
  if (!find_tile(a.offsets, a.K, T, lane, e, row0, nrows)) return;
  const int n = lane & 15, G = lane >> 4;
  const bool valid = n < nrows;
  const int q = row0 + (valid ? n : 0);
  const int tok = a.perm[q];
  const uint16_t* Bt = adapter_B<INDIRECT>(a.tgt, e);
  const int d_out = a.tgt.d_out;
  const int cols = d_out / a.col_groups;
  const int c0 = g * cols;
  const int nblk = cols / kColBlock;
  const char* y0row = reinterpret_cast<const char*>(a.y0) + (size_t)tok * d_out * (Y0F32 ? 4 : 2);
  char* yrow = reinterpret_cast<char*>(a.y) + (size_t)tok * d_out * (YF32 ? 4 : 2);
  bf16x8_t hb[RB];
  h_operand_from_ws<RB>(hb, a.hpart, a.P, a.nsplit, q, valid, lane);
  for (int blk = wave; blk < nblk; blk += 4) {
    RowChunk<Y0F32> cur;
    load_row_chunk<Y0F32>(cur, y0row, c0 + blk * kColBlock, G);
    f32x4_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    expand_mfma<RB>(o, hb, Bt, a.tgt.r_pad, c0 + blk * kColBlock, lane);
    if (valid) epilogue_store<Y0F32, YF32>(o, cur, yrow, c0 + blk * kColBlock, G);
  }
}

// k > 1: grid = ceil(N/16) token tiles * col_groups.  KMAX bounds k (register arrays).
template <int RB, int KMAX, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(256) void expand_tokens(ExpandArgs a) {
  __shared__ int offs[65];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x <= a.K) offs[threadIdx.x] = a.offsets[threadIdx.x];
  __syncthreads();
  const int g = blockIdx.x % a.col_groups, tt = blockIdx.x / a.col_groups;
  const int n = lane & 15, G = lane >> 4;
  const int t0 = tt * 16;
  const int tok = t0 + n;
  const bool valid = tok < a.N;
  const int tokc = valid ? tok : t0;
  // the token's slots: grouped position and adapter, and its h operand per slot
  int es[KMAX];
  bf16x8_t hs[KMAX][RB];
  uint64_t mine = 0;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    es[s] = -1;
    int q = -1;
    if (s < a.k && valid) q = a.inv[(long long)tokc * a.k + s];
    if (q >= 0) {
      es[s] = segment_of(offs, a.K, q);
      mine |= 1ull << es[s];
    }
    h_operand_from_ws<RB>(hs[s], a.hpart, a.P, a.nsplit, q < 0 ? 0 : q, q >= 0, lane);
  }
  // adapters used by any token of the tile (every wave of the block computes the same set)
  uint64_t used = mine;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)used, d, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(used >> 32), d, kWave);
    used |= ((uint64_t)hi << 32) | lo;
  }
  const int d_out = a.tgt.d_out;
  const int cols = d_out / a.col_groups;
  const int c0 = g * cols;
  const int nblk = cols / kColBlock;
  const char* y0row = reinterpret_cast<const char*>(a.y0) + (size_t)tokc * d_out * (Y0F32 ? 4 : 2);
  char* yrow = reinterpret_cast<char*>(a.y) + (size_t)tokc * d_out * (YF32 ? 4 : 2);
  for (int blk = wave; blk < nblk; blk += 4) {
    RowChunk<Y0F32> cur;
    load_row_chunk<Y0F32>(cur, y0row, c0 + blk * kColBlock, G);
    f32x4_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint64_t rem = used;
    while (rem) {
      const int e = __builtin_ctzll(rem);
      rem &= rem - 1;
      bf16x8_t hb[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) hb[u] = bf16x8_t{};
#pragma unroll
      for (int s = 0; s < KMAX; ++s)
        if (es[s] == e) {
#pragma unroll
          for (int u = 0; u < RB; ++u) hb[u] = hs[s][u];
        }
      expand_mfma<RB>(o, hb, adapter_B<INDIRECT>(a.tgt, e), a.tgt.r_pad, c0 + blk * kColBlock, lane);
    }
    if (valid) epilogue_store<Y0F32, YF32>(o, cur, yrow, c0 + blk * kColBlock, G);
  }
}

// --------------------------------------------------------------------------------------
// host side

int apply_resolve_path(int N, int k, int path) {
  if (path != 0) return path;
  const long long P = (long long)N * k;
  if (k == 1) return P >= 192 ? 1 : 2;
  return P >= 1024 ? 1 : 2;
}

static int skinny_splits(int d_in) {
  const int S = d_in / kStepK;  // steps of 128
  int ns = S / 4;               // 512 reduction elements per split
  if (ns < 1) ns = 1;
  if (ns > 16) ns = 16;
  return ns;
}

size_t apply_ws_bytes(int N, int k, int r_pad, int d_in, int path) {
  const int p = apply_resolve_path(N, k, path);
  if (k == 1 && p == 1) return 0;
  const int ns = (p == 2) ? skinny_splits(d_in) : 1;
  return (size_t)ns * (size_t)N * (size_t)k * (size_t)r_pad * sizeof(float);
}

static int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

// Column groups: enough workgroups to cover the chip (about two per CU) while every wave
// keeps at least one 128-column block.
static int choose_col_groups(long long tiles, int d_out, int target_blocks) {
  const int nblk = d_out / kColBlock;
  int c = 1;
  while (tiles * c < target_blocks && nblk % (2 * c) == 0 && nblk / (2 * c) >= 4) c *= 2;
  return c;
}

template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_fused_t(const FusedArgs& fa, int grid, hipStream_t s) {
  hipLaunchKernelGGL((apply_fused_k1<RB, IND, Y0F, YF>), dim3(grid), dim3(256), 0, s, fa);
  return hipGetLastError();
}
template <int RB, bool IND>
static hipError_t launch_shrink_t(const ShrinkArgs& sa, int tiles, hipStream_t s) {
  hipLaunchKernelGGL((shrink_grouped<RB, IND>), dim3(tiles, sa.nsplit), dim3(256), 0, s, sa);
  return hipGetLastError();
}
template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_expand_k1_t(const ExpandArgs& ea, int grid, hipStream_t s) {
  hipLaunchKernelGGL((expand_grouped_k1<RB, IND, Y0F, YF>), dim3(grid), dim3(256), 0, s, ea);
  return hipGetLastError();
}
template <int RB, int KM, bool IND, bool Y0F, bool YF>
static hipError_t launch_expand_tok_t(const ExpandArgs& ea, int grid, hipStream_t s) {
  hipLaunchKernelGGL((expand_tokens<RB, KM, IND, Y0F, YF>), dim3(grid), dim3(256), 0, s, ea);
  return hipGetLastError();
}

// Dispatch a runtime (RB, indirect, y0 f32, y f32) to the template instance.
#define MOLORA_DISPATCH_RB(RBV, ...)                                     \
  switch (RBV) {                                                         \
    case 1: { constexpr int RB = 1; __VA_ARGS__; } break;                \
    case 2: { constexpr int RB = 2; __VA_ARGS__; } break;                \
    case 3: { constexpr int RB = 3; __VA_ARGS__; } break;                \
    case 4: { constexpr int RB = 4; __VA_ARGS__; } break;                \
    default: return hipErrorInvalidValue;                                \
  }
#define MOLORA_DISPATCH_BOOL(V, NAME, ...) \
  if (V) { constexpr bool NAME = true; __VA_ARGS__; } else { constexpr bool NAME = false; __VA_ARGS__; }

hipError_t launch_apply(const ApplyLaunch& a, hipStream_t s) {
  const long long P = (long long)a.N * a.k;
  const int RBv = a.tgt.r_pad / 16;
  const long long tiles = P / kTileRows + a.K + 1;  // upper bound on tiles of any grouping
  const bool in_place = (a.y0 == a.y);
  const int copy_blocks = in_place ? 0 : (int)std::min<long long>((a.N + 255) / 256, 64);
  hipError_t err = hipSuccess;

  if (a.k == 1 && a.path == 1) {
    FusedArgs fa;
    fa.tgt = a.tgt; fa.x = a.x; fa.y0 = a.y0; fa.y = a.y;
    fa.offsets = a.offsets; fa.perm = a.perm; fa.perm_w = a.perm_w; fa.inv = a.inv;
    fa.N = a.N; fa.K = a.K; fa.scale = a.scale;
    int cg = a.col_groups > 0 ? a.col_groups : env_int("MOLORA_APPLY_COLGROUPS", 0);
    if (cg <= 0 || (a.tgt.d_out / kColBlock) % cg != 0) cg = choose_col_groups(tiles, a.tgt.d_out, 512);
    fa.col_groups = cg;
    fa.tiles_per_xcd = (int)((tiles + 7) / 8);
    fa.copy_blocks = copy_blocks;
    const int grid = 8 * fa.tiles_per_xcd * cg + copy_blocks;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_fused_t<RB, IND, Y0F, YF>(fa, grid, s))))));
    return err;
  }

  // two-kernel paths: grouped shrink into the workspace, then an expand
  const int nsplit = (a.path == 2) ? skinny_splits(a.tgt.d_in) : 1;
  ShrinkArgs sa;
  sa.tgt = a.tgt; sa.x = a.x; sa.offsets = a.offsets; sa.perm = a.perm; sa.perm_w = a.perm_w;
  sa.K = a.K; sa.k = a.k; sa.scale = a.scale; sa.hpart = a.ws; sa.P = P; sa.nsplit = nsplit;
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND,
      err = (launch_shrink_t<RB, IND>(sa, (int)tiles, s))));
  if (err != hipSuccess) return err;

  ExpandArgs ea;
  ea.tgt = a.tgt; ea.y0 = a.y0; ea.y = a.y; ea.offsets = a.offsets; ea.perm = a.perm; ea.inv = a.inv;
  ea.hpart = a.ws; ea.P = P; ea.nsplit = nsplit; ea.N = a.N; ea.K = a.K; ea.k = a.k;
  ea.copy_blocks = copy_blocks;
  if (a.k == 1) {
    const int cg = choose_col_groups(tiles, a.tgt.d_out, 512);
    ea.col_groups = cg;
    ea.main_blocks = (int)tiles * cg;
    const int grid = ea.main_blocks + copy_blocks;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_expand_k1_t<RB, IND, Y0F, YF>(ea, grid, s))))));
    return err;
  }
  const long long ttiles = (a.N + 15) / 16;
  const int cg = choose_col_groups(ttiles, a.tgt.d_out, 512);
  ea.col_groups = cg;
  ea.main_blocks = (int)(ttiles * cg);
  ea.copy_blocks = 0;  // every token is visited
  const int grid = ea.main_blocks;
#define MOLORA_TOK(KM)                                                                                  \
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,      \
      MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_expand_tok_t<RB, KM, IND, Y0F, YF>(ea, grid, s))))))
  if (a.k <= 2) { MOLORA_TOK(2) }
  else if (a.k <= 4) { MOLORA_TOK(4) }
  else { MOLORA_TOK(8) }
#undef MOLORA_TOK
  return err;
}

// --------------------------------------------------------------------------------------
// hot-set relayout: A [d_in][r] -> A^T [r_pad][d_in]; B [r][d_out] -> B^T [d_out][r_pad];
// rank padding rows/columns are zero.
__global__ void relayout_A(const uint16_t* __restrict__ A, uint16_t* __restrict__ At, int d_in, int r,
                           int r_pad) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)r_pad * d_in) return;
  const int j = (int)(i / d_in), c = (int)(i % d_in);
  At[i] = (j < r) ? A[(long long)c * r + j] : (uint16_t)0;
}
__global__ void relayout_B(const uint16_t* __restrict__ B, uint16_t* __restrict__ Bt, int d_out, int r,
                           int r_pad) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)d_out * r_pad) return;
  const int c = (int)(i / r_pad), j = (int)(i % r_pad);
  Bt[i] = (j < r) ? B[(long long)j * d_out + c] : (uint16_t)0;
}

hipError_t launch_relayout(const uint16_t* A, const uint16_t* B, int d_in, int d_out, int r, int r_pad,
                           uint16_t* At, uint16_t* Bt, hipStream_t s) {
  const long long na = (long long)r_pad * d_in, nb = (long long)d_out * r_pad;
  hipLaunchKernelGGL(relayout_A, dim3((unsigned)((na + 255) / 256)), dim3(256), 0, s, A, At, d_in, r, r_pad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(relayout_B, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, B, Bt, d_out, r, r_pad);
  return hipGetLastError();
}

// --------------------------------------------------------------------------------------
// per-sequence comparator metadata: pass e routes every token to e with weight [idx[t] == e].
__global__ void seqpass_meta(const int32_t* __restrict__ idx, int N, int K, int32_t* __restrict__ offsets,
                             int32_t* __restrict__ perm, float* __restrict__ perm_w) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) perm[i] = (int32_t)i;
  if (i < (long long)K * (K + 1)) {
    const int e = (int)(i / (K + 1)), j = (int)(i % (K + 1));
    offsets[i] = (j <= e) ? 0 : N;
  }
  if (i < (long long)K * N) {
    const int e = (int)(i / N), t = (int)(i % N);
    perm_w[i] = (idx[t] == e) ? 1.0f : 0.0f;
  }
}

hipError_t launch_seqpass_meta(const int32_t* idx, int N, int K, int32_t* offsets, int32_t* perm,
                               float* perm_w, hipStream_t s) {
  long long n = (long long)K * N;
  if (n < (long long)K * (K + 1)) n = (long long)K * (K + 1);
  hipLaunchKernelGGL(seqpass_meta, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, N, K, offsets,
                     perm, perm_w);
  return hipGetLastError();
}

}  // namespace molora
