// Grouped LoRA application on gfx950: shrink h = x_t A_e (d_in -> r), expand
// delta = h B_e (r -> d_out), and the gate-weighted, alpha/r-scaled add into y.
//
// MoLoRA pages (thelatestinai.com): Figure 2 (tokens grouped by selected adapter, a grouped
// GEMM, outputs combined by a weighted sum), Table 10 (A is (K, d, r), B is (K, r, d)),
// Figure 4 / Table 2 (hot-set adapters at fixed addresses, direct or indirect layout),
// Figure 5 / Figure 9 (a matrix-core kernel for large batches, a skinny kernel for small ones).
//
// Kernels:
//   apply_tile         token-major tiles with grouping inside the tile (any k, K <= 16): a
//                      workgroup owns 16 consecutive tokens and a slice of output columns;
//                      its x / y0 / y rows depend only on the token index, so those streams
//                      start as soon as the (small) routing loads are done; for every adapter
//                      used in the tile (ascending) one MFMA shrink over the 16 rows and one
//                      masked MFMA expand, summed in registers; y is written once.
//   apply_fused_k1     globally grouped tiles, one adapter per token: a workgroup owns 16
//                      grouped rows of one adapter (gathered through perm) and a slice of the
//                      output columns; shrink and expand fused; each token written once.
//   shrink_grouped     the grouped shrink into an fp32 workspace (weighted by gate and
//                      alpha/r), optionally split over d_in (the skinny path), for
//   expand_grouped_k1  (one adapter per token) and
//   expand_tokens      (k > 1: token-major, every adapter of the tile, fixed order).
//   copy_unrouted      y = y0 for tokens that no adapter was applied to (out-of-place calls).
//
// The shrink result h stays fp32 and enters the expand MFMA as a bf16 hi/lo pair
// (h = hi + lo to about 2^-17 relative).  Workgroups that share x rows are numbered so that
// they run back to back on the same XCD (block b runs on XCD b % 8) and share its L2.
#include <algorithm>
#include <cstdlib>

#include "dispatch_dev.h"
#include "molora_launch.h"
#include "molora_mfma.h"

namespace molora {

constexpr int kWaves8 = 8;    // waves per workgroup of the fused kernels
constexpr int kPrefetch = 2;  // expand blocks per wave whose y0 is requested up front
constexpr int kTileMaxU = kApplyTileMaxAdapters;

// Rows of tokens 4G..4G+3 of a tile, given the token held by each lane n < 16.
template <typename P>
__device__ __forceinline__ void tile_rows(P base, size_t row_bytes, int tok_of_lane, int G, P (&rows)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = __shfl(tok_of_lane, 4 * G + i, kWave);
    rows[i] = base + (size_t)t * row_bytes;
  }
}

// --------------------------------------------------------------------------------------
// y = y0 for rows no tile writes (k = 1, out of place).  Token t is unrouted iff inv[t] < 0.
template <bool Y0F32, bool YF32, int NW>
__device__ void copy_unrouted(const void* y0, void* y, const int32_t* __restrict__ inv, int N, int d_out, int cb,
                              int ncb) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int base = (cb * NW + wave) * kWave; base < N; base += ncb * NW * kWave) {
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
// Tile-local grouping (token-major), any k, K <= 16.
struct TileArgs {
  TargetDev tgt;
  const uint16_t* x;
  const void* y0;
  void* y;
  const int32_t* offsets;
  const float* perm_w;
  const int32_t* inv;
  int N, K, k;
  float scale;
  int col_groups;
  int tiles;          // token tiles (ceil(N / 16))
  int tiles_per_xcd;  // grid = 8 * tiles_per_xcd * col_groups
};

template <int RB>
struct TileGroup {
  static constexpr int UP = RB == 1 ? 4 : (RB == 2 ? 2 : 1);  // adapters per shrink group
};

template <int RB>
struct TileLds {
  float red[TileGroup<RB>::UP * RedLds<RB, kWaves8>::kFloats];  // the waves' partials of one adapter group
  u32x4_t hbl[kTileMaxU * 16 * RB * 4];                         // per used adapter: [token][u][G] operand
};

// Body of one tile workgroup, given the token slots of this lane's token (adapter es[s] and
// gate weight times alpha/r ws[s]; es = -1 for none).  Every thread of the workgroup calls it.
template <int RB, int KMAX, bool INDIRECT, bool Y0F32, bool YF32>
__device__ __forceinline__ void tile_body(const TileArgs& a, TileLds<RB>& L, int tt, int g, const int (&es)[KMAX],
                                          const float (&ws)[KMAX]) {
  constexpr int NW = kWaves8;
  constexpr int PF = kPrefetch;
  constexpr int UP = TileGroup<RB>::UP;
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int t0 = tt * 16;
  const int tok = t0 + n;
  const int tokc = tok < a.N ? tok : a.N - 1;
  const int d_in = a.tgt.d_in, d_out = a.tgt.d_out;
  const int cols = d_out / a.col_groups;
  const int c0 = g * cols;
  const int nblk = cols / kColBlock;

  uint64_t mine = 0;
#pragma unroll
  for (int s = 0; s < KMAX; ++s)
    if (es[s] >= 0) mine |= 1ull << es[s];
  uint64_t used = mine;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)used, d, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(used >> 32), d, kWave);
    used |= ((uint64_t)hi << 32) | lo;
  }
  const int nU = __popcll(used);

  // y0 rows of the first output blocks
  const char* y0rows[4];
  char* yrows[4];
  unsigned vmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * G + i;
    const int tc = t < a.N ? t : a.N - 1;
    vmask |= (t < a.N ? 1u : 0u) << i;
    y0rows[i] = reinterpret_cast<const char*>(a.y0) + (size_t)tc * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(a.y) + (size_t)tc * d_out * yb;
  }
  RowChunk<Y0F32> y0c[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int blk = wave + i * NW;
    if (blk < nblk) load_row_chunk<Y0F32>(y0c[i], y0rows, c0 + blk * kColBlock, n);
  }

  // shrink in groups of UP used adapters (ascending): x is loaded once per group and contracted
  // with each adapter's A; the waves' partials meet in LDS and wave j reduces group slot j into
  // that adapter's expand operand in hbl
  const int S = d_in / kStepK;
  const int s0 = (S * wave) / NW, s1 = (S * (wave + 1)) / NW;
  uint64_t rem = used;
  for (int base = 0; base < nU; base += UP) {
    const int nP = min(UP, nU - base);
    int eu[UP];
    const uint16_t* At[UP];
#pragma unroll
    for (int j = 0; j < UP; ++j) {
      eu[j] = -1;
      At[j] = a.tgt.At;  // never read for j >= nP
      if (j < nP) {
        eu[j] = __builtin_ctzll(rem);
        rem &= rem - 1;
        At[j] = adapter_A<INDIRECT>(a.tgt, eu[j]);
      }
    }
    f32x4_t acc[UP][RB];
#pragma unroll
    for (int j = 0; j < UP; ++j)
#pragma unroll
      for (int u = 0; u < RB; ++u) acc[j][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    shrink_multi<RB, UP>(acc, a.x + (size_t)tokc * d_in, At, nP, d_in, s0, s1, lane);
#pragma unroll
    for (int j = 0; j < UP; ++j)
      if (j < nP) shrink_to_lds<RB, NW>(acc[j], L.red + j * RedLds<RB, NW>::kFloats, wave, lane);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < UP; ++j) {
      if (j < nP && j == wave) {
        float wt = 0.f;
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
          if (es[s] == eu[j]) wt += ws[s];
        bf16x8_t hb[RB];
        h_operand_from_lds<RB, NW>(hb, L.red + j * RedLds<RB, NW>::kFloats, wt, lane);
#pragma unroll
        for (int u = 0; u < RB; ++u)
          L.hbl[(((base + j) * 16 + n) * RB + u) * 4 + G] = __builtin_bit_cast(u32x4_t, hb[u]);
      }
    }
    __syncthreads();  // hbl of the group complete; red free for the next group
  }

  // expand: every used adapter accumulated in registers, then y = y0 + acc
  for (int r0 = 0; wave + r0 * NW < nblk; r0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int blk = wave + (r0 + i) * NW;
      if (blk < nblk) {
        f32x4_t o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        uint64_t r2 = used;
        for (int sl = 0; sl < nU; ++sl) {
          const int e = __builtin_ctzll(r2);
          r2 &= r2 - 1;
          bf16x8_t hb[RB];
#pragma unroll
          for (int u = 0; u < RB; ++u) hb[u] = __builtin_bit_cast(bf16x8_t, L.hbl[((sl * 16 + n) * RB + u) * 4 + G]);
          expand_mfma<RB>(o, hb, adapter_B<INDIRECT>(a.tgt, e), a.tgt.r_pad, c0 + blk * kColBlock, lane);
        }
        epilogue_store<Y0F32, YF32>(o, y0c[i], yrows, c0 + blk * kColBlock, n, vmask);
      }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int blk = wave + (r0 + PF + i) * NW;
      if (blk < nblk) load_row_chunk<Y0F32>(y0c[i], y0rows, c0 + blk * kColBlock, n);
    }
  }
}

// Block b runs on XCD b % 8; slots of one XCD enumerate (tile, column group), column group
// fastest, so the column groups of a tile run back to back on one XCD and share its L2.
__device__ __forceinline__ void tile_of_block(int b, int col_groups, int& tt, int& g) {
  const int xcd = b & 7, slot = b >> 3;
  g = slot % col_groups;
  tt = (slot / col_groups) * 8 + xcd;
}

template <int RB, int KMAX, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kWaves8 * 64) void apply_tile(TileArgs a) {
  __shared__ TileLds<RB> L;
  __shared__ int offs[65];
  int tt, g;
  tile_of_block(blockIdx.x, a.col_groups, tt, g);
  if (tt >= a.tiles) return;
  const int lane = threadIdx.x & 63, n = lane & 15;
  const int tok = tt * 16 + n;
  const bool valid = tok < a.N;
  // routing of the tile's tokens (small loads, done before the large streams start)
  if (threadIdx.x <= a.K) offs[threadIdx.x] = a.offsets[threadIdx.x];
  __syncthreads();
  int es[KMAX];
  float ws[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    es[s] = -1;
    ws[s] = 0.f;
    if (s < a.k && valid) {
      const int q = a.inv[(long long)tok * a.k + s];
      if (q >= 0) {
        es[s] = segment_of(offs, a.K, q);
        ws[s] = a.perm_w[q] * a.scale;
      }
    }
  }
  tile_body<RB, KMAX, INDIRECT, Y0F32, YF32>(a, L, tt, g, es, ws);
}

// --------------------------------------------------------------------------------------
// One launch of the vocabulary-routed step (k = 1): workgroup 0 routes every token, writes
// idx / w and runs the stable counting sort (dispatch_block) before its own tile; every tile
// workgroup routes its 16 tokens from their ids with the same range lookup, so the apply never
// waits for the dispatch and no workgroup waits for another.
constexpr int kStepDispatchThreads = kWaves8 * 64;

struct StepArgs {
  TileArgs t;
  VocabBounds bounds;
  const int32_t* ids;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  float* perm_w;
  int32_t* inv;
};

struct VocabSource {
  const int32_t* ids;
  const int* bl;
  int K;
  __device__ __forceinline__ void operator()(int p, int& e, float& wv) const {
    e = vocab_owner(ids[p], bl, K);
    wv = (e >= 0) ? 1.0f : 0.0f;
  }
};

template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kWaves8 * 64) void step_vocab(StepArgs a) {
  __shared__ TileLds<RB> L;
  __shared__ DispatchLds<kStepDispatchThreads> DL;
  __shared__ int bl[65];
  const int K = a.t.K, N = a.t.N;
  bounds_to_lds(a.bounds, bl, K);
  __syncthreads();
  if (blockIdx.x == 0) {
    const VocabSource src{a.ids, bl, K};
    for (int t = threadIdx.x; t < N; t += kStepDispatchThreads) {
      int e;
      float wv;
      src(t, e, wv);
      a.idx[t] = e;
      a.w[t] = wv;
    }
    dispatch_block<kStepDispatchThreads>(DL, src, N, K, a.counts, a.offsets, a.perm, a.perm_w, a.inv);
  }
  int tt, g;
  tile_of_block(blockIdx.x, a.t.col_groups, tt, g);
  if (tt >= a.t.tiles) return;
  const int n = threadIdx.x & 15;
  const int tok = tt * 16 + n;
  int es[1] = {-1};
  float ws[1] = {0.f};
  if (tok < N) {
    es[0] = vocab_owner(a.ids[tok], bl, K);
    ws[0] = (es[0] >= 0) ? 1.0f * a.t.scale : 0.f;
  }
  tile_body<RB, 1, INDIRECT, Y0F32, YF32>(a.t, L, tt, g, es, ws);
}

// --------------------------------------------------------------------------------------
// Globally grouped tiles, one adapter per token.
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

template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kWaves8 * 64) void apply_fused_k1(FusedArgs a) {
  constexpr int NW = kWaves8;
  constexpr int PF = kPrefetch;
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  __shared__ float red[RedLds<RB, NW>::kFloats];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int main_blocks = 8 * a.tiles_per_xcd * a.col_groups;
  if (b >= main_blocks) {
    copy_unrouted<Y0F32, YF32, NW>(a.y0, a.y, a.inv, a.N, a.tgt.d_out, b - main_blocks, a.copy_blocks);
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
  const char* y0rows[4];
  char* yrows[4];
  tile_rows<const char*>(reinterpret_cast<const char*>(a.y0), (size_t)d_out * y0b, tok, G, y0rows);
  tile_rows<char*>(reinterpret_cast<char*>(a.y), (size_t)d_out * yb, tok, G, yrows);
  unsigned vmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) vmask |= ((4 * G + i) < nrows ? 1u : 0u) << i;

  RowChunk<Y0F32> y0c[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int blk = wave + i * NW;
    if (blk < nblk) load_row_chunk<Y0F32>(y0c[i], y0rows, c0 + blk * kColBlock, n);
  }
  f32x4_t acc[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int S = d_in / kStepK;
  shrink_steps_batched<RB, true>(acc, a.x + (size_t)tok * d_in, At, d_in, (S * wave) / NW, (S * (wave + 1)) / NW,
                                 lane);
  shrink_to_lds<RB, NW>(acc, red, wave, lane);
  __syncthreads();
  bf16x8_t hb[RB];
  h_operand_from_lds<RB, NW>(hb, red, wgt, lane);

  for (int r0 = 0; wave + r0 * NW < nblk; r0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int blk = wave + (r0 + i) * NW;
      if (blk < nblk) {
        f32x4_t o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        expand_mfma<RB>(o, hb, Bt, a.tgt.r_pad, c0 + blk * kColBlock, lane);
        epilogue_store<Y0F32, YF32>(o, y0c[i], yrows, c0 + blk * kColBlock, n, vmask);
      }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int blk = wave + (r0 + PF + i) * NW;
      if (blk < nblk) load_row_chunk<Y0F32>(y0c[i], y0rows, c0 + blk * kColBlock, n);
    }
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
  float* hpart;  // [nsplit][P][r_pad] fp32, row q = grouped position
  long long P;   // rows per split slice
  int nsplit;
};

// grid (tile slots, nsplit).  Writes perm_w * scale * (partial h) for valid rows only.
template <int RB, bool INDIRECT>
__global__ __launch_bounds__(256) void shrink_grouped(ShrinkArgs a) {
  __shared__ float red[RedLds<RB>::kFloats];
  constexpr int RS = RedLds<RB>::RS;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  shrink_steps_batched<RB, true>(acc, a.x + (size_t)tok * d_in, At, d_in, sa + (len * wave) / 4,
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
__device__ __forceinline__ void h_operand_from_ws(bf16x8_t (&hb)[RB], const float* __restrict__ hpart, long long P,
                                                  int nsplit, int q, bool valid, int lane) {
  const int G = lane >> 4;
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
    if (valid) {
      for (int sp = 0; sp < nsplit; ++sp) {
        const float* p = hpart + ((long long)sp * P + q) * (RB * 16) + u * 16 + (G & 1) * 8;
        const u32x4_t x0 = ld16(p), x1 = ld16(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] += __uint_as_float(x0[i]);
          v[i + 4] += __uint_as_float(x1[i]);
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
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  if (b >= a.main_blocks) {
    copy_unrouted<Y0F32, YF32, 4>(a.y0, a.y, a.inv, a.N, a.tgt.d_out, b - a.main_blocks, a.copy_blocks);
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
  const char* y0rows[4];
  char* yrows[4];
  tile_rows<const char*>(reinterpret_cast<const char*>(a.y0), (size_t)d_out * y0b, tok, G, y0rows);
  tile_rows<char*>(reinterpret_cast<char*>(a.y), (size_t)d_out * yb, tok, G, yrows);
  unsigned vmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) vmask |= ((4 * G + i) < nrows ? 1u : 0u) << i;
  bf16x8_t hb[RB];
  h_operand_from_ws<RB>(hb, a.hpart, a.P, a.nsplit, q, valid, lane);
  for (int blk = wave; blk < nblk; blk += 4) {
    RowChunk<Y0F32> cur;
    load_row_chunk<Y0F32>(cur, y0rows, c0 + blk * kColBlock, n);
    f32x4_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    expand_mfma<RB>(o, hb, Bt, a.tgt.r_pad, c0 + blk * kColBlock, lane);
    epilogue_store<Y0F32, YF32>(o, cur, yrows, c0 + blk * kColBlock, n, vmask);
  }
}

// k > 1: grid = ceil(N/16) token tiles * col_groups.  KMAX bounds k (register arrays).
template <int RB, int KMAX, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(256) void expand_tokens(ExpandArgs a) {
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  __shared__ int offs[65];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x <= a.K) offs[threadIdx.x] = a.offsets[threadIdx.x];
  __syncthreads();
  const int g = blockIdx.x % a.col_groups, tt = blockIdx.x / a.col_groups;
  const int n = lane & 15, G = lane >> 4;
  const int t0 = tt * 16;
  const int tok = t0 + n;
  const bool valid = tok < a.N;
  const int tokc = valid ? tok : a.N - 1;
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
  const char* y0rows[4];
  char* yrows[4];
  unsigned vmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * G + i;
    const int tc = t < a.N ? t : a.N - 1;
    vmask |= (t < a.N ? 1u : 0u) << i;
    y0rows[i] = reinterpret_cast<const char*>(a.y0) + (size_t)tc * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(a.y) + (size_t)tc * d_out * yb;
  }
  for (int blk = wave; blk < nblk; blk += 4) {
    RowChunk<Y0F32> cur;
    load_row_chunk<Y0F32>(cur, y0rows, c0 + blk * kColBlock, n);
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
    epilogue_store<Y0F32, YF32>(o, cur, yrows, c0 + blk * kColBlock, n, vmask);
  }
}

// --------------------------------------------------------------------------------------
// host side

int apply_resolve_path(int N, int k, int path, int K, int r_pad) {
  if (path != 0) return path;
  const long long P = (long long)N * k;
  if (K <= kTileMaxU && r_pad <= 32 && P >= 192) return 3;  // few, small adapters: tile-local grouping
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

size_t apply_ws_bytes(int N, int k, int K, int r_pad, int d_in, int path) {
  const int p = apply_resolve_path(N, k, path, K, r_pad);
  if (p == 3 || (k == 1 && p == 1)) return 0;
  const int ns = (p == 2) ? skinny_splits(d_in) : 1;
  return (size_t)ns * (size_t)N * (size_t)k * (size_t)r_pad * sizeof(float);
}

static int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

// Column groups: enough workgroups to cover the chip while every wave keeps output blocks.
static int choose_col_groups(long long tiles, int d_out, int target_blocks, int min_blocks_per_group) {
  const int nblk = d_out / kColBlock;
  int c = 1;
  while (tiles * c < target_blocks && nblk % (2 * c) == 0 && nblk / (2 * c) >= min_blocks_per_group) c *= 2;
  return c;
}

static int col_groups_for(int requested, long long tiles, int d_out, int target, int minb) {
  int cg = requested > 0 ? requested : env_int("MOLORA_APPLY_COLGROUPS", 0);
  if (cg <= 0 || (d_out / kColBlock) % cg != 0) cg = choose_col_groups(tiles, d_out, target, minb);
  return cg;
}

static TileArgs tile_args(const ApplyLaunch& a) {
  TileArgs ta;
  ta.tgt = a.tgt; ta.x = a.x; ta.y0 = a.y0; ta.y = a.y; ta.offsets = a.offsets; ta.perm_w = a.perm_w;
  ta.inv = a.inv; ta.N = a.N; ta.K = a.K; ta.k = a.k; ta.scale = a.scale;
  ta.tiles = (a.N + 15) / 16;
  ta.col_groups = col_groups_for(a.col_groups, ta.tiles, a.tgt.d_out, 256, kWaves8);
  ta.tiles_per_xcd = (ta.tiles + 7) / 8;
  return ta;
}

template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_fused_t(const FusedArgs& fa, int grid, hipStream_t s) {
  hipLaunchKernelGGL((apply_fused_k1<RB, IND, Y0F, YF>), dim3(grid), dim3(kWaves8 * 64), 0, s, fa);
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
static hipError_t launch_tile_t(const TileArgs& ta, int grid, hipStream_t s) {
  hipLaunchKernelGGL((apply_tile<RB, KM, IND, Y0F, YF>), dim3(grid), dim3(kWaves8 * 64), 0, s, ta);
  return hipGetLastError();
}
template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_step_t(const StepArgs& sa, int grid, hipStream_t s) {
  hipLaunchKernelGGL((step_vocab<RB, IND, Y0F, YF>), dim3(grid), dim3(kWaves8 * 64), 0, s, sa);
  return hipGetLastError();
}
template <int RB, int KM, bool IND, bool Y0F, bool YF>
static hipError_t launch_expand_tok_t(const ExpandArgs& ea, int grid, hipStream_t s) {
  hipLaunchKernelGGL((expand_tokens<RB, KM, IND, Y0F, YF>), dim3(grid), dim3(256), 0, s, ea);
  return hipGetLastError();
}

// Runtime (RB, indirect, y0 f32, y f32) -> template instance.
#define MOLORA_DISPATCH_RB(RBV, ...)                      \
  switch (RBV) {                                          \
    case 1: { constexpr int RB = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int RB = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int RB = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int RB = 4; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                 \
  }
#define MOLORA_DISPATCH_BOOL(V, NAME, ...) \
  if (V) { constexpr bool NAME = true; __VA_ARGS__; } else { constexpr bool NAME = false; __VA_ARGS__; }

hipError_t launch_apply(const ApplyLaunch& a, hipStream_t s) {
  const long long P = (long long)a.N * a.k;
  const int RBv = a.tgt.r_pad / 16;
  const long long tiles = P / kTileRows + a.K + 1;  // upper bound on tiles of any grouping
  const bool in_place = (a.y0 == a.y);
  hipError_t err = hipSuccess;

  if (a.path == 3) {
    const TileArgs ta = tile_args(a);
    const int grid = 8 * ta.tiles_per_xcd * ta.col_groups;
#define MOLORA_TILE(KM)                                                                                \
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,  \
      MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_tile_t<RB, KM, IND, Y0F, YF>(ta, grid, s))))))
    if (a.k == 1) { MOLORA_TILE(1) }
    else if (a.k <= 2) { MOLORA_TILE(2) }
    else if (a.k <= 4) { MOLORA_TILE(4) }
    else { MOLORA_TILE(8) }
#undef MOLORA_TILE
    return err;
  }

  if (a.k == 1 && a.path == 1) {
    FusedArgs fa;
    fa.tgt = a.tgt; fa.x = a.x; fa.y0 = a.y0; fa.y = a.y;
    fa.offsets = a.offsets; fa.perm = a.perm; fa.perm_w = a.perm_w; fa.inv = a.inv;
    fa.N = a.N; fa.K = a.K; fa.scale = a.scale;
    fa.col_groups = col_groups_for(a.col_groups, tiles, a.tgt.d_out, 256, kWaves8);
    fa.tiles_per_xcd = (int)((tiles + 7) / 8);
    fa.copy_blocks = in_place ? 0 : (int)std::min<long long>((a.N + 511) / 512, 64);
    const int grid = 8 * fa.tiles_per_xcd * fa.col_groups + fa.copy_blocks;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_fused_t<RB, IND, Y0F, YF>(fa, grid, s))))));
    return err;
  }

  // two-kernel paths: grouped shrink into the workspace, then an expand
  const int nsplit = (a.path == 2) ? skinny_splits(a.tgt.d_in) : 1;
  ShrinkArgs sa;
  sa.tgt = a.tgt; sa.x = a.x; sa.offsets = a.offsets; sa.perm = a.perm; sa.perm_w = a.perm_w;
  sa.K = a.K; sa.k = a.k; sa.scale = a.scale; sa.hpart = a.ws; sa.P = P; sa.nsplit = nsplit;
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, err = (launch_shrink_t<RB, IND>(sa, (int)tiles, s))));
  if (err != hipSuccess) return err;

  ExpandArgs ea;
  ea.tgt = a.tgt; ea.y0 = a.y0; ea.y = a.y; ea.offsets = a.offsets; ea.perm = a.perm; ea.inv = a.inv;
  ea.hpart = a.ws; ea.P = P; ea.nsplit = nsplit; ea.N = a.N; ea.K = a.K; ea.k = a.k;
  if (a.k == 1) {
    ea.col_groups = choose_col_groups(tiles, a.tgt.d_out, 512, 4);
    ea.main_blocks = (int)tiles * ea.col_groups;
    ea.copy_blocks = in_place ? 0 : (int)std::min<long long>((a.N + 255) / 256, 64);
    const int grid = ea.main_blocks + ea.copy_blocks;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_expand_k1_t<RB, IND, Y0F, YF>(ea, grid, s))))));
    return err;
  }
  const long long ttiles = (a.N + 15) / 16;
  ea.col_groups = choose_col_groups(ttiles, a.tgt.d_out, 512, 4);
  ea.main_blocks = (int)(ttiles * ea.col_groups);
  ea.copy_blocks = 0;  // every token is visited
  const int grid = ea.main_blocks;
#define MOLORA_TOK(KM)                                                                                \
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,  \
      MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_expand_tok_t<RB, KM, IND, Y0F, YF>(ea, grid, s))))))
  if (a.k <= 2) { MOLORA_TOK(2) }
  else if (a.k <= 4) { MOLORA_TOK(4) }
  else { MOLORA_TOK(8) }
#undef MOLORA_TOK
  return err;
}

hipError_t launch_step_vocab(const StepVocabLaunch& a, hipStream_t s) {
  StepArgs sa;
  sa.t = tile_args(a.apply);
  sa.bounds = a.bounds;
  sa.ids = a.ids; sa.idx = a.idx; sa.w = a.w; sa.counts = a.counts; sa.offsets = a.offsets; sa.perm = a.perm;
  sa.perm_w = a.perm_w; sa.inv = a.inv;
  const int grid = 8 * sa.t.tiles_per_xcd * sa.t.col_groups;
  const int RBv = a.apply.tgt.r_pad / 16;
  hipError_t err = hipSuccess;
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.apply.indirect, IND, MOLORA_DISPATCH_BOOL(a.apply.y0_f32, Y0F,
      MOLORA_DISPATCH_BOOL(a.apply.y_f32, YF, err = (launch_step_t<RB, IND, Y0F, YF>(sa, grid, s))))));
  return err;
}

// --------------------------------------------------------------------------------------
// Hot-set relayout of one adapter.
//   A [d_in][r] -> swizzled slab blocks (see a_swz_index); ranks r..r_pad-1 are zero.
//   B [r][d_out] -> B^T [d_out][r_pad] with the columns of each 128-column block permuted
//   (slab row w holds column b_perm_col(w)); ranks r..r_pad-1 are zero.
__global__ void relayout_A(const uint16_t* __restrict__ A, uint16_t* __restrict__ As, int d_in, int r, int r_pad) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)r_pad * d_in) return;
  const int RB = r_pad / 16;
  long long v = idx;
  const int i = (int)(v % 8); v /= 8;
  const int G = (int)(v % 4); v /= 4;
  const int n = (int)(v % 16); v /= 16;
  const int u = (int)(v % RB); v /= RB;
  const int c = (int)(v % 4); v /= 4;
  const int s = (int)v;
  const int j = u * 16 + n;
  const int col = s * kStepK + c * 32 + G * 8 + i;
  As[idx] = (j < r) ? A[(long long)col * r + j] : (uint16_t)0;
}
__global__ void relayout_B(const uint16_t* __restrict__ B, uint16_t* __restrict__ Bt, int d_out, int r, int r_pad) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)d_out * r_pad) return;
  const int row = (int)(i / r_pad), j = (int)(i % r_pad);
  const int col = b_perm_col(row);
  Bt[i] = (j < r) ? B[(long long)j * d_out + col] : (uint16_t)0;
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

hipError_t launch_seqpass_meta(const int32_t* idx, int N, int K, int32_t* offsets, int32_t* perm, float* perm_w,
                               hipStream_t s) {
  long long n = (long long)K * N;
  if (n < (long long)K * (K + 1)) n = (long long)K * (K + 1);
  hipLaunchKernelGGL(seqpass_meta, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, N, K, offsets, perm,
                     perm_w);
  return hipGetLastError();
}

}  // namespace molora
