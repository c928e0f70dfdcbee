// Grouped tiles of 64 rows of one adapter (MoLoRA pages, thelatestinai.com: Figure 2 right,
// tokens grouped by their selected adapter and one grouped GEMM per adapter; Table 10 shapes).
//
// A workgroup (8 waves) takes 64 consecutive rows of one adapter's segment of a grouped order
// and a slice of the output columns.  Wave w works on row block rb = w % 4 (16 rows) and half
// hf = w / 4: in the shrink, half hf takes one half of the reduction steps; in the expand, the
// 128-column blocks alternate between the halves.  The adapter pieces are staged in LDS (two
// buffers; each stage is loaded into registers one stage ahead and written to LDS when its
// buffer is free, one barrier per stage) and shared by the four row blocks, so a workgroup
// reads its adapter's A and B once per 64 rows (at rank 64 and d = 4096: 1 MB per 64 rows
// instead of per 16).
//
// Rows are grouped positions r of a pass; the row's source position q = order[r] (or r), its
// pair p = perm[q], token p / k, and gate weight wts[r] (times alpha/r).  Rows past the end of
// a tile repeat the tile's first row in the arithmetic and are not stored (another wave may be
// storing that token's row at the same time).
#pragma once

#include "molora_mfma.h"

namespace molora {

constexpr int kGMRows = 64;
constexpr int kGMWaves = 8;
constexpr int kGMThreads = kGMWaves * kWave;

struct GMArgs {
  TargetDev tgt;
  const uint16_t* x;
  const void* y0;
  void* y;
  int N, k;
  int key0, nkeys;          // keys [key0, key0 + nkeys) of offsets; adapter = key - key0
  const int32_t* offsets;   // grouped start of each key (key0 + nkeys + 1 entries used)
  const int32_t* order;     // row -> source position (nullptr: the row itself)
  const int32_t* perm;      // source position -> pair id
  const float* wts;         // row -> gate weight
  float scale;
  int col_groups;           // output-column slices per tile
  int tiles_per_xcd;        // grid = 8 * tiles_per_xcd * col_groups
};

template <int RB>
struct GMLds {
  alignas(16) uint16_t stage[2][8 * RB * 512];   // two stages of 8 RB pieces of 1 KB
  float red[2][4][16][RB * 16 + 4];              // shrink halves of each row block
  alignas(16) uint16_t hb[2][kGMRows][RB * 16];  // h hi / lo per row
  int tok[kGMRows];
};

// Tile T of the keys' segments (64 rows each, numbered key by key): key e, first row, rows.
__device__ __forceinline__ bool gm_find_tile(const int* __restrict__ offsets, int nkeys, int T, int lane, int& e,
                                             int& row0, int& nrows) {
  int lo = 0, hi = 0;
  if (lane < nkeys) {
    lo = offsets[lane];
    hi = offsets[lane + 1];
  }
  const int nt = (hi - lo + kGMRows - 1) / kGMRows;
  const int incl = wave_incl_scan(nt, lane);
  const int excl = incl - nt;
  const uint64_t m = __ballot(lane < nkeys && T >= excl && T < incl);
  if (m == 0) return false;
  const int el = __builtin_ctzll(m);
  e = el;
  const int lo_e = __shfl(lo, el, kWave), hi_e = __shfl(hi, el, kWave), ex_e = __shfl(excl, el, kWave);
  row0 = lo_e + (T - ex_e) * kGMRows;
  nrows = min(kGMRows, hi_e - row0);
  return true;
}

// One stage of adapter pieces: piece i (1 KB) from src(i), loaded by wave i % 8 (16 bytes per
// lane) into registers, written to LDS one stage later (the compiler then waits on exactly the
// loads it needs).
template <int RB, typename Src>
__device__ __forceinline__ void gm_stage_load(u32x4_t (&v)[RB], Src src) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < RB; ++j) v[j] = ld16(src(wave + kGMWaves * j) + 8 * lane);
}
template <int RB>
__device__ __forceinline__ void gm_stage_store(uint16_t* dst, const u32x4_t (&v)[RB]) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < RB; ++j)
    *reinterpret_cast<u32x4_t*>(dst + (size_t)(wave + kGMWaves * j) * 512 + 8 * lane) = v[j];
}

template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__device__ void gm_tile(const GMArgs& a, GMLds<RB>& L, int T, int g) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int rb = wave & 3, hf = wave >> 2;
  int e, row0, nrows;
  if (!gm_find_tile(a.offsets + a.key0, a.nkeys, T, lane, e, row0, nrows)) return;
  const int d_in = a.tgt.d_in, d_out = a.tgt.d_out, r_pad = a.tgt.r_pad;
  // the tile's rows: token of each (rows past the end repeat row 0)
  if (threadIdx.x < kGMRows) {
    const int rr = row0 + (threadIdx.x < nrows ? (int)threadIdx.x : 0);
    const int q = a.order != nullptr ? a.order[rr] : rr;
    L.tok[threadIdx.x] = a.perm[q] / a.k;
  }
  const int myrow = 16 * rb + n;
  __syncthreads();
  const uint16_t* At = adapter_A<INDIRECT>(a.tgt, e);
  const uint16_t* Bt = adapter_B<INDIRECT>(a.tgt, e);

  // ---------------- shrink: half 0 takes steps [0, S0), half 1 steps [S0, S); stage i holds
  // step i of half 0 (pieces 0 .. 4RB-1) and step S0 + i of half 1 (pieces 4RB .. 8RB-1)
  const int S = d_in / kStepK, S0 = (S + 1) / 2;
  const size_t piece = (size_t)RB * 16 * kStepK;  // elements of one step's 4 RB pieces
  const uint16_t* xrow = a.x + (size_t)L.tok[myrow] * d_in + 8 * G;
  auto a_src = [&](int i_stage) {
    return [=](int pi) {
      const int h = pi / (4 * RB), w = pi % (4 * RB);
      const int s = min(i_stage + h * S0, S - 1);
      return At + (size_t)s * piece + (size_t)w * 512;
    };
  };
  auto x_load = [&](u32x4_t (&xv)[4], int i_stage) {
    const int s = min(i_stage + hf * S0, S - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[c] = ld16_nt(xrow + s * kStepK + 32 * c);
  };
  f32x4_t acc[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto shrink_stage = [&](int i, const u32x4_t (&xv)[4], const uint16_t* st) {
    if (i + hf * S0 < S) {
      const uint16_t* ap = st + (size_t)hf * 4 * RB * 512;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const u32x4_t av = *reinterpret_cast<const u32x4_t*>(ap + ((c * RB + u) * 64 + 4 * n + G) * 8);
          acc[u] = mfma16x16x32(as_bf16x8(xv[c]), as_bf16x8(av), acc[u]);
        }
    }
  };
  {
    u32x4_t sa[RB], sb[RB], xa[4], xb[4];
    gm_stage_load<RB>(sa, a_src(0));
    x_load(xa, 0);
    for (int i = 0; i < S0; i += 2) {
      gm_stage_load<RB>(sb, a_src(min(i + 1, S0 - 1)));
      x_load(xb, min(i + 1, S0 - 1));
      gm_stage_store<RB>(L.stage[0], sa);
      __syncthreads();
      shrink_stage(i, xa, L.stage[0]);
      if (i + 1 >= S0) break;
      gm_stage_load<RB>(sa, a_src(min(i + 2, S0 - 1)));
      x_load(xa, min(i + 2, S0 - 1));
      gm_stage_store<RB>(L.stage[1], sb);
      __syncthreads();
      shrink_stage(i + 1, xb, L.stage[1]);
    }
  }
  // the two halves meet in LDS; 512 threads form h = (sum) x weight as a bf16 hi / lo pair
#pragma unroll
  for (int u = 0; u < RB; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) L.red[hf][rb][4 * G + i][u * 16 + n] = acc[u][i];
  __syncthreads();
  for (int v = threadIdx.x; v < kGMRows * RB * 16; v += kGMThreads) {
    const int row = v / (RB * 16), rk = v % (RB * 16);
    const int rbv = row >> 4, rw = row & 15;
    const int rrv = row0 + (row < nrows ? row : 0);
    const float h = (L.red[0][rbv][rw][rk] + L.red[1][rbv][rw][rk]) * (a.wts[rrv] * a.scale);
    const __bf16 hi = (__bf16)h;
    const __bf16 lo = (__bf16)(h - (float)hi);
    L.hb[0][row][rk] = __builtin_bit_cast(uint16_t, hi);
    L.hb[1][row][rk] = __builtin_bit_cast(uint16_t, lo);
  }
  __syncthreads();

  // ---------------- expand: the group's 128-column blocks in pairs (block 2j to half 0, 2j+1
  // to half 1), B^T rows of the pair staged in LDS
  const int cols = d_out / a.col_groups;
  const int c0 = g * cols;
  const int nblk = cols / kColBlock;
  const int npairs = (nblk + 1) / 2;
  auto b_src = [&](int j) {
    return [=](int pi) {
      const int h = pi / (4 * RB), w = pi % (4 * RB);
      const int blk = min(2 * j + h, nblk - 1);
      return Bt + (size_t)(c0 + blk * kColBlock) * r_pad + (size_t)w * 512;
    };
  };
  // A operand: row n of the row block; groups 0, 1 carry hi of ranks 16u + 8(G & 1) ..,
  // groups 2, 3 lo of the same ranks
  bf16x8_t hbv[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u)
    hbv[u] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&L.hb[G >> 1][myrow][u * 16 + 8 * (G & 1)]));
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  const char* y0rows[4];
  char* yrows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = L.tok[16 * rb + 4 * G + i];
    y0rows[i] = reinterpret_cast<const char*>(a.y0) + (size_t)t * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(a.y) + (size_t)t * d_out * yb;
  }
  unsigned vmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) vmask |= (16 * rb + 4 * G + i < nrows ? 1u : 0u) << i;
  auto my_col = [&](int j) { return c0 + min(2 * j + hf, nblk - 1) * kColBlock; };
  auto expand_stage = [&](int j, const RowChunk<Y0F32>& yc, const uint16_t* st) {
    const int blk = 2 * j + hf;
    const uint16_t* bl = st + (size_t)hf * 4 * RB * 512 + (size_t)n * r_pad + 8 * (G & 1);
    f32x4_t o[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) o[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(bl + (size_t)16 * jj * r_pad + 16 * u);
        o[jj] = mfma16x16x32(hbv[u], as_bf16x8(bv), o[jj]);
      }
    if (blk < nblk) epilogue_store<Y0F32, YF32>(o, yc, yrows, c0 + blk * kColBlock, n, vmask);
  };
  {
    u32x4_t sa[RB], sb[RB];
    RowChunk<Y0F32> ya, ybk;
    gm_stage_load<RB>(sa, b_src(0));
    load_row_chunk<Y0F32>(ya, y0rows, my_col(0), n);
    for (int j = 0; j < npairs; j += 2) {
      gm_stage_load<RB>(sb, b_src(min(j + 1, npairs - 1)));
      load_row_chunk<Y0F32>(ybk, y0rows, my_col(min(j + 1, npairs - 1)), n);
      gm_stage_store<RB>(L.stage[0], sa);
      __syncthreads();
      expand_stage(j, ya, L.stage[0]);
      if (j + 1 >= npairs) break;
      gm_stage_load<RB>(sa, b_src(min(j + 2, npairs - 1)));
      load_row_chunk<Y0F32>(ya, y0rows, my_col(min(j + 2, npairs - 1)), n);
      gm_stage_store<RB>(L.stage[1], sb);
      __syncthreads();
      expand_stage(j + 1, ybk, L.stage[1]);
    }
  }
}

}  // namespace molora
