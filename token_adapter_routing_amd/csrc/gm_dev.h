// Grouped tiles of up to 64 rows of one adapter (MoLoRA pages, thelatestinai.com: Figure 2
// right, tokens grouped by their selected adapter and one grouped GEMM per adapter; Table 10
// shapes).
//
// The rows of a pass (a grouped order, adapter by adapter) are cut into tiles of at most 64
// rows, one per workgroup and column slice, that never span two adapters: each adapter's
// segment gets ceil(count / bound) tiles of equal height (the bound aims at 256 tiles per pass,
// one round on 256 CUs), or, for the fixed-tiling comparator, 64-row tiles.
//
// A workgroup (8 waves) takes a sub-tile: wave w works on row block rb = w % 4 (16 rows) and
// half hf = w / 4.  In the shrink, half hf takes one half of the reduction steps; in the
// expand, the 128-column blocks alternate between the halves.  The adapter pieces of a stage
// (A for the shrink, B^T for the expand) are loaded into registers three stages ahead, written
// to one of three LDS buffers (one barrier per stage) and shared by the four row blocks, so a
// workgroup reads its adapter once per sub-tile.  The expand's first stages and its y0 chunks
// are requested before the shrink result is reduced, so those loads overlap the reduction.
//
// Rows are grouped positions r of a pass; the row's source position q = order[r] (or r), its
// pair p = perm[q], token p / k, and gate weight wts[r] (times alpha/r).  Rows past the end of
// a sub-tile repeat its first row in the arithmetic and are not stored.
#pragma once

#include "molora_mfma.h"

namespace molora {

constexpr int kGMRows = 64;
constexpr int kGMWaves = 8;
constexpr int kGMThreads = kGMWaves * kWave;
constexpr int kGMDepth = 3;  // stages in flight

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
  int col_groups;           // output-column slices
  int nwg;                  // row tiles (a multiple of 8, at least the tiles of a pass); grid = nwg * col_groups
  int tile_rows;            // tile height bound (GMTiling::rows)
  int fixed;                // GMTiling::fixed
  float* hout;              // shrink-only mode: unscaled h of grouped position q at [q][r_pad]
  uint16_t* hs_out;         // shrink-only mode, instead: bf16 hi / lo of wts * scale * h at
                            // [q][2][r_pad] (the token-block expand's MFMA operand rows)
};

template <int RB>
struct GMLds {
  static constexpr int kStage = 8 * RB * 512;  // elements: 8 RB pieces of 1 KB
  // three stage buffers; after the shrink the first ones' bytes hold the halves' partial sums
  alignas(16) uint16_t stage[kGMDepth][kStage];
  alignas(16) uint16_t hb[2][kGMRows][RB * 16];  // h hi / lo per row
  float wt[kGMRows];                             // gate weight x alpha/r per row
  __device__ float* red() { return reinterpret_cast<float*>(&stage[0][0]); }
  static_assert(sizeof(float) * 2 * 4 * 16 * (RB * 16 + 4) <= sizeof(stage), "partial sums fit in the stage buffers");
};

// LDS placement of the staged pieces.  LDS serves a 16-byte read per lane in groups of 8
// lanes, conflict-free when the 8 lanes' 16-byte slots differ in their low 3 bits.
//  A piece (64 slots): the shrink's lane (n, G) reads slot 4n + G, the stage store writes slot
//  lane; slot p is kept at gm_a_slot(p), whose low bits (p1^p4, p0^p3, p2) are a bijection both
//  over 8 consecutive p and over the 8 n of one G.
//  B^T block (128 rows of 2RB slots): the expand's lane (n, G) reads row 16jj + n, slot
//  2u + (G & 1); slot cs of a row is XORed with row bits chosen so 8 consecutive rows land on
//  8 bank groups (rank 16, 32, 64; rank 48 keeps the plain layout).
__device__ __forceinline__ int gm_a_slot(int p) {
  return (p & ~7) | ((((p >> 1) ^ (p >> 4)) & 1) << 2) | (((p ^ (p >> 3)) & 1) << 1) | ((p >> 2) & 1);
}
template <int RB>
__device__ __forceinline__ int gm_b_swz(int row) {
  constexpr int spr = 2 * RB;
  if constexpr (RB == 1 || RB == 2 || RB == 4) return (row / (8 / spr)) & (spr - 1);
  else return 0;
}
template <int RB>
__device__ __forceinline__ int gm_b_slot(int S) {  // S: slot in the block, row-major
  constexpr int spr = 2 * RB;
  const int row = S / spr, cs = S % spr;
  return row * spr + (cs ^ gm_b_swz<RB>(row));
}

// Stage loads: piece i (1 KB) from src(i), loaded by wave i % 8 (16 bytes per lane).
template <int RB, typename Src>
__device__ __forceinline__ void gm_stage_load(u32x4_t (&v)[RB], Src src) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < RB; ++j) v[j] = ld16(src(wave + kGMWaves * j) + 8 * lane);
}
// A stage: pieces 0 .. 8RB-1, each kept in its own 1 KB with the gm_a_slot placement.
template <int RB>
__device__ __forceinline__ void gm_stage_store_a(uint16_t* dst, const u32x4_t (&v)[RB]) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sl = gm_a_slot(lane);
#pragma unroll
  for (int j = 0; j < RB; ++j)
    *reinterpret_cast<u32x4_t*>(dst + ((size_t)(wave + kGMWaves * j) * 64 + sl) * 8) = v[j];
}
// B stage: pieces h * 4RB + w hold slots w * 64 + lane of half h's 128-row block.
template <int RB>
__device__ __forceinline__ void gm_stage_store_b(uint16_t* dst, const u32x4_t (&v)[RB]) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int pi = wave + kGMWaves * j;
    const int h = pi / (4 * RB), w = pi % (4 * RB);
    *reinterpret_cast<u32x4_t*>(dst + ((size_t)h * 4 * RB * 64 + gm_b_slot<RB>(w * 64 + lane)) * 8) = v[j];
  }
}

template <int RB>
struct GMShrinkSet {
  u32x4_t a[RB];
  u32x4_t x[4];
};
template <int RB, bool Y0F32>
struct GMExpandSet {
  u32x4_t b[RB];
  RowChunk<Y0F32> y;
};

// One sub-tile: rows [row0, row0 + nrows) of adapter e, output columns [c0, c0 + cols).
// SHRINK_ONLY: stop after the reduction and write the rows' unscaled h to a.hout (the
// backward's per-pair h and g).
template <int RB, bool INDIRECT, bool Y0F32, bool YF32, bool SHRINK_ONLY = false>
__device__ void gm_tile(const GMArgs& a, GMLds<RB>& L, int e, int row0, int nrows, int c0, int cols) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int rb = wave & 3, hf = wave >> 2;
  const int d_in = a.tgt.d_in, d_out = a.tgt.d_out, r_pad = a.tgt.r_pad;
  // lane n (of every group) holds the token of row 16 rb + n
  int tokl;
  {
    const int rl = 16 * rb + n;
    const int rr = row0 + (rl < nrows ? rl : 0);
    const int q = a.order != nullptr ? a.order[rr] : rr;
    tokl = a.perm[q] / a.k;
  }
  if (!SHRINK_ONLY && threadIdx.x < kGMRows)
    L.wt[threadIdx.x] = a.wts[row0 + ((int)threadIdx.x < nrows ? (int)threadIdx.x : 0)] * a.scale;
  const uint16_t* At = adapter_A<INDIRECT>(a.tgt, e);
  const uint16_t* Bt = adapter_B<INDIRECT>(a.tgt, e);

  // ---------------- shrink: half 0 takes steps [0, S0), half 1 steps [S0, S); stage i holds
  // step i of half 0 (pieces 0 .. 4RB-1) and step S0 + i of half 1 (pieces 4RB .. 8RB-1)
  const int S = d_in / kStepK, S0 = (S + 1) / 2;
  const size_t piece = (size_t)RB * 16 * kStepK;  // elements of one step's 4 RB pieces
  const uint16_t* xrow = a.x + (size_t)tokl * d_in + 8 * G;
  // Each set's registers are reloaded right after their last use and loads issue in program
  // order (scheduling barriers), so the compiler's waits name exactly the stage they need.
  auto load_a = [&](GMShrinkSet<RB>& st, int i) {
    i = min(i, S0 - 1);
    gm_stage_load<RB>(st.a, [=](int pi) {
      const int h = pi / (4 * RB), w = pi % (4 * RB);
      const int s = min(i + h * S0, S - 1);
      return At + (size_t)s * piece + (size_t)w * 512;
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_x = [&](GMShrinkSet<RB>& st, int i) {
    const int s = min(min(i, S0 - 1) + hf * S0, S - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) st.x[c] = ld16_nt(xrow + s * kStepK + 32 * c);
    __builtin_amdgcn_sched_barrier(0);
  };
  f32x4_t acc[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int a_sl = gm_a_slot(4 * n + G);
  auto shrink_stage = [&](int i, const u32x4_t (&xv)[4], const uint16_t* st) {
    if (i < S0 && i + hf * S0 < S) {
      const uint16_t* ap = st + (size_t)hf * 4 * RB * 512;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const u32x4_t av = *reinterpret_cast<const u32x4_t*>(ap + ((c * RB + u) * 64 + a_sl) * 8);
          acc[u] = mfma16x16x32(as_bf16x8(xv[c]), as_bf16x8(av), acc[u]);
        }
    }
  };

  // ---------------- expand geometry: the slice's 128-column blocks in pairs (block 2j to half 0,
  // 2j+1 to half 1); stage j holds the B^T rows of pair j
  const int nblk = cols / kColBlock;
  const int npairs = (nblk + 1) / 2;
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  const char* y0rows[4];
  char* yrows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = __shfl(tokl, 4 * G + i, kWave);
    y0rows[i] = reinterpret_cast<const char*>(a.y0) + (size_t)t * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(a.y) + (size_t)t * d_out * yb;
  }
  unsigned vmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) vmask |= (16 * rb + 4 * G + i < nrows ? 1u : 0u) << i;
  auto my_col = [&](int j) { return c0 + min(2 * j + hf, nblk - 1) * kColBlock; };
  auto load_b = [&](GMExpandSet<RB, Y0F32>& st, int j) {
    j = min(j, npairs - 1);
    gm_stage_load<RB>(st.b, [=](int pi) {
      const int h = pi / (4 * RB), w = pi % (4 * RB);
      const int blk = min(2 * j + h, nblk - 1);
      return Bt + (size_t)(c0 + blk * kColBlock) * r_pad + (size_t)w * 512;
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_y = [&](GMExpandSet<RB, Y0F32>& st, int j) {
    load_row_chunk<Y0F32>(st.y, y0rows, my_col(min(j, npairs - 1)), n);
    __builtin_amdgcn_sched_barrier(0);
  };

  GMExpandSet<RB, Y0F32> e0, e1, e2;
  {
    GMShrinkSet<RB> s0, s1, s2;
    load_a(s0, 0);
    load_x(s0, 0);
    load_a(s1, 1);
    load_x(s1, 1);
    load_a(s2, 2);
    load_x(s2, 2);
    // unconditional (clamped) reloads keep the count of loads in flight the same on every path
    auto step = [&](GMShrinkSet<RB>& st, int i, int buf) {
      gm_stage_store_a<RB>(L.stage[buf], st.a);
      load_a(st, i + kGMDepth);
      __syncthreads();
      shrink_stage(i, st.x, L.stage[buf]);
      load_x(st, i + kGMDepth);
    };
    // whole rounds of three stages (no exits inside a round: the waits stay exact); stages
    // past S0 only store and reload
    for (int i = 0; i < S0; i += 3) {
      step(s0, i, 0);
      step(s1, i + 1, 1);
      step(s2, i + 2, 2);
    }
  }
  // the expand's first stages and y0 chunks go out now and land during the reduction
  if constexpr (!SHRINK_ONLY) {
    load_b(e0, 0);
    load_y(e0, 0);
    load_b(e1, 1);
    load_y(e1, 1);
    load_b(e2, 2);
    load_y(e2, 2);
  }
  __syncthreads();  // every wave is done with the stage buffers: the partial sums go there
  float* red = L.red();
  constexpr int kRS = RB * 16 + 4;
#pragma unroll
  for (int u = 0; u < RB; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((hf * 4 + rb) * 16 + 4 * G + i) * kRS + u * 16 + n] = acc[u][i];
  __syncthreads();
  if constexpr (SHRINK_ONLY) {
    for (int v = threadIdx.x; v < kGMRows * RB * 16; v += kGMThreads) {
      const int row = v / (RB * 16), rk = v % (RB * 16);
      if (row < nrows) {
        const int rbv = row >> 4, rw = row & 15;
        const int rr = row0 + row;
        const int q = a.order != nullptr ? a.order[rr] : rr;
        const float h = red[(rbv * 16 + rw) * kRS + rk] + red[((4 + rbv) * 16 + rw) * kRS + rk];
        if (a.hs_out != nullptr) {
          const float v = h * a.wts[rr] * a.scale;
          const __bf16 hi = (__bf16)v;
          a.hs_out[(size_t)q * (2 * RB * 16) + rk] = __builtin_bit_cast(uint16_t, hi);
          a.hs_out[(size_t)q * (2 * RB * 16) + RB * 16 + rk] = __builtin_bit_cast(uint16_t, (__bf16)(v - (float)hi));
        } else {
          a.hout[(size_t)q * (RB * 16) + rk] = h;
        }
      }
    }
    __syncthreads();  // the next sub-tile reuses the buffers
    return;
  }
  for (int v = threadIdx.x; v < kGMRows * RB * 16; v += kGMThreads) {
    const int row = v / (RB * 16), rk = v % (RB * 16);
    const int rbv = row >> 4, rw = row & 15;
    const float h = (red[(rbv * 16 + rw) * kRS + rk] + red[((4 + rbv) * 16 + rw) * kRS + rk]) * L.wt[row];
    const __bf16 hi = (__bf16)h;
    const __bf16 lo = (__bf16)(h - (float)hi);
    L.hb[0][row][rk] = __builtin_bit_cast(uint16_t, hi);
    L.hb[1][row][rk] = __builtin_bit_cast(uint16_t, lo);
  }
  __syncthreads();

  // A operand: row n of the row block; groups 0, 1 carry hi of ranks 16u + 8(G & 1) ..,
  // groups 2, 3 lo of the same ranks
  bf16x8_t hbv[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u)
    hbv[u] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&L.hb[G >> 1][16 * rb + n][u * 16 + 8 * (G & 1)]));
  // lane's B^T slots: row 16jj + n, slot 2u + (G & 1), XOR-placed (the row swizzle depends on n only)
  int b_sl[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) b_sl[u] = n * 2 * RB + ((2 * u + (G & 1)) ^ gm_b_swz<RB>(n));
  auto expand_step = [&](GMExpandSet<RB, Y0F32>& st, int j, int buf) {
    gm_stage_store_b<RB>(L.stage[buf], st.b);
    load_b(st, j + kGMDepth);
    __syncthreads();
    const int blk = 2 * j + hf;
    if (j < npairs) {
    const uint16_t* bl = L.stage[buf] + (size_t)hf * 4 * RB * 512;
    f32x4_t o[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) o[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(bl + ((size_t)jj * 16 * 2 * RB + b_sl[u]) * 8);
        o[jj] = mfma16x16x32(hbv[u], as_bf16x8(bv), o[jj]);
      }
    if (blk < nblk) epilogue_store<Y0F32, YF32>(o, st.y, yrows, c0 + blk * kColBlock, n, vmask);
    }
    load_y(st, j + kGMDepth);
  };
  for (int j = 0; j < npairs; j += 3) {
    expand_step(e0, j, 0);
    expand_step(e1, j + 1, 1);
    expand_step(e2, j + 2, 2);
  }
  __syncthreads();  // the next sub-tile reuses the buffers
}

// The workgroup's row tile and column slice.  Segment e (adapter e of the pass) of count c is
// cut into nt = ceil(c / tile_rows) tiles: balanced (tile i: rows c*i/nt .. c*(i+1)/nt) or,
// fixed, tile_rows rows each but the last; the tiles are numbered segment by segment, so
// consecutive tiles (which run on one XCD) mostly share their adapter in its L2.
// Tile w of the pass (every lane of the wave calls it): its adapter e and rows [r0, r1);
// false past the pass's tiles (the same answer in every wave).
__device__ __forceinline__ bool gm_locate(const GMArgs& a, int w, int& e, int& r0, int& r1) {
  const int lane = threadIdx.x & 63;
  const int M = a.tile_rows;
  const int s0l = lane < a.nkeys ? a.offsets[a.key0 + lane] : 0;
  const int cl = lane < a.nkeys ? a.offsets[a.key0 + lane + 1] - s0l : 0;
  const int ntl = (cl + M - 1) / M;
  const int incl = wave_incl_scan(ntl, lane);
  const uint64_t m = __ballot(lane < a.nkeys && w >= incl - ntl && w < incl);
  if (m == 0) return false;
  e = __builtin_ctzll(m);
  const int s0 = __shfl(s0l, e, kWave), c = __shfl(cl, e, kWave), nt = __shfl(ntl, e, kWave);
  const int i = w - (__shfl(incl, e, kWave) - nt);
  if (a.fixed) {
    r0 = s0 + i * M;
    r1 = min(s0 + c, r0 + M);
  } else {
    r0 = s0 + (int)((long long)c * i / nt);
    r1 = s0 + (int)((long long)c * (i + 1) / nt);
  }
  return true;
}

template <int RB, bool INDIRECT, bool Y0F32, bool YF32, bool SHRINK_ONLY = false>
__device__ void gm_range(const GMArgs& a, GMLds<RB>& L) {
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_xcd = a.nwg >> 3;
  const int g = slot % a.col_groups;
  const int w = xcd * per_xcd + slot / a.col_groups;
  int e, r0, r1;
  if (!gm_locate(a, w, e, r0, r1)) return;
  const int cols = a.tgt.d_out / a.col_groups;
  gm_tile<RB, INDIRECT, Y0F32, YF32, SHRINK_ONLY>(a, L, e, r0, r1 - r0, g * cols, cols);
}

}  // namespace molora
