// Grouped tiles of up to 64 rows of one adapter (MoLoRA pages, thelatestinai.com: Figure 2
// right, tokens grouped by their selected adapter and one grouped GEMM per adapter; Table 10
// shapes).
//
// The rows of a pass (a grouped order, adapter by adapter) are cut into tiles of at most 64
// rows that never span two adapters: each adapter's segment gets ceil(count / bound) tiles of
// equal height (the bound aims at 256 workgroups per pass, one round on 256 CUs), or, for the
// fixed-tiling comparator, 64-row tiles.  gm_locate maps a tile number to its adapter and rows;
// the apply passes run the tiles split over 512-wide slices (gsplit.hip).
//
// gm_shrink_tile: one workgroup (8 waves) per tile computes the unscaled h = x_t A_e of every
// row (the backward's per-pair h and g): wave w works on row block rb = w % 4 (16 rows) and
// half hf = w / 4 of the reduction steps.  The A pieces of a stage are loaded into registers
// three stages ahead, written to one of three LDS buffers (one barrier per stage) and shared
// by the four row blocks, so a workgroup reads its adapter once per tile.
//
// Rows are grouped positions r of a pass; the row's source position q = order[r] (or r), its
// pair p = perm[q], token p / k, and gate weight wts[r] (times alpha/r).  Rows past the end of
// a tile repeat its first row in the arithmetic and are not stored.
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
  int nwg;                  // row tiles (a multiple of 8, at least the tiles of a pass)
  int tile_rows;            // tile height bound (GMTiling::rows)
  int fixed;                // GMTiling::fixed
  float* hout;              // gm_shrink_tile: unscaled h of grouped position q at [q][r_pad]
};

template <int RB>
struct GMLds {
  static constexpr int kStage = 8 * RB * 512;  // elements: 8 RB pieces of 1 KB
  // three stage buffers; after the shrink the first ones' bytes hold the halves' partial sums
  alignas(16) uint16_t stage[kGMDepth][kStage];
  __device__ float* red() { return reinterpret_cast<float*>(&stage[0][0]); }
  static_assert(sizeof(float) * 2 * 4 * 16 * (RB * 16 + 4) <= sizeof(stage), "partial sums fit in the stage buffers");
};

// LDS placement of staged pieces.  LDS serves a 16-byte read per lane in groups of 8 lanes,
// conflict-free when the 8 lanes' 16-byte slots differ in their low 3 bits.
//  A piece (64 slots): the shrink's lane (n, G) reads slot 4n + G, the stage store writes slot
//  lane; slot p is kept at gm_a_slot(p), whose low bits (p1^p4, p0^p3, p2) are a bijection both
//  over 8 consecutive p and over the 8 n of one G.
//  B^T rows of 2RB slots (the split expand): lane (n, G) reads row 16jj + n, slot 2u + (G & 1);
//  slot cs of a row is XORed with gm_b_swz(row), row bits chosen so 8 consecutive rows land on
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
template <int RB>
struct GMShrinkSet {
  u32x4_t a[RB];
  u32x4_t x[4];
};

// One tile: rows [row0, row0 + nrows) of adapter e; the rows' unscaled h go to a.hout.
template <int RB, bool INDIRECT>
__device__ void gm_shrink_rows(const GMArgs& a, GMLds<RB>& L, int e, int row0, int nrows) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int rb = wave & 3, hf = wave >> 2;
  const int d_in = a.tgt.d_in;
  // lane n holds the token of row 16 rb + n
  int tokl;
  {
    const int rl = 16 * rb + n;
    const int rr = row0 + (rl < nrows ? rl : 0);
    const int q = a.order != nullptr ? a.order[rr] : rr;
    tokl = a.perm[q] / a.k;
  }
  const uint16_t* At = adapter_A<INDIRECT>(a.tgt, e);

  // half 0 takes steps [0, S0), half 1 steps [S0, S); stage i holds
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
  __syncthreads();  // every wave is done with the stage buffers: the partial sums go there
  float* red = L.red();
  constexpr int kRS = RB * 16 + 4;
#pragma unroll
  for (int u = 0; u < RB; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((hf * 4 + rb) * 16 + 4 * G + i) * kRS + u * 16 + n] = acc[u][i];
  __syncthreads();
  for (int v = threadIdx.x; v < kGMRows * RB * 16; v += kGMThreads) {
    const int row = v / (RB * 16), rk = v % (RB * 16);
    if (row < nrows) {
      const int rbv = row >> 4, rw = row & 15;
      const int rr = row0 + row;
      const int q = a.order != nullptr ? a.order[rr] : rr;
      a.hout[(size_t)q * (RB * 16) + rk] = red[(rbv * 16 + rw) * kRS + rk] + red[((4 + rbv) * 16 + rw) * kRS + rk];
    }
  }
}

// Segment e (adapter e of the pass) of count c is cut into nt = ceil(c / tile_rows) tiles:
// balanced (tile i: rows c*i/nt .. c*(i+1)/nt) or, fixed, tile_rows rows each but the last; the
// tiles are numbered segment by segment, so consecutive tiles (which run on one XCD) mostly
// share their adapter in its L2.
// Tile w of the pass (every lane of the wave calls it): its adapter e and rows [r0, r1);
// false past the pass's tiles (the same answer in every wave).
__device__ __forceinline__ bool gm_locate(const GMArgs& a, int w, int& e, int& r0, int& r1) {
  const int lane = threadIdx.x & 63;
  const int M = a.tile_rows;
  int before = 0;  // tiles of the keys of the earlier 64-key chunks
  for (int kc = 0; kc < a.nkeys; kc += kWave) {
    const int key = kc + lane;
    const bool in = key < a.nkeys;
    const int s0l = in ? a.offsets[a.key0 + key] : 0;
    const int cl = in ? a.offsets[a.key0 + key + 1] - s0l : 0;
    const int ntl = (cl + M - 1) / M;
    const int incl = before + wave_incl_scan(ntl, lane);
    const uint64_t m = __ballot(in && w >= incl - ntl && w < incl);
    if (m != 0) {
      const int l = __builtin_ctzll(m);
      e = kc + l;
      const int s0 = __shfl(s0l, l, kWave), c = __shfl(cl, l, kWave), nt = __shfl(ntl, l, kWave);
      const int i = w - (__shfl(incl, l, kWave) - nt);
      if (a.fixed) {
        r0 = s0 + i * M;
        r1 = min(s0 + c, r0 + M);
      } else {
        r0 = s0 + (int)((long long)c * i / nt);
        r1 = s0 + (int)((long long)c * (i + 1) / nt);
      }
      return true;
    }
    before = __shfl(incl, kWave - 1, kWave);
  }
  return false;
}

// Workgroup b takes tile (b % 8) * nwg / 8 + b / 8: consecutive tiles (mostly of one adapter)
// on one XCD.
template <int RB, bool INDIRECT>
__device__ void gm_shrink_tile(const GMArgs& a, GMLds<RB>& L) {
  const int w = (blockIdx.x & 7) * (a.nwg >> 3) + (blockIdx.x >> 3);
  int e, r0, r1;
  if (!gm_locate(a, w, e, r0, r1)) return;
  gm_shrink_rows<RB, INDIRECT>(a, L, e, r0, r1 - r0);
}

}  // namespace molora
