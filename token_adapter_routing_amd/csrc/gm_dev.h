// Grouped tiles of up to 64 rows of one adapter (MoLoRA pages, thelatestinai.com: Figure 2
// right, tokens grouped by their selected adapter and one grouped GEMM per adapter; Table 10
// shapes).
//
// The rows of a pass (a grouped order, adapter by adapter) are cut into tiles of at most 64
// rows that never span two adapters: each adapter's segment gets ceil(count / bound) tiles of
// equal height (the bound aims at 256 workgroups per pass, one round on 256 CUs), or, for the
// fixed-tiling comparator, 64-row tiles.  gm_locate maps a tile number to its adapter and rows;
// the passes run the tiles split over 512-wide slices (gsplit.hip).
//
// Rows are grouped positions r of a pass; the row's source position q = order[r] (or r), its
// pair p = perm[q], token p / k, and gate weight wts[r] (times alpha/r).  Rows past the end of
// a tile repeat its first row in the arithmetic and are not stored.
#pragma once

#include "molora_mfma.h"

namespace molora {

constexpr int kGMRows = 64;

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
};

// LDS placement of staged B^T rows of 2RB 16-byte slots (the split expands).  LDS serves a
// 16-byte read per lane in groups of 8 lanes, conflict-free when the 8 lanes' slots differ in
// their low 3 bits: lane (n, G) reads row 16jj + n, slot 2u + (G & 1); slot cs of a row is
// XORed with gm_b_swz(row), row bits chosen so 8 consecutive rows land on 8 bank groups (rank
// 16, 32, 64; rank 48 keeps the plain layout).
template <int RB>
__device__ __forceinline__ int gm_b_swz(int row) {
  constexpr int spr = 2 * RB;
  if constexpr (RB == 1 || RB == 2 || RB == 4) return (row / (8 / spr)) & (spr - 1);
  else return 0;
}

// Segment e (adapter e of the pass) of count c is cut into nt = ceil(c / tile_rows) tiles:
// balanced (heights c / nt, the first c % nt tiles one row taller) or, fixed, tile_rows rows
// each but the last; the tiles are numbered segment by segment, so consecutive tiles (which run
// on one XCD) mostly share their adapter in its L2.
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
      } else {  // the first c % nt tiles one row taller
        const int h = c / nt, rem = c - h * nt;
        r0 = s0 + i * h + min(i, rem);
        r1 = r0 + h + (i < rem ? 1 : 0);
      }
      return true;
    }
    before = __shfl(incl, kWave - 1, kWave);
  }
  return false;
}

}  // namespace molora
