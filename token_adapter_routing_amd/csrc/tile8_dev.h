// Token-major 8-token tiles: one workgroup (8 waves) applies every adapter its 8 tokens use
// to a slice of the output columns (MoLoRA pages, thelatestinai.com: per-token routing, Figure 2
// right and Table 1; the gate-weighted sum of the selected adapters' low-rank deltas).
//
// Shrink (x * A_e, d_in -> r).  MFMA rows carry the tile's 8 tokens twice: rows 0..7 take the
// even 32-element chunk of a 64-element pair of chunks, rows 8..15 the odd one, so all 64 lanes
// load x (lane (n, G): token n % 8, 16 bytes).  Two MFMAs per pair of chunks, against the A
// pieces of the even and of the odd chunk, accumulate into acc0 (rows 0..7 valid) and acc1
// (rows 8..15 valid); acc0 + acc1 is the token's partial over the wave's reduction range.
// The 8 waves split d_in; their partials meet in LDS.
//
// Expand (h * B_e, r -> d_out), in units of 256 output columns (two 128-column slab blocks):
// the A operand is h as a bf16 hi/lo pair in two MFMAs; rows 0..7 carry the tokens' h in
// k-slots 0..15 (zeros in 16..31), rows 8..15 carry it in k-slots 16..31.  The B operand takes
// block 0 of the unit in k-slots 0..15 and block 1 in 16..31, so rows 0..7 of D are the
// tokens against block 0 and rows 8..15 against block 1.  With the slab's column permutation
// inside 128-column blocks, lane (n, G) ends up holding 8 contiguous output columns of 4
// tokens: every y0 load and y store moves 16 bytes per lane, 512 contiguous bytes per row.
//
// Every store is unconditional: tile positions past the last token are clones of token N - 1
// (same x row, routing and y0 row, hence bit-identical results written to the same place),
// and in a last unit of only 128 columns both row halves carry h in k-slots 0..15 against
// block 0, so the lanes of block 1 write the same bytes as those of block 0.
//
// Load order follows use order, because vector-memory counters retire in issue order: the
// callers issue the small routing loads, then x (nontemporal); the body then requests the
// adapter pieces (read many times, they stay in L2) and the first unit's y0 rows, and only
// after the shrink MFMAs the other units' y0 rows, which then stream during the reduction.
#pragma once

#include "molora_mfma.h"

namespace molora {

constexpr int kT8Tokens = 8;
constexpr int kT8Waves = 8;
constexpr int kT8Threads = kT8Waves * kWave;
constexpr int kT8Unit = 256;    // output columns per expand unit (the last one may have 128)
constexpr int kT8MaxU = 16;     // distinct adapters per tile (K <= 16)

template <int RB>
struct T8Cfg {
  static constexpr int XS = 4;                                 // x steps held in registers
  static constexpr int SB = RB == 1 ? 4 : (RB == 2 ? 2 : 1);  // A steps per register batch (divides XS)
  static constexpr int JB = RB == 1 ? 8 : 4;                   // MFMA columns per B register batch
};

template <int RB>
struct T8Lds {
  float red[kT8Waves][RB * 128];                 // wave partials: [wave][u][rank][token]
  float wt[kT8MaxU][kT8Tokens];                  // gate weight x scale of (slot, token)
  alignas(16) uint16_t hb[kT8MaxU][2][RB][kT8Tokens][16];  // h hi / lo: [slot][part][u][token][rank]
};

struct T8Args {
  TargetDev tgt;
  const uint16_t* x;
  const void* y0;
  void* y;
  int N, K, k;
  float scale;
  int col_groups;     // output-column slices per tile
  int tiles;          // ceil(N / 8)
  int tiles_per_xcd;  // grid = 8 * tiles_per_xcd * col_groups
};

// Block b runs on XCD b % 8.  Each XCD takes a contiguous range of tiles (neighbouring tokens
// tend to share adapters, whose pieces then stay in that XCD's L2); the column groups of a tile
// are consecutive slots of one XCD.
__device__ __forceinline__ void t8_tile_of_block(int b, const T8Args& a, int& tt, int& g) {
  const int xcd = b & 7, slot = b >> 3;
  g = slot % a.col_groups;
  tt = xcd * a.tiles_per_xcd + slot / a.col_groups;
}

// Registers and addresses that carry from the prefetch to the body.
template <int RB, bool Y0F32>
struct T8Stream {
  u32x4_t xv[T8Cfg<RB>::XS][2];
  RowChunk<Y0F32> y0c0;   // y0 rows of the wave's first unit
  const uint16_t* xp;
  int trow;     // token of the lane's first output row (4 rows: trow .. trow + 3, clamped to N - 1)
  int s0, s1;   // the wave's reduction steps
  int c0, cend, nunits;
};

// First column of the lane's 128-column block in the unit at colbase (block G / 2); in a last
// unit of only 128 columns every lane takes block 0.
__device__ __forceinline__ int t8_block_col(int colbase, int cend, int G) {
  const bool has1 = colbase + kT8Unit <= cend;
  return colbase + ((G >= 2 && has1) ? 128 : 0);
}

// Set up the wave's ranges and issue the y0 rows of its first unit: they do not depend on the
// routing and keep HBM busy while the routing loads are answered.  Every thread calls it; the
// loads are issued unconditionally (clamped), so that later waits are exact counts.
template <bool Y0F32>
__device__ __forceinline__ void t8_load_y0(RowChunk<Y0F32>& r, const T8Args& a, int trow, int col, int n);

template <int RB, bool Y0F32, bool YF32>
__device__ __forceinline__ void t8_prefetch(const T8Args& a, int tt, int g, T8Stream<RB, Y0F32>& st) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int t0 = tt * kT8Tokens;
  const int d_in = a.tgt.d_in, d_out = a.tgt.d_out;
  const int tx = min(t0 + (n & 7), a.N - 1);
  st.xp = a.x + (size_t)tx * d_in + 32 * (n >> 3) + 8 * G;
  const int S = d_in / kStepK;
  st.s0 = (S * wave) / kT8Waves;
  st.s1 = (S * (wave + 1)) / kT8Waves;
  const int cols = d_out / a.col_groups;
  st.c0 = g * cols;
  st.cend = st.c0 + cols;
  st.nunits = (cols + kT8Unit - 1) / kT8Unit;
  st.trow = t0 + 4 * (G & 1);
  const int cb0 = st.c0 + min(wave, st.nunits - 1) * kT8Unit;
  t8_load_y0<Y0F32>(st.y0c0, a, st.trow, t8_block_col(cb0, st.cend, G), n);
}

// y0 rows / y rows of the lane's 4 tokens (addresses formed at each use, not held).
// Addresses are formed where they are used: the empty asm makes the row index opaque, so the
// compiler cannot compute the 64-bit addresses early and keep (or spill) them across the body.
__device__ __forceinline__ int t8_opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <bool Y0F32>
__device__ __forceinline__ void t8_load_y0(RowChunk<Y0F32>& r, const T8Args& a, int trow, int col, int n) {
  constexpr size_t y0b = Y0F32 ? 4 : 2;
  trow = t8_opaque(trow);
  const char* rows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    rows[i] = reinterpret_cast<const char*>(a.y0) + (size_t)min(trow + i, a.N - 1) * a.tgt.d_out * y0b;
  load_row_chunk<Y0F32>(r, rows, col, n);
}
template <bool Y0F32, bool YF32>
__device__ __forceinline__ void t8_store_y(const f32x4_t (&o)[8], const RowChunk<Y0F32>& y0c, const T8Args& a, int trow,
                                           int col, int n) {
  constexpr size_t yb = YF32 ? 4 : 2;
  trow = t8_opaque(trow);
  char* rows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    rows[i] = reinterpret_cast<char*>(a.y) + (size_t)min(trow + i, a.N - 1) * a.tgt.d_out * yb;
  epilogue_store<Y0F32, YF32>(o, y0c, rows, col, n, 0xFu);
}

// B pieces of MFMA columns j0 .. j0 + J - 1 of one expand unit, adapter B^T at Bt.
template <int RB, int J>
__device__ __forceinline__ void t8_load_b(u32x4_t (&bv)[J][RB], const uint16_t* __restrict__ Bt, int r_pad,
                                          int colbase, int cend, int lane, int j0) {
  const int n = lane & 15, G = lane >> 4;
  const uint16_t* bp = Bt + (size_t)(t8_block_col(t8_opaque(colbase), cend, G) + n) * r_pad + (G & 1) * 8;
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int u = 0; u < RB; ++u) bv[j][u] = ld16(bp + (size_t)(j0 + j) * 16 * r_pad + u * 16);
}

// Expand operands of adapter slot sl: this lane's 8 k-slots of h hi and lo for each rank block.
template <int RB>
__device__ __forceinline__ void t8_h_operands(const T8Lds<RB>& L, int sl, bool half, int lane, bf16x8_t (&hh)[RB],
                                              bf16x8_t (&hl)[RB]) {
  const int n = lane & 15, G = lane >> 4;
  const bool active = half ? (G < 2) : ((G >> 1) == (n >> 3));
  const int tl = n & 7, rr = 8 * (G & 1);
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    u32x4_t vh = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
    if (active) {
      vh = *reinterpret_cast<const u32x4_t*>(&L.hb[sl][0][u][tl][rr]);
      vl = *reinterpret_cast<const u32x4_t*>(&L.hb[sl][1][u][tl][rr]);
    }
    hh[u] = as_bf16x8(vh);
    hl[u] = as_bf16x8(vl);
  }
}

template <int RB, int J>
__device__ __forceinline__ void t8_expand_mfma(f32x4_t (&o)[8], const bf16x8_t (&hh)[RB], const bf16x8_t (&hl)[RB],
                                               const u32x4_t (&bv)[J][RB], int j0) {
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      o[j0 + j] = mfma16x16x32(hh[u], as_bf16x8(bv[j][u]), o[j0 + j]);
      o[j0 + j] = mfma16x16x32(hl[u], as_bf16x8(bv[j][u]), o[j0 + j]);
    }
}

// Main body, after t8_prefetch.  Lane l < 8k of every wave holds pair l of the tile (token
// t0 + l / k, slot l % k; positions past the last token hold a copy of token N - 1's pairs):
// adapter pe (-1: none) and pw = gate weight x scale.  `mid` runs once per wave after the
// first adapter loads are issued, before the shrink waits for its data.  Every thread of the
// workgroup calls this; control flow is uniform across the workgroup.
template <int RB, bool INDIRECT, bool Y0F32, bool YF32, typename Mid>
__device__ __forceinline__ void t8_main(const T8Args& a, T8Lds<RB>& L, T8Stream<RB, Y0F32>& st, int pe, float pw,
                                        Mid mid) {
  constexpr int XS = T8Cfg<RB>::XS;
  constexpr int SB = T8Cfg<RB>::SB;
  constexpr int JB = T8Cfg<RB>::JB;
  constexpr int NW = kT8Waves;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int r_pad = a.tgt.r_pad;

  // adapters used by the tile, ascending (one ballot per adapter index; K <= 16)
  uint32_t used = 0;
#pragma unroll
  for (int e = 0; e < kT8MaxU; ++e)
    if (e < a.K && __ballot(pe == e) != 0) used |= 1u << e;
  const int nU = __popc(used);
  const int e0 = nU > 0 ? __builtin_ctz(used) : 0;
  const int myunits = wave < st.nunits ? (st.nunits - 1 - wave) / NW + 1 : 0;
  // clamped unit columns: the loads below are issued by every wave
  const int cb0 = st.c0 + min(wave, st.nunits - 1) * kT8Unit;
  const int cb1 = st.c0 + min(wave + NW, st.nunits - 1) * kT8Unit;

  // first adapter's A pieces and the first unit's B pieces (they do not depend on h), ahead of
  // the x stream so that they are not queued behind it
  const bool x_resident = st.s1 - st.s0 <= XS;
  u32x4_t av[SB][4][RB];
  auto load_a = [&](const uint16_t* Ap, int sfirst) {
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int s = max(min(sfirst + i, st.s1 - 1), 0);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int u = 0; u < RB; ++u) av[i][c][u] = ld16(Ap + a_swz_index(RB, s, c, u, n, G, 0));
    }
  };
  load_a(adapter_A<INDIRECT>(a.tgt, e0), st.s0);
  u32x4_t b0[JB][RB], b1[JB][RB];
  t8_load_b<RB, JB>(b0, adapter_B<INDIRECT>(a.tgt, e0), r_pad, cb0, st.cend, lane, 0);
  // the wave's x steps (the first XS; a wave without reduction steps re-reads step 0)
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    const int s = max(min(st.s0 + i, st.s1 - 1), 0);
    st.xv[i][0] = ld16_nt(st.xp + s * kStepK);
    st.xv[i][1] = ld16_nt(st.xp + s * kStepK + 64);
  }
  RowChunk<Y0F32> y0c0 = st.y0c0, y0c1;
  mid();

  // shrink: one pass per used adapter; x stays in registers when the wave's steps fit; each
  // batch's A pieces are requested after the previous batch's MFMAs are issued
  uint32_t rem = used;
  for (int base = 0; base < nU; ++base) {
    const uint16_t* Acur = adapter_A<INDIRECT>(a.tgt, __builtin_ctz(rem));
    rem &= rem - 1;
    f32x4_t acc0[RB], acc1[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      acc0[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc1[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int xs0 = st.s0; xs0 < st.s1; xs0 += XS) {
      const int nx = min(XS, st.s1 - xs0);
      if (!x_resident && !(base == 0 && xs0 == st.s0)) {
#pragma unroll
        for (int i = 0; i < XS; ++i) {
          const int s = min(xs0 + i, st.s1 - 1);
          st.xv[i][0] = ld16_nt(st.xp + s * kStepK);
          st.xv[i][1] = ld16_nt(st.xp + s * kStepK + 64);
        }
      }
#pragma unroll
      for (int bi = 0; bi < XS / SB; ++bi) {
        if (bi * SB < nx) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < SB; ++i) {
            if (bi * SB + i < nx) {
#pragma unroll
              for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int u = 0; u < RB; ++u) {
                  const bf16x8_t xo = as_bf16x8(st.xv[bi * SB + i][p]);
                  acc0[u] = mfma16x16x32(xo, as_bf16x8(av[i][2 * p][u]), acc0[u]);
                  acc1[u] = mfma16x16x32(xo, as_bf16x8(av[i][2 * p + 1][u]), acc1[u]);
                }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          const int snext = xs0 + (bi + 1) * SB;
          if (snext < st.s1) load_a(Acur, snext);
        }
      }
    }
    // the next adapter's first A pieces stream during this adapter's reduction
    if (base + 1 < nU) load_a(adapter_A<INDIRECT>(a.tgt, __builtin_ctz(rem)), st.s0);
    if (base == nU - 1) {
      // the expand's second batch of B pieces, then the second unit's y0 rows, stream during
      // the last reduction.  Loads return in issue order, so every piece that the expand needs
      // before the second unit's store must be requested ahead of those rows: with one adapter
      // that is the second unit's pieces, with several (rank block 1) the first unit's pieces
      // of the second adapter.
      if (nU == 1 || JB == 8)
        t8_load_b<RB, JB>(b1, adapter_B<INDIRECT>(a.tgt, nU == 1 ? e0 : __builtin_ctz(used & (used - 1))), r_pad,
                          nU == 1 ? cb1 : cb0, st.cend, lane, 0);
      t8_load_y0<Y0F32>(y0c1, a, st.trow, t8_block_col(cb1, st.cend, G), n);
    }
    if (base == 0) {
      // weight table (slot, token): the sum of the token's gate weights on the slot's adapter;
      // the shuffles run with every lane of wave 0 active
      if (wave == 0) {
        for (int l0 = 0; l0 < kT8Tokens * nU; l0 += kWave) {
          const int l = l0 + lane;
          const int j = l >> 3, t = l & 7;
          uint32_t m = used;
          for (int i = 0; i < j && m != 0; ++i) m &= m - 1;
          const int e = m != 0 ? __builtin_ctz(m) : -2;
          float wsum = 0.f;
          for (int s = 0; s < a.k; ++s) {
            const int src = t * a.k + s;
            const int es = __shfl(pe, src, kWave);
            const float wv = __shfl(pw, src, kWave);
            if (es == e) wsum += wv;
          }
          if (l < kT8Tokens * nU) L.wt[j][t] = wsum;
        }
      }
    }
    // acc0 rows 0..7 (lanes G < 2) plus acc1 rows 8..15 (lanes G >= 2) of the same tokens
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const f32x4_t mine = (G < 2) ? acc0[u] : acc1[u];
      f32x4_t s;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = mine[i] + __shfl_xor(mine[i], 32, kWave);
      if (G < 2) *reinterpret_cast<f32x4_t*>(&L.red[wave][(u * 16 + n) * 8 + 4 * G]) = s;
    }
    __syncthreads();
    // 128 * RB threads sum the 8 partials of one (rank, token) in wave order, weight, split
    for (int v = threadIdx.x; v < RB * 128; v += kT8Threads) {
      const int tok = v & 7, rank = (v >> 3) & 15, u = v >> 7;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += L.red[w][v];
      const float h = sum * L.wt[base][tok];
      const __bf16 hi = (__bf16)h;
      const __bf16 lo = (__bf16)(h - (float)hi);
      L.hb[base][0][u][tok][rank] = __builtin_bit_cast(uint16_t, hi);
      L.hb[base][1][u][tok][rank] = __builtin_bit_cast(uint16_t, lo);
    }
    __syncthreads();
  }

  // a tile of unrouted tokens skipped the shrink, where the second unit's y0 rows are requested
  if (nU == 0) t8_load_y0<Y0F32>(y0c1, a, st.trow, t8_block_col(cb1, st.cend, G), n);

  // expand, y = y0 + sum over the used adapters (ascending) of h_e B_e
  if (myunits == 0) return;
  if (nU <= 1 && JB == 8) {
    // at most one adapter: the wave's units in pairs with two B buffers; the pieces of unit
    // i + 2 are requested right after unit i's MFMAs
    bf16x8_t hh[RB], hl[RB];
    for (int ui = 0; ui < myunits; ui += 2) {
      const int cba = st.c0 + (wave + ui * NW) * kT8Unit, cbb = cba + NW * kT8Unit;
      f32x4_t o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (nU == 1) {
        t8_h_operands<RB>(L, 0, cba + kT8Unit > st.cend, lane, hh, hl);
        t8_expand_mfma<RB, JB>(o, hh, hl, b0, 0);
      }
      t8_store_y<Y0F32, YF32>(o, y0c0, a, st.trow, t8_block_col(cba, st.cend, G), n);
      if (ui + 2 < myunits) {
        const int cbn = cba + 2 * NW * kT8Unit;
        if (nU == 1) t8_load_b<RB, JB>(b0, adapter_B<INDIRECT>(a.tgt, e0), r_pad, cbn, st.cend, lane, 0);
        t8_load_y0<Y0F32>(y0c0, a, st.trow, t8_block_col(cbn, st.cend, G), n);
      }
      if (ui + 1 < myunits) {
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (nU == 1) {
          t8_h_operands<RB>(L, 0, cbb + kT8Unit > st.cend, lane, hh, hl);
          t8_expand_mfma<RB, JB>(o, hh, hl, b1, 0);
        }
        t8_store_y<Y0F32, YF32>(o, y0c1, a, st.trow, t8_block_col(cbb, st.cend, G), n);
        if (ui + 3 < myunits) {
          const int cbn = cbb + 2 * NW * kT8Unit;
          if (nU == 1) t8_load_b<RB, JB>(b1, adapter_B<INDIRECT>(a.tgt, e0), r_pad, cbn, st.cend, lane, 0);
          t8_load_y0<Y0F32>(y0c1, a, st.trow, t8_block_col(cbn, st.cend, G), n);
        }
      }
    }
    return;
  }
  // several adapters (or large ranks): batch i = (unit, adapter slot, JB-column batch) in that
  // order, two B buffers in ping-pong: batch i + 1 is requested before batch i's MFMAs, so every
  // L2 round trip after the first overlaps the previous batch.  b0 holds batch 0 (requested
  // before the shrink).  Requests past the last batch repeat it (their data is not used), so
  // the number of loads in flight at every wait is the same on all paths.
  if (nU == 0) {
    // no routed token: y = y0
    for (int ui = 0; ui < myunits; ++ui) {
      const int cb = st.c0 + (wave + ui * NW) * kT8Unit;
      RowChunk<Y0F32> yc;
      if (ui == 0) yc = y0c0;
      else if (ui == 1) yc = y0c1;
      else t8_load_y0<Y0F32>(yc, a, st.trow, t8_block_col(cb, st.cend, G), n);
      f32x4_t o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      t8_store_y<Y0F32, YF32>(o, yc, a, st.trow, t8_block_col(cb, st.cend, G), n);
    }
    return;
  }
  constexpr int NBP = 8 / JB;  // batches per (unit, adapter)
  const int per_unit = nU * NBP;
  const int total = myunits * per_unit;
  auto batch_load = [&](u32x4_t (&bv)[JB][RB], int i) {
    i = min(i, total - 1);
    const int ui = i / per_unit, rem = i - ui * per_unit, sl = rem / NBP, jb = rem - sl * NBP;
    uint32_t m = used;
    for (int q = 0; q < sl; ++q) m &= m - 1;
    const int cb = st.c0 + (wave + ui * NW) * kT8Unit;
    t8_load_b<RB, JB>(bv, adapter_B<INDIRECT>(a.tgt, __builtin_ctz(m)), r_pad, cb, st.cend, lane, jb * JB);
  };
  f32x4_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  RowChunk<Y0F32> yc = y0c0;
  auto consume = [&](const u32x4_t (&bv)[JB][RB], int i) {
    const int ui = i / per_unit, rem = i - ui * per_unit, sl = rem / NBP, jb = rem - sl * NBP;
    const int cb = st.c0 + (wave + ui * NW) * kT8Unit;
    bf16x8_t hh[RB], hl[RB];
    t8_h_operands<RB>(L, sl, cb + kT8Unit > st.cend, lane, hh, hl);
    __builtin_amdgcn_sched_barrier(0);
    if (NBP == 1 || jb == 0) t8_expand_mfma<RB, JB>(o, hh, hl, bv, 0);
    else t8_expand_mfma<RB, JB>(o, hh, hl, bv, JB);
    __builtin_amdgcn_sched_barrier(0);
    if (rem == per_unit - 1) {
      t8_store_y<Y0F32, YF32>(o, yc, a, st.trow, t8_block_col(cb, st.cend, G), n);
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (ui + 1 == 1) yc = y0c1;
      else if (ui + 1 < myunits) t8_load_y0<Y0F32>(yc, a, st.trow, t8_block_col(cb + NW * kT8Unit, st.cend, G), n);
    }
  };
  // first pair of batches: with rank block 1, b1 already holds batch 1
  if constexpr (JB != 8) batch_load(b1, 1);
  consume(b0, 0);
  batch_load(b0, 2);
  if (1 < total) consume(b1, 1);
  for (int i = 2; i < total; i += 2) {
    batch_load(b1, i + 1);
    consume(b0, i);
    batch_load(b0, i + 2);
    if (i + 1 < total) consume(b1, i + 1);
  }
}

}  // namespace molora
