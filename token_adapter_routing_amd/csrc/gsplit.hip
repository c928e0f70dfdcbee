// Grouped tiles split over 512-wide slices (MoLoRA pages, thelatestinai.com: Figure 2 right,
// tokens grouped by their selected adapter and one grouped GEMM per adapter; Table 10 shapes,
// adapters up to rank 64).
//
// One pass over a grouped order (the tiles of gm_locate: each adapter segment cut into tiles of
// at most 64 rows) in three launches, so that a workgroup's loads are one slice of the tile
// instead of the whole of d_in and d_out:
//   gs_shrink    (tile pair, d_in slice of 512): the x rows of two consecutive tiles over the
//                slice against the adapter's A slice (straight into LDS, shared when both tiles
//                belong to one adapter); the two halves of the slice meet in LDS and the
//                partial x A of each tile's 64 rows goes to part[tile][slice] (fp32).
//   gs_finalize  (tile): h = (sum of the slices in order) x gate weight x alpha/r per row, as
//                bf16 hi / lo rows hb[tile] -- the expand's MFMA A operand (or by grouped
//                position: hq for the pair passes, unscaled fp32 hout for the backward).
//   gs_expand    (tile, d_out slice of 512): the adapter's B^T slice (straight into LDS, in the
//                XOR placement of the 64-row tiles, so the operand reads are conflict-free), the
//                h rows and the tile's y0 rows are requested at once; y = y0 + h B for the rows
//                of the tile (token rows; within a pass a token has at most one row).
// Every launch numbers the tiles the same way: tile w runs on XCD w / (nwg / 8), with the
// tiles of one adapter mostly on one XCD, whose L2 then holds the adapter's slices and the
// tile's partials and h rows.
#include <climits>

#include "gm_dev.h"
#include "molora.h"
#include "molora_launch.h"

namespace molora {

namespace {

constexpr int kGSThreads = 512;
constexpr int kGSSteps = kBSlice / kStepK;  // 4

struct GSArgs {
  GMArgs g;        // the pass: tiles, rows, routing, adapters, x, y0 / y, scale
  float* part;     // [nwg][kslices][64][r_pad] fp32
  uint16_t* hb;    // [nwg][2][64][r_pad] bf16 hi / lo of the weighted h
  uint16_t* hq;    // instead of hb (a pass over every pair, no order): [q][2][r_pad] by grouped position
  float* hout;     // instead of hb: the unscaled h of grouped position q, [q][r_pad] fp32
  int kslices, cslices;
  FinishArgs fin;  // the expand's first nfin8 workgroups finish the tokens the pass skips
  int nfin8;       // a multiple of 8, so the other workgroups keep their XCDs
};

constexpr int gs_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Finishing workgroup blk: tokens [blk * kFinishTok, + kFinishTok), a wave per 64; a token to
// finish is copied by its whole wave (row dtypes chosen at run time: these rows are few).
__device__ void finish_rows(const FinishArgs& f, int blk) {
  const int lane = threadIdx.x & 63;
  const int base = (blk * (kFinishTok / kWave) + (int)(threadIdx.x >> 6)) * kWave;
  const int t = base + lane;
  int c = 0;
  if (t < f.N)
    for (int j = 0; j < f.k; ++j) c += f.inv[(long long)t * f.k + j] >= 0 ? 1 : 0;
  uint64_t m = __ballot(t < f.N && ((f.copy_y0 && c == 0) || (f.copy_z && c > 0 && c < f.c_last)));
  while (m) {
    const int l = __builtin_ctzll(m);
    m &= m - 1;
    const int tt = base + l;
    const bool from_y0 = __shfl(c, l, kWave) == 0;
    for (int col = lane * 4; col < f.d_out; col += kWave * 4) {
      float v[4];
      const size_t o = (size_t)tt * f.d_out + col;
      if (!from_y0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = f.z[o + i];
      } else if (f.y0_f32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const float*>(f.y0)[o + i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = bf16_to_f32(reinterpret_cast<const uint16_t*>(f.y0)[o + i]);
      }
      if (f.y_f32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) reinterpret_cast<float*>(f.y)[o + i] = v[i];
      } else {
        uint32_t* p = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(f.y) + o);
        p[0] = pack_bf16x2(v[0], v[1]);
        p[1] = pack_bf16x2(v[2], v[3]);
      }
    }
  }
}

// Tile and slice of workgroup b, for `slices` slices per tile (grid nwg * slices).
__device__ __forceinline__ void gs_tile_slice(const GMArgs& g, int slices, int& w, int& sl, int b = blockIdx.x) {
  const int xcd = b & 7, q = b >> 3;
  w = xcd * (g.nwg >> 3) + q / slices;
  sl = q % slices;
}

// Token of row rl of tile rows [r0, r0 + nrows) (rows past the end repeat the first).
__device__ __forceinline__ int gs_token(const GMArgs& g, int r0, int nrows, int rl) {
  const int rr = r0 + (rl < nrows ? rl : 0);
  const int q = g.order != nullptr ? g.order[rr] : rr;
  return g.perm[q] / g.k;
}

// One adapter's A slice against the x rows of one tile, or of two tiles of that adapter (TWO):
// every A operand read from LDS then feeds both tiles' MFMAs, so a workgroup streams the slice
// once for up to 128 rows.  The two halves of the slice's steps meet in LDS; half 0 stores the
// partials of each tile at part[tile][slice].
template <int RB, bool INDIRECT, bool TWO>
__device__ __forceinline__ void gs_shrink_rows(const GSArgs& a, uint16_t* As, int e, int sl, const int (&wt)[2],
                                               const int (&r0)[2], const int (&nrows)[2]) {
  constexpr int T = TWO ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4, rb = wave & 3, kh = wave >> 2;
  const int d_in = a.g.tgt.d_in, r_pad = a.g.tgt.r_pad;
  const int S = d_in / kStepK;
  const int s0 = sl * kGSSteps, s1 = min(s0 + kGSSteps, S), ns = s1 - s0;
  constexpr int piece = RB * 16 * kStepK;  // elements of one step's pieces
  // the x rows of the lane's MFMA row (16 rb + n) in each tile: tokens first (the HBM stream waits on them)
  const uint16_t* xp[T];
#pragma unroll
  for (int t = 0; t < T; ++t) xp[t] = a.g.x + (size_t)gs_token(a.g, r0[t], nrows[t], 16 * rb + n) * d_in + 8 * G;
  __builtin_amdgcn_sched_barrier(0);
  // the adapter's A slice straight into LDS
  {
    const char* src = reinterpret_cast<const char*>(adapter_A<INDIRECT>(a.g.tgt, e) + (size_t)s0 * piece);
    char* dst = reinterpret_cast<char*>(As);
    for (int off = wave * 1024; off < ns * piece * 2; off += 8 * 1024)
      __builtin_amdgcn_global_load_lds(src + off + 16 * lane, dst + off, 16, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // this wave's half of the slice (2 steps) of each x row
  const int w0 = min(s0 + 2 * kh, s1), w1 = min(w0 + 2, s1);
  u32x4_t xv[T][2][4];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int st = max(min(w0 + i, w1 - 1), s0);
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[t][i][c] = ld16_nt(xp[t] + (size_t)st * kStepK + 32 * c);
    }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(gs_vmcnt(8 * T));  // this wave's A pieces have landed (only x is younger)
  __syncthreads();
  f32x4_t acc[T][RB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int u = 0; u < RB; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (w0 + i < w1) {
      const uint16_t* ap = As + (size_t)(w0 + i - s0) * piece;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          // lane (n, G) takes its 16 bytes at position 4n + G of the 1 KB piece (slab swizzle)
          const u32x4_t av = *reinterpret_cast<const u32x4_t*>(ap + ((c * RB + u) * 64 + 4 * n + G) * 8);
#pragma unroll
          for (int t = 0; t < T; ++t) acc[t][u] = mfma16x16x32(as_bf16x8(xv[t][i][c]), as_bf16x8(av), acc[t][u]);
        }
    }
  }
  // the halves meet in LDS (the A pieces' bytes); half 0 stores the sums
  __syncthreads();
  constexpr int kRS = RB * 16 + 4;
  float* red = reinterpret_cast<float*>(As);
  static_assert(sizeof(float) * 2 * 4 * 16 * kRS <= sizeof(uint16_t) * kGSSteps * 4 * RB * 512,
                "two tiles' partial sums fit in the A pieces' LDS");
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((t * 4 + rb) * 16 + 4 * G + i) * kRS + u * 16 + n] = acc[t][u][i];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float* dst = a.part + (((size_t)wt[t] * a.kslices + sl) * kGMRows + 16 * rb) * r_pad;
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(size_t)(4 * G + i) * r_pad + u * 16 + n] =
              acc[t][u][i] + red[((t * 4 + rb) * 16 + 4 * G + i) * kRS + u * 16 + n];
    }
  }
}

// Workgroup = tiles (2j, 2j + 1) of its XCD's run x one 512-wide d_in slice (grid nwg / 2 x
// kslices; nwg a multiple of 16).  Two tiles of one adapter share the A slice; a pair that
// straddles two adapters runs one tile after the other.
template <int RB, bool INDIRECT>
__global__ __launch_bounds__(kGSThreads, 2) void gs_shrink(const GSArgs a) {
  __shared__ alignas(16) uint16_t As[kGSSteps * 4 * RB * 512];  // [step][chunk][u] pieces of 1 KB
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int j = q / a.kslices, sl = q - j * a.kslices;
  const int wa = xcd * (a.g.nwg >> 3) + 2 * j;
  int ea, ra0, ra1, eb, rb0, rb1;
  if (!gm_locate(a.g, wa, ea, ra0, ra1)) return;
  const bool hasb = gm_locate(a.g, wa + 1, eb, rb0, rb1);
  if (hasb && eb == ea) {
    gs_shrink_rows<RB, INDIRECT, true>(a, As, ea, sl, {wa, wa + 1}, {ra0, rb0}, {ra1 - ra0, rb1 - rb0});
    return;
  }
  gs_shrink_rows<RB, INDIRECT, false>(a, As, ea, sl, {wa, 0}, {ra0, 0}, {ra1 - ra0, 1});
  if (hasb) {
    __syncthreads();  // every wave has read its partial sums out of the A pieces' LDS
    gs_shrink_rows<RB, INDIRECT, false>(a, As, eb, sl, {wa + 1, 0}, {rb0, 0}, {rb1 - rb0, 1});
  }
}

template <int RB>
__global__ __launch_bounds__(kGSThreads) void gs_finalize(const GSArgs a) {
  constexpr int RP = RB * 16, RQ = RP / 4;
  constexpr int QPT = (kGMRows * RQ + kGSThreads - 1) / kGSThreads;  // 16-byte quads per thread
  constexpr int KS = 8;                                               // slices requested together
  int w, sl, e, r0, r1;
  gs_tile_slice(a.g, 1, w, sl);
  if (!gm_locate(a.g, w, e, r0, r1)) return;
  const int nrows = r1 - r0;
  const float* base = a.part + (size_t)w * a.kslices * kGMRows * RP;
  uint16_t* hb = a.hb != nullptr ? a.hb + (size_t)w * 2 * kGMRows * RP : nullptr;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int v = j * kGSThreads + (int)threadIdx.x;
    if (v >= kGMRows * RQ) break;
    const int row = v / RQ, rk = 4 * (v % RQ);
    const float wt = a.hout != nullptr ? 1.f : row < nrows ? a.g.wts[r0 + row] * a.g.scale : 0.f;
    const float* src = base + (size_t)row * RP + rk;
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.kslices; s0 += KS) {
      u32x4_t pv[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        if (s0 + s < a.kslices) pv[s] = ld16(src + (size_t)(s0 + s) * kGMRows * RP);
#pragma unroll
      for (int s = 0; s < KS; ++s)
        if (s0 + s < a.kslices)
#pragma unroll
          for (int c = 0; c < 4; ++c) sum[c] += __uint_as_float(pv[s][c]);
    }
    if (a.hout != nullptr) {
      if (row < nrows)
        *reinterpret_cast<u32x4_t*>(a.hout + (size_t)(r0 + row) * RP + rk) =
            u32x4_t{__float_as_uint(sum[0]), __float_as_uint(sum[1]), __float_as_uint(sum[2]), __float_as_uint(sum[3])};
      continue;
    }
    uint32_t hi2[2], lo2[2];
#pragma unroll
    for (int c = 0; c < 4; c += 2) {
      float hv[2], lv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        hv[t] = sum[c + t] * wt;
        lv[t] = hv[t] - (float)(__bf16)hv[t];
      }
      hi2[c / 2] = pack_bf16x2(hv[0], hv[1]);
      lo2[c / 2] = pack_bf16x2(lv[0], lv[1]);
    }
    if (a.hq != nullptr) {
      if (row < nrows) {
        uint16_t* hq = a.hq + (size_t)(r0 + row) * 2 * RP + rk;
        *reinterpret_cast<uint2*>(hq) = make_uint2(hi2[0], hi2[1]);
        *reinterpret_cast<uint2*>(hq + RP) = make_uint2(lo2[0], lo2[1]);
      }
    } else {
      *reinterpret_cast<uint2*>(hb + (size_t)row * RP + rk) = make_uint2(hi2[0], hi2[1]);
      *reinterpret_cast<uint2*>(hb + (size_t)(kGMRows + row) * RP + rk) = make_uint2(lo2[0], lo2[1]);
    }
  }
}

template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kGSThreads, 2) void gs_expand(const GSArgs a) {
  constexpr int RP = RB * 16, SPR = 2 * RB;  // 16-byte slots per B^T row
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  constexpr int NY0 = Y0F32 ? 16 : 8;
  __shared__ alignas(16) uint16_t Bs[kBSlice * RP];  // B^T rows of the slice, XOR-placed slots
  if ((int)blockIdx.x < a.nfin8) {
    finish_rows(a.fin, blockIdx.x);
    return;
  }
  int w, cs, e, r0, r1;
  gs_tile_slice(a.g, a.cslices, w, cs, blockIdx.x - a.nfin8);
  if (!gm_locate(a.g, w, e, r0, r1)) return;
  const int nrows = r1 - r0;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4, rb = wave & 3, ch = wave >> 2;
  const int d_out = a.g.tgt.d_out;
  const int c0 = cs * kBSlice, c1 = min(c0 + kBSlice, d_out);
  const int nb = (c1 - c0) / kColBlock;
  const int b0 = min(2 * ch, nb - 1), b1 = min(2 * ch + 1, nb - 1);
  const bool has0 = 2 * ch < nb, has1 = 2 * ch + 1 < nb;
  // 0. the tokens of the lane's rows 4G + i of its row block (rows past the tile repeat its
  //    first and are not stored): first, since the y0 stream waits on them
  const int tokl = gs_token(a.g, r0, nrows, 16 * rb + n);
  const char* y0rows[4];
  char* yrows[4];
  unsigned vmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = __shfl(tokl, 4 * G + i, kWave);
    y0rows[i] = reinterpret_cast<const char*>(a.g.y0) + (size_t)t * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(a.g.y) + (size_t)t * d_out * yb;
    vmask |= (16 * rb + 4 * G + i < nrows ? 1u : 0u) << i;
  }
  __builtin_amdgcn_sched_barrier(0);
  // 1. the B^T slice: LDS slot P (row P / SPR, slot P % SPR) holds the row's slot P % SPR XOR
  //    gm_b_swz(row), so lane l of a 1 KB piece fetches the source slot that belongs at l
  {
    const char* src = reinterpret_cast<const char*>(adapter_B<INDIRECT>(a.g.tgt, e) + (size_t)c0 * RP);
    char* dst = reinterpret_cast<char*>(Bs);
    const int npieces = (c1 - c0) * SPR / 64;
    for (int p = wave; p < npieces; p += 8) {
      const int P = 64 * p + lane, row = P / SPR, slot = (P % SPR) ^ gm_b_swz<RB>(row);
      __builtin_amdgcn_global_load_lds(src + ((size_t)row * SPR + slot) * 16, dst + (size_t)p * 1024, 16, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // 2. the A operand: h rows of the tile (groups 0, 1 hi of ranks 16u + 8(G & 1) .., 2, 3 lo)
  u32x4_t hv[RB];
  {
    const uint16_t* hrow = a.hb + ((size_t)w * 2 * kGMRows + (size_t)(G >> 1) * kGMRows + 16 * rb + n) * RP;
#pragma unroll
    for (int u = 0; u < RB; ++u) hv[u] = ld16(hrow + u * 16 + 8 * (G & 1));
  }
  __builtin_amdgcn_sched_barrier(0);
  // 3. the y0 rows
  RowChunk<Y0F32> yc0, yc1;
  load_row_chunk<Y0F32>(yc0, y0rows, c0 + b0 * kColBlock, n);
  load_row_chunk<Y0F32>(yc1, y0rows, c0 + b1 * kColBlock, n);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(gs_vmcnt(NY0));  // B pieces and h rows have landed (y0 may not)
  __syncthreads();
  // lane's B^T slots: row 16j + n of the block, slot 2u + (G & 1), XOR-placed
  int b_sl[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) b_sl[u] = (2 * u + (G & 1)) ^ gm_b_swz<RB>(n);
  // the two column blocks one after the other (one set of accumulators: two workgroups per CU)
  auto block = [&](int b, const RowChunk<Y0F32>& yc, bool hs) {
    const uint16_t* bl = Bs + (size_t)(b * kColBlock + n) * RP;
    f32x4_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(bl + (size_t)16 * j * RP + 8 * b_sl[u]);
        o[j] = mfma16x16x32(as_bf16x8(hv[u]), as_bf16x8(v), o[j]);
      }
    if (hs) epilogue_store<Y0F32, YF32>(o, yc, yrows, c0 + b * kColBlock, n, vmask);
  };
  block(b0, yc0, has0);
  block(b1, yc1, has1);
}

// ---- pair passes (k > 1): pass m applies a token's routed pairs of rank 2m and 2m + 1 in one
// tile row.  The shrink and finalize above run once over every pair in the dispatch's grouped
// order and leave h by grouped position (hq); the tuple sort lists each pass's tokens by the
// adapter pair (a, b) of those two pairs (b = K: the token has no pair of rank 2m + 1); the
// pair expand cuts each key's rows into tiles like any other pass and applies
// y = src + h_a B_a + h_b B_b (the two products summed in the MFMA accumulators, in that order).
// A row's result does not depend on the other rows of its tile, so the order of a key's rows
// (the sort is not stable) leaves every output bit unchanged.

constexpr int kTSThreads = kTupleWGTokens;
constexpr int kTCols = 2 * kColBlock;  // pair expand: output columns per workgroup

struct TupleSortArgs {
  const int32_t* offsets;  // the dispatch's offsets [K + 1]
  const int32_t* inv;      // pair -> grouped position (-1: unrouted)
  int N, k, K, nkeys;      // nkeys = passes x K (K + 1)
  int m2, kk;              // passes, keys per pass
  int tile_rows, fixed;    // the expand's tiling (GMTiling)
  int tmax;                // tile entries per pass
  int32_t* bcnt;           // [gridDim][nkeys]: the workgroup's counts, then its first positions
  int32_t* toff;           // [nkeys + 1]
  int4* tiles;             // [m2][tmax]: (key in the pass, first row, end row, 0)
  int32_t* ntile;          // [m2]
  int32_t* etok;
  int32_t* eqa;
  int32_t* eqb;
};

// f(key, q_a, q_b) for every pass of token t: its routed pairs ordered by adapter (equal
// adapters by slot), taken two by two, so the keys of a pass concentrate on fewer adapter
// pairs than in rank order.  Registers only: k <= MOLORA_MAX_TOPK, every loop unrolled.
template <typename F>
__device__ __forceinline__ void token_tuples(const TupleSortArgs& a, const int* offs, int t, F f) {
  constexpr int KM = MOLORA_MAX_TOPK;
  const int K1 = a.K + 1, KK = a.K * K1;
  int ev[KM], qv[KM], pos[KM];
  int c = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int q = j < a.k ? a.inv[(long long)t * a.k + j] : -1;
    qv[j] = q;
    ev[j] = q >= 0 ? segment_of(offs, a.K, q) : INT_MAX;  // unrouted pairs sort last
    c += q >= 0 ? 1 : 0;
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    int p = 0;
#pragma unroll
    for (int i = 0; i < KM; ++i) p += (ev[i] < ev[j] || (ev[i] == ev[j] && i < j)) ? 1 : 0;
    pos[j] = p;
  }
#pragma unroll
  for (int m = 0; m < KM / 2; ++m) {
    if (2 * m >= c) break;
    int ea = 0, qa = -1, eb = a.K, qb = -1;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (pos[j] == 2 * m) { ea = ev[j]; qa = qv[j]; }
      if (pos[j] == 2 * m + 1 && 2 * m + 1 < c) { eb = ev[j]; qb = qv[j]; }
    }
    f(m * KK + ea * K1 + eb, qa, qb);
  }
}

// LDS: offs [K + 1], then one counter per key
__global__ __launch_bounds__(kTSThreads) void tuple_count(const TupleSortArgs a) {
  extern __shared__ int ts_lds[];
  int* offs = ts_lds;
  int* cnt = ts_lds + a.K + 1;
  for (int i = threadIdx.x; i <= a.K; i += kTSThreads) offs[i] = a.offsets[i];
  for (int i = threadIdx.x; i < a.nkeys; i += kTSThreads) cnt[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * kTSThreads + (int)threadIdx.x;
  if (t < a.N) token_tuples(a, offs, t, [&](int key, int, int) { atomicAdd(&cnt[key], 1); });
  __syncthreads();
  for (int i = threadIdx.x; i < a.nkeys; i += kTSThreads) a.bcnt[(size_t)blockIdx.x * a.nkeys + i] = cnt[i];
}

// One workgroup: thread i owns a run of consecutive keys; toff = exclusive scan of the key
// totals, and bcnt[b][key] becomes workgroup b's first position in the key.
__global__ __launch_bounds__(kTSThreads) void tuple_scan(const TupleSortArgs a, int nb) {
  __shared__ int wsum[kTSThreads / kWave];
  const int per = (a.nkeys + kTSThreads - 1) / kTSThreads;
  const int k0 = min((int)threadIdx.x * per, a.nkeys), k1 = min(k0 + per, a.nkeys);
  constexpr int CH = 16;  // counts requested together (their loads do not wait on each other)
  int tot = 0;
  for (int key = k0; key < k1; ++key)
    for (int b0 = 0; b0 < nb; b0 += CH) {
      int cv[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) cv[j] = b0 + j < nb ? a.bcnt[(size_t)(b0 + j) * a.nkeys + key] : 0;
#pragma unroll
      for (int j = 0; j < CH; ++j) tot += cv[j];
    }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(tot, lane);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int pos = incl - tot;
  for (int w = 0; w < wave; ++w) pos += wsum[w];
  for (int key = k0; key < k1; ++key) {
    a.toff[key] = pos;
    for (int b0 = 0; b0 < nb; b0 += CH) {
      int cv[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) cv[j] = b0 + j < nb ? a.bcnt[(size_t)(b0 + j) * a.nkeys + key] : 0;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        if (b0 + j < nb) a.bcnt[(size_t)(b0 + j) * a.nkeys + key] = pos;
        pos += cv[j];
      }
    }
  }
  if (threadIdx.x == kTSThreads - 1) a.toff[a.nkeys] = pos;  // the last thread ends at the total
  __syncthreads();
  // each pass's tiles: key c rows -> nt = ceil(c / tile_rows) tiles, balanced (the first c % nt
  // tiles one row taller) or fixed (tile_rows rows but the last), numbered key by key; thread i
  // takes a run of consecutive keys of the pass
  const int M = a.tile_rows;
  const int per2 = (a.kk + kTSThreads - 1) / kTSThreads;
  for (int m = 0; m < a.m2; ++m) {
    const int q0 = min((int)threadIdx.x * per2, a.kk), q1 = min(q0 + per2, a.kk);
    int nt = 0, sq[2], cq[2];  // per2 <= 2: K (K + 1) <= 2 kTSThreads
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = q0 + j;
      sq[j] = q < q1 ? a.toff[m * a.kk + q] : 0;
      cq[j] = q < q1 ? a.toff[m * a.kk + q + 1] - sq[j] : 0;
      nt += (cq[j] + M - 1) / M;
    }
    const int tincl = wave_incl_scan(nt, lane);
    __syncthreads();  // wsum's previous readers are done
    if (lane == kWave - 1) wsum[wave] = tincl;
    __syncthreads();
    int w = tincl - nt;
    for (int v = 0; v < wave; ++v) w += wsum[v];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = q0 + j, s0 = sq[j], c = cq[j];
      const int ntq = (c + M - 1) / M;  // 0 past the run
      const int h = a.fixed ? M : (ntq > 0 ? c / ntq : 0), rem = a.fixed ? 0 : c - h * max(ntq, 1);
      int r0 = s0;
      for (int i = 0; i < ntq; ++i, ++w) {
        const int r1 = min(s0 + c, r0 + h + (i < rem ? 1 : 0));
        a.tiles[(size_t)m * a.tmax + w] = make_int4(q, r0, r1, 0);
        r0 = r1;
      }
    }
    if (threadIdx.x == kTSThreads - 1) a.ntile[m] = w;  // the last thread ends at the pass's count
  }
}

__global__ __launch_bounds__(kTSThreads) void tuple_scatter(const TupleSortArgs a) {
  extern __shared__ int ts_lds[];
  int* offs = ts_lds;
  int* cur = ts_lds + a.K + 1;
  for (int i = threadIdx.x; i <= a.K; i += kTSThreads) offs[i] = a.offsets[i];
  for (int i = threadIdx.x; i < a.nkeys; i += kTSThreads) cur[i] = a.bcnt[(size_t)blockIdx.x * a.nkeys + i];
  __syncthreads();
  const int t = blockIdx.x * kTSThreads + (int)threadIdx.x;
  if (t < a.N)
    token_tuples(a, offs, t, [&](int key, int qa, int qb) {
      const int p = atomicAdd(&cur[key], 1);
      a.etok[p] = t;
      a.eqa[p] = qa;
      a.eqb[p] = qb;
    });
}

struct TupleArgs {
  FinishArgs fin;  // the first nfin8 workgroups finish the tokens the pass skips
  int nfin8;       // a multiple of 8, so the other workgroups keep their XCDs
  GMArgs g;  // the pass: target, y0 / y (g.nwg: the grid's tile slots, a multiple of 8)
  const int4* tiles;     // the pass's tiles (key in the pass, first row, end row)
  const int32_t* ntile;  // the pass's tile count
  const int32_t* etok;
  const int32_t* eqa;
  const int32_t* eqb;
  const uint16_t* hq;  // [P][2][r_pad] bf16 hi / lo of gate weight x alpha/r x h by grouped position
  int K1;              // K + 1
  int cslices;         // 256-wide column slices
};

// Workgroup = one tile (up to kPairTileRows = 128 rows) x one 256-wide d_out slice; wave w takes
// row block w and both 128-column blocks of the slice, one after the other.  The tiles are spread over the XCDs in runs of ceil(count / 8)
// consecutive tiles (mostly of one first adapter), so each XCD's L2 holds few B^T slices.  The
// B^T slices of a (and b) go straight into LDS in the XOR placement, the rows' h operands and
// y0 rows are requested behind them.
template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kGSThreads, 4) void gs_expand_pairs(const TupleArgs a) {
  constexpr int RP = RB * 16, SPR = 2 * RB;  // 16-byte slots per B^T row
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  constexpr int NY0 = Y0F32 ? 8 : 4;
  __shared__ alignas(16) uint16_t Bs[2][kTCols * RP];
  if ((int)blockIdx.x < a.nfin8) {
    finish_rows(a.fin, blockIdx.x);
    return;
  }
  const int bid = blockIdx.x - a.nfin8;
  const int nt = *a.ntile, per = (nt + 7) / 8;
  const int q = bid >> 3, wl = q / a.cslices, cs = q - wl * a.cslices;
  const int w = (bid & 7) * per + wl;
  if (wl >= per || w >= nt) return;
  const int4 tl = a.tiles[w];
  const int e = tl.x, r0 = tl.y, r1 = tl.z;
  const int ea = e / a.K1, eb = e - ea * a.K1;
  const bool hasb = eb < a.K1 - 1;  // the same in every lane
  const int nrows = r1 - r0;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4, rb = wave;  // 8 row blocks of 16 rows
  const int d_out = a.g.tgt.d_out;
  const int c0 = cs * kTCols, c1 = min(c0 + kTCols, d_out);
  const int nb = (c1 - c0) / kColBlock;  // 1 or 2 column blocks, both taken by every wave
  // 0. the entry of the lane's MFMA row 16 rb + n (rows past the tile repeat its first and are
  //    not stored): first, since the h and y0 streams wait on it
  const int rl = 16 * rb + n, rr = r0 + (rl < nrows ? rl : 0);
  const int tokl = a.etok[rr];
  const int qal = a.eqa[rr];
  const int qbl = hasb ? a.eqb[rr] : qal;
  const char* y0rows[4];
  char* yrows[4];
  unsigned vmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = __shfl(tokl, 4 * G + i, kWave);
    y0rows[i] = reinterpret_cast<const char*>(a.g.y0) + (size_t)t * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(a.g.y) + (size_t)t * d_out * yb;
    vmask |= (16 * rb + 4 * G + i < nrows ? 1u : 0u) << i;
  }
  // the lane's h rows: groups 0, 1 hi of ranks 16u + 8(G & 1) .., groups 2, 3 lo (addresses
  // formed here, so the loads below wait on nothing)
  const uint16_t* pa = a.hq + ((size_t)qal * 2 + (G >> 1)) * RP + 8 * (G & 1);
  const uint16_t* pb = a.hq + ((size_t)qbl * 2 + (G >> 1)) * RP + 8 * (G & 1);
  __builtin_amdgcn_sched_barrier(0);
  // 1. the B^T slices: LDS slot P (row P / SPR) holds the row's slot P % SPR XOR gm_b_swz(row)
  {
    const int npieces = (c1 - c0) * SPR / 64;
    for (int h = 0; h < (hasb ? 2 : 1); ++h) {
      const char* src = reinterpret_cast<const char*>(adapter_B<INDIRECT>(a.g.tgt, h ? eb : ea) + (size_t)c0 * RP);
      char* dst = reinterpret_cast<char*>(Bs[h]);
      for (int p = wave; p < npieces; p += 8) {
        const int P = 64 * p + lane, row = P / SPR, slot = (P % SPR) ^ gm_b_swz<RB>(row);
        __builtin_amdgcn_global_load_lds(src + ((size_t)row * SPR + slot) * 16, dst + (size_t)p * 1024, 16, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // 2. the A operands
  u32x4_t hva[RB], hvb[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) hva[u] = ld16(pa + u * 16);
#pragma unroll
  for (int u = 0; u < RB; ++u) hvb[u] = ld16(pb + u * 16);
  __builtin_amdgcn_sched_barrier(0);
  // 3. the y0 rows of both column blocks
  //    (fp32 rows: the second block's after the first block's MFMAs, which keeps the kernel at
  //    128 VGPRs, two workgroups per CU)
  RowChunk<Y0F32> yc0, yc1;
  load_row_chunk<Y0F32>(yc0, y0rows, c0, n);
  if constexpr (!Y0F32) load_row_chunk<Y0F32>(yc1, y0rows, c0 + min(1, nb - 1) * kColBlock, n);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(gs_vmcnt(Y0F32 ? NY0 : 2 * NY0));  // B pieces and h rows have landed (y0 may not)
  __syncthreads();
  int b_sl[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) b_sl[u] = (2 * u + (G & 1)) ^ gm_b_swz<RB>(n);
  // the two column blocks one after the other (one set of accumulators)
  auto block = [&](int blk, const RowChunk<Y0F32>& yc) {
    const size_t roff = (size_t)(blk * kColBlock + n) * RP;
    f32x4_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Bs[0] + roff + (size_t)16 * j * RP + 8 * b_sl[u]);
        o[j] = mfma16x16x32(as_bf16x8(hva[u]), as_bf16x8(v), o[j]);
      }
    if (hasb) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Bs[1] + roff + (size_t)16 * j * RP + 8 * b_sl[u]);
          o[j] = mfma16x16x32(as_bf16x8(hvb[u]), as_bf16x8(v), o[j]);
        }
    }
    epilogue_store<Y0F32, YF32>(o, yc, yrows, c0 + blk * kColBlock, n, vmask);
  };
  block(0, yc0);
  if (nb > 1) {
    if constexpr (Y0F32) load_row_chunk<Y0F32>(yc1, y0rows, c0 + kColBlock, n);
    block(1, yc1);
  }
}

}  // namespace

#define MOLORA_GS_RB(...)                                 \
  switch (g.tgt.r_pad / 16) {                             \
    case 1: { constexpr int RB = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int RB = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int RB = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int RB = 4; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                 \
  }
#define MOLORA_GS_BOOL(V, NAME, ...) \
  if (V) { constexpr bool NAME = true; __VA_ARGS__; } else { constexpr bool NAME = false; __VA_ARGS__; }

// gs_shrink over (tile, d_in slice), then gs_finalize per tile.
static hipError_t gs_shrink_finalize(const GMArgs& g, const GSArgs& a, bool indirect, hipStream_t s) {
  if (g.nwg % 16 != 0) return hipErrorInvalidValue;  // tile pairs within each XCD's run
  hipError_t err = hipSuccess;
  MOLORA_GS_RB(MOLORA_GS_BOOL(indirect, IND, {
    hipLaunchKernelGGL((gs_shrink<RB, IND>), dim3(g.nwg / 2 * a.kslices), dim3(kGSThreads), 0, s, a);
    err = hipGetLastError();
  }))
  if (err != hipSuccess) return err;
  MOLORA_GS_RB({
    hipLaunchKernelGGL((gs_finalize<RB>), dim3(g.nwg), dim3(kGSThreads), 0, s, a);
    err = hipGetLastError();
  })
  return err;
}

hipError_t launch_gs_pass(const GMArgs& g, float* part, uint16_t* hb, bool y0_f32, bool y_f32, bool indirect,
                          hipStream_t s, const FinishArgs* fin) {
  GSArgs a{};
  a.g = g;
  a.part = part;
  a.hb = hb;
  a.kslices = (g.tgt.d_in + kBSlice - 1) / kBSlice;
  a.cslices = (g.tgt.d_out + kBSlice - 1) / kBSlice;
  if (fin != nullptr) {
    a.fin = *fin;
    a.nfin8 = ((fin->N + kFinishTok - 1) / kFinishTok + 7) / 8 * 8;
  }
  hipError_t err = gs_shrink_finalize(g, a, indirect, s);
  if (err != hipSuccess) return err;
  MOLORA_GS_RB(MOLORA_GS_BOOL(indirect, IND, MOLORA_GS_BOOL(y0_f32, Y0F, MOLORA_GS_BOOL(y_f32, YF, {
    hipLaunchKernelGGL((gs_expand<RB, IND, Y0F, YF>), dim3(a.nfin8 + g.nwg * a.cslices), dim3(kGSThreads), 0, s, a);
    err = hipGetLastError();
  }))))
  return err;
}

hipError_t launch_gs_pair_shrink(const GMArgs& g, float* part, uint16_t* hq, bool indirect, hipStream_t s) {
  if (g.order != nullptr) return hipErrorInvalidValue;  // hq is indexed by the row's grouped position
  GSArgs a{};
  a.g = g;
  a.part = part;
  a.hq = hq;
  a.kslices = (g.tgt.d_in + kBSlice - 1) / kBSlice;
  a.cslices = 0;
  return gs_shrink_finalize(g, a, indirect, s);
}

hipError_t launch_pair_shrink_gm(const TargetDev& tgt, bool indirect, const uint16_t* x, const int32_t* offsets,
                                 const int32_t* perm, int K, int k, long long P, float* hout, float* part,
                                 hipStream_t s) {
  const int kslices = (tgt.d_in + kBSlice - 1) / kBSlice;
  const GMTiling tl = gm_tiling(kPathGrouped, P, K, kslices);
  GMArgs g{};
  g.tgt = tgt; g.x = x; g.k = k; g.perm = perm; g.offsets = offsets; g.key0 = 0; g.nkeys = K; g.order = nullptr;
  g.tile_rows = tl.rows; g.fixed = tl.fixed;
  g.nwg = gs_region(kPathGrouped, P, K, tgt.r_pad, tgt.d_in, false).nwg;
  GSArgs a{};
  a.g = g;
  a.part = part;
  a.hout = hout;
  a.kslices = kslices;
  return gs_shrink_finalize(g, a, indirect, s);
}

hipError_t launch_tuple_sort(const int32_t* offsets, const int32_t* inv, int N, int k, int K, char* region,
                             const TupleSortPlan& tp, const GMTiling& tl, hipStream_t s) {
  // the tile table holds ceil(N / 16) + keys per pass; the scan's threads take 2 keys of a pass at most
  if (tl.rows < 16 || tp.kk > 2 * kTSThreads) return hipErrorInvalidValue;
  TupleSortArgs a{};
  a.offsets = offsets;
  a.inv = inv;
  a.N = N; a.k = k; a.K = K; a.nkeys = tp.nkeys;
  a.m2 = tp.m2; a.kk = tp.kk;
  a.tile_rows = tl.rows; a.fixed = tl.fixed; a.tmax = tp.tmax;
  a.tiles = reinterpret_cast<int4*>(region + tp.tiles_off);
  a.ntile = reinterpret_cast<int32_t*>(region + tp.ntile_off);
  a.bcnt = reinterpret_cast<int32_t*>(region + tp.bcnt_off);
  a.toff = reinterpret_cast<int32_t*>(region + tp.toff_off);
  a.etok = reinterpret_cast<int32_t*>(region + tp.etok_off);
  a.eqa = reinterpret_cast<int32_t*>(region + tp.eqa_off);
  a.eqb = reinterpret_cast<int32_t*>(region + tp.eqb_off);
  const size_t lds = (size_t)(K + 1 + tp.nkeys) * sizeof(int);
  hipLaunchKernelGGL(tuple_count, dim3(tp.nb), dim3(kTSThreads), lds, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(tuple_scan, dim3(1), dim3(kTSThreads), 0, s, a, tp.nb);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(tuple_scatter, dim3(tp.nb), dim3(kTSThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_gs_expand_pairs(const GMArgs& g, const char* region, const TupleSortPlan& tp, int m,
                                  const uint16_t* hq, int K, bool y0_f32, bool y_f32, bool indirect, hipStream_t s,
                                  const FinishArgs* fin) {
  TupleArgs a{};
  a.g = g;
  if (fin != nullptr) {
    a.fin = *fin;
    a.nfin8 = ((fin->N + kFinishTok - 1) / kFinishTok + 7) / 8 * 8;
  }
  a.tiles = reinterpret_cast<const int4*>(region + tp.tiles_off) + (size_t)m * tp.tmax;
  a.ntile = reinterpret_cast<const int32_t*>(region + tp.ntile_off) + m;
  a.etok = reinterpret_cast<const int32_t*>(region + tp.etok_off);
  a.eqa = reinterpret_cast<const int32_t*>(region + tp.eqa_off);
  a.eqb = reinterpret_cast<const int32_t*>(region + tp.eqb_off);
  a.hq = hq;
  a.K1 = K + 1;
  a.cslices = (g.tgt.d_out + kTCols - 1) / kTCols;
  hipError_t err = hipSuccess;
  MOLORA_GS_RB(MOLORA_GS_BOOL(indirect, IND, MOLORA_GS_BOOL(y0_f32, Y0F, MOLORA_GS_BOOL(y_f32, YF, {
    hipLaunchKernelGGL((gs_expand_pairs<RB, IND, Y0F, YF>), dim3(a.nfin8 + g.nwg * a.cslices), dim3(kGSThreads), 0, s,
                       a);
    err = hipGetLastError();
  }))))
  return err;
}

#undef MOLORA_GS_RB
#undef MOLORA_GS_BOOL

}  // namespace molora
