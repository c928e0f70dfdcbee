// Grouped LoRA application on gfx950: shrink h = x_t A_e (d_in -> r), expand
// delta = h B_e (r -> d_out), and the gate-weighted, alpha/r-scaled add into y.
//
// MoLoRA pages (thelatestinai.com): Figure 2 (tokens grouped by selected adapter, a grouped
// GEMM, outputs combined by a weighted sum), Table 10 (A is (K, d, r), B is (K, r, d)),
// Figure 4 / Table 2 (hot-set adapters at fixed addresses, direct or indirect layout),
// Figure 5 / Figure 9 (a matrix-core kernel for large batches, a skinny kernel for small ones).
//
// Kernels (paths of molora_apply in brackets):
//   step_vocab         the whole vocabulary-routed step in one launch (k = 1): every workgroup
//                      routes its 8 tokens, applies them as apply_t8 does and writes its share
//                      of the dispatch outputs, counting all ids itself (no grid barrier).
//   apply_t8           [TILE] 8 consecutive tokens per workgroup (tile8_dev.h), every adapter
//                      the tile uses applied in turn; x / y0 / y rows depend only on the token
//                      index, so those streams start before the routing is known.
//   shrink_block, expand_block
//                      [BLOCK] 64-token blocks in two launches (block_dev.h): partial shrinks
//                      per 512-wide d_in slice into the workspace, then expands per 512-wide
//                      column slice; step_shrink_block / step_expand_block route from the ids.
//   gs_shrink, gs_finalize, gs_expand
//                      [GROUPED, rank > 32 or k > 1] one pass over the 64-row tiles of the
//                      grouped order (gm_dev.h tiling) in three launches split over 512-wide
//                      slices (gsplit.hip); k > 1 from 32 K (K + 1) tokens: pair passes, each
//                      applying two of a token's routed pairs (gs_expand_pairs over the tuple
//                      sort's tiles); below that slot_sort (or slot_hist + slot_scatter)
//                      orders the pairs by (rank among the token's pairs, adapter), one pass
//                      per rank.  Within a pass every token has at most one row, so no two
//                      workgroups write one row; the passes carry the sum in fp32 and leading
//                      workgroups of the last expand write the tokens it does not reach.
//   apply_fused_k1     [GROUPED, k = 1, rank <= 32] 16 grouped rows of one adapter (gathered
//                      through perm) and a slice of output columns; shrink and expand fused.
//   shrink_grouped     [SKINNY, GROUPED k > 1 with k*K > 64] the grouped shrink into an fp32
//                      workspace (weighted by gate and alpha/r), split over d_in, then
//   expand_grouped_k1  one adapter per token, or one pass per rank (k*K <= 64), or
//   expand_tokens      token-major over every adapter of a 16-token tile (k*K > 64), or
//   hsum_multi +       [SKINNY, k = 2..4, N <= 1024, K*r_pad <= 1024] the h rows by pair id,
//   expand_decode_multi then one launch over 32-column slices, every adapter's B^T slice in
//                      LDS and each token's routed pairs summed in registers.
//   *_multi            the same phases for several targets sharing one routing, one launch
//                      per phase (molora_apply_multi).
//   relayout_A / _B, seqpass_meta: hot-set layout and the per-sequence comparator's metadata.
//
// The shrink result h stays fp32 and enters the expand MFMA as a bf16 hi/lo pair
// (h = hi + lo to about 2^-17 relative).  Workgroups that share x rows are numbered so that
// they run back to back on the same XCD (block b runs on XCD b % 8) and share its L2.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "dispatch_dev.h"
#include "molora_launch.h"
#include "molora_mfma.h"
#include "tile8_dev.h"
#include "block_dev.h"
#include "gm_dev.h"

namespace molora {

constexpr int kWaves8 = 8;    // waves per workgroup of the fused kernels
constexpr int kPrefetch = 2;  // expand blocks per wave whose y0 is requested up front
static_assert(kT8MaxU == kApplyTileMaxAdapters, "tile path adapter bound");

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
// Token-major 8-token tiles (any k, K <= 16): the routing of a tile's pairs comes from the
// dispatch outputs (inv gives the grouped position q of pair p, offsets its adapter, perm_w
// its gate weight).  The inverse-permutation loads are issued before the x / y0 streams; the
// gate-weight loads after them (they are first needed after the shrink).
struct T8ApplyArgs {
  T8Args t;
  const int32_t* offsets;
  const float* perm_w;
  const int32_t* inv;
};

template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kT8Threads) void apply_t8(T8ApplyArgs a) {
  __shared__ T8Lds<RB> L;
  int tt, g;
  t8_tile_of_block(blockIdx.x, a.t, tt, g);
  if (tt >= a.t.tiles) return;
  const int lane = threadIdx.x & 63;
  const int k = a.t.k, K = a.t.K;
  // lane l < 8k: pair (token t0 + l / k, slot l % k), tokens past N - 1 cloned from N - 1;
  // the small loads go first, unconditionally, so that the later waits on them are exact
  const int tc = min(tt * kT8Tokens + lane / k, a.t.N - 1);
  const bool mine = lane < kT8Tokens * k;
  const int qv = a.inv[(long long)tc * k + lane % k];
  const int ov = a.offsets[min(lane, K)];  // lane i holds offsets[i]
  T8Stream<RB, Y0F32> st;
  t8_prefetch<RB, Y0F32, YF32>(a.t, tt, g, st);
  // adapter of grouped position q: the number of segment starts offsets[1 .. K-1] at or below q
  const int q = mine ? qv : -1;
  int seg = 0;
  for (int i = 1; i < K; ++i) seg += (__shfl(ov, i, kWave) <= q) ? 1 : 0;
  const int pe = q >= 0 ? seg : -1;
  const float pw = q >= 0 ? a.perm_w[q] * a.t.scale : 0.f;
  t8_main<RB, INDIRECT, Y0F32, YF32>(a.t, L, st, pe, pw, [] {});
}

// --------------------------------------------------------------------------------------
// One launch of the vocabulary-routed step (k = 1).  Every workgroup routes its 8 tokens from
// their ids and applies the adapters, as apply_t8 does.  It also derives its share of the
// dispatch outputs without waiting for any other workgroup: it counts the adapters of all N
// tokens and of the tokens before its tile (the same range lookup on every id), which gives
// the offsets and each of its tokens' positions in the stable grouped order.  This runs after
// the apply body, while its stores drain.  Workgroups of column group 0 write their tokens'
// idx / w / inv / perm / perm_w; the first tile writes counts and offsets.
constexpr int kStepIdsPerThread = 4;  // ids held from the start: N <= 512 * 4 in one pass
constexpr int kSWavesMax = 8;         // waves of the workgroups that count ids

// Vocabulary ranges as kernel arguments: [lo, hi) is routed; the owner of v is the number of
// interior bounds b[1..K-1] at or below v (mid[i - 1] = b[i]; unused entries hold INT_MAX).
struct StepBounds {
  int lo, hi;
  int mid[kT8MaxU - 1];
};
__device__ __forceinline__ int step_owner(int v, const StepBounds& b) {
  int e = 0;
#pragma unroll
  for (int i = 0; i < kT8MaxU - 1; ++i) e += (v >= b.mid[i]) ? 1 : 0;
  return (v >= b.lo && v < b.hi) ? e : -1;
}

struct StepArgs {
  T8Args t;
  StepBounds bounds;
  const int32_t* ids;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  float* perm_w;
  int32_t* inv;
  int dispatch_share;  // the launches write idx .. inv (split: from per-block counts; tile: every
                       // workgroup counts all N ids itself)
};

struct StepLds {
  int gcnt[64];   // adapter counts over all tokens
  int pcnt[64];   // adapter counts over the tokens before the tile
  int offs[65];
};

// Count ids [c0 .. c0 + 512 * kStepIdsPerThread) (held in v) into gcnt and, for tokens below
// t0, pcnt.  Wave-level match masks make one LDS atomic per group of equal adapters.
__device__ __forceinline__ void step_count(StepLds& S, const StepBounds& bd, const int (&v)[kStepIdsPerThread],
                                           int c0, int N, int nbits, int t0) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lanemask_lt(lane);
#pragma unroll
  for (int j = 0; j < kStepIdsPerThread; ++j) {
    const int t = c0 + j * kT8Threads + threadIdx.x;
    const int e = t < N ? step_owner(v[j], bd) : -1;
    const bool valid = e >= 0;
    const uint64_t m = match_mask(e, valid, nbits);
    if (valid && (m & lt) == 0) atomicAdd(&S.gcnt[e], __popcll(m));
    const uint64_t mp = m & __ballot(t < t0);
    if (valid && t < t0 && (mp & lt) == 0) atomicAdd(&S.pcnt[e], __popcll(mp));
  }
}

// The same counts as step_count, with per-wave ballots per adapter (no LDS atomics while the
// ids are counted): wave w's counts of ids [c0 .. c0 + 512 * kStepIdsPerThread) land in
// wg[w][e] / wp[w][e] (tokens below t0); the caller sums the waves in order.
__device__ __forceinline__ void step_count_waves(int (&wg)[kSWavesMax][kT8MaxU], int (&wp)[kSWavesMax][kT8MaxU],
                                                 const StepBounds& bd, const int (&v)[kStepIdsPerThread], int c0,
                                                 int N, int K, int t0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int e[kStepIdsPerThread];
  uint64_t below[kStepIdsPerThread];
#pragma unroll
  for (int j = 0; j < kStepIdsPerThread; ++j) {
    const int t = c0 + j * (int)blockDim.x + (int)threadIdx.x;
    e[j] = t < N ? step_owner(v[j], bd) : -1;
    below[j] = __ballot(t < t0);
  }
#pragma unroll
  for (int ee = 0; ee < kT8MaxU; ++ee) {
    if (ee >= K) break;
    int cg = 0, cp = 0;
#pragma unroll
    for (int j = 0; j < kStepIdsPerThread; ++j) {
      const uint64_t m = __ballot(e[j] == ee);
      cg += __popcll(m);
      cp += __popcll(m & below[j]);
    }
    if (lane == 0) {
      wg[wave][ee] += cg;
      wp[wave][ee] += cp;
    }
  }
}

template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kT8Threads) void step_vocab(StepArgs a) {
  __shared__ T8Lds<RB> L;
  __shared__ StepLds S;
  int tt, g;
  t8_tile_of_block(blockIdx.x, a.t, tt, g);
  if (tt >= a.t.tiles) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = a.t.N, K = a.t.K;
  const int t0 = tt * kT8Tokens;
  // small loads first, unconditionally (indices clamped): the tile's ids (positions past N - 1
  // clone token N - 1), then this thread's share of the first 2048 ids
  if (threadIdx.x < 64) {
    S.gcnt[threadIdx.x] = 0;
    S.pcnt[threadIdx.x] = 0;
  }
  __syncthreads();  // counters cleared (before any load is in flight, so this costs nothing)
  const int tok = t0 + lane;
  const int myid = a.ids[min(tok, N - 1)];
  int dv[kStepIdsPerThread];
#pragma unroll
  for (int j = 0; j < kStepIdsPerThread; ++j) dv[j] = a.ids[min(j * kT8Threads + (int)threadIdx.x, N - 1)];
  T8Stream<RB, Y0F32> st;
  t8_prefetch<RB, Y0F32, YF32>(a.t, tt, g, st);
  const int pe = lane < kT8Tokens ? step_owner(myid, a.bounds) : -1;
  const float pw = pe >= 0 ? 1.0f * a.t.scale : 0.f;
  int nbits = 0;
  while ((1 << nbits) < K) ++nbits;
  // the dispatch counts run while the first adapter loads are in flight
  t8_main<RB, INDIRECT, Y0F32, YF32>(a.t, L, st, pe, pw, [&] {
    step_count(S, a.bounds, dv, 0, N, nbits, t0);
    for (int c0 = kStepIdsPerThread * kT8Threads; c0 < N; c0 += kStepIdsPerThread * kT8Threads) {
#pragma unroll
      for (int j = 0; j < kStepIdsPerThread; ++j) dv[j] = a.ids[min(c0 + j * kT8Threads + (int)threadIdx.x, N - 1)];
      step_count(S, a.bounds, dv, c0, N, nbits, t0);
    }
  });

  // dispatch share: offsets, then this tile's tokens' grouped positions
  __syncthreads();
  if (wave == 0) {
    const int c = lane < K ? S.gcnt[lane] : 0;
    const int incl = wave_incl_scan(c, lane);
    if (lane < K) S.offs[lane] = incl - c;
    if (tt == 0 && g == 0) {
      if (lane < K) {
        a.counts[lane] = c;
        a.offsets[lane + 1] = incl;
      }
      if (lane == 0) a.offsets[0] = 0;
    }
  }
  __syncthreads();
  if (wave == 0 && g == 0) {
    // the tile's tokens in lanes 0..7: rank among the tile's earlier tokens of the same adapter
    const bool real = tok < N;
    const bool valid = real && pe >= 0;
    const uint64_t m = match_mask(pe, valid, nbits);
    if (lane < kT8Tokens && real) {
      a.idx[tok] = pe;
      a.w[tok] = valid ? 1.0f : 0.0f;
      if (valid) {
        const int pos = S.offs[pe] + S.pcnt[pe] + __popcll(m & lanemask_lt(lane));
        a.inv[tok] = pos;
        a.perm[pos] = tok;
        a.perm_w[pos] = 1.0f;
      } else {
        a.inv[tok] = -1;
      }
    }
  }
}

// --------------------------------------------------------------------------------------
// 64-token blocks, shrink launch then expand launch (any k, K <= 16): routing from
// the dispatch outputs.  Lane i of a wave holds offsets[i]; the adapter of grouped position q
// is the number of segment starts offsets[1 .. K-1] at or below q.
struct BlockApplyArgs {
  BlockArgs b;
  const int32_t* offsets;
  const float* perm_w;
  const int32_t* inv;
};

struct DispatchRoute {
  const int32_t* inv;
  const float* perm_w;
  int k, K;
  float scale;
  int ov;  // offsets[lane]
  __device__ __forceinline__ int operator()(int t, int s, float& w) const {
    const int q = inv[(long long)t * k + s];
    int seg = 0;
    for (int i = 1; i < K; ++i) seg += (__shfl(ov, i, kWave) <= q) ? 1 : 0;
    w = q >= 0 ? perm_w[q] * scale : 0.f;
    return q >= 0 ? seg : -1;
  }
};

// Block and slice of workgroup b: every slice of block tb runs on XCD tb mod 8 (workgroups are
// dispatched round robin over the XCDs; a launch has 8 * ceil(nblocks / 8) * slices of them),
// so the expand finds the partials that the shrink wrote in the same L2.
__device__ __forceinline__ bool block_slice_of(int b, int nblocks, int slices, int& tb, int& sl) {
  const int q = b >> 3;
  tb = (q / slices) * 8 + (b & 7);
  sl = q % slices;
  return tb < nblocks;
}
__host__ inline int block_grid(int nblocks, int slices) { return 8 * ((nblocks + 7) / 8) * slices; }

template <int RB, bool INDIRECT>
__global__ __launch_bounds__(kBThreads, 2) void shrink_block(BlockApplyArgs a) {
  __shared__ BlockLds<RB> L;
  const int lane = threadIdx.x & 63;
  const DispatchRoute rt{a.inv, a.perm_w, a.b.k, a.b.K, a.b.scale, a.offsets[min(lane, a.b.K)]};
  int tb, sl;
  if (!block_slice_of(blockIdx.x, a.b.nblocks, a.b.kslices, tb, sl)) return;
  block_shrink<RB, INDIRECT>(a.b, L, rt, tb, sl);
}

template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kBThreads, 2) void expand_block(BlockApplyArgs a) {
  __shared__ BlockLds<RB> L;
  const int lane = threadIdx.x & 63;
  const DispatchRoute rt{a.inv, a.perm_w, a.b.k, a.b.K, a.b.scale, a.offsets[min(lane, a.b.K)]};
  int tb, cs;
  if (!block_slice_of(blockIdx.x, a.b.nblocks, a.b.cslices, tb, cs)) return;
  block_expand<RB, INDIRECT, Y0F32, YF32>(a.b, L, rt, tb, cs, [] {});
}

// Several targets sharing one routing: entry blockIdx.y of the array, workgroups past that
// target's own grid return.
struct BlockMulti {
  BlockApplyArgs a[8];
};
template <int RB, bool INDIRECT>
__global__ __launch_bounds__(kBThreads, 2) void shrink_block_multi(BlockMulti m) {
  __shared__ BlockLds<RB> L;
  const BlockApplyArgs& a = m.a[blockIdx.y];
  int tb, sl;
  if (!block_slice_of(blockIdx.x, a.b.nblocks, a.b.kslices, tb, sl)) return;
  const int lane = threadIdx.x & 63;
  const DispatchRoute rt{a.inv, a.perm_w, a.b.k, a.b.K, a.b.scale, a.offsets[min(lane, a.b.K)]};
  block_shrink<RB, INDIRECT>(a.b, L, rt, tb, sl);
}
template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kBThreads, 2) void expand_block_multi(BlockMulti m) {
  __shared__ BlockLds<RB> L;
  const BlockApplyArgs& a = m.a[blockIdx.y];
  int tb, cs;
  if (!block_slice_of(blockIdx.x, a.b.nblocks, a.b.cslices, tb, cs)) return;
  const int lane = threadIdx.x & 63;
  const DispatchRoute rt{a.inv, a.perm_w, a.b.k, a.b.K, a.b.scale, a.offsets[min(lane, a.b.K)]};
  block_expand<RB, INDIRECT, Y0F32, YF32>(a.b, L, rt, tb, cs, [] {});
}

// The vocabulary-routed step split over the reduction and output dimensions, in two launches
// (k = 1).  Every token's h is the sum of per-slice partials, so a workgroup reads only a
// 512-wide slice of each adapter it uses (A: 16 KB, B: 16 KB per adapter at rank 16) instead of
// the whole matrices: an 8-token tile reads 256 KB of adapter data per adapter for 192 KB of
// its own rows, and a tile that spans a run boundary reads it twice.
//   split_shrink  (64-token block, d_in slice of 512): routes the block's tokens from their
//                 ids, stages the A slices of the adapters the block uses in LDS, and writes
//                 the partial h of every token against its own adapter (rows of other adapters
//                 are discarded, so the partial workspace does not grow with the adapters in a
//                 block).  Workgroups of slice 0 also write the block's adapter counts.
//   split_expand  (64-token block, d_out slice of 512): sums the partials in slice order,
//                 scales, stages the B slices in LDS and writes y = y0 + sum_e mask_e(h) B_e;
//                 and, from all blocks' adapter counts (offsets, and the tokens of earlier
//                 blocks per adapter), the dispatch outputs of its share of the block's tokens
//                 (the block's column slices split its 64 tokens).
// The launch boundary orders the partials' writes before their reads.  Workgroups are dispatched
// round robin over the 8 XCDs (workgroup b runs on XCD b % 8); both launches place every slice of
// block tb on XCD tb % 8, so the partials that the shrink writes are still in that XCD's L2 when
// the expand reads them.
constexpr int kSWaves = 8;
constexpr int kSThreads = kSWaves * kWave;
// adapters whose slices are staged in LDS together (64 KB)
template <int RB>
constexpr int split_group() {
  return RB == 1 ? 4 : (RB == 2 ? 2 : 1);
}

struct SplitGeom {
  int nblocks, kslices, cslices;  // grid of a launch: 8 * ceil(nblocks / 8) * slices
  float* part;  // [nblocks][kslices][64][r_pad] fp32: partial h of each token on its own adapter
  int32_t* bcnt;  // [K][split_count_stride(nblocks)]: routed tokens per adapter in each block
};
constexpr int kSMaxCounts = 1024;  // K * split_count_stride(nblocks) for N <= kStepMaxN, K <= 16
static_assert(kSMaxCounts >= kApplyTileMaxAdapters * (kStepMaxN / kSTok) && kSMaxCounts % kSThreads == 0,
              "per-block counts of the split step's dispatch share");

template <int RB>
struct ShrinkLds {
  alignas(16) uint16_t As[split_group<RB>()][4 * RB * 16 * kStepK];
  float red[4][16][RB * 16 + 4];
};

// Partial h of block tb, reduction slice sl (and, when disp, the block's adapter counts).
template <int RB, bool INDIRECT>
__device__ __forceinline__ void shrink_slice(const StepArgs& a, const SplitGeom& g, int tb, int sl, bool disp,
                                             ShrinkLds<RB>& L) {
  constexpr int GA = split_group<RB>();
  constexpr int piece = RB * 16 * kStepK;  // elements of one reduction step's A pieces
  auto& As = L.As;
  auto& red = L.red;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4, rb = wave & 3, kh = wave >> 2;
  const int N = a.t.N, K = a.t.K, d_in = a.t.tgt.d_in, r_pad = a.t.tgt.r_pad;
  const int t0 = tb * kSTok;
  // loads in use order: the block's ids (lane l: token t0 + l, clones of N - 1 past the end),
  // then the x rows
  const int myid = a.ids[min(t0 + lane, N - 1)];
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order (data returns in issue order)
  const int S_all = d_in / kStepK;
  const int s0 = sl * (kSSlice / kStepK), s1 = min(s0 + kSSlice / kStepK, S_all);
  const int w0 = min(s0 + 2 * kh, s1), w1 = min(w0 + 2, s1);  // this wave's steps
  const int row = min(t0 + 16 * rb + n, N - 1);
  const uint16_t* xp = a.t.x + (size_t)row * d_in + 8 * G;
  u32x4_t xv[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int st = max(min(w0 + i, w1 - 1), s0);
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[i][c] = ld16_nt(xp + st * kStepK + 32 * c);
  }
  const int ns = s1 - s0;
  __builtin_amdgcn_sched_barrier(0);
  const int pe = step_owner(myid, a.bounds);
  uint32_t used = 0;
#pragma unroll
  for (int e = 0; e < kT8MaxU; ++e)
    if (e < K && __ballot(pe == e) != 0) used |= 1u << e;
  const int nU = __popc(used);
  // adapters of the lane's four MFMA rows (tokens 16 rb + 4G + i)
  int erow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) erow[i] = __shfl(pe, 16 * rb + 4 * G + i, kWave);
  if (disp && wave == 0) {
    // the block's routed tokens per adapter (clones of token N - 1 past the end do not count),
    // stored while the x rows are in flight
    const bool real = t0 + lane < N;
    int mine = 0;
#pragma unroll
    for (int e = 0; e < kT8MaxU; ++e)
      if (e < K) {
        const int c = __popcll(__ballot(real && pe == e));
        if (lane == e) mine = c;
      }
    if (lane < K) g.bcnt[(size_t)lane * split_count_stride(g.nblocks) + tb] = mine;
  }

  f32x4_t hs[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) hs[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t rem = used;
  for (int base = 0; base < max(nU, 1); base += GA) {
    const int ng = min(GA, nU - base);
    // the used adapters' slices of this group (requested once the routing is known: staging
    // every adapter's slice up front costs more in extra traffic than it saves in latency)
    if (base > 0) __syncthreads();  // the previous group's slices are consumed
    uint32_t r2 = rem;
    for (int gi = 0; gi < ng; ++gi) {
      lds_copy_1k(As[gi], adapter_A<INDIRECT>(a.t.tgt, __builtin_ctz(r2)) + (size_t)s0 * piece, ns * piece * 2);
      r2 &= r2 - 1;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int gi = 0; gi < ng; ++gi) {
      const int e = __builtin_ctz(rem);
      rem &= rem - 1;
      if (__ballot(erow[0] == e || erow[1] == e || erow[2] == e || erow[3] == e) == 0) continue;
      f32x4_t acc[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (w0 + i < w1) {
          const uint16_t* ap = As[gi] + (size_t)(w0 + i - s0) * piece;
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int u = 0; u < RB; ++u) {
              // lane (n, G) takes its 16 bytes at position 4n + G of the 1 KB piece (slab swizzle)
              const u32x4_t av = *reinterpret_cast<const u32x4_t*>(ap + ((c * RB + u) * 64 + 4 * n + G) * 8);
              acc[u] = mfma16x16x32(as_bf16x8(xv[i][c]), as_bf16x8(av), acc[u]);
            }
        }
      }
      // keep the rows whose token uses this adapter (adding to zero: exact)
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) hs[u][i] += (erow[i] == e) ? acc[u][i] : 0.f;
    }
  }
  // the two reduction halves of a row block meet in LDS; the first half stores the sums
  if (kh == 1) {
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[rb][4 * G + i][u * 16 + n] = hs[u][i];
  }
  __syncthreads();
  if (kh == 0) {
    float* dst = g.part + split_part_index(tb, sl, g.kslices, r_pad) + (size_t)16 * rb * r_pad;
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(size_t)(4 * G + i) * r_pad + u * 16 + n] = hs[u][i] + red[rb][4 * G + i][u * 16 + n];
  }
}

template <int RB, bool INDIRECT>
__global__ __launch_bounds__(kSThreads) void split_shrink(StepArgs a, SplitGeom g) {
  __shared__ ShrinkLds<RB> L;
  const int q = blockIdx.x >> 3;
  const int tb = (q / g.kslices) * 8 + (blockIdx.x & 7), sl = q % g.kslices;
  if (tb >= g.nblocks) return;
  shrink_slice<RB, INDIRECT>(a, g, tb, sl, sl == 0 && a.dispatch_share, L);  // slice 0: the block's counts
}

// ALLB (rank block 1, K <= 4): the B slices of all K adapters fit in LDS and are requested
// before the y0 rows without waiting for the routing, so h and the MFMAs run while the y0 rows
// are still arriving.  Otherwise the used adapters' slices are requested once the ids are in.
template <int RB, bool INDIRECT, bool Y0F32, bool YF32, bool ALLB>
__global__ __launch_bounds__(kSThreads) void split_expand(StepArgs a, SplitGeom g) {
  constexpr int GB = split_group<RB>();
  constexpr int RP = RB * 16;
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  __shared__ alignas(16) uint16_t Bs[GB][kSSlice * RP];  // B^T rows of the slice [512][r_pad]
  __shared__ alignas(16) uint16_t hb[2][kSTok][RP];      // h hi / lo [part][token][rank]
  __shared__ alignas(16) int cntl[kSMaxCounts];          // all blocks' adapter counts [K][cstride]
  const int q = blockIdx.x >> 3;
  const int tb = (q / g.cslices) * 8 + (blockIdx.x & 7), cs = q % g.cslices;
  if (tb >= g.nblocks) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave: row block rb (16 tokens) x two 128-column blocks of the slice (512 contiguous bytes
  // of each y0 / y row)
  const int n = lane & 15, G = lane >> 4, rb = wave & 3, ch = wave >> 2;
  const int N = a.t.N, K = a.t.K, d_out = a.t.tgt.d_out;
  const int t0 = tb * kSTok;
  const int c0 = cs * kSSlice, c1 = min(c0 + kSSlice, d_out);
  const int nb = (c1 - c0) / kColBlock;  // 128-column blocks in the slice
  const int b0 = min(2 * ch, nb - 1), b1 = min(2 * ch + 1, nb - 1);
  const bool has0 = 2 * ch < nb, has1 = 2 * ch + 1 < nb;
  // loads: the ids, the y0 rows of the first column block (ALLB: after the B slices), the
  // partials (every thread 16 bytes of each slice), the B slices (straight into LDS), then the
  // y0 rows of the second column block.  Loads return in issue order: the first block's output
  // is stored while the second block's y0 rows are still arriving.
  static_assert(!ALLB || RB == 1, "all-adapter staging holds four rank-16 slices");
  const int myid = a.ids[min(t0 + lane, N - 1)];
  // dispatch share: all blocks' adapter counts, 2 per thread (unconditional, clamped loads)
  const int cstride = split_count_stride(g.nblocks), ncnt = K * cstride;
  int cv[kSMaxCounts / kSThreads];
  if (a.dispatch_share) {
#pragma unroll
    for (int j = 0; j < kSMaxCounts / kSThreads; ++j) cv[j] = g.bcnt[min(j * kSThreads + (int)threadIdx.x, ncnt - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order (data returns in issue order)
  const char* y0rows[4];
  char* yrows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = min(t0 + 16 * rb + 4 * G + i, N - 1);
    y0rows[i] = reinterpret_cast<const char*>(a.t.y0) + (size_t)t * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(a.t.y) + (size_t)t * d_out * yb;
  }
  RowChunk<Y0F32> yc0, yc1;
  if constexpr (!ALLB) load_row_chunk<Y0F32>(yc0, y0rows, c0 + b0 * kColBlock, n);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int QPT = (kSTok * RP / 4 + kSThreads - 1) / kSThreads;  // 16-byte quads per thread
  constexpr int KSMAX = 8;  // slices loaded up front (the rest, d_in > 4096, at the sum)
  u32x4_t pv[QPT][KSMAX];
  const float* pbase = g.part + split_part_index(tb, 0, g.kslices, RP);
#pragma unroll
  for (int q = 0; q < QPT; ++q) {
    const int qi = min(q * kSThreads + (int)threadIdx.x, kSTok * RP / 4 - 1);
#pragma unroll
    for (int s = 0; s < KSMAX; ++s)
      if (s < g.kslices) pv[q][s] = ld16(pbase + (size_t)s * kSTok * RP + 4 * qi);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int bbytes = (c1 - c0) * RP * 2;
  if constexpr (ALLB) {
    for (int e2 = 0; e2 < K; ++e2)
      lds_copy_1k(Bs[e2], adapter_B<INDIRECT>(a.t.tgt, e2) + (size_t)c0 * RP, bbytes);
    __builtin_amdgcn_sched_barrier(0);
    load_row_chunk<Y0F32>(yc0, y0rows, c0 + b0 * kColBlock, n);
  }
  const int pe = step_owner(myid, a.bounds);
  uint32_t used = 0;
#pragma unroll
  for (int e = 0; e < kT8MaxU; ++e)
    if (e < K && __ballot(pe == e) != 0) used |= 1u << e;
  const int nU = __popc(used);
  if constexpr (!ALLB) {
    uint32_t r2 = used;
    for (int gi = 0; gi < min(GB, nU); ++gi) {
      lds_copy_1k(Bs[gi], adapter_B<INDIRECT>(a.t.tgt, __builtin_ctz(r2)) + (size_t)c0 * RP, bbytes);
      r2 &= r2 - 1;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  load_row_chunk<Y0F32>(yc1, y0rows, c0 + b1 * kColBlock, n);
  __builtin_amdgcn_sched_barrier(0);
  // everything before the y0 rows still to come has arrived (vmcnt = those rows' loads)
  if constexpr (ALLB) __builtin_amdgcn_s_waitcnt(0x0F70 | (Y0F32 ? 16 : 8));
  else __builtin_amdgcn_s_waitcnt(0x0F70 | (Y0F32 ? 8 : 4));
  // h = scale x (sum of the slices in order), split into bf16 hi / lo; unrouted tokens get 0
#pragma unroll
  for (int q = 0; q < QPT; ++q) {
    const int qi = q * kSThreads + (int)threadIdx.x;
    const int tok = min(qi, kSTok * RP / 4 - 1) / (RP / 4), rk = 4 * (qi % (RP / 4));
    const float wt = __shfl(pe, tok, kWave) >= 0 ? a.t.scale : 0.f;
    if (qi < kSTok * RP / 4) {
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSMAX; ++s)
        if (s < g.kslices)
#pragma unroll
          for (int c = 0; c < 4; ++c) sum[c] += __uint_as_float(pv[q][s][c]);
      for (int s = KSMAX; s < g.kslices; ++s) {
        const u32x4_t v = ld16(pbase + (size_t)s * kSTok * RP + 4 * qi);
#pragma unroll
        for (int c = 0; c < 4; ++c) sum[c] += __uint_as_float(v[c]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float h = sum[c] * wt;
        const __bf16 hi = (__bf16)h;
        const __bf16 lo = (__bf16)(h - (float)hi);
        hb[0][tok][rk + c] = __builtin_bit_cast(uint16_t, hi);
        hb[1][tok][rk + c] = __builtin_bit_cast(uint16_t, lo);
      }
    }
  }
  f32x4_t o0[8], o1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    o0[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    o1[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if (a.dispatch_share) {
#pragma unroll
    for (int j = 0; j < kSMaxCounts / kSThreads; ++j)
      if (j * kSThreads + (int)threadIdx.x < ncnt) cntl[j * kSThreads + threadIdx.x] = cv[j];
  }
  const int erow = __shfl(pe, 16 * rb + n, kWave);  // adapter of the lane's A-operand row
  uint32_t rem = used;
  for (int base = 0; base < nU; base += GB) {
    const int ng = min(GB, nU - base);
    if (!ALLB && base > 0) {
      __syncthreads();  // the previous group's slices are consumed
      uint32_t r3 = rem;
      for (int gi = 0; gi < ng; ++gi) {
        lds_copy_1k(Bs[gi], adapter_B<INDIRECT>(a.t.tgt, __builtin_ctz(r3)) + (size_t)c0 * RP, bbytes);
        r3 &= r3 - 1;
      }
    }
    if (base > 0) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // the group's B slices and h (and the counts) are in LDS
    for (int gi = 0; gi < ng; ++gi) {
      const int e = __builtin_ctz(rem);
      rem &= rem - 1;
      if (__ballot(erow == e) == 0) continue;  // no token of this row block uses adapter e
      const uint16_t* Bl = Bs[ALLB ? e : gi];
      // A operand: row n of the row block, kept only if that token uses adapter e; k-slot
      // groups 0, 1 carry hi of ranks 16u + 8(G & 1) .., groups 2, 3 lo of the same ranks
      bf16x8_t hv[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(&hb[G >> 1][16 * rb + n][u * 16 + 8 * (G & 1)]);
        if (erow != e) v = u32x4_t{0u, 0u, 0u, 0u};
        hv[u] = as_bf16x8(v);
      }
      const uint16_t* bp0 = Bl + (size_t)(b0 * kColBlock + n) * RP + 8 * (G & 1);
      const uint16_t* bp1 = Bl + (size_t)(b1 * kColBlock + n) * RP + 8 * (G & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(bp0 + (size_t)16 * j * RP + 16 * u);
          const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(bp1 + (size_t)16 * j * RP + 16 * u);
          o0[j] = mfma16x16x32(hv[u], as_bf16x8(v0), o0[j]);
          o1[j] = mfma16x16x32(hv[u], as_bf16x8(v1), o1[j]);
        }
    }
  }
  if (nU == 0 && a.dispatch_share) __syncthreads();  // the counts are in LDS (no group loop ran)
  if (a.dispatch_share && wave == 0) {
    // dispatch share, before the y stores so that its own stores go out first (issued after
    // them they would extend the launch): lane e < K sums adapter e's row of block counts (all
    // blocks, and those before tb) with 16-byte LDS reads; a uniform loop over the adapters
    // turns the totals into offsets.  A token's grouped position is its adapter's offset, plus
    // that adapter's tokens in earlier blocks, plus its rank among the block's earlier tokens of
    // the same adapter.  This workgroup writes the outputs of block tokens [l0, l1) (the column
    // slices split the block).
    int tot = 0, bef = 0;
    if (lane < K) {
      const int* row = cntl + lane * cstride;
#pragma unroll
      for (int j = 0; j < kStepMaxN / kSTok / 4; ++j) {
        if (4 * j < cstride) {  // entries past nblocks are padding, never written
          const int4 v = *reinterpret_cast<const int4*>(row + 4 * j);
          const int nb = g.nblocks;
          tot += (4 * j < nb ? v.x : 0) + (4 * j + 1 < nb ? v.y : 0) + (4 * j + 2 < nb ? v.z : 0) +
                 (4 * j + 3 < nb ? v.w : 0);
          bef += (4 * j < tb ? v.x : 0) + (4 * j + 1 < tb ? v.y : 0) + (4 * j + 2 < tb ? v.z : 0) +
                 (4 * j + 3 < tb ? v.w : 0);
        }
      }
    }
    int start = 0, off = 0;
    for (int e = 0; e < K; ++e) {
      const int tot_e = __builtin_amdgcn_readlane(tot, e), bef_e = __builtin_amdgcn_readlane(bef, e);
      if (pe == e) start = off + bef_e;
      if (tb == 0 && cs == 0 && lane == e) {
        a.counts[e] = tot_e;
        a.offsets[e] = off;
      }
      off += tot_e;
    }
    if (tb == 0 && cs == 0 && lane == 0) a.offsets[K] = off;
    int nbits = 0;
    while ((1 << nbits) < K) ++nbits;
    const int tok = t0 + lane;
    const bool real = tok < N;
    const bool valid = real && pe >= 0;
    const uint64_t mm = match_mask(pe, valid, nbits);
    const int tpw = (kSTok + g.cslices - 1) / g.cslices;
    const int l0 = cs * tpw, l1 = min(kSTok, l0 + tpw);
    if (real && lane >= l0 && lane < l1) {
      a.idx[tok] = pe;
      a.w[tok] = valid ? 1.0f : 0.0f;
      if (valid) {
        const int pos = start + __popcll(mm & lanemask_lt(lane));
        a.inv[tok] = pos;
        a.perm[pos] = tok;
        a.perm_w[pos] = 1.0f;
      } else {
        a.inv[tok] = -1;
      }
    }
  }
  if (has0) epilogue_store<Y0F32, YF32>(o0, yc0, yrows, c0 + b0 * kColBlock, n, 0xFu);
  if (has1) epilogue_store<Y0F32, YF32>(o1, yc1, yrows, c0 + b1 * kColBlock, n, 0xFu);
}

// Key of grouped position q: (rank of its pair among the token's routed pairs) * K + adapter;
// weight: its gate weight.  Ranking the routed pairs (instead of using the slot index) makes
// pass 0 hold every token's first routed pair, so only pass 0 reads y0.
struct SlotKeySource {
  const int32_t* perm;
  const float* perm_w;
  const int32_t* inv;
  const int* offs;  // LDS copy of the dispatch offsets
  int k, K;
  __device__ __forceinline__ void operator()(int q, int& e, float& wv) const {
    const int p = perm[q];
    const int t = p / k, s = p - t * k;
    int rank = 0;
    for (int j = 0; j < s; ++j) rank += inv[(long long)t * k + j] >= 0 ? 1 : 0;
    e = rank * K + segment_of(offs, K, q);
    wv = perm_w[q];
  }
};

__global__ __launch_bounds__(1024) void slot_sort(const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                                                  const float* __restrict__ perm_w, const int32_t* __restrict__ inv,
                                                  int k, int K, int32_t* __restrict__ counts2,
                                                  int32_t* __restrict__ offsets2, int32_t* __restrict__ perm2,
                                                  float* __restrict__ perm_w2) {
  __shared__ DispatchLds<1024> DL;
  __shared__ int offs[65];
  if (threadIdx.x <= K) offs[threadIdx.x] = offsets[threadIdx.x];
  __syncthreads();
  const int P = offs[K];
  dispatch_block<1024>(DL, SlotKeySource{perm, perm_w, inv, offs, k, K}, P, k * K, counts2, offsets2, perm2, perm_w2,
                       nullptr);
}

// The same sort over many pairs: histogram and scatter launches over nb workgroups.
__global__ __launch_bounds__(1024) void slot_hist(const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                                                  const float* __restrict__ perm_w, const int32_t* __restrict__ inv,
                                                  int k, int K, int C, int32_t* __restrict__ bcnt) {
  __shared__ DispatchLds<1024> DL;
  __shared__ int offs[65];
  if (threadIdx.x <= K) offs[threadIdx.x] = offsets[threadIdx.x];
  __syncthreads();
  dispatch_hist_part<1024>(DL, SlotKeySource{perm, perm_w, inv, offs, k, K}, offs[K], k * K, C, bcnt);
}
__global__ __launch_bounds__(1024) void slot_scatter(const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ perm, const float* __restrict__ perm_w,
                                                     const int32_t* __restrict__ inv, int k, int K, int C, int nb,
                                                     const int32_t* __restrict__ bcnt, int32_t* __restrict__ counts2,
                                                     int32_t* __restrict__ offsets2, int32_t* __restrict__ perm2,
                                                     float* __restrict__ perm_w2) {
  __shared__ DispatchLds<1024> DL;
  __shared__ int offs[65];
  if (threadIdx.x <= K) offs[threadIdx.x] = offsets[threadIdx.x];
  __syncthreads();
  dispatch_scatter_part<1024>(DL, SlotKeySource{perm, perm_w, inv, offs, k, K}, offs[K], k * K, C, nb, bcnt, counts2,
                              offsets2, perm2, perm_w2, nullptr);
}

// After the passes: y = y0 for tokens with no routed pair (copy_y0, out-of-place calls) and
// y = z (the fp32 pass buffer) for tokens whose routed pairs end before the last pass, i.e.
// fewer than c_last of them (copy_z, when z is not y itself).  One wave per 64 tokens.
template <bool Y0F32, bool YF32>
__device__ __forceinline__ void finish_body(const void* y0, const float* z, void* y, const int32_t* __restrict__ inv,
                                            int N, int k, int c_last, int d_out, int copy_y0, int copy_z, int blk) {
  const int lane = threadIdx.x & 63;
  const int base = (blk * 4 + (threadIdx.x >> 6)) * kWave;
  const int t = base + lane;
  int c = 0;
  if (t < N)
    for (int j = 0; j < k; ++j) c += inv[(long long)t * k + j] >= 0 ? 1 : 0;
  uint64_t m = __ballot(t < N && ((copy_y0 && c == 0) || (copy_z && c > 0 && c < c_last)));
  while (m) {
    const int l = __builtin_ctzll(m);
    m &= m - 1;
    const int tt = base + l;
    const bool from_y0 = __shfl(c, l, kWave) == 0;
    for (int col = lane * 4; col < d_out; col += kWave * 4) {
      float v[4];
      if (from_y0) {
        if constexpr (Y0F32) {
          const float* p = reinterpret_cast<const float*>(y0) + (size_t)tt * d_out + col;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = p[i];
        } else {
          const uint16_t* p = reinterpret_cast<const uint16_t*>(y0) + (size_t)tt * d_out + col;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = bf16_to_f32(p[i]);
        }
      } else {
        const float* p = z + (size_t)tt * d_out + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = p[i];
      }
      if constexpr (YF32) {
        float* p = reinterpret_cast<float*>(y) + (size_t)tt * d_out + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = v[i];
      } else {
        uint32_t* p = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(y) + (size_t)tt * d_out + col);
        p[0] = pack_bf16x2(v[0], v[1]);
        p[1] = pack_bf16x2(v[2], v[3]);
      }
    }
  }
}
template <bool Y0F32, bool YF32>
__global__ __launch_bounds__(256) void finish_tokens(const void* y0, const float* z, void* y,
                                                     const int32_t* __restrict__ inv, int N, int k, int c_last,
                                                     int d_out, int copy_y0, int copy_z) {
  finish_body<Y0F32, YF32>(y0, z, y, inv, N, k, c_last, d_out, copy_y0, copy_z, blockIdx.x);
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
  // one step per load batch (fewer registers, more waves per SIMD; measured faster at decode sizes)
  shrink_steps_batched<RB, true, 1>(acc, a.x + (size_t)tok * d_in, At, d_in, (S * wave) / NW, (S * (wave + 1)) / NW,
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
__device__ __forceinline__ void shrink_grouped_body(const ShrinkArgs& a, float* red, int T, int sp) {
  constexpr int RS = RedLds<RB>::RS;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  // one step per batch: fewer registers, more waves per SIMD (the skinny workgroups are many
  // and short; measured faster than two-step batches at rank 64)
  shrink_steps_batched<RB, true, RB == 1 ? 4 : 1>(acc, a.x + (size_t)tok * d_in, At, d_in, sa + (len * wave) / 4,
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
template <int RB, bool INDIRECT>
__global__ __launch_bounds__(256) void shrink_grouped(ShrinkArgs a) {
  __shared__ float red[RedLds<RB>::kFloats];
  const int T = xcd_tile_slot(a.offsets, a.K, blockIdx.x, threadIdx.x & 63);
  if (T < 0) return;
  shrink_grouped_body<RB, INDIRECT>(a, red, T, blockIdx.y);
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
  const int32_t* offsets;  // expand_grouped_k1: grouped start of each key (key0 .. key0 + K)
  const int32_t* order;    // expand_grouped_k1: row -> grouped position of the shrink (nullptr: the row)
  int key0;
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

// One adapter per token (k = 1), or one pass over the j-th routed pairs of the tokens (k > 1:
// keys key0 .. key0 + K of the rank-sorted order, rows mapped to the shrink's grouped positions
// by `order`): grid = tile slots * col_groups (+ copy blocks).
template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__device__ __forceinline__ void expand_grouped_body(const ExpandArgs& a, int b) {
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (b >= a.main_blocks) {
    copy_unrouted<Y0F32, YF32, 4>(a.y0, a.y, a.inv, a.N, a.tgt.d_out, b - a.main_blocks, a.copy_blocks);
    return;
  }
  const int g = b % a.col_groups, T = b / a.col_groups;
  int e, row0, nrows;
  if (!find_tile(a.offsets + a.key0, a.K, T, lane, e, row0, nrows)) return;
  const int n = lane & 15, G = lane >> 4;
  const bool valid = n < nrows;
  const int qr = row0 + (valid ? n : 0);
  const int q = a.order != nullptr ? a.order[qr] : qr;  // the row's grouped position in the shrink
  const int tok = a.perm[q] / a.k;
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
  // the first block's y0 rows and B pieces do not depend on h: they go out before the partials
  RowChunk<Y0F32> cur;
  u32x4_t bv[8][RB];
  const int blk0 = min(wave, nblk - 1);
  load_row_chunk<Y0F32>(cur, y0rows, c0 + blk0 * kColBlock, n);
  expand_load_b<RB>(bv, Bt, a.tgt.r_pad, c0 + blk0 * kColBlock, lane);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t hb[RB];
  h_operand_from_ws<RB>(hb, a.hpart, a.P, a.nsplit, q, valid, lane);
  for (int blk = wave; blk < nblk; blk += 4) {
    if (blk != wave) {
      load_row_chunk<Y0F32>(cur, y0rows, c0 + blk * kColBlock, n);
      expand_load_b<RB>(bv, Bt, a.tgt.r_pad, c0 + blk * kColBlock, lane);
    }
    f32x4_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    expand_mfma_regs<RB>(o, hb, bv);
    epilogue_store<Y0F32, YF32>(o, cur, yrows, c0 + blk * kColBlock, n, vmask);
  }
}
template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(256) void expand_grouped_k1(ExpandArgs a) {
  expand_grouped_body<RB, INDIRECT, Y0F32, YF32>(a, blockIdx.x);
}

// Several projections that share one routing (the targets of a layer), one launch per phase:
// target i's arguments are entry i of an array passed by value; the grid's last dimension
// selects the entry and workgroups past a target's own grid return.
struct ShrinkMulti {
  ShrinkArgs a[kApplyMaxMulti];
};
struct ExpandMulti {
  ExpandArgs a[kApplyMaxMulti];
};
struct FinishMulti {
  const void* y0[kApplyMaxMulti];
  const float* z[kApplyMaxMulti];
  void* y[kApplyMaxMulti];
  int d_out[kApplyMaxMulti];
  const int32_t* inv;
  int N, k, copy_y0[kApplyMaxMulti], copy_z[kApplyMaxMulti];
};
template <int RB, bool INDIRECT>
__global__ __launch_bounds__(256) void shrink_grouped_multi(ShrinkMulti m) {
  __shared__ float red[RedLds<RB>::kFloats];
  const ShrinkArgs& a = m.a[blockIdx.z];
  if ((int)blockIdx.y >= a.nsplit) return;
  const int T = xcd_tile_slot(a.offsets, a.K, blockIdx.x, threadIdx.x & 63);
  if (T < 0) return;
  shrink_grouped_body<RB, INDIRECT>(a, red, T, blockIdx.y);
}
template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(256) void expand_grouped_multi(ExpandMulti m) {
  const ExpandArgs& a = m.a[blockIdx.y];
  if ((int)blockIdx.x >= a.main_blocks + a.copy_blocks) return;
  expand_grouped_body<RB, INDIRECT, Y0F32, YF32>(a, blockIdx.x);
}
template <bool Y0F32, bool YF32>
__global__ __launch_bounds__(256) void finish_tokens_multi(FinishMulti m) {
  const int i = blockIdx.y;
  finish_body<Y0F32, YF32>(m.y0[i], m.z[i], m.y[i], m.inv, m.N, m.k, m.k, m.d_out[i], m.copy_y0[i], m.copy_z[i],
                           blockIdx.x);
}

// ---- decode-sized expand (k = 2..4, at most kDXMaxTok tokens, K * r_pad <= kDXMaxKR): the
// summed h rows of every pair first, by pair id (hsum_multi), then one launch over (target,
// 32-column slice).  A workgroup holds that slice of every adapter's B^T in LDS and covers every token:
// each wave owns 16-token row blocks and adds, in registers, the token's routed pairs in
// adapter order (a repeated adapter once per slot, in slot order), then writes y = y0 + sum.
// Each adapter's B^T is read once per call, and no sum is carried between launches.
struct HsumMulti {
  const float* hpart[kApplyMaxMulti];
  uint16_t* hq[kApplyMaxMulti];   // [P][2][r_pad] bf16 hi / lo by pair id
  int32_t* eid[kApplyMaxMulti];   // [P] adapter of each routed pair
  int nsplit[kApplyMaxMulti];
  const int32_t* offsets;
  const int32_t* perm;
  long long P;
  int K;
};

// For grouped position q < offsets[K]: hq[perm[q]] = bf16 hi and lo of the sum over the splits
// (in order) of the weighted partials of q, and eid[perm[q]] = its adapter; a thread per 8
// ranks of a row.  The expand then finds a token's pairs at fixed addresses.
template <int RB>
__global__ __launch_bounds__(256) void hsum_multi(HsumMulti m) {
  constexpr int RP = RB * 16, CH = RP / 8;
  __shared__ int offs[65];
  if ((int)threadIdx.x <= m.K) offs[threadIdx.x] = m.offsets[threadIdx.x];
  __syncthreads();
  const int i = blockIdx.y;
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  if (v >= (long long)offs[m.K] * CH) return;
  const long long q = v / CH;
  const int c = (int)(v - q * CH);
  float sum[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sum[j] = 0.f;
  for (int sp = 0; sp < m.nsplit[i]; ++sp) {
    const float* p = m.hpart[i] + ((long long)sp * m.P + q) * RP + 8 * c;
    const u32x4_t x0 = ld16(p), x1 = ld16(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sum[j] += __uint_as_float(x0[j]);
      sum[j + 4] += __uint_as_float(x1[j]);
    }
  }
  const int pid = m.perm[q];
  uint16_t* dst = m.hq[i] + (size_t)pid * 2 * RP + 8 * c;
  *reinterpret_cast<bf16x8_t*>(dst) = split_hilo(sum, false);
  *reinterpret_cast<bf16x8_t*>(dst + RP) = split_hilo(sum, true);
  if (c == 0) m.eid[i][pid] = segment_of(offs, m.K, (int)q);
}

struct DecodeMulti {
  TargetDev tgt[kApplyMaxMulti];
  const void* y0[kApplyMaxMulti];
  void* y[kApplyMaxMulti];
  const uint16_t* hq[kApplyMaxMulti];   // by pair id (hsum_multi)
  const int32_t* eid[kApplyMaxMulti];   // adapter by pair id
  const int32_t* inv;
  int N, k, K;
};

constexpr int kDXThreads = 512;

// Workgroup (slice x, target y): columns [32 x, 32 x + 32) of target y.  LDS row L of adapter
// e's 32-row region holds output column 2 (L & 15) + (L >> 4) of the slice (the slab row of
// that column within its 128-column block, 16-byte slots XORed with gm_b_swz(L)), so MFMA c's
// lane n produces column 2n + c and a lane's two columns are adjacent in y.
template <int RB, int KMAX, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kDXThreads, 2) void expand_decode_multi(const DecodeMulti m) {
  constexpr int RP = RB * 16, SPR = 2 * RB, NPC = kDXCols * SPR / 64;  // 1 KB pieces per adapter
  static_assert(kDXCols == 32, "two MFMA column blocks per slice");
  __shared__ alignas(16) uint16_t Bs[kDXMaxKR * kDXCols];
  const int i = blockIdx.y;
  const TargetDev& tg = m.tgt[i];
  const int d_out = tg.d_out;
  const int c0 = blockIdx.x * kDXCols;
  if (c0 >= d_out) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  // 1. the slice of every adapter's B^T, straight into LDS
  {
    const int blk0 = c0 & ~(kColBlock - 1), cw = c0 & (kColBlock - 1);
    for (int p = wave; p < m.K * NPC; p += kDXThreads / kWave) {
      const int e = p / NPC, pp = p - e * NPC;
      const int P = 64 * pp + lane, L = P / SPR, slot = (P % SPR) ^ gm_b_swz<RB>(L);
      const int lc = cw + 2 * (L & 15) + (L >> 4);  // column within the 128-column block
      const int w = 16 * (lc & 7) + (lc >> 3);      // its slab row (the inverse of b_perm_col)
      const char* src = reinterpret_cast<const char*>(adapter_B<INDIRECT>(tg, e) + (size_t)(blk0 + w) * RP) + slot * 16;
      __builtin_amdgcn_global_load_lds(src, reinterpret_cast<char*>(Bs) + (size_t)p * 1024, 16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  const uint16_t* hq = m.hq[i];
  const int32_t* eid = m.eid[i];
  const int N = m.N, k = m.k;
  int b_sl[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) b_sl[u] = (2 * u + (G & 1)) ^ gm_b_swz<RB>(n);
  for (int rb = wave; rb * 16 < N; rb += kDXThreads / kWave) {
    // the lane's A row: token 16 rb + n, its routed pairs' adapters and h operands
    const int tn = 16 * rb + n;
    int es[KMAX];
    bf16x8_t hs[KMAX][RB];
    uint64_t mine = 0;
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      // the pair's routing, adapter and h operands are requested together (fixed addresses)
      const bool in = s < k && tn < N;
      const long long pid = in ? (long long)tn * k + s : 0;
      const int q = in ? m.inv[pid] : -1;
      const int e = in ? eid[pid] : 0;
      const uint16_t* hp = hq + ((size_t)pid * 2 + (G >> 1)) * RP + 8 * (G & 1);
      u32x4_t hv[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) hv[u] = in ? ld16(hp + 16 * u) : u32x4_t{0u, 0u, 0u, 0u};
      es[s] = q >= 0 ? e : -1;
      if (q >= 0) mine |= 1ull << e;
#pragma unroll
      for (int u = 0; u < RB; ++u) hs[s][u] = q >= 0 ? as_bf16x8(hv[u]) : bf16x8_t{};
    }
    // the y0 values of the lane's outputs: rows 4G + j, columns c0 + 2n, + 1
    const int tb = 16 * rb + 4 * G;
    float yv[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t o = (size_t)min(tb + j, N - 1) * d_out + c0 + 2 * n;
      if constexpr (Y0F32) {
        const float2 v = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(m.y0[i]) + o);
        yv[j][0] = v.x;
        yv[j][1] = v.y;
      } else {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(m.y0[i]) + o);
        yv[j][0] = __uint_as_float(v << 16);
        yv[j][1] = __uint_as_float(v & 0xffff0000u);
      }
    }
    uint64_t used = mine;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)used, d, kWave);
      const uint32_t hi = __shfl_xor((uint32_t)(used >> 32), d, kWave);
      used |= ((uint64_t)hi << 32) | lo;
    }
    f32x4_t o[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    while (used) {
      const int e = __builtin_ctzll(used);
      used &= used - 1;
      const uint16_t* Be = Bs + (size_t)e * kDXCols * RP;
      unsigned pend = 0;
#pragma unroll
      for (int s = 0; s < KMAX; ++s) pend |= (es[s] == e ? 1u : 0u) << s;
      // one round per occurrence of e among a token's slots (normally one)
      do {
        const int s0 = pend != 0 ? __builtin_ctz(pend) : -1;
        pend &= pend - 1;
        bf16x8_t hb[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) hb[u] = bf16x8_t{};
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
          if (s == s0) {
#pragma unroll
            for (int u = 0; u < RB; ++u) hb[u] = hs[s][u];
          }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Be + (size_t)(16 * c + n) * RP + 8 * b_sl[u]);
            o[c] = mfma16x16x32(hb[u], as_bf16x8(v), o[c]);
          }
      } while (__ballot(pend != 0) != 0);
    }
    // y = y0 + the sum; a token without routed pairs keeps its y0 value
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb + j;
      const bool routed = __shfl(mine != 0 ? 1 : 0, 4 * G + j, kWave) != 0;
      if (t >= N) continue;
      const float v0 = routed ? yv[j][0] + o[0][j] : yv[j][0];
      const float v1 = routed ? yv[j][1] + o[1][j] : yv[j][1];
      const size_t off = (size_t)t * d_out + c0 + 2 * n;
      if constexpr (YF32) {
        *reinterpret_cast<float2*>(reinterpret_cast<float*>(m.y[i]) + off) = make_float2(v0, v1);
      } else {
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(m.y[i]) + off) = pack_bf16x2(v0, v1);
      }
    }
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
      unsigned pend = 0;
#pragma unroll
      for (int s = 0; s < KMAX; ++s) pend |= (es[s] == e ? 1u : 0u) << s;
      // one round per occurrence of e among a token's slots (normally one)
      do {
        const int s0 = pend != 0 ? __builtin_ctz(pend) : -1;
        pend &= pend - 1;
        bf16x8_t hb[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) hb[u] = bf16x8_t{};
#pragma unroll
        for (int s = 0; s < KMAX; ++s)
          if (s == s0) {
#pragma unroll
            for (int u = 0; u < RB; ++u) hb[u] = hs[s][u];
          }
        expand_mfma<RB>(o, hb, adapter_B<INDIRECT>(a.tgt, e), a.tgt.r_pad, c0 + blk * kColBlock, lane);
      } while (__ballot(pend != 0) != 0);
    }
    epilogue_store<Y0F32, YF32>(o, cur, yrows, c0 + blk * kColBlock, n, vmask);
  }
}

// --------------------------------------------------------------------------------------
// host side

// Column groups: enough workgroups to cover the chip while every wave keeps output blocks.
static int choose_col_groups(long long tiles, int d_out, int target_blocks, int min_blocks_per_group) {
  const int nblk = d_out / kColBlock;
  int c = 1;
  while (tiles * c < target_blocks && nblk % (2 * c) == 0 && nblk / (2 * c) >= min_blocks_per_group) c *= 2;
  return c;
}

static int col_groups_for(int requested, long long tiles, int d_out, int target, int minb) {
  if (requested > 0 && (d_out / kColBlock) % requested == 0) return requested;
  return choose_col_groups(tiles, d_out, target, minb);
}

// Column groups of the 8-token tiles: more workgroups while there are fewer tiles than compute
// units, as long as every wave of a group keeps a 256-column unit.
static int t8_col_groups(int requested, long long tiles, int d_out) {
  const int nblk = d_out / kColBlock;
  if (requested > 0 && nblk % requested == 0) return requested;
  int cg = 1;
  while (tiles * cg < 256 && nblk % (2 * cg) == 0 && nblk / (2 * cg) >= 2 * kT8Waves) cg *= 2;
  return cg;
}

static BlockArgs block_args(const ApplyLaunch& a, void* ws) {
  BlockArgs b;
  b.tgt = a.tgt; b.x = a.x; b.y0 = a.y0; b.y = a.y;
  b.N = a.N; b.K = a.K; b.k = a.k; b.scale = a.scale;
  const BlockGeom g = block_geom(a.N, a.k, a.K, a.tgt.d_in, a.tgt.d_out);
  b.nblocks = g.nblocks;
  b.kslices = g.kslices;
  b.cslices = g.cslices;
  b.slotmax = g.slotmax;
  b.part = reinterpret_cast<float*>(ws);
  return b;
}

static T8Args t8_args(const ApplyLaunch& a) {
  T8Args t;
  t.tgt = a.tgt; t.x = a.x; t.y0 = a.y0; t.y = a.y;
  t.N = a.N; t.K = a.K; t.k = a.k; t.scale = a.scale;
  t.tiles = (a.N + kT8Tokens - 1) / kT8Tokens;
  t.col_groups = t8_col_groups(a.col_groups, t.tiles, a.tgt.d_out);
  t.tiles_per_xcd = (t.tiles + 7) / 8;
  return t;
}

template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_fused_t(const FusedArgs& fa, int grid, hipStream_t s) {
  hipLaunchKernelGGL((apply_fused_k1<RB, IND, Y0F, YF>), dim3(grid), dim3(kWaves8 * 64), 0, s, fa);
  return hipGetLastError();
}
template <int RB, bool IND>
static hipError_t launch_shrink_t(const ShrinkArgs& sa, int tiles, hipStream_t s) {
  hipLaunchKernelGGL((shrink_grouped<RB, IND>), dim3((tiles + 7) / 8 * 8, sa.nsplit), dim3(256), 0, s, sa);
  return hipGetLastError();
}
template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_expand_k1_t(const ExpandArgs& ea, int grid, hipStream_t s) {
  hipLaunchKernelGGL((expand_grouped_k1<RB, IND, Y0F, YF>), dim3(grid), dim3(256), 0, s, ea);
  return hipGetLastError();
}
template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_t8_t(const T8ApplyArgs& ta, int grid, hipStream_t s) {
  hipLaunchKernelGGL((apply_t8<RB, IND, Y0F, YF>), dim3(grid), dim3(kT8Threads), 0, s, ta);
  return hipGetLastError();
}
template <bool Y0F, bool YF>
static hipError_t launch_finish_t(const void* y0, const float* z, void* y, const int32_t* inv, int N, int k,
                                  int d_out, bool copy_y0, bool copy_z, hipStream_t s, int c_last = 0) {
  hipLaunchKernelGGL((finish_tokens<Y0F, YF>), dim3((N + 255) / 256), dim3(256), 0, s, y0, z, y, inv, N, k,
                     c_last > 0 ? c_last : k, d_out, (int)copy_y0, (int)copy_z);
  return hipGetLastError();
}
template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_block_t(const BlockApplyArgs& ba, hipStream_t s) {
  hipLaunchKernelGGL((shrink_block<RB, IND>), dim3(block_grid(ba.b.nblocks, ba.b.kslices)), dim3(kBThreads), 0, s, ba);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((expand_block<RB, IND, Y0F, YF>), dim3(block_grid(ba.b.nblocks, ba.b.cslices)), dim3(kBThreads), 0, s,
                     ba);
  return hipGetLastError();
}
template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_split_t(const StepArgs& sa, const SplitGeom& g, hipStream_t s) {
  const int nb8 = 8 * ((g.nblocks + 7) / 8);
  const bool allb = RB == 1 && sa.t.K <= split_group<1>();
  hipLaunchKernelGGL((split_shrink<RB, IND>), dim3(nb8 * g.kslices), dim3(kSThreads), 0, s, sa, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (RB == 1) {
    if (allb) {
      hipLaunchKernelGGL((split_expand<RB, IND, Y0F, YF, true>), dim3(nb8 * g.cslices), dim3(kSThreads), 0, s, sa, g);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((split_expand<RB, IND, Y0F, YF, false>), dim3(nb8 * g.cslices), dim3(kSThreads), 0, s, sa, g);
  return hipGetLastError();
}
template <int RB, bool IND, bool Y0F, bool YF>
static hipError_t launch_step_t(const StepArgs& sa, int grid, hipStream_t s) {
  hipLaunchKernelGGL((step_vocab<RB, IND, Y0F, YF>), dim3(grid), dim3(kT8Threads), 0, s, sa);
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

// The decode expand of n targets (hsum_multi, then expand_decode_multi): hm and dm hold every
// target's pointers; max_dout is the widest d_out.
static hipError_t launch_decode_expand(const HsumMulti& hm, const DecodeMulti& dm, int n, int max_dout, int RBv,
                                       bool indirect, bool y0_f32, bool y_f32, hipStream_t s) {
  if (dm.k < 2 || dm.k > 4 || dm.N > kDXMaxTok || dm.K * RBv * 16 > kDXMaxKR || dm.K > 64 || dm.inv == nullptr ||
      hm.K != dm.K)
    return hipErrorInvalidValue;
  if (hm.P == 0) return hipSuccess;
  const long long hthreads = hm.P * 2 * RBv;
  MOLORA_DISPATCH_RB(RBv, hipLaunchKernelGGL((hsum_multi<RB>), dim3((unsigned)((hthreads + 255) / 256), n), dim3(256),
                                             0, s, hm));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid(max_dout / kDXCols, n);
#define MOLORA_DX(KM)                                                                                      \
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(indirect, IND, MOLORA_DISPATCH_BOOL(y0_f32, Y0F,             \
      MOLORA_DISPATCH_BOOL(y_f32, YF,                                                                      \
          hipLaunchKernelGGL((expand_decode_multi<RB, KM, IND, Y0F, YF>), grid, dim3(kDXThreads), 0, s, dm)))))
  if (dm.k <= 2) { MOLORA_DX(2) }
  else { MOLORA_DX(4) }
#undef MOLORA_DX
  return hipGetLastError();
}

// Rank sort of the grouped pairs for k > 1 passes, in the region of rank_sort_plan() at wsb
// (counts2 and offsets2, perm2 and w2 = the order and weights, the chip-wide sort's counts).
struct RankSort {
  int32_t* offsets2;
  int32_t* perm2;
  float* w2;
};
static hipError_t launch_rank_sort(const ApplyLaunch& a, char* wsb, long long P, hipStream_t s, RankSort& o) {
  const RankSortPlan rp = rank_sort_plan(P, a.k, a.K);
  int32_t* counts2 = reinterpret_cast<int32_t*>(wsb + rp.counts2_off);
  o.offsets2 = reinterpret_cast<int32_t*>(wsb + rp.offsets2_off);
  o.perm2 = reinterpret_cast<int32_t*>(wsb + rp.perm2_off);
  o.w2 = reinterpret_cast<float*>(wsb + rp.w2_off);
  int32_t* bcnt = reinterpret_cast<int32_t*>(wsb + rp.bcnt_off);
  const DispatchSplit ds = dispatch_split(P);
  if (ds.nb > 1) {
    hipLaunchKernelGGL(slot_hist, dim3(ds.nb), dim3(1024), 0, s, a.offsets, a.perm, a.perm_w, a.inv, a.k, a.K, ds.C,
                       bcnt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(slot_scatter, dim3(ds.nb), dim3(1024), 0, s, a.offsets, a.perm, a.perm_w, a.inv, a.k, a.K, ds.C,
                       ds.nb, bcnt, counts2, o.offsets2, o.perm2, o.w2);
  } else {
    hipLaunchKernelGGL(slot_sort, dim3(1), dim3(1024), 0, s, a.offsets, a.perm, a.perm_w, a.inv, a.k, a.K, counts2,
                       o.offsets2, o.perm2, o.w2);
  }
  return hipGetLastError();
}

hipError_t launch_apply(const ApplyLaunch& a, hipStream_t s) {
  const long long P = (long long)a.N * a.k;
  const ApplyPlan plan = apply_plan(a.N, a.k, a.K, a.tgt.r_pad, a.tgt.d_in, a.tgt.d_out, a.y_f32, a.path);
  char* const wsb = reinterpret_cast<char*>(a.ws);
  // fp32 carry of the k > 1 passes: y itself when y is fp32, else the plan's buffer
  float* const zbuf = a.y_f32 ? reinterpret_cast<float*>(a.y) : reinterpret_cast<float*>(wsb + plan.z_off);
  const int RBv = a.tgt.r_pad / 16;
  const long long tiles = P / kTileRows + a.K + 1;  // upper bound on tiles of any grouping
  const bool in_place = (a.y0 == a.y);
  hipError_t err = hipSuccess;

  if (a.path == 3) {
    T8ApplyArgs ta;
    ta.t = t8_args(a);
    ta.offsets = a.offsets; ta.perm_w = a.perm_w; ta.inv = a.inv;
    const int grid = 8 * ta.t.tiles_per_xcd * ta.t.col_groups;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_t8_t<RB, IND, Y0F, YF>(ta, grid, s))))));
    return err;
  }

  if (a.path == 4) {
    bool taken = false;
    const size_t off = plan.block_off;
    err = launch_dense_block(&a, 1, &off, s, &taken);
    if (taken || err != hipSuccess) return err;
    BlockApplyArgs ba;
    ba.b = block_args(a, wsb + plan.block_off);
    ba.offsets = a.offsets; ba.perm_w = a.perm_w; ba.inv = a.inv;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_block_t<RB, IND, Y0F, YF>(ba, s))))));
    return err;
  }

  if (gm_path(a.path, a.k, a.K, a.tgt.r_pad)) {
    // 64-row grouped tiles split over 512-wide slices (k = 1: one pass; k > 1: below).
    const bool in_place = (a.y0 == a.y);
    GMArgs ga{};
    ga.tgt = a.tgt; ga.x = a.x; ga.N = a.N; ga.k = a.k; ga.scale = a.scale; ga.perm = a.perm; ga.nkeys = a.K;
    // row tiles per segment, each run as one workgroup per 512-wide slice (the tiling of the
    // plan's grouped-split region)
    const long long rows_max = a.k == 1 ? P : a.N;  // rows of one pass
    const GMTiling tl = gm_tiling(a.path, rows_max, a.K, (a.tgt.d_in + kBSlice - 1) / kBSlice);
    ga.tile_rows = tl.rows;
    ga.fixed = tl.fixed;
    // a pass = three launches over 512-wide slices of the tiles (gsplit.hip)
    float* gs_part = reinterpret_cast<float*>(wsb + plan.gs_off);
    uint16_t* gs_hb = reinterpret_cast<uint16_t*>(wsb + plan.gs_off + plan.gs.hb_off);
    auto pass = [&](const void* src, bool src_f32, void* dst, bool dst_f32, const FinishArgs* fin) {
      ga.y0 = src;
      ga.y = dst;
      ga.nwg = plan.gs.nwg;
      return launch_gs_pass(ga, gs_part, gs_hb, src_f32, dst_f32, a.indirect, s, fin);
    };
    // the tokens the last pass does not reach, finished by extra workgroups of its expand:
    // y0 for tokens without a routed pair (out of place), the fp32 carry z for tokens whose
    // routed pairs end before the last pass (when z is not y itself)
    auto finish = [&](const float* z, int c_last, bool copy_z) {
      FinishArgs f{};
      f.y0 = a.y0; f.z = z; f.y = a.y; f.inv = a.inv;
      f.N = a.N; f.k = a.k; f.c_last = c_last; f.d_out = a.tgt.d_out;
      f.y0_f32 = a.y0_f32; f.y_f32 = a.y_f32; f.copy_y0 = in_place ? 0 : 1; f.copy_z = copy_z ? 1 : 0;
      return f;
    };
    if (a.k == 1) {
      ga.key0 = 0; ga.offsets = a.offsets; ga.order = nullptr; ga.wts = a.perm_w;
      const FinishArgs f = finish(nullptr, 1, false);
      return pass(a.y0, a.y0_f32, a.y, a.y_f32, in_place ? nullptr : &f);
    }
    if (plan.tuples) {
      // k > 1 in pair passes: h of every pair by grouped position (one split shrink over the
      // dispatch's order), the tuple sort, then pass m applies each token's routed pairs of rank
      // 2m and 2m + 1; pass 0 reads y0, the last writes y, the passes between carry the sum in
      // fp32 (in y itself when y is fp32, else in z)
      const int kslices = (a.tgt.d_in + kBSlice - 1) / kBSlice;
      const GMTiling tp = gm_tiling(a.path, P, a.K, kslices);
      uint16_t* hq = reinterpret_cast<uint16_t*>(wsb + plan.hq_off);
      ga.key0 = 0; ga.offsets = a.offsets; ga.order = nullptr; ga.wts = a.perm_w;
      ga.tile_rows = tp.rows; ga.fixed = tp.fixed; ga.nwg = plan.gs.nwg;
      err = launch_gs_pair_shrink(ga, gs_part, hq, a.indirect, s);
      if (err != hipSuccess) return err;
      const TupleSortPlan& tsp = plan.tsort;
      char* tsr = wsb + plan.tsort_off;
      // pair-expand tiles: balanced heights up to kPairTileRows rows (fixed tiling: 64-row tiles)
      GMTiling te{};
      te.fixed = a.path == kPathGroupedFixed ? 1 : 0;
      te.rows = te.fixed ? kGMRows : kPairTileRows;
      te.max_tiles = (a.N + te.rows - 1) / te.rows + tsp.kk;
      err = launch_tuple_sort(a.offsets, a.inv, a.N, a.k, a.K, tsr, tsp, te, s);
      if (err != hipSuccess) return err;
      GMArgs ge = ga;
      ge.nwg = (int)((te.max_tiles + 7) / 8 * 8);
      float* z = zbuf;
      const bool copy_z = tsp.m2 > 1 && static_cast<void*>(z) != a.y;
      const FinishArgs f = finish(z, 2 * tsp.m2 - 1, copy_z);
      for (int m = 0; m < tsp.m2; ++m) {
        const bool last = m == tsp.m2 - 1;
        ge.y0 = m == 0 ? a.y0 : static_cast<const void*>(z);
        ge.y = last ? a.y : static_cast<void*>(z);
        err = launch_gs_expand_pairs(ge, tsr, tsp, m, hq, a.K, m == 0 ? (bool)a.y0_f32 : true,
                                     last ? (bool)a.y_f32 : true, a.indirect, s,
                                     last && (!in_place || copy_z) ? &f : nullptr);
        if (err != hipSuccess) return err;
      }
      return err;
    }
    // k > 1: pass j applies the j-th routed pair of every token over the (rank, adapter)
    // order of the slot sort; pass 0 reads y0, the last pass writes y and the passes in between
    // carry the sum in fp32 (in y itself when y is fp32, else in z), so a bf16 y is rounded once.
    RankSort rs;
    err = launch_rank_sort(a, wsb + plan.sort_off, P, s, rs);
    if (err != hipSuccess) return err;
    int32_t* offsets2 = rs.offsets2;
    int32_t* perm2 = rs.perm2;
    float* w2 = rs.w2;
    float* z = zbuf;
    const bool copy_z = static_cast<void*>(z) != a.y;
    const FinishArgs f = finish(z, a.k, copy_z);
    ga.offsets = offsets2; ga.order = perm2; ga.wts = w2;
    for (int j = 0; j < a.k; ++j) {
      ga.key0 = j * a.K;
      const bool last = j == a.k - 1;
      err = pass(j == 0 ? a.y0 : static_cast<const void*>(z), j == 0 ? (bool)a.y0_f32 : true,
                 last ? a.y : static_cast<void*>(z), last ? (bool)a.y_f32 : true,
                 last && (!in_place || copy_z) ? &f : nullptr);
      if (err != hipSuccess) return err;
    }
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
  sa.K = a.K; sa.k = a.k; sa.scale = a.scale; sa.P = P; sa.nsplit = nsplit;
  sa.hpart = reinterpret_cast<float*>(wsb + plan.hpart_off);
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, err = (launch_shrink_t<RB, IND>(sa, (int)tiles, s))));
  if (err != hipSuccess) return err;

  ExpandArgs ea;
  ea.tgt = a.tgt; ea.y0 = a.y0; ea.y = a.y; ea.offsets = a.offsets; ea.perm = a.perm; ea.inv = a.inv;
  ea.hpart = sa.hpart; ea.P = P; ea.nsplit = nsplit; ea.N = a.N; ea.K = a.K; ea.k = a.k;
  ea.order = nullptr;
  ea.key0 = 0;
  if (a.k == 1) {
    ea.col_groups = choose_col_groups(tiles, a.tgt.d_out, 512, 4);
    ea.main_blocks = (int)tiles * ea.col_groups;
    ea.copy_blocks = in_place ? 0 : (int)std::min<long long>((a.N + 255) / 256, 64);
    const int grid = ea.main_blocks + ea.copy_blocks;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a.y_f32, YF, err = (launch_expand_k1_t<RB, IND, Y0F, YF>(ea, grid, s))))));
    return err;
  }
  if (a.path == 2 && decode_expand_fits(a.N, a.k, a.K, a.tgt.r_pad)) {
    HsumMulti hm{};
    DecodeMulti dm{};
    hm.hpart[0] = sa.hpart;
    hm.hq[0] = reinterpret_cast<uint16_t*>(wsb + plan.hq_off);
    hm.eid[0] = reinterpret_cast<int32_t*>(wsb + plan.hq_off + decode_eid_off(P, a.tgt.r_pad));
    hm.nsplit[0] = nsplit;
    hm.offsets = a.offsets; hm.perm = a.perm; hm.P = P; hm.K = a.K;
    dm.tgt[0] = a.tgt; dm.y0[0] = a.y0; dm.y[0] = a.y; dm.hq[0] = hm.hq[0]; dm.eid[0] = hm.eid[0];
    dm.inv = a.inv; dm.N = a.N; dm.k = a.k; dm.K = a.K;
    return launch_decode_expand(hm, dm, 1, a.tgt.d_out, RBv, a.indirect, a.y0_f32, a.y_f32, s);
  }
  if (a.path == 2 && a.k * a.K <= 64) {
    // one grouped expand pass per rank of the routed pairs (as on the 64-row tiles), over
    // (adapter, 16-row tile, column group) workgroups, the sum carried in fp32
    RankSort rs;
    err = launch_rank_sort(a, wsb + plan.sort_off, P, s, rs);
    if (err != hipSuccess) return err;
    const long long ptiles = (a.N + 15) / 16 + a.K;  // 16-row tiles of one pass
    ea.offsets = rs.offsets2;
    ea.order = rs.perm2;
    ea.col_groups = choose_col_groups(ptiles, a.tgt.d_out, 512, 4);
    ea.main_blocks = (int)(ptiles * ea.col_groups);
    ea.copy_blocks = 0;
    const int grid = ea.main_blocks;
    for (int j = 0; j < a.k; ++j) {
      const bool last = j == a.k - 1;
      ea.key0 = j * a.K;
      ea.y0 = j == 0 ? a.y0 : static_cast<const void*>(zbuf);
      ea.y = last ? a.y : static_cast<void*>(zbuf);
      const bool y0f = j == 0 ? (bool)a.y0_f32 : true, yf = last ? (bool)a.y_f32 : true;
      MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.indirect, IND, MOLORA_DISPATCH_BOOL(y0f, Y0F,
          MOLORA_DISPATCH_BOOL(yf, YF, err = (launch_expand_k1_t<RB, IND, Y0F, YF>(ea, grid, s))))));
      if (err != hipSuccess) return err;
    }
    const bool copy_z = static_cast<void*>(zbuf) != a.y;
    if (in_place && !copy_z) return err;
    MOLORA_DISPATCH_BOOL(a.y0_f32, Y0F, MOLORA_DISPATCH_BOOL(a.y_f32, YF,
        err = (launch_finish_t<Y0F, YF>(a.y0, zbuf, a.y, a.inv, a.N, a.k, a.tgt.d_out, !in_place, copy_z, s))));
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

// Several targets sharing one routing.  The skinny path runs each phase for all targets in one
// launch (the rank sort once); other paths apply the targets in turn, each with its own slice of
// the workspace.  Workspace: [rank sort] then per target [h partials][fp32 carry].
hipError_t launch_apply_multi(const ApplyLaunch* as, int n, hipStream_t s) {
  const ApplyLaunch& a0 = as[0];
  hipError_t err = hipSuccess;
  char* wsb = reinterpret_cast<char*>(a0.ws);
  int d_in[kApplyMaxMulti], d_out[kApplyMaxMulti];
  for (int i = 0; i < n; ++i) {
    d_in[i] = as[i].tgt.d_in;
    d_out[i] = as[i].tgt.d_out;
  }
  const MultiPlan mp = apply_multi_plan(n, d_in, d_out, a0.N, a0.k, a0.K, a0.tgt.r_pad, a0.y_f32, a0.path);
  if (a0.path == 4) {
    // 64-token blocks: one shrink launch and one expand launch for all targets
    bool taken = false;
    err = launch_dense_block(as, n, mp.tgt_off, s, &taken);
    if (taken || err != hipSuccess) return err;
    static_assert(sizeof(BlockMulti) / sizeof(BlockApplyArgs) == kApplyMaxMulti, "multi size");
    BlockMulti bm;
    int gs = 1, ge = 1;
    for (int i = 0; i < n; ++i) {
      const ApplyLaunch& b = as[i];
      bm.a[i].b = block_args(b, wsb + mp.tgt_off[i]);
      bm.a[i].offsets = b.offsets;
      bm.a[i].perm_w = b.perm_w;
      bm.a[i].inv = b.inv;
      gs = std::max(gs, block_grid(bm.a[i].b.nblocks, bm.a[i].b.kslices));
      ge = std::max(ge, block_grid(bm.a[i].b.nblocks, bm.a[i].b.cslices));
    }
    const int RBv = a0.tgt.r_pad / 16;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a0.indirect, IND,
        hipLaunchKernelGGL((shrink_block_multi<RB, IND>), dim3(gs, n), dim3(kBThreads), 0, s, bm)));
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a0.indirect, IND, MOLORA_DISPATCH_BOOL(a0.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a0.y_f32, YF,
            hipLaunchKernelGGL((expand_block_multi<RB, IND, Y0F, YF>), dim3(ge, n), dim3(kBThreads), 0, s, bm)))));
    return hipGetLastError();
  }
  if (!mp.fused) {
    for (int i = 0; i < n; ++i) {
      ApplyLaunch b = as[i];
      b.ws = reinterpret_cast<float*>(wsb + mp.tgt_off[i]);
      err = launch_apply(b, s);
      if (err != hipSuccess) return err;
    }
    return err;
  }
  const long long P = (long long)a0.N * a0.k;
  const long long tiles = P / kTileRows + a0.K + 1;
  const int RBv = a0.tgt.r_pad / 16;
  ShrinkMulti sm;
  float* z[kApplyMaxMulti];
  int max_split = 1;
  for (int i = 0; i < n; ++i) {
    const ApplyLaunch& a = as[i];
    ShrinkArgs& sa = sm.a[i];
    sa.tgt = a.tgt; sa.x = a.x; sa.offsets = a.offsets; sa.perm = a.perm; sa.perm_w = a.perm_w;
    sa.K = a.K; sa.k = a.k; sa.scale = a.scale; sa.P = P; sa.nsplit = skinny_splits(a.tgt.d_in);
    sa.hpart = reinterpret_cast<float*>(wsb + mp.hpart_off[i]);
    z[i] = a.y_f32 ? reinterpret_cast<float*>(a.y) : nullptr;
    if (a.k > 1 && !a.y_f32) z[i] = reinterpret_cast<float*>(wsb + mp.z_off[i]);
    max_split = std::max(max_split, sa.nsplit);
  }
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a0.indirect, IND,
      hipLaunchKernelGGL((shrink_grouped_multi<RB, IND>), dim3((int)(tiles + 7) / 8 * 8, max_split, n), dim3(256), 0, s, sm)));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mp.decode) {
    HsumMulti hm{};
    DecodeMulti dm{};
    int max_dout = 0;
    for (int i = 0; i < n; ++i) {
      hm.hpart[i] = sm.a[i].hpart;
      hm.hq[i] = reinterpret_cast<uint16_t*>(wsb + mp.hq_off[i]);
      hm.eid[i] = reinterpret_cast<int32_t*>(wsb + mp.hq_off[i] + decode_eid_off(P, a0.tgt.r_pad));
      hm.nsplit[i] = sm.a[i].nsplit;
      dm.tgt[i] = as[i].tgt; dm.y0[i] = as[i].y0; dm.y[i] = as[i].y; dm.hq[i] = hm.hq[i]; dm.eid[i] = hm.eid[i];
      max_dout = std::max(max_dout, as[i].tgt.d_out);
    }
    hm.offsets = a0.offsets; hm.perm = a0.perm; hm.P = P; hm.K = a0.K;
    dm.inv = a0.inv; dm.N = a0.N; dm.k = a0.k; dm.K = a0.K;
    return launch_decode_expand(hm, dm, n, max_dout, RBv, a0.indirect, a0.y0_f32, a0.y_f32, s);
  }

  ExpandMulti em;
  auto expand_args = [&](int i, long long t) {
    const ApplyLaunch& a = as[i];
    ExpandArgs& ea = em.a[i];
    ea.tgt = a.tgt; ea.y0 = a.y0; ea.y = a.y; ea.offsets = a.offsets; ea.perm = a.perm; ea.inv = a.inv;
    ea.hpart = sm.a[i].hpart; ea.P = P; ea.nsplit = sm.a[i].nsplit; ea.N = a.N; ea.K = a.K; ea.k = a.k;
    ea.order = nullptr;
    ea.key0 = 0;
    ea.col_groups = choose_col_groups(t, a.tgt.d_out, 512, 8);  // measured on the 28-layer decode stack
    ea.main_blocks = (int)(t * ea.col_groups);
    ea.copy_blocks = 0;
    return ea.main_blocks;
  };
  if (a0.k == 1) {
    int gx = 1;
    for (int i = 0; i < n; ++i) {
      expand_args(i, tiles);
      ExpandArgs& ea = em.a[i];
      ea.copy_blocks = as[i].y0 == as[i].y ? 0 : (int)std::min<long long>((as[i].N + 255) / 256, 64);
      gx = std::max(gx, ea.main_blocks + ea.copy_blocks);
    }
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a0.indirect, IND, MOLORA_DISPATCH_BOOL(a0.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a0.y_f32, YF,
            hipLaunchKernelGGL((expand_grouped_multi<RB, IND, Y0F, YF>), dim3(gx, n), dim3(256), 0, s, em)))));
    return hipGetLastError();
  }
  // k > 1: the rank sort once (shared routing), then one pass per rank over all targets
  RankSort rs;
  err = launch_rank_sort(a0, wsb + mp.sort_off, P, s, rs);
  if (err != hipSuccess) return err;
  const long long ptiles = (a0.N + 15) / 16 + a0.K;
  int gx = 1;
  for (int i = 0; i < n; ++i) gx = std::max(gx, expand_args(i, ptiles));
  for (int i = 0; i < n; ++i) {
    em.a[i].offsets = rs.offsets2;
    em.a[i].order = rs.perm2;
  }
  for (int j = 0; j < a0.k; ++j) {
    const bool last = j == a0.k - 1;
    for (int i = 0; i < n; ++i) {
      em.a[i].key0 = j * a0.K;
      em.a[i].y0 = j == 0 ? as[i].y0 : static_cast<const void*>(z[i]);
      em.a[i].y = last ? as[i].y : static_cast<void*>(z[i]);
    }
    const bool y0f = j == 0 ? (bool)a0.y0_f32 : true, yf = last ? (bool)a0.y_f32 : true;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a0.indirect, IND, MOLORA_DISPATCH_BOOL(y0f, Y0F,
        MOLORA_DISPATCH_BOOL(yf, YF,
            hipLaunchKernelGGL((expand_grouped_multi<RB, IND, Y0F, YF>), dim3(gx, n), dim3(256), 0, s, em)))));
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  FinishMulti fm;
  bool any = false;
  for (int i = 0; i < n; ++i) {
    fm.y0[i] = as[i].y0;
    fm.z[i] = z[i];
    fm.y[i] = as[i].y;
    fm.d_out[i] = as[i].tgt.d_out;
    fm.copy_y0[i] = as[i].y0 != as[i].y;
    fm.copy_z[i] = static_cast<void*>(z[i]) != as[i].y;
    any = any || fm.copy_y0[i] || fm.copy_z[i];
  }
  if (!any) return err;
  fm.inv = a0.inv;
  fm.N = a0.N;
  fm.k = a0.k;
  MOLORA_DISPATCH_BOOL(a0.y0_f32, Y0F, MOLORA_DISPATCH_BOOL(a0.y_f32, YF,
      hipLaunchKernelGGL((finish_tokens_multi<Y0F, YF>), dim3((a0.N + 255) / 256, n), dim3(256), 0, s, fm)));
  return hipGetLastError();
}

hipError_t launch_step_vocab(const StepVocabLaunch& a, hipStream_t s) {
  StepArgs sa;
  sa.t = t8_args(a.apply);
  const int K = a.apply.K;
  sa.bounds.lo = a.bounds.b[0];
  sa.bounds.hi = a.bounds.b[K];
  for (int i = 0; i < kT8MaxU - 1; ++i) sa.bounds.mid[i] = (i + 1 < K) ? a.bounds.b[i + 1] : INT_MAX;
  sa.ids = a.ids; sa.idx = a.idx; sa.w = a.w; sa.counts = a.counts; sa.offsets = a.offsets; sa.perm = a.perm;
  sa.perm_w = a.perm_w; sa.inv = a.inv;
  sa.dispatch_share = a.dispatch_share ? 1 : 0;
  const int RBv = a.apply.tgt.r_pad / 16;
  hipError_t err = hipSuccess;
  if (a.part != nullptr) {
    SplitGeom g;
    g.nblocks = (a.apply.N + kSTok - 1) / kSTok;
    g.kslices = (a.apply.tgt.d_in + kSSlice - 1) / kSSlice;
    g.cslices = (a.apply.tgt.d_out + kSSlice - 1) / kSSlice;
    g.part = a.part;
    g.bcnt = a.bcnt;
    MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.apply.indirect, IND, MOLORA_DISPATCH_BOOL(a.apply.y0_f32, Y0F,
        MOLORA_DISPATCH_BOOL(a.apply.y_f32, YF, err = (launch_split_t<RB, IND, Y0F, YF>(sa, g, s))))));
    return err;
  }
  const int grid = 8 * sa.t.tiles_per_xcd * sa.t.col_groups;
  MOLORA_DISPATCH_RB(RBv, MOLORA_DISPATCH_BOOL(a.apply.indirect, IND, MOLORA_DISPATCH_BOOL(a.apply.y0_f32, Y0F,
      MOLORA_DISPATCH_BOOL(a.apply.y_f32, YF, err = (launch_step_t<RB, IND, Y0F, YF>(sa, grid, s))))));
  return err;
}

// --------------------------------------------------------------------------------------
// Hot-set relayout of one adapter.
//   A [d_in][r] -> swizzled slab blocks (see a_swz_index); ranks r..r_pad-1 are zero.
//   B [r][d_out] -> B^T [d_out][r_pad] with the columns of each 128-column block permuted
//   (slab row w holds column b_perm_col(w)); ranks r..r_pad-1 are zero.
//   Source strides: element (row, rank j) of the [d][r] matrix being laid out is read at
//   src[row * s_row + j * s_j] (A itself: s_row = r, s_j = 1; the transposed twin's A = B^T
//   of a forward adapter: s_row = 1, s_j = d).
__global__ void relayout_A(const uint16_t* __restrict__ A, uint16_t* __restrict__ As, int d_in, int r, int r_pad,
                           long long s_row, long long s_j) {
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
  As[idx] = (j < r) ? A[(long long)col * s_row + (long long)j * s_j] : (uint16_t)0;
}
// Element (rank j, column col) of the [r][d] matrix is read at src[j * s_j + col * s_col] (B
// itself: s_j = d_out, s_col = 1; the twin's B = A^T of a forward adapter: s_j = 1, s_col = r).
__global__ void relayout_B(const uint16_t* __restrict__ B, uint16_t* __restrict__ Bt, int d_out, int r, int r_pad,
                           long long s_j, long long s_col) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)d_out * r_pad) return;
  const int row = (int)(i / r_pad), j = (int)(i % r_pad);
  const int col = b_perm_col(row);
  Bt[i] = (j < r) ? B[(long long)j * s_j + (long long)col * s_col] : (uint16_t)0;
}

hipError_t launch_relayout(const uint16_t* A, const uint16_t* B, int d_in, int d_out, int r, int r_pad,
                           uint16_t* At, uint16_t* Bt, hipStream_t s, bool transposed) {
  const long long na = (long long)r_pad * d_in, nb = (long long)d_out * r_pad;
  // transposed: the slab adapter (d_in x r, r x d_out) is (B^T, A^T) of the forward adapter
  // whose A is [d_out][r] and B is [r][d_in]
  const uint16_t* srcA = transposed ? B : A;
  const uint16_t* srcB = transposed ? A : B;
  const long long sa_row = transposed ? 1 : r, sa_j = transposed ? d_in : 1;
  const long long sb_j = transposed ? 1 : d_out, sb_col = transposed ? r : 1;
  hipLaunchKernelGGL(relayout_A, dim3((unsigned)((na + 255) / 256)), dim3(256), 0, s, srcA, At, d_in, r, r_pad,
                     sa_row, sa_j);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(relayout_B, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, srcB, Bt, d_out, r, r_pad,
                     sb_j, sb_col);
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

// --------------------------------------------------------------------------------------
// Scratch memory of the entry points that allocate nothing: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in symbol); it takes each device's address once with
// hipGetSymbolAddress, with that device current, and passes that address.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_addr;  // per device ordinal; nullptr until looked up
}  // namespace

hipError_t scratch_setup(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_addr.size()) g_scratch_addr.resize((size_t)dev + 1, nullptr);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  if (out != nullptr) *out = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace molora
