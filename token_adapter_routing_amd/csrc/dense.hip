// Dense-slot 64-token blocks for small hot sets (MoLoRA pages, thelatestinai.com: per-token
// routing, Figure 2 right -- every token's delta is the gate-weighted sum of its selected
// adapters' x A_e B_e; Table 1 rows "Routing decision" and "Grouped LoRA shrink / expand").
//
// When the 512-wide slices of all K adapters of a target fit in LDS together (K * r_pad <= 64:
// four adapters of rank 16, two of rank 32), the block path needs no per-block adapter list:
//
//   shrink_dense  workgroup = 128 tokens (two 64-token blocks) x one 512-wide d_in slice of one
//                 target.  The A slices of all K adapters go straight into LDS; each of the 8
//                 waves takes one 16-token row block through every step of the slice and every
//                 adapter, then scales each row's partial by that token's gate weight on the
//                 adapter (the sum of its slots' weights there, 0 if it does not use it) and
//                 stores one partial plane per adapter, [block][plane][slice][64][r_pad] fp32 --
//                 or, when a token has fewer slots than there are adapters (k < K), one plane
//                 per slot holding its adapter's partial (a slot that repeats an earlier slot's
//                 adapter holds 0).
//                 The routing (grouped position -> adapter from the offsets, gate weight from
//                 perm_w) returns while the x rows are in flight.
//   expand_dense  workgroup = 64 tokens x one 512-wide d_out slice of one target.  The B^T
//                 slices of all K adapters (straight into LDS), the slots' adapters (per-slot
//                 planes), the partials and the y0 rows are requested at once, in that order
//                 (loads return in issue order), so h
//                 (alpha/r x the slice sum, split into bf16 hi / lo) and the MFMAs run while
//                 the y0 rows are still arriving; y = y0 + sum_e h_e B_e.
// With one slot per token of weight 1 (vocabulary routing) every rounding step is the split
// step's -- the two half-slice chains of the shrink, the slice sum in order, then alpha/r -- so
// the two give the same bits.
//
// Several targets run in one launch of each kernel: workgroup b works on the (target, slice)
// item of a table in the arguments.  In the shrink, the targets that read the same x form a
// column per slice; an XCD runs the columns in turn, each over its pair blocks with the
// column's targets back to back, so the x rows of a block and the column's A slices stay in
// its L2 (workgroups are dispatched round robin over the 8 XCDs).  Every item of pair block pb
// runs on XCD pb mod 8 in both kernels, where the expand finds the partials the shrink wrote.
#include "dispatch_dev.h"
#include "molora_launch.h"
#include "molora_mfma.h"

namespace molora {

namespace {

constexpr int kDTok = 2 * kBTok;                    // shrink: tokens per workgroup
constexpr int kDWaves = 8;
constexpr int kDThreads = kDWaves * kWave;
constexpr int kDLdsElems = 4 * kBSlice * 16;       // all adapters' slices of one 512 slice: 64 KB
constexpr int kDStepsPerSlice = kBSlice / kStepK;  // 4

struct DenseTarget {
  TargetDev tgt;
  const uint16_t* x;
  const void* y0;
  void* y;
  float* part;  // [nblocks][K][kslices][64][r_pad] fp32
  int kslices, cslices;
};

struct DenseArgs {
  DenseTarget t[kApplyMaxMulti];
  const int32_t* offsets;
  const float* perm_w;
  const int32_t* inv;
  DenseFuse fuse;  // routing as (idx, w) and, from disp_wgs leading workgroups, the dispatch
  int disp_wgs;
  int per_slot;    // k < K: one partial plane per routed slot (else one per adapter)
  int N, K, k;
  float scale;
  int nblocks, npairs;  // 64-token blocks, 128-token pair blocks
  int items_s, items_e;
  uint16_t item_s[kDenseMaxItems];  // shrink items: (target << 8) | d_in slice
  uint16_t col_start[kDenseMaxItems];  // the shrink column (x group, slice) of each item
  uint8_t col_len[kDenseMaxItems];
  uint16_t item_e[kDenseMaxItems];  // expand items: (target << 8) | d_out slice
};

// (adapter, gate weight) of pair p from the routing arrays (the dispatch's source)
struct PairSource {
  const int32_t* idx;
  const float* w;
  __device__ __forceinline__ void operator()(int p, int& e, float& wv) const {
    e = idx[p];
    wv = w[p];
  }
};

// s_waitcnt immediate for "at most n vector memory operations outstanding" (gfx9 encoding:
// vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt at their no-wait maxima).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Copy `bytes` (a multiple of 1 KB) from global src to LDS dst: each wave instruction moves
// 1 KB, lane l's 16 bytes landing at dst + 16 l; wave w takes the pieces w, w + 8, ...
__device__ __forceinline__ void dense_lds_copy(void* dst, const void* src, int bytes, int wave, int lane) {
  for (int off = wave * 1024; off < bytes; off += kDWaves * 1024)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + off + 16 * lane,
                                     reinterpret_cast<char*>(dst) + off, 16, 0, 0);
}

// DIRECT: the pairs' adapters and weights come from the routing arrays (idx, w); the leading
// a.disp_wgs workgroups run the dispatch of those pairs instead of a shrink item.
template <int RB, bool INDIRECT, int KM, bool DIRECT>
__global__ __launch_bounds__(kDThreads, 2) void shrink_dense(const DenseArgs a) {
  __shared__ alignas(16) uint16_t As[kDLdsElems];  // [adapter][step][chunk][u][64 lanes x 16 B]
  int bid = blockIdx.x;
  if constexpr (DIRECT) {
    if (bid < a.disp_wgs) {
      const int P = a.N * a.k;
      if (bid * kDThreads >= P) return;  // past the pairs (the count rounds up to whole XCD rounds)
      static_assert(sizeof(DispatchLds<kDThreads>) <= sizeof(As), "dispatch tables in the shrink's LDS");
      dispatch_wide_part<kDThreads, PairSource, 4>(*reinterpret_cast<DispatchLds<kDThreads>*>(As),
                                                   PairSource{a.fuse.idx, a.fuse.w}, P, a.K, bid, a.fuse.counts,
                                                   a.fuse.offsets, a.fuse.perm, a.fuse.perm_w, a.fuse.inv);
      return;
    }
    bid -= a.disp_wgs;  // a multiple of 8: the XCD of every item is unchanged
  }
  const int xcd = bid & 7, qb = bid >> 3;
  // an XCD takes the columns (one x group at one slice) in turn, each over its pair blocks, and
  // a column's targets back to back: the x rows and the column's A slices stay in its L2
  const int npg = (a.npairs + 7) / 8;
  const int i0 = qb / npg;  // an item of this workgroup's column
  const int cs = a.col_start[i0], len = a.col_len[i0];
  const int local = qb - npg * cs;
  const int pb = (local / len) * 8 + xcd;
  if (pb >= a.npairs) return;
  const int item = a.item_s[cs + local % len];
  const DenseTarget& T = a.t[item >> 8];
  const int sl = item & 255;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int N = a.N, K = a.K, k = a.k;
  const int d_in = T.tgt.d_in, r_pad = T.tgt.r_pad;
  const int S = d_in / kStepK;
  const int s0 = sl * kDStepsPerSlice, s1 = min(s0 + kDStepsPerSlice, S), ns = s1 - s0;
  const int r0 = pb * kDTok + kWave / 4 * wave;  // first token of the wave's row block
  constexpr size_t piece = (size_t)RB * 16 * kStepK;  // elements of one step's pieces
  constexpr int kAdapterElems = kDStepsPerSlice * (int)piece;

  // 1. routing of the lane's MFMA rows (tokens r0 + 4G + i): segment starts, and the grouped
  // positions of the rows' pairs, spread over the 16 lanes of a lane group: lane n takes the
  // slots n % 4, n % 4 + 4, .. of row n / 4
  constexpr int PPL = (KM + 3) / 4;  // pairs per lane
  int seg_start[3] = {0x7fffffff, 0x7fffffff, 0x7fffffff};
  if constexpr (!DIRECT) {
#pragma unroll
    for (int i = 0; i < 3; ++i) seg_start[i] = (i + 1 < K) ? a.offsets[i + 1] : 0x7fffffff;
  }
  int qv[PPL];
  float wd[PPL];
  {
    const long long t = min(r0 + 4 * G + (n >> 2), N - 1);
#pragma unroll
    for (int m = 0; m < PPL; ++m) {
      const long long p = t * k + min((n & 3) + 4 * m, k - 1);
      if constexpr (DIRECT) {
        qv[m] = a.fuse.idx[p];
        wd[m] = a.fuse.w[p];
      } else {
        qv[m] = a.inv[p];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // 2. the slice of every adapter's A, straight into LDS
  for (int e = 0; e < K; ++e)
    dense_lds_copy(As + e * kAdapterElems, adapter_A<INDIRECT>(T.tgt, e) + (size_t)s0 * piece, ns * (int)piece * 2,
                   wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  // 3. the x rows of the wave's 16 tokens over the slice (steps past the end re-read the last)
  const int row = min(r0 + n, N - 1);
  const uint16_t* xp = T.x + (size_t)row * d_in + 8 * G;
  u32x4_t xv[kDStepsPerSlice][4];
#pragma unroll
  for (int i = 0; i < kDStepsPerSlice; ++i) {
    const int st = min(s0 + i, s1 - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[i][c] = ld16(xp + (size_t)st * kStepK + 32 * c);
  }
  __builtin_amdgcn_sched_barrier(0);
  // everything but the x rows has arrived: routing in registers, this wave's A pieces in LDS
  __builtin_amdgcn_s_waitcnt(vmcnt_only(kDStepsPerSlice * 4));
  int ev[PPL];
  float wv[PPL];
#pragma unroll
  for (int m = 0; m < PPL; ++m) {
    const bool slot = (n & 3) + 4 * m < k;
    if constexpr (DIRECT) {
      // the pair's adapter as given (outside [0, K): unrouted) and its weight, the values the
      // dispatch copies into perm_w
      ev[m] = (slot && qv[m] >= 0 && qv[m] < K) ? qv[m] : -1;
      wv[m] = wd[m];
    } else {
      const int q = slot ? qv[m] : -1;
      ev[m] = q < 0 ? -1 : (q >= seg_start[0]) + (q >= seg_start[1]) + (q >= seg_start[2]);
      wv[m] = a.perm_w[max(q, 0)];  // returns behind the x rows
    }
  }
  __syncthreads();  // every wave's A pieces are in LDS
  // gate weight of each of the lane's rows on each adapter: the sum over the row's slots (the
  // four lanes of the row, then to every lane of the group); alpha/r follows the slice sum
  float wt[4 / RB][4];
  auto fold_weights = [&] {
#pragma unroll
    for (int e = 0; e < 4 / RB; ++e) {
      float v = 0.f;
#pragma unroll
      for (int m = 0; m < PPL; ++m) v += (ev[m] == e) ? wv[m] : 0.f;
      v += __shfl_xor(v, 1, kWave);
      v += __shfl_xor(v, 2, kWave);
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[e][i] = __shfl(v, 16 * G + 4 * i, kWave);
    }
  };

  // two chains per adapter, steps 0-1 and 2-3 of the slice, added at the end (the split
  // step's order, so that its results and these agree bit for bit)
  f32x4_t acc[2][4 / RB][RB];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 4 / RB; ++e)
#pragma unroll
      for (int u = 0; u < RB; ++u) acc[hh][e][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4 / RB; ++e) {
    if (e < K) {
#pragma unroll
      for (int i = 0; i < kDStepsPerSlice; ++i) {
        if (i < ns) {
          const uint16_t* ap = As + e * kAdapterElems + (size_t)i * piece;
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int u = 0; u < RB; ++u) {
              // lane (n, G) takes its 16 bytes at position 4n + G of the 1 KB piece (slab swizzle)
              const u32x4_t av = *reinterpret_cast<const u32x4_t*>(ap + ((c * RB + u) * 64 + 4 * n + G) * 8);
              acc[i >> 1][e][u] = mfma16x16x32(as_bf16x8(xv[i][c]), as_bf16x8(av), acc[i >> 1][e][u]);
            }
        }
      }
    }
  }
  // partial x A_e of each row, times the row's gate weight on e
  const int tb = r0 / kBTok;
  if (tb >= a.nblocks) return;  // second half of an odd last pair: no such block (wave-uniform)
  const int rowb = r0 % kBTok;
  fold_weights();
  if (a.per_slot) {
    // one plane per routed slot s: the partial of the slot's adapter times the token's weight
    // on it; a slot repeating an earlier slot's adapter stores 0 (the earlier one holds the sum)
    static_assert(PPL == 1, "a row's slots sit in four lanes");
    int es[4][4];  // [row i][slot s]: lane 4i + s of the group holds the pair
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) es[i][t] = __shfl(ev[0], 16 * G + 4 * i + t, kWave);
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      if (t < k) {
        float* dst = T.part + block_part_index(tb, t, sl, K, T.kslices, r_pad) + (size_t)(rowb + 4 * G) * r_pad + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = es[i][t];
          bool first = e >= 0;
#pragma unroll
          for (int t2 = 0; t2 < KM; ++t2)
            if (t2 < t) first = first && es[i][t2] != e;
#pragma unroll
          for (int u = 0; u < RB; ++u) {
            float v = 0.f;
#pragma unroll
            for (int ee = 0; ee < 4 / RB; ++ee)
              if (first && ee == e) v = (acc[0][ee][u][i] + acc[1][ee][u][i]) * wt[ee][i];
            dst[(size_t)i * r_pad + 16 * u] = v;
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4 / RB; ++e) {
    if (e < K) {
      float* dst = T.part + block_part_index(tb, e, sl, K, T.kslices, r_pad) + (size_t)(rowb + 4 * G) * r_pad + n;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < RB; ++u) dst[(size_t)i * r_pad + 16 * u] = (acc[0][e][u][i] + acc[1][e][u][i]) * wt[e][i];
    }
  }
}

template <int RB, bool INDIRECT, bool Y0F32, bool YF32>
__global__ __launch_bounds__(kDThreads, 2) void expand_dense(const DenseArgs a) {
  constexpr int RP = RB * 16;
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  constexpr int NY0 = Y0F32 ? 16 : 8;  // y0 loads per lane (two 128-column blocks)
  constexpr int KS = Y0F32 ? 4 : 8;    // slices per item requested ahead of the y0 rows
  constexpr int RQ = RP / 4;           // 16-byte rank quads per row
  constexpr int NQ = (4 / RB) * kBTok * RQ;            // items (adapter, token, quad) at K = 4 / RB
  constexpr int QPT = (NQ + kDThreads - 1) / kDThreads;  // items per thread
  __shared__ alignas(16) uint16_t Bs[kDLdsElems];            // [adapter][512][r_pad] B^T rows of the slice
  __shared__ alignas(16) uint16_t hb[(4 / RB) * 2 * kBTok * RP];  // [adapter][hi, lo][token][rank]
  const int xcd = blockIdx.x & 7, qb = blockIdx.x >> 3;
  const int per = 2 * a.items_e;
  const int pb = (qb / per) * 8 + xcd;
  const int rem = qb % per;
  const int tb = 2 * pb + rem / a.items_e;
  if (pb >= a.npairs || tb >= a.nblocks) return;
  const int item = a.item_e[rem % a.items_e];
  const DenseTarget& T = a.t[item >> 8];
  const int cs = item & 255;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4, rb = wave & 3, ch = wave >> 2;
  const int N = a.N, K = a.K;
  const int d_out = T.tgt.d_out;
  const int t0 = tb * kBTok;
  const int c0 = cs * kBSlice, c1 = min(c0 + kBSlice, d_out);
  const int nb = (c1 - c0) / kColBlock;  // 128-column blocks in the slice
  const int b0 = min(2 * ch, nb - 1), b1 = min(2 * ch + 1, nb - 1);
  const bool has0 = 2 * ch < nb, has1 = 2 * ch + 1 < nb;

  const bool per_slot = a.per_slot != 0;
  if (per_slot) {
    // h rows of the adapters a token does not use stay 0
    for (int i = threadIdx.x; i < (int)(sizeof(hb) / 16); i += kDThreads)
      reinterpret_cast<u32x4_t*>(hb)[i] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  // 1. every adapter's B^T rows of the slice, straight into LDS
  for (int e = 0; e < K; ++e)
    dense_lds_copy(Bs + e * kBSlice * RP, adapter_B<INDIRECT>(T.tgt, e) + (size_t)c0 * RP, (c1 - c0) * RP * 2, wave,
                   lane);
  __builtin_amdgcn_sched_barrier(0);
  // per-slot planes: the adapter of every slot of each item's token (grouped position -> adapter
  // by the offsets, or the routing as given)
  const int kk = a.k;
  const int nplanes = per_slot ? kk : K;
  int rq_[QPT][4];
  int seg_start[3] = {0x7fffffff, 0x7fffffff, 0x7fffffff};
  if (per_slot) {
    if (a.fuse.idx == nullptr) {
#pragma unroll
      for (int i = 0; i < 3; ++i) seg_start[i] = (i + 1 < K) ? a.offsets[i + 1] : 0x7fffffff;
    }
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int v = min(j * kDThreads + (int)threadIdx.x, nplanes * kBTok * RQ - 1);
      const long long t = min(t0 + (v / RQ) % kBTok, N - 1);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const long long pp = t * kk + min(s2, kk - 1);
        rq_[j][s2] = a.fuse.idx != nullptr ? a.fuse.idx[pp] : a.inv[pp];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // 2. the partials: thread item v = (plane, token, rank quad), its first KS slices
  const int nq = nplanes * kBTok * RQ;
  const float* pbase = T.part + block_part_index(tb, 0, 0, K, T.kslices, RP);
  const size_t slice_f = (size_t)kBTok * RP, adapter_f = (size_t)T.kslices * slice_f;
  u32x4_t pv[QPT][KS];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int v = min(j * kDThreads + (int)threadIdx.x, nq - 1);
    const float* src = pbase + (size_t)(v / (kBTok * RQ)) * adapter_f + (size_t)4 * (v % (kBTok * RQ));
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (s < T.kslices) pv[j][s] = ld16(src + (size_t)s * slice_f);
  }
  __builtin_amdgcn_sched_barrier(0);
  // 3. the y0 rows of the wave's tokens 4G..4G+3 of its row block (clones of N - 1 past the end)
  const char* y0rows[4];
  char* yrows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = min(t0 + 16 * rb + 4 * G + i, N - 1);
    y0rows[i] = reinterpret_cast<const char*>(T.y0) + (size_t)t * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(T.y) + (size_t)t * d_out * yb;
  }
  RowChunk<Y0F32> yc0, yc1;
  load_row_chunk<Y0F32>(yc0, y0rows, c0 + b0 * kColBlock, n);
  load_row_chunk<Y0F32>(yc1, y0rows, c0 + b1 * kColBlock, n);
  __builtin_amdgcn_sched_barrier(0);
  // everything before the y0 rows has arrived (vmcnt = those rows' loads)
  __builtin_amdgcn_s_waitcnt(vmcnt_only(NY0));
  // 4. h = alpha/r x the sum of the (gate-weighted) slices in order, split into bf16 hi / lo
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    const int v = j * kDThreads + (int)threadIdx.x;
    if (v < nq) {
      const int plane = v / (kBTok * RQ), tok = (v / RQ) % kBTok, rk = 4 * (v % RQ);
      // the adapter whose h row this plane fills: the plane itself, or the slot's adapter
      // (nothing for an unrouted slot or one that repeats an earlier slot's adapter)
      int e = plane;
      if (per_slot) {
        int es[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const int q = rq_[j][s2];
          if (a.fuse.idx != nullptr) es[s2] = (s2 < kk && q >= 0 && q < K) ? q : -1;
          else es[s2] = (s2 < kk && q >= 0) ? (q >= seg_start[0]) + (q >= seg_start[1]) + (q >= seg_start[2]) : -1;
        }
        e = -1;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          if (s2 == plane) e = es[s2];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          if (s2 < plane && es[s2] == e) e = -1;
      }
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        if (s < T.kslices)
#pragma unroll
          for (int c = 0; c < 4; ++c) sum[c] += __uint_as_float(pv[j][s][c]);
      const float* src = pbase + (size_t)plane * adapter_f + (size_t)4 * (v % (kBTok * RQ));
      for (int s = KS; s < T.kslices; ++s) {
        const u32x4_t pw = ld16(src + (size_t)s * slice_f);
#pragma unroll
        for (int c = 0; c < 4; ++c) sum[c] += __uint_as_float(pw[c]);
      }
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float hv = sum[c] * a.scale;
        const __bf16 h = (__bf16)hv;
        hi[c] = __builtin_bit_cast(uint16_t, h);
        lo[c] = __builtin_bit_cast(uint16_t, (__bf16)(hv - (float)h));
      }
      if (e >= 0) {
        uint16_t* hp = hb + ((size_t)(e * 2) * kBTok + tok) * RP + rk;
        *reinterpret_cast<uint2*>(hp) = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
        *reinterpret_cast<uint2*>(hp + kBTok * RP) =
            make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
      }
    }
  }
  __syncthreads();  // h and every wave's B pieces are in LDS
  // 5. y = y0 + sum_e h_e B_e: A operand row n of the row block, groups 0, 1 hi of ranks
  // 16u + 8(G & 1) .., groups 2, 3 lo of the same ranks
  f32x4_t o0[8], o1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    o0[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    o1[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int e = 0; e < 4 / RB; ++e) {
    if (e < K) {
      bf16x8_t hv[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u)
        hv[u] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
            hb + ((size_t)(e * 2 + (G >> 1)) * kBTok + 16 * rb + n) * RP + u * 16 + 8 * (G & 1)));
      const uint16_t* Bl = Bs + e * kBSlice * RP;
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
  if (has0) epilogue_store<Y0F32, YF32>(o0, yc0, yrows, c0 + b0 * kColBlock, n, 0xFu);
  if (has1) epilogue_store<Y0F32, YF32>(o1, yc1, yrows, c0 + b1 * kColBlock, n, 0xFu);
}

template <int RB, bool IND, int KM, bool DIRECT>
hipError_t launch_shrink_dense_t(const DenseArgs& da, int grid, hipStream_t s) {
  hipLaunchKernelGGL((shrink_dense<RB, IND, KM, DIRECT>), dim3(grid), dim3(kDThreads), 0, s, da);
  return hipGetLastError();
}
template <int RB, bool IND, bool Y0F, bool YF>
hipError_t launch_expand_dense_t(const DenseArgs& da, int grid, hipStream_t s) {
  hipLaunchKernelGGL((expand_dense<RB, IND, Y0F, YF>), dim3(grid), dim3(kDThreads), 0, s, da);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_block(const ApplyLaunch* as, int n, const size_t* ws_off, hipStream_t s, bool* taken,
                              const DenseFuse* fuse) {
  const ApplyLaunch& a0 = as[0];
  *taken = false;
  // k <= K <= 4 here (a token's slots: at most four)
  if (!dense_block_ok(a0.K, a0.tgt.r_pad) || a0.k > 4) return hipSuccess;
  const long long P = (long long)a0.N * a0.k;
  if (fuse != nullptr && P > kDenseFuseMaxPairs) return hipSuccess;  // K <= 4 here
  DenseArgs da{};
  if (fuse != nullptr) {
    da.fuse = *fuse;
    da.disp_wgs = (int)(8 * ((P + 8 * kDThreads - 1) / (8 * kDThreads)));
  }
  da.offsets = a0.offsets;
  da.perm_w = a0.perm_w;
  da.inv = a0.inv;
  da.N = a0.N;
  da.K = a0.K;
  da.k = a0.k;
  da.scale = a0.scale;
  da.nblocks = (a0.N + kBTok - 1) / kBTok;
  da.per_slot = a0.k < a0.K;
  da.npairs = (a0.N + kDTok - 1) / kDTok;
  int kslices[kApplyMaxMulti], cslices[kApplyMaxMulti];
  for (int i = 0; i < n; ++i) {
    const ApplyLaunch& b = as[i];
    DenseTarget& t = da.t[i];
    t.tgt = b.tgt;
    t.x = b.x;
    t.y0 = b.y0;
    t.y = b.y;
    t.part = reinterpret_cast<float*>(reinterpret_cast<char*>(a0.ws) + ws_off[i]);
    const BlockGeom g = block_geom(b.N, b.k, b.K, b.tgt.d_in, b.tgt.d_out);
    t.kslices = kslices[i] = g.kslices;
    t.cslices = cslices[i] = g.cslices;
  }
  // targets reading the same x rows share a group (the first such target's index)
  int xg[kApplyMaxMulti];
  for (int i = 0; i < n; ++i) {
    xg[i] = i;
    for (int j = 0; j < i; ++j)
      if (as[j].x == as[i].x && as[j].tgt.d_in == as[i].tgt.d_in) {
        xg[i] = xg[j];
        break;
      }
  }
  const DenseItems it = dense_items(n, xg, kslices, cslices);
  if (!it.ok) return hipSuccess;  // more work items than the table holds: the general block kernels
  *taken = true;
  da.items_s = it.n_s;
  da.items_e = it.n_e;
  for (int i = 0; i < it.n_s; ++i) {
    da.item_s[i] = it.s[i];
    da.col_start[i] = it.col_start[i];
    da.col_len[i] = it.col_len[i];
  }
  for (int i = 0; i < it.n_e; ++i) da.item_e[i] = it.e[i];
  const int groups = (da.npairs + 7) / 8;
  const int grid_s = da.disp_wgs + 8 * groups * da.items_s, grid_e = 8 * groups * 2 * da.items_e;
  const int RBv = a0.tgt.r_pad / 16;
  hipError_t err = hipSuccess;
#define MOLORA_DENSE_RB(...)                                  \
  switch (RBv) {                                              \
    case 1: { constexpr int RB = 1; __VA_ARGS__; } break;     \
    case 2: { constexpr int RB = 2; __VA_ARGS__; } break;     \
    case 3: { constexpr int RB = 3; __VA_ARGS__; } break;     \
    case 4: { constexpr int RB = 4; __VA_ARGS__; } break;     \
    default: return hipErrorInvalidValue;                     \
  }
#define MOLORA_DENSE_BOOL(V, NAME, ...) \
  if (V) { constexpr bool NAME = true; __VA_ARGS__; } else { constexpr bool NAME = false; __VA_ARGS__; }
  const bool direct = fuse != nullptr;
  if (a0.k <= 2) {
    MOLORA_DENSE_RB(MOLORA_DENSE_BOOL(a0.indirect, IND, MOLORA_DENSE_BOOL(direct, DIR,
        err = (launch_shrink_dense_t<RB, IND, 2, DIR>(da, grid_s, s)))))
  } else {
    MOLORA_DENSE_RB(MOLORA_DENSE_BOOL(a0.indirect, IND, MOLORA_DENSE_BOOL(direct, DIR,
        err = (launch_shrink_dense_t<RB, IND, 4, DIR>(da, grid_s, s)))))
  }
  if (err != hipSuccess) return err;
  MOLORA_DENSE_RB(MOLORA_DENSE_BOOL(a0.indirect, IND, MOLORA_DENSE_BOOL(a0.y0_f32, Y0F,
      MOLORA_DENSE_BOOL(a0.y_f32, YF, err = (launch_expand_dense_t<RB, IND, Y0F, YF>(da, grid_e, s))))))
#undef MOLORA_DENSE_RB
#undef MOLORA_DENSE_BOOL
  return err;
}

}  // namespace molora
