// 64-token blocks split over workgroups (MoLoRA pages, thelatestinai.com: per-token routing,
// Figure 2 right and Table 1; the gate-weighted sum of the selected adapters' deltas).
//
// A block of 64 consecutive tokens is handled in two launches (8 waves per workgroup):
//   shrink  (block, reduction slice of 512):  partial h = x[64 tokens, slice] * A_e[slice] for
//           every adapter e the block uses, written to a workspace.
//   expand  (block, column slice of 512):  sums the block's partials in slice order, weights
//           them (gate weight x alpha/r per token and adapter), and writes
//           y = y0 + sum_e h_e B_e[:, slice] for the 64 tokens.
// The launch boundary orders the partials' writes before their reads.  The adapter pieces of a
// slice (A: 16 KB, B: 16 KB per adapter at rank 16) are read once per workgroup, straight into
// LDS, and shared by the four row-block waves, so the per-CU load volume is dominated by the x
// and y0 streams (an 8-token tile reads every adapter's whole A and B: twice its own stream).
// Every slice of block tb runs on XCD tb mod 8 (workgroups are dispatched round robin over the
// 8 XCDs; the kernels map workgroup ids accordingly), so the expand finds the partials that the
// shrink wrote in the same L2.
//
// MFMA layouts (v_mfma_f32_16x16x32_bf16): the shrink uses the swizzled A pieces with rows =
// 16 tokens; the expand uses h as a bf16 hi/lo pair stacked along k and the slab's permuted
// B^T columns, so that lane (n, G) holds 8 contiguous output columns of tokens 4G..4G+3.
#pragma once

#include "molora_mfma.h"

namespace molora {

constexpr int kBWaves = 8;
constexpr int kBThreads = kBWaves * kWave;
constexpr int kBMaxU = 16;        // adapters per block (K <= 16)
// adapters whose pieces are staged in LDS at once (one at ranks above 32: LDS size)
template <int RB>
constexpr int block_group() {
  return RB <= 2 ? 2 : 1;
}

struct BlockArgs {
  TargetDev tgt;
  const uint16_t* x;
  const void* y0;
  void* y;
  int N, K, k;
  float scale;
  int nblocks;   // ceil(N / 64)
  int kslices;   // ceil(d_in / 512)
  int cslices;   // ceil(d_out / 512)
  int slotmax;   // partial slots per block: min(K, 64 k)
  float* part;   // [nblocks][slotmax][kslices][64][r_pad] fp32
};

template <int RB>
struct BlockLds {
  // shrink: A pieces [slot][step][chunk][u][64 lanes x 16 B]; expand: B^T rows [slot][512][r_pad]
  alignas(16) uint16_t ab[block_group<RB>()][kBSlice * RB * 16];
  float red[2][4][16][RB * 16 + 4];          // shrink: the two reduction halves of each row block
  alignas(16) uint16_t hb[block_group<RB>()][2][kBTok][RB * 16];  // expand: h hi / lo [slot][part][token][rank]
  float wt[kBMaxU][kBTok];                    // expand: weight of (slot, token)
};

// Adapter of the pair (token t, slot s) and its weight x alpha/r, for the tokens of a block;
// tokens past N - 1 are clones of token N - 1 (same routing, so identical results).
// Every wave calls block_used with all lanes active.
template <typename Route>
__device__ __forceinline__ uint32_t block_used(const Route& rt, int t0, int N, int k, int K) {
  const int lane = threadIdx.x & 63;
  uint32_t used = 0;
  for (int j = 0; j < k; ++j) {
    const int pl = lane + kWave * j;
    const int tc = min(t0 + pl / k, N - 1);
    float w;
    const int e = rt(tc, pl % k, w);
#pragma unroll
    for (int ee = 0; ee < kBMaxU; ++ee)
      if (ee < K && __ballot(e == ee) != 0) used |= 1u << ee;
  }
  return used;
}

// Slot of adapter e among the used adapters (ascending).
__device__ __forceinline__ int slot_of(uint32_t used, int e) { return __popc(used & ((1u << e) - 1u)); }

// Copy `bytes` (a multiple of 1 KB) from global src to LDS dst, split over the workgroup's waves:
// each wave instruction moves 1 KB, lane l's 16 bytes landing at dst + 16 l.
__device__ __forceinline__ void lds_copy_1k(void* dst, const void* src, int bytes) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int off = wave * 1024; off < bytes; off += kBWaves * 1024)
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + off + 16 * lane,
                                     reinterpret_cast<char*>(dst) + off, 16, 0, 0);
}

// Copy `bytes` (a multiple of 1 KB, at most 2 RB KB per wave) from global src to LDS dst through
// registers: wave w's 1 KB pieces w, w + 8, ..; the loads are unconditional (clamped), the
// stores only for pieces inside `bytes`.
template <int RB>
__device__ __forceinline__ void lds_stage_regs(void* dst, const void* src, int bytes) {
  constexpr int C = (kBSlice * RB * 16 * 2) / (kBWaves * 1024);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  u32x4_t v[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int off = min((wave + kBWaves * c) * 1024, bytes - 1024);
    v[c] = ld16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(src) + off) + 8 * lane);
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int off = (wave + kBWaves * c) * 1024;
    if (off < bytes) *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(dst) + off + 16 * lane) = v[c];
  }
}

// ------------------------------------------------------------------------------------------
// shrink workgroup: block tb, reduction slice sl.  Wave w: row block rb = w % 4 (16 tokens),
// reduction half kh = w / 4 (two steps of 128).
template <int RB, bool INDIRECT, typename Route>
__device__ void block_shrink(const BlockArgs& a, BlockLds<RB>& L, const Route& rt, int tb, int sl) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int rb = wave & 3, kh = wave >> 2;
  const int t0 = tb * kBTok;
  const int d_in = a.tgt.d_in, r_pad = a.tgt.r_pad;
  const int S = d_in / kStepK;
  const int s0 = sl * (kBSlice / kStepK), s1 = min(s0 + kBSlice / kStepK, S);  // the slice's steps
  const int ns = s1 - s0;
  const int w0 = min(s0 + 2 * kh, s1), w1 = min(w0 + 2, s1);                       // this wave's steps
  // x rows of the wave's 16 tokens, its (up to) two steps: issued first
  const int row = min(t0 + 16 * rb + n, a.N - 1);
  const uint16_t* xp = a.x + (size_t)row * d_in + 8 * G;
  u32x4_t xv[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int s = max(min(w0 + i, w1 - 1), 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[i][c] = ld16_nt(xp + s * kStepK + 32 * c);
  }
  const uint32_t used = block_used(rt, t0, a.N, a.k, a.K);
  const int nU = __popc(used);
  const size_t piece = (size_t)RB * 16 * kStepK;  // elements of one step's pieces (4 chunks x RB)
  uint32_t rem = used;
  for (int base = 0; base < nU; base += block_group<RB>()) {
    const int ng = min(block_group<RB>(), nU - base);
    // stage the group's A pieces of the slice: [g][step][chunk][u][1 KB]
    uint32_t r2 = rem;
    for (int g = 0; g < ng; ++g) {
      const uint16_t* Ap = adapter_A<INDIRECT>(a.tgt, __builtin_ctz(r2)) + (size_t)s0 * piece;
      r2 &= r2 - 1;
      lds_copy_1k(L.ab[g], Ap, ns * (int)piece * 2);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int g = 0; g < ng; ++g) {
      f32x4_t acc[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (w0 + i < w1) {
          const uint16_t* ap = L.ab[g] + (size_t)(w0 + i - s0) * piece;
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
      // the two reduction halves of a row block meet in LDS; 512 threads store the sums
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) L.red[kh][rb][4 * G + i][u * 16 + n] = acc[u][i];
      __syncthreads();
      const int slot = base + g;
      float* dst = a.part + block_part_index(tb, slot, sl, a.slotmax, a.kslices, r_pad);
      for (int v = threadIdx.x; v < kBTok * RB * 16; v += kBThreads) {
        const int tok = v / (RB * 16), rk = v % (RB * 16);
        const int rbv = tok >> 4, rw = tok & 15;
        dst[(size_t)tok * r_pad + rk] = L.red[0][rbv][rw][rk] + L.red[1][rbv][rw][rk];
      }
      __syncthreads();
    }
    for (int g = 0; g < ng; ++g) rem &= rem - 1;
  }
}

// ------------------------------------------------------------------------------------------
// expand workgroup: block tb, column slice cs.  Wave w: row block rb = w % 4, column half
// ch = w / 4 (two blocks of 128 columns).  `hook` runs while the y0 rows and B pieces are in
// flight (the step kernel counts its dispatch there).
template <int RB, bool INDIRECT, bool Y0F32, bool YF32, typename Route, typename Hook>
__device__ void block_expand(const BlockArgs& a, BlockLds<RB>& L, const Route& rt, int tb, int cs, Hook hook) {
  constexpr size_t y0b = Y0F32 ? 4 : 2, yb = YF32 ? 4 : 2;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int rb = wave & 3, ch = wave >> 2;
  const int t0 = tb * kBTok;
  const int d_out = a.tgt.d_out, r_pad = a.tgt.r_pad;
  const int c0 = cs * kBSlice, c1 = min(c0 + kBSlice, d_out);
  const int nb = (c1 - c0) / kColBlock;                      // 128-column blocks in the slice
  const int b0 = min(2 * ch, nb - 1), b1 = min(2 * ch + 1, nb - 1);
  const bool has0 = 2 * ch < nb, has1 = 2 * ch + 1 < nb;
  // y0 rows of the wave's tokens 4G..4G+3 of its row block (clones past N - 1), both blocks
  const char* y0rows[4];
  char* yrows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = min(t0 + 16 * rb + 4 * G + i, a.N - 1);
    y0rows[i] = reinterpret_cast<const char*>(a.y0) + (size_t)t * d_out * y0b;
    yrows[i] = reinterpret_cast<char*>(a.y) + (size_t)t * d_out * yb;
  }
  // the y0 rows first: they do not depend on the routing and are the HBM stream of this launch
  // (everything requested after them returns after them, and is needed before them only by
  // work that is short next to their latency)
  RowChunk<Y0F32> yc0, yc1;
  load_row_chunk<Y0F32>(yc0, y0rows, c0 + b0 * kColBlock, n);
  load_row_chunk<Y0F32>(yc1, y0rows, c0 + b1 * kColBlock, n);
  __builtin_amdgcn_sched_barrier(0);
  // routing: used adapters and the (slot, token) weights; token thread t sums its pairs in order
  const uint32_t used = block_used(rt, t0, a.N, a.k, a.K);
  const int nU = __popc(used);
  if (threadIdx.x < kBTok) {
    const int tc = min(t0 + (int)threadIdx.x, a.N - 1);
    for (int j = 0; j < nU; ++j) L.wt[j][threadIdx.x] = 0.f;
    for (int s = 0; s < a.k; ++s) {
      float w;
      const int e = rt(tc, s, w);
      if (e >= 0) L.wt[slot_of(used, e)][threadIdx.x] += w;
    }
  }
  constexpr int BG = block_group<RB>();
  const int bbytes = (c1 - c0) * r_pad * 2;  // B^T rows of the slice, one adapter
  // a group's B^T rows into LDS through registers (the waits then name exactly these loads)
  auto stage_b = [&](uint32_t r2, int ng) {
    for (int g = 0; g < ng; ++g) {
      lds_stage_regs<RB>(L.ab[g], adapter_B<INDIRECT>(a.tgt, __builtin_ctz(r2)) + (size_t)c0 * r_pad, bbytes);
      r2 &= r2 - 1;
    }
  };
  // h of a group's slots: sum the slices in order, weight, split into hi / lo.  A thread takes
  // 4 consecutive ranks (16 bytes) of one (slot, token) and requests all its slices at once.
  auto group_h = [&](int base, int ng) {
    constexpr int KS = 8;  // slices requested together
    for (int v = threadIdx.x; v < ng * kBTok * RB * 4; v += kBThreads) {
      const int g = v / (kBTok * RB * 4), vi = v % (kBTok * RB * 4);
      const int tok = vi / (RB * 4), rk = 4 * (vi % (RB * 4));
      const float* src = a.part + block_part_index(tb, base + g, 0, a.slotmax, a.kslices, r_pad) + (size_t)tok * r_pad + rk;
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < a.kslices; s0 += KS) {
        u32x4_t pv[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
          if (s0 + s < a.kslices) pv[s] = ld16(src + (size_t)(s0 + s) * kBTok * r_pad);
#pragma unroll
        for (int s = 0; s < KS; ++s)
          if (s0 + s < a.kslices)
#pragma unroll
            for (int c = 0; c < 4; ++c) sum[c] += __uint_as_float(pv[s][c]);
      }
      const float wgt = L.wt[base + g][tok];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float h = sum[c] * wgt;
        const __bf16 hi = (__bf16)h;
        const __bf16 lo = (__bf16)(h - (float)hi);
        L.hb[g][0][tok][rk + c] = __builtin_bit_cast(uint16_t, hi);
        L.hb[g][1][tok][rk + c] = __builtin_bit_cast(uint16_t, lo);
      }
    }
  };
  f32x4_t o0[8], o1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    o0[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    o1[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  auto group_mfma = [&](int ng) {
    for (int g = 0; g < ng; ++g) {
      // A operand: row n of the row block; groups 0, 1 carry hi of ranks 16u + 8(G & 1) ..,
      // groups 2, 3 lo of the same ranks
      bf16x8_t hb[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u)
        hb[u] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&L.hb[g][G >> 1][16 * rb + n][u * 16 + 8 * (G & 1)]));
      const uint16_t* bl = L.ab[g];
      // B pieces straight from LDS into the MFMAs (the same pieces serve the 4 row blocks)
      const uint16_t* bp0 = bl + (size_t)(b0 * kColBlock + n) * r_pad + 8 * (G & 1);
      const uint16_t* bp1 = bl + (size_t)(b1 * kColBlock + n) * r_pad + 8 * (G & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < RB; ++u) {
          const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(bp0 + (size_t)16 * j * r_pad + 16 * u);
          const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(bp1 + (size_t)16 * j * r_pad + 16 * u);
          o0[j] = mfma16x16x32(hb[u], as_bf16x8(v0), o0[j]);
          o1[j] = mfma16x16x32(hb[u], as_bf16x8(v1), o1[j]);
        }
    }
  };
  // first group: B rows and h (requested behind the y0 rows)
  const int ng0 = min(BG, nU);
  stage_b(used, ng0);
  hook();
  __syncthreads();  // the weight table is complete
  group_h(0, ng0);
  __syncthreads();  // B rows and h of the group are in LDS
  group_mfma(ng0);
  uint32_t rem = used;
  for (int g = 0; g < ng0; ++g) rem &= rem - 1;
  for (int base = BG; base < nU; base += BG) {
    const int ng = min(BG, nU - base);
    __syncthreads();  // LDS pieces free for the next group
    stage_b(rem, ng);
    group_h(base, ng);
    __syncthreads();
    group_mfma(ng);
    for (int g = 0; g < ng; ++g) rem &= rem - 1;
  }
  if (has0) epilogue_store<Y0F32, YF32>(o0, yc0, yrows, c0 + b0 * kColBlock, n, 0xFu);
  if (has1) epilogue_store<Y0F32, YF32>(o1, yc1, yrows, c0 + b1 * kColBlock, n, 0xFu);
}

}  // namespace molora
