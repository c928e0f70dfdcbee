// Routing decisions on gfx950 (MoLoRA pages, thelatestinai.com, Table 1 "Routing decision":
// the vocabulary range function R_vocab(v), cost O(1), or TopK over a learned gate
// g_theta(x), cost O(64d + 64K); Figure 2: the k selected adapters are combined by a
// weighted sum, here the softmax over the selected logits).
//
//   route_vocab_k   one thread per token: binary search of the id in the K+1 range bounds (LDS).
//   route_topk_k    router mode, a workgroup owns 16 tokens: the first layer x W1^T (d -> 64)
//                   is an MFMA product with the same gather/shrink core as the LoRA shrink,
//                   8 waves splitting d (every workgroup reads all of W1) and meeting in LDS;
//                   bias and ReLU follow in LDS.  With a workspace the first layer runs as a
//                   launch of its own over 128-token x d/8 workgroups (router_l1_chunk_k, W1
//                   read once per 128 tokens) and route_topk_k sums its chunks -- the same
//                   arithmetic in the same order, so the same bits;
//                   the second layer (64 -> K) runs on the VALU with one lane per adapter.
//                   Selection: one wave per token holds the K logits in its lanes; k rounds of
//                   (wave max, ballot of lanes equal to it, lowest lane wins) pick the top-k
//                   with ties to the lower adapter index; one more round gives the (k+1)-th
//                   value for the near-tie flag, whose margin is taken in fp64.
//   topk_logits_k   given logits: the same selection for 64 / SEG tokens per wave at once, one
//                   per SEG-lane segment (SEG = 16, 32 or 64 >= K).
#include <cmath>

#include "molora_launch.h"
#include "molora_mfma.h"

namespace molora {

// Copy the K+1 bounds from kernel arguments into LDS (static indices only).
__device__ __forceinline__ void bounds_to_lds(const VocabBounds& vb, int* lds, int K) {
#pragma unroll
  for (int i = 0; i < 65; ++i)
    if ((int)threadIdx.x == i && i <= K) lds[i] = vb.b[i];
}

__global__ __launch_bounds__(256) void route_vocab_k(const int32_t* __restrict__ ids, int N, VocabBounds b,
                                                     int K, int32_t* __restrict__ idx, float* __restrict__ w) {
  __shared__ int bl[65];
  bounds_to_lds(b, bl, K);
  __syncthreads();
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const int e = vocab_owner(ids[i], bl, K);
  idx[i] = e;
  w[i] = (e >= 0) ? 1.0f : 0.0f;
}

hipError_t launch_route_vocab(const int32_t* ids, int N, const VocabBounds& bounds, int K, int32_t* idx,
                              float* w, hipStream_t s) {
  hipLaunchKernelGGL(route_vocab_k, dim3((N + 255) / 256), dim3(256), 0, s, ids, N, bounds, K, idx, w);
  return hipGetLastError();
}

// Top-k of one token whose logit for adapter `lane` is `l` (lanes >= K hold nothing).
__device__ __forceinline__ void topk_one_token(float l, int K, int k, int lane, int32_t* __restrict__ idx_row,
                                               float* __restrict__ w_row, uint8_t* flag) {
  const bool mine = lane < K;
  uint64_t taken = 0;
  float vmax = 0.f, kth = 0.f;
  for (int s = 0; s < k; ++s) {
    const bool avail = mine && !((taken >> lane) & 1ull);
    const float m = wave_max(avail ? l : -INFINITY);
    uint64_t bm = __ballot(avail && l == m);
    if (bm == 0) bm = __ballot(avail);  // only reachable with non-finite logits
    taken |= 1ull << __builtin_ctzll(bm);
    if (s == 0) vmax = m;
    kth = m;
  }
  bool near_tie = false;
  if (k < K) {
    const bool avail = mine && !((taken >> lane) & 1ull);
    const float m2 = wave_max(avail ? l : -INFINITY);
    near_tie = ((double)kth - (double)m2) < 1e-4;
  }
  const bool sel = (taken >> lane) & 1ull;
  const float ex = sel ? expf(l - vmax) : 0.f;
  const float sum = wave_sum(ex);
  if (sel) {
    const int slot = __popcll(taken & lanemask_lt(lane));
    idx_row[slot] = lane;
    w_row[slot] = ex / sum;
  }
  if (flag != nullptr && lane == 0) *flag = near_tie ? 1 : 0;
}

struct TopkArgs {
  const uint16_t* x;
  int N, d;
  const uint16_t* W1;  // [64][d]
  const float* b1;
  const uint16_t* W2;  // [K][64]
  const float* b2;
  float* logits;
  int K, k;
  int32_t* idx;
  float* w;
  uint8_t* flags;
  const float* part;  // first layer split over d: [kRouterChunks][N][64] fp32, or NULL
};

// First router layer x W1^T (+ b1) of tokens [t0, t0 + 16) into out[16][64] (LDS): 8 waves
// split d (the same MFMA shrink core as the LoRA shrink) and meet in LDS.  relu: apply the
// ReLU.  Ends with a barrier; `red` holds RedLds<4, 8>::kFloats floats.
__device__ __forceinline__ void router_layer1(const uint16_t* x, int N, int d, const uint16_t* W1, const float* b1,
                                              int t0, float* red, float* out, bool relu) {
  constexpr int NW = 8, RB = 4;
  constexpr int RS = RedLds<RB, NW>::RS;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok = min(t0 + (lane & 15), N - 1);
  // b1 of the hidden unit this thread finishes below (threadIdx.x mod 64), requested first
  const float b1v = b1 != nullptr ? b1[threadIdx.x & 63] : 0.f;
  f32x4_t acc[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int S = d / kStepK;
  shrink_steps_batched<RB, false>(acc, x + (size_t)tok * d, W1, d, (S * wave) / NW, (S * (wave + 1)) / NW, lane);
  shrink_to_lds<RB, NW>(acc, red, wave, lane);
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 64; i += NW * 64) {
    const int row = i >> 6, j = i & 63;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[(w * 16 + row) * RS + j];
    if (b1 != nullptr) v += b1v;
    out[i] = relu ? (v > 0.f ? v : 0.f) : v;
  }
  __syncthreads();
}

// The first layer split over d, for a workspace: chunk c of the reduction steps is exactly
// the range router_layer1's wave c takes, [S c / 8, S (c + 1) / 8) of S = d / 128 steps, and a
// workgroup takes 128 tokens (one 16-token row block per wave) of one chunk.  The chunk's W1
// pieces go straight into LDS once for the 128 tokens (instead of every 16-token workgroup
// reading all of W1), each wave runs the same MFMA chain as router_layer1's wave c on its
// rows, and part[c][t][64] holds the chunk's sum.  Summing the 8 chunks in order, then b1,
// repeats router_layer1's LDS reduction: the two give the same bits.  Workgroup b takes chunk
// b mod 8, so every XCD keeps one chunk of W1 in its L2.
constexpr int kRouterChunkTok = 128;

__global__ __launch_bounds__(512) void router_l1_chunk_k(const uint16_t* __restrict__ x, int N, int d,
                                                         const uint16_t* __restrict__ W1, float* __restrict__ part) {
  extern __shared__ __align__(16) uint16_t Wl[];  // [step][c][u] pieces of 64 lanes x 16 bytes
  const int ch = blockIdx.x % kRouterChunks, tt = blockIdx.x / kRouterChunks;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int S = d / kStepK;
  const int s0 = (S * ch) / kRouterChunks, s1 = (S * (ch + 1)) / kRouterChunks, ns = s1 - s0;
  // W1 piece p = (step, c, u): lane (n, G) brings its own operand (hidden unit 16u + n,
  // reduction index 128 step + 32c + 8G ..) to offset 16 lane of the piece
  for (int p = wave; p < ns * 16; p += 8) {
    const int si = p >> 4, c = (p >> 2) & 3, u = p & 3;
    __builtin_amdgcn_global_load_lds(W1 + (size_t)(u * 16 + n) * d + (size_t)(s0 + si) * kStepK + c * 32 + 8 * G,
                                     Wl + (size_t)p * 512, 16, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int t0 = tt * kRouterChunkTok + 16 * wave;
  const uint16_t* xp = x + (size_t)min(t0 + n, N - 1) * d + 8 * G;
  f32x4_t acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int SB = 2;  // steps per x batch
  for (int sb = 0; sb < max(ns, 1); sb += SB) {
    u32x4_t xv[SB][4];
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int st = s0 + min(sb + i, max(ns - 1, 0));
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[i][c] = ld16(xp + (size_t)st * kStepK + 32 * c);
    }
    if (sb == 0) {
      // this wave's W1 pieces have landed (only the x rows are younger); then everyone's
      __builtin_amdgcn_s_waitcnt((SB * 4 & 15) | (((SB * 4) >> 4) << 14) | (7 << 4) | (15 << 8));
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if (sb + i < ns) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(Wl + (size_t)(((sb + i) * 4 + c) * 4 + u) * 512 + 8 * lane);
            acc[u] = mfma16x16x32(as_bf16x8(xv[i][c]), as_bf16x8(wv), acc[u]);
          }
      }
    }
  }
  float* dst = part + ((size_t)ch * N) * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * G + i;
    if (t < N) {
#pragma unroll
      for (int u = 0; u < 4; ++u) dst[(size_t)t * 64 + u * 16 + n] = acc[u][i];
    }
  }
}

// Hidden layer of tokens [t0, t0 + 16) from the chunk sums: sum in chunk order, b1, ReLU (the
// arithmetic of router_layer1's reduction).  Ends with a barrier.
__device__ __forceinline__ void router_from_chunks(const float* __restrict__ part, int N, const float* b1, int t0,
                                                   float* out) {
  for (int i = threadIdx.x; i < 16 * 64; i += blockDim.x) {
    const int row = i >> 6, j = i & 63;
    const float* src = part + (size_t)min(t0 + row, N - 1) * 64 + j;
    float pv[kRouterChunks];
#pragma unroll
    for (int c = 0; c < kRouterChunks; ++c) pv[c] = src[(size_t)c * N * 64];
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < kRouterChunks; ++c) v += pv[c];
    if (b1 != nullptr) v += b1[j];
    out[i] = v > 0.f ? v : 0.f;
  }
  __syncthreads();
}

// Router mode: 8 waves (splitting d in the first layer), 16 tokens per workgroup.
// PART: the router's first layer comes from the chunk sums of router_l1_chunk_k.
template <bool PART>
__global__ __launch_bounds__(512) void route_topk_k(TopkArgs a) {
  constexpr int NW = 8;
  __shared__ float red[!PART ? RedLds<4, 8>::kFloats : 1];
  __shared__ float hid[16 * 64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * 16;
  // lane e < K's row of W2 (64 bf16) and b2[e], requested before the first layer so that the
  // second layer does not wait on them
  u32x4_t w2r[8];
  float b2v = 0.f;
  {
    const uint16_t* w2 = a.W2 + (size_t)min(lane, a.K - 1) * 64;
#pragma unroll
    for (int q = 0; q < 8; ++q) w2r[q] = ld16(w2 + 8 * q);
    if (a.b2 != nullptr) b2v = a.b2[min(lane, a.K - 1)];
    if constexpr (PART) router_from_chunks(a.part, a.N, a.b1, t0, hid);
    else router_layer1(a.x, a.N, a.d, a.W1, a.b1, t0, red, hid, true);
  }
  constexpr int RPW = 16 / NW;  // tokens per wave in the selection
  for (int r = 0; r < RPW; ++r) {
    const int row = wave * RPW + r;
    const int tok = t0 + row;
    if (tok >= a.N) break;  // uniform per wave
    float l = -INFINITY;
    if (lane < a.K) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        const uint32_t pair = w2r[j >> 3][(j >> 1) & 3];
        s = fmaf(hid[row * 64 + j], bf16_to_f32((j & 1) ? (pair >> 16) : (pair & 0xffffu)), s);
      }
      if (a.b2 != nullptr) s += b2v;
      l = s;
      a.logits[(size_t)tok * a.K + lane] = l;
    }
    topk_one_token(l, a.K, a.k, lane, a.idx + (size_t)tok * a.k, a.w + (size_t)tok * a.k,
                   a.flags ? a.flags + tok : nullptr);
  }
}

// Given logits: a wave holds 64 / SEG tokens, one per SEG-lane segment (SEG >= K, lane e of a
// segment = adapter e), and runs the selection of topk_one_token on all of them at once with
// reductions over the segment (butterflies of SEG lanes).  For K <= SEG the lanes past K hold
// -inf and 0, so every max and sum takes the same operands in the same order as the 64-lane
// version: the same bits.
template <int SEG>
__global__ __launch_bounds__(256) void topk_logits_k(const float* __restrict__ logits, int N, int K, int k,
                                                     int32_t* __restrict__ idx, float* __restrict__ w,
                                                     uint8_t* __restrict__ flags) {
  constexpr int TPW = kWave / SEG;  // tokens per wave
  const int lane = threadIdx.x & 63, seg = lane / SEG, e = lane % SEG;
  const int tok = (blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * TPW + seg;
  const bool mine = e < K && tok < N;
  const float l = mine ? logits[(size_t)tok * K + e] : -INFINITY;
  const uint64_t segbits = SEG == kWave ? ~0ull : (((1ull << SEG) - 1) << (seg * SEG));
  auto seg_max = [&](float v) {
#pragma unroll
    for (int d = SEG / 2; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
    return v;
  };
  auto seg_sum = [&](float v) {
#pragma unroll
    for (int d = SEG / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
  };
  uint64_t taken = 0;  // this segment's selected lanes
  float vmax = 0.f, kth = 0.f;
  for (int s = 0; s < k; ++s) {
    const bool avail = mine && !((taken >> lane) & 1ull);
    const float m = seg_max(avail ? l : -INFINITY);
    uint64_t bm = __ballot(avail && l == m) & segbits;
    if (bm == 0) bm = __ballot(avail) & segbits;  // only reachable with non-finite logits
    if (bm != 0) taken |= 1ull << __builtin_ctzll(bm);
    if (s == 0) vmax = m;
    kth = m;
  }
  bool near_tie = false;
  if (k < K) {
    const bool avail = mine && !((taken >> lane) & 1ull);
    const float m2 = seg_max(avail ? l : -INFINITY);
    near_tie = ((double)kth - (double)m2) < 1e-4;
  }
  const bool sel = (taken >> lane) & 1ull;
  const float ex = sel ? expf(l - vmax) : 0.f;
  const float sum = seg_sum(ex);
  if (sel) {
    const int slot = __popcll(taken & lanemask_lt(lane));  // ascending adapter order
    idx[(size_t)tok * k + slot] = e;
    w[(size_t)tok * k + slot] = ex / sum;
  }
  if (flags != nullptr && e == 0 && tok < N) flags[tok] = near_tie ? 1 : 0;
}

hipError_t launch_route_topk(const uint16_t* x, int N, int d, const uint16_t* W1, const float* b1,
                             const uint16_t* W2, const float* b2, float* logits, int K, int k, int32_t* idx,
                             float* w, uint8_t* flags, float* part, hipStream_t s) {
  TopkArgs a{x, N, d, W1, b1, W2, b2, logits, K, k, idx, w, flags, part};
  const dim3 grid((N + 15) / 16);
  if (W1 != nullptr && part != nullptr && router_chunked(d)) {
    const int tiles = (N + kRouterChunkTok - 1) / kRouterChunkTok;
    const int ns_max = (d / kStepK + kRouterChunks - 1) / kRouterChunks;
    hipLaunchKernelGGL(router_l1_chunk_k, dim3(tiles * kRouterChunks), dim3(512), (size_t)ns_max * 16 * 1024, s, x, N,
                       d, W1, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((route_topk_k<true>), grid, dim3(512), 0, s, a);
  } else if (W1 != nullptr) {
    hipLaunchKernelGGL((route_topk_k<false>), grid, dim3(512), 0, s, a);
  } else {
    // given logits: 4 waves of 64 / SEG tokens per workgroup
    const int seg = K <= 16 ? 16 : K <= 32 ? 32 : 64, per_wg = 4 * (kWave / seg);
    const dim3 g2((N + per_wg - 1) / per_wg);
    if (seg == 16) hipLaunchKernelGGL((topk_logits_k<16>), g2, dim3(256), 0, s, logits, N, K, k, idx, w, flags);
    else if (seg == 32) hipLaunchKernelGGL((topk_logits_k<32>), g2, dim3(256), 0, s, logits, N, K, k, idx, w, flags);
    else hipLaunchKernelGGL((topk_logits_k<64>), g2, dim3(256), 0, s, logits, N, K, k, idx, w, flags);
  }
  return hipGetLastError();
}

// Pre-activation x W1^T + b1 of every token, fp32 [N][64] (the router's backward).
__global__ __launch_bounds__(512) void router_pre_k(const uint16_t* __restrict__ x, int N, int d,
                                                    const uint16_t* __restrict__ W1, const float* __restrict__ b1,
                                                    float* __restrict__ pre) {
  __shared__ float red[RedLds<4, 8>::kFloats];
  __shared__ float out[16 * 64];
  const int t0 = blockIdx.x * 16;
  router_layer1(x, N, d, W1, b1, t0, red, out, false);
  for (int i = threadIdx.x; i < 16 * 64; i += 512)
    if (t0 + (i >> 6) < N) pre[(size_t)t0 * 64 + i] = out[i];
}

hipError_t launch_router_pre(const uint16_t* x, int N, int d, const uint16_t* W1, const float* b1, float* pre,
                             hipStream_t s) {
  hipLaunchKernelGGL(router_pre_k, dim3((N + 15) / 16), dim3(512), 0, s, x, N, d, W1, b1, pre);
  return hipGetLastError();
}

}  // namespace molora
