// Dispatch on gfx950: per-adapter histogram, exclusive scan into offsets, and the stable
// grouping permutation (MoLoRA pages, thelatestinai.com, Table 1 rows "Histogram
// computation" and "Pointer arrays"; Figure 2 right: tokens grouped by selected adapter).
//
// One workgroup of 1024 threads (16 waves) sorts all pairs by counting:
//   pass 1  wave64 "match" masks (ballots over the bits of the adapter index) give each group
//           of equal adapters in a wave its size; the group's lowest lane adds it to an LDS
//           counter.  Wave 0 scans the K counters into offsets.
//   pass 2  pairs are taken in chunks of E*1024 (E <= 8), pair p = chunk + j*1024 + tid.  A
//           lane's rank among equal adapters of its wave is popcount(match & lanes below);
//           the groups' sizes go to LDS as [j][wave][adapter]; 16 threads per adapter scan
//           those sizes in (j, wave) order -- ascending pair id -- on top of the adapter's
//           offset and the pairs of earlier chunks, which makes the permutation stable and
//           identical on every run.
#include "molora_launch.h"

namespace molora {

constexpr int kDispThreads = 1024;
constexpr int kDispWaves = kDispThreads / kWave;
constexpr int kDispMaxE = 8;

// Lanes of the wave that hold the same adapter index as this lane (valid lanes only).
__device__ __forceinline__ uint64_t match_mask(int e, bool v, int nbits) {
  uint64_t m = __ballot(v);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = v && ((e >> b) & 1);
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__global__ __launch_bounds__(kDispThreads) void dispatch_single(const int32_t* __restrict__ idx,
                                                                const float* __restrict__ w, int P, int K,
                                                                int nbits, int E, int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ perm,
                                                                float* __restrict__ perm_w,
                                                                int32_t* __restrict__ inv) {
  __shared__ int cnt[64];
  __shared__ int offs[65];
  __shared__ int base[64];
  __shared__ int wcnt[kDispMaxE * kDispWaves * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint64_t lt = lanemask_lt(lane);
  if (tid < 64) {
    cnt[tid] = 0;
    base[tid] = 0;
  }
  __syncthreads();

  // pass 1: histogram
  for (int p0 = 0; p0 < P; p0 += kDispThreads) {
    const int p = p0 + tid;
    const int e = (p < P) ? idx[p] : -1;
    const bool v = (e >= 0) && (e < K);
    const uint64_t m = match_mask(e, v, nbits);
    if (v && (m & lt) == 0) atomicAdd(&cnt[e], __popcll(m));
  }
  __syncthreads();
  if (wave == 0) {
    const int c = (lane < K) ? cnt[lane] : 0;
    const int incl = wave_incl_scan(c, lane);
    if (lane < K) {
      counts[lane] = c;
      offsets[lane + 1] = incl;
      offs[lane] = incl - c;
    }
    if (lane == 0) offsets[0] = 0;
  }
  __syncthreads();

  // pass 2: stable scatter
  const int chunk = E * kDispThreads;
  for (int c0 = 0; c0 < P; c0 += chunk) {
    for (int i = tid; i < E * kDispWaves * 64; i += kDispThreads) wcnt[i] = 0;
    __syncthreads();
    int ev[kDispMaxE], rk[kDispMaxE];
#pragma unroll
    for (int j = 0; j < kDispMaxE; ++j) {
      ev[j] = -1;
      rk[j] = 0;
      if (j < E) {
        const int p = c0 + j * kDispThreads + tid;
        const int e = (p < P) ? idx[p] : -1;
        const bool v = (e >= 0) && (e < K);
        const uint64_t m = match_mask(e, v, nbits);
        if (v) {
          ev[j] = e;
          rk[j] = __popcll(m & lt);
          if (rk[j] == 0) wcnt[(j * kDispWaves + wave) * 64 + e] = __popcll(m);
        }
      }
    }
    __syncthreads();
    {
      // adapter ae's E*16 group sizes, in (j, wave) order, split over 16 threads of one wave
      const int ae = tid >> 4, pi = tid & 15;
      int loc[kDispMaxE];
      int sum = 0;
#pragma unroll
      for (int i = 0; i < kDispMaxE; ++i) {
        loc[i] = 0;
        if (i < E) {
          loc[i] = wcnt[(pi * E + i) * 64 + ae];
          sum += loc[i];
        }
      }
      int incl = sum;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) {
        const int o = __shfl_up(incl, d, 16);
        if (pi >= d) incl += o;
      }
      const int b0 = (ae < K) ? offs[ae] + base[ae] : 0;
      int run = b0 + incl - sum;
#pragma unroll
      for (int i = 0; i < kDispMaxE; ++i) {
        if (i < E) {
          wcnt[(pi * E + i) * 64 + ae] = run;
          run += loc[i];
        }
      }
      if (pi == 15 && ae < K) base[ae] = base[ae] + incl;  // same wave read base[ae] above
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kDispMaxE; ++j) {
      if (j < E) {
        const int p = c0 + j * kDispThreads + tid;
        if (ev[j] >= 0) {
          const int pos = wcnt[(j * kDispWaves + wave) * 64 + ev[j]] + rk[j];
          perm[pos] = p;
          perm_w[pos] = w[p];
          if (inv != nullptr) inv[p] = pos;
        } else if (p < P && inv != nullptr) {
          inv[p] = -1;
        }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_dispatch(const int32_t* idx, const float* w, int P, int K, int32_t* counts, int32_t* offsets,
                           int32_t* perm, float* perm_w, int32_t* inv, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < K) ++nbits;
  int E = (P + kDispThreads - 1) / kDispThreads;
  if (E < 1) E = 1;
  if (E > kDispMaxE) E = kDispMaxE;
  hipLaunchKernelGGL(dispatch_single, dim3(1), dim3(kDispThreads), 0, s, idx, w, P, K, nbits, E, counts,
                     offsets, perm, perm_w, inv);
  return hipGetLastError();
}

}  // namespace molora
