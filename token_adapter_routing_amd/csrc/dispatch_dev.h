// Stable counting sort of routed pairs by adapter (MoLoRA pages, thelatestinai.com, Table 1
// rows "Histogram computation" and "Pointer arrays"; Figure 2 right: tokens grouped by their
// selected adapter), in one workgroup or, for many pairs, in two chip-wide launches.
//
// NT threads (NW = NT/64 waves).  Pairs are produced by a source functor src(p) -> (e, w).
//   pass 1  wave64 "match" masks (ballots over the bits of the adapter index) give each group
//           of equal adapters in a wave its size; the group's lowest lane adds it to an LDS
//           counter.  Wave 0 scans the K counters into offsets.
//   pass 2  pairs are taken in chunks of E*NT (E <= 8), pair p = chunk + j*NT + tid.  A lane's
//           rank among equal adapters of its wave is popcount(match & lanes below); group
//           sizes go to LDS as [j][wave][adapter]; NT/64 threads per adapter scan them in
//           (j, wave) order -- ascending pair id -- on top of the adapter's offset and the
//           pairs of earlier chunks, which makes the permutation stable and deterministic.
#pragma once

#include "molora_dev.h"

namespace molora {

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

template <int NT>
struct DispatchLds {
  static constexpr int NW = NT / kWave;
  int cnt[64];
  int offs[64];
  int base[64];
  int wcnt[kDispMaxE * NW * 64];
};

// Pairs c0 + j*NT + tid (j < E, below c1) from the source: adapter (outside [0, K) = unrouted)
// and gate weight; missing pairs get -1.
template <int NT, typename Src>
__device__ __forceinline__ void disp_load(Src src, int c0, int c1, int E, int (&ev)[kDispMaxE], float (&wv)[kDispMaxE]) {
#pragma unroll
  for (int j = 0; j < kDispMaxE; ++j) {
    ev[j] = -1;
    wv[j] = 0.f;
    const int p = c0 + j * NT + (int)threadIdx.x;
    if (j < E && p < c1) src(p, ev[j], wv[j]);
  }
}

// Histogram of loaded pairs into L.cnt: one LDS atomic per group of equal adapters of a wave.
template <int NT>
__device__ __forceinline__ void disp_count(DispatchLds<NT>& L, const int (&ev)[kDispMaxE], int E, int K, int nbits) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lanemask_lt(lane);
#pragma unroll
  for (int j = 0; j < kDispMaxE; ++j) {
    if (j < E) {
      const bool v = (ev[j] >= 0) && (ev[j] < K);
      const uint64_t m = match_mask(ev[j], v, nbits);
      if (v && (m & lt) == 0) atomicAdd(&L.cnt[ev[j]], __popcll(m));
    }
  }
}

// Stable scatter of the loaded pairs c0 + j*NT + tid: pair p of adapter e goes to
// L.offs[e] + L.base[e] + (its rank among the chunk's pairs of e in ascending p); L.base[e]
// then advances by the chunk's count.  Callers set L.offs and L.base.
template <int NT>
__device__ void disp_scatter(DispatchLds<NT>& L, int (&ev)[kDispMaxE], const float (&wv)[kDispMaxE], int c0, int c1,
                             int E, int K, int nbits, int32_t* __restrict__ perm, float* __restrict__ perm_w,
                             int32_t* __restrict__ inv) {
  constexpr int NW = NT / kWave;
  constexpr int TPA = NT / 64;  // threads per adapter in the scan
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint64_t lt = lanemask_lt(lane);
  for (int i = tid; i < E * NW * 64; i += NT) L.wcnt[i] = 0;
  __syncthreads();
  int rk[kDispMaxE];
#pragma unroll
  for (int j = 0; j < kDispMaxE; ++j) {
    rk[j] = 0;
    if (j < E) {
      const bool v = (ev[j] >= 0) && (ev[j] < K);
      const uint64_t m = match_mask(ev[j], v, nbits);
      if (v) {
        rk[j] = __popcll(m & lt);
        if (rk[j] == 0) L.wcnt[(j * NW + wave) * 64 + ev[j]] = __popcll(m);
      } else {
        ev[j] = -1;
      }
    }
  }
  __syncthreads();
  {
    // adapter ae's E*NW group sizes in (j, wave) order, split over TPA threads of one wave;
    // thread pi takes the entries [pi * E * NW / TPA, (pi + 1) * E * NW / TPA)
    const int ae = tid / TPA, pi = tid % TPA;
    constexpr int PER = kDispMaxE * NW / TPA;  // upper bound of entries per thread
    const int per = E * NW / TPA;
    int loc[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      loc[i] = 0;
      if (i < per) {
        loc[i] = L.wcnt[(pi * per + i) * 64 + ae];
        sum += loc[i];
      }
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < TPA; d <<= 1) {
      const int o = __shfl_up(incl, d, TPA);
      if (pi >= d) incl += o;
    }
    const int b0 = (ae < K) ? L.offs[ae] + L.base[ae] : 0;
    int run = b0 + incl - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (i < per) {
        L.wcnt[(pi * per + i) * 64 + ae] = run;
        run += loc[i];
      }
    }
    if (pi == TPA - 1 && ae < K) L.base[ae] = L.base[ae] + incl;  // same wave read base[ae] above
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kDispMaxE; ++j) {
    if (j < E) {
      const int p = c0 + j * NT + tid;
      if (ev[j] >= 0) {
        const int pos = L.wcnt[(j * NW + wave) * 64 + ev[j]] + rk[j];
        perm[pos] = p;
        perm_w[pos] = wv[j];
        if (inv != nullptr) inv[p] = pos;
      } else if (p < c1 && inv != nullptr) {
        inv[p] = -1;
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int disp_nbits(int K) {
  int nbits = 0;
  while ((1 << nbits) < K) ++nbits;
  return nbits;
}

// One workgroup sorts all P pairs: histogram, scan, scatter.  src(p) returns adapter e
// (outside [0, K) = unrouted) and gate weight w of pair p < P.
template <int NT, typename Src>
__device__ void dispatch_block(DispatchLds<NT>& L, Src src, int P, int K, int32_t* __restrict__ counts,
                               int32_t* __restrict__ offsets, int32_t* __restrict__ perm, float* __restrict__ perm_w,
                               int32_t* __restrict__ inv) {
  static_assert(NT % 64 == 0 && NT / 64 >= 1 && NT / 64 <= 16, "dispatch block size");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbits = disp_nbits(K);
  int E = (P + NT - 1) / NT;
  if (E < 1) E = 1;
  if (E > kDispMaxE) E = kDispMaxE;
  if (tid < 64) {
    L.cnt[tid] = 0;
    L.base[tid] = 0;
  }
  __syncthreads();
  // pass 1: histogram.  When all pairs fit in one chunk the values stay in registers for pass 2.
  const int chunk = E * NT;
  const bool one_chunk = P <= chunk;
  int ev[kDispMaxE];
  float wv[kDispMaxE];
  for (int c0 = 0; c0 < P; c0 += chunk) {
    disp_load<NT>(src, c0, P, E, ev, wv);
    disp_count<NT>(L, ev, E, K, nbits);
  }
  __syncthreads();
  if (wave == 0) {
    const int c = (lane < K) ? L.cnt[lane] : 0;
    const int incl = wave_incl_scan(c, lane);
    if (lane < K) {
      counts[lane] = c;
      offsets[lane + 1] = incl;
      L.offs[lane] = incl - c;
    }
    if (lane == 0) offsets[0] = 0;
  }
  __syncthreads();
  // pass 2: stable scatter
  for (int c0 = 0; c0 < P; c0 += chunk) {
    if (!one_chunk) disp_load<NT>(src, c0, P, E, ev, wv);
    disp_scatter<NT>(L, ev, wv, c0, P, E, K, nbits, perm, perm_w, inv);
  }
}

// Several workgroups (chip-wide sort, two launches).  Workgroup b owns pairs [b*C, (b+1)*C).
// Launch 1: its histogram to bcnt[b][K].
template <int NT, typename Src>
__device__ void dispatch_hist_part(DispatchLds<NT>& L, Src src, int P, int K, int C, int32_t* __restrict__ bcnt) {
  const int tid = threadIdx.x;
  const int nbits = disp_nbits(K);
  if (tid < 64) L.cnt[tid] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * C, c1 = min(P, c0 + C);
  const int E = min(kDispMaxE, (C + NT - 1) / NT);  // pairs per thread and pass (uniform)
  int ev[kDispMaxE];
  float wv[kDispMaxE];
  for (int s0 = c0; s0 < c1; s0 += E * NT) {
    disp_load<NT>(src, s0, c1, E, ev, wv);
    disp_count<NT>(L, ev, E, K, nbits);
  }
  __syncthreads();
  if (tid < K) bcnt[(size_t)blockIdx.x * K + tid] = L.cnt[tid];
}

// Launch 2: every workgroup sums the nb histograms (totals and the part before its own range),
// scans the totals into offsets (workgroup 0 writes counts and offsets) and scatters its range.
template <int NT, typename Src>
__device__ void dispatch_scatter_part(DispatchLds<NT>& L, Src src, int P, int K, int C, int nb,
                                      const int32_t* __restrict__ bcnt, int32_t* __restrict__ counts,
                                      int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                      float* __restrict__ perm_w, int32_t* __restrict__ inv) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbits = disp_nbits(K);
  const int b = blockIdx.x;
  if (tid < 64) {
    L.cnt[tid] = 0;
    L.base[tid] = 0;
  }
  __syncthreads();
  // totals and the part before this workgroup, per adapter: every count loaded by its own
  // thread and added in LDS (integer sums: the order does not matter)
  for (int i = tid; i < nb * K; i += NT) {
    const int j = i / K, e = i - j * K;
    const int c = bcnt[i];
    atomicAdd(&L.cnt[e], c);
    if (j < b) atomicAdd(&L.base[e], c);
  }
  __syncthreads();
  if (wave == 0) {
    const int c = (lane < K) ? L.cnt[lane] : 0;
    const int incl = wave_incl_scan(c, lane);
    if (lane < K) L.offs[lane] = incl - c;
    if (b == 0) {
      if (lane < K) {
        counts[lane] = c;
        offsets[lane + 1] = incl;
      }
      if (lane == 0) offsets[0] = 0;
    }
  }
  __syncthreads();
  const int c0 = b * C, c1 = min(P, c0 + C);
  const int E = min(kDispMaxE, (C + NT - 1) / NT);
  int ev[kDispMaxE];
  float wv[kDispMaxE];
  for (int s0 = c0; s0 < c1; s0 += E * NT) {
    disp_load<NT>(src, s0, c1, E, ev, wv);
    disp_scatter<NT>(L, ev, wv, s0, c1, E, K, nbits, perm, perm_w, inv);
  }
}

// One launch over several workgroups for few adapters (K <= kDispWideMaxK): workgroup b of the
// dispatch owns the pairs [b*NT, min(P, (b+1)*NT)).  Every workgroup loads all P adapters --
// thread t holds pairs s0 + j*NT + t, so its own pair is one of them -- and counts them per
// adapter with one ballot per adapter and wave load (no atomics), in total (-> offsets) and
// before its own range (-> where its pairs of each adapter start), then scatters its range
// stably.  Workgroup 0 writes counts and offsets.  Each workgroup reads every pair, so this
// suits up to a few thousand pairs.
constexpr int kDispWideMaxK = 16;
template <int NT, typename Src, int MAXK = kDispWideMaxK>  // MAXK: a bound on K known at compile time
__device__ void dispatch_wide_part(DispatchLds<NT>& L, Src src, int P, int K, int b, int32_t* __restrict__ counts,
                                   int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                   float* __restrict__ perm_w, int32_t* __restrict__ inv) {
  constexpr int NW = NT / kWave;
  static_assert(2 * NW * 64 <= kDispMaxE * NW * 64, "per-wave count table");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = b * NT, c1 = min(P, c0 + NT);
  int tot[MAXK], pre[MAXK];
#pragma unroll
  for (int e = 0; e < MAXK; ++e) tot[e] = pre[e] = 0;
  int eo = -1;  // this thread's own pair c0 + tid: adapter and gate weight
  float wo = 0.f;
  for (int s0 = 0; s0 < P; s0 += kDispMaxE * NT) {
    int ev[kDispMaxE];
#pragma unroll
    for (int j = 0; j < kDispMaxE; ++j) {
      const int p = s0 + j * NT + tid;
      float wd = 0.f;
      ev[j] = -1;
      if (p < P) src(p, ev[j], wd);
      if (s0 + j * NT == c0) {  // uniform: the load that holds this workgroup's range
        eo = ev[j];
        wo = wd;
      }
    }
#pragma unroll
    for (int j = 0; j < kDispMaxE; ++j) {
      const uint64_t before = __ballot(s0 + j * NT + tid < c0);
#pragma unroll
      for (int e = 0; e < MAXK; ++e)
        if (e < K) {
          const uint64_t m = __ballot(ev[j] == e);
          tot[e] += __popcll(m);
          pre[e] += __popcll(m & before);
        }
    }
  }
  int mt = 0, mp = 0;
#pragma unroll
  for (int e = 0; e < MAXK; ++e)
    if (lane == e) {
      mt = tot[e];
      mp = pre[e];
    }
  L.wcnt[wave * 64 + lane] = mt;
  L.wcnt[(NW + wave) * 64 + lane] = mp;
  __syncthreads();
  if (wave == 0) {
    int c = 0, pr = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      c += L.wcnt[w * 64 + lane];
      pr += L.wcnt[(NW + w) * 64 + lane];
    }
    if (lane >= K) c = pr = 0;
    const int incl = wave_incl_scan(c, lane);
    L.offs[lane] = incl - c;
    L.base[lane] = pr;
    if (b == 0) {
      if (lane < K) {
        counts[lane] = c;
        offsets[lane + 1] = incl;
      }
      if (lane == 0) offsets[0] = 0;
    }
  }
  __syncthreads();
  int ev[kDispMaxE];
  float wv[kDispMaxE];
  ev[0] = eo;
  wv[0] = wo;
  disp_scatter<NT>(L, ev, wv, c0, c1, 1, K, disp_nbits(K), perm, perm_w, inv);
}

}  // namespace molora
