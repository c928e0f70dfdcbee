// Dispatch on gfx950: per-adapter histogram, exclusive scan into offsets, and the stable
// grouping permutation of the routed pairs (MoLoRA pages, thelatestinai.com, Table 1 rows
// "Histogram computation" and "Pointer arrays"; Figure 2 right).  1024-thread workgroups run
// the counting sort of dispatch_dev.h over the pairs' (idx, w): one workgroup for few pairs,
// one launch of a workgroup per 1024 pairs for 4097..8192 pairs over at most 16 adapters
// (each counts all pairs and scatters its own), two launches above that.
#include "dispatch_dev.h"
#include "molora_launch.h"

namespace molora {

constexpr int kDispThreads = 1024;
// Up to kDispMaxE * kDispThreads (= kDispChunk) pairs: above kDispWideMin pairs (few adapters)
// one launch of a workgroup per kDispThreads pairs, below that one workgroup.
constexpr int kDispWideMin = 4096;  // the one-workgroup sort costs about 2.3 us + 1.45 ns per pair
static_assert(kDispMaxE * kDispThreads == kDispChunk, "one load per thread and chunk covers a dispatch chunk");

struct ArraySource {
  const int32_t* idx;
  const float* w;
  __device__ __forceinline__ void operator()(int p, int& e, float& wv) const {
    e = idx[p];
    wv = w[p];
  }
};

__global__ __launch_bounds__(kDispThreads) void dispatch_single(const int32_t* __restrict__ idx,
                                                                const float* __restrict__ w, int P, int K,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ perm, float* __restrict__ perm_w,
                                                                int32_t* __restrict__ inv) {
  __shared__ DispatchLds<kDispThreads> L;
  dispatch_block<kDispThreads>(L, ArraySource{idx, w}, P, K, counts, offsets, perm, perm_w, inv);
}

__global__ __launch_bounds__(kDispThreads) void dispatch_hist(const int32_t* __restrict__ idx,
                                                              const float* __restrict__ w, int P, int K, int C,
                                                              int32_t* __restrict__ bcnt) {
  __shared__ DispatchLds<kDispThreads> L;
  dispatch_hist_part<kDispThreads>(L, ArraySource{idx, w}, P, K, C, bcnt);
}

__global__ __launch_bounds__(kDispThreads) void dispatch_scatter(const int32_t* __restrict__ idx,
                                                                 const float* __restrict__ w, int P, int K, int C,
                                                                 int nb, const int32_t* __restrict__ bcnt,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ perm,
                                                                 float* __restrict__ perm_w, int32_t* __restrict__ inv) {
  __shared__ DispatchLds<kDispThreads> L;
  dispatch_scatter_part<kDispThreads>(L, ArraySource{idx, w}, P, K, C, nb, bcnt, counts, offsets, perm, perm_w, inv);
}

__global__ __launch_bounds__(kDispThreads) void dispatch_wide(const int32_t* __restrict__ idx,
                                                              const float* __restrict__ w, int P, int K,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm, float* __restrict__ perm_w,
                                                              int32_t* __restrict__ inv) {
  __shared__ DispatchLds<kDispThreads> L;
  dispatch_wide_part<kDispThreads>(L, ArraySource{idx, w}, P, K, blockIdx.x, counts, offsets, perm, perm_w, inv);
}

hipError_t launch_dispatch(const int32_t* idx, const float* w, int P, int K, int32_t* counts, int32_t* offsets,
                           int32_t* perm, float* perm_w, int32_t* inv, void* ws, hipStream_t s) {
  const DispatchSplit d = dispatch_split(P);
  if (d.nb > 1 && ws != nullptr) {
    int32_t* bcnt = reinterpret_cast<int32_t*>(ws);
    hipLaunchKernelGGL(dispatch_hist, dim3(d.nb), dim3(kDispThreads), 0, s, idx, w, P, K, d.C, bcnt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dispatch_scatter, dim3(d.nb), dim3(kDispThreads), 0, s, idx, w, P, K, d.C, d.nb, bcnt, counts,
                       offsets, perm, perm_w, inv);
    return hipGetLastError();
  }
  if (P > kDispWideMin && P <= kDispMaxE * kDispThreads && K <= kDispWideMaxK) {
    // a workgroup per kDispThreads pairs, each counting all of them
    const int nb = (P + kDispThreads - 1) / kDispThreads;
    hipLaunchKernelGGL(dispatch_wide, dim3(nb), dim3(kDispThreads), 0, s, idx, w, P, K, counts,
                       offsets, perm, perm_w, inv);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_single, dim3(1), dim3(kDispThreads), 0, s, idx, w, P, K, counts, offsets, perm, perm_w,
                     inv);
  return hipGetLastError();
}

}  // namespace molora
