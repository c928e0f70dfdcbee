// Elementwise and row kernels of the synthetic decoder with per-token LoRA (MoLoRA pages,
// thelatestinai.com, Table 7: an end-to-end transformer with per-token routing; Table 8: the
// interleaved two-modality batch).  bf16 tensors, fp32 arithmetic.
//
//   xf_rmsnorm_k          a workgroup per token row: y = x / sqrt(mean(x^2) + eps) * w.
//   xf_softmax_causal_k   a wave per score row i of one (sequence, head): softmax over
//                         columns 0..i (the row's own and earlier tokens), zeros after.
//   xf_swiglu_k           g = silu(g) * up, 8 elements per thread.
//   xf_add_k              y = a + b (the residual stream), 8 elements per thread.
#include <cmath>

#include "molora_launch.h"
#include "molora_dev.h"

namespace molora {

__global__ __launch_bounds__(256) void xf_rmsnorm_k(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                    uint16_t* __restrict__ y, int d, float eps) {
  __shared__ float part[4];
  const uint16_t* xr = x + (size_t)blockIdx.x * d;
  uint16_t* yr = y + (size_t)blockIdx.x * d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ss = 0.f;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    const u32x4_t v = ld16(xr + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_to_f32(v[i] & 0xffffu), b = bf16_to_f32(v[i] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  const float inv = rsqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)d + eps);
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    const u32x4_t v = ld16(xr + c), wv = ld16(w + c);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(bf16_to_f32(v[i] & 0xffffu) * inv * bf16_to_f32(wv[i] & 0xffffu),
                         bf16_to_f32(v[i] >> 16) * inv * bf16_to_f32(wv[i] >> 16));
    st16(yr + c, o);
  }
}

__global__ __launch_bounds__(256) void xf_softmax_causal_k(const float* __restrict__ S, uint16_t* __restrict__ P,
                                                           int seq, long long rows) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(row % seq);
  const float* sr = S + row * seq;
  uint16_t* pr = P + row * seq;
  float m = -INFINITY;
  for (int j = lane; j <= i; j += kWave) m = fmaxf(m, sr[j]);
  m = wave_max(m);
  float sum = 0.f;
  for (int j = lane; j <= i; j += kWave) sum += expf(sr[j] - m);
  sum = wave_sum(sum);
  const float inv = 1.f / sum;
  for (int j = lane; j < seq; j += kWave) {
    const __bf16 v = (__bf16)(j <= i ? expf(sr[j] - m) * inv : 0.f);
    pr[j] = __builtin_bit_cast(uint16_t, v);
  }
}

__global__ __launch_bounds__(256) void xf_swiglu_k(uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
                                                   long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4_t gv = ld16(g + 8 * i), uv = ld16(u + 8 * i);
  u32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float g0 = bf16_to_f32(gv[k] & 0xffffu), g1 = bf16_to_f32(gv[k] >> 16);
    const float s0 = g0 / (1.f + expf(-g0)), s1 = g1 / (1.f + expf(-g1));
    o[k] = pack_bf16x2(s0 * bf16_to_f32(uv[k] & 0xffffu), s1 * bf16_to_f32(uv[k] >> 16));
  }
  st16(g + 8 * i, o);
}

__global__ __launch_bounds__(256) void xf_add_k(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                                uint16_t* __restrict__ y, long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4_t av = ld16(a + 8 * i), bv = ld16(b + 8 * i);
  u32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = pack_bf16x2(bf16_to_f32(av[k] & 0xffffu) + bf16_to_f32(bv[k] & 0xffffu),
                       bf16_to_f32(av[k] >> 16) + bf16_to_f32(bv[k] >> 16));
  st16(y + 8 * i, o);
}

hipError_t launch_xf_rmsnorm(const uint16_t* x, const uint16_t* w, uint16_t* y, int N, int d, float eps,
                             hipStream_t s) {
  hipLaunchKernelGGL(xf_rmsnorm_k, dim3(N), dim3(256), 0, s, x, w, y, d, eps);
  return hipGetLastError();
}
hipError_t launch_xf_softmax_causal(const float* S, uint16_t* P, int seq, long long rows, hipStream_t s) {
  hipLaunchKernelGGL(xf_softmax_causal_k, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, S, P, seq, rows);
  return hipGetLastError();
}
hipError_t launch_xf_swiglu(uint16_t* g, const uint16_t* u, long long n, hipStream_t s) {
  const long long n8 = n / 8;
  hipLaunchKernelGGL(xf_swiglu_k, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, g, u, n8);
  return hipGetLastError();
}
hipError_t launch_xf_add(const uint16_t* a, const uint16_t* b, uint16_t* y, long long n, hipStream_t s) {
  const long long n8 = n / 8;
  hipLaunchKernelGGL(xf_add_k, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a, b, y, n8);
  return hipGetLastError();
}

}  // namespace molora
