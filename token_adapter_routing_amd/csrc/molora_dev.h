// Device-side helpers shared by the gfx950 kernels of the adapter-routing library.
//
// Wave64 throughout.  MFMA operand conventions (v_mfma_f32_16x16x32_bf16, D = A*B + C,
// A 16x32, B 32x16, D 16x16):
//   A operand: lane l supplies row m = l%16, k-slots 8*(l/16) .. 8*(l/16)+7 (8 bf16)
//   B operand: lane l supplies column n = l%16, the same k-slots
//   D        : lane l holds column n = l%16, rows 4*(l/16) .. 4*(l/16)+3 (4 fp32)
// Any bijection between k-slots and physical reduction indices may be used as long as
// both operands follow it; the kernels choose one that lets every lane read 64
// contiguous bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "molora_plan.h"

namespace molora {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

template <bool INDIRECT>
__device__ __forceinline__ const uint16_t* adapter_A(const TargetDev& t, int e) {
  if constexpr (INDIRECT) return t.ptrA[e];
  else return t.At + (long long)e * t.strideA;
}
template <bool INDIRECT>
__device__ __forceinline__ const uint16_t* adapter_B(const TargetDev& t, int e) {
  if constexpr (INDIRECT) return t.ptrB[e];
  else return t.Bt + (long long)e * t.strideB;
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ void st16_nt(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Two floats -> packed bf16 pair (round to nearest even; hardware cvt on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Wave64 inclusive prefix sum of an int.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// Tile lookup over the grouped order: adapter e's segment [offsets[e], offsets[e+1]) is cut
// into ceil(count/16) tiles of 16 rows; tiles are numbered adapter by adapter.  Every lane of
// the wave must call this.  Returns false when T is past the last tile.
__device__ __forceinline__ bool find_tile(const int* __restrict__ offsets, int K, int T, int lane,
                                          int& e, int& row0, int& nrows) {
  int lo = 0, hi = 0;
  if (lane < K) {
    lo = offsets[lane];
    hi = offsets[lane + 1];
  }
  const int nt = (hi - lo + kTileRows - 1) / kTileRows;
  const int incl = wave_incl_scan(nt, lane);
  const int excl = incl - nt;
  const uint64_t m = __ballot(lane < K && T >= excl && T < incl);
  if (m == 0) return false;
  const int el = __builtin_ctzll(m);
  e = el;
  const int lo_e = __shfl(lo, el, kWave);
  const int hi_e = __shfl(hi, el, kWave);
  const int ex_e = __shfl(excl, el, kWave);
  row0 = lo_e + (T - ex_e) * kTileRows;
  nrows = min(kTileRows, hi_e - row0);
  return true;
}

// Tile slot of workgroup x for the tiles of find_tile spread over the 8 XCDs in runs: XCD
// x % 8 takes tiles [j per, (j + 1) per) with per = ceil(tiles / 8), so an adapter's tiles
// share an XCD's L2.  The grid's x extent must be a multiple of 8 and at least 8 per; returns
// -1 for workgroups past the tiles.  Every lane of the wave must call this.
__device__ __forceinline__ int xcd_tile_slot(const int* __restrict__ offsets, int K, int x, int lane) {
  int nt = 0;
  if (lane < K) nt = (offsets[lane + 1] - offsets[lane] + kTileRows - 1) / kTileRows;
  const int total = __shfl(wave_incl_scan(nt, lane), kWave - 1, kWave);
  const int per = (total + 7) / 8, j = x >> 3;
  return j < per ? (x & 7) * per + j : -1;
}

// Vocabulary range lookup (largest e with b[e] <= v, if b[0] <= v < b[K]; else -1), on bounds
// held in LDS or registers.
__device__ __forceinline__ int vocab_owner(int v, const int* b, int K) {
  if (v < b[0] || v >= b[K]) return -1;
  int lo = 0, hi = K;  // b[lo] <= v < b[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (b[mid] <= v) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Adapter owning grouped position q (offsets in LDS, K+1 entries): largest e with offsets[e] <= q.
__device__ __forceinline__ int segment_of(const int* offs, int K, int q) {
  int lo = 0, hi = K;  // invariant: offs[lo] <= q < offs[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offs[mid] <= q) lo = mid;
    else hi = mid;
  }
  return lo;
}

}  // namespace molora
