// Host-side launchers of the gfx950 kernels (internal to the library).  Every launcher
// assumes its arguments were validated by the C-ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "molora_dev.h"

namespace molora {

struct VocabBounds {
  int b[65];
};

// Copy the K+1 bounds from kernel arguments into LDS (static indices only).
__device__ __forceinline__ void bounds_to_lds(const VocabBounds& vb, int* lds, int K) {
#pragma unroll
  for (int i = 0; i < 65; ++i)
    if ((int)threadIdx.x == i && i <= K) lds[i] = vb.b[i];
}

hipError_t launch_route_vocab(const int32_t* ids, int N, const VocabBounds& bounds, int K,
                              int32_t* idx, float* w, hipStream_t s);

hipError_t launch_route_topk(const uint16_t* x, int N, int d, const uint16_t* W1, const float* b1,
                             const uint16_t* W2, const float* b2, float* logits, int K, int k,
                             int32_t* idx, float* w, uint8_t* flags, hipStream_t s);

// Chip-wide dispatch split: nb workgroups of C pairs (nb == 1: one workgroup sorts all).
struct DispatchSplit {
  int nb, C;
};
constexpr int kDispMaxParts = 128;
DispatchSplit dispatch_split(long long P);
size_t dispatch_ws_bytes(long long P, int K);  // per-workgroup counts of the chip-wide sort
// ws: at least dispatch_ws_bytes(P, K) bytes, or nullptr (then one workgroup sorts all pairs)
hipError_t launch_dispatch(const int32_t* idx, const float* w, int P, int K, int32_t* counts, int32_t* offsets,
                           int32_t* perm, float* perm_w, int32_t* inv, void* ws, hipStream_t s);

hipError_t launch_relayout(const uint16_t* A, const uint16_t* B, int d_in, int d_out, int r,
                           int r_pad, uint16_t* At, uint16_t* Bt, hipStream_t s);

struct ApplyLaunch {
  TargetDev tgt;
  bool indirect;
  const uint16_t* x;
  const void* y0;
  void* y;
  int y0_f32, y_f32;
  int N, k, K;
  float scale;
  const int32_t* offsets;
  const int32_t* perm;
  const float* perm_w;
  const int32_t* inv;
  int path;          // resolved path (1 GROUPED, 2 SKINNY, 3 TILE, 4 BLOCK)
  float* ws;         // workspace (partials of the shrink; for BLOCK control words first)
  int col_groups;    // 0 = choose
};

// Workspace bytes a resolved apply needs.
size_t apply_ws_bytes(int N, int k, int K, int r_pad, int d_in, int d_out, bool y_f32, int path);
int apply_resolve_path(int N, int k, int path, int K, int r_pad);
constexpr int kApplyTileMaxAdapters = 16;  // tile-local path: distinct adapters per tile
hipError_t launch_apply(const ApplyLaunch& a, hipStream_t s);
// Targets sharing one routing (same N, k, K, rank, path and dtypes); as[0].ws holds the
// whole workspace of apply_multi_ws_bytes bytes.
constexpr int kApplyMaxMulti = 8;
int apply_multi_resolve_path(int n, int N, int k, int path, int K, int r_pad);
size_t apply_multi_ws_bytes(int n, const int* d_in, const int* d_out, int N, int k, int K, int r_pad, bool y_f32,
                            int path);
hipError_t launch_apply_multi(const ApplyLaunch* as, int n, hipStream_t s);

struct StepVocabLaunch {
  ApplyLaunch apply;  // x, y0, y, N, K, scale, target; k = 1
  VocabBounds bounds;
  const int32_t* ids;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  float* perm_w;
  int32_t* inv;
  void* ws;           // NULL: tile apply; else the block apply's workspace
};
// Workspace bytes of the one-launch step on 64-token blocks.
size_t step_ws_bytes(int N, int K, int r_pad, int d_in);
// True when the one-launch step handles N tokens (its per-workgroup dispatch share reads all N
// ids); larger batches run route, dispatch and the tile apply as three launches.
bool step_vocab_fused(int N);
hipError_t launch_step_vocab(const StepVocabLaunch& a, hipStream_t s);

hipError_t launch_seqpass_meta(const int32_t* idx, int N, int K, int32_t* offsets, int32_t* perm,
                               float* perm_w, hipStream_t s);

}  // namespace molora
