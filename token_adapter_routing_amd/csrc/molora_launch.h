// Host-side launchers of the gfx950 kernels (internal to the library).  Every launcher
// assumes its arguments were validated by the C-ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "molora_plan.h"

namespace molora {

struct VocabBounds {
  int b[65];
};

hipError_t launch_route_vocab(const int32_t* ids, int N, const VocabBounds& bounds, int K,
                              int32_t* idx, float* w, hipStream_t s);

// part != NULL (router mode, router_chunked(d)): the first layer split over d into part,
// route_topk_ws_bytes(N, d) bytes; the same results.
hipError_t launch_route_topk(const uint16_t* x, int N, int d, const uint16_t* W1, const float* b1,
                             const uint16_t* W2, const float* b2, float* logits, int K, int k,
                             int32_t* idx, float* w, uint8_t* flags, float* part, hipStream_t s);

// ws: at least dispatch_ws_bytes(P, K) bytes, or nullptr (then one workgroup sorts all pairs)
hipError_t launch_dispatch(const int32_t* idx, const float* w, int P, int K, int32_t* counts, int32_t* offsets,
                           int32_t* perm, float* perm_w, int32_t* inv, void* ws, hipStream_t s);

hipError_t launch_relayout(const uint16_t* A, const uint16_t* B, int d_in, int d_out, int r, int r_pad,
                           uint16_t* At, uint16_t* Bt, hipStream_t s, bool transposed);

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
  float* ws;         // workspace of apply_plan() for this apply (NULL when it needs none)
  int col_groups;    // 0 = choose
};

// Block path (64-token blocks) for small hot sets (dense_block_ok): n targets sharing one
// routing, target i's partials at (char*)as[0].ws + ws_off[i] (block_ws_bytes each).  Sets
// *taken = false and enqueues nothing when the hot set or the targets' slices do not fit the
// dense kernels.
// fuse != NULL: the routing comes as (idx, w) [N*k] (inv, perm_w and offsets unused) and the
// shrink launch also runs the dispatch of those pairs into the given outputs (up to
// kDenseFuseMaxPairs pairs; above that *taken = false).
struct DenseFuse {
  const int32_t* idx;
  const float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  float* perm_w;
  int32_t* inv;
};
hipError_t launch_dense_block(const ApplyLaunch* as, int n, const size_t* ws_off, hipStream_t s, bool* taken,
                              const DenseFuse* fuse = nullptr);

// The tokens a pass does not reach, finished by extra workgroups at the start of the pass's
// last expand launch (rows disjoint from the pass's own): y = y0 for tokens without a routed pair
// (copy_y0), y = z (the fp32 carry) for tokens with fewer than c_last routed pairs (copy_z).
struct FinishArgs {
  const void* y0;
  const float* z;
  void* y;
  const int32_t* inv;
  int N, k, c_last, d_out;
  int y0_f32, y_f32, copy_y0, copy_z;
};
constexpr int kFinishTok = 512;  // tokens per finishing workgroup (8 waves of 64)

struct GMArgs;  // gm_dev.h
// One pass of the 64-row grouped tiles (g: the pass's rows, routing and tiling; g.nwg from
// gs_region) in three launches over 512-wide slices: partials into part, h rows into hb
// (gs_region's layout).
hipError_t launch_gs_pass(const GMArgs& g, float* part, uint16_t* hb, bool y0_f32, bool y_f32, bool indirect,
                          hipStream_t s, const FinishArgs* fin = nullptr);
// fin (optional): extra workgroups of the expand launch finish the tokens the pass does not reach.
// Pair passes (k > 1): the shrink and finalize of one pass over every pair of the dispatch's
// grouped order (g.order null, g.nwg from gs_region over P rows), writing h by grouped position
// into hq [P][2][r_pad]; the tuple sort into its region (tuple_sort_plan's layout), with each
// pass's tiles of tiling tl (rows >= 16); the pair expand of pass m (g: target, y0 / y; g.nwg a
// multiple of 8, at least the pass's tiles, over 256-wide column slices).
hipError_t launch_gs_pair_shrink(const GMArgs& g, float* part, uint16_t* hq, bool indirect, hipStream_t s);
hipError_t launch_tuple_sort(const int32_t* offsets, const int32_t* inv, int N, int k, int K, char* region,
                             const TupleSortPlan& tp, const GMTiling& tl, hipStream_t s);
hipError_t launch_gs_expand_pairs(const GMArgs& g, const char* region, const TupleSortPlan& tp, int m,
                                  const uint16_t* hq, int K, bool y0_f32, bool y_f32, bool indirect, hipStream_t s,
                                  const FinishArgs* fin = nullptr);

// Per-pair shrink without gate weight or scale into hout [P][r_pad] fp32 by grouped position:
// the split shrink and finalize over the 64-row tiles of the dispatch's grouped order; part
// holds the slice partials (gs_region(kPathGrouped, P, K, r_pad, d_in, false).part_bytes).
hipError_t launch_pair_shrink_gm(const TargetDev& tgt, bool indirect, const uint16_t* x, const int32_t* offsets,
                                 const int32_t* perm, int K, int k, long long P, float* hout, float* part,
                                 hipStream_t s);

// Backward of the routed LoRA except dx: dA, dB, dw (any may be NULL) from x, gy and the
// forward routing; ws holds bwd_plan() for these shapes.
struct BackwardLaunch {
  TargetDev tgt, tgt_t;  // forward adapters and their transposed twin (same target)
  bool indirect, indirect_t;
  const uint16_t* x;
  const uint16_t* gy;
  const int32_t* offsets;
  const int32_t* perm;
  const float* perm_w;
  const int32_t* inv;
  int N, k, K, r;
  float scale;
  float* dA;
  float* dB;
  float* dw;
  char* ws;
  bool dx_f32;  // the plan's dx apply (placement of the later regions only)
  int dx_path;
};
hipError_t launch_backward(const BackwardLaunch& a, hipStream_t s);

// Router backward: dL/dlogits of the top-k softmax; the MLP's parameter gradients and dx.
hipError_t launch_route_topk_backward(const int32_t* idx, const float* w, const float* dw, int N, int K, int k,
                                      float* dl, hipStream_t s);
hipError_t launch_router_pre(const uint16_t* x, int N, int d, const uint16_t* W1, const float* b1, float* pre,
                             hipStream_t s);
struct RouterBackwardLaunch {
  const uint16_t* x;   // [N][d] bf16
  int N, d, K;
  const uint16_t* W1;  // [64][d] bf16
  const float* b1;     // [64] or NULL
  const uint16_t* W2;  // [K][64] bf16
  const float* dl;     // dL/dlogits [N][K] fp32
  float* dW1;          // [64][d] or NULL
  float* db1;          // [64] or NULL
  float* dW2;          // [K][64] or NULL
  float* db2;          // [K] or NULL
  const float* dx0;    // [N][d] fp32 or NULL
  float* dx;           // [N][d] fp32 or NULL
  char* ws;            // router_bwd_plan()
};
hipError_t launch_router_backward(const RouterBackwardLaunch& a, hipStream_t s);

// Synthetic decoder forward (xfmr.cpp): base projections on the GEMM library, norms,
// attention softmax, SwiGLU and residual adds on this library's kernels (xf.hip), the
// per-token LoRA of each projection through launch_apply / launch_apply_multi.
enum { kXfQ, kXfK, kXfV, kXfO, kXfGate, kXfUp, kXfDown, kXfTargets };
struct XfLayerDev {
  const uint16_t* norm1;
  const uint16_t* norm2;
  const uint16_t* W[kXfTargets];  // nn.Linear layout [out][in]
  TargetDev tgt[kXfTargets];
  bool lora, indirect;
  float scale;
};
struct XfLaunch {
  int d, f, n_seq, seq_len, n_layers, K, k;
  float eps;
  const XfLayerDev* layers;
  const uint16_t* x_in;
  uint16_t* x_out;
  const int32_t* offsets;
  const int32_t* perm;
  const float* perm_w;
  const int32_t* inv;
  int path_qkv, path_o, path_gu, path_down;  // resolved apply paths
  size_t lora_bytes;                         // the LoRA applies' workspace (xf_plan's lora region)
  char* ws;                                  // xf_plan(n_seq, seq_len, d, f, lora_bytes)
  const char** what;                         // out: what failed
};
hipError_t launch_xf_forward(const XfLaunch& a, hipStream_t s);
hipError_t launch_xf_rmsnorm(const uint16_t* x, const uint16_t* w, uint16_t* y, int N, int d, float eps, hipStream_t s);
hipError_t launch_xf_softmax_causal(const float* S, uint16_t* P, int seq, long long rows, hipStream_t s);
hipError_t launch_xf_swiglu(uint16_t* g, const uint16_t* u, long long n, hipStream_t s);
hipError_t launch_xf_add(const uint16_t* a, const uint16_t* b, uint16_t* y, long long n, hipStream_t s);

// a.ws: the workspace of apply_plan() for a's shape and resolved path.
hipError_t launch_apply(const ApplyLaunch& a, hipStream_t s);
// Targets sharing one routing (same N, k, K, rank, path and dtypes); as[0].ws holds the
// whole workspace of apply_multi_plan().
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
  float* part;         // NULL: the one-launch tile step; else the split launches' partials
  int32_t* bcnt;        // split launches with dispatch_share: per-block adapter counts
  bool dispatch_share;  // the launches write idx .. inv (N <= kStepMaxN); else they only apply
};
hipError_t launch_step_vocab(const StepVocabLaunch& a, hipStream_t s);

// The calling thread's current device's scratch array (kScratchBytes, 256-byte aligned): looked
// up once per device with hipGetSymbolAddress, then cached.  out may be NULL (set-up only).
hipError_t scratch_setup(void** out);

hipError_t launch_seqpass_meta(const int32_t* idx, int N, int K, int32_t* offsets, int32_t* perm,
                               float* perm_w, hipStream_t s);

}  // namespace molora
