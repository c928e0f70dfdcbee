// Sizes and placements shared by the host launchers and the kernels: tile constants, the
// workspace layout of every path, and the index formulas the kernels write partial sums with.
// Plain C++ without HIP types, so the host-side arithmetic also builds for a CPU-only test
// (under AddressSanitizer / UndefinedBehaviorSanitizer) that checks every workspace a kernel
// writes against the bytes the entry points require.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIP__)
#define MOLORA_HD __host__ __device__
#else
#define MOLORA_HD
#endif

namespace molora {

constexpr int kWave = 64;
constexpr int kTileRows = 16;    // rows (pairs) per MFMA tile
constexpr int kStepK = 128;      // reduction elements one wave consumes per shrink step
constexpr int kColBlock = 128;   // output columns one wave produces per expand block

constexpr int kBTok = 64;        // block path: tokens per block
constexpr int kBSlice = 512;     // block path: reduction or output columns per workgroup
constexpr int kSTok = 64;        // split step: tokens per block
constexpr int kSSlice = 512;     // split step: reduction or output columns per workgroup
constexpr int kStepMaxN = 4096;  // the vocabulary step's fused launches handle N <= this
constexpr int kDispChunk = 8192; // pairs one 1024-thread dispatch workgroup sorts per pass
constexpr int kDispMaxParts = 128;
constexpr int kDispMinPart = 1024;  // pairs of one chip-wide dispatch workgroup, at least
constexpr int kApplyTileMaxAdapters = 16;  // tile and block paths: distinct adapters (K <= 16)
constexpr int kApplyMaxMulti = 8;          // targets of one molora_apply_multi call
constexpr size_t kScratchBytes = size_t(8) << 20;  // device scratch of the allocation-free step
                                                   // (MOLORA_NOALLOC_SCRATCH_BYTES)

enum { kPathAuto = 0, kPathGrouped = 1, kPathSkinny = 2, kPathTile = 3, kPathBlock = 4, kPathGroupedFixed = 5 };

// Per-target adapter addressing, as the kernels see it.
struct TargetDev {
  const uint16_t* At;            // direct: A of adapter 0 in the slab's swizzled layout
  const uint16_t* Bt;            // direct: B^T of adapter 0, [d_out][r_pad] bf16
  long long strideA;             // elements between consecutive adapters' A
  long long strideB;             // elements between consecutive adapters' B^T
  const uint16_t* const* ptrA;   // indirect: device table of K A addresses
  const uint16_t* const* ptrB;   // indirect: device table of K B^T addresses
  int d_in, d_out, r_pad;
};

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// ---- dispatch: above kDispChunk pairs the sort runs over nb workgroups of C pairs each, whose
// per-adapter counts ([nb][K] int32) live in the workspace.
struct DispatchSplit {
  int nb, C;
};
DispatchSplit dispatch_split(long long P);
size_t dispatch_ws_bytes(long long P, int K);

// ---- block path: partial sums of the shrink launch, [nblocks][slotmax][kslices][64][r_pad]
// fp32; (tb, slot, sl) starts at block_part_index and holds 64 rows of r_pad floats.
MOLORA_HD inline size_t block_part_index(int tb, int slot, int sl, int slotmax, int kslices, int r_pad) {
  return ((((size_t)tb * slotmax + slot) * kslices + sl) * kBTok) * r_pad;
}
MOLORA_HD inline size_t block_part_floats(int nblocks, int slotmax, int kslices, int r_pad) {
  return (size_t)nblocks * slotmax * kslices * kBTok * r_pad;
}
struct BlockGeom {
  int nblocks, kslices, cslices, slotmax;
};
BlockGeom block_geom(int N, int k, int K, int d_in, int d_out);
size_t block_ws_bytes(int N, int k, int K, int r_pad, int d_in);

// ---- dense-slot blocks: when the 512-wide slices of all K adapters fit in LDS together
// (K * r_pad <= 64) the block path keeps a partial for every adapter (slot = adapter index, the
// same region size since slotmax = K) and runs from a table of (target, slice) work items:
// shrink items grouped by the x they read (per slice, the group's targets in turn), expand
// items per target in slice order.  An item is (target << 8) | slice.
constexpr int kDenseMaxItems = 256;
constexpr int kDenseFuseMaxPairs = 8192;  // pairs whose dispatch rides in the dense shrink launch
MOLORA_HD inline bool dense_block_ok(int K, int r_pad) { return K >= 1 && K * r_pad <= 64; }
struct DenseItems {
  bool ok;    // false: more items than the table holds, or a target with more than 255 slices
  int n_s, n_e;
  uint16_t s[kDenseMaxItems], e[kDenseMaxItems];
  // shrink columns: the items of one x group at one slice, s[col_start[i] .. + col_len[i])
  // for every item i of the column
  uint16_t col_start[kDenseMaxItems];
  uint8_t col_len[kDenseMaxItems];
};
// x_group[i]: index of the first target that reads the same x rows as target i.
DenseItems dense_items(int n, const int* x_group, const int* kslices, const int* cslices);

// ---- split step (vocabulary routing, k = 1): partial h of every token on its own adapter,
// [nblocks][kslices][64][r_pad] fp32; (tb, sl) starts at split_part_index.
MOLORA_HD inline size_t split_part_index(int tb, int sl, int kslices, int r_pad) {
  return (((size_t)tb * kslices + sl) * kSTok) * r_pad;
}
MOLORA_HD inline size_t split_part_floats(int N, int d_in, int r_pad) {
  return (size_t)((N + kSTok - 1) / kSTok) * ((d_in + kSSlice - 1) / kSSlice) * kSTok * r_pad;
}

// Per-block adapter counts of the split step's dispatch share, adapter-major: [K][stride]
// int32 with the block count rounded up to a multiple of 4 (rows read 16 bytes at a time; the
// padding entries are never written and never counted).
MOLORA_HD inline int split_count_stride(int nblocks) { return (nblocks + 3) / 4 * 4; }

// Workspace of molora_step_vocab with a workspace: the split launches' partials at part_off.
// N <= kStepMaxN: those launches also produce the dispatch outputs (fused_dispatch), through
// per-block adapter counts (at cnt_off) that the first launch writes and the second scans.  Larger N: route and a chip-wide dispatch (its per-workgroup counts at disp_off)
// run first.
struct StepPlan {
  bool fused_dispatch;
  size_t disp_off, disp_bytes;
  size_t part_off, part_bytes;
  size_t cnt_off, cnt_bytes;
  size_t total;
};
StepPlan step_plan(int N, int K, int r_pad, int d_in);

// ---- apply paths
int apply_resolve_path(int N, int k, int path, int K, int r_pad);
int apply_multi_resolve_path(int n, int N, int k, int path, int K, int r_pad);
int skinny_splits(int d_in);

// Decode-sized skinny apply with k > 1: one expand launch per call over (target, 32-column
// slice) workgroups that hold the B^T slices of every adapter in LDS and sum each token's
// routed pairs in registers (no rank passes, no fp32 carry).  Bounds: 2 <= k <= 4, N tokens
// at most kDXMaxTok, K * r_pad at most kDXMaxKR (64 KB of B^T per workgroup).
constexpr int kDXCols = 32;
constexpr int kDXMaxTok = 1024;
constexpr int kDXMaxKR = 1024;
bool decode_expand_fits(int N, int k, int K, int r_pad);
// The decode region: h rows [P][2][r_pad] bf16 by pair id, then the pairs' adapters [P] int32.
size_t decode_eid_off(long long P, int r_pad);
size_t decode_hq_bytes(long long P, int r_pad);
// 64-row grouped tiles (r > 32, or k > 1 with k*K <= 64)
bool use_gm(int k, int K, int r_pad);
// The resolved path runs the 64-row grouped kernel: the grouped path where use_gm holds, and
// the fixed-tiling comparator wherever its rank passes apply (k == 1 or k*K <= 64).
// k > 1 runs one split pass per pair rank with an fp32 carry (measured at K = 16, rank 64,
// 16384 tokens, k = 4: 799 us, against 982 us for a token-block expand that read y0 once).
bool gm_path(int path, int k, int K, int r_pad);
// Row tiles of the 64-row grouped kernel: per segment (adapter) of a pass, ceil(count / rows)
// tiles, balanced inside the segment (adaptive) or of exactly `rows` rows but the last (fixed).
struct GMTiling {
  int rows;      // tile height bound (16 .. 64)
  int fixed;     // 1: fixed 64-row tiles per segment
  long long max_tiles;  // upper bound on the tiles of a pass: ceil(rows_of_pass / rows) + keys
};
// slices: workgroups per tile (the d_in slices of a split pass; 1 for one workgroup per tile).
GMTiling gm_tiling(int path, long long rows_of_pass, int nkeys, int slices);

// Rank sort of k > 1 (grouped and skinny paths): counts2 [k*K] and offsets2 [k*K+1] in a
// 256-byte-aligned head, then perm2 [P] int32 and w2 [P] fp32, then the chip-wide sort's
// per-workgroup counts; offsets relative to the start of the sort's region.
struct RankSortPlan {
  size_t counts2_off, offsets2_off, perm2_off, w2_off, bcnt_off, bytes;
};
RankSortPlan rank_sort_plan(long long P, int k, int K);

// Workspace of one molora_apply on a resolved path: [skinny/grouped h partials][rank sort][z],
// where z is the fp32 [N][d_out] carry of the k > 1 passes when y is bf16.
// ---- grouped tiles split over 512-wide slices (a pass of the 64-row grouped tiles in three
// launches): the pass's slice partials [nwg][kslices][64][r_pad] fp32, then its h rows
// [nwg][2][64][r_pad] bf16; nwg = the pass's tile bound rounded up to a multiple of 16 (whole
// XCD rounds of tile pairs).
struct GSRegion {
  int nwg;
  size_t part_bytes, hb_off, total;
};
// with_hb = false: the partials only (a shrink whose finalize writes h by grouped position).
GSRegion gs_region(int path, long long rows_of_pass, int K, int r_pad, int d_in, bool with_hb = true);

// ---- k > 1 in passes over pairs of a token's routed pairs (the 64-row grouped tiles): pass m
// applies the token's routed pairs of rank 2m and 2m + 1 together, so a k = 4 call reads and
// writes the carry twice instead of four times.  A pass's keys are the adapter pairs (a, b),
// b = K for "no second pair": K (K + 1) keys; the tuples are taken when the keys hold 32 rows
// on average or more (N >= 32 K (K + 1)), below that the tiles would be mostly short.
constexpr int kTupleWGTokens = 1024;  // tokens per workgroup of the tuple sort
constexpr int kPairTileRows = 128;    // pair-expand tile height bound (8 row blocks of 16)
bool gm_tuples(int N, int k, int K);
// The tuple sort's region: per-workgroup key counts bcnt [nb][nkeys] (then the workgroups'
// first positions), the pass offsets toff [nkeys + 1], each pass's tiles [m2][tmax] (int4: key
// in the pass, first row, end row) and tile count ntile [m2], and the entries (token, grouped
// position of the first pair, of the second pair or -1) etok / eqa / eqb [m2 * N]; offsets
// relative to the region's start.  tmax = ceil(N / 16) + K (K + 1) bounds a pass's tiles for
// any tile height from 16 rows.
struct TupleSortPlan {
  int m2, kk, nkeys, nb;  // passes ceil(k / 2), keys per pass K (K + 1), all keys, workgroups
  int tmax;
  size_t bcnt_off, toff_off, tiles_off, ntile_off, etok_off, eqa_off, eqb_off, bytes;
};
TupleSortPlan tuple_sort_plan(int N, int k, int K);

struct ApplyPlan {
  int path;
  size_t hpart_off, hpart_bytes;  // shrink partials ([nsplit][P][r_pad] fp32): two-kernel paths,
                                  // and h of every pair for k > 1 on the 64-row grouped tiles
  size_t block_off, block_bytes;  // block path partials
  size_t sort_off;                // rank sort region (k > 1 on the grouped / skinny passes)
  RankSortPlan sort;
  size_t z_off, z_bytes;          // fp32 carry
  size_t gs_off;                  // 64-row grouped passes: the slice partials and h rows
  GSRegion gs;
  int tuples;                     // k > 1 in pair passes: the shrink of every pair, then
  size_t hq_off, hq_bytes;        //   its h by grouped position [P][2][r_pad] bf16 hi / lo,
  size_t tsort_off;               //   the tuple sort and the carry z
  TupleSortPlan tsort;
  size_t total;
};
ApplyPlan apply_plan(int N, int k, int K, int r_pad, int d_in, int d_out, bool y_f32, int path);
size_t apply_ws_bytes(int N, int k, int K, int r_pad, int d_in, int d_out, bool y_f32, int path);

// Workspace of molora_apply_multi (n targets sharing one routing): on the fused skinny path
// [rank sort][per target: h partials, z], or per target [h partials, h rows] when the decode
// expand takes the call; otherwise one apply_plan region per target.
struct MultiPlan {
  int path;
  bool fused;
  size_t sort_off;
  RankSortPlan sort;
  size_t tgt_off[kApplyMaxMulti];   // start of target i's region
  size_t hpart_off[kApplyMaxMulti]; // fused: its h partials
  size_t z_off[kApplyMaxMulti];     // fused: its fp32 carry (bf16 y, k > 1), else 0
  bool decode;                      // fused, decode_expand_fits: h rows instead of sort and carry
  size_t hq_off[kApplyMaxMulti];    // decode: its h rows and pair adapters (decode_hq_bytes)
  size_t total;
};
MultiPlan apply_multi_plan(int n, const int* d_in, const int* d_out, int N, int k, int K, int r_pad, bool y_f32,
                           int path);

// ---- backward (molora_backward): per-pair h = x A_e and g = gy B_e^T from two grouped
// shrinks (unscaled, one partial each), a pair pass that writes
// dL/dw and the scaled h, g as bf16 hi/lo chunks [nchunks][2][r_pad][Qc] (rank-major, pairs
// contiguous, zero past the segment), then the weight-gradient reductions over each
// segment's pairs: partials [nchunks][D / 128][128][r_pad] fp32, summed chunk by chunk.
constexpr int kWStep = 64;   // pairs per LDS step of the weight-gradient kernel
constexpr int kWCols = 128;  // columns of x / gy per weight-gradient workgroup
struct BwdPlan {
  int nsh, nsg;            // splits of the h shrink (over d_in) and the g shrink (over d_out)
  int Qc;                  // pairs per chunk, a multiple of kWStep
  long long nchunks;       // upper bound on chunks: ceil(P / Qc) + K
  size_t h_off, h_bytes;   // h partials [nsh][P][r_pad] fp32
  size_t g_off, g_bytes;   // g partials [nsg][P][r_pad] fp32
  size_t gs_off, gs_bytes; // the h and g shrinks' slice partials (one shrink at a time)
  size_t sa_off, sb_off, s_bytes;  // hi/lo chunks of scale*w*g (for dA) and scale*w*h (for dB)
  size_t part_off, part_bytes;     // weight-gradient partials, shared by dA then dB
  size_t apply_off, apply_bytes;   // dx: the apply on the transposed adapters
  size_t total;
};
int wgrad_chunk(long long P, int D);
// dx_path: the resolved path of the dx apply (apply_resolve_path on the transposed shapes).
BwdPlan bwd_plan(int N, int k, int K, int r_pad, int d_in, int d_out, bool dx_f32, int dx_path);
// bf16 elements of one chunk's hi (or lo) plane; the lo plane follows the hi plane.
MOLORA_HD inline size_t bwd_s_chunk_elems(int r_pad, int Qc) { return (size_t)r_pad * Qc; }

// ---- router first layer split over d (molora_route_topk with a workspace): chunk c of the
// S = d / 128 reduction steps is [S c / 8, S (c + 1) / 8); the workspace holds each chunk's
// sum, [kRouterChunks][N][64] fp32.  Used for d <= 128 * 8 * kRouterMaxChunkSteps.
constexpr int kRouterChunks = 8;
constexpr int kRouterMaxChunkSteps = 4;  // d <= 4096: at most 64 KB of W1 pieces in LDS
MOLORA_HD inline bool router_chunked(int d) {
  return d > 0 && (d / 128 + kRouterChunks - 1) / kRouterChunks <= kRouterMaxChunkSteps;
}
inline size_t route_topk_ws_bytes(int N, int d) {
  return router_chunked(d) ? (size_t)kRouterChunks * N * 64 * sizeof(float) : 0;
}

// ---- router backward (molora_router_backward), hidden width kRouterHidden: the
// pre-activation [N][64] fp32, dL/d(pre-activation) [N][64] fp32, its hi/lo chunk planes for
// the dW1 reduction (one segment: all tokens in order), that reduction's partials, per
// 64-token block partial sums of dW2, db2, db1, and the two-entry segment offsets.
constexpr int kRouterHidden = 64;
constexpr int kRouterTokBlock = 64;
struct RouterBwdPlan {
  int Qc;
  long long nchunks;
  int ntb;  // 64-token blocks
  size_t pre_off, da_off, s_off, part_off, small_off, offs_off, total;
};
RouterBwdPlan router_bwd_plan(int N, int d, int K);
MOLORA_HD inline int router_small_floats(int K) { return K * kRouterHidden + K + kRouterHidden; }

// ---- synthetic decoder (molora_xf_forward): per forward, bf16 activations h (norm output),
// q, k, v, attention output, o (projection output), gate and up [N][f] (the product written
// into gate), the scores [n_seq][heads][S][S] fp32 and probabilities (bf16), the LoRA applies'
// workspace and the GEMM library's workspace.
constexpr int kXfHeadDim = 128;
constexpr size_t kXfBlasBytes = size_t(64) << 20;
struct XfPlan {
  size_t h_off, q_off, k_off, v_off, att_off, o_off, g_off, u_off, s_off, p_off;
  size_t lora_off, lora_bytes, blas_off, blas_bytes, total;
};
XfPlan xf_plan(int n_seq, int seq_len, int d, int f, size_t lora_bytes);

}  // namespace molora
