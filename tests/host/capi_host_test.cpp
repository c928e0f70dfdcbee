// CPU test of the C ABI's host layer, built with AddressSanitizer and UndefinedBehaviorSanitizer.
//
// capi.cpp and plan.cpp are compiled as shipped.  The kernel launchers and the three HIP runtime
// calls that capi.cpp makes are replaced by stand-ins that launch nothing; instead each stand-in
// performs, on host memory, every workspace and slab write the replaced kernels make (from the
// same index helpers the kernels use), so a workspace or slab that the *_workspace / *_bytes
// queries size too small, or a plan whose regions overlap, shows up as a sanitizer error or a
// failed check.  "Device" buffers are host allocations of exactly the queried size.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "molora.h"
#include "molora_launch.h"

using namespace molora;

static int g_fail = 0;
static int g_checks = 0;
#define CHECK(c, ...)                                             \
  do {                                                            \
    ++g_checks;                                                   \
    if (!(c)) {                                                   \
      ++g_fail;                                                   \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);        \
      fprintf(stderr, __VA_ARGS__);                               \
      fprintf(stderr, " [%s]\n", molora_last_error());            \
    }                                                             \
  } while (0)

// ------------------------------------------------------------------ write recording
// Byte ranges written into the current workspace by the stand-in kernels of one call, with the
// name of the array they belong to; ranges of different arrays must not overlap.
struct Range {
  size_t lo, hi;
  std::string what;
};
static std::vector<Range> g_ranges;
static char* g_ws_base = nullptr;
static size_t g_ws_bytes = 0;

// Write `count` elements of T at base[first ..] (every element: the sanitizer checks each).
template <typename T>
static void write_span(void* base, size_t first, size_t count, const char* what) {
  if (count == 0) return;
  T* p = static_cast<T*>(base);
  for (size_t i = 0; i < count; ++i) p[first + i] = T(1);
  char* lo = reinterpret_cast<char*>(p + first);
  if (g_ws_base != nullptr && lo >= g_ws_base && lo < g_ws_base + g_ws_bytes + 1)
    g_ranges.push_back({(size_t)(lo - g_ws_base), (size_t)(lo - g_ws_base) + count * sizeof(T), what});
}

static void check_disjoint(const char* call) {
  std::vector<Range> r = g_ranges;
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < r.size(); ++i)
    CHECK(r[i].lo >= r[i - 1].hi || r[i].what == r[i - 1].what, "%s: %s [%zu, %zu) overlaps %s [%zu, %zu)", call,
          r[i].what.c_str(), r[i].lo, r[i].hi, r[i - 1].what.c_str(), r[i - 1].lo, r[i - 1].hi);
  for (const Range& x : r) CHECK(x.hi <= g_ws_bytes, "%s: %s ends at %zu > %zu", call, x.what.c_str(), x.hi, g_ws_bytes);
}

// ------------------------------------------------------------------ stand-in kernels
static int g_launches = 0;
static int g_last_apply_path = -1;

static void rank_sort_writes(char* region, long long P, int k, int K) {
  const RankSortPlan rp = rank_sort_plan(P, k, K);
  write_span<int32_t>(region + rp.counts2_off, 0, (size_t)k * K, "counts2");
  write_span<int32_t>(region + rp.offsets2_off, 0, (size_t)k * K + 1, "offsets2");
  write_span<int32_t>(region + rp.perm2_off, 0, (size_t)P, "perm2");
  write_span<float>(region + rp.w2_off, 0, (size_t)P, "w2");
  const DispatchSplit ds = dispatch_split(P);
  if (ds.nb > 1) write_span<int32_t>(region + rp.bcnt_off, 0, (size_t)ds.nb * k * K, "rank bcnt");
}

static void block_writes(const ApplyLaunch& a, char* base) {
  const BlockGeom g = block_geom(a.N, a.k, a.K, a.tgt.d_in, a.tgt.d_out);
  for (int tb = 0; tb < g.nblocks; ++tb)
    for (int slot = 0; slot < g.slotmax; ++slot)
      for (int sl = 0; sl < g.kslices; ++sl)
        write_span<float>(base, block_part_index(tb, slot, sl, g.slotmax, g.kslices, a.tgt.r_pad),
                          (size_t)kBTok * a.tgt.r_pad, "block partials");
}

// What launch_apply's kernels write into a.ws for a's resolved path (apply.hip, launch_apply).
static void apply_writes(const ApplyLaunch& a) {
  const ApplyPlan p = apply_plan(a.N, a.k, a.K, a.tgt.r_pad, a.tgt.d_in, a.tgt.d_out, a.y_f32, a.path);
  CHECK(p.path == a.path, "resolved path %d vs plan %d", a.path, p.path);
  char* ws = reinterpret_cast<char*>(a.ws);
  const long long P = (long long)a.N * a.k;
  if (p.total > 0) CHECK(ws != nullptr, "path %d needs a workspace of %zu bytes", a.path, p.total);
  if (ws == nullptr) return;
  if (a.path == kPathBlock) {
    block_writes(a, ws + p.block_off);
    return;
  }
  if (a.path == kPathTile || (a.path == kPathGrouped && a.k == 1)) return;  // no workspace
  if (gm_path(a.path, a.k, a.K, a.tgt.r_pad)) {
    // a pass's slice partials (every tile of the bound, every 512-wide d_in slice) and h rows
    auto gs_writes = [&](long long rows) {
      const GSRegion g = gs_region(a.path, rows, a.K, a.tgt.r_pad, a.tgt.d_in);
      CHECK(g.nwg == p.gs.nwg && g.total == p.gs.total, "split pass region");
      const long long kslices = (a.tgt.d_in + kBSlice - 1) / kBSlice;
      write_span<float>(ws + p.gs_off, 0, (size_t)g.nwg * kslices * 64 * a.tgt.r_pad, "gs partials");
      write_span<uint16_t>(ws + p.gs_off + g.hb_off, 0, (size_t)g.nwg * 2 * 64 * a.tgt.r_pad, "gs h rows");
    };
    if (a.k == 1) {
      gs_writes(P);
      return;
    }
    if (gm_tuples(a.N, a.k, a.K)) {
      // the pair shrink (partials of every pair's tiles), h by grouped position, the tuple
      // sort (counts, offsets, at most N entries per pass) and the carry of k > 2
      CHECK(p.tuples == 1, "pair passes planned");
      const GSRegion g = gs_region(a.path, P, a.K, a.tgt.r_pad, a.tgt.d_in, false);
      const long long kslices = (a.tgt.d_in + kBSlice - 1) / kBSlice;
      write_span<float>(ws + p.gs_off, 0, (size_t)g.nwg * kslices * 64 * a.tgt.r_pad, "pair partials");
      write_span<uint16_t>(ws + p.hq_off, 0, (size_t)P * 2 * a.tgt.r_pad, "pair h");
      const int m2 = (a.k + 1) / 2, nkeys = m2 * a.K * (a.K + 1);
      const int nb = (a.N + kTupleWGTokens - 1) / kTupleWGTokens;
      const TupleSortPlan& t = p.tsort;
      write_span<int32_t>(ws + p.tsort_off + t.bcnt_off, 0, (size_t)nb * nkeys, "tuple counts");
      write_span<int32_t>(ws + p.tsort_off + t.toff_off, 0, (size_t)nkeys + 1, "tuple offsets");
      // a pass's tiles: at most ceil(N / rows) + keys of the expand's tiling (rows >= 16)
      const GMTiling te = gm_tiling(a.path, a.N, a.K * (a.K + 1), (a.tgt.d_out + 255) / 256);
      CHECK(te.rows >= 16 && te.max_tiles <= t.tmax, "tile table bound");
      write_span<int32_t>(ws + p.tsort_off + t.tiles_off, 0, (size_t)m2 * t.tmax * 4, "tuple tiles");
      write_span<int32_t>(ws + p.tsort_off + t.ntile_off, 0, (size_t)m2, "tuple tile counts");
      write_span<int32_t>(ws + p.tsort_off + t.etok_off, 0, (size_t)m2 * a.N, "tuple tokens");
      write_span<int32_t>(ws + p.tsort_off + t.eqa_off, 0, (size_t)m2 * a.N, "tuple first pairs");
      write_span<int32_t>(ws + p.tsort_off + t.eqb_off, 0, (size_t)m2 * a.N, "tuple second pairs");
      if (!a.y_f32 && m2 > 1) write_span<float>(ws + p.z_off, 0, (size_t)a.N * a.tgt.d_out, "z");
      return;
    }
    CHECK(p.tuples == 0, "rank passes planned");
    rank_sort_writes(ws + p.sort_off, P, a.k, a.K);
    if (!a.y_f32) write_span<float>(ws + p.z_off, 0, (size_t)a.N * a.tgt.d_out, "z");
    gs_writes(a.N);
    return;
  }
  const int ns = a.path == kPathSkinny ? skinny_splits(a.tgt.d_in) : 1;
  write_span<float>(ws + p.hpart_off, 0, (size_t)ns * P * a.tgt.r_pad, "hpart");
  if (a.path == kPathSkinny && decode_expand_fits(a.N, a.k, a.K, a.tgt.r_pad)) {
    // the decode expand: the summed h rows [P][2][r_pad] bf16 and the pairs' adapters, by pair
    // id (no sort, no carry)
    write_span<uint16_t>(ws + p.hq_off, 0, (size_t)P * 2 * a.tgt.r_pad, "decode h rows");
    write_span<int32_t>(ws + p.hq_off + decode_eid_off(P, a.tgt.r_pad), 0, (size_t)P, "decode adapters");
  } else if (a.path == kPathSkinny && a.k > 1 && a.k * a.K <= 64) {
    rank_sort_writes(ws + p.sort_off, P, a.k, a.K);
    if (!a.y_f32) write_span<float>(ws + p.z_off, 0, (size_t)a.N * a.tgt.d_out, "z");
  }
}

namespace molora {

hipError_t launch_route_vocab(const int32_t*, int, const VocabBounds&, int, int32_t*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_route_topk(const uint16_t*, int N, int d, const uint16_t* W1, const float*, const uint16_t*,
                             const float*, float*, int, int, int32_t*, float*, uint8_t*, float* part, hipStream_t) {
  ++g_launches;
  // the split first layer writes kRouterChunks x N x 64 floats into the workspace
  if (part != nullptr) {
    CHECK(W1 != nullptr && router_chunked(d), "split router layer for d=%d", d);
    write_span<float>(part, 0, (size_t)kRouterChunks * N * 64, "route part");
  }
  return hipSuccess;
}
hipError_t launch_dispatch(const int32_t*, const float*, int P, int K, int32_t*, int32_t*, int32_t*, float*, int32_t*,
                           void* ws, hipStream_t) {
  ++g_launches;
  const DispatchSplit d = dispatch_split(P);
  if (d.nb > 1 && ws != nullptr) write_span<int32_t>(ws, 0, (size_t)d.nb * K, "dispatch bcnt");
  return hipSuccess;
}
hipError_t launch_relayout(const uint16_t*, const uint16_t*, int d_in, int d_out, int, int r_pad, uint16_t* At,
                           uint16_t* Bt, hipStream_t, bool) {
  ++g_launches;
  write_span<uint16_t>(At, 0, (size_t)r_pad * d_in, "A slot");
  write_span<uint16_t>(Bt, 0, (size_t)d_out * r_pad, "B slot");
  return hipSuccess;
}
// What launch_backward's kernels write into the workspace (backward.hip): the h and g
// partials, the hi/lo chunk planes, and the weight-gradient partials (dA, then dB, in one
// region the two reductions take in turn).
static int g_last_backward_outputs = 0;
hipError_t launch_backward(const BackwardLaunch& a, hipStream_t) {
  ++g_launches;
  const BwdPlan p = bwd_plan(a.N, a.k, a.K, a.tgt.r_pad, a.tgt.d_in, a.tgt.d_out, a.dx_f32, a.dx_path);
  const long long P = (long long)a.N * a.k;
  CHECK(a.tgt.d_in == a.tgt_t.d_out && a.tgt.d_out == a.tgt_t.d_in, "twin shapes");
  g_last_backward_outputs = (a.dA != nullptr) + 2 * (a.dB != nullptr) + 4 * (a.dw != nullptr);
  const bool need_h = a.dB != nullptr || a.dw != nullptr, need_g = a.dA != nullptr || a.dw != nullptr;
  if (P > 0) {
    // the split shrinks' partials: every tile of the bound, every 512-wide slice of d_in (h) or d_out (g)
    for (int d : {need_h ? a.tgt.d_in : 0, need_g ? a.tgt.d_out : 0}) {
      if (d == 0) continue;
      const int kslices = (d + kBSlice - 1) / kBSlice;
      const GMTiling tl = gm_tiling(kPathGrouped, P, a.K, kslices);
      const long long nwg = (tl.max_tiles + 15) / 16 * 16;  // whole XCD rounds of tile pairs
      CHECK(nwg == gs_region(kPathGrouped, P, a.K, a.tgt.r_pad, d, false).nwg, "bwd shrink tiles");
      write_span<float>(a.ws + p.gs_off, 0, (size_t)nwg * kslices * 64 * a.tgt.r_pad, "bwd shrink partials");
    }
    if (need_h) write_span<float>(a.ws + p.h_off, 0, (size_t)p.nsh * P * a.tgt.r_pad, "bwd h");
    if (need_g) write_span<float>(a.ws + p.g_off, 0, (size_t)p.nsg * P * a.tgt.r_pad, "bwd g");
    const size_t planes = (size_t)p.nchunks * 2 * bwd_s_chunk_elems(a.tgt.r_pad, p.Qc);
    if (a.dA != nullptr) write_span<uint16_t>(a.ws + p.sa_off, 0, planes, "bwd s for dA");
    if (a.dB != nullptr) write_span<uint16_t>(a.ws + p.sb_off, 0, planes, "bwd s for dB");
    CHECK(p.Qc % kWStep == 0 && p.Qc >= kWStep, "chunk of %d pairs", p.Qc);
    CHECK(p.nchunks >= (P + p.Qc - 1) / p.Qc + a.K, "chunk bound");
  }
  if (a.dA != nullptr && P > 0)
    write_span<float>(a.ws + p.part_off, 0, (size_t)p.nchunks * a.tgt.d_in * a.tgt.r_pad, "bwd wgrad part");
  if (a.dB != nullptr && P > 0)
    write_span<float>(a.ws + p.part_off, 0, (size_t)p.nchunks * a.tgt.d_out * a.tgt.r_pad, "bwd wgrad part");
  return hipSuccess;
}
hipError_t launch_route_topk_backward(const int32_t*, const float*, const float*, int, int, int, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
// What launch_router_backward's kernels write into the workspace (backward.hip).
hipError_t launch_router_backward(const RouterBackwardLaunch& a, hipStream_t) {
  ++g_launches;
  const RouterBwdPlan p = router_bwd_plan(a.N, a.d, a.K);
  write_span<float>(a.ws + p.pre_off, 0, (size_t)a.N * kRouterHidden, "router pre");
  write_span<float>(a.ws + p.da_off, 0, (size_t)a.N * kRouterHidden, "router da");
  if (a.N > 0) {
    // the planes of every token block's chunk, up to the block-rounded token count
    const long long last = ((long long)p.ntb * kRouterTokBlock - 1) / p.Qc;
    CHECK(last < p.nchunks, "router chunk %lld of %lld", last, p.nchunks);
    write_span<uint16_t>(a.ws + p.s_off, 0, (size_t)(last + 1) * 2 * bwd_s_chunk_elems(kRouterHidden, p.Qc),
                         "router s");
    write_span<float>(a.ws + p.part_off, 0, (size_t)p.nchunks * a.d * kRouterHidden, "router part");
  }
  write_span<float>(a.ws + p.small_off, 0, (size_t)p.ntb * router_small_floats(a.K), "router small");
  write_span<int32_t>(a.ws + p.offs_off, 0, 2, "router offsets");
  return hipSuccess;
}
// What launch_xf_forward writes into the workspace (xfmr.cpp): every activation region, the
// LoRA applies' workspace of each call and the GEMM library's workspace.
hipError_t launch_xf_forward(const XfLaunch& a, hipStream_t) {
  ++g_launches;
  const XfPlan p = xf_plan(a.n_seq, a.seq_len, a.d, a.f, a.lora_bytes);
  const size_t N = (size_t)a.n_seq * a.seq_len, H = a.d / kXfHeadDim, ss = (size_t)a.n_seq * H * a.seq_len * a.seq_len;
  write_span<uint16_t>(a.ws + p.h_off, 0, N * a.d, "xf h");
  write_span<uint16_t>(a.ws + p.q_off, 0, N * a.d, "xf q");
  write_span<uint16_t>(a.ws + p.k_off, 0, N * a.d, "xf k");
  write_span<uint16_t>(a.ws + p.v_off, 0, N * a.d, "xf v");
  write_span<uint16_t>(a.ws + p.att_off, 0, N * a.d, "xf att");
  write_span<uint16_t>(a.ws + p.o_off, 0, N * a.d, "xf o");
  write_span<uint16_t>(a.ws + p.g_off, 0, N * a.f, "xf gate");
  write_span<uint16_t>(a.ws + p.u_off, 0, N * a.f, "xf up");
  write_span<float>(a.ws + p.s_off, 0, ss, "xf scores");
  write_span<uint16_t>(a.ws + p.p_off, 0, ss, "xf probs");
  write_span<char>(a.ws + p.blas_off, 0, p.blas_bytes, "xf blas");
  for (int l = 0; l < a.n_layers; ++l) {
    const XfLayerDev& L = a.layers[l];
    if (!L.lora) continue;
    ApplyLaunch m{};
    m.N = (int)N; m.k = a.k; m.K = a.K; m.y_f32 = 0; m.ws = reinterpret_cast<float*>(a.ws + p.lora_off);
    // the single-target applies (o, down) at their own shapes; the multi applies' plans
    for (int t : {kXfO, kXfDown}) {
      m.tgt = L.tgt[t];
      m.path = t == kXfO ? a.path_o : a.path_down;
      const size_t before = g_ranges.size();
      apply_writes(m);
      // the applies run one after another in the same region: one array for the overlap check
      for (size_t i = before; i < g_ranges.size(); ++i) g_ranges[i].what = "xf lora";
    }
    int din[3], dout[3];
    for (int i = 0; i < 3; ++i) { din[i] = L.tgt[i].d_in; dout[i] = L.tgt[i].d_out; }
    const MultiPlan mq = apply_multi_plan(3, din, dout, (int)N, a.k, a.K, L.tgt[0].r_pad, false, kPathAuto);
    CHECK(mq.path == a.path_qkv, "q/k/v path %d vs %d", mq.path, a.path_qkv);
    write_span<char>(a.ws + p.lora_off, 0, mq.total, "xf lora");
    for (int i = 0; i < 2; ++i) { din[i] = L.tgt[kXfGate + i].d_in; dout[i] = L.tgt[kXfGate + i].d_out; }
    const MultiPlan mg = apply_multi_plan(2, din, dout, (int)N, a.k, a.K, L.tgt[0].r_pad, false, kPathAuto);
    write_span<char>(a.ws + p.lora_off, 0, mg.total, "xf lora");
  }
  return hipSuccess;
}
hipError_t launch_apply(const ApplyLaunch& a, hipStream_t) {
  ++g_launches;
  g_last_apply_path = a.path;
  apply_writes(a);
  return hipSuccess;
}
hipError_t launch_apply_multi(const ApplyLaunch* as, int n, hipStream_t) {
  ++g_launches;
  const ApplyLaunch& a0 = as[0];
  g_last_apply_path = a0.path;
  int d_in[kApplyMaxMulti], d_out[kApplyMaxMulti];
  for (int i = 0; i < n; ++i) {
    d_in[i] = as[i].tgt.d_in;
    d_out[i] = as[i].tgt.d_out;
  }
  const MultiPlan mp = apply_multi_plan(n, d_in, d_out, a0.N, a0.k, a0.K, a0.tgt.r_pad, a0.y_f32, a0.path);
  char* ws = reinterpret_cast<char*>(a0.ws);
  if (mp.total > 0) CHECK(ws != nullptr, "multi needs %zu bytes", mp.total);
  if (ws == nullptr) return hipSuccess;
  if (!mp.fused) {
    for (int i = 0; i < n; ++i) {
      ApplyLaunch b = as[i];
      b.ws = reinterpret_cast<float*>(ws + mp.tgt_off[i]);
      apply_writes(b);
    }
    return hipSuccess;
  }
  const long long P = (long long)a0.N * a0.k;
  CHECK(mp.decode == (decode_expand_fits(a0.N, a0.k, a0.K, a0.tgt.r_pad) && a0.path == kPathSkinny), "decode plan");
  if (a0.k > 1 && !mp.decode) rank_sort_writes(ws + mp.sort_off, P, a0.k, a0.K);
  for (int i = 0; i < n; ++i) {
    write_span<float>(ws + mp.hpart_off[i], 0, (size_t)skinny_splits(d_in[i]) * P * a0.tgt.r_pad, "hpart (multi)");
    if (mp.decode) {
      write_span<uint16_t>(ws + mp.hq_off[i], 0, (size_t)P * 2 * a0.tgt.r_pad, "decode h rows (multi)");
      write_span<int32_t>(ws + mp.hq_off[i] + decode_eid_off(P, a0.tgt.r_pad), 0, (size_t)P, "decode adapters (multi)");
    } else if (a0.k > 1 && !a0.y_f32) {
      write_span<float>(ws + mp.z_off[i], 0, (size_t)a0.N * d_out[i], "z (multi)");
    }
  }
  return hipSuccess;
}
hipError_t launch_dense_block(const ApplyLaunch* as, int n, const size_t* ws_off, hipStream_t, bool* taken,
                              const DenseFuse* fuse) {
  // the device side's own conditions, then the two launches' workspace writes (partials of
  // every adapter per block and slice for each target)
  const ApplyLaunch& a0 = as[0];
  *taken = false;
  if (!dense_block_ok(a0.K, a0.tgt.r_pad) || a0.k > 4) return hipSuccess;
  if (fuse != nullptr && ((long long)a0.N * a0.k > kDenseFuseMaxPairs || a0.K > 16)) return hipSuccess;
  int xg[kApplyMaxMulti], ks[kApplyMaxMulti], cs[kApplyMaxMulti];
  for (int i = 0; i < n; ++i) {
    xg[i] = i;
    for (int j = 0; j < i; ++j)
      if (as[j].x == as[i].x && as[j].tgt.d_in == as[i].tgt.d_in) {
        xg[i] = xg[j];
        break;
      }
    const BlockGeom g = block_geom(as[i].N, as[i].k, as[i].K, as[i].tgt.d_in, as[i].tgt.d_out);
    ks[i] = g.kslices;
    cs[i] = g.cslices;
  }
  if (!dense_items(n, xg, ks, cs).ok) return hipSuccess;
  *taken = true;
  g_launches += 2;
  g_last_apply_path = a0.path;
  if (fuse != nullptr) CHECK(fuse->idx != nullptr && fuse->w != nullptr && fuse->inv != nullptr, "fused routing arrays");
  for (int i = 0; i < n; ++i) {
    const BlockGeom g = block_geom(as[i].N, as[i].k, as[i].K, as[i].tgt.d_in, as[i].tgt.d_out);
    CHECK(g.slotmax == as[i].K, "dense partials need one slot per adapter");
    write_span<float>(reinterpret_cast<char*>(a0.ws) + ws_off[i], 0,
                      block_part_floats(g.nblocks, g.slotmax, g.kslices, as[i].tgt.r_pad), "dense partials");
  }
  return hipSuccess;
}
hipError_t launch_step_vocab(const StepVocabLaunch& a, hipStream_t) {
  ++g_launches;
  CHECK(a.apply.N <= kStepMaxN || !a.dispatch_share, "fused dispatch share above %d tokens (N=%d)", kStepMaxN,
        a.apply.N);
  if (a.part == nullptr) return hipSuccess;  // the one-launch tile step writes no workspace
  const int nblocks = (a.apply.N + kSTok - 1) / kSTok;
  const int kslices = (a.apply.tgt.d_in + kSSlice - 1) / kSSlice;
  for (int tb = 0; tb < nblocks; ++tb)
    for (int sl = 0; sl < kslices; ++sl)
      write_span<float>(a.part, split_part_index(tb, sl, kslices, a.apply.tgt.r_pad), (size_t)kSTok * a.apply.tgt.r_pad,
                        "split partials");
  if (a.dispatch_share) {  // the first launch's per-block adapter counts
    CHECK(a.bcnt != nullptr, "per-block counts buffer missing");
    if (a.bcnt != nullptr) write_span<int32_t>(a.bcnt, 0, (size_t)a.apply.K * split_count_stride(nblocks), "block counts");
  }
  return hipSuccess;
}
static char* g_scratch = nullptr;  // host stand-in of the device scratch array
hipError_t scratch_setup(void** out) {
  if (g_scratch == nullptr) {
    void* p = nullptr;
    if (posix_memalign(&p, 256, kScratchBytes) != 0) return hipErrorOutOfMemory;
    g_scratch = static_cast<char*>(p);
  }
  if (out != nullptr) *out = g_scratch;
  return hipSuccess;
}
hipError_t launch_seqpass_meta(const int32_t*, int, int, int32_t*, int32_t*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

}  // namespace molora

extern "C" {
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);  // the indirect layout's pointer tables, written into the host "slab"
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stand-in"; }
}

// ------------------------------------------------------------------ helpers
static void* fake(size_t addr) { return reinterpret_cast<void*>(addr); }  // aligned, never dereferenced

struct HostHotset {
  molora_hotset* hs = nullptr;
  std::vector<char> slab;
};

static bool make_hotset(HostHotset& h, int K, int r, const std::vector<std::pair<int, int>>& dims, int layout,
                        bool transposed = false) {
  auto init = transposed ? molora_hotset_init_transposed : molora_hotset_init;
  std::vector<molora_target> tg;
  for (auto& d : dims) tg.push_back({d.first, d.second, fake(0x10000), fake(0x20000)});
  size_t bytes = 0;
  int rc = molora_hotset_bytes(K, r, (int)tg.size(), tg.data(), layout, &bytes);
  CHECK(rc == MOLORA_OK, "hotset_bytes K=%d r=%d", K, r);
  if (rc != MOLORA_OK) return false;
  h.slab.assign(bytes + 256, 0);  // + room to align the base to 256 bytes
  char* base = h.slab.data();
  base += (256 - reinterpret_cast<uintptr_t>(base) % 256) % 256;
  // a slab one byte short is refused before anything is written
  rc = init(&h.hs, K, r, 2.0f, (int)tg.size(), tg.data(), layout, base, bytes - 1, nullptr);
  CHECK(rc == MOLORA_ENOSPC && h.hs == nullptr, "short slab accepted");
  g_ws_base = base;  // slot and table writes must land inside [base, base + bytes)
  g_ws_bytes = bytes;
  g_ranges.clear();
  rc = init(&h.hs, K, r, 2.0f, (int)tg.size(), tg.data(), layout, base, bytes, nullptr);
  CHECK(rc == MOLORA_OK, "hotset_init K=%d r=%d layout=%d transposed=%d", K, r, layout, (int)transposed);
  for (const Range& x : g_ranges) CHECK(x.hi <= bytes, "slab write %s ends at %zu > %zu", x.what.c_str(), x.hi, bytes);
  g_ws_base = nullptr;
  return rc == MOLORA_OK;
}

// Host buffer of exactly n bytes, 256-byte aligned (n == 0: none); the sanitizer flags any
// access past its n-th byte.
static void* exact_alloc(size_t n) {
  if (n == 0) return nullptr;
  void* p = nullptr;
  if (posix_memalign(&p, 256, n) != 0) return nullptr;
  return p;
}

static const size_t kMaxBuf = 192ull << 20;  // skip combinations whose workspace exceeds this

// ------------------------------------------------------------------ tests
static void test_step(int K, int r, int d_in, int d_out, int N, int layout) {
  HostHotset h;
  if (!make_hotset(h, K, r, {{d_in, d_out}}, layout)) return;
  std::vector<int32_t> bounds(K + 1);
  for (int e = 0; e <= K; ++e) bounds[e] = 8192 * e;
  size_t need = 0;
  CHECK(molora_step_workspace(h.hs, 0, N, &need) == MOLORA_OK, "step_workspace N=%d", N);
  const StepPlan sp = step_plan(N, K, (r + 15) / 16 * 16, d_in);
  CHECK(need == sp.total, "step_workspace %zu vs plan %zu", need, sp.total);
  if (need > kMaxBuf) {
    molora_hotset_destroy(h.hs);
    return;
  }
  // exact-size workspace: every write the launches make must land inside it
  char* ws = static_cast<char*>(exact_alloc(need));
  g_ws_base = ws;
  g_ws_bytes = need;
  g_ranges.clear();
  const int l0 = g_launches;
  int rc = molora_step_vocab(h.hs, 0, (int32_t*)fake(0x1000), N, bounds.data(), fake(0x2000), fake(0x3000),
                             MOLORA_BF16, fake(0x4000), MOLORA_BF16, (int32_t*)fake(0x5000), (float*)fake(0x6000),
                             (int32_t*)fake(0x7000), (int32_t*)fake(0x8000), (int32_t*)fake(0x9000),
                             (float*)fake(0xa000), (int32_t*)fake(0xb000), ws, need, nullptr);
  if (K <= kApplyTileMaxAdapters) {
    CHECK(rc == MOLORA_OK, "step N=%d K=%d r=%d d=%d", N, K, r, d_in);
    const int launches = g_launches - l0;
    if (N == 0) CHECK(launches == 0, "N=0 launched %d", launches);
    else if (N <= kStepMaxN) CHECK(launches == 1, "N=%d: %d launch calls", N, launches);
    else CHECK(launches == 3, "N=%d: %d launch calls (route, dispatch, split)", N, launches);
    check_disjoint("step");
    // one byte short: refused, nothing launched
    if (need > 0 && N > 0) {
      const int l1 = g_launches;
      rc = molora_step_vocab(h.hs, 0, (int32_t*)fake(0x1000), N, bounds.data(), fake(0x2000), fake(0x3000), MOLORA_BF16,
                             fake(0x4000), MOLORA_BF16, (int32_t*)fake(0x5000), (float*)fake(0x6000),
                             (int32_t*)fake(0x7000), (int32_t*)fake(0x8000), (int32_t*)fake(0x9000),
                             (float*)fake(0xa000), (int32_t*)fake(0xb000), ws, need - 1, nullptr);
      CHECK(rc == MOLORA_ENOSPC && g_launches == l1, "short step workspace accepted (N=%d)", N);
    }
    // without a workspace: the tile step (no workspace writes)
    g_ranges.clear();
    rc = molora_step_vocab(h.hs, 0, (int32_t*)fake(0x1000), N, bounds.data(), fake(0x2000), fake(0x3000), MOLORA_BF16,
                           fake(0x4000), MOLORA_BF16, (int32_t*)fake(0x5000), (float*)fake(0x6000),
                           (int32_t*)fake(0x7000), (int32_t*)fake(0x8000), (int32_t*)fake(0x9000), (float*)fake(0xa000),
                           (int32_t*)fake(0xb000), nullptr, 0, nullptr);
    CHECK(rc == MOLORA_OK && g_ranges.empty(), "tile step N=%d", N);
  } else {
    CHECK(rc == MOLORA_ENOTSUP, "step with K=%d accepted", K);
  }
  g_ws_base = nullptr;
  free(ws);
  molora_hotset_destroy(h.hs);
}

static void test_apply(int K, int r, int d_in, int d_out, int N, int k, int path, int y_dtype) {
  HostHotset h;
  if (!make_hotset(h, K, r, {{d_in, d_out}}, MOLORA_LAYOUT_DIRECT)) return;
  size_t need = 0;
  int rc = molora_apply_workspace(h.hs, 0, N, k, y_dtype, path, &need);
  if (k > K) {
    CHECK(rc != MOLORA_OK, "k > K accepted");
    molora_hotset_destroy(h.hs);
    return;
  }
  CHECK(rc == MOLORA_OK, "apply_workspace");
  if (need > kMaxBuf) {
    molora_hotset_destroy(h.hs);
    return;
  }
  char* ws = static_cast<char*>(exact_alloc(need));
  g_ws_base = ws;
  g_ws_bytes = need;
  g_ranges.clear();
  g_last_apply_path = -1;
  rc = molora_apply(h.hs, 0, fake(0x2000), fake(0x3000), y_dtype, fake(0x4000), y_dtype, N, k, (int32_t*)fake(0x8000),
                    (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000), path, ws, need, nullptr);
  const bool tile_like = path == MOLORA_PATH_TILE || path == MOLORA_PATH_BLOCK;
  if (tile_like && K > kApplyTileMaxAdapters) {
    CHECK(rc == MOLORA_ENOTSUP, "tile/block with K=%d accepted", K);
  } else {
    CHECK(rc == MOLORA_OK, "apply N=%d k=%d K=%d r=%d path=%d", N, k, K, r, path);
    if (N > 0) CHECK(g_last_apply_path == apply_resolve_path(N, k, path, K, (r + 15) / 16 * 16), "path");
    int reported = -1;
    CHECK(molora_apply_path(h.hs, 0, N, k, path, &reported) == MOLORA_OK &&
              (N == 0 || reported == g_last_apply_path),
          "molora_apply_path reports %d, the launch ran %d", reported, g_last_apply_path);
    check_disjoint("apply");
    if (need > 0 && N > 0) {
      const int l1 = g_launches;
      rc = molora_apply(h.hs, 0, fake(0x2000), fake(0x3000), y_dtype, fake(0x4000), y_dtype, N, k,
                        (int32_t*)fake(0x8000), (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000),
                        path, ws, need - 1, nullptr);
      CHECK(rc == MOLORA_ENOSPC && g_launches == l1, "short apply workspace accepted");
    }
  }
  g_ws_base = nullptr;
  free(ws);
  molora_hotset_destroy(h.hs);
}

static void test_backward(int K, int r, int d_in, int d_out, int N, int k, int dx_dtype, int layout, int outputs) {
  HostHotset f, t;
  if (!make_hotset(f, K, r, {{d_in, d_out}}, layout)) return;
  if (!make_hotset(t, K, r, {{d_in, d_out}}, layout, true)) {
    molora_hotset_destroy(f.hs);
    return;
  }
  size_t need = 0;
  int rc = molora_backward_workspace(f.hs, t.hs, 0, N, k, dx_dtype, &need);
  if (k > K) {
    CHECK(rc != MOLORA_OK, "backward k > K accepted");
  } else if (need <= kMaxBuf) {
    CHECK(rc == MOLORA_OK, "backward_workspace K=%d r=%d N=%d k=%d", K, r, N, k);
    // swapped or mismatched hot sets are refused before anything is enqueued
    CHECK(molora_backward_workspace(t.hs, f.hs, 0, N, k, dx_dtype, &need) == MOLORA_EINVAL, "swapped pair accepted");
    CHECK(molora_backward_workspace(f.hs, f.hs, 0, N, k, dx_dtype, &need) == MOLORA_EINVAL, "forward as twin accepted");
    rc = molora_backward_workspace(f.hs, t.hs, 0, N, k, dx_dtype, &need);
    char* ws = static_cast<char*>(exact_alloc(need));
    g_ws_base = ws;
    g_ws_bytes = need;
    g_ranges.clear();
    void* dx = (outputs & 8) ? fake(0x4000) : nullptr;
    float* dA = (outputs & 1) ? (float*)fake(0xc000) : nullptr;
    float* dB = (outputs & 2) ? (float*)fake(0xd000) : nullptr;
    float* dw = (outputs & 4) ? (float*)fake(0xe000) : nullptr;
    const int l0 = g_launches;
    g_last_backward_outputs = -1;
    rc = molora_backward(f.hs, t.hs, 0, fake(0x2000), fake(0x3000), fake(0x5000), dx_dtype, dx, dx_dtype, N, k,
                         (int32_t*)fake(0x8000), (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000),
                         dA, dB, dw, ws, need, nullptr);
    if (outputs == 0) {
      CHECK(rc == MOLORA_EINVAL && g_launches == l0, "backward without outputs accepted");
    } else {
      CHECK(rc == MOLORA_OK, "backward K=%d r=%d d=%d/%d N=%d k=%d outputs=%d", K, r, d_in, d_out, N, k, outputs);
      const bool wgrads = (outputs & 7) != 0;
      if (wgrads) CHECK(g_last_backward_outputs == (outputs & 7), "backward outputs %d", g_last_backward_outputs);
      check_disjoint("backward");
      if (need > 0 && N > 0) {
        const int l1 = g_launches;
        rc = molora_backward(f.hs, t.hs, 0, fake(0x2000), fake(0x3000), fake(0x5000), dx_dtype, dx, dx_dtype, N, k,
                             (int32_t*)fake(0x8000), (int32_t*)fake(0x9000), (float*)fake(0xa000),
                             (int32_t*)fake(0xb000), dA, dB, dw, ws, need - 1, nullptr);
        CHECK(rc == MOLORA_ENOSPC && g_launches == l1, "short backward workspace accepted");
      }
    }
    g_ws_base = nullptr;
    free(ws);
  }
  molora_hotset_destroy(f.hs);
  molora_hotset_destroy(t.hs);
}

static void test_router_backward(int N, int d, int K) {
  size_t need = 0;
  CHECK(molora_router_backward_workspace(N, d, K, &need) == MOLORA_OK, "router_backward_workspace");
  if (need > kMaxBuf) return;
  char* ws = static_cast<char*>(exact_alloc(need));
  g_ws_base = ws;
  g_ws_bytes = need;
  g_ranges.clear();
  const int l0 = g_launches;
  int rc = molora_router_backward(fake(0x1000), N, d, fake(0x2000), (float*)fake(0x3000), fake(0x4000), K,
                                  (float*)fake(0x5000), (float*)fake(0x6000), (float*)fake(0x7000),
                                  (float*)fake(0x8000), (float*)fake(0x9000), nullptr, (float*)fake(0xa000), ws, need,
                                  nullptr);
  CHECK(rc == MOLORA_OK && g_launches == l0 + 1, "router_backward N=%d d=%d K=%d", N, d, K);
  check_disjoint("router_backward");
  const int l1 = g_launches;
  rc = molora_router_backward(fake(0x1000), N, d, fake(0x2000), nullptr, fake(0x4000), K, (float*)fake(0x5000),
                              (float*)fake(0x6000), nullptr, nullptr, nullptr, nullptr, nullptr, ws, need - 1, nullptr);
  CHECK(rc == MOLORA_ENOSPC && g_launches == l1, "short router workspace accepted");
  rc = molora_router_backward(fake(0x1000), N, d, fake(0x2000), nullptr, fake(0x4000), K, (float*)fake(0x5000),
                              nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, ws, need, nullptr);
  CHECK(rc == MOLORA_EINVAL && g_launches == l1, "router backward without outputs accepted");
  g_ws_base = nullptr;
  free(ws);
  CHECK(molora_router_backward_workspace(N, 100, K, &need) == MOLORA_ENOTSUP, "d=100 accepted");
  CHECK(molora_route_topk_backward(nullptr, nullptr, nullptr, 4, K, K + 1, nullptr, nullptr) == MOLORA_ENOTSUP,
        "k > K accepted");
}

// molora_route_topk with a workspace: the split first layer writes only inside it, for the d
// it covers; larger d and logits mode leave it alone; a short workspace is refused.
static void test_route_topk_ws(int N, int d) {
  size_t need = 1;
  CHECK(molora_route_topk_workspace(N, d, &need) == MOLORA_OK, "route_topk_workspace N=%d d=%d", N, d);
  CHECK(need == (molora::router_chunked(d) ? (size_t)8 * N * 64 * 4 : 0), "route_topk workspace %zu", need);
  const size_t alloc = std::max<size_t>(need, 256);
  if (alloc > kMaxBuf) return;
  char* ws = static_cast<char*>(exact_alloc(alloc));
  g_ws_base = ws;
  g_ws_bytes = need;
  g_ranges.clear();
  const int l0 = g_launches;
  int rc = molora_route_topk(fake(0x1000), N, d, fake(0x2000), nullptr, fake(0x4000), nullptr, (float*)fake(0x5000),
                             4, 2, (int32_t*)fake(0x6000), (float*)fake(0x7000), nullptr, ws, need, nullptr);
  CHECK(rc == MOLORA_OK && g_launches == l0 + (N > 0 ? 1 : 0), "route_topk with workspace N=%d d=%d", N, d);
  check_disjoint("route_topk");
  if (need > 0) {
    rc = molora_route_topk(fake(0x1000), N, d, fake(0x2000), nullptr, fake(0x4000), nullptr, (float*)fake(0x5000), 4,
                           2, (int32_t*)fake(0x6000), (float*)fake(0x7000), nullptr, ws, need - 1, nullptr);
    CHECK(rc == MOLORA_ENOSPC, "short route_topk workspace accepted");
  }
  g_ws_base = nullptr;
  free(ws);
}

static void test_xf(int d, int f, int L, int n_seq, int seq_len, int K, int r, int k, bool lora) {
  std::vector<HostHotset> hsv(L);
  std::vector<molora_xf_layer> layers(L);
  for (int l = 0; l < L; ++l) {
    molora_xf_layer& X = layers[l];
    X.norm1 = fake(0x1000);
    X.norm2 = fake(0x1100);
    for (int t = 0; t < 7; ++t) X.W[t] = fake(0x2000 + 0x100 * t);
    X.lora = nullptr;
    if (lora) {
      if (!make_hotset(hsv[l], K, r, {{d, d}, {d, d}, {d, d}, {d, d}, {d, f}, {d, f}, {f, d}}, MOLORA_LAYOUT_DIRECT)) return;
      X.lora = hsv[l].hs;
    }
  }
  size_t need = 0;
  int rc = molora_xf_workspace(d, f, L, layers.data(), n_seq, seq_len, k, &need);
  if (lora && k > K) {
    CHECK(rc == MOLORA_ENOTSUP, "xf k > K accepted");
  } else {
    CHECK(rc == MOLORA_OK, "xf_workspace d=%d f=%d L=%d N=%dx%d", d, f, L, n_seq, seq_len);
    if (need <= kMaxBuf) {
      char* ws = static_cast<char*>(exact_alloc(need));
      g_ws_base = ws;
      g_ws_bytes = need;
      g_ranges.clear();
      const int l0 = g_launches;
      rc = molora_xf_forward(d, f, L, layers.data(), n_seq, seq_len, fake(0x3000), fake(0x4000), k,
                             (int32_t*)fake(0x8000), (int32_t*)fake(0x9000), (float*)fake(0xa000),
                             (int32_t*)fake(0xb000), ws, need, nullptr);
      CHECK(rc == MOLORA_OK && g_launches == l0 + 1, "xf_forward");
      check_disjoint("xf_forward");
      rc = molora_xf_forward(d, f, L, layers.data(), n_seq, seq_len, fake(0x3000), fake(0x4000), k,
                             (int32_t*)fake(0x8000), (int32_t*)fake(0x9000), (float*)fake(0xa000),
                             (int32_t*)fake(0xb000), ws, need - 1, nullptr);
      CHECK(rc == MOLORA_ENOSPC, "short xf workspace accepted");
      g_ws_base = nullptr;
      free(ws);
    }
    // a LoRA layer with the wrong shapes is refused
    if (lora) {
      HostHotset bad;
      if (make_hotset(bad, K, r, {{d, d}, {d, d}, {d, d}, {d, d}, {d, f}, {d, f}, {d, f}}, MOLORA_LAYOUT_DIRECT)) {
        const molora_hotset* keep = layers[0].lora;
        layers[0].lora = bad.hs;
        CHECK(molora_xf_workspace(d, f, L, layers.data(), n_seq, seq_len, k, &need) == MOLORA_EINVAL,
              "mismatched LoRA targets accepted");
        layers[0].lora = keep;
        molora_hotset_destroy(bad.hs);
      }
    }
  }
  for (auto& h : hsv) molora_hotset_destroy(h.hs);
}

static void test_multi(int K, int r, int N, int k, int path, int y_dtype) {
  const std::vector<std::pair<int, int>> qwen = {{2048, 2048}, {2048, 1024}, {2048, 1024}, {2048, 2048},
                                                 {2048, 6144}, {2048, 6144}, {6144, 2048}};
  HostHotset h;
  if (!make_hotset(h, K, r, qwen, MOLORA_LAYOUT_INDIRECT)) return;
  const int n = 7;
  int targets[n];
  const void* xs[n];
  const void* y0s[n];
  void* ys[n];
  for (int i = 0; i < n; ++i) {
    targets[i] = i;
    xs[i] = fake(0x100000 + 0x1000 * i);
    y0s[i] = fake(0x200000 + 0x1000 * i);
    ys[i] = fake(0x300000 + 0x1000 * i);
  }
  size_t need = 0;
  int rc = molora_apply_multi_workspace(h.hs, n, targets, N, k, y_dtype, path, &need);
  CHECK(rc == MOLORA_OK, "multi_workspace");
  if (need > kMaxBuf) {
    molora_hotset_destroy(h.hs);
    return;
  }
  char* ws = static_cast<char*>(exact_alloc(need));
  g_ws_base = ws;
  g_ws_bytes = need;
  g_ranges.clear();
  rc = molora_apply_multi(h.hs, n, targets, xs, y0s, y_dtype, ys, y_dtype, N, k, (int32_t*)fake(0x8000),
                          (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000), path, ws, need, nullptr);
  CHECK(rc == MOLORA_OK, "multi N=%d k=%d path=%d", N, k, path);
  check_disjoint("apply_multi");
  if (need > 0) {
    rc = molora_apply_multi(h.hs, n, targets, xs, y0s, y_dtype, ys, y_dtype, N, k, (int32_t*)fake(0x8000),
                            (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000), path, ws, need - 1,
                            nullptr);
    CHECK(rc == MOLORA_ENOSPC, "short multi workspace accepted");
  }
  g_ws_base = nullptr;
  free(ws);
  // dispatch + apply in one call: the apply's regions, then the dispatch's counts
  size_t need2 = 0;
  rc = molora_dispatch_apply_multi_workspace(h.hs, n, targets, N, k, y_dtype, path, &need2);
  CHECK(rc == MOLORA_OK && need2 == align256(need) + dispatch_ws_bytes((long long)N * k, K),
        "dispatch_apply_multi_workspace %zu", need2);
  if (need2 <= kMaxBuf) {
    char* ws2 = static_cast<char*>(exact_alloc(std::max<size_t>(need2, 1)));
    g_ws_base = ws2;
    g_ws_bytes = need2;
    g_ranges.clear();
    const int l0 = g_launches;
    rc = molora_dispatch_apply_multi(h.hs, n, targets, xs, y0s, y_dtype, ys, y_dtype, N, k, (int32_t*)fake(0x7000),
                                     (float*)fake(0x7800), (int32_t*)fake(0x8000), (int32_t*)fake(0x8800),
                                     (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000), path, ws2,
                                     need2, nullptr);
    CHECK(rc == MOLORA_OK && g_launches == l0 + (N > 0 ? 2 : 0), "dispatch_apply_multi N=%d k=%d path=%d (%d launches)",
          N, k, path, g_launches - l0);
    check_disjoint("dispatch_apply_multi");
    if (need2 > 0) {
      rc = molora_dispatch_apply_multi(h.hs, n, targets, xs, y0s, y_dtype, ys, y_dtype, N, k, (int32_t*)fake(0x7000),
                                       (float*)fake(0x7800), (int32_t*)fake(0x8000), (int32_t*)fake(0x8800),
                                       (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000), path,
                                       ws2, need2 - 1, nullptr);
      CHECK(rc == MOLORA_ENOSPC, "short dispatch_apply_multi workspace accepted");
    }
    rc = molora_dispatch_apply_multi(h.hs, n, targets, xs, y0s, y_dtype, ys, y_dtype, N, k, (int32_t*)fake(0x7000),
                                     (float*)fake(0x7800), (int32_t*)fake(0x8000), (int32_t*)fake(0x8800),
                                     (int32_t*)fake(0x9000), (float*)fake(0xa000), nullptr, path, ws2, need2, nullptr);
    CHECK(rc == MOLORA_EINVAL || N == 0, "dispatch_apply_multi without inv accepted");
    g_ws_base = nullptr;
    free(ws2);
  }
  molora_hotset_destroy(h.hs);
}

static void test_dispatch() {
  for (long long N : {1LL, 8192LL, 8193LL, 16384LL, 100000LL, 1048579LL})
    for (int k : {1, 2, 4})
      for (int K : {1, 4, 16, 64}) {
        size_t need = 0;
        CHECK(molora_dispatch_workspace((int)N, k, K, &need) == MOLORA_OK, "dispatch_workspace");
        char* ws = static_cast<char*>(exact_alloc(need));
        g_ws_base = ws;
        g_ws_bytes = need;
        g_ranges.clear();
        int rc = molora_dispatch((int32_t*)fake(0x1000), (float*)fake(0x2000), (int)N, k, K, (int32_t*)fake(0x3000),
                                 (int32_t*)fake(0x4000), (int32_t*)fake(0x5000), (float*)fake(0x6000),
                                 (int32_t*)fake(0x7000), ws, need, nullptr);
        CHECK(rc == MOLORA_OK, "dispatch N=%lld k=%d K=%d", N, k, K);
        check_disjoint("dispatch");
        if (need > 0) {
          rc = molora_dispatch((int32_t*)fake(0x1000), (float*)fake(0x2000), (int)N, k, K, (int32_t*)fake(0x3000),
                               (int32_t*)fake(0x4000), (int32_t*)fake(0x5000), (float*)fake(0x6000),
                               (int32_t*)fake(0x7000), ws, need - 4, nullptr);
          CHECK(rc == MOLORA_ENOSPC, "short dispatch workspace accepted");
        }
        g_ws_base = nullptr;
        free(ws);
      }
}

static void test_validation() {
  // argument errors are reported before anything is launched
  const int l0 = g_launches;
  int32_t b[3] = {0, 10, 5};
  CHECK(molora_route_vocab((int32_t*)fake(0x1000), 4, b, 2, (int32_t*)fake(0x2000), (float*)fake(0x3000), nullptr) ==
            MOLORA_EINVAL && std::strstr(molora_last_error(), "non-decreasing") != nullptr,
        "decreasing bounds");
  CHECK(molora_route_vocab((int32_t*)fake(0x1002), 4, b + 0, 1, (int32_t*)fake(0x2000), (float*)fake(0x3000),
                           nullptr) == MOLORA_EINVAL,
        "misaligned ids");
  CHECK(molora_route_topk(nullptr, 4, 0, nullptr, nullptr, nullptr, nullptr, (float*)fake(0x1000), 4, 5,
                          (int32_t*)fake(0x2000), (float*)fake(0x3000), nullptr, nullptr, 0, nullptr) == MOLORA_ENOTSUP,
        "k > K");
  CHECK(molora_dispatch((int32_t*)fake(0x1000), (float*)fake(0x2000), 1 << 29, 8, 4, (int32_t*)fake(0x3000),
                        (int32_t*)fake(0x4000), (int32_t*)fake(0x5000), (float*)fake(0x6000), nullptr, nullptr, 0,
                        nullptr) == MOLORA_ENOTSUP,
        "N*k overflow");
  HostHotset h;
  if (make_hotset(h, 4, 16, {{512, 512}}, MOLORA_LAYOUT_DIRECT)) {
    size_t sz = 0;
    CHECK(molora_apply_workspace(h.hs, 1, 4, 1, 0, 0, &sz) == MOLORA_EINVAL, "target out of range");
    CHECK(molora_apply_workspace(h.hs, 0, 4, 5, 0, 0, &sz) == MOLORA_EINVAL, "k > K");
    CHECK(molora_apply(h.hs, 0, fake(0x2008), fake(0x3000), 0, fake(0x4000), 0, 4, 1, (int32_t*)fake(0x8000),
                       (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000), 0, nullptr, 0,
                       nullptr) == MOLORA_EINVAL,
          "misaligned x");
    CHECK(molora_apply(h.hs, 0, fake(0x2000), fake(0x3000), 0, fake(0x3000), 1, 4, 1, (int32_t*)fake(0x8000),
                       (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000), 0, nullptr, 0,
                       nullptr) == MOLORA_EINVAL,
          "in place with two dtypes");
    CHECK(molora_hotset_load(h.hs, 0, 4, fake(0x10), fake(0x10), nullptr) == MOLORA_EINVAL, "adapter out of range");
    molora_hotset_destroy(h.hs);
  }
  CHECK(g_launches == l0 + 4, "launches during validation: %d", g_launches - l0);  // init: one relayout per adapter
}

// The allocation-free step: workspace from the scratch stand-in (exactly kScratchBytes), size
// limit enforced before anything is launched.
static void test_noalloc() {
  HostHotset h;
  if (!make_hotset(h, 4, 16, {{4096, 4096}}, MOLORA_LAYOUT_DIRECT)) return;
  int32_t bounds[5] = {0, 8192, 16384, 24576, 32768};
  void* sp = nullptr;
  CHECK(scratch_setup(&sp) == hipSuccess, "scratch stand-in");
  for (int N : {1, 2048, 4096, 4097, 8192, 16383, 16384, 65536}) {
    const StepPlan plan = step_plan(N, 4, 16, 4096);
    g_ws_base = static_cast<char*>(sp);
    g_ws_bytes = kScratchBytes;
    g_ranges.clear();
    const int l0 = g_launches;
    const int rc = molora_step_vocab_noalloc(h.hs, 0, (int32_t*)fake(0x1000), N, bounds, fake(0x2000), fake(0x3000),
                                             MOLORA_BF16, fake(0x4000), MOLORA_BF16, (int32_t*)fake(0x5000),
                                             (float*)fake(0x6000), (int32_t*)fake(0x7000), (int32_t*)fake(0x8000),
                                             (int32_t*)fake(0x9000), (float*)fake(0xa000), (int32_t*)fake(0xb000),
                                             nullptr);
    if (plan.total <= kScratchBytes) {
      CHECK(rc == MOLORA_OK, "noalloc N=%d", N);
      check_disjoint("noalloc");
    } else {
      CHECK(rc == MOLORA_ENOSPC && g_launches == l0 && std::strstr(molora_last_error(), "scratch") != nullptr,
            "noalloc N=%d above the scratch size accepted", N);
    }
  }
  g_ws_base = nullptr;
  molora_hotset_destroy(h.hs);
}

// Work items of the dense-slot block kernels: every (target, slice) exactly once; shrink items
// of one x group interleaved per slice; the table's capacity enforced.
static void test_dense_items() {
  using namespace molora;
  CHECK(dense_block_ok(4, 16) && dense_block_ok(2, 32) && dense_block_ok(1, 64) && !dense_block_ok(5, 16) &&
            !dense_block_ok(2, 48) && !dense_block_ok(0, 16),
        "dense_block_ok");
  // a transformer layer's 7 projections: q, k, v, gate, up read x; o and down their own rows
  const int xg[7] = {0, 0, 0, 3, 0, 0, 6};
  const int ks[7] = {4, 4, 4, 4, 4, 4, 12}, cs[7] = {4, 2, 2, 4, 12, 12, 4};
  const DenseItems d = dense_items(7, xg, ks, cs);
  CHECK(d.ok && d.n_s == 36 && d.n_e == 40, "dense items %d %d", d.n_s, d.n_e);
  int seen_s[7][256] = {}, seen_e[7][256] = {};
  for (int i = 0; i < d.n_s; ++i) ++seen_s[d.s[i] >> 8][d.s[i] & 255];
  for (int i = 0; i < d.n_e; ++i) ++seen_e[d.e[i] >> 8][d.e[i] & 255];
  for (int t = 0; t < 7; ++t) {
    for (int sl = 0; sl < 256; ++sl) CHECK(seen_s[t][sl] == (sl < ks[t] ? 1 : 0), "shrink item (%d, %d)", t, sl);
    for (int c = 0; c < 256; ++c) CHECK(seen_e[t][c] == (c < cs[t] ? 1 : 0), "expand item (%d, %d)", t, c);
  }
  // the x group of target 0 comes first, slice by slice: q, k, v, gate, up of slice 0, ...
  const int first[5] = {0, 1, 2, 4, 5};
  for (int sl = 0; sl < 4; ++sl)
    for (int j = 0; j < 5; ++j)
      CHECK(d.s[5 * sl + j] == ((first[j] << 8) | sl), "group order at %d: %04x", 5 * sl + j, d.s[5 * sl + j]);
  // columns: one x group at one slice; the kernel's decode of a workgroup number covers every
  // (pair block group, item) once for any number of pair block groups
  for (int i = 0; i < d.n_s; ++i) {
    const int c0 = d.col_start[i], len = d.col_len[i];
    CHECK(c0 <= i && i < c0 + len && c0 + len <= d.n_s, "column of item %d", i);
    for (int j = c0; j < c0 + len; ++j)
      CHECK((d.s[j] & 255) == (d.s[i] & 255) && xg[d.s[j] >> 8] == xg[d.s[i] >> 8], "column mixes items %d, %d", i, j);
  }
  for (int npg : {1, 3, 4, 7}) {
    std::vector<int> seen((size_t)npg * d.n_s, 0);
    for (int q = 0; q < npg * d.n_s; ++q) {
      const int i0 = q / npg, c0 = d.col_start[i0], len = d.col_len[i0], local = q - npg * c0;
      const int pbg = local / len, item = c0 + local % len;
      CHECK(pbg >= 0 && pbg < npg && item >= c0 && item < c0 + len, "decode q=%d npg=%d", q, npg);
      if (pbg >= 0 && pbg < npg) ++seen[(size_t)pbg * d.n_s + item];
    }
    for (int v : seen) CHECK(v == 1, "decode coverage npg=%d", npg);
  }
  // capacity: 8 targets of 33 slices overflow the shrink table
  int xg8[8], ks8[8], cs8[8];
  for (int i = 0; i < 8; ++i) {
    xg8[i] = i;
    ks8[i] = 33;
    cs8[i] = 1;
  }
  CHECK(!dense_items(8, xg8, ks8, cs8).ok, "shrink table overflow accepted");
  ks8[0] = 256;
  CHECK(!dense_items(1, xg8, ks8, cs8).ok, "256 slices accepted");
  const int bad[2] = {1, 1};
  CHECK(!dense_items(2, bad, ks, cs).ok, "x group pointing forward accepted");
}

int main() {
  test_dense_items();
  for (int N : {0, 1, 100, 4096, 4097})
    for (int d : {128, 640, 2048, 4096, 4224, 8192}) test_route_topk_ws(N, d);
  test_noalloc();
  test_validation();
  test_dispatch();
  for (int layout : {MOLORA_LAYOUT_DIRECT, MOLORA_LAYOUT_INDIRECT})
    for (int K : {1, 4, 16, 17})
      for (int r : {8, 16, 64})
        for (int N : {0, 1, 63, 64, 2048, 4096, 4097, 8192, 8193, 65536})
          test_step(K, r, 4096, 4096, N, layout);
  test_step(4, 16, 512, 1536, 5000, MOLORA_LAYOUT_DIRECT);
  for (int path : {MOLORA_PATH_AUTO, MOLORA_PATH_GROUPED, MOLORA_PATH_SKINNY, MOLORA_PATH_TILE, MOLORA_PATH_BLOCK,
                   MOLORA_PATH_GROUPED_FIXED})
    for (int K : {1, 4, 16, 64})
      for (int r : {8, 16, 48, 64})
        for (int k : {1, 2, 3, 4, 8})
          for (int N : {0, 1, 100, 1024, 4097})
            for (int yd : {MOLORA_BF16, MOLORA_F32}) test_apply(K, r, 1024, 2048, N, k, path, yd);
  for (int N : {16384}) test_apply(16, 64, 4096, 4096, N, 4, MOLORA_PATH_AUTO, MOLORA_BF16);
  for (int k : {2, 3, 4})  // pair passes at the stress shape
    for (int yd : {MOLORA_BF16, MOLORA_F32}) test_apply(16, 64, 4096, 4096, 16384, k, MOLORA_PATH_GROUPED, yd);
  for (int N : {2303, 2304, 65536})  // K (K + 1) = 72 keys per pass, four passes at k = 8
    for (int k : {7, 8}) test_apply(8, 64, 512, 640, N, k, MOLORA_PATH_GROUPED, MOLORA_BF16);
  for (int path : {MOLORA_PATH_AUTO, MOLORA_PATH_SKINNY, MOLORA_PATH_BLOCK, MOLORA_PATH_GROUPED})
    for (int k : {1, 2})
      for (int N : {1, 256, 4096})
        for (int yd : {MOLORA_BF16, MOLORA_F32}) test_multi(4, 16, N, k, path, yd);
  for (int k : {2, 3, 4})  // the decode expand (K * r_pad = 1024) and just past its token bound
    for (int N : {1, 256, 1024, 1025})
      for (int yd : {MOLORA_BF16, MOLORA_F32}) test_multi(16, 64, N, k, MOLORA_PATH_SKINNY, yd);
  test_multi(16, 16, 4096, 2, MOLORA_PATH_BLOCK, MOLORA_BF16);  // no dense kernels: dispatch, then apply
  test_multi(4, 16, 8192, 2, MOLORA_PATH_BLOCK, MOLORA_BF16);   // 16384 pairs: dispatch, then apply
  for (int layout : {MOLORA_LAYOUT_DIRECT, MOLORA_LAYOUT_INDIRECT})
    for (int K : {1, 4, 16, 64})
      for (int r : {8, 16, 64})
        for (int k : {1, 2, 4})
          for (int N : {0, 1, 100, 2048, 16384})
            test_backward(K, r, 1024, 2048, N, k, MOLORA_BF16, layout, 15);
  for (int outputs = 0; outputs < 16; ++outputs) test_backward(4, 16, 512, 256, 777, 2, MOLORA_F32, MOLORA_LAYOUT_DIRECT, outputs);
  test_backward(16, 64, 4096, 4096, 16384, 1, MOLORA_BF16, MOLORA_LAYOUT_DIRECT, 15);
  for (int N : {0, 1, 63, 64, 65, 4096, 5000, 65536})
    for (int d : {128, 2048, 4096})
      for (int K : {1, 4, 64}) test_router_backward(N, d, K);
  test_xf(256, 768, 2, 2, 64, 4, 8, 1, true);
  test_xf(256, 768, 1, 3, 17, 2, 16, 2, true);
  test_xf(256, 768, 2, 2, 64, 4, 8, 1, false);
  test_xf(1024, 2816, 2, 16, 512, 4, 16, 1, true);
  test_xf(512, 1408, 1, 1, 100, 2, 16, 3, true);
  free(g_scratch);
  fprintf(stderr, "%d checks, %d failures\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
