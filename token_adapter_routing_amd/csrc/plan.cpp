// Host-side sizes and placements of every workspace (declared in molora_plan.h).  Plain C++:
// the library builds it with the kernels, and a CPU-only test builds it with the sanitizers.
#include "molora_plan.h"

#include <algorithm>

namespace molora {

DispatchSplit dispatch_split(long long P) {
  DispatchSplit d{1, (int)P};
  if (P <= kDispChunk) return d;
  // parts of kDispMinPart pairs (one per thread) up to kDispMaxParts parts, then larger ones
  long long C = std::max<long long>(kDispMinPart, (P + kDispMaxParts - 1) / kDispMaxParts);
  C = (C + kDispMinPart - 1) / kDispMinPart * kDispMinPart;
  d.C = (int)C;
  d.nb = (int)((P + C - 1) / C);
  return d;
}

size_t dispatch_ws_bytes(long long P, int K) {
  const DispatchSplit d = dispatch_split(P);
  return d.nb > 1 ? (size_t)d.nb * K * sizeof(int32_t) : 0;
}

BlockGeom block_geom(int N, int k, int K, int d_in, int d_out) {
  BlockGeom g;
  g.nblocks = (N + kBTok - 1) / kBTok;
  g.kslices = (d_in + kBSlice - 1) / kBSlice;
  g.cslices = (d_out + kBSlice - 1) / kBSlice;
  g.slotmax = std::min(K, kBTok * k);
  return g;
}

size_t block_ws_bytes(int N, int k, int K, int r_pad, int d_in) {
  const BlockGeom g = block_geom(N, k, K, d_in, kBSlice);
  return block_part_floats(g.nblocks, g.slotmax, g.kslices, r_pad) * sizeof(float);
}

DenseItems dense_items(int n, const int* x_group, const int* kslices, const int* cslices) {
  DenseItems d{};
  d.ok = n >= 1 && n <= kApplyMaxMulti;
  for (int i = 0; i < n && d.ok; ++i)
    if (kslices[i] < 1 || kslices[i] > 255 || cslices[i] < 1 || cslices[i] > 255 || x_group[i] < 0 ||
        x_group[i] > i || x_group[x_group[i]] != x_group[i])
      d.ok = false;
  if (!d.ok) return d;
  for (int g = 0; g < n; ++g) {
    if (x_group[g] != g) continue;  // not the first target of its group
    for (int sl = 0; sl < kslices[g]; ++sl) {
      const int c0 = d.n_s;
      for (int i = g; i < n; ++i)
        if (x_group[i] == g && sl < kslices[i]) {
          if (d.n_s == kDenseMaxItems) {
            d.ok = false;
            return d;
          }
          d.s[d.n_s++] = (uint16_t)((i << 8) | sl);
        }
      for (int i = c0; i < d.n_s; ++i) {
        d.col_start[i] = (uint16_t)c0;
        d.col_len[i] = (uint8_t)(d.n_s - c0);
      }
    }
  }
  for (int i = 0; i < n; ++i)
    for (int cs = 0; cs < cslices[i]; ++cs) {
      if (d.n_e == kDenseMaxItems) {
        d.ok = false;
        return d;
      }
      d.e[d.n_e++] = (uint16_t)((i << 8) | cs);
    }
  return d;
}

StepPlan step_plan(int N, int K, int r_pad, int d_in) {
  StepPlan p{};
  p.fused_dispatch = N <= kStepMaxN;
  p.disp_off = 0;
  p.disp_bytes = p.fused_dispatch ? 0 : dispatch_ws_bytes(N, K);
  p.part_off = align256(p.disp_bytes);
  p.part_bytes = split_part_floats(N, d_in, r_pad) * sizeof(float);
  p.cnt_off = align256(p.part_off + p.part_bytes);
  p.cnt_bytes = p.fused_dispatch ? (size_t)K * split_count_stride((N + kSTok - 1) / kSTok) * sizeof(int32_t) : 0;
  p.total = p.cnt_off + p.cnt_bytes;
  return p;
}

int apply_resolve_path(int N, int k, int path, int K, int r_pad) {
  if (path != kPathAuto) return path;
  const long long P = (long long)N * k;
  // Measured at d = 4096, rank 16 (dispatch + apply, uniform routing, 1..2048 tokens, 4..64
  // adapters): for k = 1 the grouped 16-row tiles win at every batch up to 512 tokens and for
  // more than 4 adapters at every size (an 8-token tile reads every adapter its tokens use:
  // 1.3-3.4x slower with 8-16 adapters); the tile path wins from 1024 pairs with at most 4
  // adapters.  For k > 1 the tile path applies a token's pairs in one workgroup, where the
  // grouped path would carry the sum through memory between rank passes.  Ranks above 32: the
  // 64-row grouped tiles from 1024 pairs on; below that the skinny path's split reductions.
  // Small hot sets (every adapter's 512-wide slice in LDS at once, K * r_pad <= 64): the
  // dense-slot 64-token blocks from 192 pairs at k > 1 and from 4096 tokens at k = 1 (measured
  // at d = 2048..6144, 256..8192 tokens, K = 2..4, r = 16 and 32: 1.1-1.5x over the tile path,
  // which reads every adapter a tile uses whole).  Below 4096 tokens at k = 1 their shrink has
  // fewer workgroups than the chip has CUs and loses to the tile path with cold inputs.
  if (dense_block_ok(K, r_pad)) {
    if (k > 1) return P >= 192 ? kPathBlock : kPathGrouped;
    if (N >= 4096) return kPathBlock;
  }
  if (r_pad <= 32) {
    if (k > 1) return (K <= kApplyTileMaxAdapters && P >= 192) ? kPathTile : kPathGrouped;
    return (P >= 1024 && K <= 4) ? kPathTile : kPathGrouped;
  }
  return P >= 1024 ? kPathGrouped : kPathSkinny;
}

// AUTO for several targets: as for one, except that tile-local applies with k > 1 become the
// 64-token blocks, whose two launches then cover every target, and that small hot sets take
// the dense-slot blocks from 192 pairs at any k (one launch per phase for all targets: 2-3.4x
// over the grouped tiles at 256..1024 tokens, measured).
int apply_multi_resolve_path(int n, int N, int k, int path, int K, int r_pad) {
  const int p = apply_resolve_path(N, k, path, K, r_pad);
  if (path == kPathAuto && n > 1 && dense_block_ok(K, r_pad) && (long long)N * k >= 192) return kPathBlock;
  return (path == kPathAuto && p == kPathTile && k > 1 && n > 1) ? kPathBlock : p;
}

int skinny_splits(int d_in) {
  int ns = (d_in / kStepK) / 4;  // 512 reduction elements per split
  if (ns < 1) ns = 1;
  if (ns > 16) ns = 16;
  return ns;
}

bool decode_expand_fits(int N, int k, int K, int r_pad) {
  return k >= 2 && k <= 4 && N <= kDXMaxTok && K * r_pad <= kDXMaxKR;
}

size_t decode_eid_off(long long P, int r_pad) { return align256((size_t)P * 2 * r_pad * sizeof(uint16_t)); }
size_t decode_hq_bytes(long long P, int r_pad) {
  return decode_eid_off(P, r_pad) + align256((size_t)P * sizeof(int32_t));
}

bool use_gm(int k, int K, int r_pad) { return (k > 1 && k * K <= 64) || (k == 1 && r_pad > 32); }

bool gm_path(int path, int k, int K, int r_pad) {
  if (path == kPathGrouped) return use_gm(k, K, r_pad);
  return path == kPathGroupedFixed && (k == 1 || k * K <= 64);
}

// Adaptive: every segment is cut into ceil(count / rows) tiles of balanced height, so no tile
// spans two adapters and a small segment gets one short tile.  The height bound is 64 rows when
// a tile runs as several workgroups (one per 512-wide slice: measured at 512 tokens, K = 4,
// rank 64, 16-row tiles took 44.0 us against 41.0 us for 64-row ones, since every tile reads its
// adapter's whole slices); with one workgroup per tile it aims at 256 workgroups over the pass
// (one round on the chip), between 16 and 64 rows.  Fixed: 64-row tiles per segment whatever
// its size (the fixed-tiling comparator).
GMTiling gm_tiling(int path, long long rows_of_pass, int nkeys, int slices) {
  GMTiling t{};
  t.fixed = path == kPathGroupedFixed ? 1 : 0;
  if (t.fixed || slices > 1) {
    t.rows = 64;
  } else {
    const long long per = (rows_of_pass + 255) / 256;
    t.rows = (int)std::min<long long>(64, std::max<long long>(16, (per + 15) / 16 * 16));
  }
  t.max_tiles = (rows_of_pass + t.rows - 1) / t.rows + nkeys;
  return t;
}

RankSortPlan rank_sort_plan(long long P, int k, int K) {
  RankSortPlan s{};
  s.counts2_off = 0;
  s.offsets2_off = (size_t)k * K * sizeof(int32_t);
  const size_t head = align256((size_t)(2 * k * K + 1) * sizeof(int32_t));
  s.perm2_off = head;
  s.w2_off = head + (size_t)P * sizeof(int32_t);
  s.bcnt_off = head + align256((size_t)P * (sizeof(int32_t) + sizeof(float)));
  s.bytes = s.bcnt_off + align256(dispatch_ws_bytes(P, k * K));
  return s;
}

GSRegion gs_region(int path, long long rows_of_pass, int K, int r_pad, int d_in, bool with_hb) {
  GSRegion g{};
  const int kslices = (d_in + kBSlice - 1) / kBSlice;
  const GMTiling tl = gm_tiling(path, rows_of_pass, K, kslices);
  g.nwg = (int)((tl.max_tiles + 15) / 16 * 16);  // tile pairs within each XCD's run
  g.part_bytes = (size_t)g.nwg * kslices * 64 * r_pad * sizeof(float);
  g.hb_off = align256(g.part_bytes);
  g.total = with_hb ? g.hb_off + (size_t)g.nwg * 2 * 64 * r_pad * sizeof(uint16_t) : g.part_bytes;
  return g;
}

bool gm_tuples(int N, int k, int K) { return k > 1 && (long long)N >= 32LL * K * (K + 1); }

TupleSortPlan tuple_sort_plan(int N, int k, int K) {
  TupleSortPlan t{};
  t.m2 = (k + 1) / 2;
  t.kk = K * (K + 1);
  t.nkeys = t.m2 * t.kk;
  t.nb = std::max(1, (N + kTupleWGTokens - 1) / kTupleWGTokens);
  const size_t ent = align256((size_t)t.m2 * N * sizeof(int32_t));
  t.tmax = (N + 15) / 16 + t.kk;
  t.bcnt_off = 0;
  t.toff_off = align256((size_t)t.nb * t.nkeys * sizeof(int32_t));
  t.tiles_off = t.toff_off + align256((size_t)(t.nkeys + 1) * sizeof(int32_t));
  t.ntile_off = t.tiles_off + align256((size_t)t.m2 * t.tmax * 4 * sizeof(int32_t));
  t.etok_off = t.ntile_off + align256((size_t)t.m2 * sizeof(int32_t));
  t.eqa_off = t.etok_off + ent;
  t.eqb_off = t.eqa_off + ent;
  t.bytes = t.eqb_off + ent;
  return t;
}

ApplyPlan apply_plan(int N, int k, int K, int r_pad, int d_in, int d_out, bool y_f32, int path) {
  ApplyPlan a{};
  a.path = apply_resolve_path(N, k, path, K, r_pad);
  const long long P = (long long)N * k;
  const size_t zb = y_f32 ? 0 : (size_t)N * d_out * sizeof(float);
  if (a.path == kPathBlock) {
    a.block_bytes = block_ws_bytes(N, k, K, r_pad, d_in);
    a.total = a.block_bytes;
    return a;
  }
  if (gm_path(a.path, k, K, r_pad)) {
    if (k == 1) {  // one pass over the grouped order
      a.gs_off = 0;
      a.gs = gs_region(a.path, P, K, r_pad, d_in);
      a.total = a.gs.total;
      return a;
    }
    if (gm_tuples(N, k, K)) {
      a.tuples = 1;
      a.gs_off = 0;
      a.gs = gs_region(a.path, P, K, r_pad, d_in, false);  // the shrink over every pair
      a.hq_off = align256(a.gs.total);
      a.hq_bytes = align256((size_t)P * 2 * r_pad * sizeof(uint16_t));
      a.tsort_off = a.hq_off + a.hq_bytes;
      a.tsort = tuple_sort_plan(N, k, K);
      a.z_off = align256(a.tsort_off + a.tsort.bytes);
      a.z_bytes = a.tsort.m2 > 1 ? zb : 0;
      a.total = a.z_off + a.z_bytes;
      return a;
    }
    a.sort_off = 0;
    a.sort = rank_sort_plan(P, k, K);
    a.z_off = a.sort.bytes;
    a.z_bytes = zb;
    a.gs_off = align256(a.z_off + a.z_bytes);  // one pass at a time: N rows each
    a.gs = gs_region(a.path, N, K, r_pad, d_in);
    a.total = a.gs_off + a.gs.total;
    return a;
  }
  if (a.path == kPathTile || (k == 1 && a.path == kPathGrouped)) return a;
  const int ns = a.path == kPathSkinny ? skinny_splits(d_in) : 1;
  a.hpart_off = 0;
  a.hpart_bytes = align256((size_t)ns * (size_t)P * (size_t)r_pad * sizeof(float));
  a.total = a.hpart_bytes;
  if (a.path == kPathSkinny && decode_expand_fits(N, k, K, r_pad)) {  // h rows for the decode expand
    a.hq_off = a.hpart_bytes;
    a.hq_bytes = decode_hq_bytes(P, r_pad);
    a.total = a.hq_off + a.hq_bytes;
  } else if (a.path == kPathSkinny && k > 1 && k * K <= 64) {  // one expand pass per rank of the pairs
    a.sort_off = a.hpart_bytes;
    a.sort = rank_sort_plan(P, k, K);
    a.z_off = a.sort_off + a.sort.bytes;
    a.z_bytes = zb;
    a.total = a.z_off + a.z_bytes;
  }
  return a;
}

size_t apply_ws_bytes(int N, int k, int K, int r_pad, int d_in, int d_out, bool y_f32, int path) {
  return apply_plan(N, k, K, r_pad, d_in, d_out, y_f32, path).total;
}

MultiPlan apply_multi_plan(int n, const int* d_in, const int* d_out, int N, int k, int K, int r_pad, bool y_f32,
                           int path) {
  MultiPlan m{};
  m.path = apply_multi_resolve_path(n, N, k, path, K, r_pad);
  m.decode = m.path == kPathSkinny && decode_expand_fits(N, k, K, r_pad);
  m.fused = m.path == kPathSkinny && (k == 1 || k * K <= 64 || m.decode);
  size_t off = 0;
  if (!m.fused) {
    for (int i = 0; i < n; ++i) {
      m.tgt_off[i] = off;
      off += align256(apply_ws_bytes(N, k, K, r_pad, d_in[i], d_out[i], y_f32, m.path));
    }
    m.total = off;
    return m;
  }
  const long long P = (long long)N * k;
  if (k > 1 && !m.decode) {
    m.sort_off = 0;
    m.sort = rank_sort_plan(P, k, K);
    off = align256(m.sort.bytes);
  }
  for (int i = 0; i < n; ++i) {
    m.tgt_off[i] = off;
    m.hpart_off[i] = off;
    off += align256((size_t)skinny_splits(d_in[i]) * (size_t)P * (size_t)r_pad * sizeof(float));
    if (m.decode) {
      m.hq_off[i] = off;
      off += decode_hq_bytes(P, r_pad);
    } else if (k > 1 && !y_f32) {
      m.z_off[i] = off;
      off += align256((size_t)N * d_out[i] * sizeof(float));
    }
  }
  m.total = off;
  return m;
}

// Pairs per weight-gradient chunk: about 512 workgroups of (chunk, 128 columns), two per
// compute unit, between 256 and 4096 pairs each.  A chunk's fp32 partial (128 x r_pad) costs
// 2 r_pad / Qc of the bf16 rows it reads, written and read once, so chunks stay long.
int wgrad_chunk(long long P, int D) {
  const long long ncb = D / kWCols;
  const long long steps = std::max<long long>(4, std::min<long long>(64, P * ncb / (512LL * kWStep)));
  return (int)(steps * kWStep);
}

BwdPlan bwd_plan(int N, int k, int K, int r_pad, int d_in, int d_out, bool dx_f32, int dx_path) {
  BwdPlan b{};
  const long long P = (long long)N * k;
  b.nsh = 1;  // the split shrink's finalize sums the slices per row
  b.nsg = 1;
  b.Qc = wgrad_chunk(P, std::min(d_in, d_out));
  b.nchunks = (P + b.Qc - 1) / b.Qc + K;
  size_t off = 0;
  b.h_off = off;
  b.h_bytes = align256((size_t)b.nsh * P * r_pad * sizeof(float));
  off += b.h_bytes;
  b.g_off = off;
  b.g_bytes = align256((size_t)b.nsg * P * r_pad * sizeof(float));
  off += b.g_bytes;
  b.gs_off = off;
  b.gs_bytes = P > 0 ? align256(std::max(gs_region(kPathGrouped, P, K, r_pad, d_in, false).part_bytes,
                                         gs_region(kPathGrouped, P, K, r_pad, d_out, false).part_bytes))
                     : 0;
  off += b.gs_bytes;
  b.s_bytes = align256((size_t)b.nchunks * 2 * bwd_s_chunk_elems(r_pad, b.Qc) * sizeof(uint16_t));
  b.sa_off = off;
  off += b.s_bytes;
  b.sb_off = off;
  off += b.s_bytes;
  const int D = std::max(d_in, d_out);
  b.part_off = off;
  b.part_bytes = align256((size_t)b.nchunks * D * r_pad * sizeof(float));
  off += b.part_bytes;
  b.apply_off = off;
  b.apply_bytes = align256(apply_ws_bytes(N, k, K, r_pad, d_out, d_in, dx_f32, dx_path));
  off += b.apply_bytes;
  b.total = off;
  return b;
}

RouterBwdPlan router_bwd_plan(int N, int d, int K) {
  RouterBwdPlan p{};
  p.Qc = wgrad_chunk(N, d);
  p.nchunks = ((long long)N + p.Qc - 1) / p.Qc + 1;
  p.ntb = (N + kRouterTokBlock - 1) / kRouterTokBlock;
  size_t off = 0;
  p.pre_off = off;
  off += align256((size_t)N * kRouterHidden * sizeof(float));
  p.da_off = off;
  off += align256((size_t)N * kRouterHidden * sizeof(float));
  p.s_off = off;
  off += align256((size_t)p.nchunks * 2 * bwd_s_chunk_elems(kRouterHidden, p.Qc) * sizeof(uint16_t));
  p.part_off = off;
  off += align256((size_t)p.nchunks * d * kRouterHidden * sizeof(float));
  p.small_off = off;
  off += align256((size_t)p.ntb * router_small_floats(K) * sizeof(float));
  p.offs_off = off;
  off += 256;
  p.total = off;
  return p;
}

XfPlan xf_plan(int n_seq, int seq_len, int d, int f, size_t lora_bytes) {
  XfPlan p{};
  const size_t N = (size_t)n_seq * seq_len;
  const size_t H = (size_t)d / kXfHeadDim;
  const size_t nd = align256(N * d * sizeof(uint16_t)), nf = align256(N * f * sizeof(uint16_t));
  const size_t ss = (size_t)n_seq * H * seq_len * seq_len;
  size_t off = 0;
  p.h_off = off; off += nd;
  p.q_off = off; off += nd;
  p.k_off = off; off += nd;
  p.v_off = off; off += nd;
  p.att_off = off; off += nd;
  p.o_off = off; off += nd;
  p.g_off = off; off += nf;
  p.u_off = off; off += nf;
  p.s_off = off; off += align256(ss * sizeof(float));
  p.p_off = off; off += align256(ss * sizeof(uint16_t));
  p.lora_off = off;
  p.lora_bytes = align256(lora_bytes);
  off += p.lora_bytes;
  p.blas_off = off;
  p.blas_bytes = kXfBlasBytes;
  off += p.blas_bytes;
  p.total = off;
  return p;
}

}  // namespace molora
