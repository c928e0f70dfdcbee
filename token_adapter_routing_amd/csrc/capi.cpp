// C-ABI entry points: argument validation on the host, hot-set slab layout, launches.
// Every check that can be made without reading device memory is made here, before anything
// is enqueued; kernels then assume valid shapes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <utility>
#include <new>
#include <string>
#include <vector>

#include "molora.h"
#include "molora_launch.h"

static_assert(MOLORA_NOALLOC_SCRATCH_BYTES == molora::kScratchBytes, "scratch size in the header and the library");

struct molora_hotset {
  int K = 0, r = 0, r_pad = 0, layout = 0, n_targets = 0;
  float scale = 1.f;
  bool transposed = false;  // holds (B^T, A^T) of the given adapters (molora_hotset_init_transposed)
  std::vector<molora::TargetDev> tg;
  void* slab = nullptr;
  size_t slab_bytes = 0;
  // host copies of every adapter's slot addresses, [target][adapter] (both layouts)
  std::vector<std::vector<uint16_t*>> slotA, slotB;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MOLORA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOLORA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int rank_pad(int r) { return (r + 15) / 16 * 16; }

// Slot of adapter e in the indirect layout: a fixed permutation of [0, K) so that adapter
// addresses are not an affine function of e.
int indirect_slot(int e, int K) {
  const int mult = (K % 37 == 0) ? 41 : 37;
  return (int)(((long long)e * mult + 11) % K);
}

struct SlabPlan {
  struct T {
    size_t offA, offB, offPA, offPB, sizeA, sizeB;
  };
  std::vector<T> t;
  size_t total = 0;
};

int check_targets(int K, int r, int n_targets, const molora_target* targets, bool need_ptrs) {
  if (K < 1 || K > MOLORA_MAX_ADAPTERS) return fail(MOLORA_ENOTSUP, "K=%d outside [1, %d]", K, MOLORA_MAX_ADAPTERS);
  if (r < 1 || r > MOLORA_MAX_RANK) return fail(MOLORA_ENOTSUP, "r=%d outside [1, %d]", r, MOLORA_MAX_RANK);
  if (n_targets < 1 || n_targets > 16) return fail(MOLORA_EINVAL, "n_targets=%d outside [1, 16]", n_targets);
  if (targets == nullptr) return fail(MOLORA_EINVAL, "targets is NULL");
  for (int t = 0; t < n_targets; ++t) {
    const molora_target& g = targets[t];
    if (g.d_in <= 0 || g.d_out <= 0 || g.d_in % 128 != 0 || g.d_out % 128 != 0)
      return fail(MOLORA_ENOTSUP, "target %d: d_in=%d d_out=%d must be positive multiples of 128", t, g.d_in,
                  g.d_out);
    if (need_ptrs) {
      if (g.A == nullptr || g.B == nullptr) return fail(MOLORA_EINVAL, "target %d: A or B is NULL", t);
      if (!aligned(g.A, 2) || !aligned(g.B, 2)) return fail(MOLORA_EINVAL, "target %d: A or B misaligned", t);
    }
  }
  return MOLORA_OK;
}

SlabPlan plan_slab(int K, int r, int n_targets, const molora_target* targets, int layout) {
  SlabPlan p;
  const int rp = rank_pad(r);
  size_t cur = 0;
  for (int t = 0; t < n_targets; ++t) {
    SlabPlan::T s{};
    s.sizeA = align_up((size_t)rp * targets[t].d_in * 2, 256);
    s.sizeB = align_up((size_t)targets[t].d_out * rp * 2, 256);
    s.offA = cur;
    cur += (size_t)K * s.sizeA;
    s.offB = cur;
    cur += (size_t)K * s.sizeB;
    if (layout == MOLORA_LAYOUT_INDIRECT) {
      s.offPA = cur;
      cur = align_up(cur + (size_t)K * sizeof(void*), 256);
      s.offPB = cur;
      cur = align_up(cur + (size_t)K * sizeof(void*), 256);
    }
    p.t.push_back(s);
  }
  p.total = cur;
  return p;
}

}  // namespace

extern "C" {

const char* molora_last_error(void) { return g_err.c_str(); }

int molora_hotset_bytes(int K, int r, int n_targets, const molora_target* targets, int layout, size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  if (layout != MOLORA_LAYOUT_DIRECT && layout != MOLORA_LAYOUT_INDIRECT)
    return fail(MOLORA_EINVAL, "unknown layout %d", layout);
  const int rc = check_targets(K, r, n_targets, targets, false);
  if (rc != MOLORA_OK) return rc;
  *bytes = plan_slab(K, r, n_targets, targets, layout).total;
  return ok();
}

}  // extern "C"

namespace {

int hotset_init_impl(molora_hotset** out, int K, int r, float scale, int n_targets, const molora_target* targets,
                     int layout, void* slab, size_t slab_bytes, void* stream, bool transposed) {
  if (out == nullptr) return fail(MOLORA_EINVAL, "out is NULL");
  *out = nullptr;
  if (layout != MOLORA_LAYOUT_DIRECT && layout != MOLORA_LAYOUT_INDIRECT)
    return fail(MOLORA_EINVAL, "unknown layout %d", layout);
  int rc = check_targets(K, r, n_targets, targets, true);
  if (rc != MOLORA_OK) return rc;
  if (slab == nullptr || !aligned(slab, 256)) return fail(MOLORA_EINVAL, "slab is NULL or not 256-byte aligned");
  // the slab's own targets: the twin's target t maps d_out -> d_in
  std::vector<molora_target> slab_targets(targets, targets + n_targets);
  if (transposed)
    for (molora_target& g : slab_targets) std::swap(g.d_in, g.d_out);
  const SlabPlan plan = plan_slab(K, r, n_targets, slab_targets.data(), layout);
  if (slab_bytes < plan.total)
    return fail(MOLORA_ENOSPC, "slab holds %zu bytes, %zu needed", slab_bytes, plan.total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  molora_hotset* hs = new (std::nothrow) molora_hotset;
  if (hs == nullptr) return fail(MOLORA_EINVAL, "out of host memory");
  hs->K = K;
  hs->r = r;
  hs->r_pad = rank_pad(r);
  hs->layout = layout;
  hs->n_targets = n_targets;
  hs->scale = scale;
  hs->slab = slab;
  hs->slab_bytes = slab_bytes;
  hs->transposed = transposed;
  char* base = reinterpret_cast<char*>(slab);
  std::vector<std::vector<const void*>> tablesA(n_targets), tablesB(n_targets);
  for (int t = 0; t < n_targets; ++t) {
    const molora_target& g = targets[t];
    const SlabPlan::T& p = plan.t[t];
    molora::TargetDev d{};
    d.d_in = slab_targets[t].d_in;
    d.d_out = slab_targets[t].d_out;
    d.r_pad = hs->r_pad;
    for (int e = 0; e < K; ++e) {
      const int slot = (layout == MOLORA_LAYOUT_DIRECT) ? e : indirect_slot(e, K);
      uint16_t* At = reinterpret_cast<uint16_t*>(base + p.offA + (size_t)slot * p.sizeA);
      uint16_t* Bt = reinterpret_cast<uint16_t*>(base + p.offB + (size_t)slot * p.sizeB);
      const uint16_t* A = reinterpret_cast<const uint16_t*>(g.A) + (size_t)e * g.d_in * r;
      const uint16_t* B = reinterpret_cast<const uint16_t*>(g.B) + (size_t)e * r * g.d_out;
      hipError_t err = molora::launch_relayout(A, B, d.d_in, d.d_out, r, hs->r_pad, At, Bt, s, transposed);
      if (err != hipSuccess) {
        delete hs;
        return hip_fail(err, "hot-set relayout");
      }
      tablesA[t].push_back(At);
      tablesB[t].push_back(Bt);
    }
    if (layout == MOLORA_LAYOUT_DIRECT) {
      d.At = reinterpret_cast<const uint16_t*>(base + p.offA);
      d.Bt = reinterpret_cast<const uint16_t*>(base + p.offB);
      d.strideA = (long long)(p.sizeA / 2);
      d.strideB = (long long)(p.sizeB / 2);
    } else {
      d.ptrA = reinterpret_cast<const uint16_t* const*>(base + p.offPA);
      d.ptrB = reinterpret_cast<const uint16_t* const*>(base + p.offPB);
      hipError_t err = hipMemcpyAsync(base + p.offPA, tablesA[t].data(), (size_t)K * sizeof(void*),
                                      hipMemcpyHostToDevice, s);
      if (err == hipSuccess)
        err = hipMemcpyAsync(base + p.offPB, tablesB[t].data(), (size_t)K * sizeof(void*), hipMemcpyHostToDevice, s);
      if (err != hipSuccess) {
        delete hs;
        return hip_fail(err, "pointer tables");
      }
    }
    hs->tg.push_back(d);
    hs->slotA.emplace_back();
    hs->slotB.emplace_back();
    for (int e = 0; e < K; ++e) {
      hs->slotA.back().push_back(const_cast<uint16_t*>(static_cast<const uint16_t*>(tablesA[t][e])));
      hs->slotB.back().push_back(const_cast<uint16_t*>(static_cast<const uint16_t*>(tablesB[t][e])));
    }
  }
  hipError_t err = hipStreamSynchronize(s);  // host tables above must outlive the copies
  // this device's scratch array (molora_step_vocab_noalloc), looked up once per device here
  if (err == hipSuccess) err = molora::scratch_setup(nullptr);
  if (err != hipSuccess) {
    delete hs;
    return hip_fail(err, "hot-set init");
  }
  *out = hs;
  return ok();
}

}  // namespace

extern "C" {

int molora_hotset_init(molora_hotset** out, int K, int r, float scale, int n_targets, const molora_target* targets,
                       int layout, void* slab, size_t slab_bytes, void* stream) {
  return hotset_init_impl(out, K, r, scale, n_targets, targets, layout, slab, slab_bytes, stream, false);
}

int molora_hotset_init_transposed(molora_hotset** out, int K, int r, float scale, int n_targets,
                                  const molora_target* targets, int layout, void* slab, size_t slab_bytes,
                                  void* stream) {
  return hotset_init_impl(out, K, r, scale, n_targets, targets, layout, slab, slab_bytes, stream, true);
}

int molora_hotset_load(molora_hotset* hs, int target, int e, const void* A, const void* B, void* stream) {
  if (hs == nullptr) return fail(MOLORA_EINVAL, "hs is NULL");
  if (target < 0 || target >= hs->n_targets)
    return fail(MOLORA_EINVAL, "target %d outside [0, %d)", target, hs->n_targets);
  if (e < 0 || e >= hs->K) return fail(MOLORA_EINVAL, "adapter %d outside [0, %d)", e, hs->K);
  if (A == nullptr || B == nullptr) return fail(MOLORA_EINVAL, "A or B is NULL");
  if (!aligned(A, 2) || !aligned(B, 2)) return fail(MOLORA_EINVAL, "misaligned pointer");
  const molora::TargetDev& d = hs->tg[target];
  const hipError_t err =
      molora::launch_relayout(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), d.d_in, d.d_out,
                              hs->r, hs->r_pad, hs->slotA[target][e], hs->slotB[target][e],
                              reinterpret_cast<hipStream_t>(stream), hs->transposed);
  return err == hipSuccess ? ok() : hip_fail(err, "hot-set load");
}

int molora_hotset_destroy(molora_hotset* hs) {
  delete hs;
  return ok();
}

int molora_route_vocab(const int32_t* ids, int N, const int32_t* bounds, int K, int32_t* idx, float* w,
                       void* stream) {
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (K < 1 || K > MOLORA_MAX_ADAPTERS) return fail(MOLORA_ENOTSUP, "K=%d outside [1, %d]", K, MOLORA_MAX_ADAPTERS);
  if (bounds == nullptr) return fail(MOLORA_EINVAL, "bounds is NULL");
  molora::VocabBounds vb{};
  for (int e = 0; e <= K; ++e) {
    vb.b[e] = bounds[e];
    if (e > 0 && bounds[e] < bounds[e - 1]) return fail(MOLORA_EINVAL, "bounds must be non-decreasing");
  }
  if (N == 0) return ok();
  if (ids == nullptr || idx == nullptr || w == nullptr) return fail(MOLORA_EINVAL, "ids, idx or w is NULL");
  if (!aligned(ids, 4) || !aligned(idx, 4) || !aligned(w, 4)) return fail(MOLORA_EINVAL, "misaligned pointer");
  const hipError_t e = molora::launch_route_vocab(ids, N, vb, K, idx, w, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "route_vocab launch");
}

int molora_route_topk_workspace(int N, int d, size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (d <= 0 || d % 128 != 0) return fail(MOLORA_ENOTSUP, "d=%d must be a positive multiple of 128", d);
  *bytes = molora::route_topk_ws_bytes(N, d);
  return ok();
}

int molora_route_topk(const void* x, int N, int d, const void* W1, const float* b1, const void* W2, const float* b2,
                      float* logits, int K, int k, int32_t* idx, float* w, uint8_t* flags, void* ws, size_t ws_bytes,
                      void* stream) {
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (K < 1 || K > MOLORA_MAX_ADAPTERS) return fail(MOLORA_ENOTSUP, "K=%d outside [1, %d]", K, MOLORA_MAX_ADAPTERS);
  if (k < 1 || k > K || k > MOLORA_MAX_TOPK) return fail(MOLORA_ENOTSUP, "k=%d outside [1, min(K, %d)]", k, MOLORA_MAX_TOPK);
  if (W1 != nullptr) {
    if (d <= 0 || d % 128 != 0) return fail(MOLORA_ENOTSUP, "router mode needs d a positive multiple of 128 (d=%d)", d);
    if (W2 == nullptr) return fail(MOLORA_EINVAL, "router mode needs W2");
    if (N > 0 && x == nullptr) return fail(MOLORA_EINVAL, "router mode needs x");
    if (!aligned(W1, 16) || !aligned(W2, 16) || (x != nullptr && !aligned(x, 16)))
      return fail(MOLORA_EINVAL, "x, W1 and W2 must be 16-byte aligned");
    if ((b1 != nullptr && !aligned(b1, 4)) || (b2 != nullptr && !aligned(b2, 4)))
      return fail(MOLORA_EINVAL, "misaligned bias");
  }
  // the split first layer: router mode, a workspace, and d within its range
  float* part = nullptr;
  if (W1 != nullptr && ws != nullptr && molora::router_chunked(d)) {
    const size_t need = molora::route_topk_ws_bytes(N, d);
    if (ws_bytes < need) return fail(MOLORA_ENOSPC, "route_topk workspace %zu < %zu bytes", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(MOLORA_EINVAL, "workspace must be 256-byte aligned");
    part = static_cast<float*>(ws);
  }
  if (N == 0) return ok();
  if (logits == nullptr || idx == nullptr || w == nullptr) return fail(MOLORA_EINVAL, "logits, idx or w is NULL");
  if (!aligned(logits, 4) || !aligned(idx, 4) || !aligned(w, 4)) return fail(MOLORA_EINVAL, "misaligned pointer");
  const hipError_t e = molora::launch_route_topk(
      reinterpret_cast<const uint16_t*>(x), N, d, reinterpret_cast<const uint16_t*>(W1), b1,
      reinterpret_cast<const uint16_t*>(W2), b2, logits, K, k, idx, w, flags, part,
      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "route_topk launch");
}

int molora_dispatch_workspace(int N, int k, int K, size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  if (N < 0 || k < 1 || k > MOLORA_MAX_TOPK) return fail(MOLORA_EINVAL, "bad N=%d or k=%d", N, k);
  if (K < 1 || K > MOLORA_MAX_ADAPTERS) return fail(MOLORA_ENOTSUP, "K=%d outside [1, %d]", K, MOLORA_MAX_ADAPTERS);
  *bytes = molora::dispatch_ws_bytes((long long)N * k, K);
  return ok();
}

int molora_dispatch(const int32_t* idx, const float* w, int N, int k, int K, int32_t* counts, int32_t* offsets,
                    int32_t* perm, float* perm_w, int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (k < 1 || k > MOLORA_MAX_TOPK) return fail(MOLORA_ENOTSUP, "k=%d outside [1, %d]", k, MOLORA_MAX_TOPK);
  if (K < 1 || K > MOLORA_MAX_ADAPTERS) return fail(MOLORA_ENOTSUP, "K=%d outside [1, %d]", K, MOLORA_MAX_ADAPTERS);
  if ((long long)N * k >= (1ll << 31)) return fail(MOLORA_ENOTSUP, "N*k too large");
  if (N == 0) return ok();
  if (idx == nullptr || w == nullptr || counts == nullptr || offsets == nullptr || perm == nullptr || perm_w == nullptr)
    return fail(MOLORA_EINVAL, "a required pointer is NULL");
  if (!aligned(idx, 4) || !aligned(w, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(perm, 4) ||
      !aligned(perm_w, 4) || (inv != nullptr && !aligned(inv, 4)))
    return fail(MOLORA_EINVAL, "misaligned pointer");
  const size_t need = molora::dispatch_ws_bytes((long long)N * k, K);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 4)))
    return fail(MOLORA_ENOSPC, "dispatch workspace of %zu bytes needed, %zu given", need, ws_bytes);
  const hipError_t e = molora::launch_dispatch(idx, w, N * k, K, counts, offsets, perm, perm_w, inv, ws,
                                               reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "dispatch launch");
}

int molora_apply_workspace(const molora_hotset* hs, int target, int N, int k, int y_dtype, int path, size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  if (hs == nullptr) return fail(MOLORA_EINVAL, "hot set is NULL");
  if (target < 0 || target >= hs->n_targets) return fail(MOLORA_EINVAL, "target %d outside [0, %d)", target, hs->n_targets);
  if (N < 0 || k < 1 || k > MOLORA_MAX_TOPK || k > hs->K) return fail(MOLORA_EINVAL, "bad N=%d or k=%d", N, k);
  if (path < MOLORA_PATH_AUTO || path > MOLORA_PATH_GROUPED_FIXED) return fail(MOLORA_EINVAL, "unknown path %d", path);
  if (y_dtype != MOLORA_BF16 && y_dtype != MOLORA_F32) return fail(MOLORA_EINVAL, "unknown dtype");
  *bytes = molora::apply_ws_bytes(N, k, hs->K, hs->r_pad, hs->tg[target].d_in, hs->tg[target].d_out,
                                  y_dtype == MOLORA_F32, path);
  return ok();
}

int molora_apply_path(const molora_hotset* hs, int target, int N, int k, int path, int* resolved) {
  if (resolved == nullptr) return fail(MOLORA_EINVAL, "resolved is NULL");
  if (hs == nullptr) return fail(MOLORA_EINVAL, "hot set is NULL");
  if (target < 0 || target >= hs->n_targets) return fail(MOLORA_EINVAL, "target %d outside [0, %d)", target, hs->n_targets);
  if (N < 0 || k < 1 || k > MOLORA_MAX_TOPK || k > hs->K) return fail(MOLORA_EINVAL, "bad N=%d or k=%d", N, k);
  if (path < MOLORA_PATH_AUTO || path > MOLORA_PATH_GROUPED_FIXED) return fail(MOLORA_EINVAL, "unknown path %d", path);
  *resolved = molora::apply_resolve_path(N, k, path, hs->K, hs->r_pad);
  return ok();
}

int molora_apply(const molora_hotset* hs, int target, const void* x, const void* y0, int y0_dtype, void* y, int y_dtype,
                 int N, int k, const int32_t* offsets, const int32_t* perm, const float* perm_w, const int32_t* inv,
                 int path, void* ws, size_t ws_bytes, void* stream) {
  if (hs == nullptr) return fail(MOLORA_EINVAL, "hot set is NULL");
  if (target < 0 || target >= hs->n_targets) return fail(MOLORA_EINVAL, "target %d outside [0, %d)", target, hs->n_targets);
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (k < 1 || k > MOLORA_MAX_TOPK || k > hs->K) return fail(MOLORA_ENOTSUP, "k=%d outside [1, min(K, %d)]", k, MOLORA_MAX_TOPK);
  if ((long long)N * k >= (1ll << 31)) return fail(MOLORA_ENOTSUP, "N*k too large");
  if ((y0_dtype != MOLORA_BF16 && y0_dtype != MOLORA_F32) || (y_dtype != MOLORA_BF16 && y_dtype != MOLORA_F32))
    return fail(MOLORA_EINVAL, "unknown dtype");
  if (path < MOLORA_PATH_AUTO || path > MOLORA_PATH_GROUPED_FIXED) return fail(MOLORA_EINVAL, "unknown path %d", path);
  if ((path == MOLORA_PATH_TILE || path == MOLORA_PATH_BLOCK) && hs->K > molora::kApplyTileMaxAdapters)
    return fail(MOLORA_ENOTSUP, "the tile and block paths support K <= %d", molora::kApplyTileMaxAdapters);
  if (y0 == y && y0_dtype != y_dtype) return fail(MOLORA_EINVAL, "in-place apply needs y0_dtype == y_dtype");
  if (N == 0) return ok();
  if (x == nullptr || y0 == nullptr || y == nullptr) return fail(MOLORA_EINVAL, "x, y0 or y is NULL");
  if (!aligned(x, 16) || !aligned(y0, 16) || !aligned(y, 16)) return fail(MOLORA_EINVAL, "x, y0 and y must be 16-byte aligned");
  if (offsets == nullptr || perm == nullptr || perm_w == nullptr || inv == nullptr)
    return fail(MOLORA_EINVAL, "offsets, perm, perm_w and inv are required");
  if (!aligned(offsets, 4) || !aligned(perm, 4) || !aligned(perm_w, 4) || !aligned(inv, 4))
    return fail(MOLORA_EINVAL, "misaligned pointer");
  const molora::TargetDev& tg = hs->tg[target];
  const size_t need = molora::apply_ws_bytes(N, k, hs->K, hs->r_pad, tg.d_in, tg.d_out, y_dtype == MOLORA_F32, path);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 16)))
    return fail(MOLORA_ENOSPC, "workspace of %zu bytes (16-byte aligned) needed, %zu given", need, ws_bytes);
  molora::ApplyLaunch a{};
  a.tgt = tg;
  a.indirect = hs->layout == MOLORA_LAYOUT_INDIRECT;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.y0 = y0;
  a.y = y;
  a.y0_f32 = y0_dtype == MOLORA_F32;
  a.y_f32 = y_dtype == MOLORA_F32;
  a.N = N;
  a.k = k;
  a.K = hs->K;
  a.scale = hs->scale;
  a.offsets = offsets;
  a.perm = perm;
  a.perm_w = perm_w;
  a.inv = inv;
  a.path = molora::apply_resolve_path(N, k, path, hs->K, hs->r_pad);
  a.ws = reinterpret_cast<float*>(ws);
  a.col_groups = 0;
  const hipError_t e = molora::launch_apply(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "apply launch");
}

static int check_multi_targets(const molora_hotset* hs, int n, const int* targets, int* d_in, int* d_out) {
  if (hs == nullptr) return fail(MOLORA_EINVAL, "hot set is NULL");
  if (n < 1 || n > molora::kApplyMaxMulti) return fail(MOLORA_ENOTSUP, "n=%d outside [1, %d]", n, molora::kApplyMaxMulti);
  if (targets == nullptr) return fail(MOLORA_EINVAL, "targets is NULL");
  for (int i = 0; i < n; ++i) {
    if (targets[i] < 0 || targets[i] >= hs->n_targets)
      return fail(MOLORA_EINVAL, "targets[%d]=%d outside [0, %d)", i, targets[i], hs->n_targets);
    d_in[i] = hs->tg[targets[i]].d_in;
    d_out[i] = hs->tg[targets[i]].d_out;
  }
  return MOLORA_OK;
}

int molora_apply_multi_workspace(const molora_hotset* hs, int n, const int* targets, int N, int k, int y_dtype,
                                 int path, size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  int d_in[molora::kApplyMaxMulti], d_out[molora::kApplyMaxMulti];
  const int rc = check_multi_targets(hs, n, targets, d_in, d_out);
  if (rc != MOLORA_OK) return rc;
  if (N < 0 || k < 1 || k > MOLORA_MAX_TOPK || k > hs->K) return fail(MOLORA_EINVAL, "bad N=%d or k=%d", N, k);
  if (path < MOLORA_PATH_AUTO || path > MOLORA_PATH_GROUPED_FIXED) return fail(MOLORA_EINVAL, "unknown path %d", path);
  if (y_dtype != MOLORA_BF16 && y_dtype != MOLORA_F32) return fail(MOLORA_EINVAL, "unknown dtype");
  *bytes = molora::apply_multi_plan(n, d_in, d_out, N, k, hs->K, hs->r_pad, y_dtype == MOLORA_F32, path).total;
  return ok();
}

// Arguments of an n-target apply other than the routing arrays and the workspace; fills the
// launch records (routing and workspace pointers left for the caller).  *empty: N == 0.
static int check_multi_io(const molora_hotset* hs, int n, const int* targets, const void* const* x,
                          const void* const* y0, int y0_dtype, void* const* y, int y_dtype, int N, int k, int path,
                          int* d_in, int* d_out, molora::ApplyLaunch* as, bool* empty) {
  const int rc = check_multi_targets(hs, n, targets, d_in, d_out);
  if (rc != MOLORA_OK) return rc;
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (k < 1 || k > MOLORA_MAX_TOPK || k > hs->K) return fail(MOLORA_ENOTSUP, "k=%d outside [1, min(K, %d)]", k, MOLORA_MAX_TOPK);
  if ((long long)N * k >= (1ll << 31)) return fail(MOLORA_ENOTSUP, "N*k too large");
  if ((y0_dtype != MOLORA_BF16 && y0_dtype != MOLORA_F32) || (y_dtype != MOLORA_BF16 && y_dtype != MOLORA_F32))
    return fail(MOLORA_EINVAL, "unknown dtype");
  if (path < MOLORA_PATH_AUTO || path > MOLORA_PATH_GROUPED_FIXED) return fail(MOLORA_EINVAL, "unknown path %d", path);
  if ((path == MOLORA_PATH_TILE || path == MOLORA_PATH_BLOCK) && hs->K > molora::kApplyTileMaxAdapters)
    return fail(MOLORA_ENOTSUP, "the tile and block paths support K <= %d", molora::kApplyTileMaxAdapters);
  if (x == nullptr || y0 == nullptr || y == nullptr) return fail(MOLORA_EINVAL, "x, y0 or y array is NULL");
  *empty = N == 0;
  if (N == 0) return MOLORA_OK;
  for (int i = 0; i < n; ++i) {
    if (x[i] == nullptr || y0[i] == nullptr || y[i] == nullptr) return fail(MOLORA_EINVAL, "x, y0 or y [%d] is NULL", i);
    if (!aligned(x[i], 16) || !aligned(y0[i], 16) || !aligned(y[i], 16))
      return fail(MOLORA_EINVAL, "x, y0 and y [%d] must be 16-byte aligned", i);
    if (y0[i] == y[i] && y0_dtype != y_dtype) return fail(MOLORA_EINVAL, "in-place apply needs y0_dtype == y_dtype");
    for (int j = 0; j < i; ++j)
      if (targets[j] == targets[i] || y[j] == y[i]) return fail(MOLORA_EINVAL, "targets and outputs must be distinct");
  }
  const int rp = molora::apply_multi_resolve_path(n, N, k, path, hs->K, hs->r_pad);
  for (int i = 0; i < n; ++i) {
    molora::ApplyLaunch& a = as[i];
    a = molora::ApplyLaunch{};
    a.tgt = hs->tg[targets[i]];
    a.indirect = hs->layout == MOLORA_LAYOUT_INDIRECT;
    a.x = reinterpret_cast<const uint16_t*>(x[i]);
    a.y0 = y0[i];
    a.y = y[i];
    a.y0_f32 = y0_dtype == MOLORA_F32;
    a.y_f32 = y_dtype == MOLORA_F32;
    a.N = N;
    a.k = k;
    a.K = hs->K;
    a.scale = hs->scale;
    a.path = rp;
    a.col_groups = 0;
  }
  return MOLORA_OK;
}

int molora_apply_multi(const molora_hotset* hs, int n, const int* targets, const void* const* x,
                       const void* const* y0, int y0_dtype, void* const* y, int y_dtype, int N, int k,
                       const int32_t* offsets, const int32_t* perm, const float* perm_w, const int32_t* inv, int path,
                       void* ws, size_t ws_bytes, void* stream) {
  int d_in[molora::kApplyMaxMulti], d_out[molora::kApplyMaxMulti];
  molora::ApplyLaunch as[molora::kApplyMaxMulti];
  bool empty = false;
  const int rc = check_multi_io(hs, n, targets, x, y0, y0_dtype, y, y_dtype, N, k, path, d_in, d_out, as, &empty);
  if (rc != MOLORA_OK || empty) return rc == MOLORA_OK ? ok() : rc;
  if (offsets == nullptr || perm == nullptr || perm_w == nullptr || inv == nullptr)
    return fail(MOLORA_EINVAL, "offsets, perm, perm_w and inv are required");
  if (!aligned(offsets, 4) || !aligned(perm, 4) || !aligned(perm_w, 4) || !aligned(inv, 4))
    return fail(MOLORA_EINVAL, "misaligned pointer");
  const size_t need =
      molora::apply_multi_plan(n, d_in, d_out, N, k, hs->K, hs->r_pad, y_dtype == MOLORA_F32, path).total;
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 256)))
    return fail(MOLORA_ENOSPC, "workspace of %zu bytes (256-byte aligned) needed, %zu given", need, ws_bytes);
  for (int i = 0; i < n; ++i) {
    as[i].offsets = offsets;
    as[i].perm = perm;
    as[i].perm_w = perm_w;
    as[i].inv = inv;
    as[i].ws = reinterpret_cast<float*>(ws);
  }
  const hipError_t e = molora::launch_apply_multi(as, n, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "apply launch");
}

int molora_dispatch_apply_multi_workspace(const molora_hotset* hs, int n, const int* targets, int N, int k,
                                          int y_dtype, int path, size_t* bytes) {
  size_t apply_bytes = 0;
  const int rc = molora_apply_multi_workspace(hs, n, targets, N, k, y_dtype, path, &apply_bytes);
  if (rc != MOLORA_OK) return rc;
  *bytes = molora::align256(apply_bytes) + molora::dispatch_ws_bytes((long long)N * k, hs->K);
  return ok();
}

int molora_dispatch_apply_multi(const molora_hotset* hs, int n, const int* targets, const void* const* x,
                                const void* const* y0, int y0_dtype, void* const* y, int y_dtype, int N, int k,
                                const int32_t* idx, const float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                                float* perm_w, int32_t* inv, int path, void* ws, size_t ws_bytes, void* stream) {
  int d_in[molora::kApplyMaxMulti], d_out[molora::kApplyMaxMulti];
  molora::ApplyLaunch as[molora::kApplyMaxMulti];
  bool empty = false;
  const int rc = check_multi_io(hs, n, targets, x, y0, y0_dtype, y, y_dtype, N, k, path, d_in, d_out, as, &empty);
  if (rc != MOLORA_OK || empty) return rc == MOLORA_OK ? ok() : rc;
  if (idx == nullptr || w == nullptr || counts == nullptr || offsets == nullptr || perm == nullptr ||
      perm_w == nullptr || inv == nullptr)
    return fail(MOLORA_EINVAL, "idx, w, counts, offsets, perm, perm_w and inv are required");
  if (!aligned(idx, 4) || !aligned(w, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(perm, 4) ||
      !aligned(perm_w, 4) || !aligned(inv, 4))
    return fail(MOLORA_EINVAL, "misaligned pointer");
  const long long P = (long long)N * k;
  const molora::MultiPlan mp =
      molora::apply_multi_plan(n, d_in, d_out, N, k, hs->K, hs->r_pad, y_dtype == MOLORA_F32, path);
  const size_t disp_off = molora::align256(mp.total);
  const size_t need = disp_off + molora::dispatch_ws_bytes(P, hs->K);
  if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned(ws, 256)))
    return fail(MOLORA_ENOSPC, "workspace of %zu bytes (256-byte aligned) needed, %zu given", need, ws_bytes);
  for (int i = 0; i < n; ++i) {
    as[i].offsets = offsets;
    as[i].perm = perm;
    as[i].perm_w = perm_w;
    as[i].inv = inv;
    as[i].ws = reinterpret_cast<float*>(ws);
  }
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (as[0].path == MOLORA_PATH_BLOCK) {
    // small hot sets: the dispatch rides in the block shrink's launch, which reads the routing
    // as given
    const molora::DenseFuse f{idx, w, counts, offsets, perm, perm_w, inv};
    bool taken = false;
    const hipError_t e = molora::launch_dense_block(as, n, mp.tgt_off, s, &taken, &f);
    if (e != hipSuccess) return hip_fail(e, "dispatch + apply launch");
    if (taken) return ok();
  }
  char* dws = need > disp_off ? static_cast<char*>(ws) + disp_off : nullptr;
  hipError_t e = molora::launch_dispatch(idx, w, (int)P, hs->K, counts, offsets, perm, perm_w, inv, dws, s);
  if (e != hipSuccess) return hip_fail(e, "dispatch launch");
  e = molora::launch_apply_multi(as, n, s);
  return e == hipSuccess ? ok() : hip_fail(e, "apply launch");
}

int molora_step_workspace(const molora_hotset* hs, int target, int N, size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  if (hs == nullptr) return fail(MOLORA_EINVAL, "hot set is NULL");
  if (target < 0 || target >= hs->n_targets) return fail(MOLORA_EINVAL, "target %d outside [0, %d)", target, hs->n_targets);
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  *bytes = molora::step_plan(N, hs->K, hs->r_pad, hs->tg[target].d_in).total;
  return ok();
}

int molora_step_vocab(const molora_hotset* hs, int target, const int32_t* ids, int N, const int32_t* bounds,
                      const void* x, const void* y0, int y0_dtype, void* y, int y_dtype, int32_t* idx, float* w,
                      int32_t* counts, int32_t* offsets, int32_t* perm, float* perm_w, int32_t* inv, void* ws,
                      size_t ws_bytes, void* stream) {
  if (hs == nullptr) return fail(MOLORA_EINVAL, "hot set is NULL");
  if (target < 0 || target >= hs->n_targets) return fail(MOLORA_EINVAL, "target %d outside [0, %d)", target, hs->n_targets);
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (hs->K > molora::kApplyTileMaxAdapters)
    return fail(MOLORA_ENOTSUP, "the one-launch step supports K <= %d", molora::kApplyTileMaxAdapters);
  if (bounds == nullptr) return fail(MOLORA_EINVAL, "bounds is NULL");
  molora::StepVocabLaunch st{};
  for (int e = 0; e <= hs->K; ++e) {
    st.bounds.b[e] = bounds[e];
    if (e > 0 && bounds[e] < bounds[e - 1]) return fail(MOLORA_EINVAL, "bounds must be non-decreasing");
  }
  if ((y0_dtype != MOLORA_BF16 && y0_dtype != MOLORA_F32) || (y_dtype != MOLORA_BF16 && y_dtype != MOLORA_F32))
    return fail(MOLORA_EINVAL, "unknown dtype");
  if (y0 == y && y0_dtype != y_dtype) return fail(MOLORA_EINVAL, "in-place step needs y0_dtype == y_dtype");
  if (N == 0) return ok();
  if (ids == nullptr || x == nullptr || y0 == nullptr || y == nullptr || idx == nullptr || w == nullptr ||
      counts == nullptr || offsets == nullptr || perm == nullptr || perm_w == nullptr || inv == nullptr)
    return fail(MOLORA_EINVAL, "a required pointer is NULL");
  if (!aligned(x, 16) || !aligned(y0, 16) || !aligned(y, 16)) return fail(MOLORA_EINVAL, "x, y0 and y must be 16-byte aligned");
  if (!aligned(ids, 4) || !aligned(idx, 4) || !aligned(w, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(perm, 4) || !aligned(perm_w, 4) || !aligned(inv, 4))
    return fail(MOLORA_EINVAL, "misaligned pointer");
  const molora::StepPlan plan = molora::step_plan(N, hs->K, hs->r_pad, hs->tg[target].d_in);
  if (ws != nullptr && (ws_bytes < plan.total || !aligned(ws, 256)))
    return fail(MOLORA_ENOSPC, "step workspace of %zu bytes (256-byte aligned) needed, %zu given", plan.total, ws_bytes);
  molora::ApplyLaunch& a = st.apply;
  a.tgt = hs->tg[target];
  a.indirect = hs->layout == MOLORA_LAYOUT_INDIRECT;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.y0 = y0;
  a.y = y;
  a.y0_f32 = y0_dtype == MOLORA_F32;
  a.y_f32 = y_dtype == MOLORA_F32;
  a.N = N;
  a.k = 1;
  a.K = hs->K;
  a.scale = hs->scale;
  a.offsets = offsets;
  a.perm = perm;
  a.perm_w = perm_w;
  a.inv = inv;
  a.path = molora::kPathTile;
  a.ws = nullptr;
  a.col_groups = 0;
  st.part = ws != nullptr ? reinterpret_cast<float*>(static_cast<char*>(ws) + plan.part_off) : nullptr;
  st.bcnt = ws != nullptr ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + plan.cnt_off) : nullptr;
  st.dispatch_share = true;
  st.ids = ids;
  st.idx = idx;
  st.w = w;
  st.counts = counts;
  st.offsets = offsets;
  st.perm = perm;
  st.perm_w = perm_w;
  st.inv = inv;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N <= molora::kStepMaxN) {  // one or two launches that also route and write the dispatch outputs
    const hipError_t e = molora::launch_step_vocab(st, s);
    return e == hipSuccess ? ok() : hip_fail(e, "step launch");
  }
  // Above kStepMaxN tokens the routing and the dispatch run as launches of their own (chip-wide
  // with a workspace, else one workgroup); then the split launches apply (same arithmetic, so y
  // is bit-identical at every N), or, without a workspace, the tile path.
  char* wsb = static_cast<char*>(ws);
  void* dws = (ws != nullptr && plan.disp_bytes > 0) ? wsb + plan.disp_off : nullptr;
  hipError_t e = molora::launch_route_vocab(ids, N, st.bounds, hs->K, idx, w, s);
  if (e == hipSuccess) e = molora::launch_dispatch(idx, w, N, hs->K, counts, offsets, perm, perm_w, inv, dws, s);
  if (e == hipSuccess) {
    if (ws != nullptr) {
      st.part = reinterpret_cast<float*>(wsb + plan.part_off);
      st.bcnt = nullptr;
      st.dispatch_share = false;
      e = molora::launch_step_vocab(st, s);
    } else {
      e = molora::launch_apply(a, s);
    }
  }
  return e == hipSuccess ? ok() : hip_fail(e, "step launch");
}

int molora_step_vocab_noalloc(const molora_hotset* hs, int target, const int32_t* ids, int N, const int32_t* bounds,
                              const void* x, const void* y0, int y0_dtype, void* y, int y_dtype, int32_t* idx,
                              float* w, int32_t* counts, int32_t* offsets, int32_t* perm, float* perm_w,
                              int32_t* inv, void* stream) {
  if (hs == nullptr) return fail(MOLORA_EINVAL, "hot set is NULL");
  if (target < 0 || target >= hs->n_targets) return fail(MOLORA_EINVAL, "target %d outside [0, %d)", target, hs->n_targets);
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  const molora::StepPlan plan = molora::step_plan(N, hs->K, hs->r_pad, hs->tg[target].d_in);
  if (plan.total > molora::kScratchBytes)
    return fail(MOLORA_ENOSPC, "this step needs %zu bytes of scratch; the allocation-free step holds %zu", plan.total,
                molora::kScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = molora::scratch_setup(&scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch lookup");
  return molora_step_vocab(hs, target, ids, N, bounds, x, y0, y0_dtype, y, y_dtype, idx, w, counts, offsets, perm,
                           perm_w, inv, scratch, molora::kScratchBytes, stream);
}

namespace {

// Checks shared by molora_backward_workspace and molora_backward.
int check_backward_pair(const molora_hotset* hs, const molora_hotset* hs_t, int target, int N, int k) {
  if (hs == nullptr || hs_t == nullptr) return fail(MOLORA_EINVAL, "hot set is NULL");
  if (hs->transposed || !hs_t->transposed)
    return fail(MOLORA_EINVAL, "hs must be a forward hot set and hs_t one built by molora_hotset_init_transposed");
  if (hs->K != hs_t->K || hs->r != hs_t->r || hs->n_targets != hs_t->n_targets || hs->scale != hs_t->scale)
    return fail(MOLORA_EINVAL, "hs and hs_t differ in K, r, targets or scale");
  if (target < 0 || target >= hs->n_targets) return fail(MOLORA_EINVAL, "target %d outside [0, %d)", target, hs->n_targets);
  if (hs->tg[target].d_in != hs_t->tg[target].d_out || hs->tg[target].d_out != hs_t->tg[target].d_in)
    return fail(MOLORA_EINVAL, "hs_t's target %d is not the transpose of hs's", target);
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (k < 1 || k > MOLORA_MAX_TOPK || k > hs->K) return fail(MOLORA_ENOTSUP, "k=%d outside [1, min(K, %d)]", k, MOLORA_MAX_TOPK);
  if ((long long)N * k >= (1ll << 31)) return fail(MOLORA_ENOTSUP, "N*k too large");
  return MOLORA_OK;
}

molora::BwdPlan backward_plan(const molora_hotset* hs, int target, int N, int k, bool dx_f32, int* dx_path) {
  const molora::TargetDev& tg = hs->tg[target];
  const int path = molora::apply_resolve_path(N, k, MOLORA_PATH_AUTO, hs->K, hs->r_pad);
  if (dx_path != nullptr) *dx_path = path;
  return molora::bwd_plan(N, k, hs->K, hs->r_pad, tg.d_in, tg.d_out, dx_f32, path);
}

}  // namespace

int molora_backward_workspace(const molora_hotset* hs, const molora_hotset* hs_t, int target, int N, int k,
                              int dx_dtype, size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  const int rc = check_backward_pair(hs, hs_t, target, N, k);
  if (rc != MOLORA_OK) return rc;
  if (dx_dtype != MOLORA_BF16 && dx_dtype != MOLORA_F32) return fail(MOLORA_EINVAL, "unknown dtype");
  *bytes = backward_plan(hs, target, N, k, dx_dtype == MOLORA_F32, nullptr).total;
  return ok();
}

int molora_backward(const molora_hotset* hs, const molora_hotset* hs_t, int target, const void* x, const void* gy,
                    const void* dx0, int dx0_dtype, void* dx, int dx_dtype, int N, int k, const int32_t* offsets,
                    const int32_t* perm, const float* perm_w, const int32_t* inv, float* dA, float* dB, float* dw,
                    void* ws, size_t ws_bytes, void* stream) {
  int rc = check_backward_pair(hs, hs_t, target, N, k);
  if (rc != MOLORA_OK) return rc;
  if ((dx0_dtype != MOLORA_BF16 && dx0_dtype != MOLORA_F32) || (dx_dtype != MOLORA_BF16 && dx_dtype != MOLORA_F32))
    return fail(MOLORA_EINVAL, "unknown dtype");
  if (dx != nullptr && dx0 == dx && dx0_dtype != dx_dtype) return fail(MOLORA_EINVAL, "in-place dx needs dx0_dtype == dx_dtype");
  if (dx == nullptr && dA == nullptr && dB == nullptr && dw == nullptr)
    return fail(MOLORA_EINVAL, "dx, dA, dB and dw are all NULL");
  if ((dA != nullptr && !aligned(dA, 4)) || (dB != nullptr && !aligned(dB, 4)) || (dw != nullptr && !aligned(dw, 4)))
    return fail(MOLORA_EINVAL, "misaligned pointer");
  const bool any_pairs = N > 0;
  if (any_pairs) {
    if (x == nullptr || gy == nullptr) return fail(MOLORA_EINVAL, "x or gy is NULL");
    if (!aligned(x, 16) || !aligned(gy, 16)) return fail(MOLORA_EINVAL, "x and gy must be 16-byte aligned");
    if (offsets == nullptr || perm == nullptr || perm_w == nullptr || inv == nullptr)
      return fail(MOLORA_EINVAL, "offsets, perm, perm_w and inv are required");
    if (!aligned(offsets, 4) || !aligned(perm, 4) || !aligned(perm_w, 4) || !aligned(inv, 4))
      return fail(MOLORA_EINVAL, "misaligned pointer");
    if (dx != nullptr && (dx0 == nullptr || !aligned(dx0, 16) || !aligned(dx, 16)))
      return fail(MOLORA_EINVAL, "dx needs dx0; both 16-byte aligned");
  } else if ((dA != nullptr || dB != nullptr) && offsets == nullptr) {
    return fail(MOLORA_EINVAL, "offsets is required");
  }
  int dx_path = 0;
  const molora::BwdPlan plan = backward_plan(hs, target, N, k, dx_dtype == MOLORA_F32, &dx_path);
  const bool need_ws = any_pairs || dA != nullptr || dB != nullptr;
  if (need_ws && (ws == nullptr || ws_bytes < plan.total || !aligned(ws, 256)))
    return fail(MOLORA_ENOSPC, "workspace of %zu bytes (256-byte aligned) needed, %zu given", plan.total, ws_bytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* wsb = reinterpret_cast<char*>(ws);
  if (dx != nullptr && any_pairs) {
    molora::ApplyLaunch a{};
    a.tgt = hs_t->tg[target];
    a.indirect = hs_t->layout == MOLORA_LAYOUT_INDIRECT;
    a.x = reinterpret_cast<const uint16_t*>(gy);
    a.y0 = dx0;
    a.y = dx;
    a.y0_f32 = dx0_dtype == MOLORA_F32;
    a.y_f32 = dx_dtype == MOLORA_F32;
    a.N = N;
    a.k = k;
    a.K = hs->K;
    a.scale = hs->scale;
    a.offsets = offsets;
    a.perm = perm;
    a.perm_w = perm_w;
    a.inv = inv;
    a.path = dx_path;
    a.ws = reinterpret_cast<float*>(wsb + plan.apply_off);
    a.col_groups = 0;
    const hipError_t e = molora::launch_apply(a, s);
    if (e != hipSuccess) return hip_fail(e, "backward dx launch");
  }
  if (dA == nullptr && dB == nullptr && dw == nullptr) return ok();
  molora::BackwardLaunch b{};
  b.tgt = hs->tg[target];
  b.tgt_t = hs_t->tg[target];
  b.indirect = hs->layout == MOLORA_LAYOUT_INDIRECT;
  b.indirect_t = hs_t->layout == MOLORA_LAYOUT_INDIRECT;
  b.x = reinterpret_cast<const uint16_t*>(x);
  b.gy = reinterpret_cast<const uint16_t*>(gy);
  b.offsets = offsets;
  b.perm = perm;
  b.perm_w = perm_w;
  b.inv = inv;
  b.N = N;
  b.k = k;
  b.K = hs->K;
  b.r = hs->r;
  b.scale = hs->scale;
  b.dA = dA;
  b.dB = dB;
  b.dw = dw;
  b.ws = wsb;
  b.dx_f32 = dx_dtype == MOLORA_F32;
  b.dx_path = dx_path;
  const hipError_t e = molora::launch_backward(b, s);
  return e == hipSuccess ? ok() : hip_fail(e, "backward launch");
}

int molora_route_topk_backward(const int32_t* idx, const float* w, const float* dw, int N, int K, int k,
                               float* dlogits, void* stream) {
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (K < 1 || K > MOLORA_MAX_ADAPTERS) return fail(MOLORA_ENOTSUP, "K=%d outside [1, %d]", K, MOLORA_MAX_ADAPTERS);
  if (k < 1 || k > K || k > MOLORA_MAX_TOPK) return fail(MOLORA_ENOTSUP, "k=%d outside [1, min(K, %d)]", k, MOLORA_MAX_TOPK);
  if (N == 0) return ok();
  if (idx == nullptr || w == nullptr || dw == nullptr || dlogits == nullptr)
    return fail(MOLORA_EINVAL, "idx, w, dw or dlogits is NULL");
  if (!aligned(idx, 4) || !aligned(w, 4) || !aligned(dw, 4) || !aligned(dlogits, 4))
    return fail(MOLORA_EINVAL, "misaligned pointer");
  const hipError_t e = molora::launch_route_topk_backward(idx, w, dw, N, K, k, dlogits, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "route_topk_backward launch");
}

int molora_router_backward_workspace(int N, int d, int K, size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (d <= 0 || d % 128 != 0) return fail(MOLORA_ENOTSUP, "d=%d must be a positive multiple of 128", d);
  if (K < 1 || K > MOLORA_MAX_ADAPTERS) return fail(MOLORA_ENOTSUP, "K=%d outside [1, %d]", K, MOLORA_MAX_ADAPTERS);
  *bytes = molora::router_bwd_plan(N, d, K).total;
  return ok();
}

int molora_router_backward(const void* x, int N, int d, const void* W1, const float* b1, const void* W2, int K,
                           const float* dlogits, float* dW1, float* db1, float* dW2, float* db2, const float* dx0,
                           float* dx, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  int rc = molora_router_backward_workspace(N, d, K, &need);
  if (rc != MOLORA_OK) return rc;
  if (dW1 == nullptr && db1 == nullptr && dW2 == nullptr && db2 == nullptr && dx == nullptr)
    return fail(MOLORA_EINVAL, "every output is NULL");
  if (W1 == nullptr || W2 == nullptr) return fail(MOLORA_EINVAL, "W1 or W2 is NULL");
  if (!aligned(W1, 16) || !aligned(W2, 16)) return fail(MOLORA_EINVAL, "W1 and W2 must be 16-byte aligned");
  if (N > 0) {
    if (x == nullptr || dlogits == nullptr) return fail(MOLORA_EINVAL, "x or dlogits is NULL");
    if (!aligned(x, 16) || !aligned(dlogits, 4)) return fail(MOLORA_EINVAL, "misaligned x or dlogits");
  }
  if ((b1 != nullptr && !aligned(b1, 4)) || (dW1 != nullptr && !aligned(dW1, 4)) || (db1 != nullptr && !aligned(db1, 4)) ||
      (dW2 != nullptr && !aligned(dW2, 4)) || (db2 != nullptr && !aligned(db2, 4)) || (dx0 != nullptr && !aligned(dx0, 8)) ||
      (dx != nullptr && !aligned(dx, 8)))
    return fail(MOLORA_EINVAL, "misaligned pointer");
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(MOLORA_ENOSPC, "workspace of %zu bytes (256-byte aligned) needed, %zu given", need, ws_bytes);
  molora::RouterBackwardLaunch a{};
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.N = N;
  a.d = d;
  a.K = K;
  a.W1 = reinterpret_cast<const uint16_t*>(W1);
  a.b1 = b1;
  a.W2 = reinterpret_cast<const uint16_t*>(W2);
  a.dl = dlogits;
  a.dW1 = dW1;
  a.db1 = db1;
  a.dW2 = dW2;
  a.db2 = db2;
  a.dx0 = dx0;
  a.dx = dx;
  a.ws = reinterpret_cast<char*>(ws);
  const hipError_t e = molora::launch_router_backward(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "router_backward launch");
}

namespace {

// Shapes of the decoder's seven LoRA targets (q, k, v, o, gate, up, down).
void xf_dims(int d, int f, int* din, int* dout) {
  const int di[molora::kXfTargets] = {d, d, d, d, d, d, f};
  const int dn[molora::kXfTargets] = {d, d, d, d, f, f, d};
  for (int t = 0; t < molora::kXfTargets; ++t) {
    din[t] = di[t];
    dout[t] = dn[t];
  }
}

// Validates the model description; on success *K is the adapters per target (0: no layer
// has LoRA) and *lora_bytes the largest workspace of one layer's applies.
int xf_check(int d, int f, int n_layers, const molora_xf_layer* layers, int n_seq, int seq_len, int k, int* K,
             size_t* lora_bytes, int* paths) {
  if (d <= 0 || f <= 0 || d % 128 != 0 || f % 128 != 0)
    return fail(MOLORA_ENOTSUP, "d=%d and f=%d must be positive multiples of 128", d, f);
  if (n_layers < 1 || n_layers > 1024 || layers == nullptr) return fail(MOLORA_EINVAL, "n_layers=%d or layers", n_layers);
  if (n_seq < 1 || seq_len < 1) return fail(MOLORA_EINVAL, "n_seq=%d seq_len=%d", n_seq, seq_len);
  const long long N = (long long)n_seq * seq_len;
  if (N * std::max(d, f) >= (1ll << 31) || (long long)n_seq * (d / 128) * seq_len * (long long)seq_len >= (1ll << 31))
    return fail(MOLORA_ENOTSUP, "batch too large");
  if (k < 1 || k > MOLORA_MAX_TOPK) return fail(MOLORA_ENOTSUP, "k=%d outside [1, %d]", k, MOLORA_MAX_TOPK);
  int din[molora::kXfTargets], dout[molora::kXfTargets];
  xf_dims(d, f, din, dout);
  *K = 0;
  *lora_bytes = 0;
  for (int l = 0; l < n_layers; ++l) {
    const molora_xf_layer& L = layers[l];
    if (L.norm1 == nullptr || L.norm2 == nullptr || !aligned(L.norm1, 16) || !aligned(L.norm2, 16))
      return fail(MOLORA_EINVAL, "layer %d: norm weights NULL or misaligned", l);
    for (int t = 0; t < molora::kXfTargets; ++t)
      if (L.W[t] == nullptr || !aligned(L.W[t], 16)) return fail(MOLORA_EINVAL, "layer %d: W[%d] NULL or misaligned", l, t);
    const molora_hotset* hs = L.lora;
    if (hs == nullptr) continue;
    if (hs->transposed || hs->n_targets != molora::kXfTargets)
      return fail(MOLORA_EINVAL, "layer %d: the LoRA hot set needs the 7 forward targets", l);
    for (int t = 0; t < molora::kXfTargets; ++t)
      if (hs->tg[t].d_in != din[t] || hs->tg[t].d_out != dout[t])
        return fail(MOLORA_EINVAL, "layer %d: LoRA target %d is %dx%d, %dx%d needed", l, t, hs->tg[t].d_in,
                    hs->tg[t].d_out, din[t], dout[t]);
    if (*K != 0 && hs->K != *K) return fail(MOLORA_EINVAL, "layer %d: K=%d differs from %d", l, hs->K, *K);
    *K = hs->K;
    if (k > hs->K) return fail(MOLORA_ENOTSUP, "k=%d > K=%d", k, hs->K);
    const int rp = hs->r_pad;
    const int pq = molora::apply_multi_resolve_path(3, (int)N, k, MOLORA_PATH_AUTO, hs->K, rp);
    const int pg = molora::apply_multi_resolve_path(2, (int)N, k, MOLORA_PATH_AUTO, hs->K, rp);
    const int po = molora::apply_resolve_path((int)N, k, MOLORA_PATH_AUTO, hs->K, rp);
    if (paths != nullptr) {
      paths[0] = pq; paths[1] = po; paths[2] = pg; paths[3] = po;
    }
    const size_t b[4] = {
        molora::apply_multi_plan(3, din, dout, (int)N, k, hs->K, rp, false, MOLORA_PATH_AUTO).total,
        molora::apply_ws_bytes((int)N, k, hs->K, rp, d, d, false, MOLORA_PATH_AUTO),
        molora::apply_multi_plan(2, din + molora::kXfGate, dout + molora::kXfGate, (int)N, k, hs->K, rp, false,
                                 MOLORA_PATH_AUTO).total,
        molora::apply_ws_bytes((int)N, k, hs->K, rp, f, d, false, MOLORA_PATH_AUTO)};
    for (size_t v : b) *lora_bytes = std::max(*lora_bytes, v);
  }
  return MOLORA_OK;
}

}  // namespace

int molora_xf_workspace(int d, int f, int n_layers, const molora_xf_layer* layers, int n_seq, int seq_len, int k,
                        size_t* bytes) {
  if (bytes == nullptr) return fail(MOLORA_EINVAL, "bytes is NULL");
  int K = 0;
  size_t lb = 0;
  const int rc = xf_check(d, f, n_layers, layers, n_seq, seq_len, k, &K, &lb, nullptr);
  if (rc != MOLORA_OK) return rc;
  *bytes = molora::xf_plan(n_seq, seq_len, d, f, lb).total;
  return ok();
}

int molora_xf_forward(int d, int f, int n_layers, const molora_xf_layer* layers, int n_seq, int seq_len,
                      const void* x_in, void* x_out, int k, const int32_t* offsets, const int32_t* perm,
                      const float* perm_w, const int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
  int K = 0;
  size_t lb = 0;
  int paths[4] = {0, 0, 0, 0};
  int rc = xf_check(d, f, n_layers, layers, n_seq, seq_len, k, &K, &lb, paths);
  if (rc != MOLORA_OK) return rc;
  if (x_in == nullptr || x_out == nullptr || !aligned(x_in, 16) || !aligned(x_out, 16))
    return fail(MOLORA_EINVAL, "x_in or x_out NULL or not 16-byte aligned");
  if (K > 0) {
    if (offsets == nullptr || perm == nullptr || perm_w == nullptr || inv == nullptr)
      return fail(MOLORA_EINVAL, "offsets, perm, perm_w and inv are required with LoRA layers");
    if (!aligned(offsets, 4) || !aligned(perm, 4) || !aligned(perm_w, 4) || !aligned(inv, 4))
      return fail(MOLORA_EINVAL, "misaligned pointer");
  }
  const molora::XfPlan plan = molora::xf_plan(n_seq, seq_len, d, f, lb);
  if (ws == nullptr || ws_bytes < plan.total || !aligned(ws, 256))
    return fail(MOLORA_ENOSPC, "workspace of %zu bytes (256-byte aligned) needed, %zu given", plan.total, ws_bytes);
  std::vector<molora::XfLayerDev> dev(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    const molora_xf_layer& L = layers[l];
    molora::XfLayerDev& D = dev[l];
    D.norm1 = static_cast<const uint16_t*>(L.norm1);
    D.norm2 = static_cast<const uint16_t*>(L.norm2);
    for (int t = 0; t < molora::kXfTargets; ++t) D.W[t] = static_cast<const uint16_t*>(L.W[t]);
    D.lora = L.lora != nullptr;
    if (D.lora) {
      for (int t = 0; t < molora::kXfTargets; ++t) D.tgt[t] = L.lora->tg[t];
      D.indirect = L.lora->layout == MOLORA_LAYOUT_INDIRECT;
      D.scale = L.lora->scale;
    }
  }
  const char* what = "";
  molora::XfLaunch a{};
  a.d = d; a.f = f; a.n_seq = n_seq; a.seq_len = seq_len; a.n_layers = n_layers; a.K = K; a.k = k;
  a.eps = 1e-6f;
  a.layers = dev.data();
  a.x_in = static_cast<const uint16_t*>(x_in);
  a.x_out = static_cast<uint16_t*>(x_out);
  a.offsets = offsets; a.perm = perm; a.perm_w = perm_w; a.inv = inv;
  a.path_qkv = paths[0]; a.path_o = paths[1]; a.path_gu = paths[2]; a.path_down = paths[3];
  a.lora_bytes = lb;
  a.ws = static_cast<char*>(ws);
  a.what = &what;
  const hipError_t e = molora::launch_xf_forward(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOLORA_EHIP, "decoder forward (%s): %s", what, hipGetErrorString(e));
  return ok();
}

int molora_seqpass_meta(const int32_t* idx, int N, int K, int32_t* offsets, int32_t* perm, float* perm_w, void* stream) {
  if (N < 0) return fail(MOLORA_EINVAL, "N=%d < 0", N);
  if (K < 1 || K > MOLORA_MAX_ADAPTERS) return fail(MOLORA_ENOTSUP, "K=%d outside [1, %d]", K, MOLORA_MAX_ADAPTERS);
  if (N == 0) return ok();
  if (idx == nullptr || offsets == nullptr || perm == nullptr || perm_w == nullptr)
    return fail(MOLORA_EINVAL, "a required pointer is NULL");
  const hipError_t e =
      molora::launch_seqpass_meta(idx, N, K, offsets, perm, perm_w, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "seqpass_meta launch");
}

}  // extern "C"
