// Synthetic decoder forward with per-token LoRA (MoLoRA pages, thelatestinai.com, Table 7: an
// end-to-end transformer whose projections all take the per-token adapters, against a
// per-sequence simulation of one forward pass per adapter; Table 8: the same on an interleaved
// two-modality batch).
//
// Per layer, on one stream:
//   h = rmsnorm(x)                                  xf_rmsnorm_k
//   q, k, v = h W^T  (+ per-token LoRA, in place)   GEMM library; launch_apply_multi (3 targets)
//   S = q k^T / sqrt(128) per (sequence, head)      strided-batched GEMM, fp32 scores
//   P = causal softmax(S)                           xf_softmax_causal_k
//   att = P v                                       strided-batched GEMM
//   o = att Wo^T (+ LoRA);  x += o                  GEMM; launch_apply; xf_add_k
//   h = rmsnorm(x);  gate, up = h W^T (+ LoRA)      xf_rmsnorm_k; GEMMs; launch_apply_multi
//   a = silu(gate) * up;  o = a Wdown^T (+ LoRA)    xf_swiglu_k; GEMM; launch_apply
//   x += o                                          xf_add_k
// The base projections are plain dense GEMMs: they go to rocBLAS (bf16 operands, fp32
// accumulation, bf16 results), with a workspace carved from the caller's so nothing is
// allocated.  The LoRA deltas are this library's grouped kernels, added to the stored base
// output in place.  Matrices are row-major; rocBLAS is column-major, so each product is
// issued as its transpose.
#include <rocblas/rocblas.h>

#include <cmath>
#include <map>
#include <mutex>

#include "molora_launch.h"

namespace molora {

namespace {

std::mutex g_blas_mu;
std::map<int, rocblas_handle> g_blas;  // one handle per device, created on first use

rocblas_handle blas_for_current_device(const char** what) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *what = "hipGetDevice";
    return nullptr;
  }
  auto it = g_blas.find(dev);
  if (it != g_blas.end()) return it->second;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success) {
    *what = "rocblas_create_handle";
    return nullptr;
  }
  g_blas[dev] = h;
  return h;
}

// Row-major Y [rows][out] = X [rows][in] W^T with W [out][in] (nn.Linear layout).
rocblas_status linear(rocblas_handle h, const uint16_t* X, const uint16_t* W, uint16_t* Y, int rows, int in, int out) {
  const float one = 1.f, zero = 0.f;
  return rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, out, rows, in, &one, W,
                         rocblas_datatype_bf16_r, in, X, rocblas_datatype_bf16_r, in, &zero, Y,
                         rocblas_datatype_bf16_r, out, Y, rocblas_datatype_bf16_r, out, rocblas_datatype_f32_r,
                         rocblas_gemm_algo_standard, 0, 0);
}

ApplyLaunch lora_launch(const XfLaunch& a, const XfLayerDev& L, int t, const uint16_t* x, uint16_t* y, int path,
                        char* ws) {
  ApplyLaunch p{};
  p.tgt = L.tgt[t];
  p.indirect = L.indirect;
  p.x = x;
  p.y0 = y;
  p.y = y;
  p.N = a.n_seq * a.seq_len;
  p.k = a.k;
  p.K = a.K;
  p.scale = L.scale;
  p.offsets = a.offsets;
  p.perm = a.perm;
  p.perm_w = a.perm_w;
  p.inv = a.inv;
  p.path = path;
  p.ws = reinterpret_cast<float*>(ws);
  return p;
}

}  // namespace

hipError_t launch_xf_forward(const XfLaunch& a, hipStream_t s) {
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle h = blas_for_current_device(a.what);
  if (h == nullptr) return hipErrorUnknown;
  const XfPlan p = xf_plan(a.n_seq, a.seq_len, a.d, a.f, a.lora_bytes);
  if (rocblas_set_stream(h, s) != rocblas_status_success ||
      rocblas_set_workspace(h, a.ws + p.blas_off, p.blas_bytes) != rocblas_status_success) {
    *a.what = "rocblas stream / workspace";
    return hipErrorUnknown;
  }
  auto P = [&](size_t off) { return reinterpret_cast<uint16_t*>(a.ws + off); };
  uint16_t* hb = P(p.h_off);
  uint16_t* q = P(p.q_off);
  uint16_t* k = P(p.k_off);
  uint16_t* v = P(p.v_off);
  uint16_t* att = P(p.att_off);
  uint16_t* o = P(p.o_off);
  uint16_t* g = P(p.g_off);
  uint16_t* u = P(p.u_off);
  float* S = reinterpret_cast<float*>(a.ws + p.s_off);
  uint16_t* Pr = P(p.p_off);
  char* lws = a.ws + p.lora_off;
  const int N = a.n_seq * a.seq_len, d = a.d, f = a.f, T = a.seq_len, H = d / kXfHeadDim;
  const long long nd = (long long)N * d, nf = (long long)N * f;
  const float qk_scale = 1.f / std::sqrt((float)kXfHeadDim), one = 1.f, zero = 0.f;
  hipError_t err = hipSuccess;
#define XF_HIP(call, name)      \
  if ((err = (call)) != hipSuccess) { \
    *a.what = name;             \
    return err;                 \
  }
#define XF_BLAS(call, name)                             \
  if ((call) != rocblas_status_success) {               \
    *a.what = name;                                     \
    return hipErrorUnknown;                             \
  }
  const uint16_t* cur = a.x_in;
  for (int l = 0; l < a.n_layers; ++l) {
    const XfLayerDev& L = a.layers[l];
    XF_HIP(launch_xf_rmsnorm(cur, L.norm1, hb, N, d, a.eps, s), "rmsnorm");
    XF_BLAS(linear(h, hb, L.W[kXfQ], q, N, d, d), "q projection");
    XF_BLAS(linear(h, hb, L.W[kXfK], k, N, d, d), "k projection");
    XF_BLAS(linear(h, hb, L.W[kXfV], v, N, d, d), "v projection");
    if (L.lora) {
      ApplyLaunch m[3] = {lora_launch(a, L, kXfQ, hb, q, a.path_qkv, lws), lora_launch(a, L, kXfK, hb, k, a.path_qkv, lws),
                          lora_launch(a, L, kXfV, hb, v, a.path_qkv, lws)};
      XF_HIP(launch_apply_multi(m, 3, s), "q/k/v LoRA");
    }
    for (int b = 0; b < a.n_seq; ++b) {
      const size_t tok0 = (size_t)b * T * d;
      float* Sb = S + (size_t)b * H * T * T;
      uint16_t* Pb = Pr + (size_t)b * H * T * T;
      // column-major S^T[j][i] = k_j . q_i, i.e. row-major S[i][j], per head (stride 128)
      XF_BLAS(rocblas_gemm_strided_batched_ex(h, rocblas_operation_transpose, rocblas_operation_none, T, T, kXfHeadDim,
                                              &qk_scale, k + tok0, rocblas_datatype_bf16_r, d, kXfHeadDim, q + tok0,
                                              rocblas_datatype_bf16_r, d, kXfHeadDim, &zero, Sb,
                                              rocblas_datatype_f32_r, T, (rocblas_stride)T * T, Sb,
                                              rocblas_datatype_f32_r, T, (rocblas_stride)T * T, H,
                                              rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0),
              "attention scores");
      XF_HIP(launch_xf_softmax_causal(Sb, Pb, T, (long long)H * T, s), "softmax");
      // column-major att^T[c][i] = sum_j v_j[c] P[i][j]
      XF_BLAS(rocblas_gemm_strided_batched_ex(h, rocblas_operation_none, rocblas_operation_none, kXfHeadDim, T, T, &one,
                                              v + tok0, rocblas_datatype_bf16_r, d, kXfHeadDim, Pb,
                                              rocblas_datatype_bf16_r, T, (rocblas_stride)T * T, &zero, att + tok0,
                                              rocblas_datatype_bf16_r, d, kXfHeadDim, att + tok0,
                                              rocblas_datatype_bf16_r, d, kXfHeadDim, H, rocblas_datatype_f32_r,
                                              rocblas_gemm_algo_standard, 0, 0),
              "attention values");
    }
    XF_BLAS(linear(h, att, L.W[kXfO], o, N, d, d), "o projection");
    if (L.lora) {
      const ApplyLaunch m = lora_launch(a, L, kXfO, att, o, a.path_o, lws);
      XF_HIP(launch_apply(m, s), "o LoRA");
    }
    XF_HIP(launch_xf_add(cur, o, a.x_out, nd, s), "residual");
    cur = a.x_out;
    XF_HIP(launch_xf_rmsnorm(cur, L.norm2, hb, N, d, a.eps, s), "rmsnorm");
    XF_BLAS(linear(h, hb, L.W[kXfGate], g, N, d, f), "gate projection");
    XF_BLAS(linear(h, hb, L.W[kXfUp], u, N, d, f), "up projection");
    if (L.lora) {
      ApplyLaunch m[2] = {lora_launch(a, L, kXfGate, hb, g, a.path_gu, lws),
                          lora_launch(a, L, kXfUp, hb, u, a.path_gu, lws)};
      XF_HIP(launch_apply_multi(m, 2, s), "gate/up LoRA");
    }
    XF_HIP(launch_xf_swiglu(g, u, nf, s), "swiglu");
    XF_BLAS(linear(h, g, L.W[kXfDown], o, N, f, d), "down projection");
    if (L.lora) {
      const ApplyLaunch m = lora_launch(a, L, kXfDown, g, o, a.path_down, lws);
      XF_HIP(launch_apply(m, s), "down LoRA");
    }
    XF_HIP(launch_xf_add(cur, o, a.x_out, nd, s), "residual");
  }
#undef XF_HIP
#undef XF_BLAS
  return hipSuccess;
}

}  // namespace molora
