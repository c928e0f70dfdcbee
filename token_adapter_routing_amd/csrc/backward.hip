// Backward of the routed LoRA on gfx950 (MoLoRA pages, thelatestinai.com, Figure 2: tokens
// grouped by their selected adapter, each group one grouped GEMM; the same grouping serves the
// gradients, read backwards; Table 13: adapters and router are trained from the loss alone).
//
// For a routed pair q (token t, adapter e, gate weight w, LoRA scale s), with h = x_t A_e and
// g = gy_t B_e^T:
//   dA_e = sum_q x_t^T (s w g)      dB_e = sum_q (s w h)^T gy_t      dL/dw_q = s (h . g)
// dx is the forward apply of the transposed adapters (B^T, A^T) on gy (launched by the C ABI).
//
//   pair shrinks  the 64-row grouped kernel in shrink-only mode (A staged in LDS once per tile)
//                 gives unscaled h and g per grouped pair.
//   bwd_pairs     a workgroup owns 64 consecutive pairs of one chunk: sums the partials, writes
//                 dL/dw at the pair id and s w g, s w h as bf16 hi/lo planes [rank][pair] of
//                 the chunk (pairs past the segment hold zeros).
//   bwd_wgrad     a workgroup owns (chunk, 128 columns of x or gy): per step of 64 pairs it
//                 stages the gathered rows transposed in LDS (pairs contiguous, 16-byte groups
//                 XOR-swizzled by row), and the chunk's hi/lo planes; the 8 waves (16 columns
//                 each) take D[rank][col] += S^T[rank][pair] X[pair][col] with
//                 v_mfma_f32_16x16x32_bf16 (hi and lo: fp32-accurate S), and write the
//                 chunk's partial [col][rank] in fp32.
//   bwd_reduce    a workgroup owns (adapter, 128 columns): sums the adapter's chunk partials
//                 in chunk order (deterministic) into dA [K][d_in][r] or dB [K][r][d_out];
//                 an adapter without pairs gets zeros.
#include "molora_launch.h"
#include "molora_dev.h"

namespace molora {

// Chunk cg of the segments cut into ceil(count / Qc) chunks each, numbered segment by
// segment: its adapter and pair range [q0, q1).  False past the last chunk (wave-uniform).
__device__ __forceinline__ bool chunk_of(const int32_t* __restrict__ offsets, int K, int Qc, long long cg, int lane,
                                         int& e, int& q0, int& q1) {
  const int lo = lane < K ? offsets[lane] : 0;
  const int cnt = lane < K ? offsets[lane + 1] - lo : 0;
  const int nch = (cnt + Qc - 1) / Qc;
  const int incl = wave_incl_scan(nch, lane);
  const uint64_t m = __ballot(lane < K && cg >= incl - nch && cg < incl);
  if (m == 0) return false;
  e = __builtin_ctzll(m);
  const int lo_e = __shfl(lo, e, kWave), cnt_e = __shfl(cnt, e, kWave);
  const int first = __shfl(incl, e, kWave) - __shfl(nch, e, kWave);
  q0 = lo_e + (int)(cg - first) * Qc;
  q1 = min(lo_e + cnt_e, q0 + Qc);
  return true;
}

__global__ __launch_bounds__(256) void fill_zero_k(float* __restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ------------------------------------------------------------------------------ pair pass
struct BwdPairArgs {
  const float* hp;  // [nsh][P][r_pad] unscaled h partials, or nullptr
  const float* gp;  // [nsg][P][r_pad] unscaled g partials, or nullptr
  int nsh, nsg;
  long long P;
  const int32_t* offsets;
  const int32_t* perm;
  const float* perm_w;
  const int32_t* inv;
  int K, r_pad, Qc;
  float scale;
  uint16_t* sa;  // chunks of s w g (dA), or nullptr
  uint16_t* sb;  // chunks of s w h (dB), or nullptr
  float* dw;     // [P] by pair id, or nullptr
  long long chunk_blocks;
  int zero_blocks;
};

__device__ __forceinline__ void sum_partials(float (&v)[16], const float* __restrict__ p, int ns, long long P, int q,
                                             int r_pad, int j0, int nj) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = 0.f;
  for (int sp = 0; sp < ns; ++sp) {
    const float* row = p + ((long long)sp * P + q) * r_pad + j0;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      if (i < nj) {
        const u32x4_t x = ld16(row + i);
        v[i] += __uint_as_float(x[0]);
        v[i + 1] += __uint_as_float(x[1]);
        v[i + 2] += __uint_as_float(x[2]);
        v[i + 3] += __uint_as_float(x[3]);
      }
    }
  }
}

__device__ __forceinline__ void put_hilo(uint16_t* __restrict__ plane, size_t lo_off, int Qc, int j, int col,
                                         float v) {
  const __bf16 hi = (__bf16)v;
  const __bf16 lo = (__bf16)(v - (float)hi);
  plane[(size_t)j * Qc + col] = __builtin_bit_cast(uint16_t, hi);
  plane[lo_off + (size_t)j * Qc + col] = __builtin_bit_cast(uint16_t, lo);
}

__global__ __launch_bounds__(256) void bwd_pairs(BwdPairArgs a) {
  __shared__ float dot[4][64];
  const int lane = threadIdx.x & 63, jg = threadIdx.x >> 6;
  if ((long long)blockIdx.x >= a.chunk_blocks) {
    if (a.dw == nullptr) return;
    const long long stride = (long long)a.zero_blocks * 256;
    for (long long p = ((long long)blockIdx.x - a.chunk_blocks) * 256 + threadIdx.x; p < a.P; p += stride)
      if (a.inv[p] < 0) a.dw[p] = 0.f;
    return;
  }
  const int spc = a.Qc / kWStep;
  const long long cg = (long long)blockIdx.x / spc;
  const int col = (int)((long long)blockIdx.x % spc) * kWStep + lane;
  int e, q0, q1;
  if (!chunk_of(a.offsets, a.K, a.Qc, cg, lane, e, q0, q1)) return;
  const int q = q0 + col;
  const bool valid = q < q1;
  const int nj = a.r_pad / 4, j0 = jg * nj;
  float h[16], g[16];
  if (valid && a.hp != nullptr) sum_partials(h, a.hp, a.nsh, a.P, q, a.r_pad, j0, nj);
  else
#pragma unroll
    for (int i = 0; i < 16; ++i) h[i] = 0.f;
  if (valid && a.gp != nullptr) sum_partials(g, a.gp, a.nsg, a.P, q, a.r_pad, j0, nj);
  else
#pragma unroll
    for (int i = 0; i < 16; ++i) g[i] = 0.f;
  const float c = valid ? a.scale * a.perm_w[q] : 0.f;
  const size_t plane = bwd_s_chunk_elems(a.r_pad, a.Qc);
  const size_t base = (size_t)cg * 2 * plane;
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < nj) {
      d += h[i] * g[i];
      if (a.sa != nullptr) put_hilo(a.sa + base, plane, a.Qc, j0 + i, col, c * g[i]);
      if (a.sb != nullptr) put_hilo(a.sb + base, plane, a.Qc, j0 + i, col, c * h[i]);
    }
  }
  if (a.dw == nullptr) return;
  dot[jg][lane] = d;
  __syncthreads();
  if (jg == 0 && valid) a.dw[a.perm[q]] = a.scale * (((dot[0][lane] + dot[1][lane]) + dot[2][lane]) + dot[3][lane]);
}

// ------------------------------------------------------------------------------ weight gradient
struct BwdWgradArgs {
  const uint16_t* X;  // [rows][D] bf16 (x for dA, gy for dB)
  int D;
  const int32_t* offsets;
  const int32_t* perm;  // grouped position -> pair id; nullptr: the position is the row
  int k, K;
  const uint16_t* S;    // chunks [nchunks][2][r_pad][Qc] bf16 hi / lo
  int Qc, r_pad, ncb;
  float* part;          // [nchunks][ncb][128][r_pad] fp32
};

constexpr int kWThreads = 512;

template <int RB>
struct WgradLds {
  uint32_t xt[kWCols][kWStep / 2];        // X^T: row = column of X, dword = two pairs; 16-byte
                                          // groups (8 pairs) at group ^ (row & 7)
  u32x4_t st[2][RB * 16][kWStep / 8];     // S^T hi / lo: row = rank, groups at g ^ (row & 7)
};

template <int RB>
__global__ __launch_bounds__(kWThreads) void bwd_wgrad(BwdWgradArgs a) {
  __shared__ WgradLds<RB> L;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long cg = (long long)blockIdx.x / a.ncb;
  const int b = (int)((long long)blockIdx.x % a.ncb);
  int e, q0, q1;
  if (!chunk_of(a.offsets, a.K, a.Qc, cg, lane, e, q0, q1)) return;
  const int n = lane & 15, G = lane >> 4;
  // staging roles: X rows (2p, 2p+1) of the step, columns [8c, 8c + 8) of the block
  const int p = threadIdx.x & 31, c = threadIdx.x >> 5;
  const uint16_t* xcol = a.X + (size_t)b * kWCols + 8 * c;
  const uint16_t* schunk = a.S + (size_t)cg * 2 * bwd_s_chunk_elems(a.r_pad, a.Qc);
  constexpr int kSPieces = 2 * RB * 16 * (kWStep / 8);  // 16-byte pieces of S per step
  auto row_of = [&](int q) {
    q = min(q, q1 - 1);  // rows past the range: any valid row (their S is zero)
    return a.perm != nullptr ? a.perm[q] / a.k : q;
  };
  // two steps of rows in flight: register sets A and B alternate
  struct Regs {
    u32x4_t xv[2], sv[2];
  };
  Regs ra, rb;
  auto load = [&](Regs& R, int qs) {
    R.xv[0] = ld16(xcol + (size_t)row_of(qs + 2 * p) * a.D);
    R.xv[1] = ld16(xcol + (size_t)row_of(qs + 2 * p + 1) * a.D);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = threadIdx.x + i * kWThreads;
      if (v < kSPieces) {
        const int pl = v / (RB * 16 * 8), rem = v % (RB * 16 * 8);
        const int j = rem >> 3, gq = rem & 7;
        R.sv[i] = ld16(schunk + (size_t)pl * bwd_s_chunk_elems(a.r_pad, a.Qc) + (size_t)j * a.Qc + (qs - q0) + 8 * gq);
      }
    }
  };
  auto store = [&](const Regs& R) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int row = 8 * c + s;
      const uint32_t lo = (s & 1) ? (R.xv[0][s >> 1] >> 16) : (R.xv[0][s >> 1] & 0xffffu);
      const uint32_t hi = (s & 1) ? (R.xv[1][s >> 1] >> 16) : (R.xv[1][s >> 1] & 0xffffu);
      L.xt[row][4 * ((p >> 2) ^ s) + (p & 3)] = lo | (hi << 16);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = threadIdx.x + i * kWThreads;
      if (v < kSPieces) {
        const int pl = v / (RB * 16 * 8), rem = v % (RB * 16 * 8);
        const int j = rem >> 3, gq = rem & 7;
        L.st[pl][j][gq ^ (j & 7)] = R.sv[i];
      }
    }
  };
  f32x4_t acc[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int xrow = 16 * wave + n;
  auto products = [&]() {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int gq = 4 * ks + G;
      const u32x4_t xb = *reinterpret_cast<const u32x4_t*>(&L.xt[xrow][4 * (gq ^ (xrow & 7))]);
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int j = 16 * u + n;
        const u32x4_t sh = L.st[0][j][gq ^ (j & 7)];
        const u32x4_t sl = L.st[1][j][gq ^ (j & 7)];
        acc[u] = mfma16x16x32(as_bf16x8(sh), as_bf16x8(xb), acc[u]);
        acc[u] = mfma16x16x32(as_bf16x8(sl), as_bf16x8(xb), acc[u]);
      }
    }
  };
  // one step: its rows go to LDS, the step two ahead is loaded into the freed registers
  auto step = [&](Regs& R, int qs) {
    __syncthreads();  // the previous step's operands are consumed
    store(R);
    __syncthreads();
    if (qs + 2 * kWStep < q1) load(R, qs + 2 * kWStep);
    products();
  };
  load(ra, q0);
  if (q0 + kWStep < q1) load(rb, q0 + kWStep);
  for (int qs = q0; qs < q1; qs += 2 * kWStep) {
    step(ra, qs);
    if (qs + kWStep < q1) step(rb, qs + kWStep);
  }
  // D[rank 16u + 4G + i][column 16 wave + n]
  float* dst = a.part + (((size_t)cg * a.ncb + b) * kWCols + 16 * wave + n) * a.r_pad + 4 * G;
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[u][i]);
    st16(dst + 16 * u, v);
  }
}

// ------------------------------------------------------------------------------ reduction
struct BwdReduceArgs {
  const float* part;
  const int32_t* offsets;
  int K, Qc, r, r_pad, ncb, D;
  float* out;
  int rank_major;  // 0: out [K][D][r] (dA); 1: out [K][r][D] (dB)
};

// A workgroup owns (adapter e, 128 columns, 16 ranks): each thread sums 8 (column, rank)
// elements over e's chunks in chunk order (reads 64-byte rank runs of the partials), then
// writes them rank-contiguous (dA) or, through an LDS transpose, column-contiguous (dB).
__global__ __launch_bounds__(256) void bwd_reduce(BwdReduceArgs a) {
  __shared__ float tr[16][kWCols + 1];
  const int RBv = a.r_pad / 16;
  const int u = blockIdx.x % RBv;
  const int b = (blockIdx.x / RBv) % a.ncb;
  const int e = blockIdx.x / (RBv * a.ncb);
  const int lane = threadIdx.x & 63;
  const int cnt = lane < a.K ? a.offsets[lane + 1] - a.offsets[lane] : 0;
  const int nchl = (cnt + a.Qc - 1) / a.Qc;
  const int incl = wave_incl_scan(nchl, lane);
  const int nch = __shfl(nchl, e, kWave);
  const int first = __shfl(incl, e, kWave) - nch;
  const int jj = threadIdx.x & 15, c0 = threadIdx.x >> 4;  // rank 16u + jj, columns c0 + 16 i
  const int j = 16 * u + jj;
  float sum[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sum[i] = 0.f;
  for (int ch = 0; ch < nch; ++ch) {
    const float* src = a.part + ((size_t)(first + ch) * a.ncb + b) * kWCols * a.r_pad + j;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum[i] += src[(size_t)(c0 + 16 * i) * a.r_pad];
  }
  const size_t gcol0 = (size_t)b * kWCols;
  if (!a.rank_major) {
    if (j < a.r)
#pragma unroll
      for (int i = 0; i < 8; ++i) a.out[((size_t)e * a.D + gcol0 + c0 + 16 * i) * a.r + j] = sum[i];
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) tr[jj][c0 + 16 * i] = sum[i];
  __syncthreads();
  for (int v = threadIdx.x; v < 16 * kWCols; v += 256) {
    const int jr = v / kWCols, col = v % kWCols;
    if (16 * u + jr < a.r) a.out[((size_t)e * a.r + 16 * u + jr) * a.D + gcol0 + col] = tr[jr][col];
  }
}

// ------------------------------------------------------------------------------ host side
static hipError_t launch_wgrad_reduce(const BackwardLaunch& a, const BwdPlan& plan, const uint16_t* X, int D,
                                      const uint16_t* S, float* out, int rank_major, hipStream_t s) {
  const int ncb = D / kWCols;
  float* part = reinterpret_cast<float*>(a.ws + plan.part_off);
  if (a.N > 0) {
    BwdWgradArgs w;
    w.X = X; w.D = D; w.offsets = a.offsets; w.perm = a.perm; w.k = a.k; w.K = a.K;
    w.S = S; w.Qc = plan.Qc; w.r_pad = a.tgt.r_pad; w.ncb = ncb; w.part = part;
    const long long grid = plan.nchunks * ncb;
    switch (a.tgt.r_pad / 16) {
      case 1: hipLaunchKernelGGL(bwd_wgrad<1>, dim3((unsigned)grid), dim3(kWThreads), 0, s, w); break;
      case 2: hipLaunchKernelGGL(bwd_wgrad<2>, dim3((unsigned)grid), dim3(kWThreads), 0, s, w); break;
      case 3: hipLaunchKernelGGL(bwd_wgrad<3>, dim3((unsigned)grid), dim3(kWThreads), 0, s, w); break;
      case 4: hipLaunchKernelGGL(bwd_wgrad<4>, dim3((unsigned)grid), dim3(kWThreads), 0, s, w); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  BwdReduceArgs r;
  r.part = part; r.offsets = a.offsets; r.K = a.K; r.Qc = plan.Qc; r.r = a.r; r.r_pad = a.tgt.r_pad;
  r.ncb = ncb; r.D = D; r.out = out; r.rank_major = rank_major;
  hipLaunchKernelGGL(bwd_reduce, dim3((unsigned)(a.K * ncb * (a.tgt.r_pad / 16))), dim3(256), 0, s, r);
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardLaunch& a, hipStream_t s) {
  const BwdPlan plan = bwd_plan(a.N, a.k, a.K, a.tgt.r_pad, a.tgt.d_in, a.tgt.d_out, a.dx_f32, a.dx_path);
  const long long P = (long long)a.N * a.k;
  const bool need_h = a.dB != nullptr || a.dw != nullptr;
  const bool need_g = a.dA != nullptr || a.dw != nullptr;
  float* hp = need_h ? reinterpret_cast<float*>(a.ws + plan.h_off) : nullptr;
  float* gp = need_g ? reinterpret_cast<float*>(a.ws + plan.g_off) : nullptr;
  uint16_t* sa = a.dA != nullptr ? reinterpret_cast<uint16_t*>(a.ws + plan.sa_off) : nullptr;
  uint16_t* sb = a.dB != nullptr ? reinterpret_cast<uint16_t*>(a.ws + plan.sb_off) : nullptr;
  float* gsp = reinterpret_cast<float*>(a.ws + plan.gs_off);  // the shrinks' slice partials
  hipError_t err = hipSuccess;
  if (P > 0) {
    if (need_h) {
      err = launch_pair_shrink_gm(a.tgt, a.indirect, a.x, a.offsets, a.perm, a.K, a.k, P, hp, gsp, s);
      if (err != hipSuccess) return err;
    }
    if (need_g) {
      err = launch_pair_shrink_gm(a.tgt_t, a.indirect_t, a.gy, a.offsets, a.perm, a.K, a.k, P, gp, gsp, s);
      if (err != hipSuccess) return err;
    }
    BwdPairArgs pa;
    pa.hp = hp; pa.gp = gp; pa.nsh = plan.nsh; pa.nsg = plan.nsg; pa.P = P;
    pa.offsets = a.offsets; pa.perm = a.perm; pa.perm_w = a.perm_w; pa.inv = a.inv;
    pa.K = a.K; pa.r_pad = a.tgt.r_pad; pa.Qc = plan.Qc; pa.scale = a.scale;
    pa.sa = sa; pa.sb = sb; pa.dw = a.dw;
    pa.chunk_blocks = plan.nchunks * (plan.Qc / kWStep);
    pa.zero_blocks = a.dw != nullptr ? (int)std::min<long long>((P + 255) / 256, 64) : 0;
    hipLaunchKernelGGL(bwd_pairs, dim3((unsigned)(pa.chunk_blocks + pa.zero_blocks)), dim3(256), 0, s, pa);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.dA != nullptr) {
    err = launch_wgrad_reduce(a, plan, a.x, a.tgt.d_in, sa, a.dA, 0, s);
    if (err != hipSuccess) return err;
  }
  if (a.dB != nullptr) err = launch_wgrad_reduce(a, plan, a.gy, a.tgt.d_out, sb, a.dB, 1, s);
  return err;
}

// ------------------------------------------------------------------------------ router
// dL/dlogits through the softmax over the selected logits: the selected logit of slot j gets
// w_j (dw_j - sum_i w_i dw_i), every other logit 0.  One thread per (token, adapter).
__global__ __launch_bounds__(256) void route_topk_bwd_k(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                        const float* __restrict__ dw, int N, int K, int k,
                                                        float* __restrict__ dl) {
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  if (v >= (long long)N * K) return;
  const int t = (int)(v / K), e = (int)(v % K);
  const int32_t* ir = idx + (size_t)t * k;
  const float* wr = w + (size_t)t * k;
  const float* dr = dw + (size_t)t * k;
  float mean = 0.f, mine = 0.f, wmine = 0.f;
  bool sel = false;
  for (int j = 0; j < k; ++j) {
    mean += wr[j] * dr[j];
    if (ir[j] == e) {
      sel = true;
      mine = dr[j];
      wmine = wr[j];
    }
  }
  dl[v] = sel ? wmine * (mine - mean) : 0.f;
}

hipError_t launch_route_topk_backward(const int32_t* idx, const float* w, const float* dw, int N, int K, int k,
                                      float* dl, hipStream_t s) {
  const long long n = (long long)N * K;
  hipLaunchKernelGGL(route_topk_bwd_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, idx, w, dw, N, K, k, dl);
  return hipGetLastError();
}

// Per 64-token block: dL/d(hidden) = dlogits W2, masked by the ReLU of the recomputed
// pre-activation (the forward's own fp32 decision), written fp32 [N][64] and as the dW1
// reduction's hi/lo planes; the block's partial sums of dW2 = sum dlogits^T relu(pre),
// db2 = sum dlogits and db1 = sum dL/d(pre) go to `small` [block][K*64 + K + 64].
struct RouterTokArgs {
  const float* pre;
  const float* dl;
  const uint16_t* W2;  // [K][64] bf16
  int N, K, Qc;
  float* da;
  uint16_t* S;
  float* small;
  int32_t* offs;
};

__global__ __launch_bounds__(256) void router_bwd_tok_k(RouterTokArgs a) {
  constexpr int H = kRouterHidden, T = kRouterTokBlock;
  __shared__ float w2[64][H];
  __shared__ float dls[T][65];
  __shared__ float hid[T][H + 1];
  __shared__ float das[T][H + 1];
  const int t0 = blockIdx.x * T;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.offs[0] = 0;
    a.offs[1] = a.N;
  }
  for (int v = threadIdx.x; v < a.K * H; v += 256) w2[v / H][v % H] = bf16_to_f32(a.W2[v]);
  for (int v = threadIdx.x; v < T * a.K; v += 256) {
    const int tl = v / a.K, e = v % a.K;
    dls[tl][e] = t0 + tl < a.N ? a.dl[(size_t)(t0 + tl) * a.K + e] : 0.f;
  }
  __syncthreads();
  const int tl = threadIdx.x & 63, hg = threadIdx.x >> 6;
  const int t = t0 + tl;
  const bool valid = t < a.N;
  const size_t plane = bwd_s_chunk_elems(H, a.Qc);
  uint16_t* sc = a.S + (size_t)(t / a.Qc) * 2 * plane;
  const int col = t % a.Qc;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int h = hg * 16 + i;
    float dh = 0.f;
    for (int e = 0; e < a.K; ++e) dh = fmaf(dls[tl][e], w2[e][h], dh);
    const float p = valid ? a.pre[(size_t)t * H + h] : 0.f;
    const float g = (valid && p > 0.f) ? dh : 0.f;
    hid[tl][h] = p > 0.f ? p : 0.f;
    das[tl][h] = g;
    if (valid) a.da[(size_t)t * H + h] = g;
    const __bf16 hi = (__bf16)g;
    const __bf16 lo = (__bf16)(g - (float)hi);
    sc[(size_t)h * a.Qc + col] = __builtin_bit_cast(uint16_t, hi);
    sc[plane + (size_t)h * a.Qc + col] = __builtin_bit_cast(uint16_t, lo);
  }
  __syncthreads();
  float* out = a.small + (size_t)blockIdx.x * router_small_floats(a.K);
  for (int v = threadIdx.x; v < router_small_floats(a.K); v += 256) {
    float sum = 0.f;
    if (v < a.K * H) {
      const int e = v / H, h = v % H;
      for (int i = 0; i < T; ++i) sum = fmaf(dls[i][e], hid[i][h], sum);
    } else if (v < a.K * H + a.K) {
      const int e = v - a.K * H;
      for (int i = 0; i < T; ++i) sum += dls[i][e];
    } else {
      const int h = v - a.K * H - a.K;
      for (int i = 0; i < T; ++i) sum += das[i][h];
    }
    out[v] = sum;
  }
}

// Sum the blocks' partials in block order into dW2 [K][64], db2 [K], db1 [64].
__global__ __launch_bounds__(256) void router_bwd_small_k(const float* __restrict__ small, int ntb, int K,
                                                          float* __restrict__ dW2, float* __restrict__ db2,
                                                          float* __restrict__ db1) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  const int n = router_small_floats(K);
  if (v >= n) return;
  float sum = 0.f;
  for (int b = 0; b < ntb; ++b) sum += small[(size_t)b * n + v];
  if (v < K * kRouterHidden) {
    if (dW2 != nullptr) dW2[v] = sum;
  } else if (v < K * kRouterHidden + K) {
    if (db2 != nullptr) db2[v - K * kRouterHidden] = sum;
  } else if (db1 != nullptr) {
    db1[v - K * kRouterHidden - K] = sum;
  }
}

// dx = dx0 + dL/d(pre) W1 on the VALU: a workgroup owns 16 tokens x 512 columns, two columns
// per thread, the 16 tokens' gradients in LDS.
__global__ __launch_bounds__(256) void router_bwd_dx_k(const float* __restrict__ da, const uint16_t* __restrict__ W1,
                                                       const float* __restrict__ dx0, float* __restrict__ dx, int N,
                                                       int d) {
  constexpr int H = kRouterHidden;
  __shared__ float g[16][H];
  const int t0 = blockIdx.x * 16;
  for (int v = threadIdx.x; v < 16 * H; v += 256) {
    const int tl = v / H;
    g[tl][v % H] = t0 + tl < N ? da[(size_t)(t0 + tl) * H + v % H] : 0.f;
  }
  __syncthreads();
  const int c = blockIdx.y * 512 + 2 * threadIdx.x;
  if (c >= d) return;
  float acc[16][2];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t][0] = acc[t][1] = 0.f;
  for (int h = 0; h < H; ++h) {
    const uint32_t wv = *reinterpret_cast<const uint32_t*>(W1 + (size_t)h * d + c);
    const float w0 = bf16_to_f32(wv & 0xffffu), w1 = bf16_to_f32(wv >> 16);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      acc[t][0] = fmaf(g[t][h], w0, acc[t][0]);
      acc[t][1] = fmaf(g[t][h], w1, acc[t][1]);
    }
  }
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    if (t0 + t >= N) break;
    const size_t o = (size_t)(t0 + t) * d + c;
    const float b0 = dx0 != nullptr ? dx0[o] : 0.f, b1v = dx0 != nullptr ? dx0[o + 1] : 0.f;
    dx[o] = b0 + acc[t][0];
    dx[o + 1] = b1v + acc[t][1];
  }
}

hipError_t launch_router_backward(const RouterBackwardLaunch& a, hipStream_t s) {
  const RouterBwdPlan p = router_bwd_plan(a.N, a.d, a.K);
  float* pre = reinterpret_cast<float*>(a.ws + p.pre_off);
  float* da = reinterpret_cast<float*>(a.ws + p.da_off);
  uint16_t* S = reinterpret_cast<uint16_t*>(a.ws + p.s_off);
  float* part = reinterpret_cast<float*>(a.ws + p.part_off);
  float* small = reinterpret_cast<float*>(a.ws + p.small_off);
  int32_t* offs = reinterpret_cast<int32_t*>(a.ws + p.offs_off);
  hipError_t err = hipSuccess;
  if (a.N > 0) {
    err = launch_router_pre(a.x, a.N, a.d, a.W1, a.b1, pre, s);
    if (err != hipSuccess) return err;
    RouterTokArgs t{pre, a.dl, a.W2, a.N, a.K, p.Qc, da, S, small, offs};
    hipLaunchKernelGGL(router_bwd_tok_k, dim3((unsigned)p.ntb), dim3(256), 0, s, t);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (a.dW2 != nullptr || a.db2 != nullptr || a.db1 != nullptr) {
    if (a.N > 0) {
      const int n = router_small_floats(a.K);
      hipLaunchKernelGGL(router_bwd_small_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, small, p.ntb, a.K,
                         a.dW2, a.db2, a.db1);
    } else {
      // no tokens: the parameter gradients are zero (a fill kernel, capturable)
      hipLaunchKernelGGL(router_bwd_small_k, dim3((unsigned)((router_small_floats(a.K) + 255) / 256)), dim3(256), 0,
                         s, small, 0, a.K, a.dW2, a.db2, a.db1);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (a.dW1 != nullptr) {
    const int ncb = a.d / kWCols;
    if (a.N > 0) {
      BwdWgradArgs w;
      w.X = a.x; w.D = a.d; w.offsets = offs; w.perm = nullptr; w.k = 1; w.K = 1;
      w.S = S; w.Qc = p.Qc; w.r_pad = kRouterHidden; w.ncb = ncb; w.part = part;
      hipLaunchKernelGGL(bwd_wgrad<4>, dim3((unsigned)(p.nchunks * ncb)), dim3(kWThreads), 0, s, w);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      BwdReduceArgs r;
      r.part = part; r.offsets = offs; r.K = 1; r.Qc = p.Qc; r.r = kRouterHidden; r.r_pad = kRouterHidden;
      r.ncb = ncb; r.D = a.d; r.out = a.dW1; r.rank_major = 1;
      hipLaunchKernelGGL(bwd_reduce, dim3((unsigned)(ncb * (kRouterHidden / 16))), dim3(256), 0, s, r);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    } else {
      hipLaunchKernelGGL(fill_zero_k, dim3((unsigned)(((size_t)kRouterHidden * a.d + 255) / 256)), dim3(256), 0, s,
                         a.dW1, (long long)kRouterHidden * a.d);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  if (a.dx != nullptr && a.N > 0) {
    hipLaunchKernelGGL(router_bwd_dx_k, dim3((unsigned)((a.N + 15) / 16), (unsigned)((a.d + 511) / 512)), dim3(256), 0,
                       s, da, a.W1, a.dx0, a.dx, a.N, a.d);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace molora
