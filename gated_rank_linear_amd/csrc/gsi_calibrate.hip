// Calibration of a layer's activation basis V_k on the GPU, with the depth cascade.
//
// Method: "Gated Subspace Inference for transformer acceleration" technical summary
// (gist.science, arXiv 2605.03109), §2.3 (depth cascade and calibration): a layer's basis is
// computed once from a calibration forward pass; the next layer's basis starts from this one
// and needs only a few rank-1 (DGKS) corrections instead of a full SVD per layer.
//
// One calibration call runs n_iter steps of subspace iteration
//     Q <- orth(A^T (A Q)),   A [n, d] calibration activations (one token per row)
// where orth is Gram-Schmidt over the columns in order, each column projected against the
// orthonormal columns before it (a rank-1 extension of the factor) and projected a second time
// when the first projection leaves less than eta = 1/sqrt(2) of its norm (the Daniel-Gragg-
// Kaufman-Stewart criterion). The start Q0 is a Gaussian draw for the first layer and the
// previous layer's basis for the cascade. Bases are stored by rows: Qt [k, d], row j = column j.
//
// Kernels: the two products run on the float32 NT GEMM of the dense path (Zt = Qt A^T, then
// Yt = Zt (A^T)^T with A^T transposed once per call). The orthonormalisation goes by panels of
// rows: each panel is projected against the earlier rows on the whole chip (H = Y_panel Q^T split
// over K, then Y_panel -= H Q), and Gram-Schmidt inside the panel runs in one workgroup, since
// column j depends on every column before it.
#include <cmath>

#include "gsi_internal.h"

namespace gsi {
namespace {

constexpr int kOrthThreads = 1024;
constexpr int kOrthWaves = kOrthThreads / 64;
constexpr int kOrthMaxD = 16384;  // a thread holds at most 16 elements of a panel row
constexpr int kOrthMaxK = 512;
constexpr int kCalMaxIter = 64;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the workgroup in a fixed order (butterflies inside each wave, then the wave sums in
// index order); every thread receives the result. Also a barrier for LDS and global memory.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();  // red is free, and every write before this call is visible after the next
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kOrthWaves; ++i) s += red[i];
  return s;
}

// Gram-Schmidt with DGKS reorthogonalisation inside one panel of `rows` rows (j0 .. j0 + rows - 1
// of Y, each d long), result in the same rows of Q (a different buffer). One workgroup; thread
// tid holds elements tid + 1024 u (u < EPT) of every row of the panel in registers, so a column
// costs workgroup sums only: v = y_j; h_i = <q_i, v> for the panel rows i < j (per-thread
// partial products, then one fixed-order workgroup sum per i); v -= sum h_i q_i; a second
// projection when |v|^2 fell below eta2 of its value before; q_j = v / |v|.
template <int EPT>
__global__ __launch_bounds__(kOrthThreads) void dgks_panel_kernel(const float* __restrict__ Y, float* __restrict__ Q,
                                                                  int j0, int rows, int d, float eta2) {
  constexpr int PMAX = EPT >= 8 ? 64 / EPT : 16;  // rows held per thread (registers)
  __shared__ float red[PMAX][kOrthWaves];
  __shared__ float h[PMAX];
  __shared__ float nred[kOrthWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float yv[PMAX][EPT];
#pragma unroll
  for (int r = 0; r < PMAX; ++r)
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = tid + kOrthThreads * u;
      yv[r][u] = (r < rows && e < d) ? Y[(long long)(j0 + r) * d + e] : 0.f;
    }
  auto norm2 = [&](const float (&v)[EPT]) {
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < EPT; ++u) s = __builtin_fmaf(v[u], v[u], s);
    return block_sum(s, nred);
  };
#pragma clang loop unroll(full)
  for (int j = 0; j < PMAX; ++j) {
    if (j >= rows) continue;  // uniform
    float v[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) v[u] = yv[j][u];
    const float before = norm2(v);
    float after = before;
    for (int pass = 0; pass < 2 && j > 0; ++pass) {
      // h_i = <q_i, v>, i < j: per-thread partials, wave sums, then the wave sums in index order
#pragma unroll
      for (int i = 0; i < PMAX; ++i) {
        if (i < j) {  // uniform
          float a = 0.f;
#pragma unroll
          for (int u = 0; u < EPT; ++u) a = __builtin_fmaf(yv[i][u], v[u], a);
          a = wave_sum(a);
          if (lane == 0) red[i][wave] = a;
        }
      }
      __syncthreads();
      if (tid < j) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kOrthWaves; ++w) sum += red[tid][w];
        h[tid] = sum;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < EPT; ++u) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < PMAX; ++i)
          if (i < j) acc = __builtin_fmaf(h[i], yv[i][u], acc);
        v[u] -= acc;
      }
      after = norm2(v);
      if (!(after < eta2 * before)) break;  // enough of the column survived one projection
    }
    const float inv = 1.0f / sqrtf(after);
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      yv[j][u] = v[u] * inv;
      const int e = tid + kOrthThreads * u;
      if (e < d) Q[(long long)(j0 + j) * d + e] = yv[j][u];
    }
  }
}

// Rows per panel for a row length d: a thread holds ceil(d / 1024) elements of each panel row.
int panel_rows(int d) { return d <= 4096 ? 16 : d <= 8192 ? 8 : 4; }

int launch_dgks_panel(const float* Y, float* Q, int j0, int rows, int d, float eta2, hipStream_t s) {
  const int ept = (d + kOrthThreads - 1) / kOrthThreads;
  if (ept <= 1) dgks_panel_kernel<1><<<1, kOrthThreads, 0, s>>>(Y, Q, j0, rows, d, eta2);
  else if (ept <= 2) dgks_panel_kernel<2><<<1, kOrthThreads, 0, s>>>(Y, Q, j0, rows, d, eta2);
  else if (ept <= 4) dgks_panel_kernel<4><<<1, kOrthThreads, 0, s>>>(Y, Q, j0, rows, d, eta2);
  else if (ept <= 8) dgks_panel_kernel<8><<<1, kOrthThreads, 0, s>>>(Y, Q, j0, rows, d, eta2);
  else dgks_panel_kernel<16><<<1, kOrthThreads, 0, s>>>(Y, Q, j0, rows, d, eta2);
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

// One projection of a panel of rows against every earlier row of Q, on the whole chip:
// Y[r, e] -= sum_{i < p0} H[r, i] Q[i, e] for the `rows` rows of the panel, H = Y_panel Q^T
// ([rows, p0], computed before by the NT GEMM). One thread per column e, the panel's rows of H
// staged in LDS, fixed order over i.
constexpr int kPanel = 16;
__global__ __launch_bounds__(256) void panel_project_kernel(float* __restrict__ Y, const float* __restrict__ H,
                                                            const float* __restrict__ Q, int rows, int p0, int d) {
  __shared__ float hs[kPanel][kOrthMaxK];
  for (int idx = threadIdx.x; idx < rows * p0; idx += 256) hs[idx / p0][idx % p0] = H[idx];
  __syncthreads();
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= d) return;
  float acc[kPanel];
#pragma unroll
  for (int r = 0; r < kPanel; ++r) acc[r] = 0.f;
  for (int i = 0; i < p0; ++i) {
    const float q = Q[(long long)i * d + e];
#pragma unroll
    for (int r = 0; r < kPanel; ++r) acc[r] = __builtin_fmaf(hs[r][i], q, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < kPanel; ++r)
    if (r < rows) Y[(long long)r * d + e] -= acc[r];
}

struct CalWs {
  float* At;  // [d, n]
  float* Zt;  // [k, n]
  float* Yt;  // [k, d]
  float* H;   // [kPanel, k] projections of a panel on the earlier rows
  float* Hp;  // [kHSplits, kPanel, k] split-K partial sums of H
  float* P;   // [kPSplits, k, max(n, d)] split-K partial sums of the token products
};
constexpr int kHSplits = 16;
constexpr int kPSplits = 8;
inline long long prod_part_elems(int n, int d, int k) { return (long long)kPSplits * k * (n > d ? n : d); }

size_t cal_ws_bytes(int n, int d, int k) {
  return align256((size_t)d * n * 4) + align256((size_t)k * n * 4) + align256((size_t)k * d * 4) +
         align256((size_t)kPanel * k * 4) + align256((size_t)kHSplits * kPanel * k * 4) +
         align256((size_t)prod_part_elems(n, d, k) * 4);
}

CalWs cal_ws_carve(void* ws, int n, int d, int k) {
  char* c = (char*)ws;
  CalWs w;
  w.At = (float*)c;
  c += align256((size_t)d * n * 4);
  w.Zt = (float*)c;
  c += align256((size_t)k * n * 4);
  w.Yt = (float*)c;
  c += align256((size_t)k * d * 4);
  w.H = (float*)c;
  c += align256((size_t)kPanel * k * 4);
  w.Hp = (float*)c;
  c += align256((size_t)kHSplits * kPanel * k * 4);
  w.P = (float*)c;
  return w;
}

int cal_shape(int n, int d, int k, int n_iter) {
  if (k < 8 || k > kOrthMaxK) return GSI_ERR_SHAPE;
  if (d < k || d > kOrthMaxD || d % 8 != 0) return GSI_ERR_SHAPE;
  if (n < k || n % 8 != 0 || n > (1 << 20)) return GSI_ERR_SHAPE;
  if (n_iter < 1 || n_iter > kCalMaxIter) return GSI_ERR_SHAPE;
  return GSI_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace
}  // namespace gsi

using namespace gsi;

extern "C" {

size_t gsi_calibrate_workspace_bytes(int n, int d, int k) {
  if (cal_shape(n, d, k, 1) != GSI_OK) return 0;
  return cal_ws_bytes(n, d, k);
}

int gsi_calibrate(int n, int d, int k, const float* A, const float* Q0t, int n_iter, float* Qt, void* ws,
                  size_t ws_bytes, void* stream) {
  int rc = cal_shape(n, d, k, n_iter);
  if (rc != GSI_OK) return rc;
  if (!A || !Q0t || !Qt || !ws) return GSI_ERR_NULL;
  if (!aligned16(A) || !aligned16(Q0t) || !aligned16(Qt) || !aligned16(ws)) return GSI_ERR_ALIGN;
  if (ws_bytes < cal_ws_bytes(n, d, k)) return GSI_ERR_WORKSPACE;
  // the result must not overlap the inputs it is computed from, except Qt == Q0t exactly
  const char* qa = (const char*)Qt;
  const char* qe = qa + (size_t)k * d * 4;
  const char* aa = (const char*)A;
  const char* ae = aa + (size_t)n * d * 4;
  const char* wa = (const char*)ws;
  const char* we = wa + cal_ws_bytes(n, d, k);
  const char* sa = (const char*)Q0t;
  const char* se = sa + (size_t)k * d * 4;
  if ((qa < ae && aa < qe) || (qa < we && wa < qe) || (sa != qa && qa < se && sa < qe)) return GSI_ERR_SHAPE;
  if ((rc = gsi_device_check()) != GSI_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  const CalWs w = cal_ws_carve(ws, n, d, k);
  // A^T [d, n] once per call: the second product contracts over the tokens
  if ((rc = launch_transpose(GSI_F32, A, w.At, n, d, LayerDesc{}, 0, nullptr, s)) != GSI_OK) return rc;
  const float eta2 = 0.5f;  // eta = 1/sqrt(2)
  for (int it = 0; it < n_iter; ++it) {
    const float* Qin = it == 0 ? Q0t : Qt;
    // Zt [k, n] = Qt A^T: row j holds (A q_j)^T
    const long long pe = prod_part_elems(n, d, k);
    if ((rc = launch_gemm_nt_f32_splitk(Qin, d, A, d, w.Zt, n, k, n, d, w.P, pe, s)) != GSI_OK) return rc;
    // Yt [k, d] = Zt A: row j holds (A^T A q_j)^T
    if ((rc = launch_gemm_nt_f32_splitk(w.Zt, n, w.At, n, w.Yt, d, k, d, n, w.P, pe, s)) != GSI_OK) return rc;
    // orth(Yt) by panels of up to kPanel rows: each panel is projected against all earlier rows
    // twice on the whole chip (the second projection is the DGKS reorthogonalisation, taken
    // always), then Gram-Schmidt with the DGKS criterion runs inside the panel in one workgroup
    const int panel = panel_rows(d);
    for (int p0 = 0; p0 < k; p0 += panel) {
      const int rows = k - p0 < panel ? k - p0 : panel;
      float* Yp = w.Yt + (long long)p0 * d;
      for (int pass = 0; pass < 2 && p0 > 0; ++pass) {
        if ((rc = launch_gemm_nt_f32_splitk(Yp, d, Qt, d, w.H, p0, rows, p0, d, w.Hp,
                                            (long long)kHSplits * kPanel * k, s)) != GSI_OK)
          return rc;
        panel_project_kernel<<<(d + 255) / 256, 256, 0, s>>>(Yp, w.H, Qt, rows, p0, d);
        if (hipGetLastError() != hipSuccess) return GSI_ERR_HIP;
      }
      if ((rc = launch_dgks_panel(w.Yt, Qt, p0, rows, d, eta2, s)) != GSI_OK) return rc;
    }
  }
  return GSI_OK;
}

}  // extern "C"
