// Internal declarations shared by the libgsi translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/gsi.h"
#include "gsi_plan.h"

namespace gsi {

typedef unsigned long long u64;

// ---------------------------------------------------------------------------------------------
// Element types. Storage is raw bits; conversions are explicit so every rounding is visible.
// ---------------------------------------------------------------------------------------------
struct bf16_t { uint16_t b; };
struct f16_t { uint16_t b; };

__host__ __device__ __forceinline__ float to_f32(float v) { return v; }
__host__ __device__ __forceinline__ float to_f32(bf16_t v) {
  union { uint32_t u; float f; } c;
  c.u = (uint32_t)v.b << 16;
  return c.f;
}
__device__ __forceinline__ float to_f32(f16_t v) {
  _Float16 h;
  __builtin_memcpy(&h, &v.b, 2);
  return (float)h;
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
// round to nearest even; NaN stays NaN (quiet)
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  uint32_t u = c.u;
  bf16_t r;
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
    r.b = (uint16_t)((u >> 16) | 0x40u);
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);
    r.b = (uint16_t)(u >> 16);
  }
  return r;
}
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  f16_t r;
  __builtin_memcpy(&r.b, &h, 2);
  return r;
}

template <typename T> struct elem_size { static constexpr int v = sizeof(T); };

// 16-byte vector of elements and its conversion to floats
template <typename T> struct vec16 {
  static constexpr int N = 16 / sizeof(T);
};

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& q, float* out) {
  const T* e = reinterpret_cast<const T*>(&q);
#pragma unroll
  for (int i = 0; i < vec16<T>::N; ++i) out[i] = to_f32(e[i]);
}

inline size_t dtype_size(int dtype) { return dtype == GSI_F32 ? 4 : 2; }
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------------------------
// Layer and stack handles
// ---------------------------------------------------------------------------------------------
}  // namespace gsi

struct gsi_layer {
  int dtype, d_out, d, k;
  int P, xr;                 // decode grid and input window the plan was made for
  gsi::LayerDesc desc;       // x_off = y_off = 0, mode = gated
  gsi::PlanRow* plan;        // [P] plan rows of the decode kernel, in the layer's aux buffer
};

struct gsi_stack {
  int dtype, n_sites, k_max, d_max, d_out_max;
  int P, xr;
  long long x_ld, y_ld;
  gsi::PlanRow* d_plan;     // [n_sites][P] plan rows (device, owned)
  gsi::LayerDesc* h_table;  // host copy of the site descriptors
  gsi_layer** layers;       // host copy of the borrowed handles
};

namespace gsi {

// Workspace header (start of every workspace)
struct WsHeader {
  unsigned long long epoch;       // exchange tag base, advanced by every persistent launch
  unsigned long long abort_mark;  // epoch + 1 of a launch that gave up waiting
  int status;                     // GSI_OK or GSI_ERR_TIMEOUT (sticky until read by gsi_workspace_status)
  unsigned pad[59];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

// ---------------------------------------------------------------------------------------------
// Persistent decode kernel (tokens processed one at a time through the sites)
// ---------------------------------------------------------------------------------------------
constexpr int kReplicas = 8;       // one mailbox copy per XCD
constexpr int kMaxBlocks = 256;    // persistent blocks (one per CU)
constexpr int kMaxK = 512;
constexpr int kSyncThreads = 64;   // 1 sync wave
constexpr int kDecodeThreads = kDataThreads + kSyncThreads;
constexpr int kYPart = 2048;         // rows of y per block held in LDS before they are stored
constexpr int kMinBlocks = kMaxK / 4;  // the decode grid needs at least this many blocks

struct DecodeArgs {
  const PlanRow* plan;  // [n_sites][P]
  int n_sites, n_steps, t_step;
  const void* X;
  long long x_ld;
  void* Y;
  long long y_ld;
  uint8_t* gates;
  float* rho;
  int gate_ld;
  float eps;
  void* ws;  // workspace: header and mailboxes (decode_ws_bytes)
  int P, xr;
};

size_t decode_ws_bytes();
// input window (16-byte chunks per data thread) the kernel needs for these sites
int decode_window(int dtype, const LayerDesc* sites, int n_sites);
// co-resident grid (a power of two >= kMinBlocks) for the kernel with that window; 0 if none
int decode_grid(int dtype, int xr);
// plan rows of one site for a grid of P blocks, computed on the device into out[0..P)
int launch_plan(const LayerDesc& d, int P, int es, PlanRow* out, hipStream_t s);
int launch_decode(int dtype, const DecodeArgs& a, hipStream_t s);
// the same kernel and grid as an ordinary (not cooperative) launch, for one-token calls
int launch_decode_resident(int dtype, const DecodeArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Dense helpers (create time and the batched path)
// ---------------------------------------------------------------------------------------------
// C[m, n] = alpha-free sum_i A[a_row(m), i] * B[n, i]  (both operands K-contiguous, "NT")
//   a_idx: optional row gather for A (device int32 list), c_idx: optional row scatter for C,
//   m_count: optional device int32 giving the number of valid rows (else m).
//   sub_identity: C[m][n] -= (m == n) (for V^T V - I).
int launch_gemm_nt(int a_type, int b_type, int c_type, const void* A, long long lda, const int* a_idx,
                   const void* B, long long ldb, void* C, long long ldc, const int* c_idx, int m, int n, int kdim,
                   const int* m_count, int sub_identity, hipStream_t s);
// Create-time products M = W V and V^T V - I (float32); with a workspace of at least
// precompute_ws_bytes() they run split over K with fixed-order reductions (0: no workspace used)
// and, for 16-bit weights, *dd receives the split D = V^T V - I that launch_vdt takes (inside ws;
// null on the path without a workspace)
size_t precompute_ws_bytes(int dtype, int d_out, int d, int k);
int launch_precompute(int dtype, const void* W, const void* Vt, void* M, float* Dl, int d_out, int d, int k,
                      void* ws, size_t ws_bytes, const void** dd, hipStream_t s);
// VDt[k, d] = (V (V^T V - I))^T from D = V^T V - I and V (d x k), in the weight dtype: one
// matrix-core product from dd when given, else from Dl (float32) on the vector ALU
int launch_vdt(int dtype, const float* Dl, const void* dd, const void* V, void* VDt, int d, int k, hipStream_t s);
// dst[k, d] = transpose(src[d, k]); with `plan` (P <= 256 entries), also the decode plan rows of
// the layer described by desc
int launch_transpose(int dtype, const void* src, void* dst, int d, int k, const LayerDesc& desc, int P,
                     PlanRow* plan, hipStream_t s);
// float32 C[m, n] = A B^T for a small output and a long K, K split over blocks (partial sums in
// part, at least part_elems floats), reduced in chunk order
int launch_gemm_nt_f32_splitk(const float* A, long long lda, const float* B, long long ldb, float* C, long long ldc,
                              int m, int n, int kdim, float* part, long long part_elems, hipStream_t s);

struct BatchedWs {
  float* G;      // [T, k]  g = V^T x per token
  float* H;      // [T, k]  (V^T V - I) g per token
  float* nx2;    // [T]
  int* fast_idx; // [T]
  int* slow_idx; // [T]
  int* counts;   // [2]
  float* part;   // [kMaxSplit, T, d_out] split-K partial sums of the fast product (and the projection)
  float* part2;  // [kMaxSplit, T, d_out] split-K partial sums of the slow product
  long long part_elems;
  // two-launch path (chunks of at most 64 tokens), two sets of the projection's outputs: one
  // launch writes one set while the products of the same launch read the other
  float* Pp[2];    // [kMaxProjChunks][64][2 k] projection chunk sums
  float* gq[2];    // [64][kMaxK / 16][2] per token and 32-column tile: sum g^2, sum g h
  float* nx2p[2];  // [64][kMaxProjChunks] per token, chunk sums of |x|^2
  int* cnt;        // [kBatchedCounters] arrival counters (projection tiles, then row tiles), zero between launches
};
constexpr int kMaxProjChunks = 16;
constexpr int kMaxProdChunks = 4;  // K chunks of the two-launch path's products
constexpr int kBatchedCounters = 4096;  // arrival counters of the two-launch path (16 KB)
// K chunks of the two-launch batched path of one site (zp == 0 and zy == 0: not applicable)
struct BatchedSplit {
  int zp, kc;         // projection: chunks of x's K and their width
  int zy, kcw, kcm;   // products: chunks of W's K (slow product) and their width; M's chunk width
  int zf;             // chunks of M's K (fast product, one or none)
};
constexpr int kMaxSplit = 8;  // K chunks of a split product
// partial-sum elements the batched path may use (none when every call runs one token)
inline long long split_part_elems(int T, int d_out) { return T > 1 ? (long long)kMaxSplit * T * d_out : 0; }
size_t batched_ws_bytes(int k, int T, int d_out);
BatchedWs batched_ws_carve(void* base, int k, int T, int d_out);
int launch_gemm_nt_split(int a_type, int b_type, int c_type, const void* A, long long lda, const int* a_idx,
                         const void* B, long long ldb, void* C, long long ldc, const int* c_idx, int m, int n,
                         int kdim, const int* m_count, float* part, long long part_elems, hipStream_t s);
// the skinny kernel's K chunks for an m <= 64 row product (0: not applicable), its partial sums
// without reduction, and one reduction of two token lists into C
int skinny_splits(int a_type, int b_type, int m, int n, int kdim, long long part_elems);
int launch_skinny_partials(int a_type, int b_type, const void* A, long long lda, const int* a_idx, const void* B,
                           long long ldb, int m, int n, int kdim, const int* m_count, int splits, float* part,
                           hipStream_t s);
int launch_reduce2(int c_type, const float* pa, int sa, const int* ca, const int* ia, const float* pb, int sb,
                   const int* cb, const int* ib, int m, int n, void* C, long long ldc, hipStream_t s);
int launch_gate_batched(int dtype, const LayerDesc& L, const void* X, long long x_ld, int T, float eps,
                        const BatchedWs& w, uint8_t* gate, int gate_ld, float* rho, hipStream_t s);
BatchedSplit batched_split(int dtype, const LayerDesc& L, int ntok);
// One site over ntok <= 64 tokens on the two-launch path: its projection (g split in two 16-bit
// halves, the gate pieces) writes buffer set `set`, which its products read.
struct BatchedUnit {
  const LayerDesc* L;
  BatchedSplit sp;
  const void* X;
  long long x_ld;
  int ntok;
  float eps;
  void* Y;
  long long y_ld;
  uint8_t* gate;
  int gate_ld;
  float* rho;
  const BatchedWs* w;
  int set;  // 0 or 1
};
// One launch: the projection of `proj` and the products of `prod` (either may be null; a dense
// site's projection is skipped); the two must use different buffer sets.
int launch_batched_step(int dtype, const BatchedUnit* proj, const BatchedUnit* prod, hipStream_t s);

}  // namespace gsi
