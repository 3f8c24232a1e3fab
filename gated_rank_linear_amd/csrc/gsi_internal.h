// Internal declarations shared by the libgsi translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/gsi.h"

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
struct LayerDesc {  // device-side description of one site (also used host-side)
  const void* Vt;     // [k, d]
  const void* M;      // [d_out, k]
  const float* Dl;    // [k, k] = V^T V - I
  const void* W;      // [d_out, d]
  int d, d_out, k, pad;
  long long x_off, y_off;  // column offsets into stacked X / Y rows
};

}  // namespace gsi

struct gsi_layer {
  int dtype, d_out, d, k;
  gsi::LayerDesc desc;       // x_off = y_off = 0
  gsi::LayerDesc* dev_desc;  // device copy, stored in the layer's aux buffer
};

struct gsi_stack {
  int dtype, n_sites, k_max, d_max, d_out_max;
  long long x_ld, y_ld;
  gsi::LayerDesc* d_table;  // device copy
  gsi::LayerDesc* h_table;  // host copy
  gsi_layer** layers;       // host copy of the borrowed handles
};

namespace gsi {

// Workspace header (start of every workspace)
struct WsHeader {
  unsigned epoch;  // exchange tag base, advanced by every persistent launch
  int status;      // GSI_OK or GSI_ERR_TIMEOUT (sticky until read by gsi_workspace_status)
  unsigned abort_tag;  // tag base + 1 of a launch that gave up waiting
  unsigned pad[61];
};

// ---------------------------------------------------------------------------------------------
// Persistent decode kernel (batch of n_tokens processed one token at a time through all sites)
// ---------------------------------------------------------------------------------------------
constexpr int kReplicas = 8;       // one mailbox copy per XCD
constexpr int kMaxBlocks = 256;    // persistent blocks (one per CU)
constexpr int kMaxK = 512;
constexpr int kDataThreads = 256;  // 4 data waves
constexpr int kSyncThreads = 64;   // 1 sync wave
constexpr int kDecodeThreads = kDataThreads + kSyncThreads;
constexpr int kRegionChunks = 4096;  // 16-byte chunks per LDS site region (two regions, 64 KB each)
constexpr int kYPart = 2048;         // rows of y per block held in LDS before they are stored
constexpr int kMinBlocks = kMaxK / 4;  // the decode grid needs at least this many blocks

struct DecodeParams {
  const LayerDesc* sites;  // device table of n_sites descriptors
  int n_sites, n_tokens;
  const void* X;
  long long x_ld;
  void* Y;
  long long y_ld;
  uint8_t* gates;  // [n_tokens, gate_ld]
  float* rho;      // optional
  int gate_ld, site0;  // column of site 0 in gates/rho
  float eps;
  int k_max, d_max;
  WsHeader* hdr;
  u64* box_g;  // [kReplicas][kMaxK]       g values
  u64* box_p;  // [kReplicas][kMaxBlocks]  per-block gate pieces
  u64* box_f;  // [kReplicas][kMaxBlocks]  slow-path completion
};

size_t decode_ws_bytes();
// host_sites: host copy of the n_sites descriptors (used to size the register windows)
int launch_decode(int dtype, const DecodeParams& p, const LayerDesc* host_sites, hipStream_t s);
// enqueue a copy of `d` (passed by value) into device memory `dst`
int launch_write_desc(const LayerDesc& d, LayerDesc* dst, hipStream_t s);

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
// dst[k, d] = transpose(src[d, k])
int launch_transpose(int dtype, const void* src, void* dst, int d, int k, hipStream_t s);
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

}  // namespace gsi
