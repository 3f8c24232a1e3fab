// The kernels of one batch-1 decode step of a GPT-J-shaped parallel block that are not GSI sites:
// LayerNorm, plain softmax attention over the key/value cache, GELU and the residual add. The
// pages run every linear map as a GSI site and leave attention unchanged [GSI §3 item 4, §5];
// the block's form (one LayerNorm feeding attention and MLP, tanh GELU, no positional rotation)
// is the plainest GPT-J-shaped reading. All arithmetic is float32 on 16-bit stored values; every
// result is rounded once to the stored type.
#include <algorithm>
#include <cmath>

#include "gsi_step.h"

namespace gsi {

namespace {

template <typename T>
__device__ __forceinline__ T bits_as(unsigned short v) {
  T t;
  t.b = v;
  return t;
}

// EPL consecutive 16-bit elements starting at p (aligned to 2 EPL bytes), as float32
template <typename T, int EPL>
__device__ __forceinline__ void load_row(const T* p, float (&out)[EPL]) {
  const unsigned short* q = reinterpret_cast<const unsigned short*>(p);
  if constexpr (EPL == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(q);
    out[0] = to_f32(bits_as<T>(v.x & 0xffffu));
    out[1] = to_f32(bits_as<T>(v.x >> 16));
    out[2] = to_f32(bits_as<T>(v.y & 0xffffu));
    out[3] = to_f32(bits_as<T>(v.y >> 16));
  } else if constexpr (EPL == 2) {
    const unsigned v = *reinterpret_cast<const unsigned*>(q);
    out[0] = to_f32(bits_as<T>(v & 0xffffu));
    out[1] = to_f32(bits_as<T>(v >> 16));
  } else {
    out[0] = to_f32(bits_as<T>(q[0]));
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// sum over the block's waves in wave order (deterministic); every thread gets the result
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // red is free
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[w];
  return s;
}

// LayerNorm blocks: 1024 threads; thread t holds the groups of 4 consecutive row elements
// 4096 c + 4 t .. + 3 (c < kLnChunks; d a multiple of 4, d <= 16384), read and written 8 bytes at
// a time, with gamma and beta loaded together with the row
constexpr int kLnChunks = 16384 / 4096;
template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]) {
  const T a0 = from_f32<T>(v[0]), a1 = from_f32<T>(v[1]), a2 = from_f32<T>(v[2]), a3 = from_f32<T>(v[3]);
  uint2 w;
  w.x = (unsigned)a0.b | ((unsigned)a1.b << 16);
  w.y = (unsigned)a2.b | ((unsigned)a3.b << 16);
  *reinterpret_cast<uint2*>(p) = w;
}
// LayerNorm of the row held in v (groups as above, zero past d), written twice to xa: the stack's
// two sites read the same input
template <typename T>
__device__ __forceinline__ void ln_dup_row(const float (&v)[kLnChunks][4], const float (&gm)[kLnChunks][4],
                                           const float (&bt)[kLnChunks][4], int d, T* __restrict__ xa,
                                           float* red) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += v[c][e];
  const float mean = block_sum<16>(s, red) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    if (4096 * c + 4 * (int)threadIdx.x < d) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dv = v[c][e] - mean;
        q = __builtin_fmaf(dv, dv, q);
      }
    }
  }
  const float var = block_sum<16>(q, red) / (float)d;
  const float rs = 1.0f / sqrtf(var + kLnEps);
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int i = 4096 * c + 4 * (int)threadIdx.x;
    if (i < d) {
      float a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = (v[c][e] - mean) * rs * gm[c][e] + bt[c][e];
      store4<T>(xa + i, a);
      store4<T>(xa + d + i, a);
    }
  }
}
template <typename T>
__global__ __launch_bounds__(1024) void ln_dup_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                                                      const T* __restrict__ beta, int d, T* __restrict__ xa) {
  __shared__ float red[16];
  float v[kLnChunks][4], gm[kLnChunks][4], bt[kLnChunks][4];
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int i = 4096 * c + 4 * (int)threadIdx.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[c][e] = gm[c][e] = bt[c][e] = 0.f;
    if (i < d) {
      load_row<T, 4>(x + i, v[c]);
      load_row<T, 4>(gamma + i, gm[c]);
      load_row<T, 4>(beta + i, bt[c]);
    }
  }
  ln_dup_row<T>(v, gm, bt, d, xa, red);
}
// x += yb[0:d] + yb[d:2d] (rounded and stored), then the next block's LayerNorm of the stored row
// to xa: the same values as the residual kernel followed by ln_dup_kernel, in one launch
template <typename T>
__global__ __launch_bounds__(1024) void residual_ln_kernel(T* __restrict__ x, const T* __restrict__ yb,
                                                           const T* __restrict__ gamma, const T* __restrict__ beta,
                                                           int d, T* __restrict__ xa) {
  __shared__ float red[16];
  float v[kLnChunks][4], gm[kLnChunks][4], bt[kLnChunks][4];
#pragma unroll
  for (int c = 0; c < kLnChunks; ++c) {
    const int i = 4096 * c + 4 * (int)threadIdx.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[c][e] = gm[c][e] = bt[c][e] = 0.f;
    if (i < d) {
      float xv[4], y0[4], y1[4];
      load_row<T, 4>(x + i, xv);
      load_row<T, 4>(yb + i, y0);
      load_row<T, 4>(yb + d + i, y1);
      load_row<T, 4>(gamma + i, gm[c]);
      load_row<T, 4>(beta + i, bt[c]);
      float xn[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xn[e] = (xv[e] + y0[e]) + y1[e];
        v[c][e] = to_f32(from_f32<T>(xn[e]));
      }
      store4<T>(x + i, xn);
    }
  }
  ln_dup_row<T>(v, gm, bt, d, xa, red);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {  // this wave's vector memory operations, down to N
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One launch: blocks 0 .. H nsplit - 1 are (head h, chunk c) = (i / nsplit, i mod nsplit) of the
// attention, the rest compute u = gelu(f) for 256 elements each (f = ya[3d:3d+dff], u to
// xb[d:d+dff]).
// Attention block (h, c): head h over the positions of chunk c, [c lc, min(L, (c + 1) lc)),
// L = pos + 1. Wave w takes positions c lc + w, + 4, ...; lane l holds elements EPL l .. + EPL - 1 of
// the head. Per group of positions: the scores <q, k> / sqrt(dh) (wave sums), then the running
// maximum m, the running sum l of exp(s - m) and the running exp(s - m)-weighted sum of the value
// rows. The
// four waves are merged through LDS and the chunk's (m, l, sums) stored with device-scope stores;
// the head's last chunk to arrive (counter cnt[h], zero between launches) adds the chunks in chunk
// order, o_h = sum_c e^(m_c - M) sums_c / sum_c e^(m_c - M) l_c, to xb[h dh ..]. Position pos reads
// the new token's k and v from ya, and the chunk holding it writes them into row pos of the caches.
// Position chunks of the attention over L positions with n_heads heads: at most
// split_count_max(n_heads), chunks of at least 16 positions (the same rule on the host and in
// the kernel).
__host__ __device__ inline int split_count_max(int n_heads) {
  const int want = (512 + n_heads - 1) / n_heads;
  return want < 1 ? 1 : (want > kMaxAttnSplit ? kMaxAttnSplit : want);
}
__host__ __device__ inline int split_count(int L, int n_heads) {
  const int want = split_count_max(n_heads);
  const int lc0 = (L + want - 1) / want;
  const int lc = lc0 < 16 ? 16 : lc0;
  return (L + lc - 1) / lc;
}

// pos_dev (optional): the position is read from device memory instead (a step replayed from a
// captured graph); the grid then holds gsplit = split_count_max(n_heads) chunk blocks per head,
// those past the position's chunk count leave at once, and a position outside [0, cap) runs no
// attention block (nothing is written to the caches).
template <typename T, int EPL>
__global__ __launch_bounds__(256) void attn_gelu_kernel(const T* __restrict__ ya, T* __restrict__ kc,
                                                        T* __restrict__ vc, int pos_arg, int d, int n_heads,
                                                        int lc_arg, int nsplit_arg, float* __restrict__ part,
                                                        int* __restrict__ cnt, int dff, T* __restrict__ xb,
                                                        uint8_t* __restrict__ gate_dup, float* __restrict__ rho_dup,
                                                        const int* __restrict__ pos_dev, int cap, int gsplit) {
  constexpr int dh = 64 * EPL;
  int pos = pos_arg, lc = lc_arg, nsplit = nsplit_arg;
  if (pos_dev) {
    pos = *pos_dev;
    const int L = pos + 1;
    nsplit = split_count(L > 0 ? L : 1, n_heads);
    lc = (L + nsplit - 1) / nsplit;
  }
  // a shared-input site's gate (and ratio), decided by the stack launch before this one, is
  // reported for both of its maps
  if (gate_dup && blockIdx.x == 0 && threadIdx.x == 0) {
    gate_dup[1] = gate_dup[0];
    if (rho_dup) rho_dup[1] = rho_dup[0];
  }
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[4][dh];
  __shared__ int s_last;
  const int na = n_heads * gsplit;
  if ((int)blockIdx.x >= na) {
    const int i = ((int)blockIdx.x - na) * 256 + threadIdx.x;
    if (i >= dff) return;
    const float z = to_f32(ya[3 * (long long)d + i]);
    const float u = 0.5f * z * (1.0f + tanhf(0.7978845608028654f * (z + 0.044715f * z * z * z)));
    xb[d + i] = from_f32<T>(u);
    return;
  }
  const int h = blockIdx.x / gsplit, c = blockIdx.x % gsplit;
  if (pos_dev && (pos < 0 || pos >= cap || c >= nsplit)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = h * dh + lane * EPL;
  const int j0 = c * lc, j1 = min(pos + 1, j0 + lc);
  float q[EPL];
  load_row<T, EPL>(ya + col, q);
  const float scale = 1.0f / sqrtf((float)dh);
  if (wave == 0 && pos >= j0 && pos < j1) {
    // the new token joins the caches (this launch reads row pos from ya only)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      kc[(long long)pos * d + col + e] = ya[d + col + e];
      vc[(long long)pos * d + col + e] = ya[2 * d + col + e];
    }
  }
  float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  // PP positions of the wave at a time (positions jb, jb + 4, ...): every key and value row
  // loaded first, then PP independent scores, then one rescale of the running sums
  constexpr int PP = 8;
  for (int jb = j0 + wave; jb < j1; jb += 4 * PP) {
    float kv[PP][EPL], vv[PP][EPL];
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      const int j = jb + 4 * p;
      const int jr = j < j1 ? j : jb;  // rows past the chunk read a valid row and are not used
      const T* kr = jr == pos ? ya + d : kc + (long long)jr * d;
      const T* vr = jr == pos ? ya + 2 * d : vc + (long long)jr * d;
      load_row<T, EPL>(kr + col, kv[p]);
      load_row<T, EPL>(vr + col, vv[p]);
    }
    float sc[PP];
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(q[e], kv[p][e], dot);
      sc[p] = wave_sum(dot) * scale;
    }
    float mn = m;
#pragma unroll
    for (int p = 0; p < PP; ++p)
      if (jb + 4 * p < j1) mn = fmaxf(mn, sc[p]);
    const float cf = expf(m - mn);
    l *= cf;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= cf;
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      if (jb + 4 * p < j1) {
        const float w = expf(sc[p] - mn);
        l += w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(w, vv[p][e], acc[e]);
      }
    }
    m = mn;
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[wave][lane * EPL + e] = acc[e];
  __syncthreads();
  float* ph = part + (long long)h * nsplit * (dh + 2);
  float* out = ph + (long long)c * (dh + 2);
  const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  if (threadIdx.x < dh) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) a += s_acc[w][threadIdx.x] * expf(s_m[w] - M);
    __hip_atomic_store(out + 2 + threadIdx.x, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == 0) {
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += s_l[w] * expf(s_m[w] - M);
    __hip_atomic_store(out, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(out + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // hand-off: every wave's stores complete, then one count per block; the last chunk combines
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&cnt[h], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
  __syncthreads();
  if (!s_last) return;
  // one device-scope acquire, then ordinary loads: the chunks' maxima and sums through LDS, the
  // value sums straight from memory, all independent
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __shared__ float s_cm[kMaxAttnSplit], s_cl[kMaxAttnSplit];
  if ((int)threadIdx.x < nsplit) {
    s_cm[threadIdx.x] = ph[(long long)threadIdx.x * (dh + 2)];
    s_cl[threadIdx.x] = ph[(long long)threadIdx.x * (dh + 2) + 1];
  }
  __syncthreads();
  float Mx = -INFINITY;
  for (int cc = 0; cc < nsplit; ++cc) Mx = fmaxf(Mx, s_cm[cc]);
  if (threadIdx.x < dh) {
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int cc = 0; cc < nsplit; ++cc) {
      const float w = expf(s_cm[cc] - Mx);
      den = __builtin_fmaf(s_cl[cc], w, den);
      num = __builtin_fmaf(ph[(long long)cc * (dh + 2) + 2 + threadIdx.x], w, num);
    }
    xb[h * dh + threadIdx.x] = from_f32<T>(num / den);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&cnt[h], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__global__ __launch_bounds__(256) void residual_kernel(T* __restrict__ x, const T* __restrict__ yb, int d) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < d) x[i] = from_f32<T>((to_f32(x[i]) + to_f32(yb[i])) + to_f32(yb[d + i]));
}

}  // namespace

int attn_splits(int L, int n_heads) { return split_count(L, n_heads); }

__global__ void pos_advance_kernel(int* pos) {
  if (threadIdx.x == 0) *pos += 1;
}

int launch_pos_advance(int* pos, hipStream_t s) {
  pos_advance_kernel<<<1, 64, 0, s>>>(pos);
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

// partial sums, then one arrival counter per head (zero between launches)
size_t attn_ws_bytes(int d, int n_heads) {
  return align256((size_t)kMaxAttnSplit * (d + 2 * (size_t)n_heads) * 4) + align256((size_t)n_heads * 4);
}

int launch_ln_dup(int dtype, const void* x, const void* gamma, const void* beta, int d, void* xa, hipStream_t s) {
  if (d < 4 || d > 16384 || d % 4 != 0) return GSI_ERR_SHAPE;
  if (dtype == GSI_BF16)
    ln_dup_kernel<bf16_t><<<1, 1024, 0, s>>>((const bf16_t*)x, (const bf16_t*)gamma, (const bf16_t*)beta, d,
                                             (bf16_t*)xa);
  else if (dtype == GSI_F16)
    ln_dup_kernel<f16_t><<<1, 1024, 0, s>>>((const f16_t*)x, (const f16_t*)gamma, (const f16_t*)beta, d,
                                            (f16_t*)xa);
  else
    return GSI_ERR_DTYPE;
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

template <typename T, int EPL>
static void attention_launch(const void* ya, void* kc, void* vc, int pos, int d, int n_heads, int dff, void* xb,
                             float* part, uint8_t* gate_dup, float* rho_dup, const int* pos_dev, int cap,
                             hipStream_t s) {
  const int L = pos + 1;
  const int nsplit = attn_splits(L, n_heads);
  const int lc = (L + nsplit - 1) / nsplit;
  const int gsplit = pos_dev ? split_count_max(n_heads) : nsplit;
  int* cnt = (int*)((char*)part + align256((size_t)kMaxAttnSplit * (d + 2 * (size_t)n_heads) * 4));
  const unsigned nb = (unsigned)(n_heads * gsplit + (dff + 255) / 256);
  attn_gelu_kernel<T, EPL><<<nb, 256, 0, s>>>((const T*)ya, (T*)kc, (T*)vc, pos, d, n_heads, lc, nsplit, part, cnt,
                                               dff, (T*)xb, gate_dup, rho_dup, pos_dev, cap, gsplit);
}

int launch_attention_gelu(int dtype, const void* ya, void* k_cache, void* v_cache, int pos, int d, int n_heads,
                          int dff, void* xb, float* part, uint8_t* gate_dup, float* rho_dup, const int* pos_dev,
                          int cap, hipStream_t s) {
  if (n_heads < 1 || d % n_heads != 0 || pos < 0) return GSI_ERR_SHAPE;
  const int dh = d / n_heads;
  const bool bf = dtype == GSI_BF16;
  if (dtype != GSI_BF16 && dtype != GSI_F16) return GSI_ERR_DTYPE;
  if (dh == 64) {
    if (bf) attention_launch<bf16_t, 1>(ya, k_cache, v_cache, pos, d, n_heads, dff, xb, part, gate_dup, rho_dup, pos_dev, cap, s);
    else attention_launch<f16_t, 1>(ya, k_cache, v_cache, pos, d, n_heads, dff, xb, part, gate_dup, rho_dup, pos_dev, cap, s);
  } else if (dh == 128) {
    if (bf) attention_launch<bf16_t, 2>(ya, k_cache, v_cache, pos, d, n_heads, dff, xb, part, gate_dup, rho_dup, pos_dev, cap, s);
    else attention_launch<f16_t, 2>(ya, k_cache, v_cache, pos, d, n_heads, dff, xb, part, gate_dup, rho_dup, pos_dev, cap, s);
  } else if (dh == 256) {
    if (bf) attention_launch<bf16_t, 4>(ya, k_cache, v_cache, pos, d, n_heads, dff, xb, part, gate_dup, rho_dup, pos_dev, cap, s);
    else attention_launch<f16_t, 4>(ya, k_cache, v_cache, pos, d, n_heads, dff, xb, part, gate_dup, rho_dup, pos_dev, cap, s);
  } else {
    return GSI_ERR_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

int launch_residual_ln(int dtype, void* x, const void* yb, const void* gamma, const void* beta, int d, void* xa,
                      hipStream_t s) {
  if (d < 4 || d > 16384 || d % 4 != 0) return GSI_ERR_SHAPE;
  if (dtype == GSI_BF16)
    residual_ln_kernel<bf16_t><<<1, 1024, 0, s>>>((bf16_t*)x, (const bf16_t*)yb, (const bf16_t*)gamma,
                                                  (const bf16_t*)beta, d, (bf16_t*)xa);
  else if (dtype == GSI_F16)
    residual_ln_kernel<f16_t><<<1, 1024, 0, s>>>((f16_t*)x, (const f16_t*)yb, (const f16_t*)gamma,
                                                 (const f16_t*)beta, d, (f16_t*)xa);
  else
    return GSI_ERR_DTYPE;
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

int launch_residual(int dtype, void* x, const void* yb, int d, hipStream_t s) {
  const unsigned nb = (unsigned)((d + 255) / 256);
  if (dtype == GSI_BF16)
    residual_kernel<bf16_t><<<nb, 256, 0, s>>>((bf16_t*)x, (const bf16_t*)yb, d);
  else if (dtype == GSI_F16)
    residual_kernel<f16_t><<<nb, 256, 0, s>>>((f16_t*)x, (const f16_t*)yb, d);
  else
    return GSI_ERR_DTYPE;
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

}  // namespace gsi
