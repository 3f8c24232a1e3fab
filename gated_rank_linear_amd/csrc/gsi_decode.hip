// Persistent batch-1 GSI decode kernel for gfx950.
//
// Method: "Gated Subspace Inference for transformer acceleration" technical summary
// (gist.science, arXiv 2605.03109). Per token and per site (linear layer) [GSI §2.1-§2.2]:
//   g = V^T x;  nr2 = |x - V g|^2 = |x|^2 - |g|^2 + g^T (V^T V - I) g;  fast iff nr2 < eps^2 |x|^2
//   fast: y = M g (M = W V cached)      slow: y = W x
// Every linear site of every block runs in order [GSI §3], one token at a time.
//
// Design (one block per CU, all blocks co-resident via a cooperative launch):
//  * Work split per site: block b owns the g columns j = b, b + P, ... (rows of V^T, contiguous
//    d-long rows, so each g_j is a complete dot product inside one block) and a contiguous slice
//    of output rows of M / W. The slice of every site is prefetched into registers while the
//    previous site is still waiting on its exchanges, so HBM reads overlap synchronisation.
//  * Two all-gather exchanges per site: (E1) every block needs all of g for its rows of M g;
//    (E2) the gate needs the global sum of per-block pieces of g^T (V^T V - I) g, and its
//    completion also means every block has written its rows of y. A slow token adds (E3), the
//    completion of the W x rows.
//  * Exchanges use tagged 64-bit mailbox words (tag << 32 | payload) with one copy per XCD, so
//    a block polls the copy its own XCD reads most cheaply; stores and polls are device-scope.
//    Tags grow monotonically across launches (base kept in the workspace header), so no
//    clearing is needed. A mailbox slot is rewritten only after every reader has consumed it
//    (the other exchange sits between two uses), which the ordering E1 < E2 < E1 ... guarantees.
//  * One wave per block (the sync wave) does all polling; four data waves do loads and math.
//    Every wait is bounded: past the bound the kernel records GSI_ERR_TIMEOUT and all blocks
//    leave, so a lost block can never hang the device.
//  * Gate arithmetic is done identically (same data, same order) in every block, so all blocks
//    take the same branch.
#include "gsi_internal.h"

namespace gsi {

constexpr int kMaxJ = 4;        // g columns per block (k <= 512, P >= 128)
constexpr int kVRegs = 16;      // prefetched 16-byte chunks per data thread for V^T rows
constexpr int kMRegs = 16;      // ... for M rows
constexpr int kDRegs = 4;       // ... for (V^T V - I) rows
constexpr unsigned long long kWaitTicks = 200000000ull;  // 2 s at the 100 MHz wall clock

__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xfu;
}
__device__ __forceinline__ u64 ld_dev(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_dev(u64* p, u64 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u64 pack(unsigned tag, float v) { return ((u64)tag << 32) | (u64)__float_as_uint(v); }

template <typename T>
__device__ __forceinline__ float dot_chunk(const uint4& a, const uint4& b, float acc) {
  float fa[vec16<T>::N], fb[vec16<T>::N];
  unpack16<T>(a, fa);
  unpack16<T>(b, fb);
#pragma unroll
  for (int i = 0; i < vec16<T>::N; ++i) acc = __builtin_fmaf(fa[i], fb[i], acc);
  return acc;
}
template <typename T>
__device__ __forceinline__ float sq_chunk(const uint4& a, float acc) {
  float fa[vec16<T>::N];
  unpack16<T>(a, fa);
#pragma unroll
  for (int i = 0; i < vec16<T>::N; ++i) acc = __builtin_fmaf(fa[i], fa[i], acc);
  return acc;
}
// 16-byte chunk of T elements against 16/sizeof(T) consecutive float32 values in LDS
template <typename T>
__device__ __forceinline__ float dot_chunk_lds(const uint4& a, const float* g, float acc) {
  float fa[vec16<T>::N];
  unpack16<T>(a, fa);
#pragma unroll
  for (int i = 0; i < vec16<T>::N; ++i) acc = __builtin_fmaf(fa[i], g[i], acc);
  return acc;
}
__device__ __forceinline__ float dot_f32x4_lds(const uint4& a, const float* g, float acc) {
  acc = __builtin_fmaf(__uint_as_float(a.x), g[0], acc);
  acc = __builtin_fmaf(__uint_as_float(a.y), g[1], acc);
  acc = __builtin_fmaf(__uint_as_float(a.z), g[2], acc);
  acc = __builtin_fmaf(__uint_as_float(a.w), g[3], acc);
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float group_sum(float v, int width) {  // width: power of two <= 64
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

struct SiteGeom {
  int d, d_out, k;
  int nJ;        // g columns owned by this block
  int cprd;      // 16-byte chunks per V^T / W row (d / VW)
  int cprk;      // 16-byte chunks per M row (k / VW)
  int r0, nrows; // output rows owned
};

template <typename T>
__device__ __forceinline__ SiteGeom geom(const LayerDesc& L, int b, int P) {
  constexpr int VW = vec16<T>::N;
  SiteGeom g;
  g.d = L.d; g.d_out = L.d_out; g.k = L.k;
  g.nJ = b < L.k ? (L.k - 1 - b) / P + 1 : 0;
  g.cprd = L.d / VW;
  g.cprk = L.k / VW;
  const int rpb = (L.d_out + P - 1) / P;
  g.r0 = min(L.d_out, b * rpb);
  g.nrows = min(L.d_out, g.r0 + rpb) - g.r0;
  return g;
}

// Issue the loads of one site's block-owned weight slices into registers.
template <typename T>
__device__ __forceinline__ void prefetch_site(const LayerDesc& L, const SiteGeom& g, int b, int P, int tid,
                                              uint4 (&vreg)[kVRegs], uint4 (&mreg)[kMRegs], uint4 (&dreg)[kDRegs]) {
  constexpr int VW = vec16<T>::N;
  const uint4* vt = reinterpret_cast<const uint4*>(L.Vt);
  const int nv = g.nJ * g.cprd;
#pragma unroll
  for (int u = 0; u < kVRegs; ++u) {
    const int c = tid + u * kDataThreads;
    if (c < nv) {
      const int jl = c / g.cprd, cc = c - jl * g.cprd;
      const long long j = b + (long long)jl * P;
      vreg[u] = vt[j * g.cprd + cc];
    }
  }
  const uint4* m = reinterpret_cast<const uint4*>(L.M) + (long long)g.r0 * g.cprk;
  const int nm = g.nrows * g.cprk;
#pragma unroll
  for (int u = 0; u < kMRegs; ++u) {
    const int c = tid + u * kDataThreads;
    if (c < nm) mreg[u] = *(m + c);
  }
  const int cpk4 = g.k / 4;  // float32 chunks per (V^T V - I) row
  const int nd = g.nJ * cpk4;
  const uint4* dl = reinterpret_cast<const uint4*>(L.Dl);
#pragma unroll
  for (int u = 0; u < kDRegs; ++u) {
    const int c = tid + u * kDataThreads;
    if (c < nd) {
      const int jl = c / cpk4, cc = c - jl * cpk4;
      const long long j = b + (long long)jl * P;
      dreg[u] = dl[j * cpk4 + cc];
    }
  }
  (void)VW;
}

// A block whose wait runs past its bound marks this launch (tag base + 1) as aborted; every other
// block polls that mark while it waits, so the whole grid leaves promptly. The mark of an older
// launch never matches because every launch advances the tag base.
__device__ __forceinline__ bool aborted(const DecodeParams& p, unsigned base) {
  return __hip_atomic_load(&p.hdr->abort_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == base + 1u;
}
__device__ __forceinline__ void record_abort(const DecodeParams& p, unsigned base) {
  __hip_atomic_store(&p.hdr->abort_tag, base + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p.hdr->status, (int)GSI_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
  constexpr int VW = vec16<T>::N;
  __shared__ float gsh[kMaxK];
  __shared__ float red[kDecodeThreads / 64][kMaxJ + 2];
  __shared__ float ypart[256];
  __shared__ float s_nx2, s_gg, s_gj[kMaxJ];
  __shared__ int s_gate, s_abort;
  __shared__ unsigned s_base;

  const int tid = threadIdx.x;
  const int b = blockIdx.x, P = gridDim.x;
  const bool is_sync = tid >= kDataThreads;
  const int lane = tid & 63, wave = tid >> 6;
  const unsigned rep = xcc_id() % kReplicas;

  if (tid == 0) {
    s_abort = 0;
    s_base = __hip_atomic_load(&p.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const unsigned base = s_base;
  const long long Q = (long long)p.n_tokens * p.n_sites;

  uint4 vreg[kVRegs], mreg[kMRegs], dreg[kDRegs];
  if (!is_sync && Q > 0) {
    const LayerDesc& L0 = p.sites ? p.sites[0] : p.one;
    prefetch_site<T>(L0, geom<T>(L0, b, P), b, P, tid, vreg, mreg, dreg);
  }

  for (long long q = 0; q < Q; ++q) {
    const int t = (int)(q / p.n_sites), s = (int)(q - (long long)t * p.n_sites);
    const LayerDesc L = p.sites ? p.sites[s] : p.one;
    const SiteGeom g = geom<T>(L, b, P);
    const unsigned tag = base + (unsigned)(q * 4);
    const unsigned tag_g = tag + 1, tag_p = tag + 2, tag_f = tag + 3;
    const T* x = reinterpret_cast<const T*>(p.X) + (long long)t * p.x_ld + L.x_off;
    const uint4* x4 = reinterpret_cast<const uint4*>(x);

    // ---------------- phase A: g_j for owned columns, |x|^2 ----------------
    if (!is_sync) {
      float acc[kMaxJ];
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) acc[j] = 0.f;
      const int nv = g.nJ * g.cprd;
#pragma unroll
      for (int u = 0; u < kVRegs; ++u) {
        const int c = tid + u * kDataThreads;
        if (c < nv) {
          const int jl = c / g.cprd, cc = c - jl * g.cprd;
          const uint4 xv = x4[cc];
          const float part = dot_chunk<T>(vreg[u], xv, 0.f);
#pragma unroll
          for (int j = 0; j < kMaxJ; ++j) acc[j] += (j == jl) ? part : 0.f;
        }
      }
      // rows longer than the prefetch window (very large d): stream the rest now
      for (int c = tid + kVRegs * kDataThreads; c < nv; c += kDataThreads) {
        const int jl = c / g.cprd, cc = c - jl * g.cprd;
        const long long j = b + (long long)jl * P;
        const uint4 vv = reinterpret_cast<const uint4*>(L.Vt)[j * g.cprd + cc];
        const float part = dot_chunk<T>(vv, x4[cc], 0.f);
#pragma unroll
        for (int jj = 0; jj < kMaxJ; ++jj) acc[jj] += (jj == jl) ? part : 0.f;
      }
      float sx = 0.f;
      for (int c = tid; c < g.cprd; c += kDataThreads) sx = sq_chunk<T>(x4[c], sx);
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) acc[j] = wave_sum(acc[j]);
      sx = wave_sum(sx);
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) red[wave][j] = acc[j];
        red[wave][kMaxJ] = sx;
      }
    }
    __syncthreads();
    if (tid == 0) {
      const float nx2 = ((red[0][kMaxJ] + red[1][kMaxJ]) + red[2][kMaxJ]) + red[3][kMaxJ];
      s_nx2 = nx2;
      for (int jl = 0; jl < g.nJ; ++jl) {
        const float gj = ((red[0][jl] + red[1][jl]) + red[2][jl]) + red[3][jl];
        s_gj[jl] = gj;
        const long long j = b + (long long)jl * P;
        for (int r = 0; r < kReplicas; ++r) st_dev(p.box_g + (long long)r * kMaxK + j, pack(tag_g, gj));
      }
    }
    // ---------------- E1: all-gather g (sync wave) ----------------
    if (is_sync) {
      const u64* mb = p.box_g + (long long)rep * kMaxK;
      const unsigned long long t0 = wall_clock64();
      float gv[kMaxK / 64];
      while (true) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < kMaxK / 64; ++i) {
          const int j = lane + 64 * i;
          if (j < g.k) {
            const u64 w = ld_dev(mb + j);
            ok &= (unsigned)(w >> 32) == tag_g;
            gv[i] = __uint_as_float((unsigned)w);
          } else {
            gv[i] = 0.f;
          }
        }
        if (__all(ok)) break;
        if (wall_clock64() - t0 > kWaitTicks || aborted(p, base)) {
          if (lane == 0) {
            s_abort = 1;
            record_abort(p, base);
          }
          break;
        }
      }
      float gg = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxK / 64; ++i) {
        const int j = lane + 64 * i;
        if (j < g.k) gsh[j] = gv[i];
        gg = __builtin_fmaf(gv[i], gv[i], gg);
      }
      gg = wave_sum(gg);
      if (lane == 0) s_gg = gg;
    }
    __syncthreads();
    if (s_abort) break;

    // ---------------- phase B: p_b = sum_j g_j ((V^T V - I) g)_j and y = M g rows ----------------
    if (!is_sync) {
      const int cpk4 = g.k / 4;
      const int nd = g.nJ * cpk4;
      float pp = 0.f;
#pragma unroll
      for (int u = 0; u < kDRegs; ++u) {
        const int c = tid + u * kDataThreads;
        if (c < nd) {
          const int jl = c / cpk4, cc = c - jl * cpk4;
          pp += s_gj[jl] * dot_f32x4_lds(dreg[u], gsh + cc * 4, 0.f);
        }
      }
      for (int c = tid + kDRegs * kDataThreads; c < nd; c += kDataThreads) {
        const int jl = c / cpk4, cc = c - jl * cpk4;
        const long long j = b + (long long)jl * P;
        pp += s_gj[jl] * dot_f32x4_lds(reinterpret_cast<const uint4*>(L.Dl)[j * cpk4 + cc], gsh + cc * 4, 0.f);
      }
      pp = wave_sum(pp);
      if (lane == 0) red[wave][0] = pp;

      // y rows: the block's M slice is nrows * cprk contiguous chunks; chunk c = tid + u*256
      // belongs to row c / cprk. Rows are reduced inside lane groups of width min(cprk, 64)
      // and, for cprk > 64, across groups through LDS in index order.
      const int nm = g.nrows * g.cprk;
      const int gw = min(g.cprk, 64);
      const int segs = g.cprk / gw;
      T* yrow = reinterpret_cast<T*>(p.Y) + (long long)t * p.y_ld + L.y_off + g.r0;
#pragma unroll
      for (int u = 0; u < kMRegs; ++u) {
        const int c0 = u * kDataThreads;
        if (c0 >= nm) break;
        const int c = tid + c0;
        float v = 0.f;
        if (c < nm) v = dot_chunk_lds<T>(mreg[u], gsh + (c % g.cprk) * VW, 0.f);
        v = group_sum(v, gw);
        if (c < nm && (c % gw) == 0) {
          if (segs == 1) yrow[c / g.cprk] = from_f32<T>(v);
          else ypart[(c / gw) % 256] = v;
        }
      }
      for (int c0 = kMRegs * kDataThreads; c0 < nm; c0 += kDataThreads) {
        const int c = tid + c0;
        float v = 0.f;
        if (c < nm) v = dot_chunk_lds<T>(reinterpret_cast<const uint4*>(L.M)[(long long)g.r0 * g.cprk + c],
                                         gsh + (c % g.cprk) * VW, 0.f);
        v = group_sum(v, gw);
        if (c < nm && (c % gw) == 0) {
          if (segs == 1) yrow[c / g.cprk] = from_f32<T>(v);
          else ypart[(c / gw) % 256] = v;
        }
      }
    }
    __syncthreads();
    if (!is_sync) {
      const int gw = min(g.cprk, 64);
      const int segs = g.cprk / gw;
      if (segs > 1) {  // combine row segments in index order (nrows * segs <= 256 by construction)
        T* yrow = reinterpret_cast<T*>(p.Y) + (long long)t * p.y_ld + L.y_off + g.r0;
        for (int r = tid; r < g.nrows; r += kDataThreads) {
          float v = 0.f;
          for (int sg = 0; sg < segs; ++sg) v += ypart[(r * segs + sg) % 256];
          yrow[r] = from_f32<T>(v);
        }
      }
      if (tid == 0) {
        const float pb = ((red[0][0] + red[1][0]) + red[2][0]) + red[3][0];
        for (int r = 0; r < kReplicas; ++r) st_dev(p.box_p + (long long)r * kMaxBlocks + b, pack(tag_p, pb));
      }
      // prefetch the next site's slices while the gate is being resolved
      if (q + 1 < Q) {
        const int sn = (int)((q + 1) % p.n_sites);
        const LayerDesc& Ln = p.sites ? p.sites[sn] : p.one;
        prefetch_site<T>(Ln, geom<T>(Ln, b, P), b, P, tid, vreg, mreg, dreg);
      }
    } else {
      // ---------------- E2: all-gather the per-block pieces, resolve the gate ----------------
      const u64* mb = p.box_p + (long long)rep * kMaxBlocks;
      const unsigned long long t0 = wall_clock64();
      float pv[kMaxBlocks / 64];
      while (true) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < kMaxBlocks / 64; ++i) {
          const int bb = lane + 64 * i;
          if (bb < P) {
            const u64 w = ld_dev(mb + bb);
            ok &= (unsigned)(w >> 32) == tag_p;
            pv[i] = __uint_as_float((unsigned)w);
          } else {
            pv[i] = 0.f;
          }
        }
        if (__all(ok)) break;
        if (wall_clock64() - t0 > kWaitTicks || aborted(p, base)) {
          if (lane == 0) {
            s_abort = 1;
            record_abort(p, base);
          }
          break;
        }
      }
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxBlocks / 64; ++i) ps += pv[i];
      ps = wave_sum(ps);
      if (lane == 0) {
        const float nx2 = s_nx2;
        const float nr2 = (nx2 - s_gg) + ps;
        const float thr = p.eps * p.eps;
        const float rhs = thr * nx2;
        const int slow = (nr2 < rhs) ? 0 : 1;
        s_gate = slow;
        if (b == 0) {
          const long long o = (long long)t * p.gate_ld + p.site0 + s;
          p.gates[o] = (uint8_t)slow;
          if (p.rho) p.rho[o] = sqrtf(fmaxf(nr2, 0.f) / nx2);
        }
      }
    }
    __syncthreads();
    if (s_abort) break;

    // ---------------- slow path: y = W x for the owned rows, then E3 ----------------
    if (s_gate) {
      if (!is_sync) {
        const uint4* w4 = reinterpret_cast<const uint4*>(L.W);
        T* yrow = reinterpret_cast<T*>(p.Y) + (long long)t * p.y_ld + L.y_off;
        for (int r = g.r0 + wave; r < g.r0 + g.nrows; r += kDataThreads / 64) {
          const uint4* wr = w4 + (long long)r * g.cprd;
          float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
          int c = lane;
          for (; c + 192 < g.cprd; c += 256) {
            a0 = dot_chunk<T>(wr[c], x4[c], a0);
            a1 = dot_chunk<T>(wr[c + 64], x4[c + 64], a1);
            a2 = dot_chunk<T>(wr[c + 128], x4[c + 128], a2);
            a3 = dot_chunk<T>(wr[c + 192], x4[c + 192], a3);
          }
          for (; c < g.cprd; c += 64) a0 = dot_chunk<T>(wr[c], x4[c], a0);
          const float v = wave_sum((a0 + a1) + (a2 + a3));
          if (lane == 0) yrow[r] = from_f32<T>(v);
        }
      }
      __syncthreads();
      if (tid == 0)
        for (int r = 0; r < kReplicas; ++r) st_dev(p.box_f + (long long)r * kMaxBlocks + b, pack(tag_f, 0.f));
      if (is_sync) {
        const u64* mb = p.box_f + (long long)rep * kMaxBlocks;
        const unsigned long long t0 = wall_clock64();
        while (true) {
          bool ok = true;
#pragma unroll
          for (int i = 0; i < kMaxBlocks / 64; ++i) {
            const int bb = lane + 64 * i;
            if (bb < P) ok &= (unsigned)(ld_dev(mb + bb) >> 32) == tag_f;
          }
          if (__all(ok)) break;
          if (wall_clock64() - t0 > kWaitTicks || aborted(p, base)) {
            if (lane == 0) {
              s_abort = 1;
              record_abort(p, base);
            }
            break;
          }
        }
      }
      __syncthreads();
      if (s_abort) break;
    }
  }
  // advance the tag base for the next launch (also after an abort, so its mark goes stale)
  if (b == 0 && tid == 0)
    __hip_atomic_store(&p.hdr->epoch, base + (unsigned)(Q * 4) + 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

size_t decode_ws_bytes() {
  return sizeof(WsHeader) + (size_t)kReplicas * kMaxK * 8 + 2 * (size_t)kReplicas * kMaxBlocks * 8;
}

static const void* decode_fn(int dtype) {
  switch (dtype) {
    case GSI_F32: return (const void*)decode_kernel<float>;
    case GSI_F16: return (const void*)decode_kernel<f16_t>;
    case GSI_BF16: return (const void*)decode_kernel<bf16_t>;
  }
  return nullptr;
}

int decode_grid_blocks(int dtype) {
  const void* fn = decode_fn(dtype);
  if (!fn) return 0;
  int dev = 0, ncu = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kDecodeThreads, 0) != hipSuccess) return 0;
  long long cap = (long long)ncu * per;
  return (int)(cap < kMaxBlocks ? cap : kMaxBlocks);
}

int launch_decode(int dtype, const DecodeParams& prm, hipStream_t s) {
  const void* fn = decode_fn(dtype);
  if (!fn) return GSI_ERR_DTYPE;
  const int P = decode_grid_blocks(dtype);
  if (P < kMaxK / kMaxJ) return GSI_ERR_DEVICE;
  DecodeParams p = prm;
  void* args[] = {&p};
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(P), dim3(kDecodeThreads), args, 0, s);
  return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

}  // namespace gsi
