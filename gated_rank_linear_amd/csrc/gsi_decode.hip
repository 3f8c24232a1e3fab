// Persistent batch-1 GSI decode kernel for gfx950.
//
// Method: "Gated Subspace Inference for transformer acceleration" technical summary
// (gist.science, arXiv 2605.03109). Per token and per site (linear layer) [GSI §2.1-§2.2]:
//   g = V^T x;  nr2 = |x - V g|^2 = |x|^2 - |g|^2 + g^T (V^T V - I) g;  fast iff nr2 < eps^2 |x|^2
//   fast: y = M g (M = W V cached)      slow: y = W x
// Every linear site of every block runs in order [GSI §3], one token at a time.
//
// Design (one block per CU, all blocks co-resident via a cooperative launch):
//  * Work split per site: block b owns the g columns j = b, b + P, ... (rows of V^T: each g_j is
//    one complete d-long dot product inside one block) and a contiguous slice of output rows of
//    M / W. Its slices of the next site (V^T rows, M rows, (V^T V - I) rows) and the next input
//    row are loaded into registers while the current site waits on its exchanges, so the HBM
//    stream overlaps synchronisation. Prefetch loads are unconditional (out-of-range slots read a
//    valid dummy chunk) so the compiler keeps them in flight across barriers.
//  * Two all-gather exchanges per site: (E1) every block needs all of g for its rows of M g;
//    (E2) the gate needs the global sum of per-block pieces of g^T (V^T V - I) g, and its
//    completion also means every block has written its rows of y. A slow token adds (E3), the
//    completion of the W x rows.
//  * Exchanges use tagged 64-bit mailbox words (tag << 32 | payload) with one copy per XCD, so
//    a block polls the copy on its own XCD's side; stores and polls are device-scope. Tags grow
//    monotonically across launches (base kept in the workspace header), so nothing is cleared.
//    A slot is rewritten only after every reader consumed it (the other exchange always sits in
//    between two uses of one mailbox).
//  * One wave per block (the sync wave) does all polling; four data waves load and compute.
//    Every wait is bounded: past the bound the launch is marked aborted and every block leaves,
//    so a lost block cannot hang the device.
//  * Gate arithmetic is done identically (same data, same order) in every block, so all blocks
//    take the same branch.
#include <algorithm>

#include "gsi_internal.h"

namespace gsi {

constexpr int kMaxJ = 4;   // g columns per block (k <= 512 with at least 128 blocks)
constexpr int kSyncDRegs = 2;  // (V^T V - I) chunks per sync-wave lane held in registers
constexpr int kSlowBatch = 8;  // W / x chunk pairs per lane in flight on the slow path
constexpr unsigned long long kWaitTicks = 200000000ull;  // 2 s at the 100 MHz wall clock

// A 16-byte chunk as a built-in vector (address-space-qualified pointers to it copy cleanly).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* g4p;  // global memory, read

__device__ __forceinline__ u32x4 ldg(g4p p, long long i) { return p[i]; }

// Descriptor table entries are read through the constant address space so the compiler issues
// scalar loads (the index is uniform across the block).
__device__ __forceinline__ LayerDesc load_desc(const LayerDesc* tab, int s) {
  static_assert(sizeof(LayerDesc) % 8 == 0, "descriptor must be a whole number of 8-byte words");
  typedef const unsigned long long __attribute__((address_space(4)))* cw;
  const cw src = (cw)(tab + s);
  LayerDesc d;
  unsigned long long* dst = reinterpret_cast<unsigned long long*>(&d);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(LayerDesc) / 8); ++i) dst[i] = src[i];
  return d;
}

__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xfu;
}
__device__ __forceinline__ u64 ld_dev(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_dev(u64* p, u64 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u64 pack(unsigned tag, float v) { return ((u64)tag << 32) | (u64)__float_as_uint(v); }

template <typename T>
__device__ __forceinline__ void unpack(const u32x4& q, float* out) {
  const T* e = reinterpret_cast<const T*>(&q);
#pragma unroll
  for (int i = 0; i < vec16<T>::N; ++i) out[i] = to_f32(e[i]);
}

template <typename T>
__device__ __forceinline__ float dot_chunk(const u32x4& a, const u32x4& b, float acc) {
  float fa[vec16<T>::N], fb[vec16<T>::N];
  unpack<T>(a, fa);
  unpack<T>(b, fb);
#pragma unroll
  for (int i = 0; i < vec16<T>::N; ++i) acc = __builtin_fmaf(fa[i], fb[i], acc);
  return acc;
}
template <typename T>
__device__ __forceinline__ float sq_chunk(const u32x4& a, float acc) {
  float fa[vec16<T>::N];
  unpack<T>(a, fa);
#pragma unroll
  for (int i = 0; i < vec16<T>::N; ++i) acc = __builtin_fmaf(fa[i], fa[i], acc);
  return acc;
}
template <typename T>
__device__ __forceinline__ float dot_chunk_lds(const u32x4& a, const float* g, float acc) {
  float fa[vec16<T>::N];
  unpack<T>(a, fa);
#pragma unroll
  for (int i = 0; i < vec16<T>::N; ++i) acc = __builtin_fmaf(fa[i], g[i], acc);
  return acc;
}
__device__ __forceinline__ float dot_f32x4_lds(const u32x4& a, const float* g, float acc) {
  acc = __builtin_fmaf(__uint_as_float(a.x), g[0], acc);
  acc = __builtin_fmaf(__uint_as_float(a.y), g[1], acc);
  acc = __builtin_fmaf(__uint_as_float(a.z), g[2], acc);
  acc = __builtin_fmaf(__uint_as_float(a.w), g[3], acc);
  return acc;
}

// Cross-lane sums on the VALU through DPP (row shifts inside 16-lane rows, then row broadcasts).
// The sum of each aligned group of `width` lanes (a power of two <= 64) lands in the group's LAST
// lane; every lane position always adds in the same order, so results are reproducible.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_src(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
__device__ __forceinline__ float group_reduce(float v, int width) {
  if (width >= 2) v += dpp_src<0x111, 0xF>(v);   // row_shr:1
  if (width >= 4) v += dpp_src<0x112, 0xF>(v);   // row_shr:2
  if (width >= 8) v += dpp_src<0x114, 0xF>(v);   // row_shr:4
  if (width >= 16) v += dpp_src<0x118, 0xF>(v);  // row_shr:8
  if (width >= 32) v += dpp_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if (width >= 64) v += dpp_src<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
// Whole-wave sum, valid in lane 63.
__device__ __forceinline__ float wave_reduce(float v) {
  v += dpp_src<0x111, 0xF>(v);
  v += dpp_src<0x112, 0xF>(v);
  v += dpp_src<0x114, 0xF>(v);
  v += dpp_src<0x118, 0xF>(v);
  v += dpp_src<0x142, 0xA>(v);
  v += dpp_src<0x143, 0xC>(v);
  return v;
}

struct SiteGeom {
  int nJ;        // g columns owned by this block
  int cprd;      // 16-byte chunks per V^T / W row (d / VW)
  int nx;        // x chunks per data thread (ceil(cprd / 256))
  int cprk;      // 16-byte chunks per M row (k / VW)
  int r0, nrows; // output rows owned
  int nm;        // M chunks owned (nrows * cprk)
  int nd;        // (V^T V - I) float4 chunks owned (nJ * k / 4)
};

template <typename T>
__device__ __forceinline__ SiteGeom geom(const LayerDesc& L, int b, int P) {
  constexpr int VW = vec16<T>::N;
  SiteGeom g;
  g.nJ = b < L.k ? (L.k - 1 - b) / P + 1 : 0;
  g.cprd = L.d / VW;
  g.nx = (g.cprd + kDataThreads - 1) / kDataThreads;
  g.cprk = L.k / VW;
  const int rpb = (L.d_out + P - 1) / P;
  g.r0 = min(L.d_out, b * rpb);
  g.nrows = min(L.d_out, g.r0 + rpb) - g.r0;
  g.nm = g.nrows * g.cprk;
  g.nd = g.nJ * (L.k / 4);
  return g;
}

// Register windows: JR x XR chunks of V^T rows (column jl, x chunk tid + 256 u), XR chunks of the
// input row, and MR chunks of M rows (chunk tid + 256 u of the block's slice).
template <int JR, int XR, int MR>
struct Window {
  u32x4 v[JR][XR];
  u32x4 x[XR];
  u32x4 m[MR];
};

// Loads of one site's slices (and its input row) into the window, in two parts: the V^T rows and
// the input row (consumed in phase A), then the M and (V^T V - I) rows (consumed in phase B). All
// loads are unconditional: each reads through a pointer selected beforehand (the real chunk or a
// valid dummy chunk), so exactly one load is issued per slot and it never leaves a valid buffer.
template <typename T, int JR, int XR, int MR>
__device__ __forceinline__ void prefetch_proj(const LayerDesc& L, const SiteGeom& g, const void* xrow, int b, int P,
                                              int tid, const u32x4* dummy, Window<JR, XR, MR>& w) {
  const g4p vt = (g4p)L.Vt;
  const g4p dm = (g4p)dummy;
#pragma unroll
  for (int jl = 0; jl < JR; ++jl) {
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      const int cc = tid + u * kDataThreads;
      const bool ok = jl < g.nJ && cc < g.cprd;
      const long long j = b + (long long)jl * P;
      const g4p src = ok ? vt + (j * g.cprd + cc) : dm;
      w.v[jl][u] = src[0];
    }
  }
  const g4p xp = (g4p)xrow;
#pragma unroll
  for (int u = 0; u < XR; ++u) {
    const int cc = tid + u * kDataThreads;
    w.x[u] = xp[cc < g.cprd ? cc : 0];
  }
}
template <typename T, int JR, int XR, int MR>
__device__ __forceinline__ void prefetch_image(const LayerDesc& L, const SiteGeom& g, int b, int P, int tid,
                                               const u32x4* dummy, Window<JR, XR, MR>& w) {
  const g4p dm = (g4p)dummy;
  const g4p mp = (g4p)L.M + (long long)g.r0 * g.cprk;
#pragma unroll
  for (int u = 0; u < MR; ++u) {
    const int c = tid + u * kDataThreads;
    const g4p src = c < g.nm ? mp + c : dm;
    w.m[u] = src[0];
  }
}

// Sync wave: load this block's rows of V^T V - I for the next site (chunk c = lane + 64 u).
__device__ __forceinline__ void prefetch_sync_delta(const LayerDesc& L, const SiteGeom& g, int b, int P, int lane,
                                                    const u32x4* dummy, u32x4 (&sdl)[kSyncDRegs]) {
  const g4p dm = (g4p)dummy;
  const int cpk4 = L.k / 4;
  const g4p dl = (g4p)L.Dl;
#pragma unroll
  for (int u = 0; u < kSyncDRegs; ++u) {
    const int c = lane + 64 * u;
    const bool ok = c < g.nd;
    const int jl = ok ? c / cpk4 : 0, cc = ok ? c - jl * cpk4 : 0;
    const long long j = b + (long long)jl * P;
    const g4p src = ok ? dl + (j * cpk4 + cc) : dm;
    sdl[u] = src[0];
  }
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

// Sync wave: poll `n` tagged words of mailbox copy `mb` until all carry `tag`; values go to `out`
// (per lane, entries lane + 64 i; zero past n). One poll issues all of its loads back to back
// (slots past n re-read entry n - 1) together with the launch's abort mark, then waits once, so
// a poll costs one memory round trip. Returns false on timeout or abort.
template <int NI>
__device__ __forceinline__ bool gather(const DecodeParams& p, unsigned base, const u64* mb, int n, unsigned tag,
                                       int lane, float (&out)[NI]) {
  const unsigned long long t0 = wall_clock64();
  while (true) {
    u64 wv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = lane + 64 * i;
      wv[i] = ld_dev(mb + (j < n ? j : n - 1));
    }
    const unsigned ab = __hip_atomic_load(&p.hdr->abort_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      ok &= (unsigned)(wv[i] >> 32) == tag;
      out[i] = (lane + 64 * i < n) ? __uint_as_float((unsigned)wv[i]) : 0.f;
    }
    if (__all(ok)) return true;
    if (ab == base + 1u || wall_clock64() - t0 > kWaitTicks) {
      if (lane == 0) record_abort(p, base);
      return false;
    }
  }
}

template <typename T, int JR, int XR, int MR>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
  constexpr int VW = vec16<T>::N;
  __shared__ float gsh[kMaxK];
  __shared__ float red[kDecodeThreads / 64][kMaxJ + 2];
  __shared__ float ypart[256];
  __shared__ float s_nx2, s_gg;
  __shared__ int s_gate, s_abort;
  __shared__ unsigned s_base;

  const int tid = threadIdx.x;
  const int b = blockIdx.x, P = gridDim.x;
  const bool is_sync = tid >= kDataThreads;
  const int lane = tid & 63, wave = tid >> 6;
  const unsigned rep = xcc_id() % kReplicas;
  const LayerDesc* tab = p.sites;
  const u32x4* dummy = reinterpret_cast<const u32x4*>(p.hdr);

  if (tid == 0) {
    s_abort = 0;
    s_base = __hip_atomic_load(&p.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const unsigned base = s_base;
  const long long Q = (long long)p.n_tokens * p.n_sites;

  Window<JR, XR, MR> w;
  u32x4 sdl[kSyncDRegs];
  if (Q > 0) {
    const LayerDesc L0 = load_desc(tab, 0);
    const SiteGeom g0 = geom<T>(L0, b, P);
    if (!is_sync) {
      prefetch_proj<T>(L0, g0, reinterpret_cast<const T*>(p.X) + L0.x_off, b, P, tid, dummy, w);
      prefetch_image<T>(L0, g0, b, P, tid, dummy, w);
    } else {
      prefetch_sync_delta(L0, g0, b, P, lane, dummy, sdl);
    }
  }

  for (long long q = 0; q < Q; ++q) {
    const int t = (int)(q / p.n_sites), s = (int)(q - (long long)t * p.n_sites);
    const LayerDesc L = load_desc(tab, s);
    const SiteGeom g = geom<T>(L, b, P);
    const unsigned tag = base + (unsigned)(q * 4);
    const unsigned tag_g = tag + 1, tag_p = tag + 2, tag_f = tag + 3;
    const T* x = reinterpret_cast<const T*>(p.X) + (long long)t * p.x_ld + L.x_off;

    // ---------------- phase A: g_j for owned columns and |x|^2, from the window ----------------
    if (!is_sync) {
      float acc[kMaxJ];
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) acc[j] = 0.f;
#pragma unroll
      for (int jl = 0; jl < JR; ++jl)
#pragma unroll
        for (int u = 0; u < XR; ++u) {
          const int cc = tid + u * kDataThreads;
          const float part = dot_chunk<T>(w.v[jl][u], w.x[u], 0.f);
          acc[jl] += (jl < g.nJ && cc < g.cprd) ? part : 0.f;
        }
      float sx = 0.f;
#pragma unroll
      for (int u = 0; u < XR; ++u) {
        const float v = sq_chunk<T>(w.x[u], 0.f);
        sx += (tid + u * kDataThreads < g.cprd) ? v : 0.f;
      }
      // inputs longer than the window (d beyond XR * 256 chunks, or more columns than JR)
      if (g.nx > XR || g.nJ > JR) {
        const g4p x4 = (g4p)x;
        for (int cc = tid + XR * kDataThreads; cc < g.cprd; cc += kDataThreads) sx = sq_chunk<T>(ldg(x4, cc), sx);
        for (int jl = 0; jl < g.nJ; ++jl) {
          const long long j = b + (long long)jl * P;
          const g4p vr = (g4p)L.Vt + j * g.cprd;
          float a = 0.f;
          for (int cc = tid + (jl < JR ? XR : 0) * kDataThreads; cc < g.cprd; cc += kDataThreads)
            a = dot_chunk<T>(ldg(vr, cc), ldg(x4, cc), a);
#pragma unroll
          for (int jj = 0; jj < kMaxJ; ++jj) acc[jj] += (jj == jl) ? a : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) acc[j] = wave_reduce(acc[j]);
      sx = wave_reduce(sx);
      if (lane == 63) {
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) red[wave][j] = acc[j];
        red[wave][kMaxJ] = sx;
      }
    }
    __syncthreads();
    // ---- E1 (sync wave): publish this block's g_j, all-gather g, then the gate piece p_b ----
    // The sync wave computes p_b = sum_j g_j ((V^T V - I) g)_j from its own prefetched rows of
    // V^T V - I and publishes it before releasing the data waves, so E2 runs concurrently with
    // phase B and the store is queued ahead of the data waves' next prefetch. Lane r < kReplicas
    // writes mailbox copy r.
    if (is_sync) {
      const float nx2 = ((red[0][kMaxJ] + red[1][kMaxJ]) + red[2][kMaxJ]) + red[3][kMaxJ];
      float gj_own[kMaxJ];
#pragma unroll
      for (int jl = 0; jl < kMaxJ; ++jl) gj_own[jl] = ((red[0][jl] + red[1][jl]) + red[2][jl]) + red[3][jl];
      for (int jl = 0; jl < g.nJ; ++jl) {
        const long long j = b + (long long)jl * P;
        if (lane < kReplicas) st_dev(p.box_g + (long long)lane * kMaxK + j, pack(tag_g, gj_own[jl]));
      }
      if (lane == 0) s_nx2 = nx2;
      float gv[kMaxK / 64];
      const bool ok = gather(p, base, p.box_g + (long long)rep * kMaxK, L.k, tag_g, lane, gv);
      if (!ok && lane == 0) s_abort = 1;
      float gg = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxK / 64; ++i) {
        const int j = lane + 64 * i;
        if (j < L.k) gsh[j] = gv[i];
        gg = __builtin_fmaf(gv[i], gv[i], gg);
      }
      gg = wave_reduce(gg);
      // p_b from the prefetched rows: chunk c = lane + 64 u covers row jl = c / (k/4), columns
      // 4 (c mod k/4) .. + 3; g is read back from LDS (written above by this wave, in order)
      const int cpk4 = L.k / 4;
      float pp = 0.f;
#pragma unroll
      for (int u = 0; u < kSyncDRegs; ++u) {
        const int c = lane + 64 * u;
        const bool okc = c < g.nd;
        const int jl = okc ? c / cpk4 : 0, cc = okc ? c - jl * cpk4 : 0;
        float gjl = gj_own[0];
#pragma unroll
        for (int jj = 1; jj < kMaxJ; ++jj) gjl = (jl == jj) ? gj_own[jj] : gjl;
        const float v = dot_f32x4_lds(sdl[u], gsh + cc * 4, 0.f) * gjl;
        pp += okc ? v : 0.f;
      }
      for (int c = lane + 64 * kSyncDRegs; c < g.nd; c += 64) {  // rows beyond the sync window
        const int jl = c / cpk4, cc = c - jl * cpk4;
        const long long j = b + (long long)jl * P;
        float gjl = gj_own[0];
#pragma unroll
        for (int jj = 1; jj < kMaxJ; ++jj) gjl = (jl == jj) ? gj_own[jj] : gjl;
        pp += dot_f32x4_lds(ldg((g4p)L.Dl, j * cpk4 + cc), gsh + cc * 4, 0.f) * gjl;
      }
      pp = wave_reduce(pp);
      const float pb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), 63));
      if (lane < kReplicas) st_dev(p.box_p + (long long)lane * kMaxBlocks + b, pack(tag_p, pb));
      if (lane == 63) s_gg = gg;
    }
    __syncthreads();
    if (s_abort) break;

    const bool has_next = q + 1 < Q;
    const long long qn = q + 1;
    const int tn = (int)(qn / p.n_sites), sn = (int)(qn - (long long)tn * p.n_sites);
    const LayerDesc Ln = load_desc(tab, has_next ? sn : s);
    const SiteGeom gn = geom<T>(Ln, b, P);
    if (!is_sync) {
      // ------- phase B (data waves): y = M g for the owned rows, while E2 runs -------
      // the next site's V^T rows and input row stream in now (phase A consumed those slots)
      if (has_next)
        prefetch_proj<T>(Ln, gn, reinterpret_cast<const T*>(p.X) + (long long)tn * p.x_ld + Ln.x_off, b, P, tid,
                         dummy, w);
      // The block's M slice is nrows * cprk contiguous chunks; chunk c = tid + 256 u belongs to
      // row c / cprk. Rows are reduced inside lane groups of width min(cprk, 64) and, for
      // cprk > 64, across groups through LDS in index order.
      const int gw = min(g.cprk, 64);
      const int segs = g.cprk / gw;
      T* yrow = reinterpret_cast<T*>(p.Y) + (long long)t * p.y_ld + L.y_off + g.r0;
#pragma unroll
      for (int u = 0; u < MR; ++u) {
        const int c = tid + u * kDataThreads;
        if (u * kDataThreads < g.nm) {  // uniform across the block
          const bool ok = c < g.nm;
          const int cm = ok ? c : 0;
          float v = dot_chunk_lds<T>(w.m[u], gsh + (cm % g.cprk) * VW, 0.f);
          v = group_reduce(ok ? v : 0.f, gw);
          if (ok && (c % gw) == gw - 1) {
            if (segs == 1) yrow[c / g.cprk] = from_f32<T>(v);
            else ypart[c / gw] = v;
          }
        }
      }
      for (int c0 = MR * kDataThreads; c0 < g.nm; c0 += kDataThreads) {  // slices beyond the window
        const int c = tid + c0;
        const bool ok = c < g.nm;
        const int cm = ok ? c : 0;
        float v = dot_chunk_lds<T>(ldg((g4p)L.M, (long long)g.r0 * g.cprk + cm), gsh + (cm % g.cprk) * VW, 0.f);
        v = group_reduce(ok ? v : 0.f, gw);
        if (ok && (c % gw) == gw - 1) {
          if (segs == 1) yrow[c / g.cprk] = from_f32<T>(v);
          else ypart[c / gw] = v;
        }
      }
      // the next site's M rows stream in while the gate is being resolved
      if (has_next) prefetch_image<T>(Ln, gn, b, P, tid, dummy, w);
    } else {
      // ---------------- E2 (sync wave): all-gather the pieces, resolve the gate ----------------
      float pv[kMaxBlocks / 64];
      const bool ok = gather(p, base, p.box_p + (long long)rep * kMaxBlocks, P, tag_p, lane, pv);
      if (!ok && lane == 0) s_abort = 1;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxBlocks / 64; ++i) ps += pv[i];
      ps = wave_reduce(ps);
      if (lane == 63) {
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
      // prefetch the next site's rows of V^T V - I for the next p_b
      if (has_next) prefetch_sync_delta(Ln, gn, b, P, lane, dummy, sdl);
    }
    __syncthreads();
    if (s_abort) break;
    if (!is_sync && g.cprk / min(g.cprk, 64) > 1) {  // rows split over several lane groups
      const int segs = g.cprk / min(g.cprk, 64);
      T* yrow = reinterpret_cast<T*>(p.Y) + (long long)t * p.y_ld + L.y_off + g.r0;
      for (int r = tid; r < g.nrows; r += kDataThreads) {
        float v = 0.f;
        for (int sg = 0; sg < segs; ++sg) v += ypart[r * segs + sg];
        yrow[r] = from_f32<T>(v);
      }
    }

    // ---------------- slow path: y = W x for the owned rows, then E3 ----------------
    if (s_gate) {
      if (!is_sync) {
        // one wave per row; each lane keeps kSlowBatch chunk pairs in flight per batch
        const g4p x4 = (g4p)x;
        T* yrow = reinterpret_cast<T*>(p.Y) + (long long)t * p.y_ld + L.y_off;
        for (int r = g.r0 + wave; r < g.r0 + g.nrows; r += kDataThreads / 64) {
          const g4p wr = (g4p)L.W + (long long)r * g.cprd;
          float a = 0.f;
          for (int c0 = 0; c0 < g.cprd; c0 += kSlowBatch * 64) {
            u32x4 wv[kSlowBatch], xv[kSlowBatch];
#pragma unroll
            for (int i = 0; i < kSlowBatch; ++i) {
              const int c = c0 + lane + 64 * i;
              const int cc = c < g.cprd ? c : 0;
              wv[i] = wr[cc];
              xv[i] = x4[cc];
            }
#pragma unroll
            for (int i = 0; i < kSlowBatch; ++i) {
              const float v = dot_chunk<T>(wv[i], xv[i], 0.f);
              a += (c0 + lane + 64 * i < g.cprd) ? v : 0.f;
            }
          }
          a = wave_reduce(a);
          if (lane == 63) yrow[r] = from_f32<T>(a);
        }
      }
      __syncthreads();
      if (is_sync) {
        if (lane < kReplicas) st_dev(p.box_f + (long long)lane * kMaxBlocks + b, pack(tag_f, 0.f));
        float fv[kMaxBlocks / 64];
        if (!gather(p, base, p.box_f + (long long)rep * kMaxBlocks, P, tag_f, lane, fv) && lane == 0) s_abort = 1;
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

// Instantiated register windows: JR columns, XR input chunks per thread (XR * 256 chunks of 16
// bytes cover the input row), MR M chunks per thread. Larger sites fall back to streaming loops.
template <typename T, int XR>
static const void* pick_jm(int jr, int mr) {
  if (jr <= 1 && mr <= 8) return (const void*)decode_kernel<T, 1, XR, 8>;
  if (jr <= 2) return (const void*)decode_kernel<T, 2, XR, 16>;
  return (const void*)decode_kernel<T, 4, XR, 16>;
}
template <typename T>
static const void* pick(int jr, int xr, int mr) {
  return xr <= 2 ? pick_jm<T, 2>(jr, mr) : pick_jm<T, 8>(jr, mr);
}

static const void* decode_fn(int dtype, int jr, int xr, int mr) {
  switch (dtype) {
    case GSI_F32: return pick<float>(jr, xr, mr);
    case GSI_F16: return pick<f16_t>(jr, xr, mr);
    case GSI_BF16: return pick<bf16_t>(jr, xr, mr);
  }
  return nullptr;
}

static int grid_blocks(const void* fn) {
  int dev = 0, ncu = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kDecodeThreads, 0) != hipSuccess) return 0;
  long long cap = (long long)ncu * per;
  return (int)(cap < kMaxBlocks ? cap : kMaxBlocks);
}

int launch_decode(int dtype, const DecodeParams& prm, const LayerDesc* host_sites, hipStream_t s) {
  // size the register windows for the largest site at the full grid
  const int es = dtype == GSI_F32 ? 4 : 2;
  int need_x = 1;
  for (int i = 0; i < prm.n_sites; ++i)
    need_x = std::max(need_x, (host_sites[i].d * es / 16 + kDataThreads - 1) / kDataThreads);
  const int xr = need_x <= 2 ? 2 : 8;
  int jr = 1, mr = 8;
  for (int pass = 0; pass < 2; ++pass) {
    const void* fn = decode_fn(dtype, jr, xr, mr);
    if (!fn) return GSI_ERR_DTYPE;
    const int P = grid_blocks(fn);
    if (P < kMaxK / kMaxJ) return GSI_ERR_DEVICE;
    int need_j = 1, need_m = 1;
    for (int i = 0; i < prm.n_sites; ++i) {
      const LayerDesc& L = host_sites[i];
      need_j = std::max(need_j, (L.k + P - 1) / P);
      const int rpb = (L.d_out + P - 1) / P;
      const int cprk = L.k * es / 16;
      need_m = std::max(need_m, (rpb * cprk + kDataThreads - 1) / kDataThreads);
    }
    const int jr2 = (need_j <= 1 && need_m <= 8) ? 1 : need_j <= 2 ? 2 : 4;
    const int mr2 = jr2 == 1 ? 8 : 16;
    if (jr2 == jr && mr2 == mr) {
      DecodeParams p = prm;
      void* args[] = {&p};
      hipError_t e = hipLaunchCooperativeKernel(fn, dim3(P), dim3(kDecodeThreads), args, 0, s);
      return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
    }
    jr = jr2;
    mr = mr2;
  }
  return GSI_ERR_DEVICE;
}

}  // namespace gsi
