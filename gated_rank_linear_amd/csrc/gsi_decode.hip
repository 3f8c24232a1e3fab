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
//    M / W.
//  * Two all-gather exchanges per site: (E1) every block needs all of g for its rows of M g;
//    (E2) the gate needs the global sum of per-block pieces of g^T (V^T V - I) g. A block posts
//    its E2 word only after its rows of y are stored, so E2 is also the completion of the site:
//    no block starts the next site before every block has finished this one. A slow token adds
//    (E3), the completion of the W x rows.
//  * Weights stream into LDS ahead of use: two 64 KB site regions alternate with the site
//    parity. Right after posting its E1 word, a block's data waves copy its slices of site s + 1
//    (its V^T rows, its rows of V^T V - I and its rows of M) from HBM straight into the other
//    region (global_load_lds, 16 bytes per lane, no registers); the copy drains while E1
//    resolves and lands long before site s + 1 needs it. Nothing bulky is in flight on the CU
//    while E2 resolves: only the next input row, read into registers after this block's rows of y
//    are stored and used only after E2 has completed. Slices that do not fit a region are read
//    from global memory when used.
//  * Exchanges use tagged 64-bit mailbox words (tag << 32 | payload) with one copy per XCD, so
//    a block polls the copy on its own XCD's side; stores and polls are device-scope. Tags grow
//    monotonically across launches (base kept in the workspace header), so nothing is cleared.
//    A slot is rewritten only after every reader consumed it (the other exchange always sits in
//    between two uses of one mailbox).
//  * One wave per block (the sync wave) does all polling and posting; four data waves copy and
//    compute. Every wait is bounded: past the bound the launch is marked aborted and every block
//    leaves, so a lost block cannot hang the device.
//  * Gate arithmetic is done identically (same data, same order) in every block, so all blocks
//    take the same branch.
#include <algorithm>

#include "gsi_internal.h"

namespace gsi {

constexpr int kMaxJ = 4;       // g columns per block (k <= 512 with at least 128 blocks)
constexpr int kSlowBatch = 8;  // W / x chunk pairs per lane in flight on the slow path
constexpr unsigned long long kWaitTicks = 200000000ull;  // 2 s at the 100 MHz wall clock

// A 16-byte chunk as a built-in vector (address-space-qualified pointers to it copy cleanly).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* g4p;  // global memory, read
typedef __attribute__((address_space(3))) void lds_void;
typedef u32x4 __attribute__((address_space(3))) lu32x4;  // a 16-byte chunk in LDS
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Wait until at most N vector-memory operations of this wave are outstanding (expcnt and
// lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that orders LDS only: it waits for this wave's LDS operations, not for its
// outstanding global loads, so copies into LDS and mailbox stores stay in flight across it.
// (Vector-memory data is always waited for explicitly before it is used.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
// Dot product of two 16-byte chunks of the same element type, accumulated in float32 (bf16 and
// f16 pairs through v_dot2: the products are exact in float32). The 32-bit words are copied to
// scalars before they are reinterpreted: reinterpreting a member of a vector held by reference
// in place reads the vector's first word for every member with this compiler.
template <typename T>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b, float acc);
template <>
__device__ __forceinline__ float dot16<bf16_t>(const u32x4& a, const u32x4& b, float acc) {
  const unsigned aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw[i]), __builtin_bit_cast(bf16x2, bw[i]), acc,
                                          false);
  return acc;
}
template <>
__device__ __forceinline__ float dot16<f16_t>(const u32x4& a, const u32x4& b, float acc) {
  const unsigned aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, aw[i]), __builtin_bit_cast(f16x2, bw[i]), acc, false);
  return acc;
}
template <>
__device__ __forceinline__ float dot16<float>(const u32x4& a, const u32x4& b, float acc) {
  return dot_chunk<float>(a, b, acc);
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

// Block b's share of one site and the layout of its LDS region (in 16-byte chunks). The region
// holds [V^T rows | (V^T V - I) rows | M rows], each part starting on a 64-chunk boundary so that
// every 1 KB copy instruction lies inside one part.
struct SiteGeom {
  int nJ;        // g columns owned by this block
  int cprd;      // 16-byte chunks per V^T / W row (d / VW)
  int nx;        // x chunks per data thread (ceil(cprd / 256))
  int cprk;      // 16-byte chunks per M row (k / VW)
  int cpk4;      // float4 chunks per (V^T V - I) row (k / 4)
  int r0, nrows; // output rows owned
  int nm;        // M chunks owned (nrows * cprk)
  int nd;        // (V^T V - I) chunks owned (nJ * cpk4)
  int vj, v_n;   // V^T rows held in the region and their chunks (at offset 0)
  int d_off, d_n;  // (V^T V - I) part: offset and chunks held (all or none)
  int m_off, m_n;  // M part: offset and chunks held
  int m_rows;    // rows of the M slice held in the region (the rest is read from HBM)
  bool mf;       // matrix-core layout of the M part (bf16 with k >= 128): 16-row x 32-column
                 // tiles, tile (rt, kt) being one 1 KB block whose lane l holds row 16 rt +
                 // l mod 16, columns 32 kt + 8 (l / 16) .. + 7, i.e. the A operand of
                 // v_mfma_f32_16x16x32_bf16; otherwise the rows are stored as they are, and the
                 // part held is all of the slice or a multiple of 256 chunks so that one pass of
                 // the data waves never mixes LDS and global reads
  int n_inst;    // 1 KB copy instructions that fill the region
};

__device__ __forceinline__ int align64(int v) { return (v + 63) & ~63; }

template <typename T> struct is_bf16 { static constexpr bool v = false; };
template <> struct is_bf16<bf16_t> { static constexpr bool v = true; };

template <typename T>
__device__ __forceinline__ SiteGeom geom(const LayerDesc& L, int b, int P) {
  constexpr int VW = vec16<T>::N;
  const int sh_P = __builtin_ctz(P);  // the grid is a power of two
  SiteGeom g;
  g.nJ = b < L.k ? ((L.k - 1 - b) >> sh_P) + 1 : 0;
  g.cprd = L.d / VW;
  g.nx = (g.cprd + kDataThreads - 1) / kDataThreads;
  g.cprk = L.k / VW;
  g.cpk4 = L.k / 4;
  const int rpb = (L.d_out + P - 1) >> sh_P;
  g.r0 = min(L.d_out, b * rpb);
  g.nrows = min(L.d_out, g.r0 + rpb) - g.r0;
  g.nm = g.nrows * g.cprk;
  g.nd = g.nJ * g.cpk4;
  g.vj = g.nJ;  // V^T rows that fit the region (at most kMaxJ: compares, no division)
#pragma unroll
  for (int r = kMaxJ; r >= 1; --r) g.vj = (g.vj >= r && r * g.cprd > kRegionChunks) ? r - 1 : g.vj;
  g.v_n = g.vj * g.cprd;
  g.d_off = align64(g.v_n);
  g.d_n = g.d_off + g.nd <= kRegionChunks ? g.nd : 0;
  g.m_off = align64(g.d_off + g.d_n);
  g.mf = is_bf16<T>::v && L.k >= 128;
  const int sh_cprk = __builtin_ctz(g.cprk);  // k / VW is a power of two
  if (g.mf) {
    const int tiles = min((g.nrows + 15) / 16, max(0, kRegionChunks - g.m_off) >> (sh_cprk + 4));  // 16 cprk a tile
    g.m_n = tiles << (sh_cprk + 4);
    g.m_rows = min(g.nrows, tiles * 16);
  } else {
    g.m_n = g.m_off + g.nm <= kRegionChunks ? g.nm : max(0, (kRegionChunks - g.m_off) / kDataThreads * kDataThreads);
    g.m_rows = g.m_n >> sh_cprk;
  }
  g.n_inst = (g.m_off + g.m_n + 63) / 64;
  return g;
}

// Copy instructions [i0, i1) of a site's region fill; instruction i (chunks 64 i .. 64 i + 63 of
// the region) is issued by data wave i mod 4. Each lane reads one 16-byte chunk from global
// memory straight into LDS at region + 16 (64 i + lane). Lanes past the end of a part read a
// valid dummy chunk into the part's padding, so every lane issues exactly one load.
template <typename T>
__device__ __forceinline__ void fill_region(const LayerDesc& L, const SiteGeom& g, int b, int P, int wave, int lane,
                                            int i0, int i1, lu32x4* region,
                                            const u32x4* dummy) {
  const char* vt = reinterpret_cast<const char*>(L.Vt);
  const char* dl = reinterpret_cast<const char*>(L.Dl);
  const char* mp = reinterpret_cast<const char*>(L.M) + (long long)g.r0 * g.cprk * 16;
  // k, k / 4, k / 32 and k / VW are powers of two: shifts instead of divisions
  const int sh_cpk4 = __builtin_ctz(g.cpk4);
  const int sh_kt = g.mf ? __builtin_ctz(g.cprk / 4) : 0;
  for (int i = i0 + ((wave - i0) & 3); i < i1; i += 4) {
    const int c = i * 64 + lane;
    const char* src = reinterpret_cast<const char*>(dummy);
    if (c < g.v_n) {  // V^T row jl = c / cprd (at most kMaxJ rows: compares, no division)
      int jl = 0;
#pragma unroll
      for (int r = 1; r < kMaxJ; ++r) jl += c >= r * g.cprd ? 1 : 0;
      const int cc = c - jl * g.cprd;
      src = vt + ((long long)(b + jl * P) * g.cprd + cc) * 16;
    } else if (c >= g.d_off && c < g.d_off + g.d_n) {
      const int e = c - g.d_off;
      const int jl = e >> sh_cpk4, cc = e & (g.cpk4 - 1);
      src = dl + ((long long)(b + jl * P) * g.cpk4 + cc) * 16;
    } else if (c >= g.m_off && c < g.m_off + g.m_n) {
      if (g.mf) {  // tile (rt, kk) = instruction (i - m_off / 64) in row-tile-major order
        const int it = i - g.m_off / 64;
        const int rt = it >> sh_kt, kk = it & ((1 << sh_kt) - 1);
        const int row = rt * 16 + (lane & 15);
        if (row < g.nrows) src = mp + ((long long)row * g.cprk + kk * 4 + (lane >> 4)) * 16;
      } else {
        src = mp + (long long)(c - g.m_off) * 16;
      }
    }
    // streamed once per token: non-temporal, so the copy does not displace cached lines
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(region + i * 64), 16, 0, 2 /* nt */);
  }
}

// The input row's chunks tid + 256 u (u < XR) into registers; slots past the row re-read chunk 0.
template <typename T, int XR>
__device__ __forceinline__ void load_x(const void* xrow, const SiteGeom& g, int tid, u32x4 (&xw)[XR]) {
  const g4p xp = (g4p)xrow;
#pragma unroll
  for (int u = 0; u < XR; ++u) {
    const int cc = tid + u * kDataThreads;
    xw[u] = xp[cc < g.cprd ? cc : 0];
  }
}

// A block whose wait runs past its bound marks this launch (tag base + 1) as aborted; every other
// block polls that mark while it waits, so the whole grid leaves promptly. The mark of an older
// launch never matches because every launch advances the tag base.
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

// LDS shared by the phases of one site (the two site regions are separate arrays so that the
// compiler can tell a copy into one region from reads of the other).
struct Shared {
  float* gsh;    // [kMaxK] gathered g
  lu32x4* gb;    // [kGbChunks] B operands of the matrix-core path (see mfma_rows)
  float* ypart;  // [kYPart] this block's rows of y (float32) before rounding
  float (*red)[kMaxJ + 2];  // [4][kMaxJ + 2] per-wave partial sums of phase A
  float* s_nx2;
  float* s_gg;
  int* s_gate;
  int* s_abort;
};

// Vector-ALU rows of y = M g. Each row is covered by Lr = cprk / CPL lanes of one wave, lane
// (r, lc) holding chunks lc + Lr i (i < CPL) of row r, so a row's sum takes log2(Lr) DPP steps
// and every thread reads its CPL slices of g once. Slots i >= CPL (rows shorter than 4 chunks)
// read chunk 0 and g entries below 4 VW <= kMaxK, all in bounds, and are masked out of the sum.
struct RowLanes {
  int CPL, Lr, rpw, lr, lc;
  int ch[4];
};
template <typename T>
__device__ __forceinline__ RowLanes row_lanes(const SiteGeom& g, int lane) {
  RowLanes q;
  q.CPL = min(4, g.cprk);
  q.Lr = g.cprk >> __builtin_ctz(q.CPL);  // lanes per row (a power of two <= 32)
  q.rpw = 64 / q.Lr;      // rows per wave per pass
  q.lr = lane >> __builtin_ctz(q.Lr);
  q.lc = lane & (q.Lr - 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) q.ch[i] = i < q.CPL ? q.lc + q.Lr * i : 0;
  return q;
}
template <typename T>
__device__ __forceinline__ void g_slices(const Shared& sh, const RowLanes& q, float (&gl)[4][vec16<T>::N]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < vec16<T>::N; ++e) gl[i][e] = sh.gsh[(q.lc + q.Lr * i) * vec16<T>::N + e];
}
// rows [0, m_rows) from the region (stored as they are)
template <typename T>
__device__ __forceinline__ void row_sums_lds(const SiteGeom& g, const lu32x4* cur, const Shared& sh, int wave,
                                             int lane) {
  const RowLanes q = row_lanes<T>(g, lane);
  float gl[4][vec16<T>::N];
  g_slices<T>(sh, q, gl);
  for (int rp = 0; rp < g.m_rows; rp += 4 * q.rpw) {
    const int r = rp + wave * q.rpw + q.lr;
    const bool ok = r < g.m_rows;
    const int rb = g.m_off + (ok ? r : 0) * g.cprk;
    u32x4 mv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mv[i] = cur[rb + q.ch[i]];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = dot_chunk_lds<T>(mv[i], gl[i], 0.f);
      acc += i < q.CPL ? d : 0.f;
    }
    acc = group_reduce(ok ? acc : 0.f, q.Lr);
    if (ok && q.lc == q.Lr - 1) sh.ypart[r] = acc;
  }
}
// rows [m_rows, nrows) read from HBM (slices that do not fit the region)
template <typename T>
__device__ __forceinline__ void row_sums_hbm(const LayerDesc& L, const SiteGeom& g, const Shared& sh, int wave,
                                             int lane) {
  const RowLanes q = row_lanes<T>(g, lane);
  float gl[4][vec16<T>::N];
  g_slices<T>(sh, q, gl);
  const g4p mrow = (g4p)L.M + (long long)g.r0 * g.cprk;
  for (int rp = g.m_rows; rp < g.nrows; rp += 4 * q.rpw) {
    const int r = rp + wave * q.rpw + q.lr;
    const bool ok = r < g.nrows;
    const long long rb = (long long)(ok ? r : 0) * g.cprk;
    u32x4 mv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mv[i] = ldg(mrow, rb + q.ch[i]);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = dot_chunk_lds<T>(mv[i], gl[i], 0.f);
      acc += i < q.CPL ? d : 0.f;
    }
    acc = group_reduce(ok ? acc : 0.f, q.Lr);
    if (ok && q.lc == q.Lr - 1) sh.ypart[r] = acc;
  }
}

// Matrix-core rows of y = M g (bf16, k = 32 KT). Wave w takes the 16-row tiles w, w + 4, ...
// of the region's M part (stored as A operands of v_mfma_f32_16x16x32_bf16). B carries g as two
// bf16 columns, column 0 its high part and column 1 the low part (g - high), every other column
// zero; B for 32-column step s and lane group h = l / 16 is chunk 8 s + 2 h + column of sh.gb,
// read once per site. Two accumulator chains (even and odd steps) are added at the end; then
// D[r][0] + D[r][1] (lane l and lane l + 1 of each 16-lane row, a DPP shift) is row r of y.
// Marks every chunk of `v` as needed here, so all of their loads are issued (and waited for once)
// before any later use, instead of each load being issued just before its use.
template <int N>
__device__ __forceinline__ void hold(const u32x4 (&v)[N]) {
  static_assert(N == 4 || N == 8, "operand group of 4 or 8 chunks");
  if constexpr (N == 4) {
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
  } else {
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
  }
}

constexpr int kGbZero = kMaxK / 32 * 8;  // index of an all-zero chunk of sh.gb
constexpr int kGbChunks = kGbZero + 1;
template <int KT>
__device__ __forceinline__ void mfma_rows(const SiteGeom& g, const lu32x4* cur, const Shared& sh, int wave, int lane) {
  constexpr int KH = KT < 8 ? KT : 8;  // steps held in registers at a time
  constexpr int NH = KT / KH;
  const int col = lane & 15, grp = lane >> 4;
  const int tiles = (g.m_rows + 15) / 16;
  u32x4 bv[KH];
  auto load_b = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KH; ++i) bv[i] = sh.gb[col < 2 ? (k0 + i) * 8 + grp * 2 + col : kGbZero];
    hold(bv);
  };
  if (NH == 1) load_b(0);
  for (int rt = wave; rt < tiles; rt += 4) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      if (NH > 1) load_b(hh * KH);
      u32x4 av[KH];
#pragma unroll
      for (int i = 0; i < KH; ++i) av[i] = cur[g.m_off + (rt * KT + hh * KH + i) * 64 + lane];
      hold(av);
#pragma unroll
      for (int i = 0; i < KH; ++i) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, av[i]);
        const bf16x8 B = __builtin_bit_cast(bf16x8, bv[i]);
        if (i & 1) a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, a1, 0, 0, 0);
        else a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, a0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = a0[r] + a1[r];
      const float w = v + dpp_src<0x101, 0xF>(v);  // row_shl:1: lane l + 1's value
      const int row = rt * 16 + 4 * grp + r;
      if (col == 0 && row < g.m_rows) sh.ypart[row] = w;
    }
  }
}

// One (token, site) step. `cur` holds this site's slices (filled during the previous step);
// `nxt` receives the next site's. Returns false when the launch was aborted.
template <typename T, int XR>
__device__ __forceinline__ bool site_step(const DecodeParams& p, long long q, int t, int s, long long Q, unsigned base,
                                          int b, int P,
                                          int tid, unsigned rep, const u32x4* dummy,
                                          const lu32x4* cur, lu32x4* nxt, u32x4 (&xw)[XR],
                                          const Shared& sh) {
  constexpr int VW = vec16<T>::N;
  const bool is_sync = tid >= kDataThreads;
  const int lane = tid & 63, wave = tid >> 6;
  const LayerDesc L = load_desc(p.sites, s);
  const SiteGeom g = geom<T>(L, b, P);
  const unsigned tag = base + (unsigned)(q * 4);
  const unsigned tag_g = tag + 1, tag_p = tag + 2, tag_f = tag + 3;
  const T* x = reinterpret_cast<const T*>(p.X) + (long long)t * p.x_ld + L.x_off;
  const bool has_next = q + 1 < Q;
  const int sn = s + 1 < p.n_sites ? s + 1 : 0, tn = s + 1 < p.n_sites ? t : t + 1;
  const LayerDesc Ln = load_desc(p.sites, has_next ? sn : s);
  const SiteGeom gn = geom<T>(Ln, b, P);

  // ---------------- phase A (data waves): g_j for owned columns and |x|^2 ----------------
  if (!is_sync) {
    float acc[kMaxJ];
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j) acc[j] = 0.f;
    float sx = 0.f;
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      if (u * kDataThreads < g.cprd) {  // uniform: slots past the input row are skipped
        const float v = dot16<T>(xw[u], xw[u], 0.f);
        sx += tid + u * kDataThreads < g.cprd ? v : 0.f;
      }
    }
#pragma unroll
    for (int jl = 0; jl < kMaxJ; ++jl) {
      if (jl < g.vj) {  // uniform
        const int rb = jl * g.cprd;
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < XR; ++u) {
          if (u * kDataThreads < g.cprd) {  // uniform
            const int cc = tid + u * kDataThreads;
            const bool in = cc < g.cprd;
            const u32x4 vv = cur[rb + (in ? cc : 0)];
            const float part = dot16<T>(vv, xw[u], 0.f);
            a += in ? part : 0.f;
          }
        }
        acc[jl] = a;
      }
    }
    // columns not held in the region, and inputs longer than the register window
    if (g.vj < g.nJ || g.nx > XR) {
      const g4p x4 = (g4p)x;
      for (int cc = tid + XR * kDataThreads; cc < g.cprd; cc += kDataThreads) {
        const u32x4 xv = ldg(x4, cc);
        sx = dot16<T>(xv, xv, sx);
      }
      for (int jl = 0; jl < g.nJ; ++jl) {
        const long long j = b + (long long)jl * P;
        const g4p vr = (g4p)L.Vt + j * g.cprd;
        float a = 0.f;
        for (int cc = tid + (jl < g.vj ? XR : 0) * kDataThreads; cc < g.cprd; cc += kDataThreads)
          a = dot16<T>(ldg(vr, cc), ldg(x4, cc), a);
#pragma unroll
        for (int jj = 0; jj < kMaxJ; ++jj) acc[jj] += (jj == jl) ? a : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxJ; ++j)
      if (j < g.nJ) acc[j] = wave_reduce(acc[j]);  // uniform
    sx = wave_reduce(sx);
    if (lane == 63) {
#pragma unroll
      for (int j = 0; j < kMaxJ; ++j) sh.red[wave][j] = acc[j];
      sh.red[wave][kMaxJ] = sx;
    }
  }
  lds_barrier();
  // ---------------- E1: post this block's g_j, then all-gather g ----------------
  float gj_own[kMaxJ];
  if (is_sync) {
#pragma unroll
    for (int jl = 0; jl < kMaxJ; ++jl)
      gj_own[jl] = ((sh.red[0][jl] + sh.red[1][jl]) + sh.red[2][jl]) + sh.red[3][jl];
    for (int jl = 0; jl < g.nJ; ++jl) {
      const long long j = b + (long long)jl * P;
      if (lane < kReplicas) st_dev(p.box_g + (long long)lane * kMaxK + j, pack(tag_g, gj_own[jl]));
    }
    if (lane == 0) *sh.s_nx2 = ((sh.red[0][kMaxJ] + sh.red[1][kMaxJ]) + sh.red[2][kMaxJ]) + sh.red[3][kMaxJ];
  }
  lds_barrier();  // the g words are issued ahead of the copy below
  if (!is_sync) {
    if (has_next) fill_region<T>(Ln, gn, b, P, wave, lane, 0, gn.n_inst, nxt, dummy);
  } else {
    float gv[kMaxK / 64];
    const bool ok = gather(p, base, p.box_g + (long long)rep * kMaxK, L.k, tag_g, lane, gv);
    if (!ok && lane == 0) *sh.s_abort = 1;
    float gg = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxK / 64; ++i) {
      const int j = lane + 64 * i;
      if (j < L.k) {
        sh.gsh[j] = gv[i];
        if (g.mf) {  // g = hi + lo + O(2^-18 |g|), both parts bf16 (exact products with M)
          const bf16_t hi = from_f32<bf16_t>(gv[i]);
          const bf16_t lo = from_f32<bf16_t>(gv[i] - to_f32(hi));
          auto* gb16 = reinterpret_cast<__attribute__((address_space(3))) uint16_t*>(sh.gb);
          const int c0 = ((j >> 5) * 4 + ((j >> 3) & 3)) * 2;  // chunk of (step j / 32, lane group)
          gb16[c0 * 8 + (j & 7)] = hi.b;
          gb16[(c0 + 1) * 8 + (j & 7)] = lo.b;
        }
      }
      gg = __builtin_fmaf(gv[i], gv[i], gg);
    }
    gg = wave_reduce(gg);
    if (lane == 63) *sh.s_gg = gg;
  }
  lds_barrier();
  if (*sh.s_abort) return false;

  // ------- phase B (data waves): this block's rows of y = M g; (sync wave) the gate piece -------
  float pb = 0.f;
  if (!is_sync) {
    if (g.mf) {
      switch (g.cprk / 4) {  // 32-column steps per row: k / 32
        case 4: mfma_rows<4>(g, cur, sh, wave, lane); break;
        case 8: mfma_rows<8>(g, cur, sh, wave, lane); break;
        default: mfma_rows<16>(g, cur, sh, wave, lane); break;
      }
    } else {
      row_sums_lds<T>(g, cur, sh, wave, lane);
    }
    if (g.m_rows < g.nrows) row_sums_hbm<T>(L, g, sh, wave, lane);
  } else {
    // p_b = sum_j g_j ((V^T V - I) g)_j over the owned columns; chunk c covers row c / cpk4,
    // columns 4 (c mod cpk4) .. + 3
    float pp = 0.f;
    if (g.d_n > 0) {
      for (int c = lane; c < g.nd; c += 64) {
        const int jl = c >> __builtin_ctz(g.cpk4), cc = c & (g.cpk4 - 1);
        float gjl = gj_own[0];
#pragma unroll
        for (int jj = 1; jj < kMaxJ; ++jj) gjl = (jl == jj) ? gj_own[jj] : gjl;
        const u32x4 dv = cur[g.d_off + c];
        pp += dot_f32x4_lds(dv, sh.gsh + cc * 4, 0.f) * gjl;
      }
    } else {
      for (int c = lane; c < g.nd; c += 64) {
        const int jl = c >> __builtin_ctz(g.cpk4), cc = c & (g.cpk4 - 1);
        float gjl = gj_own[0];
#pragma unroll
        for (int jj = 1; jj < kMaxJ; ++jj) gjl = (jl == jj) ? gj_own[jj] : gjl;
        const u32x4 dv = ldg((g4p)L.Dl, (long long)(b + (long long)jl * P) * g.cpk4 + cc);
        pp += dot_f32x4_lds(dv, sh.gsh + cc * 4, 0.f) * gjl;
      }
    }
    pp = wave_reduce(pp);
    pb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), 63));
  }
  lds_barrier();
  // ---- the sync wave stores this block's rows of y, then posts its E2 word (site done) ----
  if (is_sync) {
    T* yrow = reinterpret_cast<T*>(p.Y) + (long long)t * p.y_ld + L.y_off + g.r0;
    for (int r = lane; r < g.nrows; r += 64) yrow[r] = from_f32<T>(sh.ypart[r]);
    if (lane < kReplicas) st_dev(p.box_p + (long long)lane * kMaxBlocks + b, pack(tag_p, pb));
  }
  lds_barrier();  // the y rows and the E2 word are issued ahead of the loads below
  if (!is_sync) {
    // the next input row streams in while E2 resolves
    if (has_next) load_x<T, XR>(reinterpret_cast<const T*>(p.X) + (long long)tn * p.x_ld + Ln.x_off, gn, tid, xw);
    wait_vmcnt<0>();  // the next region and input row are complete before the barrier below
  } else {
    // ---------------- E2: all-gather the pieces, resolve the gate ----------------
    float pv[kMaxBlocks / 64];
    const bool ok = gather(p, base, p.box_p + (long long)rep * kMaxBlocks, P, tag_p, lane, pv);
    if (!ok && lane == 0) *sh.s_abort = 1;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxBlocks / 64; ++i) ps += pv[i];
    ps = wave_reduce(ps);
    if (lane == 63) {
      const float nx2 = *sh.s_nx2;
      const float nr2 = (nx2 - *sh.s_gg) + ps;
      const float thr = p.eps * p.eps;
      const float rhs = thr * nx2;
      const int slow = (nr2 < rhs) ? 0 : 1;
      *sh.s_gate = slow;
      if (b == 0) {
        const long long o = (long long)t * p.gate_ld + p.site0 + s;
        p.gates[o] = (uint8_t)slow;
        if (p.rho) p.rho[o] = sqrtf(fmaxf(nr2, 0.f) / nx2);
      }
    }
    wait_vmcnt<0>();  // this block's fast-path rows of y are written before a slow path rewrites them
  }
  lds_barrier();
  if (*sh.s_abort) return false;

  // ---------------- slow path: y = W x for the owned rows, then E3 ----------------
  if (*sh.s_gate) {
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
            const float v = dot16<T>(wv[i], xv[i], 0.f);
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
      if (!gather(p, base, p.box_f + (long long)rep * kMaxBlocks, P, tag_f, lane, fv) && lane == 0) *sh.s_abort = 1;
    }
    __syncthreads();
    if (*sh.s_abort) return false;
  }
  return true;
}

template <typename T, int XR>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
  __shared__ u32x4 region0[kRegionChunks];
  __shared__ u32x4 region1[kRegionChunks];
  __shared__ float gsh[kMaxK];
  __shared__ u32x4 gb[kGbChunks];
  __shared__ float ypart[kYPart];
  __shared__ float red[kDecodeThreads / 64][kMaxJ + 2];
  __shared__ float s_nx2, s_gg;
  __shared__ int s_gate, s_abort;
  __shared__ unsigned s_base;

  const int tid = threadIdx.x;
  const int b = blockIdx.x, P = gridDim.x;
  const bool is_sync = tid >= kDataThreads;
  const int lane = tid & 63, wave = tid >> 6;
  const unsigned rep = xcc_id() % kReplicas;
  const u32x4* dummy = reinterpret_cast<const u32x4*>(p.hdr);
  const Shared sh{gsh, (lu32x4*)gb, ypart, red, &s_nx2, &s_gg, &s_gate, &s_abort};
  lu32x4* const r0 = (lu32x4*)region0;
  lu32x4* const r1 = (lu32x4*)region1;

  if (tid == 0) {
    gb[kGbZero] = u32x4{0u, 0u, 0u, 0u};
    s_abort = 0;
    s_base = __hip_atomic_load(&p.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const long long Q = (long long)p.n_tokens * p.n_sites;

  u32x4 xw[XR];
  if (Q > 0 && !is_sync) {  // site 0's region and input row
    const LayerDesc L0 = load_desc(p.sites, 0);
    const SiteGeom g0 = geom<T>(L0, b, P);
    load_x<T, XR>(reinterpret_cast<const T*>(p.X) + L0.x_off, g0, tid, xw);
    fill_region<T>(L0, g0, b, P, wave, lane, 0, g0.n_inst, (lu32x4*)region0, dummy);
    wait_vmcnt<0>();
  }
  __syncthreads();
  const unsigned base = s_base;

  int t = 0, s = 0;  // token and site of step q
  auto advance = [&]() {
    if (++s == p.n_sites) {
      s = 0;
      ++t;
    }
  };
  for (long long q = 0; q < Q; q += 2) {
    if (!site_step<T, XR>(p, q, t, s, Q, base, b, P, tid, rep, dummy, r0, r1, xw, sh)) break;
    advance();
    if (q + 1 < Q && !site_step<T, XR>(p, q + 1, t, s, Q, base, b, P, tid, rep, dummy, r1, r0, xw, sh)) break;
    advance();
  }
  if (!is_sync) wait_vmcnt<0>();  // no copy into LDS outlives the block
  // advance the tag base for the next launch (also after an abort, so its mark goes stale)
  if (b == 0 && tid == 0)
    __hip_atomic_store(&p.hdr->epoch, base + (unsigned)(Q * 4) + 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

size_t decode_ws_bytes() {
  return sizeof(WsHeader) + (size_t)kReplicas * kMaxK * 8 + 2 * (size_t)kReplicas * kMaxBlocks * 8;
}

// Instantiated input windows: XR chunks of 16 bytes per data thread (XR * 256 chunks cover the
// input row); longer rows are finished by a streaming loop.
template <typename T>
static const void* pick(int xr) {
  return xr <= 2 ? (const void*)decode_kernel<T, 2> : (const void*)decode_kernel<T, 8>;
}

static const void* decode_fn(int dtype, int xr) {
  switch (dtype) {
    case GSI_F32: return pick<float>(xr);
    case GSI_F16: return pick<f16_t>(xr);
    case GSI_BF16: return pick<bf16_t>(xr);
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
  const int es = dtype == GSI_F32 ? 4 : 2;
  int need_x = 1;
  for (int i = 0; i < prm.n_sites; ++i)
    need_x = std::max(need_x, (host_sites[i].d * es / 16 + kDataThreads - 1) / kDataThreads);
  const void* fn = decode_fn(dtype, need_x);
  if (!fn) return GSI_ERR_DTYPE;
  int P = grid_blocks(fn);
  while (P & (P - 1)) P &= P - 1;  // a power of two: the kernel splits work with shifts
  if (P < kMinBlocks) return GSI_ERR_DEVICE;
  DecodeParams p = prm;
  void* args[] = {&p};
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(P), dim3(kDecodeThreads), args, 0, s);
  return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

}  // namespace gsi
