// Persistent batch-1 GSI decode kernel for gfx950.
//
// Method: "Gated Subspace Inference for transformer acceleration" technical summary
// (gist.science, arXiv 2605.03109). Per token and per site (linear layer) [GSI §2.1-§2.2]:
//   g = V^T x;  nr2 = |x - V g|^2 = |x|^2 - |g|^2 + g^T (V^T V - I) g;  fast iff nr2 < eps^2 |x|^2
//   fast: y = M g (M = W V cached)      slow: y = W x
// Every linear site of every block runs in order [GSI §3], one token at a time.
//
// Design (one block per CU, all blocks co-resident via a cooperative launch):
//  * Work split per site (gsi_plan.h): block b owns the g columns j = b, b + P, ... (rows of V^T:
//    each g_j is one complete d-long dot product inside one block) and a contiguous slice of
//    output rows of M / W. The split of every (site, block) is precomputed at creation as a
//    128-byte plan row; every wave loads the row it needs a step ahead into its own registers and
//    moves it to scalar registers while it waits anyway, so a step starts without waiting for
//    descriptor loads or index arithmetic.
//  * Two all-gather exchanges per site: (E1) every block needs all of g for its rows of M g;
//    (E2) the gate needs the global sum of per-block pieces of g^T (V^T V - I) g. A block posts
//    its E2 word only after its rows of y are stored, so E2 is also the completion of the site:
//    no block starts the next site before every block has finished this one. A slow token adds
//    (E3), the completion of the W x rows.
//  * Weights stream into LDS ahead of use: two 64 KB site regions alternate with the step
//    parity. Right after posting its E1 word, a block's data waves copy its slices of the next
//    step's site (its V^T rows, its rows of V^T V - I and its rows of M) from HBM straight into
//    the other region (global_load_lds, 16 bytes per lane, no registers); the copy drains while
//    E1 resolves. Nothing bulky is in flight on the CU while E2 resolves: only the next input row,
//    read into registers after this block's rows of y are stored and used only after E2 has
//    completed. Slices that do not fit a region are read from global memory when used.
//  * y = M g runs on the vector ALU (each row split over a few lanes of one wave, DPP sums): at
//    batch 1 the product is a matrix-vector product, bound by the bytes of M, not by arithmetic.
//  * Exchanges use tagged 64-bit mailbox words (tag << 32 | payload) with one copy per XCD, so
//    a block polls the copy on its own XCD's side; stores and polls are device-scope. Tags come
//    from the workspace's 64-bit epoch (gsi_plan.h: step_tag); every launch first rewrites the
//    words it owns with a tag no poll uses, so no word older than the previous launch survives.
//  * One wave per block (the sync wave) does all polling and posting; four data waves copy and
//    compute. Every wait is bounded: past the bound the launch is marked aborted and every block
//    leaves, so a lost block cannot hang the device.
//  * Gate arithmetic is done identically (same data, same order) in every block, so all blocks
//    take the same branch.
//  * Site modes (gsi_plan.h): a static-projection site skips the V^T V - I rows and the gate
//    (y = M g, E2 as the completion only); a dense site skips g and E1 (y = W x, then E2).
#include <algorithm>

#include "gsi_internal.h"

namespace gsi {

// Phase timeline (a build option for profiling; compiled out of libgsi): with GSI_PHASE_STAMPS,
// the sync wave of blocks 0, 100 and 200 stores a wall-clock stamp at each phase boundary of the
// 16 site steps q = GSI_PHASE_Q0 .. + 15 of a launch; gsi_phase_stamps copies them out.
#ifdef GSI_PHASE_STAMPS
#ifndef GSI_PHASE_Q0
#define GSI_PHASE_Q0 512
#endif
__device__ unsigned long long g_phase_stamps[3][16][11];
#define GSI_PHASE(i)                                                                                   \
  do {                                                                                                 \
    if (c.tid == kDataThreads && c.q >= GSI_PHASE_Q0 && c.q < GSI_PHASE_Q0 + 16) {                     \
      const int bi_ = c.b == 0 ? 0 : (c.b == 100 ? 1 : (c.b == 200 ? 2 : -1));                          \
      if (bi_ >= 0) g_phase_stamps[bi_][c.q - GSI_PHASE_Q0][i] = wall_clock64();                       \
    }                                                                                                  \
  } while (0)
#else
#define GSI_PHASE(i) \
  do {               \
  } while (0)
#endif

constexpr int kSlowBatch = 8;  // W / x chunk pairs per lane in flight on the W x rows
constexpr unsigned long long kWaitTicks = 200000000ull;  // 2 s at the 100 MHz wall clock

// A 16-byte chunk as a built-in vector (address-space-qualified pointers to it copy cleanly).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* g4p;  // global memory, read
typedef __attribute__((address_space(3))) void lds_void;
typedef u32x4 __attribute__((address_space(3))) lu32x4;  // a 16-byte chunk in LDS
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ldg(g4p p, long long i) { return p[i]; }
__device__ __forceinline__ g4p gptr(unsigned long long a) { return (g4p)(uintptr_t)a; }

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
  acc = __builtin_fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = __builtin_fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = __builtin_fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = __builtin_fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  return acc;
}

// One 16-byte chunk of a weight row against float32 values of g held in registers.
template <typename T>
__device__ __forceinline__ float dot_chunk_g(const u32x4& a, const float* g, float acc) {
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
__device__ __forceinline__ float wave_reduce(float v) { return group_reduce(v, 64); }

// Plan rows travel through each wave's own registers: lane l (l < 5) loads 16-byte chunk l of the
// row (the other lanes load the last chunk again, unused), and plan_unpack moves the 20 words to
// scalar registers. A wave only ever reads rows it loaded itself, so no wave waits on another's.
__device__ __forceinline__ u32x4 plan_load(const PlanRow* table, int s, int b, int P, int lane) {
  return ldg((g4p)(table + (long long)s * P + b), lane < kPlanChunks ? lane : kPlanChunks - 1);
}
__device__ __forceinline__ PlanRow plan_unpack(const u32x4& v) {
  PlanRow p;
  unsigned* dst = reinterpret_cast<unsigned*>(&p);
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < (int)(sizeof(PlanRow) / 4); ++i)
    dst[i] = (unsigned)__builtin_amdgcn_readlane((int)w[i & 3], i >> 2);
  return p;
}

// Copy instructions of a site's region fill; instruction i (chunks 64 i .. 64 i + 63 of the
// region) is issued by data wave i mod 4. Each lane reads one 16-byte chunk from global memory
// straight into LDS at region + 16 (64 i + lane). Padding chunks read a valid dummy chunk, so
// every lane issues exactly one load.
__device__ __forceinline__ void fill_region(const PlanRow& g, int P, int wave, int lane, lu32x4* region,
                                            const u32x4* dummy) {
  for (int i = wave; i < g.n_inst; i += 4) {
    const unsigned long long a = fill_source(g, P, i, lane);
    const void* src = a ? (const void*)(uintptr_t)a : (const void*)dummy;
    // streamed once per token: non-temporal, so the copy does not displace cached lines
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(region + i * 64), 16, 0, 2 /* nt */);
  }
}

// The input row's chunks tid + 256 u (u < XR) into registers; slots past the row re-read chunk 0.
template <int XR>
__device__ __forceinline__ void load_x(const void* xrow, int cprd, int tid, u32x4 (&xw)[XR]) {
  const g4p xp = (g4p)xrow;
#pragma unroll
  for (int u = 0; u < XR; ++u) {
    const int cc = tid + u * kDataThreads;
    xw[u] = xp[cc < cprd ? cc : 0];
  }
}

struct DecodeParams {
  const PlanRow* plan;  // [n_sites][P] plan rows
  int n_sites, n_steps, t_step;
  const void* X;
  long long x_ld;
  void* Y;
  long long y_ld;
  uint8_t* gates;  // [n_steps * t_step, gate_ld]
  float* rho;      // optional
  int gate_ld;
  float eps;
  WsHeader* hdr;
  u64* box_g;  // [kReplicas][kMaxK]       g values
  u64* box_p;  // [kReplicas][kMaxBlocks]  per-block gate pieces / site completion
  u64* box_f;  // [kReplicas][kMaxBlocks]  W x completion
};

// Order of the steps: steps of t_step tokens in order; inside a step the sites in order; inside a
// site the step's tokens in order.
struct Cursor {
  int s, tis, step;
  __device__ __forceinline__ void advance(int n_sites, int t_step) {
    if (++tis == t_step) {
      tis = 0;
      if (++s == n_sites) {
        s = 0;
        ++step;
      }
    }
  }
  __device__ __forceinline__ long long token(int t_step) const { return (long long)step * t_step + tis; }
};

// A block whose wait runs past its bound marks this launch (epoch + 1) as aborted; every other
// block polls that mark while it waits, so the whole grid leaves promptly. The mark of an older
// launch never matches because every launch advances the epoch.
__device__ __forceinline__ void record_abort(const DecodeParams& p, unsigned long long base) {
  __hip_atomic_store(&p.hdr->abort_mark, base + 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p.hdr->status, (int)GSI_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sync wave: poll `n` tagged words of mailbox copy `mb` until all carry `tag`; values go to `out`
// (per lane, entries lane + 64 i; zero past n). One poll issues all of its loads back to back
// (slots past n re-read entry n - 1) together with the launch's abort mark, then waits once, so
// a poll costs one memory round trip. Returns false on timeout or abort.
template <int NI>
__device__ __forceinline__ bool gather(const DecodeParams& p, unsigned long long base, const u64* mb, int n,
                                       unsigned tag, int lane, float (&out)[NI]) {
  const unsigned long long t0 = wall_clock64();
  while (true) {
    u64 wv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = lane + 64 * i;
      wv[i] = ld_dev(mb + (j < n ? j : n - 1));
    }
    const unsigned long long ab = __hip_atomic_load(&p.hdr->abort_mark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      ok &= (unsigned)(wv[i] >> 32) == tag;
      out[i] = (lane + 64 * i < n) ? __uint_as_float((unsigned)wv[i]) : 0.f;
    }
    if (__all(ok)) return true;
    if (ab == base + 1ull || wall_clock64() - t0 > kWaitTicks) {
      if (lane == 0) record_abort(p, base);
      return false;
    }
  }
}

// LDS shared by the phases of one site (the two site regions are separate arrays so that the
// compiler can tell a copy into one region from reads of the other).
struct Shared {
  float* gsh;    // [kMaxK] gathered g
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
__device__ __forceinline__ RowLanes row_lanes(int cprk, int lane) {
  RowLanes q;
  q.CPL = min(4, cprk);
  q.Lr = cprk >> __builtin_ctz(q.CPL);  // lanes per row (a power of two <= 32)
  q.rpw = 64 / q.Lr;                    // rows per wave per pass
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
// rows [0, m_rows) from the region, rows [m_rows, nrows) from HBM
template <typename T>
__device__ __forceinline__ void fast_rows(const PlanRow& g, const lu32x4* cur, const Shared& sh, int wave, int lane) {
  const RowLanes q = row_lanes(g.cprk, lane);
  float gl[4][vec16<T>::N];
  g_slices<T>(sh, q, gl);
  for (int rp = 0; rp < g.m_rows; rp += 4 * q.rpw) {
    const int r = rp + wave * q.rpw + q.lr;
    const bool ok = r < g.m_rows;
    const int rr = ok ? r : 0;
    u32x4 mv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mv[i] = cur[lds_m(g, rr, q.ch[i])];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = dot_chunk_g<T>(mv[i], gl[i], 0.f);
      acc += i < q.CPL ? d : 0.f;
    }
    acc = group_reduce(ok ? acc : 0.f, q.Lr);
    if (ok && q.lc == q.Lr - 1) sh.ypart[r] = acc;
  }
  if (g.m_rows < g.nrows) {
    const g4p mrow = gptr(g.m);
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
        const float d = dot_chunk_g<T>(mv[i], gl[i], 0.f);
        acc += i < q.CPL ? d : 0.f;
      }
      acc = group_reduce(ok ? acc : 0.f, q.Lr);
      if (ok && q.lc == q.Lr - 1) sh.ypart[r] = acc;
    }
  }
}

// The block's rows of y = W x straight from HBM: one wave per row, each lane keeping kSlowBatch
// chunk pairs in flight.
template <typename T>
__device__ __forceinline__ void dense_rows(unsigned long long w, int nrows, int cprd, const T* x, T* yrow, int wave,
                                           int lane) {
  const g4p x4 = (g4p)x;
  for (int r = wave; r < nrows; r += kDataThreads / 64) {
    const g4p wr = gptr(w) + (long long)r * cprd;
    float a = 0.f;
    for (int c0 = 0; c0 < cprd; c0 += kSlowBatch * 64) {
      u32x4 wv[kSlowBatch], xv[kSlowBatch];
#pragma unroll
      for (int i = 0; i < kSlowBatch; ++i) {
        const int c = c0 + lane + 64 * i;
        const int cc = c < cprd ? c : 0;
        wv[i] = wr[cc];
        xv[i] = x4[cc];
      }
#pragma unroll
      for (int i = 0; i < kSlowBatch; ++i) {
        const float v = dot16<T>(wv[i], xv[i], 0.f);
        a += (c0 + lane + 64 * i < cprd) ? v : 0.f;
      }
    }
    a = wave_reduce(a);
    if (lane == 63) yrow[r] = from_f32<T>(a);
  }
}

struct StepCtx {
  long long q, Q;
  unsigned long long base;
  int b, P, tid;
  unsigned rep;
  const u32x4* dummy;
};

// One (token, site) step. `cur` holds this step's slices (filled during the previous step); `nxt`
// receives the next step's. Plan rows arrive in scalar registers: g is this step's (every wave),
// gn the next step's (data waves only). Each wave loads the row it will need one step later at the
// start of this step (data waves: the row after next; the sync wave: the next) and unpacks it where
// it would otherwise wait: the data waves once their own loads have completed, the sync wave right
// after posting its E2 word. Returns false when the launch was aborted.
template <typename T, int XR>
__device__ __forceinline__ bool site_step(const DecodeParams& p, const StepCtx& c, const Cursor& cq, const lu32x4* cur,
                                          lu32x4* nxt, u32x4 (&xw)[XR], const Shared& sh, PlanRow& g, PlanRow& gn) {
  const int tid = c.tid, b = c.b, P = c.P;
  const bool is_sync = tid >= kDataThreads;
  const int lane = tid & 63, wave = tid >> 6;
  const bool has_next = c.q + 1 < c.Q, has_next2 = c.q + 2 < c.Q;
  // what the step still needs after g and gn are replaced by the next step's rows
  const int mode = g.mode, nrows = g.nrows, cprd = g.cprd;
  const unsigned long long w_rows = g.w;
  GSI_PHASE(10);  // step entry
  Cursor cn = cq;
  cn.advance(p.n_sites, p.t_step);
  Cursor c2 = cn;
  c2.advance(p.n_sites, p.t_step);
  const long long t = cq.token(p.t_step);
  // the plan row this wave needs one step from now (loads of a row in bounds even when unused)
  const u32x4 plan_ahead = is_sync ? plan_load(p.plan, has_next ? cn.s : cq.s, b, P, lane)
                                   : plan_load(p.plan, has_next2 ? c2.s : cq.s, b, P, lane);
  const unsigned tag_g = step_tag(c.base, c.q, 1), tag_p = step_tag(c.base, c.q, 2), tag_f = step_tag(c.base, c.q, 3);
  const T* x = reinterpret_cast<const T*>(p.X) + t * p.x_ld + g.x_off;
  T* yrow = reinterpret_cast<T*>(p.Y) + t * p.y_ld + g.y_off;
  const long long vt_stride = (long long)P * g.cprd;  // chunks between owned V^T rows

  if (mode == kSiteDense) {
    // ---------------- dense site: y = W x for the owned rows, then the completion exchange -------------
    if (!is_sync) {
      dense_rows<T>(w_rows, nrows, cprd, x, yrow, wave, lane);
      if (has_next) {
        fill_region(gn, P, wave, lane, nxt, c.dummy);
        load_x<XR>(reinterpret_cast<const T*>(p.X) + cn.token(p.t_step) * p.x_ld + gn.x_off, gn.cprd, tid, xw);
      }
      wait_vmcnt<0>();  // rows of y stored; next region, plan row and input row complete
      g = gn;
      gn = plan_unpack(plan_ahead);
    }
    __syncthreads();
    if (is_sync) {
      if (lane < kReplicas) st_dev(p.box_p + (long long)lane * kMaxBlocks + b, pack(tag_p, 0.f));
      g = plan_unpack(plan_ahead);
      float pv[kMaxBlocks / 64];
      const bool ok = gather(p, c.base, p.box_p + (long long)c.rep * kMaxBlocks, P, tag_p, lane, pv);
      if (!ok && lane == 0) *sh.s_abort = 1;
      if (b == 0 && lane == 0) {
        const long long o = t * p.gate_ld + cq.s;
        p.gates[o] = 1;
        if (p.rho) p.rho[o] = __builtin_nanf("");
      }
    }
    __syncthreads();
    return !*sh.s_abort;
  }

  // ---------------- phase A (data waves): g_j for owned columns and |x|^2 ----------------
  GSI_PHASE(0);
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
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < XR; ++u) {
          if (u * kDataThreads < g.cprd) {  // uniform
            const int cc = tid + u * kDataThreads;
            const bool in = cc < g.cprd;
            const u32x4 vv = cur[lds_vt(g, jl, in ? cc : 0)];
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
        const g4p vr = gptr(g.vt) + (long long)jl * vt_stride;
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
  GSI_PHASE(1);
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
  GSI_PHASE(2);
  if (!is_sync) {
    if (has_next) fill_region(gn, P, wave, lane, nxt, c.dummy);
  } else {
    float gv[kMaxK / 64];
    const bool ok = gather(p, c.base, p.box_g + (long long)c.rep * kMaxK, g.k, tag_g, lane, gv);
    GSI_PHASE(3);
    if (!ok && lane == 0) *sh.s_abort = 1;
    float gg = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxK / 64; ++i) {
      const int j = lane + 64 * i;
      if (j < g.k) sh.gsh[j] = gv[i];
      gg = __builtin_fmaf(gv[i], gv[i], gg);
    }
    gg = wave_reduce(gg);
    if (lane == 63) *sh.s_gg = gg;
  }
  lds_barrier();
  GSI_PHASE(4);
  if (*sh.s_abort) return false;

  // ------- phase B (data waves): this block's rows of y = M g; (sync wave) the gate piece -------
  float pb = 0.f;
  if (!is_sync) {
    fast_rows<T>(g, cur, sh, wave, lane);
  } else if (mode == kSiteGated) {
    // p_b = sum_j g_j ((V^T V - I) g)_j over the owned columns; chunk e covers owned row
    // e / cpk4, columns 4 (e mod cpk4) .. + 3
    const int nd = g.nJ * g.cpk4;
    const int sh4 = __builtin_ctz(g.cpk4);
    float pp = 0.f;
    for (int e = lane; e < nd; e += 64) {
      const int jl = e >> sh4, cc = e & (g.cpk4 - 1);
      float gjl = gj_own[0];
#pragma unroll
      for (int jj = 1; jj < kMaxJ; ++jj) gjl = (jl == jj) ? gj_own[jj] : gjl;
      const u32x4 dv = g.d_n > 0 ? cur[lds_dl(g, e)] : ldg(gptr(g.dl), (long long)jl * P * g.cpk4 + cc);
      pp += dot_f32x4_lds(dv, sh.gsh + cc * 4, 0.f) * gjl;
    }
    pp = wave_reduce(pp);
    pb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pp), 63));
  }
  lds_barrier();
  // ---- the sync wave stores this block's rows of y, then posts its E2 word (site done) ----
  GSI_PHASE(5);
  if (is_sync) {
    for (int r = lane; r < nrows; r += 64) yrow[r] = from_f32<T>(sh.ypart[r]);
    if (lane < kReplicas) st_dev(p.box_p + (long long)lane * kMaxBlocks + b, pack(tag_p, pb));
  }
  lds_barrier();  // the y rows and the E2 word are issued ahead of the loads below
  GSI_PHASE(6);
  if (!is_sync) {
    // the next input row streams in while E2 resolves
    if (has_next) load_x<XR>(reinterpret_cast<const T*>(p.X) + cn.token(p.t_step) * p.x_ld + gn.x_off, gn.cprd, tid, xw);
    wait_vmcnt<0>();  // the next region, plan row and input row are complete before the barrier below
    g = gn;
    gn = plan_unpack(plan_ahead);
  } else {
    g = plan_unpack(plan_ahead);  // overlaps the wait for the other blocks' E2 words
    // ---------------- E2: all-gather the pieces, resolve the gate ----------------
    float pv[kMaxBlocks / 64];
    const bool ok = gather(p, c.base, p.box_p + (long long)c.rep * kMaxBlocks, P, tag_p, lane, pv);
    GSI_PHASE(7);
    if (!ok && lane == 0) *sh.s_abort = 1;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxBlocks / 64; ++i) ps += pv[i];
    ps = wave_reduce(ps);
    if (lane == 63) {
      int slow = 0;
      float r = __builtin_nanf("");
      if (mode == kSiteGated) {
        const float nx2 = *sh.s_nx2;
        const float nr2 = (nx2 - *sh.s_gg) + ps;
        const float thr = p.eps * p.eps;
        const float rhs = thr * nx2;
        slow = (nr2 < rhs) ? 0 : 1;
        r = sqrtf(fmaxf(nr2, 0.f) / nx2);
      }
      *sh.s_gate = slow;
      if (b == 0) {
        const long long o = t * p.gate_ld + cq.s;
        p.gates[o] = (uint8_t)slow;
        if (p.rho) p.rho[o] = r;
      }
    }
  }
  lds_barrier();
  GSI_PHASE(8);
  if (*sh.s_abort) return false;

  // ---------------- slow path: y = W x for the owned rows, then E3 ----------------
  if (*sh.s_gate) {
    // the sync wave's fast-path stores to these rows of y complete before the W x rows replace
    // them (only here: on the fast path nothing waits for stores)
    if (is_sync) wait_vmcnt<0>();
    __syncthreads();
    if (!is_sync) {
      dense_rows<T>(w_rows, nrows, cprd, x, yrow, wave, lane);
      wait_vmcnt<0>();
    }
    __syncthreads();
    if (is_sync) {
      if (lane < kReplicas) st_dev(p.box_f + (long long)lane * kMaxBlocks + b, pack(tag_f, 0.f));
      float fv[kMaxBlocks / 64];
      if (!gather(p, c.base, p.box_f + (long long)c.rep * kMaxBlocks, P, tag_f, lane, fv) && lane == 0) *sh.s_abort = 1;
    }
    __syncthreads();
    if (*sh.s_abort) return false;
  }
  GSI_PHASE(9);
  return true;
}

template <typename T, int XR>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
  __shared__ u32x4 region0[kRegionChunks];
  __shared__ u32x4 region1[kRegionChunks];
  __shared__ float gsh[kMaxK];
  __shared__ float ypart[kYPart];
  __shared__ float red[kDecodeThreads / 64][kMaxJ + 2];
  __shared__ float s_nx2, s_gg;
  __shared__ int s_gate, s_abort;
  __shared__ unsigned long long s_base;

  const int tid = threadIdx.x;
  const int b = blockIdx.x, P = gridDim.x;
  const bool is_sync = tid >= kDataThreads;
  const int lane = tid & 63, wave = tid >> 6;
  const Shared sh{gsh, ypart, red, &s_nx2, &s_gg, &s_gate, &s_abort};
  lu32x4* const r0 = (lu32x4*)region0;
  lu32x4* const r1 = (lu32x4*)region1;
  const long long Q = (long long)p.n_steps * p.t_step * p.n_sites;

  if (tid == 0) {
    s_abort = 0;
    s_base = __hip_atomic_load(&p.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const unsigned long long base = s_base;
  if (is_sync && lane < kReplicas) {
    // rewrite every mailbox word this block owns (all replicas) with the launch's unused tag
    const u64 w0 = pack((unsigned)base, 0.f);
    for (int j = b; j < kMaxK; j += P) st_dev(p.box_g + (long long)lane * kMaxK + j, w0);
    for (int j = b; j < kMaxBlocks; j += P) {
      st_dev(p.box_p + (long long)lane * kMaxBlocks + j, w0);
      st_dev(p.box_f + (long long)lane * kMaxBlocks + j, w0);
    }
  }
  const StepCtx c0{0, Q, base, b, P, tid, xcc_id() % kReplicas, reinterpret_cast<const u32x4*>(p.hdr)};

  u32x4 xw[XR];
  // plan rows of steps 0 and 1 (every wave its own copy), step 0's region and input row
  const int s1 = p.t_step > 1 ? 0 : (p.n_sites > 1 ? 1 : 0);
  PlanRow g = plan_unpack(plan_load(p.plan, 0, b, P, lane));
  PlanRow gn = plan_unpack(plan_load(p.plan, s1, b, P, lane));
  if (Q > 0 && !is_sync) {
    load_x<XR>(reinterpret_cast<const T*>(p.X) + g.x_off, g.cprd, tid, xw);
    fill_region(g, P, wave, lane, r0, c0.dummy);
    wait_vmcnt<0>();
  }
  __syncthreads();

  Cursor cq{0, 0, 0};
  StepCtx c = c0;
  for (long long q = 0; q < Q; q += 2) {
    c.q = q;
    if (!site_step<T, XR>(p, c, cq, r0, r1, xw, sh, g, gn)) break;
    cq.advance(p.n_sites, p.t_step);
    if (q + 1 >= Q) break;
    c.q = q + 1;
    if (!site_step<T, XR>(p, c, cq, r1, r0, xw, sh, g, gn)) break;
    cq.advance(p.n_sites, p.t_step);
  }
  if (!is_sync) wait_vmcnt<0>();  // no copy into LDS outlives the block
  // advance the epoch for the next launch (also after an abort, so its mark goes stale)
  if (b == 0 && tid == 0)
    __hip_atomic_store(&p.hdr->epoch, next_epoch(base, Q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

size_t decode_ws_bytes() {
  return sizeof(WsHeader) + (size_t)kReplicas * kMaxK * 8 + 2 * (size_t)kReplicas * kMaxBlocks * 8;
}

void decode_boxes(void* ws, WsHeader** hdr, u64** box_g, u64** box_p, u64** box_f) {
  char* c = (char*)ws;
  *hdr = (WsHeader*)c;
  c += sizeof(WsHeader);
  *box_g = (u64*)c;
  c += (size_t)kReplicas * kMaxK * 8;
  *box_p = (u64*)c;
  c += (size_t)kReplicas * kMaxBlocks * 8;
  *box_f = (u64*)c;
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

int decode_window(int dtype, const LayerDesc* sites, int n_sites) {
  const int es = dtype == GSI_F32 ? 4 : 2;
  int need_x = 1;
  for (int i = 0; i < n_sites; ++i) need_x = std::max(need_x, (sites[i].d * es / 16 + kDataThreads - 1) / kDataThreads);
  return need_x;
}

int decode_grid(int dtype, int xr) {
  const void* fn = decode_fn(dtype, xr);
  if (!fn) return 0;
  int dev = 0, ncu = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kDecodeThreads, 0) != hipSuccess) return 0;
  long long cap = (long long)ncu * per;
  int P = (int)(cap < kMaxBlocks ? cap : kMaxBlocks);
  while (P & (P - 1)) P &= P - 1;  // a power of two: the work split uses shifts
  return P < kMinBlocks ? 0 : P;
}

__global__ void plan_kernel(LayerDesc d, int P, int es, PlanRow* out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < P) out[b] = make_plan_row(d, b, P, es);
}

int launch_plan(const LayerDesc& d, int P, int es, PlanRow* out, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3((P + 255) / 256), dim3(256), 0, s, d, P, es, out);
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

static int launch_decode_as(int dtype, const DecodeArgs& a, hipStream_t s, bool cooperative) {
  const void* fn = decode_fn(dtype, a.xr);
  if (!fn) return GSI_ERR_DTYPE;
  DecodeParams p;
  p.plan = a.plan;
  p.n_sites = a.n_sites;
  p.n_steps = a.n_steps;
  p.t_step = a.t_step;
  p.X = a.X;
  p.x_ld = a.x_ld;
  p.Y = a.Y;
  p.y_ld = a.y_ld;
  p.gates = a.gates;
  p.rho = a.rho;
  p.gate_ld = a.gate_ld;
  p.eps = a.eps;
  decode_boxes(a.ws, &p.hdr, &p.box_g, &p.box_p, &p.box_f);
  void* args[] = {&p};
  hipError_t e = cooperative ? hipLaunchCooperativeKernel(fn, dim3(a.P), dim3(kDecodeThreads), args, 0, s)
                             : hipLaunchKernel(fn, dim3(a.P), dim3(kDecodeThreads), args, 0, s);
  return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

int launch_decode(int dtype, const DecodeArgs& a, hipStream_t s) { return launch_decode_as(dtype, a, s, true); }

// The same grid as an ordinary launch. The grid is one a device holds at once (decode_grid), the
// launch starts after the stream's earlier work has finished, and every wait inside the kernel is
// bounded, so a block that becomes resident late only delays the others. The cooperative launch
// switches queues before and after the kernel (about 10 us each way); a call that decodes a single
// token would spend more time there than in the kernel.
int launch_decode_resident(int dtype, const DecodeArgs& a, hipStream_t s) {
  return launch_decode_as(dtype, a, s, false);
}

}  // namespace gsi

#ifdef GSI_PHASE_STAMPS
// the phase stamps of the last launch: 3 blocks x 16 site steps x 11 stamps, wall-clock ticks
extern "C" int gsi_phase_stamps(unsigned long long* out) {
  return hipMemcpyFromSymbol(out, HIP_SYMBOL(gsi::g_phase_stamps), sizeof(gsi::g_phase_stamps)) == hipSuccess ? 0 : -1;
}
#endif
