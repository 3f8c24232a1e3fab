// Work split of the persistent batch-1 decode kernel: which slices of a site each block owns,
// where they sit in the block's LDS region, and where every 16-byte chunk of the region is copied
// from. Plain C++ (no HIP types), compiled into the kernels and into the host-side check of the
// index arithmetic, so both use exactly these functions.
//
// Method: "Gated Subspace Inference for transformer acceleration" technical summary
// (gist.science, arXiv 2605.03109), §2.1-§2.2: per token, g = V^T x, the residual norm, the
// gate, then y = M g (fast) or y = W x (slow).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define GSI_HD __host__ __device__ __forceinline__
#else
#define GSI_HD inline
#endif

namespace gsi {

// What a site computes. GATED is the method [GSI §2.2]; STATIC is the gateless fast path
// y = M g for every token (static projection, the eps > 1 limit of the gate); DENSE is y = W x for
// every token (a linear map left outside the method, e.g. attention maps when only the MLP maps
// are gated).
enum SiteMode { kSiteGated = 0, kSiteStatic = 1, kSiteDense = 2 };

// One site as the library stores it (device and host copies).
struct LayerDesc {
  const void* Vt;     // [k, d]
  const void* M;      // [d_out, k]
  const float* Dl;    // [k, k] = V^T V - I
  const void* W;      // [d_out, d]
  const void* VDt;    // [k, d] = (V (V^T V - I))^T in the weight dtype (16-bit layers; batched gate)
  int d, d_out, k, mode;
  long long x_off, y_off;  // column offsets into stacked X / Y rows
};

constexpr int kMaxJ = 4;             // g columns per block (k <= 512 with at least 128 blocks)
constexpr int kRegionChunks = 4096;  // 16-byte chunks per LDS site region (64 KB)
constexpr int kDataThreads = 256;    // 4 data waves per block
constexpr int kPlanChunks = 5;       // 16-byte chunks of one plan row

// Block b's share of one site, for a grid of P blocks (P a power of two). Addresses are byte
// addresses already offset to the block's first owned row.
//  * g columns: j = b, b + P, ... < k (nJ of them), i.e. complete d-long rows of V^T.
//  * output rows: [r0, r0 + nrows), contiguous, ceil(d_out / P) per block.
//  * LDS region (16-byte chunks): [V^T rows | (V^T V - I) rows | M rows], each part starting on a
//    64-chunk boundary so that one 64-lane copy instruction lies inside one part. Parts that do
//    not fit are read from global memory when used: V^T rows from vj on, all of V^T V - I when it
//    does not fit, M rows from m_rows on (m_n is all of the slice or a multiple of 256 chunks, so
//    one pass of the 256 data threads never mixes LDS and global reads).
// Counts are 16-bit (every one is at most 8192 for the shapes the library accepts) so that a row
// is 80 bytes and two of them fit in a wave's scalar registers.
struct alignas(16) PlanRow {
  unsigned long long vt;  // V^T row b; owned row jl is vt + jl * P * cprd * 16
  unsigned long long dl;  // row b of V^T V - I; owned row jl is dl + jl * P * cpk4 * 16
  unsigned long long m;   // M row r0
  unsigned long long w;   // W row r0
  int x_off;              // element offset of the site's input in a stacked input row
  int y_off;              // element offset of output row r0 in a stacked output row
  unsigned short mode;    // SiteMode
  unsigned short k;
  unsigned short nJ;      // g columns owned
  unsigned short vj;      // V^T rows held in the region
  unsigned short cprd;    // 16-byte chunks per V^T / W row (d / elements per chunk)
  unsigned short nx;      // input chunks per data thread (ceil(cprd / 256))
  unsigned short cprk;    // 16-byte chunks per M row
  unsigned short cpk4;    // 16-byte chunks per (V^T V - I) row (k / 4, float32)
  unsigned short nrows;   // output rows owned
  unsigned short m_rows;  // rows of the M slice held in the region
  unsigned short v_n;     // V^T chunks held (at offset 0)
  unsigned short d_off, d_n;  // (V^T V - I) part: offset and chunks held (all or none)
  unsigned short m_off, m_n;  // M part: offset and chunks held
  unsigned short n_inst;      // 64-chunk copy instructions that fill the region
  int r0;                 // first output row owned
  int pad;
};
static_assert(sizeof(PlanRow) == kPlanChunks * 16, "a plan row is five 16-byte chunks");

GSI_HD int plan_align64(int v) { return (v + 63) & ~63; }
GSI_HD int plan_ctz(unsigned v) { return __builtin_ctz(v); }  // v > 0
GSI_HD int plan_min(int a, int b) { return a < b ? a : b; }
GSI_HD int plan_max(int a, int b) { return a > b ? a : b; }

// es: bytes per element of W, V^T, M, x (2 or 4). P: blocks of the grid (a power of two).
GSI_HD PlanRow make_plan_row(const LayerDesc& L, int b, int P, int es) {
  const int VW = 16 / es;  // elements per 16-byte chunk
  const int sh_P = plan_ctz((unsigned)P);
  const int cprd = L.d / VW, cprk = L.k / VW, cpk4 = L.k / 4;
  const int rpb = (L.d_out + P - 1) >> sh_P;
  const int r0 = plan_min(L.d_out, b * rpb);
  const int nrows = plan_min(L.d_out, r0 + rpb) - r0;
  const bool dense = L.mode == kSiteDense;
  const int nJ = (!dense && b < L.k) ? ((L.k - 1 - b) >> sh_P) + 1 : 0;
  int vj = nJ;  // V^T rows that fit the region
  while (vj > 0 && vj * cprd > kRegionChunks) --vj;
  const int v_n = vj * cprd;
  const int d_off = plan_align64(v_n);
  const int nd = L.mode == kSiteGated ? nJ * cpk4 : 0;
  const int d_n = d_off + nd <= kRegionChunks ? nd : 0;
  const int m_off = plan_align64(d_off + d_n);
  const int nm = dense ? 0 : nrows * cprk;
  const int m_n = m_off + nm <= kRegionChunks ? nm : plan_max(0, (kRegionChunks - m_off) / kDataThreads * kDataThreads);
  PlanRow p;
  p.mode = (unsigned short)L.mode;
  p.k = (unsigned short)L.k;
  p.nJ = (unsigned short)nJ;
  p.vj = (unsigned short)vj;
  p.cprd = (unsigned short)cprd;
  p.nx = (unsigned short)((cprd + kDataThreads - 1) / kDataThreads);
  p.cprk = (unsigned short)cprk;
  p.cpk4 = (unsigned short)cpk4;
  p.nrows = (unsigned short)nrows;
  p.m_rows = (unsigned short)(cprk > 0 ? m_n / cprk : 0);
  p.v_n = (unsigned short)v_n;
  p.d_off = (unsigned short)d_off;
  p.d_n = (unsigned short)d_n;
  p.m_off = (unsigned short)m_off;
  p.m_n = (unsigned short)m_n;
  p.n_inst = (unsigned short)((m_off + m_n + 63) / 64);
  p.vt = (unsigned long long)(uintptr_t)L.Vt + (unsigned long long)b * cprd * 16;
  p.dl = (unsigned long long)(uintptr_t)L.Dl + (unsigned long long)b * cpk4 * 16;
  p.m = (unsigned long long)(uintptr_t)L.M + (unsigned long long)r0 * cprk * 16;
  p.w = (unsigned long long)(uintptr_t)L.W + (unsigned long long)r0 * cprd * 16;
  p.x_off = (int)L.x_off;
  p.y_off = (int)(L.y_off + r0);
  p.r0 = r0;
  p.pad = 0;
  return p;
}

// Source address of region chunk c = 64 i + lane (copy instruction i, lane 0..63), or 0 for a
// padding chunk (the caller reads a valid dummy chunk there).
GSI_HD unsigned long long fill_source(const PlanRow& p, int P, int i, int lane) {
  const int c = i * 64 + lane;
  if (c < p.v_n) {  // V^T row jl = c / cprd (at most kMaxJ rows: compares, no division)
    int jl = 0;
    for (int r = 1; r < kMaxJ; ++r) jl += c >= r * p.cprd ? 1 : 0;
    const int cc = c - jl * p.cprd;
    return p.vt + ((unsigned long long)jl * P * p.cprd + cc) * 16;
  }
  if (c >= p.d_off && c < p.d_off + p.d_n) {
    const int e = c - p.d_off;
    const int sh = plan_ctz((unsigned)p.cpk4);
    const int jl = e >> sh, cc = e & (p.cpk4 - 1);
    return p.dl + ((unsigned long long)jl * P * p.cpk4 + cc) * 16;
  }
  if (c >= p.m_off && c < p.m_off + p.m_n) return p.m + (unsigned long long)(c - p.m_off) * 16;
  return 0;
}

// Region chunk holding chunk cc of owned V^T row jl (jl < vj), chunk e = jl * cpk4 + cc of the
// owned (V^T V - I) rows (when d_n > 0), chunk ch of owned M row r (r < m_rows).
GSI_HD int lds_vt(const PlanRow& p, int jl, int cc) { return jl * p.cprd + cc; }
GSI_HD int lds_dl(const PlanRow& p, int e) { return p.d_off + e; }
GSI_HD int lds_m(const PlanRow& p, int r, int ch) { return p.m_off + r * p.cprk + ch; }

// Mailbox tags. A launch reads the 64-bit epoch E of its workspace and tags the words of step q
// with the low 32 bits of E + 4 q + kind (g words 1, gate pieces 2, slow-path completion 3). Every
// block first rewrites every mailbox word it owns (all replicas) with the tag of E itself, which
// no poll uses, and block 0 finally advances the epoch to E + 4 Q + 4 for a launch of Q steps.
// A word polled at step q of a launch therefore holds either a write of this launch (tag E + 4 q'
// + kind' for some q' <= q, or E) or, before this launch's rewrite of it lands, a write of the
// previous launch on the workspace (tags in [E - 4 Q_prev - 4, E - 1]). Both differ from the
// polled tag modulo 2^32 unless the word was written at step q with the same kind, as long as
// 4 (Q_prev + Q) + 8 < 2^32; launches are limited to Q < 2^28 steps, which guarantees it.
constexpr long long kMaxStepsPerLaunch = 1ll << 28;
GSI_HD unsigned step_tag(unsigned long long epoch, long long q, int kind) {
  return (unsigned)(epoch + 4ull * (unsigned long long)q + (unsigned long long)kind);
}
GSI_HD unsigned long long next_epoch(unsigned long long epoch, long long Q) {
  return epoch + 4ull * (unsigned long long)Q + 4ull;
}

}  // namespace gsi
