// Host-side check of the batch-1 decode kernel's work split and mailbox tags, built from the same
// header the kernels include (gated_rank_linear_amd/csrc/gsi_plan.h). Built and run on the CPU by
// tests/test_plan.py; prints one line per failure and exits non-zero if there is any.
//
// For every site shape of the synthetic workloads (and edge shapes) at every rank k, element size,
// site mode and grid size it checks, block by block:
//   * every g column and every output row is owned by exactly one block;
//   * the LDS region fits, its parts are 64-chunk aligned and disjoint;
//   * simulating the copy instructions, every region chunk that phase A (V^T rows), the gate piece
//     ((V^T V - I) rows) and phase B (M rows) read holds exactly the global chunk it stands for,
//     and the addresses used for the parts read from global memory are the right ones.
// Then it checks the mailbox tag arithmetic against an explicit model of the mailbox words.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <vector>

#include "gsi_plan.h"

using namespace gsi;
typedef unsigned long long u64;

static int failures = 0;
#define CHECK(cond, ...)                                            \
  do {                                                              \
    if (!(cond)) {                                                  \
      if (failures < 50) {                                          \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__);            \
        std::printf(__VA_ARGS__);                                   \
        std::printf("\n");                                          \
      }                                                             \
      ++failures;                                                   \
    }                                                               \
  } while (0)

static const u64 kVT = 1ull << 40, kDL = 2ull << 40, kM = 3ull << 40, kW = 4ull << 40;

static void check_site(int d, int d_out, int k, int es, int mode, int P) {
  LayerDesc L;
  L.Vt = (const void*)kVT;
  L.M = (const void*)kM;
  L.Dl = (const float*)kDL;
  L.W = (const void*)kW;
  L.d = d;
  L.d_out = d_out;
  L.k = k;
  L.mode = mode;
  L.x_off = 12345;
  L.y_off = 678;
  const int VW = 16 / es;
  const int cprd = d / VW, cprk = k / VW, cpk4 = k / 4;
  std::vector<int> col_owner(k, -1), row_owner(d_out, -1);
  for (int b = 0; b < P; ++b) {
    const PlanRow p = make_plan_row(L, b, P, es);
    const char* tag = "";
    (void)tag;
#define WHERE "d=%d d_out=%d k=%d es=%d mode=%d P=%d b=%d"
#define ARGS d, d_out, k, es, mode, P, b
    CHECK(p.cprd == cprd && p.cprk == cprk && p.cpk4 == cpk4, WHERE " chunk counts", ARGS);
    CHECK(p.x_off == L.x_off && p.y_off == L.y_off + p.r0, WHERE " offsets", ARGS);
    // ownership
    if (mode != kSiteDense) {
      for (int jl = 0; jl < p.nJ; ++jl) {
        const int j = b + jl * P;
        CHECK(j < k, WHERE " column %d past k", ARGS, j);
        if (j < k) {
          CHECK(col_owner[j] == -1, WHERE " column %d owned twice", ARGS, j);
          col_owner[j] = b;
        }
      }
      CHECK(p.nJ <= kMaxJ, WHERE " nJ %d > kMaxJ", ARGS, p.nJ);
    } else {
      CHECK(p.nJ == 0 && p.n_inst == 0, WHERE " dense site holds region parts", ARGS);
    }
    CHECK(p.r0 >= 0 && p.nrows >= 0 && p.r0 + p.nrows <= d_out, WHERE " rows out of range", ARGS);
    for (int r = 0; r < p.nrows; ++r) {
      CHECK(row_owner[p.r0 + r] == -1, WHERE " row %d owned twice", ARGS, p.r0 + r);
      row_owner[p.r0 + r] = b;
    }
    // region layout
    CHECK(p.n_inst * 64 <= kRegionChunks, WHERE " region overflow %d instructions", ARGS, p.n_inst);
    CHECK(p.d_off % 64 == 0 && p.m_off % 64 == 0, WHERE " parts not 64-chunk aligned", ARGS);
    CHECK(p.v_n == p.vj * cprd && p.vj <= p.nJ, WHERE " V^T part", ARGS);
    CHECK(p.v_n <= p.d_off && p.d_off + p.d_n <= p.m_off && p.m_off + p.m_n <= p.n_inst * 64 + 0 * 1,
          WHERE " parts overlap", ARGS);
    CHECK(p.d_n == 0 || p.d_n == p.nJ * cpk4, WHERE " (V^T V - I) part neither all nor none", ARGS);
    if (mode != kSiteGated) CHECK(p.d_n == 0, WHERE " (V^T V - I) held outside the gated mode", ARGS);
    CHECK(p.m_rows * cprk == p.m_n && p.m_rows <= p.nrows, WHERE " M part", ARGS);
    if (p.m_rows < p.nrows) CHECK(p.m_n % kDataThreads == 0, WHERE " partial M part not a multiple of 256", ARGS);
    // simulate the fill
    std::vector<u64> region((size_t)p.n_inst * 64, ~0ull);
    for (int i = 0; i < p.n_inst; ++i)
      for (int lane = 0; lane < 64; ++lane) region[(size_t)i * 64 + lane] = fill_source(p, P, i, lane);
    std::set<u64> seen;
    for (u64 a : region)
      if (a) {
        CHECK(seen.insert(a).second, WHERE " global chunk %llx copied twice", ARGS, a);
      }
    // phase A: V^T rows
    for (int jl = 0; jl < p.vj; ++jl)
      for (int cc = 0; cc < cprd; ++cc) {
        const u64 want = kVT + ((u64)(b + jl * P) * cprd + cc) * 16;
        const int c = lds_vt(p, jl, cc);
        CHECK(c >= 0 && c < (int)region.size() && region[c] == want, WHERE " V^T row %d chunk %d", ARGS, jl, cc);
      }
    for (int jl = p.vj; jl < p.nJ; ++jl)
      for (int cc = 0; cc < cprd; cc += 97) {
        const u64 got = p.vt + ((u64)jl * P * cprd + cc) * 16;
        CHECK(got == kVT + ((u64)(b + jl * P) * cprd + cc) * 16, WHERE " global V^T row %d", ARGS, jl);
      }
    // gate piece: rows of V^T V - I
    if (mode == kSiteGated) {
      for (int e = 0; e < p.nJ * cpk4; ++e) {
        const int jl = e / cpk4, cc = e % cpk4;
        const u64 want = kDL + ((u64)(b + jl * P) * cpk4 + cc) * 16;
        if (p.d_n > 0) {
          const int c = lds_dl(p, e);
          CHECK(c < (int)region.size() && region[c] == want, WHERE " (V^T V - I) chunk %d", ARGS, e);
        } else {
          CHECK(p.dl + ((u64)jl * P * cpk4 + cc) * 16 == want, WHERE " global (V^T V - I) chunk %d", ARGS, e);
        }
      }
    }
    // phase B: rows of M, then W rows of the slow path / a dense site
    for (int r = 0; r < p.m_rows; ++r)
      for (int ch = 0; ch < cprk; ++ch) {
        const int c = lds_m(p, r, ch);
        const u64 want = kM + ((u64)(p.r0 + r) * cprk + ch) * 16;
        CHECK(c < (int)region.size() && region[c] == want, WHERE " M row %d chunk %d", ARGS, r, ch);
      }
    for (int r = p.m_rows; r < p.nrows && mode != kSiteDense; r += 7)
      CHECK(p.m + ((u64)r * cprk + cprk - 1) * 16 == kM + ((u64)(p.r0 + r) * cprk + cprk - 1) * 16,
            WHERE " global M row %d", ARGS, r);
    for (int r = 0; r < p.nrows; r += 5)
      CHECK(p.w + ((u64)r * cprd + cprd - 1) * 16 == kW + ((u64)(p.r0 + r) * cprd + cprd - 1) * 16,
            WHERE " W row %d", ARGS, r);
    // every chunk copied is one some phase reads (no stray copies beyond padding)
    size_t used = (size_t)p.v_n + (size_t)p.d_n + (size_t)p.m_n;
    CHECK(seen.size() == used, WHERE " %zu chunks copied, %zu read", ARGS, seen.size(), used);
    // the M rows of phase B: lanes per row a power of two that divides a wave
    if (mode != kSiteDense) {
      const int CPL = cprk < 4 ? cprk : 4;
      const int Lr = cprk / CPL;
      CHECK(Lr >= 1 && Lr <= 64 && (64 % Lr) == 0, WHERE " lanes per row %d", ARGS, Lr);
    }
#undef WHERE
#undef ARGS
  }
  if (mode != kSiteDense)
    for (int j = 0; j < k; ++j) CHECK(col_owner[j] >= 0, "d=%d k=%d P=%d: column %d unowned", d, k, P, j);
  for (int r = 0; r < d_out; ++r) CHECK(row_owner[r] >= 0, "d_out=%d P=%d: row %d unowned", d_out, P, r);
}

// Mailbox model: every word remembers the tag of its last write. Launch after launch on one
// workspace, each block rewrites its owned words with the launch's base tag, then step q writes
// the words of its kind with step_tag(E, q, kind). A poll at step q must match a word only when
// that word was written at step q (with the same kind). Both orders of "rewrite lands before /
// after the poll" are modelled: a poll sees either the value before this launch's rewrite (the
// last value of the previous launch) or any value written in this launch up to step q.
static void check_tags() {
  const u64 starts[] = {0ull, 1ull, 0xfffffff0ull, 0xffffffffull, 0x1fffffff8ull, 0x7ffffffffffff000ull};
  const long long launches[][3] = {{1, 3, 2}, {5, 1, 7}, {64, 64, 64}, {1, 1, 1}, {1000, 3, 40}};
  for (u64 e0 : starts)
    for (const auto& ql : launches) {
      u64 E = e0;
      // one word per kind; value of a word = (tag, launch index, step, kind) of its last write
      struct W { unsigned tag; int launch; long long step; int kind; };
      std::map<int, W> last_prev;  // last value of each kind at the end of the previous launch
      for (int kind = 1; kind <= 3; ++kind) last_prev[kind] = W{(unsigned)E, -1, -1, kind};
      for (int li = 0; li < 3; ++li) {
        const long long Q = ql[li];
        std::map<int, std::vector<W>> writes;  // writes of this launch per kind, in order
        for (int kind = 1; kind <= 3; ++kind) writes[kind].push_back(W{(unsigned)E, li, -1, kind});
        for (long long q = 0; q < Q; ++q) {
          for (int kind = 1; kind <= 3; ++kind) {
            // the live write of this step (kind 3 only on some steps, as on slow sites)
            const bool writes_now = kind != 3 || (q % 3 == 1);
            if (writes_now) writes[kind].push_back(W{step_tag(E, q, kind), li, q, kind});
            if (!writes_now) continue;
            const unsigned want = step_tag(E, q, kind);
            // every value the poll might see: the previous launch's last value or any write so far
            std::vector<W> seen = writes[kind];
            seen.push_back(last_prev[kind]);
            for (const W& w : seen) {
              const bool match = w.tag == want;
              const bool live = w.launch == li && w.step == q;
              CHECK(match == live, "epoch %llx launch %d step %lld kind %d: stale tag %x (launch %d step %lld) "
                                   "matches=%d", (unsigned long long)E, li, q, kind, w.tag, w.launch, w.step,
                    (int)match);
            }
            // a word of another kind never carries this kind's tag either
            for (int other = 1; other <= 3; ++other)
              if (other != kind) CHECK(step_tag(E, q, other) != want, "kinds collide");
          }
        }
        for (int kind = 1; kind <= 3; ++kind) last_prev[kind] = writes[kind].back();
        const u64 En = next_epoch(E, Q);
        CHECK(En > E && En - E == 4ull * Q + 4, "epoch advance");
        E = En;
      }
    }
  // The bound the library enforces: with both launches below kMaxStepsPerLaunch steps the span of
  // tags a poll can see is below 2^32, so no stale tag can wrap onto a live one.
  const u64 span = 4ull * (u64)(kMaxStepsPerLaunch - 1) + 4ull + 4ull * (u64)(kMaxStepsPerLaunch - 1) + 3ull;
  CHECK(span < (1ull << 32), "launch bound does not keep tags apart");
  // the largest launch: its own first and last step tags of one kind stay apart
  CHECK(step_tag(0xfffffffcull, 0, 1) != step_tag(0xfffffffcull, kMaxStepsPerLaunch - 1, 1), "wrap inside a launch");
}

int main() {
  const int sites[][2] = {
      {768, 768},   {768, 2304},   {768, 3072},   {3072, 768},  {4096, 12288}, {4096, 4096}, {4096, 16384},
      {16384, 4096}, {4096, 28672}, {40, 100},    {64, 257},    {520, 1000},   {24, 3},      {1032, 700},
      {1024, 12300}, {65536, 64},  {64, 262144}, {2048, 1000}, {4096, 300},   {8, 1},       {16, 24}};
  for (const auto& s : sites) {
    const int d = s[0], d_out = s[1];
    for (int es : {2, 4})
      for (int k = 8; k <= 512 && k <= d; k *= 2)
        for (int mode : {kSiteGated, kSiteStatic})
          for (int P : {128, 256}) {
            if ((d_out + P - 1) / P > 2048) continue;  // the library rejects this shape
            check_site(d, d_out, k, es, mode, P);
          }
    for (int es : {2, 4})
      for (int P : {128, 256})
        if ((d_out + P - 1) / P <= 2048) check_site(d, d_out, 0, es, kSiteDense, P);
  }
  check_tags();
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("plan and tag checks passed\n");
  return 0;
}
