// Dense kernels of libgsi: the create-time precomputation (V^T, M = W V, V^T V - I) and the
// batched (T >= 16) path: projection, device-side gate with fast/slow token compaction, and the
// fast (M g) and slow (W x) products. Method: "Gated Subspace Inference for transformer
// acceleration" technical summary (gist.science, arXiv 2605.03109), §2.1-§2.2.
#include "gsi_internal.h"

#include <algorithm>
#include <type_traits>

namespace gsi {

template <typename T> __device__ __forceinline__ float ld_f32(const void* p, long long i) {
  return to_f32(reinterpret_cast<const T*>(p)[i]);
}
template <typename T> __device__ __forceinline__ void st_from_f32(void* p, long long i, float v) {
  reinterpret_cast<T*>(p)[i] = from_f32<T>(v);
}

// ---------------------------------------------------------------------------------------------
// NT GEMM on the vector ALU, float32 accumulation: C[m, n] = sum_i A[ra(m), i] * B[n, i].
// 64x64 output tile per 256-thread block, K staged through LDS in chunks of 32 (converted to
// float32 once), 4x4 outputs per thread. Each output is one thread's fixed-order sum, so results
// are reproducible run to run.
// ---------------------------------------------------------------------------------------------
constexpr int GBM = 64, GBN = 64, GBK = 32;

template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const void* __restrict__ A, long long lda,
                                                      const int* __restrict__ a_idx, const void* __restrict__ B,
                                                      long long ldb, void* __restrict__ C, long long ldc,
                                                      const int* __restrict__ c_idx, int m, int n, int kdim,
                                                      const int* __restrict__ m_count, int sub_identity) {
  __shared__ float As[GBK][GBM + 4];
  __shared__ float Bs[GBK][GBN + 4];
  const int mv = m_count ? min(m, *m_count) : m;
  const int m0 = blockIdx.y * GBM, n0 = blockIdx.x * GBN;
  if (m0 >= mv) return;
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  // loader mapping: 64 rows x 32 k per tile = 2048 elements, 8 per thread (one row, 8 consecutive k)
  const int lr = tid / 4, lk = (tid % 4) * 8;
  const int am = m0 + lr;
  const bool a_ok = am < mv;
  const long long a_row = a_ok ? (long long)(a_idx ? a_idx[am] : am) : 0;
  const int bn = n0 + lr;
  const bool b_ok = bn < n;

  for (int k0 = 0; k0 < kdim; k0 += GBK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = k0 + lk + e;
      As[lk + e][lr] = (a_ok && kk < kdim) ? ld_f32<TA>(A, a_row * lda + kk) : 0.f;
      Bs[lk + e][lr] = (b_ok && kk < kdim) ? ld_f32<TB>(B, (long long)bn * ldb + kk) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < GBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mm = m0 + ty * 4 + i;
    if (mm >= mv) continue;
    const long long crow = c_idx ? c_idx[mm] : mm;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nn = n0 + tx * 4 + j;
      if (nn >= n) continue;
      float v = acc[i][j];
      if (sub_identity && mm == nn) v -= 1.0f;
      st_from_f32<TC>(C, crow * ldc + nn, v);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// NT GEMM on the matrix cores (v_mfma_f32_16x16x32_{bf16,f16}), float32 accumulation:
// C[m, n] = sum_i A[ra(m), i] * B[n, i], both operands K-contiguous. 64x64 output tile per block
// of 4 waves (2 x 2, 32x32 each: 2 x 2 tiles of 16x16). Per 32-column step, lane l of a wave
// holds, for each of its 16-row tiles, 8 consecutive K elements of row l mod 16 starting at
// 8 (l / 16) (the A operand layout), and the same for its B tiles; fragments are loaded straight
// from global memory one step ahead of their use. Rows past m (or the device count) and K past
// kdim read a valid location and are zeroed. A float32 A (with bf16 B) is split into bf16 high
// and low parts, each multiplied exactly: |a - hi - lo| <= 2^-18 |a|.
// ---------------------------------------------------------------------------------------------
typedef __bf16 mbf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 mf16x8 __attribute__((ext_vector_type(8)));
typedef float mf32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int mu32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct mfma_op;
template <> struct mfma_op<bf16_t> {
  static __device__ __forceinline__ mf32x4 run(mu32x4 a, mu32x4 b, mf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mbf16x8, a), __builtin_bit_cast(mbf16x8, b), c, 0,
                                                  0, 0);
  }
};
template <> struct mfma_op<f16_t> {
  static __device__ __forceinline__ mf32x4 run(mu32x4 a, mu32x4 b, mf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mf16x8, a), __builtin_bit_cast(mf16x8, b), c, 0,
                                                 0, 0);
  }
};

template <typename TA, typename TB, typename TC>
__global__ __launch_bounds__(256) void gemm_nt_mfma_kernel(const void* __restrict__ A, long long lda,
                                                           const int* __restrict__ a_idx, const void* __restrict__ B,
                                                           long long ldb, void* __restrict__ C, long long ldc,
                                                           const int* __restrict__ c_idx, int m, int n, int kdim,
                                                           const int* __restrict__ m_count, int sub_identity,
                                                           int k_chunk, float* __restrict__ part) {
  constexpr bool kSplit = sizeof(TA) == 4;  // float32 A against bf16 B
  constexpr int kGroup = 4;                 // K steps of 32 whose loads are issued together
  const int mv = m_count ? min(m, *m_count) : m;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  if (m0 >= mv) return;
  // split K: block z takes columns [kb, ke) and, when part is given, writes its raw sums there
  const int kb = blockIdx.z * k_chunk, ke = min(kdim, kb + k_chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, kq = lane >> 4;
  // rows of A (through the gather list) and of B used by this lane; invalid ones read row 0
  long long arow[2], brow[2];
  bool aok[2], bok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int mm = m0 + wm * 32 + i * 16 + r16;
    aok[i] = mm < mv;
    arow[i] = aok[i] ? (long long)(a_idx ? a_idx[mm] : mm) * lda : 0;
    const int nn = n0 + wn * 32 + i * 16 + r16;
    bok[i] = nn < n;
    brow[i] = bok[i] ? (long long)nn * ldb : 0;
  }
  mf32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = mf32x4{0.f, 0.f, 0.f, 0.f};

  // raw 16-byte chunks of one K step (A as loaded; the bf16 split of a float32 A happens at use)
  struct Frag {
    mu32x4 a[2][kSplit ? 2 : 1];
    mu32x4 b[2];
  };
  auto load_step = [&](int k0, Frag& f) {
    const int kk = k0 + kq * 8;
    const bool kin = kk < ke;  // kdim and the chunk bounds are multiples of 8: a chunk is all in or out
    const int kc = kin ? kk : kb;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool ok = aok[i] && kin;
      if constexpr (kSplit) {
        const mu32x4* pa = reinterpret_cast<const mu32x4*>(reinterpret_cast<const float*>(A) + arow[i] + kc);
        f.a[i][0] = ok ? pa[0] : mu32x4{0u, 0u, 0u, 0u};
        f.a[i][1] = ok ? pa[1] : mu32x4{0u, 0u, 0u, 0u};
      } else {
        const mu32x4 v = reinterpret_cast<const mu32x4*>(reinterpret_cast<const TA*>(A) + arow[i] + kc)[0];
        f.a[i][0] = ok ? v : mu32x4{0u, 0u, 0u, 0u};
      }
      const mu32x4 w = reinterpret_cast<const mu32x4*>(reinterpret_cast<const TB*>(B) + brow[i] + kc)[0];
      f.b[i] = (bok[i] && kin) ? w : mu32x4{0u, 0u, 0u, 0u};
    }
  };
  auto compute_step = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      mu32x4 ah, al = mu32x4{0u, 0u, 0u, 0u};
      if constexpr (kSplit) {
        const mu32x4 r0 = f.a[i][0], r1 = f.a[i][1];
        const unsigned raw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        unsigned short h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = __uint_as_float(raw[e]);
          const bf16_t hb = from_f32<bf16_t>(v);
          const bf16_t lb = from_f32<bf16_t>(v - to_f32(hb));
          h[e] = hb.b;
          l[e] = lb.b;
        }
        ah = mu32x4{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16), h[4] | ((unsigned)h[5] << 16),
                    h[6] | ((unsigned)h[7] << 16)};
        al = mu32x4{l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16), l[4] | ((unsigned)l[5] << 16),
                    l[6] | ((unsigned)l[7] << 16)};
      } else {
        ah = f.a[i][0];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = mfma_op<TB>::run(ah, f.b[j], acc[i][j]);
        if constexpr (kSplit) acc[i][j] = mfma_op<TB>::run(al, f.b[j], acc[i][j]);
      }
    }
  };

  // groups of kGroup steps, double-buffered: the next group's loads are all issued before this
  // group's products, so up to 2 kGroup steps of loads are in flight (steps past the chunk load
  // zeros)
  Frag cur[kGroup], nxt[kGroup];
#pragma unroll
  for (int u = 0; u < kGroup; ++u) load_step(kb + 32 * u, cur[u]);
  for (int k0 = kb; k0 < ke; k0 += 32 * kGroup) {
#pragma unroll
    for (int u = 0; u < kGroup; ++u) load_step(k0 + 32 * (kGroup + u), nxt[u]);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) compute_step(cur[u]);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) cur[u] = nxt[u];
  }
  if (part) {  // raw partial sums of this K chunk: part[z][mm][nn]
    float* pz = part + (long long)blockIdx.z * m * n;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = m0 + wm * 32 + i * 16 + 4 * kq + r;
        if (mm >= mv) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int nn = n0 + wn * 32 + j * 16 + r16;
          if (nn < n) pz[(long long)mm * n + nn] = acc[i][j][r];
        }
      }
    return;
  }
  // D of a 16x16 tile: lane l holds column l mod 16, rows 4 (l / 16) .. + 3
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = m0 + wm * 32 + i * 16 + 4 * kq + r;
      if (mm >= mv) continue;
      const long long crow = c_idx ? c_idx[mm] : mm;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nn = n0 + wn * 32 + j * 16 + r16;
        if (nn >= n) continue;
        float v = acc[i][j][r];
        if (sub_identity && mm == nn) v -= 1.0f;
        st_from_f32<TC>(C, crow * ldc + nn, v);
      }
    }
}

// Skinny NT GEMM on the matrix cores for products with at most 64 rows of A whose count is a
// device-side token count (the batched fast product, float32 g rows against bf16 M, and slow
// product, 16-bit x rows against W): a block covers 64 columns of C and wave w the 16-column tile
// n0 + 16 w, so every element of B is loaded once per block; each wave runs only the
// NRT = ceil(mv / 16) row tiles that hold valid rows (mv is uniform, read once). The rows of A
// are staged once per block through LDS. K is split over blockIdx.z; the raw float32 sums of a
// chunk go to part[z][mm][nn] (rows mm < mv; row o_idx[mm] when an output list is given), added
// later in chunk order (with `coherent`, by device-scope stores another block can read without a
// cache flush). Per sub-chunk of 256 K columns the block copies its A rows (mv valid, the
// rest zero) into LDS, a float32 A split into high and low parts in B's 16-bit type (bf16:
// |a - hi - lo| <= 2^-18 |a|; f16: 2^-22 |a| within its normal range), stored in the A-operand order of
// v_mfma_f32_16x16x32_{bf16,f16} (row tile t, step s, lane l at ((t * 8 + s) * 64 + l)), so every
// element is read from global memory (and split) once per block instead of once per wave and
// every LDS read is one conflict-free 16-byte load; the eight steps of B of a sub-chunk are
// loaded before its products, and the next sub-chunk's A fragments (into registers) and B steps
// before this one's products.
// B steps of one 256-column sub-chunk for this lane (row nn of B, the lane's 8-element K groups);
// steps outside [kb, ke) read column kb and are zeroed
// bx: the block's column tile (columns 64 bx .. 64 bx + 63 of C). With B2, column tile bx takes
// its first 32 columns from rows 32 bx .. of B and the next 32 from the same rows of B2 (waves 0-1
// and 2-3).
template <typename TB>
__device__ __forceinline__ void skinny_load_b(const TB* __restrict__ B, long long ldb, int n, int kb, int ke, int k0,
                                              mu32x4 (&bv)[8], int bx, const TB* __restrict__ B2 = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nn = bx * 64 + wave * 16 + (lane & 15);
  const bool bok = nn < n;
  const int brow_i = B2 ? bx * 32 + (wave & 1) * 16 + (lane & 15) : nn;
  if (B2 && wave >= 2) B = B2;
  const long long brow = bok ? (long long)brow_i * ldb : 0;
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const int kk = k0 + 32 * st + 8 * (lane >> 4);
    const bool kin = kk < ke;  // K bounds are multiples of 8: a chunk is all in or all out
    const mu32x4 w = reinterpret_cast<const mu32x4*>(B + brow + (kin ? kk : kb))[0];
    bv[st] = (bok && kin) ? w : mu32x4{0u, 0u, 0u, 0u};
  }
}

template <typename TA, typename TB, int NRT, bool kPre = false, int kPreB = 0>
__device__ __forceinline__ void skinny_staged_tiles(const TA* __restrict__ A, long long lda,
                                                    const int* __restrict__ a_idx, const TB* __restrict__ B,
                                                    long long ldb, int mv, int n, int kb, int ke,
                                                    float* __restrict__ part, mu32x4* __restrict__ lds_hi,
                                                    mu32x4* __restrict__ lds_lo, const int* __restrict__ o_idx,
                                                    bool coherent, const TA* __restrict__ A_lo, mu32x4 (&pb0)[8],
                                                    mu32x4 (&pb1)[8], int bx, const TB* __restrict__ B2 = nullptr,
                                                    float* __restrict__ x2out = nullptr, TB* __restrict__ yout = nullptr,
                                                    long long y_ld = 0) {
  // bx: the block's column tile; yout: the sums are complete (one K chunk) and go straight to
  // yout[row][nn] rounded to TB instead of to part
  // B2: second row source (skinny_load_b); x2out (16-bit A): each A row's sum of squares over
  // [kb, ke) to x2out[row * kMaxProjChunks]
  // kPreB (16-bit A only): the caller has already loaded the first kPreB sub-chunks' B steps into
  // pb0 (and pb1) with skinny_load_b
  // kF32: A is float32 and is split here; kPre: A arrives split, high parts at A and low parts at
  // A_lo (16-bit, B's type); either way each step takes two products
  constexpr bool kF32 = sizeof(TA) == 4;
  constexpr bool kSplit = kF32 || kPre;
  constexpr int kSteps = 8;  // 32-column steps per sub-chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int nn = bx * 64 + wave * 16 + r16;
  const bool bok = nn < n;
  mf32x4 acc[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) acc[t] = mf32x4{0.f, 0.f, 0.f, 0.f};
  static_assert(kSteps == 8, "skinny_load_b loads eight steps");
  auto load_b = [&](int k0, mu32x4 (&bv)[kSteps]) { skinny_load_b(B, ldb, n, kb, ke, k0, bv, bx, B2); };
  // A fragments of a sub-chunk: thread tid takes fragments f = tid + 256 i (i < 2 NRT); they are
  // loaded into registers one sub-chunk ahead and written to LDS (split, for a float32 A) at the
  // start of the sub-chunk that uses them
  constexpr int NF = NRT * kSteps * 64 / 256;
  constexpr int AW = kSplit ? 2 : 1;  // 16-byte loads per fragment
  mu32x4 areg[NF][AW];
  // each fragment's A row is the same in every sub-chunk: its offset is looked up once (the list
  // may sit in LDS, and a load through a generic pointer would make every later wait drain all
  // memory loads in flight)
  // 16-bit A is read coalesced: element e = tid + 256 i of a sub-chunk is row e / 32, 16-byte
  // chunk e mod 32 (32 consecutive threads read one row's 512 bytes) and is written to its place
  // in the A-operand order; a float32 A is read per fragment
  auto a_row_of = [&](int e) { return kF32 ? 16 * (e >> 9) + (e & 15) : e >> 5; };
  auto a_lds_of = [&](int e) {
    return kF32 ? e : (((e >> 9) * kSteps + ((e & 31) >> 2)) * 64 + ((e >> 5) & 15) + 16 * (e & 3));
  };
  long long arow[NF];
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int mm = a_row_of(tid + 256 * i);
    arow[i] = mm < mv ? (long long)(a_idx ? a_idx[mm] : mm) * lda : -1;
  }
  // output rows of this lane's results, looked up before any store is issued (a lookup after a
  // store would wait for that store to complete)
  int orow[NRT][4];
#pragma unroll
  for (int t = 0; t < NRT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = 16 * t + 4 * kq + r;
      orow[t][r] = mm < mv ? (o_idx ? o_idx[mm] : mm) : -1;
    }
  auto load_a_into = [&](int k0, mu32x4(&areg)[NF][AW]) {
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int f = tid + 256 * i;
      const int l = f & 63, st = (f >> 6) & (kSteps - 1);
      const int kk = kF32 ? k0 + 32 * st + 8 * (l >> 4) : k0 + 8 * (f & 31);
      const bool in = arow[i] >= 0 && kk < ke;
      const long long row = in ? arow[i] + kk : 0;
      const mu32x4* pa = reinterpret_cast<const mu32x4*>(A + row);
      if constexpr (kPre) {
        const mu32x4 vh = pa[0];
        const mu32x4 vl = reinterpret_cast<const mu32x4*>(A_lo + row)[0];
        areg[i][0] = in ? vh : mu32x4{0u, 0u, 0u, 0u};
        areg[i][1] = in ? vl : mu32x4{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int h = 0; h < AW; ++h) {
          const mu32x4 v = pa[h];
          areg[i][h] = in ? v : mu32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto load_a = [&](int k0) { load_a_into(k0, areg); };
  // rows (tid / 32) + 8 i: their sums of squares, complete in lane tid mod 32 == 0
  float xs[NF];
#pragma unroll
  for (int i = 0; i < NF; ++i) xs[i] = 0.f;
  auto store_a_from = [&](const mu32x4(&areg)[NF][AW]) {
    if constexpr (!kSplit) {
      if (x2out) {  // uniform
#pragma unroll
        for (int i = 0; i < NF; ++i) {
          float v = 0.f;
          const TA* e = reinterpret_cast<const TA*>(&areg[i][0]);
#pragma unroll
          for (int j = 0; j < 8; ++j) v = __builtin_fmaf(to_f32(e[j]), to_f32(e[j]), v);
#pragma unroll
          for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
          xs[i] += v;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int f = a_lds_of(tid + 256 * i);
      if constexpr (kPre) {
        lds_hi[f] = areg[i][0];
        lds_lo[f] = areg[i][1];
      } else if constexpr (kF32) {
        const unsigned raw[8] = {areg[i][0].x, areg[i][0].y, areg[i][0].z, areg[i][0].w,
                                 areg[i][AW - 1].x, areg[i][AW - 1].y, areg[i][AW - 1].z, areg[i][AW - 1].w};
        unsigned short h[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // split in B's own 16-bit type, the type the matrix-core product reads both operands in
          const float v = __uint_as_float(raw[e]);
          const TB hb = from_f32<TB>(v);
          const TB lb = from_f32<TB>(v - to_f32(hb));
          h[e] = hb.b;
          lo[e] = lb.b;
        }
        lds_hi[f] = mu32x4{h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16),
                           h[4] | ((unsigned)h[5] << 16), h[6] | ((unsigned)h[7] << 16)};
        lds_lo[f] = mu32x4{lo[0] | ((unsigned)lo[1] << 16), lo[2] | ((unsigned)lo[3] << 16),
                           lo[4] | ((unsigned)lo[5] << 16), lo[6] | ((unsigned)lo[7] << 16)};
      } else {
        lds_hi[f] = areg[i][0];
      }
    }
  };
  auto store_a = [&]() { store_a_from(areg); };
  // per step the high parts of every tile, then the low parts: consecutive products never use the
  // same accumulator
  auto products = [&](const mu32x4(&bv)[kSteps]) {
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
#pragma unroll
      for (int t = 0; t < NRT; ++t) acc[t] = mfma_op<TB>::run(lds_hi[(t * kSteps + st) * 64 + lane], bv[st], acc[t]);
      if constexpr (kSplit) {
#pragma unroll
        for (int t = 0; t < NRT; ++t) acc[t] = mfma_op<TB>::run(lds_lo[(t * kSteps + st) * 64 + lane], bv[st], acc[t]);
      }
    }
  };
  constexpr int S = 32 * kSteps;
  // two sub-chunks ahead only while the registers allow it (one or two row tiles of 16-bit A)
  constexpr bool kDeep = !kSplit && NRT <= 2;
  if constexpr (kDeep) {
    // 16-bit A: two sub-chunks of A and B in flight ahead of the products. Three register sets,
    // named in a loop unrolled by three; loads past the chunk read its first columns and are
    // zeroed, so every step issues the same loads.
    mu32x4 a0[NF][AW], a1[NF][AW], a2[NF][AW], b2[kSteps];
    mu32x4(&b0)[kSteps] = pb0;
    mu32x4(&b1)[kSteps] = pb1;
    if constexpr (kPreB < 1) load_b(kb, b0);
    load_a_into(kb, a0);
    if constexpr (kPreB < 2) load_b(kb + S, b1);
    load_a_into(kb + S, a1);
#define GSI_SKSTEP(KC, ACUR, BCUR, ANX, BNX)                                                              \
  do {                                                                                                   \
    __syncthreads();                                                                                     \
    store_a_from(ACUR);                                                                                  \
    __syncthreads();                                                                                     \
    load_a_into((KC) + 2 * S, ANX);                                                                      \
    load_b((KC) + 2 * S, BNX);                                                                           \
    products(BCUR);                                                                                      \
  } while (0)
    for (int k0 = kb;; k0 += 3 * S) {
      GSI_SKSTEP(k0, a0, b0, a2, b2);
      if (k0 + S >= ke) break;
      GSI_SKSTEP(k0 + S, a1, b1, a0, b0);
      if (k0 + 2 * S >= ke) break;
      GSI_SKSTEP(k0 + 2 * S, a2, b2, a1, b1);
      if (k0 + 3 * S >= ke) break;
    }
#undef GSI_SKSTEP
  }
  mu32x4 bcur[kSteps], bnxt[kSteps];
  if constexpr (kPre) {
    // A arrives split (the batched fast product, K of one or two sub-chunks): each sub-chunk's
    // loads issued together, no registers held for the next one
    for (int k0 = kb; k0 < ke; k0 += 32 * kSteps) {
      load_a(k0);
      load_b(k0, bcur);
      __syncthreads();  // the previous sub-chunk's A fragments are no longer read
      store_a();
      __syncthreads();
      products(bcur);
    }
  }
  constexpr bool kNext = kF32 || (!kSplit && !kDeep);  // one sub-chunk ahead
  if constexpr (kNext) {
    if constexpr (kPreB >= 1) {
#pragma unroll
      for (int st = 0; st < kSteps; ++st) bcur[st] = pb0[st];
    } else {
      load_b(kb, bcur);
    }
    load_a(kb);
  }
  for (int k0 = kb; kNext && k0 < ke; k0 += 32 * kSteps) {
    __syncthreads();  // the previous sub-chunk's A fragments are no longer read
    store_a();
    __syncthreads();
    if (k0 + 32 * kSteps < ke) {  // uniform: the next sub-chunk's A and B in flight during the products
      load_a(k0 + 32 * kSteps);
      load_b(k0 + 32 * kSteps, bnxt);
    }
    products(bcur);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) bcur[st] = bnxt[st];
  }
#pragma unroll
  for (int t = 0; t < NRT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (orow[t][r] >= 0 && bok) {
        float* q = part + (long long)orow[t][r] * n + nn;
        if (yout)  // uniform
          yout[(long long)orow[t][r] * y_ld + nn] = from_f32<TB>(acc[t][r]);
        else if (coherent)  // read by another block of the same launch
          __hip_atomic_store(q, acc[t][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *q = acc[t][r];
      }
    }
  if constexpr (!kSplit) {
    if (x2out && (tid & 31) == 0) {
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int mm = (tid >> 5) + 8 * i;
        if (mm < mv) x2out[(long long)mm * kMaxProjChunks] = xs[i];
      }
    }
  }
}

template <typename TA, typename TB>
__global__ __launch_bounds__(256) void gemm_nt_skinny_staged_kernel(const void* __restrict__ A, long long lda,
                                                                    const int* __restrict__ a_idx,
                                                                    const void* __restrict__ B, long long ldb, int m,
                                                                    int n, int kdim, const int* __restrict__ m_count,
                                                                    int k_chunk, float* __restrict__ part) {
  constexpr bool kSplit = sizeof(TA) == 4;
  __shared__ mu32x4 lds_hi[4 * 8 * 64], lds_lo[kSplit ? 4 * 8 * 64 : 1];  // 64 KB (32 KB for 16-bit A)
  const int mv = m_count ? min(m, *m_count) : m;
  if (mv <= 0) return;
  const int kb = blockIdx.z * k_chunk, ke = min(kdim, kb + k_chunk);
  float* pz = part + (long long)blockIdx.z * m * n;
  const TA* a = reinterpret_cast<const TA*>(A);
  const TB* b = reinterpret_cast<const TB*>(B);
  mu32x4 b0[8], b1[8];  // loaded inside (no early B loads here)
  switch ((mv + 15) >> 4) {  // uniform
    case 1: skinny_staged_tiles<TA, TB, 1>(a, lda, a_idx, b, ldb, mv, n, kb, ke, pz, lds_hi, lds_lo, nullptr, false, nullptr, b0, b1, blockIdx.x); break;
    case 2: skinny_staged_tiles<TA, TB, 2>(a, lda, a_idx, b, ldb, mv, n, kb, ke, pz, lds_hi, lds_lo, nullptr, false, nullptr, b0, b1, blockIdx.x); break;
    case 3: skinny_staged_tiles<TA, TB, 3>(a, lda, a_idx, b, ldb, mv, n, kb, ke, pz, lds_hi, lds_lo, nullptr, false, nullptr, b0, b1, blockIdx.x); break;
    default: skinny_staged_tiles<TA, TB, 4>(a, lda, a_idx, b, ldb, mv, n, kb, ke, pz, lds_hi, lds_lo, nullptr, false, nullptr, b0, b1, blockIdx.x); break;
  }
}

// Sum of split-K partials in chunk order, C[c_row(mm)][nn] = sum_z part[z][mm][nn] for the
// mv = min(m, *m_count) valid rows.
template <typename TC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int m, int n,
                                                            const int* __restrict__ m_count, void* __restrict__ C,
                                                            long long ldc, const int* __restrict__ c_idx) {
  const int mm = blockIdx.y;
  const int mv = m_count ? min(m, *m_count) : m;
  if (mm >= mv) return;
  const long long crow = c_idx ? c_idx[mm] : mm;
  for (int nn = blockIdx.x * 256 + threadIdx.x; nn < n; nn += gridDim.x * 256) {
    float v = 0.f;
    for (int z = 0; z < splits; ++z) v += part[((long long)z * m + mm) * n + nn];
    st_from_f32<TC>(C, crow * ldc + nn, v);
  }
}

// Precompute reduction. Blocks [0, nb_img): rows of M, one thread per four columns, summing the
// sw chunks at pw (chunk stride cw floats) into running sum z mod 8 (eight loads in flight), the
// eight sums added in a fixed tree, rounded to TC. Blocks from nb_img on: rows of V^T V (n x n),
// eight threads per four columns, thread u summing chunks u, u + 8, ... of the sd chunks at pd
// (chunk stride cd), the eight threads' sums added in a fixed butterfly; stored to Dl as float32
// with I subtracted and, when DD is given, also split into two parts of TC, hi = round(v) and
// lo = round(v - hi), stored as row r of DD = [hi | lo] (n x 2n). Results do not depend on timing.
template <typename TC>
__global__ __launch_bounds__(256) void precompute_reduce_kernel(const float* __restrict__ pw, int sw, long long cw,
                                                                const float* __restrict__ pd, int sd, long long cd,
                                                                int m_img, int n, void* __restrict__ M,
                                                                float* __restrict__ Dl, TC* __restrict__ DD,
                                                                int nb_img) {
  if ((int)blockIdx.x < nb_img) {
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;  // group of 4 columns
    if (q >= (long long)m_img * (n / 4)) return;
    const int r = (int)(q / (n / 4)), n4 = (int)(q % (n / 4)) * 4;
    const float4* pp = reinterpret_cast<const float4*>(pw + (long long)r * n + n4);
    const long long stride = cw / 4;
    float a[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u][0] = a[u][1] = a[u][2] = a[u][3] = 0.f;
    int z = 0;
    for (; z + 8 <= sw; z += 8) {
      float4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = pp[(long long)(z + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a[u][0] += w[u].x;
        a[u][1] += w[u].y;
        a[u][2] += w[u].z;
        a[u][3] += w[u].w;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // the last sw mod 8 chunks (z is a multiple of 8 here)
      if (z + u < sw) {
        const float4 w = pp[(long long)(z + u) * stride];
        a[u][0] += w.x;
        a[u][1] += w.y;
        a[u][2] += w.z;
        a[u][3] += w.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      st_from_f32<TC>(M, (long long)r * n + n4 + e,
                      ((a[0][e] + a[1][e]) + (a[2][e] + a[3][e])) + ((a[4][e] + a[5][e]) + (a[6][e] + a[7][e])));
    return;
  }
  const long long q8 = (long long)(blockIdx.x - nb_img) * 256 + threadIdx.x;
  const long long q = q8 >> 3;  // group of 4 columns of V^T V
  const int u = (int)(q8 & 7);
  const bool valid = q < (long long)n * (n / 4);
  const int r = valid ? (int)(q / (n / 4)) : 0, n4 = valid ? (int)(q % (n / 4)) * 4 : 0;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const float4* pp = reinterpret_cast<const float4*>(pd + (long long)r * n + n4);
    const long long stride = cd / 4;
    for (int z = u; z < sd; z += 8) {
      const float4 w = pp[(long long)z * stride];
      acc[0] += w.x;
      acc[1] += w.y;
      acc[2] += w.z;
      acc[3] += w.w;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {  // the 8 lanes of a group are adjacent: butterfly over lane bits 0..2
    float v = acc[e];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    acc[e] = v;
  }
  if (valid && u == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = acc[e] - (r == n4 + e ? 1.0f : 0.0f);
      Dl[(long long)r * n + n4 + e] = v;
      if (DD) {
        const TC hi = from_f32<TC>(v);
        DD[(long long)r * 2 * n + n4 + e] = hi;
        DD[(long long)r * 2 * n + n + n4 + e] = from_f32<TC>(v - to_f32(hi));
      }
    }
  }
}

// The same sum for a dense m x n output read and written four columns at a time (n a multiple of
// 4), with I subtracted on request (V^T V - I).
template <typename TC>
__global__ __launch_bounds__(256) void splitk_reduce4_kernel(const float* __restrict__ part, int splits, int m, int n,
                                                             void* __restrict__ C, long long ldc, int sub_identity) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;  // group of 4 columns
  const long long total = (long long)m * (n / 4);
  if (q >= total) return;
  const int mm = (int)(q / (n / 4)), n4 = (int)(q % (n / 4)) * 4;
  const long long stride = (long long)m * n;
  const float4* p = reinterpret_cast<const float4*>(part + (long long)mm * n + n4);
  float4 v = p[0];
  for (int z = 1; z < splits; ++z) {
    const float4 w = p[z * (stride / 4)];
    v.x += w.x;
    v.y += w.y;
    v.z += w.z;
    v.w += w.w;
  }
  float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (sub_identity && mm == n4 + e) vv[e] -= 1.0f;
    st_from_f32<TC>(C, (long long)mm * ldc + n4 + e, vv[e]);
  }
}

// ---------------------------------------------------------------------------------------------
// Matrix-core NT GEMM for 16-bit A and B with K a multiple of 32, staged through LDS: 128x128
// output tile per block of 4 waves (2 x 2, 64x64 each = 4 x 4 tiles of 16x16). Each 32-column
// K step is 16 operand blocks of 1 KB (8 of A, 8 of B), copied from global memory straight into
// LDS (global_load_lds_dwordx4, 4 per wave) in the operand order of v_mfma_f32_16x16x32_*, so a
// fragment is one conflict-free 16-byte LDS read per lane. Three stages in flight; the stage
// buffers are separate LDS arrays and the K loop is unrolled by three, so reads of one stage
// never wait for copies into another. Rows past m (or the device count) and columns past n read
// row 0 and are not stored.
// ---------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void dlds_void;
typedef mu32x4 __attribute__((address_space(3))) dlu32x4;

template <int N>
__device__ __forceinline__ void dwait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void dlds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T, typename TC>
__global__ __launch_bounds__(256) void gemm_nt_mfma_lds_kernel(const void* __restrict__ A, long long lda,
                                                               const int* __restrict__ a_idx,
                                                               const void* __restrict__ B, long long ldb,
                                                               void* __restrict__ C, long long ldc,
                                                               const int* __restrict__ c_idx, int m, int n, int kdim,
                                                               const int* __restrict__ m_count, int sub_identity) {
  __shared__ mu32x4 st0[16 * 64], st1[16 * 64], st2[16 * 64];  // 3 stages x 16 operand blocks
  const int mv = m_count ? min(m, *m_count) : m;
  const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
  if (m0 >= mv) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // the 4 operand blocks this wave copies per step: blocks wave + 4 u; block q < 8 is A rows
  // m0 + 16 q .., block q >= 8 is B rows n0 + 16 (q - 8) ..; lane l reads row + (l mod 16),
  // elements 8 (l / 16) .. + 7 of the step
  const T* src[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = wave + 4 * u;
    if (q < 8) {
      const int mm = m0 + 16 * q + (lane & 15);
      const long long row = mm < mv ? (long long)(a_idx ? a_idx[mm] : mm) : 0;
      src[u] = reinterpret_cast<const T*>(A) + row * lda + 8 * (lane >> 4);
    } else {
      const int nn = n0 + 16 * (q - 8) + (lane & 15);
      const long long row = nn < n ? nn : 0;
      src[u] = reinterpret_cast<const T*>(B) + row * ldb + 8 * (lane >> 4);
    }
  }
  mf32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mf32x4{0.f, 0.f, 0.f, 0.f};
// the stage arrays are named directly in every copy and read, so the compiler can tell them apart
#define GSI_ISSUE(STAGE, K0)                                                                           \
  do {                                                                                                 \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) __builtin_amdgcn_global_load_lds(                    \
        (const void*)(src[u] + (K0)), (dlds_void*)((dlu32x4*)(STAGE) + (wave + 4 * u) * 64), 16, 0, 0);              \
  } while (0)
#define GSI_COMPUTE(STAGE)                                                                             \
  do {                                                                                                 \
    mu32x4 af[4], bf[4];                                                                               \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) af[i] = ((const dlu32x4*)(STAGE))[(wm * 4 + i) * 64 + lane]; \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) bf[j] = ((const dlu32x4*)(STAGE))[(8 + wn * 4 + j) * 64 + lane]; \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                      \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[i][j] = mfma_op<T>::run(af[i], bf[j], acc[i][j]); \
  } while (0)
// every step issues exactly 4 copies per wave (past the last stage they re-read the last K step
// into a stage nobody reads again), so at step s the copies still outstanding are stage s and
// stage s + 1, and waiting until at most 4 remain always completes stage s
#define GSI_STEP(CUR, FUT, ST)                                                                          \
  do {                                                                                                 \
    dwait_vmcnt<4>();                                                                                  \
    dlds_barrier();                                                                                    \
    GSI_ISSUE(FUT, min((ST) + 2, nk - 1) * 32);                                                        \
    GSI_COMPUTE(CUR);                                                                                  \
  } while (0)
  const int nk = kdim / 32;
  GSI_ISSUE(st0, 0);
  GSI_ISSUE(st1, min(1, nk - 1) * 32);
  int s0 = 0;
  for (; s0 + 3 <= nk; s0 += 3) {
    GSI_STEP(st0, st2, s0);
    GSI_STEP(st1, st0, s0 + 1);
    GSI_STEP(st2, st1, s0 + 2);
  }
  if (s0 < nk) GSI_STEP(st0, st2, s0);
  if (s0 + 1 < nk) GSI_STEP(st1, st0, s0 + 1);
  dwait_vmcnt<0>();  // no copy may land in LDS after the block ends
#undef GSI_STEP
#undef GSI_COMPUTE
#undef GSI_ISSUE
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
      if (mm >= mv) continue;
      const long long crow = c_idx ? c_idx[mm] : mm;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int nn = n0 + wn * 64 + j * 16 + (lane & 15);
        if (nn >= n) continue;
        float v = acc[i][j][r];
        if (sub_identity && mm == nn) v -= 1.0f;
        st_from_f32<TC>(C, crow * ldc + nn, v);
      }
    }
}

// ---------------------------------------------------------------------------------------------
// Matrix-core NT GEMM for a short, wide B (n a multiple of 256, the rank k of M = W V): MT x 256
// output tile per block of 4 waves (MT = 16, 32 or 64 rows), so A (the weight, d_out x d)
// streams from memory once per 256 columns. Wave w owns columns 64 w .. 64 w + 63. A 64-column
// K step is NB operand blocks of 1 KB, each holding 8 rows x 128 bytes (A: MT / 8 blocks; B: 32),
// copied straight into LDS, three stages in flight. Eight consecutive lanes of a copy read one
// row's whole 128-byte segment (one cache line), with the 16-byte chunks permuted within the
// row: row r of an operand sits at block r / 8, row slot (r mod 8) xor (block parity), chunk
// slot c xor (r mod 8). With that swizzle the MFMA operand reads (lane l: row l mod 16 of a tile,
// chunk 4 u + l / 16 of sub-step u) hit 16 distinct 16-byte bank groups in every 16 lanes.
// Every wave issues the same number of copies per step: when NB is not a multiple of 4 the spare
// copies repeat the first blocks (same data to the same place).
// Split K: block z covers K columns [z k_chunk, (z + 1) k_chunk) (k_chunk a multiple of 64) and,
// when `part` is given, stores its raw float32 sums to part[z][m][n] for a reduction in chunk
// order; otherwise (k_chunk >= kdim) it writes C.
// ---------------------------------------------------------------------------------------------
template <typename T, typename TC, int MT>
__global__ __launch_bounds__(256) void gemm_nt_wide_kernel(const void* __restrict__ A, long long lda,
                                                           const int* __restrict__ a_idx,
                                                           const void* __restrict__ B, long long ldb,
                                                           void* __restrict__ C, long long ldc,
                                                           const int* __restrict__ c_idx, int m, int n, int kdim,
                                                           const int* __restrict__ m_count, int sub_identity,
                                                           int k_chunk, float* __restrict__ part,
                                                           const void* __restrict__ A2, int m_split) {
  constexpr int RT = MT / 16, NA = 2 * RT, NB = NA + 32, CPW = (NB + 3) / 4;
  __shared__ mu32x4 st0[NB * 64], st1[NB * 64], st2[NB * 64];
  const int mv = m_count ? min(m, *m_count) : m;
  const int m0 = blockIdx.x * MT, n0 = blockIdx.y * 256;
  if (m0 >= mv) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // copy t of this wave fills operand block qd = (wave + 4 t) mod NB (qd < NA: A rows
  // 8 qd .. 8 qd + 7; else B rows 8 (qd - NA) ..). Lane l fills row slot l / 8, chunk slot l mod 8:
  // row 8 q + ((l / 8) xor (q mod 2)) of the operand, 16-byte chunk (l mod 8) xor (row mod 8).
  // Rows of A from m_split on come from A2 (row m_split of the product is row 0 of A2).
  const T* src[CPW];
  int dst[CPW];
#pragma unroll
  for (int t = 0; t < CPW; ++t) {
    const int q = wave + 4 * t;
    const int qd = q < NB ? q : q - NB;
    const int qo = qd < NA ? qd : qd - NA;
    const int r = 8 * qo + ((lane >> 3) ^ (qo & 1));
    const int ko = 8 * ((lane & 7) ^ (r & 7));
    dst[t] = qd * 64;
    if (qd < NA) {
      const int mm = m0 + r;
      const long long row = mm < mv ? (long long)(a_idx ? a_idx[mm] : mm) : 0;
      const T* abase = row < m_split ? reinterpret_cast<const T*>(A) + row * lda
                                     : reinterpret_cast<const T*>(A2) + (row - m_split) * lda;
      src[t] = abase + ko;
    } else {
      const long long row = n0 + r;
      src[t] = reinterpret_cast<const T*>(B) + row * ldb + ko;
    }
  }
  // LDS place of this lane's operand fragment (row l mod 16 of a 16-row tile, chunk 4 u + l / 16)
  // relative to the tile's first block: independent of the tile
  int rd[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    rd[u] = ((lane >> 3) & 1) * 64 + 8 * ((lane & 7) ^ ((lane >> 3) & 1)) + ((4 * u + (lane >> 4)) ^ (lane & 7));
  mf32x4 acc[RT][4];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mf32x4{0.f, 0.f, 0.f, 0.f};
#define GSI_WISSUE(STAGE, K0)                                                                          \
  do {                                                                                                 \
    _Pragma("unroll") for (int t = 0; t < CPW; ++t) __builtin_amdgcn_global_load_lds(                  \
        (const void*)(src[t] + (K0)), (dlds_void*)((dlu32x4*)(STAGE) + dst[t]), 16, 0, 0);             \
  } while (0)
// both sub-steps' operand fragments are read before the first product, so the LDS latency is
// paid once per step
#define GSI_WCOMPUTE(STAGE)                                                                            \
  do {                                                                                                 \
    mu32x4 af[2][RT], bf[2][4];                                                                        \
    _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                                    \
      _Pragma("unroll") for (int i = 0; i < RT; ++i) af[u][i] = ((const dlu32x4*)(STAGE))[2 * i * 64 + rd[u]]; \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                    \
        bf[u][j] = ((const dlu32x4*)(STAGE))[(NA + 2 * (wave * 4 + j)) * 64 + rd[u]];                 \
    }                                                                                                  \
    _Pragma("unroll") for (int u = 0; u < 2; ++u)                                                      \
      _Pragma("unroll") for (int i = 0; i < RT; ++i)                                                   \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[i][j] = mfma_op<T>::run(af[u][i], bf[u][j], acc[i][j]); \
  } while (0)
// every step issues exactly CPW copies per wave (past the last stage they re-read the last K step
// into a stage nobody reads again), so waiting until at most CPW remain completes the current one
#define GSI_WSTEP(CUR, FUT, ST)                                                                         \
  do {                                                                                                 \
    dwait_vmcnt<CPW>();                                                                                \
    dlds_barrier();                                                                                    \
    GSI_WISSUE(FUT, kb + min((ST) + 2, nk - 1) * 64);                                                  \
    GSI_WCOMPUTE(CUR);                                                                                 \
  } while (0)
  const int kb = (int)blockIdx.z * k_chunk;
  const int nk = (min(kdim, kb + k_chunk) - kb) / 64;
  GSI_WISSUE(st0, kb);
  GSI_WISSUE(st1, kb + min(1, nk - 1) * 64);
  int s0 = 0;
  for (; s0 + 3 <= nk; s0 += 3) {
    GSI_WSTEP(st0, st2, s0);
    GSI_WSTEP(st1, st0, s0 + 1);
    GSI_WSTEP(st2, st1, s0 + 2);
  }
  if (s0 < nk) GSI_WSTEP(st0, st2, s0);
  if (s0 + 1 < nk) GSI_WSTEP(st1, st0, s0 + 1);
  dwait_vmcnt<0>();  // no copy may land in LDS after the block ends
#undef GSI_WSTEP
#undef GSI_WCOMPUTE
#undef GSI_WISSUE
  if (part) {
    float* pz = part + (long long)blockIdx.z * m * n;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = m0 + i * 16 + 4 * (lane >> 4) + r;
        if (mm >= mv) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) pz[(long long)mm * n + n0 + wave * 64 + j * 16 + (lane & 15)] = acc[i][j][r];
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = m0 + i * 16 + 4 * (lane >> 4) + r;
      if (mm >= mv) continue;
      const long long crow = c_idx ? c_idx[mm] : mm;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int nn = n0 + wave * 64 + j * 16 + (lane & 15);
        float v = acc[i][j][r];
        if (sub_identity && mm == nn) v -= 1.0f;
        st_from_f32<TC>(C, crow * ldc + nn, v);
      }
    }
}

// ---------------------------------------------------------------------------------------------
// Products of the create-time precompute ([W; V^T] (V^T)^T and V^T V split over K, and
// (V^T V - I) V^T): a 128 x 256 output tile per block of 8 waves, two waves per SIMD; wave w owns
// rows 64 (w / 4) .. + 63 and columns 64 (w mod 4) .. + 63 of the tile (16 tiles of
// v_mfma_f32_16x16x32, 64 accumulator registers per lane). Operands are copied straight into LDS
// (global_load_lds_dwordx4) in blocks of 1 KB = 8 rows x 128 bytes of a 64-column K step, with
// the block layout and xor swizzle of gemm_nt_wide_kernel, so operand reads are one conflict-free
// 16-byte LDS read per lane. One copy ring per operand: waves 0-3 copy only A (16 blocks per K
// step, 4 copies per wave) into RA stages, waves 4-7 only B (32 blocks, 8 copies per wave) into
// RB stages; each group waits on its own copies (A issued RA - 1 steps ahead, B RB - 1), and the
// barrier after the waits joins them. B's column index wraps at kwrap_b (its kwrap_b columns
// serve an A with kdim = a multiple of them). Rows from m_split on come from A2. Block z covers K
// columns [z k_chunk, (z + 1) k_chunk); with C given (one K chunk) results are rounded to T and
// stored to C (row stride ldc), otherwise raw float32 sums go to part[z][m][n].
// ---------------------------------------------------------------------------------------------
constexpr int ring_gcd(int a, int b) { return b == 0 ? a : ring_gcd(b, a % b); }

template <int I, int L, typename F>
__device__ __forceinline__ void unroll_steps(F&& f) {
  if constexpr (I < L) {
    f(std::integral_constant<int, I>{});
    unroll_steps<I + 1, L>(f);
  }
}

template <typename T, int RA, int RB>
__global__ __launch_bounds__(512) void gemm_nt_ring_kernel(const void* __restrict__ A, const void* __restrict__ A2,
                                                           int m_split, long long lda, const void* __restrict__ B,
                                                           long long ldb, int kwrap_b, int m, int n, int kdim,
                                                           int k_chunk, float* __restrict__ part, void* __restrict__ C,
                                                           long long ldc) {
  static_assert(RA >= 2 && RA <= 6 && RB >= 2 && RB <= 3 && RA + RB <= 8, "ring depths");
  constexpr int CA = 4, CB = 8;  // copies per wave and K step
  // one LDS object per ring slot: the compiler then knows which copies a slot's reads wait for
  // (with one array and a run-time slot it would wait for every copy in flight before any read)
  __shared__ mu32x4 sa0[16 * 64], sa1[16 * 64], sa2[RA > 2 ? 16 * 64 : 1], sa3[RA > 3 ? 16 * 64 : 1],
      sa4[RA > 4 ? 16 * 64 : 1], sa5[RA > 5 ? 16 * 64 : 1];
  __shared__ mu32x4 sb0[32 * 64], sb1[32 * 64], sb2[RB > 2 ? 32 * 64 : 1];
  const int m0 = blockIdx.x * 128, n0 = blockIdx.y * 256;
  if (m0 >= m) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 2, wc = wave & 3;
  const bool copies_a = wave < 4;
  // copy t of this wave fills operand block q = (wave mod 4) + 4 t of its operand: row
  // 8 q + ((l / 8) xor (q mod 2)), 16-byte chunk (l mod 8) xor (row mod 8) for lane l
  const T* src[CB];
#pragma unroll
  for (int t = 0; t < CB; ++t) {
    const int q = (wave & 3) + 4 * t;
    const int r = 8 * q + ((lane >> 3) ^ (q & 1));
    const int ko = 8 * ((lane & 7) ^ (r & 7));
    if (copies_a) {
      const int mm = m0 + (t < CA ? r : 0);
      const long long row = mm < m ? mm : 0;
      const T* abase = row < m_split ? reinterpret_cast<const T*>(A) + row * lda
                                     : reinterpret_cast<const T*>(A2) + (row - m_split) * lda;
      src[t] = abase + ko;
    } else {
      src[t] = reinterpret_cast<const T*>(B) + (long long)(n0 + r) * ldb + ko;
    }
  }
  int rd[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    rd[u] = ((lane >> 3) & 1) * 64 + 8 * ((lane & 7) ^ ((lane >> 3) & 1)) + ((4 * u + (lane >> 4)) ^ (lane & 7));
  mf32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mf32x4{0.f, 0.f, 0.f, 0.f};
  const int kb = (int)blockIdx.z * k_chunk;
  const int nk = (min(kdim, kb + k_chunk) - kb) / 64;  // >= 1: the launch checks the split
  const int wave4 = wave & 3;
  auto slot_a = [&](auto ic) -> dlu32x4* {
    constexpr int i = decltype(ic)::value;
    if constexpr (i == 0) return (dlu32x4*)sa0;
    else if constexpr (i == 1) return (dlu32x4*)sa1;
    else if constexpr (i == 2) return (dlu32x4*)sa2;
    else if constexpr (i == 3) return (dlu32x4*)sa3;
    else if constexpr (i == 4) return (dlu32x4*)sa4;
    else return (dlu32x4*)sa5;
  };
  auto slot_b = [&](auto ic) -> dlu32x4* {
    constexpr int i = decltype(ic)::value;
    if constexpr (i == 0) return (dlu32x4*)sb0;
    else if constexpr (i == 1) return (dlu32x4*)sb1;
    else return (dlu32x4*)sb2;
  };
  auto issue_a = [&](int step, dlu32x4* dst) {
#pragma unroll
    for (int t = 0; t < CA; ++t)
      __builtin_amdgcn_global_load_lds((const void*)(src[t] + kb + step * 64), (dlds_void*)(dst + (wave4 + 4 * t) * 64),
                                       16, 0, 0);
  };
  auto issue_b = [&](int step, dlu32x4* dst) {
    const int kbb = (kb + step * 64) % kwrap_b;
#pragma unroll
    for (int t = 0; t < CB; ++t)
      __builtin_amdgcn_global_load_lds((const void*)(src[t] + kbb), (dlds_void*)(dst + (wave4 + 4 * t) * 64), 16, 0, 0);
  };
  constexpr int DA = RA - 1, DB = RB - 1;  // steps issued ahead
  constexpr int L = RA * RB / ring_gcd(RA, RB);  // the slots repeat after L steps
  // the K loop, once per copy group: each copy of it holds only its group's copies (the waits
  // the compiler adds for LDS reads then see only the copies this wave can have in flight) and
  // both pass the same barriers
  auto k_loop = [&](auto group) {
    constexpr bool kA = decltype(group)::value;
    constexpr int D = kA ? DA : DB;
    // every step issues exactly its copies (past the last K step they re-read that step into a
    // slot nobody reads again), so one fixed wait completes the current step: the copies of the
    // D - 1 later steps may stay in flight
    auto refill = [&](int step, auto slot) {
      if constexpr (kA)
        issue_a(min(step, nk - 1), slot_a(slot));
      else
        issue_b(min(step, nk - 1), slot_b(slot));
    };
    unroll_steps<0, D>([&](auto ic) { refill(decltype(ic)::value, ic); });
    auto step = [&](auto ic, int s) {
      constexpr int I = decltype(ic)::value;  // s mod L
      dwait_vmcnt<(kA ? CA : CB) * (D - 1)>();
      dlds_barrier();
      // refill the slot every wave finished reading in step s - 1
      refill(s + D, std::integral_constant<int, (I + D) % (kA ? RA : RB)>{});
      const dlu32x4* pa = slot_a(std::integral_constant<int, I % RA>{});
      const dlu32x4* pb = slot_b(std::integral_constant<int, I % RB>{});
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        mu32x4 af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = pa[2 * (4 * wr + i) * 64 + rd[u]];
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = pb[2 * (4 * wc + j) * 64 + rd[u]];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma_op<T>::run(af[i], bf[j], acc[i][j]);
      }
    };
    // whole groups of L steps, then the last nk mod L (kept apart so the loop body has no
    // data-dependent step: the waits the compiler derives for it then match the fixed ones)
    int s0 = 0;
    for (; s0 + L <= nk; s0 += L) unroll_steps<0, L>([&](auto ic) { step(ic, s0 + decltype(ic)::value); });
    unroll_steps<0, L - 1>([&](auto ic) {
      if (s0 + decltype(ic)::value < nk) step(ic, s0 + decltype(ic)::value);
    });
  };
  if (copies_a)
    k_loop(std::true_type{});
  else
    k_loop(std::false_type{});
  dwait_vmcnt<0>();  // every copy was waited for above; kept so no copy can outlive the block
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = m0 + wr * 64 + i * 16 + 4 * (lane >> 4) + r;
      if (mm >= m) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int nn = n0 + wc * 64 + j * 16 + (lane & 15);
        if (C)
          reinterpret_cast<T*>(C)[(long long)mm * ldc + nn] = from_f32<T>(acc[i][j][r]);
        else
          part[((long long)blockIdx.z * m + mm) * n + nn] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------------------------
// Matrix-core NT GEMM for a small output with a long K (V^T V - I, the batched projection
// X V): one 16x16 output tile per block; wave w accumulates the 32-column K steps w, w + 4, ...
// from global memory (8 steps of loads in flight), and the four partial tiles are added in a
// fixed order through LDS, so results are reproducible run to run.
// ---------------------------------------------------------------------------------------------
template <typename T, typename TC>
__global__ __launch_bounds__(256) void gemm_nt_kslice_kernel(const void* __restrict__ A, long long lda,
                                                             const void* __restrict__ B, long long ldb,
                                                             void* __restrict__ C, long long ldc, int m, int n,
                                                             int kdim, int sub_identity, int k_chunk,
                                                             float* __restrict__ part) {
  __shared__ mf32x4 part_w[3][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tm = blockIdx.y * 16, tn = blockIdx.x * 16;
  const int ra = min(tm + (lane & 15), m - 1), rb = min(tn + (lane & 15), n - 1);
  const mu32x4* pa = reinterpret_cast<const mu32x4*>(reinterpret_cast<const T*>(A) + (long long)ra * lda) + (lane >> 4);
  const mu32x4* pb = reinterpret_cast<const mu32x4*>(reinterpret_cast<const T*>(B) + (long long)rb * ldb) + (lane >> 4);
  // K steps of 32 columns (4 chunks of 16 bytes per row) of this block's K chunk (split K: block
  // z takes [z k_chunk, (z + 1) k_chunk) and writes its raw sums to part[z])
  const int s_end = min(kdim, (int)(blockIdx.z + 1) * k_chunk) / 32;
  mf32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  int s = (int)blockIdx.z * k_chunk / 32 + wave;
  for (; s + 28 < s_end; s += 32) {
    mu32x4 a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = pa[(s + 4 * u) * 4];
      b[u] = pb[(s + 4 * u) * 4];
    }
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      acc0 = mfma_op<T>::run(a[u], b[u], acc0);
      acc1 = mfma_op<T>::run(a[u + 1], b[u + 1], acc1);
    }
  }
  for (; s < s_end; s += 4) acc0 = mfma_op<T>::run(pa[s * 4], pb[s * 4], acc0);
  mf32x4 acc = acc0 + acc1;
  if (wave > 0) part_w[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    acc = ((acc + part_w[0][lane]) + part_w[1][lane]) + part_w[2][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = tm + 4 * (lane >> 4) + r, nn = tn + (lane & 15);
      if (mm >= m || nn >= n) continue;
      if (part) {
        part[((long long)blockIdx.z * m + mm) * n + nn] = acc[r];
      } else {
        float v = acc[r];
        if (sub_identity && mm == nn) v -= 1.0f;
        st_from_f32<TC>(C, (long long)mm * ldc + nn, v);
      }
    }
  }
}

template <typename T, int MT>
static void* pick_wide_c(int c_type) {
  switch (c_type) {
    case GSI_F32: return (void*)gemm_nt_wide_kernel<T, float, MT>;
    case GSI_F16: return (void*)gemm_nt_wide_kernel<T, f16_t, MT>;
    case GSI_BF16: return (void*)gemm_nt_wide_kernel<T, bf16_t, MT>;
  }
  return nullptr;
}

template <typename T>
static void* pick_wide(int mt, int c_type) {
  return mt == 64 ? pick_wide_c<T, 64>(c_type)
         : mt == 32 ? pick_wide_c<T, 32>(c_type)
                    : pick_wide_c<T, 16>(c_type);
}

template <typename T>
static void* pick_kslice_c(int c_type) {
  switch (c_type) {
    case GSI_F32: return (void*)gemm_nt_kslice_kernel<T, float>;
    case GSI_F16: return (void*)gemm_nt_kslice_kernel<T, f16_t>;
    case GSI_BF16: return (void*)gemm_nt_kslice_kernel<T, bf16_t>;
  }
  return nullptr;
}

template <typename T>
static void* pick_mfma_lds_c(int c_type) {
  switch (c_type) {
    case GSI_F32: return (void*)gemm_nt_mfma_lds_kernel<T, float>;
    case GSI_F16: return (void*)gemm_nt_mfma_lds_kernel<T, f16_t>;
    case GSI_BF16: return (void*)gemm_nt_mfma_lds_kernel<T, bf16_t>;
  }
  return nullptr;
}

template <typename TA, typename TB>
static void* pick_mfma_c(int c_type) {
  switch (c_type) {
    case GSI_F32: return (void*)gemm_nt_mfma_kernel<TA, TB, float>;
    case GSI_F16: return (void*)gemm_nt_mfma_kernel<TA, TB, f16_t>;
    case GSI_BF16: return (void*)gemm_nt_mfma_kernel<TA, TB, bf16_t>;
  }
  return nullptr;
}

template <typename TA, typename TB>
static void* pick_c(int c_type) {
  switch (c_type) {
    case GSI_F32: return (void*)gemm_nt_kernel<TA, TB, float>;
    case GSI_F16: return (void*)gemm_nt_kernel<TA, TB, f16_t>;
    case GSI_BF16: return (void*)gemm_nt_kernel<TA, TB, bf16_t>;
  }
  return nullptr;
}
template <typename TA>
static void* pick_b(int b_type, int c_type) {
  switch (b_type) {
    case GSI_F32: return pick_c<TA, float>(c_type);
    case GSI_F16: return pick_c<TA, f16_t>(c_type);
    case GSI_BF16: return pick_c<TA, bf16_t>(c_type);
  }
  return nullptr;
}

// the register-fed matrix-core kernel for these operand types, or null
static void* pick_mfma(int a_type, int b_type, int c_type) {
  if (a_type == GSI_BF16 && b_type == GSI_BF16) return pick_mfma_c<bf16_t, bf16_t>(c_type);
  if (a_type == GSI_F16 && b_type == GSI_F16) return pick_mfma_c<f16_t, f16_t>(c_type);
  if (a_type == GSI_F32 && b_type == GSI_BF16) return pick_mfma_c<float, bf16_t>(c_type);
  return nullptr;
}

// ---------------------------------------------------------------------------------------------
// Small float32 NT GEMM on the vector ALU (the batched G (V^T V - I), T x k x k): one 16x16
// output tile per block, one output per thread. K is staged through LDS 512 columns at a time
// (one load phase for k <= 512, so the product waits for memory once); each output is a
// fixed-order sum.
// ---------------------------------------------------------------------------------------------
constexpr int kSmallK = 512;
__global__ __launch_bounds__(256) void gemm_nt_small_f32_kernel(const float* __restrict__ A, long long lda,
                                                                const float* __restrict__ B, long long ldb,
                                                                float* __restrict__ C, long long ldc, int m, int n,
                                                                int kdim, int k_chunk, float* __restrict__ part) {
  // rows padded by 4 floats: the 16 rows of B read at one K index fall in 16 different banks
  __shared__ float As[16][kSmallK + 4], Bs[16][kSmallK + 4];
  const int tm = blockIdx.y * 16, tn = blockIdx.x * 16;
  const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
  // K split over blockIdx.z (raw sums of chunk z to part[z][m][n]) when part is given
  const int kb = blockIdx.z * k_chunk, ke = min(kdim, kb + k_chunk);
  float acc = 0.f;
  for (int k0 = kb; k0 < ke; k0 += kSmallK) {
    const int kn = min(kSmallK, ke - k0);  // a multiple of 4 (kdim and k_chunk are multiples of 8)
    // 16 rows x kn columns of each operand as float4: kn / 4 per row
    for (int idx = threadIdx.x; idx < 16 * (kSmallK / 4); idx += 256) {
      const int rr = idx / (kSmallK / 4), q = idx % (kSmallK / 4);
      if (4 * q < kn) {
        const int ra = min(tm + rr, m - 1), rb = min(tn + rr, n - 1);
        const float4 va = *reinterpret_cast<const float4*>(A + (long long)ra * lda + k0 + 4 * q);
        const float4 vb = *reinterpret_cast<const float4*>(B + (long long)rb * ldb + k0 + 4 * q);
        As[rr][4 * q] = va.x; As[rr][4 * q + 1] = va.y; As[rr][4 * q + 2] = va.z; As[rr][4 * q + 3] = va.w;
        Bs[rr][4 * q] = vb.x; Bs[rr][4 * q + 1] = vb.y; Bs[rr][4 * q + 2] = vb.z; Bs[rr][4 * q + 3] = vb.w;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kn; ++kk) acc = __builtin_fmaf(As[r][kk], Bs[c][kk], acc);
    __syncthreads();
  }
  if (tm + r < m && tn + c < n) {
    if (part)
      part[((long long)blockIdx.z * m + tm + r) * n + tn + c] = acc;
    else
      C[(long long)(tm + r) * ldc + tn + c] = acc;
  }
}

static void* pick_reduce(int c_type) {
  switch (c_type) {
    case GSI_F32: return (void*)splitk_reduce_kernel<float>;
    case GSI_F16: return (void*)splitk_reduce_kernel<f16_t>;
    case GSI_BF16: return (void*)splitk_reduce_kernel<bf16_t>;
  }
  return nullptr;
}

int launch_gemm_nt(int a_type, int b_type, int c_type, const void* A, long long lda, const int* a_idx,
                   const void* B, long long ldb, void* C, long long ldc, const int* c_idx, int m, int n, int kdim,
                   const int* m_count, int sub_identity, hipStream_t s) {
  if (m <= 0 || n <= 0) return GSI_OK;
  void* fn = nullptr;
  const bool same16 = a_type == b_type && (a_type == GSI_BF16 || a_type == GSI_F16);
  // float32 products too small to fill the chip with 64x64 tiles: 16x16 tiles
  if (a_type == GSI_F32 && b_type == GSI_F32 && c_type == GSI_F32 && !a_idx && !c_idx && !m_count && !sub_identity &&
      (long long)((m + 63) / 64) * ((n + 63) / 64) < 128) {
    dim3 grid((n + 15) / 16, (m + 15) / 16);
    gemm_nt_small_f32_kernel<<<grid, 256, 0, s>>>((const float*)A, lda, (const float*)B, ldb, (float*)C, ldc, m, n,
                                                 kdim, kdim, nullptr);
    return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
  }
  // a small output with a long K and no row lists: one 16x16 tile per block, K split over 4 waves
  if (same16 && kdim % 32 == 0 && kdim >= 1024 && !a_idx && !c_idx && !m_count && m <= 1024 && n <= 1024) {
    fn = a_type == GSI_BF16 ? pick_kslice_c<bf16_t>(c_type) : pick_kslice_c<f16_t>(c_type);
    if (!fn) return GSI_ERR_DTYPE;
    dim3 grid((n + 15) / 16, (m + 15) / 16);
    int k_chunk = kdim;
    float* part = nullptr;
    void* args[] = {&A, &lda, &B, &ldb, &C, &ldc, &m, &n, &kdim, &sub_identity, &k_chunk, &part};
    hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
    return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
  }
  // a tall A against a short, wide B (M = W V with k a multiple of 256): A streams once
  if (same16 && kdim % 64 == 0 && n % 256 == 0 && m >= 256) {
    // rows per tile: the most that still gives about one block per CU (a block's time is set by
    // its copies in flight, so more blocks, not bigger ones, raise the rate)
    const long long cols = n / 256;
    const int mt = (m + 63) / 64 * cols >= 192 ? 64 : (m + 31) / 32 * cols >= 192 ? 32 : 16;
    fn = a_type == GSI_BF16 ? pick_wide<bf16_t>(mt, c_type) : pick_wide<f16_t>(mt, c_type);
    if (!fn) return GSI_ERR_DTYPE;
    dim3 grid((m + mt - 1) / mt, n / 256);
    int k_chunk = kdim;
    float* no_part = nullptr;
    const void* no_a2 = nullptr;
    int m_split = m;
    void* args[] = {&A, &lda, &a_idx, &B, &ldb, &C, &ldc, &c_idx, &m, &n, &kdim, &m_count, &sub_identity,
                    &k_chunk, &no_part, &no_a2, &m_split};
    hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
    return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
  }
  // LDS-staged matrix cores: one 16-bit type for A and B, K in whole 32-column steps, and enough
  // rows to fill 128-row tiles (the small-m products of the batched path use the direct kernel)
  if (kdim % 32 == 0 && m >= 128 && a_type == b_type && (a_type == GSI_BF16 || a_type == GSI_F16)) {
    fn = a_type == GSI_BF16 ? pick_mfma_lds_c<bf16_t>(c_type) : pick_mfma_lds_c<f16_t>(c_type);
    if (!fn) return GSI_ERR_DTYPE;
    dim3 grid((n + 127) / 128, (m + 127) / 128);
    void* args[] = {&A, &lda, &a_idx, &B, &ldb, &C, &ldc, &c_idx, &m, &n, &kdim, &m_count, &sub_identity};
    hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
    return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
  }
  // matrix cores for 16-bit operands of one type (float32 A with bf16 B through the bf16 split);
  // the vector-ALU kernel for the rest. Operand rows must start on 16 bytes (d and k are
  // multiples of 8 elements).
  fn = pick_mfma(a_type, b_type, c_type);
  if (fn) {
    dim3 grid((n + 63) / 64, (m + 63) / 64);
    int k_chunk = kdim;
    float* part = nullptr;
    void* args[] = {&A, &lda, &a_idx, &B, &ldb, &C, &ldc, &c_idx, &m, &n, &kdim, &m_count, &sub_identity,
                    &k_chunk, &part};
    hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
    return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
  }
  switch (a_type) {
    case GSI_F32: fn = pick_b<float>(b_type, c_type); break;
    case GSI_F16: fn = pick_b<f16_t>(b_type, c_type); break;
    case GSI_BF16: fn = pick_b<bf16_t>(b_type, c_type); break;
  }
  if (!fn) return GSI_ERR_DTYPE;
  dim3 grid((n + GBN - 1) / GBN, (m + GBM - 1) / GBM);
  void* args[] = {&A, &lda, &a_idx, &B, &ldb, &C, &ldc, &c_idx, &m, &n, &kdim, &m_count, &sub_identity};
  hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
  return e == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

// Float32 NT GEMM with K split over blockIdx.z (the calibration's token products, whose 64 x 64
// tiles alone would not fill the chip): the tile scheme of gemm_nt_kernel over the columns
// [z k_chunk, (z + 1) k_chunk), raw sums to part[z][m][n].
__global__ __launch_bounds__(256) void gemm_nt_f32_tile64_kernel(const float* __restrict__ A, long long lda,
                                                                 const float* __restrict__ B, long long ldb, int m,
                                                                 int n, int kdim, int k_chunk,
                                                                 float* __restrict__ part) {
  __shared__ float As[GBK][GBM + 4];
  __shared__ float Bs[GBK][GBN + 4];
  const int m0 = blockIdx.y * GBM, n0 = blockIdx.x * GBN;
  const int kb = blockIdx.z * k_chunk, ke = min(kdim, kb + k_chunk);
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  const int lr = tid / 4, lk = (tid % 4) * 8;
  const int am = m0 + lr, bn = n0 + lr;
  const bool a_ok = am < m, b_ok = bn < n;
  const float* arow = A + (long long)(a_ok ? am : 0) * lda;
  const float* brow = B + (long long)(b_ok ? bn : 0) * ldb;
  for (int k0 = kb; k0 < ke; k0 += GBK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = k0 + lk + e;
      As[lk + e][lr] = (a_ok && kk < ke) ? arow[kk] : 0.f;
      Bs[lk + e][lr] = (b_ok && kk < ke) ? brow[kk] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < GBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* pz = part + (long long)blockIdx.z * m * n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mm = m0 + ty * 4 + i;
    if (mm >= m) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nn = n0 + tx * 4 + j;
      if (nn < n) pz[(long long)mm * n + nn] = acc[i][j];
    }
  }
}

// Float32 C[m, n] = A B^T with K split over blocks (the calibration's products): for a large
// output 64 x 64 tiles in up to 8 K chunks, for a small output with a long K (a panel against the
// earlier rows) 16 x 16 tiles in up to 16 chunks; raw sums per chunk into part ([splits, m, n], at
// least part_elems long), then their sum in chunk order into C. One chunk (no reduction) when
// part is too small.
int launch_gemm_nt_f32_splitk(const float* A, long long lda, const float* B, long long ldb, float* C, long long ldc,
                              int m, int n, int kdim, float* part, long long part_elems, hipStream_t s) {
  if (m <= 0 || n <= 0) return GSI_OK;
  const long long tiles64 = (long long)((n + 63) / 64) * ((m + 63) / 64);
  if (tiles64 >= 32 && part) {
    // a large output: 64 x 64 tiles, K split so that about 512 blocks run (at least 512 columns
    // per chunk, at most 8 chunks)
    int splits = (int)std::min<long long>(8, std::max<long long>(1, (512 + tiles64 - 1) / tiles64));
    splits = std::min(splits, std::max(1, kdim / 512));
    while (splits > 1 && (long long)splits * m * n > part_elems) --splits;
    if (splits < 2)
      return launch_gemm_nt(GSI_F32, GSI_F32, GSI_F32, A, lda, nullptr, B, ldb, C, ldc, nullptr, m, n, kdim, nullptr,
                            0, s);
    int k_chunk = ((kdim + splits - 1) / splits + GBK - 1) / GBK * GBK;
    splits = (kdim + k_chunk - 1) / k_chunk;
    dim3 grid((n + GBN - 1) / GBN, (m + GBM - 1) / GBM, splits);
    gemm_nt_f32_tile64_kernel<<<grid, 256, 0, s>>>(A, lda, B, ldb, m, n, kdim, k_chunk, part);
    if (hipGetLastError() != hipSuccess) return GSI_ERR_HIP;
    const float* cpart = part;
    const int* no_count = nullptr;
    const int* no_idx = nullptr;
    void* Cv = C;
    void* rargs[] = {&cpart, &splits, &m, &n, &no_count, &Cv, &ldc, &no_idx};
    dim3 rgrid((unsigned)std::min(16, (n + 255) / 256), m);
    return hipLaunchKernel((void*)splitk_reduce_kernel<float>, rgrid, dim3(256), rargs, 0, s) == hipSuccess
               ? GSI_OK
               : GSI_ERR_HIP;
  }
  const long long tiles = (long long)((n + 15) / 16) * ((m + 15) / 16);
  int splits = (int)std::min<long long>(16, std::max<long long>(1, (256 + tiles - 1) / tiles));
  splits = std::min(splits, std::max(1, kdim / 256));
  while (splits > 1 && (long long)splits * m * n > part_elems) --splits;
  int k_chunk = ((kdim + splits - 1) / splits + 7) / 8 * 8;
  splits = (kdim + k_chunk - 1) / k_chunk;
  dim3 grid((n + 15) / 16, (m + 15) / 16, splits);
  if (splits < 2 || !part) {
    gemm_nt_small_f32_kernel<<<dim3(grid.x, grid.y), 256, 0, s>>>(A, lda, B, ldb, C, ldc, m, n, kdim, kdim, nullptr);
    return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
  }
  gemm_nt_small_f32_kernel<<<grid, 256, 0, s>>>(A, lda, B, ldb, C, ldc, m, n, kdim, k_chunk, part);
  if (hipGetLastError() != hipSuccess) return GSI_ERR_HIP;
  const float* cpart = part;
  const int* no_count = nullptr;
  const int* no_idx = nullptr;
  void* Cv = C;
  void* rargs[] = {&cpart, &splits, &m, &n, &no_count, &Cv, &ldc, &no_idx};
  dim3 rgrid((unsigned)std::min(16, (n + 255) / 256), m);
  return hipLaunchKernel((void*)splitk_reduce_kernel<float>, rgrid, dim3(256), rargs, 0, s) == hipSuccess ? GSI_OK
                                                                                                     : GSI_ERR_HIP;
}

// K chunks the skinny kernel takes for an m <= 64 row product (0 when it does not apply): the
// split rule of launch_gemm_nt_split, about 1024 blocks, at least 256 K columns per chunk.
int skinny_splits(int a_type, int b_type, int m, int n, int kdim, long long part_elems) {
  const bool ok = (a_type == GSI_BF16 && b_type == GSI_BF16) || (a_type == GSI_F16 && b_type == GSI_F16) ||
                  (a_type == GSI_F32 && b_type == GSI_BF16);
  if (!ok || m > 64 || m <= 0 || n <= 0) return 0;
  const long long tiles = (long long)((n + 63) / 64);
  int splits = (int)std::min<long long>(kMaxSplit, std::max<long long>(1, (1024 + tiles - 1) / tiles));
  splits = std::min(splits, std::max(1, kdim / 256));
  while (splits > 1 && (long long)splits * m * n > part_elems) --splits;
  if (splits < 2) return 0;
  const int k_chunk = ((kdim + splits - 1) / splits + 31) / 32 * 32;
  return (kdim + k_chunk - 1) / k_chunk;
}

// The skinny kernel's raw K-chunk sums only (no reduction): part[z][mm][nn] for the mv valid
// rows, `splits` from skinny_splits.
int launch_skinny_partials(int a_type, int b_type, const void* A, long long lda, const int* a_idx, const void* B,
                           long long ldb, int m, int n, int kdim, const int* m_count, int splits, float* part,
                           hipStream_t s) {
  int k_chunk = ((kdim + splits - 1) / splits + 31) / 32 * 32;
  void* sk = a_type == GSI_BF16 ? (void*)gemm_nt_skinny_staged_kernel<bf16_t, bf16_t>
             : a_type == GSI_F16 ? (void*)gemm_nt_skinny_staged_kernel<f16_t, f16_t>
                                 : (void*)gemm_nt_skinny_staged_kernel<float, bf16_t>;
  dim3 grid((n + 63) / 64, 1, splits);
  void* args[] = {&A, &lda, &a_idx, &B, &ldb, &m, &n, &kdim, &m_count, &k_chunk, &part};
  return hipLaunchKernel(sk, grid, dim3(256), args, 0, s) == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

// One reduction for two token lists (the batched fast and slow products): row slot mm < *ca takes
// list a (partials pa, sa chunks, output row ia[mm]), the next *cb slots list b; sums in chunk
// order.
template <typename TC>
__global__ __launch_bounds__(256) void splitk_reduce2_kernel(const float* __restrict__ pa, int sa,
                                                             const int* __restrict__ ca, const int* __restrict__ ia,
                                                             const float* __restrict__ pb, int sb,
                                                             const int* __restrict__ cb, const int* __restrict__ ib,
                                                             int m, int n, void* __restrict__ C, long long ldc) {
  const int na = min(m, *ca), nb = min(m, *cb);
  int mm = blockIdx.y;
  const float* part = pa;
  int splits = sa;
  const int* idx = ia;
  if (mm >= na) {
    mm -= na;
    if (mm >= nb) return;
    part = pb;
    splits = sb;
    idx = ib;
  }
  const long long crow = idx[mm];
  for (int nn = blockIdx.x * 256 + threadIdx.x; nn < n; nn += gridDim.x * 256) {
    float v = 0.f;
    for (int z = 0; z < splits; ++z) v += part[((long long)z * m + mm) * n + nn];
    st_from_f32<TC>(C, crow * ldc + nn, v);
  }
}

int launch_reduce2(int c_type, const float* pa, int sa, const int* ca, const int* ia, const float* pb, int sb,
                   const int* cb, const int* ib, int m, int n, void* C, long long ldc, hipStream_t s) {
  void* fn = c_type == GSI_F32 ? (void*)splitk_reduce2_kernel<float>
             : c_type == GSI_F16 ? (void*)splitk_reduce2_kernel<f16_t>
                                 : (void*)splitk_reduce2_kernel<bf16_t>;
  void* args[] = {&pa, &sa, &ca, &ia, &pb, &sb, &cb, &ib, &m, &n, &C, &ldc};
  dim3 grid((unsigned)std::min(16, (n + 255) / 256), m);
  return hipLaunchKernel(fn, grid, dim3(256), args, 0, s) == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

// Split-K variant for products with few output tiles and a long K (the batched fast and slow
// paths): the register-fed matrix-core kernel over S chunks of K, raw sums into part
// ([S, m, n] float32, at least part_elems long), then their sum in chunk order into C. Falls back
// to launch_gemm_nt when the types have no matrix-core kernel or S would be 1.
// ---------------------------------------------------------------------------------------------
// Create-time precompute with a workspace [GSI §2.1]: M = W V on 128 x 256 tiles split over K
// (each K chunk at least 512 columns, about 192 or more blocks in all) with a fixed-order
// reduction, and V^T V - I on 16 x 16 tiles split over K the same way. Without a workspace (or
// for shapes the tiles do not fit) the single-pass kernels run instead.
// ---------------------------------------------------------------------------------------------
// Split plan of the create-time products on 128 x 256 tiles (one block per CU, 256 CUs):
//   fused:  [W; V^T] (V^T)^T = [M; V^T V] in one launch of sm K chunks;
//   else:   W (V^T)^T in sm chunks, then V^T (V^T)^T in sd chunks, two launches.
// The fused launch is taken when it keeps at least 3/4 of the blocks of the separate one within
// one wave of blocks. sm = 0: the shape does not take the split path.
struct PrecomputePlan {
  int sm, sd;  // K chunks of the image product and (when sd > 0) of the separate V^T V product
  bool fused;
};

static int best_splits(long long tiles, int d) {
  // the most chunks (a power of two) that keep tiles x chunks within 256 blocks, with every chunk
  // at least 256 columns (four K steps: fewer partial sums to add, and copy rings that fill) and a
  // whole number of 64-column steps
  int sp = 1;
  while (tiles * sp * 2 <= 256 && d % (2 * sp) == 0 && d / (2 * sp) >= 256 && (d / (2 * sp)) % 64 == 0) sp *= 2;
  return sp;
}

static PrecomputePlan precompute_plan(int dtype, int d_out, int d, int k) {
  PrecomputePlan pl{0, 0, false};
  if (dtype == GSI_F32 || k % 256 != 0 || d % 512 != 0 || d_out < 128) return pl;
  const long long cols = k / 256;
  const long long tiles_w = (long long)((d_out + 127) / 128) * cols, tiles_f = (long long)((d_out + k + 127) / 128) * cols;
  // the image product: K chunks of at least 512 columns
  auto img_splits = [&](long long tiles) {
    int sp = 1;
    while (tiles * sp * 2 <= 256 && d % (2 * sp) == 0 && d / (2 * sp) >= 512 && (d / (2 * sp)) % 64 == 0) sp *= 2;
    return sp;
  };
  const int sw = img_splits(tiles_w), sf = img_splits(tiles_f);
  if (tiles_f * sf * 4 >= tiles_w * sw * 3 && tiles_f * sf <= 256) {
    pl.sm = sf;
    pl.fused = true;
  } else {
    pl.sm = sw;
    pl.sd = best_splits((long long)(k / 128) * cols, d);
  }
  return pl;
}

int precompute_splits(int dtype, int d_out, int d, int k) { return precompute_plan(dtype, d_out, d, k).sm; }

// (V^T V - I) V^T on matrix cores: D = V^T V - I split into 16-bit high and low parts by the
// precompute reduction, stored as DD = [D_hi | D_lo] (k x 2k), and one product of DD against V's
// rows with V's k columns used twice (every product exact, float32 sums), rounded to the dtype
static bool vdt_on_mfma(int dtype, int d, int k) { return dtype != GSI_F32 && d % 256 == 0 && k % 64 == 0 && k >= 64; }
static size_t dd_bytes(int dtype, int d, int k) {
  return vdt_on_mfma(dtype, d, k) ? align256((size_t)2 * k * k * 2) : 0;
}

// create workspace: [DD][K-chunk partials of M (or [M; V^T V])][K-chunk partials of V^T V]
size_t precompute_ws_bytes(int dtype, int d_out, int d, int k) {
  const PrecomputePlan pl = precompute_plan(dtype, d_out, d, k);
  if (pl.sm == 0) return 0;
  const size_t img = (size_t)pl.sm * (pl.fused ? d_out + k : d_out) * k * 4;
  const size_t gram = pl.fused ? 0 : (size_t)pl.sd * k * k * 4;
  return dd_bytes(dtype, d, k) + align256(img) + align256(gram);
}

// depths of the two copy rings of gemm_nt_ring_kernel (A steps, B steps; 16 KB and 32 KB each)
constexpr int kRingA = 4, kRingB = 3;

static int launch_ring(int dtype, const void* A, const void* A2, int m_split, long long lda, const void* B,
                       long long ldb, int kwrap_b, int m, int n, int kdim, int splits, float* part, void* C,
                       long long ldc, hipStream_t s) {
  void* fn = dtype == GSI_BF16 ? (void*)gemm_nt_ring_kernel<bf16_t, kRingA, kRingB>
                               : (void*)gemm_nt_ring_kernel<f16_t, kRingA, kRingB>;
  int k_chunk = kdim / splits;
  // every block needs at least one whole 64-column step of K, n whole 256-column tiles, and B
  // steps that do not straddle its wrap
  if (splits < 1 || kdim % splits != 0 || k_chunk % 64 != 0 || k_chunk < 64 || n % 256 != 0 || kwrap_b % 64 != 0 ||
      kdim % kwrap_b != 0 || (C && splits != 1) || (!C && !part))
    return GSI_ERR_SHAPE;
  dim3 grid((m + 127) / 128, n / 256, splits);
  void* args[] = {&A, &A2, &m_split, &lda, &B, &ldb, &kwrap_b, &m, &n, &kdim, &k_chunk, &part, &C, &ldc};
  return hipLaunchKernel(fn, grid, dim3(512), args, 0, s) == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

// With the workspace: the split products above, then one reduction that rounds M, subtracts I
// from V^T V and (16-bit layers) writes DD for launch_vdt (*dd then points to it). Without: the
// single-pass kernels (*dd = null).
int launch_precompute(int dtype, const void* W, const void* Vt, void* M, float* Dl, int d_out, int d, int k,
                      void* ws, size_t ws_bytes, const void** dd, hipStream_t s) {
  *dd = nullptr;
  const PrecomputePlan pl = precompute_plan(dtype, d_out, d, k);
  if (ws && pl.sm > 0 && precompute_ws_bytes(dtype, d_out, d, k) <= ws_bytes) {
    const size_t ddb = dd_bytes(dtype, d, k);
    float* pw = (float*)((char*)ws + ddb);
    const int m_img = pl.fused ? d_out + k : d_out;
    int rc = launch_ring(dtype, W, Vt, d_out, d, Vt, d, d, m_img, k, d, pl.sm, pw, nullptr, 0, s);
    if (rc != GSI_OK) return rc;
    const long long cw = (long long)m_img * k;
    const float* pd = pw + (long long)d_out * k;  // fused: the V^T V rows follow the image rows
    long long cd = cw;
    int sd = pl.sm;
    if (!pl.fused) {
      float* pg = (float*)((char*)pw + align256((size_t)pl.sm * d_out * k * 4));
      rc = launch_ring(dtype, Vt, Vt, k, d, Vt, d, d, k, k, d, pl.sd, pg, nullptr, 0, s);
      if (rc != GSI_OK) return rc;
      pd = pg;
      cd = (long long)k * k;
      sd = pl.sd;
    }
    const int nb_img = (int)(((long long)d_out * (k / 4) + 255) / 256);
    const int nb_gram = (int)(((long long)k * (k / 4) * 8 + 255) / 256);
    const unsigned nb = (unsigned)(nb_img + nb_gram);
    void* ddp = ddb ? ws : nullptr;
    if (dtype == GSI_BF16)
      precompute_reduce_kernel<bf16_t><<<nb, 256, 0, s>>>(pw, pl.sm, cw, pd, sd, cd, d_out, k, M, Dl, (bf16_t*)ddp, nb_img);
    else
      precompute_reduce_kernel<f16_t><<<nb, 256, 0, s>>>(pw, pl.sm, cw, pd, sd, cd, d_out, k, M, Dl, (f16_t*)ddp, nb_img);
    if (hipGetLastError() != hipSuccess) return GSI_ERR_HIP;
    *dd = ddp;
    return GSI_OK;
  }
  const int rc = launch_gemm_nt(dtype, dtype, dtype, W, d, nullptr, Vt, d, M, k, nullptr, d_out, k, d, nullptr, 0, s);
  if (rc != GSI_OK) return rc;
  return launch_gemm_nt(dtype, dtype, GSI_F32, Vt, d, nullptr, Vt, d, Dl, k, nullptr, k, k, d, nullptr, 1, s);
}

int launch_vdt(int dtype, const float* Dl, const void* dd, const void* V, void* VDt, int d, int k, hipStream_t s) {
  if (dd && vdt_on_mfma(dtype, d, k))  // row j: sum over K < 2k of DD[j][K] V[:, K mod k]
    return launch_ring(dtype, dd, dd, k, 2LL * k, V, k, k, k, d, 2 * k, 1, nullptr, VDt, d, s);
  // row j of (V (V^T V - I))^T = sum_l D[j][l] V[:, l]: D against V's rows
  return launch_gemm_nt(GSI_F32, dtype, dtype, Dl, k, nullptr, V, k, VDt, d, nullptr, k, d, k, nullptr, 0, s);
}

int launch_gemm_nt_split(int a_type, int b_type, int c_type, const void* A, long long lda, const int* a_idx,
                         const void* B, long long ldb, void* C, long long ldc, const int* c_idx, int m, int n,
                         int kdim, const int* m_count, float* part, long long part_elems, hipStream_t s) {
  if (m <= 0 || n <= 0) return GSI_OK;
  const bool same16 = a_type == b_type && (a_type == GSI_BF16 || a_type == GSI_F16);
  if (same16 && kdim % 32 == 0 && kdim >= 1024 && !a_idx && !c_idx && !m_count && m <= 1024 && n <= 1024 && part) {
    // 16x16 tiles with K split over the four waves of a block and over blocks
    const long long tiles16 = (long long)((n + 15) / 16) * ((m + 15) / 16);
    int splits = (int)std::min<long long>(kMaxSplit, std::max<long long>(1, (1024 + tiles16 - 1) / tiles16));
    splits = std::min(splits, std::max(1, kdim / 512));
    while (splits > 1 && (long long)splits * m * n > part_elems) --splits;
    if (splits > 1) {
      void* kf = a_type == GSI_BF16 ? pick_kslice_c<bf16_t>(GSI_F32) : pick_kslice_c<f16_t>(GSI_F32);
      int k_chunk = ((kdim + splits - 1) / splits + 31) / 32 * 32;
      splits = (kdim + k_chunk - 1) / k_chunk;
      int sub_identity = 0;
      void* c_unused = part;
      long long ldc_unused = n;
      dim3 grid((n + 15) / 16, (m + 15) / 16, splits);
      void* args[] = {&A, &lda, &B, &ldb, &c_unused, &ldc_unused, &m, &n, &kdim, &sub_identity, &k_chunk, &part};
      if (hipLaunchKernel(kf, grid, dim3(256), args, 0, s) != hipSuccess) return GSI_ERR_HIP;
      void* rf = pick_reduce(c_type);
      if (!rf) return GSI_ERR_DTYPE;
      const float* cpart = part;
      const int* no_count = nullptr;
      void* rargs[] = {&cpart, &splits, &m, &n, &no_count, &C, &ldc, &c_idx};
      dim3 rgrid((unsigned)std::min(16, (n + 255) / 256), m);
      return hipLaunchKernel(rf, rgrid, dim3(256), rargs, 0, s) == hipSuccess ? GSI_OK : GSI_ERR_HIP;
    }
  }
  void* fn = pick_mfma(a_type, b_type, c_type);
  const long long tiles = (long long)((n + 63) / 64) * ((m + 63) / 64);
  // about 1024 blocks, at least 256 K columns (8 steps) per chunk, at most kMaxSplit chunks
  int splits = (int)std::min<long long>(kMaxSplit, std::max<long long>(1, (1024 + tiles - 1) / tiles));
  splits = std::min(splits, std::max(1, kdim / 256));
  while (splits > 1 && (long long)splits * m * n > part_elems) --splits;
  if (!fn || splits < 2 || !part)
    return launch_gemm_nt(a_type, b_type, c_type, A, lda, a_idx, B, ldb, C, ldc, c_idx, m, n, kdim, m_count, 0, s);
  int k_chunk = ((kdim + splits - 1) / splits + 31) / 32 * 32;
  splits = (kdim + k_chunk - 1) / k_chunk;
  if (m <= 64) {  // at most 64 rows (a token list): the skinny kernel, B loaded once per block
    void* sk = a_type == GSI_BF16 && b_type == GSI_BF16 ? (void*)gemm_nt_skinny_staged_kernel<bf16_t, bf16_t>
               : a_type == GSI_F16 && b_type == GSI_F16 ? (void*)gemm_nt_skinny_staged_kernel<f16_t, f16_t>
               : a_type == GSI_F32 && b_type == GSI_BF16 ? (void*)gemm_nt_skinny_staged_kernel<float, bf16_t>
                                                        : nullptr;
    if (sk) {
      dim3 grid((n + 63) / 64, 1, splits);
      void* args[] = {&A, &lda, &a_idx, &B, &ldb, &m, &n, &kdim, &m_count, &k_chunk, &part};
      if (hipLaunchKernel(sk, grid, dim3(256), args, 0, s) != hipSuccess) return GSI_ERR_HIP;
      void* rf = pick_reduce(c_type);
      if (!rf) return GSI_ERR_DTYPE;
      const float* cpart = part;
      void* rargs[] = {&cpart, &splits, &m, &n, &m_count, &C, &ldc, &c_idx};
      dim3 rgrid((unsigned)std::min(16, (n + 255) / 256), m);
      return hipLaunchKernel(rf, rgrid, dim3(256), rargs, 0, s) == hipSuccess ? GSI_OK : GSI_ERR_HIP;
    }
  }
  int sub_identity = 0;
  void* fn_out = pick_mfma(a_type, b_type, GSI_F32);
  dim3 grid((n + 63) / 64, (m + 63) / 64, splits);
  void* c_unused = part;       // the kernel writes part when it is given, never C
  long long ldc_unused = n;
  void* args[] = {&A, &lda, &a_idx, &B, &ldb, &c_unused, &ldc_unused, &c_idx, &m, &n, &kdim, &m_count,
                  &sub_identity, &k_chunk, &part};
  if (hipLaunchKernel(fn_out, grid, dim3(256), args, 0, s) != hipSuccess) return GSI_ERR_HIP;
  void* rf = pick_reduce(c_type);
  if (!rf) return GSI_ERR_DTYPE;
  const float* cpart = part;
  void* rargs[] = {&cpart, &splits, &m, &n, &m_count, &C, &ldc, &c_idx};
  dim3 rgrid((unsigned)std::min(16, (n + 255) / 256), m);
  return hipLaunchKernel(rf, rgrid, dim3(256), rargs, 0, s) == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

// ---------------------------------------------------------------------------------------------
// dst[k, d] = transpose(src[d, k]), 64 x 64 tiles through LDS. A whole tile is read and written
// in 16-byte pieces (rows of both matrices are whole multiples of 16 bytes: d and k are multiples
// of 8); tiles cut by the matrix edge (d or k not a multiple of 64) go element by element.
// ---------------------------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E* __restrict__ src, E* __restrict__ dst, int d, int k,
                                                        LayerDesc desc, int P, PlanRow* __restrict__ plan) {
  constexpr int T = 64, VE = 16 / (int)sizeof(E), CPR = T / VE;  // elements per piece, pieces per tile row
  __shared__ E t[T][T + 2];
  // block (0, 0) also writes the decode kernel's plan rows of the layer (one per grid block)
  if (plan && blockIdx.x == 0 && blockIdx.y == 0 && (int)threadIdx.x < P)
    plan[threadIdx.x] = make_plan_row(desc, threadIdx.x, P, (int)sizeof(E));
  const int c0 = blockIdx.x * T, r0 = blockIdx.y * T;  // src rows r (d), cols c (k)
  if (r0 + T <= d && c0 + T <= k) {
    for (int q = threadIdx.x; q < T * CPR; q += 256) {
      const int r = q / CPR, c = (q % CPR) * VE;
      const mu32x4 v = *reinterpret_cast<const mu32x4*>(src + (long long)(r0 + r) * k + c0 + c);
      const E* e = reinterpret_cast<const E*>(&v);
#pragma unroll
      for (int i = 0; i < VE; ++i) t[r][c + i] = e[i];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < T * CPR; q += 256) {
      const int c = q / CPR, r = (q % CPR) * VE;
      mu32x4 v;
      E* e = reinterpret_cast<E*>(&v);
#pragma unroll
      for (int i = 0; i < VE; ++i) e[i] = t[r + i][c];
      *reinterpret_cast<mu32x4*>(dst + (long long)(c0 + c) * d + r0 + r) = v;
    }
    return;
  }
  for (int q = threadIdx.x; q < T * T; q += 256) {
    const int r = q / T, c = q % T;
    if (r0 + r < d && c0 + c < k) t[r][c] = src[(long long)(r0 + r) * k + c0 + c];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < T * T; q += 256) {
    const int c = q / T, r = q % T;
    if (r0 + r < d && c0 + c < k) dst[(long long)(c0 + c) * d + r0 + r] = t[r][c];
  }
}

int launch_transpose(int dtype, const void* src, void* dst, int d, int k, const LayerDesc& desc, int P,
                     PlanRow* plan, hipStream_t s) {
  if (plan && (P < 1 || P > 256)) return GSI_ERR_DEVICE;
  dim3 grid((k + 63) / 64, (d + 63) / 64);
  if (dtype == GSI_F32)
    transpose_kernel<uint32_t><<<grid, 256, 0, s>>>((const uint32_t*)src, (uint32_t*)dst, d, k, desc, P, plan);
  else
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, d, k, desc, P, plan);
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

// ---------------------------------------------------------------------------------------------
// Batched gate: one block per token. nx2 = |x|^2, gg = |g|^2, q = g^T (V^T V - I) g, then
// nr2 = nx2 - gg + q (= |x - V g|^2 exactly in real arithmetic) and the float32 comparison
// nr2 < fl(fl(eps^2) * nx2) -> fast [GSI §2.2]. Fixed-order block reductions.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float block_sum_256(float v, float* red) {
  // wave reduction (fixed butterfly order), then the 4 wave sums in index order
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

template <typename T>
__global__ __launch_bounds__(256) void gate_batched_kernel(const void* __restrict__ X, long long x_ld, int d, int k,
                                                           const float* __restrict__ G, const float* __restrict__ H,
                                                           float eps, uint8_t* __restrict__ gate, int gate_ld,
                                                           float* __restrict__ rho, float* __restrict__ nx2_out) {
  __shared__ float red[8];
  const int t = blockIdx.x;
  const T* x = reinterpret_cast<const T*>(X) + (long long)t * x_ld;
  float sx = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) {
    float v = to_f32(x[i]);
    sx = __builtin_fmaf(v, v, sx);
  }
  float sg = 0.f, sq = 0.f;
  for (int j = threadIdx.x; j < k; j += 256) {
    const float gj = G[(long long)t * k + j];
    sg = __builtin_fmaf(gj, gj, sg);
    sq = __builtin_fmaf(gj, H[(long long)t * k + j], sq);
  }
  const float nx2 = block_sum_256(sx, red);
  const float gg = block_sum_256(sg, red + 4);
  __syncthreads();
  const float q = block_sum_256(sq, red);
  if (threadIdx.x == 0) {
    const float nr2 = (nx2 - gg) + q;
    const float thr = eps * eps;
    const float rhs = thr * nx2;
    const bool fast = nr2 < rhs;
    gate[(long long)t * gate_ld] = fast ? 0 : 1;
    if (rho) rho[(long long)t * gate_ld] = sqrtf(fmaxf(nr2, 0.f) / nx2);
    nx2_out[t] = nx2;
  }
}

// Token compaction in token order: fast_idx / slow_idx lists and counts[0] (fast), counts[1] (slow).
__global__ __launch_bounds__(1024) void compact_kernel(const uint8_t* __restrict__ gate, int gate_ld, int T,
                                                       int* __restrict__ fast_idx, int* __restrict__ slow_idx,
                                                       int* __restrict__ counts) {
  __shared__ int wsum[2][16];
  __shared__ int base[2];
  if (threadIdx.x == 0) base[0] = base[1] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x / 64;
  for (int t0 = 0; t0 < T; t0 += 1024) {
    const int t = t0 + threadIdx.x;
    const bool valid = t < T;
    const bool slow = valid && gate[(long long)t * gate_ld] != 0;
    const bool fast = valid && !slow;
    const u64 mf = __ballot(fast), ms = __ballot(slow);
    const u64 below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int pf = __popcll(mf & below), ps = __popcll(ms & below);
    if (lane == 0) { wsum[0][w] = __popcll(mf); wsum[1][w] = __popcll(ms); }
    __syncthreads();
    int of = base[0], os = base[1];
    for (int i = 0; i < w; ++i) { of += wsum[0][i]; os += wsum[1][i]; }
    if (fast) fast_idx[of + pf] = t;
    if (slow) slow_idx[os + ps] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int i = 0; i < 16; ++i) { base[0] += wsum[0][i]; base[1] += wsum[1][i]; }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) { counts[0] = base[0]; counts[1] = base[1]; }
}

static size_t proj_bytes(int k, int T) {
  const size_t t = (size_t)std::min(T, 64);
  return align256((size_t)kMaxProjChunks * t * 2 * k * 4) + align256((size_t)(kMaxK / 16) * t * 2 * 4) +
         align256((size_t)kMaxProjChunks * t * 4);
}
size_t batched_ws_bytes(int k, int T, int d_out) {
  return kBatchedCounters * 4 + 2 * align256((size_t)T * k * 4) + align256((size_t)T * 4) * 3 + align256(2 * 4) +
         2 * align256(split_part_elems(T, d_out) * 4) + 2 * proj_bytes(k, T);
}
BatchedWs batched_ws_carve(void* base, int k, int T, int d_out) {
  char* p = (char*)base;
  BatchedWs w;
  // the counters first, at an offset and size that do not depend on the site's shape: they must
  // stay zero between calls whatever else the workspace was carved into
  w.cnt = (int*)p;
  p += kBatchedCounters * 4;
  w.part_elems = split_part_elems(T, d_out);
  w.G = (float*)p; p += align256((size_t)T * k * 4);
  w.H = (float*)p; p += align256((size_t)T * k * 4);
  w.nx2 = (float*)p; p += align256((size_t)T * 4);
  w.fast_idx = (int*)p; p += align256((size_t)T * 4);
  w.slow_idx = (int*)p; p += align256((size_t)T * 4);
  w.counts = (int*)p; p += align256(2 * 4);
  w.part = w.part_elems ? (float*)p : nullptr;
  p += align256(w.part_elems * 4);
  w.part2 = w.part_elems ? (float*)p : nullptr;
  p += align256(w.part_elems * 4);
  const size_t t = (size_t)std::min(T, 64);
  for (int set = 0; set < 2; ++set) {
    w.Pp[set] = (float*)p; p += align256((size_t)kMaxProjChunks * t * 2 * k * 4);
    w.gq[set] = (float*)p; p += align256((size_t)(kMaxK / 16) * t * 2 * 4);
    w.nx2p[set] = (float*)p; p += align256((size_t)kMaxProjChunks * t * 4);
  }
  return w;
}

// Gate bits and token lists of a site without a gate: a static-projection site sends every token
// to the fast path, a dense site every token to the slow path; rho is reported as NaN.
__global__ __launch_bounds__(256) void mode_lists_kernel(int T, int slow, uint8_t* __restrict__ gate, int gate_ld,
                                                         float* __restrict__ rho, int* __restrict__ fast_idx,
                                                         int* __restrict__ slow_idx, int* __restrict__ counts) {
  for (int t = threadIdx.x; t < T; t += 256) {
    gate[(long long)t * gate_ld] = (uint8_t)slow;
    if (rho) rho[(long long)t * gate_ld] = __builtin_nanf("");
    (slow ? slow_idx : fast_idx)[t] = t;
  }
  if (threadIdx.x == 0) {
    counts[0] = slow ? 0 : T;
    counts[1] = slow ? T : 0;
  }
}

int launch_gate_batched(int dtype, const LayerDesc& L, const void* X, long long x_ld, int T, float eps,
                        const BatchedWs& w, uint8_t* gate, int gate_ld, float* rho, hipStream_t s) {
  if (L.mode == kSiteDense) {
    mode_lists_kernel<<<1, 256, 0, s>>>(T, 1, gate, gate_ld, rho, w.fast_idx, w.slow_idx, w.counts);
    return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
  }
  // G = X V as X (V^T)^T: [T, k] float32
  int rc = launch_gemm_nt_split(dtype, dtype, GSI_F32, X, x_ld, nullptr, L.Vt, L.d, w.G, L.k, nullptr, T, L.k, L.d,
                                nullptr, w.part, w.part_elems, s);
  if (rc != GSI_OK) return rc;
  if (L.mode == kSiteStatic) {
    mode_lists_kernel<<<1, 256, 0, s>>>(T, 0, gate, gate_ld, rho, w.fast_idx, w.slow_idx, w.counts);
    return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
  }
  // H = G (V^T V - I)  (the matrix is symmetric, so its rows serve as the K-contiguous operand)
  rc = launch_gemm_nt(GSI_F32, GSI_F32, GSI_F32, w.G, L.k, nullptr, L.Dl, L.k, w.H, L.k, nullptr, T, L.k, L.k,
                      nullptr, 0, s);
  if (rc != GSI_OK) return rc;
  if (dtype == GSI_F32)
    gate_batched_kernel<float><<<T, 256, 0, s>>>(X, x_ld, L.d, L.k, w.G, w.H, eps, gate, gate_ld, rho, w.nx2);
  else if (dtype == GSI_F16)
    gate_batched_kernel<f16_t><<<T, 256, 0, s>>>(X, x_ld, L.d, L.k, w.G, w.H, eps, gate, gate_ld, rho, w.nx2);
  else
    gate_batched_kernel<bf16_t><<<T, 256, 0, s>>>(X, x_ld, L.d, L.k, w.G, w.H, eps, gate, gate_ld, rho, w.nx2);
  if (hipGetLastError() != hipSuccess) return GSI_ERR_HIP;
  compact_kernel<<<1, 1024, 0, s>>>(gate, gate_ld, T, w.fast_idx, w.slow_idx, w.counts);
  if (hipGetLastError() != hipSuccess) return GSI_ERR_HIP;
  return GSI_OK;
}


// Cross-block hand-off inside one launch without cache flushes: partial sums are written with
// device-scope stores (coherent across the XCDs' L2s), every wave waits until its stores have
// completed, then one thread counts the block in; the block that counts last reads the partial
// sums with device-scope loads and resets the counter for the next launch.
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool arrive_last(int* cnt, int total, int* s_last) {
  dwait_vmcnt<0>();  // this wave's device-scope stores are complete
  __syncthreads();   // ... and every other wave's
  if (threadIdx.x == 0)
    *s_last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1;
  __syncthreads();
  return *s_last;
}

// ---------------------------------------------------------------------------------------------
// Batched path in two launches per site and chunk of at most 64 tokens (16-bit weights).
//
// bproj_kernel: [G | H] = X [V_k | V_k (V_k^T V_k - I)] on matrix cores, h = (V^T V - I) g being
// the second half [GSI §2.2: the residual norm from g and the stored basis]. Block (b, z) streams
// rows 32 b .. 32 b + 31 of V^T and of (V (V^T V - I))^T (the skinny tiles, x staged in LDS) over
// K chunk z and stores the raw float32 sums for every token; blocks of tile 0 also store each
// token's |x|^2 over the chunk. The last block of a tile to finish adds the chunks in chunk order,
// stores g split into high and low parts in the weight dtype, and per token the tile's sums of
// g^2 and g h.
// ---------------------------------------------------------------------------------------------
struct BProjArgs {
  const void* X;
  long long x_ld;
  int ntok, d, k, with_h, kc;
  const void* Vt;
  const void* VDt;
  float* Pp;    // [Zp][ntok][2 k]: tile b's 32 g then 32 h columns at 64 b
  float* nx2p;  // [ntok][kMaxProjChunks]
  void* Ghi;    // [ntok][k] high parts of g in the weight dtype
  void* Glo;    // [ntok][k] low parts: g - Ghi rounded to the weight dtype
  float* gq;    // [ntok][kMaxK / 16][2], tiles of 32 columns
  int* cnt;     // [k / 32], zero between launches
};

// one block of the projection: column tile b, K chunk z of nz (lds_a: 32 KB)
template <typename T>
__device__ __forceinline__ void bproj_block(const BProjArgs& p, int b, int z, int nz, mu32x4* lds_a, int& s_last) {
  const int k2 = 2 * p.k;
  const int kb = z * p.kc, ke = min(p.d, kb + p.kc);
  float* pz = p.Pp + (long long)z * p.ntok * k2;
  const T* x = reinterpret_cast<const T*>(p.X);
  const T* vt = reinterpret_cast<const T*>(p.Vt);
  const T* vd = p.with_h ? reinterpret_cast<const T*>(p.VDt) : vt;
  float* x2 = b == 0 ? p.nx2p + z : nullptr;
  mu32x4 b0[8], b1[8];
  switch ((p.ntok + 15) >> 4) {  // uniform
    case 1: skinny_staged_tiles<T, T, 1>(x, p.x_ld, nullptr, vt, p.d, p.ntok, k2, kb, ke, pz, lds_a, lds_a, nullptr, true, nullptr, b0, b1, b, vd, x2); break;
    case 2: skinny_staged_tiles<T, T, 2>(x, p.x_ld, nullptr, vt, p.d, p.ntok, k2, kb, ke, pz, lds_a, lds_a, nullptr, true, nullptr, b0, b1, b, vd, x2); break;
    case 3: skinny_staged_tiles<T, T, 3>(x, p.x_ld, nullptr, vt, p.d, p.ntok, k2, kb, ke, pz, lds_a, lds_a, nullptr, true, nullptr, b0, b1, b, vd, x2); break;
    default: skinny_staged_tiles<T, T, 4>(x, p.x_ld, nullptr, vt, p.d, p.ntok, k2, kb, ke, pz, lds_a, lds_a, nullptr, true, nullptr, b0, b1, b, vd, x2); break;
  }
  if (!arrive_last(&p.cnt[b], nz, &s_last)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // the tile's last block: thread (t, q) = (tid / 4, tid mod 4) takes columns 8 q .. 8 q + 7 of
  // the tile's g and h for token t, summing the chunks in chunk order
  const int t = threadIdx.x >> 2, q = threadIdx.x & 3;
  const bool ok = t < p.ntok;
  float g[8], h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) g[e] = h[e] = 0.f;
  if (ok) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float4 v[kMaxProjChunks][2];
#pragma unroll
      for (int zz = 0; zz < kMaxProjChunks; ++zz) {
        if (zz < nz) {
          const float4* src = reinterpret_cast<const float4*>(p.Pp + ((long long)zz * p.ntok + t) * k2 + 64 * b +
                                                              32 * half + 8 * q);
          v[zz][0] = src[0];
          v[zz][1] = src[1];
        }
      }
      float* o = half ? h : g;
#pragma unroll
      for (int zz = 0; zz < kMaxProjChunks; ++zz) {
        if (zz < nz) {
          o[0] += v[zz][0].x; o[1] += v[zz][0].y; o[2] += v[zz][0].z; o[3] += v[zz][0].w;
          o[4] += v[zz][1].x; o[5] += v[zz][1].y; o[6] += v[zz][1].z; o[7] += v[zz][1].w;
        }
      }
    }
  }
  float gg = 0.f, gh = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    gg = __builtin_fmaf(g[e], g[e], gg);
    gh = __builtin_fmaf(g[e], h[e], gh);
  }
  gg += __shfl_xor(gg, 1, 64);
  gh += __shfl_xor(gh, 1, 64);
  gg += __shfl_xor(gg, 2, 64);
  gh += __shfl_xor(gh, 2, 64);
  if (ok) {
    // g split once here for the fast product's matrix-core passes (|g - hi - lo| <= 2^-18 |g|
    // for bf16)
    unsigned short hv[8], lv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const T hi = from_f32<T>(g[e]);
      const T lo = from_f32<T>(g[e] - to_f32(hi));
      hv[e] = hi.b;
      lv[e] = lo.b;
    }
    const long long off = (long long)t * p.k + 32 * b + 8 * q;
    *reinterpret_cast<mu32x4*>(reinterpret_cast<T*>(p.Ghi) + off) =
        mu32x4{hv[0] | ((unsigned)hv[1] << 16), hv[2] | ((unsigned)hv[3] << 16), hv[4] | ((unsigned)hv[5] << 16),
               hv[6] | ((unsigned)hv[7] << 16)};
    *reinterpret_cast<mu32x4*>(reinterpret_cast<T*>(p.Glo) + off) =
        mu32x4{lv[0] | ((unsigned)lv[1] << 16), lv[2] | ((unsigned)lv[3] << 16), lv[4] | ((unsigned)lv[5] << 16),
               lv[6] | ((unsigned)lv[7] << 16)};
    if (q == 0) {
      p.gq[((long long)t * (kMaxK / 16) + b) * 2 + 0] = gg;
      p.gq[((long long)t * (kMaxK / 16) + b) * 2 + 1] = gh;
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(&p.cnt[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__global__ __launch_bounds__(256) void bproj_kernel(BProjArgs p) {
  __shared__ mu32x4 lds_a[4 * 8 * 64];
  __shared__ int s_last;
  bproj_block<T>(p, blockIdx.x, blockIdx.z, gridDim.z, lds_a, s_last);
}

// ---------------------------------------------------------------------------------------------
// bprod_kernel: gate and both products of one site for the chunk's tokens. Every block first
// forms the gate of every token from the projection's pieces, in one fixed order (nr2 =
// (|x|^2 - |g|^2) + g^T h, fast iff nr2 < fl(eps^2) |x|^2 [GSI §2.2]), so all blocks agree, and
// lists the fast and slow tokens in token order in LDS; block (0, nz - 1) stores the gate bits
// and rho. Block (b, z) then owns output rows 64 b .. 64 b + 63: the first zf blocks of a row tile
// (zf = 1, none on a dense site) compute y = M g over the fast tokens and all of M's K (g as its
// two 16-bit parts, two matrix-core passes), the other zs blocks y = W x over the slow tokens and
// chunk z - zf of W's K, both on the staged skinny tiles. A product that one block computes whole
// (M g; W x when W's K is one chunk) is rounded and stored as y rows by that block; a slow product
// split over K leaves raw float32 sums in Py[chunk][t][row], which the last slow block of the row
// tile adds in chunk order.
// A static-projection site lists every token as fast, a dense site every token as slow.
// ---------------------------------------------------------------------------------------------
struct BProdArgs {
  const void* X;
  long long x_ld;
  int ntok, d, d_out, k, mode;
  float eps;
  const void* Ghi;    // [ntok][k] g, high and low parts in the weight dtype
  const void* Glo;
  const float* gq;    // [ntok][kMaxK / 16][2]
  const float* nx2p;  // [ntok][kMaxProjChunks]
  int zp;
  const void* M;
  const void* W;
  int kcm, kcw;
  int zs;     // K chunks of the slow product (the last zs blocks in z); the first are the fast product's
  float* Py;  // [zf + zs][ntok][d_out]
  int* cnt;   // [d_out / 64], zero between launches
  void* Y;
  long long y_ld;
  uint8_t* gate;
  int gate_ld;
  float* rho;
};

// LDS of a products block
struct BProdLds {
  mu32x4 hi[4 * 8 * 64], lo[4 * 8 * 64];  // staged A fragments (high and low parts), 64 KB
  int fast[64], slow[64];                 // token lists
  unsigned char isfast[64];
  int n[2], last;
};

// one block of the products: row tile bx, block bz of nz (the first zf take the fast product)
template <typename T>
__device__ __forceinline__ void bprod_block(const BProdArgs& p, int bx, int bz, int nz, BProdLds& L) {
  mu32x4* lds_hi = L.hi;
  mu32x4* lds_lo = L.lo;
  int* s_fast = L.fast;
  int* s_slow = L.slow;
  unsigned char* s_isfast = L.isfast;
  int* s_n = L.n;
  // blocks z < zf (dispatched first) take the fast product, blocks zf .. zf + zs - 1 chunk
  // z - zf of the slow product; the two kinds run side by side
  const int zf = nz - p.zs;
  const bool slow_blk = bz >= zf;
  const int z = slow_blk ? bz - zf : bz;
  // a slow block requests its first sub-chunk of W before the gate is known: it arrives while the
  // gate is formed (a gated site with no slow token wastes it)
  const T* wt = reinterpret_cast<const T*>(p.W);
  const int kbw = z * p.kcw, kew = min(p.d, kbw + p.kcw);
  mu32x4 wb0[8], wb1[8];  // wb1 is loaded by the slow pass itself (registers)
  if (slow_blk && p.mode != kSiteStatic) skinny_load_b(wt, p.d, p.d_out, kbw, kew, kbw, wb0, bx);
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    bool fast = false;
    float r = __builtin_nanf("");
    if (t < p.ntok) {
      if (p.mode == kSiteGated) {
        // this token's pieces are contiguous: all loaded at once, then added in a fixed order
        // tiles of 32 columns: k / 32 (g^2, g h) pairs
        float4 xv[kMaxProjChunks / 4], qv[kMaxK / 64];
        const float4* xp = reinterpret_cast<const float4*>(p.nx2p + (long long)t * kMaxProjChunks);
        const float4* qp = reinterpret_cast<const float4*>(p.gq + (long long)t * (kMaxK / 16) * 2);
#pragma unroll
        for (int i = 0; i < kMaxProjChunks / 4; ++i) xv[i] = xp[i];
#pragma unroll
        for (int i = 0; i < kMaxK / 64; ++i)
          if (i < (p.k / 32 + 1) / 2) qv[i] = qp[i];
        float nx2 = 0.f, gg = 0.f, q = 0.f;
#pragma unroll
        for (int i = 0; i < kMaxProjChunks; ++i) {
          const float v = i % 4 == 0 ? xv[i / 4].x : i % 4 == 1 ? xv[i / 4].y : i % 4 == 2 ? xv[i / 4].z : xv[i / 4].w;
          if (i < p.zp) nx2 += v;
        }
#pragma unroll
        for (int c = 0; c < kMaxK / 32; ++c) {
          const float4 v = qv[c / 2];
          if (c < p.k / 32) {
            gg += c % 2 == 0 ? v.x : v.z;
            q += c % 2 == 0 ? v.y : v.w;
          }
        }
        const float nr2 = (nx2 - gg) + q;
        const float thr = p.eps * p.eps;
        fast = nr2 < thr * nx2;
        r = sqrtf(fmaxf(nr2, 0.f) / nx2);
      } else {
        fast = p.mode == kSiteStatic;
      }
    }
    const bool valid = t < p.ntok;
    const u64 mf = __ballot(valid && fast), ms = __ballot(valid && !fast);
    const u64 below = t ? (~0ull >> (64 - t)) : 0ull;
    if (valid && fast) s_fast[__popcll(mf & below)] = t;
    if (valid && !fast) s_slow[__popcll(ms & below)] = t;
    s_isfast[t] = fast ? 1 : 0;
    if (t == 0) {
      s_n[0] = __popcll(mf);
      s_n[1] = __popcll(ms);
    }
    if (bx == 0 && bz == nz - 1 && valid) {
      p.gate[(long long)t * p.gate_ld] = fast ? 0 : 1;
      if (p.rho) p.rho[(long long)t * p.gate_ld] = r;
    }
  }
  __syncthreads();
  const int nf = s_n[0], ns = s_n[1];
  // a token whose product one block computes whole (every fast token; the slow tokens when W's K
  // is one chunk) gets its y row straight from that block; only a slow product split over K
  // leaves partial sums for the last block of the row tile. ns is the same in every block.
  if (slow_blk && ns == 0) {
    dwait_vmcnt<0>();  // the early W loads have landed
    return;
  }
  const bool direct = !slow_blk || p.zs == 1;
  T* yd = direct ? reinterpret_cast<T*>(p.Y) : nullptr;
  float* pz = p.Py + (long long)z * p.ntok * p.d_out;
  if (!slow_blk && nf > 0) {  // fast tokens: y = M g     [GSI §2.2]
    const int kb = z * p.kcm, ke = min(p.k, kb + p.kcm);
    const T* gh = reinterpret_cast<const T*>(p.Ghi);
    const T* gl = reinterpret_cast<const T*>(p.Glo);
    const T* m = reinterpret_cast<const T*>(p.M);
    switch ((nf + 15) >> 4) {
      case 1: skinny_staged_tiles<T, T, 1, true>(gh, p.k, s_fast, m, p.k, nf, p.d_out, kb, ke, pz, lds_hi, lds_lo, s_fast, true, gl, wb0, wb1, bx, nullptr, nullptr, yd, p.y_ld); break;
      case 2: skinny_staged_tiles<T, T, 2, true>(gh, p.k, s_fast, m, p.k, nf, p.d_out, kb, ke, pz, lds_hi, lds_lo, s_fast, true, gl, wb0, wb1, bx, nullptr, nullptr, yd, p.y_ld); break;
      case 3: skinny_staged_tiles<T, T, 3, true>(gh, p.k, s_fast, m, p.k, nf, p.d_out, kb, ke, pz, lds_hi, lds_lo, s_fast, true, gl, wb0, wb1, bx, nullptr, nullptr, yd, p.y_ld); break;
      default: skinny_staged_tiles<T, T, 4, true>(gh, p.k, s_fast, m, p.k, nf, p.d_out, kb, ke, pz, lds_hi, lds_lo, s_fast, true, gl, wb0, wb1, bx, nullptr, nullptr, yd, p.y_ld); break;
    }
  }
  if (slow_blk && ns > 0) {  // slow tokens: y = W x     [GSI §2.2]
    const T* xa = reinterpret_cast<const T*>(p.X);
    switch ((ns + 15) >> 4) {
      case 1: skinny_staged_tiles<T, T, 1, false, 1>(xa, p.x_ld, s_slow, wt, p.d, ns, p.d_out, kbw, kew, pz, lds_hi, lds_lo, s_slow, true, nullptr, wb0, wb1, bx, nullptr, nullptr, yd, p.y_ld); break;
      case 2: skinny_staged_tiles<T, T, 2, false, 1>(xa, p.x_ld, s_slow, wt, p.d, ns, p.d_out, kbw, kew, pz, lds_hi, lds_lo, s_slow, true, nullptr, wb0, wb1, bx, nullptr, nullptr, yd, p.y_ld); break;
      case 3: skinny_staged_tiles<T, T, 3, false, 1>(xa, p.x_ld, s_slow, wt, p.d, ns, p.d_out, kbw, kew, pz, lds_hi, lds_lo, s_slow, true, nullptr, wb0, wb1, bx, nullptr, nullptr, yd, p.y_ld); break;
      default: skinny_staged_tiles<T, T, 4, false, 1>(xa, p.x_ld, s_slow, wt, p.d, ns, p.d_out, kbw, kew, pz, lds_hi, lds_lo, s_slow, true, nullptr, wb0, wb1, bx, nullptr, nullptr, yd, p.y_ld); break;
    }
  }
  if (direct || !arrive_last(&p.cnt[bx], p.zs, &L.last)) return;
  // the last slow block of the row tile: thread i takes rows 64 b + 4 (i mod 16) .. + 3 of the
  // slow tokens i / 16 + 16 s, summing the chunks in chunk order; one device-scope acquire, then
  // ordinary 16-byte loads, all in flight at once
  const int row = bx * 64 + 4 * (threadIdx.x & 15);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  float4 pv[4][kMaxProdChunks];
#pragma unroll
  for (int sg = 0; sg < 4; ++sg) {
    const int i = (threadIdx.x >> 4) + 16 * sg;
    if (i >= ns) continue;
    const int t = s_slow[i];
#pragma unroll
    for (int zz = 0; zz < kMaxProdChunks; ++zz)
      if (zz < p.zs) pv[sg][zz] = *reinterpret_cast<const float4*>(p.Py + ((long long)zz * p.ntok + t) * p.d_out + row);
  }
#pragma unroll
  for (int sg = 0; sg < 4; ++sg) {
    const int i = (threadIdx.x >> 4) + 16 * sg;
    if (i >= ns) continue;
    const int t = s_slow[i];
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int zz = 0; zz < kMaxProdChunks; ++zz) {
      if (zz < p.zs) {
        a[0] += pv[sg][zz].x;
        a[1] += pv[sg][zz].y;
        a[2] += pv[sg][zz].z;
        a[3] += pv[sg][zz].w;
      }
    }
    T* yr = reinterpret_cast<T*>(p.Y) + (long long)t * p.y_ld + row;
#pragma unroll
    for (int e = 0; e < 4; ++e) yr[e] = from_f32<T>(a[e]);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&p.cnt[bx], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__global__ __launch_bounds__(256) void bprod_kernel(BProdArgs p) {
  __shared__ BProdLds lds;
  bprod_block<T>(p, blockIdx.x, blockIdx.z, gridDim.z, lds);
}

// One launch of the pipelined stack: the projection of one unit (np_x column tiles x np_z K
// chunks) beside the products of the unit before it (nq_x row tiles x nq_z blocks, the first zf
// of a row tile the fast product's). Dispatch order: the slow product's blocks (the longest:
// they stream W), then the projection's, then the fast product's. The two units share no
// buffer: the projection writes one set of g, gate pieces and chunk sums while the products read
// the other set, written by the previous launch.
template <typename T>
__global__ __launch_bounds__(256) void bstep_kernel(BProjArgs pa, int np_x, int np_z, BProdArgs pb, int nq_x,
                                                    int nq_z) {
  __shared__ BProdLds lds;
  const int np = np_x * np_z, zf = nq_z - pb.zs, nslow = nq_x * pb.zs;
  int i = blockIdx.x;
  if (i < nslow) {
    bprod_block<T>(pb, i % nq_x, zf + i / nq_x, nq_z, lds);
    return;
  }
  i -= nslow;
  if (i < np)
    bproj_block<T>(pa, i % np_x, i / np_x, np_z, lds.hi, lds.last);
  else
    bprod_block<T>(pb, (i - np) % nq_x, (i - np) / nq_x, nq_z, lds);
}

// the products' partial sums (slow chunks) and the fast chunk fit the split-K buffer
static_assert(kMaxProdChunks + 1 <= kMaxSplit, "products chunks exceed the partial-sum buffer");

BatchedSplit batched_split(int dtype, const LayerDesc& L, int ntok) {
  BatchedSplit sp{0, 0, 0, 0, 0, 0};
  if (dtype == GSI_F32 || ntok < 1 || ntok > 64) return sp;
  if (L.d % 32 != 0 || L.d_out % 64 != 0 || L.k % 32 != 0 || L.k > kMaxK) return sp;
  if (kMaxK / 16 + L.d_out / 64 > kBatchedCounters) return sp;
  if (L.mode != kSiteDense && (L.k == 0 || !L.VDt)) return sp;
  // projection: tiles of 32 columns (of g and of h), about 256 blocks, at most kMaxProjChunks
  // chunks of K, every chunk non-empty
  if (L.mode != kSiteDense) {
    int zp = std::max(1, std::min(kMaxProjChunks, 256 / (L.k / 32)));
    for (;; --zp) {
      const int kc = ((L.d + zp - 1) / zp + 7) / 8 * 8;
      if ((long long)(zp - 1) * kc < L.d || zp == 1) {
        sp.zp = zp;
        sp.kc = kc;
        break;
      }
    }
  }
  // products: the fast one in one block per row tile over all of M's K (a dense site has none),
  // the slow one beside it in chunks of W's K (at most kMaxProdChunks, non-empty), about 512
  // blocks of 64 output rows in all (two per CU)
  const int nrt = L.d_out / 64;
  sp.zf = L.mode == kSiteDense ? 0 : 1;
  int zy = std::max(1, std::min(kMaxProdChunks, (512 - nrt * sp.zf) / nrt));
  for (;; --zy) {
    const int kcw = ((L.d + zy - 1) / zy + 7) / 8 * 8;
    if ((long long)(zy - 1) * kcw < L.d || zy == 1) {
      sp.zy = zy;
      sp.kcw = kcw;
      break;
    }
  }
  sp.kcm = L.mode == kSiteDense ? 8 : L.k;
  return sp;
}

// the projection's and the products' arguments of one unit; g of the unit's buffer set sits in
// the G (set 0) or H (set 1) region as its two 16-bit halves
static void unit_g(const BatchedUnit& u, void** hi, void** lo) {
  char* g = (char*)(u.set ? u.w->H : u.w->G);
  *hi = g;
  *lo = g + (size_t)u.ntok * u.L->k * 2;
}

static BProjArgs proj_args(const BatchedUnit& u) {
  BProjArgs a;
  a.X = u.X;
  a.x_ld = u.x_ld;
  a.ntok = u.ntok;
  a.d = u.L->d;
  a.k = u.L->k;
  a.with_h = u.L->mode == kSiteGated;
  a.kc = u.sp.kc;
  a.Vt = u.L->Vt;
  a.VDt = u.L->VDt;
  a.Pp = u.w->Pp[u.set];
  a.nx2p = u.w->nx2p[u.set];
  unit_g(u, &a.Ghi, &a.Glo);
  a.gq = u.w->gq[u.set];
  a.cnt = u.w->cnt;
  return a;
}

static BProdArgs prod_args(const BatchedUnit& u) {
  BProdArgs b;
  b.X = u.X;
  b.x_ld = u.x_ld;
  b.ntok = u.ntok;
  b.d = u.L->d;
  b.d_out = u.L->d_out;
  b.k = u.L->k;
  b.mode = u.L->mode;
  b.eps = u.eps;
  void *hi, *lo;
  unit_g(u, &hi, &lo);
  b.Ghi = hi;
  b.Glo = lo;
  b.gq = u.w->gq[u.set];
  b.nx2p = u.w->nx2p[u.set];
  b.zp = u.sp.zp;
  b.M = u.L->M;
  b.W = u.L->W;
  b.kcm = u.sp.kcm;
  b.kcw = u.sp.kcw;
  b.zs = u.sp.zy;
  b.Py = u.w->part;
  b.cnt = u.w->cnt + kMaxK / 16;
  b.Y = u.Y;
  b.y_ld = u.y_ld;
  b.gate = u.gate;
  b.gate_ld = u.gate_ld;
  b.rho = u.rho;
  return b;
}

int launch_batched_step(int dtype, const BatchedUnit* proj, const BatchedUnit* prod, hipStream_t s) {
  if (proj && proj->L->mode == kSiteDense) proj = nullptr;  // a dense site has no projection
  if (proj && prod && proj->set == prod->set) return GSI_ERR_SHAPE;
  const bool bf = dtype == GSI_BF16;
  if (proj && !prod) {
    const dim3 grid(proj->L->k / 32, 1, proj->sp.zp);
    if (bf)
      bproj_kernel<bf16_t><<<grid, 256, 0, s>>>(proj_args(*proj));
    else
      bproj_kernel<f16_t><<<grid, 256, 0, s>>>(proj_args(*proj));
  } else if (prod && !proj) {
    const dim3 grid(prod->L->d_out / 64, 1, prod->sp.zy + prod->sp.zf);
    if (bf)
      bprod_kernel<bf16_t><<<grid, 256, 0, s>>>(prod_args(*prod));
    else
      bprod_kernel<f16_t><<<grid, 256, 0, s>>>(prod_args(*prod));
  } else if (proj && prod) {
    const int np_x = proj->L->k / 32, np_z = proj->sp.zp;
    const int nq_x = prod->L->d_out / 64, nq_z = prod->sp.zy + prod->sp.zf;
    const unsigned nb = (unsigned)(np_x * np_z + nq_x * nq_z);
    if (bf)
      bstep_kernel<bf16_t><<<nb, 256, 0, s>>>(proj_args(*proj), np_x, np_z, prod_args(*prod), nq_x, nq_z);
    else
      bstep_kernel<f16_t><<<nb, 256, 0, s>>>(proj_args(*proj), np_x, np_z, prod_args(*prod), nq_x, nq_z);
  }
  return hipGetLastError() == hipSuccess ? GSI_OK : GSI_ERR_HIP;
}

}  // namespace gsi
