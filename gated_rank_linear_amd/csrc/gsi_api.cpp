// C ABI of libgsi (declared in include/gsi.h): argument validation, handles, and enqueueing of
// the HIP kernels. Every argument check runs before the first HIP call, so an invalid call
// enqueues nothing and never touches the device.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>

#include "gsi_internal.h"
#include "gsi_step.h"

using namespace gsi;

namespace {

bool dtype_ok(int dtype) { return dtype == GSI_F32 || dtype == GSI_F16 || dtype == GSI_BF16; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Shape rules shared by every entry point (see include/gsi.h).
int check_shape(int dtype, int d_out, int d, int k) {
  if (!dtype_ok(dtype)) return GSI_ERR_DTYPE;
  if (d_out < 1 || d < 8 || d % 8 != 0 || d > 65536) return GSI_ERR_SHAPE;
  if (k < 8 || k > 512 || k > d || !pow2(k)) return GSI_ERR_SHAPE;
  // a decode block holds its rows of y in LDS: at most kYPart rows for the largest row share,
  // ceil(d_out / kMinBlocks)
  if (((long long)d_out + kMinBlocks - 1) / kMinBlocks > kYPart) return GSI_ERR_SHAPE;
  return GSI_OK;
}

// A dense layer (k = 0): W only.
int check_dense_shape(int dtype, int d_out, int d) {
  if (!dtype_ok(dtype)) return GSI_ERR_DTYPE;
  if (d_out < 1 || d < 8 || d % 8 != 0 || d > 65536) return GSI_ERR_SHAPE;
  if (((long long)d_out + kMinBlocks - 1) / kMinBlocks > kYPart) return GSI_ERR_SHAPE;
  return GSI_OK;
}

int check_eps(float eps) {
  if (std::isnan(eps) || eps < 0.f) return GSI_ERR_EPS;
  return GSI_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? GSI_OK : GSI_ERR_HIP; }

// aux = [V^T (k x d, weight dtype)] [V^T V - I (k x k, float32)] [decode plan rows (kMaxBlocks)]
//       [(V (V^T V - I))^T (k x d, weight dtype; 16-bit layers only)]
// (a dense layer, k = 0, holds the plan rows only)
size_t aux_vt_off(int, int, int) { return 0; }
size_t aux_dl_off(int dtype, int d, int k) { return align256((size_t)k * d * dtype_size(dtype)); }
size_t aux_plan_off(int dtype, int d, int k) { return aux_dl_off(dtype, d, k) + align256((size_t)k * k * 4); }
size_t aux_vdt_off(int dtype, int d, int k) { return align256(aux_plan_off(dtype, d, k) + sizeof(PlanRow) * kMaxBlocks); }
bool has_vdt(int dtype, int k) { return dtype != GSI_F32 && k > 0; }
size_t aux_bytes(int dtype, int d, int k) {
  return aux_vdt_off(dtype, d, k) + (has_vdt(dtype, k) ? align256((size_t)k * d * dtype_size(dtype)) : 0);
}

// The decode kernel's grid, one answer per (device, dtype, input window class): the occupancy
// query behind it costs tens of microseconds, once per layer creation otherwise.
int cached_decode_grid(int dtype, int xr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> known[kMaxDevices][3][2];  // 0 unknown, else grid + 1
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int inst = xr <= 2 ? 0 : 1;
  const bool cacheable = dev >= 0 && dev < kMaxDevices && dtype >= 0 && dtype < 3;
  if (cacheable) {
    const int v = known[dev][dtype][inst].load(std::memory_order_relaxed);
    if (v != 0) return v - 1;
  }
  const int P = decode_grid(dtype, xr);
  if (cacheable) known[dev][dtype][inst].store(P + 1, std::memory_order_relaxed);
  return P;
}

// the decode kernel's input window and grid for one layer (before anything is enqueued)
int layer_grid(gsi_layer* L) {
  L->xr = decode_window(L->dtype, &L->desc, 1);
  L->P = cached_decode_grid(L->dtype, L->xr);
  return L->P == 0 ? GSI_ERR_DEVICE : GSI_OK;
}

size_t ws_bytes_for(int k, int d_out, int T) {
  return align256(decode_ws_bytes()) + batched_ws_bytes(k, T < 1 ? 1 : T, d_out);
}

WsHeader* ws_header(void* ws) { return reinterpret_cast<WsHeader*>(ws); }

BatchedWs batched_part(void* ws, int k, int T, int d_out) {
  return batched_ws_carve((char*)ws + align256(decode_ws_bytes()), k, T, d_out);
}

// Units of the two-launch batched path in flight on one stream: each unit's projection runs in
// the same launch as the products of the unit before it. A unit's inputs are given when it is
// enqueued and its projection reads nothing the earlier unit writes, so the two are independent;
// the projection's latency is then spent while the earlier products stream their weights. The
// two alternate between the workspace's two sets of projection buffers.
class BatchedPipe {
 public:
  BatchedPipe(int dtype, const BatchedWs& w, hipStream_t s) : dtype_(dtype), w_(&w), s_(s) {}
  int push(BatchedUnit u) {
    u.w = w_;
    u.set = set_;
    set_ ^= 1;
    const int rc = launch_batched_step(dtype_, &u, pending_ ? &prev_ : nullptr, s_);
    prev_ = u;
    pending_ = rc == GSI_OK;
    return rc;
  }
  // the products of the last unit
  int flush() {
    if (!pending_) return GSI_OK;
    pending_ = false;
    return launch_batched_step(dtype_, nullptr, &prev_, s_);
  }

 private:
  int dtype_;
  const BatchedWs* w_;
  hipStream_t s_;
  bool pending_ = false;
  BatchedUnit prev_{};
  int set_ = 0;
};

// Batched path for one site over T tokens whose rows sit at X (+ row stride x_ld) and Y; w is the
// batched part of the workspace, carved for the largest k and d_out of the call.
int run_batched(int dtype, const LayerDesc& L, const void* X, long long x_ld, int T, float eps, void* Y,
                long long y_ld, uint8_t* gate, int gate_ld, float* rho, const BatchedWs& w, BatchedPipe& pipe,
                hipStream_t s) {
  if (batched_split(dtype, L, std::min(T, 64)).zy > 0) {
    // two launches per chunk of at most 64 tokens, overlapped with the units around it
    for (int t0 = 0; t0 < T; t0 += 64) {
      BatchedUnit u{};
      u.L = &L;
      u.ntok = std::min(64, T - t0);
      u.sp = batched_split(dtype, L, u.ntok);
      u.X = (const char*)X + (size_t)t0 * x_ld * dtype_size(dtype);
      u.x_ld = x_ld;
      u.eps = eps;
      u.Y = (char*)Y + (size_t)t0 * y_ld * dtype_size(dtype);
      u.y_ld = y_ld;
      u.gate = gate + (size_t)t0 * gate_ld;
      u.gate_ld = gate_ld;
      u.rho = rho ? rho + (size_t)t0 * gate_ld : nullptr;
      const int rc = pipe.push(u);
      if (rc != GSI_OK) return rc;
    }
    return GSI_OK;
  }
  // the kernels below use the workspace's other regions: the units in flight finish first
  int rc = pipe.flush();
  if (rc != GSI_OK) return rc;
  rc = launch_gate_batched(dtype, L, X, x_ld, T, eps, w, gate, gate_ld, rho, s);
  if (rc != GSI_OK) return rc;
  if (L.mode == kSiteDense)  // every token: y = W x
    return launch_gemm_nt_split(dtype, dtype, dtype, X, x_ld, w.slow_idx, L.W, L.d, Y, y_ld, w.slow_idx, T, L.d_out,
                                L.d, w.counts + 1, w.part, w.part_elems, s);
  if (L.mode == kSiteStatic)  // every token: y = M g
    return launch_gemm_nt_split(GSI_F32, dtype, dtype, w.G, L.k, w.fast_idx, L.M, L.k, Y, y_ld, w.fast_idx, T,
                                L.d_out, L.k, w.counts + 0, w.part, w.part_elems, s);
  // both products on the skinny kernel: their K-chunk sums in two buffers, one reduction into y
  const int sa = skinny_splits(GSI_F32, dtype, T, L.d_out, L.k, w.part_elems);
  const int sb = skinny_splits(dtype, dtype, T, L.d_out, L.d, w.part_elems);
  if (sa >= 2 && sb >= 2 && w.part2) {
    // fast tokens: y = M g; slow tokens: y = W x     [GSI §2.2]
    rc = launch_skinny_partials(GSI_F32, dtype, w.G, L.k, w.fast_idx, L.M, L.k, T, L.d_out, L.k, w.counts + 0, sa,
                                w.part, s);
    if (rc != GSI_OK) return rc;
    rc = launch_skinny_partials(dtype, dtype, X, x_ld, w.slow_idx, L.W, L.d, T, L.d_out, L.d, w.counts + 1, sb,
                                w.part2, s);
    if (rc != GSI_OK) return rc;
    return launch_reduce2(dtype, w.part, sa, w.counts + 0, w.fast_idx, w.part2, sb, w.counts + 1, w.slow_idx, T,
                          L.d_out, Y, y_ld, s);
  }
  // fast tokens: y = M g     [GSI §2.2]
  rc = launch_gemm_nt_split(GSI_F32, dtype, dtype, w.G, L.k, w.fast_idx, L.M, L.k, Y, y_ld, w.fast_idx, T, L.d_out,
                            L.k, w.counts + 0, w.part, w.part_elems, s);
  if (rc != GSI_OK) return rc;
  // slow tokens: y = W x     [GSI §2.2]
  return launch_gemm_nt_split(dtype, dtype, dtype, X, x_ld, w.slow_idx, L.W, L.d, Y, y_ld, w.slow_idx, T, L.d_out,
                              L.d, w.counts + 1, w.part, w.part_elems, s);
}

}  // namespace

extern "C" {

const char* gsi_status_string(int code) {
  switch (code) {
    case GSI_OK: return "ok";
    case GSI_ERR_NULL: return "null pointer argument";
    case GSI_ERR_SHAPE: return "dimension out of range (d, k multiples of 8, k a power of two <= min(d, 512))";
    case GSI_ERR_DTYPE: return "unknown or mismatched dtype";
    case GSI_ERR_EPS: return "eps must be >= 0 and not NaN";
    case GSI_ERR_WORKSPACE: return "workspace missing or too small";
    case GSI_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case GSI_ERR_DEVICE: return "current device is not gfx950 or cannot co-schedule the persistent grid";
    case GSI_ERR_HIP: return "HIP runtime error";
    case GSI_ERR_TIMEOUT: return "an in-kernel wait exceeded its bound";
  }
  return "unknown status";
}

int gsi_device_check(void) {
  // the answer per device is cached: reading the device properties costs about a millisecond
  constexpr int kMaxDevices = 64;
  static std::atomic<int> known[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GSI_ERR_DEVICE;
  if (dev >= 0 && dev < kMaxDevices) {
    const int k = known[dev].load(std::memory_order_relaxed);
    if (k != 0) return k == 1 ? GSI_OK : GSI_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GSI_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < kMaxDevices) known[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? GSI_OK : GSI_ERR_DEVICE;
}

size_t gsi_layer_aux_bytes(int dtype, int d_out, int d, int k) {
  if (k == 0) return check_dense_shape(dtype, d_out, d) == GSI_OK ? aux_bytes(dtype, d, 0) : 0;
  if (check_shape(dtype, d_out, d, k) != GSI_OK) return 0;
  return aux_bytes(dtype, d, k);
}

size_t gsi_layer_create_workspace_bytes(int dtype, int d_out, int d, int k) {
  if (check_shape(dtype, d_out, d, k) != GSI_OK) return 0;
  return precompute_ws_bytes(dtype, d_out, d, k);
}

int gsi_layer_create(gsi_layer** out, int dtype, int d_out, int d, int k, const void* W, const void* V, void* M,
                     void* aux, size_t aux_nbytes, void* ws, size_t ws_nbytes, void* stream) {
  if (!out) return GSI_ERR_NULL;
  *out = nullptr;
  int rc = check_shape(dtype, d_out, d, k);
  if (rc != GSI_OK) return rc;
  if (!W || !V || !M || !aux) return GSI_ERR_NULL;
  if (!aligned16(W) || !aligned16(V) || !aligned16(M) || !aligned16(aux) || !aligned16(ws)) return GSI_ERR_ALIGN;
  if (aux_nbytes < aux_bytes(dtype, d, k)) return GSI_ERR_WORKSPACE;
  if (ws && ws_nbytes < precompute_ws_bytes(dtype, d_out, d, k)) return GSI_ERR_WORKSPACE;
  if ((rc = gsi_device_check()) != GSI_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  gsi_layer* L = new (std::nothrow) gsi_layer;
  if (!L) return GSI_ERR_NULL;
  void* Vt = (char*)aux + aux_vt_off(dtype, d, k);
  float* Dl = (float*)((char*)aux + aux_dl_off(dtype, d, k));
  L->plan = (PlanRow*)((char*)aux + aux_plan_off(dtype, d, k));
  L->dtype = dtype;
  L->d_out = d_out;
  L->d = d;
  L->k = k;
  L->desc.Vt = Vt;
  L->desc.M = M;
  L->desc.Dl = Dl;
  L->desc.W = W;
  L->desc.VDt = has_vdt(dtype, k) ? (char*)aux + aux_vdt_off(dtype, d, k) : nullptr;
  L->desc.d = d;
  L->desc.d_out = d_out;
  L->desc.k = k;
  L->desc.mode = kSiteGated;
  L->desc.x_off = 0;
  L->desc.y_off = 0;
  if ((rc = layer_grid(L)) != GSI_OK) {
    delete L;
    return rc;
  }
  // V^T (k x d) and the decode plan, then M = W V = W (V^T)^T and V^T V - I   [GSI §2.1]; for the
  // batched gate also (V (V^T V - I))^T = (V^T V - I) V^T, row j of it = sum_l D[j][l] V[:, l]
  const void* dd = nullptr;
  if ((rc = launch_transpose(dtype, V, Vt, d, k, L->desc, L->P, L->plan, s)) != GSI_OK ||
      (rc = launch_precompute(dtype, W, Vt, M, Dl, d_out, d, k, ws, ws ? ws_nbytes : 0, &dd, s)) != GSI_OK ||
      (L->desc.VDt && (rc = launch_vdt(dtype, Dl, dd, V, (void*)L->desc.VDt, d, k, s)) != GSI_OK)) {
    delete L;
    return rc;
  }
  *out = L;
  return GSI_OK;
}

int gsi_layer_create_dense(gsi_layer** out, int dtype, int d_out, int d, const void* W, void* aux, size_t aux_nbytes,
                           void* stream) {
  if (!out) return GSI_ERR_NULL;
  *out = nullptr;
  int rc = check_dense_shape(dtype, d_out, d);
  if (rc != GSI_OK) return rc;
  if (!W || !aux) return GSI_ERR_NULL;
  if (!aligned16(W) || !aligned16(aux)) return GSI_ERR_ALIGN;
  if (aux_nbytes < aux_bytes(dtype, d, 0)) return GSI_ERR_WORKSPACE;
  if ((rc = gsi_device_check()) != GSI_OK) return rc;
  gsi_layer* L = new (std::nothrow) gsi_layer;
  if (!L) return GSI_ERR_NULL;
  L->plan = (PlanRow*)((char*)aux + aux_plan_off(dtype, d, 0));
  L->dtype = dtype;
  L->d_out = d_out;
  L->d = d;
  L->k = 0;
  L->desc.Vt = nullptr;
  L->desc.M = nullptr;
  L->desc.Dl = nullptr;
  L->desc.W = W;
  L->desc.VDt = nullptr;
  L->desc.d = d;
  L->desc.d_out = d_out;
  L->desc.k = 0;
  L->desc.mode = kSiteDense;
  L->desc.x_off = 0;
  L->desc.y_off = 0;
  if ((rc = layer_grid(L)) != GSI_OK ||
      (rc = launch_plan(L->desc, L->P, (int)dtype_size(dtype), L->plan, (hipStream_t)stream)) != GSI_OK) {
    delete L;
    return rc;
  }
  *out = L;
  return GSI_OK;
}

int gsi_layer_destroy(gsi_layer* L) {
  delete L;
  return GSI_OK;
}

size_t gsi_workspace_bytes(int dtype, int d_out, int d, int k, int T_max) {
  if (T_max < 0) return 0;
  if (k == 0 ? check_dense_shape(dtype, d_out, d) != GSI_OK : check_shape(dtype, d_out, d, k) != GSI_OK) return 0;
  return ws_bytes_for(k, d_out, T_max);
}

int gsi_forward(const gsi_layer* L, const void* x, int T, float eps, void* y, uint8_t* gate, float* rho, void* ws,
                size_t ws_nbytes, void* stream) {
  if (!L) return GSI_ERR_NULL;
  if (T < 0) return GSI_ERR_SHAPE;
  int rc = check_eps(eps);
  if (rc != GSI_OK) return rc;
  if (T == 0) return GSI_OK;
  if (!x || !y || !gate || !ws) return GSI_ERR_NULL;
  if (!aligned16(x) || !aligned16(ws)) return GSI_ERR_ALIGN;
  if (ws_nbytes < ws_bytes_for(L->k, L->d_out, T)) return GSI_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (T < 16) {
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.plan = L->plan;
    a.n_sites = 1;
    a.n_steps = 1;
    a.t_step = T;
    a.X = x;
    a.x_ld = L->d;
    a.Y = y;
    a.y_ld = L->d_out;
    a.gates = gate;
    a.rho = rho;
    a.gate_ld = 1;
    a.eps = eps;
    a.ws = ws;
    a.P = L->P;
    a.xr = L->xr;
    return launch_decode(L->dtype, a, s);
  }
  const BatchedWs w = batched_part(ws, L->k, T, L->d_out);
  BatchedPipe pipe(L->dtype, w, s);
  rc = run_batched(L->dtype, L->desc, x, L->d, T, eps, y, L->d_out, gate, 1, rho, w, pipe, s);
  return rc != GSI_OK ? rc : pipe.flush();
}

int gsi_stack_create_modes(gsi_stack** out, gsi_layer* const* sites, const int* modes, int n_sites) {
  if (!out) return GSI_ERR_NULL;
  *out = nullptr;
  if (!sites) return GSI_ERR_NULL;
  if (n_sites < 1) return GSI_ERR_SHAPE;
  for (int i = 0; i < n_sites; ++i) {
    if (!sites[i]) return GSI_ERR_NULL;
    if (sites[i]->dtype != sites[0]->dtype) return GSI_ERR_DTYPE;
    if (modes) {
      const int m = modes[i];
      if (m != GSI_SITE_GATED && m != GSI_SITE_STATIC && m != GSI_SITE_DENSE) return GSI_ERR_SHAPE;
      if (sites[i]->k == 0 && m != GSI_SITE_DENSE) return GSI_ERR_SHAPE;  // a dense layer has no basis
    }
  }
  LayerDesc* table = (LayerDesc*)std::malloc(sizeof(LayerDesc) * n_sites);
  gsi_layer** layers = (gsi_layer**)std::malloc(sizeof(gsi_layer*) * n_sites);
  gsi_stack* S = new (std::nothrow) gsi_stack;
  if (!table || !layers || !S) {
    std::free(table);
    std::free(layers);
    delete S;
    return GSI_ERR_NULL;
  }
  long long xo = 0, yo = 0;
  int kmax = 0, dmax = 0, domax = 0;
  for (int i = 0; i < n_sites; ++i) {
    table[i] = sites[i]->desc;
    if (modes) table[i].mode = modes[i];
    table[i].x_off = xo;
    table[i].y_off = yo;
    xo += sites[i]->d;
    yo += sites[i]->d_out;
    kmax = sites[i]->k > kmax ? sites[i]->k : kmax;
    dmax = sites[i]->d > dmax ? sites[i]->d : dmax;
    domax = sites[i]->d_out > domax ? sites[i]->d_out : domax;
    layers[i] = sites[i];
  }
  S->dtype = sites[0]->dtype;
  S->n_sites = n_sites;
  S->k_max = kmax;
  S->d_max = dmax;
  S->d_out_max = domax;
  S->x_ld = xo;
  S->y_ld = yo;
  S->layers = layers;
  S->h_table = table;
  S->d_plan = nullptr;
  // plan rows hold element offsets into stacked rows as 32-bit integers
  if (xo >= (1ll << 31) || yo >= (1ll << 31)) {
    std::free(table);
    std::free(layers);
    delete S;
    return GSI_ERR_SHAPE;
  }
  S->xr = decode_window(S->dtype, table, n_sites);
  S->P = cached_decode_grid(S->dtype, S->xr);
  auto fail = [&](int code) {
    if (S->d_plan) (void)hipFree(S->d_plan);
    std::free(table);
    std::free(layers);
    delete S;
    return code;
  };
  if (S->P == 0) return fail(GSI_ERR_DEVICE);
  // plan rows of every (site, block), made on the host by the same code the kernels use
  const size_t plan_bytes = sizeof(PlanRow) * (size_t)n_sites * S->P;
  PlanRow* h_plan = (PlanRow*)std::malloc(plan_bytes);
  if (!h_plan) return fail(GSI_ERR_NULL);
  const int es = (int)dtype_size(S->dtype);
  for (int i = 0; i < n_sites; ++i)
    for (int b = 0; b < S->P; ++b) h_plan[(size_t)i * S->P + b] = make_plan_row(table[i], b, S->P, es);
  hipError_t e = hipMalloc((void**)&S->d_plan, plan_bytes);
  if (e == hipSuccess) e = hipMemcpy(S->d_plan, h_plan, plan_bytes, hipMemcpyHostToDevice);
  std::free(h_plan);
  if (e != hipSuccess) return fail(GSI_ERR_HIP);
  *out = S;
  return GSI_OK;
}

int gsi_stack_create(gsi_stack** out, gsi_layer* const* sites, int n_sites) {
  return gsi_stack_create_modes(out, sites, nullptr, n_sites);
}

int gsi_stack_destroy(gsi_stack* S) {
  if (!S) return GSI_OK;
  int rc = GSI_OK;
  if (S->d_plan && hipFree(S->d_plan) != hipSuccess) rc = GSI_ERR_HIP;
  std::free(S->layers);
  std::free(S->h_table);
  delete S;
  return rc;
}

size_t gsi_stack_workspace_bytes(const gsi_stack* S, int T_step) {
  if (!S || T_step < 1) return 0;
  return ws_bytes_for(S->k_max, S->d_out_max, T_step);
}

int gsi_stack_decode(gsi_stack* S, const void* X, int n_steps, int T_step, float eps, void* Y, uint8_t* gates,
                     float* rho, void* ws, size_t ws_nbytes, void* stream) {
  if (!S) return GSI_ERR_NULL;
  if (n_steps < 0 || T_step < 1) return GSI_ERR_SHAPE;
  int rc = check_eps(eps);
  if (rc != GSI_OK) return rc;
  if (n_steps == 0) return GSI_OK;
  if (!X || !Y || !gates || !ws) return GSI_ERR_NULL;
  if (!aligned16(X) || !aligned16(ws)) return GSI_ERR_ALIGN;
  if (ws_nbytes < ws_bytes_for(S->k_max, S->d_out_max, T_step)) return GSI_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (T_step < 16) {
    if ((long long)n_steps * T_step * S->n_sites >= kMaxStepsPerLaunch) return GSI_ERR_SHAPE;
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.plan = S->d_plan;
    a.n_sites = S->n_sites;
    a.n_steps = n_steps;
    a.t_step = T_step;
    a.X = X;
    a.x_ld = S->x_ld;
    a.Y = Y;
    a.y_ld = S->y_ld;
    a.gates = gates;
    a.rho = rho;
    a.gate_ld = S->n_sites;
    a.eps = eps;
    a.ws = ws;
    a.P = S->P;
    a.xr = S->xr;
    return launch_decode(S->dtype, a, s);
  }
  const size_t es = dtype_size(S->dtype);
  // one carving of the workspace for every site (k_max, d_out_max): units of different sites are
  // in flight together
  const BatchedWs w = batched_part(ws, S->k_max, T_step, S->d_out_max);
  BatchedPipe pipe(S->dtype, w, s);
  for (int st = 0; st < n_steps; ++st) {
    const long long row0 = (long long)st * T_step;
    for (int i = 0; i < S->n_sites; ++i) {
      const LayerDesc& L = S->h_table[i];
      const char* xs = (const char*)X + (size_t)(row0 * S->x_ld + L.x_off) * es;
      char* ys = (char*)Y + (size_t)(row0 * S->y_ld + L.y_off) * es;
      uint8_t* gs = gates + row0 * S->n_sites + i;
      float* rs = rho ? rho + row0 * S->n_sites + i : nullptr;
      rc = run_batched(S->dtype, L, xs, S->x_ld, T_step, eps, ys, S->y_ld, gs, S->n_sites, rs, w, pipe, s);
      if (rc != GSI_OK) return rc;
    }
  }
  return pipe.flush();
}

int gsi_workspace_status(void* ws, size_t ws_nbytes, int* host_status, void* stream) {
  if (!ws || !host_status) return GSI_ERR_NULL;
  if (ws_nbytes < sizeof(WsHeader)) return GSI_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int rc = hip_rc(hipStreamSynchronize(s));
  if (rc != GSI_OK) return rc;
  int v = 0;
  rc = hip_rc(hipMemcpy(&v, &ws_header(ws)->status, sizeof(int), hipMemcpyDeviceToHost));
  if (rc != GSI_OK) return rc;
  *host_status = v;
  int zero = 0;
  return hip_rc(hipMemcpy(&ws_header(ws)->status, &zero, sizeof(int), hipMemcpyHostToDevice));
}

// ---- one decode-step block: GSI sites around an unchanged plain attention ----

// A: [QKV, fc_in] (d -> 3 d, d -> dff), or one shared-input site d -> 3 d + dff (QKV and fc_in
// stacked: one basis, one g, one gate); B: [out, fc_out] (d -> d, dff -> d)
static bool block_shapes(const gsi_stack* A, const gsi_stack* B, int n_heads, int* d_out, int* dff_out) {
  if ((A->n_sites != 1 && A->n_sites != 2) || B->n_sites != 2) return false;
  const LayerDesc &q = A->h_table[0], &o = B->h_table[0], &m = B->h_table[1];
  const int d = q.d, dff = m.d;
  if (d < 64 || d > 16384 || n_heads < 1 || d % n_heads != 0 || dff < 1) return false;
  const int dh = d / n_heads;
  if (dh != 64 && dh != 128 && dh != 256) return false;
  if (A->n_sites == 2) {
    const LayerDesc& f = A->h_table[1];
    if (q.d_out != 3 * d || f.d != d || f.d_out != dff) return false;
  } else if ((long long)q.d_out != 3LL * d + dff) {
    return false;
  }
  if (o.d != d || o.d_out != d || m.d_out != d) return false;
  *d_out = d;
  *dff_out = dff;
  return true;
}

// one token through a stack on the batch-1 kernel, launched as an ordinary launch (arguments
// already checked by the caller)
static int stack_one_token(gsi_stack* S, const void* X, float eps, void* Y, uint8_t* gates, float* rho, void* ws,
                           hipStream_t s) {
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.plan = S->d_plan;
  a.n_sites = S->n_sites;
  a.n_steps = 1;
  a.t_step = 1;
  a.X = X;
  a.x_ld = S->x_ld;
  a.Y = Y;
  a.y_ld = S->y_ld;
  a.gates = gates;
  a.rho = rho;
  a.gate_ld = S->n_sites;
  a.eps = eps;
  a.ws = ws;
  a.P = S->P;
  a.xr = S->xr;
  return launch_decode_resident(S->dtype, a, s);
}

size_t gsi_block_step_workspace_bytes(const gsi_stack* A, const gsi_stack* B, int n_heads) {
  int d = 0, dff = 0;
  if (!A || !B || !block_shapes(A, B, n_heads, &d, &dff)) return 0;
  const size_t st = std::max(ws_bytes_for(A->k_max, A->d_out_max, 1), ws_bytes_for(B->k_max, B->d_out_max, 1));
  return align256(st) + align256(attn_ws_bytes(d, n_heads));
}

// checks of one block's arguments (nothing enqueued); d and dff of the block on success
static int block_check(gsi_stack* A, gsi_stack* B, const void* gamma, const void* beta, void* x, void* k_cache,
                       void* v_cache, int pos, int n_heads, float eps, void* xa, void* ya, void* xb, void* yb,
                       uint8_t* gates, void* ws, size_t ws_bytes, int* d, int* dff) {
  if (!A || !B || !gamma || !beta || !x || !k_cache || !v_cache || !xa || !ya || !xb || !yb || !gates || !ws)
    return GSI_ERR_NULL;
  if (A->dtype != B->dtype || (A->dtype != GSI_BF16 && A->dtype != GSI_F16)) return GSI_ERR_DTYPE;
  if (!block_shapes(A, B, n_heads, d, dff) || pos < 0 || pos >= (1 << 24)) return GSI_ERR_SHAPE;
  int rc = check_eps(eps);
  if (rc != GSI_OK) return rc;
  for (const void* p : {gamma, beta, (const void*)x, (const void*)k_cache, (const void*)v_cache, (const void*)xa,
                        (const void*)ya, (const void*)xb, (const void*)yb, (const void*)ws})
    if (!aligned16(p)) return GSI_ERR_ALIGN;
  if (ws_bytes < gsi_block_step_workspace_bytes(A, B, n_heads)) return GSI_ERR_WORKSPACE;
  return GSI_OK;
}

// enqueue one checked block. ln_done: xa already holds this block's LayerNorm (the previous
// block's residual launch formed it); next_gamma / next_beta (optional): the residual launch also
// forms the next block's LayerNorm into xa.
static int block_enqueue(gsi_stack* A, gsi_stack* B, const void* gamma, const void* beta, void* x, void* k_cache,
                         void* v_cache, int pos, int n_heads, float eps, void* xa, void* ya, void* xb, void* yb,
                         uint8_t* gates, float* rho, void* ws, int d, int dff, hipStream_t s, bool ln_done = false,
                         const void* next_gamma = nullptr, const void* next_beta = nullptr,
                         const int* pos_dev = nullptr, int cap = 0) {
  const size_t st = align256(std::max(ws_bytes_for(A->k_max, A->d_out_max, 1), ws_bytes_for(B->k_max, B->d_out_max, 1)));
  float* part = (float*)((char*)ws + st);
  int rc = ln_done ? GSI_OK : launch_ln_dup(A->dtype, x, gamma, beta, d, xa, s);
  if (rc != GSI_OK) return rc;
  rc = stack_one_token(A, xa, eps, ya, gates, rho, ws, s);
  if (rc != GSI_OK) return rc;
  // a shared-input stack A decides one gate for QKV and fc_in: the attention launch repeats it
  const bool shared = A->n_sites == 1;
  rc = launch_attention_gelu(A->dtype, ya, k_cache, v_cache, pos, d, n_heads, dff, xb, part,
                             shared ? gates : nullptr, shared ? rho : nullptr, pos_dev, cap, s);
  if (rc != GSI_OK) return rc;
  rc = stack_one_token(B, xb, eps, yb, gates + 2, rho ? rho + 2 : nullptr, ws, s);
  if (rc != GSI_OK) return rc;
  return next_gamma ? launch_residual_ln(A->dtype, x, yb, next_gamma, next_beta, d, xa, s)
                    : launch_residual(A->dtype, x, yb, d, s);
}

int gsi_block_step(gsi_stack* A, gsi_stack* B, const void* gamma, const void* beta, void* x, void* k_cache,
                   void* v_cache, int pos, int n_heads, float eps, void* xa, void* ya, void* xb, void* yb,
                   uint8_t* gates, float* rho, void* ws, size_t ws_bytes, void* stream) {
  int d = 0, dff = 0;
  const int rc = block_check(A, B, gamma, beta, x, k_cache, v_cache, pos, n_heads, eps, xa, ya, xb, yb, gates, ws,
                             ws_bytes, &d, &dff);
  if (rc != GSI_OK) return rc;
  return block_enqueue(A, B, gamma, beta, x, k_cache, v_cache, pos, n_heads, eps, xa, ya, xb, yb, gates, rho, ws, d,
                       dff, (hipStream_t)stream);
}

// the step at host position pos, or (pos_dev) at the device position *pos_dev, advanced afterwards
static int decode_step_impl(int n_blocks, gsi_stack* const* A, gsi_stack* const* B, const void* const* gamma,
                            const void* const* beta, void* const* k_cache, void* const* v_cache, int pos, int* pos_dev,
                            int cap, int n_heads, float eps, void* x, void* xa, void* ya, void* xb, void* yb,
                            uint8_t* gates, float* rho, void* ws, size_t ws_bytes, void* stream) {
  if (n_blocks < 1) return GSI_ERR_SHAPE;
  if (!A || !B || !gamma || !beta || !k_cache || !v_cache) return GSI_ERR_NULL;
  int d0 = 0, dff0 = 0;
  for (int b = 0; b < n_blocks; ++b) {  // every block checked before anything is enqueued
    int d = 0, dff = 0;
    const int rc = block_check(A[b], B[b], gamma[b], beta[b], x, k_cache[b], v_cache[b], pos, n_heads, eps, xa, ya,
                               xb, yb, gates, ws, ws_bytes, &d, &dff);
    if (rc != GSI_OK) return rc;
    if (b == 0) {
      d0 = d;
      dff0 = dff;
    } else if (d != d0 || dff != dff0 || A[b]->dtype != A[0]->dtype) {
      return GSI_ERR_SHAPE;
    }
  }
  hipStream_t s = (hipStream_t)stream;
  for (int b = 0; b < n_blocks; ++b) {
    // each block's residual add also forms the next block's LayerNorm (one launch fewer per block)
    const bool more = b + 1 < n_blocks;
    const int rc = block_enqueue(A[b], B[b], gamma[b], beta[b], x, k_cache[b], v_cache[b], pos, n_heads, eps, xa, ya,
                                 xb, yb, gates + 4 * b, rho ? rho + 4 * b : nullptr, ws, d0, dff0, s, b > 0,
                                 more ? gamma[b + 1] : nullptr, more ? beta[b + 1] : nullptr, pos_dev, cap);
    if (rc != GSI_OK) return rc;
  }
  return pos_dev ? launch_pos_advance(pos_dev, s) : GSI_OK;
}

int gsi_decode_step(int n_blocks, gsi_stack* const* A, gsi_stack* const* B, const void* const* gamma,
                    const void* const* beta, void* const* k_cache, void* const* v_cache, int pos, int n_heads,
                    float eps, void* x, void* xa, void* ya, void* xb, void* yb, uint8_t* gates, float* rho, void* ws,
                    size_t ws_bytes, void* stream) {
  return decode_step_impl(n_blocks, A, B, gamma, beta, k_cache, v_cache, pos, nullptr, 0, n_heads, eps, x, xa, ya, xb,
                          yb, gates, rho, ws, ws_bytes, stream);
}

int gsi_decode_step_devpos(int n_blocks, gsi_stack* const* A, gsi_stack* const* B, const void* const* gamma,
                           const void* const* beta, void* const* k_cache, void* const* v_cache, int* pos,
                           int cache_rows, int n_heads, float eps, void* x, void* xa, void* ya, void* xb, void* yb,
                           uint8_t* gates, float* rho, void* ws, size_t ws_bytes, void* stream) {
  if (!pos) return GSI_ERR_NULL;
  if (cache_rows < 1 || cache_rows > (1 << 24) || ((uintptr_t)pos & 3)) return GSI_ERR_SHAPE;
  // the block checks see position 0; the kernels bound the device position by cache_rows
  return decode_step_impl(n_blocks, A, B, gamma, beta, k_cache, v_cache, 0, pos, cache_rows, n_heads, eps, x, xa, ya,
                          xb, yb, gates, rho, ws, ws_bytes, stream);
}

}  // extern "C"
