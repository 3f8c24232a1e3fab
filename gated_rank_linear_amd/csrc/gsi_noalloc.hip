// gsi_stack_decode_noalloc: the batch-1 stack decode for callers that cannot allocate device
// memory (code under stream capture, serving loops, harnesses that forbid allocation). The only
// device memory the batch-1 kernel needs beyond its inputs and outputs is its exchange state
// (workspace header and mailboxes, decode_ws_bytes() = 65,792 bytes); here it lives in a
// file-scope device array, one copy per GPU for the life of the process.
#include <cmath>
#include <mutex>

#include "gsi_internal.h"

namespace {

constexpr size_t kScratchBytes = 65792;  // header + g / gate-piece / completion mailboxes
constexpr int kMaxDevices = 64;

// Zero at load: the exchange protocol needs zeros only before its first use; afterwards every
// launch keeps the array consistent (its 64-bit epoch advances, stale words never match a tag).
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` per device, looked up once with that device current. In host code
// the array's name is only a stand-in for the symbol; kernels get the looked-up address.
void* g_scratch[kMaxDevices];
std::once_flag g_once[kMaxDevices];
int g_rc[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GSI_ERR_DEVICE;
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = e == hipSuccess ? p : nullptr;
    g_rc[dev] = e == hipSuccess && p ? GSI_OK : GSI_ERR_HIP;
  });
  *out = g_scratch[dev];
  return g_rc[dev];
}

}  // namespace

extern "C" int gsi_stack_decode_noalloc(gsi_stack* S, const void* X, int n_steps, int T_step, float eps, void* Y,
                                        uint8_t* gates, float* rho, void* stream) {
  static_assert(kScratchBytes >= 256 + (size_t)gsi::kReplicas * gsi::kMaxK * 8 +
                                      2 * (size_t)gsi::kReplicas * gsi::kMaxBlocks * 8,
                "scratch holds the workspace header and the three mailboxes");
  if (!S) return GSI_ERR_NULL;
  if (n_steps < 0 || T_step < 1) return GSI_ERR_SHAPE;
  if (std::isnan(eps) || eps < 0.f) return GSI_ERR_EPS;
  // the batched path (T_step >= 16) needs split-product scratch that grows with T_step and
  // d_out; only the per-token path fits the fixed array
  if (T_step >= 16) return GSI_ERR_WORKSPACE;
  if (gsi::decode_ws_bytes() > kScratchBytes) return GSI_ERR_WORKSPACE;
  if (n_steps == 0) return GSI_OK;
  if (!X || !Y || !gates) return GSI_ERR_NULL;
  if (((uintptr_t)X & 15u) != 0) return GSI_ERR_ALIGN;
  if ((long long)n_steps * T_step * S->n_sites >= gsi::kMaxStepsPerLaunch) return GSI_ERR_SHAPE;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != GSI_OK) return rc;
  gsi::DecodeArgs a;
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
  return gsi::launch_decode(S->dtype, a, (hipStream_t)stream);
}
