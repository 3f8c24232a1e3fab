// Host-side sanitizer run of the C ABI's argument validation: the library's host code is built
// with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_abi_sanitize.py) and every
// entry point is called with invalid arguments on a machine without a usable GPU. Each call must
// return its documented status without touching device memory; the sanitizers report any invalid
// host memory access or undefined behaviour on the way. Prints one line per failure.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "../include/gsi.h"

static int failures = 0;
#define EXPECT(call, want)                                                                        \
  do {                                                                                            \
    const long long got_ = (long long)(call);                                                     \
    if (got_ != (long long)(want)) {                                                              \
      std::printf("FAIL line %d: %s returned %lld, expected %lld\n", __LINE__, #call, got_,        \
                  (long long)(want));                                                             \
      ++failures;                                                                                 \
    }                                                                                             \
  } while (0)

int main() {
  const float nan = std::numeric_limits<float>::quiet_NaN();
  alignas(16) static unsigned char buf[4096];
  void* p = buf;
  // status strings: every code and an unknown one
  for (int c = -12; c <= 2; ++c) {
    const char* s = gsi_status_string(c);
    if (!s || !s[0]) {
      std::printf("FAIL: empty status string for %d\n", c);
      ++failures;
    }
  }
  // size queries: invalid shapes and dtypes give 0
  EXPECT(gsi_layer_aux_bytes(GSI_BF16, 0, 64, 16), 0);
  EXPECT(gsi_layer_aux_bytes(GSI_BF16, 64, 0, 16), 0);
  EXPECT(gsi_layer_aux_bytes(GSI_BF16, 64, 64, -8), 0);
  EXPECT(gsi_layer_aux_bytes(GSI_BF16, 64, 64, 4096), 0);
  EXPECT(gsi_layer_aux_bytes(99, 64, 64, 16), 0);
  EXPECT(gsi_layer_aux_bytes(GSI_BF16, 64, 60, 16), 0);  // d not a multiple of 8
  EXPECT(gsi_layer_create_workspace_bytes(-1, 64, 64, 16), 0);
  EXPECT(gsi_workspace_bytes(99, 64, 64, 16, 16), 0);
  EXPECT(gsi_stack_workspace_bytes(nullptr, 1), 0);
  EXPECT(gsi_calibrate_workspace_bytes(0, 64, 16), 0);
  // creation: NULL handles, shapes, alignment
  gsi_layer* L = reinterpret_cast<gsi_layer*>(0x1);
  EXPECT(gsi_layer_create(nullptr, GSI_BF16, 64, 64, 16, p, p, p, p, sizeof(buf), nullptr, 0, nullptr), GSI_ERR_NULL);
  EXPECT(gsi_layer_create(&L, GSI_BF16, 64, 64, 16, nullptr, p, p, p, sizeof(buf), nullptr, 0, nullptr), GSI_ERR_NULL);
  EXPECT(L == nullptr, 1);
  EXPECT(gsi_layer_create(&L, GSI_BF16, 64, 64, 16, p, p, p, nullptr, sizeof(buf), nullptr, 0, nullptr), GSI_ERR_NULL);
  EXPECT(gsi_layer_create(&L, GSI_BF16, -64, 64, 16, p, p, p, p, sizeof(buf), nullptr, 0, nullptr), GSI_ERR_SHAPE);
  EXPECT(gsi_layer_create(&L, 7, 64, 64, 16, p, p, p, p, sizeof(buf), nullptr, 0, nullptr), GSI_ERR_DTYPE);
  EXPECT(gsi_layer_create(&L, GSI_BF16, 64, 64, 16, buf + 2, p, p, p, sizeof(buf), nullptr, 0, nullptr), GSI_ERR_ALIGN);
  EXPECT(gsi_layer_create(&L, GSI_BF16, 64, 64, 16, p, p, p, p, 16, nullptr, 0, nullptr), GSI_ERR_WORKSPACE);
  EXPECT(gsi_layer_create_dense(nullptr, GSI_BF16, 64, 64, p, p, sizeof(buf), nullptr), GSI_ERR_NULL);
  EXPECT(gsi_layer_create_dense(&L, GSI_BF16, 64, 64, nullptr, p, sizeof(buf), nullptr), GSI_ERR_NULL);
  EXPECT(gsi_layer_create_dense(&L, GSI_BF16, 0, 64, p, p, sizeof(buf), nullptr), GSI_ERR_SHAPE);
  EXPECT(gsi_layer_create_dense(&L, GSI_BF16, 64, 64, p, p, 8, nullptr), GSI_ERR_WORKSPACE);
  EXPECT(gsi_layer_destroy(nullptr), GSI_OK);
  // forward: NULL layer first, then argument checks that need no device
  EXPECT(gsi_forward(nullptr, p, 4, 0.1f, p, buf, nullptr, p, sizeof(buf), nullptr), GSI_ERR_NULL);
  // stacks
  gsi_stack* S = reinterpret_cast<gsi_stack*>(0x1);
  EXPECT(gsi_stack_create(nullptr, nullptr, 1), GSI_ERR_NULL);
  EXPECT(gsi_stack_create(&S, nullptr, 1), GSI_ERR_NULL);
  EXPECT(S == nullptr, 1);
  gsi_layer* none[2] = {nullptr, nullptr};
  EXPECT(gsi_stack_create(&S, none, 0), GSI_ERR_SHAPE);
  EXPECT(gsi_stack_create(&S, none, 2), GSI_ERR_NULL);
  const int bad_modes[1] = {5};
  EXPECT(gsi_stack_create_modes(&S, none, bad_modes, 1), GSI_ERR_NULL);
  EXPECT(gsi_stack_destroy(nullptr), GSI_OK);
  EXPECT(gsi_stack_decode(nullptr, p, 1, 1, 0.1f, p, buf, nullptr, p, sizeof(buf), nullptr), GSI_ERR_NULL);
  EXPECT(gsi_stack_decode_noalloc(nullptr, p, 1, 1, 0.1f, p, buf, nullptr, nullptr), GSI_ERR_NULL);
  // status read: NULL workspace / output
  int st = 0;
  EXPECT(gsi_workspace_status(nullptr, 0, &st, nullptr), GSI_ERR_NULL);
  EXPECT(gsi_workspace_status(p, sizeof(buf), nullptr, nullptr), GSI_ERR_NULL);
  // decode-step block: NULL stacks or buffers are refused before anything else
  EXPECT(gsi_block_step_workspace_bytes(nullptr, nullptr, 16), 0);
  EXPECT(gsi_block_step(nullptr, nullptr, p, p, p, p, p, 0, 16, 0.1f, p, p, p, p, buf, nullptr, p, sizeof(buf),
                        nullptr), GSI_ERR_NULL);
  gsi_stack* stacks[1] = {nullptr};
  const void* cptr[1] = {p};
  void* vptr[1] = {p};
  EXPECT(gsi_decode_step(0, stacks, stacks, cptr, cptr, vptr, vptr, 0, 16, 0.1f, p, p, p, p, p, buf, nullptr, p,
                         sizeof(buf), nullptr), GSI_ERR_SHAPE);
  EXPECT(gsi_decode_step(1, nullptr, stacks, cptr, cptr, vptr, vptr, 0, 16, 0.1f, p, p, p, p, p, buf, nullptr, p,
                         sizeof(buf), nullptr), GSI_ERR_NULL);
  EXPECT(gsi_decode_step(1, stacks, stacks, cptr, cptr, vptr, vptr, 0, 16, 0.1f, p, p, p, p, p, buf, nullptr, p,
                         sizeof(buf), nullptr), GSI_ERR_NULL);
  // calibration
  EXPECT(gsi_calibrate(0, 64, 16, (const float*)p, (const float*)p, 1, (float*)p, p, sizeof(buf), nullptr), GSI_ERR_SHAPE);
  EXPECT(gsi_calibrate(32, 64, 16, nullptr, (const float*)p, 1, (float*)p, p, sizeof(buf), nullptr), GSI_ERR_NULL);
  (void)nan;
  std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
