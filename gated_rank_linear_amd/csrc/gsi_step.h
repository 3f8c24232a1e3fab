// Kernels around the GSI sites in one batch-1 decode step of a GPT-J-shaped parallel block
// (LayerNorm, plain attention, GELU, residual add); declarations shared with gsi_api.cpp.
#pragma once

#include "gsi_internal.h"

namespace gsi {

constexpr int kMaxAttnSplit = 64;  // position chunks of one head's attention
constexpr float kLnEps = 1e-5f;

// position chunks of the attention over L positions with n_heads heads
int attn_splits(int L, int n_heads);
// scratch of the attention: per (head, chunk) its max, sum and dh float32 values, then one
// arrival counter per head (zero before the first launch; each launch leaves them zero)
size_t attn_ws_bytes(int d, int n_heads);

// xa[0:d] = xa[d:2d] = LayerNorm(x) (unit row, float32 statistics, rounded to the dtype); d a
// multiple of 4, at most 16384
int launch_ln_dup(int dtype, const void* x, const void* gamma, const void* beta, int d, void* xa, hipStream_t s);
// attention of the query q = ya[0:d] over cache rows 0 .. pos - 1 and the new k, v = ya[d:2d],
// ya[2d:3d] (row pos of the caches is written with them); o to xb[0:d]; u = gelu(ya[3d:3d+dff]) to
// xb[d:d+dff]; with gate_dup (and rho_dup), entry 0 is also copied to entry 1 (the gate of a
// shared-input site reported for both of its maps); with pos_dev the position is read from device
// memory when the launch runs (pos is then unused) and must lie in [0, cap) for the attention to run
int launch_attention_gelu(int dtype, const void* ya, void* k_cache, void* v_cache, int pos, int d, int n_heads,
                          int dff, void* xb, float* part, uint8_t* gate_dup, float* rho_dup, const int* pos_dev,
                          int cap, hipStream_t s);
// *pos += 1 (one thread)
int launch_pos_advance(int* pos, hipStream_t s);
// x += yb[0:d] + yb[d:2d]
int launch_residual(int dtype, void* x, const void* yb, int d, hipStream_t s);
// x += yb[0:d] + yb[d:2d], then xa = [a | a] with a = LayerNorm(x) for the next block (the values
// of launch_residual followed by launch_ln_dup)
int launch_residual_ln(int dtype, void* x, const void* yb, const void* gamma, const void* beta, int d, void* xa,
                       hipStream_t s);

}  // namespace gsi
