// Internal launchers behind the C ABI (see include/trellis.h for the public contract).
// Arguments here are already validated by api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/trellis.h"

namespace trellis {

hipError_t launch_decode_tiles(const int16_t *code, int K, int in_features, int out_features,
                               uint16_t *w_hat, uint16_t *states, hipStream_t stream);

hipError_t launch_decode_tiles_e4m3(const int16_t *code, int K, int in_features, int out_features, uint8_t *w8,
                                    hipStream_t stream);

// y = had(x*r*s)*norm (post = 0) or had(x)*r*s*norm (post = 1) on 128-blocks; had() is
// the UNNORMALISED Sylvester butterfly, `norm` the factor applied (1/sqrt(128) for the
// public entry point).
hipError_t launch_had128(const void *x, int x_is_fp32, int rows, int n, const uint16_t *r,
                         const float *s, int post, float norm, void *y, int y_is_fp32,
                         hipStream_t stream);

// How the finishing launch combines the column blocks of a GEMV problem list.
enum GemvFinish {
  kFinishPlain = 0,     // y[p] = had(y_pre[p]) * sv_p for every problem p
  kFinishSwiGLU = 1,    // problems in slots of 2H (H gate entries, then H up entries):
                        // y[slot][h-th slice] = silu(gate_h) * up_h   (B = 1)
  kFinishWeighted = 2,  // y = had(sum_p w[p] * y_pre[p]) * sv, sv shared   (B = 1)
};

// One product problem list: either a single layer (table == NULL) or the routed entries of
// a device table.  With `group` entries per expert, problem p uses table entry
// routed[p / group] * group + p % group.
struct GemvLaunch {
  trellis_linear single;         // used when table == NULL
  const trellis_linear *table;   // device table [E * group] or NULL
  int E;                         // experts (valid routed ids are 0..E-1)
  int group;                     // table entries per expert (>= 1)
  const int32_t *routed;         // device [n_problems / group] (table mode)
  int n_problems;
  int in_features, out_features, B;
  const uint16_t *x;
  int x_per_problem;
  uint16_t *y;
  const uint16_t *shared_r;
  const float *shared_s;
  int shared_side;
  int finish;                    // GemvFinish
  int halves;                    // kFinishSwiGLU: H
  const float *router_w;         // kFinishWeighted: device f32 [n_problems]
};

// Workspace bytes for a GEMV launch with n_problems problems of [in, out] at batch B.
size_t gemv_workspace_bytes(int n_problems, int in_features, int out_features, int B);
// Upper bound on n_problems * out_features / 128 for one GEMV/MoE call.
int gemv_max_column_blocks();
hipError_t launch_gemv(const GemvLaunch &a, void *ws, size_t ws_bytes, hipStream_t stream);

// Routed-expert MLP of one token: gate/up halves (table [E][2H]) -> silu(g)*u -> down
// (table [E]) -> router-weighted sum with one output rotation.
struct MlpLaunch {
  const trellis_linear *gate_up, *down;
  int E, halves, n, hidden, inter;
  const int32_t *routed;
  const float *router_w;
  const uint16_t *x;
  const uint16_t *r_hidden_in, *r_hidden_out;
  const float *s_hidden_in, *s_hidden_out;
  uint16_t *act;  // fp16 [n][inter] or NULL (then held in the workspace)
  uint16_t *y;
};
size_t moe_mlp_workspace_bytes(int hidden, int inter, int halves, int n);

// Tail-biting Viterbi encoder: targets f32 [T][16][16] -> code [T][16K] (+ states).
size_t encode_workspace_bytes(int n_tiles);
hipError_t launch_encode_tiles(const float *targets, int T, int K, int cb, int16_t *code, uint16_t *states,
                               void *ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_moe_mlp(const MlpLaunch &m, void *ws, size_t ws_bytes, hipStream_t stream);

size_t gemm_workspace_bytes(int in_features, int out_features, int M);
hipError_t launch_gemm(const trellis_linear &L, const uint16_t *x, int M, uint16_t *y, void *ws,
                       size_t ws_bytes, hipStream_t stream);

// The FP8 prefill: E4M3 weights (cb = 2) against E4M3 activations with per-row scales.
size_t gemm_fp8_workspace_bytes(int in_features, int out_features, int M);
hipError_t launch_gemm_fp8(const trellis_linear &L, const uint16_t *x, int M, uint16_t *y, void *ws,
                           size_t ws_bytes, hipStream_t stream);

}  // namespace trellis
