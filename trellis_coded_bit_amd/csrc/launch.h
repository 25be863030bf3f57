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

// y = had(x*r*s)*norm (post = 0) or had(x)*r*s*norm (post = 1) on 128-blocks; had() is
// the UNNORMALISED Sylvester butterfly, `norm` the factor applied (1/sqrt(128) for the
// public entry point).
hipError_t launch_had128(const void *x, int x_is_fp32, int rows, int n, const uint16_t *r,
                         const float *s, int post, float norm, void *y, int y_is_fp32,
                         hipStream_t stream);

// One product problem list: either a single layer (table == NULL) or `n` routed entries of
// a device table.
struct GemvLaunch {
  trellis_linear single;         // used when table == NULL
  const trellis_linear *table;   // device table or NULL
  int E;
  const int32_t *routed;         // device [n] (table mode)
  int n_problems;
  int in_features, out_features, B;
  const uint16_t *x;
  int x_per_problem;
  uint16_t *y;
  const uint16_t *shared_r;
  const float *shared_s;
  int shared_side;
};

// Workspace bytes for a GEMV launch with n_problems problems of [in, out] at batch B.
size_t gemv_workspace_bytes(int n_problems, int in_features, int out_features, int B);
// Upper bound on n_problems * out_features / 128 for one GEMV/MoE call.
int gemv_max_column_blocks();
hipError_t launch_gemv(const GemvLaunch &a, void *ws, size_t ws_bytes, hipStream_t stream);

size_t gemm_workspace_bytes(int in_features, int out_features, int M);
hipError_t launch_gemm(const trellis_linear &L, const uint16_t *x, int M, uint16_t *y, void *ws,
                       size_t ws_bytes, hipStream_t stream);

}  // namespace trellis
