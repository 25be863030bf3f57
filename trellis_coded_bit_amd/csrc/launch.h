// Internal launchers behind the C ABI (see include/trellis.h for the public contract).
// Arguments here are already validated by api.cpp.
#pragma once
#include <hip/hip_runtime_api.h>
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

// Every workspace starts with the same reserved region, so that one zero-filled buffer can
// serve every entry point in any order:
//   [0, 256)                 header; word 0 is the error word (sticky: kernels only OR bits
//                            into it, the caller clears it); the other words are unused
//   [256, 256 + 64 KiB)      the small-batch products' column-block counters: zero between
//                            calls (each call's finishing workgroups reset the ones it used);
//                            no other entry point writes them
//   [kWsReserved, ...)       the entry point's own scratch
constexpr size_t kWsHeaderBytes = 256;
constexpr int kMaxFinishGroups = 16384;
constexpr size_t kWsCounterBytes = (size_t)kMaxFinishGroups * 4;
constexpr size_t kWsReserved = kWsHeaderBytes + kWsCounterBytes;
// Error-word bits.
constexpr uint32_t kErrBadEntry = 1u;    // a routed id out of range or a table entry with bad K / cb
constexpr uint32_t kErrWaitExpired = 2u; // a bounded wait for another workgroup ran out (prefill)

// How the small-batch products finish a column block.
enum GemvFinish {
  kFinishPlain = 0,     // y[p] = had(y_pre[p]) * sv_p for every problem p
  kFinishSwiGLU = 1,    // problems in slots of 2H (H gate entries, then H up entries):
                        // y[slot][h-th slice] = silu(gate_h) * up_h   (B = 1)
  kFinishWeighted = 2,  // y = had(sum_p w[p] * y_pre[p]) * sv, sv shared   (B = 1)
};

// One layer of a list-mode launch: its descriptor and its own input and output.
constexpr int kMaxList = 8;
struct GemvItem {
  trellis_linear L;
  const uint16_t *x;  // fp16 [B][L.in_features]
  uint16_t *y;        // fp16 [B][L.out_features]
};

// One product problem list, in one of two modes:
//   list mode  (table == NULL): n_list layers of any shapes, each with its own x and y;
//   table mode (table != NULL): the routed entries of a device table, all [in, out]; with
//     `group` entries per expert, problem p uses entry routed[p / group] * group + p % group.
struct GemvLaunch {
  int n_list;
  GemvItem list[kMaxList];
  const trellis_linear *table;   // device table [E * group] or NULL
  int E;                         // experts (valid routed ids are 0..E-1)
  int group;                     // table entries per expert (>= 1)
  const int32_t *routed;         // device [n_problems / group] (table mode)
  int n_problems;                // table mode
  int in_features, out_features; // table mode
  int B;
  const uint16_t *x;             // table mode
  int x_per_problem;
  uint16_t *y;                   // table mode
  const uint16_t *shared_r;
  const float *shared_s;
  int shared_side;
  int finish;                    // GemvFinish (table mode; list mode is always plain)
  int halves;                    // kFinishSwiGLU: H
  const float *router_w;         // kFinishWeighted: device f32 [n_problems]
};

// Workspace bytes of a launch (including the reserved region); 0 if it is not supported
// (more column blocks than the counter region holds, or too many units).
size_t gemv_workspace_bytes(const GemvLaunch &a);
// The same for a table-mode launch of n_problems [in, out] problems at batch B.
size_t gemv_workspace_bytes(int n_problems, int in_features, int out_features, int B);
// The launch: one kernel (plus nothing else), or a zero fill for an empty weighted sum.
hipError_t launch_gemv(const GemvLaunch &a, void *ws, size_t ws_bytes, hipStream_t stream);
// The library-held scratch of the allocation-free entry point (the current device's copy).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void **ptr);

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

// Microbenchmarks (include/trellis_micro.h).
int micro_cus();
hipError_t launch_micro_stream_read(const void *buf, size_t bytes, int blocks, uint32_t *sink, hipStream_t stream);
hipError_t launch_micro_valu(int op, int iters, int waves_per_simd, uint64_t *cycles, uint64_t *ticks, uint32_t *sink,
                             hipStream_t stream, int *blocks_out);
hipError_t launch_micro_mfma(int kind, int iters, int waves_per_simd, uint64_t *cycles, uint64_t *ticks, float *sink,
                             hipStream_t stream, int *blocks_out);

}  // namespace trellis
