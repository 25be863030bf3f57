// C ABI of libtrellis.so: argument validation, error reporting and dispatch to the gfx950
// launchers.  The contract (meaning, layout, ownership, errors) is in include/trellis.h.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/trellis.h"
#include "../../include/trellis_micro.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return TRELLIS_OK;
  return fail(TRELLIS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_linear(const trellis_linear *L, int need_side_vectors) {
  if (!L) return fail(TRELLIS_EINVAL, "layer descriptor is NULL");
  if (L->K < 2 || L->K > 4) return fail(TRELLIS_EINVAL, "K=%d not in {2,3,4}", L->K);
  if (L->cb != 1 && L->cb != 2)
    return fail(TRELLIS_EINVAL, "cb=%d: 1 (MCG codebook) or 2 (MCG rounded to E4M3) expected", L->cb);
  if (L->in_features <= 0 || L->out_features <= 0 || L->in_features % 128 || L->out_features % 128)
    return fail(TRELLIS_EINVAL, "in=%d out=%d must be positive multiples of 128", L->in_features,
                L->out_features);
  if (!L->code) return fail(TRELLIS_EINVAL, "code is NULL");
  if (!aligned(L->code, 16)) return fail(TRELLIS_EALIGN, "code must be 16-byte aligned");
  if (need_side_vectors && (!L->rin || !L->rout)) return fail(TRELLIS_EINVAL, "rin/rout is NULL");
  if ((L->rin && !aligned(L->rin, 2)) || (L->rout && !aligned(L->rout, 2)) ||
      (L->s_in && !aligned(L->s_in, 4)) || (L->s_out && !aligned(L->s_out, 4)))
    return fail(TRELLIS_EALIGN, "side vectors must be naturally aligned");
  return TRELLIS_OK;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int trellis_abi_version(void) { return TRELLIS_ABI_VERSION; }

const char *trellis_last_error(void) { return g_err; }

int trellis_decode_tiles(const int16_t *code, int K, int in_features, int out_features,
                         uint16_t *w_hat, uint16_t *states, void *stream) {
  g_err[0] = 0;
  if (K < 2 || K > 4) return fail(TRELLIS_EINVAL, "K=%d not in {2,3,4}", K);
  if (in_features < 0 || out_features < 0 || in_features % 16 || out_features % 16)
    return fail(TRELLIS_EINVAL, "in=%d out=%d must be non-negative multiples of 16", in_features,
                out_features);
  if ((long long)in_features * out_features == 0) return TRELLIS_OK;
  if (!code || !w_hat) return fail(TRELLIS_EINVAL, "code or w_hat is NULL");
  if (!aligned(code, 16) || !aligned(w_hat, 16) || (states && !aligned(states, 16)))
    return fail(TRELLIS_EALIGN, "code, w_hat and states must be 16-byte aligned");
  return hip_status(trellis::launch_decode_tiles(code, K, in_features, out_features, w_hat, states,
                                                 as_stream(stream)),
                    "trellis_decode_tiles launch");
}

int had128_scale(const void *x, int x_is_fp32, int rows, int n, const uint16_t *r, const float *s,
                 int post, void *y, int y_is_fp32, void *stream) {
  g_err[0] = 0;
  if (rows < 0 || n <= 0 || n % 128) return fail(TRELLIS_EINVAL, "rows=%d n=%d: need rows >= 0, n a positive multiple of 128", rows, n);
  if (post != 0 && post != 1) return fail(TRELLIS_EINVAL, "post=%d must be 0 or 1", post);
  if ((long long)rows * (n / 128) > (1LL << 33)) return fail(TRELLIS_EINVAL, "too many rows");
  if (rows == 0) return TRELLIS_OK;
  if (!x || !y) return fail(TRELLIS_EINVAL, "x or y is NULL");
  if (!aligned(x, x_is_fp32 ? 4 : 2) || !aligned(y, y_is_fp32 ? 4 : 2) ||
      (r && !aligned(r, 2)) || (s && !aligned(s, 4)))
    return fail(TRELLIS_EALIGN, "arrays must be naturally aligned");
  if (x != y) {
    // partial overlap is not supported (exact aliasing is)
    const char *xa = static_cast<const char *>(x), *ya = static_cast<const char *>(y);
    const size_t xb = (size_t)rows * n * (x_is_fp32 ? 4 : 2), yb = (size_t)rows * n * (y_is_fp32 ? 4 : 2);
    if (xa < ya + yb && ya < xa + xb) return fail(TRELLIS_EINVAL, "x and y overlap without being identical");
  } else if (x_is_fp32 != y_is_fp32) {
    return fail(TRELLIS_EINVAL, "in-place use needs x and y of the same type");
  }
  const float norm = 0.08838834764831845f;  // 1/sqrt(128)
  return hip_status(trellis::launch_had128(x, x_is_fp32, rows, n, r, s, post, norm, y, y_is_fp32,
                                           as_stream(stream)),
                    "had128_scale launch");
}

size_t trellis_workspace_bytes(int op, const trellis_linear *L, int batch_or_M, int n_routed) {
  if (!L || L->in_features <= 0 || L->out_features <= 0 || L->in_features % 128 ||
      L->out_features % 128)
    return 0;
  switch (op) {
    case TRELLIS_OP_GEMV: {
      if (batch_or_M < 1 || batch_or_M > 8) return 0;
      trellis::GemvLaunch a{};
      a.n_list = 1;
      a.list[0].L = *L;
      a.B = batch_or_M;
      return trellis::gemv_workspace_bytes(a);
    }
    case TRELLIS_OP_GEMM:
      if (batch_or_M < 0) return 0;
      return trellis::gemm_workspace_bytes(L->in_features, L->out_features, batch_or_M);
    case TRELLIS_OP_MOE_GEMV:
      if (n_routed < 0) return 0;
      return trellis::gemv_workspace_bytes(n_routed, L->in_features, L->out_features, 1);
    case TRELLIS_OP_GEMM_FP8:
      if (batch_or_M < 0) return 0;
      return trellis::gemm_fp8_workspace_bytes(L->in_features, L->out_features, batch_or_M);
    default:
      return 0;
  }
}

int trellis_gemv(const trellis_linear *L, const uint16_t *x, int B, uint16_t *y, void *ws,
                 size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  int st = check_linear(L, 1);
  if (st) return st;
  trellis_gemv_item it;
  it.L = *L;
  it.x = x;
  it.y = y;
  return trellis_gemv_list(&it, 1, B, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Checks a list of small-batch problems and fills the launch description.
int make_list_launch(const trellis_gemv_item *items, int n, int B, trellis::GemvLaunch *a) {
  if (!items) return fail(TRELLIS_EINVAL, "items is NULL");
  if (n < 1 || n > TRELLIS_GEMV_LIST_MAX) return fail(TRELLIS_EINVAL, "n=%d not in 1..%d", n, TRELLIS_GEMV_LIST_MAX);
  if (B < 1 || B > 8) return fail(TRELLIS_EINVAL, "B=%d not in 1..8", B);
  *a = trellis::GemvLaunch{};
  for (int p = 0; p < n; ++p) {
    const trellis_gemv_item &it = items[p];
    int st = check_linear(&it.L, 1);
    if (st) {
      char tmp[512];
      snprintf(tmp, sizeof(tmp), "item %d: %.480s", p, g_err);
      snprintf(g_err, sizeof(g_err), "%s", tmp);
      return st;
    }
    if (!it.x || !it.y) return fail(TRELLIS_EINVAL, "item %d: x or y is NULL", p);
    if (!aligned(it.x, 2) || !aligned(it.y, 2)) return fail(TRELLIS_EALIGN, "item %d: x/y must be 2-byte aligned", p);
    a->list[p].L = it.L;
    a->list[p].x = it.x;
    a->list[p].y = it.y;
  }
  // outputs must not overlap each other or any input (every output is written once, after
  // every input of the launch may still be read)
  for (int p = 0; p < n; ++p) {
    const char *y0 = reinterpret_cast<const char *>(items[p].y);
    const char *y1 = y0 + (size_t)B * items[p].L.out_features * 2;
    for (int q = 0; q < n; ++q) {
      const char *x0 = reinterpret_cast<const char *>(items[q].x);
      const char *x1 = x0 + (size_t)B * items[q].L.in_features * 2;
      if (y0 < x1 && x0 < y1) return fail(TRELLIS_EINVAL, "item %d's output overlaps item %d's input", p, q);
      if (q != p) {
        const char *z0 = reinterpret_cast<const char *>(items[q].y);
        const char *z1 = z0 + (size_t)B * items[q].L.out_features * 2;
        if (y0 < z1 && z0 < y1) return fail(TRELLIS_EINVAL, "outputs of items %d and %d overlap", p, q);
      }
    }
  }
  a->n_list = n;
  a->table = nullptr;
  a->B = B;
  a->shared_side = -1;
  a->finish = trellis::kFinishPlain;
  return TRELLIS_OK;
}

}  // namespace

extern "C" {

size_t trellis_gemv_list_workspace_bytes(const trellis_gemv_item *items, int n, int B) {
  trellis::GemvLaunch a;
  if (make_list_launch(items, n, B, &a) != TRELLIS_OK) return 0;
  return trellis::gemv_workspace_bytes(a);
}

int trellis_gemv_list(const trellis_gemv_item *items, int n, int B, void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  trellis::GemvLaunch a;
  int st = make_list_launch(items, n, B, &a);
  if (st) return st;
  const size_t need = trellis::gemv_workspace_bytes(a);
  if (need == 0)
    return fail(TRELLIS_EUNSUPPORTED, "more than %d output column blocks or 2^31 units in one call",
                trellis::kMaxFinishGroups);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(TRELLIS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  return hip_status(trellis::launch_gemv(a, ws, ws_bytes, as_stream(stream)), "trellis_gemv launch");
}

int trellis_gemv_list_noalloc(const trellis_gemv_item *items, int n, int B, void *stream) {
  g_err[0] = 0;
  trellis::GemvLaunch a;
  int st = make_list_launch(items, n, B, &a);
  if (st) return st;
  const size_t need = trellis::gemv_workspace_bytes(a);
  if (need == 0)
    return fail(TRELLIS_EUNSUPPORTED, "more than %d output column blocks or 2^31 units in one call",
                trellis::kMaxFinishGroups);
  if (need > trellis::kNoAllocScratchBytes)
    return fail(TRELLIS_EUNSUPPORTED, "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu",
                need, trellis::kNoAllocScratchBytes);
  void *ws = nullptr;
  st = hip_status(trellis::noalloc_scratch(&ws), "trellis_gemv_list_noalloc scratch lookup");
  if (st) return st;
  return hip_status(trellis::launch_gemv(a, ws, trellis::kNoAllocScratchBytes, as_stream(stream)),
                    "trellis_gemv_list_noalloc launch");
}

int trellis_gemm(const trellis_linear *L, const uint16_t *x, int M, uint16_t *y, void *ws,
                 size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  int st = check_linear(L, 1);
  if (st) return st;
  if (M < 0) return fail(TRELLIS_EINVAL, "M=%d < 0", M);
  if (M == 0) return TRELLIS_OK;
  if ((long long)M > (1LL << 24)) return fail(TRELLIS_EINVAL, "M=%d too large", M);
  if (!x || !y) return fail(TRELLIS_EINVAL, "x or y is NULL");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(TRELLIS_EALIGN, "x/y must be 16-byte aligned");
  const size_t need = trellis::gemm_workspace_bytes(L->in_features, L->out_features, M);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(TRELLIS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  return hip_status(trellis::launch_gemm(*L, x, M, y, ws, ws_bytes, as_stream(stream)),
                    "trellis_gemm launch");
}

int trellis_gemm_fp8(const trellis_linear *L, const uint16_t *x, int M, uint16_t *y, void *ws,
                     size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  int st = check_linear(L, 1);
  if (st) return st;
  if (L->cb != 2) return fail(TRELLIS_EINVAL, "trellis_gemm_fp8 needs the E4M3 codebook (cb=2), got cb=%d", L->cb);
  if (M < 0) return fail(TRELLIS_EINVAL, "M=%d < 0", M);
  if (M == 0) return TRELLIS_OK;
  if ((long long)M > (1LL << 24)) return fail(TRELLIS_EINVAL, "M=%d too large", M);
  if (!x || !y) return fail(TRELLIS_EINVAL, "x or y is NULL");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(TRELLIS_EALIGN, "x/y must be 16-byte aligned");
  const size_t need = trellis::gemm_fp8_workspace_bytes(L->in_features, L->out_features, M);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(TRELLIS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  return hip_status(trellis::launch_gemm_fp8(*L, x, M, y, ws, ws_bytes, as_stream(stream)),
                    "trellis_gemm_fp8 launch");
}

int trellis_decode_tiles_e4m3(const int16_t *code, int K, int in_features, int out_features, uint8_t *w8,
                              void *stream) {
  g_err[0] = 0;
  if (K < 2 || K > 4) return fail(TRELLIS_EINVAL, "K=%d not in {2,3,4}", K);
  if (in_features < 0 || out_features < 0 || in_features % 16 || out_features % 16)
    return fail(TRELLIS_EINVAL, "in=%d out=%d must be non-negative multiples of 16", in_features,
                out_features);
  if ((long long)in_features * out_features == 0) return TRELLIS_OK;
  if (!code || !w8) return fail(TRELLIS_EINVAL, "code or w8 is NULL");
  if (!aligned(code, 16) || !aligned(w8, 16)) return fail(TRELLIS_EALIGN, "code and w8 must be 16-byte aligned");
  return hip_status(trellis::launch_decode_tiles_e4m3(code, K, in_features, out_features, w8, as_stream(stream)),
                    "trellis_decode_tiles_e4m3 launch");
}

int trellis_moe_gemv(const trellis_linear *experts, int E, const int32_t *routed, int n,
                     int in_features, int out_features, const uint16_t *x, int x_per_expert,
                     const uint16_t *shared_r, const float *shared_s, int shared_side,
                     uint16_t *y, void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (E <= 0 || !experts) return fail(TRELLIS_EINVAL, "empty or NULL expert table");
  if (n < 0) return fail(TRELLIS_EINVAL, "n=%d < 0", n);
  if (in_features <= 0 || out_features <= 0 || in_features % 128 || out_features % 128)
    return fail(TRELLIS_EINVAL, "in=%d out=%d must be positive multiples of 128", in_features, out_features);
  if (shared_side < -1 || shared_side > 1) return fail(TRELLIS_EINVAL, "shared_side=%d", shared_side);
  if (shared_side >= 0 && !shared_r) return fail(TRELLIS_EINVAL, "shared_r is NULL");
  if (x_per_expert != 0 && x_per_expert != 1) return fail(TRELLIS_EINVAL, "x_per_expert must be 0 or 1");
  if (n == 0) return TRELLIS_OK;
  if (!routed || !x || !y) return fail(TRELLIS_EINVAL, "routed, x or y is NULL");
  if (!aligned(experts, 8) || !aligned(routed, 4) || !aligned(x, 2) || !aligned(y, 2))
    return fail(TRELLIS_EALIGN, "misaligned table, routed, x or y");
  const size_t need = trellis::gemv_workspace_bytes(n, in_features, out_features, 1);
  if (need == 0)
    return fail(TRELLIS_EUNSUPPORTED, "n*out/128 exceeds %d column blocks", trellis::kMaxFinishGroups);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(TRELLIS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  trellis::GemvLaunch a{};
  a.table = experts;
  a.E = E;
  a.group = 1;
  a.routed = routed;
  a.n_problems = n;
  a.in_features = in_features;
  a.out_features = out_features;
  a.B = 1;
  a.x = x;
  a.x_per_problem = x_per_expert;
  a.y = y;
  a.shared_r = shared_r;
  a.shared_s = shared_s;
  a.shared_side = shared_side;
  return hip_status(trellis::launch_gemv(a, ws, ws_bytes, as_stream(stream)), "trellis_moe_gemv launch");
}

size_t trellis_moe_mlp_workspace_bytes(int hidden, int inter, int halves, int n) {
  if (hidden <= 0 || inter <= 0 || halves < 1 || n < 0 || hidden % 128 || inter % (128 * halves)) return 0;
  if ((long long)n * (inter / 128) * (hidden / 128) >= (1LL << 30)) return 0;
  return trellis::moe_mlp_workspace_bytes(hidden, inter, halves, n);
}

int trellis_moe_mlp(const trellis_linear *gate_up, const trellis_linear *down, int E, int halves,
                    const int32_t *routed, const float *router_w, int n, int hidden, int inter,
                    const uint16_t *x, const uint16_t *r_hidden_in, const float *s_hidden_in,
                    const uint16_t *r_hidden_out, const float *s_hidden_out, uint16_t *act,
                    uint16_t *y, void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (E <= 0 || !gate_up || !down) return fail(TRELLIS_EINVAL, "empty or NULL expert tables");
  if (halves < 1) return fail(TRELLIS_EINVAL, "halves=%d < 1", halves);
  if (n < 0) return fail(TRELLIS_EINVAL, "n=%d < 0", n);
  if (hidden <= 0 || inter <= 0 || hidden % 128 || inter % (128 * halves))
    return fail(TRELLIS_EINVAL, "hidden=%d must be a positive multiple of 128 and inter=%d of 128*halves",
                hidden, inter);
  if ((long long)n * (inter / 128) * (hidden / 128) >= (1LL << 30))
    return fail(TRELLIS_EINVAL, "n=%d routed experts of %dx%d exceed the work limit", n, hidden, inter);
  if (!y || !r_hidden_out) return fail(TRELLIS_EINVAL, "y or r_hidden_out is NULL");
  if (n > 0 && (!routed || !router_w || !x || !r_hidden_in))
    return fail(TRELLIS_EINVAL, "routed, router_w, x or r_hidden_in is NULL");
  if (!aligned(gate_up, 8) || !aligned(down, 8) || !aligned(routed, 4) || !aligned(router_w, 4) ||
      !aligned(x, 2) || !aligned(y, 2) || !aligned(act, 2) || !aligned(r_hidden_in, 2) ||
      !aligned(r_hidden_out, 2) || !aligned(s_hidden_in, 4) || !aligned(s_hidden_out, 4))
    return fail(TRELLIS_EALIGN, "misaligned table, vector or buffer");
  const size_t need = trellis::moe_mlp_workspace_bytes(hidden, inter, halves, n);
  if (need == 0)
    return fail(TRELLIS_EUNSUPPORTED, "n*inter/128 exceeds %d column blocks", 2 * trellis::kMaxFinishGroups);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(TRELLIS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  trellis::MlpLaunch m{};
  m.gate_up = gate_up;
  m.down = down;
  m.E = E;
  m.halves = halves;
  m.n = n;
  m.hidden = hidden;
  m.inter = inter;
  m.routed = routed;
  m.router_w = router_w;
  m.x = x;
  m.r_hidden_in = r_hidden_in;
  m.s_hidden_in = s_hidden_in;
  m.r_hidden_out = r_hidden_out;
  m.s_hidden_out = s_hidden_out;
  m.act = act;
  m.y = y;
  return hip_status(trellis::launch_moe_mlp(m, ws, ws_bytes, as_stream(stream)), "trellis_moe_mlp launch");
}

size_t trellis_encode_workspace_bytes(int n_tiles) {
  if (n_tiles < 0) return 0;
  return trellis::encode_workspace_bytes(n_tiles);
}

int trellis_encode_tiles(const float *targets, int n_tiles, int K, int cb, int16_t *code, uint16_t *states,
                         void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (K < 2 || K > 4) return fail(TRELLIS_EINVAL, "K=%d not in {2,3,4}", K);
  if (cb != 1 && cb != 2) return fail(TRELLIS_EINVAL, "cb=%d: 1 (MCG) or 2 (E4M3) expected", cb);
  if (n_tiles < 0) return fail(TRELLIS_EINVAL, "n_tiles=%d < 0", n_tiles);
  if (n_tiles == 0) return TRELLIS_OK;
  if (!targets || !code) return fail(TRELLIS_EINVAL, "targets or code is NULL");
  if (!aligned(targets, 4) || !aligned(code, 4) || !aligned(states, 2))
    return fail(TRELLIS_EALIGN, "targets/code must be 4-byte and states 2-byte aligned");
  const size_t need = trellis::encode_workspace_bytes(n_tiles);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(TRELLIS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  return hip_status(trellis::launch_encode_tiles(targets, n_tiles, K, cb, code, states, ws, ws_bytes,
                                                 as_stream(stream)),
                    "trellis_encode_tiles launch");
}

int trellis_validate_table(const trellis_linear *host_table, int E, int in_features,
                           int out_features, int shared_side) {
  g_err[0] = 0;
  if (!host_table || E <= 0) return fail(TRELLIS_EINVAL, "empty or NULL table");
  for (int e = 0; e < E; ++e) {
    const trellis_linear &L = host_table[e];
    trellis_linear c = L;
    if (shared_side == 0 && !c.rin) c.rin = reinterpret_cast<const uint16_t *>(&L);  // shared: may be NULL
    if (shared_side == 1 && !c.rout) c.rout = reinterpret_cast<const uint16_t *>(&L);
    int st = check_linear(&c, 1);
    if (st) {
      char tmp[512];
      snprintf(tmp, sizeof(tmp), "entry %d: %.480s", e, g_err);
      snprintf(g_err, sizeof(g_err), "%s", tmp);
      return st;
    }
    if (L.in_features != in_features || L.out_features != out_features)
      return fail(TRELLIS_EINVAL, "entry %d: shape %dx%d differs from %dx%d", e, L.in_features,
                  L.out_features, in_features, out_features);
  }
  return TRELLIS_OK;
}

// ---------------------------------------------------------------------------------------
// Microbenchmarks (include/trellis_micro.h)
// ---------------------------------------------------------------------------------------

int trellis_micro_cus(void) { return trellis::micro_cus(); }

int trellis_micro_stream_read(const void *buf, size_t bytes, int blocks, uint32_t *sink, void *stream) {
  g_err[0] = 0;
  if (!buf || !sink) return fail(TRELLIS_EINVAL, "buf or sink is NULL");
  if (bytes < 16 || bytes % 16) return fail(TRELLIS_EINVAL, "bytes=%zu must be a positive multiple of 16", bytes);
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(TRELLIS_EALIGN, "buf must be 16-byte aligned");
  if (blocks < 0 || blocks > (1 << 20)) return fail(TRELLIS_EINVAL, "blocks=%d out of range", blocks);
  return hip_status(trellis::launch_micro_stream_read(buf, bytes, blocks, sink, as_stream(stream)),
                    "trellis_micro_stream_read launch");
}

int trellis_micro_valu(int op, int iters, int waves_per_simd, uint64_t *cycles, uint64_t *ticks, uint32_t *sink,
                       void *stream) {
  g_err[0] = 0;
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 8)
    return fail(TRELLIS_EINVAL, "iters=%d >= 1 and waves_per_simd=%d in 1..8 expected", iters, waves_per_simd);
  if (!cycles || !ticks || !sink) return fail(TRELLIS_EINVAL, "cycles, ticks or sink is NULL");
  if (!aligned(cycles, 8) || !aligned(ticks, 8) || !aligned(sink, 4)) return fail(TRELLIS_EALIGN, "misaligned output");
  int blocks = 0;
  const hipError_t e = trellis::launch_micro_valu(op, iters, waves_per_simd, cycles, ticks, sink, as_stream(stream), &blocks);
  if (e == hipErrorInvalidValue) return fail(TRELLIS_EINVAL, "unknown micro kernel %d", op);
  const int st = hip_status(e, "trellis_micro_valu launch");
  return st ? st : blocks;
}

int trellis_micro_mfma(int kind, int iters, int waves_per_simd, uint64_t *cycles, uint64_t *ticks, float *sink,
                       void *stream) {
  g_err[0] = 0;
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 4)
    return fail(TRELLIS_EINVAL, "iters=%d >= 1 and waves_per_simd=%d in 1..4 expected", iters, waves_per_simd);
  if (!cycles || !ticks || !sink) return fail(TRELLIS_EINVAL, "cycles, ticks or sink is NULL");
  if (!aligned(cycles, 8) || !aligned(ticks, 8) || !aligned(sink, 4)) return fail(TRELLIS_EALIGN, "misaligned output");
  int blocks = 0;
  const hipError_t e = trellis::launch_micro_mfma(kind, iters, waves_per_simd, cycles, ticks, sink, as_stream(stream), &blocks);
  if (e == hipErrorInvalidValue) return fail(TRELLIS_EINVAL, "unknown matrix kernel %d", kind);
  const int st = hip_status(e, "trellis_micro_mfma launch");
  return st ? st : blocks;
}

}  // extern "C"
