// Host-only driver of libtrellis's C-ABI layer (csrc/api.cpp) for AddressSanitizer and
// UndefinedBehaviorSanitizer builds with the host compiler.  The device launchers are stubs
// that count their calls and check what the ABI layer hands them (non-null pointers, sizes
// inside the workspace), so every entry point's validation and marshalling runs without a GPU.
// Exit status 0 when every expectation holds; the sanitizers abort on any memory or
// undefined-behaviour error.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/trellis.h"
#include "../../include/trellis_micro.h"
#include "../../trellis_coded_bit_amd/csrc/launch.h"

static int g_launches = 0, g_fail = 0;
#define EXPECT(c)                                                            \
  do {                                                                       \
    if (!(c)) {                                                              \
      std::fprintf(stderr, "expectation failed at line %d: %s (last error: %s)\n", __LINE__, #c, \
                   trellis_last_error());                                    \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

extern "C" const char *hipGetErrorString(hipError_t) { return "stub HIP error"; }

namespace trellis {
static hipError_t launched() { ++g_launches; return hipSuccess; }
hipError_t launch_decode_tiles(const int16_t *code, int, int, int, uint16_t *w, uint16_t *, hipStream_t) {
  EXPECT(code && w);
  return launched();
}
hipError_t launch_decode_tiles_e4m3(const int16_t *code, int, int, int, uint8_t *w8, hipStream_t) {
  EXPECT(code && w8);
  return launched();
}
hipError_t launch_had128(const void *x, int, int, int, const uint16_t *, const float *, int, float, void *y, int,
                         hipStream_t) {
  EXPECT(x && y);
  return launched();
}
size_t gemv_workspace_bytes(const GemvLaunch &a) {
  const int n = a.table ? a.n_problems : a.n_list;
  return kWsReserved + (size_t)(n > 0 ? n : 0) * 4096;
}
size_t gemv_workspace_bytes(int n_problems, int, int, int) { return kWsReserved + (size_t)n_problems * 4096; }
hipError_t launch_gemv(const GemvLaunch &a, void *ws, size_t ws_bytes, hipStream_t) {
  EXPECT(ws && ws_bytes >= gemv_workspace_bytes(a));
  if (!a.table)
    for (int p = 0; p < a.n_list; ++p) EXPECT(a.list[p].x && a.list[p].y && a.list[p].L.code);
  return launched();
}
static char g_scratch[1 << 12];
hipError_t noalloc_scratch(void **ptr) { *ptr = g_scratch; return hipSuccess; }
size_t moe_mlp_workspace_bytes(int, int, int, int n) { return kWsReserved + (size_t)n * 8192; }
size_t encode_workspace_bytes(int n) { return (size_t)n << 20; }
hipError_t launch_encode_tiles(const float *t, int, int, int, int16_t *code, uint16_t *, void *ws, size_t, hipStream_t) {
  EXPECT(t && code && ws);
  return launched();
}
hipError_t launch_moe_mlp(const MlpLaunch &m, void *ws, size_t, hipStream_t) {
  EXPECT(ws && m.gate_up && m.down && m.y);
  return launched();
}
size_t gemm_workspace_bytes(int in, int, int M) { return kWsReserved + (size_t)M * in * 2; }
hipError_t launch_gemm(const trellis_linear &L, const uint16_t *x, int, uint16_t *y, void *ws, size_t, hipStream_t) {
  EXPECT(L.code && x && y && ws);
  return launched();
}
size_t gemm_fp8_workspace_bytes(int in, int, int M) { return kWsReserved + (size_t)M * in; }
hipError_t launch_gemm_fp8(const trellis_linear &L, const uint16_t *x, int, uint16_t *y, void *ws, size_t,
                           hipStream_t) {
  EXPECT(L.code && x && y && ws && L.cb == 2);
  return launched();
}
int micro_cus() { return 256; }
hipError_t launch_micro_stream_read(const void *b, size_t, int, uint32_t *s, hipStream_t) {
  EXPECT(b && s);
  return launched();
}
hipError_t launch_micro_valu(int op, int, int wps, uint64_t *, uint64_t *, uint32_t *, hipStream_t, int *blocks) {
  *blocks = 256 * wps;
  return op < 0 ? hipErrorInvalidValue : launched();
}
hipError_t launch_micro_mfma(int kind, int, int wps, uint64_t *, uint64_t *, float *, hipStream_t, int *blocks) {
  *blocks = 256 * wps;
  return kind < 0 ? hipErrorInvalidValue : launched();
}
}  // namespace trellis

// Fake, never dereferenced device addresses (16-byte aligned unless made otherwise).
template <typename T>
static T *dev(unsigned long a) { return reinterpret_cast<T *>(a << 12); }

static trellis_linear layer(int K, int in, int out, int cb = 1) {
  trellis_linear L;
  L.code = dev<const int16_t>(0x100);
  L.rin = dev<const uint16_t>(0x200);
  L.rout = dev<const uint16_t>(0x300);
  L.s_in = dev<const float>(0x400);
  L.s_out = dev<const float>(0x500);
  L.K = K;
  L.in_features = in;
  L.out_features = out;
  L.cb = cb;
  return L;
}

int main() {
  EXPECT(trellis_abi_version() == TRELLIS_ABI_VERSION);
  // decode / Hadamard
  EXPECT(trellis_decode_tiles(dev<int16_t>(1), 3, 512, 256, dev<uint16_t>(2), nullptr, nullptr) == TRELLIS_OK);
  EXPECT(trellis_decode_tiles(dev<int16_t>(1), 5, 512, 256, dev<uint16_t>(2), nullptr, nullptr) == TRELLIS_EINVAL);
  EXPECT(std::strlen(trellis_last_error()) > 0);
  EXPECT(trellis_decode_tiles_e4m3(dev<int16_t>(1), 2, 64, 64, dev<uint8_t>(2), nullptr) == TRELLIS_OK);
  EXPECT(had128_scale(dev<void>(1), 0, 4, 256, nullptr, nullptr, 0, dev<void>(1), 0, nullptr) == TRELLIS_OK);
  EXPECT(had128_scale(dev<void>(1), 0, 4, 256, nullptr, nullptr, 0, dev<char>(1) + 128, 0, nullptr) == TRELLIS_EINVAL);
  // single and list GEMV
  trellis_linear L = layer(3, 512, 384);
  const size_t nb = trellis_workspace_bytes(TRELLIS_OP_GEMV, &L, 4, 0);
  EXPECT(nb > 0);
  EXPECT(trellis_gemv(&L, dev<uint16_t>(0x600), 4, dev<uint16_t>(0x700), dev<void>(0x800), nb, nullptr) == TRELLIS_OK);
  EXPECT(trellis_gemv(&L, dev<uint16_t>(0x600), 9, dev<uint16_t>(0x700), dev<void>(0x800), nb, nullptr) == TRELLIS_EINVAL);
  EXPECT(trellis_gemv(nullptr, dev<uint16_t>(0x600), 1, dev<uint16_t>(0x700), dev<void>(0x800), nb, nullptr) == TRELLIS_EINVAL);
  trellis_gemv_item items[TRELLIS_GEMV_LIST_MAX + 1];
  for (int i = 0; i <= TRELLIS_GEMV_LIST_MAX; ++i) {
    items[i].L = layer(2 + i % 3, 256 * (1 + i % 2), 128 * (1 + i % 4), 1 + i % 2);
    items[i].x = dev<const uint16_t>(0x1000 + 16 * i);
    items[i].y = dev<uint16_t>(0x2000 + 16 * i);
  }
  const size_t lb = trellis_gemv_list_workspace_bytes(items, TRELLIS_GEMV_LIST_MAX, 8);
  EXPECT(lb > 0);
  EXPECT(trellis_gemv_list(items, TRELLIS_GEMV_LIST_MAX, 8, dev<void>(0x800), lb, nullptr) == TRELLIS_OK);
  EXPECT(trellis_gemv_list(items, TRELLIS_GEMV_LIST_MAX + 1, 8, dev<void>(0x800), lb, nullptr) == TRELLIS_EINVAL);
  EXPECT(trellis_gemv_list(items, 0, 8, dev<void>(0x800), lb, nullptr) == TRELLIS_EINVAL);
  EXPECT(trellis_gemv_list(items, 2, 1, dev<void>(0x800), 10, nullptr) == TRELLIS_EWORKSPACE);
  EXPECT(trellis_gemv_list_noalloc(items, 3, 2, nullptr) == TRELLIS_OK);
  items[1].y = items[0].y;  // outputs overlap
  EXPECT(trellis_gemv_list(items, 2, 1, dev<void>(0x800), lb, nullptr) == TRELLIS_EINVAL);
  items[1].y = dev<uint16_t>(0x2010);
  items[2].L.K = 9;
  EXPECT(trellis_gemv_list(items, 3, 1, dev<void>(0x800), lb, nullptr) == TRELLIS_EINVAL);
  EXPECT(std::strstr(trellis_last_error(), "item 2") != nullptr);
  // prefill
  const size_t gb = trellis_workspace_bytes(TRELLIS_OP_GEMM, &L, 300, 0);
  EXPECT(trellis_gemm(&L, dev<uint16_t>(0x600), 300, dev<uint16_t>(0x700), dev<void>(0x800), gb, nullptr) == TRELLIS_OK);
  EXPECT(trellis_gemm(&L, dev<uint16_t>(0x600), -3, dev<uint16_t>(0x700), dev<void>(0x800), gb, nullptr) == TRELLIS_EINVAL);
  trellis_linear L8 = layer(3, 512, 384, 2);
  const size_t fb = trellis_workspace_bytes(TRELLIS_OP_GEMM_FP8, &L8, 64, 0);
  EXPECT(trellis_gemm_fp8(&L8, dev<uint16_t>(0x600), 64, dev<uint16_t>(0x700), dev<void>(0x800), fb, nullptr) == TRELLIS_OK);
  EXPECT(trellis_gemm_fp8(&L, dev<uint16_t>(0x600), 64, dev<uint16_t>(0x700), dev<void>(0x800), fb, nullptr) == TRELLIS_EINVAL);
  // MoE tables
  trellis_linear table[6];
  for (int e = 0; e < 6; ++e) table[e] = layer(2 + e % 3, 768, 256);
  EXPECT(trellis_validate_table(table, 6, 768, 256, -1) == TRELLIS_OK);
  table[4].K = 1;
  EXPECT(trellis_validate_table(table, 6, 768, 256, -1) == TRELLIS_EINVAL);
  EXPECT(std::strstr(trellis_last_error(), "entry 4") != nullptr);
  const size_t mb = trellis_workspace_bytes(TRELLIS_OP_MOE_GEMV, &table[0], 1, 5);
  EXPECT(trellis_moe_gemv(dev<trellis_linear>(0x900), 6, dev<int32_t>(0xA00), 5, 768, 256, dev<uint16_t>(0x600), 0,
                          dev<uint16_t>(0x610), nullptr, 0, dev<uint16_t>(0x700), dev<void>(0x800), mb, nullptr) == TRELLIS_OK);
  EXPECT(trellis_moe_gemv(dev<trellis_linear>(0x900), 6, dev<int32_t>(0xA00), 5, 768, 256, dev<uint16_t>(0x600), 0,
                          nullptr, nullptr, 0, dev<uint16_t>(0x700), dev<void>(0x800), mb, nullptr) == TRELLIS_EINVAL);
  const size_t pb = trellis_moe_mlp_workspace_bytes(768, 512, 2, 3);
  EXPECT(trellis_moe_mlp(dev<trellis_linear>(0x900), dev<trellis_linear>(0x901), 6, 2, dev<int32_t>(0xA00),
                         dev<float>(0xA01), 3, 768, 512, dev<uint16_t>(0x600), dev<uint16_t>(0x610), nullptr,
                         dev<uint16_t>(0x620), nullptr, nullptr, dev<uint16_t>(0x700), dev<void>(0x800), pb, nullptr) == TRELLIS_OK);
  // encoder and microbenchmarks
  const size_t eb = trellis_encode_workspace_bytes(8);
  EXPECT(trellis_encode_tiles(dev<float>(0x100), 8, 3, 1, dev<int16_t>(0x200), nullptr, dev<void>(0x300), eb, nullptr) == TRELLIS_OK);
  EXPECT(trellis_encode_tiles(dev<float>(0x100), 8, 3, 3, dev<int16_t>(0x200), nullptr, dev<void>(0x300), eb, nullptr) == TRELLIS_EINVAL);
  EXPECT(trellis_micro_stream_read(dev<void>(0x100), 1 << 20, 0, dev<uint32_t>(0x200), nullptr) == TRELLIS_OK);
  EXPECT(trellis_micro_valu(TRELLIS_MICRO_DECODE_TILE_MFMA, 10, 4, dev<uint64_t>(1), dev<uint64_t>(2), dev<uint32_t>(3), nullptr) == 1024);
  EXPECT(trellis_micro_mfma(TRELLIS_MICRO_MFMA_F16_32X32X16, 10, 2, dev<uint64_t>(1), dev<uint64_t>(2), dev<float>(3), nullptr) == 512);
  std::printf("launches %d, failures %d\n", g_launches, g_fail);
  return g_fail == 0 && g_launches == 14 ? 0 : 1;
}
