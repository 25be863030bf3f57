// trellis_gemm: prefill product Y = had(had(X*su) @ W_hat) * sv for M rows.
//
// ("Escha-W2 runs on Metal", reconstruction paragraph; decode as in decode.hip.)
//
// Two launches:
//   1. had128 pre-pass: XH = H128(X*su) (unnormalised butterfly) as fp16 in the workspace;
//   2. the fused GEMM: each 256-thread workgroup owns a 256 (M) x 128 (N) output tile.  Per
//      k-step of 32 input rows it decodes the 2x8 trellis tiles of that step into LDS as
//      fp16 (the format's exact fp16 codebook values, one v_add_f16 rounding) and runs
//      v_mfma_f32_16x16x32_f16 with fp32 accumulation; wave w owns output rows
//      64w..64w+63.  The epilogue applies the output Hadamard across the tile's 128 columns
//      (16 lanes x 8 registers per row), the scales and the exact 1/128, and writes fp16.
#include "launch.h"
#include "trellis_device.h"

namespace trellis {

namespace {

constexpr int kMT = 256;     // output rows per workgroup
constexpr int kNT = 128;     // output columns per workgroup (one Hadamard block)
constexpr int kKS = 32;      // input rows per k-step (two tile rows)
constexpr int kBPitch = kKS + 8;  // LDS row pitch (halves) of the transposed B tile

template <int K>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t *__restrict__ xh, int M, int in,
                                                   const uint32_t *__restrict__ code, int out,
                                                   const uint16_t *__restrict__ rout,
                                                   const float *__restrict__ s_out,
                                                   uint16_t *__restrict__ y) {
  constexpr int NW = 8 * K;
  __shared__ __attribute__((aligned(16))) uint16_t bt[kNT][kBPitch];  // [n][k]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int Tj = out / 16;
  const int row_base = mt * kMT + wave * 64;
  const LaneWindow lw = lane_window(lane, K);
  const int n16 = lane & 15, kg = lane >> 4;

  floatx4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = in / kKS;
  for (int ks = 0; ks < nsteps; ++ks) {
    __syncthreads();
    // decode the step's 16 tiles: wave w takes tiles 4w..4w+3 (tile row t>>3, column t&7)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int t = wave * 4 + t4;
      const int ti = t >> 3, tj = t & 7;
      const uint32_t *tile = code + ((size_t)(ks * 2 + ti) * Tj + (size_t)nt * 8 + tj) * NW;
      const uint32_t bits = lane_bits(tile[lw.d0], tile[lw.d1], lw.sh);
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = __builtin_bit_cast(uint16_t, mcg_value(mcg_hash(lane_state<K>(bits, j))));
      uint32_t *dst = reinterpret_cast<uint32_t *>(&bt[16 * tj + n16][16 * ti + 2 * kg]);
      dst[0] = v[0] | (v[1] << 16);   // rows 2g, 2g+1
      dst[4] = v[2] | (v[3] << 16);   // rows 2g+8, 2g+9
    }
    __syncthreads();
    // A fragments: rows row_base + 16*mb + (lane&15), k = 8*kg .. 8*kg+7 of this step
    half8 af[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int row = row_base + 16 * mb + n16;
      u32x4 a = {0u, 0u, 0u, 0u};
      if (row < M) a = *reinterpret_cast<const u32x4 *>(xh + (size_t)row * in + ks * kKS + 8 * kg);
      af[mb] = __builtin_bit_cast(half8, a);
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const half8 bf = *reinterpret_cast<const half8 *>(&bt[16 * nb + n16][8 * kg]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bf, acc[mb][nb], 0, 0, 0);
    }
  }

  // Epilogue.  Lane holds rows 16*mb + 4*(lane>>4) + r, columns 16*nb + (lane&15).
  // Column index bits 0..3 are lane bits, bits 4..6 the register index nb.
  float sv[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int col = nt * kNT + 16 * nb + n16;
    float s = h2f(rout[col]) * (1.0f / 128.0f);
    if (s_out) s *= s_out[col];
    sv[nb] = s;
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb] = acc[mb][nb][r];
      // register stages (column strides 16, 32, 64)
#pragma unroll
      for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          if ((nb & h) == 0) {
            const float a = v[nb], b = v[nb + h];
            v[nb] = a + b;
            v[nb + h] = a - b;
          }
        }
      }
      // lane stages (column strides 1, 2, 4, 8) inside each 16-lane group
#pragma unroll
      for (int h = 1; h < 16; h <<= 1) {
        const bool up = (lane & h) != 0;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const float p = __shfl_xor(v[nb], h, 64);
          v[nb] = up ? (p - v[nb]) : (v[nb] + p);
        }
      }
      const int row = row_base + 16 * mb + 4 * (lane >> 4) + r;
      if (row < M) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
          y[(size_t)row * out + nt * kNT + 16 * nb + n16] = f2h(v[nb] * sv[nb]);
      }
    }
  }
}

}  // namespace

size_t gemm_workspace_bytes(int in_features, int out_features, int M) {
  (void)out_features;
  return ((size_t)M * in_features * 2 + 255) / 256 * 256;
}

hipError_t launch_gemm(const trellis_linear &L, const uint16_t *x, int M, uint16_t *y, void *ws,
                       size_t ws_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (ws_bytes < gemm_workspace_bytes(L.in_features, L.out_features, M)) return hipErrorInvalidValue;
  uint16_t *xh = static_cast<uint16_t *>(ws);
  hipError_t e = launch_had128(x, 0, M, L.in_features, L.rin, L.s_in, 0, 1.0f, xh, 0, stream);
  if (e != hipSuccess) return e;
  dim3 grid(L.out_features / kNT, (M + kMT - 1) / kMT), block(256);
  const uint32_t *c = reinterpret_cast<const uint32_t *>(L.code);
  switch (L.K) {
    case 2: gemm_kernel<2><<<grid, block, 0, stream>>>(xh, M, L.in_features, c, L.out_features, L.rout, L.s_out, y); break;
    case 3: gemm_kernel<3><<<grid, block, 0, stream>>>(xh, M, L.in_features, c, L.out_features, L.rout, L.s_out, y); break;
    case 4: gemm_kernel<4><<<grid, block, 0, stream>>>(xh, M, L.in_features, c, L.out_features, L.rout, L.s_out, y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trellis
