// trellis_decode_tiles: packed trellis tiles -> codebook-domain fp16 matrix, bit-exact.
//
// ("The escha W2 format, recovered and verified", "Bit layout" and "Codebook: cb=1";
//  "Escha-W2 runs on Metal", tile/permutation paragraph; the E4M3 variant: "EXLR8" page,
//  E4M3 paragraph.)
//
// Work split: one 256-thread workgroup per (tile row i, group of 8 tile columns).  Each
// wave decodes two tiles; lane l decodes its four symbols (trellis_device.h) and drops the
// fp16 values into an LDS staging block [16 rows][128 cols], which the workgroup then
// writes out as 16 coalesced 256-byte row segments.
#include "launch.h"
#include "trellis_device.h"

namespace trellis {

template <int K>
__global__ __launch_bounds__(256) void decode_tiles_kernel(const uint32_t *__restrict__ code,
                                                           int Tj, uint16_t *__restrict__ w_hat,
                                                           int out_features,
                                                           uint16_t *__restrict__ states) {
  constexpr int NW = 8 * K;  // 32-bit words per tile
  __shared__ uint16_t stage[16][128 + 8];
  const int i = blockIdx.y;
  const int j0 = blockIdx.x * 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const LaneWindow lw = lane_window(lane, K);
  const int n = lane & 15;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int jj = 2 * wave + t;
    const int j = j0 + jj;
    if (j < Tj) {
      const uint32_t *tile = code + ((size_t)i * Tj + j) * NW;
      const uint32_t bits = lane_bits(tile[lw.d0], tile[lw.d1], lw.sh);
      uint32_t st[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        st[q] = lane_state<K>(bits, q);
        stage[lane_row(lane, q)][16 * jj + n] = __builtin_bit_cast(uint16_t, mcg_value(mcg_hash(st[q])));
      }
      if (states) {
        const int s0 = 32 * (n & 7) + 8 * (lane >> 4) + 4 * (n >> 3);
        uint2 pk;
        pk.x = st[0] | (st[1] << 16);
        pk.y = st[2] | (st[3] << 16);
        *reinterpret_cast<uint2 *>(states + ((size_t)i * Tj + j) * 256 + s0) = pk;
      }
    }
  }
  __syncthreads();
  // 16 rows x (8 tiles x 16 cols): thread -> (row, 8-column chunk)
  const int row = threadIdx.x >> 4, chunk = threadIdx.x & 15;
  const int col = 16 * j0 + 8 * chunk;
  if (col < out_features) {
    const uint16_t *src = &stage[row][8 * chunk];
    uint4 v;
    v.x = src[0] | ((uint32_t)src[1] << 16);
    v.y = src[2] | ((uint32_t)src[3] << 16);
    v.z = src[4] | ((uint32_t)src[5] << 16);
    v.w = src[6] | ((uint32_t)src[7] << 16);
    *reinterpret_cast<uint4 *>(w_hat + (size_t)(16 * i + row) * out_features + col) = v;
  }
}

// The E4M3 codebook variant ("EXLR8" page, E4M3 paragraph): the same decode, each value
// rounded to E4M3 and written as one byte.  Workgroup per (tile row i, 16 tile columns),
// each wave decoding four tiles; the 16 x 256 bytes are staged in LDS and written as 16
// bytes per thread.
template <int K>
__global__ __launch_bounds__(256) void decode_tiles_e4m3_kernel(const uint32_t *__restrict__ code, int Tj,
                                                                uint8_t *__restrict__ w8, int out_features) {
  constexpr int NW = 8 * K;
  __shared__ __attribute__((aligned(16))) uint8_t stage[16][256 + 16];
  const int i = blockIdx.y;
  const int j0 = blockIdx.x * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const LaneWindow lw = lane_window(lane, K);
  const int n = lane & 15;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int jj = 4 * wave + t;
    const int j = j0 + jj;
    if (j < Tj) {
      const uint32_t *tile = code + ((size_t)i * Tj + j) * NW;
      const uint32_t bits = lane_bits(tile[lw.d0], tile[lw.d1], lw.sh);
      const uint32_t q = e4m3_pack4(mcg_hash(lane_state<K>(bits, 0)), mcg_hash(lane_state<K>(bits, 1)),
                                    mcg_hash(lane_state<K>(bits, 2)), mcg_hash(lane_state<K>(bits, 3)));
#pragma unroll
      for (int s = 0; s < 4; ++s) stage[lane_row(lane, s)][16 * jj + n] = (uint8_t)(q >> (8 * s));
    }
  }
  __syncthreads();
  const int row = threadIdx.x >> 4, chunk = threadIdx.x & 15;
  const int col = 16 * j0 + 16 * chunk;
  if (col < out_features)
    *reinterpret_cast<u32x4 *>(w8 + (size_t)(16 * i + row) * out_features + col) =
        *reinterpret_cast<const u32x4 *>(&stage[row][16 * chunk]);
}

hipError_t launch_decode_tiles_e4m3(const int16_t *code, int K, int in_features, int out_features, uint8_t *w8,
                                    hipStream_t stream) {
  const int Ti = in_features / 16, Tj = out_features / 16;
  if (Ti == 0 || Tj == 0) return hipSuccess;
  dim3 grid((Tj + 15) / 16, Ti), block(256);
  const uint32_t *c = reinterpret_cast<const uint32_t *>(code);
  switch (K) {
    case 2: decode_tiles_e4m3_kernel<2><<<grid, block, 0, stream>>>(c, Tj, w8, out_features); break;
    case 3: decode_tiles_e4m3_kernel<3><<<grid, block, 0, stream>>>(c, Tj, w8, out_features); break;
    case 4: decode_tiles_e4m3_kernel<4><<<grid, block, 0, stream>>>(c, Tj, w8, out_features); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_tiles(const int16_t *code, int K, int in_features, int out_features,
                               uint16_t *w_hat, uint16_t *states, hipStream_t stream) {
  const int Ti = in_features / 16, Tj = out_features / 16;
  if (Ti == 0 || Tj == 0) return hipSuccess;
  dim3 grid((Tj + 7) / 8, Ti), block(256);
  const uint32_t *c = reinterpret_cast<const uint32_t *>(code);
  switch (K) {
    case 2: decode_tiles_kernel<2><<<grid, block, 0, stream>>>(c, Tj, w_hat, out_features, states); break;
    case 3: decode_tiles_kernel<3><<<grid, block, 0, stream>>>(c, Tj, w_hat, out_features, states); break;
    case 4: decode_tiles_kernel<4><<<grid, block, 0, stream>>>(c, Tj, w_hat, out_features, states); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trellis
