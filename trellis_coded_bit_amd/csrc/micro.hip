// Microbenchmarks of the hardware ceilings under the trellis-coded products (the public
// contract is in include/trellis_micro.h): cold HBM stream read, vector-instruction issue
// costs of the codebook decode, and matrix-instruction rates.
//
// Each timed loop reads the shader clock (s_memtime) and the constant 100 MHz clock
// (s_memrealtime) before and after; the host turns cycles into clocks per instruction per
// SIMD and the ratio of the two clocks into the shader frequency under that load.
#include "../../include/trellis_micro.h"
#include "launch.h"
#include "trellis_device.h"

namespace trellis {
namespace {

constexpr int kMicroThreads = 256;  // four waves: one per SIMD when a CU holds one workgroup

struct Clocks {
  uint64_t c, t;
};
__device__ __forceinline__ Clocks clocks_now() {
  Clocks k;
  asm volatile("s_memtime %0\n s_memrealtime %1\n s_waitcnt lgkmcnt(0)" : "=s"(k.c), "=s"(k.t));
  return k;
}
__device__ __forceinline__ void clocks_store(const Clocks &a, const Clocks &b, uint64_t *cycles, uint64_t *ticks) {
  if (threadIdx.x == 0) {
    cycles[blockIdx.x] = b.c - a.c;
    ticks[blockIdx.x] = b.t - a.t;
  }
}

// ---------------------------------------------------------------------------------------
// Stream read
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kMicroThreads) void stream_read_kernel(const u32x4 *buf, size_t n16, uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * kMicroThreads;
  size_t i = (size_t)blockIdx.x * kMicroThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i), b = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride), d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
  sink[(size_t)blockIdx.x * kMicroThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// ---------------------------------------------------------------------------------------
// Single vector instructions: 8 independent chains, 64 instructions per iteration.
// ---------------------------------------------------------------------------------------
template <int OP>
__device__ __forceinline__ void one_op(uint32_t &a, uint32_t s1, uint32_t v2) {
  if constexpr (OP == TRELLIS_MICRO_V_ADD_U32) asm volatile("v_add_u32 %0, %0, %1" : "+v"(a) : "v"(v2));
  else if constexpr (OP == TRELLIS_MICRO_V_MUL_LO_U32) asm volatile("v_mul_lo_u32 %0, %0, %1" : "+v"(a) : "s"(s1));
  else if constexpr (OP == TRELLIS_MICRO_V_MUL_U32_U24) asm volatile("v_mul_u32_u24 %0, %1, %0" : "+v"(a) : "s"(s1));
  else if constexpr (OP == TRELLIS_MICRO_V_MAD_U32_U24) asm volatile("v_mad_u32_u24 %0, %0, %1, %2" : "+v"(a) : "s"(s1), "v"(v2));
  else if constexpr (OP == TRELLIS_MICRO_V_MAD_U32_U16)
    asm volatile("v_mad_u32_u16 %0, %0, %1, %2 op_sel:[1,0,0,0]" : "+v"(a) : "s"(s1), "v"(v2));
  else if constexpr (OP == TRELLIS_MICRO_V_MUL_LO_U16_SDWA)
    asm volatile("v_mul_lo_u16_sdwa %0, %0, %1 dst_sel:WORD_1 dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:WORD_0"
                 : "+v"(a) : "v"(v2));
  else if constexpr (OP == TRELLIS_MICRO_V_PK_MUL_LO_U16) asm volatile("v_pk_mul_lo_u16 %0, %0, %1" : "+v"(a) : "v"(v2));
  else if constexpr (OP == TRELLIS_MICRO_V_BFE_U32) asm volatile("v_bfe_u32 %0, %0, 7, 16" : "+v"(a));
  else if constexpr (OP == TRELLIS_MICRO_V_ALIGNBIT_B32) asm volatile("v_alignbit_b32 %0, %0, %1, %2" : "+v"(a) : "v"(v2), "v"(s1));
  else if constexpr (OP == TRELLIS_MICRO_V_PERM_B32) asm volatile("v_perm_b32 %0, %0, %1, %2" : "+v"(a) : "v"(v2), "s"(s1));
  else if constexpr (OP == TRELLIS_MICRO_V_BITOP3_B32)
    asm volatile("v_bitop3_b32 %0, %0, %1, %2 bitop3:0x6a" : "+v"(a) : "s"(s1), "v"(v2));
  else if constexpr (OP == TRELLIS_MICRO_V_LSHRREV_B32) asm volatile("v_lshrrev_b32 %0, 3, %0" : "+v"(a));
  else if constexpr (OP == TRELLIS_MICRO_V_ADD_F16_SDWA)
    asm volatile("v_add_f16_sdwa %0, %0, %0 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0 src1_sel:WORD_1"
                 : "+v"(a));
  else if constexpr (OP == TRELLIS_MICRO_V_MUL_U32_U24_SDWA)
    asm volatile("v_mul_u32_u24_sdwa %0, %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
                 : "+v"(a) : "s"(s1));
  else if constexpr (OP == TRELLIS_MICRO_V_FMA_F32) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a) : "s"(s1), "v"(v2));
}

template <int OP>
__global__ __launch_bounds__(kMicroThreads) void valu_kernel(int iters, uint32_t s1, uint64_t *cycles, uint64_t *ticks,
                                                             uint32_t *sink) {
  uint32_t a[8];
  const uint32_t v2 = threadIdx.x * 0x9E3779B9u + 0x3C00u;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (threadIdx.x + 1u) * (2u * i + 3u) + 0x3C003C00u;
  const Clocks k0 = clocks_now();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) one_op<OP>(a[i], s1, v2);
  }
  const Clocks k1 = clocks_now();
  clocks_store(k0, k1, cycles, ticks);
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) x ^= a[i];
  sink[(size_t)blockIdx.x * kMicroThreads + threadIdx.x] = x;
}

// ---------------------------------------------------------------------------------------
// Whole per-tile decodes.  Each wave holds 16 tiles' code words in LDS (K = 3: 24 words
// per tile); per tile a lane reads its two window words, decodes its four states and hands
// the four hash words on (to LDS, or to one MFMA).  The LDS traffic is what the products
// have per tile; the vector instructions are the decode's.
// ---------------------------------------------------------------------------------------
constexpr int kDecK = 3, kDecNW = 8 * kDecK, kDecTiles = 16;

// The 24-bit form: v = s * 0xCBAC1FED mod 2^32 = s * 0xAC1FED + ((s * 0xCB) mod 2^8) << 24,
// each product on the 24-bit multiplier reading the state's 16-bit half directly.
__device__ __forceinline__ uint32_t hash_u24_hi(uint32_t x, uint32_t c24, uint32_t c8) {
  uint32_t p, t;
  asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
      : "=v"(p) : "v"(x), "s"(c24));
  asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
      : "=v"(t) : "v"(x), "s"(c8));
  return ((p + t) & 0x8FFF8FFFu) ^ 0x3B603B60u;
}
__device__ __forceinline__ uint32_t hash_u24_lo(uint32_t x, uint32_t c24, uint32_t c8) {
  uint32_t p, t;
  asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:DWORD"
      : "=v"(p) : "v"(x), "s"(c24));
  asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:DWORD"
      : "=v"(t) : "v"(x), "s"(c8));
  return ((p + t) & 0x8FFF8FFFu) ^ 0x3B603B60u;
}

template <int OP>
__global__ __launch_bounds__(kMicroThreads) void decode_kernel(int iters, uint32_t c24, uint64_t *cycles, uint64_t *ticks,
                                                               uint32_t *sink) {
  __shared__ uint32_t words[4][kDecTiles * kDecNW];
  __shared__ u32x4 out[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = lane; i < kDecTiles * kDecNW; i += 64) words[wave][i] = (i + 1u) * 0x9E3779B9u ^ threadIdx.x;
  __syncthreads();
  const LaneWindow lw = lane_window(lane, kDecK);
  const uint32_t *w = words[wave];
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const half8 av = __builtin_bit_cast(half8, u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
  u32x4 fold = {0u, 0u, 0u, 0u};
  const Clocks k0 = clocks_now();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < kDecTiles; ++t) {
      const uint32_t *tw = w + t * kDecNW;
      uint32_t w0 = tw[lw.d0], w1 = tw[lw.d1];
      asm volatile("" : "+v"(w0), "+v"(w1));  // new words every iteration for the compiler
      u32x4 bw;
      if constexpr (OP == TRELLIS_MICRO_DECODE_TILE_U24) {
        // states at stream offsets 16, 13, 10, 7 of the lane's 32-bit window: the first is
        // the high half of the funnel, the others the low half of three more funnels
        const uint32_t b0 = lane_bits(w0, w1, lw.sh);
        const uint32_t b1 = lane_bits(w0, w1, (lw.sh + 13) & 31), b2 = lane_bits(w0, w1, (lw.sh + 10) & 31),
                       b3 = lane_bits(w0, w1, (lw.sh + 7) & 31);
        bw[0] = hash_u24_hi(b0, c24, 0xCBu);
        bw[1] = hash_u24_lo(b1, c24, 0xCBu);
        bw[2] = hash_u24_lo(b2, c24, 0xCBu);
        bw[3] = hash_u24_lo(b3, c24, 0xCBu);
      } else {
        const uint32_t bits = lane_bits(w0, w1, lw.sh);
        bw[0] = mcg_hash(lane_state<kDecK>(bits, 0));
        bw[1] = mcg_hash(lane_state<kDecK>(bits, 1));
        bw[2] = mcg_hash(lane_state<kDecK>(bits, 2));
        bw[3] = mcg_hash(lane_state<kDecK>(bits, 3));
      }
      if constexpr (OP == TRELLIS_MICRO_DECODE_TILE_MFMA)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8, bw), acc, 0, 0, 0);
      else
        asm volatile("" ::"v"(bw[0]), "v"(bw[1]), "v"(bw[2]), "v"(bw[3]));  // the words are used
    }
  }
  out[wave][lane] = u32x4{w[lane], w[lane + 64], w[lane + 128], w[lane + 192]};
  const Clocks k1 = clocks_now();
  clocks_store(k0, k1, cycles, ticks);
  fold = out[wave][lane];
  sink[(size_t)blockIdx.x * kMicroThreads + threadIdx.x] =
      fold[0] ^ fold[1] ^ fold[2] ^ fold[3] ^ __builtin_bit_cast(uint32_t, acc[0] + acc[1] + acc[2] + acc[3]);
}

// ---------------------------------------------------------------------------------------
// Matrix instructions: 8 independent accumulators per wave.
// ---------------------------------------------------------------------------------------
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(kMicroThreads) void mfma_kernel(int iters, uint64_t *cycles, uint64_t *ticks, float *sink) {
  const u32x4 ai = {threadIdx.x, 0x3C003C00u, 0x38003800u, 0x34003400u};
  const half8 ha = __builtin_bit_cast(half8, ai), hb = __builtin_bit_cast(half8, ai ^ 0x00010001u);
  const intx8 fa = {(int)threadIdx.x, 0x38383838, 0x30303030, 0x28282828, 1, 2, 3, 4};
  const intx8 fb = {0x38383838, (int)threadIdx.x, 5, 6, 7, 8, 0x30303030, 0x28282828};
  float s = 0.f;
  Clocks k0, k1;
  if constexpr (KIND == TRELLIS_MICRO_MFMA_F16_16X16X32 || KIND == TRELLIS_MICRO_MFMA_F8_16X16X128) {
    floatx4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // (a run-time start value: from constants the compiler builds the accumulators out of
      // overlapping register ranges and copies them every iteration)
      const float f = (float)(threadIdx.x + j);
      acc[j] = floatx4{f, f, f, f};
    }
    k0 = clocks_now();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (KIND == TRELLIS_MICRO_MFMA_F16_16X16X32)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, hb, acc[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb, acc[j], 0, 0, 0, 0, 0, 0);
      }
      // (keeps each accumulator in one accumulator-register range across iterations)
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[j]));
    }
    k1 = clocks_now();
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][3];
  } else {
    floatx16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = (float)(j + e);
    k0 = clocks_now();
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (KIND == TRELLIS_MICRO_MFMA_F16_32X32X16)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, hb, acc[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[j], 0, 0, 0, 0, 0, 0);
      }
    k1 = clocks_now();
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][15];
  }
  clocks_store(k0, k1, cycles, ticks);
  sink[(size_t)blockIdx.x * kMicroThreads + threadIdx.x] = s;
}

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

}  // namespace

int micro_cus() { return cu_count(); }

hipError_t launch_micro_stream_read(const void *buf, size_t bytes, int blocks, uint32_t *sink, hipStream_t stream) {
  if (blocks <= 0) blocks = 8 * cu_count();
  stream_read_kernel<<<blocks, kMicroThreads, 0, stream>>>(static_cast<const u32x4 *>(buf), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_micro_valu(int op, int iters, int wps, uint64_t *cycles, uint64_t *ticks, uint32_t *sink,
                             hipStream_t stream, int *blocks_out) {
  const int blocks = cu_count() * wps;
  *blocks_out = blocks;
  const uint32_t s1 = 0xCBAC1FEDu;
#define TRELLIS_MICRO_V(ID) \
  case ID: valu_kernel<ID><<<blocks, kMicroThreads, 0, stream>>>(iters, s1, cycles, ticks, sink); break;
  switch (op) {
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_ADD_U32)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_MUL_LO_U32)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_MUL_U32_U24)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_MAD_U32_U24)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_MAD_U32_U16)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_MUL_LO_U16_SDWA)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_PK_MUL_LO_U16)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_BFE_U32)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_ALIGNBIT_B32)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_PERM_B32)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_BITOP3_B32)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_LSHRREV_B32)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_ADD_F16_SDWA)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_MUL_U32_U24_SDWA)
    TRELLIS_MICRO_V(TRELLIS_MICRO_V_FMA_F32)
    case TRELLIS_MICRO_DECODE_TILE:
      decode_kernel<TRELLIS_MICRO_DECODE_TILE><<<blocks, kMicroThreads, 0, stream>>>(iters, 0xAC1FEDu, cycles, ticks, sink);
      break;
    case TRELLIS_MICRO_DECODE_TILE_MFMA:
      decode_kernel<TRELLIS_MICRO_DECODE_TILE_MFMA><<<blocks, kMicroThreads, 0, stream>>>(iters, 0xAC1FEDu, cycles, ticks,
                                                                                          sink);
      break;
    case TRELLIS_MICRO_DECODE_TILE_U24:
      decode_kernel<TRELLIS_MICRO_DECODE_TILE_U24><<<blocks, kMicroThreads, 0, stream>>>(iters, 0xAC1FEDu, cycles, ticks,
                                                                                         sink);
      break;
    default: return hipErrorInvalidValue;
  }
#undef TRELLIS_MICRO_V
  return hipGetLastError();
}

hipError_t launch_micro_mfma(int kind, int iters, int wps, uint64_t *cycles, uint64_t *ticks, float *sink,
                             hipStream_t stream, int *blocks_out) {
  const int blocks = cu_count() * wps;
  *blocks_out = blocks;
  switch (kind) {
    case TRELLIS_MICRO_MFMA_F16_16X16X32:
      mfma_kernel<TRELLIS_MICRO_MFMA_F16_16X16X32><<<blocks, kMicroThreads, 0, stream>>>(iters, cycles, ticks, sink);
      break;
    case TRELLIS_MICRO_MFMA_F16_32X32X16:
      mfma_kernel<TRELLIS_MICRO_MFMA_F16_32X32X16><<<blocks, kMicroThreads, 0, stream>>>(iters, cycles, ticks, sink);
      break;
    case TRELLIS_MICRO_MFMA_F8_16X16X128:
      mfma_kernel<TRELLIS_MICRO_MFMA_F8_16X16X128><<<blocks, kMicroThreads, 0, stream>>>(iters, cycles, ticks, sink);
      break;
    case TRELLIS_MICRO_MFMA_F8_32X32X64:
      mfma_kernel<TRELLIS_MICRO_MFMA_F8_32X32X64><<<blocks, kMicroThreads, 0, stream>>>(iters, cycles, ticks, sink);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trellis
