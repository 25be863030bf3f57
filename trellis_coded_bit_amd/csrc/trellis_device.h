// Device-side building blocks shared by the gfx950 kernels of libtrellis.
//
// Method sources (page title, section):
//   * "The escha W2 format, recovered and verified": "Bit layout" (tile words read as
//     32-bit words, MSB-first windows ending at each symbol's own K bits, circular) and
//     "Codebook: cb=1 (MCG), verified" (multiply, mask/xor, sum of two fp16 halves).
//   * "Escha-W2 runs on Metal": tile/permutation paragraph (symbol -> tile row/column).
//
// Lane <-> symbol assignment used by every kernel.  Lane l of a wave (n = l & 15,
// g = l >> 4) owns the four consecutive symbols s0 + {0,1,2,3} of a tile with
//     s0 = 32*(n & 7) + 8*g + 4*(n >> 3).
// By the tile permutation these four symbols all lie in tile column n and in tile rows
// {2g, 2g+1, 2g+8, 2g+9}.  Their four 16-bit windows span 16 + 3K <= 28 consecutive
// stream bits, so one 32-bit funnel shift of two tile words holds all of them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trellis {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

// The MCG hash ("Codebook: cb=1"): v = s * 0xCBAC1FED mod 2^32, then (v & 0x8FFF8FFF) ^
// 0x3B603B60.  The result, read as two fp16 halves, sums to the codebook value.
__device__ __forceinline__ uint32_t mcg_hash(uint32_t state) {
  uint32_t v = state * 0xCBAC1FEDu;
  return (v & 0x8FFF8FFFu) ^ 0x3B603B60u;
}

// fp16 codebook value: one binary16 round-to-nearest-even of lo + hi.
__device__ __forceinline__ _Float16 mcg_value(uint32_t h) {
  _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
  _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(h >> 16));
  return lo + hi;
}

// Codebook values of two hash words as an fp16 pair (a in the low half, b in the high
// half), one round-to-nearest-even per value.  Each value is one fp16 add of a word's two
// halves with SDWA operand selects; the second writes the high half and keeps the low one.
// Two instructions per pair, against two v_perm_b32 and a packed add when the halves are
// gathered first.
__device__ __forceinline__ uint32_t mcg_value2(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_add_f16_sdwa %0, %1, %1 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:WORD_1"
      : "=v"(r) : "v"(a));
  asm("v_add_f16_sdwa %0, %1, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0 src1_sel:WORD_1"
      : "+v"(r) : "v"(b));
  return r;
}

// The E4M3 codebook ("EXLR8" page, E4M3 paragraph: every codebook value is rounded to E4M3,
// nearest with ties to even, saturating).  Four hash words -> their fp16 values -> four
// E4M3 bytes, value j in byte j.  gfx950's scaled conversion with scale 1.0 rounds to
// nearest even; the codebook's magnitudes stay below 4, far inside E4M3's range of 448, so
// how it saturates never matters here.
__device__ __forceinline__ uint32_t e4m3_pack4(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3) {
  typedef _Float16 hv2 __attribute__((ext_vector_type(2)));
  typedef short sv2 __attribute__((ext_vector_type(2)));
  const sv2 zero = {0, 0};
  sv2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(zero, __builtin_bit_cast(hv2, mcg_value2(h0, h1)), 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, __builtin_bit_cast(hv2, mcg_value2(h2, h3)), 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Per-lane window geometry inside a tile of K-bit symbols (8K 32-bit words).
// The lane's four windows start at stream bit `start` = K*s0 + K - 16 (mod 256K).
// Writing start = 32*d0 + off with off in [1, 32], the 32 stream bits beginning at `start`
// are alignbit(word[d0], word[d1], 32 - off) with d1 = d0 + 1 (mod 8K); window j is then
// bits [16 - j*K, 32 - j*K) of that register.
struct LaneWindow {
  uint32_t d0, d1, sh;
};

__device__ __forceinline__ LaneWindow lane_window(int lane, int K) {
  const int n = lane & 15, g = lane >> 4;
  const int s0 = 32 * (n & 7) + 8 * g + 4 * (n >> 3);
  const int nbits = 256 * K, nwords = 8 * K;
  int start = K * s0 + K - 16;
  if (start <= 0) start += nbits;  // start in [1, nbits]
  const int d0 = (start - 1) >> 5;
  const int off = start - 32 * d0;  // [1, 32]
  LaneWindow w;
  w.d0 = (uint32_t)d0;
  w.d1 = (uint32_t)((d0 + 1) % nwords);
  w.sh = (uint32_t)(32 - off);
  return w;
}

// 32 stream bits starting at the lane's first window.
__device__ __forceinline__ uint32_t lane_bits(uint32_t w0, uint32_t w1, uint32_t sh) {
  return __builtin_amdgcn_alignbit(w0, w1, sh);
}

// State of the lane's symbol s0 + j.
template <int K>
__device__ __forceinline__ uint32_t lane_state(uint32_t bits, int j) {
  return (bits >> (16 - j * K)) & 0xFFFFu;
}

// Tile row of the lane's symbol s0 + j (j = 0..3): 2g, 2g+1, 2g+8, 2g+9.
__device__ __forceinline__ int lane_row(int lane, int j) {
  return 2 * (lane >> 4) + (j & 1) + 8 * (j >> 1);
}

// threadIdx.x, opaque to the optimiser: values derived from it are recomputed where they
// are used instead of being hoisted to kernel entry and kept live across loops (in kernels
// that inline several code paths the hoisted copies of every path's lane constants spill).
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Loads through the global address space (the pointers reach the kernels inside structs,
// so the compiler cannot infer the address space and would otherwise emit flat loads).
template <typename T>
__device__ __forceinline__ T ldg(const T *p) {
  return *(const __attribute__((address_space(1))) T *)p;
}

// Raw buffer resource over `bytes` bytes at `base` (loads past the end return zero, stores
// past it are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Cache-policy operand of the buffer intrinsics: SC1, device (agent) scope.  Data that one
// workgroup stores and another (possibly on another XCD, with its own L2) reads after a
// device-scope atomic is written and read with it.
constexpr int kSC1 = 16;

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Value of lane (lane ^ m) for m = 1, 2, 4, 8 (DPP within rows of 16), 16 (swizzle within
// halves of the wave) and 32 (bpermute).  The DPP forms (every source lane valid) are
// written as updates with bound_ctrl so the compiler can fold the move into the VALU
// operation that consumes it.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __builtin_bit_cast(int, v);
  int r;
  if constexpr (M == 1) r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true);   // quad_perm 1,0,3,2
  else if constexpr (M == 2) r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
  else if constexpr (M == 4)  // row_half_mirror (i -> 7 - i) then quad_perm 3,2,1,0: i -> i ^ 4
    r = __builtin_amdgcn_update_dpp(0, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true), 0x1B, 0xF, 0xF,
                                    true);
  else if constexpr (M == 8) r = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, true);  // row_ror 8
  else if constexpr (M == 16) r = __builtin_amdgcn_ds_swizzle(x, 0x401F);                 // xor 16
  else r = __shfl_xor(x, M, 64);
  return __builtin_bit_cast(float, r);
}

// One butterfly stage across lanes: partner + own on the lane whose stride bit is clear,
// partner - own on the other (one sign select and one add that takes the partner by DPP).
template <int M>
__device__ __forceinline__ void fwht_stage(float &a, float &b, int lane) {
  const float sg = (lane & M) ? -1.f : 1.f;
  a = lane_xor<M>(a) + sg * a;
  b = lane_xor<M>(b) + sg * b;
}

// The four butterfly stages across the 16 lanes of a row (strides 1, 2, 4, 8), for values
// held one per lane and row.
__device__ __forceinline__ void fwht_stage1(float &v, int lane) {
  v = lane_xor<1>(v) + ((lane & 1) ? -v : v);
  v = lane_xor<2>(v) + ((lane & 2) ? -v : v);
  v = lane_xor<4>(v) + ((lane & 4) ? -v : v);
  v = lane_xor<8>(v) + ((lane & 8) ? -v : v);
}

// Unnormalised Sylvester Hadamard butterfly over 128 values held two per lane: element
// e = 64*h + lane in (a, b)[h] with the in-register stage pairing h, or any other fixed
// assignment of the seven index bits to (h, lane bits) -- H_128 is the tensor product of
// seven 2x2 butterflies, so the stages may run in any order and the output uses the same
// assignment as the input.
__device__ __forceinline__ void wave_fwht128(float &a, float &b) {
  const int lane = opaque_tid() & 63;
  const float s = a + b, d = a - b;
  a = s;
  b = d;
  fwht_stage<1>(a, b, lane);
  fwht_stage<2>(a, b, lane);
  fwht_stage<4>(a, b, lane);
  fwht_stage<8>(a, b, lane);
  fwht_stage<16>(a, b, lane);
  fwht_stage<32>(a, b, lane);
}

}  // namespace trellis
