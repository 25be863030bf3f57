// trellis_gemm: prefill product Y = had(had(X*su) @ W_hat) * sv for M rows.
//
// ("Escha-W2 runs on Metal", reconstruction paragraph; decode as in decode.hip.)
//
// Two launches:
//   1. rotate: XH = H128(X*su) (unnormalised butterfly, times an exact 2^-4) as fp16 in the
//      workspace (after its reserved region), stored in
//      1 KB blocks of 16 rows x one k-step laid out exactly as the MFMA A operands are held
//      by the lanes, so every A-operand load is one contiguous, fully used 1 KB piece.  It
//      also clears the split-tile counters.
//   2. the stream-K product.  Output tiles are 512 rows x 128 columns (one Hadamard block)
//      and a tile's k-steps are 32 input rows (two trellis tile rows), taken in pairs.  The
//      (tile, k-step pair) iterations are numbered tile-major and each of the G workgroups
//      (one per CU) takes one contiguous range of them, so every workgroup does the same
//      work whatever the tile count; consecutive ranges go to the same XCD (the dispatcher
//      deals workgroups round-robin over the XCDs).
//
//      A workgroup is 8 waves; wave w owns output rows 64w..64w+63 of the tile (4 x 8
//      blocks of 16x16, fp32 accumulators) and, per k-step, decodes the two trellis tile
//      rows of column block w directly into one MFMA B operand: by the lane assignment of
//      the decoder a lane's four symbols of a tile sit in one tile column and four tile
//      rows, so the lane holds, for its column, eight weights along k -- exactly one B
//      operand of v_mfma_f32_16x16x32_f16 once k inside the step is numbered as the lanes
//      hold it.  The operands go through a two-slot LDS ring (1 KB per column block) so all
//      waves use all eight column blocks; half of them are read right after the barrier
//      that publishes a step and half a step later, behind 16 MFMAs.  Codes (one 4-byte
//      word per lane covers a step's two tiles) go through a wave-private LDS ring; codes
//      and activations are loaded two k-steps ahead into registers.  The codebook's fp16
//      addition (one rounding) happens in the decoder, so B holds the format's exact fp16
//      weights.
//
//      A range covering a whole tile finishes it: output Hadamard across the tile's 128
//      columns (16 lanes x 8 registers per row), scales, the exact 2^-3 left of the two
//      1/sqrt(128) (2^-7 for the FP8 product, whose row scales undo the quantisation), fp16
//      stores.
//      A tile split between two ranges: the first contributor to arrive stores its fp32
//      partial tile; the second adds it to its registers and finishes the tile.  Tiles
//      split among three or more (short ranges): every contributor stores, the last to
//      arrive adds all partials in range order.  Nobody waits for a workgroup that has not
//      arrived.
#include <cstdlib>

#include "launch.h"
#include "trellis_device.h"

namespace trellis {

namespace {

constexpr int kMT = 512;      // output rows per tile
constexpr int kNT = 128;      // output columns per tile (one Hadamard block)
constexpr int kKS = 32;       // input rows per k-step (two trellis tile rows)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileFloats = kMT * kNT;
constexpr int kMinSteps = 4;  // fewest k-step pairs per workgroup worth a split

struct GemmParams {
  const uint16_t *xh;  // rotated activations in 16-row x k-step blocks (rotate_kernel;
                       // E4M3 bytes for the FP8 product)
  const float *rowscale;  // FP8 product: per-row dequantisation scale [Mpad], else unused
  const uint32_t *code;
  const uint16_t *rout;
  const float *s_out;
  uint16_t *y;
  float *partials;     // [2G][kTileFloats]
  uint32_t *counters;  // [T][2] (arrived, stored) per tile, zeroed by the rotation launch
  uint32_t *errword;   // the workspace's error word
  int M, in, out;
  int S;               // k-step pairs per tile (the unit of the ranges)
  int nNT;             // column tiles
  int G;               // workgroups
  int q;               // iterations per workgroup (the first r take one more)
  int r;
};

// Iteration counts fit in 32 bits (checked at launch).
__device__ __forceinline__ int range_start(const GemmParams &P, int g) {
  return g * P.q + (g < P.r ? g : P.r);
}

__device__ __forceinline__ int range_owner(const GemmParams &P, int i) {
  const int big = P.r * (P.q + 1);
  return i < big ? i / (P.q + 1) : P.r + (i - big) / P.q;
}

// Workgroup b runs on XCD b % 8; give each XCD a contiguous block of ranges.
__device__ __forceinline__ int xcd_range(int b, int G) {
  const int x = b & 7, j = b >> 3;
  return x * (G >> 3) + min(x, G & 7) + j;
}

// Layout of the rotated activations XH: blocks of 16 rows x one k-step (32 input rows),
// 1 KB each, ordered [row block][k-step]; inside a block, MFMA lane l = 16*g + (m & 15)
// owns 16 contiguous bytes holding its eight A-operand elements j = 0..7, which are the
// step's input rows 16*(j >> 2) + 2*g + (j & 1) + 8*((j >> 1) & 1) -- the tile rows of the
// decoder's symbols j & 3 in the step's tile row j >> 2 (trellis_device.h).  Every
// A-operand load is then one contiguous, fully used 1 KB piece.
//
// XH = H128(X*su): a workgroup per (16-row block, 128-column block), 16 lanes per row with
// 8 consecutive elements each (three in-register butterfly stages, four across the 16
// lanes).  The 4 KB of output (four consecutive 1 KB k-step blocks) is assembled in LDS and
// stored with 16 contiguous bytes per thread.  Rows past M are written as zeros.
// VEC: rin and s_in are 16-byte aligned (vector loads), else element loads.
template <bool VEC>
__global__ __launch_bounds__(256) void rotate_kernel(const uint16_t *__restrict__ x, int rows, int n,
                                                     const uint16_t *__restrict__ r,
                                                     const float *__restrict__ s,
                                                     uint16_t *__restrict__ xh,
                                                     uint32_t *__restrict__ counters, int ncounters) {
  __shared__ __attribute__((aligned(16))) uint16_t stage[4 * 512];
  for (int c = blockIdx.x * 256 + threadIdx.x; c < ncounters; c += gridDim.x * 256) counters[c] = 0;
  const int nb = n / 128;
  const int rb = blockIdx.x / nb, blk = blockIdx.x - rb * nb;
  const int q = threadIdx.x >> 4;  // row of the block
  const int i = threadIdx.x & 15;  // elements 8i .. 8i+7 of the 128-block
  const int row = 16 * rb + q;
  const int c = blk * 128 + 8 * i;
  float v[8];
  if (row < rows) {
    const u32x4 xv = *reinterpret_cast<const u32x4 *>(x + (size_t)row * n + c);
    if (VEC) {
      const u32x4 rv = *reinterpret_cast<const u32x4 *>(r + c);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t xw = xv[t >> 1], rw = rv[t >> 1];
        const uint16_t xs = (t & 1) ? (uint16_t)(xw >> 16) : (uint16_t)xw;
        const uint16_t rs = (t & 1) ? (uint16_t)(rw >> 16) : (uint16_t)rw;
        v[t] = h2f(xs) * h2f(rs);
      }
      if (s) {
        const floatx4 s0 = *reinterpret_cast<const floatx4 *>(s + c);
        const floatx4 s1 = *reinterpret_cast<const floatx4 *>(s + c + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[t] *= s0[t];
          v[t + 4] *= s1[t];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t xw = xv[t >> 1];
        const uint16_t xs = (t & 1) ? (uint16_t)(xw >> 16) : (uint16_t)xw;
        v[t] = h2f(xs) * h2f(r[c + t]);
        if (s) v[t] *= s[c + t];
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = 0.f;
  }
  // element index bits 0..2: register t, bits 3..6: lane i
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if ((t & h) == 0) {
        const float a = v[t], b = v[t + h];
        v[t] = a + b;
        v[t + h] = a - b;
      }
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    float p;
    p = lane_xor<1>(v[t]);
    v[t] = (lane & 1) ? (p - v[t]) : (v[t] + p);
    p = lane_xor<2>(v[t]);
    v[t] = (lane & 2) ? (p - v[t]) : (v[t] + p);
    p = lane_xor<4>(v[t]);
    v[t] = (lane & 4) ? (p - v[t]) : (v[t] + p);
    p = lane_xor<8>(v[t]);
    v[t] = (lane & 8) ? (p - v[t]) : (v[t] + p);
  }
  // element 8i + t is row kk = 8*(i & 3) + t of the block's k-step i >> 2: operand group
  // g = t >> 1, element j = 2*(i & 3) + (t & 1), stored at lane slot 16*g + q
  uint16_t *dst = stage + (i >> 2) * 512 + q * 8 + 2 * (i & 3);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    // stored times 2^-4 (exact): close to the normalised 2^-3.5, so a block whose normalised
    // rotation fits fp16 does not overflow here
    const half2_t pr = {(_Float16)(v[2 * g] * 0.0625f), (_Float16)(v[2 * g + 1] * 0.0625f)};
    *reinterpret_cast<half2_t *>(dst + 16 * 8 * g) = pr;
  }
  __syncthreads();
  const int S32 = n / 32;
  uint16_t *out = xh + ((size_t)rb * S32 + 4 * blk) * 512;
  reinterpret_cast<u32x4 *>(out)[threadIdx.x] = reinterpret_cast<const u32x4 *>(stage)[threadIdx.x];
}

// Four symbols of one tile for this lane -> fp16 codebook values packed in pairs
// (symbols 0,1 and 2,3: tile rows 2g, 2g+1 and 2g+8, 2g+9 of column n).  CB = 2: each
// value rounded to E4M3 and converted back to fp16 (exact), the E4M3 codebook ("EXLR8").
template <int K, int CB = 1>
__device__ __forceinline__ u32x2 decode_pairs(uint32_t w0, uint32_t w1, uint32_t sh) {
  const uint32_t bits = lane_bits(w0, w1, sh);
  uint32_t h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = mcg_hash(lane_state<K>(bits, j));
  u32x2 out;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if constexpr (CB == 1) {
      // one fp16 add of each word's halves (SDWA selects), value 2p low, 2p + 1 high
      out[p] = mcg_value2(h[2 * p], h[2 * p + 1]);
    } else {
      const uint32_t lo = __builtin_amdgcn_perm(h[2 * p + 1], h[2 * p], 0x05040100u);  // lo halves
      const uint32_t hi = __builtin_amdgcn_perm(h[2 * p + 1], h[2 * p], 0x07060302u);  // hi halves
      const half2_t v = __builtin_bit_cast(half2_t, lo) + __builtin_bit_cast(half2_t, hi);
      typedef short sv2 __attribute__((ext_vector_type(2)));
      const sv2 q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(sv2{0, 0}, v, 1.0f, false);
      out[p] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_bit_cast(uint32_t, q), 1.0f, false));
    }
  }
  return out;
}

// Waits for this wave's LDS operations, then a workgroup barrier.  Unlike __syncthreads()
// it does not wait for outstanding global loads (the prefetched operands).  No instruction
// is scheduled across it, so each half-step's decode stays after the loads it consumes
// were given a full half-step to arrive.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

typedef floatx4 Acc[4][8];

// Output Hadamard, scales and stores for tile (mt, nt).  Lane holds rows
// 64*wave + 16*mb + 4*(lane >> 4) + r and columns 16*nb + (lane & 15).

// Staging through LDS uses the wave's own 1 KB of B ring slot 0 (idle between pieces).
// F8: the rows carry the activations' dequantisation scales (rowscale), applied with sv.
template <bool F8 = false>
__device__ __forceinline__ void finish_tile(const GemmParams &P, Acc &acc, int mt, int nt, u32x4 *ring0) {
  const int lane = threadIdx.x & 63, n16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float sg1 = (lane & 1) ? -1.f : 1.f, sg2 = (lane & 2) ? -1.f : 1.f;
  const float sg4 = (lane & 4) ? -1.f : 1.f, sg8 = (lane & 8) ? -1.f : 1.f;
  uint16_t *stage = reinterpret_cast<uint16_t *>(ring0 + (F8 ? 128 : 64) * wave);
  // the wave's 64 rows of the tile's output (uniform); stores to rows past M fall outside
  // the buffer range and are dropped
  const int wrow0 = mt * kMT + 64 * wave;
  const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(P.y + (size_t)wrow0 * P.out + nt * kNT,
                                                (long long)(P.M - wrow0) * P.out * 2 - nt * kNT * 2);
  float sv[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int col = nt * kNT + 16 * nb + n16;
    // fp16 product: the activations were stored times 2^-4, so 2^-7 / 2^-4 remains; FP8:
    // the row scales restore the unnormalised activations, 2^-7 remains
    float s = h2f(P.rout[col]) * (F8 ? (1.0f / 128.0f) : (1.0f / 8.0f));
    if (P.s_out) s *= P.s_out[col];
    sv[nb] = s;
  }
  uint32_t rs[4][4];  // f32 bits
  if constexpr (F8) {
    // rows past the padded row count read as zero (their stores are dropped anyway)
    const int Mpad = (P.M + 15) & ~15;
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(P.rowscale + wrow0, (long long)(Mpad - wrow0) * 4);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rs[mb][r] = __builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)(16 * mb + 4 * (lane >> 4) + r) * 4, 0, 0);
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb] = acc[mb][nb][r];
      if constexpr (F8) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) v[nb] *= __builtin_bit_cast(float, rs[mb][r]);
      }
      // column strides 16, 32, 64: register index nb
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
      // column strides 1, 2, 4, 8: lanes inside each group of 16 (partner + own where the
      // stride bit is clear, partner - own where it is set).
      // (stage by stage over the eight values: eight independent DPP chains in flight)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb] = lane_xor<1>(v[nb]) + sg1 * v[nb];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb] = lane_xor<2>(v[nb]) + sg2 * v[nb];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb] = lane_xor<4>(v[nb]) + sg4 * v[nb];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb] = lane_xor<8>(v[nb]) + sg8 * v[nb];
      // The wave's four rows of this (mb, r) go through LDS so that every lane stores 16
      // contiguous bytes (8 columns): lane l takes row l >> 4, columns 8 * (l & 15) ...
      // (The lane index is re-derived here: kept live across the groups it gets spilled.)
      int l = threadIdx.x & 63;
      asm volatile("" : "+v"(l));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) stage[(l >> 4) * 128 + 16 * nb + (l & 15)] = f2h(v[nb] * sv[nb]);
      __builtin_amdgcn_wave_barrier();
      const u32x4 out8 = *reinterpret_cast<const u32x4 *>(stage + (l >> 4) * 128 + 8 * (l & 15));
      __builtin_amdgcn_wave_barrier();  // the next group's writes come after these reads
      const int rr = 16 * mb + 4 * (l >> 4) + r;  // row inside the wave's 64
      __builtin_amdgcn_raw_buffer_store_b128(out8, ry, (uint32_t)(rr * P.out * 2 + 16 * (l & 15)), 0, 0);
    }
  }
}


// Partial tiles in the workspace: slot-major, then wave, (mb, nb), lane, four floats each
// (coalesced 1 KB per instruction).  They are written and read with device-scope
// coherence (the sc1 cache policy: through the per-XCD L2s), because the workgroup that
// adds them may run on another XCD.

__device__ __forceinline__ void store_partial(const GemmParams &P, int slot, const Acc &acc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t rp =
      buffer_rsrc(P.partials + (size_t)slot * kTileFloats, (long long)kTileFloats * 4);
  const uint32_t off = (uint32_t)(wave * 32 * 64 + lane) * 16;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      __builtin_amdgcn_raw_buffer_store_b128(acc[mb][nb], rp, off, (mb * 8 + nb) * 64 * 16, kSC1);
}

__device__ __forceinline__ void add_partial(const GemmParams &P, int slot, Acc &acc, bool init) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t rp =
      buffer_rsrc(P.partials + (size_t)slot * kTileFloats, (long long)kTileFloats * 4);
  const uint32_t off = (uint32_t)(wave * 32 * 64 + lane) * 16;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const floatx4 v = __builtin_amdgcn_raw_buffer_load_b128(rp, off, (mb * 8 + nb) * 64 * 16, kSC1);
      acc[mb][nb] = init ? v : acc[mb][nb] + v;
    }
}

// Accumulates k-step pairs [k0, k1) of tile t (k-steps 2*k0 .. 2*k1 - 1).
template <int K, int CB = 1>
__device__ __forceinline__ void run_piece(const GemmParams &P, u32x4 (*ring)[8][64],
                                          u32x4 (*cring)[4 * 2 * 32 / 4], int t, int k0, int k1, Acc &acc,
                                          int signal) {
  constexpr int NW = 8 * K;  // 32-bit words per trellis tile
  // The lane's constants are recomputed per piece rather than kept live across the
  // epilogue (where they would be spilled and reloaded just before the loop, and the wait
  // for those reloads would then sit inside the loop).
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mt = t / P.nNT, nt = t - mt * P.nNT;
  const LaneWindow lw = lane_window(lane, K);

  // A operands: row blocks row0/16 + mb of XH (rows 64*wave + 16*mb + (lane & 15) of the
  // tile), one 1 KB block per step.  Blocks past the last row block read as zero.
  const int row0 = mt * kMT + 64 * wave;
  const int S32 = 2 * P.S;  // k-steps per row block
  const int Mpad = (P.M + 15) & ~15;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(P.xh + (size_t)(row0 >> 4) * S32 * 512,
                                                (long long)(Mpad - row0) * P.in * 2);
  const uint32_t a_off = (uint32_t)lane * 16;
  const int a_mb = S32 * 1024;  // bytes between row blocks
  // Codes: column block `wave` of the tile, tile rows 2*step + ti.  The step's two tiles
  // (2 * NW words) are loaded with one 4-byte word per lane (lanes past 2 * NW repeat
  // the first ones) and staged in a wave-private four-step LDS ring, from which every
  // lane reads the two words of each tile that hold its windows.  Steps past the end of
  // the code array read as zero (their results are never used).
  const long long row_bytes = (long long)(P.out / 16) * NW * 4;
  const long long code_bytes = (long long)(P.in / 16) * row_bytes;
  const long long col_off = (long long)(nt * 8 + wave) * NW * 4;
  const int cword = lane % (2 * NW);  // word of the step's two tiles this lane loads
  const uint32_t c_off = (uint32_t)((cword / NW) * row_bytes + 4 * (cword % NW));
  uint32_t *cw = reinterpret_cast<uint32_t *>(cring[wave]);  // [4 slots][2 * NW] words

  auto load_a = [&](u32x4 (&a)[4], int s) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      a[mb] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_off, s * 1024 + mb * a_mb, 0);
  };
  auto load_c = [&](uint32_t &c, int s) {
    const long long off = 2LL * s * row_bytes + col_off;
    const __amdgpu_buffer_rsrc_t rc =
        buffer_rsrc(reinterpret_cast<const char *>(P.code) + off, code_bytes - off);
    c = __builtin_amdgcn_raw_buffer_load_b32(rc, c_off, 0, 0);
  };
  auto stage_c = [&](uint32_t c, int slot) {
    cw[slot * 2 * NW + cword] = c;  // repeated lanes store equal data
  };
  // The decode's window words are read from the code ring half a step before the decode
  // (into W), so the decode does not start with an LDS round trip.
  u32x4 W;
  auto fetch_words = [&](int cslot) {
    const uint32_t *w = cw + cslot * 2 * NW;
    W = u32x4{w[lw.d0], w[lw.d1], w[NW + lw.d0], w[NW + lw.d1]};
  };
  auto decode_to = [&](int slot) {
    const u32x2 t0 = decode_pairs<K, CB>(W[0], W[1], lw.sh);
    const u32x2 t1 = decode_pairs<K, CB>(W[2], W[3], lw.sh);
    ring[slot][wave][lane] = u32x4{t0[0], t0[1], t1[0], t1[1]};
  };
  // B operands of one step: column blocks 0..3 are read from the ring right after the
  // barrier that publishes the step and 4..7 half a step later, so each group's LDS
  // latency hides behind 16 MFMAs of the other.
  u32x4 B[8];
  auto read_b = [&](int slot, int nb0) {
#pragma unroll
    for (int nb = nb0; nb < nb0 + 4; ++nb) B[nb] = ring[slot][nb][lane];
  };
  // The second half of a step: activation row block mb's last four MFMAs, then its load for
  // two steps ahead (the activation loads go out one at a time between MFMAs instead of as
  // one burst from every wave right after the barrier; 338 -> 336 us per call).
  auto mfma_half_load = [&](u32x4 (&a)[4], int s_next) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int nb = 4; nb < 8; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a[mb]),
                                                             __builtin_bit_cast(half8, B[nb]), acc[mb][nb], 0, 0, 0);
      a[mb] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_off, s_next * 1024 + mb * a_mb, 0);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // four MFMAs
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one activation load
    }
  };
  auto mfma_half = [&](const u32x4 (&a)[4], int nb0) {
#pragma unroll
    for (int nb = nb0; nb < nb0 + 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a[mb]),
                                                             __builtin_bit_cast(half8, B[nb]), acc[mb][nb], 0, 0, 0);
  };

#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int s0 = 2 * k0, s1 = 2 * k1;
  u32x4 A0[4], A1[4];
  uint32_t CR0, CR1;
  // Step s (relative r = s - s0) uses B ring slot r & 1 and A registers of that parity; its
  // codes sit in code ring slot r & 3.  During step s the codes of step s+1 are decoded
  // into the other B slot and the codes of step s+2 are staged; codes and activations
  // are loaded two steps ahead (past the piece they fetch unused data).
  // The previous piece's output stores must have completed first: with stores and loads
  // both outstanding the compiler can no longer count loads in order and would wait for
  // all of them inside the loop.  The loads left outstanding when the loop starts are
  // issued in the order one iteration leaves them (codes s+2, activations s, codes s+3,
  // activations s+1): the compiler counts outstanding loads per instruction position and
  // takes, at the loop head, the stricter of the entry and the back edge, so any other
  // order would make each iteration wait for loads issued only just before.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  load_c(CR0, s0);
  load_c(CR1, s0 + 1);
  stage_c(CR0, 0);
  stage_c(CR1, 1);
  __builtin_amdgcn_sched_barrier(0);
  load_c(CR0, s0 + 2);
  __builtin_amdgcn_sched_barrier(0);
  load_a(A0, s0);
  __builtin_amdgcn_sched_barrier(0);
  load_c(CR1, s0 + 3);
  __builtin_amdgcn_sched_barrier(0);
  load_a(A1, s0 + 1);
  __builtin_amdgcn_sched_barrier(0);
  fetch_words(0);
  decode_to(0);
  fetch_words(1);
  lds_barrier();
  // Every thread passed vmcnt(0) above, so partial-tile stores issued before this piece
  // have completed: publish them now (their latency was hidden behind the prologue).
  if (signal >= 0 && threadIdx.x == 0)
    __hip_atomic_fetch_add(P.counters + 2 * signal + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  read_b(0, 0);
  // Before each barrier a wave has 16 MFMAs and one step's decode (about 40 VALU
  // instructions); they are issued interleaved so that the matrix core and the vector ALU
  // work at the same time (the two waves of a SIMD reach this point together).
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
    }
  };
  for (int s = s0, r = 0; s < s1; s += 2, r += 2) {
    // step s (B slot 0)
    mfma_half(A0, 0);
    read_b(0, 4);
    stage_c(CR0, (r + 2) & 3);  // codes of step s + 2
    load_c(CR0, s + 4);
    decode_to(1);  // step s + 1 (words fetched half a step ago)
    interleave();
    fetch_words((r + 2) & 3);  // step s + 2's words (staged above: same wave, in order)
    lds_barrier();
    read_b(1, 0);
    mfma_half_load(A0, s + 2);
    // (keeps the next step's MFMAs out of this group: hoisted here they would wait on
    // activations loaded only half a step earlier)
    __builtin_amdgcn_sched_barrier(0);
    // step s + 1 (B slot 1)
    mfma_half(A1, 0);
    read_b(1, 4);
    stage_c(CR1, (r + 3) & 3);  // codes of step s + 3
    load_c(CR1, s + 5);
    decode_to(0);  // step s + 2 (unused after the last pair)
    interleave();
    fetch_words((r + 3) & 3);
    lds_barrier();
    read_b(0, 0);               // step s + 2 (unused after the last pair)
    mfma_half_load(A1, s + 3);
    __builtin_amdgcn_sched_barrier(0);
    // Keeps these B reads in this iteration: with nothing that may write memory after
    // them, the compiler would merge them with the prologue's identical reads into one
    // read at the top of the loop, right before the MFMAs that wait for it.
    asm volatile("" ::: "memory");
  }
  lds_barrier();  // the rings' last reads are done before the next piece writes them
}

// ---------------------------------------------------------------------------------------
// The FP8 product ("EXLR8" page: decoded weights are exactly E4M3, so prefill runs on FP8
// matrix multiplies).  The activations are rotated, then quantised per row to E4M3 with
// the scale max|row| / 448 (two launches: the rows' block maxima, then the codes), and the
// product runs on v_mfma_f32_16x16x128_f8f6f4 with k-steps of 128 input rows (eight
// trellis tile rows).  A lane's 32 B operand: byte j is tile row j >> 2 of the step and the
// lane's symbol j & 3 (rows 2g, 2g+1, 2g+8, 2g+9 of that tile, g = lane >> 4) -- for B the
// four E4M3 bytes of one decoded tile are one register; A is stored in the same order.
// ---------------------------------------------------------------------------------------

// One 128-block of 16 rows rotated: thread (row q = tid >> 4, i = tid & 15) returns
// elements 8i..8i+7 of H128(x*su) (unnormalised), zeros for rows past M.  VEC: r and s are
// 16-byte aligned (vector loads), else element loads.
template <bool VEC>
__device__ __forceinline__ void rotate_block(const uint16_t *__restrict__ x, int rows, int n,
                                             const uint16_t *__restrict__ r, const float *__restrict__ s, int row,
                                             int c, float (&v)[8]) {
  if (row < rows) {
    const u32x4 xv = *reinterpret_cast<const u32x4 *>(x + (size_t)row * n + c);
    float rv[8], sv[8];
    if (VEC) {
      const u32x4 r4 = *reinterpret_cast<const u32x4 *>(r + c);
#pragma unroll
      for (int t = 0; t < 8; ++t) rv[t] = h2f((t & 1) ? (uint16_t)(r4[t >> 1] >> 16) : (uint16_t)r4[t >> 1]);
      if (s) {
        const floatx4 s0 = *reinterpret_cast<const floatx4 *>(s + c);
        const floatx4 s1 = *reinterpret_cast<const floatx4 *>(s + c + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sv[t] = s0[t];
          sv[t + 4] = s1[t];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        rv[t] = h2f(r[c + t]);
        if (s) sv[t] = s[c + t];
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t xw = xv[t >> 1];
      const uint16_t xs = (t & 1) ? (uint16_t)(xw >> 16) : (uint16_t)xw;
      v[t] = h2f(xs) * rv[t];
      if (s) v[t] *= sv[t];
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = 0.f;
  }
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if ((t & h) == 0) {
        const float a = v[t], b = v[t + h];
        v[t] = a + b;
        v[t + h] = a - b;
      }
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    float p;
    p = lane_xor<1>(v[t]);
    v[t] = (lane & 1) ? (p - v[t]) : (v[t] + p);
    p = lane_xor<2>(v[t]);
    v[t] = (lane & 2) ? (p - v[t]) : (v[t] + p);
    p = lane_xor<4>(v[t]);
    v[t] = (lane & 4) ? (p - v[t]) : (v[t] + p);
    p = lane_xor<8>(v[t]);
    v[t] = (lane & 8) ? (p - v[t]) : (v[t] + p);
  }
}

// Maximum over the 16 lanes of a row (lanes 16q .. 16q+15 of a wave).
__device__ __forceinline__ float row16_max(float m) {
  m = fmaxf(m, lane_xor<1>(m));
  m = fmaxf(m, lane_xor<2>(m));
  m = fmaxf(m, lane_xor<4>(m));
  m = fmaxf(m, lane_xor<8>(m));
  return m;
}

// Launch 1: workgroup per (16-row block rb, 128-block blk); pmax[row][blk] = max |xh| of
// the row over the block.  Also clears the split-tile counters.
template <bool VEC>
__global__ __launch_bounds__(256) void rowmax_kernel(const uint16_t *__restrict__ x, int rows, int n,
                                                     const uint16_t *__restrict__ r, const float *__restrict__ s,
                                                     float *__restrict__ pmax, uint32_t *__restrict__ counters,
                                                     int ncounters) {
  for (int c = blockIdx.x * 256 + threadIdx.x; c < ncounters; c += gridDim.x * 256) counters[c] = 0;
  const int nb = n / 128;
  const int rb = blockIdx.x / nb, blk = blockIdx.x - rb * nb;
  const int q = threadIdx.x >> 4, i = threadIdx.x & 15;
  const int row = 16 * rb + q;
  float v[8];
  rotate_block<VEC>(x, rows, n, r, s, row, blk * 128 + 8 * i, v);
  float m = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(v[t]));
  m = row16_max(m);
  if (i == 0) pmax[(size_t)row * nb + blk] = m;
}

// Launch 2: same grid.  The row's maximum a, the codes e4m3(xh * 448 / a) (clamped to
// +-448 first, so the conversion never saturates), written as 2 KB blocks [row block]
// [k-step] in the operand order above; block 0 also writes rowscale[row] = a / 448.
template <bool VEC>
__global__ __launch_bounds__(256) void quant8_kernel(const uint16_t *__restrict__ x, int rows, int n,
                                                     const uint16_t *__restrict__ r, const float *__restrict__ s,
                                                     const float *__restrict__ pmax, uint8_t *__restrict__ xq,
                                                     float *__restrict__ rowscale) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[2048];
  const int nb = n / 128;
  const int rb = blockIdx.x / nb, blk = blockIdx.x - rb * nb;
  const int q = threadIdx.x >> 4, i = threadIdx.x & 15;
  const int row = 16 * rb + q;
  float m = 0.f;
  for (int b = i; b < nb; b += 16) m = fmaxf(m, pmax[(size_t)row * nb + b]);
  m = row16_max(m);
  const float inv = m > 0.f ? 448.0f / m : 0.f;
  if (blk == 0 && i == 0) rowscale[row] = m * (1.0f / 448.0f);
  float v[8];
  rotate_block<VEC>(x, rows, n, r, s, row, blk * 128 + 8 * i, v);
  // element 8i + t: tile row i >> 1 of the step, tile-internal row 8(i & 1) + t, so lane
  // group g = t >> 1 and byte j = 4(i >> 1) + 2(i & 1) + (t & 1) of lane 16g + q
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const float a = fminf(fmaxf(v[2 * g] * inv, -448.f), 448.f);
    const float b = fminf(fmaxf(v[2 * g + 1] * inv, -448.f), 448.f);
    const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    *reinterpret_cast<uint16_t *>(stage + (16 * g + q) * 32 + 4 * (i >> 1) + 2 * (i & 1)) = (uint16_t)pk;
  }
  __syncthreads();
  uint8_t *out = xq + ((size_t)rb * nb + blk) * 2048;
  reinterpret_cast<uint2 *>(out)[threadIdx.x] = reinterpret_cast<const uint2 *>(stage)[threadIdx.x];
}

typedef int intx8 __attribute__((ext_vector_type(8)));

// Accumulates k-steps [k0, k1) of tile t (128 input rows each) on the FP8 matrix core.
// B ring: [2 slots][8 column blocks][2 halves][64 lanes] (2 KB per column block); code
// ring: per wave [4 slots][64 chunks of 16 B] (the step's eight tiles of the wave's column
// block, tile ti at chunks 2K*ti ..).
template <int K>
__device__ __forceinline__ void run_piece_f8(const GemmParams &P, u32x4 (*ring)[8][2][64], u32x4 (*cring)[4 * 64],
                                             int t, int k0, int k1, Acc &acc, int signal) {
  constexpr int NW = 8 * K;  // 32-bit words per trellis tile
  constexpr int CH = 2 * K;  // 16-byte chunks per trellis tile
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mt = t / P.nNT, nt = t - mt * P.nNT;
  const LaneWindow lw = lane_window(lane, K);
  // A: 2 KB blocks [row block][step]; the lane's 32 bytes at 32 * lane.  Blocks past the
  // last row block read as zero.
  const int row0 = mt * kMT + 64 * wave;
  const int Mpad = (P.M + 15) & ~15;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(reinterpret_cast<const uint8_t *>(P.xh) + (size_t)(row0 >> 4) * P.S * 2048,
                                                (long long)(Mpad - row0) * P.in);
  const uint32_t a_off = (uint32_t)lane * 32;
  const int a_mb = P.S * 2048;  // bytes between row blocks
  // Codes: column block `wave`, tile rows 8s .. 8s+7; lane loads chunk lane % (8 CH).
  const long long row_bytes = (long long)(P.out / 16) * NW * 4;
  const long long code_bytes = (long long)(P.in / 16) * row_bytes;
  const long long col_off = (long long)(nt * 8 + wave) * NW * 4;
  const int cc = lane % (8 * CH);
  const uint32_t c_off = (uint32_t)((cc / CH) * row_bytes + 16 * (cc % CH));
  u32x4 *cw = cring[wave];

  auto load_a = [&](u32x4 (&a)[4][2], int st) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int h = 0; h < 2; ++h) a[mb][h] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_off, st * 2048 + mb * a_mb + 16 * h, 0);
  };
  auto load_c = [&](u32x4 &c, int st) {
    const long long off = 8LL * st * row_bytes + col_off;
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(reinterpret_cast<const char *>(P.code) + off, code_bytes - off);
    c = __builtin_amdgcn_raw_buffer_load_b128(rc, c_off, 0, 0);
  };
  auto stage_c = [&](const u32x4 &c, int slot) { cw[slot * 64 + cc] = c; };  // repeated lanes store equal data
  // The decode of the piece's first step (before the loop; the loop decodes in `step`).
  auto decode_to = [&](int cslot, int slot) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(cw + cslot * 64);
    uint32_t q[8];
    // the window words of tiles ti + 2, ti + 3 are read while tiles ti, ti + 1 decode
    u32x4 cur = {w[lw.d0], w[lw.d1], w[NW + lw.d0], w[NW + lw.d1]};
#pragma unroll
    for (int ti = 0; ti < 8; ti += 2) {
      u32x4 nxt = cur;
      if (ti + 2 < 8)
        nxt = u32x4{w[(ti + 2) * NW + lw.d0], w[(ti + 2) * NW + lw.d1], w[(ti + 3) * NW + lw.d0], w[(ti + 3) * NW + lw.d1]};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t bits = lane_bits(cur[2 * h], cur[2 * h + 1], lw.sh);
        q[ti + h] = e4m3_pack4(mcg_hash(lane_state<K>(bits, 0)), mcg_hash(lane_state<K>(bits, 1)),
                               mcg_hash(lane_state<K>(bits, 2)), mcg_hash(lane_state<K>(bits, 3)));
      }
      cur = nxt;
    }
    ring[slot][wave][0][lane] = u32x4{q[0], q[1], q[2], q[3]};
    ring[slot][wave][1][lane] = u32x4{q[4], q[5], q[6], q[7]};
  };
  // One step: its 32 MFMAs on B slot `slot` (column block nb + 1's operand is read while
  // nb's four MFMAs run) and the decode of the next step's eight tiles (codes in code ring
  // slot `cslot`, into B slot `dslot`), one tile per column block, issued between the MFMAs
  // five vector instructions at a time.
  auto step = [&](const u32x4 (&a)[4][2], int slot, int cslot, int dslot) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(cw + cslot * 64);
    uint32_t wd0[8], wd1[8];
#pragma unroll
    for (int ti = 0; ti < 8; ++ti) {
      wd0[ti] = w[ti * NW + lw.d0];
      wd1[ti] = w[ti * NW + lw.d1];
    }
    uint32_t q[8];
    u32x4 c0 = ring[slot][0][0][lane], c1 = ring[slot][0][1][lane];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const u32x4 b0 = c0, b1 = c1;
      if (nb + 1 < 8) {
        c0 = ring[slot][nb + 1][0][lane];
        c1 = ring[slot][nb + 1][1][lane];
      }
      const intx8 bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const intx8 av = {(int)a[mb][0][0], (int)a[mb][0][1], (int)a[mb][0][2], (int)a[mb][0][3],
                          (int)a[mb][1][0], (int)a[mb][1][1], (int)a[mb][1][2], (int)a[mb][1][3]};
        acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[mb][nb], 0, 0, 0, 0, 0, 0);
      }
      const uint32_t bits = lane_bits(wd0[nb], wd1[nb], lw.sh);
      q[nb] = e4m3_pack4(mcg_hash(lane_state<K>(bits, 0)), mcg_hash(lane_state<K>(bits, 1)),
                         mcg_hash(lane_state<K>(bits, 2)), mcg_hash(lane_state<K>(bits, 3)));
    }
    ring[dslot][wave][0][lane] = u32x4{q[0], q[1], q[2], q[3]};
    ring[dslot][wave][1][lane] = u32x4{q[4], q[5], q[6], q[7]};
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five vector instructions
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
  };

#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  u32x4 A0[4][2], A1[4][2];
  u32x4 CR0, CR1;
  // Step s (relative r = s - k0) uses B ring slot r & 1 and A registers of that parity; its
  // codes sit in code ring slot r & 3.  During step s the codes of step s+1 are decoded
  // into the other B slot and those of step s+2 staged; codes and activations are loaded
  // two steps ahead (past the piece they fetch unused data, bounded by the resources).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the previous piece's stores are done
  load_c(CR0, k0);
  load_c(CR1, k0 + 1);
  stage_c(CR0, 0);
  stage_c(CR1, 1);
  // The loads left in flight when the loop starts are issued in the order one iteration
  // leaves them (codes of step k0 + 2, activations of k0, codes of k0 + 3, activations of
  // k0 + 1): the compiler counts outstanding loads per position and takes, at the loop
  // head, the stricter of the entry and the back edge, so any other order makes every
  // iteration wait for loads issued only just before.
  __builtin_amdgcn_sched_barrier(0);
  load_c(CR0, k0 + 2);
  __builtin_amdgcn_sched_barrier(0);
  load_a(A0, k0);
  __builtin_amdgcn_sched_barrier(0);
  load_c(CR1, k0 + 3);
  __builtin_amdgcn_sched_barrier(0);
  load_a(A1, k0 + 1);
  __builtin_amdgcn_sched_barrier(0);
  decode_to(0, 0);
  lds_barrier();
  if (signal >= 0 && threadIdx.x == 0)
    __hip_atomic_fetch_add(P.counters + 2 * signal + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int st = k0, r = 0; st < k1; st += 2, r += 2) {
    // step st: B slot 0, A0
    stage_c(CR0, (r + 2) & 3);
    load_c(CR0, st + 4);
    step(A0, 0, (r + 1) & 3, 1);  // MFMAs of step st, decode of step st + 1
    lds_barrier();
    load_a(A0, st + 2);
    if (st + 1 < k1) {  // (uniform) step st + 1: B slot 1, A1
      stage_c(CR1, (r + 3) & 3);
      step(A1, 1, (r + 2) & 3, 0);  // MFMAs of step st + 1, decode of step st + 2
      lds_barrier();
    }
    // The second step's loads are issued on both paths (unused after an odd last step), so
    // the compiler counts the same loads in flight at the loop head whichever path ran, and
    // waits only for the ones a step uses.
    load_c(CR1, st + 5);
    load_a(A1, st + 3);
  }
  lds_barrier();  // the rings' last reads are done before the next piece writes them
}

// The workgroup's range: pieces, split tiles, epilogues (shared by the fp16 and FP8 products).
// F8: the FP8 product; CB: the codebook of the fp16 product.
template <int K, bool F8, int CB, typename Ring, typename CRing>
__device__ __forceinline__ void gemm_ranges(const GemmParams &P, Ring ring, CRing cring) {
  __shared__ uint32_t arrivals;
  const int g = xcd_range(blockIdx.x, P.G);
  const int it0 = range_start(P, g);
  const int end = range_start(P, g + 1);
  int signal = -1;  // split tile whose stored partial is still to be published
  // The range covers tiles tf..tl.  A split tile's two contributors meet in the middle of
  // the tile: one at the end of its range, the other at the start of its range.  The piece
  // at the end of the range is done FIRST (then the start piece, then the whole tiles), so
  // both contributors of a split tile reach it early and its partial tile is stored and
  // added while other workgroups still compute, rather than in the kernel's tail.
  const int tf = it0 < end ? it0 / P.S : 0, tl = it0 < end ? (end - 1) / P.S : -1;
  const bool end_first = tl > tf && end - tl * P.S < P.S;
  for (int j = 0; j <= tl - tf; ++j) {
    const int t = end_first ? (j == 0 ? tl : tf + j - 1) : tf + j;
    const int ts = t * P.S;
    const int k0 = t == tf ? it0 - ts : 0;
    const int k1 = t == tl ? end - ts : P.S;
    Acc acc;
    if constexpr (F8) run_piece_f8<K>(P, ring, cring, t, k0, k1, acc, signal);
    else run_piece<K, CB>(P, ring, cring, t, k0, k1, acc, signal);
    signal = -1;
    bool finish = k0 == 0 && k1 == P.S;  // one epilogue call site (register allocation)
    if (!finish) {
      const int g0 = range_owner(P, ts), g1 = range_owner(P, ts + P.S - 1);
      const int own = 2 * g + (t == tf ? 0 : 1);  // slot 2g: the range's start piece
      if (g1 == g0 + 1) {
        // Two contributors.  Counters (arrived, stored) per tile.  The first to arrive
        // stores its partial tile and publishes it later (start of its next piece, or
        // its end); the second adds that partial to its own registers (two terms: the
        // sum does not depend on the order) and finishes the tile.  The second only
        // waits for a contributor that has already arrived, i.e. is running.
        if (threadIdx.x == 0)
          arrivals = __hip_atomic_fetch_add(P.counters + 2 * t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrivals == 0) {
          store_partial(P, own, acc);
          signal = t;
        } else {
          if (threadIdx.x == 0) {
            // Bounded: the other contributor has arrived (it is running) and publishes its
            // partial within one piece.  If the wait ever ran out, the sum would miss that
            // partial; the error word says so.
            bool seen = false;
            for (int spin = 0; spin < (1 << 24) && !seen; ++spin) {
              seen = __hip_atomic_load(P.counters + 2 * t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
              if (!seen) __builtin_amdgcn_s_sleep(2);
            }
            if (!seen) __hip_atomic_fetch_or(P.errword, kErrWaitExpired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          __syncthreads();
          // the partial is read after its publication was seen, with device-scope (sc1) loads,
          // which read the coherent copy: no cache invalidation is needed
          const int c = g0 + g1 - g;  // the other contributor
          add_partial(P, 2 * c + (range_start(P, c) >= ts ? 0 : 1), acc, false);
          finish = true;
        }
      } else {
        // Three or more contributors (ranges shorter than a tile): every one stores its
        // partial tile; the last to arrive adds all of them in range order, so the sum
        // does not depend on which one arrives last.
        store_partial(P, own, acc);
        // Every thread waits for its own partial stores before the barrier (the barrier
        // alone does not wait for global stores), so the arrival below publishes them.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (threadIdx.x == 0)
          arrivals = __hip_atomic_fetch_add(P.counters + 2 * t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrivals == (uint32_t)(g1 - g0)) {  // (the others' partials: sc1 loads after their arrivals)
          // A contributor's piece of tile t is the start piece of its range (slot 2c) when
          // its range starts inside t, else the end piece (slot 2c + 1).
          for (int c = g0; c <= g1; ++c)
            add_partial(P, 2 * c + (range_start(P, c) >= ts ? 0 : 1), acc, c == g0);
          finish = true;
        }
      }
    }
    if (finish) finish_tile<F8>(P, acc, t / P.nNT, t % P.nNT, reinterpret_cast<u32x4 *>(ring));
  }
  if (signal >= 0) {
    // every thread's stores of the last piece's partial have completed, then the barrier
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(P.counters + 2 * signal + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int K, int CB>
__global__ __launch_bounds__(kThreads, 2) void gemm_sk_kernel(GemmParams P) {  // 2 waves per SIMD
  __shared__ __attribute__((aligned(16))) u32x4 ring[2][8][64];         // decoded B operands
  __shared__ __attribute__((aligned(16))) u32x4 cring[kWaves][4 * 2 * 32 / 4];  // staged codes
  gemm_ranges<K, false, CB>(P, ring, cring);
}

template <int K>
__global__ __launch_bounds__(kThreads, 2) void gemm_f8_kernel(GemmParams P) {  // 2 waves per SIMD
  __shared__ __attribute__((aligned(16))) u32x4 ring[2][8][2][64];  // decoded B operands (E4M3)
  __shared__ __attribute__((aligned(16))) u32x4 cring[kWaves][4 * 64];  // staged codes
  gemm_ranges<K, true, 1>(P, ring, cring);
}

int device_cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

struct Plan {
  int S, nNT, T, G;
  long long I;
  int q, r;
  size_t xh_bytes, xh_off, pmax_off, rowscale_off, partials_off, counters_off, bytes;
};

// f8: iterations are single 128-row k-steps and the activations are E4M3 bytes, with the
// row maxima and scales after them.
Plan plan(int in_features, int out_features, int M, bool f8 = false) {
  Plan p;
  p.S = f8 ? in_features / 128 : in_features / (2 * kKS);
  p.nNT = out_features / kNT;
  p.T = (M + kMT - 1) / kMT * p.nNT;
  p.I = (long long)p.T * p.S;
  long long G = device_cu_count();  // one workgroup (8 waves) per CU
  const long long by_work = (p.I + kMinSteps - 1) / kMinSteps;
  if (G > by_work) G = by_work;
  // Debug/test override of the workgroup count (exercises many split patterns).
  if (const char *env = getenv("TRELLIS_GEMM_WGS")) {
    const long long v = atoll(env);
    if (v > 0) G = v;
  }
  if (G > p.I) G = p.I;
  if (G < 1) G = 1;
  p.G = (int)G;
  p.q = (int)(p.I / G);
  p.r = (int)(p.I % G);
  const size_t Mpad = (size_t)((M + 15) / 16) * 16;  // whole 16-row blocks
  p.xh_bytes = Mpad * in_features * (f8 ? 1 : 2);
  p.xh_off = kWsReserved;  // (the reserved region of every workspace is left alone)
  p.pmax_off = p.xh_off + (p.xh_bytes + 255) / 256 * 256;
  p.rowscale_off = p.pmax_off + (f8 ? (Mpad * (in_features / 128) * 4 + 255) / 256 * 256 : 0);
  p.partials_off = p.rowscale_off + (f8 ? (Mpad * 4 + 255) / 256 * 256 : 0);
  p.counters_off = p.partials_off + (size_t)2 * p.G * kTileFloats * sizeof(float);
  p.bytes = p.counters_off + ((size_t)p.T * 8 + 255) / 256 * 256;
  return p;
}

}  // namespace

size_t gemm_workspace_bytes(int in_features, int out_features, int M) {
  if (M <= 0) return kWsReserved;
  return plan(in_features, out_features, M).bytes;
}

size_t gemm_fp8_workspace_bytes(int in_features, int out_features, int M) {
  if (M <= 0) return kWsReserved;
  return plan(in_features, out_features, M, true).bytes;
}

hipError_t launch_gemm_fp8(const trellis_linear &L, const uint16_t *x, int M, uint16_t *y, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const Plan p = plan(L.in_features, L.out_features, M, true);
  if (ws_bytes < p.bytes) return hipErrorInvalidValue;
  if (p.G > (1 << 20)) return hipErrorInvalidValue;
  if (p.I >= (1LL << 31)) return hipErrorInvalidValue;  // 32-bit iteration arithmetic
  if ((long long)(M + 15) / 16 * (L.in_features / 128) >= (1LL << 31)) return hipErrorInvalidValue;
  char *w = static_cast<char *>(ws);
  uint8_t *xq = reinterpret_cast<uint8_t *>(w + p.xh_off);
  float *pmax = reinterpret_cast<float *>(w + p.pmax_off);
  float *rowscale = reinterpret_cast<float *>(w + p.rowscale_off);
  uint32_t *counters = reinterpret_cast<uint32_t *>(w + p.counters_off);
  const unsigned rgrid = (unsigned)((M + 15) / 16 * (L.in_features / 128));
  const bool vec = (reinterpret_cast<uintptr_t>(L.rin) % 16) == 0 && (reinterpret_cast<uintptr_t>(L.s_in) % 16) == 0;
  if (vec) rowmax_kernel<true><<<rgrid, 256, 0, stream>>>(x, M, L.in_features, L.rin, L.s_in, pmax, counters, 2 * p.T);
  else rowmax_kernel<false><<<rgrid, 256, 0, stream>>>(x, M, L.in_features, L.rin, L.s_in, pmax, counters, 2 * p.T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (vec) quant8_kernel<true><<<rgrid, 256, 0, stream>>>(x, M, L.in_features, L.rin, L.s_in, pmax, xq, rowscale);
  else quant8_kernel<false><<<rgrid, 256, 0, stream>>>(x, M, L.in_features, L.rin, L.s_in, pmax, xq, rowscale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmParams P;
  P.xh = reinterpret_cast<const uint16_t *>(xq);
  P.rowscale = rowscale;
  P.code = reinterpret_cast<const uint32_t *>(L.code);
  P.rout = L.rout;
  P.s_out = L.s_out;
  P.y = y;
  P.partials = reinterpret_cast<float *>(w + p.partials_off);
  P.counters = counters;
  P.errword = reinterpret_cast<uint32_t *>(w);
  P.M = M;
  P.in = L.in_features;
  P.out = L.out_features;
  P.S = p.S;
  P.nNT = p.nNT;
  P.G = p.G;
  P.q = p.q;
  P.r = p.r;
  switch (L.K) {
    case 2: gemm_f8_kernel<2><<<p.G, kThreads, 0, stream>>>(P); break;
    case 3: gemm_f8_kernel<3><<<p.G, kThreads, 0, stream>>>(P); break;
    case 4: gemm_f8_kernel<4><<<p.G, kThreads, 0, stream>>>(P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const trellis_linear &L, const uint16_t *x, int M, uint16_t *y, void *ws,
                       size_t ws_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const Plan p = plan(L.in_features, L.out_features, M);
  if (ws_bytes < p.bytes) return hipErrorInvalidValue;
  if (p.G > (1 << 20)) return hipErrorInvalidValue;
  if (p.I >= (1LL << 31)) return hipErrorInvalidValue;  // 32-bit iteration arithmetic
  uint16_t *xh = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + p.xh_off);
  uint32_t *counters = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + p.counters_off);
  if ((long long)(M + 15) / 16 * (L.in_features / 128) >= (1LL << 31)) return hipErrorInvalidValue;
  const unsigned rgrid = (unsigned)((M + 15) / 16 * (L.in_features / 128));
  const bool vec = (reinterpret_cast<uintptr_t>(L.rin) % 16) == 0 && (reinterpret_cast<uintptr_t>(L.s_in) % 16) == 0;
  if (vec)
    rotate_kernel<true><<<rgrid, 256, 0, stream>>>(x, M, L.in_features, L.rin, L.s_in, xh, counters, 2 * p.T);
  else
    rotate_kernel<false><<<rgrid, 256, 0, stream>>>(x, M, L.in_features, L.rin, L.s_in, xh, counters, 2 * p.T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmParams P;
  P.xh = xh;
  P.rowscale = nullptr;
  P.code = reinterpret_cast<const uint32_t *>(L.code);
  P.rout = L.rout;
  P.s_out = L.s_out;
  P.y = y;
  P.partials = reinterpret_cast<float *>(static_cast<char *>(ws) + p.partials_off);
  P.counters = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + p.counters_off);
  P.errword = static_cast<uint32_t *>(ws);
  P.M = M;
  P.in = L.in_features;
  P.out = L.out_features;
  P.S = p.S;
  P.nNT = p.nNT;
  P.G = p.G;
  P.q = p.q;
  P.r = p.r;
  switch (L.K + 4 * (L.cb - 1)) {
    case 2: gemm_sk_kernel<2, 1><<<p.G, kThreads, 0, stream>>>(P); break;
    case 3: gemm_sk_kernel<3, 1><<<p.G, kThreads, 0, stream>>>(P); break;
    case 4: gemm_sk_kernel<4, 1><<<p.G, kThreads, 0, stream>>>(P); break;
    case 6: gemm_sk_kernel<2, 2><<<p.G, kThreads, 0, stream>>>(P); break;
    case 7: gemm_sk_kernel<3, 2><<<p.G, kThreads, 0, stream>>>(P); break;
    case 8: gemm_sk_kernel<4, 2><<<p.G, kThreads, 0, stream>>>(P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trellis
