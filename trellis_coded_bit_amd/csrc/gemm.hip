// trellis_gemm: prefill product Y = had(had(X*su) @ W_hat) * sv for M rows.
//
// ("Escha-W2 runs on Metal", reconstruction paragraph; decode as in decode.hip.)
//
// Three launches:
//   1. rotate: XH = H128(X*su) (unnormalised butterfly) as fp16 in the workspace, with the
//      32 input channels of every k-step stored in the order the MFMA operands take them
//      (below), so every A-operand load is one contiguous 16-byte piece;
//   2. the stream-K product.  Output tiles are 256 rows x 128 columns (one Hadamard block)
//      and a tile's k-steps are 32 input rows (two trellis tile rows).  The (tile, k-step)
//      iterations are numbered tile-major and every workgroup takes one contiguous range
//      of them, so all workgroups do the same work whatever the tile count; consecutive
//      ranges go to the same XCD (the dispatcher deals workgroups round-robin over the
//      XCDs), so an XCD works on one band of rows and keeps its activations in its L2.
//      A workgroup is 4 waves; wave w owns output rows 64w..64w+63 of the tile (4 x 8
//      blocks of 16x16, fp32 accumulators) and, per k-step, decodes the two trellis tile
//      rows of column blocks 2w and 2w+1 directly into MFMA B operands: by the lane
//      assignment of the decoder a lane's four symbols of a tile sit in one tile column and
//      four tile rows, so the lane holds, for its column, eight weights along k -- exactly
//      one B operand of v_mfma_f32_16x16x32_f16 once k inside the step is numbered as the
//      lanes hold it.  The operands go through a two-slot LDS ring (1 KB per column block)
//      so all four waves use all eight column blocks.  Codes and activations are loaded
//      two k-steps ahead into registers.  The codebook's fp16 addition (one rounding)
//      happens in the decoder, so B holds the format's exact fp16 weights.
//      A range covering a whole tile finishes it: output Hadamard across the tile's 128
//      columns (16 lanes x 8 registers per row), scales, the exact 1/128, fp16 stores.
//      The first or last piece of a range that covers only part of a tile is stored as an
//      fp32 partial tile in the workspace instead;
//   3. fix-up: one workgroup per split tile adds its partial tiles in range order
//      (deterministic) and finishes the tile as above.
#include <cstdlib>

#include "launch.h"
#include "trellis_device.h"

namespace trellis {

namespace {

constexpr int kMT = 256;      // output rows per tile
constexpr int kNT = 128;      // output columns per tile (one Hadamard block)
constexpr int kKS = 32;       // input rows per k-step (two trellis tile rows)
constexpr int kThreads = 256;
constexpr int kTileFloats = kMT * kNT;
constexpr int kMinSteps = 4;  // fewest k-step pairs per workgroup worth a split

struct GemmParams {
  const uint16_t *xh;  // [M][in] rotated activations, k permuted inside each 32-group
  const uint32_t *code;
  const uint16_t *rout;
  const float *s_out;
  uint16_t *y;
  float *partials;     // [2G][kTileFloats]
  int M, in, out;
  int S;               // k-step pairs per tile (the unit of the ranges)
  int nNT;             // column tiles
  int G;               // workgroups
  long long q;         // iterations per workgroup (the first r take one more)
  int r;
};

__device__ __forceinline__ long long range_start(const GemmParams &P, int g) {
  return (long long)g * P.q + (g < P.r ? g : P.r);
}

__device__ __forceinline__ int range_owner(const GemmParams &P, long long i) {
  const long long big = (long long)P.r * (P.q + 1);
  return i < big ? (int)(i / (P.q + 1)) : (int)(P.r + (i - big) / P.q);
}

// Workgroup b runs on XCD b % 8; give each XCD a contiguous block of ranges.
__device__ __forceinline__ int xcd_range(int b, int G) {
  const int x = b & 7, j = b >> 3;
  return x * (G >> 3) + min(x, G & 7) + j;
}

// Position, inside a k-step, of input row kk of the step: the MFMA operand element 8*g + j
// of lane group g holds row 16*(j >> 2) + 2*g + (j & 1) + 8*((j >> 1) & 1), which is the
// tile row of the decoder's symbol j & 3 in tile row-pair j >> 2 (trellis_device.h).
__device__ __forceinline__ int kperm_pos(int kk) {
  return 8 * ((kk >> 1) & 3) + 4 * (kk >> 4) + 2 * ((kk >> 3) & 1) + (kk & 1);
}

// XH = H128(X*su), one wave per (row, 128-block), k-permuted fp16 output.
__global__ __launch_bounds__(256) void rotate_kernel(const uint16_t *__restrict__ x, int rows, int n,
                                                     const uint16_t *__restrict__ r,
                                                     const float *__restrict__ s,
                                                     uint16_t *__restrict__ xh) {
  const int nb = n / 128;
  const long long task = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= (long long)rows * nb) return;
  const int row = (int)(task / nb), blk = (int)(task % nb);
  const int lane = threadIdx.x & 63;
  const size_t base = (size_t)row * n + (size_t)blk * 128;
  const int c0 = blk * 128 + lane, c1 = c0 + 64;
  float a = h2f(x[base + lane]), b = h2f(x[base + lane + 64]);
  float sa = h2f(r[c0]), sb = h2f(r[c1]);
  if (s) {
    sa *= s[c0];
    sb *= s[c1];
  }
  a *= sa;
  b *= sb;
  wave_fwht128(a, b);
  const int e0 = lane, e1 = lane + 64;  // block element of a and b
  xh[base + (e0 & ~31) + kperm_pos(e0 & 31)] = f2h(a);
  xh[base + (e1 & ~31) + kperm_pos(e1 & 31)] = f2h(b);
}

// Four symbols of one tile for this lane -> fp16 codebook values packed in pairs
// (symbols 0,1 and 2,3: tile rows 2g, 2g+1 and 2g+8, 2g+9 of column n).
template <int K>
__device__ __forceinline__ u32x2 decode_pairs(uint32_t w0, uint32_t w1, uint32_t sh) {
  const uint32_t bits = lane_bits(w0, w1, sh);
  uint32_t h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = mcg_hash(lane_state<K>(bits, j));
  u32x2 out;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t lo = __builtin_amdgcn_perm(h[2 * p + 1], h[2 * p], 0x05040100u);  // lo halves
    const uint32_t hi = __builtin_amdgcn_perm(h[2 * p + 1], h[2 * p], 0x07060302u);  // hi halves
    const half2_t v = __builtin_bit_cast(half2_t, lo) + __builtin_bit_cast(half2_t, hi);
    out[p] = __builtin_bit_cast(uint32_t, v);
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
__device__ __forceinline__ void finish_tile(const GemmParams &P, Acc &acc, int mt, int nt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n16 = lane & 15;
  float sv[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int col = nt * kNT + 16 * nb + n16;
    float s = h2f(P.rout[col]) * (1.0f / 128.0f);
    if (P.s_out) s *= P.s_out[col];
    sv[nb] = s;
  }
  const int row0 = mt * kMT + 64 * wave + 4 * (lane >> 4);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) v[nb] = acc[mb][nb][r];
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
      // column strides 1, 2, 4, 8: lanes inside each group of 16
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        float p;
        p = lane_xor<1>(v[nb]);
        v[nb] = (lane & 1) ? (p - v[nb]) : (v[nb] + p);
        p = lane_xor<2>(v[nb]);
        v[nb] = (lane & 2) ? (p - v[nb]) : (v[nb] + p);
        p = lane_xor<4>(v[nb]);
        v[nb] = (lane & 4) ? (p - v[nb]) : (v[nb] + p);
        p = lane_xor<8>(v[nb]);
        v[nb] = (lane & 8) ? (p - v[nb]) : (v[nb] + p);
      }
      const int row = row0 + 16 * mb + r;
      if (row < P.M) {
        uint16_t *yr = P.y + (size_t)row * P.out + nt * kNT + n16;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) yr[16 * nb] = f2h(v[nb] * sv[nb]);
      }
    }
  }
}

// Partial tiles: wave-major, then (mb, nb), then lane, four floats each (coalesced).
__device__ __forceinline__ float *partial_ptr(const GemmParams &P, int slot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return P.partials + (size_t)slot * kTileFloats + (size_t)(wave * 32 * 64 + lane) * 4;
}

// Raw buffer resource over `bytes` bytes at `base` (loads past the end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Accumulates k-step pairs [k0, k1) of tile t (k-steps 2*k0 .. 2*k1 - 1).
template <int K>
__device__ __forceinline__ void run_piece(const GemmParams &P, u32x4 (*ring)[8][64], int t, int k0,
                                          int k1, Acc &acc) {
  constexpr int NW = 8 * K;  // 32-bit words per trellis tile
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mt = t / P.nNT, nt = t - mt * P.nNT;
  const LaneWindow lw = lane_window(lane, K);

  // A operands: rows 64*wave + 16*mb + (lane & 15) of the tile, 8 halves at 8*(lane >> 4)
  // of each step.  Rows past M lie past the resource's end and read as zero.
  const int row0 = mt * kMT + 64 * wave;
  const __amdgpu_buffer_rsrc_t ra =
      buffer_rsrc(P.xh + (size_t)row0 * P.in, (long long)(P.M - row0) * P.in * 2);
  const uint32_t a_off = (uint32_t)(((lane & 15) * P.in + 8 * (lane >> 4)) * 2);
  const int a_mb = 16 * P.in * 2;  // bytes between m-blocks
  // Codes: column blocks 2*wave + j of the tile, tile rows 2*step + ti; steps past the end
  // of the code array read as zero (their results are never used).
  const long long row_bytes = (long long)(P.out / 16) * NW * 4;
  const long long code_bytes = (long long)(P.in / 16) * row_bytes;
  const long long col_off = (long long)(nt * 8 + 2 * wave) * NW * 4;
  const uint32_t d0 = lw.d0 * 4, d1 = lw.d1 * 4;

  auto load_a = [&](u32x4 (&a)[4], int s) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      a[mb] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_off, s * kKS * 2 + mb * a_mb, 0);
  };
  auto load_c = [&](uint32_t (&c)[8], int s) {
    const long long off = 2LL * s * row_bytes + col_off;
    const __amdgpu_buffer_rsrc_t rc =
        buffer_rsrc(reinterpret_cast<const char *>(P.code) + off, code_bytes - off);
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const int so = ti * (int)row_bytes;
      c[2 * ti] = __builtin_amdgcn_raw_buffer_load_b32(rc, d0, so, 0);
      c[2 * ti + 1] = __builtin_amdgcn_raw_buffer_load_b32(rc, d1, so, 0);
      c[4 + 2 * ti] = __builtin_amdgcn_raw_buffer_load_b32(rc, d0 + NW * 4, so, 0);
      c[4 + 2 * ti + 1] = __builtin_amdgcn_raw_buffer_load_b32(rc, d1 + NW * 4, so, 0);
    }
  };
  auto decode_to = [&](const uint32_t (&c)[8], int slot) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x2 t0 = decode_pairs<K>(c[4 * j], c[4 * j + 1], lw.sh);
      const u32x2 t1 = decode_pairs<K>(c[4 * j + 2], c[4 * j + 3], lw.sh);
      ring[slot][2 * wave + j][lane] = u32x4{t0[0], t0[1], t1[0], t1[1]};
    }
  };
  auto mfma_step = [&](const u32x4 (&a)[4], int slot) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const half8 bf = __builtin_bit_cast(half8, ring[slot][nb][lane]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a[mb]), bf, acc[mb][nb], 0, 0, 0);
    }
  };

#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int s0 = 2 * k0, s1 = 2 * k1;
  u32x4 A0[4], A1[4];
  uint32_t C0[8], C1[8];
  // Step s uses slot (s - s0) & 1, A(s) in A[that slot]; C(s+1) is decoded during step s.
  // Loads run two steps ahead; past the piece they fetch unused data.
  load_a(A0, s0);
  load_a(A1, s0 + 1);
  load_c(C0, s0);
  load_c(C1, s0 + 1);
  decode_to(C0, 0);
  load_c(C0, s0 + 2);
  lds_barrier();
  for (int s = s0; s < s1; s += 2) {
    decode_to(C1, 1);  // step s + 1
    load_c(C1, s + 3);
    mfma_step(A0, 0);  // step s
    load_a(A0, s + 2);
    lds_barrier();
    decode_to(C0, 0);  // step s + 2 (unused after the last pair)
    load_c(C0, s + 4);
    mfma_step(A1, 1);  // step s + 1
    load_a(A1, s + 3);
    lds_barrier();
  }
}

template <int K>
__global__ __launch_bounds__(kThreads, 2) void gemm_sk_kernel(GemmParams P) {
  __shared__ __attribute__((aligned(16))) u32x4 ring[2][8][64];
  const int g = xcd_range(blockIdx.x, P.G);
  long long it = range_start(P, g);
  const long long end = range_start(P, g + 1);
  bool first = true;
  while (it < end) {
    const int t = (int)(it / P.S);
    const int k0 = (int)(it - (long long)t * P.S);
    const int k1 = (int)min((long long)P.S, (long long)k0 + (end - it));
    Acc acc;
    run_piece<K>(P, ring, t, k0, k1, acc);
    if (k0 == 0 && k1 == P.S) {
      finish_tile(P, acc, t / P.nNT, t % P.nNT);
    } else {
      float *dst = partial_ptr(P, 2 * g + (first ? 0 : 1));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
          *reinterpret_cast<floatx4 *>(dst + (size_t)(mb * 8 + nb) * 64 * 4) = acc[mb][nb];
    }
    it += k1 - k0;
    first = false;
  }
}

// Workgroup f finishes the tile that its range ends in when that tile is split and f is
// its first contributor.  A contributor's piece of tile t is its first piece (slot 2c)
// when its range starts inside t, else its last piece (slot 2c + 1).
__global__ __launch_bounds__(kThreads) void gemm_fixup_kernel(GemmParams P) {
  const int f = blockIdx.x;
  const long long e = range_start(P, f + 1) - 1;
  const int t = (int)(e / P.S);
  const long long ts = (long long)t * P.S;
  const int g0 = range_owner(P, ts), g1 = range_owner(P, ts + P.S - 1);
  if (g0 == g1 || g0 != f) return;
  Acc acc;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int c = g0; c <= g1; ++c) {
    const float *src = partial_ptr(P, 2 * c + (range_start(P, c) >= ts ? 0 : 1));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        acc[mb][nb] += *reinterpret_cast<const floatx4 *>(src + (size_t)(mb * 8 + nb) * 64 * 4);
  }
  finish_tile(P, acc, t / P.nNT, t % P.nNT);
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
  long long I, q;
  int r;
  size_t xh_bytes, bytes;
};

Plan plan(int in_features, int out_features, int M) {
  Plan p;
  p.S = in_features / (2 * kKS);
  p.nNT = out_features / kNT;
  p.T = (M + kMT - 1) / kMT * p.nNT;
  p.I = (long long)p.T * p.S;
  long long G = 2LL * device_cu_count();  // two workgroups per CU
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
  p.q = p.I / G;
  p.r = (int)(p.I % G);
  p.xh_bytes = ((size_t)M * in_features * 2 + 255) / 256 * 256;
  p.bytes = p.xh_bytes + (size_t)2 * p.G * kTileFloats * sizeof(float);
  return p;
}

}  // namespace

size_t gemm_workspace_bytes(int in_features, int out_features, int M) {
  if (M <= 0) return 256;
  return plan(in_features, out_features, M).bytes;
}

hipError_t launch_gemm(const trellis_linear &L, const uint16_t *x, int M, uint16_t *y, void *ws,
                       size_t ws_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const Plan p = plan(L.in_features, L.out_features, M);
  if (ws_bytes < p.bytes) return hipErrorInvalidValue;
  if (p.G > (1 << 20)) return hipErrorInvalidValue;
  uint16_t *xh = static_cast<uint16_t *>(ws);
  const long long tasks = (long long)M * (L.in_features / 128);
  rotate_kernel<<<(unsigned)((tasks + 3) / 4), 256, 0, stream>>>(x, M, L.in_features, L.rin, L.s_in, xh);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmParams P;
  P.xh = xh;
  P.code = reinterpret_cast<const uint32_t *>(L.code);
  P.rout = L.rout;
  P.s_out = L.s_out;
  P.y = y;
  P.partials = reinterpret_cast<float *>(static_cast<char *>(ws) + p.xh_bytes);
  P.M = M;
  P.in = L.in_features;
  P.out = L.out_features;
  P.S = p.S;
  P.nNT = p.nNT;
  P.G = p.G;
  P.q = p.q;
  P.r = p.r;
  switch (L.K) {
    case 2: gemm_sk_kernel<2><<<p.G, kThreads, 0, stream>>>(P); break;
    case 3: gemm_sk_kernel<3><<<p.G, kThreads, 0, stream>>>(P); break;
    case 4: gemm_sk_kernel<4><<<p.G, kThreads, 0, stream>>>(P); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  gemm_fixup_kernel<<<p.G, kThreads, 0, stream>>>(P);
  return hipGetLastError();
}

}  // namespace trellis
