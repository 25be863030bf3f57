// trellis_encode_tiles: the tail-biting Viterbi encoder (the encode side of the format).
//
// ("EXLR8" page, tile-coding paragraph: a 16x16 tile is one path through a 16-bit-state
//  trellis, each weight contributing K new bits, and a Viterbi search picks the path with
//  the least squared error against the MCG codebook; E4M3 paragraph: with the E4M3 codebook
//  the rounding happens inside the search.  The pages do not say how the circular
//  constraint is met; here, as in the oracle, two passes: a free pass whose best end state
//  fixes the wrap bits O, then a pass whose start states have high bits O and end states
//  low bits O, so that the path closes on itself.  Ties go to the lowest index.)
//
// One 1024-thread workgroup per tile.  All 65 536 path costs stay in registers, 64 per
// thread.  State n = (t << L) | (q << K) | b with L = 16 - K: a thread owns, for its q,
// every b and a range of t.  A step has two halves:
//   * best[m] = min over t of cost[(t << L) | m] for the groups m = (q << K) | b the thread
//     owns (for K = 4 the 16 t values are spread over four adjacent lanes), written to LDS
//     with the argmin t (the decision kept for the backtrack);
//   * cost'[n] = best[n >> K] + (x_s - value(n))^2, where n >> K = (t << (L - K)) | q does
//     not depend on b: one LDS read serves all b of a (q, t).
// The costs are float32, each step one subtraction, one multiplication and one addition,
// each rounded (no fused multiply-add), so the decisions match a float32 search that does
// the same operations.  The decisions of the second pass (one word per thread and step)
// go to the workspace; a second launch walks them back from the best end state, one thread
// per tile, and packs the symbols' bits into the tile's 16K words.
#include "launch.h"
#include "trellis_device.h"

namespace trellis {

namespace {

constexpr int kEncThreads = 1024;

template <int K>
struct Enc {
  static constexpr int L = 16 - K;
  static constexpr int NB = 1 << K;           // b values (and t values)
  static constexpr int QPT = K == 2 ? 4 : 1;   // q values per thread
  static constexpr int TPT = K == 4 ? 4 : NB;  // t values per thread
  static constexpr int STATES = QPT * TPT * NB;
  static_assert(STATES == 64, "64 states per thread");
};

template <int K>
__device__ __forceinline__ int thread_q(int j, int i) {
  return K == 2 ? j + kEncThreads * i : (K == 3 ? j : j >> 2);
}

// Codebook value of state n as float (cb = 2: rounded to E4M3).
template <int CB>
__device__ __forceinline__ _Float16 enc_value(uint32_t n) {
  _Float16 v = mcg_value(mcg_hash(n));
  if constexpr (CB == 2) {
    typedef _Float16 hv2 __attribute__((ext_vector_type(2)));
    typedef short sv2 __attribute__((ext_vector_type(2)));
    const hv2 pr = {v, v};
    const sv2 q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(sv2{0, 0}, pr, 1.0f, false);
    v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_bit_cast(uint32_t, q), 1.0f, false)[0];
  }
  return v;
}

// (value, index) minimum with ties to the lower index.
__device__ __forceinline__ void argmin_merge(float &v, int &n, float ov, int on) {
  if (ov < v || (ov == v && on < n)) {
    v = ov;
    n = on;
  }
}

template <int K, int CB>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(const float *__restrict__ targets,
                                                             uint32_t *__restrict__ dec, int *__restrict__ ends) {
#pragma clang fp contract(off)
  using E = Enc<K>;
  constexpr int L = E::L, NB = E::NB, QPT = E::QPT, TPT = E::TPT;
  constexpr uint32_t mask_lo = (1u << L) - 1;
  __shared__ float x[256];
  __shared__ float best[2][1 << L];
  __shared__ float red_v[kEncThreads / 64];
  __shared__ int red_n[kEncThreads / 64];
  __shared__ int wrap;
  const int tile = blockIdx.x;
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6;
  // symbol s of the tile sits at row 8 ((s >> 1) & 1) + 2 ((s >> 3) & 3) + (s & 1), column
  // 8 ((s >> 2) & 1) + (s >> 5) (the tile permutation)
  if (j < 256) {
    const int s = j;
    const int r = 8 * ((s >> 1) & 1) + 2 * ((s >> 3) & 3) + (s & 1), c = 8 * ((s >> 2) & 1) + (s >> 5);
    x[s] = targets[(size_t)tile * 256 + r * 16 + c];
  }
  const int t0 = K == 4 ? 4 * (j & 3) : 0;
  // the owned states' codebook values, two fp16 per register
  uint32_t cv[E::STATES / 2];
#pragma unroll
  for (int i = 0; i < QPT; ++i)
#pragma unroll
    for (int tt = 0; tt < TPT; ++tt)
#pragma unroll
      for (int b = 0; b < NB; b += 2) {
        const uint32_t n = ((uint32_t)(t0 + tt) << L) | ((uint32_t)thread_q<K>(j, i) << K) | b;
        const _Float16 v0 = enc_value<CB>(n), v1 = enc_value<CB>(n + 1);
        cv[((i * TPT + tt) * NB + b) >> 1] =
            (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
      }
  // (unpacked at every use: kept as floats across the steps they would need 64 more
  // registers than a thread has)
  auto value = [&](int i, int tt, int b) -> float {
    uint32_t w = cv[((i * TPT + tt) * NB + b) >> 1];
    asm volatile("" : "+v"(w));
    return h2f((b & 1) ? (uint16_t)(w >> 16) : (uint16_t)w);
  };
  __syncthreads();

  float cost[QPT][TPT][NB];
  for (int pass = 0; pass < 2; ++pass) {
    const uint32_t O = pass ? (uint32_t)wrap : 0u;
    // step 0
    {
      const float xs = x[0];
#pragma unroll
      for (int i = 0; i < QPT; ++i)
#pragma unroll
        for (int tt = 0; tt < TPT; ++tt) {
          // n >> K = (t << (L - K)) | q
          const uint32_t hi = ((uint32_t)(t0 + tt) << (L - K)) | (uint32_t)thread_q<K>(j, i);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const float d = xs - value(i, tt, b);
            cost[i][tt][b] = (pass && hi != O) ? __builtin_inff() : d * d;
          }
        }
    }
    for (int s = 1; s < 256; ++s) {
      // best and argmin over t for the owned groups m = (q << K) | b
      uint32_t word = 0;
      float *bw = best[s & 1];
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        const int q = thread_q<K>(j, i);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float bv = cost[i][0][b];
          int bt = t0;
#pragma unroll
          for (int tt = 1; tt < TPT; ++tt)
            if (cost[i][tt][b] < bv) {
              bv = cost[i][tt][b];
              bt = t0 + tt;
            }
          if constexpr (K == 4) {  // the four lanes of q hold t = 0..3, 4..7, 8..11, 12..15
            {  // (DPP moves within each quad of lanes; the index travels as raw bits)
              float ov = lane_xor<1>(bv);
              int ot = __builtin_bit_cast(int, lane_xor<1>(__builtin_bit_cast(float, bt)));
              argmin_merge(bv, bt, ov, ot);
              ov = lane_xor<2>(bv);
              ot = __builtin_bit_cast(int, lane_xor<2>(__builtin_bit_cast(float, bt)));
              argmin_merge(bv, bt, ov, ot);
            }
            if ((b >> 2) == (j & 3)) word |= (uint32_t)bt << (4 * (b & 3));
            if ((j & 3) == 0) bw[(q << K) | b] = bv;
          } else {
            word |= (uint32_t)bt << (K * (i * NB + b));
            bw[(q << K) | b] = bv;
          }
        }
      }
      if (pass) dec[((size_t)tile * 256 + s) * kEncThreads + j] = word;
      __syncthreads();
      const float xs = x[s];
#pragma unroll
      for (int i = 0; i < QPT; ++i)
#pragma unroll
        for (int tt = 0; tt < TPT; ++tt) {
          const float bb = bw[((t0 + tt) << (L - K)) | thread_q<K>(j, i)];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const float d = xs - value(i, tt, b);
            cost[i][tt][b] = bb + d * d;
          }
        }
    }
    // the best end state (pass 2: low bits O), ties to the lowest index
    float mv = __builtin_inff();
    int mn = 1 << 16;
#pragma unroll
    for (int i = 0; i < QPT; ++i)
#pragma unroll
      for (int tt = 0; tt < TPT; ++tt)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const uint32_t m = ((uint32_t)thread_q<K>(j, i) << K) | b;
          const int n = (int)(((uint32_t)(t0 + tt) << L) | m);
          const float c = (pass && m != O) ? __builtin_inff() : cost[i][tt][b];
          argmin_merge(mv, mn, c, n);
        }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const float ov = __shfl_xor(mv, sh, 64);
      const int on = __shfl_xor(mn, sh, 64);
      argmin_merge(mv, mn, ov, on);
    }
    if (lane == 0) {
      red_v[wave] = mv;
      red_n[wave] = mn;
    }
    __syncthreads();
    if (j == 0) {
      float v = red_v[0];
      int n = red_n[0];
      for (int w = 1; w < kEncThreads / 64; ++w) argmin_merge(v, n, red_v[w], red_n[w]);
      if (pass == 0) wrap = (int)((uint32_t)n & mask_lo);
      else ends[tile] = n;
    }
    __syncthreads();
  }
}

// One thread per tile: walk the decisions back from the end state and pack the symbols'
// bits (symbol s's K bits at stream bits sK.., most significant first; 32-bit words, most
// significant bit first, stored little-endian as int16 pairs).
template <int K>
__global__ __launch_bounds__(256) void backtrack_kernel(const uint32_t *__restrict__ dec, const int *__restrict__ ends,
                                                        int T, uint32_t *__restrict__ code, uint16_t *__restrict__ states) {
  constexpr int L = 16 - K;
  const int tile = blockIdx.x * 256 + threadIdx.x;
  if (tile >= T) return;
  uint32_t st = (uint32_t)ends[tile];
  uint32_t *cw = code + (size_t)tile * 8 * K;
  uint64_t acc = 0;
  int nbits = 0, widx = 8 * K - 1;
  for (int s = 255; s >= 0; --s) {
    if (states) states[(size_t)tile * 256 + s] = (uint16_t)st;
    acc |= (uint64_t)(st & ((1u << K) - 1)) << nbits;
    nbits += K;
    if (nbits >= 32) {
      cw[widx--] = (uint32_t)acc;
      acc >>= 32;
      nbits -= 32;
    }
    if (s > 0) {
      const uint32_t m = st >> K, q = m >> K, b = m & ((1u << K) - 1);
      int jj, sh;
      if (K == 2) {
        jj = (int)(q & (kEncThreads - 1));
        sh = (int)(K * ((q >> 10) * 4 + b));
      } else if (K == 3) {
        jj = (int)q;
        sh = (int)(K * b);
      } else {
        jj = (int)(4 * q + (b >> 2));
        sh = (int)(4 * (b & 3));
      }
      const uint32_t w = dec[((size_t)tile * 256 + s) * kEncThreads + jj];
      const uint32_t t = (w >> sh) & ((1u << K) - 1);
      st = (t << L) | m;
    }
  }
}

}  // namespace

size_t encode_workspace_bytes(int n_tiles) {
  if (n_tiles <= 0) return 256;
  return (size_t)n_tiles * 256 * kEncThreads * 4 + (((size_t)n_tiles * 4 + 255) & ~(size_t)255);
}

hipError_t launch_encode_tiles(const float *targets, int T, int K, int cb, int16_t *code, uint16_t *states,
                               void *ws, size_t ws_bytes, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (ws_bytes < encode_workspace_bytes(T)) return hipErrorInvalidValue;
  uint32_t *dec = static_cast<uint32_t *>(ws);
  int *ends = reinterpret_cast<int *>(static_cast<char *>(ws) + (size_t)T * 256 * kEncThreads * 4);
  switch (K + 4 * (cb - 1)) {
    case 2: encode_kernel<2, 1><<<T, kEncThreads, 0, stream>>>(targets, dec, ends); break;
    case 3: encode_kernel<3, 1><<<T, kEncThreads, 0, stream>>>(targets, dec, ends); break;
    case 4: encode_kernel<4, 1><<<T, kEncThreads, 0, stream>>>(targets, dec, ends); break;
    case 6: encode_kernel<2, 2><<<T, kEncThreads, 0, stream>>>(targets, dec, ends); break;
    case 7: encode_kernel<3, 2><<<T, kEncThreads, 0, stream>>>(targets, dec, ends); break;
    case 8: encode_kernel<4, 2><<<T, kEncThreads, 0, stream>>>(targets, dec, ends); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t *cw = reinterpret_cast<uint32_t *>(code);
  const unsigned g = (unsigned)((T + 255) / 256);
  if (K == 2) backtrack_kernel<2><<<g, 256, 0, stream>>>(dec, ends, T, cw, states);
  else if (K == 3) backtrack_kernel<3><<<g, 256, 0, stream>>>(dec, ends, T, cw, states);
  else backtrack_kernel<4><<<g, 256, 0, stream>>>(dec, ends, T, cw, states);
  return hipGetLastError();
}

}  // namespace trellis
