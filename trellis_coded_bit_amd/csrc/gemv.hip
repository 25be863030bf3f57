// trellis_gemv / trellis_moe_gemv: fused small-batch products against trellis-coded weights.
//
// y = had(had(x*su) @ W_hat) * sv  ("Escha-W2 runs on Metal", reconstruction paragraph),
// for B = 1..8 rows, over a list of problems (one layer, or the routed entries of an expert
// pointer table -- "EXLR8" page: per-expert widths, a pointer table re-read every launch,
// one hidden-side rotation shared by all experts).
//
// Work decomposition (stream-K over "units").  A unit is one 128-row input block I times
// one 128-column output block J of one problem p, i.e. 8x8 tiles; units are numbered
// u = (p*nJ + J)*nI + I and the G workgroups take equal contiguous ranges of u, so every
// workgroup streams the same number of code bytes whatever the matrix shape.  A range that
// cuts a column block leaves a partial sum in the workspace; the last workgroup to finish
// a column block (agent-scope counter) adds the partials in a fixed order, applies the
// output Hadamard and the scales, writes fp16 y and resets the counter.  Partial sums are
// written and read with agent-scope atomic accesses, which are coherent across the XCDs'
// L2 caches without the full L2 write-back a device-wide fence would cost.
//
// Inside a workgroup (4 waves) every wave takes two of the unit's eight tile rows:
//   * loads: the wave's 2 x 8 tiles are 2 x 256K contiguous bytes; each lane loads 8-byte
//     pieces (fully coalesced) several units ahead of use (a ring of kPrefetch units in
//     registers keeps a few KB per wave in flight) and stages them in a wave-private LDS
//     buffer; each tile is stored with a copy of its last word in front, so every lane's
//     circular window is two adjacent LDS words;
//   * input rotation: for each group of kSuper units the workgroup butterflies x*su
//     (unnormalised) and stores fp16 MFMA A-operands in LDS, each value twice (below);
//   * contraction: per tile each lane decodes its four symbols (trellis_device.h) to four
//     MCG hash words and feeds them UNSUMMED to v_mfma_f32_16x16x32_f16 as eight fp16
//     B-elements along k.  The A operand repeats each activation for the lo and hi halves,
//     so the matrix core forms x*lo + x*hi in fp32 and the codebook's lo+hi addition costs
//     no VALU work.  One MFMA covers one tile; batch rows ride in the 16 M rows.  (This
//     fp32 sum of the halves is the exact value before the format's fp16 rounding; it
//     differs from the rounded codebook value by at most half an fp16 ulp.)
//   * the two 1/sqrt(128) factors are folded into one exact 1/128 at the output.
#include <cstdlib>

#include "launch.h"
#include "trellis_device.h"

namespace trellis {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxB = 8;
constexpr int kSuper = 4;        // units whose input rotation is done together
constexpr int kPrefetch = 3;     // units in flight per wave
constexpr int kTileStride = 36;  // LDS words per staged tile: 4 + 8K (K <= 4)
// Counter slots live at a fixed place in the workspace whatever the problem shape, so the
// partial sums of one call can never land on the counters of a later, larger call.
constexpr int kMaxColumnBlocks = 65536;

struct GemvParams {
  GemvLaunch L;
  uint32_t *errword;
  uint32_t *counters;
  float *partials;
  int U;  // total units
  int G;  // workgroups
  int nI, nJ, maxseg;
};

// Dynamic LDS layout for batch B.
struct Lds {
  uint32_t *a;      // [kSuper][8 tile rows][4 groups][B][4 words]
  uint32_t *tiles;  // [kWaves][16 tiles][kTileStride]
  float *red;       // [kWaves][B][128]
  float *fin;       // [B][128]
  int *flag;
};

__host__ __device__ constexpr size_t lds_a_bytes(int B) { return (size_t)kSuper * 8 * 4 * B * 16; }
__host__ __device__ constexpr size_t lds_tiles_bytes() { return (size_t)kWaves * 16 * kTileStride * 4; }
__host__ __device__ constexpr size_t lds_bytes(int B) {
  return lds_a_bytes(B) + lds_tiles_bytes() + (size_t)kWaves * B * 128 * 4 + (size_t)B * 128 * 4 + 16;
}

__device__ __forceinline__ Lds lds_carve(char *base, int B) {
  Lds s;
  s.a = reinterpret_cast<uint32_t *>(base);
  s.tiles = reinterpret_cast<uint32_t *>(base + lds_a_bytes(B));
  s.red = reinterpret_cast<float *>(base + lds_a_bytes(B) + lds_tiles_bytes());
  s.fin = s.red + kWaves * B * 128;
  s.flag = reinterpret_cast<int *>(s.fin + B * 128);
  return s;
}

struct Problem {
  const uint32_t *code;
  const uint16_t *rin, *rout;
  const float *s_in, *s_out;
  int K;
  bool ok;
};

__device__ __forceinline__ Problem get_problem(const GemvParams &P, int p) {
  trellis_linear d = P.L.single;
  bool ok = true;
  if (P.L.table) {
    const int e = P.L.routed[p];
    if (e < 0 || e >= P.L.E) ok = false;
    else d = P.L.table[e];
  }
  Problem r;
  r.code = reinterpret_cast<const uint32_t *>(d.code);
  r.K = d.K;
  r.rin = d.rin;
  r.s_in = d.s_in;
  r.rout = d.rout;
  r.s_out = d.s_out;
  if (P.L.shared_side == 0) { r.rin = P.L.shared_r; r.s_in = P.L.shared_s; }
  if (P.L.shared_side == 1) { r.rout = P.L.shared_r; r.s_out = P.L.shared_s; }
  if (ok) {
    ok = d.K >= 2 && d.K <= 4 && d.cb == 1 && d.code != nullptr && r.rin != nullptr &&
         r.rout != nullptr && d.in_features == P.L.in_features &&
         d.out_features == P.L.out_features;
  }
  r.ok = ok;
  return r;
}

struct Coords {
  int q, I, p, J;
};

__device__ __forceinline__ Coords unit_coords(const GemvParams &P, int u) {
  Coords c;
  c.q = (int)((unsigned)u / (unsigned)P.nI);
  c.I = u - c.q * P.nI;
  c.p = (int)((unsigned)c.q / (unsigned)P.nJ);
  c.J = c.q - c.p * P.nJ;
  return c;
}

// First unit of workgroup g, and the workgroup owning unit u (largest g with start(g) <= u).
__device__ __forceinline__ int wg_start(int g, int U, int G) { return (int)(((long long)g * U) / G); }
__device__ __forceinline__ int owner(int u, int U, int G) {
  return (int)((((long long)u + 1) * G - 1) / U);
}

// Orders this wave's LDS accesses (all lanes of one wave run in lockstep and the LDS
// executes one wave's operations in order; this only stops the compiler from moving them).
__device__ __forceinline__ void wave_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------------------
// Input rotation of units [u, u + n) into the A-operand buffer (whole workgroup).
// a[((s*8 + ti)*4 + g)*B + m] holds, for tile row ti of unit s and batch row m, the four
// words for rows (2g, 2g+1, 2g+8, 2g+9), each word the fp16 value twice.
// ---------------------------------------------------------------------------------------
__device__ void rotate_units(const GemvParams &P, int u, int n, const Lds &sm) {
  const int B = P.L.B, in = P.L.in_features;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int task = wave; task < n * B; task += kWaves) {
    const int s = task / B, b = task - s * B;
    const Coords c = unit_coords(P, u + s);
    const Problem pr = get_problem(P, c.p);
    float va = 0.f, vb = 0.f;
    if (pr.ok) {
      const uint16_t *x = P.L.x + (P.L.x_per_problem ? (size_t)c.p * B * in : (size_t)0) + (size_t)b * in;
      const int k0 = c.I * 128 + lane, k1 = k0 + 64;
      va = h2f(ldg(x + k0)) * h2f(ldg(pr.rin + k0));
      vb = h2f(ldg(x + k1)) * h2f(ldg(pr.rin + k1));
      if (pr.s_in) { va *= ldg(pr.s_in + k0); vb *= ldg(pr.s_in + k1); }
      wave_fwht128(va, vb);
    }
    // element k = lane (+64): tile row ti = k >> 4, in-tile row rr = k & 15
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ti = (lane >> 4) + 4 * h, rr = lane & 15;
      const int g = (rr & 7) >> 1, w = 2 * (rr >> 3) + (rr & 1);
      const uint32_t hv = f2h(h ? vb : va);
      sm.a[((((s * 8 + ti) * 4 + g) * B + b) << 2) + w] = hv | (hv << 16);
    }
  }
}

// ---------------------------------------------------------------------------------------
// End of a segment (the workgroup's share of column block q): reduce the waves'
// accumulators, publish the partial, and let the last contributor finish the block.
// ---------------------------------------------------------------------------------------
__device__ void finish_segment(const GemvParams &P, const Lds &sm, const Coords &c, const Problem &pr,
                               floatx4 (&acc)[8]) {
  const int B = P.L.B, out = P.L.out_features;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mrow = 4 * (lane >> 4) + r;
    if (mrow < B) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sm.red[(wave * B + mrow) * 128 + 16 * jj + (lane & 15)] = acc[jj][r];
    }
  }
  __syncthreads();
  const int seg = c.q - wg_start(g, P.U, P.G) / P.nI;
  float *part = P.partials + ((size_t)g * P.maxseg + seg) * kMaxB * 128;
  for (int idx = tid; idx < B * 128; idx += kThreads) {
    float v = sm.red[idx];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += sm.red[w * B * 128 + idx];
    __hip_atomic_store(part + idx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  const int g_lo = owner(c.q * P.nI, P.U, P.G), g_hi = owner((c.q + 1) * P.nI - 1, P.U, P.G);
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(P.counters + c.q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sm.flag = (old == (uint32_t)(g_hi - g_lo));
  }
  __syncthreads();
  if (*sm.flag) {
    for (int idx = tid; idx < B * 128; idx += kThreads) {
      float v = 0.f;
      for (int gg = g_lo; gg <= g_hi; ++gg) {
        const int sg = c.q - wg_start(gg, P.U, P.G) / P.nI;
        v += __hip_atomic_load(P.partials + ((size_t)gg * P.maxseg + sg) * kMaxB * 128 + idx,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      sm.fin[idx] = v;
    }
    __syncthreads();
    uint16_t *y = P.L.y + (size_t)c.p * B * out;
    for (int b = wave; b < B; b += kWaves) {
      const int c0 = c.J * 128 + lane, c1 = c0 + 64;
      float va = sm.fin[b * 128 + lane], vb = sm.fin[b * 128 + lane + 64];
      if (pr.ok) {
        wave_fwht128(va, vb);
        float sa = h2f(ldg(pr.rout + c0)) * (1.0f / 128.0f), sb = h2f(ldg(pr.rout + c1)) * (1.0f / 128.0f);
        if (pr.s_out) { sa *= ldg(pr.s_out + c0); sb *= ldg(pr.s_out + c1); }
        va *= sa;
        vb *= sb;
      } else {
        va = 0.f;
        vb = 0.f;
      }
      y[(size_t)b * out + c0] = f2h(va);
      y[(size_t)b * out + c1] = f2h(vb);
    }
    if (tid == 0) __hip_atomic_store(P.counters + c.q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------------------
// Per-lane geometry of the coalesced loads of one unit (two tile rows x 8 tiles per wave).
// ---------------------------------------------------------------------------------------
template <int K>
struct UnitLoader {
  static constexpr int NW = 8 * K;     // words per tile
  static constexpr int ROWW = 8 * NW;  // words per 8-tile row chunk
  uint32_t off[K];                     // word offset of the lane's piece t from the unit base
  uint32_t lds[K];                     // LDS word index of piece t in the wave's tile buffer
  bool prefix[K];                      // piece t ends with the tile's last word

  __device__ __forceinline__ void init(int lane, int row_stride_words) {
#pragma unroll
    for (int t = 0; t < K; ++t) {
      const int wpos = 2 * (lane + 64 * t);  // word position in the 2-row concatenation
      const int r = wpos / ROWW, o = wpos - r * ROWW;
      const int tt = o / NW, dd = o - tt * NW;
      off[t] = (uint32_t)(r * row_stride_words + o);
      lds[t] = (uint32_t)((r * 8 + tt) * kTileStride + 4 + dd);
      prefix[t] = (dd + 1 == NW - 1);
    }
  }
};

template <int K>
__device__ __forceinline__ void load_unit(uint32_t (&buf)[2 * K], const uint32_t *base, const UnitLoader<K> &ld) {
#pragma unroll
  for (int t = 0; t < K; ++t) {
    const u32x2 v = ldg(reinterpret_cast<const u32x2 *>(base + ld.off[t]));
    buf[2 * t] = v[0];
    buf[2 * t + 1] = v[1];
  }
}

// Units [ub, ue) of this workgroup, all of width K.
template <int K>
__device__ void run_range(const GemvParams &P, const Lds &sm, int ub, int ue) {
  constexpr int NW = 8 * K;
  const int n = ue - ub;
  const int B = P.L.B;
  const int Tj = P.L.out_features / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, grp = lane >> 4;
  const LaneWindow lw = lane_window(lane, K);
  // first word of the lane's pair inside the staged tile (the prefix copy sits at index 3)
  const uint32_t wbase = 4u + ((lw.d0 == (uint32_t)(NW - 1)) ? 0xFFFFFFFFu : lw.d0);
  uint32_t *tb = sm.tiles + wave * 16 * kTileStride;
  UnitLoader<K> ld;
  ld.init(lane, Tj * NW);

  auto unit_base = [&](int u) -> const uint32_t * {
    const Coords c = unit_coords(P, u);
    const Problem pr = get_problem(P, c.p);
    return pr.code + ((size_t)(8 * c.I + 2 * wave) * Tj + (size_t)8 * c.J) * NW;
  };

  uint32_t ring[kPrefetch][2 * K];
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j)
    if (j < n) load_unit<K>(ring[j], unit_base(ub + j), ld);
  floatx4 acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < n; k0 += kPrefetch) {
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      const int k = k0 + j;
      if (k >= n) break;
      // input rotation for the next kSuper units
      if (k % kSuper == 0) {
        __syncthreads();
        rotate_units(P, ub + k, min(kSuper, n - k), sm);
        __syncthreads();
      }
      // stage unit k's words in the wave's LDS buffer
#pragma unroll
      for (int t = 0; t < K; ++t) {
        *reinterpret_cast<u32x2 *>(tb + ld.lds[t]) = u32x2{ring[j][2 * t], ring[j][2 * t + 1]};
        if (ld.prefix[t]) tb[ld.lds[t] - 4 - (NW - 2) + 3] = ring[j][2 * t + 1];
      }
      // refill this ring slot with unit k + kPrefetch
      if (k + kPrefetch < n) load_unit<K>(ring[j], unit_base(ub + k + kPrefetch), ld);
      wave_sync();
      const int s = k % kSuper;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        u32x4 a = {0u, 0u, 0u, 0u};
        if (m < B) a = *reinterpret_cast<const u32x4 *>(sm.a + ((((s * 8 + 2 * wave + r) * 4 + grp) * B + m) << 2));
        const half8 av = __builtin_bit_cast(half8, a);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const uint32_t *tw = tb + (r * 8 + tt) * kTileStride + wbase;
          const uint32_t bits = lane_bits(tw[0], tw[1], lw.sh);
          u32x4 bw;
          bw[0] = mcg_hash(lane_state<K>(bits, 0));
          bw[1] = mcg_hash(lane_state<K>(bits, 1));
          bw[2] = mcg_hash(lane_state<K>(bits, 2));
          bw[3] = mcg_hash(lane_state<K>(bits, 3));
          acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8, bw), acc[tt], 0, 0, 0);
        }
      }
      wave_sync();
      const Coords c = unit_coords(P, ub + k);
      if (c.I == P.nI - 1 || k == n - 1) {
        const Problem pr = get_problem(P, c.p);
        finish_segment(P, sm, c, pr, acc);
      }
    }
  }
}

// Units of invalid problems: no loads; every segment publishes a zero partial so the column
// blocks still complete (with zero output) and the error word is set.
__device__ void run_invalid(const GemvParams &P, const Lds &sm, int ub, int ue) {
  if (threadIdx.x == 0) __hip_atomic_fetch_or(P.errword, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  floatx4 acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int u = ub; u < ue; ++u) {
    const Coords c = unit_coords(P, u);
    if (c.I == P.nI - 1 || u == ue - 1) {
      const Problem pr = get_problem(P, c.p);
      finish_segment(P, sm, c, pr, acc);
    }
  }
}

__device__ __forceinline__ int problem_class(const GemvParams &P, int p) {
  const Problem pr = get_problem(P, p);
  return pr.ok ? pr.K : 0;
}

__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams P) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const Lds sm = lds_carve(lds_raw, P.L.B);
  const int g = blockIdx.x;
  const int u0 = wg_start(g, P.U, P.G), u1 = wg_start(g + 1, P.U, P.G);
  const int per_problem = P.nI * P.nJ;
  int u = u0;
  while (u < u1) {
    int p = u / per_problem;
    const int cls = problem_class(P, p);
    int ue = min(u1, (p + 1) * per_problem);
    while (ue < u1 && problem_class(P, p + 1) == cls) {
      ++p;
      ue = min(u1, (p + 1) * per_problem);
    }
    switch (cls) {
      case 2: run_range<2>(P, sm, u, ue); break;
      case 3: run_range<3>(P, sm, u, ue); break;
      case 4: run_range<4>(P, sm, u, ue); break;
      default: run_invalid(P, sm, u, ue); break;
    }
    u = ue;
  }
}

struct DeviceInfo {
  int cus = 0;
  int occ[kMaxB + 1] = {};
};

int device_cus_and_occupancy(int B, int *cus_out) {
  static DeviceInfo cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  DeviceInfo &d = cache[dev];
  if (d.cus == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    d.cus = cus;
  }
  if (d.occ[B] == 0) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemv_kernel, kThreads, lds_bytes(B)) != hipSuccess ||
        occ <= 0)
      occ = 2;
    d.occ[B] = occ;
  }
  *cus_out = d.cus;
  return d.occ[B];
}

struct Geometry {
  int U, G, nI, nJ, maxseg, nq;
  size_t counters_off, partials_off, bytes;
};

Geometry geometry(int n_problems, int in_features, int out_features, int B) {
  Geometry gm;
  gm.nI = in_features / 128;
  gm.nJ = out_features / 128;
  gm.nq = n_problems * gm.nJ;
  const long long U = (long long)gm.nq * gm.nI;
  gm.U = (int)U;
  int cus = 0;
  const int occ = device_cus_and_occupancy(B, &cus);
  long long G = (long long)cus * occ;
  // Debug/test override of the workgroup count (exercises ranges that span column blocks).
  if (const char *env = getenv("TRELLIS_GEMV_WGS")) {
    const long long v = atoll(env);
    if (v > 0) G = v;
  }
  if (G > U) G = U;
  if (G < 1) G = 1;
  gm.G = (int)G;
  const long long per = (U + G - 1) / G;
  gm.maxseg = (int)((per + gm.nI - 1) / gm.nI + 1);
  gm.counters_off = 256;
  gm.partials_off = gm.counters_off + (size_t)kMaxColumnBlocks * 4;
  gm.bytes = gm.partials_off + (size_t)gm.G * gm.maxseg * kMaxB * 128 * sizeof(float);
  return gm;
}

}  // namespace

int gemv_max_column_blocks() { return kMaxColumnBlocks; }

size_t gemv_workspace_bytes(int n_problems, int in_features, int out_features, int B) {
  if (n_problems <= 0) return 256;
  if (B < 1) B = 1;
  if (B > kMaxB) B = kMaxB;
  return geometry(n_problems, in_features, out_features, B).bytes;
}

hipError_t launch_gemv(const GemvLaunch &a, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (a.n_problems <= 0) return hipSuccess;
  if (a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
  const long long units = (long long)a.n_problems * (a.out_features / 128) * (a.in_features / 128);
  if (units >= (1LL << 31)) return hipErrorInvalidValue;
  const Geometry gm = geometry(a.n_problems, a.in_features, a.out_features, a.B);
  if (gm.nq > kMaxColumnBlocks) return hipErrorInvalidValue;
  if (ws_bytes < gm.bytes) return hipErrorInvalidValue;
  GemvParams P;
  P.L = a;
  char *w = static_cast<char *>(ws);
  P.errword = reinterpret_cast<uint32_t *>(w);
  P.counters = reinterpret_cast<uint32_t *>(w + gm.counters_off);
  P.partials = reinterpret_cast<float *>(w + gm.partials_off);
  P.U = gm.U;
  P.G = gm.G;
  P.nI = gm.nI;
  P.nJ = gm.nJ;
  P.maxseg = gm.maxseg;
  gemv_kernel<<<gm.G, kThreads, lds_bytes(a.B), stream>>>(P);
  return hipGetLastError();
}

}  // namespace trellis
