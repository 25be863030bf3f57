// trellis_gemv / trellis_gemv_list / trellis_moe_gemv / trellis_moe_mlp: fused small-batch
// products against trellis-coded weights.
//
// y = had(had(x*su) @ W_hat) * sv  ("Escha-W2 runs on Metal", reconstruction paragraph),
// for B = 1..8 rows, over a list of problems: up to eight layers of any shapes with their
// own inputs and outputs, or the routed entries of an expert pointer table ("EXLR8" page:
// per-expert widths, a pointer table re-read every launch, one hidden-side rotation shared
// by all experts).
//
// One launch per problem list.  A "unit" is one 128-row input block I times one 128-column
// output block J of one problem, i.e. 8x8 tiles; units are numbered problem by problem,
// column block by column block, I fastest.  They are cut into "chunks" of consecutive
// units: G equal chunks, one per workgroup, every workgroup resident at once (so every one
// streams the same code bytes whatever the shapes or widths).  Inside a workgroup
// (4 waves) every wave takes two of the unit's eight tile rows:
//   * loads: the wave's 2 x 8 tiles are 2 x 256K contiguous bytes, copied straight from
//     global memory into a wave-private LDS ring (global_load_lds, 16 B per lane, fully
//     coalesced) several units ahead of use; a lane's circular window is read as two LDS
//     words of its tile;
//   * input rotation: per sub-range the workgroup butterflies x*su (unnormalised) and
//     stores fp16 MFMA A-operands in LDS, each value twice and scaled by an exact 2^-4
//     (below);
//   * contraction: per tile each lane decodes its four symbols (trellis_device.h) to four
//     MCG hash words and feeds them UNSUMMED to v_mfma_f32_16x16x32_f16 as eight fp16
//     B-elements along k.  The A operand repeats each activation for the lo and hi halves,
//     so the matrix core forms x*lo + x*hi in fp32 and the codebook's lo+hi addition costs
//     no vector instruction.  One MFMA covers one tile; batch rows ride in the 16 M rows
//     (rows past B multiply zeros and are ignored).  This fp32 sum of the
//     halves is the exact value before the format's fp16 rounding; it differs from the
//     rounded codebook value by at most half an fp16 ulp.
// Finishing, in the same launch: a chunk's fp32 partial y_pre[B][128] of each column block
// it touches (its "segments") is stored with device-scope (sc1) stores.  At the end of the
// chunk, once every thread has waited for those stores to complete, the workgroup counts the
// chunk in per column block with one device-scope atomic.  Whoever brings a block's count to
// the number of chunks that cover it adds the block's partials in chunk order (so the sum
// does not depend on who arrives last), applies the output Hadamard, the scales and the
// exact factor that remains of the two 1/sqrt(128), and writes fp16 y; then it resets the
// block's counter for the next call.  Blocks finish as soon as their last chunk is done,
// while other chunks are still decoding.
//
// Magnitudes: the butterfly of a 128-block grows values by up to 128 (sqrt(128) for random
// signs).  The rotated activations are stored as fp16 times 2^-4, close to the normalised
// 1/sqrt(128) = 2^-3.5, so any block whose normalised rotation is representable in fp16 is
// (2^-4 is exact; the output side applies 2^-7 / 2^-4 = 2^-3).
#include <climits>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "launch.h"
#include "trellis_device.h"

namespace trellis {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxB = 8;
constexpr int kMaxTasks = 4;     // (unit, batch row) rotations per wave and sub-range
constexpr int kABudget = 32768;  // LDS bytes for A operands
// Code ring per wave.  7 KB keeps a workgroup at batch 1 within 40 KB of LDS, so four
// workgroups (16 waves) share a CU; more waves per SIMD hide the decode's latencies better
// than deeper rings hide memory latency (measured).
constexpr int kRingBytes = 7168;
constexpr float kInScale = 0.0625f;  // 2^-4 on the stored rotated activations
constexpr float kOutScale = 0.125f;  // 2^-7 / 2^-4: the rest of the two 1/sqrt(128)

struct GemvParams {
  // (the fields read before a workgroup's first code copy come first)
  int U;                // total units
  int CH;               // units per chunk (chunk c = workgroup c; the last may be shorter)
  int G;                // workgroups = chunks
  int kA;               // units per sub-range (A-operand capacity)
  int maxseg;           // column blocks a chunk can touch
  int nI, nJ;           // table mode: the uniform shape in blocks
  int ubase[kMaxList + 1];  // list mode: first unit of each problem (U past the last)
  int qbase[kMaxList + 1];  // list mode: first column block of each problem
  uint32_t *errword;
  uint32_t *counters;   // [finish groups], zero between calls
  float *partials;      // [G][maxseg][B][128]
  long long partial_bytes;
  GemvLaunch L;
};

// Dynamic LDS layout for batch B.
struct Lds {
  uint32_t *a;      // [kA][8 tile rows][4 groups][B][4 words]; at the end: arrival flags
  uint32_t *tiles;  // [kWaves][kRingBytes / 4]: each wave's code ring
  float *red;       // [kWaves][B][128]; at the end: one block's sums
};

__host__ __device__ constexpr size_t lds_a_bytes(int B, int kA) { return (size_t)kA * 8 * 4 * B * 16; }
__host__ __device__ constexpr size_t lds_tiles_bytes() { return (size_t)kWaves * kRingBytes; }
__host__ __device__ constexpr size_t lds_bytes(int B, int kA) {
  return lds_a_bytes(B, kA) + lds_tiles_bytes() + (size_t)kWaves * B * 128 * 4;
}

__device__ __forceinline__ Lds lds_carve(char *base, int B, int kA) {
  Lds s;
  s.a = reinterpret_cast<uint32_t *>(base);
  s.tiles = reinterpret_cast<uint32_t *>(base + lds_a_bytes(B, kA));
  s.red = reinterpret_cast<float *>(base + lds_a_bytes(B, kA) + lds_tiles_bytes());
  return s;
}

// One problem, resolved (wave-uniform).
struct Problem {
  const uint32_t *code;
  const uint16_t *rin, *rout;
  const float *s_in, *s_out;
  const uint16_t *x;
  uint16_t *y;
  int K;
  int cb;  // 1: MCG fp16 values; 2: the same rounded to E4M3
  int in, out;
  bool ok;
};

template <bool LIST>
__device__ __forceinline__ Problem get_problem(const GemvParams &P, int p) {
  Problem r;
  const int B = P.L.B;
  if constexpr (LIST) {
    const GemvItem &it = P.L.list[p];
    r.code = reinterpret_cast<const uint32_t *>(it.L.code);
    r.rin = it.L.rin;
    r.rout = it.L.rout;
    r.s_in = it.L.s_in;
    r.s_out = it.L.s_out;
    r.K = it.L.K;
    r.cb = it.L.cb;
    r.in = it.L.in_features;
    r.out = it.L.out_features;
    r.x = it.x;
    r.y = it.y;
    r.ok = r.K >= 2 && r.K <= 4 && (r.cb == 1 || r.cb == 2);
  } else {
    const int grp = P.L.group;
    const int slot = grp == 1 ? p : p / grp;
    const int e = P.L.routed[slot];
    bool ok = e >= 0 && e < P.L.E;
    trellis_linear d{};
    if (ok) d = P.L.table[e * grp + (p - slot * grp)];
    r.code = reinterpret_cast<const uint32_t *>(d.code);
    r.K = d.K;
    r.cb = d.cb;
    r.rin = d.rin;
    r.s_in = d.s_in;
    r.rout = d.rout;
    r.s_out = d.s_out;
    if (P.L.shared_side == 0) { r.rin = P.L.shared_r; r.s_in = P.L.shared_s; }
    if (P.L.shared_side == 1) { r.rout = P.L.shared_r; r.s_out = P.L.shared_s; }
    r.in = P.L.in_features;
    r.out = P.L.out_features;
    r.x = P.L.x + (P.L.x_per_problem ? (size_t)p * B * r.in : (size_t)0);
    r.y = P.L.y + (size_t)p * B * r.out;
    r.ok = ok && d.K >= 2 && d.K <= 4 && (d.cb == 1 || d.cb == 2) && d.code != nullptr && r.rin != nullptr &&
           r.rout != nullptr && d.in_features == P.L.in_features && d.out_features == P.L.out_features;
  }
  return r;
}


// Unit and column-block numbering over the problems.
template <bool LIST>
__device__ __forceinline__ int problem_of_unit(const GemvParams &P, int u) {
  if constexpr (LIST) {
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxList; ++i) p += u >= P.ubase[i];  // (entries past the list hold U)
    return p;
  } else {
    return u / (P.nI * P.nJ);
  }
}
template <bool LIST>
__device__ __forceinline__ int problem_of_block(const GemvParams &P, int q) {
  if constexpr (LIST) {
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxList; ++i) p += q >= P.qbase[i];
    return p;
  } else {
    return q / P.nJ;
  }
}
template <bool LIST>
__device__ __forceinline__ int units_base(const GemvParams &P, int p) {
  if constexpr (LIST) return P.ubase[p];
  else return p * P.nI * P.nJ;
}
template <bool LIST>
__device__ __forceinline__ int blocks_base(const GemvParams &P, int p) {
  if constexpr (LIST) return P.qbase[p];
  else return p * P.nJ;
}
template <bool LIST>
__device__ __forceinline__ int nI_of(const GemvParams &P, int p) {
  if constexpr (LIST) return P.L.list[p].L.in_features / 128;
  else return P.nI;
}
template <bool LIST>
__device__ __forceinline__ int block_of_unit(const GemvParams &P, int u) {
  const int p = problem_of_unit<LIST>(P, u);
  return blocks_base<LIST>(P, p) + (u - units_base<LIST>(P, p)) / nI_of<LIST>(P, p);
}
// The chunks that meet column block q: c_lo .. c_hi.  Every chunk after c_lo starts inside
// block q, so q is its first segment; q is segment seg_lo of chunk c_lo.
struct BlockChunks {
  int lo, hi, seg_lo;
};
__device__ __forceinline__ int chunk_start(const GemvParams &P, int c) { return c * P.CH; }
__device__ __forceinline__ int chunk_end(const GemvParams &P, int c) { return min(P.U, (c + 1) * P.CH); }
__device__ __forceinline__ int chunk_of(const GemvParams &P, int u) { return u / P.CH; }
template <bool LIST>
__device__ __forceinline__ BlockChunks block_chunks(const GemvParams &P, int q) {
  const int p = problem_of_block<LIST>(P, q);
  const int nI = nI_of<LIST>(P, p);
  const int qs = units_base<LIST>(P, p) + (q - blocks_base<LIST>(P, p)) * nI;
  BlockChunks c;
  c.lo = chunk_of(P, qs);
  c.hi = chunk_of(P, qs + nI - 1);
  c.seg_lo = q - block_of_unit<LIST>(P, chunk_start(P, c.lo));
  return c;
}

// Finish groups: the column blocks whose partials one finishing workgroup combines.
//   plain: one block;  SwiGLU: the gate and the up block of one (slot, half, J);
//   weighted: block J of every problem.
template <bool LIST>
__device__ __forceinline__ int group_of_block(const GemvParams &P, int q) {
  if (LIST || P.L.finish == kFinishPlain) return q;
  const int p = q / P.nJ, J = q - p * P.nJ;
  if (P.L.finish == kFinishSwiGLU) {
    const int H = P.L.halves;
    const int slot = p / (2 * H), h = (p - slot * 2 * H) % H;
    return (slot * H + h) * P.nJ + J;
  }
  return J;
}
template <bool LIST>
__device__ __forceinline__ int group_arrivals(const GemvParams &P, int f) {
  auto n = [&](int q) {
    const BlockChunks c = block_chunks<LIST>(P, q);
    return c.hi - c.lo + 1;
  };
  if (LIST || P.L.finish == kFinishPlain) return n(f);
  if (P.L.finish == kFinishSwiGLU) {
    const int H = P.L.halves, nJ = P.nJ;
    const int slot = f / (H * nJ), rem = f - slot * H * nJ;
    const int pg = slot * 2 * H + rem / nJ, J = rem - (rem / nJ) * nJ;
    return n(pg * nJ + J) + n((pg + H) * nJ + J);
  }
  int t = 0;
  for (int k = 0; k < P.L.n_problems; ++k) t += n(k * P.nJ + f);
  return t;
}

// Wave issue priority (s_setprio takes an immediate).
__device__ __forceinline__ void set_priority(int prio) {
  if (prio >= 3) __builtin_amdgcn_s_setprio(3);
  else if (prio == 2) __builtin_amdgcn_s_setprio(2);
  else if (prio == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Orders this wave's LDS accesses (all lanes of one wave run in lockstep and the LDS
// executes one wave's operations in order; this only stops the compiler from moving them).
__device__ __forceinline__ void wave_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}


// ---------------------------------------------------------------------------------------
// Input rotation.  a[((s*8 + ti)*4 + g)*B + m] holds, for tile row ti of unit s and batch
// row m, the four words for rows (2g, 2g+1, 2g+8, 2g+9), each word the fp16 value twice.
// The loads of a sub-range's rotation are issued before its first code loads (vector
// memory completions are counted in issue order), the arithmetic runs after.
// ---------------------------------------------------------------------------------------
struct RotLoads {
  float x0[kMaxTasks], x1[kMaxTasks], r0[kMaxTasks], r1[kMaxTasks], s0[kMaxTasks], s1[kMaxTasks];
};

__device__ __forceinline__ void rotation_compute(int B, int n, int wave, const RotLoads &rl, const Lds &sm) {
  const int lane = opaque_tid() & 63;
#pragma unroll
  for (int t = 0; t < kMaxTasks; ++t) {
    const int task = wave + kWaves * t;
    if (task < n * B) {
      const int s = task / B, b = task - s * B;
      float va = rl.x0[t] * rl.r0[t] * rl.s0[t];
      float vb = rl.x1[t] * rl.r1[t] * rl.s1[t];
      wave_fwht128(va, vb);
      // element k = lane (+64): tile row ti = k >> 4, in-tile row rr = k & 15
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ti = (lane >> 4) + 4 * h, rr = lane & 15;
        const int g = (rr & 7) >> 1, w = 2 * (rr >> 3) + (rr & 1);
        const uint32_t hv = f2h((h ? vb : va) * kInScale);
        sm.a[((((s * 8 + ti) * 4 + g) * B + b) << 2) + w] = hv | (hv << 16);
      }
    }
  }
}

// The same rotation with 16-byte accesses (x, rin and s_in 16-byte aligned): lanes
// 16j..16j+15 of wave w take task w + kWaves*j (its unit's 128-block of one batch row), lane
// i of the group holding elements 8i..8i+7 -- four load instructions per lane for a task
// instead of six per task and wave.  Three butterfly stages run in registers and four
// across the group's 16 lanes; element k = 8i + t lands where the scalar form puts it.
struct RotVec {
  u32x4 x, r;
  floatx4 s0, s1;
};

template <bool WITH_S>
__device__ __forceinline__ RotVec rot_vec_load(const uint16_t *xp, const uint16_t *rin, const float *s_in, int in,
                                               int B, int task, int I) {
  const int i = opaque_tid() & 15;
  const int s = task / B, b = task - s * B;
  (void)s;
  const int k = I * 128 + 8 * i;
  RotVec q;
  q.x = ldg(reinterpret_cast<const u32x4 *>(xp + (size_t)b * in + k));
  q.r = ldg(reinterpret_cast<const u32x4 *>(rin + k));
  if constexpr (WITH_S) {
    q.s0 = ldg(reinterpret_cast<const floatx4 *>(s_in + k));
    q.s1 = ldg(reinterpret_cast<const floatx4 *>(s_in + k + 4));
  } else {
    q.s0 = floatx4{1.f, 1.f, 1.f, 1.f};
    q.s1 = floatx4{1.f, 1.f, 1.f, 1.f};
  }
  return q;
}

__device__ __forceinline__ void rot_vec_compute(int B, int n, int task, const RotVec &q, const Lds &sm) {
  const int lane = opaque_tid() & 63, i = lane & 15;
  float v[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t xw = q.x[t >> 1], rw = q.r[t >> 1];
    const float xs = h2f((t & 1) ? (uint16_t)(xw >> 16) : (uint16_t)xw);
    const float rs = h2f((t & 1) ? (uint16_t)(rw >> 16) : (uint16_t)rw);
    v[t] = xs * rs * (t < 4 ? q.s0[t] : q.s1[t - 4]);
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
#pragma unroll
  for (int t = 0; t < 8; ++t) fwht_stage1(v[t], lane);
  if (task < n * B) {
    const int s = task / B, b = task - s * B;
    // element k = 8i + t: tile row ti = i >> 1, in-tile row rr = 8(i & 1) + t, so group
    // g = t >> 1 and word w = 2(i & 1) + (t & 1): one 8-byte write per pair of elements
    const int ti = i >> 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t h0 = f2h(v[2 * g] * kInScale), h1 = f2h(v[2 * g + 1] * kInScale);
      *reinterpret_cast<u32x2 *>(sm.a + ((((s * 8 + ti) * 4 + g) * B + b) << 2) + 2 * (i & 1)) =
          u32x2{h0 | (h0 << 16), h1 | (h1 << 16)};
    }
  }
}

// Workgroup barrier for LDS traffic only: the waves' code copies in flight are not waited
// for (a plain __syncthreads would wait for every outstanding vector memory operation).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// End of a segment (chunk c's share of a column block, its segment seg): reduce the waves'
// accumulators and store the partial with device-scope stores.  The stores are not waited
// for here (code copies in flight keep streaming); the arrival at the end of the chunk
// waits for them.
__device__ __forceinline__ void publish_partial(const GemvParams &P, const Lds &sm, int c, int seg,
                                                floatx4 (&acc)[8]) {
  const int B = P.L.B;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int mrow = 4 * (lane >> 4) + r;
    if (mrow < B) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sm.red[(wave * B + mrow) * 128 + 16 * jj + (lane & 15)] = acc[jj][r];
    }
  }
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  lds_barrier();
  const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(P.partials, P.partial_bytes);
  const uint32_t base = (uint32_t)(((size_t)c * P.maxseg + seg) * B * 128 * 4);
  for (int idx = tid; idx < B * 128; idx += kThreads) {
    float v = sm.red[idx];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += sm.red[w * B * 128 + idx];
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rp, base + 4 * idx, 0, kSC1);
  }
  lds_barrier();
}

// ---------------------------------------------------------------------------------------
// Code streaming.  Each wave owns a ring of kRingBytes of LDS holding whole units (its two
// tile rows x 8 tiles: 16 tiles, row-major, tile (r, t) at word (8r + t) * 8K).  The rows
// are copied straight from global memory into the ring with global_load_lds (no register
// staging), so many units are in flight per wave.  These copies are not tracked by the
// compiler's wait-count insertion: the loop waits for them itself with s_waitcnt vmcnt(N),
// issuing exactly kDma copies per unit on every path (dummy copies past the end) so that N
// is a compile-time constant.  Vector memory operations complete in issue order.
// ---------------------------------------------------------------------------------------

template <int K>
struct Ring {
  static constexpr int NW = 8 * K;                      // words per tile
  static constexpr int UNIT_BYTES = 16 * NW * 4;       // 1024 / 1536 / 2048
  static constexpr int SLOTS = kRingBytes / UNIT_BYTES; // 7 / 4 / 3
  static constexpr int DMA = (K == 2) ? 1 : 2;          // copies per unit
  static constexpr int WAIT = DMA * (SLOTS - 1);        // copies younger than the unit in use
  static_assert(WAIT < 64, "vmcnt range");
};

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int imm = (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(imm);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void *lds_void_ptr;

// Copy the wave's two tile rows of a unit into ring slot `dst` (LDS).  The copies are
// buffer loads straight into LDS over the problem's code array (scalar resource `rc`):
// `off` (bytes, wave-uniform) is where the unit's first row starts, `rs` the row stride in
// words.  `real` = false: a dummy copy of the array's first bytes (the count of copies per
// unit stays fixed).  Every offset is 32-bit (a problem's code array is under 2 GiB), so no
// per-lane 64-bit address is kept live across the loop.
template <int K>
__device__ __forceinline__ void dma_unit(__amdgpu_buffer_rsrc_t rc, uint32_t off, uint32_t rs, uint32_t *dst,
                                         bool real) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // (recomputed here: cheaper than keeping it live)
  const uint32_t so = real ? off : 0u;
  if constexpr (K == 2) {
    // 2 x 512 B: lanes 0..31 take row 0, lanes 32..63 row 1, 16 B each
    const uint32_t vo = 4u * ((uint32_t)(lane >> 5) * rs + 4u * (uint32_t)(lane & 31));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void_ptr)dst, 16, vo, so, 0, 0);
  } else if constexpr (K == 3) {
    // 2 x 768 B = 96 pieces of 16 B: lanes 0..63 take pieces 0..63, then lanes 0..31 take
    // pieces 64..95 (a piece never straddles the two rows: 768 is a multiple of 16)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int piece = 64 * c + lane;
      const int r = piece >= 48 ? (piece >= 96 ? 2 : 1) : 0;
      const uint32_t vo = 4u * ((uint32_t)r * rs + 4u * (uint32_t)(piece - 48 * r));
      if (c == 0 || lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void_ptr)(dst + c * 256), 16, vo, so, 0, 0);
    }
  } else {
    // 2 x 1024 B: one copy per row, 16 B per lane
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t vo = 4u * ((uint32_t)r * rs + 4u * (uint32_t)lane);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void_ptr)(dst + r * 256), 16, vo, so, 0, 0);
    }
  }
}

// Units [ub, ue) of problem p (width K), part of chunk c, in sub-ranges of at most P.kA
// units.  Each sub-range issues its rotation loads and its first code copies, rotates while
// the code is in flight, then streams with SLOTS - 1 units in flight per wave.  q0: the
// chunk's first column block (segment numbering).  fresh: the workgroup's first part
// (nothing of an earlier part to wait for).
// CB = 2 (the E4M3 codebook, "EXLR8" page): each lane's four values are the E4M3-rounded
// codebook values, converted back to fp16 (exact) and fed to v_mfma_f32_16x16x16_f16 with
// the A operand's duplicated words repacked once per tile row into (x0, x1), (x8, x9).
template <int K, int CB, bool LIST>
__device__ void run_problem(const GemvParams &P, const Lds &sm, const Problem &pr, int p, int ub, int ue, int c,
                            int q0, bool fresh) {
  using RG = Ring<K>;
  constexpr int NW = RG::NW;
  constexpr int SLOTS = RG::SLOTS;
  const int B = P.L.B;
  const int Tj = pr.out / 16;
  const int nI = pr.in / 128;
  // The lane's constants are derived here, per call: left to itself the compiler computes
  // them once per width at kernel entry and keeps every width's set live across the chunk
  // loop, which spills in the kernels that handle several widths.
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, grp = lane >> 4;
  const LaneWindow lw = lane_window(lane, K);
  uint32_t *ring = sm.tiles + wave * (kRingBytes / 4);
  const int mc = m < B ? m : B - 1;  // batch row of the A operand (rows past B are ignored)
  const uint32_t a_lane = (uint32_t)((grp * B + mc) << 2);
  const size_t row_stride = (size_t)Tj * NW;
  // the problem's code array as a buffer; offsets in bytes from its start (32-bit: arrays
  // of 2 GiB or more are rejected at launch)
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(pr.code, (long long)(pr.in / 16) * (long long)row_stride * 4);
  const uint32_t rs = (uint32_t)row_stride;
  const uint32_t code_off = (uint32_t)(2 * wave) * rs * 4u;  // this wave's two tile rows
  const uint32_t row_block_bytes = 8u * rs * 4u;
  const int first = __builtin_amdgcn_readfirstlane(ub - units_base<LIST>(P, p));
  const int total = __builtin_amdgcn_readfirstlane(ue - ub);
  const int in = pr.in;
  const uint16_t *xp = pr.x;
  const int qp = __builtin_amdgcn_readfirstlane(blocks_base<LIST>(P, p) - q0);  // segment of J = 0

  floatx4 acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Issue priority from the share of the chunk still to do, in quarters (3 = more than three
  // quarters left).  The waves of a CU otherwise issue oldest-first, so the workgroups
  // resident on a CU would finish one after another and the last would run with few waves at
  // the end; with this rule the ones behind catch up and they finish together.  Priority p
  // applies from unit t[p] = u1 - floor((p + 1) * units / 4) on.
  const int ch_u1 = __builtin_amdgcn_readfirstlane(chunk_end(P, c));
  const int ch_units = __builtin_amdgcn_readfirstlane(ch_u1 - chunk_start(P, c));
  const int t2 = ch_u1 - (3 * ch_units) / 4, t1 = ch_u1 - (2 * ch_units) / 4, t0 = ch_u1 - ch_units / 4;
  auto prio_at = [&](int u) { return u >= t0 ? 0 : u >= t1 ? 1 : u >= t2 ? 2 : 3; };

  for (int sb = 0; sb < total; sb += P.kA) {
    const int n = __builtin_amdgcn_readfirstlane(min(P.kA, total - sb));
    int cur_I = __builtin_amdgcn_readfirstlane((first + sb) % nI);
    int cur_J = __builtin_amdgcn_readfirstlane((first + sb) / nI);
    int pre_I = cur_I;
    // next unit to request: its rows start at nxt (uniform); one step along I adds a row
    // block, the wrap to the next column block moves 8 tiles right and back to I = 0
    uint32_t nxt = code_off + (uint32_t)pre_I * row_block_bytes + (uint32_t)(8 * cur_J * NW * 4);
    const uint32_t wrap_back = (uint32_t)(nI - 1) * row_block_bytes;
    auto advance = [&]() {
      if (++pre_I == nI) {
        pre_I = 0;
        nxt = nxt - wrap_back + 8u * NW * 4u;
      } else {
        nxt += row_block_bytes;
      }
    };
    // the previous sub-range's reads of the A buffer and of the ring are finished (nothing
    // to wait for on the workgroup's first sub-range)
    if (!(fresh && sb == 0)) __syncthreads();
    // The rotation's loads, then the first unit into slot 0; units 1..SLOTS-2 are requested
    // after the rotation.  Vector memory operations complete in issue order, so loads issued
    // after a code copy would wait for it: issued first, the (cache-resident) activations
    // and side vectors arrive while the copy is in flight and the rotation runs under it.
    // At the start of the kernel every wave requests code at once: asking for one unit each
    // first lets the memory system serve everybody's first unit before the deeper
    // prefetches, so the decode starts sooner.
    auto prime = [&](int j) {
      const bool real = j < n;
      dma_unit<K>(rc, nxt, rs, ring + j * (RG::UNIT_BYTES / 4), real);
      if (real) advance();
    };
    auto first_copy = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      prime(0);
      __builtin_amdgcn_sched_barrier(0);
      if (sb == 0) set_priority(prio_at(ub));  // (after the first copy is on its way)
    };
    // Rotation loads: straight-line code (tasks past the last are clamped to it and their
    // values ignored), so all of them are in flight together.
    const bool vec = ((reinterpret_cast<uintptr_t>(xp) | reinterpret_cast<uintptr_t>(pr.rin) |
                       reinterpret_cast<uintptr_t>(pr.s_in)) & 15) == 0;
    if (vec) {
      const int task = min(wave + kWaves * (lane >> 4), n * B - 1);
      const int I = (first + sb + task / B) % nI;
      const RotVec q = pr.s_in ? rot_vec_load<true>(xp, pr.rin, pr.s_in, in, B, task, I)
                               : rot_vec_load<false>(xp, pr.rin, pr.s_in, in, B, task, I);
      first_copy();
      rot_vec_compute(B, n, wave + kWaves * (lane >> 4), q, sm);
    } else {
    RotLoads rq;
    auto load_tasks = [&](auto with_s) {
#pragma unroll
      for (int t = 0; t < kMaxTasks; ++t) {
        const int task = min(wave + kWaves * t, n * B - 1);
        const int s = task / B, b = task - s * B;
        const int I = (first + sb + s) % nI;
        const int k0 = I * 128 + lane, k1 = k0 + 64;
        rq.x0[t] = h2f(ldg(xp + (size_t)b * in + k0));
        rq.x1[t] = h2f(ldg(xp + (size_t)b * in + k1));
        rq.r0[t] = h2f(ldg(pr.rin + k0));
        rq.r1[t] = h2f(ldg(pr.rin + k1));
        if constexpr (decltype(with_s)::value) {
          rq.s0[t] = ldg(pr.s_in + k0);
          rq.s1[t] = ldg(pr.s_in + k1);
        } else {
          rq.s0[t] = 1.f;
          rq.s1[t] = 1.f;
        }
      }
    };
    if (pr.s_in) load_tasks(std::true_type{});
    else load_tasks(std::false_type{});
    first_copy();
    rotation_compute(B, n, wave, rq, sm);
    }
    __syncthreads();  // (also waits for unit 0)
#pragma unroll
    for (int j = 1; j < SLOTS - 1; ++j) prime(j);

    int slot = 0;
    // A operands, kept across units: lanes of MFMA rows past B never load theirs, so those
    // rows multiply zeros rather than copies of row B - 1 (the results of those rows are
    // ignored either way; zeros draw less power in the matrix core, measured ~1% faster).
    u32x4 areg[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    for (int k = 0; k < n; ++k) {
      // copy unit k + SLOTS - 1 into the slot unit k - 1 used (its reads are complete)
      {
        const int ws = (slot == 0 ? SLOTS : slot) - 1;
        const bool real = k + SLOTS - 1 < n;
        dma_unit<K>(rc, nxt, rs, ring + ws * (RG::UNIT_BYTES / 4), real);
        if (real) advance();
      }
      wait_vmcnt<RG::WAIT>();  // unit k has landed
      {
        const int u = ub + sb + k;
        if (u == t2 || u == t1 || u == t0) set_priority(prio_at(u));
      }
      const uint32_t *ub_ = ring + slot * (RG::UNIT_BYTES / 4);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (m < B) areg[r] = *reinterpret_cast<const u32x4 *>(sm.a + (uint32_t)(((k * 8 + 2 * wave + r) * 4 * B) << 2) + a_lane);
        const u32x4 a = areg[r];
        const half8 av = __builtin_bit_cast(half8, a);
        const u32x2 a2 = {__builtin_amdgcn_perm(a[1], a[0], 0x05040100u), __builtin_amdgcn_perm(a[3], a[2], 0x05040100u)};
        // The tile row's window words are all read before its decode starts (the reads'
        // LDS latency then overlaps the first tiles' decode instead of every second tile's).
        uint32_t W0[8], W1[8];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const uint32_t *tw = ub_ + (r * 8 + tt) * NW;
          W0[tt] = tw[lw.d0];
          W1[tt] = tw[lw.d1];
        }
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const uint32_t bits = lane_bits(W0[tt], W1[tt], lw.sh);
          u32x4 bw;
          bw[0] = mcg_hash(lane_state<K>(bits, 0));
          bw[1] = mcg_hash(lane_state<K>(bits, 1));
          bw[2] = mcg_hash(lane_state<K>(bits, 2));
          bw[3] = mcg_hash(lane_state<K>(bits, 3));
          if constexpr (CB == 1) {
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8, bw), acc[tt], 0, 0, 0);
          } else {
            const uint32_t q = e4m3_pack4(bw[0], bw[1], bw[2], bw[3]);
            const half2_t v01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q, 1.0f, false);
            const half2_t v23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q, 1.0f, true);
            const half4_t bv = {v01[0], v01[1], v23[0], v23[1]};
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a2), bv, acc[tt], 0, 0, 0);
          }
        }
      }
      wave_sync();
      if (cur_I == nI - 1 || sb + k == total - 1) publish_partial(P, sm, c, qp + cur_J, acc);
      if (++cur_I == nI) { cur_I = 0; ++cur_J; }
      slot = (slot + 1 == SLOTS) ? 0 : slot + 1;
    }
    wait_vmcnt<0>();  // the dummy copies of the tail have landed before the ring is reused
  }
}

// Units of invalid problems (table mode): no loads; each segment publishes a zero partial
// (the finish writes zeros for invalid problems anyway) and the error word is set.
template <bool LIST>
__device__ void run_invalid(const GemvParams &P, const Lds &sm, int p, int ub, int ue, int c, int q0) {
  if (threadIdx.x == 0) __hip_atomic_fetch_or(P.errword, kErrBadEntry, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  floatx4 acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int nI = nI_of<LIST>(P, p), base = units_base<LIST>(P, p), qb = blocks_base<LIST>(P, p);
  for (int u = ub; u < ue; ++u) {
    const int lu = u - base, J = lu / nI, I = lu - J * nI;
    if (I == nI - 1 || u == ue - 1) publish_partial(P, sm, c, qb + J - q0, acc);
  }
}

// ---------------------------------------------------------------------------------------
// Finishing.
// ---------------------------------------------------------------------------------------

// Sums of column block q's partials at indexes idx_i = threadIdx.x + i * kThreads (i < NI,
// idx < B*128), chunks added in chunk order starting from 0 -- the same order whoever runs
// it.  Loads are device-scope and up to 32 are in flight per thread.
template <bool LIST, int NI>
__device__ __forceinline__ void block_sums(const GemvParams &P, int q, float (&v)[NI]) {
  const int B = P.L.B;
  const BlockChunks c = block_chunks<LIST>(P, q);
  const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(P.partials, P.partial_bytes);
  constexpr int kBatch = 32 / NI;
#pragma unroll
  for (int i = 0; i < NI; ++i) v[i] = 0.f;
  for (int gb = c.lo; gb <= c.hi; gb += kBatch) {
    float part[NI][kBatch];
#pragma unroll
    for (int t = 0; t < kBatch; ++t) {
      const int gg = gb + t;
      const uint32_t slot = (uint32_t)(gg * P.maxseg + (gg == c.lo ? c.seg_lo : 0));
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int idx = threadIdx.x + i * kThreads;
        part[i][t] = 0.f;
        if (gg <= c.hi && idx < B * 128)
          part[i][t] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rp, (slot * B * 128 + idx) * 4, 0, kSC1));
      }
    }
#pragma unroll
    for (int t = 0; t < kBatch; ++t)
#pragma unroll
      for (int i = 0; i < NI; ++i) v[i] += part[i][t];
  }
}

// Output-side scales of columns J*128 + lane and + 64 (rout * s_out * the remaining factor).
__device__ __forceinline__ float2 out_scales(const uint16_t *rout, const float *s_out, int J, int lane) {
  const int c0 = J * 128 + lane, c1 = c0 + 64;
  float sa = h2f(ldg(rout + c0)) * kOutScale, sb = h2f(ldg(rout + c1)) * kOutScale;
  if (s_out) { sa *= ldg(s_out + c0); sb *= ldg(s_out + c1); }
  return float2{sa, sb};
}

template <bool LIST>
__device__ void finish_plain(const GemvParams &P, const Lds &sm, int q) {
  const int B = P.L.B;
  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6;
  const int p = problem_of_block<LIST>(P, q), J = q - blocks_base<LIST>(P, p);
  const Problem pr = get_problem<LIST>(P, p);
  float2 sc = {0.f, 0.f};
  if (pr.ok) sc = out_scales(pr.rout, pr.s_out, J, lane);
  float v[kMaxB * 128 / kThreads];
  block_sums<LIST>(P, q, v);
#pragma unroll
  for (int i = 0; i < kMaxB * 128 / kThreads; ++i) {
    const int idx = tid + i * kThreads;
    if (idx < B * 128) sm.red[idx] = v[i];
  }
  __syncthreads();
  const int c0 = J * 128 + lane;
  for (int b = wave; b < B; b += kWaves) {
    float va = sm.red[b * 128 + lane], vb = sm.red[b * 128 + lane + 64];
    wave_fwht128(va, vb);
    pr.y[(size_t)b * pr.out + c0] = f2h(va * sc.x);       // (an invalid problem has zero scales)
    pr.y[(size_t)b * pr.out + c0 + 64] = f2h(vb * sc.y);
  }
  __syncthreads();
}

// Batch 1: two plain finishes at once, waves 0-1 finishing column block qa and waves 2-3
// block qb (qb < 0: none).  A block's 128 sums need only half the workgroup, and a
// workgroup that arrives last at two blocks would otherwise pay the partials' load latency
// twice.  The partials are added in chunk order, as finish_plain adds them.
template <bool LIST>
__device__ void finish_plain_pair(const GemvParams &P, const Lds &sm, int qa, int qb) {
  const int tid = opaque_tid(), h = tid >> 7, t = tid & 127, lane = tid & 63;
  const int q = __builtin_amdgcn_readfirstlane(h ? qb : qa);
  float v = 0.f;
  if (q >= 0) {
    const BlockChunks c = block_chunks<LIST>(P, q);
    const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(P.partials, P.partial_bytes);
    constexpr int kBatch = 16;
    for (int gb = c.lo; gb <= c.hi; gb += kBatch) {
      float part[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int gg = gb + k;
        const uint32_t slot = (uint32_t)(gg * P.maxseg + (gg == c.lo ? c.seg_lo : 0));
        part[k] = gg <= c.hi ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, (slot * 128 + t) * 4, 0, kSC1))
                             : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) v += part[k];
    }
  }
  sm.red[h * 128 + t] = v;
  __syncthreads();
  if (q >= 0 && ((tid >> 6) & 1) == 0) {
    const int p = problem_of_block<LIST>(P, q), J = q - blocks_base<LIST>(P, p);
    const Problem pr = get_problem<LIST>(P, p);
    float2 sc = {0.f, 0.f};
    if (pr.ok) sc = out_scales(pr.rout, pr.s_out, J, lane);
    float va = sm.red[h * 128 + lane], vb = sm.red[h * 128 + lane + 64];
    wave_fwht128(va, vb);
    const int c0 = J * 128 + lane;
    pr.y[c0] = f2h(va * sc.x);  // (an invalid problem has zero scales)
    pr.y[c0 + 64] = f2h(vb * sc.y);
  }
  __syncthreads();
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z) ("EXLR8" page, calibration paragraph: the
// expert's down projection reads silu(gate x) * up x).  For z below about -88 e^-z is
// +inf in fp32 and the quotient is -0, the limit.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// kFinishSwiGLU, B = 1.  Group f = (slot*H + h)*nJ + J: threads 0..127 sum the gate
// entry's partials, threads 128..255 the up entry's; waves 0 and 2 rotate and scale them;
// then a = silu(g) * u is written as fp16 to y[slot][(h*nJ + J)*128 + c].
__device__ void finish_swiglu(const GemvParams &P, const Lds &sm, int f) {
  const int H = P.L.halves, nJ = P.nJ;
  const int slot = f / (H * nJ), rem = f - slot * H * nJ;
  const int pg = slot * 2 * H + rem / nJ, J = rem - (rem / nJ) * nJ;
  const int tid = opaque_tid(), c = tid & 127, which = tid >> 7, lane = tid & 63;
  const int p = which ? pg + H : pg;
  const bool rot = (tid & 127) < 64;  // waves 0 (gate) and 2 (up)
  float2 sc = {0.f, 0.f};
  if (rot) {
    const Problem pr = get_problem<false>(P, p);
    if (pr.ok) sc = out_scales(pr.rout, pr.s_out, J, lane);  // (an invalid entry's output is zero)
  }
  // each half of the workgroup sums one block: thread t of the half takes column t
  const BlockChunks cb = block_chunks<false>(P, p * nJ + J);
  const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(P.partials, P.partial_bytes);
  float v = 0.f;
  for (int gb = cb.lo; gb <= cb.hi; gb += 32) {
    float part[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int gg = gb + t;
      const uint32_t s = (uint32_t)(gg * P.maxseg + (gg == cb.lo ? cb.seg_lo : 0));
      part[t] = gg <= cb.hi ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, (s * 128 + c) * 4, 0, kSC1))
                           : 0.f;
    }
#pragma unroll
    for (int t = 0; t < 32; ++t) v += part[t];
  }
  float *gu = sm.red;  // [2][128]
  gu[which * 128 + c] = v;
  __syncthreads();
  if (rot) {
    float va = gu[which * 128 + lane], vb = gu[which * 128 + lane + 64];
    wave_fwht128(va, vb);
    gu[which * 128 + lane] = va * sc.x;
    gu[which * 128 + lane + 64] = vb * sc.y;
  }
  __syncthreads();
  if (tid < 128) {
    const int inter = H * nJ * 128;
    P.L.y[(size_t)slot * inter + rem * 128 + c] = f2h(silu(gu[c]) * gu[128 + c]);
  }
  __syncthreads();
}

// kFinishWeighted, B = 1.  Group J: thread (r, c) (r = tid / 128) adds w[k] * (sum of
// problem k's partials of block J) over k = r, r + 2, ..., in that order; the two sums are
// added in r order, rotated once and scaled by the shared sv.
__device__ void finish_weighted(const GemvParams &P, const Lds &sm, int J) {
  const int tid = opaque_tid(), c = tid & 127, r = tid >> 7, lane = tid & 63;
  const int nJ = P.nJ, n = P.L.n_problems;
  const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(P.partials, P.partial_bytes);
  float acc = 0.f;
  for (int k = r; k < n; k += 2) {
    const int q = k * nJ + J;
    const BlockChunks cb = block_chunks<false>(P, q);
    float v = 0.f;
    for (int gb = cb.lo; gb <= cb.hi; gb += 32) {
      float part[32];
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        const int gg = gb + t;
        const uint32_t s = (uint32_t)(gg * P.maxseg + (gg == cb.lo ? cb.seg_lo : 0));
        part[t] = gg <= cb.hi ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, (s * 128 + c) * 4, 0, kSC1))
                             : 0.f;
      }
#pragma unroll
      for (int t = 0; t < 32; ++t) v += part[t];
    }
    acc += ldg(P.L.router_w + k) * v;
  }
  sm.red[r * 128 + c] = acc;
  __syncthreads();
  if (tid < 64) {
    float va = sm.red[lane] + sm.red[128 + lane];
    float vb = sm.red[lane + 64] + sm.red[128 + lane + 64];
    const float2 sc = out_scales(P.L.shared_r, P.L.shared_s, J, lane);
    wave_fwht128(va, vb);
    P.L.y[J * 128 + lane] = f2h(va * sc.x);
    P.L.y[J * 128 + lane + 64] = f2h(vb * sc.y);
  }
  __syncthreads();
}

// End of chunk c: count the chunk in at the finish group of each of its segments; finish
// the groups whose count this brings to the number of chunks covering them, and reset their
// counters.
template <bool LIST>
__device__ void arrive_chunk(const GemvParams &P, const Lds &sm, int c) {
  const int cu0 = chunk_start(P, c), cu1 = chunk_end(P, c);
  const int q0 = block_of_unit<LIST>(P, cu0), q1 = block_of_unit<LIST>(P, cu1 - 1);
  __builtin_amdgcn_s_setprio(3);  // the arrivals and finishes ahead of other workgroups' decode
  // Every thread's partial stores have completed before any counter moves (a workgroup
  // barrier does not wait for global stores), so an arrival publishes complete partials.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  uint32_t *flags = sm.tiles;  // (the code ring is idle once the chunk is done)
  for (int base = q0; base <= q1; base += kThreads) {
    const int q = base + (int)threadIdx.x;
    if (q <= q1) {
      const int f = group_of_block<LIST>(P, q);
      const uint32_t old = __hip_atomic_fetch_add(P.counters + f, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      flags[threadIdx.x] = old + 1 == (uint32_t)group_arrivals<LIST>(P, f) ? 1u : 0u;
    }
    __syncthreads();
    const int cnt = min(kThreads, q1 - base + 1);
    // The other chunks' partials are read after their arrivals were seen, with device-scope
    // (sc1) loads, which read the coherent copy (the per-XCD L2s hold no stale one): no
    // cache invalidation is needed.
    if (LIST && P.L.B == 1) {
      int pend = -1;  // (uniform)
      for (int i = 0; i < cnt; ++i) {
        if (__builtin_amdgcn_readfirstlane(flags[i])) {
          const int f = group_of_block<LIST>(P, base + i);
          if (pend < 0) {
            pend = f;
            continue;
          }
          finish_plain_pair<LIST>(P, sm, pend, f);
          if (threadIdx.x == 0) {
            __hip_atomic_store(P.counters + pend, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(P.counters + f, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          pend = -1;
        }
      }
      if (pend >= 0) {
        finish_plain_pair<LIST>(P, sm, pend, -1);
        if (threadIdx.x == 0) __hip_atomic_store(P.counters + pend, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      for (int i = 0; i < cnt; ++i) {
        if (__builtin_amdgcn_readfirstlane(flags[i])) {
          const int f = group_of_block<LIST>(P, base + i);
          if (LIST || P.L.finish == kFinishPlain) finish_plain<LIST>(P, sm, f);
          else if (P.L.finish == kFinishSwiGLU) finish_swiglu(P, sm, f);
          else finish_weighted(P, sm, f);
          if (threadIdx.x == 0) __hip_atomic_store(P.counters + f, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();
  }
}

// The units [cu0, cu1) of one chunk, problem by problem.
template <bool LIST, int KS, int CBS>
__device__ __forceinline__ void run_chunk(const GemvParams &P, const Lds &sm, int c) {
  const int cu0 = chunk_start(P, c), cu1 = chunk_end(P, c);
  const int q0 = block_of_unit<LIST>(P, cu0);
  for (int u = cu0; u < cu1;) {
    const int p = problem_of_unit<LIST>(P, u);
    const int ue = min(cu1, units_base<LIST>(P, p + 1));
    const Problem pr = get_problem<LIST>(P, p);
    const bool f = u == cu0;  // (the workgroup's first part: nothing earlier to wait for)
    if constexpr (KS != 0) {
      run_problem<KS, CBS, LIST>(P, sm, pr, p, u, ue, c, q0, f);
    } else {
      const int sel = pr.ok ? pr.K + 4 * (pr.cb - 1) : 0;
      if (sel == 2) run_problem<2, 1, LIST>(P, sm, pr, p, u, ue, c, q0, f);
      else if (sel == 3) run_problem<3, 1, LIST>(P, sm, pr, p, u, ue, c, q0, f);
      else if (sel == 4) run_problem<4, 1, LIST>(P, sm, pr, p, u, ue, c, q0, f);
      else if (CBS == 0 && sel == 6) run_problem<2, 2, LIST>(P, sm, pr, p, u, ue, c, q0, f);
      else if (CBS == 0 && sel == 7) run_problem<3, 2, LIST>(P, sm, pr, p, u, ue, c, q0, f);
      else if (CBS == 0 && sel == 8) run_problem<4, 2, LIST>(P, sm, pr, p, u, ue, c, q0, f);
      else run_invalid<LIST>(P, sm, p, u, ue, c, q0);
    }
    u = ue;
  }
}

// LIST: list mode.  KS = 2, 3, 4: every problem has that width and codebook CBS (the K
// dispatch compiled away, a smaller kernel); KS = 0: per-problem K, with CBS = 1 (every
// problem on the MCG codebook) or 0 (either codebook).
template <bool LIST, int KS, int CBS>
__global__ __launch_bounds__(kThreads, 4) void gemv_kernel(GemvParams P) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const Lds sm = lds_carve(lds_raw, P.L.B, P.kA);
  const int c = blockIdx.x;  // (chunk c; the launch has exactly G = chunks workgroups)
  // Top issue priority for the chunk's set-up: its loads go out while other workgroups on
  // the CU decode (and a workgroup dispatched after its CU's others are already decoding
  // would otherwise run its prologue at the lowest priority, behind them).
  __builtin_amdgcn_s_setprio(3);
  run_chunk<LIST, KS, CBS>(P, sm, c);
  arrive_chunk<LIST>(P, sm, c);
}

// An empty weighted sum (no routed experts): y = 0.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint16_t *y, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = 0;
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemv_kernel<false, 0, 0>, kThreads,
                                                     lds_bytes(B, kWaves * kMaxTasks / B)) != hipSuccess ||
        occ <= 0)
      occ = 2;
    d.occ[B] = occ;
  }
  *cus_out = d.cus;
  return d.occ[B];
}

struct Geometry {
  bool ok = false;
  int U = 0, G = 0, CH = 0, maxseg = 0, kA = 0, nq = 0, nf = 0;
  int ubase[kMaxList + 1] = {}, qbase[kMaxList + 1] = {};
  size_t partial_bytes = 0, bytes = 0;
};

constexpr int kMinChunkAt4 = 13;

Geometry geometry(const GemvLaunch &a) {
  Geometry gm;
  const int B = a.B < 1 ? 1 : (a.B > kMaxB ? kMaxB : a.B);
  long long U = 0, nq = 0;
  int nI_min = INT_MAX;
  if (a.table == nullptr) {
    for (int p = 0; p < a.n_list; ++p) {
      gm.ubase[p] = (int)U;
      gm.qbase[p] = (int)nq;
      const int nI = a.list[p].L.in_features / 128, nJ = a.list[p].L.out_features / 128;
      U += (long long)nI * nJ;
      nq += nJ;
      nI_min = nI < nI_min ? nI : nI_min;
    }
    for (int p = a.n_list; p <= kMaxList; ++p) {
      gm.ubase[p] = (int)(U < INT_MAX ? U : INT_MAX);
      gm.qbase[p] = (int)(nq < INT_MAX ? nq : INT_MAX);
    }
  } else {
    const int nI = a.in_features / 128, nJ = a.out_features / 128;
    U = (long long)a.n_problems * nI * nJ;
    nq = (long long)a.n_problems * nJ;
    nI_min = nI;
  }
  if (U <= 0 || U >= (1LL << 31) || nq > kMaxFinishGroups) return gm;
  // code offsets are 32-bit byte offsets from each array's start: every code array is
  // under 2 GiB (in * out * K / 8 bytes, K <= 4)
  {
    const long long max_code = 1LL << 31;
    if (a.table == nullptr) {
      for (int p = 0; p < a.n_list; ++p)
        if ((long long)a.list[p].L.in_features * a.list[p].L.out_features / 2 >= max_code) return gm;
    } else if ((long long)a.in_features * a.out_features / 2 >= max_code) {
      return gm;
    }
  }
  gm.U = (int)U;
  gm.nq = (int)nq;
  gm.nf = a.table && a.finish == kFinishSwiGLU ? gm.nq / 2
        : a.table && a.finish == kFinishWeighted ? a.out_features / 128 : gm.nq;
  int cus = 0;
  const int occ_lds = device_cus_and_occupancy(B, &cus);
  int occ = occ_lds;
  // Short chunks amortise a workgroup's set-up and finish latency poorly: with fewer than
  // kMinChunkAt4 units each at four workgroups per CU, three per CU are used (measured on
  // the MoE token, whose launches give 6-12 units per workgroup: 65.5 against 70-73 us;
  // the dense MLP step, 16 units, is faster at four: 45.4 against 48.0 us).
  if (occ >= 4 && U < (long long)kMinChunkAt4 * cus * occ) occ = 3;
  long long G = (long long)cus * occ;
  // units per sub-range: the A-operand region holds kWaves * kMaxTasks (unit, row) rotations
  long long kA_max = kABudget / (512 * B);
  if (kA_max > (long long)kWaves * kMaxTasks / B) kA_max = (long long)kWaves * kMaxTasks / B;
  // Debug/test override of the workgroup count (it exercises chunks that span column blocks
  // and problems).
  bool forced = false;
  if (const char *env = getenv("TRELLIS_GEMV_WGS")) {
    const long long v = atoll(env);
    if (v > 0) {
      G = v;
      forced = true;
    }
  }
  // A chunk longer than kA_max units runs in several sub-ranges, each paying a rotation
  // and about a microsecond at its start.  When the CUs can hold the workgroups that chunks
  // of kA_max units need, use those (the small-batch step at B = 2, kA_max = 8: 880
  // workgroups of 8 units, 25.6 us, against 768 of 10 units, 27.8 us).
  if (!forced && (U + G - 1) / G > kA_max) {
    const long long Gk = (U + kA_max - 1) / kA_max;
    if (Gk <= (long long)cus * occ_lds) G = Gk;
  }
  if (G > U) G = U;
  if (G < 1) G = 1;
  // equal chunks, one per workgroup; none may be empty
  const long long CH = (U + G - 1) / G;
  G = (U + CH - 1) / CH;
  gm.CH = (int)CH;
  gm.G = (int)G;
  // a chunk of n units meets at most (n - 1) / nI_min + 2 column blocks
  const long long chmax = CH;
  const long long maxseg = (chmax - 1) / nI_min + 2;
  gm.maxseg = (int)(maxseg < nq ? maxseg : nq);
  gm.kA = (int)(chmax < kA_max ? chmax : kA_max);
  gm.partial_bytes = (size_t)gm.G * gm.maxseg * B * 128 * sizeof(float);
  if (gm.partial_bytes >= (1ULL << 31)) return gm;  // 32-bit buffer offsets
  gm.bytes = kWsReserved + gm.partial_bytes;
  gm.ok = true;
  return gm;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// The kernel launch of one problem list whose partials go to `partials` (the error word
// and the counters are the workspace's reserved region at `ws`).
hipError_t launch_list(const GemvLaunch &a, char *ws, float *partials, size_t partial_room, hipStream_t stream) {
  if (a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
  if (a.table && a.finish != kFinishPlain && a.B != 1) return hipErrorInvalidValue;
  if (!a.table && (a.n_list < 1 || a.n_list > kMaxList)) return hipErrorInvalidValue;
  const Geometry gm = geometry(a);
  if (!gm.ok || partial_room < gm.partial_bytes) return hipErrorInvalidValue;
  GemvParams P;
  P.L = a;
  if (P.L.group < 1) P.L.group = 1;
  P.errword = reinterpret_cast<uint32_t *>(ws);
  P.counters = reinterpret_cast<uint32_t *>(ws + kWsHeaderBytes);
  P.partials = partials;
  P.partial_bytes = (long long)gm.partial_bytes;
  P.U = gm.U;
  P.CH = gm.CH;
  P.G = gm.G;
  P.maxseg = gm.maxseg;
  P.kA = gm.kA;
  P.nI = a.table ? a.in_features / 128 : 0;
  P.nJ = a.table ? a.out_features / 128 : 0;
  for (int i = 0; i <= kMaxList; ++i) {
    P.ubase[i] = gm.ubase[i];
    P.qbase[i] = gm.qbase[i];
  }
  const size_t lds = lds_bytes(a.B, gm.kA);
  if (a.table) {
    gemv_kernel<false, 0, 0><<<gm.G, kThreads, lds, stream>>>(P);
    return hipGetLastError();
  }
  // list mode: a kernel specialised for one width when every layer shares it
  bool same = true, all_mcg = true;
  for (int p = 0; p < a.n_list; ++p) {
    same = same && a.list[p].L.K == a.list[0].L.K && a.list[p].L.cb == a.list[0].L.cb;
    all_mcg = all_mcg && a.list[p].L.cb == 1;
  }
  const int sel = same ? a.list[0].L.K + 4 * (a.list[0].L.cb - 1) : (all_mcg ? 1 : 0);
  switch (sel) {
    case 2: gemv_kernel<true, 2, 1><<<gm.G, kThreads, lds, stream>>>(P); break;
    case 3: gemv_kernel<true, 3, 1><<<gm.G, kThreads, lds, stream>>>(P); break;
    case 4: gemv_kernel<true, 4, 1><<<gm.G, kThreads, lds, stream>>>(P); break;
    case 6: gemv_kernel<true, 2, 2><<<gm.G, kThreads, lds, stream>>>(P); break;
    case 7: gemv_kernel<true, 3, 2><<<gm.G, kThreads, lds, stream>>>(P); break;
    case 8: gemv_kernel<true, 4, 2><<<gm.G, kThreads, lds, stream>>>(P); break;
    case 1: gemv_kernel<true, 0, 1><<<gm.G, kThreads, lds, stream>>>(P); break;
    default: gemv_kernel<true, 0, 0><<<gm.G, kThreads, lds, stream>>>(P); break;
  }
  return hipGetLastError();
}

}  // namespace

size_t gemv_workspace_bytes(const GemvLaunch &a) {
  const bool empty = a.table ? a.n_problems <= 0 : a.n_list <= 0;
  if (empty) return kWsReserved;
  const Geometry gm = geometry(a);
  return gm.ok ? gm.bytes : 0;
}

size_t gemv_workspace_bytes(int n_problems, int in_features, int out_features, int B) {
  GemvLaunch a{};
  a.table = reinterpret_cast<const trellis_linear *>(1);  // (only the mode matters here)
  a.n_problems = n_problems;
  a.in_features = in_features;
  a.out_features = out_features;
  a.B = B;
  return gemv_workspace_bytes(a);
}

// Scratch of the allocation-free entry point: a workspace (reserved region, then partials)
// in device memory that the library itself holds, one copy per device, zero at load and
// left with zero counters by every call.  In host code `scratch` is only a stand-in for the
// symbol: its device address is looked up once per device and kept in g_scratch_ptr.
__device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // (the current device's copy)
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_gemv(const GemvLaunch &a, void *ws, size_t ws_bytes, hipStream_t stream) {
  const bool empty = a.table ? a.n_problems <= 0 : a.n_list <= 0;
  if (empty) {
    if (!(a.table && a.finish == kFinishWeighted)) return hipSuccess;
    // an empty weighted sum: y = 0
    const int n = a.out_features;
    zero_fill_kernel<<<(n + 255) / 256, 256, 0, stream>>>(a.y, n);
    return hipGetLastError();
  }
  const size_t need = gemv_workspace_bytes(a);
  if (need == 0 || ws_bytes < need) return hipErrorInvalidValue;
  char *w = static_cast<char *>(ws);
  return launch_list(a, w, reinterpret_cast<float *>(w + kWsReserved), ws_bytes - kWsReserved, stream);
}

// Workspace of the routed MLP: [reserved region][activations fp16 [n][inter], 256-aligned]
// [partials: the larger of the two launches' regions].  The down launch reuses the gate/up
// partials region: it runs after the gate/up launch on the same stream.
namespace {
GemvLaunch mlp_gate_up(const MlpLaunch &m, uint16_t *act) {
  GemvLaunch gu{};
  gu.table = m.gate_up;
  gu.E = m.E;
  gu.group = 2 * m.halves;
  gu.routed = m.routed;
  gu.n_problems = m.n * 2 * m.halves;
  gu.in_features = m.hidden;
  gu.out_features = m.inter / m.halves;
  gu.B = 1;
  gu.x = m.x;
  gu.x_per_problem = 0;
  gu.y = act;
  gu.shared_r = m.r_hidden_in;
  gu.shared_s = m.s_hidden_in;
  gu.shared_side = 0;
  gu.finish = kFinishSwiGLU;
  gu.halves = m.halves;
  return gu;
}
GemvLaunch mlp_down(const MlpLaunch &m, const uint16_t *act) {
  GemvLaunch d{};
  d.table = m.down;
  d.E = m.E;
  d.group = 1;
  d.routed = m.routed;
  d.n_problems = m.n;
  d.in_features = m.inter;
  d.out_features = m.hidden;
  d.B = 1;
  d.x = act;
  d.x_per_problem = 1;
  d.y = m.y;
  d.shared_r = m.r_hidden_out;
  d.shared_s = m.s_hidden_out;
  d.shared_side = 1;
  d.finish = kFinishWeighted;
  d.router_w = m.router_w;
  return d;
}
}  // namespace

size_t moe_mlp_workspace_bytes(int hidden, int inter, int halves, int n) {
  if (n <= 0) return kWsReserved;
  MlpLaunch m{};
  m.hidden = hidden;
  m.inter = inter;
  m.halves = halves;
  m.n = n;
  m.gate_up = m.down = reinterpret_cast<const trellis_linear *>(1);  // (only the mode matters here)
  const size_t gu = gemv_workspace_bytes(mlp_gate_up(m, nullptr));
  const size_t d = gemv_workspace_bytes(mlp_down(m, nullptr));
  if (gu == 0 || d == 0) return 0;
  const size_t room = (gu > d ? gu : d) - kWsReserved;
  return kWsReserved + align256((size_t)n * inter * 2) + room;
}

hipError_t launch_moe_mlp(const MlpLaunch &m, void *ws, size_t ws_bytes, hipStream_t stream) {
  const size_t need = moe_mlp_workspace_bytes(m.hidden, m.inter, m.halves, m.n);
  if (need == 0 || ws_bytes < need) return hipErrorInvalidValue;
  char *w = static_cast<char *>(ws);
  const size_t act_bytes = m.n > 0 ? align256((size_t)m.n * m.inter * 2) : 0;
  uint16_t *act = m.act ? m.act : reinterpret_cast<uint16_t *>(w + kWsReserved);
  float *partials = reinterpret_cast<float *>(w + kWsReserved + act_bytes);
  const size_t room = ws_bytes - kWsReserved - act_bytes;
  if (m.n > 0) {
    const hipError_t e = launch_list(mlp_gate_up(m, act), w, partials, room, stream);
    if (e != hipSuccess) return e;
  }
  const GemvLaunch d = mlp_down(m, act);
  if (m.n <= 0) return launch_gemv(d, ws, ws_bytes, stream);
  return launch_list(d, w, partials, room, stream);
}

}  // namespace trellis
