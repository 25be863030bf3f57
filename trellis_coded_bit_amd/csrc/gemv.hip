// trellis_gemv / trellis_moe_gemv: fused small-batch products against trellis-coded weights.
//
// y = had(had(x*su) @ W_hat) * sv  ("Escha-W2 runs on Metal", reconstruction paragraph),
// for B = 1..8 rows, over a list of problems (one layer, or the routed entries of an expert
// pointer table -- "EXLR8" page: per-expert widths, a pointer table re-read every launch,
// one hidden-side rotation shared by all experts).
//
// Two launches.
//
// 1. gemv_partial_kernel (stream-K over "units").  A unit is one 128-row input block I
//    times one 128-column output block J of one problem p, i.e. 8x8 tiles; units are
//    numbered u = (p*nJ + J)*nI + I and the G workgroups take equal contiguous ranges of u,
//    so every workgroup streams the same number of code bytes whatever the matrix shape.
//    Each workgroup writes one fp32 partial sum y_pre[B][128] per column block it touches
//    (its "segment") into the workspace.  Inside a workgroup (4 waves) every wave takes
//    two of the unit's eight tile rows:
//      * loads: the wave's 2 x 8 tiles are 2 x 256K contiguous bytes, copied straight
//        from global memory into a wave-private LDS ring (global_load_lds, 16 B per lane,
//        fully coalesced) several units ahead of use; a lane's circular window is read as
//        two LDS words of its tile;
//      * balance: the workgroups resident on one CU set their issue priority from the
//        share of their range still to do, so they finish together;
//      * input rotation: per sub-range the workgroup butterflies x*su (unnormalised) and
//        stores fp16 MFMA A-operands in LDS, each value twice (below);
//      * contraction: per tile each lane decodes its four symbols (trellis_device.h) to
//        four MCG hash words and feeds them UNSUMMED to v_mfma_f32_16x16x32_f16 as eight
//        fp16 B-elements along k.  The A operand repeats each activation for the lo and hi
//        halves, so the matrix core forms x*lo + x*hi in fp32 and the codebook's lo+hi
//        addition costs no VALU work.  One MFMA covers one tile; batch rows ride in the
//        16 M rows (rows past B read a duplicate activation and are ignored).  This fp32
//        sum of the halves is the exact value before the format's fp16 rounding; it
//        differs from the rounded codebook value by at most half an fp16 ulp.
// 2. gemv_finish_kernel: one workgroup per column block adds its partials in workgroup
//    order (deterministic), applies the output Hadamard, the scales and the exact 1/128
//    that replaces the two 1/sqrt(128) factors, and writes fp16 y.
#include <cstdlib>
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

struct GemvParams {
  GemvLaunch L;
  uint32_t *errword;
  float *partials;
  int U;   // total units
  int G;   // workgroups of the partial kernel
  int nI, nJ, maxseg;
  int kA;  // units per sub-range (A-operand capacity)
};

// Dynamic LDS layout for batch B.
struct Lds {
  uint32_t *a;      // [kA][8 tile rows][4 groups][B][4 words]
  uint32_t *tiles;  // [kWaves][kRingBytes / 4]: each wave's code ring
  float *red;       // [kWaves][B][128]
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

struct Problem {
  const uint32_t *code;
  const uint16_t *rin, *rout;
  const float *s_in, *s_out;
  int K;
  int cb;  // 1: MCG fp16 values; 2: the same rounded to E4M3
  bool ok;
};

// TABLE = false: the launch is known to be a single layer (no table lookups at all).
template <bool TABLE = true>
__device__ __forceinline__ Problem get_problem(const GemvParams &P, int p) {
  trellis_linear d = P.L.single;
  bool ok = true;
  if (TABLE && P.L.table) {
    const int grp = P.L.group;
    const int slot = grp == 1 ? p : p / grp;
    const int e = P.L.routed[slot];
    if (e < 0 || e >= P.L.E) ok = false;
    else d = P.L.table[e * grp + (p - slot * grp)];
  }
  Problem r;
  r.code = reinterpret_cast<const uint32_t *>(d.code);
  r.K = d.K;
  r.cb = d.cb;
  r.rin = d.rin;
  r.s_in = d.s_in;
  r.rout = d.rout;
  r.s_out = d.s_out;
  if (P.L.shared_side == 0) { r.rin = P.L.shared_r; r.s_in = P.L.shared_s; }
  if (P.L.shared_side == 1) { r.rout = P.L.shared_r; r.s_out = P.L.shared_s; }
  if (ok) {
    ok = d.K >= 2 && d.K <= 4 && (d.cb == 1 || d.cb == 2) && d.code != nullptr && r.rin != nullptr &&
         r.rout != nullptr && d.in_features == P.L.in_features &&
         d.out_features == P.L.out_features;
  }
  r.ok = ok;
  return r;
}

// First unit of workgroup g, and the workgroup owning unit u (largest g with start(g) <= u).
// 32-bit arithmetic: the launch checks G * U < 2^32.
__host__ __device__ __forceinline__ int wg_start(int g, int U, int G) {
  return (int)(((unsigned)g * (unsigned)U) / (unsigned)G);
}
__host__ __device__ __forceinline__ int owner(int u, int U, int G) {
  return (int)(((unsigned)(u + 1) * (unsigned)G - 1u) / (unsigned)U);
}

// Orders this wave's LDS accesses (all lanes of one wave run in lockstep and the LDS
// executes one wave's operations in order; this only stops the compiler from moving them).
__device__ __forceinline__ void wave_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wave issue priority (s_setprio takes an immediate).
__device__ __forceinline__ void set_priority(int prio) {
  if (prio >= 3) __builtin_amdgcn_s_setprio(3);
  else if (prio == 2) __builtin_amdgcn_s_setprio(2);
  else if (prio == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
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
  const int lane = threadIdx.x & 63;
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
        const uint32_t hv = f2h(h ? vb : va);
        sm.a[((((s * 8 + ti) * 4 + g) * B + b) << 2) + w] = hv | (hv << 16);
      }
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

// End of a segment (the workgroup's share of column block q): reduce the waves'
// accumulators and store the partial (not waited for: code copies in flight keep streaming).
__device__ __forceinline__ void publish_partial(const GemvParams &P, const Lds &sm, int q, floatx4 (&acc)[8]) {
  const int B = P.L.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int g = blockIdx.x;
  const int seg = q - wg_start(g, P.U, P.G) / P.nI;
  float *part = P.partials + ((size_t)g * P.maxseg + seg) * kMaxB * 128;
  for (int idx = tid; idx < B * 128; idx += kThreads) {
    float v = sm.red[idx];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += sm.red[w * B * 128 + idx];
    part[idx] = v;
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

// Copy the wave's two tile rows of the unit whose rows start at `row0` (global words) into
// ring slot `dst` (LDS).  `real` = false: every lane reads the first 16 bytes of `row0`.
template <int K>
__device__ __forceinline__ void dma_unit(const uint32_t *row0, size_t row_stride_words, uint32_t *dst, bool real) {
  const int lane = threadIdx.x & 63;
  if constexpr (K == 2) {
    // 2 x 512 B: lanes 0..31 take row 0, lanes 32..63 row 1, 16 B each
    const uint32_t *src = row0 + (real ? ((size_t)(lane >> 5) * row_stride_words + 4 * (lane & 31)) : 0);
    __builtin_amdgcn_global_load_lds((const void *)src, (lds_void_ptr)dst, 16, 0, 0);
  } else if constexpr (K == 3) {
    // 2 x 768 B = 96 pieces of 16 B: lanes 0..63 take pieces 0..63, then lanes 0..31 take
    // pieces 64..95 (a piece never straddles the two rows: 768 is a multiple of 16)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int piece = 64 * c + lane;
      const int r = piece / 48, w = 4 * (piece - 48 * r);
      const uint32_t *src = row0 + (real ? ((size_t)r * row_stride_words + w) : 0);
      if (c == 0 || lane < 32)
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void_ptr)(dst + c * 256), 16, 0, 0);
    }
  } else {
    // 2 x 1024 B: one copy per row, 16 B per lane
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t *src = row0 + (real ? ((size_t)r * row_stride_words + 4 * lane) : 0);
      __builtin_amdgcn_global_load_lds((const void *)src, (lds_void_ptr)(dst + r * 256), 16, 0, 0);
    }
  }
}

// Units [ub, ue) of problem p (width K), in sub-ranges of at most P.kA units.  Each
// sub-range issues its rotation loads and its first code copies, rotates while the code is
// in flight, then streams with SLOTS - 1 units in flight per wave.
// CB = 2 (the E4M3 codebook, "EXLR8" page): each lane's four values are the E4M3-rounded
// codebook values, converted back to fp16 (exact) and fed to v_mfma_f32_16x16x16_f16 with
// the A operand's duplicated words repacked once per tile row into (x0, x1), (x8, x9).
template <int K, int CB = 1>
__device__ void run_problem(const GemvParams &P, const Lds &sm, const Problem &pr, int p, int ub, int ue,
                            bool fresh) {
  using RG = Ring<K>;
  constexpr int NW = RG::NW;
  constexpr int SLOTS = RG::SLOTS;
  const int B = P.L.B;
  const int Tj = P.L.out_features / 16;
  const int nI = P.nI;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, grp = lane >> 4;
  const LaneWindow lw = lane_window(lane, K);
  uint32_t *ring = sm.tiles + wave * (kRingBytes / 4);
  const int mc = m < B ? m : B - 1;  // batch row of the A operand (rows past B are ignored)
  const uint32_t a_lane = (uint32_t)((grp * B + mc) << 2);
  const size_t row_stride = (size_t)Tj * NW;
  const uint32_t *code = pr.code + (size_t)(2 * wave) * row_stride;
  const size_t row_block_words = 8 * row_stride;
  const int first = __builtin_amdgcn_readfirstlane(ub - p * P.nI * P.nJ);
  const int total = __builtin_amdgcn_readfirstlane(ue - ub);
  const int in = P.L.in_features;
  const uint16_t *xp = P.L.x + (P.L.x_per_problem ? (size_t)p * B * in : (size_t)0);

  // The workgroup's first copy goes out before the rest of the set-up (priority
  // thresholds, sub-range bookkeeping, lane constants): its address needs only the first
  // unit's (I, J).
  if (fresh) {
    const int I0 = __builtin_amdgcn_readfirstlane(first % nI), J0 = __builtin_amdgcn_readfirstlane(first / nI);
    dma_unit<K>(code + (size_t)I0 * row_block_words + (size_t)(8 * J0) * NW, row_stride, ring, true);
    __builtin_amdgcn_sched_barrier(0);
  }
  floatx4 acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Issue priority from the share of the workgroup's range still to do, in quarters (3 =
  // more than three quarters left).  The waves of a CU otherwise issue oldest-first, so the
  // workgroups resident on a CU would finish one after another and the last would run with
  // few waves at the end; with this rule the ones behind catch up and they finish together.
  // Priority p applies from unit t[p] = u1 - floor((p + 1) * units / 4) on.
  const int wg_u1 = __builtin_amdgcn_readfirstlane(wg_start(blockIdx.x + 1, P.U, P.G));
  const int wg_units = __builtin_amdgcn_readfirstlane(wg_u1 - wg_start(blockIdx.x, P.U, P.G));
  const int t2 = wg_u1 - (3 * wg_units) / 4, t1 = wg_u1 - (2 * wg_units) / 4, t0 = wg_u1 - wg_units / 4;
  auto prio_at = [&](int c) { return c >= t0 ? 0 : c >= t1 ? 1 : c >= t2 ? 2 : 3; };

  for (int sb = 0; sb < total; sb += P.kA) {
    const int n = __builtin_amdgcn_readfirstlane(min(P.kA, total - sb));
    int cur_I = __builtin_amdgcn_readfirstlane((first + sb) % nI);
    int cur_J = __builtin_amdgcn_readfirstlane((first + sb) / nI);
    int pre_I = cur_I;
    // next unit to request: its rows start at nxt (uniform); one step along I adds a row
    // block, the wrap to the next column block moves 8 tiles right and back to I = 0
    const uint32_t *nxt = code + (size_t)pre_I * row_block_words + (size_t)(8 * cur_J) * NW;
    const size_t wrap_back = (size_t)(nI - 1) * row_block_words;
    auto advance = [&]() {
      if (++pre_I == nI) {
        pre_I = 0;
        nxt = nxt - wrap_back + 8 * NW;
      } else {
        nxt += row_block_words;
      }
    };
    // the previous sub-range's reads of the A buffer and of the ring are finished (nothing
    // to wait for on the workgroup's first sub-range)
    if (!(fresh && sb == 0)) __syncthreads();
    // The first unit into slot 0, then the rotation's loads; units 1..SLOTS-2 are requested
    // after the rotation.  At the start of the kernel every wave requests code at once: asking for
    // one unit each first lets the memory system serve everybody's first unit before the
    // deeper prefetches, so the decode starts sooner.
    auto prime = [&](int j) {
      const bool real = j < n;
      dma_unit<K>(real ? nxt : code, row_stride, ring + j * (RG::UNIT_BYTES / 4), real);
      if (real) advance();
    };
    if (fresh && sb == 0) advance();  // (its copy was issued above)
    else prime(0);
    if (sb == 0) set_priority(prio_at(ub));  // (after the first copy is on its way)
    // Rotation loads: straight-line code (tasks past the last are clamped to it and their
    // values ignored), so all of them are in flight together.
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
    rotation_compute(B, n, wave, rq, sm);
    __syncthreads();  // (also waits for unit 0)
#pragma unroll
    for (int j = 1; j < SLOTS - 1; ++j) prime(j);

    int slot = 0;
    for (int k = 0; k < n; ++k) {
      // copy unit k + SLOTS - 1 into the slot unit k - 1 used (its reads are complete)
      {
        const int ws = (slot == 0 ? SLOTS : slot) - 1;
        const bool real = k + SLOTS - 1 < n;
        dma_unit<K>(real ? nxt : code, row_stride, ring + ws * (RG::UNIT_BYTES / 4), real);
        if (real) advance();
      }
      wait_vmcnt<RG::WAIT>();  // unit k has landed
      {
        const int c = ub + sb + k;
        if (c == t2 || c == t1 || c == t0) set_priority(prio_at(c));
      }
      const uint32_t *ub_ = ring + slot * (RG::UNIT_BYTES / 4);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(sm.a + (uint32_t)(((k * 8 + 2 * wave + r) * 4 * B) << 2) + a_lane);
        const half8 av = __builtin_bit_cast(half8, a);
        const u32x2 a2 = {__builtin_amdgcn_perm(a[1], a[0], 0x05040100u), __builtin_amdgcn_perm(a[3], a[2], 0x05040100u)};
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const uint32_t *tw = ub_ + (r * 8 + tt) * NW;
          const uint32_t bits = lane_bits(tw[lw.d0], tw[lw.d1], lw.sh);
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
      if (cur_I == nI - 1 || sb + k == total - 1) publish_partial(P, sm, p * P.nJ + cur_J, acc);
      if (++cur_I == nI) { cur_I = 0; ++cur_J; }
      slot = (slot + 1 == SLOTS) ? 0 : slot + 1;
    }
    wait_vmcnt<0>();  // the dummy copies of the tail have landed before the ring is reused
  }
}

// Units of invalid problems: no loads; each segment publishes a zero partial (the finishing
// kernel writes zeros for invalid problems anyway) and the error word is set.
__device__ void run_invalid(const GemvParams &P, const Lds &sm, int ub, int ue) {
  if (threadIdx.x == 0) __hip_atomic_fetch_or(P.errword, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  floatx4 acc[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int u = ub; u < ue; ++u) {
    const int q = u / P.nI, I = u - q * P.nI;
    if (I == P.nI - 1 || u == ue - 1) publish_partial(P, sm, q, acc);
  }
}

// KS = 2, 3, 4: one layer of that width (no table, the K dispatch compiled away, a smaller
// kernel); KS = 0: a list of problems with per-entry K.
template <int KS, int CBS = 1>
__global__ __launch_bounds__(kThreads, 4) void gemv_partial_kernel(GemvParams P) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const Lds sm = lds_carve(lds_raw, P.L.B, P.kA);
  // Top issue priority from the start: a workgroup dispatched after its CU's others are
  // already decoding would otherwise run its prologue at the lowest priority, behind them.
  __builtin_amdgcn_s_setprio(3);
  // The arguments needed before the first code copy, read in one round trip (left alone,
  // the compiler loads them in several dependent rounds around the early branches).
  asm volatile("" ::"s"(P.U), "s"(P.G), "s"(P.nI), "s"(P.nJ), "s"(P.kA), "s"(P.L.B), "s"(P.L.in_features),
               "s"(P.L.out_features), "s"(P.L.single.code), "s"(P.L.single.rin), "s"(P.L.single.s_in),
               "s"(P.L.x), "s"(P.L.shared_side), "s"(P.L.shared_r), "s"(P.L.shared_s), "s"(P.partials), "s"(P.L.table), "s"(P.L.E),
               "s"(P.L.routed));
  const int g = blockIdx.x;
  const int u0 = wg_start(g, P.U, P.G), u1 = wg_start(g + 1, P.U, P.G);
  if constexpr (KS != 0) {
    if (u0 < u1) run_problem<KS, CBS>(P, sm, get_problem<false>(P, 0), 0, u0, u1, true);
    return;
  }
  const int per_problem = P.nI * P.nJ;
  for (int u = u0; u < u1;) {
    const int p = u / per_problem;
    const int ue = min(u1, (p + 1) * per_problem);
    const Problem pr = get_problem(P, p);
    const bool fresh = u == u0;
    switch (pr.ok ? pr.K + 4 * (pr.cb - 1) : 0) {
      case 2: run_problem<2>(P, sm, pr, p, u, ue, fresh); break;
      case 3: run_problem<3>(P, sm, pr, p, u, ue, fresh); break;
      case 4: run_problem<4>(P, sm, pr, p, u, ue, fresh); break;
      case 6: run_problem<2, 2>(P, sm, pr, p, u, ue, fresh); break;
      case 7: run_problem<3, 2>(P, sm, pr, p, u, ue, fresh); break;
      case 8: run_problem<4, 2>(P, sm, pr, p, u, ue, fresh); break;
      default: run_invalid(P, sm, u, ue); break;
    }
    u = ue;
  }
}

// One workgroup per column block q: sum the contributors' partials in workgroup order,
// rotate, scale and write fp16 y.
constexpr int kPartialBatch = 32;  // partial loads a thread issues together

__global__ __launch_bounds__(kThreads) void gemv_finish_kernel(GemvParams P) {
  __shared__ float fin[kMaxB][128];
  // all arguments in one early round trip
  asm volatile("" ::"s"(P.U), "s"(P.G), "s"(P.nI), "s"(P.nJ), "s"(P.maxseg), "s"(P.partials), "s"(P.L.B),
               "s"(P.L.out_features), "s"(P.L.y), "s"(P.L.table), "s"(P.L.E), "s"(P.L.routed),
               "s"(P.L.single.rout), "s"(P.L.single.s_out), "s"(P.L.shared_side), "s"(P.L.shared_r),
               "s"(P.L.shared_s));
  const int B = P.L.B, out = P.L.out_features;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = blockIdx.x;
  // Contributors g_lo..g_hi.  Every contributor after the first starts its range inside
  // block q, so q is its first segment; only g_lo can reach q at a later segment.  The
  // partial loads therefore need no table and no barrier: they are issued first.
  const int g_lo = owner(q * P.nI, P.U, P.G), g_hi = owner((q + 1) * P.nI - 1, P.U, P.G);
  const int seg_lo = q - wg_start(g_lo, P.U, P.G) / P.nI;
  float v[kMaxB * 128 / kThreads];
#pragma unroll
  for (int i = 0; i < kMaxB * 128 / kThreads; ++i) v[i] = 0.f;
  for (int gb = g_lo; gb <= g_hi; gb += kPartialBatch) {
#pragma unroll
    for (int i = 0; i < kMaxB * 128 / kThreads; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < B * 128) {
        float part[kPartialBatch];
#pragma unroll
        for (int t = 0; t < kPartialBatch; ++t) {
          const int gg = gb + t;
          const size_t sl = (size_t)gg * P.maxseg + (gg == g_lo ? seg_lo : 0);
          part[t] = gg <= g_hi ? P.partials[sl * kMaxB * 128 + idx] : 0.f;
        }
#pragma unroll
        for (int t = 0; t < kPartialBatch; ++t) v[i] += part[t];
      }
    }
  }
  // the output-side vectors (their loads overlap the partials')
  const int p = q / P.nJ, J = q - p * P.nJ;
  const Problem pr = get_problem(P, p);
  const int c0 = J * 128 + lane, c1 = c0 + 64;
  float sa = 0.f, sb = 0.f;
  if (pr.ok) {
    sa = h2f(ldg(pr.rout + c0)) * (1.0f / 128.0f);
    sb = h2f(ldg(pr.rout + c1)) * (1.0f / 128.0f);
    if (pr.s_out) { sa *= ldg(pr.s_out + c0); sb *= ldg(pr.s_out + c1); }
  }
#pragma unroll
  for (int i = 0; i < kMaxB * 128 / kThreads; ++i) {
    const int idx = tid + i * kThreads;
    if (idx < B * 128) fin[idx >> 7][idx & 127] = v[i];
  }
  __syncthreads();
  uint16_t *y = P.L.y + (size_t)p * B * out;
  for (int b = wave; b < B; b += kWaves) {
    float va = fin[b][lane], vb = fin[b][lane + 64];
    if (pr.ok) {
      wave_fwht128(va, vb);
      va *= sa;
      vb *= sb;
    } else {
      va = 0.f;
      vb = 0.f;
    }
    y[(size_t)b * out + c0] = f2h(va);
    y[(size_t)b * out + c1] = f2h(vb);
  }
}

// Batch row 0 of column block q, column c: the contributors' partials added in workgroup
// order (the order gemv_finish_kernel uses).
__device__ __forceinline__ float partial_sum_b1(const GemvParams &P, int q, int c) {
  const int g_lo = owner(q * P.nI, P.U, P.G), g_hi = owner((q + 1) * P.nI - 1, P.U, P.G);
  const int seg_lo = q - wg_start(g_lo, P.U, P.G) / P.nI;
  float v = 0.f;
  for (int gb = g_lo; gb <= g_hi; gb += kPartialBatch) {
    float part[kPartialBatch];
#pragma unroll
    for (int t = 0; t < kPartialBatch; ++t) {
      const int gg = gb + t;
      const size_t sl = (size_t)gg * P.maxseg + (gg == g_lo ? seg_lo : 0);
      part[t] = gg <= g_hi ? P.partials[sl * kMaxB * 128 + c] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < kPartialBatch; ++t) v += part[t];
  }
  return v;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z) ("EXLR8" page, calibration paragraph: the
// expert's down projection reads silu(gate x) * up x).  For z below about -88 e^-z is
// +inf in fp32 and the quotient is -0, the limit.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// kFinishSwiGLU, B = 1.  Workgroup f handles output block J of slice h of routed slot k
// (f = (k*H + h)*nJ + J): threads 0..127 sum the gate entry's partials, threads 128..255
// the up entry's; waves 0 and 2 rotate and scale them; then a = silu(g) * u is written as
// fp16 to y[k][(h*nJ + J)*128 + c].
__global__ __launch_bounds__(kThreads) void gemv_finish_swiglu_kernel(GemvParams P) {
  __shared__ float gu[2][128];
  const int H = P.L.halves, nJ = P.nJ;
  const int f = blockIdx.x;
  const int slot = f / (H * nJ), rem = f - slot * H * nJ;
  const int pg = slot * 2 * H + rem / nJ, J = rem - (rem / nJ) * nJ;
  const int tid = threadIdx.x, c = tid & 127, which = tid >> 7, lane = tid & 63;
  const int p = which ? pg + H : pg;
  const float v = partial_sum_b1(P, p * nJ + J, c);
  const bool rot = (tid & 127) < 64;  // waves 0 (gate) and 2 (up)
  float sa = 0.f, sb = 0.f;
  if (rot) {
    const Problem pr = get_problem(P, p);
    if (pr.ok) {
      const int c0 = J * 128 + lane, c1 = c0 + 64;
      sa = h2f(ldg(pr.rout + c0)) * (1.0f / 128.0f);
      sb = h2f(ldg(pr.rout + c1)) * (1.0f / 128.0f);
      if (pr.s_out) { sa *= ldg(pr.s_out + c0); sb *= ldg(pr.s_out + c1); }
    }
  }
  gu[which][c] = v;
  __syncthreads();
  if (rot) {
    float va = gu[which][lane], vb = gu[which][lane + 64];
    wave_fwht128(va, vb);
    gu[which][lane] = va * sa;  // (an invalid entry has sa = sb = 0: its output is zero)
    gu[which][lane + 64] = vb * sb;
  }
  __syncthreads();
  if (tid < 128) {
    const int inter = H * nJ * 128;
    P.L.y[(size_t)slot * inter + rem * 128 + c] = f2h(silu(gu[0][c]) * gu[1][c]);
  }
}

// kFinishWeighted, B = 1.  Workgroup J: thread (r, c) (r = tid / 128, 8 of them) adds
// w[k] * (sum of problem k's partials of block J) over k = r, r + 8, ..., in that order;
// the eight sums are then added in r order, rotated once and scaled by the shared sv.
constexpr int kWeightedThreads = 1024;
__global__ __launch_bounds__(kWeightedThreads) void gemv_finish_weighted_kernel(GemvParams P) {
  __shared__ float red[kWeightedThreads / 128][128];
  const int tid = threadIdx.x, c = tid & 127, r = tid >> 7, lane = tid & 63;
  const int J = blockIdx.x, nJ = P.nJ, n = P.L.n_problems;
  float acc = 0.f;
  for (int k = r; k < n; k += kWeightedThreads / 128) acc += ldg(P.L.router_w + k) * partial_sum_b1(P, k * nJ + J, c);
  red[r][c] = acc;
  __syncthreads();
  if (tid < 64) {
    float va = 0.f, vb = 0.f;
#pragma unroll
    for (int i = 0; i < kWeightedThreads / 128; ++i) {
      va += red[i][lane];
      vb += red[i][lane + 64];
    }
    const int c0 = J * 128 + lane, c1 = c0 + 64;
    float sa = h2f(ldg(P.L.shared_r + c0)) * (1.0f / 128.0f);
    float sb = h2f(ldg(P.L.shared_r + c1)) * (1.0f / 128.0f);
    if (P.L.shared_s) { sa *= ldg(P.L.shared_s + c0); sb *= ldg(P.L.shared_s + c1); }
    wave_fwht128(va, vb);
    P.L.y[c0] = f2h(va * sa);
    P.L.y[c1] = f2h(vb * sb);
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemv_partial_kernel<0>, kThreads,
                                                     lds_bytes(B, kWaves * kMaxTasks / B)) != hipSuccess ||
        occ <= 0)
      occ = 2;
    d.occ[B] = occ;
  }
  *cus_out = d.cus;
  return d.occ[B];
}

struct Geometry {
  int U, G, nI, nJ, maxseg, nq, kA;
  size_t partials_off, bytes;
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
  long long kA_max = kABudget / (512 * B);
  if (kA_max > (long long)kWaves * kMaxTasks / B) kA_max = (long long)kWaves * kMaxTasks / B;
  gm.kA = (int)(per < kA_max ? per : kA_max);
  gm.partials_off = 256;
  gm.bytes = gm.partials_off + (size_t)gm.G * gm.maxseg * kMaxB * 128 * sizeof(float);
  return gm;
}

}  // namespace

int gemv_max_column_blocks() { return 1 << 30; }

size_t gemv_workspace_bytes(int n_problems, int in_features, int out_features, int B) {
  if (n_problems <= 0) return 256;
  if (B < 1) B = 1;
  if (B > kMaxB) B = kMaxB;
  return geometry(n_problems, in_features, out_features, B).bytes;
}

namespace {

// The partial and finishing launches of one problem list, with the error word and the
// partials region given separately (the routed MLP places two lists in one workspace).
hipError_t launch_gemv_parts(const GemvLaunch &a, uint32_t *errword, float *partials, size_t partial_bytes,
                             hipStream_t stream) {
  if (a.B < 1 || a.B > kMaxB) return hipErrorInvalidValue;
  if (a.finish != kFinishPlain && a.B != 1) return hipErrorInvalidValue;
  if (a.n_problems <= 0) {
    if (a.finish != kFinishWeighted) return hipSuccess;
    // an empty weighted sum: y = 0 (the finishing kernel reads no partials)
    GemvParams P{};
    P.L = a;
    P.L.n_problems = 0;
    P.nJ = a.out_features / 128;
    gemv_finish_weighted_kernel<<<P.nJ, kWeightedThreads, 0, stream>>>(P);
    return hipGetLastError();
  }
  const long long units = (long long)a.n_problems * (a.out_features / 128) * (a.in_features / 128);
  if (units >= (1LL << 31)) return hipErrorInvalidValue;
  const Geometry gm = geometry(a.n_problems, a.in_features, a.out_features, a.B);
  if (partial_bytes < gm.bytes - gm.partials_off) return hipErrorInvalidValue;
  if ((long long)gm.G * gm.U >= (1LL << 32)) return hipErrorInvalidValue;  // 32-bit slot arithmetic
  GemvParams P;
  P.L = a;
  if (P.L.group < 1) P.L.group = 1;
  P.errword = errword;
  P.partials = partials;
  P.U = gm.U;
  P.G = gm.G;
  P.nI = gm.nI;
  P.nJ = gm.nJ;
  P.maxseg = gm.maxseg;
  P.kA = gm.kA;
  const size_t lds = lds_bytes(a.B, gm.kA);
  const int single = a.table == nullptr ? a.single.K + 4 * (a.single.cb - 1) : 0;
  if (single == 2) gemv_partial_kernel<2><<<gm.G, kThreads, lds, stream>>>(P);
  else if (single == 3) gemv_partial_kernel<3><<<gm.G, kThreads, lds, stream>>>(P);
  else if (single == 4) gemv_partial_kernel<4><<<gm.G, kThreads, lds, stream>>>(P);
  else if (single == 6) gemv_partial_kernel<2, 2><<<gm.G, kThreads, lds, stream>>>(P);
  else if (single == 7) gemv_partial_kernel<3, 2><<<gm.G, kThreads, lds, stream>>>(P);
  else if (single == 8) gemv_partial_kernel<4, 2><<<gm.G, kThreads, lds, stream>>>(P);
  else gemv_partial_kernel<0><<<gm.G, kThreads, lds, stream>>>(P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.finish == kFinishSwiGLU) gemv_finish_swiglu_kernel<<<gm.nq / 2, kThreads, 0, stream>>>(P);
  else if (a.finish == kFinishWeighted) gemv_finish_weighted_kernel<<<gm.nJ, kWeightedThreads, 0, stream>>>(P);
  else gemv_finish_kernel<<<gm.nq, kThreads, 0, stream>>>(P);
  return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

hipError_t launch_gemv(const GemvLaunch &a, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (a.n_problems <= 0 && a.finish != kFinishWeighted) return hipSuccess;
  const size_t need = gemv_workspace_bytes(a.n_problems, a.in_features, a.out_features, a.B);
  if (ws_bytes < need) return hipErrorInvalidValue;
  char *w = static_cast<char *>(ws);
  return launch_gemv_parts(a, reinterpret_cast<uint32_t *>(w), reinterpret_cast<float *>(w + 256), ws_bytes - 256,
                           stream);
}

// Workspace of the routed MLP: [error word: 256 B][activations fp16 [n][inter], 256-aligned]
// [partials: the larger of the two launches' regions].  The down launch reuses the gate/up
// partials region: it runs after the gate/up finishing kernel on the same stream.
size_t moe_mlp_workspace_bytes(int hidden, int inter, int halves, int n) {
  if (n <= 0) return 256;
  const size_t gu = gemv_workspace_bytes(n * 2 * halves, hidden, inter / halves, 1) - 256;
  const size_t d = gemv_workspace_bytes(n, inter, hidden, 1) - 256;
  return 256 + align256((size_t)n * inter * 2) + (gu > d ? gu : d);
}

hipError_t launch_moe_mlp(const MlpLaunch &m, void *ws, size_t ws_bytes, hipStream_t stream) {
  const size_t need = moe_mlp_workspace_bytes(m.hidden, m.inter, m.halves, m.n);
  if (ws_bytes < need) return hipErrorInvalidValue;
  char *w = static_cast<char *>(ws);
  uint32_t *errword = reinterpret_cast<uint32_t *>(w);
  const size_t act_bytes = m.n > 0 ? align256((size_t)m.n * m.inter * 2) : 0;
  uint16_t *act = m.act ? m.act : reinterpret_cast<uint16_t *>(w + 256);
  float *partials = reinterpret_cast<float *>(w + 256 + act_bytes);
  const size_t partial_bytes = ws_bytes - 256 - act_bytes;

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
  if (m.n > 0) {
    const hipError_t e = launch_gemv_parts(gu, errword, partials, partial_bytes, stream);
    if (e != hipSuccess) return e;
  }
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
  return launch_gemv_parts(d, errword, partials, partial_bytes, stream);
}

}  // namespace trellis
