// had128_scale: blockwise Sylvester Hadamard-128 fused with per-channel scales.
//
// ("Escha-W2 runs on Metal", reconstruction paragraph: xh = had_blockwise(x*su),
//  y = had_blockwise(y_pre)*sv; "The escha W2 format ...", "Reconstruction": H is the
//  normalised Sylvester Hadamard of size 128.)
//
// Pointers of any natural alignment: one wave per (row, 128-block), lane l holding elements
// l and l+64; the 64-stride stage is in-register and the strides 32..1 are cross-lane
// exchanges (wave_fwht128).  16-byte-aligned operands take the vectorised kernel below.
#include "launch.h"
#include "trellis_device.h"

namespace trellis {

template <bool XF32, bool YF32>
__global__ __launch_bounds__(256) void had128_kernel(const void *x, int rows, int n,
                                                     const uint16_t *__restrict__ r,
                                                     const float *__restrict__ s, int post,
                                                     float norm, void *y) {
  const int nb = n / 128;
  const long long task = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= (long long)rows * nb) return;
  const int row = (int)(task / nb), blk = (int)(task % nb);
  const int lane = threadIdx.x & 63;
  const size_t base = (size_t)row * n + (size_t)blk * 128;
  const int c0 = blk * 128 + lane, c1 = c0 + 64;
  float a, b;
  if (XF32) {
    a = ((const float *)x)[base + lane];
    b = ((const float *)x)[base + lane + 64];
  } else {
    a = h2f(((const uint16_t *)x)[base + lane]);
    b = h2f(((const uint16_t *)x)[base + lane + 64]);
  }
  float sa = 1.f, sb = 1.f;
  if (r) { sa = h2f(r[c0]); sb = h2f(r[c1]); }
  if (s) { sa *= s[c0]; sb *= s[c1]; }
  if (!post) { a *= sa; b *= sb; }
  wave_fwht128(a, b);
  a *= norm;
  b *= norm;
  if (post) { a *= sa; b *= sb; }
  if (YF32) {
    ((float *)y)[base + lane] = a;
    ((float *)y)[base + lane + 64] = b;
  } else {
    ((uint16_t *)y)[base + lane] = f2h(a);
    ((uint16_t *)y)[base + lane + 64] = f2h(b);
  }
}

// 16-byte-aligned operands: 16 lanes per (row, 128-block), lane i holding elements
// 8i .. 8i+7 (one 16-byte fp16 load, or two for fp32), so a wave covers four blocks with
// full-width accesses.  Strides 1, 2, 4 are in-register, strides 8 .. 64 cross the 16 lanes
// (the same butterfly as above with another assignment of the index bits).
template <bool XF32, bool YF32>
__global__ __launch_bounds__(256) void had128_vec_kernel(const void *x, int rows, int n,
                                                         const uint16_t *__restrict__ r,
                                                         const float *__restrict__ s, int post,
                                                         float norm, void *y) {
  const int nb = n / 128;
  const long long task = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (task >= (long long)rows * nb) return;  // (whole 16-lane groups leave together)
  const int row = (int)(task / nb), blk = (int)(task % nb);
  const int i = threadIdx.x & 15, lane = threadIdx.x & 63;
  const int c = blk * 128 + 8 * i;
  const size_t base = (size_t)row * n + c;
  float v[8];
  if (XF32) {
    const floatx4 p0 = *reinterpret_cast<const floatx4 *>((const float *)x + base);
    const floatx4 p1 = *reinterpret_cast<const floatx4 *>((const float *)x + base + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[t] = p0[t];
      v[t + 4] = p1[t];
    }
  } else {
    const u32x4 p = *reinterpret_cast<const u32x4 *>((const uint16_t *)x + base);
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = h2f((t & 1) ? (uint16_t)(p[t >> 1] >> 16) : (uint16_t)p[t >> 1]);
  }
  float sc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) sc[t] = 1.f;
  if (r) {
    const u32x4 rv = *reinterpret_cast<const u32x4 *>(r + c);
#pragma unroll
    for (int t = 0; t < 8; ++t) sc[t] = h2f((t & 1) ? (uint16_t)(rv[t >> 1] >> 16) : (uint16_t)rv[t >> 1]);
  }
  if (s) {
    const floatx4 s0 = *reinterpret_cast<const floatx4 *>(s + c);
    const floatx4 s1 = *reinterpret_cast<const floatx4 *>(s + c + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc[t] *= s0[t];
      sc[t + 4] *= s1[t];
    }
  }
  if (!post) {
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] *= sc[t];
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
  const float sg1 = (lane & 1) ? -1.f : 1.f, sg2 = (lane & 2) ? -1.f : 1.f;
  const float sg4 = (lane & 4) ? -1.f : 1.f, sg8 = (lane & 8) ? -1.f : 1.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = lane_xor<1>(v[t]) + sg1 * v[t];
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = lane_xor<2>(v[t]) + sg2 * v[t];
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = lane_xor<4>(v[t]) + sg4 * v[t];
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = lane_xor<8>(v[t]) + sg8 * v[t];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    v[t] *= norm;
    if (post) v[t] *= sc[t];
  }
  if (YF32) {
    *reinterpret_cast<floatx4 *>((float *)y + base) = floatx4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<floatx4 *>((float *)y + base + 4) = floatx4{v[4], v[5], v[6], v[7]};
  } else {
    u32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = (uint32_t)f2h(v[2 * t]) | ((uint32_t)f2h(v[2 * t + 1]) << 16);
    *reinterpret_cast<u32x4 *>((uint16_t *)y + base) = o;
  }
}

hipError_t launch_had128(const void *x, int x_is_fp32, int rows, int n, const uint16_t *r,
                         const float *s, int post, float norm, void *y, int y_is_fp32,
                         hipStream_t stream) {
  const long long tasks = (long long)rows * (n / 128);
  if (tasks == 0) return hipSuccess;
  auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (a16(x) && a16(y) && a16(r) && a16(s)) {
    const unsigned g = (unsigned)((tasks + 15) / 16);
    if (x_is_fp32 && y_is_fp32) had128_vec_kernel<true, true><<<g, 256, 0, stream>>>(x, rows, n, r, s, post, norm, y);
    else if (x_is_fp32) had128_vec_kernel<true, false><<<g, 256, 0, stream>>>(x, rows, n, r, s, post, norm, y);
    else if (y_is_fp32) had128_vec_kernel<false, true><<<g, 256, 0, stream>>>(x, rows, n, r, s, post, norm, y);
    else had128_vec_kernel<false, false><<<g, 256, 0, stream>>>(x, rows, n, r, s, post, norm, y);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((tasks + 3) / 4);
  if (x_is_fp32 && y_is_fp32)
    had128_kernel<true, true><<<grid, 256, 0, stream>>>(x, rows, n, r, s, post, norm, y);
  else if (x_is_fp32)
    had128_kernel<true, false><<<grid, 256, 0, stream>>>(x, rows, n, r, s, post, norm, y);
  else if (y_is_fp32)
    had128_kernel<false, true><<<grid, 256, 0, stream>>>(x, rows, n, r, s, post, norm, y);
  else
    had128_kernel<false, false><<<grid, 256, 0, stream>>>(x, rows, n, r, s, post, norm, y);
  return hipGetLastError();
}

}  // namespace trellis
