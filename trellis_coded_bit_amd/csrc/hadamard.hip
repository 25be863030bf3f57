// had128_scale: blockwise Sylvester Hadamard-128 fused with per-channel scales.
//
// ("Escha-W2 runs on Metal", reconstruction paragraph: xh = had_blockwise(x*su),
//  y = had_blockwise(y_pre)*sv; "The escha W2 format ...", "Reconstruction": H is the
//  normalised Sylvester Hadamard of size 128.)
//
// One wave per (row, 128-block): lane l holds elements l and l+64, the 64-stride stage is
// in-register and the strides 32..1 are cross-lane exchanges (wave_fwht128).
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

hipError_t launch_had128(const void *x, int x_is_fp32, int rows, int n, const uint16_t *r,
                         const float *s, int post, float norm, void *y, int y_is_fp32,
                         hipStream_t stream) {
  const long long tasks = (long long)rows * (n / 128);
  if (tasks == 0) return hipSuccess;
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
