// Per-row work on either side of the projections: the RMSNorm factor of a row
// and the rotary-position table of a set of rows.
//
// Norms are folded into the projections ("llm-rs", section 4, third lesson):
// the norm's gain is multiplied into the next projection's weight columns once,
// and what remains at step time is one scalar per row, 1 / sqrt(mean(x^2) +
// eps), which the projection's epilogue applies to its outputs.  The factor is
// computed once per row here (one wave per row, 16-byte loads, a lane-ordered
// sum followed by a fixed butterfly, so the value does not depend on the batch),
// not in every workgroup of the projection; the same pass can write the bf16
// rounding of the row, which is the projection's input.
//
// Rotary positions (the pages do not describe them; the reading used here is
// the consecutive-pair form): pair i of a head of width d at position p is
// turned by p * base^(-2i / d).  The angle, its cosine and sine are evaluated
// in fp64 and stored as fp32 (cos, sin) per (row, pair), so that the epilogue
// that rotates the projection's outputs only multiplies.

#include <math.h>

#include "common.h"

namespace pkd {

__global__ __launch_bounds__(256) void rms_factor_kernel(const float* __restrict__ x, int n, int cols, float eps,
                                                         float* __restrict__ inv, uint16_t* __restrict__ xb) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), l = lane_id();
  if (r >= n) return;
  const float* row = x + (int64_t)r * cols;
  float ss = 0.f;
  // unrolled so that several 1 KiB wave loads of the row are in flight at once
#pragma unroll 4
  for (int j = l; j < cols / 4; j += 64) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + 4 * j);
    ss = fmaf(v[0], v[0], ss);
    ss = fmaf(v[1], v[1], ss);
    ss = fmaf(v[2], v[2], ss);
    ss = fmaf(v[3], v[3], ss);
    if (xb) *reinterpret_cast<u32x2*>(xb + (int64_t)r * cols + 4 * j) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  if (l == 0) inv[r] = 1.0f / sqrtf(ss / (float)cols + eps);
}

__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* pos, int n, int hd, double base, float* cs) {
  const int half = hd / 2;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, pair)
  if (t >= (int64_t)n * half) return;
  const int r = (int)(t / half), i = (int)(t % half);
  const double th = (double)pos[r] * pow(base, -2.0 * i / hd);
  double sn, c;
  sincos(th, &sn, &c);
  cs[2 * t] = (float)c;
  cs[2 * t + 1] = (float)sn;
}

pkd_status rms_factor_launch(const float* x, int32_t n_rows, int32_t cols, float eps, float* inv_rms, void* x_bf16,
                             hipStream_t stream, pkd_error* err) {
  if (n_rows <= 0) return ok(err);
  hipLaunchKernelGGL(rms_factor_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, stream, x, n_rows, cols, eps, inv_rms,
                     (uint16_t*)x_bf16);
  return check_launch(err, "rms factor");
}

pkd_status rope_table_launch(const int32_t* pos, int32_t n_rows, int32_t head_dim, float base, float* cs,
                             hipStream_t stream, pkd_error* err) {
  if (n_rows <= 0) return ok(err);
  const int64_t t = (int64_t)n_rows * (head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((t + 255) / 256)), dim3(256), 0, stream, pos, n_rows,
                     head_dim, (double)base, cs);
  return check_launch(err, "rope table");
}

}  // namespace pkd
