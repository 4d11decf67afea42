// Static low-rank factors of TTQ (paper-daily.com deep reading, section 2:
// W is split into B A plus a quantised residual; gist.science French summary,
// section 2B: B, A from the SVD of W, kept static).
//
//   ttq_residual  W_res = fp16(W - B A), once per weight.  The rank-r product
//                 is summed in fp64 (each fp32 x fp32 product is exact in
//                 fp64) and rounded once to fp16.
// (Z = X A^T, per call of the projection, is computed by the prescale pass.)
#include "ttq_internal.h"

namespace ttq {

namespace {

// fp64 -> fp16 with a single rounding to nearest even: round to fp32 with
// round-to-odd (sticky inexact bit), then fp32 -> fp16 RNE.  fp32 keeps 13
// more bits than fp16, enough for round-to-odd to make the second rounding
// exact (Boldo & Melquiond, "Emulation of FMA and correctly rounded sums:
// proved algorithms using rounding to odd").
__device__ __forceinline__ _Float16 f64_to_f16_rne(double x) {
  float f = (float)x;  // RNE
  if ((double)f != x) {
    unsigned int b = __builtin_bit_cast(unsigned int, f);
    if (fabs((double)f) > fabs(x)) b -= 1;  // truncate toward zero
    b |= 1u;                                // odd: remembers inexactness
    f = __builtin_bit_cast(float, b);
  }
  return (_Float16)f;
}

template <int R>
__global__ __launch_bounds__(256) void residual_kernel(const _Float16* __restrict__ W,
                                                       const float* __restrict__ B,
                                                       const float* __restrict__ A, int d_out,
                                                       int d_in, _Float16* __restrict__ Wres) {
  const int n = blockIdx.y;
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= d_in) return;
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < R; ++j) acc += (double)B[(int64_t)n * R + j] * (double)A[(int64_t)j * d_in + k];
  const double w = (double)W[(int64_t)n * d_in + k];
  Wres[(int64_t)n * d_in + k] = f64_to_f16_rne(w - acc);
}

}  // namespace

hipError_t launch_residual(int d_out, int d_in, int r, const void* W, const float* B,
                           const float* A, void* W_res, hipStream_t s) {
  dim3 grid((unsigned)((d_in + 255) / 256), (unsigned)d_out);
  if (r != 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL((residual_kernel<16>), grid, dim3(256), 0, s,
                     static_cast<const _Float16*>(W), B, A, d_out, d_in,
                     static_cast<_Float16*>(W_res));
  return hipGetLastError();
}

}  // namespace ttq
