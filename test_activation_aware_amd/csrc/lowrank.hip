// Static low-rank factors of TTQ (paper-daily.com deep reading, section 2:
// W is split into B A plus a quantised residual; gist.science French summary,
// section 2B: B, A from the SVD of W, kept static).
//
//   ttq_residual  W_res = fp16(W - B A), once per weight.  The rank-r product
//                 is summed in fp64 (each fp32 x fp32 product is exact in
//                 fp64) and rounded once to fp16.
//   ttq_lowrank_z Z = X A^T (fp32 [T][r]) per call of the projection; the
//                 projection adds B Z in its epilogue.  HBM-bound: X is read
//                 once.
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

// One wave per token row: lanes stride over the d_in channels, each keeps R
// partial dot products, then a butterfly across the wave.
template <typename TX, int R>
__global__ __launch_bounds__(256) void lowrank_z_kernel(const TX* __restrict__ X, int64_t T,
                                                        int d_in, int64_t ldx,
                                                        const float* __restrict__ A,
                                                        float* __restrict__ Z) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.f;
  const TX* xr = X + t * ldx;
  for (int k = lane; k < d_in; k += 64) {
    const float x = (float)xr[k];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] += x * A[(int64_t)j * d_in + k];
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float v = acc[j];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    acc[j] = v;
  }
  if (lane < R) {
    float out = acc[0];
#pragma unroll
    for (int j = 1; j < R; ++j)
      if (lane == j) out = acc[j];
    Z[t * R + lane] = out;
  }
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

hipError_t launch_lowrank_z(int64_t T, int d_in, int r, const void* X, bool x_f32, int64_t ldx,
                            const float* A, float* Z, hipStream_t s) {
  if (r != 16) return hipErrorInvalidValue;
  dim3 grid((unsigned)((T + 3) / 4));
  if (x_f32)
    hipLaunchKernelGGL((lowrank_z_kernel<float, 16>), grid, dim3(256), 0, s,
                       static_cast<const float*>(X), T, d_in, ldx, A, Z);
  else
    hipLaunchKernelGGL((lowrank_z_kernel<_Float16, 16>), grid, dim3(256), 0, s,
                       static_cast<const _Float16*>(X), T, d_in, ldx, A, Z);
  return hipGetLastError();
}

}  // namespace ttq
