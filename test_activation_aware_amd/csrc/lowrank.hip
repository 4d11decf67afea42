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

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
constexpr int kResRows = 32;  // rows of W per workgroup
constexpr int kResGrp = 4;    // rows per step; the next step's rows are loaded meanwhile

// A workgroup owns 32 rows and 1024 channels; a thread owns 4 adjacent
// channels.  Its 16 x 4 values of A are widened to fp64 once and reused for
// the 32 rows, taken 4 at a time while the next 4 rows' W are in flight.
// Each row's B values are the same for the whole workgroup.  Per element:
// the 16 exact products b_j a_j added in the order j = 0..15 starting from
// 0, then w minus that sum, rounded once.
template <int R>
__global__ __launch_bounds__(256) void residual_kernel(const _Float16* __restrict__ W,
                                                       const float* __restrict__ B,
                                                       const float* __restrict__ A, int d_out,
                                                       int d_in, _Float16* __restrict__ Wres) {
  const int k = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (k >= d_in) return;
  const int64_t n0 = (int64_t)blockIdx.y * kResRows;
  h4 wc[kResGrp];
#pragma unroll
  for (int i = 0; i < kResGrp; ++i) wc[i] = *reinterpret_cast<const h4*>(W + (n0 + i) * d_in + k);
  double a[R][4];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const float4 v = *reinterpret_cast<const float4*>(A + (int64_t)j * d_in + k);
    a[j][0] = v.x; a[j][1] = v.y; a[j][2] = v.z; a[j][3] = v.w;
  }
#pragma unroll 1
  for (int i0 = 0; i0 < kResRows; i0 += kResGrp) {
    // the next step's rows (the last step loads its own rows again)
    const int64_t nn = n0 + (i0 + kResGrp < kResRows ? i0 + kResGrp : i0);
    h4 wn[kResGrp];
#pragma unroll
    for (int i = 0; i < kResGrp; ++i) wn[i] = *reinterpret_cast<const h4*>(W + (nn + i) * d_in + k);
#pragma unroll
    for (int i = 0; i < kResGrp; ++i) {
      const float* b = B + (n0 + i0 + i) * R;
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const double bj = (double)b[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += bj * a[j][e];
      }
      h4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = f64_to_f16_rne((double)wc[i][e] - acc[e]);
      *reinterpret_cast<h4*>(Wres + (n0 + i0 + i) * d_in + k) = o;
    }
#pragma unroll
    for (int i = 0; i < kResGrp; ++i) wc[i] = wn[i];
  }
}

}  // namespace

hipError_t launch_residual(int d_out, int d_in, int r, const void* W, const float* B,
                           const float* A, void* W_res, hipStream_t s) {
  if (r != 16 || d_out % kResRows != 0 || d_in % 4 != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)((d_in + 1023) / 1024), (unsigned)(d_out / kResRows));
  hipLaunchKernelGGL((residual_kernel<16>), grid, dim3(256), 0, s,
                     static_cast<const _Float16*>(W), B, A, d_out, d_in,
                     static_cast<_Float16*>(W_res));
  return hipGetLastError();
}

}  // namespace ttq
