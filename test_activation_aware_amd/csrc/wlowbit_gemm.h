// Shared declarations of the low-bit projection's translation units: the
// launch arguments and one launcher per code width q (instantiated in
// wlowbit_gemm_q2.hip ... wlowbit_gemm_q5.hip, so the widths compile in
// parallel).
#pragma once

#include "ttq_internal.h"

namespace ttq {

// The launch arguments shared by every instance
struct GemmArgs {
  int64_t T;
  int d_in, d_out;
  const void* X;  // Xs (pre-scaled) or the raw fp16 input
  int64_t ldx;
  const void* dvh;  // fp16 D^(-1/2) (raw input only)
  const uint32_t* codes;
  const void* scales;
  const void* zeros;
  const float* B;
  const float* Z;
  void* Y;
  int64_t ldy;
};

// Launches the prefill projection for code width Q: group size g, rank r,
// fp32 or fp16 output (pre-scaled input), or the raw fp16 input with
// D^(-1/2) on the weight side (rawx, fp16 output).
template <int Q>
hipError_t launch_gemm_q(bool y_f32, bool rawx, int g, int r, const GemmArgs& a, hipStream_t s);

extern template hipError_t launch_gemm_q<2>(bool, bool, int, int, const GemmArgs&, hipStream_t);
extern template hipError_t launch_gemm_q<3>(bool, bool, int, int, const GemmArgs&, hipStream_t);
extern template hipError_t launch_gemm_q<4>(bool, bool, int, int, const GemmArgs&, hipStream_t);
extern template hipError_t launch_gemm_q<5>(bool, bool, int, int, const GemmArgs&, hipStream_t);

}  // namespace ttq
