// ttq_wlowbit_gemm: the TTQ low-bit projection (prefill form), dispatch by
// code width.  The kernel and its design notes are in wlowbit_gemm_impl.h;
// each code width is compiled in its own translation unit.
#include "wlowbit_gemm.h"

namespace ttq {

namespace {

hipError_t launch_q(int q, bool y_f32, bool rawx, int g, int r, const GemmArgs& a, hipStream_t s) {
  switch (q) {
    case 2: return launch_gemm_q<2>(y_f32, rawx, g, r, a, s);
    case 3: return launch_gemm_q<3>(y_f32, rawx, g, r, a, s);
    case 5: return launch_gemm_q<5>(y_f32, rawx, g, r, a, s);
    default: return launch_gemm_q<4>(y_f32, rawx, g, r, a, s);
  }
}

}  // namespace

hipError_t launch_wlowbit_gemm(int64_t T, int d_in, int d_out, int q, int g, int r, const void* Xs,
                               int64_t ldxs, const uint32_t* codes, const void* scales,
                               const void* zeros, const float* B, const float* Z, void* Y, bool y_f32,
                               int64_t ldy, hipStream_t s) {
  if (T == 1) return launch_wlowbit_gemv(d_in, d_out, q, g, r, Xs, codes, scales, zeros, B, Z, Y, y_f32, s);
  if (T <= kFewTokMaxT)
    return launch_wlowbit_fewtok(T, d_in, d_out, q, g, r, Xs, ldxs, nullptr, codes, scales, zeros, B, Z, Y, y_f32, ldy,
                                 s);
  if (T <= kDecodeMaxT)
    return launch_wlowbit_decode(T, d_in, d_out, q, g, r, Xs, ldxs, codes, scales, zeros, B, Z, Y, y_f32, ldy, s);
  const GemmArgs a{T, d_in, d_out, Xs, ldxs, nullptr, codes, scales, zeros, B, Z, Y, ldy};
  return launch_q(q, y_f32, false, g, r, a, s);
}

hipError_t launch_wlowbit_gemm_rawx(int64_t T, int d_in, int d_out, int q, int g, int r, const void* X,
                                    int64_t ldx, const void* dinv16, const uint32_t* codes, const void* scales,
                                    const void* zeros, const float* B, const float* Z, void* Y, int64_t ldy,
                                    hipStream_t s) {
  if (T <= kDecodeMaxT) return hipErrorInvalidValue;
  const GemmArgs a{T, d_in, d_out, X, ldx, dinv16, codes, scales, zeros, B, Z, Y, ldy};
  return launch_q(q, false, true, g, r, a, s);
}

}  // namespace ttq
