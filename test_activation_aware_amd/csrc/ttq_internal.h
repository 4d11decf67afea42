// Internal declarations shared by the HIP sources of libttq (not part of the
// public ABI in include/ttq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttq {

// Column statistic: partial sums then a fixed-order finalize.  dinv16 (may
// be NULL): an fp16 copy of D^(-1/2).
constexpr int kColstatsMaxChunks = 128;      // row chunks of the partial pass
int colstats_chunks(int64_t T);              // chunks used for T tokens
hipError_t launch_colstats(const void* X, bool x_f32, int64_t T, int64_t d, int64_t ldx,
                           float p, float lambda, float alpha, float* D, float* dinvsqrt,
                           void* dinv16, float* partial, hipStream_t s);

hipError_t launch_quantize_pack(int d_out, int d_in, int q, int g, const void* W,
                                const float* D, uint32_t* codes, void* scales, void* zeros,
                                hipStream_t s);

hipError_t launch_residual(int d_out, int d_in, int r, const void* W, const float* B,
                           const float* A, void* W_res, hipStream_t s);

// Xs = fp16(D^(-1/2) X) in the GEMM's channel order and/or Z = X A^T
// (either output may be NULL), one read of X.
hipError_t launch_prescale_z(int64_t T, int d, const void* X, bool x_f32, int64_t ldx,
                             const float* dinvsqrt, void* Xs, const float* A, float* Z,
                             hipStream_t s);

// Few-token (decode) form of the projection: split-K weight streaming.
constexpr int kDecodeMaxT = 64;
hipError_t launch_wlowbit_decode(int64_t T, int d_in, int d_out, int q, int g, int r, const void* Xs,
                                 int64_t ldxs, const uint32_t* codes, const void* scales, const void* zeros,
                                 const float* B, const float* Z, void* Y, bool y_f32, int64_t ldy,
                                 hipStream_t s);

// The same for T <= kFuseMaxT and r = 0, straight from the raw input X
// (fp16 or fp32, row stride ldx) and D^(-1/2): one launch, the pre-scaling
// done inside; Y has X's dtype.  Bit-identical to launch_prescale_z followed
// by launch_wlowbit_decode.
constexpr int kFuseMaxT = 4;
hipError_t launch_wlowbit_decode_raw(int64_t T, int d_in, int d_out, int q, int g, const void* X, bool x_f32,
                                     int64_t ldx, const float* dinvsqrt, const uint32_t* codes,
                                     const void* scales, const void* zeros, void* Y, int64_t ldy,
                                     hipStream_t s);

// The same for kFuseMaxT < T <= kDecodeMaxT and r = 0 from the raw input:
// split-K over 256-row workgroups that share one pre-scaled copy of their
// input slice, fp32 partials in `workspace` (decode_splitk_ws_bytes), then a
// reduction in split order.  Y has X's dtype.
size_t decode_splitk_ws_bytes(int64_t T, int d_in, int d_out);
hipError_t launch_wlowbit_decode_splitk(int64_t T, int d_in, int d_out, int q, int g, const void* X, bool x_f32,
                                        int64_t ldx, const float* dinvsqrt, const uint32_t* codes,
                                        const void* scales, const void* zeros, void* Y, int64_t ldy,
                                        void* workspace, hipStream_t s);

// The projection; T <= kDecodeMaxT goes to the decode kernel.
hipError_t launch_wlowbit_gemm(int64_t T, int d_in, int d_out, int q, int g, int r, const void* Xs,
                               int64_t ldxs, const uint32_t* codes, const void* scales,
                               const void* zeros, const float* B, const float* Z, void* Y, bool y_f32,
                               int64_t ldy, hipStream_t s);

// The projection for T > kDecodeMaxT straight from the raw fp16 input X (row
// stride ldx) with D^(-1/2) applied on the weight side: dinv16 is
// fp16(D^(-1/2)) [d_in].  Y is fp16.
hipError_t launch_wlowbit_gemm_rawx(int64_t T, int d_in, int d_out, int q, int g, int r, const void* X,
                                    int64_t ldx, const void* dinv16, const uint32_t* codes, const void* scales,
                                    const void* zeros, const float* B, const float* Z, void* Y, int64_t ldy,
                                    hipStream_t s);

}  // namespace ttq
