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

// The same from a fixed per-device scratch array of the library (no
// workspace argument, nothing allocated): kColstatsScratchBytes hold the
// partial sums of up to kColstatsScratchMaxD channels at any T.
// hipErrorInvalidValue when colstats_chunks(T) * d floats do not fit.  Calls that overlap on one
// GPU share the array and race.
constexpr int kColstatsScratchMaxD = 16384;
constexpr size_t kColstatsScratchBytes = (size_t)kColstatsMaxChunks * kColstatsScratchMaxD * sizeof(float);  // 8 MiB
hipError_t launch_colstats_noalloc(const void* X, bool x_f32, int64_t T, int64_t d, int64_t ldx, float p,
                                   float lambda, float alpha, float* D, float* dinvsqrt, hipStream_t s);
hipError_t launch_colstats(const void* X, bool x_f32, int64_t T, int64_t d, int64_t ldx,
                           float p, float lambda, float alpha, float* D, float* dinvsqrt,
                           void* dinv16, float* partial, hipStream_t s);

// The same statistic from fp16 X together with Z = X A^T (fp32 [T][16], A
// fp32 [16][d], d a multiple of 64): one read of X.  The partial sums take
// colstats_z_chunks(T) rows of d floats.
int colstats_z_chunks(int64_t T);
hipError_t launch_colstats_z(const void* X, int64_t T, int d, int64_t ldx, float p, float lambda, float alpha,
                             const float* A, float* D, float* dinvsqrt, void* dinv16, float* partial, float* Z,
                             hipStream_t s);

// Codes, scales and zeros of W D^(1/2); with wexp != NULL also the effective
// fp16 weight W_hat = fp16(fp16((c - z) s) * dinv16) [d_out][d_in] (dinv16:
// fp16 D^(-1/2) [d_in]), and with B, A (fp32 rank-16 factors [d_out][16],
// [16][d_in]; only together with wexp) W_hat + B A rounded once to fp16.
hipError_t launch_quantize_pack(int d_out, int d_in, int q, int g, const void* W,
                                const float* D, uint32_t* codes, void* scales, void* zeros,
                                const void* dinv16, void* wexp, const float* B, const float* A,
                                hipStream_t s);

// One online step of the rank-16 factors for a prompt's statistic D: the
// orthonormal right basis V [d_in][16] is advanced by one subspace-iteration
// step on (W D^(1/2))^T (W D^(1/2)) and B [d_out][16], A [16][d_in] are
// formed from it (all fp32).  d_in a multiple of 128, d_out of 32.
size_t lowrank_refresh_ws_bytes(int d_out, int d_in);
hipError_t launch_lowrank_refresh(int d_out, int d_in, const void* W, const float* D, float* V, float* B,
                                  float* A, void* workspace, hipStream_t s);

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

// The same for kFewTokMaxT < T <= kDecodeMaxT and r = 0 from the raw input:
// split-K over 256-row workgroups that share one pre-scaled copy of their
// input slice, fp32 partials in `workspace` (decode_splitk_ws_bytes), then a
// reduction in split order.  Y has X's dtype.
size_t decode_splitk_ws_bytes(int64_t T, int d_in, int d_out);
hipError_t launch_wlowbit_decode_splitk(int64_t T, int d_in, int d_out, int q, int g, const void* X, bool x_f32,
                                        int64_t ldx, const float* dinvsqrt, const uint32_t* codes,
                                        const void* scales, const void* zeros, void* Y, int64_t ldy,
                                        void* workspace, hipStream_t s);

// The projection of a single token (T = 1): a dot-product form of the
// decode, one workgroup per 32-row tile.  launch_wlowbit_gemv takes the
// pre-scaled input Xs [d_in] (and Z [16], B for r > 0; Y fp16 or fp32);
// launch_wlowbit_gemv_raw the raw x (fp16 or fp32) and D^(-1/2), r = 0, Y of
// x's type.  The two give the same bits for the same input.
hipError_t launch_wlowbit_gemv(int d_in, int d_out, int q, int g, int r, const void* Xs, const uint32_t* codes,
                               const void* scales, const void* zeros, const float* B, const float* Z, void* Y,
                               bool y_f32, hipStream_t s);
hipError_t launch_wlowbit_gemv_raw(int d_in, int d_out, int q, int g, const void* X, bool x_f32,
                                   const float* dinvsqrt, const uint32_t* codes, const void* scales,
                                   const void* zeros, void* Y, hipStream_t s);

// The projection of 2 <= T <= kFewTokMaxT tokens, one workgroup per 32-row
// tile on the matrix cores: dinv16 == NULL, X is the pre-scaled Xs (Y fp16 or
// fp32, B and Z for r > 0); dinv16 = fp16(D^(-1/2)), X is the raw fp16 input
// with D^(-1/2) applied on the weight side (Y fp16).  X rows of stride ldx.
constexpr int kFewTokMaxT = 16;
hipError_t launch_wlowbit_fewtok(int64_t T, int d_in, int d_out, int q, int g, int r, const void* X, int64_t ldx,
                                 const void* dinv16, const uint32_t* codes, const void* scales, const void* zeros,
                                 const float* B, const float* Z, void* Y, bool y_f32, int64_t ldy, hipStream_t s);

// The projection; T = 1 goes to the dot-product form, T <= kFewTokMaxT to the
// few-token form, T <= kDecodeMaxT to the decode kernel.
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

// The projection of a long prompt from the effective fp16 weight W_hat
// [d_out][d_in] (written by the quantiser): Y = W_hat X + B Z, fp16 X and Y.
// Same results as launch_wlowbit_gemm_rawx on the matching codes.
hipError_t launch_dense_gemm(int64_t T, int d_in, int d_out, int r, const void* X, int64_t ldx, const void* Wt,
                             const float* B, const float* Z, void* Y, int64_t ldy, hipStream_t s);

}  // namespace ttq
