// ttq_colstats: per-input-channel activation statistic of one prompt,
//   d_j = (mean_t |x_tj|^p + lambda)^alpha,  also D^(-1/2),
// the online AWQ diagonal of the TTQ paper (paper-daily.com deep reading,
// section 2; gist.science German summary, section 2: p-norm form).
//
// HBM-bound column reduction over the T rows of X [T][ldx].
//   pass 1 (colstats_partial): grid (column slabs, row chunks).  A workgroup
//     of 4 waves owns one slab of 64*VEC columns; each lane owns VEC adjacent
//     columns (one 16-byte load per row) and the 4 waves take interleaved
//     rows of the chunk.  Lane sums stay in fp32 registers, the 4 waves are
//     combined through LDS and one partial per (chunk, column) is written.
//   pass 2 (colstats_finalize): per column, 8 threads sum interleaved slices
//     of the chunk partials in fp64 and the slices are combined in a fixed
//     order; then divide by T, add lambda, raise to alpha, round once to
//     fp32.  No atomics: bitwise deterministic.
#include "ttq_internal.h"

namespace ttq {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int PMODE>
__device__ __forceinline__ float powabs(float x, float p) {
  if constexpr (PMODE == 2) {
    return x * x;
  } else if constexpr (PMODE == 1) {
    return fabsf(x);
  } else {
    return powf(fabsf(x), p);
  }
}

// VEC = 8 fp16 or 4 fp32 columns per lane (one 16-byte load per row).
template <typename TX, int PMODE>
__global__ __launch_bounds__(kThreads) void colstats_partial(const TX* __restrict__ X, int64_t T,
                                                             int64_t d, int64_t ldx, int64_t rows_per_chunk,
                                                             float p, float* __restrict__ partial) {
  constexpr int VEC = 16 / sizeof(TX);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = (int64_t)blockIdx.x * (64 * VEC) + (int64_t)lane * VEC;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = min(T, r0 + rows_per_chunk);
  const bool active = col0 < d;  // d is a multiple of VEC

  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;

  if (active) {
    const TX* base = X + col0;
    int64_t t = r0 + wave;
    // four rows in flight per lane
    for (; t + 3 * kWaves < r1; t += 4 * kWaves) {
      uint4 raw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        raw[u] = *reinterpret_cast<const uint4*>(base + (t + u * kWaves) * ldx);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const TX* e = reinterpret_cast<const TX*>(&raw[u]);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += powabs<PMODE>((float)e[v], p);
      }
    }
    for (; t < r1; t += kWaves) {
      uint4 raw = *reinterpret_cast<const uint4*>(base + t * ldx);
      const TX* e = reinterpret_cast<const TX*>(&raw);
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] += powabs<PMODE>((float)e[v], p);
    }
  }

  __shared__ float red[kWaves][64 * VEC + 1];
#pragma unroll
  for (int v = 0; v < VEC; ++v) red[wave][lane * VEC + v] = acc[v];
  __syncthreads();
  // combine the 4 waves in a fixed order and store one partial per column
  for (int c = threadIdx.x; c < 64 * VEC; c += kThreads) {
    const int64_t col = (int64_t)blockIdx.x * (64 * VEC) + c;
    if (col < d) {
      float s = red[0][c];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) s += red[w][c];
      partial[(int64_t)blockIdx.y * d + col] = s;
    }
  }
}

// 256 threads = 32 columns x 8 slices of the chunk list; slice w sums chunks
// w, w+8, w+16, ... and the 8 slice sums are added in slice order.
__global__ __launch_bounds__(256) void colstats_finalize(const float* __restrict__ partial, int chunks,
                                                         int64_t d, int64_t T, double lambda,
                                                         double alpha, float* __restrict__ D,
                                                         float* __restrict__ dinvsqrt,
                                                         _Float16* __restrict__ dinv16) {
  const int cx = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int64_t j = (int64_t)blockIdx.x * 32 + cx;
  // all of this slice's chunk partials are requested at once (clamped,
  // unconditional loads), then added in chunk order
  constexpr int kPerSlice = kColstatsMaxChunks / 8;
  const int64_t jc = j < d ? j : d - 1;
  float v[kPerSlice];
#pragma unroll
  for (int i = 0; i < kPerSlice; ++i) v[i] = partial[(int64_t)min(sl + 8 * i, chunks - 1) * d + jc];
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kPerSlice; ++i)
    if (sl + 8 * i < chunks) s += (double)v[i];
  __shared__ double red[8][32];
  red[sl][cx] = s;
  __syncthreads();
  if (sl != 0 || j >= d) return;
  double t = red[0][cx];
#pragma unroll
  for (int w = 1; w < 8; ++w) t += red[w][cx];
  const double m = t / (double)T;
  const float dj = (float)pow(m + lambda, alpha);
  D[j] = dj;
  const float r = (float)(1.0 / sqrt((double)dj));
  dinvsqrt[j] = r;
  if (dinv16 != nullptr) dinv16[j] = (_Float16)r;  // fp16 copy, rounded to nearest even
}

template <typename TX>
hipError_t launch_typed(const void* X, int64_t T, int64_t d, int64_t ldx, float p, float lambda,
                        float alpha, float* D, float* dinvsqrt, void* dinv16, float* partial, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(TX);
  const int chunks = colstats_chunks(T);
  const int64_t rows = (T + chunks - 1) / chunks;
  dim3 grid((unsigned)((d + 64 * VEC - 1) / (64 * VEC)), (unsigned)chunks);
  const TX* x = static_cast<const TX*>(X);
  if (p == 2.0f)
    hipLaunchKernelGGL((colstats_partial<TX, 2>), grid, dim3(kThreads), 0, s, x, T, d, ldx, rows, p, partial);
  else if (p == 1.0f)
    hipLaunchKernelGGL((colstats_partial<TX, 1>), grid, dim3(kThreads), 0, s, x, T, d, ldx, rows, p, partial);
  else
    hipLaunchKernelGGL((colstats_partial<TX, 0>), grid, dim3(kThreads), 0, s, x, T, d, ldx, rows, p, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colstats_finalize, dim3((unsigned)((d + 31) / 32)), dim3(256), 0, s, partial,
                     chunks, d, T, (double)lambda, (double)alpha, D, dinvsqrt, static_cast<_Float16*>(dinv16));
  return hipGetLastError();
}

}  // namespace

int colstats_chunks(int64_t T) {
  // chunks of at least 32 rows (8 per wave), at most kColstatsMaxChunks
  int64_t c = (T + 31) / 32;
  if (c > kColstatsMaxChunks) c = kColstatsMaxChunks;
  if (c < 1) c = 1;
  return (int)c;
}

hipError_t launch_colstats(const void* X, bool x_f32, int64_t T, int64_t d, int64_t ldx, float p,
                           float lambda, float alpha, float* D, float* dinvsqrt, void* dinv16, float* partial,
                           hipStream_t s) {
  if (x_f32) return launch_typed<float>(X, T, d, ldx, p, lambda, alpha, D, dinvsqrt, dinv16, partial, s);
  return launch_typed<_Float16>(X, T, d, ldx, p, lambda, alpha, D, dinvsqrt, dinv16, partial, s);
}

}  // namespace ttq
