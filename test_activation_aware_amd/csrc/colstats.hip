// ttq_colstats: per-input-channel activation statistic of one prompt,
//   d_j = (mean_t |x_tj|^p + lambda)^alpha,  also D^(-1/2),
// the online AWQ diagonal of the TTQ paper (paper-daily.com deep reading,
// section 2; gist.science German summary, section 2: p-norm form).
//
// HBM-bound column reduction over the T rows of X [T][ldx].
//   pass 1 (colstats_partial): grid (column slabs, row chunks).  A workgroup
//     of 4 waves owns one slab of 64*VEC columns; each lane owns VEC adjacent
//     columns (one 16-byte load per row, eight rows in flight, nontemporal)
//     and the 4 waves take interleaved rows of the chunk.  Lane sums stay in
//     fp32 registers, the 4 waves are
//     combined through LDS and one partial per (chunk, column) is written.
//   pass 2 (colstats_finalize): per column, 8 threads sum interleaved slices
//     of the chunk partials in fp64 and the slices are combined in a fixed
//     order; then divide by T, add lambda, raise to alpha, round once to
//     fp32.  No atomics: bitwise deterministic.
//
// With the rank-16 term (fp16 input), colstats_z_partial replaces pass 1 and
// also forms Z = X A^T, the low-rank input of the projection
// Y = Q[(W - B A) D^(1/2)] (D^(-1/2) X) + B (A X) (paper-daily.com deep
// reading, section 2: static low-rank factors applied to the raw input), from
// the same read of X.  A workgroup owns 16 TG tokens and all d channels; its
// 8 waves take 32-channel chunks round-robin.  Lane l holds token l % 16 and
// channels 8 (l / 16) .. + 8 of a chunk, the operand layout of a 16x16x32
// fp16 MFMA whose other operand is the matching slice of A^T (A split into
// two fp16 parts, so Z keeps about 22 bits; the operands of ttq_lowrank_z,
// with the chunks summed in another grouping, so Z agrees with it to fp32
// rounding, not bit for bit).  For the
// statistic each lane squares its 8 channels over its TG tokens, and the 16
// lanes that hold the same channels are added by a fixed tree of DPP row
// rotations; one partial row per workgroup (16 TG tokens) goes to the same
// finalize pass.
#include <mutex>

#include "ttq_internal.h"

// Fixed scratch of ttq_colstats_noalloc, for callers that cannot allocate
// device memory: the partial sums of the statistic, kColstatsScratchBytes on
// every GPU the library runs on, held until the process ends.  Host code
// never passes `scratch` itself to a kernel (in host code the name is a
// host-side stand-in, not a device address): it looks up each device's
// address once with hipGetSymbolAddress and passes that.
static __device__ __align__(256) float scratch[ttq::kColstatsScratchBytes / sizeof(float)];

namespace ttq {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsInFlight = 8;  // 16-byte row loads per lane in flight (partial pass)
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

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
    // eight rows in flight per lane, read with the nontemporal hint (X is
    // streamed once here): at the Qwen3-32B q_proj prompt (16384 x 5120 fp16)
    // 26.4 us cold against 31.2-32.0 us for four plain loads in flight, warm
    // unchanged; rows are still added in row order, so the sums are the same
    for (; t + (kRowsInFlight - 1) * kWaves < r1; t += kRowsInFlight * kWaves) {
      uint4 raw[kRowsInFlight];
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const u4v q = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(base + (t + u * kWaves) * ldx));
        raw[u] = make_uint4(q[0], q[1], q[2], q[3]);
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
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
// w, w+8, w+16, ... in that order and the 8 slice sums are added in slice
// order.
__global__ __launch_bounds__(256) void colstats_finalize(const float* __restrict__ partial, int chunks,
                                                         int64_t d, int64_t T, double lambda,
                                                         double alpha, float* __restrict__ D,
                                                         float* __restrict__ dinvsqrt,
                                                         _Float16* __restrict__ dinv16) {
  const int cx = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int64_t j = (int64_t)blockIdx.x * 32 + cx;
  // a slice requests kPerSlice of its chunk partials at once (clamped,
  // unconditional loads), then adds them in chunk order
  constexpr int kPerSlice = kColstatsMaxChunks / 8;
  const int64_t jc = j < d ? j : d - 1;
  double s = 0.0;
  for (int base = 0; base < chunks; base += 8 * kPerSlice) {
    float v[kPerSlice];
#pragma unroll
    for (int i = 0; i < kPerSlice; ++i) v[i] = partial[(int64_t)min(base + sl + 8 * i, chunks - 1) * d + jc];
#pragma unroll
    for (int i = 0; i < kPerSlice; ++i)
      if (base + sl + 8 * i < chunks) s += (double)v[i];
  }
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

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kRank = 16;   // rows of A
constexpr int kTok = 16;    // tokens per MFMA group
constexpr int kChunk = 32;  // channels per wave step

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k + 15), by rotations
// of 8, 4, 2 and 1 lanes: every lane of the row ends with the row's total,
// always added in the same order.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
  return v;
}

constexpr int kZWaves = 8;  // waves of the fused pass, each on every 8th chunk

template <int PMODE, int TG>
__global__ __launch_bounds__(64 * kZWaves) void colstats_z_partial(int64_t T, int d, const _Float16* __restrict__ X,
                                                          int64_t ldx, float p, const float* __restrict__ A,
                                                          float* __restrict__ partial, float* __restrict__ Z) {
  __shared__ f4 zred[kZWaves][TG][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, kb = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kTok * TG;
  const _Float16* xr[TG];
  float live[TG];  // 1 for tokens < T, 0 for the clamped rows past the end
#pragma unroll
  for (int g = 0; g < TG; ++g) {
    const int64_t t = t0 + kTok * g + row;
    xr[g] = X + (t < T ? t : T - 1) * ldx + 8 * kb;
    live[g] = t < T ? 1.f : 0.f;
  }
  const float* ar = A + (int64_t)row * d + 8 * kb;  // A^T column j = row of A
  float* prow = partial + (int64_t)blockIdx.x * d + 8 * kb;
  f4 acc[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};
  const int nchunks = d / kChunk;

  auto chunk = [&](int k0, const h8 (&x)[TG], const float (&a)[8]) {
    h8 ahi, alo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ahi[e] = (_Float16)a[e];
      alo[e] = (_Float16)(a[e] - (float)ahi[e]);
    }
#pragma unroll
    for (int g = 0; g < TG; ++g) {
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x[g], ahi, acc[g], 0, 0, 0);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x[g], alo, acc[g], 0, 0, 0);
    }
    float st[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = live[0] * powabs<PMODE>((float)x[0][e], p);
#pragma unroll
      for (int g = 1; g < TG; ++g) v += live[g] * powabs<PMODE>((float)x[g][e], p);
      st[e] = row16_sum(v);
    }
    if (row == 0) {
      float4* o = reinterpret_cast<float4*>(prow + k0);
      o[0] = make_float4(st[0], st[1], st[2], st[3]);
      o[1] = make_float4(st[4], st[5], st[6], st[7]);
    }
  };
  auto load_chunk = [&](int k0, h8 (&x)[TG], float (&a)[8]) {
#pragma unroll
    for (int g = 0; g < TG; ++g) x[g] = *reinterpret_cast<const h8*>(xr[g] + k0);
    const float4 a0 = reinterpret_cast<const float4*>(ar + k0)[0];
    const float4 a1 = reinterpret_cast<const float4*>(ar + k0)[1];
    a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
    a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
  };
  // kU chunks per pass, all their loads requested before any is used; a wave
  // accumulates its chunks in the order c = wave, wave + 8, ...
  constexpr int kU = 4;
  int c = wave;
  for (; c + kZWaves * (kU - 1) < nchunks; c += kZWaves * kU) {
    h8 x[kU][TG];
    float a[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) load_chunk((c + kZWaves * u) * kChunk, x[u], a[u]);
#pragma unroll
    for (int u = 0; u < kU; ++u) chunk((c + kZWaves * u) * kChunk, x[u], a[u]);
  }
  for (; c < nchunks; c += kZWaves) {
    h8 x[TG];
    float a[8];
    load_chunk(c * kChunk, x, a);
    chunk(c * kChunk, x, a);
  }

  // lane l holds Z[t0 + 16 g + 4 (l / 16) + i][l % 16], i = 0..3, for this
  // wave's chunks; the 8 waves' partials are added in wave order
#pragma unroll
  for (int g = 0; g < TG; ++g) zred[wave][g][lane] = acc[g];
  __syncthreads();
  if (wave < TG) {
    const int g = wave;
    f4 s = zred[0][g][lane];
#pragma unroll
    for (int w = 1; w < kZWaves; ++w) {
      const f4 v = zred[w][g][lane];
      s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tz = t0 + kTok * g + 4 * kb + i;
      if (tz < T) Z[tz * kRank + row] = s[i];
    }
  }
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

// tokens per workgroup of the fused pass: 64 while that leaves a workgroup
// per CU, else 16 tokens
int colstats_z_tg(int64_t T) { return T >= 64 * 256 ? 4 : 1; }

int colstats_z_chunks(int64_t T) {
  const int64_t tok = (int64_t)kTok * colstats_z_tg(T);
  return (int)((T + tok - 1) / tok);
}

hipError_t launch_colstats_z(const void* X, int64_t T, int d, int64_t ldx, float p, float lambda, float alpha,
                             const float* A, float* D, float* dinvsqrt, void* dinv16, float* partial, float* Z,
                             hipStream_t s) {
  const int tg = colstats_z_tg(T);
  const int chunks = colstats_z_chunks(T);
  const _Float16* x = static_cast<const _Float16*>(X);
  const dim3 grid((unsigned)chunks), block(64 * kZWaves);
#define TTQ_CZ(PM, TGV) hipLaunchKernelGGL((colstats_z_partial<PM, TGV>), grid, block, 0, s, T, d, x, ldx, p, A, partial, Z)
  if (tg == 4) {
    if (p == 2.0f) TTQ_CZ(2, 4);
    else if (p == 1.0f) TTQ_CZ(1, 4);
    else TTQ_CZ(0, 4);
  } else {
    if (p == 2.0f) TTQ_CZ(2, 1);
    else if (p == 1.0f) TTQ_CZ(1, 1);
    else TTQ_CZ(0, 1);
  }
#undef TTQ_CZ
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colstats_finalize, dim3((unsigned)((d + 31) / 32)), dim3(256), 0, s, partial, chunks, (int64_t)d,
                     T, (double)lambda, (double)alpha, D, dinvsqrt, static_cast<_Float16*>(dinv16));
  return hipGetLastError();
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The device the work of stream s runs on (the current device for the null
// stream), and that device's address of `scratch`: looked up once per device
// with that device current (the caller's current device is restored).
hipError_t scratch_for_stream(hipStream_t s, float** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (s != nullptr) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(s, &sd);
    if (e != hipSuccess) return e;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

}  // namespace

hipError_t launch_colstats_noalloc(const void* X, bool x_f32, int64_t T, int64_t d, int64_t ldx, float p,
                                   float lambda, float alpha, float* D, float* dinvsqrt, hipStream_t s) {
  if ((size_t)colstats_chunks(T) * (size_t)d * sizeof(float) > kColstatsScratchBytes) return hipErrorInvalidValue;
  float* partial = nullptr;
  hipError_t e = scratch_for_stream(s, &partial);
  if (e != hipSuccess) return e;
  // every partial the finalize pass reads is written first by the partial
  // pass of the same call: nothing needs clearing between calls
  return launch_colstats(X, x_f32, T, d, ldx, p, lambda, alpha, D, dinvsqrt, nullptr, partial, s);
}

hipError_t launch_colstats(const void* X, bool x_f32, int64_t T, int64_t d, int64_t ldx, float p,
                           float lambda, float alpha, float* D, float* dinvsqrt, void* dinv16, float* partial,
                           hipStream_t s) {
  if (x_f32) return launch_typed<float>(X, T, d, ldx, p, lambda, alpha, D, dinvsqrt, dinv16, partial, s);
  return launch_typed<_Float16>(X, T, d, ldx, p, lambda, alpha, D, dinvsqrt, dinv16, partial, s);
}

}  // namespace ttq
