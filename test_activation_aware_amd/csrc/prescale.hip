// The two per-call passes over the raw input X of the TTQ projection
//   Y = Q[(W - B A) D^(1/2)] (D^(-1/2) X) + B (A X)
// (paper-daily.com deep reading, section 2: the closed form Q[W D^(1/2)] D^(-1/2)
// and the static low-rank term B A applied to the raw input):
//
//   Xs = fp16(D^(-1/2) X)   the pre-scaled input the low-bit GEMM streams;
//   Z  = X A^T              fp32 [T][16], the rank-16 input of the epilogue.
//
// One kernel does either or both: X is read from HBM once.  Xs keeps the
// channel order of X, rows of d fp16 values.
//
// Xs is written with nontemporal stores: the GEMM reads it back from HBM
// anyway (it is far larger than the caches), and streaming it past L2 keeps
// dirty lines from piling up there (about 20 % faster than plain stores).
//
// Xs alone streams rows (8 channels per thread, D^(-1/2) held in registers).
// With Z: a workgroup owns 16 tokens; its 4 waves take 32-channel
// chunks round-robin, so at any time the workgroup streams 128 contiguous
// channels of 16 rows.  Lane l holds token l%16 and channels 8*(l/16)..+8 of
// the chunk: exactly the A operand of a 16x16x32 fp16 MFMA, whose B operand
// is the matching slice of A^T (fp32 A split into two fp16 parts so that Z
// keeps about 22 bits; fp32 X uses the 16x16x4 fp32 MFMA instead).  The four
// waves' partial Z are summed through LDS at the end.
#include "ttq_internal.h"

namespace ttq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kRank = 16;
constexpr int kTok = 16;    // tokens per workgroup
constexpr int kChunk = 32;  // channels per wave step

template <typename TX>
__device__ __forceinline__ void load8(const TX* p, float v[8]) {
  if constexpr (sizeof(TX) == 2) {
    const h8 h = *reinterpret_cast<const h8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)h[e];
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename TX, bool XS, bool ZZ, int TG>
__global__ __launch_bounds__(256) void prescale_z_kernel(int64_t T, int d, const TX* __restrict__ X,
                                                         int64_t ldx, const float* __restrict__ dinvsqrt,
                                                         _Float16* __restrict__ Xs,
                                                         const float* __restrict__ A,
                                                         float* __restrict__ Z) {
  // TG groups of 16 tokens per workgroup: each slice of A (and of D^(-1/2))
  // a wave loads serves TG groups, so A is read from L2 once per 16 TG tokens
  __shared__ f4 zred[4][TG][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, kb = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kTok * TG;
  const TX* xr[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) {
    const int64_t t = t0 + kTok * g + row;
    xr[g] = X + (t < T ? t : T - 1) * ldx + 8 * kb;  // rows past T are read clamped and not stored
  }
  const float* ar = A + (int64_t)row * d + 8 * kb;  // A^T column j = row of A
  f4 acc[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};
  const int nchunks = d / kChunk;

  // kU chunks per pass, all their loads requested before any is used (one
  // memory round trip per pass instead of per chunk); chunks are still
  // accumulated in order c = wave, wave + 4, ...
  auto chunk = [&](int k0, const float (&x)[TG][8], const float (&dv)[8], const float (&a)[8]) {
    if constexpr (XS) {
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        h8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[2 * e] = (_Float16)(x[g][2 * e] * dv[2 * e]);
          o[2 * e + 1] = (_Float16)(x[g][2 * e + 1] * dv[2 * e + 1]);
        }
        const int64_t t = t0 + kTok * g + row;
        if (t < T) __builtin_nontemporal_store(o, reinterpret_cast<h8*>(Xs + t * d + k0 + 8 * kb));
      }
    }
    if constexpr (ZZ) {
      if constexpr (sizeof(TX) == 2) {
        h8 ahi, alo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ahi[e] = (_Float16)a[e];
          alo[e] = (_Float16)(a[e] - (float)ahi[e]);
        }
#pragma unroll
        for (int g = 0; g < TG; ++g) {
          h8 xh;
#pragma unroll
          for (int e = 0; e < 8; ++e) xh[e] = (_Float16)x[g][e];  // exact: x came from fp16
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, ahi, acc[g], 0, 0, 0);
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, alo, acc[g], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int g = 0; g < TG; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[g][e], a[e], acc[g], 0, 0, 0);
      }
    }
  };
  auto load_chunk = [&](int k0, float (&x)[TG][8], float (&dv)[8], float (&a)[8]) {
#pragma unroll
    for (int g = 0; g < TG; ++g) load8<TX>(xr[g] + k0, x[g]);
    if constexpr (XS) load8<float>(dinvsqrt + k0 + 8 * kb, dv);
    if constexpr (ZZ) load8<float>(ar + k0, a);
  };
  constexpr int kU = TG >= 4 ? 2 : 4;
  int c = wave;
  for (; c + 4 * (kU - 1) < nchunks; c += 4 * kU) {
    float x[kU][TG][8], dv[kU][8], a[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) load_chunk((c + 4 * u) * kChunk, x[u], dv[u], a[u]);
#pragma unroll
    for (int u = 0; u < kU; ++u) chunk((c + 4 * u) * kChunk, x[u], dv[u], a[u]);
  }
  for (; c < nchunks; c += 4) {
    float x[TG][8], dv[8], a[8];
    load_chunk(c * kChunk, x, dv, a);
    chunk(c * kChunk, x, dv, a);
  }

  if constexpr (ZZ) {
    // lane l holds Z[t0 + 16 g + 4*(l/16) + i][l % 16], i = 0..3, for this
    // wave's chunks; the 4 waves' partials are added in wave order
#pragma unroll
    for (int g = 0; g < TG; ++g) zred[wave][g][lane] = acc[g];
    __syncthreads();
    if (wave < TG) {
      const int g = wave;
      f4 s = zred[0][g][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
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
}

// Xs only (r = 0): a pure stream.  Thread = 8 channels (one 16-byte piece of
// Xs), D^(-1/2) of its channels held in registers across kRows rows; a wave
// moves 1 KB of contiguous row bytes per load and per store.
constexpr int kRows = 32;

template <typename TX>
__global__ __launch_bounds__(256) void prescale_kernel(int64_t T, int d, const TX* __restrict__ X,
                                                       int64_t ldx, const float* __restrict__ dinvsqrt,
                                                       _Float16* __restrict__ Xs) {
  const int c8 = blockIdx.y * 256 + threadIdx.x;  // 8-channel piece
  if (c8 * 8 >= d) return;
  const int64_t t0 = (int64_t)blockIdx.x * kRows;
  const int rows = (int)min<int64_t>(kRows, T - t0);
  const float4 da = *reinterpret_cast<const float4*>(dinvsqrt + 8 * c8);
  const float4 db = *reinterpret_cast<const float4*>(dinvsqrt + 8 * c8 + 4);
  const float dv[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
  const TX* xp = X + t0 * ldx + 8 * c8;
  _Float16* yp = Xs + t0 * d + 8 * c8;
#pragma unroll 8
  for (int i = 0; i < rows; ++i) {
    float x[8];
    load8<TX>(xp + i * ldx, x);
    h8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = (_Float16)(x[2 * e] * dv[2 * e]);
      o[2 * e + 1] = (_Float16)(x[2 * e + 1] * dv[2 * e + 1]);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<h8*>(yp + (int64_t)i * d));
  }
}

template <typename TX>
hipError_t launch_tx(int64_t T, int d, const void* X, int64_t ldx, const float* dinv, void* Xs,
                     const float* A, float* Z, hipStream_t s) {
  const TX* x = static_cast<const TX*>(X);
  _Float16* xs = static_cast<_Float16*>(Xs);
  if (Xs && !Z) {
    hipLaunchKernelGGL((prescale_kernel<TX>), dim3((unsigned)((T + kRows - 1) / kRows), (unsigned)((d / 8 + 255) / 256)),
                       dim3(256), 0, s, T, d, x, ldx, dinv, xs);
    return hipGetLastError();
  }
  // 64 tokens per workgroup while that still leaves a workgroup per CU, else
  // (Z alone) 32 from two workgroups per CU on, else 16: every workgroup reads
  // all of A from L2, so fewer, wider workgroups read less of it
  const int tg = T >= 64 * 256 ? 4 : (!Xs && T >= 32 * 256 ? 2 : 1);
  const dim3 grid((unsigned)((T + kTok * tg - 1) / (kTok * tg)));
  if (Xs) {
    if (tg == 4)
      hipLaunchKernelGGL((prescale_z_kernel<TX, true, true, 4>), grid, dim3(256), 0, s, T, d, x, ldx, dinv, xs, A, Z);
    else
      hipLaunchKernelGGL((prescale_z_kernel<TX, true, true, 1>), grid, dim3(256), 0, s, T, d, x, ldx, dinv, xs, A, Z);
  } else {
    if (tg == 4)
      hipLaunchKernelGGL((prescale_z_kernel<TX, false, true, 4>), grid, dim3(256), 0, s, T, d, x, ldx, dinv, xs, A, Z);
    else if (tg == 2)
      hipLaunchKernelGGL((prescale_z_kernel<TX, false, true, 2>), grid, dim3(256), 0, s, T, d, x, ldx, dinv, xs, A, Z);
    else
      hipLaunchKernelGGL((prescale_z_kernel<TX, false, true, 1>), grid, dim3(256), 0, s, T, d, x, ldx, dinv, xs, A, Z);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prescale_z(int64_t T, int d, const void* X, bool x_f32, int64_t ldx,
                             const float* dinvsqrt, void* Xs, const float* A, float* Z,
                             hipStream_t s) {
  if (T <= 0 || (!Xs && !Z)) return hipSuccess;
  if (x_f32) return launch_tx<float>(T, d, X, ldx, dinvsqrt, Xs, A, Z, s);
  return launch_tx<_Float16>(T, d, X, ldx, dinvsqrt, Xs, A, Z, s);
}

}  // namespace ttq
