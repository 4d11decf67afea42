// ttq_quantize_pack: activation-scaled group round-to-nearest quantisation
// of W_res D^(1/2) and packing of the codes (TTQ paper: paper-daily.com deep
// reading, section 2, RTN QDQ per group and the AWQ closed form
// Q[W D^(1/2)] D^(-1/2); gist.science German summary, section 2, per-group
// scale S and zero point Z).
//
// Rules (all fp32, one rounding per operation; identical to the CPU oracle):
//   sq_j = sqrt(D_j)                    correctly rounded
//   v    = w * sq_j                     w an fp16 weight
//   mn   = min(0, min_G v), mx = max(0, max_G v)
//   s32  = (mx - mn) / N,  N = 2^q - 1  IEEE division
//   s    = smallest positive fp16 >= s32 (1 for an all-zero group)
//   z    = clamp(rint(-mn / s), 0, N)   round half to even
//   c    = clamp(rint(v / s) + z, 0, N)
//
// Work split: one lane owns one block of 32 consecutive input channels and
// keeps the same block for every row it visits, so its 32 sqrt(D) values are
// computed once and stay in registers.  A group of g = 64 or 128 channels is
// 2 or 4 adjacent lanes; their min/max meet through lane shuffles.  Lanes of
// a wave read 64 consecutive 64-byte blocks (4 KB contiguous) and write their
// q packed words contiguously: the kernel streams W once (HBM-bound).
//
// Codes use a reciprocal fast path: with r = 1/s (one IEEE division per
// group), u = fma(v, r, z) lies within 2^-18 of v/s + z, so whenever u is
// more than 2^-16 away from every half-integer, rint(u) equals
// rint(fl(v/s)) + z exactly.  Otherwise the element takes the IEEE division.
#include "ttq_internal.h"

#pragma clang fp contract(off)

namespace ttq {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float lane_min(float v, int width) {
  for (int o = 1; o < width; o <<= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float lane_max(float v, int width) {
  for (int o = 1; o < width; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// smallest positive fp16 that is >= x (x >= 0, finite)
__device__ __forceinline__ _Float16 fp16_round_up(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  unsigned short b = __builtin_bit_cast(unsigned short, h);
  if ((float)h < x) b = (unsigned short)(b + 1);  // next fp16 up (positive values)
  if (b == 0) b = 1;                              // 2^-24, smallest positive
  return __builtin_bit_cast(_Float16, b);
}

template <int Q, int G>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(
    const _Float16* __restrict__ W, const float* __restrict__ D, int d_out, int nb,
    int64_t rows_in_flight, uint32_t* __restrict__ codes, _Float16* __restrict__ scales,
    _Float16* __restrict__ zeros) {
  constexpr int LPG = G / 32;  // lanes per group
  constexpr float N = (float)((1 << Q) - 1);
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= (int64_t)nb * rows_in_flight) return;  // whole groups leave together
  const int b = (int)(t % nb);
  const int64_t row0 = t / nb;
  const int64_t d = (int64_t)nb * 32;
  const int ng = nb / LPG;

  float sq[32];
  {
    const float4* dp = reinterpret_cast<const float4*>(D + (int64_t)b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float4 v = dp[i];
      sq[4 * i + 0] = sqrtf(v.x);
      sq[4 * i + 1] = sqrtf(v.y);
      sq[4 * i + 2] = sqrtf(v.z);
      sq[4 * i + 3] = sqrtf(v.w);
    }
  }

  for (int64_t row = row0; row < d_out; row += rows_in_flight) {
    const uint4* wp = reinterpret_cast<const uint4*>(W + row * d + (int64_t)b * 32);
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = wp[i];
    const _Float16* w = reinterpret_cast<const _Float16*>(raw);

    float v[32];
    float mn = 0.f, mx = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      v[k] = (float)w[k] * sq[k];
      mn = fminf(mn, v[k]);
      mx = fmaxf(mx, v[k]);
    }
    if constexpr (LPG > 1) {
      mn = lane_min(mn, LPG);
      mx = lane_max(mx, LPG);
    }

    float s, zf;
    _Float16 s16;
    if (mx == mn) {  // all-zero group
      s16 = (_Float16)1.0f;
      s = 1.0f;
      zf = 0.0f;
    } else {
      const float s32 = (mx - mn) / N;
      s16 = fp16_round_up(s32);
      s = (float)s16;
      zf = fminf(fmaxf(rintf(-mn / s), 0.0f), N) + 0.0f;
    }
    const float rcp = 1.0f / s;

    uint32_t word[Q];
#pragma unroll
    for (int i = 0; i < Q; ++i) word[i] = 0u;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float u = __builtin_fmaf(v[k], rcp, zf);
      float c = rintf(u);
      if (fabsf(u - c) > 0.5f - 0x1p-16f) c = rintf(v[k] / s) + zf;  // near a tie: exact path
      c = fminf(fmaxf(c, 0.0f), N);
      const uint32_t ci = (uint32_t)c;
      const int bit = Q * k;
      word[bit >> 5] |= ci << (bit & 31);
      if ((bit & 31) + Q > 32) word[(bit >> 5) + 1] |= ci >> (32 - (bit & 31));
    }

    uint32_t* cp = codes + (row * nb + b) * Q;
    if constexpr (Q == 4) {
      *reinterpret_cast<uint4*>(cp) = make_uint4(word[0], word[1], word[2], word[3]);
    } else if constexpr (Q == 2) {
      *reinterpret_cast<uint2*>(cp) = make_uint2(word[0], word[1]);
    } else {
#pragma unroll
      for (int i = 0; i < Q; ++i) cp[i] = word[i];
    }
    if ((b % LPG) == 0) {
      const int64_t gi = row * ng + b / LPG;
      scales[gi] = s16;
      zeros[gi] = (_Float16)zf;
    }
  }
}

template <int Q>
hipError_t launch_q(int d_out, int d_in, int g, const _Float16* W, const float* D, uint32_t* codes,
                    _Float16* scales, _Float16* zeros, hipStream_t s) {
  const int nb = d_in / 32;
  // rows visited per lane: about 8, so each lane's sqrt(D) work is amortised
  int64_t rows_in_flight = (d_out + 7) / 8;
  if (rows_in_flight < 1) rows_in_flight = 1;
  const int64_t threads = (int64_t)nb * rows_in_flight;
  const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
  switch (g) {
    case 32:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 32>), dim3(blocks), dim3(kThreads), 0, s, W, D,
                         d_out, nb, rows_in_flight, codes, scales, zeros);
      break;
    case 64:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 64>), dim3(blocks), dim3(kThreads), 0, s, W, D,
                         d_out, nb, rows_in_flight, codes, scales, zeros);
      break;
    default:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 128>), dim3(blocks), dim3(kThreads), 0, s, W, D,
                         d_out, nb, rows_in_flight, codes, scales, zeros);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_pack(int d_out, int d_in, int q, int g, const void* W, const float* D,
                                uint32_t* codes, void* scales, void* zeros, hipStream_t s) {
  const _Float16* w = static_cast<const _Float16*>(W);
  _Float16* sc = static_cast<_Float16*>(scales);
  _Float16* ze = static_cast<_Float16*>(zeros);
  switch (q) {
    case 2: return launch_q<2>(d_out, d_in, g, w, D, codes, sc, ze, s);
    case 3: return launch_q<3>(d_out, d_in, g, w, D, codes, sc, ze, s);
    default: return launch_q<4>(d_out, d_in, g, w, D, codes, sc, ze, s);
  }
}

}  // namespace ttq
