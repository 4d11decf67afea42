// The TTQ low-bit projection for few tokens (decode, T <= 64): the same
//   Y = Q[(W - B A) D^(1/2)] (D^(-1/2) X) + B (A X)
// as ttq_wlowbit_gemm, reusing the prefill's codes, scales and zeros
// (paper-daily.com deep reading, section 6: quantisation parameters computed
// at prefill and reused by the decode steps).
//
// With T <= 64 the work is streaming the packed weight once (26 MB for the
// Qwen3-32B q_proj at q = 4): the kernel is HBM-bound, so it is built for
// memory parallelism rather than for matrix-core occupancy.
//   * One workgroup of 8 waves per 32-row tile of W (d_out / 32 workgroups);
//     wave w takes a contiguous range of the tile's 64-channel steps.  The
//     tiled code layout makes a step of a tile one contiguous 1 KB chunk
//     (q = 4), so a wave's codes are one contiguous run, and its scales and
//     zeros another.
//   * A wave first requests its scales and zeros (16-byte loads, parked in
//     LDS for per-step reads), then the codes of up to 16 steps at once
//     (registers), and keeps the pre-scaled input of the next 2 - 4 steps in
//     flight.  Per 16-channel sub-step: one v_mfma_f32_32x32x16_f16 per 32
//     tokens, A = dequantised weights (the register dequantisation of the
//     prefill kernel), B = the pre-scaled input (small; it stays in L2).
//   * The 8 partial products meet in LDS in a fixed order (deterministic) and
//     are stored as fp16 or fp32.
//   * Rank-16 term: B16 x Z_hi + B16 x Z_lo (Z split into two fp16 parts)
//     added to wave 0's accumulators.
#include "ttq_internal.h"

namespace ttq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRound = 16;  // steps whose codes a wave holds at once


__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// one step's code words of this lane (see the prefill kernel): q = 4, this
// lane half's 4 words; q = 2, the row's 4 words; q = 3, the row's 6 words
struct CodeStep {
  u4v a;
  u2v b;
};

template <int Q>
__device__ __forceinline__ CodeStep load_codes(const uint32_t* p, int hh) {
  CodeStep c;
  if constexpr (Q == 4) {
    c.a = *reinterpret_cast<const u4v*>(p + 4 * hh);
  } else if constexpr (Q == 2) {
    c.a = *reinterpret_cast<const u4v*>(p);
  } else {
    const u2v w01 = *reinterpret_cast<const u2v*>(p);
    const u2v w23 = *reinterpret_cast<const u2v*>(p + 2);
    c.b = *reinterpret_cast<const u2v*>(p + 4);
    c.a = u4v{w01[0], w01[1], w23[0], w23[1]};
  }
  return c;
}

__device__ __forceinline__ uint32_t code_word(const CodeStep& c, int i) { return i < 4 ? c.a[i] : c.b[i - 4]; }

// fp16 pairs 1024 + c for sub-step s of the step, this lane half
template <int Q>
__device__ __forceinline__ void code_pairs(const CodeStep& c, int s, int hh, uint32_t mask, uint32_t magic,
                                           uint32_t out[4]) {
  uint32_t u;
  if constexpr (Q == 4) {
    u = c.a[s];
  } else if constexpr (Q == 2) {
    u = __builtin_amdgcn_perm(0u, c.a[s] >> (16 * hh), 0x0C010C00u);
  } else {
    const int bit = 3 * (16 * (s & 1) + 8 * hh);
    const int w = bit >> 5, off = bit & 31;
    const uint32_t lo = code_word(c, 3 * (s >> 1) + w);
    const uint32_t hi = (w < 2) ? code_word(c, 3 * (s >> 1) + w + 1) : 0u;
    const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)off);
    u = (win & 0xFFFu) | ((win << 4) & 0x0FFF0000u);
  }
  constexpr int SH = (Q == 4) ? 4 : (Q == 3 ? 3 : 2);
  out[0] = and_or(u, mask, magic);
#pragma unroll
  for (int j = 1; j < 4; ++j) out[j] = and_or(u >> (SH * j), mask, magic);
}

template <typename TY>
__device__ __forceinline__ void store4(TY* p, const float* v) {
  if constexpr (sizeof(TY) == 2) {
    h2 a = {(_Float16)v[0], (_Float16)v[1]};
    h2 b = {(_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<uint2*>(p) = make_uint2(as_u32(a), as_u32(b));
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// NF = token fragments of 32 (T <= 32 * NF)
template <int Q, int G, typename TY, bool LOWRANK, int NF>
__global__ __launch_bounds__(kThreads) void wlowbit_decode_kernel(
    int T, int d_in, int d_out, const _Float16* __restrict__ Xs, int64_t ldxs,
    const uint32_t* __restrict__ codes, const _Float16* __restrict__ scales,
    const _Float16* __restrict__ zeros, const float* __restrict__ Bf, const float* __restrict__ Z,
    TY* __restrict__ Y, int64_t ldy) {
  constexpr int SW = 2 * Q;                     // code words per row per step
  constexpr int kXAhead = (NF == 1) ? 4 : 2;    // steps of input requested ahead of use
  // groups a round of kRound steps can touch, in 16-byte pieces of 8 halfs
  constexpr int kGroupPieces = ((kRound * 64 + 2 * G - 2) / G + 1 + 15) / 16 * 64;
  __shared__ f16x part[kWaves][NF][64];
  __shared__ __attribute__((aligned(16))) _Float16 sgrp[kWaves][2][kGroupPieces * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int nt = blockIdx.x;  // 32-row tile
  const int ksteps = d_in / 64;
  const int ng = d_in / G;

  uint32_t mask = (Q == 4) ? 0x000F000Fu : (Q == 3 ? 0x00070007u : 0x00030003u);
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(mask), "+v"(magic));

  f16x acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[f][e] = 0.f;

  // Wave w takes the contiguous steps [kb, ke): its codes are one contiguous
  // run of (ke - kb) KB (q = 4), its scales and zeros one run of groups.
  const int per = (ksteps + kWaves - 1) / kWaves;
  const int kb = min(wave * per, ksteps), ke = min(kb + per, ksteps);
  const uint32_t* ctile = codes + (int64_t)nt * ksteps * 32 * SW + l32 * SW;
  const _Float16* stile = scales + (int64_t)nt * ng * 32;
  const _Float16* ztile = zeros + (int64_t)nt * ng * 32;
  // this lane's token rows (rows past T read row T - 1; never stored)
  const _Float16* xrow[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) xrow[f] = Xs + (int64_t)min(32 * f + l32, T - 1) * ldxs + 8 * hh;
  auto load_x = [&](int k, h8 (&xb)[4][NF]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int f = 0; f < NF; ++f) xb[s][f] = *reinterpret_cast<const h8*>(xrow[f] + k * 64 + 16 * s);
  };
  _Float16* ssc = &sgrp[wave][0][0];
  _Float16* szr = &sgrp[wave][1][0];

  for (int k0 = kb; k0 < ke; k0 += kRound) {
    const int nk = min(kRound, ke - k0);
    // Requests in the order they are needed: the round's scales and zeros
    // (groups [g0, g1] of this tile, 32 halfs each, contiguous; 16-byte
    // pieces into this wave's LDS slice), then the codes, then the input.
    const int g0 = (k0 * 64) / G, g1 = ((k0 + nk - 1) * 64 + 63) / G;
    const int pieces = (g1 - g0 + 1) * 4;
    constexpr int SJ = kGroupPieces / 64;
    uint4 sreg[SJ], zreg[SJ];
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
      const int p = min(64 * j + lane, pieces - 1);
      sreg[j] = reinterpret_cast<const uint4*>(stile + (int64_t)g0 * 32)[p];
      zreg[j] = reinterpret_cast<const uint4*>(ztile + (int64_t)g0 * 32)[p];
    }
    // codes of up to kRound steps in flight at once
    CodeStep cs[kRound];
#pragma unroll
    for (int i = 0; i < kRound; ++i) cs[i] = load_codes<Q>(ctile + (int64_t)min(k0 + i, ke - 1) * 32 * SW, hh);
    // the pre-scaled input of the next kXAhead steps in flight (it comes from
    // L2; one step of MFMAs is far shorter than an L2 round trip)
    h8 xr[kXAhead][4][NF];
#pragma unroll
    for (int i = 0; i < kXAhead; ++i) load_x(min(k0 + i, ke - 1), xr[i]);
    // scales and zeros land first: park them in LDS, where every lane finds
    // its row's values
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
      const int p = 64 * j + lane;
      if (p < pieces) {
        reinterpret_cast<uint4*>(ssc)[p] = sreg[j];
        reinterpret_cast<uint4*>(szr)[p] = zreg[j];
      }
    }
#pragma unroll
    for (int i = 0; i < kRound; ++i) {
      const int k = k0 + i;
      if (i < nk) {
        const h8 (&xb)[4][NF] = xr[i % kXAhead];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int grp = (k * 64 + 16 * s) / G - g0;
          const _Float16 sv = ssc[grp * 32 + l32];
          const _Float16 nv = (_Float16)(-1024.0f) - szr[grp * 32 + l32];  // -(1024 + z), exact
          const h2 sc = {sv, sv}, nz = {nv, nv};
          uint32_t pr[4];
          code_pairs<Q>(cs[i], s, hh, mask, magic, pr);
          h8 a;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const h2 wv = (as_h2(pr[j]) + nz) * sc;
            a[2 * j] = wv[0];
            a[2 * j + 1] = wv[1];
          }
#pragma unroll
          for (int f = 0; f < NF; ++f) acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, xb[s][f], acc[f], 0, 0, 0);
        }
        if (i + kXAhead < nk) load_x(k + kXAhead, xr[i % kXAhead]);
      }
    }
  }

  if constexpr (LOWRANK) {
    if (wave == 0) {
      const int n = min(nt * 32 + l32, d_out - 1);
      const float4* bp = reinterpret_cast<const float4*>(Bf + (int64_t)n * 16 + 8 * hh);
      const float4 b0 = bp[0], b1 = bp[1];
      const h8 bfr = {(_Float16)b0.x, (_Float16)b0.y, (_Float16)b0.z, (_Float16)b0.w,
                      (_Float16)b1.x, (_Float16)b1.y, (_Float16)b1.z, (_Float16)b1.w};
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int t = min(32 * f + l32, T - 1);
        const float4* zp = reinterpret_cast<const float4*>(Z + (int64_t)t * 16 + 8 * hh);
        const float4 z0 = zp[0], z1 = zp[1];
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        h8 zh, zl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const _Float16 hv = (_Float16)zv[e];
          zh[e] = hv;
          zl[e] = (_Float16)(zv[e] - (float)hv);
        }
        acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr, zh, acc[f], 0, 0, 0);
        acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr, zl, acc[f], 0, 0, 0);
      }
    }
  }

  // ---- the 8 waves' partial sums, added in wave order ----
#pragma unroll
  for (int f = 0; f < NF; ++f) part[wave][f][lane] = acc[f];
  __syncthreads();
  // wave w: fragment f = w / 4, the 4 consecutive accumulator values e4 = w % 4
  // (lane holds token 32 f + l32, channels 8 e4 + 4 hh + 0..3)
  const int f = wave >> 2, e4 = wave & 3;
  if (f < NF) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f16x p = part[w][f][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += p[4 * e4 + e];
    }
    const int t = 32 * f + l32;
    const int n = nt * 32 + 8 * e4 + 4 * hh;
    if (t < T && n < d_out) store4<TY>(Y + (int64_t)t * ldy + n, v);
  }
}

template <int Q, int G, typename TY, bool LR>
hipError_t launch_nf(int T, int d_in, int d_out, const void* Xs, int64_t ldxs, const uint32_t* codes,
                     const void* scales, const void* zeros, const float* B, const float* Z, void* Y,
                     int64_t ldy, hipStream_t s) {
  const dim3 grid((unsigned)(d_out / 32));
  const _Float16* xs = static_cast<const _Float16*>(Xs);
  const _Float16* sc = static_cast<const _Float16*>(scales);
  const _Float16* ze = static_cast<const _Float16*>(zeros);
  TY* y = static_cast<TY*>(Y);
  if (T <= 32)
    hipLaunchKernelGGL((wlowbit_decode_kernel<Q, G, TY, LR, 1>), grid, dim3(kThreads), 0, s, T, d_in, d_out, xs,
                       ldxs, codes, sc, ze, B, Z, y, ldy);
  else
    hipLaunchKernelGGL((wlowbit_decode_kernel<Q, G, TY, LR, 2>), grid, dim3(kThreads), 0, s, T, d_in, d_out, xs,
                       ldxs, codes, sc, ze, B, Z, y, ldy);
  return hipGetLastError();
}

template <int Q, int G, typename TY>
hipError_t launch_lr(int r, int T, int d_in, int d_out, const void* Xs, int64_t ldxs, const uint32_t* codes,
                     const void* scales, const void* zeros, const float* B, const float* Z, void* Y,
                     int64_t ldy, hipStream_t s) {
  if (r > 0) return launch_nf<Q, G, TY, true>(T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
  return launch_nf<Q, G, TY, false>(T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
}

template <int Q, typename TY>
hipError_t launch_g(int g, int r, int T, int d_in, int d_out, const void* Xs, int64_t ldxs,
                    const uint32_t* codes, const void* scales, const void* zeros, const float* B,
                    const float* Z, void* Y, int64_t ldy, hipStream_t s) {
  switch (g) {
    case 32: return launch_lr<Q, 32, TY>(r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
    case 64: return launch_lr<Q, 64, TY>(r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
    default: return launch_lr<Q, 128, TY>(r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
  }
}

template <typename TY>
hipError_t launch_q(int q, int g, int r, int T, int d_in, int d_out, const void* Xs, int64_t ldxs,
                    const uint32_t* codes, const void* scales, const void* zeros, const float* B,
                    const float* Z, void* Y, int64_t ldy, hipStream_t s) {
  switch (q) {
    case 2: return launch_g<2, TY>(g, r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
    case 3: return launch_g<3, TY>(g, r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
    default: return launch_g<4, TY>(g, r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
  }
}

}  // namespace

hipError_t launch_wlowbit_decode(int64_t T, int d_in, int d_out, int q, int g, int r, const void* Xs,
                                 int64_t ldxs, const uint32_t* codes, const void* scales, const void* zeros,
                                 const float* B, const float* Z, void* Y, bool y_f32, int64_t ldy,
                                 hipStream_t s) {
  if (T <= 0 || T > kDecodeMaxT) return hipErrorInvalidValue;
  if (y_f32)
    return launch_q<float>(q, g, r, (int)T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
  return launch_q<_Float16>(q, g, r, (int)T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
}

}  // namespace ttq
