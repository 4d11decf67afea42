// ttq_wlowbit_gemm: the TTQ low-bit projection
//   Y[t][n] = sum_k V_hat[n][k] * (dinvsqrt[k] * X[t][k])  +  sum_j B[n][j] Z[t][j]
// with V_hat[n][k] = (code[n][k] - z[n][k/g]) * s[n][k/g], i.e.
//   Y = Q[(W - B A) D^(1/2)] (D^(-1/2) X) + B (A X)
// (TTQ paper: paper-daily.com deep reading, section 2, closed form
// Q[W D^(1/2)] D^(-1/2) and low-rank compensation; section 5, a custom kernel
// that fuses the pre-scaling of X).
//
// CDNA4 design (gfx950, wave64, MFMA v_mfma_f32_32x32x16_f16):
//   * One workgroup = 4 waves computes a BN x BM tile of Y^T (BN output
//     channels x BM tokens); waves are arranged 2 x 2, each owning a
//     (BN/2) x (BM/2) sub-tile as 32x32 MFMA fragments with fp32 accumulators.
//   * The MFMA "A" operand is the dequantised weight (rows = output channels),
//     "B" is the pre-scaled input (columns = tokens).  Accumulator lanes then
//     hold 4 consecutive output channels of one token: 8- or 16-byte stores.
//   * K loop in steps of 64 input channels, double-buffered in LDS:
//       X tile    BM x 64 fp16, pre-scaled by D^(-1/2) in fp32 and rounded once
//                 to fp16 on its way from HBM to LDS (v_fma_mix), stored in a
//                 q-specific channel order (below) with an XOR swizzle of the
//                 16-byte chunks against LDS bank conflicts;
//       codes     BN rows x 2 blocks x q words, odd row stride;
//       s, z      BN rows x (64/g or 1) pairs (s, -(1024 + z)) as fp16.
//     The next step's global loads are issued before the current step's MFMAs.
//   * Dequantisation in registers: a code nibble c is turned into the fp16
//     1024 + c by OR-ing the exponent bits 0x6400, two codes per 32-bit
//     register; (1024 + c) - (1024 + z) = c - z is exact, times s gives the
//     fp16 weight with one rounding (packed fp16 add and multiply).
//   * The OR trick naturally pairs code j with code j+4 (q = 3, 4) or j+8
//     (q = 2) of the same word; the MFMA only needs A and B to agree on the
//     channel order, so the X tile is stored in that same permuted order.
//   * Rank-r term: before the K loop each fragment gets two extra MFMAs,
//     B16 x Z_hi and B16 x Z_lo, with Z = Z_hi + Z_lo split into two fp16
//     parts so the fp32 Z keeps about 22 bits.
#include "ttq_internal.h"

namespace ttq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BK = 64;

// Position p (0..15) inside a 16-channel chunk of the X tile -> channel.
template <int Q>
__device__ __forceinline__ constexpr int chunk_perm(int p) {
  const int h = p >> 3, i = p & 7;
  if constexpr (Q == 2) return 4 * h + (i >> 1) + ((i & 1) ? 8 : 0);
  else return 8 * h + (i >> 1) + ((i & 1) ? 4 : 0);
}

// The 4 code pairs a lane feeds to one MFMA, as fp16 1024 + c in each half.
// `wrow` points at the row's 2*Q words (two 32-channel blocks) in LDS;
// s = 16-channel sub-step (0..3) of the 64-channel step, hh = lane half.
template <int Q>
__device__ __forceinline__ void code_pairs(const uint32_t* wrow, int s, int hh, uint32_t out[4]) {
  const int kb = s >> 1, half = s & 1;
  if constexpr (Q == 4) {
    const uint32_t u = wrow[kb * 4 + 2 * half + hh];
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = ((u >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
  } else if constexpr (Q == 2) {
    const uint32_t u = wrow[kb * 2 + half] >> (8 * hh);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = ((u >> (2 * j)) & 0x00030003u) | 0x64006400u;
  } else {
    const int bit = 3 * (16 * half + 8 * hh);  // 0, 24, 48, 72
    const int w = bit >> 5, off = bit & 31;
    const uint32_t lo = wrow[kb * 3 + w];
    const uint32_t hi = (w < 2) ? wrow[kb * 3 + w + 1] : 0u;
    const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)off);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j] = ((win >> (3 * j)) & 7u) | (((win >> (3 * j + 12)) & 7u) << 16) | 0x64006400u;
  }
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

template <typename TX>
__device__ __forceinline__ void store4(TX* p, const float* v) {
  if constexpr (sizeof(TX) == 2) {
    h2 a = {(_Float16)v[0], (_Float16)v[1]};
    h2 b = {(_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<uint2*>(p) = make_uint2(as_u32(a), as_u32(b));
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int Q, int G, typename TX, bool LOWRANK, int BN, int BM>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void wlowbit_gemm_kernel(int64_t T, int d_in, int d_out, const TX* __restrict__ X, int64_t ldx,
                         const float* __restrict__ dinvsqrt, const uint32_t* __restrict__ codes,
                         const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
                         const float* __restrict__ Bf, const float* __restrict__ Z,
                         TX* __restrict__ Y, int64_t ldy, int tiles_n) {
  constexpr int TN = BN / 2, TM = BM / 2;  // wave sub-tile
  constexpr int FN = TN / 32, FM = TM / 32;
  constexpr int GPK = (G <= BK) ? BK / G : 1;  // groups per K step
  constexpr int WSTR = 2 * Q + 1;               // LDS words per code row (odd)
  constexpr int XU = BM * 4 / kThreads;         // 16-channel X units per thread
  constexpr int XV = 16 * (int)sizeof(TX) / 16; // 16-byte loads per unit
  static_assert(BM * 4 % kThreads == 0, "X tile split");
  static_assert(BN <= kThreads, "one code row per thread");

  __shared__ __attribute__((aligned(16))) _Float16 xs[2][BM * BK];
  __shared__ uint32_t ws[2][BN * WSTR];
  __shared__ uint32_t szs[2][BN * GPK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave >> 1, wm = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;

  const int tile = blockIdx.x;
  const int tn = tile % tiles_n, tm = tile / tiles_n;
  const int n0 = tn * BN;
  const int64_t m0 = (int64_t)tm * BM;
  const int nb = d_in / 32;
  const int ng = d_in / G;
  const int KT = d_in / BK;

  f16x acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if constexpr (LOWRANK) {
    // B (fp32 [d_out][16]) -> fp16 A operand; Z (fp32 [T][16]) -> hi/lo fp16 B operands
    h8 bfr[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int n = n0 + wn * TN + i * 32 + l32;
      const float* bp = Bf + (int64_t)min(n, d_out - 1) * 16 + 8 * hh;
#pragma unroll
      for (int e = 0; e < 8; ++e) bfr[i][e] = (_Float16)(n < d_out ? bp[e] : 0.f);
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t t = m0 + wm * TM + j * 32 + l32;
      h8 zh, zl;
      const float* zp = Z + min(t, T - 1) * 16 + 8 * hh;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zv = t < T ? zp[e] : 0.f;
        const _Float16 hv = (_Float16)zv;
        zh[e] = hv;
        zl[e] = (_Float16)(zv - (float)hv);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr[i], zh, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr[i], zl, acc[i][j], 0, 0, 0);
      }
    }
  }

  // ---- global -> register staging ----
  uint4 xr[XU][XV];
  float dv[16];
  uint32_t wr[2 * Q];
  uint32_t sr[GPK];
  const int xc = tid & 3;  // this thread's 16-channel chunk inside the 64-channel step

  auto load_stage = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int row = (tid + u * kThreads) >> 2;
      const int64_t t = m0 + row;
      const TX* src = X + min(t, T - 1) * ldx + k0 + xc * 16;
#pragma unroll
      for (int v = 0; v < XV; ++v) {
        uint4 val = reinterpret_cast<const uint4*>(src)[v];
        if (t >= T) val = make_uint4(0u, 0u, 0u, 0u);
        xr[u][v] = val;
      }
    }
    const float4* dp = reinterpret_cast<const float4*>(dinvsqrt + k0 + xc * 16);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 f = dp[v];
      dv[4 * v + 0] = f.x;
      dv[4 * v + 1] = f.y;
      dv[4 * v + 2] = f.z;
      dv[4 * v + 3] = f.w;
    }
    if (tid < BN) {
      const int n = min(n0 + tid, d_out - 1);
      const uint32_t* cp = codes + ((int64_t)n * nb + kt * 2) * Q;
#pragma unroll
      for (int i = 0; i < 2 * Q; ++i) wr[i] = cp[i];
      const int gk = (kt * BK) / G;
#pragma unroll
      for (int i = 0; i < GPK; ++i) {
        const _Float16 s = scales[(int64_t)n * ng + gk + i];
        const _Float16 z = zeros[(int64_t)n * ng + gk + i];
        h2 p = {s, (_Float16)(-((float)z + 1024.0f))};
        sr[i] = as_u32(p);
      }
    }
  };

  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int row = (tid + u * kThreads) >> 2;
      const TX* e = reinterpret_cast<const TX*>(&xr[u][0]);
      uint32_t out[8];
#pragma unroll
      for (int p = 0; p < 16; p += 2) {
        const int k0 = chunk_perm<Q>(p), k1 = chunk_perm<Q>(p + 1);
        h2 y = {(_Float16)((float)e[k0] * dv[k0]), (_Float16)((float)e[k1] * dv[k1])};
        out[p >> 1] = as_u32(y);
      }
      // two 16-byte chunks (8 channels each) at XOR-swizzled positions
      const int c0 = (2 * xc) ^ (row & 7), c1 = (2 * xc + 1) ^ (row & 7);
      *reinterpret_cast<uint4*>(&xs[buf][row * BK + c0 * 8]) = make_uint4(out[0], out[1], out[2], out[3]);
      *reinterpret_cast<uint4*>(&xs[buf][row * BK + c1 * 8]) = make_uint4(out[4], out[5], out[6], out[7]);
    }
    if (tid < BN) {
#pragma unroll
      for (int i = 0; i < 2 * Q; ++i) ws[buf][tid * WSTR + i] = wr[i];
#pragma unroll
      for (int i = 0; i < GPK; ++i) szs[buf][tid * GPK + i] = sr[i];
    }
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_stage(kt + 1);

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h8 bx[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int row = wm * TM + j * 32 + l32;
        const int c = (2 * s + hh) ^ (row & 7);
        bx[j] = *reinterpret_cast<const h8*>(&xs[buf][row * BK + c * 8]);
      }
      const int gi = (G == 32) ? (s >> 1) : 0;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int nr = wn * TN + i * 32 + l32;
        uint32_t pr[4];
        code_pairs<Q>(&ws[buf][nr * WSTR], s, hh, pr);
        const h2 sz = as_h2(szs[buf][nr * GPK + gi]);
        const h2 sc = {sz[0], sz[0]};
        const h2 nz = {sz[1], sz[1]};
        h8 a;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h2 wv = (as_h2(pr[j]) + nz) * sc;
          a[2 * j] = wv[0];
          a[2 * j + 1] = wv[1];
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bx[j], acc[i][j], 0, 0, 0);
      }
    }

    if (kt + 1 < KT) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds token t = l32, channels 8*(e/4) + 4*hh + e%4 ----
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t t = m0 + wm * TM + j * 32 + l32;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int n = n0 + wn * TN + i * 32 + 8 * e4 + 4 * hh;
        if (n < d_out) {
          float v[4] = {acc[i][j][4 * e4 + 0], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                        acc[i][j][4 * e4 + 3]};
          store4<TX>(Y + t * ldy + n, v);
        }
      }
    }
  }
}

template <int Q, int G, typename TX, bool LR>
hipError_t launch_cfg(int64_t T, int d_in, int d_out, const void* X, int64_t ldx, const float* dinv,
                      const uint32_t* codes, const void* scales, const void* zeros,
                      const float* B, const float* Z, void* Y, int64_t ldy, hipStream_t s) {
  constexpr int BN = 256, BM = 256;
  const int tiles_n = (d_out + BN - 1) / BN;
  const int64_t tiles_m = (T + BM - 1) / BM;
  const int64_t tiles = tiles_n * tiles_m;
  hipLaunchKernelGGL((wlowbit_gemm_kernel<Q, G, TX, LR, BN, BM>), dim3((unsigned)tiles), dim3(kThreads),
                     0, s, T, d_in, d_out, static_cast<const TX*>(X), ldx, dinv, codes,
                     static_cast<const _Float16*>(scales), static_cast<const _Float16*>(zeros), B, Z,
                     static_cast<TX*>(Y), ldy, tiles_n);
  return hipGetLastError();
}

template <int Q, int G, typename TX>
hipError_t launch_lr(int r, int64_t T, int d_in, int d_out, const void* X, int64_t ldx,
                     const float* dinv, const uint32_t* codes, const void* scales, const void* zeros,
                     const float* B, const float* Z, void* Y, int64_t ldy, hipStream_t s) {
  if (r > 0) return launch_cfg<Q, G, TX, true>(T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, B, Z, Y, ldy, s);
  return launch_cfg<Q, G, TX, false>(T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, B, Z, Y, ldy, s);
}

template <int Q, typename TX>
hipError_t launch_g(int g, int r, int64_t T, int d_in, int d_out, const void* X, int64_t ldx,
                    const float* dinv, const uint32_t* codes, const void* scales, const void* zeros,
                    const float* B, const float* Z, void* Y, int64_t ldy, hipStream_t s) {
  switch (g) {
    case 32: return launch_lr<Q, 32, TX>(r, T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, B, Z, Y, ldy, s);
    case 64: return launch_lr<Q, 64, TX>(r, T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, B, Z, Y, ldy, s);
    default: return launch_lr<Q, 128, TX>(r, T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, B, Z, Y, ldy, s);
  }
}

template <typename TX>
hipError_t launch_q(int q, int g, int r, int64_t T, int d_in, int d_out, const void* X, int64_t ldx,
                    const float* dinv, const uint32_t* codes, const void* scales, const void* zeros,
                    const float* B, const float* Z, void* Y, int64_t ldy, hipStream_t s) {
  switch (q) {
    case 2: return launch_g<2, TX>(g, r, T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, B, Z, Y, ldy, s);
    case 3: return launch_g<3, TX>(g, r, T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, B, Z, Y, ldy, s);
    default: return launch_g<4, TX>(g, r, T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, B, Z, Y, ldy, s);
  }
}

}  // namespace

hipError_t launch_wlowbit_gemm(int64_t T, int d_in, int d_out, int q, int g, int r, const void* X,
                               bool x_f32, int64_t ldx, const float* dinvsqrt, const uint32_t* codes,
                               const void* scales, const void* zeros, const float* B, const float* Z,
                               void* Y, int64_t ldy, hipStream_t s) {
  if (x_f32)
    return launch_q<float>(q, g, r, T, d_in, d_out, X, ldx, dinvsqrt, codes, scales, zeros, B, Z, Y, ldy, s);
  return launch_q<_Float16>(q, g, r, T, d_in, d_out, X, ldx, dinvsqrt, codes, scales, zeros, B, Z, Y, ldy, s);
}

}  // namespace ttq
