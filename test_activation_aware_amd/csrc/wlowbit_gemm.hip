// ttq_wlowbit_gemm: the TTQ low-bit projection
//   Y[t][n] = sum_k V_hat[n][k] * (dinvsqrt[k] * X[t][k])  +  sum_j B[n][j] Z[t][j]
// with V_hat[n][k] = (code[n][k] - z[n][k/g]) * s[n][k/g], i.e.
//   Y = Q[(W - B A) D^(1/2)] (D^(-1/2) X) + B (A X)
// (TTQ paper: paper-daily.com deep reading, section 2, closed form
// Q[W D^(1/2)] D^(-1/2) and low-rank compensation; section 5, a custom kernel
// that fuses the pre-scaling of X).
//
// CDNA4 design (gfx950, wave64, MFMA v_mfma_f32_32x32x16_f16):
//   * A workgroup of 4 waves computes a 256 (output channels) x 128 (tokens)
//     tile of Y^T; wave w owns channels [64w, 64w + 64) x all 128 tokens as
//     2 x 4 fragments of 32x32 with fp32 accumulators.  Two workgroups fit on
//     a CU (<= 256 registers per lane, <= 54 KB LDS each), so one workgroup's
//     loads and barrier overlap the other's MFMAs.
//   * MFMA "A" = dequantised weight (rows = output channels), "B" = pre-scaled
//     input (columns = tokens): accumulator lanes hold 4 consecutive output
//     channels of one token, stored as 8 or 16 bytes.
//   * K loop in steps of 64 input channels, two LDS stages:
//       codes, scales, zeros  in the tiled storage order one step of one
//                 32-row tile is a contiguous chunk, so every wave load
//                 instruction moves 1 KB of contiguous bytes;
//       X         8 lanes per 128-byte row segment -> registers -> multiplied
//                 by D^(-1/2) in fp32 and rounded to fp16 (one v_fma_mix per
//                 element) -> LDS, in a permuted channel order with an XOR
//                 swizzle of 16-byte chunks (conflict-free both ways);
//       D^(-1/2)  64 floats per step through a two-slot LDS ring.
//     Loads for step k+1 are issued before the MFMAs of step k.
//   * Rows past T or d_out are read clamped to valid rows; a token's output
//     depends only on its own row, and padding outputs are never stored.
//   * Dequantisation in registers: code c becomes the fp16 1024 + c by OR-ing
//     the exponent bits 0x6400 (v_and_or_b32, two codes per register);
//     (1024 + c) - (1024 + z) = c - z exactly, times s gives the fp16 weight
//     with one rounding (packed fp16 add and multiply).  The OR trick pairs
//     code j with code j+4 of each 8-code group, so the X tile is stored in
//     the channel order 0 4 1 5 2 6 3 7 within every 8 channels: the MFMA
//     only needs A and B to agree on the order of the reduction.
//   * Rank-r term: before the K loop each fragment gets two extra MFMAs,
//     B16 x Z_hi and B16 x Z_lo with Z = Z_hi + Z_lo split into two fp16
//     parts, so the fp32 Z keeps about 22 bits.
//   * Workgroup ids go round-robin over the 8 XCDs; ids are regrouped so each
//     XCD gets a contiguous band of tiles, walked in groups of 4 token tiles
//     x all channel tiles, keeping the XCD's L2 on few X rows and W rows.
#include "ttq_internal.h"

namespace ttq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BN = 256;  // output channels per workgroup
constexpr int BM = 128;  // tokens per workgroup
constexpr int BK = 64;   // input channels per step
constexpr int FN = 2;    // 32-row fragments per wave
constexpr int FM = 4;    // 32-token fragments per wave
constexpr int kXcds = 8;

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// (a & m) | o in one VOP3 instruction (all operands in VGPRs)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// fp16 pair (low half of xa times da, low half of xb times db) or the high
// halves (HI = 1): one v_fma_mix per element, fp32 product rounded to fp16
template <int HI>
__device__ __forceinline__ uint32_t mix_pair(uint32_t xa, uint32_t xb, float da, float db) {
  uint32_t r;
  if constexpr (HI == 0) {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(xa), "v"(da));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "+v"(r) : "v"(xb), "v"(db));
  } else {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(xa), "v"(da));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(xb), "v"(db));
  }
  return r;
}

// The 4 code pairs (fp16 1024 + c in each half) a lane feeds to one MFMA.
// `rw` holds the row's step words as read from LDS (q = 4: this lane half's
// 4 words, one per sub-step; q = 2: the 4 words of the step; q = 3: the 6
// words of the step); s = 16-channel sub-step, hh = lane half.
template <int Q>
__device__ __forceinline__ void code_pairs(const uint32_t* rw, int s, int hh, uint32_t mask,
                                           uint32_t magic, uint32_t out[4]) {
  uint32_t u;
  if constexpr (Q == 4) {
    u = rw[s];
  } else if constexpr (Q == 2) {
    // the 8 two-bit codes of this lane half; spread its two bytes 16 bits apart
    u = __builtin_amdgcn_perm(0u, rw[s] >> (16 * hh), 0x0C010C00u);
  } else {
    const int bit = 3 * (16 * (s & 1) + 8 * hh);  // 0, 24, 48, 72 within the block
    const int w = bit >> 5, off = bit & 31;
    const uint32_t lo = rw[3 * (s >> 1) + w];
    const uint32_t hi = (w < 2) ? rw[3 * (s >> 1) + w + 1] : 0u;
    const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)off);  // 8 codes, 24 bits
    u = (win & 0xFFFu) | ((win << 4) & 0x0FFF0000u);                       // codes 4..7 to bit 16
  }
  constexpr int SH = (Q == 4) ? 4 : (Q == 3 ? 3 : 2);
  out[0] = and_or(u, mask, magic);
#pragma unroll
  for (int j = 1; j < 4; ++j) out[j] = and_or(u >> (SH * j), mask, magic);
}

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

template <int Q, int G, typename TX, bool LOWRANK>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void wlowbit_gemm_kernel(int64_t T, int d_in, int d_out, const TX* __restrict__ X, int64_t ldx,
                         const float* __restrict__ dinvsqrt, const uint32_t* __restrict__ codes,
                         const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
                         const float* __restrict__ Bf, const float* __restrict__ Z,
                         TX* __restrict__ Y, int64_t ldy, int tiles_n, int tiles) {
  constexpr int GPK = (G <= BK) ? BK / G : 1;   // groups per step
  constexpr int SW = 2 * Q;                      // code words per row per step
  constexpr int CW = 8 * 32 * SW;                // code words per step (8 row tiles)
  constexpr int SZ = 8 * GPK * 32;               // scales (and zeros) per step
  constexpr int XV = (int)sizeof(TX) / 2;        // 16-byte loads per 8 channels

  __shared__ __attribute__((aligned(16))) _Float16 xs[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint32_t cs[2][CW];
  __shared__ __attribute__((aligned(16))) _Float16 szs[2][2 * SZ];  // scales then zeros
  __shared__ __attribute__((aligned(16))) float dvs[2][BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  int tile = blockIdx.x;
  if (tiles % kXcds == 0) tile = (tile % kXcds) * (tiles / kXcds) + tile / kXcds;
  constexpr int kGroupM = 4;
  const int tiles_m = tiles / tiles_n;
  const int first_m = (tile / (kGroupM * tiles_n)) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = tile % (kGroupM * tiles_n);
  const int tm = first_m + in_group % gm, tn = in_group / gm;
  const int n0 = tn * BN;
  const int64_t m0 = (int64_t)tm * BM;
  const int ksteps = d_in / BK;
  const int ng = d_in / G;
  const int ntile0 = n0 / 32, ntiles = d_out / 32;

  uint32_t mask = (Q == 4) ? 0x000F000Fu : (Q == 3 ? 0x00070007u : 0x00030003u);  // code bits
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(mask), "+v"(magic));  // keep both in VGPRs for v_and_or_b32

  f16x acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if constexpr (LOWRANK) {
    h8 bfr[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int n = min(n0 + wave * 64 + i * 32 + l32, d_out - 1);
      const float4* bp = reinterpret_cast<const float4*>(Bf + (int64_t)n * 16 + 8 * hh);
      const float4 b0 = bp[0], b1 = bp[1];
      bfr[i][0] = (_Float16)b0.x; bfr[i][1] = (_Float16)b0.y;
      bfr[i][2] = (_Float16)b0.z; bfr[i][3] = (_Float16)b0.w;
      bfr[i][4] = (_Float16)b1.x; bfr[i][5] = (_Float16)b1.y;
      bfr[i][6] = (_Float16)b1.z; bfr[i][7] = (_Float16)b1.w;
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t t = min(m0 + j * 32 + l32, T - 1);
      const float4* zp = reinterpret_cast<const float4*>(Z + t * 16 + 8 * hh);
      const float4 z0 = zp[0], z1 = zp[1];
      const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      h8 zh, zl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 hv = (_Float16)zv[e];
        zh[e] = hv;
        zl[e] = (_Float16)(zv[e] - (float)hv);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr[i], zh, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr[i], zl, acc[i][j], 0, 0, 0);
      }
    }
  }

  // ---- X staging: thread -> 8-channel chunk xc, rows (tid >> 3) + 32u ----
  const int xc = tid & 7;
  const TX* xrow[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t t = min(m0 + (tid >> 3) + 32 * u, T - 1);
    xrow[u] = X + t * ldx + 8 * xc;
  }
  uint4 xr[4][XV];
  float4 dvr;  // D^(-1/2) of the step after next (threads < 16 keep it)

  // codes, scales and zeros of one step: 16-byte slots, slot p handled by
  // thread p % 256; registers now, LDS after the MFMAs of the current step.
  // (Copying them straight to LDS would make the compiler wait for every
  // outstanding load before the step's first LDS read.)
  constexpr int CSL = CW / 4;                        // code slots per step
  constexpr int CPT = (CSL + kThreads - 1) / kThreads;
  constexpr int SLOTS = SZ / 8;                      // slots per scales / zeros array
  static_assert(CPT <= 2, "code slots per thread");
  uint4 cr0, cr1;  // code slots tid and tid + 256 (scalars: an indexed array
                   // would be moved out of registers)
  uint4 sr;
  // Every thread issues every load (indices clamped into range) and only the
  // LDS stores are predicated: no divergent branch sits between a load and
  // its use, so the compiler's wait counts stay exact.
  auto load_w = [&](int kt) {
    // a tile's step chunk is 32 * 2Q words = 16Q slots: slot p -> row tile
    // p / 16Q, words 4 (p % 16Q) of that chunk
    {
      const int p = min(tid, CSL - 1);
      const int t = min(ntile0 + p / (16 * Q), ntiles - 1);
      cr0 = *reinterpret_cast<const uint4*>(codes + ((int64_t)t * ksteps + kt) * (32 * SW) + 4 * (p % (16 * Q)));
    }
    if constexpr (CPT > 1) {
      const int p = min(tid + kThreads, CSL - 1);
      const int t = min(ntile0 + p / (16 * Q), ntiles - 1);
      cr1 = *reinterpret_cast<const uint4*>(codes + ((int64_t)t * ksteps + kt) * (32 * SW) + 4 * (p % (16 * Q)));
    }
    const int p = min(tid, 2 * SLOTS - 1);  // slots < SLOTS: scales, then zeros
    const int arr = p / SLOTS, q8 = p % SLOTS;
    const int t = min(ntile0 + q8 / (4 * GPK), ntiles - 1);
    const int within = 8 * (q8 % (4 * GPK));  // halfs inside the tile's GPK x 32 chunk
    const int gk = (kt * BK) / G;
    sr = *reinterpret_cast<const uint4*>((arr == 0 ? scales : zeros) + ((int64_t)t * ng + gk) * 32 + within);
  };
  auto store_w = [&](int buf) {
    if (tid < CSL) *reinterpret_cast<uint4*>(&cs[buf][4 * tid]) = cr0;
    if constexpr (CPT > 1) {
      if (tid + kThreads < CSL) *reinterpret_cast<uint4*>(&cs[buf][4 * (tid + kThreads)]) = cr1;
    }
    if (tid < 2 * SLOTS) *reinterpret_cast<uint4*>(&szs[buf][8 * tid]) = sr;
  };

  auto load_x = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < XV; ++v) xr[u][v] = reinterpret_cast<const uint4*>(xrow[u] + k0)[v];
  };

  auto store_x = [&](int buf) {
    const float4 da = *reinterpret_cast<const float4*>(&dvs[buf][8 * xc]);
    const float4 db = *reinterpret_cast<const float4*>(&dvs[buf][8 * xc + 4]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = (tid >> 3) + 32 * u;
      uint32_t o[4];
      if constexpr (sizeof(TX) == 2) {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&xr[u][0]);
        // channel pairs (0,4) (1,5) (2,6) (3,7): halves of words (0,2) (0,2) (1,3) (1,3)
        o[0] = mix_pair<0>(w[0], w[2], da.x, db.x);
        o[1] = mix_pair<1>(w[0], w[2], da.y, db.y);
        o[2] = mix_pair<0>(w[1], w[3], da.z, db.z);
        o[3] = mix_pair<1>(w[1], w[3], da.w, db.w);
      } else {
        const float* e = reinterpret_cast<const float*>(&xr[u][0]);
        const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          h2 y = {(_Float16)(e[p] * dd[p]), (_Float16)(e[p + 4] * dd[p + 4])};
          o[p] = as_u32(y);
        }
      }
      *reinterpret_cast<uint4*>(&xs[buf][row * BK + ((xc ^ (row & 7)) * 8)]) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  // ---- prologue: D^(-1/2) of steps 0 and 1, stage 0 ----
  {
    const float4 d0 = reinterpret_cast<const float4*>(dinvsqrt)[tid & 15];
    dvr = reinterpret_cast<const float4*>(dinvsqrt + min(1, ksteps - 1) * BK)[tid & 15];
    if (tid < 16) *reinterpret_cast<float4*>(&dvs[0][4 * tid]) = d0;
  }
  load_w(0);
  load_x(0);
  __syncthreads();
  store_w(0);
  store_x(0);
  if (tid < 16 && ksteps > 1) *reinterpret_cast<float4*>(&dvs[1][4 * tid]) = dvr;
  __syncthreads();

  for (int kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ksteps) {
      load_w(kt + 1);
      load_x(kt + 1);
      dvr = reinterpret_cast<const float4*>(dinvsqrt + min(kt + 2, ksteps - 1) * BK)[tid & 15];
    }
    // keep the next step's LDS stores after this step's MFMAs: hoisted next to
    // their loads they would make every step wait out the load latency
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // this wave's code words and group parameters for the step
    uint32_t rw[FN][(Q == 3) ? 6 : 4];
    h2 sc[FN][GPK], nz[FN][GPK];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int tl = wave * 2 + i;  // row tile inside the workgroup
      const uint32_t* rowp = &cs[buf][(tl * 32 + l32) * SW];
      if constexpr (Q == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(rowp + 4 * hh);
        rw[i][0] = v.x; rw[i][1] = v.y; rw[i][2] = v.z; rw[i][3] = v.w;
      } else if constexpr (Q == 2) {
        const uint4 v = *reinterpret_cast<const uint4*>(rowp);
        rw[i][0] = v.x; rw[i][1] = v.y; rw[i][2] = v.z; rw[i][3] = v.w;
      } else {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const uint2 v = *reinterpret_cast<const uint2*>(rowp + 2 * k);
          rw[i][2 * k] = v.x;
          rw[i][2 * k + 1] = v.y;
        }
      }
#pragma unroll
      for (int gi = 0; gi < GPK; ++gi) {
        const _Float16 s = szs[buf][(tl * GPK + gi) * 32 + l32];
        const _Float16 z = szs[buf][SZ + (tl * GPK + gi) * 32 + l32];
        const _Float16 n = (_Float16)(-1024.0f) - z;  // -(1024 + z), exact
        sc[i][gi] = h2{s, s};
        nz[i][gi] = h2{n, n};
      }
    }

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h8 bx[FM];
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int row = j * 32 + l32;
        const int c = (2 * s + hh) ^ (row & 7);
        bx[j] = *reinterpret_cast<const h8*>(&xs[buf][row * BK + c * 8]);
      }
      const int gi = (G == 32) ? (s >> 1) : 0;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        uint32_t pr[4];
        code_pairs<Q>(rw[i], s, hh, mask, magic, pr);
        h8 a;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h2 wv = (as_h2(pr[j]) + nz[i][gi]) * sc[i][gi];
          a[2 * j] = wv[0];
          a[2 * j + 1] = wv[1];
        }
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bx[j], acc[i][j], 0, 0, 0);
      }
    }

    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < ksteps) {
      store_w(buf ^ 1);
      store_x(buf ^ 1);
      if (tid < 16 && kt + 2 < ksteps) *reinterpret_cast<float4*>(&dvs[buf][4 * tid]) = dvr;
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds token t = l32, channels 8*(e/4) + 4*hh + e%4 ----
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t t = m0 + j * 32 + l32;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int n = n0 + wave * 64 + i * 32 + 8 * e4 + 4 * hh;
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
  const int tiles_n = (d_out + BN - 1) / BN;
  const int64_t tiles_m = (T + BM - 1) / BM;
  const int64_t tiles = tiles_n * tiles_m;
  hipLaunchKernelGGL((wlowbit_gemm_kernel<Q, G, TX, LR>), dim3((unsigned)tiles), dim3(kThreads), 0, s, T,
                     d_in, d_out, static_cast<const TX*>(X), ldx, dinv, codes,
                     static_cast<const _Float16*>(scales), static_cast<const _Float16*>(zeros), B, Z,
                     static_cast<TX*>(Y), ldy, tiles_n, (int)tiles);
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
