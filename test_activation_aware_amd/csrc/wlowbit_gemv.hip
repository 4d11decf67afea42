// The TTQ low-bit projection of a single token (decode, T = 1):
//   y = Q[(W - B A) D^(1/2)] (D^(-1/2) x) + B (A x)
// reusing the prefill's codes, scales and zeros (paper-daily.com deep
// reading, section 6: quantisation parameters computed at prefill and reused
// by the decode steps).  The group dequantisation w = s (c - z) of the
// quantiser (paper-daily.com deep reading, section 2; thelatestinai.com,
// the method section) is not formed weight by weight: per row and group,
//   sum_k s (c_k - z) xs_k = s ( sum_k (1024 + c_k) xs_k - (1024 + z) sum_k xs_k ),
// where 1024 + c is the fp16 value the unpacking makes from a code (the code
// OR-ed into the mantissa of 1024.0, exact) and xs = D^(-1/2) x in fp16.  The
// first sum is one v_dot2_f32_f16 per pair of weights (each product exact in
// fp32, fp32 accumulation), the second is precomputed per 8-channel piece of
// xs, so each pair of weights costs one unpack and one dot instruction.
//
// With one token the work is streaming the packed weight once; there is no
// matrix product to put on the matrix cores.  Layout of the work:
//   * one workgroup per 32-row tile of W (d_out / 32 workgroups), up to 16
//     waves; wave w takes a contiguous range of the tile's 64-channel steps,
//     in rounds of up to kRound steps;
//   * per round a wave requests, in order of use: its scales and zeros
//     (direct-to-LDS), its slice of the input (one 8-channel piece per lane),
//     then the codes of all the round's steps;
//   * it pre-scales its input slice into LDS (the prescale pass's arithmetic,
//     fp16(fp32(x) * D^(-1/2))) with the fp32 sum of every piece;
//   * lane l accumulates row l % 32 over the channels of its half l / 32 (the
//     lane layout of the codes), applying s and z at each group's end;
//   * the 2 x waves partial sums of a row meet in LDS and are added in a fixed
//     order (deterministic); the rank-16 term B (A x) is added in fp32.
#include <type_traits>

#include "code_unpack.h"
#include "ttq_internal.h"

namespace ttq {

namespace {

using namespace unpack;

constexpr int kMaxWaves = 16;
constexpr int kRound = 5;  // steps per wave per round

template <int Q, int G, typename TY, bool LOWRANK, typename TX>
__global__ __launch_bounds__(64 * kMaxWaves) void wlowbit_gemv_kernel(
    int d_in, int per, const _Float16* __restrict__ Xs, const TX* __restrict__ Xr,
    const float* __restrict__ dinv,
    // (codes not __restrict__: see wlowbit_decode_kernel)
    const uint32_t* codes, const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    const float* __restrict__ Bf, const float* __restrict__ Z, TY* __restrict__ Y) {
  constexpr bool FUSED = !std::is_void<TX>::value;
  constexpr int SW = 2 * Q;  // code words per row per step
  // groups a round can touch (one more when it starts inside a group), in
  // 16-byte pieces of 8 halfs, rounded up to whole 64-lane DMA instructions
  constexpr int kGroups = (kRound * 64 + G - 1) / G + 1;
  constexpr int kSzPieces = (kGroups * 4 + 63) / 64 * 64;
  __shared__ __attribute__((aligned(16))) h8 xsl[kMaxWaves][64];      // the round's pre-scaled input pieces
  __shared__ __attribute__((aligned(16))) float psl[kMaxWaves][64];   // their fp32 sums, [step][half][sub-step]
  __shared__ __attribute__((aligned(16))) _Float16 sgrp[kMaxWaves][2][kSzPieces * 8];
  __shared__ float ypart[kMaxWaves][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int nt = blockIdx.x;  // 32-row tile
  const int ksteps = d_in / 64;
  const int ng = d_in / G;

  uint32_t mask = ((1u << Q) - 1u) * 0x00010001u;  // code bits in both halves
  uint32_t magic = 0x64006400u;                    // 1024.0 in both halves
  asm volatile("" : "+v"(mask), "+v"(magic));

  const int kb = min(wave * per, ksteps), ke = min(kb + per, ksteps);
  const uint32_t* ctile = codes + (int64_t)nt * ksteps * 32 * SW + l32 * SW;
  const _Float16* stile = scales + (int64_t)nt * ng * 32;
  const _Float16* ztile = zeros + (int64_t)nt * ng * 32;
  _Float16* ssc = &sgrp[wave][0][0];
  _Float16* szr = &sgrp[wave][1][0];
  // this lane's piece of the round's input: p = lane (8 channels), whose sum
  // goes to slot 8 i + 4 half + sub-step for p = 8 i + 2 sub-step + half
  const int pslot = (lane & ~7) | ((lane & 1) << 2) | ((lane >> 1) & 3);

  float y = 0.f;   // this lane's row, over the groups finished so far
  float t = 0.f;   // sum of (1024 + c) xs over the current group
  float sx = 0.f;  // sum of xs over the current group
  int g0 = 0;
  for (int k0 = kb; k0 < ke; k0 += kRound) {
    const int nk = min(kRound, ke - k0);
    // scales and zeros of groups [g0, g1] (32 halfs each, contiguous) to LDS
    g0 = (k0 * 64) / G;
    const int g1 = ((k0 + nk) * 64 - 1) / G;
    const int pieces = (g1 - g0 + 1) * 4;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the previous round's LDS reads are done
    {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(stile + (int64_t)g0 * 32, (int64_t)pieces * 16);
      const __amdgpu_buffer_rsrc_t rz = make_rsrc(ztile + (int64_t)g0 * 32, (int64_t)pieces * 16);
#pragma unroll
      for (int j = 0; j < kSzPieces / 64; ++j) {
        const int voff = min(64 * j + lane, pieces - 1) * 16;
        lds_dma16(rs, voff, ssc + 64 * j * 8);
        lds_dma16(rz, voff, szr + 64 * j * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the input piece (clamped to the round's last piece: unconditional load)
    const int c = k0 * 64 + 8 * min(lane, nk * 8 - 1);
    XRaw<TX> xraw;
    float4 dva, dvb;
    h8 xv;
    if constexpr (FUSED) {
      xraw.load(Xr + c);
      dva = *reinterpret_cast<const float4*>(dinv + c);
      dvb = *reinterpret_cast<const float4*>(dinv + c + 4);
    } else {
      xv = *reinterpret_cast<const h8*>(Xs + c);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the codes of the round's steps, all in flight (unconditional, clamped)
    CodeStep<Q> cs[kRound];
#pragma unroll
    for (int i = 0; i < kRound; ++i) cs[i] = load_codes<Q>(ctile + (int64_t)min(k0 + i, ke - 1) * 32 * SW, hh);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FUSED) {
      float x[8];
      xraw.get(x);
      const float dv[8] = {dva.x, dva.y, dva.z, dva.w, dvb.x, dvb.y, dvb.z, dvb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = (_Float16)(x[e] * dv[e]);
      // the correction below needs the sum of exactly the stored x~: pin its
      // bits, so that the conversion is not re-selected for the sum as one
      // rounding of the product (v_fma_mixlo) where the store rounds twice
      uint4 xb = __builtin_bit_cast(uint4, xv);
      asm volatile("" : "+v"(xb.x), "+v"(xb.y), "+v"(xb.z), "+v"(xb.w));
      xv = __builtin_bit_cast(h8, xb);
    }
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ps += (float)xv[e];
    xsl[wave][lane] = xv;
    psl[wave][pslot] = ps;

#pragma unroll
    for (int i = 0; i < kRound; ++i) {
      if (i < nk) {
        const int k = k0 + i;
        const float4 ps4 = *reinterpret_cast<const float4*>(&psl[wave][8 * i + 4 * hh]);
        const float psv[4] = {ps4.x, ps4.y, ps4.z, ps4.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const h8 xp = xsl[wave][8 * i + 2 * s + hh];
          uint32_t pr[4];
          code_pairs<Q>(cs[i], s, hh, mask, magic, pr);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const h2 xpair = {xp[2 * j], xp[2 * j + 1]};
            t = __builtin_amdgcn_fdot2(as_h2(pr[j]), xpair, t, false);
          }
          sx += psv[s];
          const int ch = k * 64 + 16 * s;  // first channel of the sub-step
          if ((ch + 16) % G == 0) {        // the group ends with this sub-step
            // (scales and zeros were copied to LDS before the codes were
            // requested: reading them after this step's codes arrived)
            const int grp = ch / G - g0 + after_load(cs[i].a[0]);
            const float sv = (float)ssc[grp * 32 + l32];
            const float zv = 1024.f + (float)szr[grp * 32 + l32];
            y += sv * (t - zv * sx);
            t = 0.f;
            sx = 0.f;
          }
        }
      }
    }
  }
  if (G > 64 && ke > kb && (ke * 64) % G != 0) {
    // the range ends inside a group (G = 128, odd end step): its share of it
    const int grp = (ke * 64 - 1) / G - g0;
    const float sv = (float)ssc[grp * 32 + l32];
    const float zv = 1024.f + (float)szr[grp * 32 + l32];
    y += sv * (t - zv * sx);
  }

  // ---- the waves' partial sums, added in (wave, half) order ----
  ypart[wave][lane] = y;
  __syncthreads();
  if (wave == 0 && lane < 32) {
    float v = 0.f;
    for (int w = 0; w < nwaves; ++w) {
      v += ypart[w][lane];
      v += ypart[w][lane + 32];
    }
    const int n = nt * 32 + lane;
    if constexpr (LOWRANK) {
      const float4* bp = reinterpret_cast<const float4*>(Bf + (int64_t)n * 16);
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const float4 b = bp[j4];
        v += b.x * Z[4 * j4] + b.y * Z[4 * j4 + 1] + b.z * Z[4 * j4 + 2] + b.w * Z[4 * j4 + 3];
      }
    }
    Y[n] = (TY)v;
  }
}

// ---------------------------------------------------------------------------
// A few tokens (2 <= T <= 16): the same layout of the work on the matrix
// cores.  Per 16-channel sub-step one v_mfma_f32_32x32x16_f16 per wave, A =
// the dequantised weights of the tile (lane layout of the codes), B = 16
// channels of the wave's input slice for the T tokens (columns past T repeat
// the last token and are never stored).  The input slice of a round (T rows
// x nk steps x 64 channels, fp16) is copied into the wave's part of LDS by
// direct-to-LDS loads before the codes are requested, 16-byte pieces of a
// token's row XOR-swizzled by the token (conflict-free reads); the round's
// step count is what fits the wave's part (6 KB, 4 KB for g = 16).
// XMODE 0: the input is the pre-scaled Xs.  XMODE 1: the raw fp16 X, with
// D^(-1/2) applied to each dequantised weight pair as
// fp16(fp16((c - z) s) * fp16(d^(-1/2))), the prefill kernel's effective
// weight.  The 16 waves' 32 x 32 partial tiles meet in LDS; thread (token,
// row) adds them in wave order.
// ---------------------------------------------------------------------------
// per wave: the round's input slice (less for g = 16, whose scales and
// zeros take more room)
__host__ __device__ constexpr int fewtok_xs_bytes(int G) { return G == 16 ? 4096 : 6144; }

__host__ __device__ inline int fewtok_round(int T, int G) {
  const int kr = fewtok_xs_bytes(G) / (128 * T);  // steps of 64 channels x T tokens x 2 bytes
  return kr > kRound ? kRound : kr;
}

template <int Q, int G, typename TY, bool LOWRANK, int XMODE>
__global__ __launch_bounds__(64 * kMaxWaves) void wlowbit_fewtok_kernel(
    int T, int d_in, int per, const _Float16* X, int64_t ldx, const _Float16* __restrict__ dinv16,
    const uint32_t* codes, const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    const float* __restrict__ Bf, const float* __restrict__ Z, TY* __restrict__ Y, int64_t ldy) {
  constexpr int SW = 2 * Q;
  constexpr int kXsBytes = fewtok_xs_bytes(G);
  // groups of a round (rounds start at a group boundary unless G > 64), in
  // 16-byte pieces, rounded up to whole 64-lane DMA instructions (lanes past
  // the round's pieces copy the last one)
  constexpr int kSzPieces = (((kRound * 64 + G - 1) / G + (G > 64 ? 1 : 0)) * 4 + 63) / 64 * 64;
  constexpr int kRedBytes = kMaxWaves * 64 * 17 * 4;  // the partial tiles, lane rows padded to 17 floats
  constexpr int kXBytes = kMaxWaves * kXsBytes;
  // one LDS object for everything the direct-to-LDS loads write (the input
  // slices, then the scales and zeros, then, XMODE 1, the round's fp16
  // D^(-1/2)), per wave
  constexpr int kSgBytes = kMaxWaves * 2 * kSzPieces * 16;
  constexpr int kDvBytes = XMODE == 1 ? kMaxWaves * 1024 : 0;
  static_assert(kRedBytes <= kXBytes + kSgBytes, "the partial tiles reuse the LDS of the slices and scales");
  __shared__ __attribute__((aligned(16))) char xbuf[kXBytes + kSgBytes + kDvBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int nt = blockIdx.x;
  const int ksteps = d_in / 64;
  const int ng = d_in / G;
  const int kr = fewtok_round(T, G);

  uint32_t mask = ((1u << Q) - 1u) * 0x00010001u;
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(mask), "+v"(magic));

  const int kb = min(wave * per, ksteps), ke = min(kb + per, ksteps);
  const uint32_t* ctile = codes + (int64_t)nt * ksteps * 32 * SW + l32 * SW;
  const _Float16* stile = scales + (int64_t)nt * ng * 32;
  const _Float16* ztile = zeros + (int64_t)nt * ng * 32;
  _Float16* ssc = reinterpret_cast<_Float16*>(xbuf + kXBytes + wave * 2 * kSzPieces * 16);
  _Float16* szr = ssc + kSzPieces * 8;
  _Float16* dvw = reinterpret_cast<_Float16*>(xbuf + kXBytes + kSgBytes + (XMODE == 1 ? wave * 1024 : 0));
  char* xw = xbuf + wave * kXsBytes;
  const int tl = min(l32, T - 1);  // this lane's token column

  f16x acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  for (int k0 = kb; k0 < ke; k0 += kr) {
    const int nk = min(kr, ke - k0);
    const int rowp = nk * 8;  // 16-byte pieces per token row of the slice
    const int g0 = (k0 * 64) / G, g1 = ((k0 + nk) * 64 - 1) / G;
    const int pieces = (g1 - g0 + 1) * 4;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the previous round's LDS reads are done
    {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(stile + (int64_t)g0 * 32, (int64_t)pieces * 16);
      const __amdgpu_buffer_rsrc_t rz = make_rsrc(ztile + (int64_t)g0 * 32, (int64_t)pieces * 16);
#pragma unroll
      for (int j = 0; j < kSzPieces / 64; ++j) {
        const int voff = min(64 * j + lane, pieces - 1) * 16;
        lds_dma16(rs, voff, ssc + 64 * j * 8);
        lds_dma16(rz, voff, szr + 64 * j * 8);
      }
      if constexpr (XMODE == 1) {
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(dinv16 + (int64_t)k0 * 64, (int64_t)nk * 128);
        lds_dma16(rd, min(lane, rowp - 1) * 16, dvw);
      }
      // the input slice: slot j of the wave's part holds token t = j / rowp,
      // piece (i, c ^ (t & 7)) for j % rowp = 8 i + c (i = step of the round,
      // c = 8-channel piece of the step); slots past T rows read clamped
      // (t = j / rowp through a float reciprocal: j < 16 * 8 * kRound and
      // rowp <= 8 * kRound, so (j + 1/2) / rowp stays at least 1 / (2 rowp)
      // from an integer and the rounding error of the product is far below
      // that; byte offsets in 32 bits: t < 16 and 2 ldx < 2^23)
      const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, ((int64_t)(T - 1) * ldx + d_in) * 2);
      const int nslot = T * rowp;
      const float inv_rowp = 1.0f / (float)rowp;
      const int ldx2 = (int)(ldx * 2);
      for (int j0 = 0; j0 < nslot; j0 += 64) {
        const int j = min(j0 + lane, nslot - 1);
        const int t = (int)(((float)j + 0.5f) * inv_rowp);
        const int rem = j - t * rowp;
        const int ch = (k0 + (rem >> 3)) * 64 + 8 * ((rem & 7) ^ (t & 7));
        lds_dma16(rx, t * ldx2 + 2 * ch, xw + j0 * 16);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    CodeStep<Q> cs[kRound];
#pragma unroll
    for (int i = 0; i < kRound; ++i) cs[i] = load_codes<Q>(ctile + (int64_t)min(k0 + i, k0 + nk - 1) * 32 * SW, hh);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < kRound; ++i) {
      if (i < nk) {
        const int k = k0 + i;
        // the step's LDS reads (scales, zeros, D^(-1/2), input slice) wait for
        // its codes, which arrive after the round's direct-to-LDS copies
        const int tie = after_load(cs[i].a[0]);
        const _Float16* sst = ssc + tie;
        const _Float16* szt = szr + tie;
        const char* xwt = xw + tie;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int grp = (k * 64 + 16 * s) / G - g0;
          const _Float16 sv = sst[grp * 32 + l32];
          const _Float16 nv = (_Float16)(-1024.0f) - szt[grp * 32 + l32];  // -(1024 + z), exact
          const h2 sc = {sv, sv}, nz = {nv, nv};
          uint32_t pr[4];
          code_pairs<Q>(cs[i], s, hh, mask, magic, pr);
          h8 dv;
          if constexpr (XMODE == 1) dv = *reinterpret_cast<const h8*>(dvw + tie + i * 64 + 16 * s + 8 * hh);
          h8 a;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            h2 wv = (as_h2(pr[j]) + nz) * sc;
            if constexpr (XMODE == 1) wv = wv * h2{dv[2 * j], dv[2 * j + 1]};
            a[2 * j] = wv[0];
            a[2 * j + 1] = wv[1];
          }
          const int piece = 8 * i + ((2 * s + hh) ^ (tl & 7));
          const h8 b = *reinterpret_cast<const h8*>(xwt + (tl * rowp + piece) * 16);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
        }
      }
    }
  }

  if constexpr (LOWRANK) {
    if (wave == 0) {
      // + B Z: B (fp16) x Z split in two fp16 parts
      const int n = nt * 32 + l32;
      const float4* bp = reinterpret_cast<const float4*>(Bf + (int64_t)n * 16 + 8 * hh);
      const float4 b0 = bp[0], b1 = bp[1];
      const h8 bfr = {(_Float16)b0.x, (_Float16)b0.y, (_Float16)b0.z, (_Float16)b0.w,
                      (_Float16)b1.x, (_Float16)b1.y, (_Float16)b1.z, (_Float16)b1.w};
      const float4* zp = reinterpret_cast<const float4*>(Z + (int64_t)tl * 16 + 8 * hh);
      const float4 z0 = zp[0], z1 = zp[1];
      const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      h8 zh, zl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 hv = (_Float16)zv[e];
        zh[e] = hv;
        zl[e] = (_Float16)(zv[e] - (float)hv);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr, zh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr, zl, acc, 0, 0, 0);
    }
  }

  // ---- the waves' 32 x 32 partial tiles, added in wave order ----
  __syncthreads();  // every wave is done with its input slice
  float* red = reinterpret_cast<float*>(xbuf);
#pragma unroll
  for (int e = 0; e < 16; ++e) red[(wave * 64 + lane) * 17 + e] = acc[e];
  __syncthreads();
  // thread (token j, row i): accumulator lane j + 32 ((i / 4) % 2), value
  // (i / 8) * 4 + i % 4 of each wave
  for (int idx = threadIdx.x; idx < T * 32; idx += blockDim.x) {
    const int j = idx >> 5, i = idx & 31;
    const int src = (j + 32 * ((i >> 2) & 1)) * 17 + (i >> 3) * 4 + (i & 3);
    float v = 0.f;
    for (int w = 0; w < nwaves; ++w) v += red[w * 64 * 17 + src];
    Y[(int64_t)j * ldy + nt * 32 + i] = (TY)v;
  }
}

struct Shape {
  int nw, per;
};
Shape gemv_shape(int d_in) {
  const int ksteps = d_in / 64;
  int nw = (ksteps + kRound - 1) / kRound;
  if (nw > kMaxWaves) nw = kMaxWaves;
  if (nw < 1) nw = 1;
  return {nw, (ksteps + nw - 1) / nw};
}

template <int Q, int G, typename TY, bool LR, typename TX>
hipError_t launch_one(int d_in, int d_out, const void* Xs, const void* X, const float* dinv, const uint32_t* codes,
                      const void* scales, const void* zeros, const float* B, const float* Z, void* Y,
                      hipStream_t s) {
  const Shape sh = gemv_shape(d_in);
  hipLaunchKernelGGL((wlowbit_gemv_kernel<Q, G, TY, LR, TX>), dim3((unsigned)(d_out / 32)), dim3(64 * sh.nw), 0, s,
                     d_in, sh.per, static_cast<const _Float16*>(Xs), static_cast<const TX*>(X), dinv, codes,
                     static_cast<const _Float16*>(scales), static_cast<const _Float16*>(zeros), B, Z,
                     static_cast<TY*>(Y));
  return hipGetLastError();
}

// TX = void: the pre-scaled input Xs (any r, Y of type TY); TX = _Float16 /
// float: the raw input x and D^(-1/2) (r = 0, Y of x's type)
template <typename TY, bool LR, typename TX>
hipError_t launch_qg(int q, int g, int d_in, int d_out, const void* Xs, const void* X, const float* dinv,
                     const uint32_t* codes, const void* scales, const void* zeros, const float* B, const float* Z,
                     void* Y, hipStream_t s) {
#define TTQ_GV_G(QQ)                                                                                           \
  switch (g) {                                                                                                 \
    case 16: return launch_one<QQ, 16, TY, LR, TX>(d_in, d_out, Xs, X, dinv, codes, scales, zeros, B, Z, Y, s); \
    case 32: return launch_one<QQ, 32, TY, LR, TX>(d_in, d_out, Xs, X, dinv, codes, scales, zeros, B, Z, Y, s); \
    case 64: return launch_one<QQ, 64, TY, LR, TX>(d_in, d_out, Xs, X, dinv, codes, scales, zeros, B, Z, Y, s); \
    default: return launch_one<QQ, 128, TY, LR, TX>(d_in, d_out, Xs, X, dinv, codes, scales, zeros, B, Z, Y, s); \
  }
  switch (q) {
    case 2: TTQ_GV_G(2)
    case 3: TTQ_GV_G(3)
    case 5: TTQ_GV_G(5)
    default: TTQ_GV_G(4)
  }
#undef TTQ_GV_G
}

}  // namespace

hipError_t launch_wlowbit_fewtok(int64_t T, int d_in, int d_out, int q, int g, int r, const void* X, int64_t ldx,
                                 const void* dinv16, const uint32_t* codes, const void* scales, const void* zeros,
                                 const float* B, const float* Z, void* Y, bool y_f32, int64_t ldy, hipStream_t s) {
  if (T < 2 || T > kFewTokMaxT || (dinv16 && y_f32)) return hipErrorInvalidValue;
  const Shape sh = gemv_shape(d_in);
  const dim3 grid((unsigned)(d_out / 32)), block(64 * sh.nw);
  const _Float16* x = static_cast<const _Float16*>(X);
  const _Float16* dv = static_cast<const _Float16*>(dinv16);
  const _Float16* sc = static_cast<const _Float16*>(scales);
  const _Float16* ze = static_cast<const _Float16*>(zeros);
#define TTQ_FT(QQ, GG, TY, LR, XM)                                                                           \
  hipLaunchKernelGGL((wlowbit_fewtok_kernel<QQ, GG, TY, LR, XM>), grid, block, 0, s, (int)T, d_in, sh.per, x, ldx, \
                     dv, codes, sc, ze, B, Z, static_cast<TY*>(Y), ldy)
#define TTQ_FT_G(QQ)                                                                                           \
  switch (g) {                                                                                                 \
    case 16: TTQ_FT_FORM(QQ, 16); break;                                                                       \
    case 32: TTQ_FT_FORM(QQ, 32); break;                                                                       \
    case 64: TTQ_FT_FORM(QQ, 64); break;                                                                       \
    default: TTQ_FT_FORM(QQ, 128); break;                                                                      \
  }
#define TTQ_FT_FORM(QQ, GG)                                    \
  if (dv) {                                                    \
    if (r > 0) TTQ_FT(QQ, GG, _Float16, true, 1);              \
    else TTQ_FT(QQ, GG, _Float16, false, 1);                   \
  } else if (y_f32) {                                          \
    if (r > 0) TTQ_FT(QQ, GG, float, true, 0);                 \
    else TTQ_FT(QQ, GG, float, false, 0);                      \
  } else {                                                     \
    if (r > 0) TTQ_FT(QQ, GG, _Float16, true, 0);              \
    else TTQ_FT(QQ, GG, _Float16, false, 0);                   \
  }
  switch (q) {
    case 2: TTQ_FT_G(2) break;
    case 3: TTQ_FT_G(3) break;
    case 5: TTQ_FT_G(5) break;
    default: TTQ_FT_G(4) break;
  }
#undef TTQ_FT_FORM
#undef TTQ_FT_G
#undef TTQ_FT
  return hipGetLastError();
}

hipError_t launch_wlowbit_gemv(int d_in, int d_out, int q, int g, int r, const void* Xs, const uint32_t* codes,
                               const void* scales, const void* zeros, const float* B, const float* Z, void* Y,
                               bool y_f32, hipStream_t s) {
  if (y_f32) {
    if (r > 0) return launch_qg<float, true, void>(q, g, d_in, d_out, Xs, nullptr, nullptr, codes, scales, zeros, B, Z, Y, s);
    return launch_qg<float, false, void>(q, g, d_in, d_out, Xs, nullptr, nullptr, codes, scales, zeros, B, Z, Y, s);
  }
  if (r > 0) return launch_qg<_Float16, true, void>(q, g, d_in, d_out, Xs, nullptr, nullptr, codes, scales, zeros, B, Z, Y, s);
  return launch_qg<_Float16, false, void>(q, g, d_in, d_out, Xs, nullptr, nullptr, codes, scales, zeros, B, Z, Y, s);
}

hipError_t launch_wlowbit_gemv_raw(int d_in, int d_out, int q, int g, const void* X, bool x_f32,
                                   const float* dinvsqrt, const uint32_t* codes, const void* scales,
                                   const void* zeros, void* Y, hipStream_t s) {
  if (x_f32)
    return launch_qg<float, false, float>(q, g, d_in, d_out, nullptr, X, dinvsqrt, codes, scales, zeros, nullptr,
                                          nullptr, Y, s);
  return launch_qg<_Float16, false, _Float16>(q, g, d_in, d_out, nullptr, X, dinvsqrt, codes, scales, zeros,
                                              nullptr, nullptr, Y, s);
}

}  // namespace ttq
