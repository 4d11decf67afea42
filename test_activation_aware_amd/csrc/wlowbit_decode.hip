// The TTQ low-bit projection for decode batches of 17 to 64 tokens (one and
// up to 16 tokens have forms of their own): the same
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
//   * A wave first requests its scales and zeros (direct-to-LDS loads, read
//     per step from LDS), then the codes of up to 16 steps at once
//     (registers), and keeps the pre-scaled input of the next 2 - 4 steps in
//     flight; requests are kept in order of use, since waiting for one load
//     waits for every older one.  Per 16-channel sub-step: one
//     v_mfma_f32_32x32x16_f16 per 32 tokens, A = dequantised weights (the
//     register dequantisation of the prefill kernel), B = the pre-scaled
//     input (small; it stays in L2).
//   * The 8 partial products meet in LDS in a fixed order (deterministic) and
//     are stored as fp16 or fp32.
//   * Rank-16 term: B16 x Z_hi + B16 x Z_lo (Z split into two fp16 parts)
//     added to wave 0's accumulators.
#include <type_traits>

#include "code_unpack.h"
#include "ttq_internal.h"

namespace ttq {

namespace {

using namespace unpack;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRound = 16;  // steps whose codes a wave holds at once


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

// NF = token fragments of 32 (T <= 32 * NF); the input is the pre-scaled Xs.
template <int Q, int G, typename TY, bool LOWRANK, int NF>
__global__ __launch_bounds__(kThreads) void wlowbit_decode_kernel(
    int T, int d_in, int d_out, const _Float16* __restrict__ Xs, int64_t ldxs,
    // (codes deliberately not __restrict__: loads from a restrict read-only
    // pointer count as invariant, and the compiler then re-issues one next to
    // its use instead of keeping the early request, which waits for all)
    const uint32_t* codes, const _Float16* __restrict__ scales,
    const _Float16* __restrict__ zeros, const float* __restrict__ Bf, const float* __restrict__ Z,
    TY* __restrict__ Y, int64_t ldy) {
  constexpr int SW = 2 * Q;                     // code words per row per step
  constexpr int kXAhead = (NF == 1) ? 4 : 2;    // steps of input requested ahead of use
  // groups a round of kRound steps can touch, in 16-byte pieces of 8 halfs
  constexpr int kGroupPieces = ((kRound * 64 + 2 * G - 2) / G + 1 + 15) / 16 * 64;
  // per wave: its partial products (NF x 64 lanes x 64 bytes)
  constexpr int kWaveBuf = NF * 64 * 64;
  __shared__ __attribute__((aligned(16))) char wbuf[kWaves][kWaveBuf];
  __shared__ __attribute__((aligned(16))) _Float16 sgrp[kWaves][2][kGroupPieces * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int nt = blockIdx.x;  // 32-row tile
  const int ksteps = d_in / 64;
  const int ng = d_in / G;

  uint32_t mask = ((1u << Q) - 1u) * 0x00010001u;  // code bits in both halves
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
    // Scales and zeros go straight to LDS (direct-to-LDS buffer loads, piece p
    // of 16 bytes at slot p; slots past the round's pieces get copies of the
    // last one).  Loads into registers would be moved by the compiler behind
    // the codes, next to their use, and then waiting for them would wait for
    // every code load too.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the previous round's LDS reads are done
    {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(stile + (int64_t)g0 * 32, (int64_t)pieces * 16);
      const __amdgpu_buffer_rsrc_t rz = make_rsrc(ztile + (int64_t)g0 * 32, (int64_t)pieces * 16);
#pragma unroll
      for (int j = 0; j < SJ; ++j) {
        const int voff = min(64 * j + lane, pieces - 1) * 16;
        lds_dma16(rs, voff, ssc + 64 * j * 8);
        lds_dma16(rz, voff, szr + 64 * j * 8);
      }
    }
    // the request order is the order of use (a wait for a load waits for every
    // older one): keep the scheduler from interleaving the groups of loads
    __builtin_amdgcn_sched_barrier(0);
    // the pre-scaled input of the next kXAhead steps in flight (from L2,
    // requested before the codes)
    h8 xr[kXAhead][4][NF];
#pragma unroll
    for (int i = 0; i < kXAhead; ++i) load_x(min(k0 + i, ke - 1), xr[i]);
    __builtin_amdgcn_sched_barrier(0);
    // codes of up to kRound steps in flight at once
    CodeStep<Q> cs[kRound];
#pragma unroll
    for (int i = 0; i < kRound; ++i)  // (unconditional: a load under a branch costs a full wait)
      cs[i] = load_codes<Q>(ctile + (int64_t)min(k0 + i, ke - 1) * 32 * SW, hh);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < kRound; ++i) {
      const int k = k0 + i;
      if (i < nk) {
        const h8 (&xb)[4][NF] = xr[i % kXAhead];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          // (scales and zeros were copied to LDS before the codes were
          // requested: read after this step's codes arrived)
          const int grp = (k * 64 + 16 * s) / G - g0 + after_load(cs[i].a[0]);
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
  for (int f = 0; f < NF; ++f) reinterpret_cast<f16x*>(&wbuf[wave][0])[f * 64 + lane] = acc[f];
  __syncthreads();
  // wave w: fragment f = w / 4, the 4 consecutive accumulator values e4 = w % 4
  // (lane holds token 32 f + l32, channels 8 e4 + 4 hh + 0..3)
  const int f = wave >> 2, e4 = wave & 3;
  if (f < NF) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f16x p = reinterpret_cast<const f16x*>(&wbuf[w][0])[f * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += p[4 * e4 + e];
    }
    const int t = 32 * f + l32;
    const int n = nt * 32 + 8 * e4 + 4 * hh;
    if (t < T && n < d_out) store4<TY>(Y + (int64_t)t * ldy + n, v);
  }
}

// ---------------------------------------------------------------------------
// Split-K form for kFewTokMaxT < T <= kDecodeMaxT (r = 0, raw input).  With 32
// rows per workgroup every workgroup re-reads the whole input, T x d_in x 2
// bytes from L2 (168 MB per call at T = 64 on the Qwen3-32B shape, six times
// the packed weight).  Here workgroup (row group, split) covers 8 tiles = 256
// rows and one range of K: its 8 waves share one pre-scaled copy of that
// input slice in LDS (the input is read once per 256 rows), each wave streams
// its own tile's codes, and the split's fp32 partial products go to the
// caller's workspace.  A second kernel adds the splits in split order.  The
// splits are the K ranges of the 8-wave kernel's waves (for d_in <= 5120), so
// the result equals that kernel's bit for bit.
// ---------------------------------------------------------------------------
constexpr int kSplitPerMax = 10;               // steps per split at most
constexpr int kSplitPitch = kSplitPerMax * 64 + 8;  // fp16 per LDS input row (16-byte pad)

__host__ __device__ inline int splitk_per(int ksteps) {
  const int ks0 = max(kWaves, (ksteps + kSplitPerMax - 1) / kSplitPerMax);
  return (ksteps + ks0 - 1) / ks0;
}
// Workgroup b of a 1-D grid of groups x parts -> (group, part).  Workgroups
// are dispatched to the 8 XCDs round-robin (b % 8); when the group count is a
// multiple of 8 every part of a group lands on the XCD of the group (group %
// 8), so what the parts of a group write stays in that XCD's L2 for the
// kernel that reads it back.
struct GroupPart {
  int group, part;
};
__host__ __device__ inline GroupPart xcd_group_part(int b, int groups, int parts) {
  if (groups % 8 != 0) return {b / parts, b % parts};
  const int xcd = b % 8, j = b / 8;
  return {xcd + 8 * (j / parts), j % parts};
}

__host__ __device__ inline int splitk_count(int ksteps) {
  const int per = splitk_per(ksteps);
  return (ksteps + per - 1) / per;
}

template <int Q, int G, int NF, typename TX>
__global__ __launch_bounds__(kThreads) void wlowbit_decode_splitk_kernel(
    int T, int d_in, int d_out, const TX* Xr, int64_t ldx, const float* dinv,
    const uint32_t* codes,  // (input pointers not __restrict__: see wlowbit_decode_kernel)
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros, float* __restrict__ P) {
  constexpr int SW = 2 * Q;
  // scale / zero pieces of 16 bytes a split can touch, per wave (a multiple of 64)
  constexpr int kPieces = ((kSplitPerMax * 64 / G + 1) * 4 + 63) / 64 * 64;
  constexpr int kTokPerThread = (kDecodeMaxT + 5) / 6;  // >= 6 thread groups stage the input
  __shared__ __attribute__((aligned(16))) _Float16 xsl[kDecodeMaxT * kSplitPitch];
  __shared__ __attribute__((aligned(16))) _Float16 sgrp[kWaves][2][kPieces * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int ksteps = d_in / 64, ng = d_in / G, ntiles = d_out / 32;
  const int per = splitk_per(ksteps);
  const GroupPart gp = xcd_group_part(blockIdx.x, (ntiles + kWaves - 1) / kWaves, splitk_count(ksteps));
  const int split = gp.part;
  const int k0 = split * per, nk = min(per, ksteps - k0);  // nk >= 1
  const bool tile_ok = gp.group * kWaves + wave < ntiles;
  const int nt = min(gp.group * kWaves + wave, ntiles - 1);  // waves past the end duplicate, never store

  uint32_t mask = ((1u << Q) - 1u) * 0x00010001u;  // code bits in both halves
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(mask), "+v"(magic));

  // 1. the raw input slice and D^(-1/2), first: thread (tg, cp) takes the
  //    8-channel piece cp of rows tg, tg + ngrp, ... (clamped, unconditional)
  const int CP = nk * 8;
  const int ngrp = kThreads / CP;
  const int cp = tid % CP, tg = tid / CP;
  const int c = (k0 + cp / 8) * 64 + 8 * (cp % 8);
  const float4 da = *reinterpret_cast<const float4*>(dinv + c);
  const float4 db = *reinterpret_cast<const float4*>(dinv + c + 4);
  XRaw<TX> xraw[kTokPerThread];
#pragma unroll
  for (int j = 0; j < kTokPerThread; ++j) xraw[j].load(Xr + (int64_t)min(tg + ngrp * j, T - 1) * ldx + c);
  __builtin_amdgcn_sched_barrier(0);

  // 2. this wave's scales and zeros (groups of its tile over the split),
  //    direct to LDS
  const int g0 = (k0 * 64) / G, g1 = ((k0 + nk) * 64 - 1) / G;
  const int pieces = (g1 - g0 + 1) * 4;
  _Float16* ssc = &sgrp[wave][0][0];
  _Float16* szr = &sgrp[wave][1][0];
  {
    const _Float16* st = scales + ((int64_t)nt * ng + g0) * 32;
    const _Float16* zt = zeros + ((int64_t)nt * ng + g0) * 32;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(st, (int64_t)pieces * 16);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(zt, (int64_t)pieces * 16);
#pragma unroll
    for (int j = 0; j < kPieces / 64; ++j) {
      const int voff = min(64 * j + lane, pieces - 1) * 16;
      lds_dma16(rs, voff, ssc + 64 * j * 8);
      lds_dma16(rz, voff, szr + 64 * j * 8);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. the codes of the split's steps, all at once, with the nontemporal
  //    hint (at T = 64 on the Qwen3-32B q_proj shape 20.0-20.4 us against
  //    21.5-23.2 us per call cold, 17.9-18.9 against 19.0-20.3 warm)
  const uint32_t* ctile = codes + (int64_t)nt * ksteps * 32 * SW + l32 * SW;
  CodeStep<Q> cs[kSplitPerMax];
#pragma unroll
  for (int i = 0; i < kSplitPerMax; ++i) cs[i] = load_codes<Q, true>(ctile + (int64_t)(k0 + min(i, nk - 1)) * 32 * SW, hh);
  __builtin_amdgcn_sched_barrier(0);

  // 4. pre-scale the input slice into LDS (the prescale pass's arithmetic,
  //    channel order kept); the wait is for the input loads only
  {
    const float dv[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
    for (int j = 0; j < kTokPerThread; ++j) {
      const int t = tg + ngrp * j;
      float x[8];
      xraw[j].get(x);
      h8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (_Float16)(x[e] * dv[e]);
      // every thread stores (rows past T and threads past the groups repeat
      // a row that another thread also writes, with the same values): a
      // store under a branch would pull the loads down behind the codes
      *reinterpret_cast<h8*>(&xsl[min(t, T - 1) * kSplitPitch + 8 * cp]) = o;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // 5. per 16-channel sub-step: dequantised weights of this wave's tile times
  //    the shared input rows
  f16x acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[f][e] = 0.f;
  int xoff[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) xoff[f] = min(32 * f + l32, T - 1) * kSplitPitch + 8 * hh;
#pragma unroll
  for (int i = 0; i < kSplitPerMax; ++i) {
    if (i < nk) {
      const int k = k0 + i;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int grp = (k * 64 + 16 * s4) / G - g0 + after_load(cs[i].a[0]);
        const _Float16 sv = ssc[grp * 32 + l32];
        const _Float16 nv = (_Float16)(-1024.0f) - szr[grp * 32 + l32];  // -(1024 + z), exact
        const h2 sc = {sv, sv}, nz = {nv, nv};
        uint32_t pr[4];
        code_pairs<Q>(cs[i], s4, hh, mask, magic, pr);
        h8 a;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h2 wv = (as_h2(pr[j]) + nz) * sc;
          a[2 * j] = wv[0];
          a[2 * j + 1] = wv[1];
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const h8 xb = *reinterpret_cast<const h8*>(&xsl[xoff[f] + i * 64 + 16 * s4]);
          acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, xb, acc[f], 0, 0, 0);
        }
      }
    }
  }

  // 6. the split's partial products: P[split][t][n], fp32
  if (tile_ok) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int t = 32 * f + l32;
      if (t < T) {
        float* pr = P + ((int64_t)split * T + t) * d_out + nt * 32 + 4 * hh;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          *reinterpret_cast<float4*>(pr + 8 * e4) =
              make_float4(acc[f][4 * e4], acc[f][4 * e4 + 1], acc[f][4 * e4 + 2], acc[f][4 * e4 + 3]);
      }
    }
  }
}

// Y[t][n] = sum of the splits' partials, in split order.  Workgroup b takes
// part of the outputs of one 256-row group (kReduceParts parts per group),
// on the XCD whose L2 holds that group's partials (xcd_group_part); each
// thread adds kReduceVec float4 of outputs, every split's partial requested
// before any is added (up to 8 splits).
constexpr int kReduceParts = 8;
constexpr int kReduceThreads = 256;
template <typename TY>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(int T, int d_out, int KS,
                                                                       const float* __restrict__ P,
                                                                       TY* __restrict__ Y, int64_t ldy) {
  const int groups = (d_out / 32 + kWaves - 1) / kWaves;
  const GroupPart gp = xcd_group_part(blockIdx.x, groups, kReduceParts);
  const int n0 = gp.group * 256;                  // first row of the group
  const int rows4 = min(256, d_out - n0) / 4;     // float4 per token row of the group
  const int per = (T * rows4 + kReduceParts - 1) / kReduceParts;
  const int i0 = gp.part * per, i1 = min(i0 + per, T * rows4);
  const int64_t sstride = (int64_t)T * (d_out / 4);  // float4 between consecutive splits
  for (int i = i0 + (int)threadIdx.x; i < i1; i += kReduceThreads) {
    const int t = i / rows4, n4 = n0 / 4 + i % rows4;
    const float4* p0 = reinterpret_cast<const float4*>(P) + (int64_t)t * (d_out / 4) + n4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](const float4& p) { v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w; };
    if (KS <= 8) {
      float4 p[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) p[s] = p0[min(s, KS - 1) * sstride];
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s < KS) add(p[s]);
    } else {
      for (int s = 0; s < KS; ++s) add(p0[s * sstride]);
    }
    store4<TY>(Y + (int64_t)t * ldy + 4 * n4, v);
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
    case 16: return launch_lr<Q, 16, TY>(r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
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
    case 5: return launch_g<5, TY>(g, r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
    default: return launch_g<4, TY>(g, r, T, d_in, d_out, Xs, ldxs, codes, scales, zeros, B, Z, Y, ldy, s);
  }
}


template <int Q, int G, typename TX>
hipError_t launch_splitk_g(int T, int d_in, int d_out, const void* X, int64_t ldx, const float* dinv,
                           const uint32_t* codes, const void* scales, const void* zeros, void* Y, int64_t ldy,
                           float* P, hipStream_t s) {
  const int ksteps = d_in / 64;
  const int groups = (d_out / 32 + kWaves - 1) / kWaves, splits = splitk_count(ksteps);
  const dim3 grid((unsigned)(groups * splits));
  const TX* x = static_cast<const TX*>(X);
  const _Float16* sc = static_cast<const _Float16*>(scales);
  const _Float16* ze = static_cast<const _Float16*>(zeros);
  if (T <= 32)
    hipLaunchKernelGGL((wlowbit_decode_splitk_kernel<Q, G, 1, TX>), grid, dim3(kThreads), 0, s, T, d_in, d_out, x,
                       ldx, dinv, codes, sc, ze, P);
  else
    hipLaunchKernelGGL((wlowbit_decode_splitk_kernel<Q, G, 2, TX>), grid, dim3(kThreads), 0, s, T, d_in, d_out, x,
                       ldx, dinv, codes, sc, ze, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((splitk_reduce_kernel<TX>), dim3((unsigned)(groups * kReduceParts)), dim3(kReduceThreads), 0, s,
                     T, d_out, splits, (const float*)P, static_cast<TX*>(Y), ldy);
  return hipGetLastError();
}

template <typename TX>
hipError_t launch_splitk(int q, int g, int T, int d_in, int d_out, const void* X, int64_t ldx, const float* dinv,
                         const uint32_t* codes, const void* scales, const void* zeros, void* Y, int64_t ldy,
                         float* P, hipStream_t s) {
#define TTQ_SPLITK_G(QQ)                                                                                      \
  switch (g) {                                                                                                \
    case 16: return launch_splitk_g<QQ, 16, TX>(T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, Y, ldy, P, s); \
    case 32: return launch_splitk_g<QQ, 32, TX>(T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, Y, ldy, P, s); \
    case 64: return launch_splitk_g<QQ, 64, TX>(T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, Y, ldy, P, s); \
    default: return launch_splitk_g<QQ, 128, TX>(T, d_in, d_out, X, ldx, dinv, codes, scales, zeros, Y, ldy, P, s); \
  }
  switch (q) {
    case 2: TTQ_SPLITK_G(2)
    case 3: TTQ_SPLITK_G(3)
    case 5: TTQ_SPLITK_G(5)
    default: TTQ_SPLITK_G(4)
  }
#undef TTQ_SPLITK_G
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

size_t decode_splitk_ws_bytes(int64_t T, int d_in, int d_out) {
  if (T <= kFewTokMaxT || T > kDecodeMaxT) return 0;
  return (size_t)splitk_count(d_in / 64) * (size_t)T * (size_t)d_out * sizeof(float);
}

hipError_t launch_wlowbit_decode_splitk(int64_t T, int d_in, int d_out, int q, int g, const void* X, bool x_f32,
                                        int64_t ldx, const float* dinvsqrt, const uint32_t* codes,
                                        const void* scales, const void* zeros, void* Y, int64_t ldy,
                                        void* workspace, hipStream_t s) {
  if (T <= kFewTokMaxT || T > kDecodeMaxT) return hipErrorInvalidValue;
  float* P = static_cast<float*>(workspace);
  if (x_f32)
    return launch_splitk<float>(q, g, (int)T, d_in, d_out, X, ldx, dinvsqrt, codes, scales, zeros, Y, ldy, P, s);
  return launch_splitk<_Float16>(q, g, (int)T, d_in, d_out, X, ldx, dinvsqrt, codes, scales, zeros, Y, ldy, P, s);
}

}  // namespace ttq
