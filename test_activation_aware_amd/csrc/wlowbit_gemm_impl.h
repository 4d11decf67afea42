// ttq_wlowbit_gemm: the TTQ low-bit projection
//   Y[t][n] = sum_k V_hat[n][k] * Xs[t][k]  +  sum_j B[n][j] Z[t][j]
// with V_hat[n][k] = (code[n][k] - z[n][k/g]) * s[n][k/g], Xs = D^(-1/2) X
// (pre-scaled by the prescale pass) and Z = A X, i.e.
//   Y = Q[(W - B A) D^(1/2)] (D^(-1/2) X) + B (A X)
// (TTQ paper: paper-daily.com deep reading, section 2, closed form
// Q[W D^(1/2)] D^(-1/2) and low-rank compensation; section 5, a low-bit kernel
// that consumes the pre-scaled input).
//
// CDNA4 design (gfx950, wave64, MFMA v_mfma_f32_32x32x16_f16):
//   * A workgroup computes a 256 (output channels) x 32*FM (tokens) tile of
//     Y^T; each wave owns FN 32-row fragments x all the tokens, i.e. FN x FM
//     fragments of 32x32 (FN = 2: 4 waves, FN = 1: 8 waves).  The fp32
//     accumulators live in the accumulator registers (AGPRs).  Long prompts
//     use FM = 8 (each weight fragment dequantised once feeds 8 MFMAs): with
//     FN = 2 one workgroup per CU (256 AGPRs), with FN = 1 two waves per SIMD
//     (128 AGPRs each, one wave's dequantisation and barrier wait overlapping
//     the other's MFMAs); short ones FM = 4 (128 AGPRs, two workgroups per
//     CU).
//   * MFMA "A" = dequantised weight (rows = output channels), "B" = pre-scaled
//     input (columns = tokens): accumulator lanes hold 4 consecutive output
//     channels of one token, stored as 8 or 16 bytes.
//   * K loop in steps of 64 input channels through a three-stage LDS ring,
//     filled only by direct-to-LDS buffer loads:
//       Xs tile   32*FM rows x 128 bytes, an XOR swizzle of 16-byte chunks
//                 applied through the source addresses (conflict-free MFMA
//                 operand reads);
//       codes     one 32-row tile's step is a contiguous chunk (tiled storage
//                 order), so each wave load moves 1 KB of contiguous bytes;
//       scales and zeros of the step.
//     Step k+2 is requested while step k runs; one wait and one barrier per
//     step.  Keeping every load of the loop direct-to-LDS keeps the compiler's
//     wait counts exact: it does not order register loads against LDS DMA and
//     would otherwise wait for the whole ring before using a register load.
//     Operands of the first sub-step of step k+1 (codes, scales, X fragments)
//     are fetched and dequantised under the last MFMAs of step k, so the
//     matrix cores do not wait at step boundaries.
//   * Inside a step, each 16-channel sub-step issues its 8 MFMAs interleaved
//     with the LDS reads and the dequantisation of the next sub-step.
//   * Dequantisation in registers: code c becomes the fp16 1024 + c by OR-ing
//     the exponent bits 0x6400 (v_and_or_b32, two codes per register);
//     (1024 + c) - (1024 + z) = c - z exactly, times s gives the fp16 weight
//     with one rounding (packed fp16 add and multiply).  The OR trick pairs
//     stored slot j with slot j+4 of each 8-code group; the quantiser stores
//     the codes of channels 0 2 4 6 1 3 5 7 in slots 0..7, so every pair is
//     two neighbouring channels and the fragment comes out in the input's own
//     channel order.
//   * Rank-r term: after the K loop each fragment gets two extra MFMAs,
//     B16 x Z_hi and B16 x Z_lo with Z = Z_hi + Z_lo split into two fp16
//     parts, so the fp32 Z keeps about 22 bits (after the loop, so that their
//     operands hold no registers during it).
//   * Rows past T or d_out are read clamped to valid rows; a token's output
//     depends only on its own row, and padding outputs are never stored.
//   * fp16 outputs leave through LDS (the free X stages after the K loop) as
//     whole 512-byte token rows of the tile: stored straight from the
//     accumulators, every store instruction writes 16 bytes into each of 32
//     rows, and with all CUs finishing their tiles together those requests
//     bound the end of every round of tiles (same-box A/B at the Qwen3-32B
//     q_proj shape: 1204-1208 us against 1238-1245 us per launch).
//   * Workgroup ids go round-robin over the 8 XCDs; ids are regrouped so each
//     XCD gets a contiguous band of tiles, walked in groups of 4 token tiles
//     x all channel tiles, keeping the XCD's L2 on few X rows and W rows.
//
// This header holds the kernel template and its launch helpers; each code
// width q is instantiated in a translation unit of its own
// (wlowbit_gemm_q<q>.hip), and wlowbit_gemm.hip dispatches on q.
#pragma once

#include <type_traits>
#include <utility>

#include "wlowbit_gemm.h"

namespace ttq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
typedef uint32_t u4a __attribute__((ext_vector_type(4), aligned(4)));  // 4 words at a word boundary

constexpr int BN = 256;  // output channels per workgroup
constexpr int BK = 64;   // input channels per step
// threads of a workgroup whose waves own FN 32-row fragments each
constexpr int threads_for(int fn) { return 64 * (BN / (32 * fn)); }
constexpr int kXcds = 8;

template <int I>
using ic = std::integral_constant<int, I>;

// f(ic<0>{}), ..., f(ic<N-1>{}): every index is a compile-time constant, so
// the register arrays indexed with it never need memory.
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(ic<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// (a & m) | o in one VOP3 instruction (all operands in VGPRs)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// The code words one lane holds for one fragment and one step: q = 4, this
// lane half's 4 words (one per sub-step); q = 2, the row's 4 words; q = 3, the
// row's 6 words (words 4 and 5 in b); q = 5, words hh .. hh + 3 of each of
// the row's two 5-word blocks (a: first block, b: second).
template <int Q>
struct CodeFrag {
  u4v a;
  u2v b;
};
template <>
struct CodeFrag<5> {
  u4v a;
  u4v b;
};

__device__ __forceinline__ uint32_t code_word(const CodeFrag<3>& c, int i) {
  return i < 4 ? c.a[i] : c.b[i - 4];
}

// The 4 code pairs (fp16 1024 + c in each half) a lane feeds to one MFMA of
// sub-step S (16 channels), lane half hh.
template <int Q, int S>
__device__ __forceinline__ void code_pairs(const CodeFrag<Q>& c, int hh, uint32_t mask, uint32_t magic,
                                           uint32_t out[4]) {
  if constexpr (Q == 5) {
    // The lane half's 8 codes start at bit 80 (S & 1) + 40 hh of block S >> 1,
    // i.e. at bit 80 (S & 1) + 8 hh of the 4 words held.  lo / hi: codes 0-3
    // and 4-7 of the 8 (20 bits each, from bit 0).
    const u4v& v = (S >> 1) ? c.b : c.a;
    const uint32_t o = 8u * (uint32_t)hh;
    uint32_t lo, hi;
    if constexpr ((S & 1) == 0) {
      lo = __builtin_amdgcn_alignbit(v[1], v[0], o);
      hi = __builtin_amdgcn_alignbit(v[1], v[0], o + 20u);
    } else {
      lo = __builtin_amdgcn_alignbit(v[3], v[2], o + 16u);
      hi = v[3] >> (o + 4u);
    }
    // bytes 0-1 of lo and hi side by side: codes 0 | 4 at bit 0, 1 | 5 at bit 5;
    // bytes 1-2: codes 2 | 6 at bit 2, 3 | 7 at bit 7
    const uint32_t ua = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    const uint32_t ub = __builtin_amdgcn_perm(hi, lo, 0x06050201u);
    out[0] = and_or(ua, mask, magic);
    out[1] = and_or(ua >> 5, mask, magic);
    out[2] = and_or(ub >> 2, mask, magic);
    out[3] = and_or(ub >> 7, mask, magic);
    return;
  }
  uint32_t u;
  if constexpr (Q == 4) {
    u = c.a[S];
  } else if constexpr (Q == 2) {
    // the 8 two-bit codes of this lane half; spread its two bytes 16 bits apart
    u = __builtin_amdgcn_perm(0u, c.a[S] >> (16 * hh), 0x0C010C00u);
  } else if constexpr (Q == 3) {
    const int bit = 3 * (16 * (S & 1) + 8 * hh);  // 0, 24, 48, 72 within the block
    const int w = bit >> 5, off = bit & 31;
    const uint32_t lo = code_word(c, 3 * (S >> 1) + w);
    const uint32_t hi = (w < 2) ? code_word(c, 3 * (S >> 1) + w + 1) : 0u;
    const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)off);  // 8 codes, 24 bits
    u = (win & 0xFFFu) | ((win << 4) & 0x0FFF0000u);                       // codes 4..7 to bit 16
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

// Raw buffer resource over [base, base + bytes): loads at offsets past the
// end return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nrec = (int)min<int64_t>(bytes, (int64_t)0x7FFFFFF0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

// 16 bytes per lane from a buffer into LDS; lane l lands at
// lds_wave_base + 16 * l (the base is the same for the whole wave)
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           voff, soff, 0, 0);
}

// XOR swizzle of the 16-byte chunks of an X row in LDS: rows r and r+1 share
// a 256-byte bank window, so the pair index picks the permutation and any 16
// consecutive rows read at one logical chunk hit 16 distinct bank groups
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N of this wave's buffer loads
// (direct-to-LDS ones included) are still in flight, and its LDS reads are done
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
}

// Workgroup barrier without a memory fence (the waits above order the
// memory traffic); the empty asm statements stop the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// FM 32-token fragments per wave: FM = 8 (256 tokens per workgroup, one
// workgroup per CU, 256 accumulator registers per lane) for long prompts,
// FM = 4 (128 tokens, two workgroups per CU) for short ones.
//
// RAWX = false: Xs is the pre-scaled input D^(-1/2) X.  RAWX = true: Xs is
// the raw fp16 input X, and D^(-1/2) is applied to the weight side of the
// same product instead, V_hat D^(-1/2) (the pages' closed form
// Q[W D^(1/2)] D^(-1/2) X can be grouped either way): dvh holds
// fp16(D^(-1/2)) and each dequantised pair is multiplied by its two entries
// (one packed multiply).  The weight side is the cheap side: a weight
// fragment feeds FM MFMAs, an input fragment FN.
template <int Q, int G, typename TY, bool LOWRANK, int FM, bool RAWX, int FN>
__global__ __attribute__((amdgpu_flat_work_group_size(threads_for(FN), threads_for(FN)),
                          // FN = 2: FM = 4 aims at two workgroups per CU (the q = 5
                          // and g = 16 forms need more than the 128 registers that
                          // allows), FM = 8 takes one.  FN = 1: two waves per SIMD.
                          amdgpu_waves_per_eu((FN == 2 && (FM == 8 || Q == 5 || G == 16)) ? 1 : 2,
                                              (FN == 2 && FM == 8) ? 1 : 2)))
void wlowbit_gemm_kernel(int64_t T, int d_in, int d_out, const _Float16* __restrict__ Xs, int64_t ldxs,
                         const _Float16* __restrict__ dvh,
                         const uint32_t* __restrict__ codes, const _Float16* __restrict__ scales,
                         const _Float16* __restrict__ zeros, const float* __restrict__ Bf,
                         const float* __restrict__ Z, TY* __restrict__ Y, int64_t ldy, int tiles_n,
                         int tiles) {
  constexpr int BM = 32 * FM;                   // tokens per workgroup
  constexpr int NW = BN / (32 * FN);            // waves
  constexpr int kThreads = 64 * NW;
  constexpr int GPK = (G <= BK) ? BK / G : 1;  // groups per step
  constexpr int SW = 2 * Q;                     // code words per row per step
  constexpr int SZ = 8 * GPK * 32;              // scales (and zeros) per step
  constexpr int SLOTS = SZ / 8;                 // 16-byte slots per scales / zeros
  constexpr int XSL = BM * BK * 2 / 16;         // 16-byte slots per X tile
  constexpr int CW = 8 * 32 * SW;               // code words per step (8 row tiles)
  constexpr int CSL = CW / 4;                   // 16-byte slots of codes per step
  constexpr int CJ = (CSL + kThreads - 1) / kThreads;
  constexpr int SJ = (SLOTS + 63) / 64;         // 16-byte loads per lane of scales / zeros
  constexpr bool WIDE_S = FN * GPK > 4;         // more than 4 groups per fragment pair (g = 16)
  static_assert(XSL % kThreads == 0 && CSL % 64 == 0 && (SLOTS <= 64 || SLOTS % 64 == 0), "slot split");

  // One array per stage: an LDS read of one array does not have to wait for
  // direct-to-LDS loads still landing in another.
  __shared__ __attribute__((aligned(16))) _Float16 xs0[BM * BK], xs1[BM * BK], xs2[BM * BK];
  __shared__ __attribute__((aligned(16))) uint32_t cs0[CW], cs1[CW], cs2[CW];
  __shared__ __attribute__((aligned(16))) _Float16 sz0[2 * SZ], sz1[2 * SZ], sz2[2 * SZ];
  constexpr int DVN = RAWX ? BK : 8;  // fp16 D^(-1/2) of the step (RAWX)
  __shared__ __attribute__((aligned(16))) _Float16 dv0[DVN], dv1[DVN], dv2[DVN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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

  uint32_t mask = ((1u << Q) - 1u) * 0x00010001u;  // code bits in both halves
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(mask), "+v"(magic));  // keep both in VGPRs for v_and_or_b32
  asm volatile("; accumulators in AGPRs" ::"a"(0.0f));

  // ---- accumulators: born from MFMAs so they live in AGPRs ----
  f16x acc[FN][FM];
  f16x c0;
#pragma unroll
  for (int e = 0; e < 16; ++e) c0[e] = 0.f;
  {
    uint32_t zr = 0u;
    asm volatile("" : "+v"(zr));
    const h2 zp = as_h2(zr);
    const h8 z8 = {zp[0], zp[1], zp[0], zp[1], zp[0], zp[1], zp[0], zp[1]};
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(z8, z8, c0, 0, 0, 0);
  }

  auto xstage = [&](auto st) -> _Float16* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return xs0;
    else if constexpr (S == 1) return xs1;
    else return xs2;
  };
  auto csstage = [&](auto st) -> uint32_t* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return cs0;
    else if constexpr (S == 1) return cs1;
    else return cs2;
  };
  auto szstage = [&](auto st) -> _Float16* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return sz0;
    else if constexpr (S == 1) return sz1;
    else return sz2;
  };
  auto dvstage = [&](auto st) -> _Float16* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return dv0;
    else if constexpr (S == 1) return dv1;
    else return dv2;
  };

  // ---- requests for one step: X, codes, scales and zeros -> LDS ----
  // Only direct-to-LDS loads run inside the K loop, and one wait per step
  // (for the loads issued a step earlier) covers them all.  Per-lane byte
  // offsets are fixed; the step enters as a scalar offset.  Rows past T and
  // row tiles past d_out fall outside the resources and read as zeros (their
  // outputs are never stored).
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(Xs + m0 * ldxs, (T - m0) * ldxs * 2);
  const int64_t ctile = (int64_t)ksteps * 32 * SW;  // words per 32-row tile
  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(codes + ntile0 * ctile, (ntiles - ntile0) * ctile * 4);
  const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(scales + (int64_t)ntile0 * ng * 32, (int64_t)(ntiles - ntile0) * ng * 64);
  const __amdgpu_buffer_rsrc_t rs_z = make_rsrc(zeros + (int64_t)ntile0 * ng * 32, (int64_t)(ntiles - ntile0) * ng * 64);
  // X slot p -> row p / 8, physical chunk p % 8 holding logical chunk
  // (p % 8) ^ swz(row); slot p + 64 NW j is row + 8 NW j with the same
  // swizzle, so the per-lane offset is shared and j enters the scalar offset
  const int xrow = wave * 8 + (lane >> 3);
  const int xoff = (int)(xrow * ldxs * 2) + 16 * ((lane & 7) ^ swz(xrow));
  const int xjstride = (int)(8 * NW * ldxs * 2);
  // codes slot p -> row tile p / (16q), 16-byte piece p % (16q) of that
  // tile's contiguous step chunk
  int coff[CJ];
#pragma unroll
  for (int j = 0; j < CJ; ++j) {
    const int p = (wave + NW * j) * 64 + lane;
    coff[j] = (int)(((p / (16 * Q)) * ctile + 4 * (p % (16 * Q))) * 4);
  }
  // scales (wave 0) and zeros (wave 1): slot p = 64 j + lane < SLOTS moves
  // 8 halfs (row tile p / (4 GPK), piece p % (4 GPK) of its step)
  int soff[SJ];
#pragma unroll
  for (int j = 0; j < SJ; ++j) {
    const int p = 64 * j + lane;
    soff[j] = ((p / (4 * GPK)) * ng * 32 + 8 * (p % (4 * GPK))) * 2;
  }
  // RAWX: the step's 64 fp16 D^(-1/2) values, lanes 0-7 of wave 2
  const __amdgpu_buffer_rsrc_t rs_d = make_rsrc(dvh, RAWX ? (int64_t)d_in * 2 : 0);

  auto load_lds = [&](int kt, _Float16* xs, uint32_t* cs, _Float16* sz, _Float16* dv) {
#pragma unroll
    for (int j = 0; j < XSL / kThreads; ++j)
      lds_dma16(rs_x, xoff, kt * BK * 2 + j * xjstride, reinterpret_cast<char*>(xs) + 16 * (wave + NW * j) * 64);
#pragma unroll
    for (int j = 0; j < CJ; ++j)
      if ((wave + NW * j) * 64 < CSL) lds_dma16(rs_c, coff[j], kt * 32 * SW * 4, cs + 4 * (wave + NW * j) * 64);
#pragma unroll
    for (int j = 0; j < SJ; ++j)
      if (wave < 2 && 64 * j + lane < SLOTS)
        lds_dma16(wave == 0 ? rs_s : rs_z, soff[j], (kt * BK / G) * 32 * 2, sz + wave * SZ + 64 * 8 * j);
    if constexpr (RAWX)
      if (wave == 2 && lane < BK / 8) lds_dma16(rs_d, 16 * lane, kt * BK * 2, dv);
  };

  // ---- operands from LDS ----
  // per fragment i and group gi (k = i * GPK + gi): the scale s and
  // -(1024 + z); up to 4 groups per fragment pair share one vector (s at
  // element k, -(1024 + z) at 4 + k), 8 (g = 16) take two
  struct ScalePair {
    h8 s, nz;
  };
  using Scales = std::conditional_t<WIDE_S, ScalePair, h8>;
  auto read_scales = [&](const _Float16* sz, Scales& out) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int gi = 0; gi < GPK; ++gi) {
        const int tl = wave * FN + i;
        const _Float16 sv = sz[(tl * GPK + gi) * 32 + l32];
        const _Float16 z = sz[SZ + (tl * GPK + gi) * 32 + l32];
        const _Float16 nzv = (_Float16)(-1024.0f) - z;  // -(1024 + z), exact
        if constexpr (WIDE_S) {
          out.s[i * GPK + gi] = sv;
          out.nz[i * GPK + gi] = nzv;
        } else {
          out[i * GPK + gi] = sv;
          out[4 + i * GPK + gi] = nzv;
        }
      }
  };
  // dvp (RAWX): this lane's 8 fp16 D^(-1/2) values of the sub-step
  auto dequant = [&](auto sc_, const CodeFrag<Q>& cf, const Scales& sv, int i, const h8& dvp) -> h8 {
    constexpr int S = decltype(sc_)::value;
    constexpr int gi = (G == 16) ? S : (G == 32) ? (S >> 1) : 0;
    uint32_t pr[4];
    code_pairs<Q, S>(cf, hh, mask, magic, pr);
    h2 sc, nz;
    if constexpr (WIDE_S) {
      sc = h2{sv.s[i * GPK + gi], sv.s[i * GPK + gi]};
      nz = h2{sv.nz[i * GPK + gi], sv.nz[i * GPK + gi]};
    } else {
      sc = h2{sv[i * GPK + gi], sv[i * GPK + gi]};
      nz = h2{sv[4 + i * GPK + gi], sv[4 + i * GPK + gi]};
    }
    h8 a;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h2 wv = (as_h2(pr[j]) + nz) * sc;  // channels 2j and 2j + 1
      if constexpr (RAWX) wv = wv * h2{dvp[2 * j], dvp[2 * j + 1]};
      a[2 * j] = wv[0];
      a[2 * j + 1] = wv[1];
    }
    return a;
  };
  auto read_dv = [&](const _Float16* dv, int S) -> h8 {
    if constexpr (RAWX) return *reinterpret_cast<const h8*>(&dv[16 * S + 8 * hh]);
    else return h8{};
  };
  auto read_codes = [&](const uint32_t* cs, CodeFrag<Q>* cf) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const uint32_t* rowp = cs + ((wave * FN + i) * 32 + l32) * SW;
      if constexpr (Q == 4) {
        cf[i].a = *reinterpret_cast<const u4v*>(rowp + 4 * hh);
      } else if constexpr (Q == 2) {
        cf[i].a = *reinterpret_cast<const u4v*>(rowp);
      } else if constexpr (Q == 5) {
        cf[i].a = *reinterpret_cast<const u4a*>(rowp + hh);
        cf[i].b = *reinterpret_cast<const u4a*>(rowp + 5 + hh);
      } else {
        const u2v w01 = *reinterpret_cast<const u2v*>(rowp);
        const u2v w23 = *reinterpret_cast<const u2v*>(rowp + 2);
        cf[i].b = *reinterpret_cast<const u2v*>(rowp + 4);
        cf[i].a = u4v{w01[0], w01[1], w23[0], w23[1]};
      }
    }
  };
  auto read_b = [&](auto sc_, const _Float16* xs, int j) -> h8 {
    constexpr int S = decltype(sc_)::value;
    const int row = j * 32 + l32;
    const int c = (2 * S + hh) ^ swz(row);
    return *reinterpret_cast<const h8*>(&xs[row * BK + c * 8]);
  };

  // ---- pipeline state carried across steps ----
  // Codes: two register sets, step kt in set kt % 2, read from LDS together
  // with the scales one sub-step before the first dequantisation that needs
  // them.
  CodeFrag<Q> cset0[FN], cset1[FN];
  auto cset = [&](auto c) -> CodeFrag<Q>* {
    if constexpr (decltype(c)::value == 0) return cset0;
    else return cset1;
  };
  h8 aop[2][FN], bop[2][FM];  // operands of even / odd sub-steps
  Scales szcur, sznext;

  // ---- prologue: steps 0 and 1 requested, step 0's first operands ready ----
  load_lds(0, xs0, cs0, sz0, dv0);
  if (ksteps > 1) load_lds(1, xs1, cs1, sz1, dv1);
  wait_vmem<0>();
  block_barrier();
  read_codes(cs0, cset0);
  read_scales(sz0, szcur);
  {
    const h8 dvp = read_dv(dv0, 0);
#pragma unroll
    for (int i = 0; i < FN; ++i) aop[0][i] = dequant(ic<0>{}, cset0[i], szcur, i, dvp);
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) bop[0][j] = read_b(ic<0>{}, xs0, j);

  // ---- one K step: LDS stage ST = kt % 3, code set CS = kt % 2 ----
  auto step = [&](auto stc, auto csc, int kt) {
    constexpr int ST = decltype(stc)::value, CS = decltype(csc)::value;
    constexpr int N1 = (ST + 1) % 3, N2 = (ST + 2) % 3;
    _Float16* xcur = xstage(ic<ST>{});
    _Float16* xnext = xstage(ic<N1>{});
    if (kt + 2 < ksteps)
      load_lds(kt + 2, xstage(ic<N2>{}), csstage(ic<N2>{}), szstage(ic<N2>{}), dvstage(ic<N2>{}));
    const CodeFrag<Q>* ccur = cset(ic<CS>{});
    CodeFrag<Q>* cnext = cset(ic<CS ^ 1>{});
    unroll<4>([&](auto sc_) {
      constexpr int S = decltype(sc_)::value;
      constexpr int P = S & 1, PN = P ^ 1;
      __builtin_amdgcn_sched_barrier(0);
      // The next sub-step's operands.  After the last step these reads fetch
      // stale, in-bounds data that is never used (no branch, so the reads and
      // the dequantisation interleave with this sub-step's MFMAs).
      if constexpr (S < 3) {
#pragma unroll
        for (int j = 0; j < FM; ++j) bop[PN][j] = read_b(ic<S + 1>{}, xcur, j);
        if constexpr (S == 2) {
          read_codes(csstage(ic<N1>{}), cnext);
          read_scales(szstage(ic<N1>{}), sznext);
        }
        const h8 dvp = read_dv(dvstage(ic<ST>{}), S + 1);
#pragma unroll
        for (int i = 0; i < FN; ++i) aop[PN][i] = dequant(ic<S + 1>{}, ccur[i], szcur, i, dvp);
      } else {
#pragma unroll
        for (int j = 0; j < FM; ++j) bop[PN][j] = read_b(ic<0>{}, xnext, j);
        const h8 dvp = read_dv(dvstage(ic<N1>{}), 0);
#pragma unroll
        for (int i = 0; i < FN; ++i) aop[PN][i] = dequant(ic<0>{}, cnext[i], sznext, i, dvp);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[P][i], bop[P][j], acc[i][j], 0, 0, 0);
      // one MFMA, then an LDS read and a few VALU operations, eight times
#pragma unroll
      for (int m = 0; m < FN * FM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, (S == 2) ? 2 : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, FM == 8 ? 2 : 4, 0);
      }
    });
    szcur = sznext;
    // This wave's share of step kt+2 has landed; after the barrier every wave
    // sees all of it, and nobody reads stage ST any more.
    wait_vmem<0>();
    block_barrier();
  };

  // Unrolled by 6 = lcm(3 stages, 2 code sets).  Leaving the loop after any
  // step (rather than skipping the rest of the body) keeps every path through
  // the body in one order, so the compiler's wait counts stay exact.
  for (int kt = 0;; kt += 6) {
    step(ic<0>{}, ic<0>{}, kt);
    if (kt + 1 >= ksteps) break;
    step(ic<1>{}, ic<1>{}, kt + 1);
    if (kt + 2 >= ksteps) break;
    step(ic<2>{}, ic<0>{}, kt + 2);
    if (kt + 3 >= ksteps) break;
    step(ic<0>{}, ic<1>{}, kt + 3);
    if (kt + 4 >= ksteps) break;
    step(ic<1>{}, ic<0>{}, kt + 4);
    if (kt + 5 >= ksteps) break;
    step(ic<2>{}, ic<1>{}, kt + 5);
    if (kt + 6 >= ksteps) break;
  }

  if constexpr (LOWRANK) {
    // the rank-16 term, added after the K loop: its operands are not held in
    // registers across the loop
    h8 bfr[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int n = min(n0 + wave * 32 * FN + i * 32 + l32, d_out - 1);
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

  // ---- epilogue: lane holds token t = l32, channels 8*(e/4) + 4*hh + e%4 ----
  if constexpr (sizeof(TY) == 2) {
    // fp16 outputs leave through LDS as whole rows: stored straight from the
    // accumulators, every store instruction would write 16 bytes into each
    // of 32 token rows.  Four passes of PT = BM / 4 tokens x the 256
    // channels (fp16, 512-byte rows), alternating between stages 0 and 1 of
    // the X ring, which the last K step has left free; the 16-byte chunks of
    // row r are XOR-swizzled by r % 32 so that the accumulator writes and
    // the row reads avoid bank conflicts.
    constexpr int PT = BM / 4;           // tokens per pass
    constexpr int FPP = PT / 32;         // fragments per pass
    constexpr int RPW = PT / NW;         // rows each wave stores per pass
    static_assert(BN == 256 && PT * 512 == BM * BK * 2 && RPW % 2 == 0, "epilogue staging shape");
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      char* yb = reinterpret_cast<char*>(pass % 2 == 0 ? xs0 : xs1);
#pragma unroll
      for (int jj = 0; jj < FPP; ++jj) {
        const int j = pass * FPP + jj;
        const int r = jj * 32 + l32;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int c = (wave * FN + i) * 4 + e4;  // 16-byte chunk (8 channels) of the row
            const h2 a = {(_Float16)acc[i][j][4 * e4 + 0], (_Float16)acc[i][j][4 * e4 + 1]};
            const h2 b = {(_Float16)acc[i][j][4 * e4 + 2], (_Float16)acc[i][j][4 * e4 + 3]};
            *reinterpret_cast<uint2*>(yb + r * 512 + ((c ^ (r & 31)) * 16) + 8 * hh) = make_uint2(as_u32(a), as_u32(b));
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      block_barrier();
#pragma unroll
      for (int ii = 0; ii < RPW / 2; ++ii) {
        const int r = wave * RPW + 2 * ii + hh;
        const int c = l32;
        const uint4 v = *reinterpret_cast<const uint4*>(yb + r * 512 + ((c ^ (r & 31)) * 16));
        const int64_t t = m0 + pass * PT + r;
        const int n = n0 + 8 * c;
        if (t < T && n < d_out) *reinterpret_cast<uint4*>(Y + t * ldy + n) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t t = m0 + j * 32 + l32;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int n = n0 + wave * 32 * FN + i * 32 + 8 * e4 + 4 * hh;
        if (n < d_out) {
          float v[4] = {acc[i][j][4 * e4 + 0], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                        acc[i][j][4 * e4 + 3]};
          store4<TY>(Y + t * ldy + n, v);
        }
      }
    }
  }
}



template <int Q, int G, typename TY, bool LR, int FM, bool RAWX, int FN>
hipError_t launch_fm(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = 32 * FM;
  const int tiles_n = (a.d_out + BN - 1) / BN;
  const int64_t tiles_m = (a.T + BM - 1) / BM;
  const int64_t tiles = tiles_n * tiles_m;
  hipLaunchKernelGGL((wlowbit_gemm_kernel<Q, G, TY, LR, FM, RAWX, FN>), dim3((unsigned)tiles), dim3(threads_for(FN)), 0, s,
                     a.T, a.d_in, a.d_out, static_cast<const _Float16*>(a.X), a.ldx,
                     static_cast<const _Float16*>(a.dvh), a.codes, static_cast<const _Float16*>(a.scales),
                     static_cast<const _Float16*>(a.zeros), a.B, a.Z, static_cast<TY*>(a.Y), a.ldy, tiles_n,
                     (int)tiles);
  return hipGetLastError();
}

// 256-token tiles (one workgroup per CU at a time) when they fill whole
// rounds of the 256 CUs or make at least four rounds; otherwise 128-token
// tiles, whose twice as many workgroups even out a partial last round.
// Measured with bit-identical outputs at d = 5120, d' = 8192: T = 2048 (256
// tiles) 153-155 against 159-162 us, T = 4096 (512) 298 against 308 us,
// T = 6144 (768) 444 against 456 us, but T = 3072 (384 tiles, 1.5 rounds)
// 259 against 240 us and T = 5120 (640, 2.5 rounds) 406 against 385 us.
// With 256-token tiles, q = 2 or 4 and g >= 32, eight waves of one fragment
// each (two per SIMD: one wave's dequantisation and barrier wait overlap the
// other's MFMAs) measured 1-1.4 % faster than four waves of two and fit 128
// registers; the other forms keep four waves.
template <int Q, int G, typename TY, bool LR, bool RAWX>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles8 = ((a.d_out + BN - 1) / BN) * ((a.T + 255) / 256);
  constexpr int FN8 = ((Q == 2 || Q == 4) && G >= 32) ? 1 : 2;
  if (tiles8 >= 1024 || (tiles8 > 0 && tiles8 % 256 == 0)) return launch_fm<Q, G, TY, LR, 8, RAWX, FN8>(a, s);
  return launch_fm<Q, G, TY, LR, 4, RAWX, 2>(a, s);
}

template <int Q, int G, typename TY, bool RAWX>
hipError_t launch_lr(int r, const GemmArgs& a, hipStream_t s) {
  if (r > 0) return launch_cfg<Q, G, TY, true, RAWX>(a, s);
  return launch_cfg<Q, G, TY, false, RAWX>(a, s);
}

template <int Q, typename TY, bool RAWX>
hipError_t launch_g(int g, int r, const GemmArgs& a, hipStream_t s) {
  switch (g) {
    case 16: return launch_lr<Q, 16, TY, RAWX>(r, a, s);
    case 32: return launch_lr<Q, 32, TY, RAWX>(r, a, s);
    case 64: return launch_lr<Q, 64, TY, RAWX>(r, a, s);
    default: return launch_lr<Q, 128, TY, RAWX>(r, a, s);
  }
}

}  // namespace

template <int Q>
hipError_t launch_gemm_q(bool y_f32, bool rawx, int g, int r, const GemmArgs& a, hipStream_t s) {
  if (rawx) return launch_g<Q, _Float16, true>(g, r, a, s);
  if (y_f32) return launch_g<Q, float, false>(g, r, a, s);
  return launch_g<Q, _Float16, false>(g, r, a, s);
}

}  // namespace ttq
