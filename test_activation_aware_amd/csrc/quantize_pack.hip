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
// Output is in the stored format of include/ttq.h: inside every 8 channels
// the codes of channels 0 2 4 6 1 3 5 7, packed as a bitstream, words in the
// tiled order (32-row tiles, one contiguous chunk per 64-channel step).
//
// Two work splits:
//   * groups of at most 64 channels without the effective weight (the
//     default prepare): one wave per (32-row tile, 64-channel step), no
//     workgroup barrier (quantize_pack_step_kernel below; the slab arrives by
//     direct-to-LDS loads marked nontemporal, W being read once);
//   * otherwise a workgroup of 128 threads owns one 32-row tile of W over
//     128 input channels (4 blocks of 32):
//     - the 32 x 128 fp16 slab (8 KB) comes in with 16-byte loads, one full
//       row per 16 lanes, and is parked in LDS (rows padded by 16 bytes, so
//       the block reads below hit 16 distinct bank groups);
//     - thread (r, b) = (row in tile, 32-channel block) quantises its block
//       from LDS (as two groups when g = 16); groups of 64 / 128 channels
//       meet through an LDS min/max exchange;
//     - codes are placed in LDS in the tiled order and leave as one
//       contiguous store of 2 steps x 32 rows x 2q words; scales and zeros
//       likewise (all with nontemporal stores, which measured about 5 %
//       faster here).
// v = w * sq is one v_fma_mix_f32 (fp16 operand, fp32 arithmetic) and the
// codes are packed bytewise with v_cvt_pk_u8_f32.
//
// Optionally (EXPAND) the workgroup also writes the effective fp16 weight of
// its slab, W_hat[n][j] = fp16(fp16((c - z) s) * fp16(d_j^(-1/2))): the
// pages' closed form Q[W D^(1/2)] D^(-1/2) (paper-daily.com deep reading,
// section 2) with exactly the fp16 operations by which the fused projection
// kernel dequantises a weight pair ((1024 + c) - (1024 + z) is c - z exactly,
// then two packed fp16 multiplies, each rounded to nearest even), so a
// dense GEMM on W_hat gives that kernel's outputs bit for bit.  The values
// replace the slab in LDS and leave as coalesced 16-byte stores.
//
// With the rank-r factors as well (LOWRANK, r = 16), the written weight is
// fp16(W_hat + B A): Y = Q[(W - B A) D^(1/2)] D^(-1/2) X + B (A X) is
// (W_hat + B A) X, so a dense GEMM on it needs no A X.  Each wave forms the
// 32 x 64 piece of B A over its two channel blocks on the matrix cores,
// v_mfma_f32_32x32x16_f16 on fp16 hi / lo splits of both factors
// (B_hi A_hi + B_hi A_lo + B_lo A_hi, fp32 accumulation: within about 2^-21
// of B A, far inside the final fp16 rounding), and adds it to W_hat in LDS
// in fp32 before the one rounding to fp16.
//
// Codes take a reciprocal fast path.  With rcp = v_rcp_f32(s) (relative
// error at most 2^-23) and u = fma(v, rcp, z), |u - (v/s + z)| < 2^-18
// because |v/s + z| <= N + 1.  Whenever u is more than 2^-16 away from every
// half-integer, rint(u) equals rint(fl(v/s)) + z, and it lies in [0, N]
// without a clamp: v/s + z stays within [-1/2, N + 1/2] up to 2^-18, so an
// out-of-range rint needs u within 2^-18 of a half-integer.  If any element
// of a thread's block comes closer, the whole block is redone with the IEEE
// division and the clamp (rare; the fast codes of the other elements would
// have been the same).  The zero point takes the same path for -mn/s.
#include "code_unpack.h"
#include "ttq_internal.h"

#pragma clang fp contract(off)

namespace ttq {

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
constexpr int kThreads = 128;
constexpr int kCols = 128;                   // channels per workgroup
constexpr int kPR = kCols / 8;               // 16-byte pieces per slab row
constexpr int kPieces = 32 * kPR / kThreads;  // slab pieces per thread
constexpr int kRowPitch = kCols + 8;         // fp16 elements per LDS row (pad: 16 bytes)

// smallest positive fp16 that is >= x (x >= 0, finite)
__device__ __forceinline__ _Float16 fp16_round_up(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  unsigned short b = __builtin_bit_cast(unsigned short, h);
  if ((float)h < x) b = (unsigned short)(b + 1);  // next fp16 up (positive values)
  if (b == 0) b = 1;                              // 2^-24, smallest positive
  return __builtin_bit_cast(_Float16, b);
}

// fp32(h) * s for the low / high fp16 of a packed pair, one rounding: an
// fma with addend -0 equals the product, sign of zero included.
__device__ __forceinline__ float mul_lo(uint32_t pair, float s) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, -0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(s));
  return r;
}
__device__ __forceinline__ float mul_hi(uint32_t pair, float s) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, -0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(s));
  return r;
}

// an integer-valued float into byte i of acc (v_cvt_pk_u8_f32 rounds to
// nearest even and saturates to [0, 255]: exact for integers in range)
__device__ __forceinline__ uint32_t put_byte(float c, int i, uint32_t acc) {
  return __builtin_amdgcn_cvt_pk_u8_f32(c, (uint32_t)i, acc);
}

// Channel (within the 32-channel block) whose code goes to stored slot k:
// inside every 8, slots 0-3 take the even channels and slots 4-7 the odd
// ones, so that a decoder pairing slot j with slot j + 4 gets the two
// neighbouring channels 2j and 2j + 1.
__device__ __forceinline__ constexpr int slot_channel(int k) {
  return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1);
}

// position of canonical word w of block-in-step h inside a row's 2q step words
template <int Q>
__device__ __forceinline__ constexpr int step_pos(int h, int w) {
  if constexpr (Q == 4) return 4 * (w % 2) + 2 * h + w / 2;
  else return Q * h + w;
}

// Scale s (fp16, and as fp32), zero point zf and 1/s of a group from its
// range mn <= 0 <= mx.
template <int Q>
__device__ __forceinline__ void group_params(float mn, float mx, _Float16& s16, float& s, float& zf, float& rcp) {
  constexpr float N = (float)((1 << Q) - 1);
  if (mx == mn) {  // all-zero group
    s16 = (_Float16)1.0f;
    s = 1.0f;
    zf = 0.0f;
  } else {
    const float s32 = (mx - mn) / N;
    s16 = fp16_round_up(s32);
    s = (float)s16;
    // z by the same reciprocal fast path as the codes
    const float x = -mn * __builtin_amdgcn_rcpf(s);
    float zr = rintf(x);
    if (fabsf(x - zr) > 0.5f - 0x1p-16f) zr = rintf(-mn / s);
    zf = fminf(fmaxf(zr, 0.0f), N) + 0.0f;
  }
  rcp = __builtin_amdgcn_rcpf(s);
}

// code(k) gives the integer-valued float stored in slot k of a 32-channel
// block; packs the block's bitstream (slot k at bit Q*k of its Q words).
template <int Q, typename F>
__device__ __forceinline__ void pack_codes(F&& code, uint32_t word[Q]) {
  if constexpr (Q == 4) {
    // bytes of lo / hi: codes 8w+2i / 8w+2i+1; lo | hi << 4 interleaves the nibbles
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t lo = 0u, hi = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo = put_byte(code(8 * w + 2 * i), i, lo);
        hi = put_byte(code(8 * w + 2 * i + 1), i, hi);
      }
      word[w] = lo | (hi << 4);
    }
  } else if constexpr (Q == 2) {
    // byte i of part m: code 16w+4i+m; four parts at shifts 0, 2, 4, 6
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t part[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) part[m] = put_byte(code(16 * w + 4 * i + m), i, part[m]);
      word[w] = part[0] | (part[1] << 2) | (part[2] << 4) | (part[3] << 6);
    }
  } else {
#pragma unroll
    for (int i = 0; i < Q; ++i) word[i] = 0u;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      // code(k) is in [0, N] (the callers' fast path by its error bound, the
      // exact one by its clamp)
      const uint32_t ci = (uint32_t)code(k);
      const int bit = Q * k;
      word[bit >> 5] |= ci << (bit & 31);
      if ((bit & 31) + Q > 32) word[(bit >> 5) + 1] |= ci >> (32 - (bit & 31));
    }
  }
}

// The packed codes of a 32-channel block v (CPG channels per group) by the
// reciprocal fast path, the whole block redone with the IEEE division and
// the clamp when any element comes within 2^-16 of a rounding boundary.
template <int Q, int CPG>
__device__ __forceinline__ void block_codes(const float v[32], const float* s, const float* zf, const float* rcp,
                                            uint32_t word[Q]) {
  constexpr float N = (float)((1 << Q) - 1);
  float far = 0.0f;  // largest distance of u from its rounded value
  pack_codes<Q>([&](int k) {
    const int ch = slot_channel(k), sg = ch / CPG;
    const float u = __builtin_fmaf(v[ch], rcp[sg], zf[sg]);
    const float c = rintf(u);
    far = fmaxf(far, fabsf(u - c));
    return c;
  }, word);
  if (far > 0.5f - 0x1p-16f)  // rare
    pack_codes<Q>([&](int k) {
      const int ch = slot_channel(k), sg = ch / CPG;
      return fminf(fmaxf(rintf(v[ch] / s[sg]) + zf[sg], 0.0f), N);
    }, word);
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));

template <int Q, int G, bool EXPAND, bool LOWRANK>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(
    const _Float16* __restrict__ W, const float* __restrict__ D, int d_in,
    uint32_t* __restrict__ codes, _Float16* __restrict__ scales, _Float16* __restrict__ zeros,
    const _Float16* __restrict__ dinv16, _Float16* __restrict__ wexp, const float* __restrict__ Bf,
    const float* __restrict__ Af) {
  static_assert(EXPAND || !LOWRANK, "the low-rank term is folded into the effective weight only");
  constexpr int LPG = G >= 32 ? G / 32 : 1;  // blocks per group
  constexpr int SG = G < 32 ? 32 / G : 1;     // groups inside one block (g = 16: 2)
  constexpr int CPG = 32 / SG;                // channels of the block per such group
  constexpr float N = (float)((1 << Q) - 1);
  constexpr int SW = 2 * Q;                 // words per row per 64-channel step
  constexpr int GPW = kCols / G;            // groups per workgroup column range

  __shared__ __attribute__((aligned(16))) _Float16 wt[32 * kRowPitch];
  __shared__ __attribute__((aligned(16))) float sq[kCols];
  __shared__ __attribute__((aligned(16))) uint32_t outc[kCols / 64 * 32 * SW];
  __shared__ __attribute__((aligned(16))) _Float16 outs[GPW * 32], outz[GPW * 32];
  __shared__ float red_mn[kCols / 32][32], red_mx[kCols / 32][32];

  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * kCols;
  const int width = min(kCols, d_in - c0);  // 64 or 128
  const int nt = blockIdx.y;                // row tile

  // D of this workgroup's channels, then the slab (piece p -> row p / kPR,
  // column 8 (p % kPR)).  All loads are unconditional, with columns past the
  // range clamped to its last piece (their LDS copies are never read): a load
  // under a branch made the compiler wait for it before issuing the next one.
  const float dj = D[c0 + min(tid, width - 1)];
  uint4 pre[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int p = tid + i * kThreads;
    const int row = p / kPR, col = min((p % kPR) * 8, width - 8);
    pre[i] = *reinterpret_cast<const uint4*>(W + (int64_t)(nt * 32 + row) * d_in + c0 + col);
  }
  // sqrt(D), correctly rounded
  sq[tid] = sqrtf(dj);
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int p = tid + i * kThreads;
    const int row = p / kPR, col = (p % kPR) * 8;
    *reinterpret_cast<uint4*>(&wt[row * kRowPitch + col]) = pre[i];
  }
  __syncthreads();

  // this thread's block: r = row in tile, bl = block in the column range
  const int r = tid & 31, bl = tid >> 5;
  const bool active = 32 * bl < width;
  const int h = bl & 1, ksl = bl >> 1;

  float v[32];
  float mn[SG], mx[SG];
#pragma unroll
  for (int sg = 0; sg < SG; ++sg) mn[sg] = mx[sg] = 0.f;
  if (active) {
    const _Float16* src = &wt[r * kRowPitch + bl * 32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * i);
      const float4 sa = *reinterpret_cast<const float4*>(&sq[bl * 32 + 8 * i]);
      const float4 sb = *reinterpret_cast<const float4*>(&sq[bl * 32 + 8 * i + 4]);
      float* o = &v[8 * i];
      o[0] = mul_lo(raw.x, sa.x); o[1] = mul_hi(raw.x, sa.y);
      o[2] = mul_lo(raw.y, sa.z); o[3] = mul_hi(raw.y, sa.w);
      o[4] = mul_lo(raw.z, sb.x); o[5] = mul_hi(raw.z, sb.y);
      o[6] = mul_lo(raw.w, sb.z); o[7] = mul_hi(raw.w, sb.w);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        mn[(8 * i + k) / CPG] = fminf(mn[(8 * i + k) / CPG], o[k]);
        mx[(8 * i + k) / CPG] = fmaxf(mx[(8 * i + k) / CPG], o[k]);
      }
    }
  }
  if constexpr (LPG > 1) {
    red_mn[bl][r] = mn[0];
    red_mx[bl][r] = mx[0];
    __syncthreads();
    const int first = bl & ~(LPG - 1);
#pragma unroll
    for (int j = 0; j < LPG; ++j) {
      mn[0] = fminf(mn[0], red_mn[first + j][r]);
      mx[0] = fmaxf(mx[0], red_mx[first + j][r]);
    }
  }

  if (active) {
    // per group of the block: scale s, zero point zf, 1/s
    float s[SG], zf[SG], rcp[SG];
    _Float16 s16[SG];
#pragma unroll
    for (int sg = 0; sg < SG; ++sg) group_params<Q>(mn[sg], mx[sg], s16[sg], s[sg], zf[sg], rcp[sg]);

    uint32_t word[Q];
    if constexpr (!EXPAND) {
      block_codes<Q, CPG>(v, s, zf, rcp, word);
    } else {
      float far = 0.0f;  // largest distance of u from its rounded value
      // the codes replace v in place (the rare exact path rereads the slab)
#pragma unroll
      for (int ch = 0; ch < 32; ++ch) {
        const int sg = ch / CPG;
        const float u = __builtin_fmaf(v[ch], rcp[sg], zf[sg]);
        v[ch] = rintf(u);
        far = fmaxf(far, fabsf(u - v[ch]));
      }
      if (far > 0.5f - 0x1p-16f) {
        const _Float16* src = &wt[r * kRowPitch + bl * 32];
#pragma unroll
        for (int ch = 0; ch < 32; ch += 2) {
          const uint32_t raw = *reinterpret_cast<const uint32_t*>(src + ch);
          const int sg = ch / CPG;
          v[ch] = fminf(fmaxf(rintf(mul_lo(raw, sq[bl * 32 + ch]) / s[sg]) + zf[sg], 0.0f), N);
          v[ch + 1] = fminf(fmaxf(rintf(mul_hi(raw, sq[bl * 32 + ch + 1]) / s[sg]) + zf[sg], 0.0f), N);
        }
      }
      pack_codes<Q>([&](int k) { return v[slot_channel(k)]; }, word);
    }
    if constexpr (EXPAND) {
      // W_hat of the block, in place of its slab in LDS (this thread's own
      // row segment: no other thread reads it)
      _Float16* dst16 = &wt[r * kRowPitch + bl * 32];
#pragma unroll
      for (int ch = 0; ch < 32; ch += 8) {
        const uint4 dv = *reinterpret_cast<const uint4*>(dinv16 + c0 + bl * 32 + ch);
        const uint32_t dvw[4] = {dv.x, dv.y, dv.z, dv.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sg = (ch + 2 * e) / CPG;
          const h2 cz = {(_Float16)(v[ch + 2 * e] - zf[sg]), (_Float16)(v[ch + 2 * e + 1] - zf[sg])};
          h2 wv = cz * h2{s16[sg], s16[sg]};
          wv = wv * __builtin_bit_cast(h2, dvw[e]);
          o[e] = __builtin_bit_cast(uint32_t, wv);
        }
        *reinterpret_cast<uint4*>(dst16 + ch) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    uint32_t* dst = &outc[(ksl * 32 + r) * SW];
#pragma unroll
    for (int w = 0; w < Q; ++w) dst[step_pos<Q>(h, w)] = word[w];
    if constexpr (SG > 1) {
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        outs[(bl * SG + sg) * 32 + r] = s16[sg];
        outz[(bl * SG + sg) * 32 + r] = (_Float16)zf[sg];
      }
    } else if ((bl % LPG) == 0) {
      outs[(bl / LPG) * 32 + r] = s16[0];
      outz[(bl / LPG) * 32 + r] = (_Float16)zf[0];
    }
  }
  // LOWRANK: this lane's operands of its wave's B A piece, loaded once the
  // quantisation no longer holds its registers.  Lane l (row l32 of the
  // tile, factor half hh) holds B[row][8 hh .. 8 hh + 7] and, for each of the
  // wave's two 32-channel blocks, A[8 hh .. 8 hh + 7][channel l32] (channels
  // past the range clamped; their results are never used).
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  float4 bq[2];
  float av[2][8];
  if constexpr (LOWRANK) {
    const float4* bp = reinterpret_cast<const float4*>(Bf + (int64_t)(nt * 32 + l32) * 16 + 8 * hh);
    bq[0] = bp[0];
    bq[1] = bp[1];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int col = c0 + min(64 * wave + 32 * blk + l32, width - 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) av[blk][e] = Af[(int64_t)(8 * hh + e) * d_in + col];
    }
  }
  __syncthreads();

  if constexpr (LOWRANK) {
    // W_hat + B A over the wave's two blocks (the wave wrote W_hat of exactly
    // these; the barrier above ordered those writes for the other lanes)
    if (64 * wave < width) {
      const float bv[8] = {bq[0].x, bq[0].y, bq[0].z, bq[0].w, bq[1].x, bq[1].y, bq[1].z, bq[1].w};
      h8 bhi, blo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bhi[e] = (_Float16)bv[e];
        blo[e] = (_Float16)(bv[e] - (float)bhi[e]);
      }
      f16x zero;
#pragma unroll
      for (int e = 0; e < 16; ++e) zero[e] = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        h8 ahi, alo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ahi[e] = (_Float16)av[blk][e];
          alo[e] = (_Float16)(av[blk][e] - (float)ahi[e]);
        }
        // rows of the product = channels (A^T), columns = weight rows (B^T)
        f16x acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bhi, zero, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, blo, acc, 0, 0, 0);
        // lane: weight row l32, channels 8 (e / 4) + 4 hh + e % 4 of the block
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          _Float16* p = &wt[l32 * kRowPitch + 64 * wave + 32 * blk + 8 * e4 + 4 * hh];
          const uint2 raw = *reinterpret_cast<const uint2*>(p);
          const h2 w01 = __builtin_bit_cast(h2, raw.x), w23 = __builtin_bit_cast(h2, raw.y);
          const h2 o01 = {(_Float16)((float)w01[0] + acc[4 * e4 + 0]), (_Float16)((float)w01[1] + acc[4 * e4 + 1])};
          const h2 o23 = {(_Float16)((float)w23[0] + acc[4 * e4 + 2]), (_Float16)((float)w23[1] + acc[4 * e4 + 3])};
          *reinterpret_cast<uint2*>(p) = make_uint2(__builtin_bit_cast(uint32_t, o01), __builtin_bit_cast(uint32_t, o23));
        }
      }
    }
    __syncthreads();
  }

  if constexpr (EXPAND) {
    // W_hat rows of the slab, the load's piece order (one row per 16 lanes)
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int p = tid + i * kThreads;
      const int row = p / kPR, col = (p % kPR) * 8;
      if (col < width)
        *reinterpret_cast<uint4*>(wexp + (int64_t)(nt * 32 + row) * d_in + c0 + col) =
            *reinterpret_cast<const uint4*>(&wt[row * kRowPitch + col]);
    }
  }
  // codes: steps [c0/64, c0/64 + width/64) of tile nt are contiguous
  {
    const int words = (width / 64) * 32 * SW;
    uint32_t* gdst = codes + ((int64_t)nt * (d_in / 64) + c0 / 64) * 32 * SW;
    for (int i = tid; i < words / 4; i += kThreads)
      __builtin_nontemporal_store(reinterpret_cast<const u4v*>(outc)[i], reinterpret_cast<u4v*>(gdst) + i);
  }
  // scales / zeros: groups [c0/G, c0/G + width/G) of tile nt are contiguous;
  // 16-byte pieces, the first threads take the scales, the next the zeros
  {
    const int pieces = (width / G) * 32 / 8;
    const int64_t off = ((int64_t)nt * (d_in / G) + c0 / G) * 32;
    if (tid < pieces)
      __builtin_nontemporal_store(reinterpret_cast<const u4v*>(outs)[tid], reinterpret_cast<u4v*>(scales + off) + tid);
    else if (tid < 2 * pieces)
      __builtin_nontemporal_store(reinterpret_cast<const u4v*>(outz)[tid - pieces], reinterpret_cast<u4v*>(zeros + off) + (tid - pieces));
  }
}

// The same quantisation without the effective weight, for groups of at most
// 64 channels, with one wave per (32-row tile, 64-channel step) and no
// workgroup barrier: each wave copies its 32 x 64 fp16 slab (4 KB) into its
// own part of LDS by direct-to-LDS loads (8 lanes per 128-byte row piece, the
// 16-byte pieces XOR-swizzled by row so the block reads below are free of
// bank conflicts), lane (r, h) = lane h * 32 + r quantises channels
// 32h .. 32h + 31 of row r (a 64-channel group meets through one lane
// exchange with lane r + 32), and the step's codes leave as the one
// contiguous chunk the tiled order gives them (Q x 256 bytes).  Waves never
// wait for one another; the four waves of a workgroup take four consecutive
// steps of a tile (32 rows x 512 bytes of W).  The slab copies carry the
// nontemporal hint: at the Qwen3-32B q_proj shape that measured 3-4 % faster
// than plain copies, warm and cold.
constexpr int kStepWaves = 4;
template <int Q, int G>
__global__ __launch_bounds__(64 * kStepWaves) void quantize_pack_step_kernel(
    const _Float16* __restrict__ W, const float* __restrict__ D, int d_in, uint32_t* __restrict__ codes,
    _Float16* __restrict__ scales, _Float16* __restrict__ zeros) {
  static_assert(G == 16 || G == 32 || G == 64, "one step holds whole groups");
  constexpr int SG = G < 32 ? 32 / G : 1;  // groups inside one 32-channel block
  constexpr int CPG = 32 / SG;
  constexpr int SW = 2 * Q;  // words per row per step
  __shared__ __attribute__((aligned(16))) uint4 slab[kStepWaves][256];  // 32 rows x 8 pieces
  __shared__ __attribute__((aligned(16))) float sqs[kStepWaves][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ksteps = d_in / 64;
  const int k = blockIdx.x * kStepWaves + wave;  // the wave's step
  if (k >= ksteps) return;                        // whole waves only: no barrier follows
  const int nt = blockIdx.y;                      // row tile
  uint4* sw = &slab[wave][0];

  // sqrt(D) of the step's channels, then the slab: LDS piece 64 i + lane
  // holds 16-byte piece (lane % 8) ^ (lane / 8) of row 8 i + lane / 8
  const float dj = D[k * 64 + lane];
  {
    const __amdgpu_buffer_rsrc_t rw = unpack::make_rsrc(W + (int64_t)nt * 32 * d_in, (int64_t)32 * d_in * 2);
    const int pr = lane >> 3, pc = (lane & 7) ^ pr;
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack::lds_dma16<2>(rw, (8 * i + pr) * d_in * 2 + k * 128 + pc * 16, sw + 64 * i);
  }
  sqs[wave][lane] = sqrtf(dj);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the copies have landed

  const int r = lane & 31, h = lane >> 5;
  float v[32];
  float mn[SG], mx[SG];
#pragma unroll
  for (int sg = 0; sg < SG; ++sg) mn[sg] = mx[sg] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 raw = sw[8 * r + ((4 * h + i) ^ (r & 7))];
    const float4 sa = *reinterpret_cast<const float4*>(&sqs[wave][32 * h + 8 * i]);
    const float4 sb = *reinterpret_cast<const float4*>(&sqs[wave][32 * h + 8 * i + 4]);
    float* o = &v[8 * i];
    o[0] = mul_lo(raw.x, sa.x); o[1] = mul_hi(raw.x, sa.y);
    o[2] = mul_lo(raw.y, sa.z); o[3] = mul_hi(raw.y, sa.w);
    o[4] = mul_lo(raw.z, sb.x); o[5] = mul_hi(raw.z, sb.y);
    o[6] = mul_lo(raw.w, sb.z); o[7] = mul_hi(raw.w, sb.w);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[(8 * i + e) / CPG] = fminf(mn[(8 * i + e) / CPG], o[e]);
      mx[(8 * i + e) / CPG] = fmaxf(mx[(8 * i + e) / CPG], o[e]);
    }
  }
  if constexpr (G == 64) {  // the group's other half is lane r + 32 (or r)
    mn[0] = fminf(mn[0], __shfl_xor(mn[0], 32));
    mx[0] = fmaxf(mx[0], __shfl_xor(mx[0], 32));
  }
  float s[SG], zf[SG], rcp[SG];
  _Float16 s16[SG];
#pragma unroll
  for (int sg = 0; sg < SG; ++sg) group_params<Q>(mn[sg], mx[sg], s16[sg], s[sg], zf[sg], rcp[sg]);
  uint32_t word[Q];
  block_codes<Q, CPG>(v, s, zf, rcp, word);

  // the step's code chunk (32 rows x SW words) through the slab's LDS, which
  // this wave alone has read
  asm volatile("" ::: "memory");
  uint32_t* oc = reinterpret_cast<uint32_t*>(sw);
#pragma unroll
  for (int w = 0; w < Q; ++w) oc[r * SW + step_pos<Q>(h, w)] = word[w];
  asm volatile("" ::: "memory");
  {
    uint32_t* gdst = codes + ((int64_t)nt * ksteps + k) * 32 * SW;
#pragma unroll
    for (int i = lane; i < 8 * SW; i += 64)
      __builtin_nontemporal_store(reinterpret_cast<const u4v*>(oc)[i], reinterpret_cast<u4v*>(gdst) + i);
  }
  // scales and zeros: group gi of tile nt at (nt * d_in / G + gi) * 32 + row
  const int64_t gbase = (int64_t)nt * (d_in / G) * 32;
  if constexpr (G == 64) {
    if (h == 0) {
      scales[gbase + (int64_t)k * 32 + r] = s16[0];
      zeros[gbase + (int64_t)k * 32 + r] = (_Float16)zf[0];
    }
  } else {
#pragma unroll
    for (int sg = 0; sg < SG; ++sg) {
      const int64_t gi = (int64_t)k * (64 / G) + h * SG + sg;
      scales[gbase + gi * 32 + r] = s16[sg];
      zeros[gbase + gi * 32 + r] = (_Float16)zf[sg];
    }
  }
}

template <int Q, bool EX, bool LR>
hipError_t launch_qe(int d_out, int d_in, int g, const _Float16* W, const float* D, uint32_t* codes,
                     _Float16* scales, _Float16* zeros, const _Float16* dinv16, _Float16* wexp, const float* B,
                     const float* A, hipStream_t s) {
  dim3 grid((unsigned)((d_in + kCols - 1) / kCols), (unsigned)(d_out / 32));
#define TTQ_QP(GV) hipLaunchKernelGGL((quantize_pack_kernel<Q, GV, EX, LR>), grid, dim3(kThreads), 0, s, W, D, d_in, \
                                      codes, scales, zeros, dinv16, wexp, B, A)
  switch (g) {
    case 16: TTQ_QP(16); break;
    case 32: TTQ_QP(32); break;
    case 64: TTQ_QP(64); break;
    default: TTQ_QP(128); break;
  }
#undef TTQ_QP
  return hipGetLastError();
}

template <int Q>
hipError_t launch_q(int d_out, int d_in, int g, const _Float16* W, const float* D, uint32_t* codes,
                    _Float16* scales, _Float16* zeros, const _Float16* dinv16, _Float16* wexp, const float* B,
                    const float* A, hipStream_t s) {
  if (wexp == nullptr && g <= 64) {
    const dim3 grid((unsigned)((d_in / 64 + kStepWaves - 1) / kStepWaves), (unsigned)(d_out / 32));
#define TTQ_QS(GV) hipLaunchKernelGGL((quantize_pack_step_kernel<Q, GV>), grid, dim3(64 * kStepWaves), 0, s, W, D, \
                                      d_in, codes, scales, zeros)
    switch (g) {
      case 16: TTQ_QS(16); break;
      case 32: TTQ_QS(32); break;
      default: TTQ_QS(64); break;
    }
#undef TTQ_QS
    return hipGetLastError();
  }
  if (wexp != nullptr && B != nullptr)
    return launch_qe<Q, true, true>(d_out, d_in, g, W, D, codes, scales, zeros, dinv16, wexp, B, A, s);
  if (wexp != nullptr)
    return launch_qe<Q, true, false>(d_out, d_in, g, W, D, codes, scales, zeros, dinv16, wexp, B, A, s);
  return launch_qe<Q, false, false>(d_out, d_in, g, W, D, codes, scales, zeros, dinv16, wexp, B, A, s);
}

}  // namespace

hipError_t launch_quantize_pack(int d_out, int d_in, int q, int g, const void* W, const float* D,
                                uint32_t* codes, void* scales, void* zeros, const void* dinv16, void* wexp,
                                const float* B, const float* A, hipStream_t s) {
  const _Float16* w = static_cast<const _Float16*>(W);
  _Float16* sc = static_cast<_Float16*>(scales);
  _Float16* ze = static_cast<_Float16*>(zeros);
  const _Float16* dv = static_cast<const _Float16*>(dinv16);
  _Float16* we = static_cast<_Float16*>(wexp);
  switch (q) {
    case 2: return launch_q<2>(d_out, d_in, g, w, D, codes, sc, ze, dv, we, B, A, s);
    case 3: return launch_q<3>(d_out, d_in, g, w, D, codes, sc, ze, dv, we, B, A, s);
    case 5: return launch_q<5>(d_out, d_in, g, w, D, codes, sc, ze, dv, we, B, A, s);
    default: return launch_q<4>(d_out, d_in, g, w, D, codes, sc, ze, dv, we, B, A, s);
  }
}

}  // namespace ttq
