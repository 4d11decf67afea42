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
// Work split: a workgroup of 128 threads owns one 32-row tile of W over 128
// input channels (4 blocks of 32), 10240 workgroups at the Qwen3-32B q_proj
// shape (small workgroups keep many slabs in flight per CU):
//   * the 32 x 128 fp16 slab (8 KB) comes in with 16-byte loads, one full
//     row per 16 lanes, and is parked in LDS (rows padded by 16 bytes, so
//     the block reads below hit 16 distinct bank groups);
//   * thread (r, b) = (row in tile, 32-channel block) quantises its block
//     from LDS (as two groups when g = 16); groups of 64 / 128 channels meet
//     through an LDS min/max exchange;
//   * codes are placed in LDS in the tiled order and leave as one contiguous
//     store of 2 steps x 32 rows x 2q words; scales and zeros likewise (all
//     with nontemporal stores, which measured about 5 % faster here).
// v = w * sq is one v_fma_mix_f32 (fp16 operand, fp32 arithmetic) and the
// codes are packed bytewise with v_cvt_pk_u8_f32.
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

template <int Q, int G>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(
    const _Float16* __restrict__ W, const float* __restrict__ D, int d_in,
    uint32_t* __restrict__ codes, _Float16* __restrict__ scales, _Float16* __restrict__ zeros) {
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
    for (int sg = 0; sg < SG; ++sg) {
      if (mx[sg] == mn[sg]) {  // all-zero group
        s16[sg] = (_Float16)1.0f;
        s[sg] = 1.0f;
        zf[sg] = 0.0f;
      } else {
        const float s32 = (mx[sg] - mn[sg]) / N;
        s16[sg] = fp16_round_up(s32);
        s[sg] = (float)s16[sg];
        // z by the same reciprocal fast path
        const float x = -mn[sg] * __builtin_amdgcn_rcpf(s[sg]);
        float zr = rintf(x);
        if (fabsf(x - zr) > 0.5f - 0x1p-16f) zr = rintf(-mn[sg] / s[sg]);
        zf[sg] = fminf(fmaxf(zr, 0.0f), N) + 0.0f;
      }
      rcp[sg] = __builtin_amdgcn_rcpf(s[sg]);
    }

    // code(k) gives the integer-valued float stored in slot k; packing into
    // the bitstream (slot k at bit Q*k of the block's Q words)
    uint32_t word[Q];
    auto pack = [&](auto&& code) {
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
          // code(k) is in [0, N] on both paths below (the fast one by its
          // error bound, the exact one by its clamp)
          const uint32_t ci = (uint32_t)code(k);
          const int bit = Q * k;
          word[bit >> 5] |= ci << (bit & 31);
          if ((bit & 31) + Q > 32) word[(bit >> 5) + 1] |= ci >> (32 - (bit & 31));
        }
      }
    };
    float far = 0.0f;  // largest distance of u from its rounded value
    pack([&](int k) {
      const int ch = slot_channel(k), sg = ch / CPG;
      const float u = __builtin_fmaf(v[ch], rcp[sg], zf[sg]);
      const float c = rintf(u);
      far = fmaxf(far, fabsf(u - c));
      return c;
    });
    if (far > 0.5f - 0x1p-16f)  // rare: redo the block with the IEEE division
      pack([&](int k) {
        const int ch = slot_channel(k), sg = ch / CPG;
        return fminf(fmaxf(rintf(v[ch] / s[sg]) + zf[sg], 0.0f), N);
      });
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
  __syncthreads();

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

template <int Q>
hipError_t launch_q(int d_out, int d_in, int g, const _Float16* W, const float* D, uint32_t* codes,
                    _Float16* scales, _Float16* zeros, hipStream_t s) {
  dim3 grid((unsigned)((d_in + kCols - 1) / kCols), (unsigned)(d_out / 32));
  switch (g) {
    case 16:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 16>), grid, dim3(kThreads), 0, s, W, D, d_in, codes,
                         scales, zeros);
      break;
    case 32:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 32>), grid, dim3(kThreads), 0, s, W, D, d_in, codes,
                         scales, zeros);
      break;
    case 64:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 64>), grid, dim3(kThreads), 0, s, W, D, d_in, codes,
                         scales, zeros);
      break;
    default:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 128>), grid, dim3(kThreads), 0, s, W, D, d_in, codes,
                         scales, zeros);
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
    case 5: return launch_q<5>(d_out, d_in, g, w, D, codes, sc, ze, s);
    default: return launch_q<4>(d_out, d_in, g, w, D, codes, sc, ze, s);
  }
}

}  // namespace ttq
