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
// Output is in the tiled storage order (32-row tiles, one contiguous chunk
// per 64-channel step; see include/ttq.h).
//
// Work split: a workgroup of 256 threads owns 256 input channels (8 blocks
// of 32) and walks 32-row tiles of W.  Per tile:
//   * the 32 x 256 fp16 slab (16 KB) comes in with 16-byte loads, two full
//     rows per wave instruction, and is parked in LDS (the next tile's loads
//     are issued before this tile is processed);
//   * thread (r, b) = (row in tile, 32-channel block) quantises its block
//     from LDS with the 32 sqrt(D) values the workgroup computed once;
//     groups of 64 / 128 channels meet through an LDS min/max exchange;
//   * codes are placed in LDS in the tiled order and leave as one contiguous
//     store of 4 steps x 32 rows x 2q words; scales and zeros likewise.
//
// Codes use a reciprocal fast path: with r = 1/s (one IEEE division per
// group), u = fma(v, r, z) lies within 2^-18 of v/s + z, so whenever u is
// more than 2^-16 away from every half-integer, rint(u) equals
// rint(fl(v/s)) + z exactly.  If any element of a thread's 32-channel block
// comes closer, the whole block is redone with the IEEE division (rare; the
// fast codes of the other elements would have been the same).
#include "ttq_internal.h"

#pragma clang fp contract(off)

namespace ttq {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 256;             // channels per workgroup
constexpr int kRowPitch = kCols + 8;   // fp16 elements per LDS row (pad: 16 bytes)

// smallest positive fp16 that is >= x (x >= 0, finite)
__device__ __forceinline__ _Float16 fp16_round_up(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  unsigned short b = __builtin_bit_cast(unsigned short, h);
  if ((float)h < x) b = (unsigned short)(b + 1);  // next fp16 up (positive values)
  if (b == 0) b = 1;                              // 2^-24, smallest positive
  return __builtin_bit_cast(_Float16, b);
}

// position of canonical word w of block-in-step h inside a row's 2q step words
template <int Q>
__device__ __forceinline__ constexpr int step_pos(int h, int w) {
  if constexpr (Q == 4) return 4 * (w % 2) + 2 * h + w / 2;
  else return Q * h + w;
}

template <int Q, int G>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(
    const _Float16* __restrict__ W, const float* __restrict__ D, int d_out, int d_in,
    int tiles_per_wg, uint32_t* __restrict__ codes, _Float16* __restrict__ scales,
    _Float16* __restrict__ zeros) {
  constexpr int LPG = G / 32;               // blocks per group
  constexpr float N = (float)((1 << Q) - 1);
  constexpr int SW = 2 * Q;                 // words per row per 64-channel step
  constexpr int GPW = kCols / G;            // groups per workgroup column range

  __shared__ __attribute__((aligned(16))) _Float16 wt[32 * kRowPitch];
  __shared__ float sq[kCols];
  __shared__ __attribute__((aligned(16))) uint32_t outc[4 * 32 * SW];
  __shared__ __attribute__((aligned(16))) _Float16 outs[GPW * 32], outz[GPW * 32];
  __shared__ float red_mn[8][32], red_mx[8][32];

  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * kCols;
  const int width = min(kCols, d_in - c0);  // 64, 128, 192 or 256
  const int n_tiles = d_out / 32;
  const int t_begin = blockIdx.y * tiles_per_wg;
  const int t_end = min(n_tiles, t_begin + tiles_per_wg);

  // sqrt(D) of this workgroup's channels, correctly rounded, once
  if (tid < width) sq[tid] = sqrtf(D[c0 + tid]);

  // slab loader: 1024 16-byte pieces, piece p -> row p / 32, column 8 * (p % 32).
  // Four named registers, not an array: an array captured by reference would
  // be placed in scratch memory.
  uint4 pre0 = make_uint4(0, 0, 0, 0), pre1 = pre0, pre2 = pre0, pre3 = pre0;
  auto piece_ptr = [&](int nt, int i) -> const uint4* {
    const int p = tid + i * kThreads;
    const int row = p >> 5, col = (p & 31) * 8;
    return reinterpret_cast<const uint4*>(W + (int64_t)(nt * 32 + row) * d_in + c0 + col);
  };
  auto piece_ok = [&](int i) { return ((tid + i * kThreads) & 31) * 8 < width; };
  auto load_tile = [&](int nt) {
    if (piece_ok(0)) pre0 = *piece_ptr(nt, 0);
    if (piece_ok(1)) pre1 = *piece_ptr(nt, 1);
    if (piece_ok(2)) pre2 = *piece_ptr(nt, 2);
    if (piece_ok(3)) pre3 = *piece_ptr(nt, 3);
  };
  if (t_begin < t_end) load_tile(t_begin);

  // this thread's block: r = row in tile, bl = block in the column range
  const int r = tid & 31, bl = tid >> 5;
  const bool active = 32 * bl < width;
  const int h = bl & 1, ksl = bl >> 1;

  for (int nt = t_begin; nt < t_end; ++nt) {
    __syncthreads();  // previous tile's LDS reads and stores are done
    auto park = [&](int i, const uint4& v) {
      const int p = tid + i * kThreads;
      const int row = p >> 5, col = (p & 31) * 8;
      if (col < width) *reinterpret_cast<uint4*>(&wt[row * kRowPitch + col]) = v;
    };
    park(0, pre0);
    park(1, pre1);
    park(2, pre2);
    park(3, pre3);
    __syncthreads();
    if (nt + 1 < t_end) load_tile(nt + 1);

    float v[32];
    float mn = 0.f, mx = 0.f;
    if (active) {
      const _Float16* src = &wt[r * kRowPitch + bl * 32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * i);
        const _Float16* e = reinterpret_cast<const _Float16*>(&raw);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v[8 * i + k] = (float)e[k] * sq[bl * 32 + 8 * i + k];
          mn = fminf(mn, v[8 * i + k]);
          mx = fmaxf(mx, v[8 * i + k]);
        }
      }
    }
    if constexpr (LPG > 1) {
      red_mn[bl][r] = mn;
      red_mx[bl][r] = mx;
      __syncthreads();
      const int first = bl & ~(LPG - 1);
#pragma unroll
      for (int j = 0; j < LPG; ++j) {
        mn = fminf(mn, red_mn[first + j][r]);
        mx = fmaxf(mx, red_mx[first + j][r]);
      }
    }

    if (active) {
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
      auto put = [&](int k, float c) {
        const uint32_t ci = (uint32_t)fminf(fmaxf(c, 0.0f), N);
        const int bit = Q * k;
        word[bit >> 5] |= ci << (bit & 31);
        if ((bit & 31) + Q > 32) word[(bit >> 5) + 1] |= ci >> (32 - (bit & 31));
      };
#pragma unroll
      for (int i = 0; i < Q; ++i) word[i] = 0u;
      bool near_tie = false;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const float u = __builtin_fmaf(v[k], rcp, zf);
        const float c = rintf(u);
        near_tie |= fabsf(u - c) > 0.5f - 0x1p-16f;
        put(k, c);
      }
      if (near_tie) {  // rare: redo the block with the IEEE division
#pragma unroll
        for (int i = 0; i < Q; ++i) word[i] = 0u;
#pragma unroll
        for (int k = 0; k < 32; ++k) put(k, rintf(v[k] / s) + zf);
      }
      uint32_t* dst = &outc[(ksl * 32 + r) * SW];
#pragma unroll
      for (int w = 0; w < Q; ++w) dst[step_pos<Q>(h, w)] = word[w];
      if ((bl % LPG) == 0) {
        outs[(bl / LPG) * 32 + r] = s16;
        outz[(bl / LPG) * 32 + r] = (_Float16)zf;
      }
    }
    __syncthreads();

    // codes: steps [c0/64, c0/64 + width/64) of tile nt are contiguous
    {
      const int words = (width / 64) * 32 * SW;
      uint32_t* gdst = codes + ((int64_t)nt * (d_in / 64) + c0 / 64) * 32 * SW;
      for (int i = tid; i < words / 4; i += kThreads)
        reinterpret_cast<uint4*>(gdst)[i] = reinterpret_cast<const uint4*>(outc)[i];
    }
    // scales / zeros: groups [c0/G, c0/G + width/G) of tile nt are contiguous;
    // 16-byte pieces, the first threads take the scales, the next the zeros
    {
      const int pieces = (width / G) * 32 / 8;
      const int64_t off = ((int64_t)nt * (d_in / G) + c0 / G) * 32;
      if (tid < pieces)
        reinterpret_cast<uint4*>(scales + off)[tid] = reinterpret_cast<const uint4*>(outs)[tid];
      else if (tid < 2 * pieces)
        reinterpret_cast<uint4*>(zeros + off)[tid - pieces] = reinterpret_cast<const uint4*>(outz)[tid - pieces];
    }
  }
}

template <int Q>
hipError_t launch_q(int d_out, int d_in, int g, const _Float16* W, const float* D, uint32_t* codes,
                    _Float16* scales, _Float16* zeros, hipStream_t s) {
  const int col_wgs = (d_in + kCols - 1) / kCols;
  const int n_tiles = d_out / 32;
  // about 8 row tiles per workgroup, but enough workgroups to fill the chip
  int per = 8;
  while (per > 1 && (int64_t)col_wgs * ((n_tiles + per - 1) / per) < 1024) per >>= 1;
  const int row_wgs = (n_tiles + per - 1) / per;
  dim3 grid((unsigned)col_wgs, (unsigned)row_wgs);
  switch (g) {
    case 32:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 32>), grid, dim3(kThreads), 0, s, W, D, d_out, d_in,
                         per, codes, scales, zeros);
      break;
    case 64:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 64>), grid, dim3(kThreads), 0, s, W, D, d_out, d_in,
                         per, codes, scales, zeros);
      break;
    default:
      hipLaunchKernelGGL((quantize_pack_kernel<Q, 128>), grid, dim3(kThreads), 0, s, W, D, d_out, d_in,
                         per, codes, scales, zeros);
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
