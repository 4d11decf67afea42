// The TTQ projection of a long prompt from the effective weight formed once
// per prompt:
//   Y = W_hat X + B Z,  W_hat[n][j] = fp16(fp16((c - z) s) * fp16(d_j^(-1/2)))
// i.e. the pages' closed form Q[W D^(1/2)] D^(-1/2) (paper-daily.com deep
// reading, section 2) materialised in fp16 by the quantiser, then applied to
// the raw input (Z = A X for the rank-16 term, gist.science French summary,
// section 2B).  The fused low-bit kernel dequantises every weight fragment
// again for each 256-token tile (64 times per weight at 16384 tokens); here it
// is done once, and this kernel is a dense fp16 GEMM.  W_hat holds exactly the
// fp16 values the fused raw-input kernel feeds its matrix cores, and the K
// order of the MFMAs is the same, so the outputs are the same bit for bit.
//
// CDNA4 design (gfx950, wave64, v_mfma_f32_32x32x16_f16):
//   * Workgroup tile 256 output channels x 256 tokens of Y^T; eight waves
//     in a 2 x 4 grid, each owning 4 x 2 fragments of 32 x 32 (128 channels x
//     64 tokens) with fp32 accumulators in AGPRs: 128 accumulator registers,
//     two waves per SIMD, 6 LDS reads per 8 MFMAs.
//   * K loop in 64-channel steps through two LDS stages (X tile and W_hat
//     tile, 32 KB each per stage: 128 KB), filled only by direct-to-LDS
//     buffer loads.  One wait and one barrier per step, before its last
//     16-channel sub-step: by then every wave has read the step's operands
//     out of its stage (the last sub-step's operands are already in
//     registers), so the loads of step k + 2 go into that stage right after
//     the barrier, while the last sub-step's MFMAs run and the next step's
//     operands come from the other stage.  A load thus has one step to land.
//     128-byte tile rows carry an XOR swizzle of their eight 16-byte chunks
//     (chunk ^ (row / 2) % 8), applied through the source offsets, so the 16
//     lanes of one LDS read phase hit 16 distinct bank groups.
//   * MFMA A = W_hat fragment (rows = output channels), B = X fragment
//     (columns = tokens); operands of the next sub-step are read from LDS
//     under the current sub-step's MFMAs.
//   * Rows past T or d_out read as zeros through the buffer resources and
//     are never stored; workgroup ids are remapped so each XCD walks a
//     contiguous band of tiles, 4 token tiles x all channel tiles at a time.
#include <type_traits>
#include <utility>

#include "ttq_internal.h"

namespace ttq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int BN = 256;  // output channels per workgroup
constexpr int BM = 256;  // tokens per workgroup
constexpr int BK = 64;   // input channels per step
constexpr int kXcds = 8;

template <int I>
using ic = std::integral_constant<int, I>;

template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(ic<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

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

// raw buffer resource over [base, base + bytes): loads past the end read zeros
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nrec = (int)min<int64_t>(bytes, (int64_t)0x7FFFFFF0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

// 16 bytes per lane from a buffer into LDS; lane l lands at lds_wave_base + 16 l
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, int voff, int soff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           voff, soff, 0, 0);
}

// XOR swizzle of the eight 16-byte chunks of a 128-byte tile row: rows 2k and
// 2k + 1 share a 256-byte bank window, so the row pair picks the permutation
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int WN, int WM, typename TY, bool LOWRANK>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WN * WM, 64 * WN * WM),
                          amdgpu_waves_per_eu(WN * WM / 4, WN * WM / 4)))
void dense_gemm_kernel(int64_t T, int d_in, int d_out, const _Float16* __restrict__ X, int64_t ldx,
                       const _Float16* __restrict__ Wt, const float* __restrict__ Bf,
                       const float* __restrict__ Z, TY* __restrict__ Y, int64_t ldy, int tiles_n, int tiles) {
  constexpr int NW = WN * WM;
  constexpr int kThreads = 64 * NW;
  constexpr int FN = 8 / WN;                 // 32-row fragments per wave
  constexpr int FM = 8 / WM;                 // 32-token fragments per wave
  constexpr int SL = BM * BK * 2 / 16;       // 16-byte slots per tile and stage (X and W alike)
  constexpr int LPW = SL / kThreads;         // loads per wave per tile and step
  static_assert(SL % kThreads == 0 && BM == BN, "slot split");

  __shared__ __attribute__((aligned(16))) _Float16 xs0[BM * BK], xs1[BM * BK];
  __shared__ __attribute__((aligned(16))) _Float16 ws0[BN * BK], ws1[BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wn = wave % WN, wm = wave / WN;

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

  asm volatile("; accumulators in AGPRs" ::"a"(0.0f));
  f16x acc[FN][FM];
  f16x c0;
#pragma unroll
  for (int e = 0; e < 16; ++e) c0[e] = 0.f;
  {
    uint32_t zr = 0u;
    asm volatile("" : "+v"(zr));
    const h2 zp = __builtin_bit_cast(h2, zr);
    const h8 z8 = {zp[0], zp[1], zp[0], zp[1], zp[0], zp[1], zp[0], zp[1]};
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(z8, z8, c0, 0, 0, 0);
  }

  auto xstage = [&](auto st) -> _Float16* {
    if constexpr (decltype(st)::value == 0) return xs0;
    else return xs1;
  };
  auto wstage = [&](auto st) -> _Float16* {
    if constexpr (decltype(st)::value == 0) return ws0;
    else return ws1;
  };

  // Loads: slot p = 64 (wave + NW j) + lane -> tile row p / 8, physical chunk
  // p % 8 holding logical chunk (p % 8) ^ swz(row); rows of slot j are row_0 +
  // 8 NW j with the same swizzle, so the lane's offset is shared and j enters
  // the scalar offset.
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(X + m0 * ldx, (T - m0) * ldx * 2);
  const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(Wt + (int64_t)n0 * d_in, (int64_t)(d_out - n0) * d_in * 2);
  const int lrow = wave * 8 + (lane >> 3);
  const int lchunk = (lane & 7) ^ swz(lrow);
  const int xoff = (int)(lrow * ldx * 2) + 16 * lchunk;
  const int woff = lrow * d_in * 2 + 16 * lchunk;
  const int xjstride = (int)(8 * NW * ldx * 2);
  const int wjstride = 8 * NW * d_in * 2;

  auto load_lds = [&](int kt, _Float16* xs, _Float16* ws) {
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      lds_dma16(rs_x, xoff, kt * BK * 2 + j * xjstride, reinterpret_cast<char*>(xs) + 16 * (wave + NW * j) * 64);
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      lds_dma16(rs_w, woff, kt * BK * 2 + j * wjstride, reinterpret_cast<char*>(ws) + 16 * (wave + NW * j) * 64);
  };

  // operand fragment (32 rows x 16 channels of sub-step S) of a stage
  auto read_frag = [&](const _Float16* st, int row0, int S) -> h8 {
    const int row = row0 + l32;
    const int c = (2 * S + hh) ^ swz(row);
    return *reinterpret_cast<const h8*>(&st[row * BK + c * 8]);
  };

  h8 aop[2][FN], bop[2][FM];

  // prologue: steps 0 and 1 requested, step 0 landed, its first operands read
  load_lds(0, xs0, ws0);
  wait_vmem<0>();
  load_lds(min(1, ksteps - 1), xs1, ws1);
  block_barrier();
#pragma unroll
  for (int i = 0; i < FN; ++i) aop[0][i] = read_frag(ws0, wn * 32 * FN + 32 * i, 0);
#pragma unroll
  for (int j = 0; j < FM; ++j) bop[0][j] = read_frag(xs0, wm * 32 * FM + 32 * j, 0);

  // one K step on stage ST
  auto step = [&](auto stc, int kt) {
    constexpr int ST = decltype(stc)::value, N1 = ST ^ 1;
    unroll<4>([&](auto sc_) {
      constexpr int S = decltype(sc_)::value;
      constexpr int P = S & 1, PN = P ^ 1;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (S == 3) {
        // step kt + 1 has landed for every wave; nobody reads stage ST any
        // more, so step kt + 2 goes there.  Unconditional (the last steps
        // repeat step ksteps - 1 into a stage nobody reads again), so the
        // loads share a block with the MFMAs they are scheduled between.
        wait_vmem<0>();
        block_barrier();
        load_lds(min(kt + 2, ksteps - 1), xstage(ic<ST>{}), wstage(ic<ST>{}));
      }
      // the next sub-step's operands (after the last step: stale, in-bounds
      // LDS data that is never used)
      const _Float16* xsrc = (S < 3) ? xstage(ic<ST>{}) : xstage(ic<N1>{});
      const _Float16* wsrc = (S < 3) ? wstage(ic<ST>{}) : wstage(ic<N1>{});
      constexpr int SN = (S + 1) & 3;
#pragma unroll
      for (int i = 0; i < FN; ++i) aop[PN][i] = read_frag(wsrc, wn * 32 * FN + 32 * i, SN);
#pragma unroll
      for (int j = 0; j < FM; ++j) bop[PN][j] = read_frag(xsrc, wm * 32 * FM + 32 * j, SN);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[P][i], bop[P][j], acc[i][j], 0, 0, 0);
      // the next sub-step's LDS reads first (a whole sub-step of MFMAs to
      // land; issued between MFMAs they left the next sub-step waiting), then
      // the MFMAs; after the barrier the step's direct-to-LDS loads go
      // between them
      __builtin_amdgcn_sched_group_barrier(0x100, FN + FM, 0);
#pragma unroll
      for (int m = 0; m < FN * FM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (S == 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    });
  };

  for (int kt = 0;; kt += 2) {
    step(ic<0>{}, kt);
    if (kt + 1 >= ksteps) break;
    step(ic<1>{}, kt + 1);
    if (kt + 2 >= ksteps) break;
  }
  wait_vmem<0>();  // the repeated tail loads

  if constexpr (LOWRANK) {
    // B16 x Z_hi + B16 x Z_lo after the K loop (Z split in two fp16 parts),
    // in the low-bit kernel's order
    h8 bfr[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int n = min(n0 + wn * 32 * FN + i * 32 + l32, d_out - 1);
      const float4* bp = reinterpret_cast<const float4*>(Bf + (int64_t)n * 16 + 8 * hh);
      const float4 b0 = bp[0], b1 = bp[1];
      bfr[i][0] = (_Float16)b0.x; bfr[i][1] = (_Float16)b0.y;
      bfr[i][2] = (_Float16)b0.z; bfr[i][3] = (_Float16)b0.w;
      bfr[i][4] = (_Float16)b1.x; bfr[i][5] = (_Float16)b1.y;
      bfr[i][6] = (_Float16)b1.z; bfr[i][7] = (_Float16)b1.w;
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int64_t t = min(m0 + wm * 32 * FM + j * 32 + l32, T - 1);
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

  // epilogue: lane holds token l32 of each token fragment, channels
  // 8 (e / 4) + 4 hh + e % 4 of each row fragment
  if constexpr (sizeof(TY) == 2 && WN == 2 && WM == 4) {
    // fp16 outputs leave through LDS as whole 512-byte token rows (stored
    // straight from the accumulators, every store instruction would write 16
    // bytes into each of 32 rows): the tile (256 tokens x 256 channels, 128
    // KB) fills the four stages, token group wm (64 tokens) in stage wm, the
    // 16-byte chunks of row r XOR-swizzled by r % 32.
    auto stage = [&](int g) -> char* {
      return reinterpret_cast<char*>(g == 0 ? xs0 : g == 1 ? xs1 : g == 2 ? ws0 : ws1);
    };
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();  // every wave is done with the stages
    {
      char* yb = stage(wm);
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int r = j * 32 + l32;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int c = (wn * FN + i) * 4 + e4;  // 16-byte chunk (8 channels) of the row
            const h2 a = {(_Float16)acc[i][j][4 * e4 + 0], (_Float16)acc[i][j][4 * e4 + 1]};
            const h2 b = {(_Float16)acc[i][j][4 * e4 + 2], (_Float16)acc[i][j][4 * e4 + 3]};
            *reinterpret_cast<uint2*>(yb + r * 512 + ((c ^ (r & 31)) * 16) + 8 * hh) =
                make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
          }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();
    {
      // wave w stores tile rows 32 w .. 32 w + 31
      const int g = wave >> 1;
      const char* yb = stage(g);
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int r = (wave & 1) * 32 + 2 * ii + hh;
        const int c = l32;
        const uint4 v = *reinterpret_cast<const uint4*>(yb + r * 512 + ((c ^ (r & 31)) * 16));
        const int64_t t = m0 + 64 * g + r;
        const int n = n0 + 8 * c;
        if (t < T && n < d_out) *reinterpret_cast<uint4*>(Y + t * ldy + n) = v;
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int64_t t = m0 + wm * 32 * FM + j * 32 + l32;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int n = n0 + wn * 32 * FN + i * 32 + 8 * e4 + 4 * hh;
        if (n < d_out) {
          float v[4] = {acc[i][j][4 * e4 + 0], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                        acc[i][j][4 * e4 + 3]};
          store4<TY>(Y + t * ldy + n, v);
        }
      }
    }
  }
}

template <int WN, int WM, bool LR>
hipError_t launch_w(int64_t T, int d_in, int d_out, const void* X, int64_t ldx, const void* Wt, const float* B,
                    const float* Z, void* Y, int64_t ldy, hipStream_t s) {
  const int tiles_n = (d_out + BN - 1) / BN;
  const int64_t tiles = (int64_t)tiles_n * ((T + BM - 1) / BM);
  hipLaunchKernelGGL((dense_gemm_kernel<WN, WM, _Float16, LR>), dim3((unsigned)tiles), dim3(64 * WN * WM), 0, s, T,
                     d_in, d_out, static_cast<const _Float16*>(X), ldx, static_cast<const _Float16*>(Wt), B, Z,
                     static_cast<_Float16*>(Y), ldy, tiles_n, (int)tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_gemm(int64_t T, int d_in, int d_out, int r, const void* X, int64_t ldx, const void* Wt,
                             const float* B, const float* Z, void* Y, int64_t ldy, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // eight waves of 128 channels x 64 tokens
  if (r > 0) return launch_w<2, 4, true>(T, d_in, d_out, X, ldx, Wt, B, Z, Y, ldy, s);
  return launch_w<2, 4, false>(T, d_in, d_out, X, ldx, Wt, B, Z, Y, ldy, s);
}

}  // namespace ttq
